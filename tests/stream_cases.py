"""Seeded contractions for the stream-plan tests (bsc_stream_plan): chain
stages with single-leg C blocks and random single-leg structures, some with C
blocks no product reaches.  Inputs only: nothing here computes a contraction."""
import numpy as np

from workloads import configs as C


def _stage(ch, si, seed):
    """Stage si of a chain with integer operands in {-2..2} (intermediate
    buffers filled with fresh integers, as if an earlier stage wrote them)."""
    st = ch.stages[si]
    rng = np.random.default_rng(seed)
    def buf(name):
        if name in ch.buffers:
            return np.asarray(ch.buffers[name], np.float64)
        return rng.integers(-2, 3, ch.sizes[name]).astype(np.float64)
    return st.con, buf(st.a_buf), buf(st.b_buf)


def _random(seed, dtype, density):
    p = C.random_problem(seed, nq=1, nkeys=(6, 5, 6), maxdim=40, qrange=1, dtype=dtype, density=density,
                         two_leg=False, int_values=True)
    return p.con, np.asarray(p.a, np.float64), np.asarray(p.b, np.float64)


# name: (factory -> (con, A values, B values), wave tile edge)
CASES = {
    "small-coop-stage1": (lambda: _stage(C.small_chain(seed=3, layout="coop", values="int"), 0, 1), 0),
    "small-coop-stage3": (lambda: _stage(C.small_chain(seed=3, layout="coop", values="int"), 2, 2), 0),
    "small-natural-f32-stage3": (lambda: _stage(C.small_chain(seed=5, layout="natural", values="int",
                                                              dtype="f32"), 2, 3), 0),
    "rabc_u1-stage3": (lambda: _stage(C.rabc_u1(layout="coop", values="int"), 2, 4), 0),
    "random-f64-sparse": (lambda: _random(7101, "f64", 0.5), 0),
    "random-f32-sparse": (lambda: _random(7102, "f32", 0.5), 0),
    "wide-f32-tile32": (lambda: _stage(C.small_chain(seed=3, layout="coop", dtype="f32", total=1024, qmax=4,
                                                     sigma=2.0, w=1, values="int"), 0, 5), 32),
    # every charge zero: 16 products per C block, each its own block, split over waves
    "neutral-f32-stage3-split": (lambda: _stage(C.neutral_chain(seed=4, layout="coop", dtype="f32"), 2, 6), 0),
}
