// The grouped contraction kernel: one launch walks a plan's whole work list
// (uni20 "block coalescing", section "Summary": issue fewer, larger kernels
// instead of one per sector GEMM).  A workgroup takes tasks blockIdx.x,
// blockIdx.x + gridDim.x, ... from a longest-first list; every C tile has
// exactly one owner, so sums need no atomics and repeat bit-for-bit.
//
// Each kernel variant (element types, the tile bodies it contains) is
// instantiated in one translation unit of its own (grouped_*.hip), so the
// variants compile in parallel; the runtime reaches them through launch.h.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "bsc_internal.h"
#include "kernels_generic.h"
#include "kernels_mfma_bf16.h"
#include "kernels_mfma_bf16_fast.h"
#include "kernels_mfma_bf16_wide.h"
#include "kernels_mfma_f.h"
#include "kernels_skinny.h"
#include "kernels_tail.h"
#include "launch.h"

namespace bsc {

// Shared memory of a grouped launch: the union of the tile bodies it contains.
template <typename TA>
struct MfmaSmemOf {
    typedef MfmaSmemF<TA> type;
};
template <>
struct MfmaSmemOf<uint16_t> {
    typedef MfmaSmemBf16 type;
};

template <typename TA, typename ACC, int32_t FEAT>
union TileSmem {
    GenericSmem<ACC> g;
    SkinnySmem<ACC> s;
    TailSmem<ACC> t;
    typename std::conditional<(FEAT & FEAT_MFMA) != 0, typename MfmaSmemOf<TA>::type, char>::type m;
    typename std::conditional<(FEAT & (FEAT_FAST_N | FEAT_FAST_K)) != 0, FastSmemBf16, char>::type f;
    typename std::conditional<(FEAT & FEAT_WIDE) != 0, WideSmemBf16, char>::type x;
};

extern __shared__ __align__(16) unsigned char bsc_dyn_smem[];

// A 256 x 128 direct-to-LDS task: a tile of at most 128 rows runs as a
// 128 x 128 tile of four 64 x 64 waves (every SIMD busy, four chunks of
// copies in flight in the same 80 KB ring), a taller one on the 256 x 128 tile.
template <typename TC, bool BN>
__device__ __forceinline__ void direct_tile_bf16(const KArgs &ka, const DFast &fd_ref, FastSmemBf16 &sm) {
    const DFast fd = fd_ref;   // one read of the record
    if (fd.mlen <= HalfTile::TM) wide_tile_body<TC, BN, HalfTile>(ka, fd, sm.op);
    else fast_tile_bf16<TC, BN>(ka, fd, sm);
}

template <typename TA, typename TC, typename ACC, int32_t FEAT>
__device__ __forceinline__ void grouped_body(const KArgs &ka) {
    TileSmem<TA, ACC, FEAT> &sm = *reinterpret_cast<TileSmem<TA, ACC, FEAT> *>(bsc_dyn_smem);
    // a task with a record finds it at its own index (record t belongs to task t)
    for (int32_t t = blockIdx.x; t < ka.ntasks; t += gridDim.x) {
        const int32_t ti = ka.task0 + t;
        const DTask task = ka.tasks[ti];
        if (task.cls == T_NOP) continue;
        if (task.cls == T_TAIL) {
            tail_bundle<TA, TC, ACC>(ka, task, sm.t);
            continue;
        }
        if (task.cls == T_SKINNY_DENSE_M) {
            skinny_dense<TA, TC, ACC, true>(ka, ka.fast[ti], sm.s);
            continue;
        }
        if (task.cls == T_SKINNY_DENSE_N) {
            skinny_dense<TA, TC, ACC, false>(ka, ka.fast[ti], sm.s);
            continue;
        }
        if (task.cls == T_SKINNY_M) {
            skinny_tile<TA, TC, ACC, true>(ka, task, sm.s);
            continue;
        }
        if (task.cls == T_SKINNY_N) {
            skinny_tile<TA, TC, ACC, false>(ka, task, sm.s);
            continue;
        }
        if constexpr ((FEAT & FEAT_FAST_N) != 0) {
            if (task.cls == T_MFMA_FAST_N) {
                direct_tile_bf16<TC, true>(ka, ka.fast[ti], sm.f);
                continue;
            }
        }
        if constexpr ((FEAT & FEAT_FAST_K) != 0) {
            if (task.cls == T_MFMA_FAST_K) {
                direct_tile_bf16<TC, false>(ka, ka.fast[ti], sm.f);
                continue;
            }
        }
        if constexpr ((FEAT & FEAT_WIDE) != 0) {
            if (task.cls == T_MFMA_WIDE_N) {
                wide_tile_bf16<TC, true>(ka, ka.fast[ti], sm.x);
                continue;
            }
            if (task.cls == T_MFMA_WIDE_K) {
                wide_tile_bf16<TC, false>(ka, ka.fast[ti], sm.x);
                continue;
            }
        }
        if constexpr ((FEAT & FEAT_MFMA) != 0) {
            if (is_mfma(task.cls)) {
                if constexpr (std::is_same<TA, uint16_t>::value) {
                    // a direct-to-LDS task run on the general tile (a launch whose operand
                    // bases are not 16-byte aligned) covers its rows and columns in
                    // general tiles; of the K-slices of a split tile, the first computes
                    // the whole tile
                    static_assert(TILE_MFMA_DENSE_M <= 2 * TILE_MFMA && TILE_WIDE <= 2 * TILE_MFMA,
                                  "a dense task fits two by two general tiles");
                    if (task.cls != T_MFMA && ka.fast[ti].nsplit > 1 && ka.fast[ti].split != 0) continue;
                    const bool rec = task.cls != T_MFMA;
                    const int32_t mh = rec && ka.fast[ti].mlen > TILE_MFMA ? 2 : 1;
                    const int32_t nh = rec && ka.fast[ti].nlen > TILE_MFMA ? 2 : 1;
                    for (int32_t a = 0; a < mh; ++a)
                        for (int32_t b = 0; b < nh; ++b) {
                            DTask part = task;
                            part.m0 += a * TILE_MFMA;
                            part.n0 += b * TILE_MFMA;
                            mfma_tile_bf16<TC>(ka, part, sm.m);
                        }
                } else {
                    mfma_tile_f<TA>(ka, task, ka.fast[ti], sm.m);
                }
                continue;
            }
        }
        generic_tile<TA, TC, ACC>(ka, task, sm.g);
    }
}

// A launch whose LDS allows only one workgroup per CU gets the whole register
// file (one wave per SIMD); the others keep two workgroups per CU.
template <typename TA, typename ACC, int32_t FEAT>
constexpr bool one_per_cu() { return sizeof(TileSmem<TA, ACC, FEAT>) > 80 * 1024; }

template <typename TA, typename TC, typename ACC, int32_t FEAT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void grouped_contract(KArgs ka) {
    grouped_body<TA, TC, ACC, FEAT>(ka);
}

template <typename TA, typename TC, typename ACC, int32_t FEAT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void grouped_contract_wide(KArgs ka) {
    grouped_body<TA, TC, ACC, FEAT>(ka);
}

// fp32 launches: the fp32 tile bodies fit in 128 VGPRs and their LDS allows
// four workgroups per CU, so they are compiled for four waves per SIMD (more
// tiles in flight to hide the per-tile chain of dependent loads).
template <typename TA, typename TC, typename ACC, int32_t FEAT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void grouped_contract_narrow(KArgs ka) {
    grouped_body<TA, TC, ACC, FEAT>(ka);
}

// Opt a kernel variant into more than the default dynamic LDS once per process.
template <typename TA, typename TC, typename ACC, int32_t FEAT>
KernelRef kernel_ref() {
    KernelFn fn;
    if constexpr (one_per_cu<TA, ACC, FEAT>()) fn = grouped_contract_wide<TA, TC, ACC, FEAT>;
    else if constexpr (std::is_same<TA, float>::value) fn = grouped_contract_narrow<TA, TC, ACC, FEAT>;
    else fn = grouped_contract<TA, TC, ACC, FEAT>;
    const size_t lds = sizeof(TileSmem<TA, ACC, FEAT>);
    static const hipError_t once = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)once;
    return {fn, lds, 256};
}

}  // namespace bsc
