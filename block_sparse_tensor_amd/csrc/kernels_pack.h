// Gather kernel: copies the operands the planner chose to pack into the
// contiguous workspace, all groups in one launch (uni20 "block coalescing",
// section "Interleaved vs contiguous — the real tradeoff is a copy": one pack
// kernel is far cheaper than one launch per sector GEMM).
//
// A task moves one tr x tc piece of one gather (rows along the group's free
// axis, columns along k; pack_tile picks the shape from the gather's width).
// When the source and the destination have the same unit-stride axis the piece
// is copied straight, element i of a wave's sweep to element i, both sides
// coalesced.  Otherwise it passes through LDS: read along the source's unit
// axis, written along the destination's.  The copy is HBM-bound: its roofline
// is 2 * bytes / 8 TB/s.
#pragma once

#include "kernels_common.h"

namespace bsc {

struct PArgs {
    const DPack *packs;
    const DTask *tasks;
    int32_t ntasks, pad;
    const void *A, *B;
    void *W;
};

// source element (x, y) of a gather
__device__ __forceinline__ int64_t pack_src(const DPack &d, int32_t x, int32_t y) {
    const int64_t ax = d.ia == 1 ? static_cast<int64_t>(x) * d.sa0
                                 : static_cast<int64_t>(x / d.ia) * d.sa0 + static_cast<int64_t>(x % d.ia) * d.sa1;
    const int64_t by = d.ib == 1 ? static_cast<int64_t>(y) * d.sb0
                                 : static_cast<int64_t>(y / d.ib) * d.sb0 + static_cast<int64_t>(y % d.ib) * d.sb1;
    return d.off + ax + by;
}

__device__ __forceinline__ int64_t pack_dst(const DPack &d, int32_t x, int32_t y) {
    return d.dmode == 0 ? d.dst + static_cast<int64_t>(x) * d.ld + y : d.dst + static_cast<int64_t>(y) * d.ld + x;
}

template <typename T>
__global__ __launch_bounds__(256) void pack_gather(PArgs pa) {
    __shared__ T lds[PACK_LDS_ELEMS];
    const int32_t tid = threadIdx.x;
    T *W = static_cast<T *>(pa.W);
    for (int32_t t = blockIdx.x; t < pa.ntasks; t += gridDim.x) {
        const DTask task = pa.tasks[t];
        const DPack d = pa.packs[task.group];
        const T *S = static_cast<const T *>(d.src == 0 ? pa.A : pa.B);
        int32_t tr = 0, tc = 0;
        const int32_t mode = pack_mode(d);
        constexpr int32_t ESZ = static_cast<int32_t>(sizeof(T));
        pack_tile(d.rows, d.cols, mode, pack_big(ESZ, mode), tr, tc);
        const int32_t x0 = task.m0, y0 = task.n0;
        const int32_t rows = min(tr, d.rows - x0), cols = min(tc, d.cols - y0);
        const int32_t n = rows * cols;
        // unit-stride axes: of the source view, and of the destination
        const bool s_k = d.ib == 1 && (d.sb0 == 1 || d.cols == 1);
        const bool s_f = d.ia == 1 && (d.sa0 == 1 || d.rows == 1);
        const bool d_k = d.dmode == 0;
        if constexpr (ESZ == 2) {
            if (pack_big(ESZ, mode)) {
                // a large bf16 piece: straight along the unit axis, PACK_BATCH
                // 16-byte vectors per lane loaded before any is stored, a
                // line's last partial vector element by element
                constexpr int32_t V = 8;
                constexpr int32_t PACK_BATCH = 4;
                const int32_t len = d_k ? cols : rows;     // extent along the unit axis
                const int32_t nv = (len + V - 1) / V;      // vectors per line
                const int32_t units = (d_k ? rows : cols) * nv;
                for (int32_t e0 = tid; e0 < units; e0 += 256 * PACK_BATCH) {
                    const T *sp[PACK_BATCH];
                    T *dp[PACK_BATCH];
                    int32_t left[PACK_BATCH];   // elements of the vector inside the line (0: past the piece)
                    uint4 v[PACK_BATCH];
#pragma unroll
                    for (int32_t b = 0; b < PACK_BATCH; ++b) {
                        const int32_t e = e0 + 256 * b;
                        left[b] = 0;
                        sp[b] = S;
                        dp[b] = W;
                        if (e < units) {
                            const int32_t line = e / nv, u = (e - line * nv) * V;
                            const int32_t x = d_k ? line : u, y = d_k ? u : line;
                            sp[b] = S + pack_src(d, x0 + x, y0 + y);
                            dp[b] = W + pack_dst(d, x0 + x, y0 + y);
                            left[b] = min(V, len - u);
                        }
                        if (left[b] == V) {
                            // (through a scalar temporary: a copy into the array
                            // element kept the whole array in private memory)
                            uint4 t;
                            __builtin_memcpy(&t, sp[b], sizeof(t));
                            v[b] = t;
                        }
                    }
#pragma unroll
                    for (int32_t b = 0; b < PACK_BATCH; ++b) {
                        if (left[b] == V) {
                            const uint4 t = v[b];
                            __builtin_memcpy(dp[b], &t, sizeof(t));
                        } else {
                            for (int32_t j = 0; j < left[b]; ++j) dp[b][j] = sp[b][j];
                        }
                    }
                }
                continue;
            }
        }
        if ((d_k && s_k) || (!d_k && s_f)) {
            // same unit axis on both sides: straight copy along it, 16 bytes
            // per lane (any element address: the code object runs in
            // unaligned-access mode), the line's last partial vector element
            // by element
            constexpr int32_t V = 16 / static_cast<int32_t>(sizeof(T));
            const int32_t len = d_k ? cols : rows;     // extent along the unit axis
            const int32_t nv = (len + V - 1) / V;      // vectors per line
            const int32_t units = (d_k ? rows : cols) * nv;
            for (int32_t e = tid; e < units; e += 256) {
                const int32_t line = e / nv, u = (e - line * nv) * V;
                const int32_t x = d_k ? line : u, y = d_k ? u : line;
                const T *sp = S + pack_src(d, x0 + x, y0 + y);
                T *dp = W + pack_dst(d, x0 + x, y0 + y);
                if (u + V <= len) {
                    uint4 v;
                    __builtin_memcpy(&v, sp, sizeof(v));
                    __builtin_memcpy(dp, &v, sizeof(v));
                } else {
                    for (int32_t j = 0; u + j < len; ++j) dp[j] = sp[j];
                }
            }
            continue;
        }
        // through LDS: [x][y] with pitch cols + 1
        const bool read_k = s_k || !s_f;
        __syncthreads();   // the previous task's LDS reads are done
        for (int32_t e = tid; e < n; e += 256) {
            const int32_t x = read_k ? e / cols : e % rows;
            const int32_t y = read_k ? e % cols : e / rows;
            lds[x * (cols + 1) + y] = S[pack_src(d, x0 + x, y0 + y)];
        }
        __syncthreads();
        for (int32_t e = tid; e < n; e += 256) {
            const int32_t x = d_k ? e / cols : e % rows;
            const int32_t y = d_k ? e % cols : e / rows;
            W[pack_dst(d, x0 + x, y0 + y)] = lds[x * (cols + 1) + y];
        }
    }
}

}  // namespace bsc
