// Gather kernel: copies the operands the planner chose to pack into the
// contiguous workspace, all groups in one launch (uni20 "block coalescing",
// section "Interleaved vs contiguous — the real tradeoff is a copy": one pack
// kernel is far cheaper than one launch per sector GEMM).
//
// A task moves a 64 x 64 piece of one gather (rows along the group's free axis,
// columns along k).  The destination is always k-contiguous, so the writes run
// along k.  The reads follow the source's own unit-stride axis: a
// k-contiguous source is read along k, a free-axis-contiguous source along the
// rows; the piece passes through LDS so both sides stay coalesced.  The copy
// is HBM-bound: its roofline is 2 * bytes / 8 TB/s.
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

template <typename T>
struct PackSmem {
    T t[TILE_PACK][TILE_PACK + 1];   // [row][k]; odd pitch keeps both access orders on distinct banks
};

// source element (x, y) of a gather
__device__ __forceinline__ int64_t pack_src(const DPack &d, int32_t x, int32_t y) {
    const int64_t ax = d.ia == 1 ? static_cast<int64_t>(x) * d.sa0
                                 : static_cast<int64_t>(x / d.ia) * d.sa0 + static_cast<int64_t>(x % d.ia) * d.sa1;
    const int64_t by = d.ib == 1 ? static_cast<int64_t>(y) * d.sb0
                                 : static_cast<int64_t>(y / d.ib) * d.sb0 + static_cast<int64_t>(y % d.ib) * d.sb1;
    return d.off + ax + by;
}

template <typename T>
__global__ __launch_bounds__(256) void pack_gather(PArgs pa) {
    __shared__ PackSmem<T> sm;
    const int32_t tid = threadIdx.x;
    T *W = static_cast<T *>(pa.W);
    for (int32_t t = blockIdx.x; t < pa.ntasks; t += gridDim.x) {
        const DTask task = pa.tasks[t];
        const DPack d = pa.packs[task.group];
        const T *S = static_cast<const T *>(d.src == 0 ? pa.A : pa.B);
        const int32_t x0 = task.m0, y0 = task.n0;
        const int32_t rows = min(TILE_PACK, d.rows - x0), cols = min(TILE_PACK, d.cols - y0);
        // a k-contiguous source (single k leg, unit stride) is read along k
        const bool along_k = d.ib == 1 && (d.sb0 == 1 || d.cols == 1);
        __syncthreads();   // the previous task's reads of the LDS piece are done
#pragma unroll 4
        for (int32_t i = 0; i < TILE_PACK * TILE_PACK / 256; ++i) {
            const int32_t e = tid + 256 * i;
            const int32_t x = along_k ? e / TILE_PACK : e % TILE_PACK;
            const int32_t y = along_k ? e % TILE_PACK : e / TILE_PACK;
            if (x < rows && y < cols) sm.t[x][y] = S[pack_src(d, x0 + x, y0 + y)];
        }
        __syncthreads();
#pragma unroll 4
        for (int32_t i = 0; i < TILE_PACK * TILE_PACK / 256; ++i) {
            const int32_t e = tid + 256 * i;
            const int32_t x = e / TILE_PACK, y = e % TILE_PACK;
            if (x < rows && y < cols)
                W[d.dst + static_cast<int64_t>(x0 + x) * d.ld + (y0 + y)] = sm.t[x][y];
        }
    }
}

}  // namespace bsc
