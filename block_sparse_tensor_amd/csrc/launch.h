// Entry points of the separately compiled kernel variants (grouped_*.hip and
// pack.hip), called by the runtime (runtime.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "bsc_internal.h"
#include "kernels_common.h"
#include "kernels_pack.h"

namespace bsc {

using KernelFn = void (*)(KArgs);

struct KernelRef {
    KernelFn fn;
    size_t lds;         // dynamic LDS bytes of the variant
    unsigned threads;   // workgroup size it is compiled for
};

// Grouped-contraction kernel of a plan dtype holding the tile bodies `feat`
// (FEAT_* bits).  For bf16, FEAT_FAST_N / FEAT_FAST_K must already be folded
// into FEAT_MFMA when an operand base is not 16-byte aligned.
KernelRef grouped_kernel_f64(int32_t feat);
KernelRef grouped_kernel_f32(int32_t feat);
KernelRef grouped_kernel_bf16_lo(int32_t feat);   // feat 0..3
KernelRef grouped_kernel_bf16_hi(int32_t feat);   // feat 4..7
KernelRef grouped_kernel_bf16_wide(int32_t feat); // FEAT_WIDE, with or without FEAT_MFMA
KernelRef grouped_kernel_bf16_wide8();            // a launch of wide tiles only (512 threads)

// Enqueue the gather kernel of a plan dtype.
void launch_pack(bsc_dtype dt, dim3 grid, hipStream_t s, const PArgs &pa);

}  // namespace bsc
