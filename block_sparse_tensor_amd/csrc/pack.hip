// The gather (pack) kernel launches, one instantiation per operand type.
#include <hip/hip_runtime.h>

#include "kernels_pack.h"
#include "launch.h"

namespace bsc {

void launch_pack(bsc_dtype dt, dim3 grid, hipStream_t s, const PArgs &pa) {
    const dim3 block(256);
    switch (dt) {
        case BSC_F64: hipLaunchKernelGGL(pack_gather<double>, grid, block, 0, s, pa); break;
        case BSC_F32: hipLaunchKernelGGL(pack_gather<float>, grid, block, 0, s, pa); break;
        case BSC_BF16_F32: hipLaunchKernelGGL(pack_gather<uint16_t>, grid, block, 0, s, pa); break;
    }
}

}  // namespace bsc
