// kern_moe_fused.hip -- launches of the fused two-GEMM MoE expert layer.
#include "internal.hpp"
#include "moe_fused.hpp"

namespace mgemm {

hipError_t launch_moe_fused(const MoeArgs &a, int in, int grid, hipStream_t s)
{
    hipLaunchKernelGGL(moe_prepare_kernel, dim3(1), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError())
        return e;
    const bool w = a.row_weight != nullptr;
    if (in == IN_BF16) {
        if (w)
            hipLaunchKernelGGL((moe_fused_kernel<IN_BF16, true>), dim3(grid), dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((moe_fused_kernel<IN_BF16, false>), dim3(grid), dim3(512), 0, s, a);
    } else {
        if (w)
            hipLaunchKernelGGL((moe_fused_kernel<IN_F16, true>), dim3(grid), dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((moe_fused_kernel<IN_F16, false>), dim3(grid), dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mgemm
