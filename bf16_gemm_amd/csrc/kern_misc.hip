// kern_misc.hip -- the zero-fill and edge-column kernels.
#include "internal.hpp"

namespace mgemm {

// D[rows x cols] = 0 (the empty sum, K == 0).
__global__ void zero_fill_kernel(char *D, int rows, int cols, int64_t ld_bytes, int esize)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)rows * cols;
    for (; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / cols, c = i % cols;
        char *p = D + r * ld_bytes + c * esize;
        if (esize == 4)
            *(float *)p = 0.0f;
        else
            *(uint16_t *)p = 0;
    }
}


template <int IN, int OUT>
static hipError_t launch_edge(const DenseArgs &a, int a_kmajor, int b_kmajor, int n_first, hipStream_t s)
{
    const int64_t items = (int64_t)a.M * (a.N - n_first);
    const int64_t blocks = (items + 3) / 4;  // one wave per output element
    hipLaunchKernelGGL((edge_cols_kernel<IN, OUT>), dim3((unsigned)blocks), dim3(256), 0, s, a, a_kmajor, b_kmajor,
                       n_first);
    return hipGetLastError();
}

EdgeFn edge_fn(int in, int out)
{
    if (in == IN_BF16)
        return out == OUT_F32 ? launch_edge<IN_BF16, OUT_F32> : out == OUT_BF16 ? launch_edge<IN_BF16, OUT_BF16> : nullptr;
    return out == OUT_F32 ? launch_edge<IN_F16, OUT_F32> : out == OUT_F16 ? launch_edge<IN_F16, OUT_F16> : nullptr;
}

hipError_t launch_zero_fill(void *D, int rows, int cols, int64_t ld_bytes, int esize, hipStream_t s)
{
    const int64_t total = (int64_t)rows * cols;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (char *)D, rows, cols, ld_bytes, esize);
    return hipGetLastError();
}

}  // namespace mgemm
