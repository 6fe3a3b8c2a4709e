// kern_misc.hip -- the zero-fill, split-reduction and edge-column kernels.
#include "internal.hpp"

namespace mgemm {

typedef float float4_t __attribute__((ext_vector_type(4)));

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


// D[r, c..c+3] = sum over splits of W[s][r, c..c+3], one thread per four
// columns: 16-byte loads of each range in increasing order, one rounding.
template <int OUT>
__global__ void __launch_bounds__(256) reduce_splits_kernel(const float *W, char *D, int M, int N4, int ldw,
                                                            int64_t split_stride, int splits, int64_t ldd)
{
    const int64_t total = (int64_t)M * N4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / N4;
        const int c = (int)(i - r * N4) * 4;
        const float *src = W + r * ldw + c;
        float4_t acc = *(const float4_t *)src;
        for (int s = 1; s < splits; ++s) {
            const float4_t v = *(const float4_t *)(src + s * split_stride);
            acc[0] += v[0];
            acc[1] += v[1];
            acc[2] += v[2];
            acc[3] += v[3];
        }
        if constexpr (OUT == OUT_F32) {
            *(float4_t *)(D + (r * ldd + c) * 4) = acc;
        } else {
            const uint32_t lo = OUT == OUT_BF16 ? pack2_bf16(acc[0], acc[1]) : pack2_f16(acc[0], acc[1]);
            const uint32_t hi = OUT == OUT_BF16 ? pack2_bf16(acc[2], acc[3]) : pack2_f16(acc[2], acc[3]);
            *(u32x2_t *)(D + (r * ldd + c) * 2) = u32x2_t{lo, hi};
        }
    }
}

hipError_t launch_reduce_splits(const float *W, void *D, int M, int N, int ldw, int64_t split_stride, int splits,
                                int64_t ldd, int out, hipStream_t s)
{
    const int N4 = N / 4;
    const int64_t total = (int64_t)M * N4;
    int64_t blocks = (total + 255) / 256;
    blocks = blocks < 1 ? 1 : (blocks > 8192 ? 8192 : blocks);
    if (out == OUT_F32)
        hipLaunchKernelGGL(reduce_splits_kernel<OUT_F32>, dim3((unsigned)blocks), dim3(256), 0, s, W, (char *)D, M, N4,
                           ldw, split_stride, splits, ldd);
    else if (out == OUT_BF16)
        hipLaunchKernelGGL(reduce_splits_kernel<OUT_BF16>, dim3((unsigned)blocks), dim3(256), 0, s, W, (char *)D, M,
                           N4, ldw, split_stride, splits, ldd);
    else
        hipLaunchKernelGGL(reduce_splits_kernel<OUT_F16>, dim3((unsigned)blocks), dim3(256), 0, s, W, (char *)D, M, N4,
                           ldw, split_stride, splits, ldd);
    return hipGetLastError();
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
