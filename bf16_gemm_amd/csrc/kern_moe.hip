// kern_moe.hip -- the MoE combine around the grouped product: each token's
// output row is the routing-weighted sum of its top-k expert rows.
#include "internal.hpp"

namespace mgemm {

typedef float f32x8_t __attribute__((ext_vector_type(8)));

template <int OUT>
__device__ __forceinline__ float half_to_float(uint32_t h)
{
    if constexpr (OUT == OUT_BF16)
        return __builtin_bit_cast(float, h << 16);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Y[t, 8c .. 8c+7] = sum_k w[t,k] * Z[pos[t,k], 8c .. 8c+7]: one lane per
// 16-byte column chunk, the k terms added in order with fused multiply-adds
// in fp32, one rounding to the 16-bit type (w null: every weight 1, a plain
// sum, for expert outputs that already carry their routing weight).  Z is
// read through a buffer resource that ends after its last row, so a
// position outside [0, z_rows) reads zeros and contributes nothing.
template <int OUT>
__global__ void __launch_bounds__(256) moe_combine_kernel(const uint16_t *Z, int64_t z_rows, int64_t ldz,
                                                          const int32_t *pos, const float *w, char *Y, int64_t ldy,
                                                          int top_k, int H8)
{
    const int64_t t = blockIdx.x;
    const uint64_t zbytes = (uint64_t)z_rows * (uint64_t)ldz * 2u;
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(Z, zbytes);
    const int32_t *pt = pos + t * top_k;
    for (int c = blockIdx.y * 256 + (int)threadIdx.x; c < H8; c += gridDim.y * 256) {
        f32x8_t acc = {};
        for (int k = 0; k < top_k; ++k) {
            const int p = pt[k];
            const float wk = w ? w[t * top_k + k] : 1.0f;
            const uint64_t row_off = (uint64_t)(int64_t)p * (uint64_t)ldz * 2u + (uint64_t)c * 16u;
            const uint32_t off = (p >= 0 && (int64_t)p < z_rows && row_off < zbytes) ? (uint32_t)row_off : kOOB;
            const u32x4_t v = bload16(rz, off);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __builtin_fmaf(wk, half_to_float<OUT>(v[q] & 0xFFFFu), acc[2 * q]);
                acc[2 * q + 1] = __builtin_fmaf(wk, half_to_float<OUT>(v[q] >> 16), acc[2 * q + 1]);
            }
        }
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = OUT == OUT_BF16 ? pack2_bf16(acc[2 * q], acc[2 * q + 1]) : pack2_f16(acc[2 * q], acc[2 * q + 1]);
        *(u32x4_t *)(Y + (t * ldy + (int64_t)c * 8) * 2) = o;
    }
}

hipError_t launch_moe_combine(const void *Z, int64_t z_rows, int64_t ldz, const int32_t *pos, const float *w,
                              void *Y, int64_t ldy, int64_t T, int top_k, int64_t H, int out, hipStream_t s)
{
    const int H8 = (int)(H / 8);
    const int gy = (H8 + 255) / 256;
    const dim3 grid((unsigned)T, (unsigned)(gy < 1 ? 1 : gy));
    if (out == OUT_BF16)
        hipLaunchKernelGGL(moe_combine_kernel<OUT_BF16>, grid, dim3(256), 0, s, (const uint16_t *)Z, z_rows, ldz, pos,
                           w, (char *)Y, ldy, top_k, H8);
    else
        hipLaunchKernelGGL(moe_combine_kernel<OUT_F16>, grid, dim3(256), 0, s, (const uint16_t *)Z, z_rows, ldz, pos,
                           w, (char *)Y, ldy, top_k, H8);
    return hipGetLastError();
}

}  // namespace mgemm
