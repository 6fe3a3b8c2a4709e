// kern_quant.hip -- blockwise FP8 quantisation of a 16-bit matrix: E4M3
// codes plus one E8M0 scale per 128 consecutive columns of a row, the
// activation layout the block-scaled products read.
#include "internal.hpp"

namespace mgemm {

// Nearest E4M3 code to a finite y with |y| <= 448, ties to the even code:
// below 2^-6 the subnormal grid of step 2^-9; above, three fraction bits at
// y's binade (a rounding up to 16 carries into the exponent field).  All
// steps are power-of-two scalings and one round-to-nearest-even.
__device__ __forceinline__ uint32_t e4m3_nearest(float y)
{
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = __builtin_fabsf(y);
    if (a < 0x1p-6f)
        return sign | (uint32_t)__builtin_rintf(a * 0x1p9f);
    int k;
    __builtin_frexpf(a, &k);
    const int e = k - 1;                                        // floor(log2 a), -6 .. 8
    const uint32_t q = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));   // 8 .. 16
    return sign | ((((uint32_t)(e + 7)) << 3) + q - 8u);
}

// One wave per (row, block of 128 columns); lane l holds columns 2l, 2l + 1
// of the block.  Scale: the smallest power of two 2^E with amax <= 448 * 2^E
// (amax = m 2^k, m in [0.5, 1): E = k - 9, or k - 8 when m > 0.875), E in
// [-127, 127]; 2^0 for an all-zero block; a block holding a non-finite value
// gets the NaN scale byte and NaN codes.
template <int IN>
__global__ void __launch_bounds__(256) quantize_e4m3_block_kernel(const uint16_t *X, int64_t rows, int64_t cols,
                                                                  int64_t ldx, uint8_t *Q, int64_t ldq, uint8_t *S,
                                                                  int64_t lds, int64_t nblk)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= rows * nblk)
        return;                                   // the whole wave leaves together
    const int64_t r = w / nblk, b = w - r * nblk;
    const int64_t c = b * 128 + 2 * lane;
    const bool in = c < cols;                     // cols is even: c + 1 < cols too
    float v0 = 0.0f, v1 = 0.0f;
    if (in) {
        const uint32_t u = *(const uint32_t *)(X + r * ldx + c);
        if constexpr (IN == IN_BF16) {
            v0 = __uint_as_float(u << 16);
            v1 = __uint_as_float(u & 0xFFFF0000u);
        } else {
            v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
            v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
        }
    }
    const bool bad = !__builtin_isfinite(v0) || !__builtin_isfinite(v1);
    const bool any_bad = __ballot(bad) != 0;
    float m = __builtin_fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        m = __builtin_fmaxf(m, __shfl_xor(m, o));
    int E = 0;
    if (m > 0.0f) {
        int k;
        const float mant = __builtin_frexpf(m, &k);
        E = k - 9 + (mant > 0.875f ? 1 : 0);
        E = E < -127 ? -127 : (E > 127 ? 127 : E);
    }
    uint32_t q0 = 0x7Fu, q1 = 0x7Fu;
    if (!any_bad) {
        q0 = e4m3_nearest(__builtin_ldexpf(v0, -E));
        q1 = e4m3_nearest(__builtin_ldexpf(v1, -E));
    }
    if (in)
        *(uint16_t *)(Q + r * ldq + c) = (uint16_t)(q0 | (q1 << 8));
    if (lane == 0)
        S[r * lds + b] = (uint8_t)(any_bad ? 255 : E + 127);
}

// The same quantisation with 16-byte loads, for cols, ldx a multiple of 8,
// X 16-byte and Q rows 8-byte aligned: lane l of a wave holds 8 consecutive
// columns, 16 lanes one block, a wave 4 consecutive blocks of one row (a
// 512-column chunk), the block maximum within each 16-lane group.  Each wave
// takes NCH consecutive chunks and issues all their loads before it
// quantises the first.
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
constexpr int kQuantChunks = 4;
template <int IN>
__global__ void __launch_bounds__(256) quantize_e4m3_block_wide_kernel(const uint16_t *X, int64_t rows, int64_t cols,
                                                                       int64_t ldx, uint8_t *Q, int64_t ldq,
                                                                       uint8_t *S, int64_t lds, int64_t chunks)
{
    constexpr int NCH = kQuantChunks;
    const int lane = threadIdx.x & 63;
    const int64_t total = rows * chunks;
    const int64_t w0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * NCH;
    if (w0 >= total)
        return;                                   // the whole wave leaves together
    u32x4_t raw[NCH];
    int64_t row[NCH], col[NCH];
    bool in[NCH];
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
        const int64_t w = w0 + h;
        row[h] = w / chunks;
        col[h] = ((w - row[h] * chunks) * 64 + lane) * 8;     // cols % 8 == 0: all 8 columns in or out
        in[h] = w < total && col[h] < cols;
        raw[h] = in[h] ? *(const u32x4_t *)(X + row[h] * ldx + col[h]) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (IN == IN_BF16) {
                v[2 * q] = __uint_as_float(raw[h][q] << 16);
                v[2 * q + 1] = __uint_as_float(raw[h][q] & 0xFFFF0000u);
            } else {
                v[2 * q] = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[h][q] & 0xFFFFu));
                v[2 * q + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[h][q] >> 16));
            }
        }
        bool bad = false;
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bad = bad || !__builtin_isfinite(v[i]);
            m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1)
            m = __builtin_fmaxf(m, __shfl_xor(m, o));
        const bool any_bad = ((__ballot(bad) >> (lane & 48)) & 0xFFFFull) != 0;   // this lane's 16-lane group
        int E = 0;
        if (m > 0.0f) {
            int k;
            const float mant = __builtin_frexpf(m, &k);
            E = k - 9 + (mant > 0.875f ? 1 : 0);
            E = E < -127 ? -127 : (E > 127 ? 127 : E);
        }
        u32x2v_t out = {0x7F7F7F7Fu, 0x7F7F7F7Fu};
        if (!any_bad) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                uint32_t word = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    word |= e4m3_nearest(__builtin_ldexpf(v[4 * g + i], -E)) << (8 * i);
                out[g] = word;
            }
        }
        if (in[h]) {
            *(u32x2v_t *)(Q + row[h] * ldq + col[h]) = out;
            if ((lane & 15) == 0)
                S[row[h] * lds + col[h] / 128] = (uint8_t)(any_bad ? 255 : E + 127);
        }
    }
}

hipError_t launch_quantize_e4m3_block(const void *X, int64_t rows, int64_t cols, int64_t ldx, int in, uint8_t *Q,
                                      int64_t ldq, uint8_t *S, int64_t lds, hipStream_t s)
{
    if (cols % 8 == 0 && ldx % 8 == 0 && ldq % 8 == 0 && ((uintptr_t)X & 15) == 0 && ((uintptr_t)Q & 7) == 0) {
        const int64_t chunks = (cols + 511) / 512;
        const unsigned grid = (unsigned)((rows * chunks + 4 * kQuantChunks - 1) / (4 * kQuantChunks));
        if (in == IN_BF16)
            hipLaunchKernelGGL(quantize_e4m3_block_wide_kernel<IN_BF16>, dim3(grid), dim3(256), 0, s,
                               (const uint16_t *)X, rows, cols, ldx, Q, ldq, S, lds, chunks);
        else
            hipLaunchKernelGGL(quantize_e4m3_block_wide_kernel<IN_F16>, dim3(grid), dim3(256), 0, s,
                               (const uint16_t *)X, rows, cols, ldx, Q, ldq, S, lds, chunks);
        return hipGetLastError();
    }
    const int64_t nblk = (cols + 127) / 128;
    const int64_t waves = rows * nblk;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    if (in == IN_BF16)
        hipLaunchKernelGGL(quantize_e4m3_block_kernel<IN_BF16>, dim3(grid), dim3(256), 0, s, (const uint16_t *)X,
                           rows, cols, ldx, Q, ldq, S, lds, nblk);
    else
        hipLaunchKernelGGL(quantize_e4m3_block_kernel<IN_F16>, dim3(grid), dim3(256), 0, s, (const uint16_t *)X,
                           rows, cols, ldx, Q, ldq, S, lds, nblk);
    return hipGetLastError();
}

}  // namespace mgemm
