/*
 * oracle.c -- plain CPU reference for the dense and grouped FP16/BF16 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests/, the smoke check and the bench's
 * CPU-baseline leg can compare the HIP library against an obviously correct
 * definition.  It shares no code, header, table or constant with the
 * library under bf16_gemm_amd/.
 *
 * What it computes (definitions restated from the pages, not their code):
 *
 *  - The GEMM itself.  "B200 的 2CTA 怎样调优" (section 七, the logical sketch
 *    under "MMA 算结果，累加缓冲存结果，epilogue 处理结果") defines one output
 *    element as an accumulator that starts at zero, adds A[i,k]*B[k,j] for
 *    every k along K, and only then hands the finished sum to an epilogue
 *    that converts it to the output type.  Here the accumulator is an IEEE
 *    double and k runs in ascending order; every product of two fp16/bf16
 *    numbers is exact in double, so the only rounding is in the additions.
 *
 *  - The output conversion.  The same sketch converts the finished sum to
 *    the output type without naming a rounding rule; this oracle reads that
 *    as IEEE round-to-nearest, ties-to-even, applied once, directly from the
 *    double sum.
 *
 *  - The SiLU gate.  The same page (section 七, "Gate／SwiGLU") defines the
 *    gated output as up x SiLU(gate); SiLU(x) = x / (1 + exp(-x)).  The pair
 *    (gate, up) is taken from one GEMM whose output columns interleave them
 *    in blocks of eight, gate first ("MegaMoE：Blackwell 与 Hopper 的融合算子
 *    解读", Hopper part, section 10 on the eight-channel interleave).
 *
 * Decoding of the 16-bit input formats and the round-to-nearest-even
 * encoders are written out here from the IEEE-754 binary16 layout and the
 * bfloat16 layout (the upper half of a binary32), so the oracle does not
 * depend on any library conversion.
 *
 * Plain means plain: no blocking, no intrinsics, no reordering of the sum.
 * Rows are split across OpenMP threads; each output element is still one
 * sequential ascending-k sum.  Build without fast-math and with
 * -ffp-contract=off so that no fused multiply-add changes a rounding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes used by this file's entry points */
enum { OR_F16 = 1, OR_BF16 = 2, OR_F32 = 3, OR_F64 = 4 };
/* operand storage: row-major (last index contiguous) or column-major */
enum { OR_ROW = 0, OR_COL = 1 };

/* ------------------------------------------------------------------ */
/* 16-bit decoders                                                     */
/* ------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^(1-15-10) */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double oracle_bf16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133); /* subnormal: f * 2^(1-127-7) */
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134); /* (1.f) * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* ------------------------------------------------------------------ */
/* round-to-nearest-even encoders                                      */
/* ------------------------------------------------------------------ */

/* Round a non-negative double that is an exact multiple of 2^-1 or finer
 * to the nearest integer, ties to the even integer. */
static double rne_integer(double v)
{
    double fl = floor(v);
    double rem = v - fl; /* exact: v and fl are close doubles */
    if (rem > 0.5)
        return fl + 1.0;
    if (rem < 0.5)
        return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Generic IEEE-style encoder for a format with `prec` significant bits
 * (implicit bit included), exponent bias `bias`, exponent field width
 * `ebits`.  Returns the bit pattern.  RNE, overflow to infinity, gradual
 * underflow. */
static uint32_t encode_rne(double x, int prec, int bias, int ebits)
{
    uint32_t sign = 0;
    uint32_t emax_field = (1u << ebits) - 1u;
    uint32_t total_bits = (uint32_t)(prec - 1) + (uint32_t)ebits; /* w/o sign */
    uint32_t inf_bits = emax_field << (prec - 1);
    if (isnan(x))
        return inf_bits | (1u << (prec - 2)); /* quiet NaN */
    if (signbit(x)) {
        sign = 1u << total_bits;
        x = -x;
    }
    if (isinf(x))
        return sign | inf_bits;
    if (x == 0.0)
        return sign;
    int emin = 1 - bias; /* exponent of the smallest normal */
    int ex;
    frexp(x, &ex);   /* x = m * 2^ex, 0.5 <= m < 1 */
    int e = ex - 1;  /* 2^e <= x < 2^(e+1) */
    if (e < emin)
        e = emin;    /* subnormal range shares the smallest normal's quantum */
    /* quantum of the format at exponent e */
    double q = rne_integer(ldexp(x, (prec - 1) - e)); /* significand, as integer */
    /* q in [2^(prec-1), 2^prec] for normals, [0, 2^(prec-1)] for subnormals
     * (where e was clamped to emin, whose biased exponent is 1).  The
     * encoding (biased exponent << (prec-1)) + (q - 2^(prec-1)) is then
     * continuous across the normal/subnormal boundary and across the carry
     * when q rounds up to 2^prec. */
    int64_t bits = ((int64_t)(e + bias) << (prec - 1)) + ((int64_t)q - ((int64_t)1 << (prec - 1)));
    if (bits >= (int64_t)inf_bits)
        bits = inf_bits; /* overflow rounds to infinity */
    return sign | (uint32_t)bits;
}

uint16_t oracle_double_to_bf16(double x) { return (uint16_t)encode_rne(x, 8, 127, 8); }
uint16_t oracle_double_to_f16(double x) { return (uint16_t)encode_rne(x, 11, 15, 5); }
uint32_t oracle_double_to_f32_bits(double x) { return encode_rne(x, 24, 127, 8); }

/* ------------------------------------------------------------------ */
/* array helpers                                                       */
/* ------------------------------------------------------------------ */

/* Decode n 16-bit values of dtype `t` into doubles. */
void oracle_decode(int t, const uint16_t *src, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = (t == OR_F16) ? oracle_f16_to_double(src[i]) : oracle_bf16_to_double(src[i]);
}

/* Round n doubles to dtype `t` (F16/BF16 -> uint16 bits, F32 -> uint32 bits). */
void oracle_encode(int t, const double *src, int64_t n, void *dst)
{
    if (t == OR_F32) {
        uint32_t *o = (uint32_t *)dst;
        for (int64_t i = 0; i < n; ++i)
            o[i] = oracle_double_to_f32_bits(src[i]);
    } else if (t == OR_F64) {
        memcpy(dst, src, (size_t)n * sizeof(double));
    } else {
        uint16_t *o = (uint16_t *)dst;
        for (int64_t i = 0; i < n; ++i)
            o[i] = (t == OR_BF16) ? oracle_double_to_bf16(src[i]) : oracle_double_to_f16(src[i]);
    }
}

/* element (r, c) of a logical rows x cols matrix stored with leading
 * dimension ld in the given layout */
static int64_t at(int layout, int64_t r, int64_t c, int64_t ld)
{
    return layout == OR_ROW ? r * ld + c : c * ld + r;
}

/* ------------------------------------------------------------------ */
/* the GEMM                                                            */
/* ------------------------------------------------------------------ */

/*
 * ref[i*N + j] = sum_{k=0}^{K-1} A(i,k) * B(k,j), in double, ascending k.
 * A is logically M x K, B is logically K x N; each is decoded exactly from
 * its 16-bit storage first.  ref is M x N row-major.
 * Returns 0 on success, -1 if a temporary cannot be allocated.
 */
int oracle_gemm_ref(int64_t M, int64_t N, int64_t K,
                    int a_type, int a_layout, const uint16_t *A, int64_t lda,
                    int b_type, int b_layout, const uint16_t *B, int64_t ldb,
                    double *ref)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (!a || !b) {
        free(a);
        free(b);
        return -1;
    }
    /* a: M x K row-major doubles; b: K x N row-major doubles */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) {
            uint16_t v = A[at(a_layout, i, k, lda)];
            a[i * K + k] = a_type == OR_F16 ? oracle_f16_to_double(v) : oracle_bf16_to_double(v);
        }
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            uint16_t v = B[at(b_layout, k, j, ldb)];
            b[k * N + j] = b_type == OR_F16 ? oracle_f16_to_double(v) : oracle_bf16_to_double(v);
        }
    /* i-k-j order: every ref[i][j] still receives its terms in ascending k,
     * one addition at a time, so each element's sum is the plain sequential
     * sum of the definition. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double *row = ref + i * N;
        for (int64_t j = 0; j < N; ++j)
            row[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double aik = a[i * K + k];
            const double *brow = b + k * N;
            for (int64_t j = 0; j < N; ++j)
                row[j] += aik * brow[j];
        }
    }
    free(a);
    free(b);
    return 0;
}

/*
 * The same sum for a list of individual elements (rows[t], cols[t]),
 * decoding operands on the fly.  Used where the full product is too large
 * for the CPU: each requested element is still the plain ascending-k sum.
 */
void oracle_gemm_ref_sampled(int64_t K,
                             int a_type, int a_layout, const uint16_t *A, int64_t lda,
                             int b_type, int b_layout, const uint16_t *B, int64_t ldb,
                             const int64_t *rows, const int64_t *cols, int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = rows[t], j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            uint16_t av = A[at(a_layout, i, k, lda)];
            uint16_t bv = B[at(b_layout, k, j, ldb)];
            double x = a_type == OR_F16 ? oracle_f16_to_double(av) : oracle_bf16_to_double(av);
            double y = b_type == OR_F16 ? oracle_f16_to_double(bv) : oracle_bf16_to_double(bv);
            s += x * y;
        }
        out[t] = s;
    }
}

/* ------------------------------------------------------------------ */
/* SiLU gate                                                           */
/* ------------------------------------------------------------------ */

double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/*
 * h[r, c] = SiLU(gate) * up for c in [0, N/2), where the GEMM output G
 * (rows x N, row-major, unrounded doubles) interleaves gate and up in blocks
 * of `il` columns, gate first: columns [2*il*b, 2*il*b + il) are gate for
 * h columns [il*b, il*b + il) and the next il columns are the matching up.
 */
void oracle_silu_gate(int64_t rows, int64_t N, int64_t il, const double *G, double *h)
{
    int64_t half = N / 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < half; ++c) {
            int64_t blk = c / il, w = c % il;
            double g = G[r * N + 2 * il * blk + w];
            double u = G[r * N + 2 * il * blk + il + w];
            h[r * half + c] = oracle_silu(g) * u;
        }
}

/*
 * The same with one weight per row multiplied into that row's outputs, after
 * SwiGLU and before any rounding (the FC1 epilogue's optional routing weight:
 * "MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 09):
 * h[r, c] = SiLU(gate) * up * w[r].
 */
void oracle_silu_gate_weighted(int64_t rows, int64_t N, int64_t il, const double *G, const double *w, double *h)
{
    int64_t half = N / 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < half; ++c) {
            int64_t blk = c / il, j = c % il;
            double g = G[r * N + 2 * il * blk + j];
            double u = G[r * N + 2 * il * blk + il + j];
            h[r * half + c] = oracle_silu(g) * u * w[r];
        }
}

/* Number of OpenMP threads a parallel region of this library would use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n =
#ifdef _OPENMP
            omp_get_num_threads();
#else
            1;
#endif
    }
    return n;
}

/* ------------------------------------------------------------------ */
/* FP8 (E4M3) GEMM with per-tensor scales                              */
/* ------------------------------------------------------------------ */

/*
 * The 8-bit input format, written out from the OCP 8-bit floating point
 * specification's E4M3 layout (the pages use FP8 without defining its bits):
 * 1 sign, 4 exponent bits with bias 7, 3 fraction bits; exponent field 0 is
 * subnormal (fraction x 2^-9); there are no infinities, and only the two
 * codes with every exponent and fraction bit set are NaN, so the largest
 * finite magnitude is 1.75 x 2^8 = 448.
 */
double oracle_e4m3_to_double(uint8_t v)
{
    const int s = v >> 7, e = (v >> 3) & 15, f = v & 7;
    double mag;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)f, -9);
    else
        mag = ldexp(1.0 + f / 8.0, e - 7);
    return s ? -mag : mag;
}

void oracle_decode_e4m3(const uint8_t *src, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_e4m3_to_double(src[i]);
}

/*
 * Per-tensor FP8 product ("MegaMoE：Blackwell 与 Hopper 的融合算子解读",
 * Hopper section 04 on FP8 quantisation: with one scale per tensor the
 * dequantisation happens once, in the epilogue): ref[i][j] = scale_a x
 * scale_b x sum_k a(i,k) b(k,j).  A is stored [M][lda] (row i holds k
 * contiguously), B is stored [N][ldb] (column j of the K x N operand holds k
 * contiguously).  The sum is the same ascending-k double sum as
 * oracle_gemm_ref (products of two E4M3 values are exact in double); the
 * product (scale_a x scale_b), formed first, multiplies the finished sum.
 */
int oracle_gemm_e4m3_ref(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B,
                         int64_t ldb, double scale_a, double scale_b, double *ref)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!a || !b) {
        free(a);
        free(b);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            a[i * K + k] = oracle_e4m3_to_double(A[i * lda + k]);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            b[j * K + k] = oracle_e4m3_to_double(B[j * ldb + k]);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += a[i * K + k] * b[j * K + k];
            ref[i * N + j] = scale_a * scale_b * acc;
        }
    free(a);
    free(b);
    return 0;
}

/* The same value at the elements (rows[t], cols[t]) only. */
/*
 * Block scales in E8M0, the OCP microscaling scale format (the pages name it
 * for MXFP8 data, one scale per block, in "MegaMoE：Blackwell 与 Hopper 的融合
 * 算子解读", the quantised-dispatch formats table): an unsigned 8-bit
 * exponent, value 2^(v - 127); 255 is NaN.
 */
double oracle_e8m0_to_double(uint8_t v)
{
    return v == 255 ? NAN : ldexp(1.0, (int)v - 127);
}

/*
 * Blockwise-scaled FP8 product (MegaMoE, Hopper section 04, the blockwise
 * path: activations scaled per token and per 128-element block of K,
 * weights per 128 x 128 block, and the dequantisation inside the K loop:
 * each K block's partial product is scaled before it joins the total).  A
 * is stored [M][lda], B [N][ldb] (k contiguous, as in oracle_gemm_e4m3_ref);
 * sa is [M][lds_a] bytes, sa[i][b] scaling row i of A over k in
 * [128 b, 128 b + 128); sb is [ceil(N / 128)][lds_b] bytes, sb[c][b]
 * scaling output columns [128 c, 128 c + 128) over the same k block:
 *   ref[i][j] = sum over b < ceil(K / 128) of
 *               e8m0(sa[i][b]) x e8m0(sb[j / 128][b]) x sum_{k in block b} a(i,k) b(k,j).
 * Each block's sum is exact in double; the scales are powers of two.
 */
int oracle_gemm_e4m3_block_ref(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B,
                               int64_t ldb, const uint8_t *sa, int64_t lds_a, const uint8_t *sb, int64_t lds_b,
                               double *ref)
{
    const int64_t nblk = (K + 127) / 128;
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!a || !b) {
        free(a);
        free(b);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            a[i * K + k] = oracle_e4m3_to_double(A[i * lda + k]);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            b[j * K + k] = oracle_e4m3_to_double(B[j * ldb + k]);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double total = 0.0;
            for (int64_t blk = 0; blk < nblk; ++blk) {
                const int64_t k1 = (blk + 1) * 128 < K ? (blk + 1) * 128 : K;
                double part = 0.0;
                for (int64_t k = blk * 128; k < k1; ++k)
                    part += a[i * K + k] * b[j * K + k];
                total += oracle_e8m0_to_double(sa[i * lds_a + blk]) *
                         oracle_e8m0_to_double(sb[(j / 128) * lds_b + blk]) * part;
            }
            ref[i * N + j] = total;
        }
    free(a);
    free(b);
    return 0;
}

void oracle_gemm_e4m3_ref_sampled(int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                                  double scale_a, double scale_b, const int64_t *rows, const int64_t *cols,
                                  int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += oracle_e4m3_to_double(A[rows[t] * lda + k]) * oracle_e4m3_to_double(B[cols[t] * ldb + k]);
        out[t] = scale_a * scale_b * acc;
    }
}
