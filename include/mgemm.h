/*
 * mgemm.h -- C ABI of the MI355X (gfx950) dense and grouped FP16/BF16 GEMM.
 *
 * The operation.  D[M,N] = A[M,K] x B[K,N]: every output element is the sum
 * over k of A[i,k]*B[k,j], accumulated in fp32, and only the finished sum is
 * converted to the output type by the epilogue ("B200 的 2CTA 怎样调优：从矩阵
 * 分块到流水线", section 七, the accumulate-then-epilogue sketch).  The
 * conversion is IEEE round-to-nearest-even.  The grouped form applies one
 * such product per expert to that expert's slice of rows, as an MoE expert
 * layer does ("MegaMoE：Blackwell 与 Hopper 的融合算子解读", Recap 1 on the MoE
 * stages), and can fuse the SwiGLU gate, h = up x SiLU(gate), into the
 * epilogue (first page, section 七, "Gate／SwiGLU"; gate and up columns
 * interleaved in blocks of eight, gate first, MegaMoE Hopper section 10).
 * The dense form also takes E4M3 (FP8) operands with one fp32 scale per
 * tensor, multiplied into the finished sum (MegaMoE Hopper section 04;
 * gemm_run_scaled).
 *
 * Launch semantics follow the execution-model page ("从 CUDA 代码到 GPU 执行",
 * the launch-configuration and Stream sections): a run call only enqueues
 * kernels on the caller's stream and returns; results are valid once that
 * stream has been synchronised, and work on one stream runs in order.
 *
 * Memory ownership.  The caller owns every device buffer (operands, output,
 * row offsets, workspace).  The library never allocates or frees device
 * memory inside a run call.  A plan holds only host memory, is immutable once
 * made, and may be used from several threads and streams at once.
 *
 * Errors.  Every call returns an mgemm_status_t; no C++ exception crosses
 * this boundary.  Argument errors are detected before anything is enqueued
 * and leave the output untouched.  gemm_last_error_message() gives a
 * thread-local description of the last failure.
 *
 * Pointers passed to run calls are device pointers on the current HIP
 * device; the stream is a hipStream_t (NULL = that device's null stream).
 */
#ifndef MGEMM_H
#define MGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t, declared here so that this header does not
 * require the HIP headers. */
struct ihipStream_t;
typedef struct ihipStream_t *mgemm_stream_t;

/* E4M3: the OCP 8-bit float with 1 sign, 4 exponent (bias 7) and 3 fraction
 * bits, subnormals, no infinities, NaN = S.1111.111 (largest finite 448).
 * An input type only, of dense and grouped plans (gemm_run_scaled,
 * gemm_run_blockscaled, grouped_gemm_run_scaled,
 * grouped_gemm_run_blockscaled). */
typedef enum { MGEMM_F16 = 1, MGEMM_BF16 = 2, MGEMM_F32 = 3, MGEMM_E4M3 = 4 } mgemm_dtype_t;

/* Storage of a logical rows x cols operand.  ROW_MAJOR: element (r,c) at
 * r*ld + c.  COL_MAJOR: element (r,c) at c*ld + r.  D is always row-major. */
typedef enum { MGEMM_ROW_MAJOR = 0, MGEMM_COL_MAJOR = 1 } mgemm_layout_t;

/* Epilogue of the grouped form.  SILU_GATE_I8: the GEMM's N output columns
 * alternate gate and up in blocks of 8 (gate[0:8], up[0:8], gate[8:16], ...);
 * the run writes N/2 columns h[r,c] = SiLU(gate) * up, with SiLU(x) =
 * x / (1 + exp(-x)), computed from the fp32 accumulators and rounded once to
 * the output type. */
typedef enum { MGEMM_EPI_NONE = 0, MGEMM_EPI_SILU_GATE_I8 = 1 } mgemm_epilogue_t;

typedef enum {
    MGEMM_OK = 0,
    MGEMM_ERR_INVALID_ARG = 1,  /* null/negative/inconsistent arguments        */
    MGEMM_ERR_UNSUPPORTED = 2,  /* valid but not supported (dtype, alignment)  */
    MGEMM_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required  */
    MGEMM_ERR_NO_MEMORY = 4,    /* host allocation of a plan failed            */
    MGEMM_ERR_HIP = 5           /* a HIP call or kernel launch failed          */
} mgemm_status_t;

typedef struct mgemm_plan *mgemm_plan_t;

/* Dense problem.  Sizes and leading dimensions are in elements.
 *  - M, N, K >= 0.  M == 0 or N == 0: the run is a no-op.  K == 0: D is
 *    filled with zeros (the empty sum).
 *  - a_type == b_type, one of F16 / BF16 / E4M3.  d_type: F32 or the input
 *    type (E4M3 inputs: F32, BF16 or F16).
 *  - E4M3 inputs: A row-major and B column-major (both k-contiguous),
 *    K, lda and ldb multiples of 16, N a multiple of 4, no split of K and
 *    no forced tile but MGEMM_PLAN_FORCE_TILE_256x256_DTL; otherwise
 *    MGEMM_ERR_UNSUPPORTED.  Grouped E4M3: see grouped_gemm_run_scaled.
 *  - K % 8 == 0; A, B, D base addresses 16-byte aligned; lda, ldb a
 *    multiple of 8 elements; ldd * sizeof(d_type) a multiple of 16 bytes.
 *    Otherwise MGEMM_ERR_UNSUPPORTED.
 *  - lda >= K (row-major A) or >= M (col-major A); ldb >= N (row-major B) or
 *    >= K (col-major B); ldd >= N.  Otherwise MGEMM_ERR_INVALID_ARG.
 *  - D must not overlap A or B. */
typedef struct {
    int64_t M, N, K;
    mgemm_dtype_t a_type, b_type, d_type;
    mgemm_layout_t a_layout, b_layout;
    int64_t lda, ldb, ldd;
} mgemm_desc_t;

/* Grouped problem: num_groups experts; expert e owns rows
 * [off[e], off[e+1]) of A and of D, where off is the device array given to
 * grouped_gemm_run (num_groups + 1 non-decreasing int32 prefix sums, off[0]
 * == 0, off[num_groups] <= max_total_rows).  Expert e's weight is the K x N
 * matrix at B + e * stride_b (elements), stored row-major ([K][N], ldb >= N)
 * or column-major ([N][K], ldb >= K).  A is row-major [rows][K] (lda >= K).
 * D is row-major with ldd >= N (EPI_NONE) or >= N/2 (SILU_GATE_I8).
 * Same dtype and alignment rules as the dense form; SILU_GATE_I8 needs
 * N % 16 == 0.  Rows of D past off[num_groups] are not written. */
typedef struct {
    int32_t num_groups;
    int64_t max_total_rows;
    int64_t N, K;
    mgemm_dtype_t a_type, b_type, d_type;
    mgemm_layout_t b_layout;
    int64_t lda, ldb, stride_b, ldd;
    mgemm_epilogue_t epilogue;
} mgemm_grouped_desc_t;

/* Plan flags (bitwise or).  0 = let the planner choose. */
#define MGEMM_PLAN_FORCE_TILE_256x256 0x1u   /* the 256x256 macro-tile  */
#define MGEMM_PLAN_FORCE_TILE_128x128 0x2u   /* the 128x128 macro-tile  */
#define MGEMM_PLAN_FORCE_TILE_32x256  0x4u   /* narrow-M (few tokens)   */
#define MGEMM_PLAN_FORCE_TILE_64x256  0x8u   /* narrow-M (few tokens)   */
/* 256x256 with loads that write LDS directly (no staging registers; four
 * waves of 128x128 in dense plans, eight waves of 128x64 in grouped plans).
 * Dense plans: row-major A only, else UNSUPPORTED; the planner uses
 * it whenever it picks the 256x256 tile for such a plan.  Grouped plans
 * (whose A is always row-major): the planner uses it for the experts of 129
 * rows or more.  In both, MGEMM_PLAN_FORCE_TILE_256x256 selects the
 * register-staged 256x256 engine instead. */
#define MGEMM_PLAN_FORCE_TILE_256x256_DTL 0x10u
/* The few-token tile: up to 128 rows of A (tokens) x 128 columns, each
 * tile computing only its valid tokens rounded up to 16 (row-major A only,
 * else UNSUPPORTED).  The planner uses it for dense plans with M <= 128 and
 * for the grouped experts of 1..128 rows. */
#define MGEMM_PLAN_FORCE_TILE_NARROW  0x20u
/* The same tile 64 and 32 columns wide (more tiles for the same N, so a
 * decode-sized product fills the CUs with fewer or no K splits). */
#define MGEMM_PLAN_FORCE_TILE_NARROW64 0x40u
#define MGEMM_PLAN_FORCE_TILE_NARROW32 0x80u
#define MGEMM_PLAN_NO_XCD_REMAP       0x100u /* plain tile order        */
/* Dense plans: fix the number of K ranges per output tile (1..64; 1 turns
 * splitting off).  Without it the planner splits K only when the output
 * tiles alone leave compute units idle and K is long, and charges the
 * reduction to the split ("B200 的 2CTA 怎样调优", section 八: for small M/N
 * with a long K, split-K raises task parallelism at the cost of a
 * reduction).  A split plan writes fp32 partial sums to the workspace
 * (gemm_plan_workspace_size) and adds them in a fixed order, so results are
 * reproducible run to run. */
#define MGEMM_PLAN_SPLIT_K(n)         ((((uint32_t)(n)) & 0xFFu) << 16)

/* Make a plan for a dense problem on the current HIP device (or, when no
 * device is visible, for a 256-CU gfx950).  *out receives the plan; free it
 * with gemm_plan_destroy. */
mgemm_status_t gemm_plan(const mgemm_desc_t *desc, uint32_t flags, mgemm_plan_t *out);

/* Make a plan for a grouped problem (same conventions). */
mgemm_status_t grouped_gemm_plan(const mgemm_grouped_desc_t *desc, uint32_t flags, mgemm_plan_t *out);

/* Device workspace in bytes that run calls with this plan need (may be 0):
 * a split dense plan's counters and fp32 partial sums, a fused MoE plan's
 * schedule and counters (moe_fused_plan), else 0.  The workspace is scratch owned by the caller; it must be
 * 16-byte aligned, and two runs in flight at once must not share it. */
mgemm_status_t gemm_plan_workspace_size(mgemm_plan_t plan, size_t *bytes);

/* Enqueue D = A x B on `stream`.  A, B, D are device pointers in the layouts
 * of the plan's descriptor.  workspace may be NULL when the plan needs none;
 * a split plan returns MGEMM_ERR_WORKSPACE (and launches nothing) when it is
 * missing, misaligned or smaller than gemm_plan_workspace_size. */
mgemm_status_t gemm_run(mgemm_plan_t plan, const void *A, const void *B, void *D,
                        void *workspace, size_t workspace_bytes, mgemm_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): gemm_run
 * without a workspace argument.  The scratch a plan needs (the fp32 partial
 * sums of a plan that splits K) comes from a device array the library
 * holds, MGEMM_NOALLOC_SCRATCH_BYTES per device, kept by every GPU the
 * library has run on until the process ends; its address is looked up on
 * the first call with a device current.  The call allocates nothing.  A
 * plan whose gemm_plan_workspace_size exceeds MGEMM_NOALLOC_SCRATCH_BYTES
 * returns MGEMM_ERR_WORKSPACE and launches nothing.  Every call on one GPU
 * shares that GPU's array and leaves its last contents there: calls that
 * overlap on one GPU (on different streams, or from different threads)
 * race and give undefined results; serialise them.  Otherwise the same
 * semantics, results and errors as gemm_run (bit for bit the same output). */
#define MGEMM_NOALLOC_SCRATCH_BYTES (32u << 20)
mgemm_status_t gemm_run_noalloc(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                mgemm_stream_t stream);

/* Enqueue D = (scale_a x scale_b) x (A x B) on `stream` for a plan with
 * E4M3 inputs, with one scale per tensor ("MegaMoE：Blackwell 与 Hopper 的融合
 * 算子解读", Hopper section 04: with per-tensor scales the dequantisation is
 * a single multiply in the epilogue).  d_scale_a and d_scale_b are device
 * pointers to one fp32 value each, read by the kernel when it runs (so they
 * may be produced on the device without a host synchronisation).  The
 * products are accumulated in fp32; each finished sum is multiplied by the
 * fp32 product scale_a x scale_b (each output is fl(fl(scale_a * scale_b) *
 * acc), an fp32 multiply) and that is rounded once to d_type.  gemm_run on an
 * E4M3 plan is the same with both scales 1.  Errors: a non-E4M3 plan gives
 * MGEMM_ERR_UNSUPPORTED; a null or misaligned scale pointer
 * MGEMM_ERR_INVALID_ARG; otherwise as gemm_run.  K == 0 writes zeros. */
mgemm_status_t gemm_run_scaled(mgemm_plan_t plan, const void *A, const void *B, void *D,
                               const float *d_scale_a, const float *d_scale_b,
                               void *workspace, size_t workspace_bytes, mgemm_stream_t stream);

/* Enqueue the blockwise-scaled product of a plan with E4M3 inputs
 * ("MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 04, the
 * blockwise path: activation scales per token and per 128-element block of
 * K, weight scales per 128 x 128 block, each K block's partial product
 * scaled before it joins the sum):
 *   D[i,j] = sum over k blocks b of sa[i][b] x sb[j / 128][b] x
 *            sum_{k in [128 b, 128 b + 128) and < K} A[i,k] B[k,j]
 * accumulated in fp32 and rounded once to d_type.  Scales are E8M0 bytes
 * (value 2^(v - 127); 255 is NaN), the power-of-two scale format of the
 * OCP microscaling blocks, applied by the matrix instruction itself.
 * d_scale_a: device bytes [M][lds_a], sa[i][b] at i * lds_a + b; d_scale_b:
 * device bytes [ceil(N / 128)][lds_b]; lds_a, lds_b >= ceil(K / 128), and
 * each array below 2^31 bytes (else MGEMM_ERR_INVALID_ARG); lds_a and lds_b
 * even (else MGEMM_ERR_UNSUPPORTED).  Bytes past ceil(K / 128) in a row are
 * padding: they may be read, never used.  Same operand
 * rules, workspace and errors as gemm_run_scaled; a non-E4M3 plan gives
 * MGEMM_ERR_UNSUPPORTED.  K == 0 writes zeros. */
mgemm_status_t gemm_run_blockscaled(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                    const uint8_t *d_scale_a, int64_t lds_a, const uint8_t *d_scale_b,
                                    int64_t lds_b, void *workspace, size_t workspace_bytes, mgemm_stream_t stream);

/* Enqueue the grouped product of a plan with E4M3 inputs: expert e's rows
 * times its weights, each finished fp32 sum multiplied by the fp32 product
 * scale_a x scale_b[e] -- fl(fl(scale_a * scale_b[e]) * acc) -- and that
 * rounded once to d_type (one scale for the activations and one per expert
 * for the weights: "MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper
 * section 04, the per-tensor path).  No gathered form (see
 * grouped_gemm_run_gather).
 * d_scale_a: device pointer to one float; d_scale_b: device pointer to
 * num_groups floats; both read by the kernel when it runs.  Grouped E4M3
 * plans need column-major expert weights, MGEMM_EPI_NONE, K, lda, ldb and
 * stride_b multiples of 16.  grouped_gemm_run on such a plan uses scales 1.
 * Errors: a non-E4M3 plan gives MGEMM_ERR_UNSUPPORTED, a null or misaligned
 * scale pointer MGEMM_ERR_INVALID_ARG, otherwise as grouped_gemm_run. */
mgemm_status_t grouped_gemm_run_scaled(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                       const int32_t *d_row_offsets, const float *d_scale_a,
                                       const float *d_scale_b, void *workspace, size_t workspace_bytes,
                                       mgemm_stream_t stream);

/* Enqueue the grouped product of a plan with E4M3 inputs with block scales
 * ("MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 04, the
 * blockwise path of the expert GEMMs): expert e's rows [off[e], off[e+1])
 * times its weight, each 128-k block's partial product scaled before it
 * joins the sum, as gemm_run_blockscaled per expert:
 *   D[r,j] = sum over k blocks b of sa[r][b] x sb[e][j / 128][b] x
 *            sum_{k in block b, k < K} A[r,k] B_e[k,j]
 * accumulated in fp32 and rounded once to d_type.  Scales are E8M0 bytes.
 * d_scale_a: device bytes [max_total_rows][lds_a], routed row r's scales at
 * r * lds_a; d_scale_b: device bytes, expert e's [ceil(N / 128)][lds_b]
 * block at e * stride_sb.  lds_a, lds_b >= ceil(K / 128) and stride_sb >=
 * ceil(N / 128) * lds_b, each array below 2^31 bytes (else
 * MGEMM_ERR_INVALID_ARG); lds_a and lds_b even (else MGEMM_ERR_UNSUPPORTED).
 * Bytes past ceil(K / 128) in a row are padding: they may be read, never
 * used.  Operands, offsets, outputs and errors as grouped_gemm_run_scaled
 * (rows past off[G] are not written); a non-E4M3 plan gives
 * MGEMM_ERR_UNSUPPORTED. */
mgemm_status_t grouped_gemm_run_blockscaled(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                            const int32_t *d_row_offsets, const uint8_t *d_scale_a, int64_t lds_a,
                                            const uint8_t *d_scale_b, int64_t lds_b, int64_t stride_sb,
                                            void *workspace, size_t workspace_bytes, mgemm_stream_t stream);

/* Enqueue the grouped product on `stream`.  d_row_offsets is a device array
 * of num_groups + 1 int32 prefix sums; it is read by the kernels only (no
 * host synchronisation).  Offsets that break the descriptor's rules give
 * undefined results but never out-of-bounds accesses beyond max_total_rows. */
mgemm_status_t grouped_gemm_run(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                const int32_t *d_row_offsets,
                                void *workspace, size_t workspace_bytes, mgemm_stream_t stream);

/* Human-readable description of the chosen variant (tile, waves, grid,
 * order); writes at most len bytes including the terminating NUL. */
mgemm_status_t gemm_plan_describe(mgemm_plan_t plan, char *buf, size_t len);

/* Numeric plan details, for logs and tests. */
typedef struct {
    int32_t block_m, block_n, block_k;   /* macro-tile                        */
    int32_t waves_m, waves_n;            /* wavefront grid inside a tile      */
    int32_t stages;                      /* LDS ring depth (deeper operand)   */
    int32_t lds_bytes;                   /* LDS per workgroup                 */
    int64_t tiles_m, tiles_n, tiles;     /* output tiles (dense form)         */
    int64_t k_steps;                     /* ceil(K / block_k)                 */
    double coverage;                     /* M*N / (tiles * block_m * block_n) */
    int32_t grid;                        /* workgroups launched               */
    int32_t group_m;                     /* tile rows per L2 group            */
    int32_t xcd_remap;                   /* 1 if the XCD-aware order is used  */
    int32_t num_cus;                     /* compute units planned for         */
    int32_t splits;                      /* K ranges per output tile (dense)  */
} mgemm_plan_info_t;

mgemm_status_t gemm_plan_info(mgemm_plan_t plan, mgemm_plan_info_t *info);

void gemm_plan_destroy(mgemm_plan_t plan);

const char *gemm_status_string(mgemm_status_t status);

/* Thread-local text of the last error raised on this thread ("" if none). */
const char *gemm_last_error_message(void);

/* Tile budget arithmetic of the planner (host only, no device needed):
 * tiles = ceil(M/BM) * ceil(N/BN); coverage = M*N / (tiles*BM*BN);
 * lds_bytes = stages * (BM*BK + BK*BN) * elt_bytes; k_steps = ceil(K/BK).
 * The tile-and-stage budget rule is the one "B200 的 2CTA 怎样调优" (section
 * 三, the CPU tile calculator) prints, without its split of the tile over a
 * CTA pair: on a CU the whole macro-tile lives in one workgroup's LDS. */
typedef struct {
    int64_t tiles;
    double coverage;
    int64_t lds_bytes;
    int64_t k_steps;
} mgemm_budget_t;

mgemm_status_t mgemm_tile_budget(int64_t M, int64_t N, int64_t K, int32_t BM, int32_t BN, int32_t BK,
                                 int32_t stages, int32_t elt_bytes, mgemm_budget_t *out);

/* L2 working set of a group of tiles: (group_m*BM + group_n*BN) * K * elt
 * bytes -- the operand rows and columns that a group of output tiles
 * shares ("GEMM优化（三）", section 3.4 on choosing the super-tile). */
int64_t mgemm_group_working_set(int32_t group_m, int32_t group_n, int32_t BM, int32_t BN,
                                int64_t K, int32_t elt_bytes);

/* Token count rounded up to the narrow tile granularity: (n + g - 1) / g * g
 * for g a power of two (MegaMoE Blackwell section 04 rounds valid tokens up
 * to a multiple of 16 before sizing the MMA). */
int64_t mgemm_round_tokens(int64_t n, int32_t granule);

/* The grouped product with A's rows gathered (the MoE dispatch fused into the
 * A loads; "MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 11, a
 * dispatch warp pulls the routed tokens' rows for the expert GEMM): routed
 * row r of the product reads row d_row_index[r] of X, a row-major
 * [x_rows][K] matrix with the plan's lda, instead of row r of a gathered A.
 * d_row_index: device int32, one entry per routed row (off[num_groups]
 * entries); an entry outside [0, x_rows) reads as a row of zeros.
 * Everything else is grouped_gemm_run's.  x_rows * lda * 2 must be below
 * 2^31 (else MGEMM_ERR_INVALID_ARG).  Only 16-bit plans whose launches use
 * the default 32x256 and direct-to-LDS 256x256 tiles take gathered rows: a
 * plan forced onto another tile, and any E4M3 plan, returns
 * MGEMM_ERR_UNSUPPORTED before anything is launched. */
mgemm_status_t grouped_gemm_run_gather(mgemm_plan_t plan, const void *X, int64_t x_rows, const void *B, void *D,
                                       const int32_t *d_row_offsets, const int32_t *d_row_index, void *workspace,
                                       size_t workspace_bytes, mgemm_stream_t stream);

/* The SiLU-gated grouped product (FC1 of an MoE layer) with each routed
 * row's output multiplied by that row's routing weight before the rounding:
 *   h[r, c] = round(SiLU(gate[r, c]) * up[r, c] * d_row_weight[r])
 * ("MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 09: the FC1
 * epilogue chain optionally multiplies by the routing weight, and taking
 * that weight into FC2's input lets the final combine add the experts'
 * contributions as they are, since p(hW2) = (ph)W2 for the linear FC2; run
 * FC2 with grouped_gemm_run, then mgemm_moe_combine with d_weights NULL).
 * SwiGLU and the weight product are fp32; one rounding to the output type.
 * d_row_weight: device fp32, 4-byte aligned, one weight per routed row
 * (off[num_groups] entries, in routed-row order: the weight of the (token,
 * choice) pair routed to that row).  d_row_index: NULL (A holds the routed
 * rows, as in grouped_gemm_run; x_rows is ignored) or the gathered form's
 * index into X = A of x_rows rows (as in grouped_gemm_run_gather, with its
 * rules on tiles).  Only plans with MGEMM_EPI_SILU_GATE_I8 (else
 * MGEMM_ERR_UNSUPPORTED); a null or misaligned d_row_weight gives
 * MGEMM_ERR_INVALID_ARG.  Everything else is grouped_gemm_run's. */
mgemm_status_t grouped_gemm_run_weighted(mgemm_plan_t plan, const void *A, int64_t x_rows, const void *B, void *D,
                                         const int32_t *d_row_offsets, const int32_t *d_row_index,
                                         const float *d_row_weight, void *workspace, size_t workspace_bytes,
                                         mgemm_stream_t stream);

/* MoE combine: every token's output row is the routing-weighted sum of the
 * rows its top-k experts produced ("MegaMoE：Blackwell 与 Hopper 的融合算子解读",
 * Blackwell section 13: a separate top-k reduce reads each branch and adds
 * them into the token's output; Hopper section 09 for the routing weight p
 * applied to an expert's output, p(hW2) = (ph)W2).
 *   Y[t, j] = sum_{k < top_k} weights[t*top_k + k] * Z[pos[t*top_k + k], j]
 * for t < T, j < H.  Z: 16-bit rows (the FC2 output in expert order),
 * z_rows x H, row pitch ldz; Y: T x H of the same type, row pitch ldy; pos
 * (int32) and weights (fp32): device arrays of T*top_k entries; weights may
 * be NULL, every weight then 1 (a plain sum, for expert outputs whose
 * routing weights were taken into FC1's epilogue by
 * grouped_gemm_run_weighted).  The terms
 * are added in k order with fp32 fused multiply-adds, then rounded once
 * (RNE) to the 16-bit type.  A position outside [0, z_rows) contributes
 * nothing.  dtype: BF16 or F16.  H % 8 == 0, ldz and ldy multiples of 8 and
 * >= H, Z and Y 16-byte aligned, z_rows * ldz * 2 <= 2^31 - 16 bytes,
 * 1 <= top_k <= 256, otherwise MGEMM_ERR_UNSUPPORTED / _INVALID_ARG.
 * T == 0 or H == 0: no-op.  Y must not overlap Z.  Asynchronous on stream. */
mgemm_status_t mgemm_moe_combine(const void *Z, int64_t z_rows, int64_t ldz, const int32_t *d_pos,
                                 const float *d_weights, void *Y, int64_t ldy, int64_t T, int32_t top_k, int64_t H,
                                 mgemm_dtype_t dtype, mgemm_stream_t stream);

/* Blockwise FP8 quantisation of a 16-bit matrix into the activation layout
 * of the block-scaled products ("MegaMoE：Blackwell 与 Hopper 的融合算子解读",
 * Hopper sections 04 and 09: after SwiGLU, each block's absolute maximum
 * gives a power-of-two E8M0 scale, and the block is multiplied by the
 * scale's reciprocal and converted to FP8).  Blocks are 128 consecutive
 * columns of a row (the last may be shorter).  Scale 2^E: the smallest
 * power of two with amax <= 448 * 2^E, E in [-127, 127]; 2^0 for an
 * all-zero block; a block with a NaN or infinity gets scale byte 255 and
 * NaN codes.  Codes: x / 2^E rounded to the nearest E4M3 value, ties to
 * the even code.  X: rows x cols, row pitch ldx elements, BF16 or F16
 * (x_type); Q: rows x cols E4M3 bytes, pitch ldq; S: rows x lds E8M0 bytes
 * (byte b of row r: the scale of columns [128 b, 128 b + 128)), lds >=
 * ceil(cols / 128); all device memory, read and written when the kernel
 * runs on `stream`.  Q and S feed gemm_run_blockscaled /
 * grouped_gemm_run_blockscaled as A and its scales (lda = ldq, lds_a = lds,
 * which those require to be even).  cols, ldx and ldq even, X 4-byte and Q
 * 2-byte aligned, else MGEMM_ERR_UNSUPPORTED; null pointers or short
 * pitches give MGEMM_ERR_INVALID_ARG.  rows or cols 0: nothing is done. */
mgemm_status_t mgemm_quantize_e4m3_block(const void *X, int64_t rows, int64_t cols, int64_t ldx,
                                         mgemm_dtype_t x_type, uint8_t *Q, int64_t ldq, uint8_t *S, int64_t lds,
                                         mgemm_stream_t stream);

/* The MoE expert layer's two GEMMs in one persistent launch ("MegaMoE：
 * Blackwell 与 Hopper 的融合算子解读", Hopper section 01 on the resident
 * FC1 -> SwiGLU -> FC2 pipeline and its fc1_done counters, Blackwell section
 * 06 on publishing a finished tile through a counter, Hopper sections 13 and
 * 15 on when to publish and how to order the tasks).  For every expert e with
 * rows [off[e], off[e+1]):
 *   FC1: H[r, :] = SiLU(gate) * up of row r of X times W1_e, the SILU_GATE_I8
 *        epilogue of grouped_gemm_run (gate and up columns of W1_e
 *        interleaved in blocks of 8, gate first), each h rounded once to dtype;
 *   FC2: Y[r, :] = H[r, :] x W2_e, accumulated in fp32, rounded once.
 * H is both an output and FC2's input: FC2 reads the rounded h, so Y equals
 * what grouped_gemm_run of FC1 then of FC2 gives, bit for bit.
 *
 * Shapes (elements):
 *  - num_experts in [1, 256]; max_total_rows < 2^30: rows of H and Y (and of
 *    X when not gathering) that exist;
 *  - hidden: FC1's K and FC2's N, a multiple of 16; inter: the h width,
 *    FC1's N is 2 * inter and FC2's K is inter, a multiple of 64;
 *  - X row-major [rows][lda], lda >= hidden; W1_e at W1 + e * stride_w1,
 *    row-major [hidden][2 * inter] with ldw1 >= 2 * inter; W2_e at W2 + e *
 *    stride_w2, row-major [inter][hidden] with ldw2 >= hidden; H row-major
 *    with ldh >= inter and ldh a multiple of 64; Y row-major, ldy >= hidden;
 *  - lda, ldw1, ldw2, ldy, stride_w1 and stride_w2 multiples of 8, leading
 *    dimensions at most 2^20, one expert's W1 or W2 below 2^30 elements;
 *  - dtype BF16 or F16 for every operand.
 * Other values: MGEMM_ERR_INVALID_ARG (inconsistent) or _UNSUPPORTED. */
typedef struct {
    int32_t num_experts;
    int64_t max_total_rows;
    int64_t hidden, inter;
    mgemm_dtype_t dtype;
    int64_t lda;
    int64_t ldw1, stride_w1;
    int64_t ldw2, stride_w2;
    int64_t ldh, ldy;
} mgemm_moe_desc_t;

/* Make a plan for the fused layer (flags must be 0).  Its workspace
 * (gemm_plan_workspace_size) holds the task schedule and the per-(expert,
 * row block) counters: 6400 + 4 * (ceil(max_total_rows / 256) + num_experts)
 * bytes rounded up to 256. */
mgemm_status_t moe_fused_plan(const mgemm_moe_desc_t *desc, uint32_t flags, mgemm_plan_t *out);

/* Enqueue the fused layer on `stream`: a one-workgroup kernel that orders
 * the experts (largest first) and clears the counters, then the persistent
 * kernel.  d_row_offsets: device int32 prefix sums as for grouped_gemm_run.
 * d_row_index: NULL (row r of FC1 reads row r of X, which has
 * max_total_rows rows), or a device int32 array with one entry per routed
 * row, row r reading X row d_row_index[r] of x_rows rows (entries outside
 * [0, x_rows) read as zeros; x_rows * lda * 2 < 2^31).  X, W1, W2, Y and
 * the workspace must be 16-byte aligned, H 128-byte aligned (each h row block
 * is written on one compute unit and read on others in the same launch, so
 * no two row blocks may share a 128-byte line), else MGEMM_ERR_UNSUPPORTED.
 * The workspace must not be shared by runs in flight at once; a missing or
 * short one gives MGEMM_ERR_WORKSPACE.  H and Y must not overlap each other
 * or the inputs.  Offsets that break the rules give undefined results but
 * no access outside the buffers. */
mgemm_status_t moe_fused_run(mgemm_plan_t plan, const void *X, int64_t x_rows, const int32_t *d_row_index,
                             const void *W1, const void *W2, void *H, void *Y, const int32_t *d_row_offsets,
                             void *workspace, size_t workspace_bytes, mgemm_stream_t stream);

/* The fused layer with each routed row's h multiplied by that row's routing
 * weight before its rounding, as grouped_gemm_run_weighted does for FC1
 * ("MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 09: the FC1
 * epilogue chain optionally applies the routing weight; FC2 being linear,
 * Y's rows are then the weighted expert outputs, p(hW2) = (ph)W2, and
 * mgemm_moe_combine with d_weights NULL adds them into the tokens' rows).
 * d_row_weight: device fp32, 4-byte aligned, one weight per routed row
 * (off[num_experts] entries in routed-row order); null or misaligned gives
 * MGEMM_ERR_INVALID_ARG.  Same tiles and k order as moe_fused_run, so h
 * and Y equal grouped_gemm_run_weighted's h and grouped_gemm_run's FC2 on
 * it bit for bit.  Everything else is moe_fused_run's. */
mgemm_status_t moe_fused_run_weighted(mgemm_plan_t plan, const void *X, int64_t x_rows, const int32_t *d_row_index,
                                      const void *W1, const void *W2, void *H, void *Y,
                                      const int32_t *d_row_offsets, const float *d_row_weight, void *workspace,
                                      size_t workspace_bytes, mgemm_stream_t stream);

/* Library version, e.g. "mgemm 0.1 gfx950". */
const char *mgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_H */
