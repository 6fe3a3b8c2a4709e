// api.cpp -- the run entry points of the C ABI and its error reporting.
//
// A run call validates its pointers and workspace, fills the kernel
// argument block from the plan and enqueues the kernels on the caller's
// stream.  It never synchronises and never allocates device memory.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.hpp"

#include <atomic>

namespace mgemm {

static thread_local char g_err[512];

// A tag per run for the split arrival counters: process-wide, never 0 or
// ~0 (the values of a zeroed or 0xFF-filled workspace).
static uint32_t next_run_tag()
{
    static std::atomic<uint32_t> counter{0};
    uint32_t t;
    do {
        t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
    } while (t == 0 || t == 0xFFFFFFFFu);
    return t;
}

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

int in_code(mgemm_dtype_t t);
int out_code(mgemm_dtype_t t);
int dtype_size(mgemm_dtype_t t);

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static mgemm_status_t hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return MGEMM_OK;
    set_error("%s: %s", what, hipGetErrorString(e));
    return MGEMM_ERR_HIP;
}

}  // namespace mgemm

using namespace mgemm;

mgemm_status_t mgemm::dense_run(mgemm_plan_t plan, const void *A, const void *B, void *D, const float *scale_a,
                                const float *scale_b, void *workspace, size_t workspace_bytes, mgemm_stream_t stream,
                                const uint8_t *block_sa, int64_t block_lda, const uint8_t *block_sb,
                                int64_t block_ldb)
{
    const mgemm_desc_t &d = plan->dense;
    if (plan->noop)
        return MGEMM_OK;
    hipStream_t s = (hipStream_t)stream;
    const int esz = dtype_size(d.d_type);
    if (!D || (!plan->zero_fill && (!A || !B))) {
        set_error("gemm_run: null operand pointer");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) {
        set_error("gemm_run: A, B and D must be 16-byte aligned");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (plan->zero_fill)
        return hip_status(launch_zero_fill(D, (int)d.M, (int)d.N, d.ldd * esz, esz, s), "gemm_run zero fill");
    const bool split = plan->splits > 1 && plan->tiles > 0;
    if (split && (!workspace || workspace_bytes < plan->workspace_bytes || !aligned16(workspace))) {
        set_error("gemm_run: the plan splits K and needs a 16-byte aligned workspace of %zu bytes (got %zu at %p)",
                  plan->workspace_bytes, workspace_bytes, workspace);
        return MGEMM_ERR_WORKSPACE;
    }

    const bool ak = d.a_layout == MGEMM_ROW_MAJOR;
    const bool bk = d.b_layout == MGEMM_COL_MAJOR;
    const int in = in_code(d.a_type), out = out_code(d.d_type);
    DenseArgs a;
    a.A = A;
    a.B = B;
    a.D = D;
    a.M = (int)d.M;
    a.N = (int)(d.N & ~(int64_t)3);
    a.K = (int)d.K;
    a.lda = (int)d.lda;
    a.ldb = (int)d.ldb;
    a.ldd = (int)d.ldd;
    a.tiles_m = (int)plan->tiles_m;
    a.tiles_n = (int)plan->tiles_n;
    a.tiles = (int)plan->tiles;
    a.group_m = plan->group_m;
    a.xcd_remap = plan->xcd_remap;
    a.splits = 1;
    a.kchunk = (int)d.K;
    a.split_stride = 0;
    a.scale_a = scale_a;
    a.scale_b = scale_b;
    a.block_sa = block_sa;
    a.block_sb = block_sb;
    a.block_lda = (int)block_lda;
    a.block_ldb = (int)block_ldb;
    if (block_sa && a.tiles > 0) {
        // E8M0 block scales: the plan's tile with the scaled matrix instruction
        DenseFn f = dense_block_fn_256x256dtl_e4m3(ak, bk, out);
        if (!f) {
            set_error("gemm_run_blockscaled: kernel missing for the planned variant");
            return MGEMM_ERR_UNSUPPORTED;
        }
        return hip_status(f(a, plan->grid, s), "gemm_run_blockscaled launch");
    }
    if (plan->sk_tiles > 0 && a.tiles > 0) {
        // stream-K: whole tiles and the cut tiles' ranges in one launch
        DenseArgs w = a;
        w.splits = plan->splits;
        w.kchunk = plan->kchunk;
        w.sk_tiles = plan->sk_tiles;
        w.ws = (char *)workspace;
        w.slab_offset = plan->slab_offset;
        w.tag = next_run_tag();
        DenseFn f = in == IN_BF16 ? dense_sk_fn_256x256dtl_bf16(bk, out) : dense_sk_fn_256x256dtl_f16(bk, out);
        if (!f) {
            set_error("gemm_run: stream-K kernel missing for the planned variant");
            return MGEMM_ERR_UNSUPPORTED;
        }
        if (mgemm_status_t st = hip_status(f(w, plan->grid, s), "gemm_run launch"))
            return st;
    } else if (is_narrow(plan->tile) && a.tiles > 0) {
        // one launch: a split's last range adds the ranges' partials itself
        DenseArgs w = a;
        w.splits = plan->splits;
        w.kchunk = plan->kchunk;
        w.tiles = a.tiles * plan->splits;
        w.ws = split ? (char *)workspace : nullptr;
        w.slab_offset = plan->slab_offset;
        w.tag = split ? next_run_tag() : 0;
        DenseFn f = dense_fn(plan->tile, ak, bk, in, out);
        if (!f) {
            set_error("gemm_run: kernel missing for the planned variant");
            return MGEMM_ERR_UNSUPPORTED;
        }
        if (mgemm_status_t st = hip_status(f(w, plan->grid, s), "gemm_run launch"))
            return st;
    } else if (split) {
        // every K range writes its fp32 partial tile into its own slab of
        // the workspace; the reduction adds the slabs into D
        DenseArgs w = a;
        w.D = workspace;
        w.ldd = a.N;
        w.splits = plan->splits;
        w.kchunk = plan->kchunk;
        w.split_stride = (int64_t)a.M * a.N;
        w.tiles = a.tiles * plan->splits;
        DenseFn f = dense_fn(plan->tile, ak, bk, in, OUT_F32);
        if (!f) {
            set_error("gemm_run: kernel missing for the planned variant");
            return MGEMM_ERR_UNSUPPORTED;
        }
        if (mgemm_status_t st = hip_status(f(w, plan->grid, s), "gemm_run launch"))
            return st;
        if (mgemm_status_t st = hip_status(launch_reduce_splits((const float *)workspace, D, a.M, a.N, a.N,
                                                                w.split_stride, plan->splits, d.ldd, out, s),
                                           "gemm_run reduce launch"))
            return st;
    } else if (a.tiles > 0) {
        DenseFn f = dense_fn(plan->tile, ak, bk, in, out);
        if (!f) {
            set_error("gemm_run: kernel missing for the planned variant");
            return MGEMM_ERR_UNSUPPORTED;
        }
        if (mgemm_status_t st = hip_status(f(a, plan->grid, s), "gemm_run launch"))
            return st;
    }
    if (a.N != d.N) {
        DenseArgs e = a;
        e.N = (int)d.N;
        EdgeFn ef = edge_fn(in, out);
        if (!ef) {
            set_error("gemm_run: edge kernel missing");
            return MGEMM_ERR_UNSUPPORTED;
        }
        return hip_status(ef(e, ak ? 1 : 0, bk ? 1 : 0, a.N, s), "gemm_run edge launch");
    }
    return MGEMM_OK;
}

extern "C" mgemm_status_t gemm_run(mgemm_plan_t plan, const void *A, const void *B, void *D, void *workspace,
                                   size_t workspace_bytes, mgemm_stream_t stream)
{
    if (!plan || plan->kind != PLAN_DENSE) {
        set_error("gemm_run: null or non-dense plan");
        return MGEMM_ERR_INVALID_ARG;
    }
    return dense_run(plan, A, B, D, nullptr, nullptr, workspace, workspace_bytes, stream);
}

extern "C" mgemm_status_t gemm_run_scaled(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                          const float *d_scale_a, const float *d_scale_b, void *workspace,
                                          size_t workspace_bytes, mgemm_stream_t stream)
{
    if (!plan || plan->kind != PLAN_DENSE) {
        set_error("gemm_run_scaled: null or non-dense plan");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (plan->dense.a_type != MGEMM_E4M3) {
        set_error("gemm_run_scaled: the plan's inputs are not E4M3");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (!d_scale_a || !d_scale_b || ((uintptr_t)d_scale_a & 3) || ((uintptr_t)d_scale_b & 3)) {
        set_error("gemm_run_scaled: scale pointers must be non-null and 4-byte aligned");
        return MGEMM_ERR_INVALID_ARG;
    }
    return dense_run(plan, A, B, D, d_scale_a, d_scale_b, workspace, workspace_bytes, stream);
}

extern "C" mgemm_status_t gemm_run_blockscaled(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                               const uint8_t *d_scale_a, int64_t lds_a, const uint8_t *d_scale_b,
                                               int64_t lds_b, void *workspace, size_t workspace_bytes,
                                               mgemm_stream_t stream)
{
    if (!plan || plan->kind != PLAN_DENSE) {
        set_error("gemm_run_blockscaled: null or non-dense plan");
        return MGEMM_ERR_INVALID_ARG;
    }
    const mgemm_desc_t &d = plan->dense;
    if (d.a_type != MGEMM_E4M3) {
        set_error("gemm_run_blockscaled: the plan's inputs are not E4M3");
        return MGEMM_ERR_UNSUPPORTED;
    }
    const int64_t kb = (d.K + 127) / 128, nb = (d.N + 127) / 128;
    if (!d_scale_a || !d_scale_b || lds_a < kb || lds_b < kb || lds_a < 1 || lds_b < 1) {
        set_error("gemm_run_blockscaled: scale pointers must be non-null and lds_a, lds_b >= ceil(K / 128) (= %lld)",
                  (long long)kb);
        return MGEMM_ERR_INVALID_ARG;
    }
    if ((lds_a | lds_b) & 1) {
        set_error("gemm_run_blockscaled: lds_a and lds_b must be even (two k blocks' scales are read at once)");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if ((uint64_t)d.M * (uint64_t)lds_a > (uint64_t)kMaxRecords ||
        (uint64_t)nb * (uint64_t)lds_b > (uint64_t)kMaxRecords) {
        set_error("gemm_run_blockscaled: each scale array must span less than 2^31 bytes");
        return MGEMM_ERR_INVALID_ARG;
    }
    return dense_run(plan, A, B, D, nullptr, nullptr, workspace, workspace_bytes, stream, d_scale_a, lds_a,
                     d_scale_b, lds_b);
}

// E4M3 block scales of the grouped product (checked by the caller).
struct GroupedBlockScales {
    const uint8_t *sa = nullptr, *sb = nullptr;
    int64_t lds_a = 0, lds_b = 0, stride_sb = 0;
};

// row_index: nullptr, or the gathered form's index (x_rows rows of A exist).
// row_weight: nullptr, or one fp32 weight per routed row for the SiLU-gate
// epilogue.  blk: nullptr, or the E4M3 block scales.
static mgemm_status_t grouped_run(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                  const int32_t *d_row_offsets, const int32_t *row_index, int64_t x_rows,
                                  mgemm_stream_t stream, const float *scale_a = nullptr,
                                  const float *scale_b = nullptr, const float *row_weight = nullptr,
                                  const GroupedBlockScales *blk = nullptr)
{
    if (!plan || plan->kind != PLAN_GROUPED) {
        set_error("grouped_gemm_run: null or non-grouped plan");
        return MGEMM_ERR_INVALID_ARG;
    }
    const mgemm_grouped_desc_t &d = plan->grouped;
    if (plan->noop)
        return MGEMM_OK;
    if (!D || !d_row_offsets || (!plan->zero_fill && (!A || !B))) {
        set_error("grouped_gemm_run: null pointer");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (row_index && d.a_type == MGEMM_E4M3) {
        // the E4M3 grouped kernel reads A's rows in place; it has no gathered form
        set_error("grouped_gemm_run_gather: E4M3 plans take no gathered rows (gather the rows first and use "
                  "grouped_gemm_run_scaled)");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (row_index && !plan->zero_fill) {
        if (x_rows < 0 || x_rows > INT32_MAX ||
            (uint64_t)x_rows * (uint64_t)d.lda * 2u > (uint64_t)kMaxRecords) {
            set_error("grouped_gemm_run_gather: x_rows=%lld out of range (x_rows * lda * 2 must be < 2^31)",
                      (long long)x_rows);
            return MGEMM_ERR_INVALID_ARG;
        }
        for (const GroupedLaunch &L : plan->launches) {
            if (L.tile != TILE_32x256 && L.tile != TILE_256x256_DTL && !is_narrow(L.tile)) {
                set_error("grouped_gemm_run_gather: the planned tile %d does not take gathered rows (the default "
                          "narrow, 32x256 and direct-to-LDS 256x256 tiles do)", L.tile);
                return MGEMM_ERR_UNSUPPORTED;
            }
        }
    }
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) {
        set_error("grouped_gemm_run: A, B and D must be 16-byte aligned");
        return MGEMM_ERR_UNSUPPORTED;
    }
    hipStream_t s = (hipStream_t)stream;
    const bool silu = d.epilogue == MGEMM_EPI_SILU_GATE_I8;
    const int esz = dtype_size(d.d_type);
    if (plan->zero_fill) {
        // K == 0: every existing output row is the empty sum (and SiLU(0)*0 = 0)
        return hip_status(launch_zero_fill(D, (int)d.max_total_rows, (int)(silu ? d.N / 2 : d.N), d.ldd * esz, esz, s),
                          "grouped_gemm_run zero fill");
    }
    const bool bk = d.b_layout == MGEMM_COL_MAJOR;
    const int in = in_code(d.a_type), out = out_code(d.d_type), epi = silu ? EPI_SILU_GATE : EPI_NONE;
    for (const GroupedLaunch &L : plan->launches) {
        const TileShape &ts = tile_shape(L.tile);
        GroupedArgs a;
        a.A = A;
        a.B = B;
        a.D = D;
        a.offs = d_row_offsets;
        a.G = d.num_groups;
        a.N = (int)d.N;
        a.K = (int)d.K;
        a.lda = (int)d.lda;
        a.ldb = (int)d.ldb;
        a.ldd = (int)d.ldd;
        a.stride_b = d.stride_b;
        a.max_rows = (int)d.max_total_rows;
        a.tiles_n = (int)((d.N + ts.bn - 1) / ts.bn);
        a.bucket_lo = L.lo;
        a.bucket_hi = L.hi;
        a.scale_a = scale_a;
        a.scale_b = scale_b;
        a.xcd_remap = plan->xcd_remap;
        a.row_index = row_index;
        a.x_rows = (int)x_rows;
        a.row_weight = row_weight;
        GroupedFn f;
        if (blk) {
            a.block_sa = blk->sa;
            a.block_sb = blk->sb;
            a.block_lda = (int)blk->lds_a;
            a.block_ldb = (int)blk->lds_b;
            a.block_stride_sb = blk->stride_sb;
            f = L.tile == TILE_256x256_DTL ? grouped_block_fn_256x256dtl_e4m3(bk, out, epi) : nullptr;
        } else {
            f = grouped_fn(L.tile, bk, in, out, epi);
        }
        if (!f) {
            set_error("grouped_gemm_run: kernel missing for the planned variant");
            return MGEMM_ERR_UNSUPPORTED;
        }
        if (mgemm_status_t st = hip_status(f(a, L.grid, s), "grouped_gemm_run launch"))
            return st;
    }
    return MGEMM_OK;
}

static mgemm_status_t moe_fused(const char *name, mgemm_plan_t plan, const void *X, int64_t x_rows,
                                const int32_t *d_row_index, const void *W1, const void *W2, void *H, void *Y,
                                const int32_t *d_row_offsets, const float *d_row_weight, void *workspace,
                                size_t workspace_bytes, mgemm_stream_t stream)
{
    if (!plan || plan->kind != PLAN_MOE) {
        set_error("%s: null or non-MoE plan", name);
        return MGEMM_ERR_INVALID_ARG;
    }
    const mgemm_moe_desc_t &d = plan->moe;
    if (plan->noop)
        return MGEMM_OK;
    if (!X || !W1 || !W2 || !H || !Y || !d_row_offsets) {
        set_error("%s: null pointer", name);
        return MGEMM_ERR_INVALID_ARG;
    }
    if (d_row_index && (x_rows < 0 || x_rows > INT32_MAX ||
                        (uint64_t)x_rows * (uint64_t)d.lda * 2u > (uint64_t)kMaxRecords)) {
        set_error("%s: x_rows=%lld out of range (x_rows * lda * 2 must be < 2^31)", name, (long long)x_rows);
        return MGEMM_ERR_INVALID_ARG;
    }
    if (!aligned16(X) || !aligned16(W1) || !aligned16(W2) || !aligned16(Y) || ((uintptr_t)H & 127u)) {
        set_error("%s: X, W1, W2 and Y must be 16-byte aligned, H 128-byte aligned", name);
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (!workspace || workspace_bytes < plan->workspace_bytes || !aligned16(workspace)) {
        set_error("%s: needs a 16-byte aligned workspace of %zu bytes (got %zu at %p)", name,
                  plan->workspace_bytes, workspace_bytes, workspace);
        return MGEMM_ERR_WORKSPACE;
    }
    MoeArgs a;
    a.X = X;
    a.row_index = d_row_index;
    a.x_rows = d_row_index ? (int)x_rows : 0;
    a.W1 = W1;
    a.W2 = W2;
    a.H = H;
    a.Y = Y;
    a.row_weight = d_row_weight;
    a.offs = d_row_offsets;
    a.G = d.num_experts;
    a.hidden = (int)d.hidden;
    a.inter = (int)d.inter;
    a.max_rows = (int)d.max_total_rows;
    a.lda = (int)d.lda;
    a.ldw1 = (int)d.ldw1;
    a.ldw2 = (int)d.ldw2;
    a.ldh = (int)d.ldh;
    a.ldy = (int)d.ldy;
    a.stride_w1 = d.stride_w1;
    a.stride_w2 = d.stride_w2;
    a.ws = (char *)workspace;
    a.max_slots = (int)plan->moe_slots;
    // about four seconds of polling before an FC2 task gives up; with valid
    // offsets every count completes long before
    a.spin_limit = 1u << 22;
    return hip_status(launch_moe_fused(a, in_code(d.dtype), plan->grid, (hipStream_t)stream), name);
}

extern "C" mgemm_status_t moe_fused_run(mgemm_plan_t plan, const void *X, int64_t x_rows, const int32_t *d_row_index,
                                        const void *W1, const void *W2, void *H, void *Y,
                                        const int32_t *d_row_offsets, void *workspace, size_t workspace_bytes,
                                        mgemm_stream_t stream)
{
    return moe_fused("moe_fused_run", plan, X, x_rows, d_row_index, W1, W2, H, Y, d_row_offsets, nullptr, workspace,
                     workspace_bytes, stream);
}

extern "C" mgemm_status_t moe_fused_run_weighted(mgemm_plan_t plan, const void *X, int64_t x_rows,
                                                 const int32_t *d_row_index, const void *W1, const void *W2, void *H,
                                                 void *Y, const int32_t *d_row_offsets, const float *d_row_weight,
                                                 void *workspace, size_t workspace_bytes, mgemm_stream_t stream)
{
    if (!d_row_weight || ((uintptr_t)d_row_weight & 3)) {
        set_error("moe_fused_run_weighted: the row weights must be a non-null, 4-byte aligned device array");
        return MGEMM_ERR_INVALID_ARG;
    }
    return moe_fused("moe_fused_run_weighted", plan, X, x_rows, d_row_index, W1, W2, H, Y, d_row_offsets,
                     d_row_weight, workspace, workspace_bytes, stream);
}

extern "C" mgemm_status_t grouped_gemm_run(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                           const int32_t *d_row_offsets, void *workspace, size_t workspace_bytes,
                                           mgemm_stream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    return grouped_run(plan, A, B, D, d_row_offsets, nullptr, 0, stream);
}

extern "C" mgemm_status_t grouped_gemm_run_gather(mgemm_plan_t plan, const void *X, int64_t x_rows, const void *B,
                                                  void *D, const int32_t *d_row_offsets,
                                                  const int32_t *d_row_index, void *workspace,
                                                  size_t workspace_bytes, mgemm_stream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (!d_row_index) {
        set_error("grouped_gemm_run_gather: null row index");
        return MGEMM_ERR_INVALID_ARG;
    }
    return grouped_run(plan, X, B, D, d_row_offsets, d_row_index, x_rows, stream);
}

extern "C" mgemm_status_t grouped_gemm_run_weighted(mgemm_plan_t plan, const void *A, int64_t x_rows, const void *B,
                                                    void *D, const int32_t *d_row_offsets,
                                                    const int32_t *d_row_index, const float *d_row_weight,
                                                    void *workspace, size_t workspace_bytes, mgemm_stream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (!plan || plan->kind != PLAN_GROUPED) {
        set_error("grouped_gemm_run_weighted: null or non-grouped plan");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (plan->grouped.epilogue != MGEMM_EPI_SILU_GATE_I8) {
        set_error("grouped_gemm_run_weighted: the row weights scale the SiLU-gate epilogue; the plan has none");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (!d_row_weight || ((uintptr_t)d_row_weight & 3)) {
        set_error("grouped_gemm_run_weighted: the row weights must be a non-null, 4-byte aligned device array");
        return MGEMM_ERR_INVALID_ARG;
    }
    return grouped_run(plan, A, B, D, d_row_offsets, d_row_index, d_row_index ? x_rows : 0, stream, nullptr,
                       nullptr, d_row_weight);
}

extern "C" mgemm_status_t grouped_gemm_run_scaled(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                                  const int32_t *d_row_offsets, const float *d_scale_a,
                                                  const float *d_scale_b, void *workspace, size_t workspace_bytes,
                                                  mgemm_stream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (!plan || plan->kind != PLAN_GROUPED) {
        set_error("grouped_gemm_run_scaled: null or non-grouped plan");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (plan->grouped.a_type != MGEMM_E4M3) {
        set_error("grouped_gemm_run_scaled: the plan's inputs are not E4M3");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (!d_scale_a || !d_scale_b || ((uintptr_t)d_scale_a & 3) || ((uintptr_t)d_scale_b & 3)) {
        set_error("grouped_gemm_run_scaled: scale pointers must be non-null and 4-byte aligned");
        return MGEMM_ERR_INVALID_ARG;
    }
    return grouped_run(plan, A, B, D, d_row_offsets, nullptr, 0, stream, d_scale_a, d_scale_b);
}

extern "C" mgemm_status_t grouped_gemm_run_blockscaled(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                                       const int32_t *d_row_offsets, const uint8_t *d_scale_a,
                                                       int64_t lds_a, const uint8_t *d_scale_b, int64_t lds_b,
                                                       int64_t stride_sb, void *workspace, size_t workspace_bytes,
                                                       mgemm_stream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (!plan || plan->kind != PLAN_GROUPED) {
        set_error("grouped_gemm_run_blockscaled: null or non-grouped plan");
        return MGEMM_ERR_INVALID_ARG;
    }
    const mgemm_grouped_desc_t &d = plan->grouped;
    if (d.a_type != MGEMM_E4M3) {
        set_error("grouped_gemm_run_blockscaled: the plan's inputs are not E4M3");
        return MGEMM_ERR_UNSUPPORTED;
    }
    const int64_t kb = (d.K + 127) / 128, nb = (d.N + 127) / 128;
    if (!d_scale_a || !d_scale_b || lds_a < kb || lds_b < kb || lds_a < 1 || lds_b < 1 || stride_sb < nb * lds_b) {
        set_error("grouped_gemm_run_blockscaled: scale pointers must be non-null, lds_a, lds_b >= ceil(K / 128) "
                  "(= %lld) and stride_sb >= ceil(N / 128) * lds_b (= %lld)", (long long)kb, (long long)(nb * lds_b));
        return MGEMM_ERR_INVALID_ARG;
    }
    if ((lds_a | lds_b) & 1) {
        set_error("grouped_gemm_run_blockscaled: lds_a and lds_b must be even (two k blocks' scales are read at once)");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if ((uint64_t)d.max_total_rows * (uint64_t)lds_a > (uint64_t)kMaxRecords ||
        (uint64_t)d.num_groups * (uint64_t)stride_sb > (uint64_t)kMaxRecords) {
        set_error("grouped_gemm_run_blockscaled: each scale array must span less than 2^31 bytes");
        return MGEMM_ERR_INVALID_ARG;
    }
    GroupedBlockScales blk;
    blk.sa = d_scale_a;
    blk.sb = d_scale_b;
    blk.lds_a = lds_a;
    blk.lds_b = lds_b;
    blk.stride_sb = stride_sb;
    return grouped_run(plan, A, B, D, d_row_offsets, nullptr, 0, stream, nullptr, nullptr, nullptr, &blk);
}

extern "C" mgemm_status_t mgemm_moe_combine(const void *Z, int64_t z_rows, int64_t ldz, const int32_t *d_pos,
                                            const float *d_weights, void *Y, int64_t ldy, int64_t T, int32_t top_k,
                                            int64_t H, mgemm_dtype_t dtype, mgemm_stream_t stream)
{
    if (T < 0 || H < 0 || z_rows < 0 || top_k < 1 || top_k > 256 || T > INT32_MAX) {
        set_error("mgemm_moe_combine: bad sizes (T=%lld H=%lld z_rows=%lld top_k=%d)", (long long)T, (long long)H,
                  (long long)z_rows, top_k);
        return MGEMM_ERR_INVALID_ARG;
    }
    if (dtype != MGEMM_BF16 && dtype != MGEMM_F16) {
        set_error("mgemm_moe_combine: dtype must be BF16 or F16");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (T == 0 || H == 0)
        return MGEMM_OK;
    if (ldz < H || ldy < H) {
        set_error("mgemm_moe_combine: ldz=%lld and ldy=%lld must be >= H=%lld", (long long)ldz, (long long)ldy,
                  (long long)H);
        return MGEMM_ERR_INVALID_ARG;
    }
    if (!Z || !Y || !d_pos) {
        set_error("mgemm_moe_combine: null pointer");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (H % 8 || ldz % 8 || ldy % 8 || !aligned16(Z) || !aligned16(Y)) {
        set_error("mgemm_moe_combine: H, ldz, ldy must be multiples of 8 and Z, Y 16-byte aligned");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if ((uint64_t)z_rows * (uint64_t)ldz * 2u > (uint64_t)kMaxRecords) {
        set_error("mgemm_moe_combine: Z spans more than %u bytes", kMaxRecords);
        return MGEMM_ERR_UNSUPPORTED;
    }
    const int out = dtype == MGEMM_BF16 ? OUT_BF16 : OUT_F16;
    return hip_status(launch_moe_combine(Z, z_rows, ldz, d_pos, d_weights, Y, ldy, T, top_k, H, out,
                                         (hipStream_t)stream),
                      "mgemm_moe_combine launch");
}

extern "C" mgemm_status_t mgemm_quantize_e4m3_block(const void *X, int64_t rows, int64_t cols, int64_t ldx,
                                                    mgemm_dtype_t x_type, uint8_t *Q, int64_t ldq, uint8_t *S,
                                                    int64_t lds, mgemm_stream_t stream)
{
    if (rows < 0 || cols < 0 || rows > INT32_MAX || cols > INT32_MAX) {
        set_error("mgemm_quantize_e4m3_block: bad sizes (rows=%lld cols=%lld)", (long long)rows, (long long)cols);
        return MGEMM_ERR_INVALID_ARG;
    }
    if (x_type != MGEMM_BF16 && x_type != MGEMM_F16) {
        set_error("mgemm_quantize_e4m3_block: x_type must be BF16 or F16");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (rows == 0 || cols == 0)
        return MGEMM_OK;
    const int64_t nblk = (cols + 127) / 128;
    if (!X || !Q || !S || ldx < cols || ldq < cols || lds < nblk) {
        set_error("mgemm_quantize_e4m3_block: null pointer, or ldx=%lld / ldq=%lld below cols=%lld, or lds=%lld "
                  "below ceil(cols / 128)=%lld", (long long)ldx, (long long)ldq, (long long)cols, (long long)lds,
                  (long long)nblk);
        return MGEMM_ERR_INVALID_ARG;
    }
    if ((cols | ldx | ldq) & 1 || ((uintptr_t)X & 3) || ((uintptr_t)Q & 1)) {
        set_error("mgemm_quantize_e4m3_block: cols, ldx and ldq must be even, X 4-byte and Q 2-byte aligned");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if ((rows * nblk + 3) / 4 > (int64_t)UINT32_MAX / 2) {
        set_error("mgemm_quantize_e4m3_block: too many blocks");
        return MGEMM_ERR_UNSUPPORTED;
    }
    return hip_status(launch_quantize_e4m3_block(X, rows, cols, ldx, in_code(x_type), Q, ldq, S, lds,
                                                 (hipStream_t)stream),
                      "mgemm_quantize_e4m3_block launch");
}

extern "C" const char *gemm_status_string(mgemm_status_t s)
{
    switch (s) {
    case MGEMM_OK: return "MGEMM_OK";
    case MGEMM_ERR_INVALID_ARG: return "MGEMM_ERR_INVALID_ARG";
    case MGEMM_ERR_UNSUPPORTED: return "MGEMM_ERR_UNSUPPORTED";
    case MGEMM_ERR_WORKSPACE: return "MGEMM_ERR_WORKSPACE";
    case MGEMM_ERR_NO_MEMORY: return "MGEMM_ERR_NO_MEMORY";
    case MGEMM_ERR_HIP: return "MGEMM_ERR_HIP";
    default: return "MGEMM_ERR_UNKNOWN";
    }
}

extern "C" const char *gemm_last_error_message(void) { return g_err; }

extern "C" const char *mgemm_version(void) { return "mgemm 0.1 gfx950"; }
