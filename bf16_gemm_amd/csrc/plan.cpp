// plan.cpp -- validation, variant choice and launch geometry (host only).
//
// A plan is made once per problem shape and reused: it fixes the macro-tile,
// the number of workgroups, the L2 group size and, for the grouped form, the
// token-count buckets and the tile each bucket runs with.  Nothing here
// touches device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "internal.hpp"

namespace mgemm {

void set_error(const char *fmt, ...);

// eff: relative MFMA efficiency the cost model assumes for the shape.
static const TileShape kTiles[NUM_TILES] = {
    /* 256x256    */ {256, 256, 2, 2, 2 * (256 + 256) * 128, 1, 1.00, false, false},
    /* 128x128    */ {128, 128, 2, 2, 2 * (128 + 128) * 128, 2, 0.80, false, false},
    /* 32x256     */ {32, 256, 1, 4, 2 * (32 + 256) * 128, 2, 0.55, true, false},
    /* 64x256     */ {64, 256, 1, 4, 2 * (64 + 256) * 128, 1, 0.70, true, false},
    /* 256x256dtl */ {256, 256, 2, 4, (3 + 2) * 256 * 128, 1, 1.00, false, true},
    /* narrow     */ {128, 128, 1, 4, 5 * (128 * 128 + 64 * 256), 1, 0.50, true, true},
    /* narrow64   */ {128, 64, 1, 4, 6 * (128 * 128 + 64 * 128), 1, 0.50, true, true},
    /* narrow32   */ {128, 32, 1, 2, 7 * (128 * 128 + 64 * 64), 1, 0.50, true, true},
};

const TileShape &tile_shape(int tile) { return kTiles[tile]; }

// LDS of one CU on gfx950.
constexpr int64_t kLdsPerCu = 160 * 1024;

// Bytes of one operand's ring: `slots` stages of rows x bk elements.  The
// stage budget of "B200 的 2CTA 怎样调优" (section 三, the tile calculator:
// stages x (BM x BK + BK x BN) x element bytes) is this for A plus this for
// B with equal stage counts (mgemm_tile_budget); the planner applies it per
// operand, since the direct-to-LDS tile gives one operand a deeper ring.
static int64_t operand_ring_bytes(int64_t rows, int64_t bk, int64_t slots, int64_t elt)
{
    return slots * rows * bk * elt;
}

static int64_t ring_lds_bytes(const TileShape &t, int a_slots, int b_slots)
{
    return operand_ring_bytes(t.bm, kBK, a_slots, 2) + operand_ring_bytes(t.bn, kBK, b_slots, 2);
}

// The few-token tile's two rings for nv token blocks (1..8): token slots
// (a) and weight slots (b), as the kernel lays them out.
template <int BN>
static void narrow_rings(int nv, int &a_slots, int &b_slots)
{
    using T = NarrowTile<IN_BF16, false, BN>;
    switch (nv) {
#define MG_R(V)                                  \
    case V:                                      \
        a_slots = T::template Ring<V>::DA;       \
        b_slots = T::template Ring<V>::DB;       \
        break;
        MG_R(1) MG_R(2) MG_R(3) MG_R(4) MG_R(5) MG_R(6) MG_R(7)
    default:
        a_slots = T::template Ring<8>::DA;
        b_slots = T::template Ring<8>::DB;
        break;
#undef MG_R
    }
}

// Wave layout and ring depths of a dense plan's tile: the direct-to-LDS
// tile runs dense plans on four waves of 128 x 128 (the tile table's 2x4 is
// its grouped launches' layout), with the 3-slot ring on B when B is
// column-major, else on A; the few-token tiles' rings (tokens as a, weights
// as b) depend on the token count.
static void dense_waves(int tile, bool bk, int &wm, int &wn, int &a_slots, int &b_slots, int64_t tokens = 128)
{
    const TileShape &ts = tile_shape(tile);
    wm = ts.wm;
    wn = ts.wn;
    a_slots = b_slots = 2;
    if (tile == TILE_256x256_DTL) {
        wn = 2;
        a_slots = bk ? 2 : 3;
        b_slots = bk ? 3 : 2;
    }
    const int nv = (int)std::min<int64_t>(std::max<int64_t>((tokens + 15) / 16, 1), 8);
    if (tile == TILE_NARROW)
        narrow_rings<128>(nv, a_slots, b_slots);
    if (tile == TILE_NARROW64)
        narrow_rings<64>(nv, a_slots, b_slots);
    if (tile == TILE_NARROW32)
        narrow_rings<32>(nv, a_slots, b_slots);
}

static const char *tile_name(int tile)
{
    static const char *n[NUM_TILES] = {"256x256", "128x128", "32x256", "64x256", "256x256dtl", "narrow128",
                                       "narrow64", "narrow32"};
    return n[tile];
}

DenseFn dense_fn(int tile, bool ak, bool bk, int in, int out)
{
    if (in == IN_E4M3)
        return tile == TILE_256x256_DTL ? dense_fn_256x256dtl_e4m3(ak, bk, out) : nullptr;
    const bool bf = in == IN_BF16;
    switch (tile) {
    case TILE_256x256: return bf ? dense_fn_256x256_bf16(ak, bk, out) : dense_fn_256x256_f16(ak, bk, out);
    case TILE_128x128: return bf ? dense_fn_128x128_bf16(ak, bk, out) : dense_fn_128x128_f16(ak, bk, out);
    case TILE_32x256: return bf ? dense_fn_32x256_bf16(ak, bk, out) : dense_fn_32x256_f16(ak, bk, out);
    case TILE_64x256: return bf ? dense_fn_64x256_bf16(ak, bk, out) : dense_fn_64x256_f16(ak, bk, out);
    case TILE_256x256_DTL: return bf ? dense_fn_256x256dtl_bf16(ak, bk, out) : dense_fn_256x256dtl_f16(ak, bk, out);
    case TILE_NARROW: return bf ? dense_fn_narrow128_bf16(ak, bk, out) : dense_fn_narrow128_f16(ak, bk, out);
    case TILE_NARROW64: return bf ? dense_fn_narrow64_bf16(ak, bk, out) : dense_fn_narrow64_f16(ak, bk, out);
    case TILE_NARROW32: return bf ? dense_fn_narrow32_bf16(ak, bk, out) : dense_fn_narrow32_f16(ak, bk, out);
    default: return nullptr;
    }
}

GroupedFn grouped_fn(int tile, bool bk, int in, int out, int epi)
{
    if (in == IN_E4M3)
        return tile == TILE_256x256_DTL ? grouped_fn_256x256dtl_e4m3(bk, out, epi) : nullptr;
    const bool bf = in == IN_BF16;
    switch (tile) {
    case TILE_256x256: return bf ? grouped_fn_256x256_bf16(bk, out, epi) : grouped_fn_256x256_f16(bk, out, epi);
    case TILE_128x128: return bf ? grouped_fn_128x128_bf16(bk, out, epi) : grouped_fn_128x128_f16(bk, out, epi);
    case TILE_32x256: return bf ? grouped_fn_32x256_bf16(bk, out, epi) : grouped_fn_32x256_f16(bk, out, epi);
    case TILE_64x256: return bf ? grouped_fn_64x256_bf16(bk, out, epi) : grouped_fn_64x256_f16(bk, out, epi);
    case TILE_256x256_DTL:
        return bf ? grouped_fn_256x256dtl_bf16(bk, out, epi) : grouped_fn_256x256dtl_f16(bk, out, epi);
    case TILE_NARROW: return bf ? grouped_fn_narrow128_bf16(bk, out, epi) : grouped_fn_narrow128_f16(bk, out, epi);
    case TILE_NARROW64: return bf ? grouped_fn_narrow64_bf16(bk, out, epi) : grouped_fn_narrow64_f16(bk, out, epi);
    case TILE_NARROW32: return bf ? grouped_fn_narrow32_bf16(bk, out, epi) : grouped_fn_narrow32_f16(bk, out, epi);
    default: return nullptr;
    }
}

int in_code(mgemm_dtype_t t) { return t == MGEMM_BF16 ? IN_BF16 : (t == MGEMM_E4M3 ? IN_E4M3 : IN_F16); }
int out_code(mgemm_dtype_t t) { return t == MGEMM_F32 ? OUT_F32 : (t == MGEMM_BF16 ? OUT_BF16 : OUT_F16); }
int dtype_size(mgemm_dtype_t t) { return t == MGEMM_F32 ? 4 : 2; }

// Compute units of the current device; a 256-CU gfx950 when none is visible
// (plans can then still be made and inspected on a host without a GPU).
static int device_cus()
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 256;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Cost model for one tile choice, in CU clocks: the busiest CU runs
// ceil(tiles / CUs) tiles, each bound by its MFMA work at the shape's
// efficiency or by the operand bytes it stages (about 64 B per clock per CU
// from L2), whichever is larger.
// sk: the tile can balance a partial last round with stream-K (then the
// busiest CU runs tiles / CUs tiles, plus a tenth of one for the fixup).
static double tile_cost(const TileShape &t, int64_t M, int64_t N, int64_t K, int cus, bool sk = false)
{
    const int64_t tiles = cdiv(M, t.bm) * cdiv(N, t.bn);
    const int64_t rem = tiles % cus;
    double per_cu = (double)cdiv(tiles, cus);
    if (sk && tiles > cus && rem > 0 && rem * 2 <= cus && cdiv(K, kBK) >= 48)
        per_cu = (double)tiles / cus + 0.1;
    const double flops = 2.0 * t.bm * t.bn * (double)std::max<int64_t>(K, 64);
    const double mfma_clk = flops / (4096.0 * t.eff);
    const double load_clk = (double)(t.bm + t.bn) * 2.0 * (double)std::max<int64_t>(K, 64) / 64.0;
    return per_cu * std::max(mfma_clk, load_clk);
}

// Time model (microseconds) for the split-K decision, fitted to measured
// small-M runs on MI355X: a task (one K range of one output tile) streams
// its operand rows at about 24 B per clock per CU (2.1 GHz) plus ~2.5 us of
// prologue and epilogue; the busiest CU runs ceil(tasks / CUs) tasks.  A
// split adds a second launch (~3 us) and its fp32 partials, written once and
// read once at ~4 TB/s.
static double task_model_us(const TileShape &t, int64_t M, int64_t N, int64_t K, int splits, int cus)
{
    const int64_t tasks = cdiv(M, t.bm) * cdiv(N, t.bn) * splits;
    const double per_cu = (double)cdiv(tasks, cus);
    const double kr = (double)std::max<int64_t>(cdiv(K, splits), 64);
    const double rows = (double)(std::min<int64_t>(t.bm, M) + std::min<int64_t>(t.bn, N));
    double us = per_cu * (rows * 2.0 * kr / (24.0 * 2100.0) + 2.5);
    if (splits > 1)
        us += 3.0 + 2.0 * (double)splits * (double)M * (double)N * 4.0 / 4.0e6;
    return us;
}

// Time model (microseconds) of a few-token plan: width `bn`, `splits` K
// ranges.  Fitted to MI355X runs of the tile on decode-sized products
// (16-128 tokens, N 2048-7168, K 2048-7168, every width and split that fits
// one round): ~2.5 us until the first K step's operands have landed, then
// each task streams its token rows and weight columns at ~55 GB/s per CU;
// a split adds its partial tiles moved at the same rate (every range writes
// one, the last reads the others).  With more than three quarters of the
// CUs streaming the per-task rate falls (the fit charges 2 us per further
// quarter).  Tasks beyond one per CU run in further rounds.  Over the
// fitted shapes the pick is within 7 % of the fastest width and split
// (2 % on average).
static double narrow_model_us(int64_t M, int64_t N, int64_t K, int bn, int splits, int cus)
{
    const double rate = 55e3;   // bytes per microsecond per CU
    const int64_t tokens = std::min<int64_t>(mgemm_round_tokens(std::min<int64_t>(M, 128), 16), 128);
    const int64_t tiles = cdiv(M, 128) * cdiv(N, bn);
    const int64_t tasks = tiles * splits;
    const double kr = (double)cdiv(K, splits);
    const double task_bytes = kr * 2.0 * (double)(tokens + bn);
    double us = 2.5 + (double)cdiv(tasks, cus) * task_bytes / rate;
    if (splits > 1)
        us += (double)splits * (double)(tokens * bn * 4) / rate;
    const int64_t busy = std::min<int64_t>(tasks, cus) - 3 * (int64_t)cus / 4;
    if (busy > 0)
        us += 2.0 * (double)busy / ((double)cus / 4.0);
    return us;
}

static bool is_in_type(mgemm_dtype_t t) { return t == MGEMM_F16 || t == MGEMM_BF16 || t == MGEMM_E4M3; }
static const char *in_name(mgemm_dtype_t t) { return t == MGEMM_BF16 ? "bf16" : (t == MGEMM_E4M3 ? "e4m3" : "f16"); }
static bool is_out_type(mgemm_dtype_t t) { return t == MGEMM_F16 || t == MGEMM_BF16 || t == MGEMM_F32; }
static bool is_layout(mgemm_layout_t l) { return l == MGEMM_ROW_MAJOR || l == MGEMM_COL_MAJOR; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxLd = (int64_t)1 << 20;

static mgemm_status_t check_types(mgemm_dtype_t a, mgemm_dtype_t b, mgemm_dtype_t d)
{
    if (!is_in_type(a) || !is_in_type(b) || !is_out_type(d)) {
        set_error("invalid dtype codes (a=%d b=%d d=%d)", (int)a, (int)b, (int)d);
        return MGEMM_ERR_INVALID_ARG;
    }
    if (a != b) {
        set_error("a_type and b_type must match");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (d != MGEMM_F32 && d != a && a != MGEMM_E4M3) {
        set_error("d_type must be F32 or the input type");
        return MGEMM_ERR_UNSUPPORTED;
    }
    return MGEMM_OK;
}

static int forced_tile(uint32_t flags)
{
    if (flags & MGEMM_PLAN_FORCE_TILE_256x256) return TILE_256x256;
    if (flags & MGEMM_PLAN_FORCE_TILE_128x128) return TILE_128x128;
    if (flags & MGEMM_PLAN_FORCE_TILE_32x256) return TILE_32x256;
    if (flags & MGEMM_PLAN_FORCE_TILE_64x256) return TILE_64x256;
    if (flags & MGEMM_PLAN_FORCE_TILE_256x256_DTL) return TILE_256x256_DTL;
    if (flags & MGEMM_PLAN_FORCE_TILE_NARROW) return TILE_NARROW;
    if (flags & MGEMM_PLAN_FORCE_TILE_NARROW64) return TILE_NARROW64;
    if (flags & MGEMM_PLAN_FORCE_TILE_NARROW32) return TILE_NARROW32;
    return -1;
}

// Tile rows per L2 group.  Tiles are issued m fastest inside groups of
// group_m tile rows, and with the XCD remap each XCD takes a run of
// consecutive tiles, so the tiles one XCD runs at once (its CUs times the
// workgroups per CU) form a group_m x group_n block sharing its L2.  Of the
// power-of-two shapes the one whose operand rows and columns --
// mgemm_group_working_set, the super-tile working set of "GEMM优化（三）"
// section 3.4 -- are fewest is taken, the one with fewer rows on a tie: 4 x 8
// for the 256 x 256 tile on 32 CUs, which measured fastest at 8192^3 (2, 8,
// 16 and 32 rows were 3-20 % slower).
static int pick_group_m(const TileShape &t, int64_t tiles_m, int cus, int occ, int64_t K)
{
    const int conc = std::max(1, cus / 8 * occ);
    int best = 1;
    int64_t best_ws = INT64_MAX;
    for (int gm = 1; gm <= conc && gm <= tiles_m; gm *= 2) {
        const int gn = (conc + gm - 1) / gm;
        const int64_t ws = mgemm_group_working_set(gm, gn, t.bm, t.bn, std::max<int64_t>(K, 1), 2);
        if (ws < best_ws) {
            best_ws = ws;
            best = gm;
        }
    }
    return best;
}

static mgemm_status_t plan_dense(const mgemm_desc_t *d, uint32_t flags, mgemm_plan *p)
{
    if (d->M < 0 || d->N < 0 || d->K < 0 || d->M >= kMaxDim || d->N >= kMaxDim || d->K >= kMaxDim) {
        set_error("M, N, K must lie in [0, 2^30): got %lld %lld %lld", (long long)d->M, (long long)d->N,
                  (long long)d->K);
        return MGEMM_ERR_INVALID_ARG;
    }
    if (mgemm_status_t s = check_types(d->a_type, d->b_type, d->d_type))
        return s;
    if (!is_layout(d->a_layout) || !is_layout(d->b_layout)) {
        set_error("invalid layout code");
        return MGEMM_ERR_INVALID_ARG;
    }
    const int64_t need_lda = d->a_layout == MGEMM_ROW_MAJOR ? d->K : d->M;
    const int64_t need_ldb = d->b_layout == MGEMM_ROW_MAJOR ? d->N : d->K;
    if (d->lda < std::max<int64_t>(need_lda, 1) || d->ldb < std::max<int64_t>(need_ldb, 1) ||
        d->ldd < std::max<int64_t>(d->N, 1)) {
        set_error("leading dimension too small (lda=%lld need %lld, ldb=%lld need %lld, ldd=%lld need %lld)",
                  (long long)d->lda, (long long)need_lda, (long long)d->ldb, (long long)need_ldb,
                  (long long)d->ldd, (long long)d->N);
        return MGEMM_ERR_INVALID_ARG;
    }
    if (d->K % 8) {
        set_error("K must be a multiple of 8 (got %lld)", (long long)d->K);
        return MGEMM_ERR_UNSUPPORTED;
    }
    const bool e4m3 = d->a_type == MGEMM_E4M3;
    if (e4m3) {
        // one kernel: k-contiguous A and B, 16-byte rows, whole tile columns
        // of four, no split of K
        const int fs = (int)((flags >> 16) & 0xFF);
        const int ft = forced_tile(flags);
        if (d->a_layout != MGEMM_ROW_MAJOR || d->b_layout != MGEMM_COL_MAJOR || d->K % 16 || d->lda % 16 ||
            d->ldb % 16 || d->N % 4 || fs > 1 || (ft >= 0 && ft != TILE_256x256_DTL)) {
            set_error("E4M3 plans need row-major A, column-major B, K, lda, ldb multiples of 16, N a multiple "
                      "of 4, no split of K and no tile but the 256x256 direct-to-LDS one");
            return MGEMM_ERR_UNSUPPORTED;
        }
    }
    const int esz = dtype_size(d->d_type);
    if (d->lda % 8 || d->ldb % 8 || (d->ldd * esz) % 16) {
        set_error("leading dimensions must give 16-byte aligned rows (lda, ldb multiples of 8; ldd*%d %% 16 == 0)",
                  esz);
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (d->lda > kMaxLd || d->ldb > kMaxLd || d->ldd > kMaxLd) {
        set_error("leading dimensions above 2^20 elements are not supported");
        return MGEMM_ERR_UNSUPPORTED;
    }
    p->kind = PLAN_DENSE;
    p->dense = *d;
    p->flags = flags;
    p->num_cus = device_cus();
    p->noop = d->M == 0 || d->N == 0;
    p->zero_fill = !p->noop && d->K == 0;
    const bool ak = d->a_layout == MGEMM_ROW_MAJOR;
    const bool bk = d->b_layout == MGEMM_COL_MAJOR;
    const int in = in_code(d->a_type), out = out_code(d->d_type);

    int tile = e4m3 ? TILE_256x256_DTL : forced_tile(flags);
    if (tile >= 0) {
        if (!dense_fn(tile, ak, bk, in, out)) {
            set_error("forced tile %s is not compiled for this layout/dtype", tile_name(tile));
            return MGEMM_ERR_UNSUPPORTED;
        }
    } else {
        double best = 0;
        for (int t = 0; t < NUM_TILES; ++t) {
            if (kTiles[t].forced_only || !dense_fn(t, ak, bk, in, out))
                continue;
            int cw, cn, ca, cb;
            dense_waves(t, bk, cw, cn, ca, cb);
            if (ring_lds_bytes(kTiles[t], ca, cb) > kLdsPerCu)
                continue;   // its ring does not fit a CU's LDS
            // the 256 x 256 tile runs on the direct-to-LDS engine where it can (stream-K tails included)
            const bool sk = t == TILE_256x256 && !e4m3 && (flags >> 16 & 0xFF) == 0 &&
                            dense_fn(TILE_256x256_DTL, ak, bk, in, out) != nullptr;
            const double c = tile_cost(kTiles[t], d->M, d->N & ~(int64_t)3, d->K, p->num_cus, sk);
            if (tile < 0 || c < best * 0.999) {
                best = c;
                tile = t;
            }
        }
    }
    if (tile < 0) {
        set_error("no kernel compiled for this layout/dtype combination");
        return MGEMM_ERR_UNSUPPORTED;
    }
    // Few tokens (M up to one narrow tile): the tokens go on the MFMA's narrow
    // side and the tile computes only their 16-row blocks ("MegaMoE", Blackwell
    // section 04: dynamic N = valid tokens rounded up to 16).
    const int64_t n_main_all = d->N & ~(int64_t)3;
    const bool narrow_rule = !e4m3 && forced_tile(flags) < 0 && d->M <= kTiles[TILE_NARROW].bm && n_main_all > 0 &&
                             dense_fn(TILE_NARROW, ak, bk, in, out) != nullptr;
    int narrow_splits = 0;
    if (narrow_rule) {
        // width and K split by the time model: 128 or 64 columns (32 is
        // left to the FORCE flag: two waves, measured slower), every split
        // count whose tasks fit one round of CUs
        const int64_t ks = std::max<int64_t>(cdiv(d->K, kBK), 1);
        double best = 0;
        for (int t : {TILE_NARROW, TILE_NARROW64}) {
            if (!dense_fn(t, ak, bk, in, out))
                continue;
            const int64_t tl = cdiv(d->M, 128) * cdiv(n_main_all, kTiles[t].bn);
            for (int sp = 1; sp <= 16; ++sp) {
                if (sp > 1 && (tl * sp > p->num_cus || cdiv(ks, sp) < 2))
                    break;
                const double c = narrow_model_us(d->M, n_main_all, d->K, kTiles[t].bn, sp, p->num_cus);
                if (narrow_splits == 0 || c < best) {
                    best = c;
                    tile = t;
                    narrow_splits = sp;
                }
            }
        }
    }
    // the 256 x 256 tile with both operands k-contiguous runs on the
    // direct-to-LDS engine (eight waves, no staging registers)
    if (tile == TILE_256x256 && forced_tile(flags) < 0 && dense_fn(TILE_256x256_DTL, ak, bk, in, out))
        tile = TILE_256x256_DTL;
    const int64_t n_main = d->N & ~(int64_t)3;
    const int64_t ksteps = cdiv(d->K, kBK);
    const int forced_splits = (int)((flags >> 16) & 0xFF);
    if (forced_splits > 64) {
        set_error("split count must lie in [1, 64] (got %d)", forced_splits);
        return MGEMM_ERR_INVALID_ARG;
    }
    int splits = 1;
    if (forced_splits > 0) {
        splits = (int)std::min<int64_t>(forced_splits, std::max<int64_t>(ksteps, 1));
    } else if (narrow_splits > 0) {
        splits = narrow_splits;   // the time model's choice (each range streams its own part of the weights)
    } else if (is_narrow(tile)) {
        // forced width: split K so that the tasks fill the CUs; the last
        // range of a tile adds the others' partials in the same launch
        const int64_t tl = cdiv(d->M, kTiles[tile].bm) * cdiv(n_main, kTiles[tile].bn);
        if (tl * 2 <= p->num_cus && ksteps >= 8)
            splits = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)p->num_cus / tl, ksteps / 4, 16}));
    } else if (!e4m3 && forced_tile(flags) < 0 && n_main > 0 && d->M > 0) {
        // Split K when the chosen tiles leave most compute units idle: the
        // tile and range count with the lowest modelled time wins if it beats
        // the unsplit plan by 10 %.
        const int64_t tl0 = cdiv(d->M, kTiles[tile].bm) * cdiv(n_main, kTiles[tile].bn);
        if (tl0 * 2 <= p->num_cus && ksteps >= 8) {
            double best = 0.9 * task_model_us(kTiles[tile], d->M, n_main, d->K, 1, p->num_cus);
            for (int t = 0; t < NUM_TILES; ++t) {
                if (kTiles[t].forced_only || !dense_fn(t, ak, bk, in, OUT_F32))
                    continue;
                const int64_t tl = cdiv(d->M, kTiles[t].bm) * cdiv(n_main, kTiles[t].bn);
                for (int sp = 2; sp <= 16; sp *= 2) {
                    const int64_t steps = cdiv(ksteps, sp);
                    if (steps < 4 || tl * sp > 2 * (int64_t)p->num_cus)
                        break;
                    const int real = (int)cdiv(ksteps, steps);
                    const double c = task_model_us(kTiles[t], d->M, n_main, d->K, real, p->num_cus);
                    if (c < best) {
                        best = c;
                        tile = t;
                        splits = real;
                    }
                }
            }
        }
    }
    const TileShape &ts = kTiles[tile];
    p->tile = tile;
    p->tiles_m = cdiv(d->M, ts.bm);
    p->tiles_n = cdiv(n_main, ts.bn);
    p->tiles = p->tiles_m * p->tiles_n;
    // Stream-K tail: the four-wave tile's last round of tiles leaves at most
    // half the CUs busy; cut those tiles into K ranges so every CU gets the
    // same K steps to within one range ("B200 的 2CTA 怎样调优", section 十:
    // uneven SM use, long tail).  Worth it when a tile is long enough that
    // the steps saved outweigh the fixup (partials written and read, ~3
    // device-scope round trips): 48 steps and more.
    p->sk_tiles = 0;
    const int64_t rem = p->tiles % p->num_cus;
    if (tile == TILE_256x256_DTL && !e4m3 && forced_splits == 0 && p->tiles > p->num_cus && rem > 0 &&
        rem * 2 <= p->num_cus && ksteps >= 48) {
        const int64_t sk = std::min<int64_t>({(int64_t)kSkMaxSplits, p->num_cus / rem, ksteps / 16});
        if (sk >= 2 && (in == IN_BF16 ? dense_sk_fn_256x256dtl_bf16(bk, out) : dense_sk_fn_256x256dtl_f16(bk, out))) {
            p->sk_tiles = (int)rem;
            splits = (int)sk;
        }
    }
    p->kchunk = (int)(cdiv(ksteps, splits) * kBK);
    p->splits = splits > 1 ? (int)cdiv(d->K, p->kchunk) : 1;
    if (p->splits > 1 && !dense_fn(tile, ak, bk, in, OUT_F32)) {
        set_error("split-K needs the fp32-output kernel of tile %s, which is not compiled", tile_name(tile));
        return MGEMM_ERR_UNSUPPORTED;
    }
    p->workspace_bytes = p->splits > 1 ? (size_t)p->splits * (size_t)d->M * (size_t)n_main * 4u : 0;
    p->slab_offset = 0;
    if (p->sk_tiles > 0) {
        // counters of the cut tiles, then one 256 x 256 fp32 partial per range
        p->slab_offset = narrow_counter_bytes(p->sk_tiles);
        p->workspace_bytes = (size_t)p->slab_offset + (size_t)p->sk_tiles * (size_t)p->splits * 256u * 256u * 4u;
    }
    if (is_narrow(tile) && p->splits > 1) {
        // counters, then one partial slab per (tile, range)
        p->slab_offset = narrow_counter_bytes(p->tiles);
        const int64_t slabs = (int64_t)p->tiles * p->splits * narrow_slab_bytes(ts.bn);
        if (slabs >= ((int64_t)1 << 31)) {
            set_error("the K split needs %lld bytes of partial tiles, more than the kernel addresses (2^31); use "
                      "fewer K ranges", (long long)slabs);
            return MGEMM_ERR_UNSUPPORTED;
        }
        p->workspace_bytes = (size_t)p->slab_offset + (size_t)slabs;
    }
    const int64_t tasks = p->sk_tiles > 0 ? p->tiles - p->sk_tiles + (int64_t)p->sk_tiles * p->splits
                                          : p->tiles * p->splits;
    int wm, wn, a_slots, b_slots;
    dense_waves(tile, bk, wm, wn, a_slots, b_slots, d->M);
    // the ring must fit the LDS, and as many workgroups per CU as the tile
    // assumes must fit beside each other, else fewer
    p->lds_bytes = ring_lds_bytes(ts, a_slots, b_slots);
    if (is_narrow(tile))   // the token slots hold the tile's token rows only
        p->lds_bytes = operand_ring_bytes(16 * std::min<int64_t>(cdiv(std::max<int64_t>(d->M, 1), 16), 8), kBK,
                                          a_slots, 2) +
                       operand_ring_bytes(ts.bn, kBK, b_slots, 2);
    if (p->lds_bytes > kLdsPerCu) {
        set_error("the %s tile's ring (%d + %d stages) needs %lld bytes of LDS, more than a CU's %lld",
                  tile_name(tile), a_slots, b_slots, (long long)p->lds_bytes, (long long)kLdsPerCu);
        return MGEMM_ERR_UNSUPPORTED;
    }
    const int occ = (int)std::min<int64_t>(ts.occupancy, kLdsPerCu / p->lds_bytes);
    const int64_t slots = (int64_t)p->num_cus * occ;
    p->grid = (int)std::max<int64_t>(1, std::min<int64_t>(tasks, slots));
    p->group_m = pick_group_m(ts, p->tiles_m, p->num_cus, occ, d->K);
    p->xcd_remap = (flags & MGEMM_PLAN_NO_XCD_REMAP) ? 0 : (p->grid % 8 == 0 ? 1 : 0);
    char stages[16];
    if (a_slots == b_slots)
        snprintf(stages, sizeof stages, "%d", a_slots);
    else
        snprintf(stages, sizeof stages, "%da/%db", a_slots, b_slots);
    char tokens[48] = "";
    if (is_narrow(tile))
        snprintf(tokens, sizeof tokens, " tokens=%lld",
                 (long long)mgemm_round_tokens(std::min<int64_t>(d->M, kTiles[TILE_NARROW].bm), 16));
    char sk_desc[64] = "";
    if (p->sk_tiles > 0)
        snprintf(sk_desc, sizeof sk_desc, " stream_k_tiles=%d", p->sk_tiles);
    char buf[384];
    snprintf(buf, sizeof buf,
             "dense M=%lld N=%lld K=%lld %s%s->%s tile=%s%s waves=%dx%d bk=%d stages=%s tiles=%lld splits=%d "
             "grid=%d group_m=%d xcd_remap=%d edge_cols=%lld%s",
             (long long)d->M, (long long)d->N, (long long)d->K, in_name(d->a_type),
             ak ? (bk ? " NT" : " NN") : (bk ? " TT" : " TN"),
             d->d_type == MGEMM_F32 ? "f32" : (d->d_type == MGEMM_BF16 ? "bf16" : "f16"), tile_name(tile), tokens, wm, wn,
             e4m3 ? 128 : 64, stages, (long long)p->tiles, p->splits, p->grid, p->group_m, p->xcd_remap, (long long)(d->N - n_main),
             sk_desc);
    p->description = buf;
    return MGEMM_OK;
}

static mgemm_status_t plan_grouped(const mgemm_grouped_desc_t *d, uint32_t flags, mgemm_plan *p)
{
    if (d->num_groups < 1 || d->num_groups > 256) {
        set_error("num_groups must lie in [1, 256] (got %d)", d->num_groups);
        return d->num_groups < 1 ? MGEMM_ERR_INVALID_ARG : MGEMM_ERR_UNSUPPORTED;
    }
    if (d->max_total_rows < 0 || d->N < 0 || d->K < 0 || d->max_total_rows >= kMaxDim || d->N >= kMaxDim ||
        d->K >= kMaxDim || d->stride_b < 0) {
        set_error("sizes must lie in [0, 2^30)");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (mgemm_status_t s = check_types(d->a_type, d->b_type, d->d_type))
        return s;
    if (!is_layout(d->b_layout) || (d->epilogue != MGEMM_EPI_NONE && d->epilogue != MGEMM_EPI_SILU_GATE_I8)) {
        set_error("invalid layout or epilogue code");
        return MGEMM_ERR_INVALID_ARG;
    }
    const bool silu = d->epilogue == MGEMM_EPI_SILU_GATE_I8;
    const int64_t out_cols = silu ? d->N / 2 : d->N;
    const int64_t need_ldb = d->b_layout == MGEMM_ROW_MAJOR ? d->N : d->K;
    if (d->lda < std::max<int64_t>(d->K, 1) || d->ldb < std::max<int64_t>(need_ldb, 1) ||
        d->ldd < std::max<int64_t>(out_cols, 1)) {
        set_error("leading dimension too small");
        return MGEMM_ERR_INVALID_ARG;
    }
    const int64_t wsize = d->b_layout == MGEMM_ROW_MAJOR ? (d->K > 0 ? (d->K - 1) * d->ldb + d->N : 0)
                                                          : (d->N > 0 ? (d->N - 1) * d->ldb + d->K : 0);
    if (d->num_groups > 1 && d->stride_b < wsize) {
        set_error("stride_b smaller than one expert's weight matrix");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (d->K % 8 || d->N % 4 || (silu && d->N % 16)) {
        set_error("grouped form needs K %% 8 == 0 and N %% 4 == 0 (N %% 16 == 0 with the SiLU gate)");
        return MGEMM_ERR_UNSUPPORTED;
    }
    const int esz = dtype_size(d->d_type);
    if (d->lda % 8 || d->ldb % 8 || (d->ldd * esz) % 16 || d->stride_b % 8) {
        set_error("leading dimensions / expert stride must give 16-byte aligned rows");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (d->lda > kMaxLd || d->ldb > kMaxLd || d->ldd > kMaxLd) {
        set_error("leading dimensions above 2^20 elements are not supported");
        return MGEMM_ERR_UNSUPPORTED;
    }
    const bool e4m3 = d->a_type == MGEMM_E4M3;
    if (e4m3 && (d->b_layout != MGEMM_COL_MAJOR || silu || d->K % 16 || d->lda % 16 || d->ldb % 16 ||
                 d->stride_b % 16 || (forced_tile(flags) >= 0 && forced_tile(flags) != TILE_256x256_DTL))) {
        set_error("grouped E4M3 plans need column-major expert weights, no epilogue, K, lda, ldb and stride_b "
                  "multiples of 16, and no tile but the 256x256 direct-to-LDS one");
        return MGEMM_ERR_UNSUPPORTED;
    }
    p->kind = PLAN_GROUPED;
    p->grouped = *d;
    p->flags = flags;
    p->num_cus = device_cus();
    p->noop = d->max_total_rows == 0 || d->N == 0;
    p->zero_fill = !p->noop && d->K == 0;
    const bool bk = d->b_layout == MGEMM_COL_MAJOR;
    const int in = in_code(d->a_type), out = out_code(d->d_type), epi = silu ? EPI_SILU_GATE : EPI_NONE;

    // Token-count buckets, each with its own launch: experts with few rows
    // take the narrow-M tile so that the padding stays small (MegaMoE,
    // Blackwell section 04 and Hopper section 03: put the few tokens on the
    // narrow tile dimension and size it to the token count), large experts
    // take the full macro-tile.  One narrow bucket up to 128 rows rather
    // than one per row class: each launch runs alone on the stream, and the
    // small classes alone (64-192 tasks) leave most CUs idle while their
    // weights stream; merged they fill the chip (measured on the 64-expert
    // layer: 3.32 ms against 3.61 ms with 32/64/128-row classes; boundaries
    // at 97 or 193 rows and a third 128x128 class were slower).
    struct B { int tile, lo, hi; };
    B buckets[2] = {{TILE_NARROW, 1, 129}, {TILE_256x256_DTL, 129, 1 << 30}};
    int nb = 2;
    const int ft = e4m3 ? TILE_256x256_DTL : forced_tile(flags);
    if (ft >= 0) {
        buckets[0] = {ft, 1, 1 << 30};
        nb = 1;
    }
    p->launches.clear();
    std::string desc;
    char buf[256];
    snprintf(buf, sizeof buf, "grouped G=%d rows<=%lld N=%lld K=%lld %s%s->%s epi=%s", d->num_groups,
             (long long)d->max_total_rows, (long long)d->N, (long long)d->K, in_name(d->a_type),
             bk ? " NT" : " NN", d->d_type == MGEMM_F32 ? "f32" : (d->d_type == MGEMM_BF16 ? "bf16" : "f16"),
             silu ? "silu_gate_i8" : "none");
    desc = buf;
    for (int i = 0; i < nb; ++i) {
        const TileShape &ts = kTiles[buckets[i].tile];
        if (!grouped_fn(buckets[i].tile, bk, in, out, epi)) {
            set_error("grouped kernel %s not compiled for this layout/dtype", tile_name(buckets[i].tile));
            return MGEMM_ERR_UNSUPPORTED;
        }
        if (ts.bn % 32) {
            set_error("internal: grouped tile width must be a multiple of 32");
            return MGEMM_ERR_UNSUPPORTED;
        }
        // upper bound on this bucket's tasks
        const int64_t lo = buckets[i].lo;
        const int64_t experts = std::min<int64_t>(d->num_groups, std::max<int64_t>(1, d->max_total_rows / lo));
        const int64_t hi_rows = std::min<int64_t>(buckets[i].hi - 1, d->max_total_rows);
        const int64_t mblocks = std::min<int64_t>(experts * cdiv(hi_rows, ts.bm), cdiv(d->max_total_rows, ts.bm) + experts);
        const int64_t tasks = mblocks * cdiv(d->N, ts.bn);
        const int64_t slots = (int64_t)p->num_cus * ts.occupancy;
        GroupedLaunch L;
        L.tile = buckets[i].tile;
        L.lo = buckets[i].lo;
        L.hi = buckets[i].hi;
        L.grid = (int)std::max<int64_t>(1, std::min<int64_t>(tasks, slots));
        if (tasks <= 0 || lo > d->max_total_rows)
            continue;
        p->launches.push_back(L);
        snprintf(buf, sizeof buf, " [%d,%s)->%s grid=%d", L.lo, L.hi >= (1 << 30) ? "inf" : std::to_string(L.hi).c_str(),
                 tile_name(L.tile), L.grid);
        desc += buf;
    }
    p->tile = p->launches.empty() ? TILE_256x256 : p->launches.back().tile;
    p->tiles_m = p->tiles_n = p->tiles = 0;
    p->grid = p->launches.empty() ? 0 : p->launches.back().grid;
    p->group_m = 1;
    p->xcd_remap = (flags & MGEMM_PLAN_NO_XCD_REMAP) ? 0 : 1;
    p->description = desc;
    return MGEMM_OK;
}

// The fused MoE layer: one persistent launch over all experts (the
// eight-wave 256 x 256 tile for experts of more than 128 rows, the
// few-token tile for the others), one workgroup per compute unit (each
// takes the whole LDS).
static mgemm_status_t plan_moe(const mgemm_moe_desc_t *d, uint32_t flags, mgemm_plan *p)
{
    if (flags) {
        set_error("moe_fused_plan takes no flags");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (d->num_experts < 1 || d->num_experts > 256) {
        set_error("num_experts must lie in [1, 256] (got %d)", d->num_experts);
        return d->num_experts < 1 ? MGEMM_ERR_INVALID_ARG : MGEMM_ERR_UNSUPPORTED;
    }
    if (d->max_total_rows < 0 || d->hidden <= 0 || d->inter <= 0 || d->max_total_rows >= kMaxDim ||
        d->hidden >= kMaxDim || d->inter >= kMaxDim || d->stride_w1 < 0 || d->stride_w2 < 0) {
        set_error("sizes must lie in [0, 2^30) and hidden, inter be positive");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (d->dtype != MGEMM_BF16 && d->dtype != MGEMM_F16) {
        set_error("the fused MoE layer takes BF16 or F16 operands");
        return (d->dtype == MGEMM_F32 || d->dtype == MGEMM_E4M3) ? MGEMM_ERR_UNSUPPORTED : MGEMM_ERR_INVALID_ARG;
    }
    const int64_t N1 = 2 * d->inter;
    if (d->lda < d->hidden || d->ldw1 < N1 || d->ldw2 < d->hidden || d->ldh < d->inter || d->ldy < d->hidden) {
        set_error("leading dimension too small");
        return MGEMM_ERR_INVALID_ARG;
    }
    const int64_t w1 = (d->hidden - 1) * d->ldw1 + N1, w2 = (d->inter - 1) * d->ldw2 + d->hidden;
    if (d->num_experts > 1 && (d->stride_w1 < w1 || d->stride_w2 < w2)) {
        set_error("stride_w1 / stride_w2 smaller than one expert's weight matrix");
        return MGEMM_ERR_INVALID_ARG;
    }
    if (d->hidden % 16 || d->inter % 64) {
        set_error("the fused MoE layer needs hidden %% 16 == 0 and inter %% 64 == 0");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (d->lda % 8 || d->ldw1 % 8 || d->ldw2 % 8 || d->ldy % 8 || d->stride_w1 % 8 || d->stride_w2 % 8 ||
        d->ldh % 64) {
        set_error("lda, ldw1, ldw2, ldy and the expert strides must be multiples of 8, ldh of 64");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (d->lda > kMaxLd || d->ldw1 > kMaxLd || d->ldw2 > kMaxLd || d->ldh > kMaxLd || d->ldy > kMaxLd) {
        set_error("leading dimensions above 2^20 elements are not supported");
        return MGEMM_ERR_UNSUPPORTED;
    }
    if (w1 >= kMaxDim || w2 >= kMaxDim) {
        set_error("one expert's W1 or W2 must hold fewer than 2^30 elements");
        return MGEMM_ERR_UNSUPPORTED;
    }
    p->kind = PLAN_MOE;
    p->moe = *d;
    p->flags = flags;
    p->num_cus = device_cus();
    p->noop = d->max_total_rows == 0;
    p->zero_fill = false;
    p->tile = TILE_256x256_DTL;
    p->tiles_m = p->tiles_n = p->tiles = 0;
    p->group_m = 1;
    p->xcd_remap = 0;
    p->splits = 1;
    // counters: sum over experts of their row blocks <= rows / 256 + experts
    p->moe_slots = cdiv(d->max_total_rows, 256) + d->num_experts;
    p->workspace_bytes = (size_t)moe_ws_bytes(p->moe_slots);
    p->grid = p->num_cus;
    char buf[320];
    snprintf(buf, sizeof buf,
             "moe_fused G=%d rows<=%lld hidden=%lld inter=%lld %s fc1+fc2 one launch: [129,inf)->256x256dtl "
             "[1,129)->narrow128 (8 waves) order=largest-first grid=%d ws=%zu",
             d->num_experts, (long long)d->max_total_rows, (long long)d->hidden, (long long)d->inter,
             in_name(d->dtype), p->grid, p->workspace_bytes);
    p->description = buf;
    return MGEMM_OK;
}

}  // namespace mgemm

using namespace mgemm;

extern "C" mgemm_status_t gemm_plan(const mgemm_desc_t *desc, uint32_t flags, mgemm_plan_t *out)
{
    if (!desc || !out) {
        set_error("gemm_plan: null argument");
        return MGEMM_ERR_INVALID_ARG;
    }
    *out = nullptr;
    mgemm_plan *p = new (std::nothrow) mgemm_plan();
    if (!p) {
        set_error("gemm_plan: out of host memory");
        return MGEMM_ERR_NO_MEMORY;
    }
    mgemm_status_t s;
    try {
        s = plan_dense(desc, flags, p);
    } catch (...) {
        s = MGEMM_ERR_NO_MEMORY;
        set_error("gemm_plan: exception while planning");
    }
    if (s != MGEMM_OK) {
        delete p;
        return s;
    }
    *out = p;
    return MGEMM_OK;
}

extern "C" mgemm_status_t grouped_gemm_plan(const mgemm_grouped_desc_t *desc, uint32_t flags, mgemm_plan_t *out)
{
    if (!desc || !out) {
        set_error("grouped_gemm_plan: null argument");
        return MGEMM_ERR_INVALID_ARG;
    }
    *out = nullptr;
    mgemm_plan *p = new (std::nothrow) mgemm_plan();
    if (!p) {
        set_error("grouped_gemm_plan: out of host memory");
        return MGEMM_ERR_NO_MEMORY;
    }
    mgemm_status_t s;
    try {
        s = plan_grouped(desc, flags, p);
    } catch (...) {
        s = MGEMM_ERR_NO_MEMORY;
        set_error("grouped_gemm_plan: exception while planning");
    }
    if (s != MGEMM_OK) {
        delete p;
        return s;
    }
    *out = p;
    return MGEMM_OK;
}

extern "C" mgemm_status_t moe_fused_plan(const mgemm_moe_desc_t *desc, uint32_t flags, mgemm_plan_t *out)
{
    if (!desc || !out) {
        set_error("moe_fused_plan: null argument");
        return MGEMM_ERR_INVALID_ARG;
    }
    *out = nullptr;
    mgemm_plan *p = new (std::nothrow) mgemm_plan();
    if (!p) {
        set_error("moe_fused_plan: out of host memory");
        return MGEMM_ERR_NO_MEMORY;
    }
    mgemm_status_t s;
    try {
        s = plan_moe(desc, flags, p);
    } catch (...) {
        s = MGEMM_ERR_NO_MEMORY;
        set_error("moe_fused_plan: exception while planning");
    }
    if (s != MGEMM_OK) {
        delete p;
        return s;
    }
    *out = p;
    return MGEMM_OK;
}

extern "C" mgemm_status_t gemm_plan_workspace_size(mgemm_plan_t plan, size_t *bytes)
{
    if (!plan || !bytes) {
        set_error("gemm_plan_workspace_size: null argument");
        return MGEMM_ERR_INVALID_ARG;
    }
    *bytes = plan->kind == PLAN_GROUPED ? 0 : plan->workspace_bytes;
    return MGEMM_OK;
}

extern "C" mgemm_status_t gemm_plan_describe(mgemm_plan_t plan, char *buf, size_t len)
{
    if (!plan || !buf || len == 0) {
        set_error("gemm_plan_describe: null argument");
        return MGEMM_ERR_INVALID_ARG;
    }
    const std::string &d = plan->description;
    size_t n = std::min(len - 1, d.size());
    memcpy(buf, d.data(), n);
    buf[n] = 0;
    return MGEMM_OK;
}

extern "C" mgemm_status_t gemm_plan_info(mgemm_plan_t plan, mgemm_plan_info_t *info)
{
    if (!plan || !info) {
        set_error("gemm_plan_info: null argument");
        return MGEMM_ERR_INVALID_ARG;
    }
    const TileShape &ts = tile_shape(plan->tile);
    memset(info, 0, sizeof *info);
    info->block_m = ts.bm;
    info->block_n = ts.bn;
    info->block_k = kBK;
    info->waves_m = ts.wm;
    info->waves_n = ts.wn;
    info->stages = plan->tile == TILE_256x256_DTL ? 3 : 2;   // the deeper ring's slots
    if (is_narrow(plan->tile))
        info->stages = ts.lds_bytes / ((ts.bm + ts.bn) * 128);   // 128 token rows and 64 k x BN weights per slot
    if (plan->kind == PLAN_DENSE) {
        int a_slots, b_slots;
        dense_waves(plan->tile, plan->dense.b_layout == MGEMM_COL_MAJOR, info->waves_m, info->waves_n, a_slots,
                    b_slots, plan->dense.M);
        info->stages = std::max(a_slots, b_slots);
    }
    info->lds_bytes = plan->kind == PLAN_DENSE ? (int32_t)plan->lds_bytes : ts.lds_bytes;
    info->tiles_m = plan->tiles_m;
    info->tiles_n = plan->tiles_n;
    info->tiles = plan->tiles;
    const int64_t K = plan->kind == PLAN_DENSE ? plan->dense.K
                      : plan->kind == PLAN_GROUPED ? plan->grouped.K : plan->moe.hidden;
    info->k_steps = cdiv(K, kBK);
    if (plan->kind == PLAN_DENSE && plan->tiles > 0)
        info->coverage = (double)plan->dense.M * (double)(plan->dense.N & ~(int64_t)3) /
                         ((double)plan->tiles * ts.bm * ts.bn);
    info->grid = plan->grid;
    info->group_m = plan->group_m;
    info->xcd_remap = plan->xcd_remap;
    info->num_cus = plan->num_cus;
    info->splits = plan->kind == PLAN_DENSE ? plan->splits : 1;
    return MGEMM_OK;
}

extern "C" void gemm_plan_destroy(mgemm_plan_t plan) { delete plan; }

extern "C" mgemm_status_t mgemm_tile_budget(int64_t M, int64_t N, int64_t K, int32_t BM, int32_t BN, int32_t BK,
                                            int32_t stages, int32_t elt_bytes, mgemm_budget_t *out)
{
    if (!out || M < 0 || N < 0 || K < 0 || BM <= 0 || BN <= 0 || BK <= 0 || stages <= 0 || elt_bytes <= 0) {
        set_error("mgemm_tile_budget: invalid argument");
        return MGEMM_ERR_INVALID_ARG;
    }
    out->tiles = cdiv(M, BM) * cdiv(N, BN);
    out->coverage = out->tiles > 0 ? (double)M * (double)N / ((double)out->tiles * BM * BN) : 0.0;
    out->lds_bytes = operand_ring_bytes(BM, BK, stages, elt_bytes) + operand_ring_bytes(BN, BK, stages, elt_bytes);
    out->k_steps = cdiv(K, BK);
    return MGEMM_OK;
}

extern "C" int64_t mgemm_group_working_set(int32_t group_m, int32_t group_n, int32_t BM, int32_t BN, int64_t K,
                                           int32_t elt_bytes)
{
    return ((int64_t)group_m * BM + (int64_t)group_n * BN) * K * elt_bytes;
}

extern "C" int64_t mgemm_round_tokens(int64_t n, int32_t granule)
{
    if (granule <= 0 || (granule & (granule - 1)))
        return -1;
    return (n + granule - 1) & ~(int64_t)(granule - 1);
}
