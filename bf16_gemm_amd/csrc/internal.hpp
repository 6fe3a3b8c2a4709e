// internal.hpp -- host-side declarations shared by the planner, the C ABI
// and the per-tile kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mgemm.h"
#include "kernels.hpp"

namespace mgemm {

using DenseFn = hipError_t (*)(const DenseArgs &, int grid, hipStream_t);
using GroupedFn = hipError_t (*)(const GroupedArgs &, int grid, hipStream_t);

// Macro-tile variants compiled into the library.
enum TileId {
    TILE_256x256 = 0,
    TILE_128x128 = 1,
    TILE_32x256 = 2,
    TILE_64x256 = 3,
    TILE_256x256_DTL = 4,  // 256 x 256 with direct-to-LDS loads (k-contiguous A and B only)
    TILE_NARROW = 5,       // up to 128 tokens x 128 columns, token blocks sized at run time (row-major A)
    TILE_NARROW64 = 6,     // the same, 64 columns
    TILE_NARROW32 = 7,     // the same, 32 columns (two waves)
    NUM_TILES = 8
};

inline bool is_narrow(int tile) { return tile == TILE_NARROW || tile == TILE_NARROW64 || tile == TILE_NARROW32; }

struct TileShape {
    int bm, bn, wm, wn;
    int lds_bytes;   // LDS of the two-slot ring
    int occupancy;   // workgroups per CU the planner assumes
    double eff;      // relative MFMA efficiency the planner assumes
    bool narrow;     // narrow-M (few tokens) shape: needs a k-contiguous A
    bool forced_only;  // not scored by the cost model (a FORCE_TILE flag, or a rule, selects it)
};

const TileShape &tile_shape(int tile);

// Kernel tables, one per (tile, input type) translation unit.
// nullptr = that combination is not compiled.
DenseFn dense_fn(int tile, bool a_kmajor, bool b_kmajor, int in, int out);
GroupedFn grouped_fn(int tile, bool b_kmajor, int in, int out, int epi);

#define MGEMM_DECLARE_TU(NAME)                              \
    DenseFn dense_fn_##NAME(bool ak, bool bk, int out);     \
    GroupedFn grouped_fn_##NAME(bool bk, int out, int epi);
MGEMM_DECLARE_TU(256x256_bf16)
MGEMM_DECLARE_TU(256x256_f16)
MGEMM_DECLARE_TU(128x128_bf16)
MGEMM_DECLARE_TU(128x128_f16)
MGEMM_DECLARE_TU(32x256_bf16)
MGEMM_DECLARE_TU(32x256_f16)
MGEMM_DECLARE_TU(64x256_bf16)
MGEMM_DECLARE_TU(64x256_f16)
MGEMM_DECLARE_TU(256x256dtl_bf16)
MGEMM_DECLARE_TU(256x256dtl_f16)
MGEMM_DECLARE_TU(narrow128_bf16)
MGEMM_DECLARE_TU(narrow128_f16)
MGEMM_DECLARE_TU(narrow64_bf16)
MGEMM_DECLARE_TU(narrow64_f16)
MGEMM_DECLARE_TU(narrow32_bf16)
MGEMM_DECLARE_TU(narrow32_f16)
#undef MGEMM_DECLARE_TU
DenseFn dense_fn_256x256dtl_e4m3(bool ak, bool bk, int out);
// the E4M3 product with E8M0 block scales
DenseFn dense_block_fn_256x256dtl_e4m3(bool ak, bool bk, int out);
// stream-K launch of the four-wave direct-to-LDS tile (row-major A)
DenseFn dense_sk_fn_256x256dtl_bf16(bool bk, int out);
DenseFn dense_sk_fn_256x256dtl_f16(bool bk, int out);
GroupedFn grouped_fn_256x256dtl_e4m3(bool bk, int out, int epi);
// the grouped E4M3 product with E8M0 block scales
GroupedFn grouped_block_fn_256x256dtl_e4m3(bool bk, int out, int epi);

using EdgeFn = hipError_t (*)(const DenseArgs &, int a_kmajor, int b_kmajor, int n_first, hipStream_t);
EdgeFn edge_fn(int in, int out);
hipError_t launch_zero_fill(void *D, int rows, int cols, int64_t ld_bytes, int esize, hipStream_t s);
// the fused MoE layer: the prepare kernel, then the persistent kernel on `grid` workgroups
hipError_t launch_moe_fused(const MoeArgs &a, int in, int grid, hipStream_t s);
hipError_t launch_quantize_e4m3_block(const void *X, int64_t rows, int64_t cols, int64_t ldx, int in, uint8_t *Q,
                                      int64_t ldq, uint8_t *S, int64_t lds, hipStream_t s);
hipError_t launch_moe_combine(const void *Z, int64_t z_rows, int64_t ldz, const int32_t *pos, const float *w,
                              void *Y, int64_t ldy, int64_t T, int top_k, int64_t H, int out, hipStream_t s);
// D[M x N] = sum over r < splits of W[r][M x N] (fp32, row pitch ldw, slabs
// split_stride apart), added in increasing r and rounded once to D's type.
hipError_t launch_reduce_splits(const float *W, void *D, int M, int N, int ldw, int64_t split_stride, int splits,
                                int64_t ldd, int out, hipStream_t s);

// One kernel launch of a grouped plan: experts whose row count lies in
// [lo, hi) run with tile `tile` on `grid` workgroups.
struct GroupedLaunch {
    int tile;
    int lo, hi;
    int grid;
};

enum PlanKind { PLAN_DENSE = 1, PLAN_GROUPED = 2, PLAN_MOE = 3 };

void set_error(const char *fmt, ...);

// Enqueue a dense plan's kernels (gemm_run, gemm_run_scaled and
// gemm_run_noalloc all end here); workspace: the plan's scratch, or null
// when it needs none.
// block_sa / block_sb: E8M0 block scales of an E4M3 plan (gemm_run_blockscaled), else null.
mgemm_status_t dense_run(mgemm_plan_t plan, const void *A, const void *B, void *D, const float *scale_a,
                         const float *scale_b, void *workspace, size_t workspace_bytes, mgemm_stream_t stream,
                         const uint8_t *block_sa = nullptr, int64_t block_lda = 0,
                         const uint8_t *block_sb = nullptr, int64_t block_ldb = 0);

}  // namespace mgemm

struct mgemm_plan {
    int kind;
    mgemm_desc_t dense;
    mgemm_grouped_desc_t grouped;
    mgemm_moe_desc_t moe;
    uint32_t flags;
    int num_cus;
    // dense
    int tile;
    int64_t tiles_m, tiles_n, tiles;
    int grid;
    int group_m;
    int xcd_remap;
    int splits;      // K ranges per output tile; > 1 writes fp32 partials to the workspace
    int kchunk;      // elements of K per range
    int64_t slab_offset;  // split reduced in the launch: bytes of arrival counters before the partial slabs
    int sk_tiles;         // stream-K: tiles cut into `splits` K ranges (the rest run whole), else 0
    int64_t lds_bytes;    // the tile's ring (dense plans), from the stage budget
    size_t workspace_bytes;
    bool zero_fill;  // K == 0
    bool noop;       // M == 0 or N == 0
    // grouped
    std::vector<mgemm::GroupedLaunch> launches;
    // fused MoE layer: row blocks its counter array holds
    int64_t moe_slots;
    std::string description;
};
