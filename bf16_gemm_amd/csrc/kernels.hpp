// kernels.hpp -- dense and grouped GEMM kernels built on the tile engine,
// and the launch-side argument structs shared with the host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engine.hpp"
#include "narrow.hpp"

namespace mgemm {

struct DenseArgs {
    const void *A;
    const void *B;
    void *D;
    int M, N, K;
    int lda, ldb, ldd;
    int tiles_m, tiles_n;
    int tiles;        // tasks: output tiles x splits
    int group_m;      // tile rows per L2 group (m fastest inside a group)
    int xcd_remap;    // 1: give each XCD a contiguous run of tiles
    int splits;       // K ranges per output tile (1: the whole K)
    int kchunk;       // elements of K per range, a multiple of 64
    int64_t split_stride;  // elements of D between the partial results of consecutive ranges
    const float *scale_a = nullptr;  // E4M3 inputs: per-tensor scales (device, one float each; null = 1)
    const float *scale_b = nullptr;
    char *ws = nullptr;               // split reduced in the launch: arrival counters, then partial slabs
    int64_t slab_offset = 0;          // bytes from ws to the first slab
    uint32_t tag = 0;                 // this run's tag for the arrival counters (never 0 or ~0)
    int sk_tiles = 0;                 // stream-K: the last sk_tiles tiles are cut into `splits` K ranges
    const uint8_t *block_sa = nullptr;  // E4M3 block scales (E8M0): [M][block_lda], one per (row, 128-k block)
    const uint8_t *block_sb = nullptr;  // [ceil(N / 128)][block_ldb], one per (128 columns, 128-k block)
    int block_lda = 0, block_ldb = 0;
};

struct GroupedArgs {
    const void *A;           // [rows][K] row-major
    const void *B;           // expert weights, expert e at B + e * stride_b
    void *D;
    const int32_t *offs;     // [G + 1] device prefix sums
    int G, N, K;
    int lda, ldb, ldd;
    int64_t stride_b;
    int max_rows;            // rows of A / D that exist
    int tiles_n;
    int bucket_lo, bucket_hi;  // only experts with bucket_lo <= rows < bucket_hi
    int xcd_remap;
    const int32_t *row_index = nullptr;  // gathered A: routed row r reads A row row_index[r]
    int x_rows = 0;                      // rows of A that exist when gathering
    const float *scale_a = nullptr;      // E4M3: the activations' scale (device, one float; null = 1)
    const float *scale_b = nullptr;      // E4M3: one weight scale per expert (device, G floats; null = 1)
    const float *row_weight = nullptr;   // SILU_GATE: routed row r's h multiplied by row_weight[r] (null = 1)
    // E4M3 block scales (E8M0 bytes): routed row r's at block_sa + r * block_lda,
    // expert e's [ceil(N/128)][block_ldb] at block_sb + e * block_stride_sb
    const uint8_t *block_sa = nullptr;
    const uint8_t *block_sb = nullptr;
    int block_lda = 0, block_ldb = 0;
    int64_t block_stride_sb = 0;
};


// The fused MoE expert layer (moe_fused.hpp).
struct MoeArgs {
    const void *X;                       // FC1 A: routed rows [rows][hidden], or token rows with row_index
    const int32_t *row_index = nullptr;  // gathered A: routed row r reads X row row_index[r]
    int x_rows = 0;
    const void *W1;                      // [G][hidden][2 inter] row-major, gate / up interleaved by 8
    const void *W2;                      // [G][inter][hidden] row-major
    void *H;                             // [rows][inter]
    void *Y;                             // [rows][hidden]
    const float *row_weight = nullptr;   // routed row r's h scaled by row_weight[r], or none
    const int32_t *offs;                 // [G + 1] device prefix sums
    int G, hidden, inter, max_rows;
    int lda, ldw1, ldw2, ldh, ldy;
    int64_t stride_w1, stride_w2;
    char *ws;                            // schedule and counters (moe_ws_bytes)
    int max_slots;                       // row blocks the counter array holds
    uint32_t spin_limit;                 // polls before an FC2 task gives up (status 1)
};

// Workspace layout (bytes):
//   0    int32 ticket counter
//   4    int32 FC1 tasks, 8: FC2 tasks (written by the prepare kernel)
//   12   int32 status: 0 = fine; 1 = an FC2 task stopped waiting (never for
//        valid offsets); 2 = offsets gave more row blocks than the counter
//        array holds (nothing computed)
//   256  per position p < 256 (experts by rows, largest first): int32 x 4
//        {expert, first row, rows, first counter}
//   4352 int32 [256] first FC1 ticket of each position (INT32_MAX past G)
//   5376 int32 [256] first FC2 ticket of each position (counted from T1)
//   6400 int32 [max_slots] completion counters, one per (expert, row block)
constexpr int kMoeTicket = 0, kMoeT1 = 4, kMoeT2 = 8, kMoeStatus = 12;
constexpr int kMoeEntries = 256, kMoeStart1 = 4352, kMoeStart2 = 5376, kMoeCounters = 6400;
__host__ __device__ constexpr int64_t moe_ws_bytes(int64_t max_slots)
{
    return (kMoeCounters + max_slots * 4 + 255) / 256 * 256;
}

// Row blocks of an expert: blocks of 256 rows on the eight-wave 256 x 256
// tile, or (at most 128 rows) one block on the few-token tile.  Column
// tiles: 256 wide on the big tile, 128 on the few-token tile.
constexpr int kMoeNarrowRows = 128;
__host__ __device__ constexpr int moe_blocks(int rows)
{
    return rows <= 0 ? 0 : (rows <= kMoeNarrowRows ? 1 : (rows + 255) / 256);
}
__host__ __device__ constexpr int moe_tasks(int rows, int n)
{
    return rows <= 0 ? 0 : (rows <= kMoeNarrowRows ? (n + 127) / 128 : (rows + 255) / 256 * ((n + 255) / 256));
}


// Workgroup id -> logical id.  Workgroups are handed to the eight XCDs
// round-robin, so id w runs on XCD w % 8.  Mapping w to
// (w % 8) * (grid / 8) + w / 8 gives every XCD a contiguous block of logical
// ids, and therefore of neighbouring tiles that share operand rows and
// columns in that XCD's L2.
__device__ __forceinline__ int logical_block(int w, int grid, int remap)
{
    if (!remap || (grid & 7))
        return w;
    return (w & 7) * (grid >> 3) + (w >> 3);
}

// Tile id -> (mb, nb) in L2 groups: group_m tile rows at a time, m fastest
// inside a group, so consecutive tiles share a column block of B and the
// group's rows of A stay resident ("GEMM优化（三）", sections 3.2-3.4: the
// super-tile order that bounds the re-read passes of the other operand).
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m, int &mb, int &nb)
{
    int per_group = group_m * tiles_n;
    int g = t / per_group;
    int first_m = g * group_m;
    int gm = min(group_m, tiles_m - first_m);
    int within = t - g * per_group;
    mb = first_m + within % gm;
    nb = within / gm;
}

// Where one tile's operand lives.  k-contiguous operand ([rows][K]): the
// origin is the tile's first row; the bytes that exist end after the last
// existing row; one K step moves 64 elements along the row.  Row-contiguous
// operand ([K][rows]): the origin is the tile's first column; the bytes end
// after element (K-1, last existing column), rounded up to its 16-byte
// chunk, so every k >= K reads as zero; one K step moves 64 rows of ld
// elements.
template <bool KMAJOR>
__device__ __forceinline__ OperandSrc operand_src(const uint16_t *tile_origin, int ld, int rows_left, int K)
{
    OperandSrc s;
    s.base = (const char *)tile_origin;
    if constexpr (KMAJOR) {
        s.bytes = (uint64_t)rows_left * (uint64_t)ld * 2u;
        s.step_bytes = kBK * 2;
    } else {
        // up to the end of the 16-byte chunk that holds the last row's last
        // element: the range check zeroes a whole dword that reaches past
        // the records, so ending at an odd element would zero the last
        // element of the last k row with its neighbour.  The chunk lies in
        // the same page as that element (16-byte aligned base and rows),
        // and its extra elements feed only rows past the operand's end.
        s.bytes = K > 0 ? ((uint64_t)(K - 1) * (uint64_t)ld + (((uint64_t)rows_left + 7u) & ~(uint64_t)7u)) * 2u : 0;
        s.step_bytes = (uint32_t)kBK * (uint32_t)ld * 2u;
    }
    return s;
}

// Tile operand A of a grouped task: the tile's own block of rows, or (with
// a row index) the whole of A, each tile row picked through the index.
__device__ __forceinline__ OperandSrc grouped_a_src(const GroupedArgs &p, int m0, int m_valid, RowGather &g)
{
    const uint16_t *A = (const uint16_t *)p.A;
    if (p.row_index) {
        g.idx = p.row_index + m0;
        g.valid = m_valid;
        g.limit = p.x_rows;
        return operand_src<true>(A, p.lda, p.x_rows, p.K);
    }
    return operand_src<true>(A + (int64_t)m0 * p.lda, p.lda, m_valid, p.K);
}

template <class T, bool A_KMAJOR, bool B_KMAJOR, int IN, int OUT>
__global__ void __launch_bounds__(T::NT) dense_kernel(DenseArgs p)
{
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    T tile;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const uint16_t *A = (const uint16_t *)p.A;
    const uint16_t *B = (const uint16_t *)p.B;
    constexpr int esize = out_size(OUT);
    for (int t = L; t < p.tiles; t += grid) {
        // task t: output tile t / splits, K range t % splits (consecutive
        // tasks, which share an XCD, are the ranges of one tile)
        const int tile_id = t / p.splits;
        const int r = t - tile_id * p.splits;
        int mb, nb;
        tile_coords(tile_id, p.tiles_m, p.tiles_n, p.group_m, mb, nb);
        const int m0 = mb * T::BM, n0 = nb * T::BN;
        const int k0 = r * p.kchunk;
        const int klen = min(p.kchunk, p.K - k0);
        const uint16_t *At = A_KMAJOR ? A + (int64_t)m0 * p.lda + k0 : A + (int64_t)k0 * p.lda + m0;
        const uint16_t *Bt = B_KMAJOR ? B + (int64_t)n0 * p.ldb + k0 : B + (int64_t)k0 * p.ldb + n0;
        const OperandSrc sa = operand_src<A_KMAJOR>(At, p.lda, p.M - m0, klen);
        const OperandSrc sb = operand_src<B_KMAJOR>(Bt, p.ldb, p.N - n0, klen);
        tile.mainloop(lds, sa, p.lda, sb, p.ldb, klen, opaque((int)threadIdx.x));
        char *Dt = (char *)p.D + ((int64_t)r * p.split_stride + (int64_t)m0 * p.ldd + n0) * esize;
        tile_epilogue<T, EPI_NONE, OUT>(tile, lds, Dt, p.ldd, min(T::BM, p.M - m0), min(T::BN, p.N - n0),
                                        opaque((int)threadIdx.x));
    }
}

// Stream-K tail balancing on the four-wave 256 x 256 tile.  When the
// output tiles leave the last round of the persistent grid partly idle
// ("B200 的 2CTA 怎样调优", section 十: uneven SM use makes a long tail),
// the plan keeps the first tiles whole (data-parallel) and cuts the last
// sk_tiles tiles into `splits` K ranges, so every CU gets the same number
// of K steps to within one range.  Ranges run first (tasks 0 ..
// sk_tiles * splits - 1), then the whole tiles.  A range stores its fp32
// partial tile (256 x 256, in the accumulators' lane order) and arrives on
// its tile's counter (split_arrive: tagged, needs no initial value); the
// last range to arrive adds the partials in range order (its own from its
// accumulators) and stores the tile through the usual epilogue.  Nothing
// waits for another workgroup.
template <class T, bool BKM, int IN, int OUT>
__global__ void __launch_bounds__(T::NT) dense_sk_kernel(DenseArgs p)
{
    static_assert(T::FM == 8 && T::FN == 8 && T::NT == 256, "the four-wave 256 x 256 tile");
    constexpr uint32_t SLAB = 256 * 256 * 4;   // bytes of one partial tile
    constexpr uint32_t BLK = T::NT * 16;       // bytes between its 16-byte blocks
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    // the arrival count goes to every wave through the deep ring's third
    // slot, which the next task's prologue does not fill (its loads go out
    // after the first barrier of that task, and the epilogue's staging meets
    // the other waves at a barrier before writing LDS)
    uint32_t *arrived = (uint32_t *)(lds + (T::DEEP_B ? T::A_SLOTS * T::OPS : 0) + 2 * T::OPS);
    T tile;
    const int tid = threadIdx.x;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const uint16_t *A = (const uint16_t *)p.A;
    const uint16_t *B = (const uint16_t *)p.B;
    constexpr int esize = out_size(OUT);
    const int tiles = p.tiles_m * p.tiles_n;
    const int dp_tiles = tiles - p.sk_tiles;
    const int sk_tasks = p.sk_tiles * p.splits;
    const int total = sk_tasks + dp_tiles;
    const __amdgpu_buffer_rsrc_t slabs = make_rsrc(p.ws + p.slab_offset, (uint64_t)sk_tasks * SLAB);
    for (int t = L; t < total; t += grid) {
        const bool sk = t < sk_tasks;
        const int tile_id = sk ? dp_tiles + t / p.splits : t - sk_tasks;
        const int r = sk ? t % p.splits : 0;
        const int k0 = r * p.kchunk;
        const int klen = sk ? min(p.kchunk, p.K - k0) : p.K;
        int mb, nb;
        tile_coords(tile_id, p.tiles_m, p.tiles_n, p.group_m, mb, nb);
        const int m0 = mb * T::BM, n0 = nb * T::BN;
        const uint16_t *At = A + (int64_t)m0 * p.lda + k0;
        const uint16_t *Bt = BKM ? B + (int64_t)n0 * p.ldb + k0 : B + (int64_t)k0 * p.ldb + n0;
        const OperandSrc sa = operand_src<true>(At, p.lda, p.M - m0, klen);
        const OperandSrc sb = operand_src<BKM>(Bt, p.ldb, p.N - n0, klen);
        tile.mainloop(lds, sa, p.lda, sb, p.ldb, klen, opaque(tid));
        if (sk) {
            // one row of 8 blocks at a time (the scheduling barriers keep
            // the accumulators' copies to 32 registers)
            const uint32_t mine = (uint32_t)t * SLAB + (uint32_t)tid * 16u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, tile.acc[i][j]), slabs,
                                                           mine + (uint32_t)(i * 8 + j) * BLK, 0, kDeviceScope);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_vm<0>();
            __syncthreads();
            if (tid == 0)
                *arrived = split_arrive((uint64_t *)p.ws + (tile_id - dp_tiles), p.tag);
            __syncthreads();
            if (*arrived != (uint32_t)p.splits)
                continue;
            if (tid == 0)
                split_reset((uint64_t *)p.ws + (tile_id - dp_tiles), p.tag);
            // sum = P0 + P1 + ... in range order, one row of blocks at a time
            // with every other range's blocks of that row in flight together;
            // x[q] holds the q-th other range (q, or q + 1 from this range on),
            // so range rr != r is x[rr] below r and x[rr - 1] above: a select
            // between two fixed registers, no indexing at run time
            const uint32_t first = (uint32_t)(t - r) * SLAB + (uint32_t)tid * 16u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                f32x4_t x[kSkMaxSplits - 1][8];
#pragma unroll
                for (int q = 0; q < kSkMaxSplits - 1; ++q) {
                    const int rr = q < r ? q : q + 1;
                    if (rr < p.splits) {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            x[q][j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                      slabs, first + (uint32_t)rr * SLAB +
                                                                                 (uint32_t)(i * 8 + j) * BLK,
                                                                      0, kDeviceScope));
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            x[q][j] = f32x4_t{};
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const f32x4_t own = tile.acc[i][j];
                    f32x4_t s = r == 0 ? own : x[0][j];
#pragma unroll
                    for (int rr = 1; rr < kSkMaxSplits; ++rr) {
                        const f32x4_t below = x[rr < kSkMaxSplits - 1 ? rr : kSkMaxSplits - 2][j];
                        const f32x4_t other = rr < r ? below : x[rr - 1][j];
                        if (rr < p.splits)
                            s += rr == r ? own : other;
                    }
                    tile.acc[i][j] = s;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + n0) * esize;
        epilogue_staged<T, OUT>(tile, lds, Dt, p.ldd, min(T::BM, p.M - m0), min(T::BN, p.N - n0), opaque(tid));
        wait_vm<0>();
    }
}

// D = scale_a x scale_b x (A x B) for E4M3 A ([M][K], lda) and B ([N][K],
// ldb), both k-contiguous, on the four-wave direct-to-LDS tile; K is not
// split.  With one scale per tensor the dequantisation is one multiply of
// the finished fp32 sums, done in the epilogue ("MegaMoE：Blackwell 与 Hopper
// 的融合算子解读", Hopper section 04).  Leading dimensions and offsets are
// in elements = bytes.
// The blockwise-scaled E4M3 product ("MegaMoE：Blackwell 与 Hopper 的融合算子
// 解读", Hopper section 04, the blockwise path: the scales change along K, so
// each K block's product is scaled inside the K loop before it joins the
// sum): here the matrix instruction applies the E8M0 scales itself
// (v_mfma_scale_f32_16x16x128_f8f6f4), one K step = one 128-k block.
template <int OUT>
__global__ void __launch_bounds__(DtlTile4E4M3::NT) dense_e4m3_block_kernel(DenseArgs p)
{
    using T = DtlTile4E4M3X<true>;
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    T tile;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const char *A = (const char *)p.A;
    const char *B = (const char *)p.B;
    constexpr int esize = out_size(OUT);
    BlockScaleSrc bs;
    bs.kb = (p.K + T::KSTEP - 1) / T::KSTEP;
    bs.lds_a = p.block_lda;
    bs.lds_b = p.block_ldb;
    bs.rb = make_rsrc(p.block_sb, (uint64_t)((p.N + 127) / 128) * (uint64_t)p.block_ldb);
    for (int t = L; t < p.tiles; t += grid) {
        int mb, nb;
        tile_coords(t, p.tiles_m, p.tiles_n, p.group_m, mb, nb);
        const int m0 = mb * T::BM, n0 = nb * T::BN;
        OperandSrc sa, sb;
        sa.base = A + (int64_t)m0 * p.lda;
        sa.bytes = (uint64_t)(p.M - m0) * (uint64_t)p.lda;
        sa.step_bytes = T::KSTEP;
        sb.base = B + (int64_t)n0 * p.ldb;
        sb.bytes = (uint64_t)(p.N - n0) * (uint64_t)p.ldb;
        sb.step_bytes = T::KSTEP;
        bs.ra = make_rsrc(p.block_sa + (int64_t)m0 * p.block_lda, (uint64_t)(p.M - m0) * (uint64_t)p.block_lda);
        bs.nblk0 = n0 / 128;
        tile.mainloop(lds, sa, p.lda, sb, p.ldb, p.K, opaque((int)threadIdx.x), bs);
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + n0) * esize;
        epilogue_staged<T, OUT>(tile, lds, Dt, p.ldd, min(T::BM, p.M - m0), min(T::BN, p.N - n0),
                                opaque((int)threadIdx.x));
        wait_vm<0>();
    }
}

template <int OUT>
__global__ void __launch_bounds__(DtlTile4E4M3::NT) dense_e4m3_kernel(DenseArgs p)
{
    using T = DtlTile4E4M3;
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    T tile;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const char *A = (const char *)p.A;
    const char *B = (const char *)p.B;
    const float scale = (p.scale_a ? *p.scale_a : 1.0f) * (p.scale_b ? *p.scale_b : 1.0f);
    constexpr int esize = out_size(OUT);
    for (int t = L; t < p.tiles; t += grid) {
        int mb, nb;
        tile_coords(t, p.tiles_m, p.tiles_n, p.group_m, mb, nb);
        const int m0 = mb * T::BM, n0 = nb * T::BN;
        OperandSrc sa, sb;
        sa.base = A + (int64_t)m0 * p.lda;
        sa.bytes = (uint64_t)(p.M - m0) * (uint64_t)p.lda;
        sa.step_bytes = T::KSTEP;
        sb.base = B + (int64_t)n0 * p.ldb;
        sb.bytes = (uint64_t)(p.N - n0) * (uint64_t)p.ldb;
        sb.step_bytes = T::KSTEP;
        tile.mainloop(lds, sa, p.lda, sb, p.ldb, p.K, opaque((int)threadIdx.x));
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + n0) * esize;
        epilogue_staged<T, OUT, true>(tile, lds, Dt, p.ldd, min(T::BM, p.M - m0), min(T::BN, p.N - n0),
                                      opaque((int)threadIdx.x), scale);
        // the next tile's loads are counted from zero (as in tile_epilogue)
        wait_vm<0>();
    }
}

template <class T, bool B_KMAJOR, int IN, int OUT, int EPI>
__global__ void __launch_bounds__(T::NT) grouped_kernel(GroupedArgs p)
{
    static_assert(T::NT >= 64, "");
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    __shared__ int task_start[257];  // exclusive prefix of tasks per expert
    __shared__ int row_start[257];
    const int tid = threadIdx.x;

    // Task table from the device offsets: expert e contributes
    // ceil(rows_e / BM) * tiles_n tasks when its rows fall in the bucket.
    int cnt = 0;
    if (tid < p.G) {
        int lo = min(max(p.offs[tid], 0), p.max_rows);
        int hi = min(max(p.offs[tid + 1], lo), p.max_rows);
        int rows = hi - lo;
        row_start[tid] = lo;
        if (rows > 0 && rows >= p.bucket_lo && rows < p.bucket_hi)
            cnt = (rows + T::BM - 1) / T::BM * p.tiles_n;
        if (tid == p.G - 1)
            row_start[p.G] = hi;
    }
    // the table has 256 entries (num_groups <= 256) whatever the workgroup
    // size; threads past it only take part in the barriers
    constexpr int TT = 256;
    if (tid < TT)
        task_start[tid + 1] = cnt;
    if (tid == 0)
        task_start[0] = 0;
    __syncthreads();
    // inclusive scan of task_start[1..TT] (Hillis-Steele)
    for (int s = 1; s < TT; s <<= 1) {
        int v = (tid < TT && tid >= s) ? task_start[tid + 1 - s] : 0;
        __syncthreads();
        if (tid < TT)
            task_start[tid + 1] += v;
        __syncthreads();
    }
    const int total = task_start[p.G];

    T tile;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const uint16_t *B = (const uint16_t *)p.B;
    constexpr int esize = out_size(OUT);
    for (int t = L; t < total; t += grid) {
        // expert: the last e with task_start[e] <= t
        int lo = 0, hi = p.G;  // invariant: task_start[lo] <= t < task_start[hi]
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if (task_start[mid] <= t)
                lo = mid;
            else
                hi = mid;
        }
        const int e = lo;
        const int local = t - task_start[e];
        const int rows0 = row_start[e];
        const int rows_e = row_start[e + 1] - rows0;
        const int tm = (rows_e + T::BM - 1) / T::BM;
        const int mb = local % tm, nb = local / tm;
        const int m0 = rows0 + mb * T::BM, n0 = nb * T::BN;
        const int m_valid = min(T::BM, rows_e - mb * T::BM);
        const uint16_t *Be = B + (int64_t)e * p.stride_b;
        const uint16_t *Bt = B_KMAJOR ? Be + (int64_t)n0 * p.ldb : Be + n0;
        RowGather ga;
        const OperandSrc sa = grouped_a_src(p, m0, m_valid, ga);
        const OperandSrc sb = operand_src<B_KMAJOR>(Bt, p.ldb, p.N - n0, p.K);
        tile.mainloop(lds, sa, p.lda, sb, p.ldb, p.K, opaque((int)threadIdx.x), ga);
        const int dcol0 = EPI == EPI_SILU_GATE ? n0 / 2 : n0;
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + dcol0) * esize;
        tile_epilogue<T, EPI, OUT>(tile, lds, Dt, p.ldd, m_valid, min(T::BN, p.N - n0), opaque((int)threadIdx.x),
                                   p.row_weight ? p.row_weight + m0 : nullptr);
    }
}

// The grouped task list without LDS, for tiles that use all of it: every
// wave builds the same per-expert task counts in registers.  Lane l holds
// experts 4l .. 4l+3 (num_groups <= 256); a wave-wide inclusive scan of the
// lanes' sums gives each lane the number of tasks before its experts, and
// the lane holding task t is the number of lanes whose tasks all come
// before t (a ballot: the prefix sums do not decrease).
struct WaveTasks {
    int cnt[4];   // tasks of experts 4 lane + i
    int row0[4];  // their first row and row count (clamped offsets)
    int nrow[4];
    int excl;     // tasks of all experts before 4 lane
    int total;

    __device__ __forceinline__ static void rows_of(const GroupedArgs &p, int e, int &lo, int &hi)
    {
        lo = min(max(p.offs[e], 0), p.max_rows);
        hi = min(max(p.offs[e + 1], lo), p.max_rows);
    }
    __device__ __forceinline__ void build(const GroupedArgs &p, int bm, int lane)
    {
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            int c = 0, lo = 0, rows = 0;
            if (e < p.G) {
                int hi;
                rows_of(p, e, lo, hi);
                rows = hi - lo;
                if (rows > 0 && rows >= p.bucket_lo && rows < p.bucket_hi)
                    c = (rows + bm - 1) / bm * p.tiles_n;
            }
            row0[i] = lo;
            nrow[i] = rows;
            cnt[i] = c;
            sum += c;
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d)
                incl += v;
        }
        excl = incl - sum;
        total = __shfl(incl, 63, 64);
    }
    // expert e, index inside it, first row and row count of task t
    // (uniform, 0 <= t < total); lane reads only, no memory access, so no
    // wait for the previous task's stores
    __device__ __forceinline__ void find(int t, int &e, int &local, int &rows0, int &rows_e) const
    {
        const int incl = excl + cnt[0] + cnt[1] + cnt[2] + cnt[3];
        const int L = __popcll(__ballot(incl <= t));
        int r = t - __builtin_amdgcn_readlane(excl, L);
        const int c0 = __builtin_amdgcn_readlane(cnt[0], L);
        const int c1 = __builtin_amdgcn_readlane(cnt[1], L);
        const int c2 = __builtin_amdgcn_readlane(cnt[2], L);
        int i = 0;
        if (r >= c0) {
            r -= c0;
            i = 1;
            if (r >= c1) {
                r -= c1;
                i = 2;
                if (r >= c2) {
                    r -= c2;
                    i = 3;
                }
            }
        }
        e = 4 * L + i;
        local = r;
        const int lo0 = __builtin_amdgcn_readlane(row0[0], L), lo1 = __builtin_amdgcn_readlane(row0[1], L);
        const int lo2 = __builtin_amdgcn_readlane(row0[2], L), lo3 = __builtin_amdgcn_readlane(row0[3], L);
        const int n0 = __builtin_amdgcn_readlane(nrow[0], L), n1 = __builtin_amdgcn_readlane(nrow[1], L);
        const int n2 = __builtin_amdgcn_readlane(nrow[2], L), n3 = __builtin_amdgcn_readlane(nrow[3], L);
        rows0 = i == 0 ? lo0 : i == 1 ? lo1 : i == 2 ? lo2 : lo3;
        rows_e = i == 0 ? n0 : i == 1 ? n1 : i == 2 ? n2 : n3;
    }
};

// grouped_kernel with the task list in registers (WaveTasks), for tiles
// whose rings fill the LDS.
template <class T, bool B_KMAJOR, int IN, int OUT, int EPI>
__global__ void __launch_bounds__(T::NT) grouped_kernel_wt(GroupedArgs p)
{
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    WaveTasks wt;
    wt.build(p, T::BM, (int)threadIdx.x & 63);
    T tile;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const uint16_t *B = (const uint16_t *)p.B;
    constexpr int esize = out_size(OUT);
    for (int t = L; t < wt.total; t += grid) {
        int e, local, rows0, rows_e;
        wt.find(t, e, local, rows0, rows_e);
        const int tm = (rows_e + T::BM - 1) / T::BM;
        const int mb = local % tm, nb = local / tm;
        const int m0 = rows0 + mb * T::BM, n0 = nb * T::BN;
        const int m_valid = min(T::BM, rows_e - mb * T::BM);
        const uint16_t *Be = B + (int64_t)e * p.stride_b;
        const uint16_t *Bt = B_KMAJOR ? Be + (int64_t)n0 * p.ldb : Be + n0;
        RowGather ga;
        const OperandSrc sa = grouped_a_src(p, m0, m_valid, ga);
        const OperandSrc sb = operand_src<B_KMAJOR>(Bt, p.ldb, p.N - n0, p.K);
        tile.mainloop(lds, sa, p.lda, sb, p.ldb, p.K, opaque((int)threadIdx.x), ga);
        const int dcol0 = EPI == EPI_SILU_GATE ? n0 / 2 : n0;
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + dcol0) * esize;
        tile_epilogue<T, EPI, OUT>(tile, lds, Dt, p.ldd, m_valid, min(T::BN, p.N - n0), opaque((int)threadIdx.x),
                                   p.row_weight ? p.row_weight + m0 : nullptr);
    }
}

// The grouped product on E4M3 inputs (expert weights column-major, [N][K]
// each) on the four-wave direct-to-LDS tile, task list in registers:
// expert e's rows are multiplied by its weights and the finished sums by
// scale_a x scale_b[e] -- one scale for the activations, one per expert for
// the weights ("MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 04,
// the per-tensor path).
template <int OUT>
__global__ void __launch_bounds__(DtlTile4E4M3::NT) grouped_e4m3_kernel(GroupedArgs p)
{
    using T = DtlTile4E4M3;
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    WaveTasks wt;
    wt.build(p, T::BM, (int)threadIdx.x & 63);
    T tile;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const char *A = (const char *)p.A;
    const char *B = (const char *)p.B;
    const float sa = p.scale_a ? *p.scale_a : 1.0f;
    constexpr int esize = out_size(OUT);
    for (int t = L; t < wt.total; t += grid) {
        int e, local, rows0, rows_e;
        wt.find(t, e, local, rows0, rows_e);
        const int tm = (rows_e + T::BM - 1) / T::BM;
        const int mb = local % tm, nb = local / tm;
        const int m0 = rows0 + mb * T::BM, n0 = nb * T::BN;
        const int m_valid = min(T::BM, rows_e - mb * T::BM);
        OperandSrc sa_src, sb_src;
        sa_src.base = A + (int64_t)m0 * p.lda;
        sa_src.bytes = (uint64_t)m_valid * (uint64_t)p.lda;
        sa_src.step_bytes = T::KSTEP;
        sb_src.base = B + (int64_t)e * p.stride_b + (int64_t)n0 * p.ldb;
        sb_src.bytes = (uint64_t)(p.N - n0) * (uint64_t)p.ldb;
        sb_src.step_bytes = T::KSTEP;
        tile.mainloop(lds, sa_src, p.lda, sb_src, p.ldb, p.K, opaque((int)threadIdx.x));
        const float scale = sa * (p.scale_b ? p.scale_b[e] : 1.0f);
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + n0) * esize;
        epilogue_staged<T, OUT, true>(tile, lds, Dt, p.ldd, m_valid, min(T::BN, p.N - n0),
                                      opaque((int)threadIdx.x), scale);
        wait_vm<0>();
    }
}

// The grouped product with block scales: the per-expert task walk of
// grouped_e4m3_kernel on the block-scaled tile of dense_e4m3_block_kernel,
// each task's A scales from its first routed row (rows past the task's
// expert read as zeros: their outputs are not stored) and its B scales
// from its expert's block ("MegaMoE", Hopper section 04, the blockwise path
// for the expert GEMMs).
template <int OUT>
__global__ void __launch_bounds__(DtlTile4E4M3::NT) grouped_e4m3_block_kernel(GroupedArgs p)
{
    using T = DtlTile4E4M3X<true>;
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    WaveTasks wt;
    wt.build(p, T::BM, (int)threadIdx.x & 63);
    T tile;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const char *A = (const char *)p.A;
    const char *B = (const char *)p.B;
    constexpr int esize = out_size(OUT);
    BlockScaleSrc bs;
    bs.kb = (p.K + T::KSTEP - 1) / T::KSTEP;
    bs.lds_a = p.block_lda;
    bs.lds_b = p.block_ldb;
    const uint64_t sb_bytes = (uint64_t)((p.N + 127) / 128) * (uint64_t)p.block_ldb;
    for (int t = L; t < wt.total; t += grid) {
        int e, local, rows0, rows_e;
        wt.find(t, e, local, rows0, rows_e);
        const int tm = (rows_e + T::BM - 1) / T::BM;
        const int mb = local % tm, nb = local / tm;
        const int m0 = rows0 + mb * T::BM, n0 = nb * T::BN;
        const int m_valid = min(T::BM, rows_e - mb * T::BM);
        OperandSrc sa_src, sb_src;
        sa_src.base = A + (int64_t)m0 * p.lda;
        sa_src.bytes = (uint64_t)m_valid * (uint64_t)p.lda;
        sa_src.step_bytes = T::KSTEP;
        sb_src.base = B + (int64_t)e * p.stride_b + (int64_t)n0 * p.ldb;
        sb_src.bytes = (uint64_t)(p.N - n0) * (uint64_t)p.ldb;
        sb_src.step_bytes = T::KSTEP;
        bs.ra = make_rsrc(p.block_sa + (int64_t)m0 * p.block_lda, (uint64_t)m_valid * (uint64_t)p.block_lda);
        bs.rb = make_rsrc(p.block_sb + (int64_t)e * p.block_stride_sb, sb_bytes);
        bs.nblk0 = n0 / 128;
        tile.mainloop(lds, sa_src, p.lda, sb_src, p.ldb, p.K, opaque((int)threadIdx.x), bs);
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + n0) * esize;
        epilogue_staged<T, OUT>(tile, lds, Dt, p.ldd, m_valid, min(T::BN, p.N - n0), opaque((int)threadIdx.x));
        wait_vm<0>();
    }
}

// Dense product on the few-token tile: output tile t / splits, K range
// t % splits (consecutive tasks -- one XCD with the remap -- are the ranges
// of one tile).  Unsplit, a task stores its tile.  Split, every range
// writes its fp32 partial tile to its slab of the workspace, publishes it
// (release fence, then an arrival on the tile's counter), and the range
// that arrives last adds all ranges' partials in increasing range order
// (its own from registers) and stores the tile: the reduction of "B200 的
// 2CTA 怎样调优" (section 八: a K split pays for its reduction) inside the
// same launch, with a result that does not depend on which range finishes
// last.  No range waits for another, so the grid needs no co-residency.
template <bool BKM, int IN, int OUT, int BN>
__global__ void __launch_bounds__((NarrowTile<IN, BKM, BN>::NT)) narrow_dense_kernel(DenseArgs p)
{
    using T = NarrowTile<IN, BKM, BN>;
    constexpr int SLAB = narrow_slab_bytes(BN);   // bytes of one partial tile
    constexpr uint32_t BSTRIDE = T::NT * 16;       // bytes between its blocks
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    // the arrival count is passed to every wave through a word that no load
    // of the rings writes
    uint32_t *arrived = (uint32_t *)(lds + T::WORDS);
    T tile;
    const int tid = threadIdx.x;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const uint16_t *A = (const uint16_t *)p.A;
    const uint16_t *B = (const uint16_t *)p.B;
    constexpr int esize = out_size(OUT);
    for (int t = L; t < p.tiles; t += grid) {
        const int tile_id = t / p.splits;
        const int r = t - tile_id * p.splits;
        int mb, nb;
        tile_coords(tile_id, p.tiles_m, p.tiles_n, p.group_m, mb, nb);
        const int m0 = mb * T::BM, n0 = nb * T::BN;
        const int m_valid = min(T::BM, p.M - m0);
        const int ntb = (m_valid + 15) >> 4;     // tokens rounded up to 16
        const int k0 = r * p.kchunk;
        const int klen = min(p.kchunk, p.K - k0);
        const uint16_t *At = A + (int64_t)m0 * p.lda + k0;
        const uint16_t *Bt = BKM ? B + (int64_t)n0 * p.ldb + k0 : B + (int64_t)k0 * p.ldb + n0;
        const OperandSrc sa = operand_src<true>(At, p.lda, m_valid, klen);
        const OperandSrc sb = operand_src<BKM>(Bt, p.ldb, p.N - n0, klen);
        tile.mainloop(lds, sa, p.lda, sb, p.ldb, klen, ntb, opaque(tid));
        f32x4_t v[T::NTB][T::NB];
        tile.values(v, ntb);
        if (p.splits > 1) {
            // the slabs of all tasks (tile-major), device-scope stores and loads
            const __amdgpu_buffer_rsrc_t slabs =
                make_rsrc(p.ws + p.slab_offset, (uint64_t)p.tiles * (uint64_t)SLAB);
            uint64_t *counter = (uint64_t *)p.ws + tile_id;
            const uint32_t mine = (uint32_t)t * (uint32_t)SLAB + (uint32_t)tid * 16u;
#pragma unroll
            for (int tb = 0; tb < T::NTB; ++tb) {
                if (tb < ntb) {
#pragma unroll
                    for (int j = 0; j < T::NB; ++j)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v[tb][j]), slabs,
                                                               mine + (uint32_t)(tb * T::NB + j) * BSTRIDE, 0,
                                                               kDeviceScope);
                }
            }
            wait_vm<0>();         // this range's partial has reached the shared level
            __syncthreads();
            if (tid == 0)
                *arrived = split_arrive(counter, p.tag);
            __syncthreads();
            if (*arrived != (uint32_t)p.splits)
                continue;         // another range arrives later and stores the tile
            if (tid == 0)
                split_reset(counter, p.tag);
            // sum = P0 + P1 + ... in range order, this range's own partial
            // from registers; one range's blocks are loaded together
            const uint32_t first = (uint32_t)(t - r) * (uint32_t)SLAB + (uint32_t)tid * 16u;
            f32x4_t sum[T::NTB][T::NB];
            for (int rr = 0; rr < p.splits; ++rr) {
                f32x4_t x[T::NTB][T::NB];
                if (rr == r) {
#pragma unroll
                    for (int tb = 0; tb < T::NTB; ++tb)
#pragma unroll
                        for (int j = 0; j < T::NB; ++j)
                            x[tb][j] = v[tb][j];
                } else {
                    const uint32_t base = first + (uint32_t)rr * (uint32_t)SLAB;
#pragma unroll
                    for (int tb = 0; tb < T::NTB; ++tb)
#pragma unroll
                        for (int j = 0; j < T::NB; ++j)
                            x[tb][j] = tb < ntb ? __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    slabs, base + (uint32_t)(tb * T::NB + j) * BSTRIDE,
                                                                    0, kDeviceScope))
                                                : f32x4_t{};
                }
#pragma unroll
                for (int tb = 0; tb < T::NTB; ++tb)
#pragma unroll
                    for (int j = 0; j < T::NB; ++j)
                        sum[tb][j] = rr == 0 ? x[tb][j] : sum[tb][j] + x[tb][j];
            }
#pragma unroll
            for (int tb = 0; tb < T::NTB; ++tb)
#pragma unroll
                for (int j = 0; j < T::NB; ++j)
                    v[tb][j] = sum[tb][j];
        }
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + n0) * esize;
        narrow_store<EPI_NONE, OUT>(v, Dt, p.ldd, m_valid, min(T::BN, p.N - n0), ntb, tid);
        wait_vm<0>();
    }
}

// Grouped product on the few-token tile (experts with at most 128 rows):
// task list in registers, each task one expert's rows against 128 of its
// weight columns, its token blocks sized to the expert's row count.
template <bool BKM, int IN, int OUT, int EPI, int BN>
__global__ void __launch_bounds__((NarrowTile<IN, BKM, BN>::NT)) narrow_grouped_kernel(GroupedArgs p)
{
    using T = NarrowTile<IN, BKM, BN>;
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    const int tid = threadIdx.x;
    WaveTasks wt;
    wt.build(p, T::BM, tid & 63);
    T tile;
    const int grid = gridDim.x;
    const int L = logical_block(blockIdx.x, grid, p.xcd_remap);
    const uint16_t *B = (const uint16_t *)p.B;
    constexpr int esize = out_size(OUT);
    for (int t = L; t < wt.total; t += grid) {
        int e, local, rows0, rows_e;
        wt.find(t, e, local, rows0, rows_e);
        const int tm = (rows_e + T::BM - 1) / T::BM;
        const int mb = local % tm, nb = local / tm;
        const int m0 = rows0 + mb * T::BM, n0 = nb * T::BN;
        const int m_valid = min(T::BM, rows_e - mb * T::BM);
        const int ntb = (m_valid + 15) >> 4;
        const uint16_t *Be = B + (int64_t)e * p.stride_b;
        const uint16_t *Bt = BKM ? Be + (int64_t)n0 * p.ldb : Be + n0;
        RowGather ga;
        const OperandSrc sa = grouped_a_src(p, m0, m_valid, ga);
        const OperandSrc sb = operand_src<BKM>(Bt, p.ldb, p.N - n0, p.K);
        tile.mainloop(lds, sa, p.lda, sb, p.ldb, p.K, ntb, opaque(tid), ga);
        f32x4_t v[T::NTB][T::NB];
        tile.values(v, ntb);
        const int dcol0 = EPI == EPI_SILU_GATE ? n0 / 2 : n0;
        char *Dt = (char *)p.D + ((int64_t)m0 * p.ldd + dcol0) * esize;
        narrow_store<EPI, OUT>(v, Dt, p.ldd, m_valid, min(T::BN, p.N - n0), ntb, tid,
                               p.row_weight ? p.row_weight + m0 : nullptr);
        wait_vm<0>();
    }
}

// The last N % 4 output columns (at most three) when N is not a multiple of
// four: one wave per (row, column) pair, fp32 partial sums over k reduced
// across the wave.  Tiny next to the tiles, so kept plain.
template <int IN>
__device__ __forceinline__ float in_value(const uint16_t *p, int64_t i)
{
    if constexpr (IN == IN_BF16)
        return (float)__builtin_bit_cast(__bf16, p[i]);
    else
        return (float)__builtin_bit_cast(_Float16, p[i]);
}

template <int IN, int OUT>
__global__ void __launch_bounds__(256) edge_cols_kernel(DenseArgs p, int a_kmajor, int b_kmajor, int n_first)
{
    const int ncols = p.N - n_first;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)p.M * ncols)
        return;
    const int m = (int)(item / ncols), n = n_first + (int)(item % ncols);
    const uint16_t *A = (const uint16_t *)p.A, *B = (const uint16_t *)p.B;
    float s = 0.0f;
    for (int k = lane; k < p.K; k += 64) {
        const float a = in_value<IN>(A, a_kmajor ? (int64_t)m * p.lda + k : (int64_t)k * p.lda + m);
        const float b = in_value<IN>(B, b_kmajor ? (int64_t)n * p.ldb + k : (int64_t)k * p.ldb + n);
        s += a * b;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        s += __shfl_xor(s, o, 64);
    if (lane == 0) {
        char *d = (char *)p.D + ((int64_t)m * p.ldd + n) * out_size(OUT);
        if constexpr (OUT == OUT_F32)
            *(float *)d = s;
        else if constexpr (OUT == OUT_BF16)
            *(__bf16 *)d = (__bf16)s;
        else
            *(_Float16 *)d = (_Float16)opaque(s);   // the fp32 sum, then one conversion (see pack2_f16)
    }
}

}  // namespace mgemm
