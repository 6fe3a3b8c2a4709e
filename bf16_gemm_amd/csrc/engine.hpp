// engine.hpp -- the gfx950 tile engine shared by the dense and grouped kernels.
//
// One workgroup computes one BM x BN output tile at a time:
//
//   * operands are staged through a two-slot LDS ring, 64 k per slot
//     (block_k), each tile row 128 bytes wide;
//   * global -> register loads are 16 bytes per lane through buffer
//     resources, so out-of-range rows and k read as zero without branches;
//   * a k-contiguous operand is written to LDS as loaded; an operand whose
//     rows run along M/N (row-major B, column-major A) is transposed in
//     registers in 8x8 blocks with v_perm_b32 so that both operands sit in
//     LDS as [row][k];
//   * inside a 128-byte LDS row the eight 16-byte chunks are XOR-permuted by
//     a function of the row.  The idea is the 128B swizzle of "GEMM优化（三）
//     大矩阵适配和极致优化" (section 2.1: a chunk's physical index is its
//     logical index XORed with the row), here with the row's bits 0-2 and
//     3-5 both folded in, because the transposing writer stores eight rows
//     that are eight apart while the MFMA fragment reader reads eight
//     consecutive rows: both groups land in eight distinct chunks;
//   * the K loop is a software pipeline: while the MFMAs of step k run on
//     one LDS slot, the registers holding step k+1 are written to the other
//     slot and the global loads of a later step (k+NS+1, with NS register
//     staging sets) are issued -- the load/compute
//     overlap that "从 CUDA 代码到 GPU 执行" (Warp Specialization section)
//     and "使用 Warp Specialization 和 Cluster 扩展 GEMM" (step 7) obtain with
//     separate roles, obtained here inside every wave;
//   * for 256 x 256 tiles whose operands are both k-contiguous, DtlTile
//     replaces the register staging with loads that write LDS directly and
//     runs eight waves instead of four;
//   * the MFMA is v_mfma_f32_32x32x16_{bf16,f16}; the B-tile fragment is
//     passed as the instruction's first operand and the A-tile fragment as
//     the second, so each lane's accumulator registers hold four consecutive
//     output columns of one output row and the epilogue writes 16-byte
//     (fp32) or 8-byte (16-bit) vectors directly from registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mgemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;                 // k per LDS slot
constexpr int kRowBytes = kBK * 2;      // bytes of one tile row in LDS
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every range
constexpr uint32_t kMaxRecords = 0x7ffffff0u;

enum InType { IN_BF16 = 0, IN_F16 = 1, IN_E4M3 = 2 };
enum OutType { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };
enum EpiKind { EPI_NONE = 0, EPI_SILU_GATE = 1 };

// Physical 16-byte chunk of logical chunk c in LDS row `row` is
// c ^ swz(row).  Any 8 consecutive rows, and any 8 rows spaced 8 apart
// starting on a multiple of 8, get 8 distinct values.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint64_t bytes)
{
    uint32_t n = bytes > kMaxRecords ? kMaxRecords : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}

// Rows of A taken through an index (the MoE dispatch fused into the A
// loads: "MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 11, a
// dispatch warp pulls the routed tokens' rows for the expert GEMM).  Tile
// row r reads A row idx[r]; rows r >= valid, and indices outside
// [0, limit), read as zeros.  idx == nullptr: tile row r is row r of the
// tile's own block of A.
struct RowGather {
    const int32_t *idx = nullptr;
    int valid = 0;
    int limit = 0;
    // byte offset of tile row r's source row (ld elements per row), or kOOB
    __device__ __forceinline__ uint32_t row_offset(int r, int ld) const
    {
        const int src = r < valid ? idx[r] : -1;
        return (src >= 0 && src < limit) ? (uint32_t)src * (uint32_t)ld * 2u : kOOB;
    }
};

__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Hide a value from loop-invariant code motion: the compiler must assume the
// value changes here, so expressions built from it are recomputed where
// they are used (a few adds) instead of being precomputed and held in
// registers for the whole kernel.
template <class V>
__device__ __forceinline__ V opaque(V v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// LDS barrier: wait for this wave's LDS traffic, then meet the other waves.
// Global loads in flight are deliberately not waited for.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Loaders: one operand tile of R rows (M or N) x 64 k per K step.
//
// The buffer resource passed to load() already points at the current K
// step (its base advances by one step per iteration and its record count
// shrinks by the same amount), so every per-lane offset below is fixed for
// the whole K loop and only a handful of registers hold addresses.
// ---------------------------------------------------------------------------

template <int R, int NT, bool KMAJOR>
struct Loader;

// k-contiguous storage: row r of the tile is 64 consecutive k, 8 chunks of
// 16 B.  Thread t handles chunk (t & 7) of rows (t >> 3) + j * NT/8, so
// eight consecutive lanes read one whole 128-byte row segment.
template <int R, int NT>
struct Loader<R, NT, true> {
    static constexpr int RSTEP = NT / 8;        // rows between a thread's chunks
    static constexpr int NC = R / RSTEP;        // chunks per thread
    static_assert(R % RSTEP == 0 && NC >= 1, "tile rows must cover the workgroup");
    static_assert(RSTEP % 64 == 0 || RSTEP == 32, "row step must keep the swizzle periodic");
    u32x4_t v[NC];
    uint32_t goff;      // byte offset of this lane's first chunk
    uint32_t gstep;     // bytes between consecutive chunks of this lane (uniform)
    int kc;             // k of this lane's chunk inside the step
    int lds_even, lds_odd;  // LDS byte offsets of chunk 0 / chunk 1

    __device__ __forceinline__ void init(int tid, int ld)
    {
        const int row = tid >> 3, c = tid & 7;
        goff = (uint32_t)row * (uint32_t)ld * 2u + (uint32_t)c * 16u;
        gstep = (uint32_t)RSTEP * (uint32_t)ld * 2u;
        kc = c * 8;
        lds_even = row * kRowBytes + ((c ^ swz(row)) << 4);
        lds_odd = (row + RSTEP) * kRowBytes + ((c ^ swz(row + RSTEP)) << 4) - RSTEP * kRowBytes;
    }
    // rows through an index (one chunk per lane only: NC == 1)
    __device__ __forceinline__ void gather(int tid, int ld, const RowGather &g)
    {
        static_assert(NC == 1, "gathered rows need one row per lane");
        const uint32_t ro = g.row_offset(tid >> 3, ld);
        goff = ro == kOOB ? kOOB : ro + (uint32_t)(tid & 7) * 16u;
    }
    // k_left: k remaining from this step's first k (>= 64 means a full step)
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int k_left)
    {
        const uint32_t base = opaque(kc < k_left ? goff : kOOB);
#pragma unroll
        for (int j = 0; j < NC; ++j)
            v[j] = bload16(r, base + (uint32_t)j * gstep);
    }
    __device__ __forceinline__ void store(char *lds) const
    {
        // rows r and r + 2*RSTEP share a swizzle (RSTEP is 32 or a multiple
        // of 64), so chunk j sits j * RSTEP rows below chunk (j & 1)
#pragma unroll
        for (int j = 0; j < NC; ++j)
            *(u32x4_t *)(lds + ((j & 1) ? lds_odd : lds_even) + j * RSTEP * kRowBytes) = v[j];
    }
    // The same work split into NP parts (chunks j with j % NP == P), so the
    // steady-state K loop can spread it between MFMA groups.  Part P's loads
    // reuse the registers that part P's store has just written out.
    // LDS writes / global loads that part P of NP issues
    template <int P, int NP>
    static constexpr int part_writes() { return P < NC ? (NC - P + NP - 1) / NP : 0; }
    template <int P, int NP>
    static constexpr int part_loads() { return part_writes<P, NP>(); }

    template <int P, int NP>
    __device__ __forceinline__ void store_part(char *lds) const
    {
#pragma unroll
        for (int j = P; j < NC; j += NP)
            *(u32x4_t *)(lds + ((j & 1) ? lds_odd : lds_even) + j * RSTEP * kRowBytes) = v[j];
    }
    template <int P, int NP>
    __device__ __forceinline__ void load_part(__amdgpu_buffer_rsrc_t r, int k_left)
    {
        if constexpr (P < NC) {
            const uint32_t base = opaque(kc < k_left ? goff : kOOB);
#pragma unroll
            for (int j = P; j < NC; j += NP)
                v[j] = bload16(r, base + (uint32_t)j * gstep);
        }
    }
};

// Row-contiguous storage ([k][row], rows contiguous): each thread loads KB
// consecutive k of 8 consecutive rows (KB x 16 B), transposes the KB x 8
// block in registers and writes 8 LDS rows of KB k each.  When KB < 8 a
// 16-byte LDS chunk (8 k of one row) holds S = 8 / KB threads' pieces; the
// S threads of one chunk are adjacent lanes, and the lanes above them take
// consecutive 8-row groups, so every load instruction still reads whole
// 128-byte segments of a k row.
template <int R, int NT>
struct Loader<R, NT, false> {
    static constexpr int NGR = R / 8;                                             // 8-row groups
    static constexpr int KB = (NGR * 8 >= NT) ? 8 : ((NGR * 16 >= NT) ? 4 : 2);   // k per block
    static constexpr int NKG = kBK / KB;                                           // k groups
    static constexpr int S = 8 / KB;                                               // pieces per chunk
    static_assert(R % 8 == 0 && NGR * NKG == NT, "transposing loader: one block per thread");
    u32x4_t v[KB];
    uint32_t goff;   // byte offset of this lane's first k row segment
    uint32_t gstep;  // bytes between consecutive k rows (uniform)
    int g, kg;       // 8-row group and k group of this lane

    __device__ __forceinline__ void init(int tid, int ld)
    {
        g = (tid / S) % NGR;
        kg = (tid / S) / NGR * S + tid % S;
        goff = (uint32_t)(kg * KB) * (uint32_t)ld * 2u + (uint32_t)g * 16u;
        gstep = (uint32_t)ld * 2u;
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int /*k_left*/)
    {
        // k past the end lies beyond the resource's records and reads as 0
        const uint32_t base = opaque(goff);
#pragma unroll
        for (int i = 0; i < KB; ++i)
            v[i] = bload16(r, base + (uint32_t)i * gstep);
    }
    // Bank order of the LDS writes.  The LDS serves a 64-lane write in
    // groups of 128 bytes (16 lanes of 8 bytes) on 32 banks; a tile row is
    // 128 bytes.  The lane mapping above puts the S pieces of each chunk in
    // one group, and the swizzle (j ^ g) & 7 sends the group's 8 row groups
    // to distinct chunks, so no group conflicts.  (With every 16-lane group on
    // one k piece the 128 x 128 tile's writes were two-way conflicts:
    // 294,912 cycles per 2048 x 2048 x 512 launch.)  Writing the group's
    // rows in the order j ^ flip, flip one lane bit above the groups of
    // 16, also keeps the writes free of conflicts where 32 lanes are served
    // at once on 64 banks, since each such set then writes both row parities
    // (both halves of the banks).
    __device__ __forceinline__ int flip() const { return KB == 2 ? (kg >> 2) & 1 : (g >> 3) & 1; }

    // LDS rows g*8 + (j ^ flip) for j in [J0, J1)
    template <int J0, int J1>
    __device__ __forceinline__ void store_rows(char *lds) const
    {
        const int f = flip();
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int jj = j ^ f;
            const int row = g * 8 + jj;
            const int d = j >> 1;   // = jj >> 1
            // the row's 16-bit halves of two k rows: lo16(a) | lo16(b) << 16
            // for even rows, hi16(a) | hi16(b) << 16 for odd rows
            const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
            auto pk = [&](uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, sel); };
            // swz(8g + jj) = (jj ^ g) & 7
            if constexpr (KB == 8) {
                u32x4_t o;
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    o[p] = pk(v[2 * p][d], v[2 * p + 1][d]);
                *(u32x4_t *)(lds + row * kRowBytes + ((kg ^ swz(row)) << 4)) = o;
            } else if constexpr (KB == 4) {
                u32x2_t o;
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    o[p] = pk(v[2 * p][d], v[2 * p + 1][d]);
                const int chunk = kg >> 1, sub = (kg & 1) * 8;
                *(u32x2_t *)(lds + row * kRowBytes + ((chunk ^ swz(row)) << 4) + sub) = o;
            } else {
                const uint32_t o = pk(v[0][d], v[1][d]);
                const int chunk = kg >> 2, sub = (kg & 3) * 4;
                *(uint32_t *)(lds + row * kRowBytes + ((chunk ^ swz(row)) << 4) + sub) = o;
            }
        }
    }
    __device__ __forceinline__ void store(char *lds) const { store_rows<0, 8>(lds); }
    template <int P, int NP>
    static constexpr int part_writes() { return 8 * (P + 1) / NP - 8 * P / NP; }
    template <int P, int NP>
    static constexpr int part_loads() { return P == NP - 1 ? KB : 0; }

    // NP parts: part P writes rows [8P/NP, 8(P+1)/NP); every row needs all KB
    // loaded registers, so the next step's loads go out with the last part.
    template <int P, int NP>
    __device__ __forceinline__ void store_part(char *lds) const
    {
        store_rows<8 * P / NP, 8 * (P + 1) / NP>(lds);
    }
    template <int P, int NP>
    __device__ __forceinline__ void load_part(__amdgpu_buffer_rsrc_t r, int k_left)
    {
        if constexpr (P == NP - 1)
            load(r, k_left);
    }
};

// Operand source: the tile's origin in global memory, the bytes that exist
// from there on, and how far one K step moves the origin.
struct OperandSrc {
    const char *base;
    uint64_t bytes;
    uint32_t step_bytes;  // 128 (k-contiguous) or 64 * ld * 2 (row-contiguous)
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t at_step(int kt) const
    {
        uint64_t adv = (uint64_t)kt * step_bytes;
        return make_rsrc(base + adv, bytes > adv ? bytes - adv : 0);
    }
};

// The same source in scalar registers (the fields are wave-uniform, but the
// compiler cannot always tell, and then builds every step's resource with
// vector compares).
__device__ __forceinline__ OperandSrc uniform_src(const OperandSrc &s)
{
    // (readfirstlane returns int: each half goes back through uint32_t, or
    // a low half with bit 31 set would sign-extend over the high half)
    auto u64 = [](uint64_t v) {
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
        return ((uint64_t)hi << 32) | (uint64_t)lo;
    };
    OperandSrc u;
    u.base = (const char *)(uintptr_t)u64((uint64_t)(uintptr_t)s.base);
    u.bytes = u64(s.bytes);
    u.step_bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)s.step_bytes);
    return u;
}

// The resource of a step that ends before the operand's last step: the base
// moved to the step, the length left as the rows bound it.  A k-contiguous
// operand's rows past the tile's last read as zero because their offsets
// pass the first step's length; a row-major B's lanes stay within one step
// of 64 rows, which such a step holds in full.  (No 64-bit compare: the
// scalar unit has none, so at_step's clamp runs on the vector unit.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t step_rsrc(const OperandSrc &u, bool kmajor, int kt)
{
    const uint64_t rec = kmajor ? u.bytes : (uint64_t)u.step_bytes;
    return make_rsrc(u.base + (uint64_t)kt * u.step_bytes, rec);
}

// ---------------------------------------------------------------------------
// The tile: accumulators, main loop, epilogue.
// ---------------------------------------------------------------------------

// Instruction interleave for one sub-step, as scheduling-group barriers:
// after MFMA i comes the i-th LDS read (the next sub-step's fragments, so
// they have the rest of the group to arrive), then the LDS writes of the
// staged step and, one slot later each, the global loads that refill those
// registers.  Groups the code does not have are simply empty.
enum : int { SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200 };

template <int I, int NM, int NR, int NW, int NV>
__device__ __forceinline__ void sched_pattern()
{
    if constexpr (I < NM) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        if constexpr (I < NR)
            __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
        else if constexpr (I - NR < NW)
            __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
        if constexpr (I - NR - 1 >= 0 && I - NR - 1 < NV)
            __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
        sched_pattern<I + 1, NM, NR, NW, NV>();
    }
}

template <int IN>
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c)
{
    if constexpr (IN == IN_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int BM_, int BN_, int WM_, int WN_, bool A_KMAJOR, bool B_KMAJOR, int IN, int NS_ = 2>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int MI = 32;   // MFMA block edge (v_mfma_f32_32x32x16)
    static constexpr int NS = NS_;  // staging register sets (global loads NS steps ahead)
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
    static constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA blocks per wave
    static constexpr int SLOT = (BM + BN) * kRowBytes;
    static constexpr int LDS_BYTES = 2 * SLOT;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");

    f32x16_t acc[FM][FN];

    // Accumulate the tile over k in [0, K).  sa: rows of A (M side),
    // sb: rows of B^T (N side).
    // tid: threadIdx.x, passed in (through opaque()) by the caller so that
    // per-lane address arithmetic is not hoisted out of the persistent tile
    // loop and held in registers across it.
    __device__ __forceinline__ void mainloop(char *lds, const OperandSrc &sa, int lda, const OperandSrc &sb, int ldb,
                                             int K, int tid, const RowGather &ga = RowGather{})
    {
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int wm0 = (wave / WN) * TM;
        const int wn0 = (wave % WN) * TN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = f32x16_t{};

        const int ksteps = (K + kBK - 1) / kBK;
        if (ksteps <= 0)
            return;
        // NS sets of staging registers: the set written to LDS in step k is
        // refilled with step k+1+NS at once, so each global load has NS full
        // K steps to arrive before its data is needed.  Narrow tiles, whose
        // sets are small and whose operands stream from HBM (few tokens
        // against a whole weight matrix), keep more steps in flight.
        Loader<BM, NT, A_KMAJOR> la[NS];
        Loader<BN, NT, B_KMAJOR> lb[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            la[s].init(tid, lda);
            lb[s].init(tid, ldb);
            if constexpr (A_KMAJOR) {
                if constexpr (Loader<BM, NT, true>::NC == 1) {
                    if (ga.idx)
                        la[s].gather(tid, lda, ga);
                }
            }
        }

        // Fragment read offsets.  Lane l reads row (l & 31) of a 32-row
        // block at 16-byte chunk 2*ks + (l >> 5).  Rows 32 apart differ in
        // swizzle by an XOR of 4 on the chunk, i.e. of 2 on ks, so block i
        // reads with base[ks ^ 2*(i & 1)] + 32*i rows.
        const int frow = lane & 31, fk = lane >> 5;
        int abase[4], bbase[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ra = wm0 + frow, rb = wn0 + frow;
            abase[ks] = ra * kRowBytes + (((2 * ks + fk) ^ swz(ra)) << 4);
            bbase[ks] = BM * kRowBytes + rb * kRowBytes + (((2 * ks + fk) ^ swz(rb)) << 4);
        }

        // Prologue: fetch steps 0 .. NS-1 into the sets, stage step 0 into
        // slot 0 and refill its set with step NS.  The loads go out part by
        // part in the same order as in the steady-state body, so the wait
        // counts the compiler derives for the loop are exact (waiting only
        // for the part about to be written).
#pragma unroll
        for (int s = 0; s < NS; ++s)
            load_parts(la[s], lb[s], sa.at_step(s), sb.at_step(s), K - s * kBK);
        la[0].store(lds);
        lb[0].store(lds + BM * kRowBytes);
        load_parts(la[0], lb[0], sa.at_step(NS), sb.at_step(NS), K - NS * kBK);
        lds_barrier();

        // Fragments are double-buffered: while the MFMAs of one 16-k
        // sub-step run from registers, the next sub-step's fragments are
        // already being read, so no MFMA waits on a fresh LDS read.
        Frags f0, f1;
        read_frags<0>(lds, abase, bbase, f0);

        // Every step runs the same branch-free body, NS steps per trip:
        // step kt writes step kt+1 (held in set (kt+1) % NS) into the other
        // slot and refills that set with step kt+1+NS.  Near the end those
        // loads fall past the operand's records (the hardware returns zeros
        // without touching memory) and the writes fill a slot nobody reads,
        // so no tail variants are needed.
        // A step count that is not a multiple of NS runs up to NS-1 extra
        // steps on all-zero slots (both operands read as zero past K), which
        // add exactly nothing.
        for (int kt = 0; kt < ksteps; kt += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u)
                step<true, true, true>(lds, kt + u, la[(u + 1) % NS], lb[(u + 1) % NS], sa, sb, K, abase, bbase, f0, f1);
        }
    }

    struct Frags {
        u32x4_t a[FM], b[FN];
    };

    __device__ __forceinline__ static void load_parts(Loader<BM, NT, A_KMAJOR> &la, Loader<BN, NT, B_KMAJOR> &lb,
                                                      __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int kleft)
    {
        la.template load_part<0, 3>(ra, kleft);
        lb.template load_part<0, 3>(rb, kleft);
        la.template load_part<1, 3>(ra, kleft);
        lb.template load_part<1, 3>(rb, kleft);
        la.template load_part<2, 3>(ra, kleft);
        lb.template load_part<2, 3>(rb, kleft);
    }
    using LoaderA = Loader<BM, NT, A_KMAJOR>;
    using LoaderB = Loader<BN, NT, B_KMAJOR>;
    template <int P> static constexpr int WA() { return LoaderA::template part_writes<P, 3>(); }
    template <int P> static constexpr int WB() { return LoaderB::template part_writes<P, 3>(); }
    template <int P> static constexpr int LA() { return LoaderA::template part_loads<P, 3>(); }
    template <int P> static constexpr int LB() { return LoaderB::template part_loads<P, 3>(); }

    template <int KS>
    __device__ __forceinline__ void read_frags(const char *slot, const int (&abase)[4], const int (&bbase)[4],
                                               Frags &f) const
    {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f.a[i] = *(const u32x4_t *)(slot + abase[KS ^ ((i & 1) * 2)] + i * 32 * kRowBytes);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            f.b[j] = *(const u32x4_t *)(slot + bbase[KS ^ ((j & 1) * 2)] + j * 32 * kRowBytes);
    }

    __device__ __forceinline__ void mfmas(const Frags &f)
    {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = mfma32<IN>(f.b[j], f.a[i], acc[i][j]);
    }

    // One K step on slot kt & 1; on entry f0 holds its first sub-step's
    // fragments, on exit (NEXT) f0 holds the next step's.
    //   STORE: write the staged registers (step kt+1) into the other slot,
    //          spread over sub-steps 0-2;
    //   LOAD:  after each part is written, fetch that part of step kt+1+NS into
    //          the same registers;
    //   NEXT:  after the barrier, read the next step's first fragments.
    // The barrier sits between the last fragment read of this step and the
    // last MFMA group, so that group covers the barrier and the next reads.
    template <bool STORE, bool LOAD, bool NEXT>
    __device__ __forceinline__ void step(char *lds, int kt, Loader<BM, NT, A_KMAJOR> &la, Loader<BN, NT, B_KMAJOR> &lb,
                                         const OperandSrc &sa, const OperandSrc &sb, int K, const int (&abase)[4],
                                         const int (&bbase)[4], Frags &f0, Frags &f1)
    {
        char *cur = lds + (kt & 1) * SLOT;
        char *nxt = lds + ((kt + 1) & 1) * SLOT;
        __amdgpu_buffer_rsrc_t ra2, rb2;
        if constexpr (LOAD) {
            ra2 = sa.at_step(kt + 1 + NS);
            rb2 = sb.at_step(kt + 1 + NS);
        }
        const int kleft2 = K - (kt + 1 + NS) * kBK;

        // sub-step 0
        read_frags<1>(cur, abase, bbase, f1);
        if constexpr (STORE) {
            la.template store_part<0, 3>(nxt);
            lb.template store_part<0, 3>(nxt + BM * kRowBytes);
        }
        if constexpr (LOAD) {
            la.template load_part<0, 3>(ra2, kleft2);
            lb.template load_part<0, 3>(rb2, kleft2);
        }
        mfmas(f0);
        sched_pattern<0, FM * FN, FM + FN, STORE ? WA<0>() + WB<0>() : 0, LOAD ? LA<0>() + LB<0>() : 0>();
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 1
        read_frags<2>(cur, abase, bbase, f0);
        if constexpr (STORE) {
            la.template store_part<1, 3>(nxt);
            lb.template store_part<1, 3>(nxt + BM * kRowBytes);
        }
        if constexpr (LOAD) {
            la.template load_part<1, 3>(ra2, kleft2);
            lb.template load_part<1, 3>(rb2, kleft2);
        }
        mfmas(f1);
        sched_pattern<0, FM * FN, FM + FN, STORE ? WA<1>() + WB<1>() : 0, LOAD ? LA<1>() + LB<1>() : 0>();
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 2
        read_frags<3>(cur, abase, bbase, f1);
        if constexpr (STORE) {
            la.template store_part<2, 3>(nxt);
            lb.template store_part<2, 3>(nxt + BM * kRowBytes);
        }
        if constexpr (LOAD) {
            la.template load_part<2, 3>(ra2, kleft2);
            lb.template load_part<2, 3>(rb2, kleft2);
        }
        mfmas(f0);
        sched_pattern<0, FM * FN, FM + FN, STORE ? WA<2>() + WB<2>() : 0, LOAD ? LA<2>() + LB<2>() : 0>();
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 3: every read of `cur` and write of `nxt` by this wave
        // is done; meet the other waves, then start on the next slot
        lds_barrier();
        if constexpr (NEXT)
            read_frags<0>(nxt, abase, bbase, f0);
        mfmas(f1);
        sched_pattern<0, FM * FN, NEXT ? FM + FN : 0, 0, 0>();
        __builtin_amdgcn_sched_barrier(0);
    }
};

// ---------------------------------------------------------------------------
// Direct-to-LDS tile: 256 x 256, both operands k-contiguous, eight waves.
//
// Global loads write LDS themselves (buffer_load ... lds: each lane's 16
// bytes land at M0 + 16 * lane), so no staging registers and no LDS-write
// instructions are involved -- the role the asynchronous tensor copy plays
// on the pages' hardware ("B200 的 2CTA 怎样调优", sections 四-五: the copy
// engine fills later K segments while the matrix unit works on the current
// one, and an issued copy is not yet usable data).  Without staging
// registers a wave needs ~80 VGPRs besides its accumulators, so the tile
// runs eight waves (two per SIMD, each 128 x 64 outputs, 128 accumulator
// registers): while one wave of a SIMD waits on a fragment read or the
// barrier, the other issues MFMAs.
//
// LDS (160 KiB): a three-slot ring for one operand ("deep": B when it is
// k-contiguous, else A) and a two-slot ring for the other, 32 KiB per
// operand step (256 rows x 128 bytes, chunks swizzled as in Tile).  During
// step k the deep operand's rows of step k+2 go into the slot freed by the
// barrier that ended step k-1, and right after the barrier that ends step k
// the other operand's rows of step k+2 go into the slot step k leaves: the
// deep operand has two steps to arrive, the other one.  The wait before
// each barrier names exactly the loads that must have landed: everything
// but this step's deep loads.
//
// One load instruction covers 8 rows x 128 bytes = 1 KiB of LDS, which is
// contiguous, so the swizzle is applied on the global side: lane l of row
// group g fetches logical chunk (l & 7) ^ swz(row) of row 8g + (l >> 3).
// Row and chunk offsets are per-lane VGPR offsets (range-checked against the
// resource, so rows past M or N read as zero); the LDS address is uniform.
template <int n>
__device__ __forceinline__ void wait_vm()
{
    // s_waitcnt with vmcnt = n (bits 3:0 and 15:14), expcnt and lgkmcnt not waited
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// One 16-byte-per-lane load from the buffer straight into LDS: lane l's
// bytes land at LDS address lds_addr + 16 l (lds_addr uniform).  Written as
// inline assembly rather than with the compiler's builtin for this load on
// purpose: the compiler's wait insertion cannot tell that a
// ds_read_b64_tr_b16 does not read what such a load is still writing, and
// puts a wait for every outstanding load (vmcnt(0)) before each transpose
// read, which throws away the ring's prefetch depth.  The loops that use
// this load count its completions themselves (s_waitcnt vmcnt before each
// barrier) and nothing else in them uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(voff),
                 "s"(r)
                 : "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const char *p) { return (uint32_t)(uintptr_t)(const lds_void_t *)p; }

typedef short i16x4_t __attribute__((ext_vector_type(4)));


template <int IN>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    if constexpr (IN == IN_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// The direct-to-LDS 256 x 256 tile.  MFMA v_mfma_f32_16x16x32 (under
// sustained load it runs ~11 % more FLOP/s than v_mfma_f32_32x32x16 at the
// power-managed clock: 1944-1976 against 1746-1790 TFLOP/s in a
// register-only loop); each wave's 128 x 64 outputs are 8 x 4 blocks of
// 16 x 16 (4 accumulators per lane each).  A 64-k step is two 32-k
// sub-steps, each run as two halves of 16 MFMAs (m blocks 0-3, then 4-7).
// A fragments rotate through two sets of four (X, Y) and B fragments
// through two (P, Q), each set read one half-step before its MFMAs:
//   half 0: MFMAs X.P (s0, m 0-3), reads Y = A(s0, m 4-7), Q = B(s1)
//   half 1: MFMAs Y.P (s0, m 4-7), reads X = A(s1, m 0-3)
//   half 2: MFMAs X.Q (s1, m 0-3), reads Y = A(s1, m 4-7)
//   half 3: barrier, then MFMAs Y.Q, reads X = A'(s0, m 0-3), P = B'(s0)
// Operand lanes: lane l holds row (l mod 16), k 8(l/16) .. 8(l/16)+7 of the
// 32-k block; B is the instruction's first operand, so the accumulator of
// lane l holds output row (l mod 16) of the block, columns 4(l/16) .. +3.
// BKM: B k-contiguous ([n][k], column-major B).  Otherwise B is row-major
// ([k][n]) and is kept that way in LDS: 64 rows of 512 bytes per step, its
// fragments read with ds_read_b64_tr_b16.  Within each group of 16 lanes
// that instruction hands lane i the elements (4j + i/4, i % 4), j = 0..3,
// of the 16 x 4 block formed by the lanes' 8-byte pieces; so when lane
// 4j + q of the group points at B[k0 + j][n0 + 4q .. n0 + 4q + 3], lane i
// receives B[k0 .. k0 + 3][n0 + i], and two reads give the eight k of a
// lane.  The 64-byte segments of row k are XOR-permuted by (k & 3), so the
// four rows one group reads fall in distinct bank groups, and the 32-byte
// halves of each segment are swapped on bit 3 of k, so that the groups
// reading k rows 8 apart (0/1, 2/3) use disjoint banks.
template <int IN, bool BKM>
struct DtlTile {
    static constexpr int BM = 256, BN = 256, WM = 2, WN = 4;
    static constexpr int MI = 16;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    static constexpr int OPS = 256 * kRowBytes;
    static constexpr bool DEEP_B = BKM;
    static constexpr int A_SLOTS = DEEP_B ? 2 : 3, B_SLOTS = DEEP_B ? 3 : 2;
    static constexpr int LDS_BYTES = (A_SLOTS + B_SLOTS) * OPS;
    static constexpr int LOADS = 256 / 8 / (NT / 64);
    static constexpr int BROW = 512;
    static_assert(FM == 8 && FN == 4, "the half-step rotation assumes 8 x 4 blocks per wave");

    f32x4_t acc[FM][FN];
    struct F4 {
        u32x4_t v[4];
    };

    uint32_t va[LOADS], vb[LOADS];
    int kc[LOADS];
    int abase[2], bbase[2];   // k-contiguous fragments of sub-step s (any block: add 16 rows per block)

    // Chunk swizzle of this tile's 128-byte rows: bits (r1, r0 ^ r3, r2) of
    // the row.  The LDS serves a 16-byte read to lanes l and l + 32 in the
    // same cycle (with 64 four-byte banks); those lanes read one row at
    // chunks c and c ^ 2, so the eight rows an 8-lane group reads must have
    // swizzles in distinct classes of {x, x ^ 2} among rows of one parity:
    // r1 and r2 give that, and r0 ^ r3 keeps 16 consecutive rows apart as
    // well.  (Tile's swz gives rows 0, 2, 4, 6 the values 0, 2, 4, 6: a
    // two-way conflict for this operand layout, measured.)  It depends on
    // the low four bits only, so blocks 16 rows apart share it.
    static __device__ __forceinline__ int dswz(int row)
    {
        return ((row >> 1) & 1) | ((((row) ^ (row >> 3)) & 1) << 1) | (((row >> 2) & 1) << 2);
    }
    int bfr[4];               // row-major B: transpose-read piece of n block jb (s = 0, h = 0)

    __device__ __forceinline__ void setup(int lane, int wave, int wm0, int wn0, int lda, int ldb)
    {
        const int r8 = lane >> 3;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int row = (wave * LOADS + j) * 8 + r8;
            const int c = (lane & 7) ^ dswz(row);
            kc[j] = c * 8;
            va[j] = (uint32_t)row * (uint32_t)lda * 2u + (uint32_t)c * 16u;
            if constexpr (BKM) {
                vb[j] = (uint32_t)row * (uint32_t)ldb * 2u + (uint32_t)c * 16u;
            } else {
                const int kr = (wave * LOADS + j) * 2 + (lane >> 5);
                const int pc = lane & 31;
                const int seg = (pc >> 2) ^ (kr & 3);
                const int w = (pc & 3) ^ (((kr >> 3) & 1) << 1);
                vb[j] = (uint32_t)kr * (uint32_t)ldb * 2u + (uint32_t)(seg * 64 + w * 16);
            }
        }
        const int r = lane & 15, q = lane >> 4;
        const int c0 = q ^ dswz(r);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            abase[s] = (wm0 + r) * kRowBytes + ((c0 ^ (4 * s)) << 4);
            bbase[s] = (wn0 + r) * kRowBytes + ((c0 ^ (4 * s)) << 4);
        }
        if constexpr (!BKM) {
            const int jj = r >> 2, qq = r & 3;
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                bfr[jb] = (8 * q + jj) * BROW + ((((wn0 >> 5) + (jb >> 1)) ^ jj) * 64) +
                          ((32 * (jb & 1) + 8 * qq) ^ (32 * (q & 1)));
        }
    }
    static __device__ __forceinline__ void dtl_load(__amdgpu_buffer_rsrc_t r, char *dst, uint32_t off)
    {
        if constexpr (BKM)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, off, 0, 0, 0);
        else
            load_to_lds16(r, lds_addr(dst), off);
    }
    // MASK: the step may end past K (a k-contiguous operand's chunks past K
    // must read as zero; a row-contiguous operand's resource already ends
    // at row K - 1).  Steps that end before the last skip the per-lane select.
    template <bool MASK = true>
    __device__ __forceinline__ void load_a(__amdgpu_buffer_rsrc_t r, char *slot, int wave, int j, int k_left) const
    {
        const uint32_t off = !MASK || kc[j] < k_left ? va[j] : kOOB;
        dtl_load(r, slot + (wave * LOADS + j) * 1024, off);
    }
    template <bool MASK = true>
    __device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t r, char *slot, int wave, int j, int k_left) const
    {
        uint32_t off = vb[j];
        if constexpr (BKM && MASK)
            off = kc[j] < k_left ? off : kOOB;
        dtl_load(r, slot + (wave * LOADS + j) * 1024, off);
    }

    // A fragments of m blocks 4 HM .. 4 HM + 3, sub-step S
    template <int S, int HM>
    __device__ __forceinline__ void read_a(const char *as, F4 &f) const
    {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            f.v[ii] = *(const u32x4_t *)(as + abase[S] + (4 * HM + ii) * 16 * kRowBytes);
    }
    // B fragments of the four n blocks, sub-step S
    template <int S>
    __device__ __forceinline__ void read_b(const char *bs, F4 &f) const
    {
        if constexpr (BKM) {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                f.v[jb] = *(const u32x4_t *)(bs + bbase[S] + jb * 16 * kRowBytes);
        } else {
            typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const char *p = bs + bfr[jb] + 32 * S * BROW;
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * BROW));
                const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
                f.v[jb] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
            }
        }
    }
    template <int HM>
    __device__ __forceinline__ void mfmas(const F4 &a, const F4 &b)
    {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                acc[4 * HM + ii][jb] = mfma16<IN>(b.v[jb], a.v[ii], acc[4 * HM + ii][jb]);
    }
    template <int I, int NR, int NV>
    static __device__ __forceinline__ void pattern()
    {
        constexpr int NM = 16;
        if constexpr (I < NM) {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            if constexpr (I < NR)
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
            if constexpr (NV > 0 && I % (NM / (NV > 0 ? NV : 1)) == 0 && I / (NM / (NV > 0 ? NV : 1)) < NV)
                __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
            pattern<I + 1, NR, NV>();
        }
    }
    static constexpr int RB = BKM ? 4 : 8;   // LDS read instructions for the four B fragments

    __device__ __forceinline__ void mainloop(char *lds, const OperandSrc &sa, int lda, const OperandSrc &sb, int ldb,
                                             int K, int tid, const RowGather &ga = RowGather{})
    {
        static_assert(LOADS % 2 == 0, "loads are issued in halves");
        constexpr int H = LOADS / 2;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm0 = (wave / WN) * TM, wn0 = (wave % WN) * TN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = f32x4_t{};
        const int ksteps = (K + kBK - 1) / kBK;
        if (ksteps <= 0)
            return;
        setup(lane, wave, wm0, wn0, lda, ldb);
        if (ga.idx) {
            // A's rows through the index: the same chunk of another row
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                const int row = (wave * LOADS + j) * 8 + (lane >> 3);
                const uint32_t ro = ga.row_offset(row, lda);
                va[j] = ro == kOOB ? kOOB : ro + (uint32_t)((lane & 7) ^ dswz(row)) * 16u;
            }
        }
        char *const A0 = lds;
        char *const B0 = lds + A_SLOTS * OPS;
        char *const D0 = DEEP_B ? B0 : A0;
        char *const S0 = DEEP_B ? A0 : B0;
        const OperandSrc ua = uniform_src(sa), ub = uniform_src(sb);
        const OperandSrc &sd = DEEP_B ? ub : ua;
        const OperandSrc &ss = DEEP_B ? ua : ub;
        constexpr bool D_KMAJOR = DEEP_B ? BKM : true, S_KMAJOR = DEEP_B ? true : BKM;
        auto load_d = [&](__amdgpu_buffer_rsrc_t r, char *slot, int j, int k_left, auto mask) {
            if constexpr (DEEP_B)
                load_b<decltype(mask)::value>(r, slot, wave, j, k_left);
            else
                load_a<decltype(mask)::value>(r, slot, wave, j, k_left);
        };
        auto load_s = [&](__amdgpu_buffer_rsrc_t r, char *slot, int j, int k_left, auto mask) {
            if constexpr (DEEP_B)
                load_a<decltype(mask)::value>(r, slot, wave, j, k_left);
            else
                load_b<decltype(mask)::value>(r, slot, wave, j, k_left);
        };
        constexpr std::true_type masked{};
        constexpr std::false_type unmasked{};
        // prologue: both operands of steps 0 and 1; wait for step 0
        {
            const auto rd0 = sd.at_step(0), rs0 = ss.at_step(0), rd1 = sd.at_step(1), rs1 = ss.at_step(1);
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                load_d(rd0, D0, j, K, masked);
                load_s(rs0, S0, j, K, masked);
            }
#pragma unroll
            for (int j = 0; j < LOADS; ++j)
                load_d(rd1, D0 + OPS, j, K - kBK, masked);
#pragma unroll
            for (int j = 0; j < LOADS; ++j)
                load_s(rs1, S0 + OPS, j, K - kBK, masked);
            wait_vm<2 * LOADS>();
        }
        lds_barrier();
        F4 X, Y, P, Q;
        read_a<0, 0>(A0, X);
        read_b<0>(B0, P);
        int sd_cur = 0, sd_next = 1, sd_fill = 2;   // deep slots of steps kt, kt+1, kt+2
        // one K step; its loads are of step kt + 2
        auto step = [&](int kt, auto mask) {
            constexpr bool M = decltype(mask)::value;
            const int s_cur = kt & 1, s_next = (kt + 1) & 1;
            const char *ac = (DEEP_B ? S0 + s_cur * OPS : D0 + sd_cur * OPS);
            const char *bc = (DEEP_B ? D0 + sd_cur * OPS : S0 + s_cur * OPS);
            const char *an = (DEEP_B ? S0 + s_next * OPS : D0 + sd_next * OPS);
            const char *bn = (DEEP_B ? D0 + sd_next * OPS : S0 + s_next * OPS);
            char *dw = D0 + sd_fill * OPS;
            char *sw = S0 + s_cur * OPS;
            const auto rD = M ? sd.at_step(kt + 2) : step_rsrc(sd, D_KMAJOR, kt + 2);
            const int kd = K - (kt + 2) * kBK;
            // half 0 (sub-step 0, m blocks 0-3): the deep operand's first loads
            read_a<0, 1>(ac, Y);
            read_b<1>(bc, Q);
#pragma unroll
            for (int j = 0; j < H; ++j)
                load_d(rD, dw, j, kd, mask);
            mfmas<0>(X, P);
            pattern<0, 4 + RB, H>();
            __builtin_amdgcn_sched_barrier(0);
            // half 1 (sub-step 0, m blocks 4-7)
            read_a<1, 0>(ac, X);
#pragma unroll
            for (int j = H; j < LOADS; ++j)
                load_d(rD, dw, j, kd, mask);
            mfmas<1>(Y, P);
            pattern<0, 4, H>();
            __builtin_amdgcn_sched_barrier(0);
            // half 2 (sub-step 1, m blocks 0-3): the last reads of step kt
            read_a<1, 1>(ac, Y);
            mfmas<0>(X, Q);
            pattern<0, 4, 0>();
            __builtin_amdgcn_sched_barrier(0);
            // half 3 (sub-step 1, m blocks 4-7): step kt+1 must be in LDS and
            // every wave done with step kt; then the 2-slot operand of step
            // kt+2 goes into the slot step kt leaves
            wait_vm<LOADS>();
            lds_barrier();
            read_a<0, 0>(an, X);
            read_b<0>(bn, P);
            {
                const auto rS = M ? ss.at_step(kt + 2) : step_rsrc(ss, S_KMAJOR, kt + 2);
                const int ks2 = K - (kt + 2) * kBK;
#pragma unroll
                for (int j = 0; j < LOADS; ++j)
                    load_s(rS, sw, j, ks2, mask);
            }
            mfmas<1>(Y, Q);
            pattern<0, 4 + RB, LOADS>();
            __builtin_amdgcn_sched_barrier(0);
            const int t = sd_cur;
            sd_cur = sd_next;
            sd_next = sd_fill;
            sd_fill = t;
        };
        // the loads of step kt + 2 need no K mask while that step is not
        // the last (kt + 2 <= ksteps - 2)
        int kt = 0;
        for (; kt < ksteps - 3; ++kt)
            step(kt, unmasked);
        for (; kt < ksteps; ++kt)
            step(kt, masked);
        // the trailing loads (empty ranges) have landed before the next tile
        wait_vm<0>();
    }
};

// acc += a . b on the matrix cores with the accumulator held in AGPRs.
// Written as assembly because the compiler, left to place 256 accumulator
// registers per lane itself, moves accumulators between AGPRs and VGPRs
// around most MFMAs (hundreds of copies per K step).  The statements are
// volatile so they keep their order with the LDS reads and loads placed
// between them.  The compiler waits for the LDS reads that feed a and b
// (it sees the registers) but inserts no wait states after these MFMAs,
// so whoever reads the accumulators with other instructions waits first
// (mfma_drain).
template <int IN>
__device__ __forceinline__ void mfma16_agpr(f32x4_t &c, const u32x4_t &a, const u32x4_t &b)
{
    if constexpr (IN == IN_BF16)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// More wait states than any MFMA result needs before other instructions
// read it, and no instruction scheduled across.
__device__ __forceinline__ void mfma_drain()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

// The same 256 x 256 direct-to-LDS tile on four waves of 128 x 128 (8 x 8
// blocks of 16 x 16, 256 accumulators per lane in AGPRs, one wave per
// SIMD): each wave reads 128 rows of A and 128 of B per 32-k sub-step for
// 64 MFMAs, two thirds of the LDS reads per MFMA of the eight-wave layout.
// Rings, swizzles and fragment addressing are DtlTile's.  A sub-step is four
// quarters of 16 MFMAs; the fragments of the next sub-step are read into the
// other set, four reads (eight transpose reads) per quarter, one after each
// of the quarter's first MFMAs:
//   sub-step 0 (X.P): reads Y = A(s1), Q = B(s1) of step kt
//   barrier (step kt+1 in LDS; every wave done with step kt's slots), then
//   sub-step 1 (Y.Q): reads X = A(s0), P = B(s0) of step kt+1, and loads
//     the shallow operand's step kt+2 (first quarter) and the deep one's
//     step kt+3 (second quarter) into the slots step kt leaves.
// The shallow operand thus has one step of lead, the deep one two.
template <int IN, bool BKM>
struct DtlTile4 {
    using Base = DtlTile<IN, BKM>;
    static constexpr int BM = 256, BN = 256, WM = 2, WN = 2;
    static constexpr int MI = 16;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    static constexpr int OPS = Base::OPS;
    static constexpr bool DEEP_B = BKM;
    static constexpr int A_SLOTS = Base::A_SLOTS, B_SLOTS = Base::B_SLOTS;
    static constexpr int LDS_BYTES = Base::LDS_BYTES;
    static constexpr int LOADS = 256 / 8 / (NT / 64);
    static constexpr int BROW = Base::BROW;
    static constexpr int RB = Base::RB;   // LDS read instructions per four B fragments
    static_assert(FM == 8 && FN == 8 && LOADS == 8, "the quarter rotation assumes 8 x 8 blocks per wave");
    using F4 = typename Base::F4;

    f32x4_t acc[FM][FN];
    uint32_t va[LOADS], vb[LOADS];
    int kc[LOADS];
    int abase[2], bbase[2];
    int bfr[FN];
    // LDS byte addresses of the 2-slot operand's fragments, per slot: A
    // (column-major B) or the transpose-read pieces of B (row-major B)
    uint32_t a_sh[2][2];
    uint32_t b_sh[2][FN];

    __device__ __forceinline__ void setup(int lane, int wave, int wm0, int wn0, int lda, int ldb)
    {
        const int r8 = lane >> 3;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int row = (wave * LOADS + j) * 8 + r8;
            const int c = (lane & 7) ^ Base::dswz(row);
            kc[j] = c * 8;
            va[j] = (uint32_t)row * (uint32_t)lda * 2u + (uint32_t)c * 16u;
            if constexpr (BKM) {
                vb[j] = (uint32_t)row * (uint32_t)ldb * 2u + (uint32_t)c * 16u;
            } else {
                const int kr = (wave * LOADS + j) * 2 + (lane >> 5);
                const int pc = lane & 31;
                const int seg = (pc >> 2) ^ (kr & 3);
                const int w = (pc & 3) ^ (((kr >> 3) & 1) << 1);
                vb[j] = (uint32_t)kr * (uint32_t)ldb * 2u + (uint32_t)(seg * 64 + w * 16);
            }
        }
        const int r = lane & 15, q = lane >> 4;
        const int c0 = q ^ Base::dswz(r);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            abase[s] = (wm0 + r) * kRowBytes + ((c0 ^ (4 * s)) << 4);
            bbase[s] = (wn0 + r) * kRowBytes + ((c0 ^ (4 * s)) << 4);
        }
        if constexpr (!BKM) {
            const int jj = r >> 2, qq = r & 3;
#pragma unroll
            for (int jb = 0; jb < FN; ++jb)
                bfr[jb] = (8 * q + jj) * BROW + ((((wn0 >> 5) + (jb >> 1)) ^ jj) * 64) +
                          ((32 * (jb & 1) + 8 * qq) ^ (32 * (q & 1)));
        }
    }
    // MASK: the step may end past K (a k-contiguous operand's chunks past K
    // must read as zero; a row-contiguous operand's resource already ends
    // at row K - 1).  Steps that end at or before K skip the per-lane select.
    template <bool MASK>
    __device__ __forceinline__ void load_a(__amdgpu_buffer_rsrc_t r, char *slot, int wave, int j, int k_left) const
    {
        const uint32_t off = !MASK || kc[j] < k_left ? va[j] : kOOB;
        load_to_lds16(r, lds_addr(slot + (wave * LOADS + j) * 1024), off);
    }
    template <bool MASK>
    __device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t r, char *slot, int wave, int j, int k_left) const
    {
        uint32_t off = vb[j];
        if constexpr (BKM && MASK)
            off = kc[j] < k_left ? off : kOOB;
        load_to_lds16(r, lds_addr(slot + (wave * LOADS + j) * 1024), off);
    }
    // LDS read number i of the A fragments of m blocks 4 H .. 4 H + 3, sub-step S
    template <int S, int H>
    __device__ __forceinline__ void read_a(const char *as, F4 &f, int i) const
    {
        f.v[i] = *(const u32x4_t *)(as + abase[S] + (4 * H + i) * 16 * kRowBytes);
    }
    // LDS read number i (of RB) of the B fragments of n blocks 4 H .. 4 H + 3, sub-step S
    template <int S, int H>
    __device__ __forceinline__ void read_b(const char *bs, F4 &f, int i) const
    {
        if constexpr (BKM) {
            f.v[i] = *(const u32x4_t *)(bs + bbase[S] + (4 * H + i) * 16 * kRowBytes);
        } else {
            typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
            const int jb = i >> 1, hi = i & 1;
            const char *p = bs + bfr[4 * H + jb] + 32 * S * BROW + 4 * BROW * hi;
            const u32x2_t w = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
            f.v[jb][2 * hi] = w[0];
            f.v[jb][2 * hi + 1] = w[1];
        }
    }
    // The same reads with the slot known: Q = the 2-slot operand's slot
    // (0 or 1), so the address is a register set up once plus an immediate
    // offset; Q < 0, or the 3-slot operand: through the slot pointer.
    template <int Q, int S, int H>
    __device__ __forceinline__ void rd_a(const char *as, F4 &f, int i) const
    {
        if constexpr (BKM && Q >= 0) {
            typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
            f.v[i] = *(const lds_u32x4 *)(uintptr_t)(a_sh[Q][S] + (4 * H + i) * 16 * kRowBytes);
        } else {
            read_a<S, H>(as, f, i);
        }
    }
    template <int Q, int S, int H>
    __device__ __forceinline__ void rd_b(const char *bs, F4 &f, int i) const
    {
        if constexpr (!BKM && Q >= 0) {
            typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
            const int jb = i >> 1, hi = i & 1;
            const uint32_t a = b_sh[Q][4 * H + jb] + 32 * S * BROW + 4 * BROW * hi;
            const u32x2_t w =
                __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)a));
            f.v[jb][2 * hi] = w[0];
            f.v[jb][2 * hi + 1] = w[1];
        } else {
            read_b<S, H>(bs, f, i);
        }
    }
    // 16 MFMAs on m blocks 4 HM .. +3 x n blocks 4 HN .. +3; read i (of NR)
    // after MFMA i, global load j (of NL) after MFMA j * 16 / NL
    static constexpr int LOFF = 2;   // MFMA after which a quarter's first load goes
    template <int HM, int HN, int NR, int NL, class RD, class LD>
    __device__ __forceinline__ void quarter(const F4 &a, const F4 &b, RD &&rd, LD &&ld)
    {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mfma16_agpr<IN>(acc[4 * HM + i / 4][4 * HN + i % 4], b.v[i % 4], a.v[i / 4]);
            if (i % (16 / NR) == 0)
                rd(i / (16 / NR));
            if constexpr (NL > 0) {
                if (i % (16 / NL) == LOFF)
                    ld(i / (16 / NL));
            }
        }
    }

    __device__ __forceinline__ void mainloop(char *lds, const OperandSrc &sa, int lda, const OperandSrc &sb, int ldb,
                                             int K, int tid)
    {
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm0 = (wave / WN) * TM, wn0 = (wave % WN) * TN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = f32x4_t{};
        const int ksteps = (K + kBK - 1) / kBK;
        if (ksteps <= 0)
            return;
        // the zeros are written here, ahead of the wait states before the
        // first MFMA (the compiler would otherwise sink them next to it)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                asm volatile("" : "+a"(acc[i][j]));
        setup(lane, wave, wm0, wn0, lda, ldb);
        char *const A0 = lds;
        char *const B0 = lds + A_SLOTS * OPS;
        char *const D0 = DEEP_B ? B0 : A0;
        char *const S0 = DEEP_B ? A0 : B0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t slot = lds_addr(S0 + q * OPS);
            if constexpr (BKM) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    a_sh[q][s] = slot + (uint32_t)abase[s];
            } else {
#pragma unroll
                for (int jb = 0; jb < FN; ++jb)
                    b_sh[q][jb] = slot + (uint32_t)bfr[jb];
            }
        }
        const OperandSrc ua = uniform_src(sa), ub = uniform_src(sb);
        const OperandSrc &sd = DEEP_B ? ub : ua;
        const OperandSrc &ss = DEEP_B ? ua : ub;
        constexpr bool D_KMAJOR = DEEP_B ? BKM : true, S_KMAJOR = DEEP_B ? true : BKM;
        auto load_d = [&](__amdgpu_buffer_rsrc_t r, char *slot, int j, int k_left, auto mask) {
            if constexpr (DEEP_B)
                load_b<decltype(mask)::value>(r, slot, wave, j, k_left);
            else
                load_a<decltype(mask)::value>(r, slot, wave, j, k_left);
        };
        auto load_s = [&](__amdgpu_buffer_rsrc_t r, char *slot, int j, int k_left, auto mask) {
            if constexpr (DEEP_B)
                load_a<decltype(mask)::value>(r, slot, wave, j, k_left);
            else
                load_b<decltype(mask)::value>(r, slot, wave, j, k_left);
        };
        constexpr std::true_type masked{};
        constexpr std::false_type unmasked{};
        // prologue: steps 0 and 1 of both operands; wait for step 0
        {
            const auto rd0 = sd.at_step(0), rs0 = ss.at_step(0), rd1 = sd.at_step(1), rs1 = ss.at_step(1);
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                load_d(rd0, D0, j, K, masked);
                load_s(rs0, S0, j, K, masked);
            }
#pragma unroll
            for (int j = 0; j < LOADS; ++j)
                load_d(rd1, D0 + OPS, j, K - kBK, masked);
#pragma unroll
            for (int j = 0; j < LOADS; ++j)
                load_s(rs1, S0 + OPS, j, K - kBK, masked);
            wait_vm<2 * LOADS>();
        }
        lds_barrier();
        F4 Xl, Xh, Pl, Ph, Yl, Yh, Ql, Qh;
        // (in the order the loop reads them, so that the LDS-read counts
        // at the loop head agree on both ways in)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            read_a<0, 0>(A0, Xl, i);
#pragma unroll
        for (int i = 0; i < RB; ++i)
            read_b<0, 0>(B0, Pl, i);
#pragma unroll
        for (int i = 0; i < RB; ++i)
            read_b<0, 1>(B0, Ph, i);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            read_a<0, 1>(A0, Xh, i);
        // the zeroed accumulators are written by ordinary instructions
        mfma_drain();
        int sd_cur = 0;   // deep slot of step kt
        // one K step; its loads are of step kt + 2.  par: the 2-slot
        // operand's slot of step kt when known at compile time (else -1)
        auto step = [&](int kt, auto mask, auto par) {
            constexpr int P = decltype(par)::value;
            constexpr int QC = P, QN = P < 0 ? -1 : (P ^ 1);
            const int s_cur = P < 0 ? (kt & 1) : P;
            const int sd_next = sd_cur == 2 ? 0 : sd_cur + 1;
            const int sd_fill = sd_next == 2 ? 0 : sd_next + 1;
            const char *ac = DEEP_B ? S0 + s_cur * OPS : D0 + sd_cur * OPS;
            const char *bc = DEEP_B ? D0 + sd_cur * OPS : S0 + s_cur * OPS;
            const char *an = DEEP_B ? S0 + (s_cur ^ 1) * OPS : D0 + sd_next * OPS;
            const char *bn = DEEP_B ? D0 + sd_next * OPS : S0 + (s_cur ^ 1) * OPS;
            // sub-step 0; the deep operand's step kt+2, two loads a quarter,
            // into the slot step kt-1 left
            const auto rD = decltype(mask)::value ? sd.at_step(kt + 2) : step_rsrc(sd, D_KMAJOR, kt + 2);
            const int kd = K - (kt + 2) * kBK;
            char *const dw = D0 + sd_fill * OPS;
            quarter<0, 0, 4, 2>(Xl, Pl, [&](int i) { rd_a<QC, 1, 0>(ac, Yl, i); },
                                [&](int j) { load_d(rD, dw, j, kd, mask); });
            quarter<0, 1, RB, 2>(Xl, Ph, [&](int i) { rd_b<QC, 1, 0>(bc, Ql, i); },
                                 [&](int j) { load_d(rD, dw, 2 + j, kd, mask); });
            quarter<1, 0, RB, 2>(Xh, Pl, [&](int i) { rd_b<QC, 1, 1>(bc, Qh, i); },
                                 [&](int j) { load_d(rD, dw, 4 + j, kd, mask); });
            quarter<1, 1, 4, 2>(Xh, Ph, [&](int i) { rd_a<QC, 1, 1>(ac, Yh, i); },
                                [&](int j) { load_d(rD, dw, 6 + j, kd, mask); });
            wait_vm<LOADS>();
            lds_barrier();
            // sub-step 1; the shallow operand's step kt+2 into the slot step
            // kt leaves
            const auto rS = decltype(mask)::value ? ss.at_step(kt + 2) : step_rsrc(ss, S_KMAJOR, kt + 2);
            const int ks = K - (kt + 2) * kBK;
            char *const sw = S0 + s_cur * OPS;
            quarter<0, 0, 4, 4>(Yl, Ql, [&](int i) { rd_a<QN, 0, 0>(an, Xl, i); },
                                [&](int j) { load_s(rS, sw, j, ks, mask); });
            quarter<0, 1, RB, 4>(Yl, Qh, [&](int i) { rd_b<QN, 0, 0>(bn, Pl, i); },
                                 [&](int j) { load_s(rS, sw, 4 + j, ks, mask); });
            quarter<1, 0, RB, 0>(Yh, Ql, [&](int i) { rd_b<QN, 0, 1>(bn, Ph, i); }, [](int) {});
            quarter<1, 1, 4, 0>(Yh, Qh, [&](int i) { rd_a<QN, 0, 1>(an, Xh, i); }, [](int) {});
            sd_cur = sd_next;
        };
        // Steps two at a time while the loads of step kt + 2 need no K mask
        // (kt + 2 <= ksteps - 2), each with its 2-slot slot fixed; the rest
        // (at most four) with the mask and the slot computed.
        int kt = 0;
        for (; kt + 1 < ksteps - 3; kt += 2) {
            step(kt, unmasked, std::integral_constant<int, 0>{});
            step(kt + 1, unmasked, std::integral_constant<int, 1>{});
        }
        for (; kt < ksteps; ++kt)
            step(kt, masked, std::integral_constant<int, -1>{});
        // the trailing loads (empty ranges) have landed before the next tile,
        // and the last MFMAs' results before the epilogue reads them
        wait_vm<0>();
        mfma_drain();
    }
};

// acc += a . b over 128 k of E4M3 (OCP FP8, 1-4-3) on the matrix cores,
// accumulator in AGPRs (same reasons as mfma16_agpr).  Operand lanes: lane l
// holds row (l mod 16) and 32 of the 128 k; the same (lane, byte) -> k
// assignment holds for both operands, so any one permutation of the 128 k
// applied to both gives the same sum.
__device__ __forceinline__ void mfma16_e4m3_agpr(f32x4_t &c, const u32x8_t &a, const u32x8_t &b)
{
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// The same with E8M0 block scales applied inside the instruction
// (v_mfma_scale_f32_16x16x128_f8f6f4): every lane's scale register scales
// the 32 k of its own row that the lane holds, for each operand (measured:
// a probe of distinct powers of two per lane recovers exactly this
// pairing), and BYTE selects which byte of each scale register is read.
template <int BYTE>
__device__ __forceinline__ void mfma16_e4m3_scaled_agpr(f32x4_t &c, const u32x8_t &a, const u32x8_t &b,
                                                        uint32_t scale_a, uint32_t scale_b)
{
    static_assert(BYTE == 0 || BYTE == 1, "");
    if constexpr (BYTE == 0)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                     : "+a"(c)
                     : "v"(a), "v"(b), "v"(scale_a), "v"(scale_b));
    else
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,1,0] op_sel_hi:[0,0,0]"
                     : "+a"(c)
                     : "v"(a), "v"(b), "v"(scale_a), "v"(scale_b));
}

// Two consecutive E8M0 scale bytes (two K steps) into bytes 0 and 1 of a
// register (buffer_load_ushort, the rest zero; the whole byte offset is in
// the per-lane offset, none in soffset, so the resource's range check
// covers all of it).  Written as assembly, like the direct-to-LDS loads, so
// that the compiler's wait insertion does not wait for every outstanding
// load before the register is read; the loops that use it count its
// completion themselves, and nothing may read the register before that.
__device__ __forceinline__ void load_scale_pair(uint32_t &reg, __amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    asm volatile("buffer_load_ushort %0, %1, %2, 0 offen" : "=v"(reg) : "v"(voff), "s"(r));
}

// Keep byte 0 only (the second step of the pair lies past K): after the
// load has been counted complete; two wait states before a matrix
// instruction reads the register.
__device__ __forceinline__ void keep_low_scale(uint32_t &reg)
{
    asm volatile("v_and_b32 %0, 0xff, %0\n\ts_nop 1" : "+v"(reg));
}

// Where a tile's block scales live (the blockwise E4M3 product): A's, one
// byte per (row, 128-k block), rows of lds_a bytes from the tile's first
// row; B's, one per (128 output columns, 128-k block), rows of lds_b bytes.
struct BlockScaleSrc {
    __amdgpu_buffer_rsrc_t ra;   // A scales from the tile's row 0 (rows past M out of range)
    __amdgpu_buffer_rsrc_t rb;   // B scales, all column blocks
    int lds_a;
    int lds_b;
    int nblk0;                   // column block of the tile's first column (n0 / 128)
    int kb;                      // k blocks (ceil(K / 128))
};

// The four-wave 256 x 256 direct-to-LDS tile for E4M3 inputs, A and B both
// k-contiguous ([M][K] and [N][K]).  A K step is 128 elements = 128 bytes of
// each tile row, so the rings (A on two slots, B on three), the global-side
// swizzle and the load assignment are the 16-bit tile's.  What differs is
// the MFMA: v_mfma_f32_16x16x128_f8f6f4 takes a whole step's 128 k per
// block at once (32 bytes per lane: the lane's chunk q and chunk q + 4 of
// the row, in both operands), so a step is one pass of 64 MFMAs, in four
// quarters of 16, each on one pair of fragment sets of four blocks (A rows
// 0-63 / 64-127 and B rows 0-63 / 64-127 of the wave: Al, Ah, Bl, Bh):
//   q0 Al.Bl  (reads Ah of this step)
//   wait for step kt+1 in LDS, barrier
//   q1 Al.Bh  (reads Bl of step kt+1 into a fifth set; loads A of kt+2)
//   q2 Ah.Bh  (reads Al of step kt+1;                 loads A of kt+2)
//   q3 Ah.Bl  (reads Bh of step kt+1;                 loads B of kt+3)
// Every set is read two quarters before the quarter that first uses it:
// with the loads writing the same LDS, a read issued one quarter ahead
// arrived too late (the step ran at twice the time of the loop without
// global loads, and of the loop without LDS reads).  Bl alternates between
// two registers sets, so steps run in pairs.  After the barrier of step kt
// no wave reads step kt's slots again: A's slot takes step kt+2 and B's
// step kt+3 (B's ring runs two steps ahead, A's one).
template <bool BS>
struct DtlTile4E4M3X {
    using Base = DtlTile<IN_BF16, true>;
    static constexpr int BM = 256, BN = 256, WM = 2, WN = 2;
    static constexpr int MI = 16;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    static constexpr int KSTEP = kRowBytes;  // E4M3 elements per K step
    static constexpr int OPS = Base::OPS;
    static constexpr int A_SLOTS = Base::A_SLOTS, B_SLOTS = Base::B_SLOTS;
    static_assert(A_SLOTS == 2 && B_SLOTS == 3, "B is the deep operand");
    static constexpr int LDS_BYTES = Base::LDS_BYTES;
    static constexpr int LOADS = 256 / 8 / (NT / 64);
    static_assert(FM == 8 && FN == 8 && LOADS == 8, "the quarter rotation assumes 8 x 8 blocks per wave");
    struct F8 {
        u32x8_t v[4];
    };

    f32x4_t acc[FM][FN];
    uint32_t va[LOADS], vb[LOADS];
    int kc[LOADS];
    int abase[2], bbase[2];
    uint32_t a_sh[2][2];  // LDS addresses of the A fragment halves, per A slot
    // Block-scaled form: two register sets of scales, one per pair of K
    // steps (set p % 2 for steps 2p, 2p + 1): sca[set][b] holds A's scale of
    // the lane's row in row block b, step 2p in byte 0 and step 2p + 1 in
    // byte 1; scb[set] B's scale of the wave's 128 columns, same bytes.
    // The loads fill only sca[set][0..1] (lane l: row l and row 64 + l of
    // the wave's rows); bcast_scales spreads them over the 8 row blocks.
    uint32_t sca[2][8], scb[2];
    uint32_t sc_lane;     // byte offset of row (lane) of the wave's A scales
    int sc_brow;          // byte offset of the wave's row of B scales

    __device__ __forceinline__ void setup(int lane, int wave, int wm0, int wn0, int lda, int ldb)
    {
        const int r8 = lane >> 3;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int row = (wave * LOADS + j) * 8 + r8;
            const int c = (lane & 7) ^ Base::dswz(row);
            kc[j] = c * 16;
            va[j] = (uint32_t)row * (uint32_t)lda + (uint32_t)c * 16u;
            vb[j] = (uint32_t)row * (uint32_t)ldb + (uint32_t)c * 16u;
        }
        const int r = lane & 15, q = lane >> 4;
        const int c0 = q ^ Base::dswz(r);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            abase[s] = (wm0 + r) * kRowBytes + ((c0 ^ (4 * s)) << 4);
            bbase[s] = (wn0 + r) * kRowBytes + ((c0 ^ (4 * s)) << 4);
        }
    }
    template <bool MASK>
    __device__ __forceinline__ void load_a(__amdgpu_buffer_rsrc_t r, char *slot, int wave, int j, int k_left) const
    {
        const uint32_t off = !MASK || kc[j] < k_left ? va[j] : kOOB;
        load_to_lds16(r, lds_addr(slot + (wave * LOADS + j) * 1024), off);
    }
    template <bool MASK>
    __device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t r, char *slot, int wave, int j, int k_left) const
    {
        const uint32_t off = !MASK || kc[j] < k_left ? vb[j] : kOOB;
        load_to_lds16(r, lds_addr(slot + (wave * LOADS + j) * 1024), off);
    }
    // half h of block 4 H + b of A (from A slot Q, an LDS address held in a
    // register plus an immediate) or of B (through the slot pointer)
    template <int Q, int H>
    __device__ __forceinline__ void rd_a(F8 &f, int i) const
    {
        typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
        const int b = i >> 1, h = i & 1;
        const u32x4_t v = *(const lds_u32x4 *)(uintptr_t)(a_sh[Q][h] + (4 * H + b) * 16 * kRowBytes);
        if (h == 0)
            f.v[b].lo = v;
        else
            f.v[b].hi = v;
    }
    template <int H>
    __device__ __forceinline__ void rd_b(const char *bs, F8 &f, int i) const
    {
        const int b = i >> 1, h = i & 1;
        const u32x4_t v = *(const u32x4_t *)(bs + bbase[h] + (4 * H + b) * 16 * kRowBytes);
        if (h == 0)
            f.v[b].lo = v;
        else
            f.v[b].hi = v;
    }
    // 16 MFMAs on m blocks 4 HM .. +3 x n blocks 4 HN .. +3 (n outer); read
    // i (of 8) after MFMAs 0, 2, .., 14, load j (of NL) after MFMA
    // j * 16 / NL + 1
    // The scales of step pair p into set SET: A's of the wave's 128 rows in
    // two loads (lane l: rows l and 64 + l; the 16 lanes of a row block read
    // 16 lines, where a load per row block had all 64 lanes read one line
    // each), then B's; two bytes (steps 2p and 2p + 1) per load (the scale
    // rows' pitches are even, so both bytes lie in the row); a pair at or
    // past the last k block, and rows past M, read as zeros through an
    // out-of-range offset.  3 loads.
    template <int SET>
    __device__ __forceinline__ void load_scales(const BlockScaleSrc &bs, int p)
    {
        const bool in_k = 2 * p < bs.kb;
        load_scale_pair(sca[SET][0], bs.ra, in_k ? sc_lane + (uint32_t)(2 * p) : kOOB);
        load_scale_pair(sca[SET][1], bs.ra, in_k ? sc_lane + (uint32_t)(64 * bs.lds_a + 2 * p) : kOOB);
        load_scale_pair(scb[SET], bs.rb, in_k ? (uint32_t)(sc_brow + 2 * p) : kOOB);
    }
    // Lane l's row of row block b is row 16b + (l mod 16), held by lane
    // 16 (b mod 4) + (l mod 16) of load b / 4: one cross-lane read per row
    // block.  Only once the set's loads have been counted complete: the
    // empty asm keeps the reads below the wait and barrier before it (the
    // compiler takes an asm load's result as written at once).
    template <int SET>
    __device__ __forceinline__ void bcast_scales(int lane)
    {
        uint32_t r0 = sca[SET][0], r1 = sca[SET][1];
        asm volatile("" : "+v"(r0), "+v"(r1));
#pragma unroll
        for (int b = 0; b < 8; ++b)
            sca[SET][b] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * (b % 4) + (lane & 15)) << 2,
                                                                 (int)(b < 4 ? r0 : r1));
    }
    // A pair whose second step lies past the last k block read a byte past
    // the scales (padding): keep only the first step's.
    template <int SET>
    __device__ __forceinline__ void trim_scales()
    {
#pragma unroll
        for (int b = 0; b < 8; ++b)
            keep_low_scale(sca[SET][b]);
        keep_low_scale(scb[SET]);
    }

    template <int HM, int HN, int NL, int SET, int P, class RD, class LD>
    __device__ __forceinline__ void quarter(const F8 &a, const F8 &b, RD &&rd, LD &&ld)
    {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (BS)
                mfma16_e4m3_scaled_agpr<P>(acc[4 * HM + i % 4][4 * HN + i / 4], b.v[i / 4], a.v[i % 4],
                                               scb[SET], sca[SET][4 * HM + i % 4]);
            else
                mfma16_e4m3_agpr(acc[4 * HM + i % 4][4 * HN + i / 4], b.v[i / 4], a.v[i % 4]);
            if (i % 2 == 0)
                rd(i / 2);
            if constexpr (NL > 0) {
                if (i % (16 / NL) == 1)
                    ld(i / (16 / NL));
            }
        }
    }

    __device__ __forceinline__ void mainloop(char *lds, const OperandSrc &sa, int lda, const OperandSrc &sb, int ldb,
                                             int K, int tid, const BlockScaleSrc &bs = BlockScaleSrc{})
    {
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm0 = (wave / WN) * TM, wn0 = (wave % WN) * TN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = f32x4_t{};
        if constexpr (BS) {
            // the wave's 128 columns are one scale block (TN == 128)
            static_assert(TN == 128, "");
            sc_lane = (uint32_t)((wm0 + lane) * bs.lds_a);
            sc_brow = (bs.nblk0 + wn0 / 128) * bs.lds_b;
        }
        const int ksteps = (K + KSTEP - 1) / KSTEP;
        if (ksteps <= 0)
            return;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                asm volatile("" : "+a"(acc[i][j]));
        setup(lane, wave, wm0, wn0, lda, ldb);
        char *const A0 = lds;                  // 2 slots: step s in slot s % 2
        char *const B0 = lds + A_SLOTS * OPS;  // 3 slots: step s in slot s % 3
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                a_sh[q][h] = lds_addr(A0 + q * OPS) + (uint32_t)abase[h];
        const OperandSrc ua = uniform_src(sa), ub = uniform_src(sb);
        constexpr std::true_type masked{};
        constexpr std::false_type unmasked{};
        // prologue: (the scales of steps 0 and 1,) A of steps 0, 1 and B of
        // steps 0, 1, 2; wait for all but B of step 2
        {
            if constexpr (BS)
                load_scales<0>(bs, 0);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const auto rb = ub.at_step(s), ra = ua.at_step(s);
#pragma unroll
                for (int j = 0; j < LOADS; ++j) {
                    load_b<true>(rb, B0 + s * OPS, wave, j, K - s * KSTEP);
                    load_a<true>(ra, A0 + s * OPS, wave, j, K - s * KSTEP);
                }
            }
            const auto rb2 = ub.at_step(2);
#pragma unroll
            for (int j = 0; j < LOADS; ++j)
                load_b<true>(rb2, B0 + 2 * OPS, wave, j, K - 2 * KSTEP);
            wait_vm<LOADS>();
        }
        lds_barrier();
        if constexpr (BS)
            bcast_scales<0>(lane);
        F8 Al, Ah, Bh, BlX, BlY;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            rd_a<0, 0>(Al, i);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            rd_b<0>(B0, BlX, i);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            rd_b<1>(B0, Bh, i);
        mfma_drain();
        int sb_cur = 0;  // B slot of step kt
        // one K step; P = kt & 1 (A's slot, and which of BlX / BlY is Bl);
        // SET = (kt / 2) & 1, the scale set of the step pair (block-scaled
        // form: the first step of pair p loads pair p + 1's scales into the
        // other set, right after its barrier; they are counted complete by
        // the next step's wait, which leaves only the last quarter's B loads
        // outstanding, and spread over the row blocks after its barrier)
        auto step = [&](int kt, auto mask, auto par, auto set) {
            constexpr int P = decltype(par)::value;
            constexpr int SET = decltype(set)::value;
            constexpr bool MASK = decltype(mask)::value;
            F8 &Bl = P == 0 ? BlX : BlY;
            F8 &Bn = P == 0 ? BlY : BlX;
            // the pair's scales have been counted complete (previous step's
            // wait); a pair ending past K drops its second step's byte
            if constexpr (BS && MASK && P == 0) {
                if (kt + 1 >= bs.kb)
                    trim_scales<SET>();
            }
            const int sb_next = sb_cur == 2 ? 0 : sb_cur + 1;
            const char *bn = B0 + sb_next * OPS;
            quarter<0, 0, 0, SET, P>(Al, Bl, [&](int i) { rd_a<P, 1>(Ah, i); }, [](int) {});
            wait_vm<LOADS>();
            lds_barrier();
            if constexpr (BS && P == 0)
                load_scales<SET ^ 1>(bs, (kt >> 1) + 1);
            if constexpr (BS && P == 1)
                bcast_scales<SET ^ 1>(lane);  // loaded by the step before, counted complete by the wait above
            const auto rA = MASK ? ua.at_step(kt + 2) : step_rsrc(ua, true, kt + 2);
            const int ka = K - (kt + 2) * KSTEP;
            char *const aw = A0 + P * OPS;
            const auto rB = MASK ? ub.at_step(kt + 3) : step_rsrc(ub, true, kt + 3);
            const int kb = K - (kt + 3) * KSTEP;
            char *const bw = B0 + sb_cur * OPS;
            quarter<0, 1, 4, SET, P>(Al, Bh, [&](int i) { rd_b<0>(bn, Bn, i); },
                                     [&](int j) { load_a<MASK>(rA, aw, wave, j, ka); });
            quarter<1, 1, 4, SET, P>(Ah, Bh, [&](int i) { rd_a<P ^ 1, 0>(Al, i); },
                                     [&](int j) { load_a<MASK>(rA, aw, wave, 4 + j, ka); });
            quarter<1, 0, 8, SET, P>(Ah, Bl, [&](int i) { rd_b<1>(bn, Bh, i); },
                                     [&](int j) { load_b<MASK>(rB, bw, wave, j, kb); });
            sb_cur = sb_next;
        };
        // Steps two at a time while every load is of a whole step
        // (kt + 4 <= ksteps - 2); the rest with the K mask.  An odd step
        // count gets one more step, whose loads were all past K: zeros.
        constexpr std::integral_constant<int, 0> p0{}, s0{};
        constexpr std::integral_constant<int, 1> p1{}, s1{};
        auto pair = [&](int kt, auto mask, auto set) {
            step(kt, mask, p0, set);
            step(kt + 1, mask, p1, set);
        };
        int kt = 0;
        if constexpr (!BS) {
            for (; kt + 1 < ksteps - 4; kt += 2)
                pair(kt, unmasked, s0);
            for (; kt < ksteps; kt += 2)
                pair(kt, masked, s0);
        } else {
            // two pairs per iteration, so that each uses its own scale set
            // without a branch (a branch on the pair's parity made the
            // compiler spill ~1700 registers); the last iteration may run up
            // to three steps past K, on zeros
            for (; kt + 3 < ksteps - 4; kt += 4) {
                pair(kt, unmasked, s0);
                pair(kt + 2, unmasked, s1);
            }
            for (; kt < ksteps; kt += 4) {
                pair(kt, masked, s0);
                pair(kt + 2, masked, s1);
            }
        }
        wait_vm<0>();
        if constexpr (BS) {
            // every scale load has landed: only now may the compiler reuse
            // their registers (the last pair's loads are never read, and
            // the compiler must not hand their registers to other values
            // while those loads are in flight)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    asm volatile("" ::"v"(sca[q][b]));
                asm volatile("" ::"v"(scb[q]));
            }
        }
        mfma_drain();
    }
};
using DtlTile4E4M3 = DtlTile4E4M3X<false>;

// ---------------------------------------------------------------------------
// Epilogue helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}
// Each fp32 value is converted as it stands (one IEEE round-to-nearest-even
// each).  The values are made opaque first: otherwise the compiler may fold
// the product that made a value and its conversion into one mixed-precision
// FMA that rounds the exact product straight to fp16, so the same epilogue
// would round differently in kernels where the fold happens and where it
// does not.
__device__ __forceinline__ uint32_t pack2_f16(float a, float b)
{
    a = opaque(a);
    b = opaque(b);
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    // SiLU(g) * u = g / (1 + e^-g) * u, with the hardware exp2 and reciprocal
    float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Four consecutive outputs -> one store of 16 B (fp32) or 8 B (16-bit) at
// byte offset `off` of resource r; offsets past the resource are dropped.
// AUX: the store's cache-policy bits (kStoreStream: non-temporal).
constexpr int kStoreStream = 2;
template <int OUT, int AUX = 0>
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v0, float v1, float v2,
                                        float v3)
{
    if constexpr (OUT == OUT_F32) {
        u32x4_t d = {__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                     __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
        __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, AUX);
    } else if constexpr (OUT == OUT_BF16) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack2_bf16(v0, v1), pack2_bf16(v2, v3)}, r, off, 0, AUX);
    } else {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack2_f16(v0, v1), pack2_f16(v2, v3)}, r, off, 0, AUX);
    }
}

constexpr int out_size(int out) { return out == OUT_F32 ? 4 : 2; }

// Write the tile.  D points at the tile's (row 0, column 0) output element
// (for SILU_GATE: the tile's first h column); m_valid / n_valid are the rows
// and GEMM columns of this tile that exist.  n_valid is a multiple of 4
// (ragged columns are written by a separate edge kernel), so each lane's
// 4-column group is wholly in or out: rows past m_valid fall beyond the
// resource and are dropped by the hardware, column groups past n_valid get
// an out-of-range offset.  No branches, so accumulators are read out one
// fragment at a time.
// AUX: the stores' cache-policy bits (kDeviceScope: written through to the
// level every XCD shares, for outputs another workgroup reads in the same
// launch).
// rw (SILU_GATE only, may be null): the tile's row weights, rw[r] for tile
// row r < m_valid; each gated value is multiplied by its row's weight before
// the rounding ("MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 09:
// the routing weight taken into FC2's input, p(hW2) = (ph)W2).
template <class T, int EPI, int OUT, int AUX = 0>
__device__ __forceinline__ void epilogue(const T &t, void *D, int64_t ldd, int m_valid, int n_valid, int tid,
                                         const float *rw = nullptr)
{
    constexpr int esize = out_size(OUT);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / T::WN) * T::TM;
    const int wn0 = (wave % T::WN) * T::TN;
    const int out_cols = EPI == EPI_SILU_GATE ? n_valid / 2 : n_valid;
    const uint32_t row_bytes = (uint32_t)ldd * (uint32_t)esize;
    if (m_valid <= 0 || n_valid <= 0)
        return;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(D, ((uint64_t)(m_valid - 1) * (uint64_t)ldd + (uint64_t)out_cols) * (uint64_t)esize);
    // row weights: rows past m_valid read 0 (their outputs are not stored)
    const __amdgpu_buffer_rsrc_t rwr = make_rsrc(rw, rw ? (uint64_t)m_valid * 4u : 0u);
    if constexpr (T::MI == 16) {
        // 16 x 16 blocks: lane l holds row (l mod 16), columns 4(l/16) .. +3
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int m = wm0 + 16 * i + (lane & 15);
            const uint32_t rowoff = (uint32_t)m * row_bytes;
            float w = 1.0f;
            if constexpr (EPI == EPI_SILU_GATE) {
                if (rw)
                    w = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rwr, (uint32_t)m * 4u, 0, 0));
            }
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const f32x4_t &a = t.acc[i][j];
                const int n = wn0 + 16 * j + 4 * (lane >> 4);
                if constexpr (EPI == EPI_NONE) {
                    const uint32_t off = n < n_valid ? rowoff + (uint32_t)n * esize : kOOB;
                    bstore4<OUT, AUX>(r, off, a[0], a[1], a[2], a[3]);
                } else {
                    // gate: columns 0-7 of the block (lanes 0-31); up: 8-15,
                    // 32 lanes further on
                    const float u0 = __shfl_xor(a[0], 32, 64), u1 = __shfl_xor(a[1], 32, 64);
                    const float u2 = __shfl_xor(a[2], 32, 64), u3 = __shfl_xor(a[3], 32, 64);
                    const int hc = (n >> 4) * 8 + (n & 15);
                    const uint32_t off = (lane < 32 && n < n_valid) ? rowoff + (uint32_t)hc * esize : kOOB;
                    float h0 = silu_mul(a[0], u0), h1 = silu_mul(a[1], u1), h2 = silu_mul(a[2], u2),
                          h3 = silu_mul(a[3], u3);
                    if (rw) {
                        h0 *= w;
                        h1 *= w;
                        h2 *= w;
                        h3 *= w;
                    }
                    bstore4<OUT, AUX>(r, off, h0, h1, h2, h3);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int m = wm0 + 32 * i + (lane & 31);
            const uint32_t rowoff = (uint32_t)m * row_bytes;
            float w = 1.0f;
            if constexpr (EPI == EPI_SILU_GATE) {
                if (rw)
                    w = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rwr, (uint32_t)m * 4u, 0, 0));
            }
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const f32x16_t &a = t.acc[i][j];
                if constexpr (EPI == EPI_NONE) {
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int n = wn0 + 32 * j + 8 * rg + 4 * (lane >> 5);
                        const uint32_t off = n < n_valid ? rowoff + (uint32_t)n * esize : kOOB;
                        bstore4<OUT, AUX>(r, off, a[4 * rg], a[4 * rg + 1], a[4 * rg + 2], a[4 * rg + 3]);
                    }
                } else {
                    // columns 8*rg..8*rg+7 of a 32-wide block are gate for rg
                    // even; the next eight are the matching up
#pragma unroll
                    for (int rg = 0; rg < 4; rg += 2) {
                        const int n = wn0 + 32 * j + 8 * rg + 4 * (lane >> 5);
                        const int hc = (n >> 4) * 8 + (n & 15);
                        const uint32_t off = n < n_valid ? rowoff + (uint32_t)hc * esize : kOOB;
                        float h0 = silu_mul(a[4 * rg + 0], a[4 * rg + 4]), h1 = silu_mul(a[4 * rg + 1], a[4 * rg + 5]);
                        float h2 = silu_mul(a[4 * rg + 2], a[4 * rg + 6]), h3 = silu_mul(a[4 * rg + 3], a[4 * rg + 7]);
                        if (rw) {
                            h0 *= w;
                            h1 *= w;
                            h2 *= w;
                            h3 *= w;
                        }
                        bstore4<OUT, AUX>(r, off, h0, h1, h2, h3);
                    }
                }
            }
        }
    }
}

// Epilogue of the 16 x 16 direct-to-LDS tile (no gate): the accumulators
// go through LDS, which the K loop no longer needs, so that every store
// instruction writes one whole tile row (64 lanes x 4 outputs: 1 KiB of
// fp32 or 512 B of 16-bit) instead of 16 rows x 64 B.  Half the tile's rows
// at a time: each wave stages its m blocks 4h .. 4h+3 (128 rows x 256
// fp32 in all = 128 KiB), the 16-byte chunks of staged row x XOR-permuted
// by (x & 15) so that the writes of 16 rows hit distinct banks; then each
// wave stores every eighth staged row.  Every wave must call it (it meets
// the others at workgroup barriers, which wait for LDS accesses only, so the
// stores of one half need not complete before the next is staged); each wave
// enters it with its own loads into the rings complete, so after the first
// barrier nothing writes the rings any more.
// SCALE: every output is first multiplied by `scale` (fp32).
template <class T, int OUT, bool SCALE = false>
__device__ __forceinline__ void epilogue_staged(const T &t, char *lds, void *D, int64_t ldd, int m_valid,
                                                int n_valid, int tid, float scale = 1.0f)
{
    static_assert(T::MI == 16 && T::BN == 256 && T::WM == 2 && T::TM == 128 && T::LDS_BYTES >= 128 * 1024, "");
    constexpr int esize = out_size(OUT);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / T::WN) * T::TM;
    const int wn0 = (wave % T::WN) * T::TN;
    if (m_valid <= 0 || n_valid <= 0)
        return;
    const uint32_t row_bytes = (uint32_t)ldd * (uint32_t)esize;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(D, ((uint64_t)(m_valid - 1) * (uint64_t)ldd + (uint64_t)n_valid) * (uint64_t)esize);
    const int n = 4 * lane;
    lds_barrier();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int x = (wm0 >> 1) + 16 * ii + (lane & 15);
#pragma unroll
            for (int jb = 0; jb < T::FN; ++jb) {
                const int c = (wn0 + 16 * jb + 4 * (lane >> 4)) >> 2;
                *(f32x4_t *)(lds + x * 1024 + ((c ^ (x & 15)) << 4)) = t.acc[4 * h + ii][jb];
            }
        }
        lds_barrier();
#pragma unroll 4
        for (int x = wave; x < 128; x += T::NT / 64) {
            f32x4_t v = *(const f32x4_t *)(lds + x * 1024 + ((lane ^ (x & 15)) << 4));
            if constexpr (SCALE)
                v *= scale;
            const int m = (x >> 6) * T::TM + 64 * h + (x & 63);
            const uint32_t off = n < n_valid ? (uint32_t)m * row_bytes + (uint32_t)n * esize : kOOB;
            // whole rows, written once and not read again here: streaming
            bstore4<OUT, kStoreStream>(r, off, v[0], v[1], v[2], v[3]);
        }
        lds_barrier();
    }
}

// The tile's epilogue: staged through LDS for the direct-to-LDS tile
// without a gate, else straight from the registers.
template <class T, int EPI, int OUT>
__device__ __forceinline__ void tile_epilogue(const T &t, char *lds, void *D, int64_t ldd, int m_valid, int n_valid,
                                              int tid, const float *rw = nullptr)
{
    if constexpr (T::MI == 16 && EPI == EPI_NONE)
        epilogue_staged<T, OUT>(t, lds, D, ldd, m_valid, n_valid, tid);
    else
        epilogue<T, EPI, OUT>(t, D, ldd, m_valid, n_valid, tid, rw);
    // The direct-to-LDS loops count their own loads with vmcnt waits, and
    // the counter also counts these stores.  Rather than rely on loads and
    // earlier stores retiring in order (the compiler's own wait placement
    // does not assume it), the next tile starts with nothing outstanding;
    // measured free, as its first wait would cover the stores anyway.
    if constexpr (T::MI == 16)
        wait_vm<0>();
}

}  // namespace mgemm
