// narrow.hpp -- the few-token tile: up to 128 rows of A (tokens) against
// 128 columns of B (weight channels), for products whose token count is
// small (the decode shape, MoE experts with few routed rows).
//
// "MegaMoE：Blackwell 与 Hopper 的融合算子解读" (Blackwell section 04, dynamic
// N and swapAB; Hopper section 03) puts the few tokens on the MMA's narrow
// dimension and sizes that dimension to the valid token count rounded up to
// a multiple of 16.  Here the matrix instruction is v_mfma_f32_16x16x32 with
// the weight fragment as its first operand and the token fragment as its
// second, so tokens are the MFMA's column side, and a tile with t valid
// tokens runs ceil(t / 16) token blocks -- decided at run time per tile, so
// one launch serves experts of every small size without padding them to a
// fixed tile height.
//
// Layout: four waves, each owning 32 of the 128 columns (two blocks of 16)
// and every token block, so each wave's MFMA count scales with the token
// count.  The weights stream from HBM once; the kernel is bound by that
// stream, so operands go straight from global memory to LDS
// (buffer_load ... lds) through two rings of 64-k steps: one for the tile's
// token rows that exist (16 per token block, 128 bytes each), loaded by half
// of the waves, and a deeper one for the step's 64 x BN weight block, loaded
// by the other half (a wave's loads complete in issue order, so token rows,
// mostly L2 hits, must not queue behind weight loads from HBM).  A tile with
// fewer tokens has smaller token slots, leaving more room to the weights.
// Every step waits for the wave's own loads of the step, meets the other
// waves at one barrier, refills the slots the previous step freed, then
// reads its fragments and issues its MFMAs.
//
// Swizzles.  Token rows (and k-contiguous weight rows, [n][k]) use the
// direct-to-LDS tile's chunk swizzle dswz (conflict-free for the 16 x 16
// fragment reads).  Row-major weights ([k][n]) stay [k][n] in LDS, 256 bytes
// per k row (8 segments of 32 bytes), read with ds_read_b64_tr_b16: each
// group of 16 lanes reads four consecutive k rows of one 32-byte segment,
// and the groups served together read rows 8 apart, so segment s of row k
// is stored at s ^ f(k), f(k) = (k & 3) | (bit 3 of k) << 2 -- eight
// distinct segments for the eight rows read in one cycle.  The permutation
// is applied on the global side of the loads (each load fills 1 KiB of
// contiguous LDS).
#pragma once

#include "engine.hpp"

namespace mgemm {

// Split-K arrival counters.  One 64-bit word per output tile: the high half
// is the tag of the run that last touched it, the low half the number of
// that run's K ranges that have arrived.  The last range sets the count back
// to zero under its tag, so replaying a launch (the same tag, e.g. a
// captured graph) counts from zero again, and a range arriving on a word
// whose tag is not its run's (an earlier run's, or a workspace that was
// never used) first claims the word for its run, so the workspace needs no
// initial value.  Returns the count including this arrival.
//
// One atomic in the usual case: the add.  When the add finds another tag,
// it went into a stale word, which the claim (tag, 1) overwrites; a range
// whose claim loses to another range's sees the new tag and adds again, so
// every range is counted exactly once.
//
// Ordering without whole-cache maintenance: each XCD has its own L2, and an
// agent-scope release / acquire fence writes back / invalidates the whole
// L2 (measured: it made a four-way split three times slower than no split).
// Instead the partial tiles are stored and loaded with the device-scope
// cache policy (kDeviceScope: written through to, and read from, the level
// every XCD shares), a range drains its stores (s_waitcnt vmcnt(0)) before
// its workgroup barrier, and only then does one lane arrive, with relaxed
// agent-scope atomics; the last range reads the others' partials after its
// arrival has returned.
__device__ __forceinline__ uint32_t split_arrive(uint64_t *word, uint32_t tag)
{
    const uint64_t old = __hip_atomic_fetch_add(word, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(old >> 32) == tag)
        return (uint32_t)old + 1u;
    uint64_t cur = old + 1;
    for (;;) {
        if ((uint32_t)(cur >> 32) == tag)
            return (uint32_t)__hip_atomic_fetch_add(word, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
                   1u;
        if (__hip_atomic_compare_exchange_strong(word, &cur, ((uint64_t)tag << 32) | 1u, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return 1u;
    }
}

// Cache-policy bits of a buffer access: sc1, device scope.
constexpr int kDeviceScope = 16;

// Most K ranges a stream-K tile is cut into (the fixup keeps the other
// ranges' blocks of one row in registers).
constexpr int kSkMaxSplits = 4;

__device__ __forceinline__ void split_reset(uint64_t *word, uint32_t tag)
{
    __hip_atomic_store(word, (uint64_t)tag << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workspace of a split narrow plan: one 8-byte counter per output tile
// (rounded up to 256 bytes), then one fp32 partial tile per (tile, range),
// 128 tokens x BN columns in the accumulators' own lane order.
__host__ __device__ constexpr int64_t narrow_counter_bytes(int64_t tiles) { return (tiles * 8 + 255) / 256 * 256; }
__host__ __device__ constexpr int narrow_slab_bytes(int bn) { return 128 * bn * 4; }

// BN_: columns per tile, 128, 64 or 32.  128 and 64: four waves, each with
// BN / 4 columns (two blocks of 16, or one); 32: two waves of 16 columns.
// NW_ > 0 sets the wave count instead (eight waves of 16 columns at 128, for
// a kernel whose workgroup also runs the eight-wave 256 x 256 tile).
// AGPR_: accumulators in AGPRs through inline assembly (a kernel of its own)
// or, false, in whatever registers the compiler picks (a kernel that also
// holds the eight-wave tile's accumulators in VGPRs).
// Every wave computes every token block of its columns.
template <int IN, bool BKM, int BN_ = 128, int NW_ = 0, bool AGPR_ = true>
struct NarrowTile {
    static constexpr int TMAX = 128;              // tokens per tile
    static constexpr int NTB = TMAX / 16;         // token blocks
    static constexpr int BM = TMAX, BN = BN_;
    static_assert(BN == 128 || BN == 64 || BN == 32, "");
    static constexpr int NW = NW_ > 0 ? NW_ : (BN >= 64 ? 4 : 2);   // waves
    static constexpr int WM = 1, WN = NW;
    static constexpr int MI = 16;
    static constexpr int NT = 64 * NW;
    static constexpr int NB = BN / 16 / NW;       // column blocks per wave
    static constexpr int B_BYTES = 64 * BN * 2;        // one step of weights
    // Two rings, one per operand.  The weights stream from HBM while the
    // token rows, read by every tile of the launch, mostly hit L2, so the
    // weights need many more bytes in flight; but one wave's loads complete
    // in the order it issued them, so in a wave that issued both kinds a
    // token row would wait behind every weight load issued before it.  The
    // first WA waves therefore load only token rows and the other waves only
    // weights, each kind into a ring of its own depth: DA token slots (one
    // 64-k step of the tile's 16 NV token rows, 128 B each) and DB weight
    // slots (one 64 x BN step).  Every wave waits for its own loads only,
    // and all waves meet at one barrier per step.  A token wave issues LA
    // loads per step (1 KiB = 8 rows each; those past the tile's rows go to
    // a 1 KiB scratch area with an out-of-range offset: zeros, no memory
    // traffic, so that every token wave counts the same loads), a weight
    // wave LBW; at most 63 loads per wave are in flight (the vmcnt range).
    // A tile with fewer tokens has smaller token slots, so its weights get
    // more of the space (up to the vmcnt bound).
    static constexpr int LDS_BYTES = 160 * 1024;
    static constexpr int WORDS = LDS_BYTES - 256;   // 256 bytes no load touches (hand-over words)
    static constexpr int SCRATCH = WORDS - 1024;    // target of the token loads past the tile's rows
    static constexpr int WA = NW / 2;               // token-loading waves; waves WA.. load weights
    static constexpr int LBW = B_BYTES / 1024 / (NW - WA);   // weight loads per weight wave and step
    static_assert(LBW * (NW - WA) * 1024 == B_BYTES, "");
    template <int NV>
    struct Ring {
        static constexpr int A_BYTES = NV * 16 * kRowBytes;
        static constexpr int LA = (2 * NV + WA - 1) / WA;
        static constexpr int DA_VM = 63 / LA + 1, DB_VM = 63 / LBW + 1;
        // token depth: up to eight steps within 7/8 of the space, at least
        // three, and never so many that fewer than three weight slots remain.
        // Token rows are re-read by every tile of the launch (from L2), so at
        // 64-128 tokens they are most of a step's bytes and their latency,
        // not the weights', sets the step rate: 128 x 7168 x 2048 ran 18.0
        // us with three token slots, 16.9 us with eight (and three weight
        // slots), 128 x 2048 x 7168 20.7 -> 19.9 us; 16 tokens unchanged.
        static constexpr int DA_FIT = SCRATCH * 7 / 8 / A_BYTES;
        static constexpr int DA_CAP = DA_FIT < 3 ? 3 : (DA_FIT > 8 ? 8 : DA_FIT);
        static constexpr int DA_ROOM = (SCRATCH - 3 * B_BYTES) / A_BYTES;
        static constexpr int DA_WANT = DA_CAP < DA_ROOM ? DA_CAP : DA_ROOM;
        static constexpr int DA = DA_WANT < DA_VM ? DA_WANT : DA_VM;
        static constexpr int DB_FIT = (SCRATCH - DA * A_BYTES) / B_BYTES;
        static constexpr int DB = DB_FIT < DB_VM ? DB_FIT : DB_VM;
        static constexpr int B_BASE = DA * A_BYTES;   // the weight ring
        static_assert(DA >= 3 && DB >= 3 && B_BASE + DB * B_BYTES <= SCRATCH, "");
    };
    static constexpr int LA_MAX = Ring<NTB>::LA;
    static constexpr int BROW = BN * 2;           // bytes of a k row of a row-major weight step
    static constexpr int RPL = 1024 / BROW;       // k rows per (1 KiB) load of a row-major weight step
    static constexpr int LG_R = BN == 128 ? 0 : (BN == 64 ? 1 : 2);   // log2 of k rows per 256 bytes
    static_assert(NB >= 1 && LBW >= 1, "");

    f32x4_t acc[NTB][NB];
    uint32_t va[LA_MAX], vb[LBW];  // per-lane global byte offsets within a step
    int kca[LA_MAX], kcb[LBW];     // k of this lane's 16-byte chunk (k-contiguous operands)
    int afr[2];                // A fragment of token block 0, sub-step s (LDS offset in a slot)
    int bfr[NB][2];            // k-contiguous B: fragment of column block nb, sub-step s (from the weights)
    int btr[NB];               // row-major B: transpose-read piece of column block nb (k row 0, from the weights)

    // Row-major weight steps: 32-byte segment s of k row k is stored at
    // s ^ bseg(k).  One ds_read_b64_tr_b16 of a 16-lane group covers k rows
    // k0 .. k0 + 3 of one segment, and the groups served in the same cycle
    // read rows 8 apart, so eight rows {k0 + j, k0 + 8 + j} share the 64
    // banks (256 bytes); rows 256 bytes apart in LDS (same k mod 256/BROW)
    // must take distinct segments: the bits of j above log2(256/BROW),
    // and bit 3 of k, above them.
    static __device__ __forceinline__ int bseg(int k)
    {
        return ((k & 3) >> LG_R) | (((k >> 3) & 1) << (2 - LG_R));
    }

    // Per-lane load offsets and fragment addresses for NV token blocks.
    template <int NV>
    __device__ __forceinline__ void setup(int lane, int wave, int lda, int ldb, const RowGather &ga)
    {
        using R = Ring<NV>;
        // A: load j of token wave w fills token rows 8 (LA w + j) .. +7 when
        // they exist, else the scratch area
#pragma unroll
        for (int j = 0; j < R::LA; ++j) {
            const int blk = wave * R::LA + j;
            const int row = blk * 8 + (lane >> 3);
            const int c = (lane & 7) ^ DtlTile<IN, true>::dswz(row);
            const bool real = blk < 2 * NV;
            kca[j] = c * 8;
            if (!real) {
                va[j] = kOOB;
            } else if (ga.idx) {
                const uint32_t ro = ga.row_offset(row, lda);
                va[j] = ro == kOOB ? kOOB : ro + (uint32_t)c * 16u;
            } else {
                va[j] = (uint32_t)row * (uint32_t)lda * 2u + (uint32_t)c * 16u;
            }
        }
        // B: load j of weight wave w (counted from WA) is the step's 1 KiB
        // piece LBW w + j (the token waves' offsets are not used)
        const int ww = wave < WA ? 0 : wave - WA;
#pragma unroll
        for (int j = 0; j < LBW; ++j) {
            if constexpr (BKM) {
                // [n][k]: piece i holds columns 8 i .. 8 i + 7
                const int row = (ww * LBW + j) * 8 + (lane >> 3);
                const int c = (lane & 7) ^ DtlTile<IN, true>::dswz(row);
                kcb[j] = c * 8;
                vb[j] = (uint32_t)row * (uint32_t)ldb * 2u + (uint32_t)c * 16u;
            } else {
                // [k][n]: piece i holds k rows RPL i .. RPL i + RPL - 1; lane l
                // the 16 bytes at 16 (l % (BROW/16)) of row l / (BROW/16), i.e.
                // physical segment (l % (BROW/16)) / 2, half l & 1
                constexpr int CPR = BROW / 16;   // 16-byte chunks per k row
                const int kr = (ww * LBW + j) * RPL + lane / CPR;
                const int pc = lane % CPR;
                const int seg = (pc >> 1) ^ bseg(kr);
                kcb[j] = 0;
                vb[j] = (uint32_t)kr * (uint32_t)ldb * 2u + (uint32_t)(seg * 32 + (pc & 1) * 16);
            }
        }
        const int r = lane & 15, q = lane >> 4;
        const int c0 = q ^ DtlTile<IN, true>::dswz(r);
#pragma unroll
        for (int s = 0; s < 2; ++s)
            afr[s] = r * kRowBytes + ((c0 ^ (4 * s)) << 4);
        const int wn0 = wave * NB * 16;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (BKM) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    bfr[nb][s] = (wn0 + 16 * nb + r) * kRowBytes + ((c0 ^ (4 * s)) << 4);
            } else {
                // lane 4 j + qq of group q points at k row 8 q + j (+ 32 s + 4 hi),
                // columns 4 qq .. 4 qq + 3 of the block's logical segment
                // (bseg of those rows does not depend on s or hi)
                const int j = r >> 2, qq = r & 3;
                const int seg = (wn0 >> 4) + nb;
                btr[nb] = (8 * q + j) * BROW + ((seg ^ bseg(8 * q + j)) * 32) + 8 * qq;
            }
        }
    }

    // A token wave's loads of one K step into token slot `slot`; ra points
    // at the step, k_left = K minus the step's first k (<= 0: a step past K,
    // all zeros)
    template <int NV>
    __device__ __forceinline__ void load_tokens(char *lds, char *slot, int wave, __amdgpu_buffer_rsrc_t ra,
                                                int k_left) const
    {
        using R = Ring<NV>;
#pragma unroll
        for (int j = 0; j < R::LA; ++j) {
            // wave-uniform: a token block of the slot, or the scratch area
            const int blk = wave * R::LA + j;
            load_to_lds16(ra, lds_addr(blk < 2 * NV ? slot + blk * 1024 : lds + SCRATCH),
                          kca[j] < k_left ? va[j] : kOOB);
        }
    }

    // A weight wave's loads of one K step into weight slot `slot`
    __device__ __forceinline__ void load_weights(char *slot, int wave, __amdgpu_buffer_rsrc_t rb, int k_left) const
    {
#pragma unroll
        for (int j = 0; j < LBW; ++j) {
            uint32_t off = vb[j];
            if constexpr (BKM)
                off = kcb[j] < k_left ? off : kOOB;
            load_to_lds16(rb, lds_addr(slot + ((wave - WA) * LBW + j) * 1024), off);
        }
    }

    // B fragments of sub-step s; wts = the slot's weights
    template <int S>
    __device__ __forceinline__ void read_b(const char *wts, u32x4_t (&b)[NB]) const
    {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (BKM) {
                b[nb] = *(const u32x4_t *)(wts + bfr[nb][S]);
            } else {
                typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
                const char *p = wts + btr[nb] + 32 * S * BROW;
                const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
                const u32x2_t hi =
                    __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * BROW)));
                b[nb] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    }

    static __device__ __forceinline__ void mma(f32x4_t &c, const u32x4_t &a, const u32x4_t &b)
    {
        if constexpr (AGPR_)
            mfma16_agpr<IN>(c, a, b);
        else
            c = mfma16<IN>(a, b, c);
    }

    // One K step on token slot `tok` and weight slot `wts`: both sub-steps'
    // fragments first, then the MFMAs of the NV token blocks.
    template <int NV>
    __device__ __forceinline__ void compute(const char *tok, const char *wts)
    {
        u32x4_t b0[NB], b1[NB], a0[NV], a1[NV];
        read_b<0>(wts, b0);
        read_b<1>(wts, b1);
#pragma unroll
        for (int tb = 0; tb < NV; ++tb) {
            a0[tb] = *(const u32x4_t *)(tok + afr[0] + tb * 16 * kRowBytes);
            a1[tb] = *(const u32x4_t *)(tok + afr[1] + tb * 16 * kRowBytes);
        }
#pragma unroll
        for (int tb = 0; tb < NV; ++tb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                mma(acc[tb][nb], b0[nb], a0[tb]);
#pragma unroll
        for (int tb = 0; tb < NV; ++tb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                mma(acc[tb][nb], b1[nb], a1[tb]);
    }

    // The K loop for NV token blocks on its two rings.  Step kt: this
    // wave's loads of step kt have landed (only those of the later steps of
    // its ring may be in flight); after the barrier every wave's have, and
    // every wave is done with step kt - 1, whose slots take the token step
    // kt + DA - 1 and the weight step kt + DB - 1.
    template <int NV>
    __device__ __forceinline__ void kloop(char *lds, const OperandSrc &sa, const OperandSrc &sb, int lda, int ldb,
                                          int K, int ksteps, int lane, int wave, const RowGather &ga)
    {
        using R = Ring<NV>;
        setup<NV>(lane, wave, lda, ldb, ga);
        const OperandSrc ua = uniform_src(sa), ub = uniform_src(sb);
        char *const wring = lds + R::B_BASE;
        const bool tw = wave < WA;   // uniform
        // prologue: token steps 0 .. DA-2 or weight steps 0 .. DB-2 (a loop
        // for the deep ring, whose unrolled buffer descriptors would all be
        // live at once)
        if (tw) {
#pragma unroll
            for (int s = 0; s < R::DA - 1; ++s)
                load_tokens<NV>(lds, lds + s * R::A_BYTES, wave, ua.at_step(s), K - s * kBK);
        } else {
#pragma unroll 1
            for (int s = 0; s < R::DB - 1; ++s)
                load_weights(wring + s * B_BYTES, wave, ub.at_step(s), K - s * kBK);
        }
        mfma_drain();
        int ta = 0, fa = R::DA - 1, tb = 0, fb = R::DB - 1;
        for (int kt = 0; kt < ksteps; ++kt) {
            if (tw)
                wait_vm<(R::DA - 2) * R::LA>();
            else
                wait_vm<(R::DB - 2) * LBW>();
            lds_barrier();
            if (tw)
                load_tokens<NV>(lds, lds + fa * R::A_BYTES, wave, ua.at_step(kt + R::DA - 1),
                                K - (kt + R::DA - 1) * kBK);
            else
                load_weights(wring + fb * B_BYTES, wave, ub.at_step(kt + R::DB - 1), K - (kt + R::DB - 1) * kBK);
            compute<NV>(lds + ta * R::A_BYTES, wring + tb * B_BYTES);
            ta = ta == R::DA - 1 ? 0 : ta + 1;
            fa = fa == R::DA - 1 ? 0 : fa + 1;
            tb = tb == R::DB - 1 ? 0 : tb + 1;
            fb = fb == R::DB - 1 ? 0 : fb + 1;
        }
    }

    // Accumulate the tile over k in [0, K): sa = its token rows (k-contiguous),
    // sb = its weight columns; ntb = token blocks to compute (1..8), the
    // tile's valid tokens rounded up to 16.
    __device__ __forceinline__ void mainloop(char *lds, const OperandSrc &sa, int lda, const OperandSrc &sb, int ldb,
                                             int K, int ntb, int tid, const RowGather &ga = RowGather{})
    {
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
        for (int i = 0; i < NTB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[i][j] = f32x4_t{};
        const int ksteps = (K + kBK - 1) / kBK;
        if (ksteps <= 0)
            return;
        if constexpr (AGPR_) {
#pragma unroll
            for (int i = 0; i < NTB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    asm volatile("" : "+a"(acc[i][j]));
        }
        switch (__builtin_amdgcn_readfirstlane(ntb)) {
        case 1: kloop<1>(lds, sa, sb, lda, ldb, K, ksteps, lane, wave, ga); break;
        case 2: kloop<2>(lds, sa, sb, lda, ldb, K, ksteps, lane, wave, ga); break;
        case 3: kloop<3>(lds, sa, sb, lda, ldb, K, ksteps, lane, wave, ga); break;
        case 4: kloop<4>(lds, sa, sb, lda, ldb, K, ksteps, lane, wave, ga); break;
        case 5: kloop<5>(lds, sa, sb, lda, ldb, K, ksteps, lane, wave, ga); break;
        case 6: kloop<6>(lds, sa, sb, lda, ldb, K, ksteps, lane, wave, ga); break;
        case 7: kloop<7>(lds, sa, sb, lda, ldb, K, ksteps, lane, wave, ga); break;
        default: kloop<8>(lds, sa, sb, lda, ldb, K, ksteps, lane, wave, ga); break;
        }
        // the trailing loads (all past K) have landed, every wave is done
        // with the ring (the next tile's prologue refills it), and the last
        // MFMAs' results are ready
        wait_vm<0>();
        lds_barrier();
        mfma_drain();
    }

    // the accumulators as ordinary registers
    __device__ __forceinline__ void values(f32x4_t (&v)[NTB][NB], int ntb) const
    {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                v[tb][nb] = tb < ntb ? acc[tb][nb] : f32x4_t{};
    }
};

// Write a narrow tile.  v[tb][nb]: lane l holds token 16 tb + (l mod 16),
// columns n0 + 16 (NB wave + nb) + 4 (l / 16) .. +3.  D points at the tile's
// (token 0, column 0) output (for SILU_GATE: its first h column); m_valid /
// n_valid: tokens and GEMM columns of the tile that exist (n_valid a
// multiple of 4).  Rows past m_valid fall past the resource; column groups
// past n_valid take an out-of-range offset.
// AUX: the stores' cache-policy bits.  rw (SILU_GATE only, may be null): the
// tile's token weights, rw[t] for token t < m_valid, multiplied into each
// gated value before the rounding (as in epilogue()).
template <int EPI, int OUT, int NTB, int NB, int AUX = 0>
__device__ __forceinline__ void narrow_store(const f32x4_t (&v)[NTB][NB], void *D, int64_t ldd, int m_valid,
                                             int n_valid, int ntb, int tid, const float *rw = nullptr)
{
    constexpr int esize = out_size(OUT);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (m_valid <= 0 || n_valid <= 0)
        return;
    const int out_cols = EPI == EPI_SILU_GATE ? n_valid / 2 : n_valid;
    const uint32_t row_bytes = (uint32_t)ldd * (uint32_t)esize;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(D, ((uint64_t)(m_valid - 1) * (uint64_t)ldd + (uint64_t)out_cols) * (uint64_t)esize);
    // token weights: tokens past m_valid read 0 (their outputs are not stored)
    const __amdgpu_buffer_rsrc_t rwr = make_rsrc(rw, rw ? (uint64_t)m_valid * 4u : 0u);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        if (tb >= ntb)
            break;
        const uint32_t rowoff = (uint32_t)(16 * tb + (lane & 15)) * row_bytes;
        float w = 1.0f;
        if constexpr (EPI == EPI_SILU_GATE) {
            if (rw)
                w = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  rwr, (uint32_t)(16 * tb + (lane & 15)) * 4u, 0, 0));
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const f32x4_t &a = v[tb][nb];
            const int n = wave * NB * 16 + 16 * nb + 4 * (lane >> 4);
            if constexpr (EPI == EPI_NONE) {
                const uint32_t off = n < n_valid ? rowoff + (uint32_t)n * esize : kOOB;
                bstore4<OUT, AUX>(r, off, a[0], a[1], a[2], a[3]);
            } else {
                // gate: columns 0-7 of the block (lanes 0-31); up: 8-15, 32 lanes on
                const float u0 = __shfl_xor(a[0], 32, 64), u1 = __shfl_xor(a[1], 32, 64);
                const float u2 = __shfl_xor(a[2], 32, 64), u3 = __shfl_xor(a[3], 32, 64);
                const int hc = (n >> 4) * 8 + (n & 15);
                const uint32_t off = (lane < 32 && n < n_valid) ? rowoff + (uint32_t)hc * esize : kOOB;
                float h0 = silu_mul(a[0], u0), h1 = silu_mul(a[1], u1), h2 = silu_mul(a[2], u2), h3 = silu_mul(a[3], u3);
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

}  // namespace mgemm
