// moe_fused.hpp -- both expert GEMMs of an MoE layer in one persistent
// launch: FC1 with the SwiGLU gate fused into its epilogue, h = SiLU(gate) x
// up, then FC2, y = h x W2, for every expert.
//
// The structure follows "MegaMoE：Blackwell 与 Hopper 的融合算子解读":
//  - one resident kernel runs FC1 and FC2 tasks and hands h from one to the
//    other through a completion count per (expert, row block) (Hopper
//    section 01, the fc1_done counter; Blackwell section 06 for the
//    write -> fence -> counter increment protocol): each FC1 task adds one
//    after its h tile is stored, and an FC2 task starts reading h once the
//    count of its row block has reached the number of FC1 column tiles;
//  - each FC1 tile adds its own count (no batching; Hopper section 13), but
//    later than the pages do: after the workgroup's next main loop, by which
//    time its h stores have drained without stalling it (FC2 tasks are handed
//    out after every FC1 task, so a later count holds up no consumer), or
//    before the workgroup first waits on a count itself;
//  - FC1 tasks of every expert are handed out before FC2 tasks, so FC2 tasks
//    find their inputs ready instead of spinning on them (Hopper section 15:
//    enough independent FC1 work between an FC2 task and its producers);
//  - experts are taken largest first, and an expert of at most 128 rows
//    runs on the few-token tile, its tokens on the matrix instruction's
//    narrow side (Blackwell section 04); larger experts run on the eight-wave
//    256 x 256 tile, as in the grouped launches, so that the layer gives
//    those launches' bits exactly.
//
// Scheduling.  Tasks are numbered by one ticket counter in the workspace:
// every FC1 task, then every FC2 task, each phase with the experts largest
// first and, inside an expert, row blocks fastest (consecutive tiles share a
// column block of the weights).  A workgroup takes a ticket, runs that task,
// and has taken its next ticket while the task ran (one ticket ahead).
// (Measured on the 64-expert layer: giving each XCD its own range of
// experts, with stealing, was 1.5 % slower than this one queue, although
// its L2 hit rate was higher; the layer's cost is the matrix rate of the
// large experts' tiles and the per-CU rate at which the small experts'
// weights stream, neither of which the order changes.)
//
// No deadlock, without assuming that all workgroups are resident at once:
// an FC2 task waits only on FC1 counts; every FC1 ticket was taken before
// any FC2 ticket; an FC1 task waits on nothing; a workgroup holding an FC1
// ticket is running (it took the ticket) and runs that task next or now (a
// ticket it holds ahead of it was taken later); and it adds the task's
// count after its next FC1 main loop (which waits on nothing), before its
// first FC2 wait, or at its end, whichever comes first.
//
// Ordering across XCDs without whole-cache maintenance (each XCD has its
// own L2): an FC1 task writes h with device-scope stores (written through
// to the level every XCD shares); each wave later waits for all its memory
// operations (vmcnt 0), the waves meet at a barrier, and only then does one
// lane add to the counter with a relaxed device-scope atomic.  An FC2 task polls the counter with atomic
// reads and then meets its waves at a barrier before any h load.  Its h
// loads may use the L2: within a launch a line of h enters an XCD's L2 only
// through loads issued after its counter completed (row blocks do not share
// cache lines when ldh is a multiple of 64 elements), and lines of earlier
// launches are dropped at the launch boundary.
#pragma once

#include "kernels.hpp"

namespace mgemm {

// One workgroup: order the experts (largest first, ties by id), lay out the
// tickets and counters, and clear the counters and the ticket counter.  Its
// writes are visible to the fused kernel that follows on the stream.
__global__ void __launch_bounds__(256) moe_prepare_kernel(MoeArgs p)
{
    __shared__ int rows_s[256];
    __shared__ int c1[257], c2[257], nb[257];
    __shared__ int ent[256][3];
    const int tid = threadIdx.x;
    const int N1 = 2 * p.inter;
    int lo = 0, rows = 0;
    if (tid < p.G) {
        lo = min(max(p.offs[tid], 0), p.max_rows);
        const int hi = min(max(p.offs[tid + 1], lo), p.max_rows);
        rows = hi - lo;
    }
    rows_s[tid] = rows;
    __syncthreads();
    if (tid < p.G) {
        int rank = 0;
        for (int j = 0; j < p.G; ++j) {
            const int r = rows_s[j];
            rank += (r > rows) || (r == rows && j < tid);
        }
        ent[rank][0] = tid;
        ent[rank][1] = lo;
        ent[rank][2] = rows;
        c1[rank + 1] = moe_tasks(rows, N1);
        c2[rank + 1] = moe_tasks(rows, p.hidden);
        nb[rank + 1] = moe_blocks(rows);
    } else {
        c1[tid + 1] = c2[tid + 1] = nb[tid + 1] = 0;
    }
    if (tid == 0)
        c1[0] = c2[0] = nb[0] = 0;
    __syncthreads();
    // inclusive scans of c1, c2, nb over positions 1..256 (Hillis-Steele)
    for (int st = 1; st < 256; st <<= 1) {
        const int a = tid >= st ? c1[tid + 1 - st] : 0;
        const int b = tid >= st ? c2[tid + 1 - st] : 0;
        const int c = tid >= st ? nb[tid + 1 - st] : 0;
        __syncthreads();
        c1[tid + 1] += a;
        c2[tid + 1] += b;
        nb[tid + 1] += c;
        __syncthreads();
    }
    const int slots = nb[256];
    const bool fits = slots <= p.max_slots;
    int32_t *w = (int32_t *)p.ws;
    int32_t *e4 = (int32_t *)(p.ws + kMoeEntries) + 4 * tid;
    if (tid < p.G) {
        e4[0] = ent[tid][0];
        e4[1] = ent[tid][1];
        e4[2] = ent[tid][2];
        e4[3] = nb[tid];
    } else {
        e4[0] = e4[1] = e4[2] = e4[3] = 0;
    }
    ((int32_t *)(p.ws + kMoeStart1))[tid] = tid < p.G ? c1[tid] : INT32_MAX;
    ((int32_t *)(p.ws + kMoeStart2))[tid] = tid < p.G ? c2[tid] : INT32_MAX;
    if (tid == 0) {
        w[kMoeTicket / 4] = 0;
        w[kMoeT1 / 4] = fits ? c1[256] : 0;
        w[kMoeT2 / 4] = fits ? c2[256] : 0;
        w[kMoeStatus / 4] = fits ? 0 : 2;
    }
    int32_t *cnt = (int32_t *)(p.ws + kMoeCounters);
    for (int i = tid; i < min(slots, p.max_slots); i += 256)
        cnt[i] = 0;
}

// The position holding ticket t (0 <= t < the phase's total) from the
// first tickets of positions 4 lane .. 4 lane + 3 held by each lane (the
// first tickets do not decrease): the last position whose first ticket is
// <= t.
__device__ __forceinline__ int moe_find(const int (&s)[4], int t, int &first)
{
    const int L = __popcll(__ballot(s[0] <= t)) - 1;
    const int s1 = __builtin_amdgcn_readlane(s[1], L), s2 = __builtin_amdgcn_readlane(s[2], L);
    const int s3 = __builtin_amdgcn_readlane(s[3], L), s0 = __builtin_amdgcn_readlane(s[0], L);
    const int i = (s1 <= t) + (s2 <= t) + (s3 <= t);
    first = i == 0 ? s0 : i == 1 ? s1 : i == 2 ? s2 : s3;
    return 4 * L + i;
}

// WEIGHTED: FC1's h rows scaled by p.row_weight (a separate instance, so
// the unweighted layer carries no weight code)
template <int IN, bool WEIGHTED>
__global__ void __launch_bounds__(512) moe_fused_kernel(MoeArgs p)
{
    using Big = DtlTile<IN, false>;
    using Nar = NarrowTile<IN, false, 128, 8, false>;
    static_assert(Big::NT == 512 && Nar::NT == 512, "both tiles run on the same eight waves");
    constexpr int LDS = Big::LDS_BYTES > Nar::LDS_BYTES ? Big::LDS_BYTES : Nar::LDS_BYTES;
    static_assert(LDS <= 160 * 1024, "");
    __shared__ __attribute__((aligned(16))) char lds[LDS];
    constexpr int OUT = IN == IN_BF16 ? OUT_BF16 : OUT_F16;
    constexpr int esize = 2;
    // the ticket hand-over word: among the narrow tile's words that no load
    // writes (the eight-wave tile's ring may cover it: it is used only while
    // every wave is between tasks)
    static_assert(LDS - 16 >= Nar::WORDS, "");
    int *const handover = (int *)(lds + LDS - 16);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int32_t *w = (const int32_t *)p.ws;
    int32_t *counters = (int32_t *)(p.ws + kMoeCounters);
    const int T1 = __builtin_amdgcn_readfirstlane(w[kMoeT1 / 4]);
    const int T2 = __builtin_amdgcn_readfirstlane(w[kMoeT2 / 4]);
    const int total = T1 + T2;
    int s1[4], s2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s1[i] = ((const int32_t *)(p.ws + kMoeStart1))[4 * lane + i];
        s2[i] = ((const int32_t *)(p.ws + kMoeStart2))[4 * lane + i];
    }
    const int N1 = 2 * p.inter;
    const int need_big = (N1 + 255) / 256, need_nar = (N1 + 127) / 128;
    const uint16_t *W1 = (const uint16_t *)p.W1, *W2 = (const uint16_t *)p.W2;
    const uint16_t *X = (const uint16_t *)p.X, *Hin = (const uint16_t *)p.H;

    int32_t *ticket = (int32_t *)(p.ws + kMoeTicket);
    if (tid == 0)
        *handover = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int t = __builtin_amdgcn_readfirstlane(*handover);
    __syncthreads();

    Big big;
    Nar nar;
    // The FC1 tile whose count this workgroup still owes (uniform; -1:
    // none).  An FC1 tile's h stores are not waited for where they are
    // issued: they drain while the next task's loads stream in, and the tile
    // is counted once every wave has since waited for all its memory
    // operations and the waves have met -- after the next task's main loop,
    // or before this workgroup waits on any count itself (an FC2 task), or at
    // the end.  So no count waits on a task that could wait on it.
    int pending = -1;
    auto publish = [&]() {
        if (pending >= 0 && tid == 0)
            __hip_atomic_fetch_add(counters + pending, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pending = -1;
    };
    while (t < total) {
        // the next ticket, taken while this task runs
        int nxt = 0;
        if (tid == 0)
            nxt = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool fc2 = t >= T1;
        const int tl = fc2 ? t - T1 : t;
        int first;
        const int pos = __builtin_amdgcn_readfirstlane(fc2 ? moe_find(s2, tl, first) : moe_find(s1, tl, first));
        const int32_t *ent = (const int32_t *)(p.ws + kMoeEntries) + 4 * pos;
        const int e = __builtin_amdgcn_readfirstlane(ent[0]);
        const int row0 = __builtin_amdgcn_readfirstlane(ent[1]);
        const int rows = __builtin_amdgcn_readfirstlane(ent[2]);
        const int slot0 = __builtin_amdgcn_readfirstlane(ent[3]);
        const int local = __builtin_amdgcn_readfirstlane(tl - first);
        const bool narrow = rows <= kMoeNarrowRows;
        int m0, n0, m_valid, slot;
        if (narrow) {
            m0 = row0;
            m_valid = rows;
            n0 = local * 128;
            slot = slot0;
        } else {
            const int tm = (rows + 255) / 256;
            const int mb = local % tm, nb = local / tm;
            m0 = row0 + mb * 256;
            m_valid = min(256, rows - mb * 256);
            n0 = nb * 256;
            slot = slot0 + mb;
        }
        if (!fc2) {
            // FC1: h[m0.., n0/2..] = SiLU(gate) x up of X_rows x W1_e[:, n0..]
            RowGather ga;
            OperandSrc sa;
            if (p.row_index) {
                ga.idx = p.row_index + m0;
                ga.valid = m_valid;
                ga.limit = p.x_rows;
                sa = operand_src<true>(X, p.lda, p.x_rows, p.hidden);
            } else {
                sa = operand_src<true>(X + (int64_t)m0 * p.lda, p.lda, m_valid, p.hidden);
            }
            const uint16_t *Bt = W1 + (int64_t)e * p.stride_w1 + n0;
            const OperandSrc sb = operand_src<false>(Bt, p.ldw1, N1 - n0, p.hidden);
            char *Ht = (char *)p.H + ((int64_t)m0 * p.ldh + n0 / 2) * esize;
            const float *rw = WEIGHTED ? p.row_weight + m0 : nullptr;
            if (narrow) {
                const int ntb = (m_valid + 15) >> 4;
                nar.mainloop(lds, sa, p.lda, sb, p.ldw1, p.hidden, ntb, opaque(tid), ga);
                wait_vm<0>();
                __syncthreads();
                publish();
                f32x4_t v[Nar::NTB][Nar::NB];
                nar.values(v, ntb);
                narrow_store<EPI_SILU_GATE, OUT, Nar::NTB, Nar::NB, kDeviceScope>(v, Ht, p.ldh, m_valid,
                                                                                   min(128, N1 - n0), ntb, tid, rw);
            } else {
                big.mainloop(lds, sa, p.lda, sb, p.ldw1, p.hidden, opaque(tid), ga);
                wait_vm<0>();
                __syncthreads();
                publish();
                epilogue<Big, EPI_SILU_GATE, OUT, kDeviceScope>(big, Ht, p.ldh, m_valid, min(256, N1 - n0),
                                                               opaque(tid), rw);
            }
            pending = slot;
        } else {
            // FC2: y[m0.., n0..] = h_rows x W2_e[:, n0..], once the row
            // block's FC1 tiles have all been counted (this workgroup's own
            // last one first)
            if (pending >= 0) {
                wait_vm<0>();
                __syncthreads();
                publish();
            }
            if (tid == 0) {
                const int need = narrow ? need_nar : need_big;
                uint32_t polls = 0;
                while (__hip_atomic_fetch_add(counters + slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                       need) {
                    if (++polls >= p.spin_limit) {
                        __hip_atomic_store((int32_t *)(p.ws + kMoeStatus), 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __syncthreads();
            const OperandSrc sa = operand_src<true>(Hin + (int64_t)m0 * p.ldh, p.ldh, m_valid, p.inter);
            const uint16_t *Bt = W2 + (int64_t)e * p.stride_w2 + n0;
            const OperandSrc sb = operand_src<false>(Bt, p.ldw2, p.hidden - n0, p.inter);
            char *Yt = (char *)p.Y + ((int64_t)m0 * p.ldy + n0) * esize;
            if (narrow) {
                const int ntb = (m_valid + 15) >> 4;
                nar.mainloop(lds, sa, p.ldh, sb, p.ldw2, p.inter, ntb, opaque(tid));
                f32x4_t v[Nar::NTB][Nar::NB];
                nar.values(v, ntb);
                narrow_store<EPI_NONE, OUT, Nar::NTB, Nar::NB>(v, Yt, p.ldy, m_valid, min(128, p.hidden - n0), ntb,
                                                               tid);
            } else {
                big.mainloop(lds, sa, p.ldh, sb, p.ldw2, p.inter, opaque(tid));
                tile_epilogue<Big, EPI_NONE, OUT>(big, lds, Yt, p.ldy, m_valid, min(256, p.hidden - n0),
                                                  opaque(tid));
            }
            wait_vm<0>();
        }
        // hand the next ticket to every wave: the rings are idle between the
        // first and the last of these barriers
        __syncthreads();
        if (tid == 0)
            *handover = nxt;
        __syncthreads();
        t = __builtin_amdgcn_readfirstlane(*handover);
        __syncthreads();
    }
    if (pending >= 0) {
        wait_vm<0>();
        __syncthreads();
        publish();
    }
}

}  // namespace mgemm
