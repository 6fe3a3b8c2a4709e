"""GPU parity of the fused MoE layer (moe_fused_run: FC1 with the SiLU gate,
then FC2, in one persistent launch) against the CPU oracle, and against the
two grouped launches it replaces.

Acceptance: h under the bf16 rule with K = hidden against the oracle's
unrounded gated sums; y against the oracle's own chain (FC2 on the oracle's
rounding of h) under the bf16 rule with K = inter, widened by the gap the
FC1 rule allows between the GPU's h and the oracle's, carried through W2.
The fused kernel runs the same tiles, with the same k order, as the default
grouped plans, so it must also give their bits exactly."""
import math
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_close, assert_close_carried, from_dev_bits, stage_gap, to_dev, values

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu

# every size class: empty, tiny, the 128 / 129 tile boundary, one and several
# 256-row blocks with ragged tails
COUNTS = [0, 1, 5, 31, 32, 33, 64, 65, 100, 128, 129, 200, 256, 257, 300, 0, 2, 600]


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def offsets(counts):
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def two_launch(A, W1, W2, offs, E, rows, H, I, dtype="bf16"):
    """The same layer as two grouped launches (default plans)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    p1 = mg.grouped_gemm_plan(E, rows, 2 * I, H, a_type=dtype, d_type=dtype, stride_b=H * 2 * I,
                              epilogue=mg.EPI_SILU_GATE_I8)
    p2 = mg.grouped_gemm_plan(E, rows, H, I, a_type=dtype, d_type=dtype, stride_b=I * H)
    h = torch.empty(rows, I, dtype=tdt, device="cuda")
    y = torch.empty(rows, H, dtype=tdt, device="cuda")
    mg.grouped_gemm_run(p1, A, W1, h, offs)
    mg.grouped_gemm_run(p2, h, W2, y, offs)
    return h, y


def fused(A, W1, W2, offs, E, rows, H, I, dtype="bf16", ws_fill=None, row_index=None, x_rows=None):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    plan = mg.moe_fused_plan(E, rows, H, I, dtype=dtype)
    h = torch.full((rows, I), -1, dtype=torch.int16, device="cuda").view(tdt)
    y = torch.full((rows, H), -1, dtype=torch.int16, device="cuda").view(tdt)
    ws = torch.empty(plan.workspace_size(), dtype=torch.uint8, device="cuda")
    if ws_fill is not None:
        ws.fill_(ws_fill)
    mg.moe_fused_run(plan, A, W1, W2, h, y, offs, workspace=ws, row_index=row_index, x_rows=x_rows)
    return h, y, plan, ws


def status(ws):
    return int(ws[12:16].cpu().numpy().view(np.int32)[0])


def fc2_carry(h_ref, W2, off, H, dtype):
    """Per routed row, the FC1 gap (GPU h against the oracle's h) carried
    through that row's expert weights."""
    carry = np.zeros((h_ref.shape[0], W2.shape[2]))
    gap = stage_gap(h_ref, H, dtype)
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            carry[lo:hi] = gap[lo:hi] @ np.abs(oracle.decode(W2[e], dtype))
    return carry


def check_oracle(A_bits, W1, W2, off, h, y, H, I, dtype, what):
    """The oracle's own chain from the inputs: FC1 + gate, its rounding of h,
    FC2 on that; y is held to the FC2 rule widened by the carried FC1 gap."""
    h_ref = oracle.silu_gate(oracle.grouped_ref(A_bits, W1, off, dtype, dtype))
    assert_close(from_dev_bits(h), h_ref, H, dtype, f"{what} FC1")
    y_ref = oracle.grouped_ref(oracle.encode(h_ref, dtype), W2, off, dtype, dtype)
    assert_close_carried(from_dev_bits(y), y_ref, I, dtype, fc2_carry(h_ref, W2, off, H, dtype), f"{what} FC2")


@pytest.mark.parametrize("variant", ["random", "int"])
def test_fused_small_moe(variant):
    """The small MoE config (ragged, empty and tiny experts) against the
    oracle and bit for bit against the two grouped launches."""
    cfg = datagen.MOE["moe_small"]
    log(f"case fused small moe {variant}")
    r, A, W1, W2 = datagen.moe_inputs_host(cfg, variant)
    rows, H, I, E = int(r.offsets[-1]), cfg.hidden, cfg.inter, cfg.num_experts
    offs = dev_i32(r.offsets)
    Ad, W1d, W2d = to_dev(A, "bf16"), to_dev(W1, "bf16"), to_dev(W2, "bf16")
    h, y, plan, ws = fused(Ad, W1d, W2d, offs, E, rows, H, I, ws_fill=0xFF)
    h2, y2 = two_launch(Ad, W1d, W2d, offs, E, rows, H, I)
    torch.cuda.synchronize()
    log("  " + plan.describe())
    assert status(ws) == 0
    check_oracle(A, W1, W2, r.offsets, h, y, H, I, "bf16", plan.describe())
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16)), "h differs from the grouped launches"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "y differs from the grouped launches"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fused_every_size_class(dtype):
    """Experts of 0..600 rows (the 128 / 129 and 256 / 257 boundaries, several
    256-row blocks), hidden and inter spanning several K steps and a ragged
    last column tile of FC2 (hidden = 400: tiles of 256 + 144)."""
    H, I = 400, 192
    E = len(COUNTS)
    off = offsets(COUNTS)
    rows = int(off[-1])
    log(f"case fused size classes {dtype} rows={rows}")
    rs = np.random.RandomState(31 if dtype == "bf16" else 32)
    A = datagen.matrix((rows, H), ("normal", 1.0), dtype, rs)
    W1 = datagen.matrix((E, H, 2 * I), ("normal", 0.05), dtype, rs)
    W2 = datagen.matrix((E, I, H), ("normal", 0.05), dtype, rs)
    Ad, W1d, W2d = to_dev(A, dtype), to_dev(W1, dtype), to_dev(W2, dtype)
    offs = dev_i32(off)
    h, y, plan, ws = fused(Ad, W1d, W2d, offs, E, rows, H, I, dtype=dtype, ws_fill=0x5A)
    h2, y2 = two_launch(Ad, W1d, W2d, offs, E, rows, H, I, dtype)
    torch.cuda.synchronize()
    assert status(ws) == 0
    check_oracle(A, W1, W2, off, h, y, H, I, dtype, plan.describe())
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def blocks(n):
    return 0 if n <= 0 else (1 if n <= 128 else -(-n // 256))


def tasks(n, cols):
    return 0 if n <= 0 else (-(-cols // 128) if n <= 128 else -(-n // 256) * -(-cols // 256))


def test_fused_schedule_table():
    """The prepare kernel's schedule: experts ranked by rows (largest first,
    ties by id); first tickets the prefix sums of each expert's tasks (one
    128-column task per 128 weight columns for an expert of at most 128
    rows, else one per 256-row block and 256 columns); one counter per row
    block, each complete after the run; every workgroup's last ticket past
    the end."""
    H, I = 256, 128
    E = len(COUNTS)
    off = offsets(COUNTS)
    rows = int(off[-1])
    rs = np.random.RandomState(33)
    A = to_dev(datagen.matrix((rows, H), ("int", 2), "bf16", rs), "bf16")
    W1 = to_dev(datagen.matrix((E, H, 2 * I), ("int", 2), "bf16", rs), "bf16")
    W2 = to_dev(datagen.matrix((E, I, H), ("int", 2), "bf16", rs), "bf16")
    h, y, plan, ws = fused(A, W1, W2, dev_i32(off), E, rows, H, I, ws_fill=0xFF)
    torch.cuda.synchronize()
    w = ws.cpu().numpy().view(np.int32)
    order = sorted(range(E), key=lambda e: (-COUNTS[e], e))
    ent = w[64:64 + 4 * E].reshape(E, 4)
    assert ent[:, 0].tolist() == order
    assert ent[:, 1].tolist() == [int(off[e]) for e in order]
    assert ent[:, 2].tolist() == [COUNTS[e] for e in order]
    c1 = [tasks(COUNTS[e], 2 * I) for e in order]
    c2 = [tasks(COUNTS[e], H) for e in order]
    nb = [blocks(COUNTS[e]) for e in order]
    assert w[1] == sum(c1) and w[2] == sum(c2)
    assert w[0] == sum(c1) + sum(c2) + plan.info().grid
    assert w[4352 // 4: 4352 // 4 + E].tolist() == list(np.cumsum([0] + c1[:-1]))
    assert w[5376 // 4: 5376 // 4 + E].tolist() == list(np.cumsum([0] + c2[:-1]))
    assert ent[:, 3].tolist() == list(np.cumsum([0] + nb[:-1]))
    cnt = w[6400 // 4: 6400 // 4 + sum(nb)]
    need = []
    for e in order:
        need += [-(-2 * I // 128) if COUNTS[e] <= 128 else -(-2 * I // 256)] * blocks(COUNTS[e])
    assert cnt.tolist() == need
    assert status(ws) == 0


def test_fused_gather_equals_pregathered():
    """FC1 reading X through the routing's row index (with entries outside X,
    read as zero rows) gives exactly the bits of the run on rows gathered
    beforehand."""
    cfg = datagen.MOE["moe_small"]
    r = datagen.moe_route(cfg)
    rows, H, I, E, T = int(r.offsets[-1]), cfg.hidden, cfg.inter, cfg.num_experts, cfg.num_tokens
    log(f"case fused gather rows={rows}")
    rs = np.random.RandomState(cfg.x_seed)
    X = datagen.matrix((T, H), ("normal", 1.0), "bf16", rs)
    _, _, W1, W2 = datagen.moe_inputs_host(cfg)
    idx = r.token_of_row.astype(np.int32).copy()
    idx[::37] = -1
    idx[7::41] = T + 5
    A = np.where(((idx >= 0) & (idx < T))[:, None], X[np.clip(idx, 0, T - 1)], 0).astype(np.uint16)
    offs = dev_i32(r.offsets)
    W1d, W2d = to_dev(W1, "bf16"), to_dev(W2, "bf16")
    h1, y1, plan, _ = fused(to_dev(A, "bf16"), W1d, W2d, offs, E, rows, H, I)
    h2, y2, _, ws = fused(to_dev(X, "bf16"), W1d, W2d, offs, E, rows, H, I, row_index=dev_i32(idx), x_rows=T)
    torch.cuda.synchronize()
    assert status(ws) == 0
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    check_oracle(A, W1, W2, r.offsets, h2, y2, H, I, "bf16", "gathered")


def test_fused_repeat_and_graph_replay():
    """Runs reuse the workspace whatever it holds; a captured graph (the
    prepare kernel clears the counters, no memset node) replays to the same
    bits every time, with eager work in between."""
    cfg = datagen.MOE["moe_small"]
    r, A, W1, W2 = datagen.moe_inputs_host(cfg, "random")
    rows, H, I, E = int(r.offsets[-1]), cfg.hidden, cfg.inter, cfg.num_experts
    Ad, W1d, W2d, offs = to_dev(A, "bf16"), to_dev(W1, "bf16"), to_dev(W2, "bf16"), dev_i32(r.offsets)
    plan = mg.moe_fused_plan(E, rows, H, I)
    ws = torch.empty(plan.workspace_size(), dtype=torch.uint8, device="cuda")
    h = torch.empty(rows, I, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(rows, H, dtype=torch.bfloat16, device="cuda")
    mg.moe_fused_run(plan, Ad, W1d, W2d, h, y, offs, workspace=ws)
    torch.cuda.synchronize()
    y_first, h_first = y.clone(), h.clone()
    for _ in range(2):
        y.zero_()
        mg.moe_fused_run(plan, Ad, W1d, W2d, h, y, offs, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_first.view(torch.int16))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mg.moe_fused_run(plan, Ad, W1d, W2d, h, y, offs, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for i in range(3):
        h.zero_()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), h_first.view(torch.int16)), f"replay {i}: h"
        assert torch.equal(y.view(torch.int16), y_first.view(torch.int16)), f"replay {i}: y"
    assert status(ws) == 0


def test_fused_moe64_full_size():
    """The 64-expert layer (4096 tokens, top-8, hidden 7168, inter 2048): bit
    for bit the two grouped launches, and sampled rows of experts of every
    size class against the oracle (FC2 on the GPU's own h)."""
    cfg = datagen.MOE["moe64"]
    log("case fused moe64 full size (device-drawn weights)")
    r, A, W1, W2 = datagen.moe_inputs_device(cfg, "cuda")
    rows, H, I, E = int(r.offsets[-1]), cfg.hidden, cfg.inter, cfg.num_experts
    offs = dev_i32(r.offsets)
    h, y, plan, ws = fused(A, W1, W2, offs, E, rows, H, I, ws_fill=0xFF)
    torch.cuda.synchronize()
    log("  " + plan.describe())
    assert status(ws) == 0
    h2, y2 = two_launch(A, W1, W2, offs, E, rows, H, I)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16)), "h differs from the grouped launches"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "y differs from the grouped launches"
    del h2, y2
    cnt = r.counts
    order = [e for e in np.argsort(cnt, kind="stable") if cnt[e] > 0]
    picks = sorted(set(order[:5] + order[len(order) // 2 - 2: len(order) // 2 + 2] + order[-4:]))
    for e in picks:
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        sel = sorted({lo, (lo + hi) // 2, hi - 1})
        g = oracle.gemm_ref(from_dev_bits(A[sel]), from_dev_bits(W1[e]), "bf16", "bf16")
        h_ref = oracle.silu_gate(g)
        assert_close(from_dev_bits(h[sel]), h_ref, H, "bf16", f"FC1 expert {e} rows {sel}")
        w2 = from_dev_bits(W2[e])
        y_ref = oracle.gemm_ref(oracle.encode(h_ref, "bf16"), w2, "bf16", "bf16")
        carry = stage_gap(h_ref, H, "bf16") @ np.abs(oracle.decode(w2, "bf16"))
        assert_close_carried(from_dev_bits(y[sel]), y_ref, I, "bf16", carry, f"FC2 expert {e} rows {sel}")
    log(f"  checked experts {picks}")


def fused_weighted(A, W1, W2, offs, w, E, rows, H, I, dtype="bf16", row_index=None, x_rows=None):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    plan = mg.moe_fused_plan(E, rows, H, I, dtype=dtype)
    h = torch.full((rows, I), -1, dtype=torch.int16, device="cuda").view(tdt)
    y = torch.full((rows, H), -1, dtype=torch.int16, device="cuda").view(tdt)
    ws = torch.full((plan.workspace_size(),), 0xA5, dtype=torch.uint8, device="cuda")
    mg.moe_fused_run_weighted(plan, A, W1, W2, h, y, offs, w, workspace=ws, row_index=row_index, x_rows=x_rows)
    return h, y, plan, ws


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fused_weighted_equals_grouped_weighted(dtype):
    """The fused layer with routing weights taken into FC1's gate epilogue:
    h bit for bit the weighted grouped FC1's and y the grouped FC2's on it
    (experts of every size class, both tiles); h against the oracle's gate
    with the row weights, y within the FC2 rule widened by the carried gap."""
    H, I = 400, 192
    E = len(COUNTS)
    off = offsets(COUNTS)
    rows = int(off[-1])
    log(f"case fused weighted {dtype} rows={rows}")
    rs = np.random.RandomState(41 if dtype == "bf16" else 42)
    A = datagen.matrix((rows, H), ("normal", 1.0), dtype, rs)
    W1 = datagen.matrix((E, H, 2 * I), ("normal", 0.05), dtype, rs)
    W2 = datagen.matrix((E, I, H), ("normal", 0.05), dtype, rs)
    w = rs.uniform(0.02, 1.0, rows).astype(np.float32)
    Ad, W1d, W2d = to_dev(A, dtype), to_dev(W1, dtype), to_dev(W2, dtype)
    offs, wd = dev_i32(off), torch.from_numpy(w).cuda()
    h, y, plan, ws = fused_weighted(Ad, W1d, W2d, offs, wd, E, rows, H, I, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    p1 = mg.grouped_gemm_plan(E, rows, 2 * I, H, a_type=dtype, d_type=dtype, stride_b=H * 2 * I,
                              epilogue=mg.EPI_SILU_GATE_I8)
    p2 = mg.grouped_gemm_plan(E, rows, H, I, a_type=dtype, d_type=dtype, stride_b=I * H)
    h2 = torch.empty(rows, I, dtype=tdt, device="cuda")
    y2 = torch.empty(rows, H, dtype=tdt, device="cuda")
    mg.grouped_gemm_run_weighted(p1, Ad, W1d, h2, offs, wd)
    mg.grouped_gemm_run(p2, h2, W2d, y2, offs)
    torch.cuda.synchronize()
    assert status(ws) == 0
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16)), "h differs from the weighted grouped FC1"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "y differs from the grouped FC2"
    h_ref = oracle.silu_gate(oracle.grouped_ref(A, W1, off, dtype, dtype), row_weight=w.astype(np.float64))
    assert_close(from_dev_bits(h), h_ref, H, dtype, f"{plan.describe()} weighted FC1")
    y_ref = oracle.grouped_ref(oracle.encode(h_ref, dtype), W2, off, dtype, dtype)
    assert_close_carried(from_dev_bits(y), y_ref, I, dtype, fc2_carry(h_ref, W2, off, H, dtype),
                         f"{plan.describe()} FC2 on weighted h")


def test_fused_weighted_power_of_two_gathered():
    """Power-of-two routing weights scale exactly: with FC1 reading X through
    the row index, the weighted fused layer's h and y are the unweighted
    layer's rows times their weights, bit for bit."""
    cfg = datagen.MOE["moe_small"]
    r = datagen.moe_route(cfg)
    rows, H, I, E, T = int(r.offsets[-1]), cfg.hidden, cfg.inter, cfg.num_experts, cfg.num_tokens
    log(f"case fused weighted power of two gathered rows={rows}")
    rs = np.random.RandomState(cfg.x_seed + 1)
    X = datagen.matrix((T, H), ("normal", 1.0), "bf16", rs)
    _, _, W1, W2 = datagen.moe_inputs_host(cfg)
    idx = dev_i32(r.token_of_row)
    w = np.ldexp(1.0, rs.randint(-3, 3, rows)).astype(np.float32)
    Xd, W1d, W2d, offs = to_dev(X, "bf16"), to_dev(W1, "bf16"), to_dev(W2, "bf16"), dev_i32(r.offsets)
    wd = torch.from_numpy(w).cuda()
    h0, y0, _, _ = fused(Xd, W1d, W2d, offs, E, rows, H, I, row_index=idx, x_rows=T)
    h1, y1, _, ws = fused_weighted(Xd, W1d, W2d, offs, wd, E, rows, H, I, row_index=idx, x_rows=T)
    torch.cuda.synchronize()
    assert status(ws) == 0
    scale = wd[:, None]
    assert torch.equal(h1.view(torch.int16), (h0.float() * scale).to(torch.bfloat16).view(torch.int16))
    assert torch.equal(y1.view(torch.int16), (y0.float() * scale).to(torch.bfloat16).view(torch.int16))
