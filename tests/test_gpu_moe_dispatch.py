"""GPU parity of the grouped product with A's rows gathered through a row
index (grouped_gemm_run_gather: the MoE dispatch fused into the A loads),
and of the whole MoE layer dispatch -> FC1 (SiLU gate) -> FC2 -> combine,
against the CPU oracle.  The oracle gathers with plain indexing, X[index]."""
import math
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal, assert_close, assert_close_carried, from_dev_bits, stage_gap, to_dev, values

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu

COUNTS = [0, 1, 5, 31, 32, 33, 64, 65, 100, 128, 129, 200, 256, 257, 300, 0, 2]


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def offsets(counts):
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("tile", ["auto", "32n", "256d"])
@pytest.mark.parametrize("epi", ["none", "silu"])
@pytest.mark.parametrize("variant", ["random", "int"])
def test_gather_against_oracle(tile, epi, variant):
    """Every expert size class; the index repeats tokens (as top-k routing
    does) and holds entries outside X, which read as zero rows."""
    flags = {"auto": 0, "32n": mg.PLAN_FORCE_TILE_32x256, "256d": mg.PLAN_FORCE_TILE_256x256_DTL}[tile]
    N, K, T = 256, 264, 700
    log(f"case gather tile={tile} epi={epi} {variant}")
    rs = np.random.RandomState(21 if variant == "random" else 22)
    off = offsets(COUNTS)
    rows = int(off[-1])
    idx = rs.randint(0, T, size=rows).astype(np.int32)
    idx[::97] = -1
    idx[5::101] = T + 3
    dist = ("normal", 1.0) if variant == "random" else ("int", 2)
    X = datagen.matrix((T, K), dist, "bf16", rs)
    W = datagen.matrix((len(COUNTS), K, N), ("normal", 0.05) if variant == "random" else ("int", 2), "bf16", rs)
    e = mg.EPI_SILU_GATE_I8 if epi == "silu" else mg.EPI_NONE
    out_cols = N // 2 if epi == "silu" else N
    D = torch.full((rows, out_cols), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    plan = mg.grouped_gemm_plan(len(COUNTS), rows, N, K, stride_b=K * N, epilogue=e, flags=flags)
    mg.grouped_gemm_run_gather(plan, to_dev(X, "bf16"), to_dev(W, "bf16"), D, dev_i32(off), dev_i32(idx))
    torch.cuda.synchronize()
    A = np.where(((idx >= 0) & (idx < T))[:, None], X[np.clip(idx, 0, T - 1)], 0).astype(np.uint16)
    ref = oracle.grouped_ref(A, W, off)
    if epi == "silu":
        ref = oracle.silu_gate(ref)
    got = from_dev_bits(D)
    if variant == "int" and epi == "none":
        assert_bits_equal(got, ref, "bf16", plan.describe())
    elif epi == "none":
        assert_close(got, ref, K, "bf16", plan.describe())
    else:
        tol = 2.0 ** -7 * np.abs(ref) + 1e-4 * math.sqrt(K)
        err = np.abs(values(got, "bf16") - ref)
        assert np.all(err <= tol), f"{plan.describe()}: max err {err.max():.3e}"


@pytest.mark.parametrize("tile", ["auto", "256d"])
def test_gather_column_major_weights_and_wide_lda(tile):
    """Column-major expert weights ([N][K] per expert) and an X whose rows are
    longer than K (lda = K + 40, the slack NaN): integer data, bit-exact."""
    flags = {"auto": 0, "256d": mg.PLAN_FORCE_TILE_256x256_DTL}[tile]
    counts = [3, 0, 140, 257, 60]
    N, K, T = 256, 200, 300
    log(f"case gather col-major weights tile={tile}")
    rs = np.random.RandomState(31)
    off = offsets(counts)
    rows = int(off[-1])
    idx = rs.randint(0, T, size=rows).astype(np.int32)
    X = datagen.matrix((T, K), ("int", 2), "bf16", rs)
    Wr = datagen.matrix((len(counts), K, N), ("int", 2), "bf16", rs)
    Wc = np.ascontiguousarray(Wr.transpose(0, 2, 1))
    lda = K + 40
    Xw = np.full((T, lda), 0x7FC1, dtype=np.uint16)
    Xw[:, :K] = X
    D = torch.empty(rows, N, dtype=torch.bfloat16, device="cuda")
    plan = mg.grouped_gemm_plan(len(counts), rows, N, K, b_layout="col", lda=lda, ldb=K, stride_b=N * K,
                                flags=flags)
    mg.grouped_gemm_run_gather(plan, to_dev(Xw, "bf16"), to_dev(Wc, "bf16"), D, dev_i32(off), dev_i32(idx))
    torch.cuda.synchronize()
    ref = oracle.grouped_ref(X[idx], Wc, off, w_layout="col")
    assert_bits_equal(from_dev_bits(D), ref, "bf16", plan.describe())


def test_gather_equals_pregathered_moe64():
    """The 64-expert layer's FC1 with the routing's row index gives exactly the
    bits of the same product on rows gathered beforehand."""
    cfg = datagen.MOE["moe64"]
    r, A, W1, _ = datagen.moe_inputs_device(cfg, "cuda")
    rows, H, I = int(r.offsets[-1]), cfg.hidden, cfg.inter
    log(f"case gather moe64 rows={rows}")
    # X: each token's row, taken back from the pre-gathered rows
    first = np.full(cfg.num_tokens, -1, dtype=np.int64)
    first[r.token_of_row[::-1]] = np.arange(rows)[::-1]
    assert np.all(first >= 0)
    X = A[torch.from_numpy(first).cuda()].contiguous()
    plan = mg.grouped_gemm_plan(cfg.num_experts, rows, 2 * I, H, stride_b=H * 2 * I, epilogue=mg.EPI_SILU_GATE_I8)
    offs = dev_i32(r.offsets)
    h1 = torch.empty(rows, I, dtype=torch.bfloat16, device="cuda")
    h2 = torch.empty_like(h1)
    mg.grouped_gemm_run(plan, A, W1, h1, offs)
    mg.grouped_gemm_run_gather(plan, X, W1, h2, offs, dev_i32(r.token_of_row))
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16)), plan.describe()


def test_moe_layer_dispatch_to_combine():
    """X -> gathered FC1 with the SiLU gate -> FC2 -> weighted top-k combine,
    on the small MoE config, against the oracle's own chain on the inputs."""
    cfg = datagen.MOE["moe_small"]
    r = datagen.moe_route(cfg)
    rows, H, I, E = int(r.offsets[-1]), cfg.hidden, cfg.inter, cfg.num_experts
    log(f"case moe layer dispatch..combine rows={rows}")
    rs = np.random.RandomState(cfg.x_seed)
    X = datagen.matrix((cfg.num_tokens, H), ("normal", cfg.x_std), "bf16", rs)
    _, _, W1, W2 = datagen.moe_inputs_host(cfg)
    offs = dev_i32(r.offsets)
    p1 = mg.grouped_gemm_plan(E, rows, 2 * I, H, stride_b=H * 2 * I, epilogue=mg.EPI_SILU_GATE_I8)
    p2 = mg.grouped_gemm_plan(E, rows, H, I, stride_b=I * H)
    h = torch.empty(rows, I, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(rows, H, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(cfg.num_tokens, H, dtype=torch.bfloat16, device="cuda")
    mg.grouped_gemm_run_gather(p1, to_dev(X, "bf16"), to_dev(W1, "bf16"), h, offs, dev_i32(r.token_of_row))
    mg.grouped_gemm_run(p2, h, to_dev(W2, "bf16"), z, offs)
    mg.moe_combine(z, dev_i32(r.pos), torch.from_numpy(r.weight).cuda(), y, cfg.top_k)
    torch.cuda.synchronize()
    # the oracle's own chain on the inputs: FC1 + gate, FC2 on its rounding
    # of h, the combine on its rounding of z; each GPU stage is held to its
    # rule widened by the gap the earlier rules allow, carried forward
    A = X[r.token_of_row]
    h_ref = oracle.silu_gate(oracle.grouped_ref(A, W1, r.offsets))
    assert_close(from_dev_bits(h), h_ref, H, "bf16", "FC1 (gathered)")
    z_ref = oracle.grouped_ref(oracle.encode(h_ref, "bf16"), W2, r.offsets)
    h_gap = stage_gap(h_ref, H, "bf16")
    z_carry = np.zeros_like(z_ref)
    for e in range(E):
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        if hi > lo:
            z_carry[lo:hi] = h_gap[lo:hi] @ np.abs(oracle.decode(W2[e], "bf16"))
    assert_close_carried(from_dev_bits(z), z_ref, I, "bf16", z_carry, "FC2")
    w = r.weight.astype(np.float64)
    y_ref = oracle.moe_combine_ref(oracle.encode(z_ref, "bf16"), r.pos, w)
    z_gap = stage_gap(z_ref, I, "bf16") + z_carry
    y_carry = np.zeros_like(y_ref)
    for k in range(r.pos.shape[1]):
        p = np.asarray(r.pos)[:, k]
        ok = (p >= 0) & (p < rows)
        y_carry[ok] += np.abs(w[ok, k])[:, None] * z_gap[p[ok]]
    err = np.abs(values(from_dev_bits(y), "bf16") - y_ref)
    tol = 2.0 ** -8 * np.abs(y_ref) + cfg.top_k * 2.0 ** -20 * np.abs(y_ref).max() + y_carry
    assert np.all(err <= tol), f"combine max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"


def test_gather_rejects_tiles_without_it():
    plan = mg.grouped_gemm_plan(2, 64, 256, 64, stride_b=64 * 256, flags=mg.PLAN_FORCE_TILE_256x256)
    X = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(2 * 64 * 256, dtype=torch.bfloat16, device="cuda")
    D = torch.zeros(64, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mg.MgemmError):
        mg.grouped_gemm_run_gather(plan, X, W, D, dev_i32([0, 32, 64]), dev_i32(np.zeros(64)))
