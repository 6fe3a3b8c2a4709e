"""GPU parity of the routing weight taken into FC1's epilogue
(grouped_gemm_run_weighted: h = round(SiLU(gate) * up * w[row]), "MegaMoE：
Blackwell 与 Hopper 的融合算子解读", Hopper section 09) and of the combine
without weights, against the CPU oracle; and, with power-of-two weights
(every scaling exact), the folded layer against the weighted-combine layer
on the GPU itself, bit for bit."""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import (assert_bits_equal, assert_close, assert_close_carried, from_dev_bits, stage_gap, to_dev,
                     values)

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu

TILES = {"auto": 0, "256": mg.PLAN_FORCE_TILE_256x256, "128": mg.PLAN_FORCE_TILE_128x128,
         "32n": mg.PLAN_FORCE_TILE_32x256, "256d": mg.PLAN_FORCE_TILE_256x256_DTL, "nrw": mg.PLAN_FORCE_TILE_NARROW}
COUNTS = [0, 1, 5, 31, 33, 64, 100, 128, 129, 200, 256, 257, 300, 0, 2]


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def offsets(counts):
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def fc1(A, W, off, N, K, w_row=None, flags=0, extra_rows=2, index=None, x_rows=None):
    """FC1 with the SiLU gate; D pre-filled with 0xFF bytes, extra_rows past
    the routed rows.  w_row None: the unweighted run."""
    rows = int(off[-1])
    D = torch.full((rows + extra_rows, N // 2), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    plan = mg.grouped_gemm_plan(len(off) - 1, rows, N, K, stride_b=K * N, epilogue=mg.EPI_SILU_GATE_I8, flags=flags)
    Ad, Wd, od = to_dev(A, "bf16"), to_dev(W, "bf16"), dev_i32(off)
    if w_row is None and index is None:
        mg.grouped_gemm_run(plan, Ad, Wd, D, od)
    elif w_row is None:
        mg.grouped_gemm_run_gather(plan, Ad, Wd, D, od, dev_i32(index), x_rows=x_rows)
    else:
        mg.grouped_gemm_run_weighted(plan, Ad, Wd, D, od, dev_f32(w_row),
                                     row_index=None if index is None else dev_i32(index), x_rows=x_rows)
    torch.cuda.synchronize()
    got = from_dev_bits(D)
    assert np.all(got[rows:] == 0xFFFF), "rows past the routed rows were written"
    return got[:rows], plan


def case(seed, variant, N=256, K=264):
    rs = np.random.RandomState(seed)
    off = offsets(COUNTS)
    rows = int(off[-1])
    dist = ("normal", 1.0) if variant == "random" else ("int", 2)
    A = datagen.matrix((rows, K), dist, "bf16", rs)
    W = datagen.matrix((len(COUNTS), K, N), ("normal", 0.05) if variant == "random" else ("int", 2), "bf16", rs)
    return A, W, off, rs


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("variant", ["random", "int"])
def test_weighted_fc1_against_oracle(tile, variant):
    """Routing-like weights in (0, 1]; every expert size class and tile."""
    log(f"case weighted fc1 tile={tile} {variant}")
    A, W, off, rs = case(31 if variant == "random" else 32, variant)
    N, K = W.shape[2], W.shape[1]
    w_row = rs.uniform(0.05, 1.0, size=int(off[-1])).astype(np.float32)
    got, plan = fc1(A, W, off, N, K, w_row, flags=TILES[tile])
    ref = oracle.silu_gate(oracle.grouped_ref(A, W, off), row_weight=w_row.astype(np.float64))
    assert_close(got, ref, K, "bf16", plan.describe())


@pytest.mark.parametrize("tile", list(TILES))
def test_weighted_power_of_two_is_the_scaled_unweighted_output(tile):
    """With w = 2^-j the product by w is exact in fp32 and commutes with the
    16-bit rounding, so each weighted row is the unweighted row times its own
    weight, bit for bit: the weight lands on its row, once."""
    log(f"case weighted pow2 tile={tile}")
    A, W, off, rs = case(33, "random")
    N, K = W.shape[2], W.shape[1]
    w_row = (2.0 ** -rs.randint(0, 6, size=int(off[-1]))).astype(np.float32)
    plain, _ = fc1(A, W, off, N, K, None, flags=TILES[tile])
    got, plan = fc1(A, W, off, N, K, w_row, flags=TILES[tile])
    want = values(plain, "bf16") * w_row[:, None].astype(np.float64)
    assert np.array_equal(values(got, "bf16"), want), plan.describe()


def test_weighted_gathered_equals_pregathered():
    """The gathered form reads X through the index; the same weights give
    the same bits as the weighted run on rows gathered beforehand."""
    log("case weighted gather")
    A, W, off, rs = case(34, "random")
    N, K = W.shape[2], W.shape[1]
    rows = int(off[-1])
    X = datagen.matrix((300, K), ("normal", 1.0), "bf16", rs)
    idx = rs.randint(0, 300, size=rows).astype(np.int32)
    w_row = rs.uniform(0.05, 1.0, size=rows).astype(np.float32)
    got_g, plan = fc1(X, W, off, N, K, w_row, index=idx, x_rows=300)
    got_p, _ = fc1(X[idx], W, off, N, K, w_row)
    assert np.array_equal(got_g, got_p), plan.describe()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_combine_without_weights_against_oracle(dtype):
    """weights NULL: the plain sum of each token's top-k rows (integer rows:
    exact; random rows: within half an ulp plus the fp32 additions)."""
    T, top_k, H, rows = 120, 8, 520, 400
    log(f"case plain combine {dtype}")
    rs = np.random.RandomState(35)
    pos = rs.randint(-2, rows + 2, size=(T, top_k)).astype(np.int32)
    for variant in ("int", "random"):
        Zb = datagen.matrix((rows, H), ("int", 4) if variant == "int" else ("normal", 1.0), dtype, rs)
        Z = to_dev(Zb, dtype)
        Y = torch.empty((T, H), dtype=Z.dtype, device="cuda")
        mg.moe_combine(Z, dev_i32(pos), None, Y, top_k)
        torch.cuda.synchronize()
        ref = oracle.moe_combine_ref(Zb, pos, None, dtype)
        got = from_dev_bits(Y)
        if variant == "int":
            assert_bits_equal(got, ref, dtype, "plain combine int")
        else:
            z = np.abs(oracle.decode(Zb, dtype))
            mag = np.zeros_like(ref)
            for k in range(top_k):
                p = pos[:, k]
                ok = (p >= 0) & (p < rows)
                mag[ok] += z[p[ok]]
            rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
            err = np.abs(values(got, dtype) - ref)
            assert np.all(err <= rel * np.abs(ref) + top_k * 2.0 ** -23 * mag), f"max err {err.max():.3e}"


def small_layer():
    cfg = datagen.MOE["moe_small"]
    r = datagen.moe_route(cfg)
    rs = np.random.RandomState(cfg.x_seed)
    X = datagen.matrix((cfg.num_tokens, cfg.hidden), ("normal", cfg.x_std), "bf16", rs)
    _, _, W1, W2 = datagen.moe_inputs_host(cfg)
    return cfg, r, X, W1, W2


def run_layer(cfg, r, X, W1, W2, w_tok, fold):
    """X -> gathered FC1 (gate; with fold, each routed row's routing weight
    in the epilogue) -> FC2 -> combine (weighted, or with fold a plain sum)."""
    rows, H, I, E = int(r.offsets[-1]), cfg.hidden, cfg.inter, cfg.num_experts
    offs = dev_i32(r.offsets)
    p1 = mg.grouped_gemm_plan(E, rows, 2 * I, H, stride_b=H * 2 * I, epilogue=mg.EPI_SILU_GATE_I8)
    p2 = mg.grouped_gemm_plan(E, rows, H, I, stride_b=I * H)
    h = torch.empty(rows, I, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(rows, H, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(cfg.num_tokens, H, dtype=torch.bfloat16, device="cuda")
    Xd, idx = to_dev(X, "bf16"), dev_i32(r.token_of_row)
    if fold:
        w_row = np.empty(rows, dtype=np.float32)
        w_row[r.pos] = w_tok
        mg.grouped_gemm_run_weighted(p1, Xd, to_dev(W1, "bf16"), h, offs, dev_f32(w_row), row_index=idx)
    else:
        mg.grouped_gemm_run_gather(p1, Xd, to_dev(W1, "bf16"), h, offs, idx)
    mg.grouped_gemm_run(p2, h, to_dev(W2, "bf16"), z, offs)
    mg.moe_combine(z, dev_i32(r.pos), None if fold else dev_f32(w_tok), y, cfg.top_k)
    torch.cuda.synchronize()
    return from_dev_bits(h), from_dev_bits(z), from_dev_bits(y)


def test_folded_layer_equals_weighted_layer_power_of_two():
    """p(hW2) = (ph)W2 on the GPU: power-of-two routing weights make every
    scaling exact (fp32 products, the 16-bit roundings, the FMAs of the
    combine), so the folded layer and the weighted-combine layer agree bit
    for bit."""
    cfg, r, X, W1, W2 = small_layer()
    log("case folded layer pow2")
    w_tok = (2.0 ** -np.random.RandomState(36).randint(0, 4, size=r.pos.shape)).astype(np.float32)
    _, _, y_w = run_layer(cfg, r, X, W1, W2, w_tok, fold=False)
    _, _, y_f = run_layer(cfg, r, X, W1, W2, w_tok, fold=True)
    assert np.array_equal(y_f, y_w)


def test_folded_layer_against_oracle():
    """The routing's own (softmax) weights folded into FC1, FC2, the plain
    combine, against the oracle's folded chain on the inputs; each GPU stage
    held to its rule widened by the gap the earlier stages allow."""
    cfg, r, X, W1, W2 = small_layer()
    rows, H, I, E = int(r.offsets[-1]), cfg.hidden, cfg.inter, cfg.num_experts
    log(f"case folded layer vs oracle rows={rows}")
    w_tok = r.weight.astype(np.float32)
    h, z, y = run_layer(cfg, r, X, W1, W2, w_tok, fold=True)
    w_row = np.empty(rows)
    w_row[r.pos] = w_tok.astype(np.float64)
    A = X[r.token_of_row]
    h_ref = oracle.silu_gate(oracle.grouped_ref(A, W1, r.offsets), row_weight=w_row)
    assert_close(h, h_ref, H, "bf16", "FC1 (weighted, gathered)")
    z_ref = oracle.grouped_ref(oracle.encode(h_ref, "bf16"), W2, r.offsets)
    h_gap = stage_gap(h_ref, H, "bf16")
    z_carry = np.zeros_like(z_ref)
    for e in range(E):
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        if hi > lo:
            z_carry[lo:hi] = h_gap[lo:hi] @ np.abs(oracle.decode(W2[e], "bf16"))
    assert_close_carried(z, z_ref, I, "bf16", z_carry, "FC2")
    y_ref = oracle.moe_combine_ref(oracle.encode(z_ref, "bf16"), r.pos, None)
    z_gap = stage_gap(z_ref, I, "bf16") + z_carry
    y_carry = np.zeros_like(y_ref)
    for k in range(r.pos.shape[1]):
        p = np.asarray(r.pos)[:, k]
        ok = (p >= 0) & (p < rows)
        y_carry[ok] += z_gap[p[ok]]
    err = np.abs(values(y, "bf16") - y_ref)
    tol = 2.0 ** -8 * np.abs(y_ref) + cfg.top_k * 2.0 ** -20 * np.abs(y_ref).max() + y_carry
    assert np.all(err <= tol), f"combine max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"
