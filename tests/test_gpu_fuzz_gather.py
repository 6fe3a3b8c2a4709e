"""Randomised MoE dispatch fused into the grouped A loads
(grouped_gemm_run_gather) on the GPU: token count, expert row counts, the
row index (with entries outside the token matrix, which read as zero rows),
N, K, weight layout, epilogue and tile (the planner's, the direct-to-LDS,
32x256 or few-token one) drawn from a fixed seed (RandomState(2037)).
Plain products on integer inputs match the oracle on the rows gathered on
the host bit for bit; gated ones meet the bf16 rule.
"""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal, assert_close, from_dev_bits, to_dev

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")
from test_gpu_grouped import counts_to_offsets  # noqa: E402

pytestmark = pytest.mark.gpu

TILES = {"auto": 0, "256d": mg.PLAN_FORCE_TILE_256x256_DTL, "32n": mg.PLAN_FORCE_TILE_32x256,
         "nrw": mg.PLAN_FORCE_TILE_NARROW}
NCASES = 24


def draw_cases():
    rs = np.random.RandomState(2037)
    cases = []
    for i in range(NCASES):
        G = int(rs.randint(1, 17))
        kinds = rs.choice(4, size=G, p=[0.15, 0.35, 0.3, 0.2])
        lo, hi = [0, 1, 17, 129], [1, 17, 129, 520]
        counts = tuple(int(rs.randint(lo[k], hi[k])) for k in kinds)
        T = int(rs.randint(1, 600))
        silu = rs.randint(3) == 0
        N = 16 * int(rs.randint(1, 33))
        K = 8 * int(rs.randint(1, 49))
        bl = ["row", "col"][rs.randint(2)]
        tile = list(TILES)[rs.randint(len(TILES))]
        cases.append((i, counts, T, N, K, bl, silu, tile))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-G{len(c[1])}-T{c[2]}-N{c[3]}-K{c[4]}-{c[5]}-{'silu' if c[6] else 'plain'}-{c[7]}"
                                             for c in CASES])
def test_random_gather(case):
    i, counts, T, N, K, bl, silu, tile = case
    G, rows = len(counts), sum(counts)
    print(f"case {i}: G={G} counts={list(counts)} T={T} N={N} K={K} {bl} silu={silu} tile={tile}", flush=True,
          file=sys.stderr)
    rs = np.random.RandomState(6000 + i)
    X = datagen.matrix((T, K), ("int", 2), "bf16", rs)
    W = datagen.matrix((G, K, N), ("int", 2), "bf16", rs)
    Wst = W if bl == "row" else np.ascontiguousarray(W.transpose(0, 2, 1))
    idx = rs.randint(0, T, size=rows).astype(np.int32)
    bad = rs.rand(rows) < 0.1
    idx[bad] = np.where(rs.rand(int(bad.sum())) < 0.5, -1 - rs.randint(0, 5, int(bad.sum())), T + rs.randint(0, 9, int(bad.sum())))
    A = np.where(((idx >= 0) & (idx < T))[:, None], X[np.clip(idx, 0, T - 1)], 0).astype(np.uint16)
    off = counts_to_offsets(list(counts))
    epi = mg.EPI_SILU_GATE_I8 if silu else mg.EPI_NONE
    out_cols = N // 2 if silu else N
    plan = mg.grouped_gemm_plan(G, max(rows, 1), N, K, b_layout=bl, stride_b=K * N, ldb=N if bl == "row" else K,
                                ldd=out_cols, epilogue=epi, flags=TILES[tile])
    raw = torch.full(((rows + 2) * out_cols * 2,), 0xFF, dtype=torch.uint8, device="cuda")
    D = raw.view(torch.bfloat16).view(rows + 2, out_cols)
    idx_dev = torch.from_numpy(idx).cuda() if rows else torch.zeros(1, dtype=torch.int32, device="cuda")
    mg.grouped_gemm_run_gather(plan, to_dev(X, "bf16"), to_dev(Wst, "bf16"), D, torch.from_numpy(off).cuda(),
                               idx_dev, x_rows=T)
    torch.cuda.synchronize()
    tail = raw[rows * out_cols * 2:].cpu().numpy()
    assert np.all(tail == 0xFF), f"case {i}: rows past the routed rows were written"
    if rows == 0:
        return
    ref = oracle.grouped_ref(A, Wst, off, w_layout=bl)
    got = from_dev_bits(D[:rows])
    if silu:
        assert_close(got, oracle.silu_gate(ref), K, "bf16", f"case {i}: {plan.describe()}")
    else:
        assert_bits_equal(got, ref, "bf16", f"case {i}: {plan.describe()}")
