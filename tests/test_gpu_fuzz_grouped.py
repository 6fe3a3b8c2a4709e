"""Randomised grouped (MoE expert) parity on the GPU: expert counts, row
counts (empty, few-token and multi-tile experts), N, K, weight layout,
output type, epilogue and forced tile drawn from a fixed seed
(RandomState(2029)).  Plain products on integer inputs must match the CPU
oracle bit for bit; SiLU-gated ones meet the bf16 rule.  D carries guard
rows past the routed rows, which must stay untouched.
"""
import sys

import numpy as np
import pytest

import oracle
from helpers import assert_bits_equal, assert_close, from_dev_bits, to_dev

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")
from test_gpu_grouped import GROUPED_TILES, grouped, make_case  # noqa: E402

pytestmark = pytest.mark.gpu

NCASES = 48


def draw_counts(rs, G):
    kinds = rs.choice(4, size=G, p=[0.2, 0.3, 0.3, 0.2])
    lo = [0, 1, 17, 129]
    hi = [1, 17, 129, 420]
    return [int(rs.randint(lo[k], hi[k])) for k in kinds]


def draw_cases():
    rs = np.random.RandomState(2029)
    cases = []
    for i in range(NCASES):
        G = int(rs.randint(1, 25))
        counts = draw_counts(rs, G)
        silu = rs.randint(3) == 0
        bl = ["row", "col"][rs.randint(2)]
        out_t = "bf16" if silu else ["bf16", "f32"][rs.randint(2)]
        # 16-byte rows: N % 8 == 0 unless the weights are [N][K] and D is fp32
        step = 16 if silu else (4 if bl == "col" and out_t == "f32" else 8)
        N = step * int(rs.randint(1, 640 // step + 1))
        K = 8 * int(rs.randint(1, 61))
        tile = list(GROUPED_TILES)[rs.randint(len(GROUPED_TILES))]
        cases.append((i, G, tuple(counts), N, K, bl, out_t, silu, tile))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-G{c[1]}-N{c[3]}-K{c[4]}-{c[5]}-{c[6]}-{'silu' if c[7] else 'plain'}-{c[8]}"
                                             for c in CASES])
def test_random_grouped(case):
    i, G, counts, N, K, bl, out_t, silu, tile = case
    print(f"case {i}: G={G} counts={list(counts)} N={N} K={K} {bl} ->{out_t} silu={silu} tile={tile}",
          flush=True, file=sys.stderr)
    A, W, off = make_case(list(counts), N, K, 7000 + i, "int")
    Wst = W if bl == "row" else np.ascontiguousarray(W.transpose(0, 2, 1))
    rows = int(off[-1])
    epi = mg.EPI_SILU_GATE_I8 if silu else mg.EPI_NONE
    D, raw, plan = grouped(to_dev(A, "bf16"), to_dev(Wst, "bf16"), torch.from_numpy(off).cuda(), G, rows, N, K,
                           out_t=out_t, epi=epi, b_layout=bl, flags=GROUPED_TILES[tile], extra_rows=2)
    ref = oracle.grouped_ref(A, Wst, off, w_layout=bl)
    got = from_dev_bits(D[:rows])
    if silu:
        assert_close(got, oracle.silu_gate(ref), K, "bf16", f"case {i}: {plan.describe()}")
    else:
        assert_bits_equal(got, ref, out_t, f"case {i}: {plan.describe()}")
    out_cols = N // 2 if silu else N
    es = 4 if out_t == "f32" else 2
    tail = raw[rows * out_cols * es:].cpu().numpy()
    assert np.all(tail == 0xFF), f"case {i}: rows past the routed rows were written"
