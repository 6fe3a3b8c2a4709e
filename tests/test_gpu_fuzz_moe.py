"""Randomised fused MoE layer (moe_fused_run) on the GPU: expert count,
per-expert row counts (empty, few-token and multi-block experts), hidden
and inter sizes drawn from a fixed seed (RandomState(2033)).  Each case must
give exactly the bits of the two grouped launches it replaces, end with a
clean status word, and meet the oracle's own chain (h under the bf16 rule,
y under it widened by the carried FC1 gap).
"""
import sys

import numpy as np
import pytest

import datagen
from helpers import to_dev

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")
from test_gpu_moe_fused import check_oracle, dev_i32, fused, offsets, status, two_launch  # noqa: E402

pytestmark = pytest.mark.gpu

NCASES = 16


def draw_cases():
    rs = np.random.RandomState(2033)
    cases = []
    for i in range(NCASES):
        E = int(rs.randint(1, 33))
        kinds = rs.choice(4, size=E, p=[0.15, 0.35, 0.3, 0.2])
        lo, hi = [0, 1, 17, 129], [1, 17, 129, 700]
        counts = tuple(int(rs.randint(lo[k], hi[k])) for k in kinds)
        H = 16 * int(rs.randint(1, 33))
        I = 64 * int(rs.randint(1, 7))
        cases.append((i, counts, H, I))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-E{len(c[1])}-rows{sum(c[1])}-H{c[2]}-I{c[3]}" for c in CASES])
def test_random_fused_moe(case):
    i, counts, H, I = case
    E, rows = len(counts), sum(counts)
    print(f"case {i}: E={E} counts={list(counts)} H={H} I={I}", flush=True, file=sys.stderr)
    off = offsets(list(counts))
    rs = np.random.RandomState(8000 + i)
    A = datagen.matrix((rows, H), ("normal", 1.0), "bf16", rs)
    W1 = datagen.matrix((E, H, 2 * I), ("normal", 0.05), "bf16", rs)
    W2 = datagen.matrix((E, I, H), ("normal", 0.05), "bf16", rs)
    Ad, W1d, W2d, offs = to_dev(A, "bf16"), to_dev(W1, "bf16"), to_dev(W2, "bf16"), dev_i32(off)
    h, y, plan, ws = fused(Ad, W1d, W2d, offs, E, rows, H, I, ws_fill=0xA5)
    torch.cuda.synchronize()
    assert status(ws) == 0, plan.describe()
    h2, y2 = two_launch(Ad, W1d, W2d, offs, E, rows, H, I)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16)), f"case {i}: h differs from the grouped launches"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"case {i}: y differs from the grouped launches"
    check_oracle(A, W1, W2, off, h, y, H, I, "bf16", f"case {i}: {plan.describe()}")
