"""Randomised E4M3 dense parity on the GPU, per-tensor (gemm_run_scaled)
and 128-block (gemm_run_blockscaled) scales: M, N, K, the output type and
the scales drawn from a fixed seed (RandomState(2031)).  Integer codes in
[-3, 3] with power-of-two scales (block scales within 2^-2..2^2, so every
partial and total sum stays exact in fp32) make every element bit-exact
against the CPU oracle.  D's padding columns start as NaN and must stay so.
"""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")
import test_gpu_fp8 as per_tensor  # noqa: E402
import test_gpu_fp8_block as block  # noqa: E402

pytestmark = pytest.mark.gpu

NCASES = 40


def draw_cases():
    rs = np.random.RandomState(2031)
    cases = []
    for i in range(NCASES):
        M = int(rs.randint(1, 700))
        N = 4 * int(rs.randint(1, 200))
        K = 16 * int(rs.randint(1, 100))
        out = ["f32", "bf16", "f16"][rs.randint(3)]
        blk = bool(rs.randint(2)) and out != "f16"
        sa, sb = 2.0 ** int(rs.randint(-3, 4)), 2.0 ** int(rs.randint(-3, 4))
        cases.append((i, M, N, K, out, blk, sa, sb))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}-{'block' if c[5] else 'tensor'}"
                                             for c in CASES])
def test_random_e4m3(case):
    i, M, N, K, out, blk, sa, sb = case
    print(f"case {i}: {M}x{N}x{K} ->{out} {'block scales' if blk else f'scales {sa} {sb}'}", flush=True,
          file=sys.stderr)
    rs = np.random.RandomState(9000 + i)
    A = datagen.matrix_e4m3((M, K), ("int", 3), rs)
    B = datagen.matrix_e4m3((N, K), ("int", 3), rs)
    if blk:
        kb = -(-K // 128)
        s_a = block.scales(M, K, -2, 2, rs, ld=kb + (kb & 1) + 2 * int(rs.randint(3)))
        s_b = block.scales(-(-N // 128), K, -2, 2, rs)
        plan, got = block.run(A, B, s_a, s_b, M, N, K, out)
        ref = oracle.gemm_e4m3_block_ref(A, B, s_a, s_b)
    else:
        plan, got = per_tensor.run(A, B, M, N, K, out, sa, sb)
        ref = oracle.gemm_e4m3_ref(A, B, sa, sb)
    assert_bits_equal(got, ref, out, f"case {i}: {plan.describe()}")
