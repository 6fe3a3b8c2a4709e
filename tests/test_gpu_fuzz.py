"""Randomised dense parity on the GPU: many small shapes, each with a layout,
input and output type, forced tile (or the planner's choice), split count
and output leading dimension drawn from a fixed seed, on integer-valued
inputs, so that every element must match the CPU oracle bit for bit.  The
output buffer is guarded on both sides (see test_gpu_gemm.run_dense).

The draws are deterministic (numpy RandomState(2027)): a failing case is
replayed by its index, which the case id and the log line name.
"""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")
from test_gpu_gemm import run_dense  # noqa: E402

pytestmark = pytest.mark.gpu

FORCE = {"auto": 0, "256": mg.PLAN_FORCE_TILE_256x256, "128": mg.PLAN_FORCE_TILE_128x128,
         "32n": mg.PLAN_FORCE_TILE_32x256, "64n": mg.PLAN_FORCE_TILE_64x256,
         "256d": mg.PLAN_FORCE_TILE_256x256_DTL, "nrw": mg.PLAN_FORCE_TILE_NARROW,
         "nrw64": mg.PLAN_FORCE_TILE_NARROW64, "nrw32": mg.PLAN_FORCE_TILE_NARROW32}
K_CONTIGUOUS_A_ONLY = {"32n", "64n", "256d", "nrw", "nrw64", "nrw32"}
SPLITTABLE = {"auto", "128", "256", "nrw", "nrw64", "nrw32"}
NCASES = 96


def draw_cases():
    rs = np.random.RandomState(2027)
    cases = []
    for i in range(NCASES):
        tile = list(FORCE)[rs.randint(len(FORCE))]
        in_t = ["bf16", "f16"][rs.randint(2)]
        out_t = ["f32", in_t][rs.randint(2)]
        al = "row" if tile in K_CONTIGUOUS_A_ONLY else ["row", "col"][rs.randint(2)]
        bl = ["row", "col"][rs.randint(2)]
        # sizes: mostly small and ragged, some a few tiles wide; few tokens
        # for the narrow tiles half of the time
        M = int(rs.randint(1, 130)) if tile.startswith("nrw") and rs.randint(2) else int(rs.randint(1, 521))
        N = int(rs.randint(1, 521))
        K = 8 * int(rs.randint(1, 66))
        splits = int(rs.choice([1, 2, 3, 5])) if tile in SPLITTABLE and rs.randint(3) == 0 else 0
        pad = int(rs.choice([0, 0, 8, 24]))
        cases.append((i, tile, in_t, out_t, al, bl, M, N, K, splits, pad))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}-{c[4]}{c[5]}-{c[6]}x{c[7]}x{c[8]}-s{c[9]}"
                                             for c in CASES])
def test_random_shape_bit_exact(case):
    i, tile, in_t, out_t, al, bl, M, N, K, splits, pad = case
    print(f"case {i}: tile={tile} {in_t}->{out_t} {al}/{bl} M={M} N={N} K={K} splits={splits} pad={pad}",
          flush=True, file=sys.stderr)
    cfg = datagen.GemmConfig("fuzz", M, N, K, in_t, out_t, al, bl, seed=3000 + i, int_seed=5000 + i)
    a, b = datagen.gemm_inputs(cfg, "int")
    flags = FORCE[tile] | (mg.PLAN_SPLIT_K(splits) if splits else 0)
    ldd = (N + 7) // 8 * 8 + pad
    got, plan = run_dense(a, b, M, N, K, in_t, out_t, al, bl, flags, ldd=ldd, sentinel=True)
    assert_bits_equal(got, oracle.gemm_ref(a, b, in_t, in_t, al, bl), out_t, f"case {i}: {plan.describe()}")
