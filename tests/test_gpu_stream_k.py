"""GPU parity of the stream-K tail on the four-wave 256 x 256 tile against
the CPU oracle.

When the output tiles leave the last round of the persistent grid at most
half busy, the plan runs the first tiles whole and cuts the last ones into
K ranges spread over the CUs; the last range of a cut tile to arrive adds
the ranges' fp32 partials in range order.  The cases have odd tile counts
(17 x 17), both B layouts, integer inputs compared bit for bit over every
output element, random inputs within the tolerance, repeated runs compared
bit for bit, and a workspace handed over full of 0xFF bytes.
"""
import sys
import zlib

import numpy as np
import pytest

import datagen
import oracle
from helpers import TORCH_OUT, assert_bits_equal, assert_close, from_dev_bits, sample_positions, to_dev

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def run(a, b, M, N, K, bl, out_t, flags=0, ws=None, plan=None):
    plan = plan or mg.gemm_plan(M, N, K, "bf16", d_type=out_t, b_layout=bl, flags=flags)
    D = torch.full((M, N), float("nan"), dtype=TORCH_OUT[out_t], device="cuda")
    if ws is None and plan.workspace_size():
        ws = torch.full((plan.workspace_size(),), 0xFF, dtype=torch.uint8, device="cuda")
    mg.gemm_run(plan, to_dev(a, "bf16"), to_dev(b, "bf16"), D, workspace=ws)
    torch.cuda.synchronize()
    return from_dev_bits(D), plan


@pytest.mark.parametrize("bl,out_t", [("row", "bf16"), ("col", "f32")])
def test_stream_k_every_element_integer(bl, out_t):
    """4352 x 4352 x 4096: 289 tiles of 256 x 256 on 256 CUs, the last 33
    cut into 4 ranges of 16 steps.  Every output element, bit-exact."""
    M = N = 4352
    K = 4096
    log(f"case stream-K {M}x{N}x{K} B {bl} -> {out_t}")
    cfg = datagen.GemmConfig("sk", M, N, K, "bf16", out_t, "row", bl, seed=61, int_seed=62 + (bl == "col"))
    a, b = datagen.gemm_inputs(cfg, "int")
    got, plan = run(a, b, M, N, K, bl, out_t)
    d = plan.describe()
    assert "tile=256x256dtl" in d and "stream_k_tiles=33" in d and "splits=4" in d, d
    assert_bits_equal(got, oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl), out_t, d)


@pytest.mark.parametrize("bl", ["row", "col"])
def test_stream_k_random_repeatable(bl):
    """Random inputs: within the tolerance on sampled outputs (tile edges,
    the cut tiles among them), and bit-identical over two runs on one
    workspace -- the fixup's order does not depend on which range arrives
    last."""
    M, N, K = 4608, 4096, 4096        # 18 x 16 = 288 tiles, the last 32 cut
    log(f"case stream-K random {M}x{N}x{K} B {bl}")
    cfg = datagen.GemmConfig("sk", M, N, K, "bf16", "bf16", "row", bl, ("normal", 1.0), ("normal", 0.02), seed=71,
                             int_seed=72)
    a, b = datagen.gemm_inputs(cfg, "random")
    plan = mg.gemm_plan(M, N, K, "bf16", d_type="bf16", b_layout=bl)
    assert "stream_k_tiles=32" in plan.describe(), plan.describe()
    ws = torch.full((plan.workspace_size(),), 0xFF, dtype=torch.uint8, device="cuda")
    g1, _ = run(a, b, M, N, K, bl, "bf16", ws=ws, plan=plan)
    g2, _ = run(a, b, M, N, K, bl, "bf16", ws=ws, plan=plan)
    assert np.array_equal(g1, g2), "stream-K results differ between runs"
    seed = zlib.crc32(f"sk{bl}".encode()) % 1000
    r, c = sample_positions(M, N, 3000, (256, 256), seed=seed)
    # the cut tiles are the last 32 in the group-of-4-rows order: rows 4096..4607
    r = np.concatenate([r, np.random.RandomState(seed).randint(4096, M, 2000)])
    c = np.concatenate([c, np.random.RandomState(seed + 1).randint(0, N, 2000)])
    ref = oracle.gemm_ref_sampled(a, b, r, c, "bf16", "bf16", "row", bl)
    assert_close(g1[r, c], ref, K, "bf16", plan.describe())


def test_stream_k_against_unbalanced_plan_integer():
    """The verdict's tail shape, 5120 x 4096 x 8192 (320 tiles: 256 whole,
    64 cut into 4 ranges), integer inputs: equal bit for bit to the plan
    that runs every tile whole (two rounds), and to the oracle on samples."""
    M, N, K = 5120, 4096, 8192
    log(f"case stream-K vs unbalanced {M}x{N}x{K}")
    cfg = datagen.GemmConfig("sk", M, N, K, "bf16", "bf16", "row", "col", seed=81, int_seed=82)
    a, b = datagen.gemm_inputs(cfg, "int")
    got, plan = run(a, b, M, N, K, "col", "bf16")
    assert "stream_k_tiles=64" in plan.describe(), plan.describe()
    whole, p1 = run(a, b, M, N, K, "col", "bf16", flags=mg.PLAN_SPLIT_K(1) | mg.PLAN_FORCE_TILE_256x256_DTL)
    assert "stream_k" not in p1.describe() and "splits=1" in p1.describe(), p1.describe()
    assert np.array_equal(got, whole)
    r, c = sample_positions(M, N, 2000, (256, 256), seed=83)
    assert_bits_equal(got[r, c], oracle.gemm_ref_sampled(a, b, r, c, "bf16", "bf16", "row", "col"), "bf16",
                      plan.describe())
