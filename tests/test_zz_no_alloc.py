"""gemm_run_noalloc (the dense run whose scratch is the library's own
per-device array, for callers that cannot allocate) against gemm_run with a
caller-owned workspace, through the C ABI.

Both run the same kernels in the same order, so their outputs must be equal
bit for bit; each is also held to the oracle (random inputs within the
tolerance, integer inputs bit-exact).  Two calls in a row, the second with a
smaller problem, so the second finds the first one's partial sums left in
the array; and a plan without a split, which needs no scratch at all.
"""
import math
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal, assert_close, from_dev_bits, to_dev

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def run_both(M, N, K, bl, splits, variant, seed, tile_flags=0):
    cfg = datagen.GemmConfig("noalloc", M, N, K, "bf16", "bf16", "row", bl, ("normal", 1.0), ("normal", 0.02),
                             seed=seed, int_seed=seed + 1)
    a, b = datagen.gemm_inputs(cfg, variant)
    A, B = to_dev(a, "bf16"), to_dev(b, "bf16")
    flags = (mg.PLAN_SPLIT_K(splits) if splits else 0) | tile_flags
    ldd = -(-N // 8) * 8                  # 16-byte output rows
    plan = mg.gemm_plan(M, N, K, "bf16", d_type="bf16", b_layout=bl, ldd=ldd, flags=flags)
    log(f"case noalloc {M}x{N}x{K} B {bl} {variant}: {plan.describe()}")
    ws_bytes = plan.workspace_size()
    assert ws_bytes <= mg.NOALLOC_SCRATCH_BYTES
    ws = torch.full((max(ws_bytes, 16),), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes
    D_ref = torch.full((M, ldd), float("nan"), dtype=torch.bfloat16, device="cuda")
    D_new = torch.full((M, ldd), float("nan"), dtype=torch.bfloat16, device="cuda")
    mg.gemm_run(plan, A, B, D_ref, workspace=ws)
    mg.gemm_run_noalloc(plan, A, B, D_new)
    torch.cuda.synchronize()
    assert torch.isnan(D_new[:, N:].float()).all(), "padding columns written"
    got_ref, got_new = from_dev_bits(D_ref[:, :N]), from_dev_bits(D_new[:, :N])
    assert np.array_equal(got_new, got_ref), f"{plan.describe()}: gemm_run_noalloc differs from gemm_run"
    ref = oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl)
    if variant == "int":
        assert_bits_equal(got_new, ref, "bf16", plan.describe())
    else:
        assert_close(got_new, ref, K, "bf16", plan.describe())
    return plan


@pytest.mark.parametrize("variant", ["random", "int"])
def test_noalloc_matches_gemm_run_two_calls_second_smaller(variant):
    # first: the decode shape on the few-token tile (128 columns) split in
    # four: 56 arrival counters and 224 partial slabs of 64 KiB, 14.7 MB
    p1 = run_both(128, 7168, 2048, "row", 4, variant, seed=71, tile_flags=mg.PLAN_FORCE_TILE_NARROW)
    assert "narrow128" in p1.describe() and p1.workspace_size() == 512 + 56 * 4 * 65536
    # second, smaller: ragged N (an edge column), column-major B, three
    # ranges; the array still holds the first call's counters and partials
    p2 = run_both(40, 1002, 1024, "col", 3, variant, seed=72)
    assert 0 < p2.workspace_size() < p1.workspace_size()
    # and a split whose partial slabs a second kernel adds (128x128 tile)
    p3 = run_both(64, 512, 1024, "row", 4, variant, seed=74, tile_flags=mg.PLAN_FORCE_TILE_128x128)
    assert "tile=128x128" in p3.describe() and p3.workspace_size() == 4 * 64 * 512 * 4


def test_noalloc_without_split_needs_no_scratch():
    p = run_both(300, 520, 392, "row", 1, "int", seed=73)
    assert p.workspace_size() == 0


def test_noalloc_rejects_plans_beyond_the_array():
    plan = mg.gemm_plan(4096, 4096, 65536, "bf16", d_type="bf16", flags=mg.PLAN_SPLIT_K(8))
    assert plan.workspace_size() > mg.NOALLOC_SCRATCH_BYTES
    D = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mg.MgemmError) as e:
        mg.gemm_run_noalloc(plan, D, D, D)
    assert e.value.status == mg.ERR_WORKSPACE
    assert (D == 0).all()


def draw_noalloc_cases():
    """Seeded split plans (RandomState(2039)) run one after another, so each
    finds the previous one's partial sums in the library's array."""
    rs = np.random.RandomState(2039)
    tiles = {"nrw": mg.PLAN_FORCE_TILE_NARROW, "nrw64": mg.PLAN_FORCE_TILE_NARROW64,
             "nrw32": mg.PLAN_FORCE_TILE_NARROW32, "128": mg.PLAN_FORCE_TILE_128x128,
             "256": mg.PLAN_FORCE_TILE_256x256}
    cases = []
    for i in range(12):
        tile = list(tiles)[rs.randint(len(tiles))]
        M = int(rs.randint(1, 129)) if tile.startswith("nrw") else int(rs.randint(1, 600))
        N = 8 * int(rs.randint(1, 88))
        K = 8 * int(rs.randint(8, 200))
        cases.append((i, M, N, K, ["row", "col"][rs.randint(2)], int(rs.randint(2, 6)), tiles[tile], tile))
    return cases


NOALLOC_CASES = draw_noalloc_cases()


def test_noalloc_random_split_plans_in_sequence():
    for i, M, N, K, bl, splits, flags, tile in NOALLOC_CASES:
        log(f"case noalloc random {i}: tile={tile} splits={splits}")
        run_both(M, N, K, bl, splits, "int", 4000 + i, tile_flags=flags)
