"""GPU parity of the grouped E4M3 product with E8M0 block scales
(grouped_gemm_run_blockscaled) against the CPU oracle
(oracle.grouped_e4m3_block_ref): expert e's routed rows [off[e], off[e+1])
times its weight, each 128-k block's partial product scaled by the routed
row's scale and by the expert's 128 x 128 weight-block scale.

Integer-valued codes with scales 2^-2 .. 2^2 are bit-exact; random codes are
held, per expert, to the dense block-scaled test's bound (the scaled
instruction's own reduction bounded per instruction, one fp32 rounding per
k block, the output rounding)."""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal, from_dev_bits, values
from test_gpu_fp8 import TORCH_OUT
from test_gpu_fp8_block import block_bound, scales

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu

# empty, tiny, one and several 256-row blocks with ragged tails
COUNTS = [0, 1, 100, 256, 257, 600, 0, 33]


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def inputs(N, K, variant, seed, counts=COUNTS, extra=5):
    rs = np.random.RandomState(seed)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows, G = int(off[-1]), len(counts)
    dist = ("int", 3) if variant == "int" else ("normal", 100.0)
    lo, hi = (-2, 2) if variant == "int" else (-6, 6)
    A = datagen.matrix_e4m3((rows + extra, K), dist, rs)   # rows past off[G]: never written
    W = datagen.matrix_e4m3((G, N, K), dist, rs)
    sa = scales(rows + extra, K, lo, hi, rs)
    sb = np.stack([scales(-(-N // 128), K, lo, hi, rs) for _ in range(G)])
    return off, A, W, sa, sb


def run(off, A, W, sa, sb, N, K, out, plan=None):
    rows, G = A.shape[0], W.shape[0]
    if plan is None:
        plan = mg.grouped_gemm_plan(G, rows, N, K, a_type="e4m3", d_type=out, b_layout="col")
    D = torch.full((rows, N), float("nan"), dtype=TORCH_OUT[out], device="cuda")
    mg.grouped_gemm_run_blockscaled(plan, torch.from_numpy(A).cuda(), torch.from_numpy(W).cuda(), D,
                                    torch.from_numpy(off).cuda(), torch.from_numpy(sa).cuda(),
                                    torch.from_numpy(np.ascontiguousarray(sb)).cuda())
    torch.cuda.synchronize()
    return plan, from_dev_bits(D)


@pytest.mark.parametrize("K", [400, 1040])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["random", "int"])
def test_grouped_blockscaled_against_oracle(K, out, variant):
    N = 520   # two full column tiles and a ragged third (5 column blocks, the last 8 wide)
    log(f"case grouped e4m3 block K={K} {out} {variant}")
    off, A, W, sa, sb = inputs(N, K, variant, seed=K + 7 * len(out) + len(variant))
    rows = int(off[-1])
    plan, got = run(off, A, W, sa, sb, N, K, out)
    assert np.isnan(values(got[rows:], out)).all(), "rows past off[G] written"
    ref = oracle.grouped_e4m3_block_ref(A, W, off, sa, sb)[:rows]
    if variant == "int":
        assert_bits_equal(got[:rows], ref, out, plan.describe())
        return
    worst = 0.0
    for e in range(W.shape[0]):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        tol, _ = block_bound(A[lo:hi], W[e], sa[lo:hi], sb[e], ref[lo:hi], out)
        err = np.abs(values(got[lo:hi], out) - ref[lo:hi])
        worst = max(worst, float((err / tol).max()))
        assert np.all(err <= tol), f"{plan.describe()}: expert {e}, worst ratio {(err / tol).max():.3f}"
    log(f"  max err / tol = {worst:.3f}")


def test_grouped_blockscaled_unit_scales_equal_per_tensor():
    """Every scale 2^0: the bits of grouped_gemm_run_scaled with scales 1."""
    N, K = 256, 512
    off, A, W, sa, sb = inputs(N, K, "random", seed=5, counts=[300, 0, 1, 299, 64])
    sa[:, :K // 128] = 127
    sb[:, :, :K // 128] = 127
    rows, G = int(off[-1]), W.shape[0]
    plan, got = run(off, A, W, sa, sb, N, K, "f32")
    D = torch.full((A.shape[0], N), float("nan"), dtype=torch.float32, device="cuda")
    mg.grouped_gemm_run_scaled(plan, torch.from_numpy(A).cuda(), torch.from_numpy(W).cuda(), D,
                               torch.from_numpy(off).cuda(), torch.ones(1, device="cuda"),
                               torch.ones(G, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(got[:rows], from_dev_bits(D)[:rows])


def test_grouped_blockscaled_scale_moves_only_its_part():
    """Raising one routed row's scale of one k block changes that row only,
    to the oracle's bits; lowering one of an expert's weight-block scales
    changes only that expert's rows in that block's 128 columns."""
    N, K = 384, 512
    off, A, W, sa, sb = inputs(N, K, "int", seed=9, counts=[40, 300, 0, 129])
    rows = int(off[-1])
    plan, base = run(off, A, W, sa, sb, N, K, "f32")
    for r, b in ((45, 1), (339, 3), (300, 0)):
        sa2 = sa.copy()
        sa2[r, b] += 1
        _, got = run(off, A, W, sa2, sb, N, K, "f32", plan)
        assert_bits_equal(got[:rows], oracle.grouped_e4m3_block_ref(A, W, off, sa2, sb)[:rows], "f32",
                          f"row {r} block {b}")
        assert np.array_equal(np.delete(got[:rows], r, 0), np.delete(base[:rows], r, 0))
    sb2 = sb.copy()
    sb2[1, 2, 1] -= 1
    _, got = run(off, A, W, sa, sb2, N, K, "f32", plan)
    assert_bits_equal(got[:rows], oracle.grouped_e4m3_block_ref(A, W, off, sa, sb2)[:rows], "f32", "weight block")
    keep = np.ones((rows, N), dtype=bool)
    keep[off[1]:off[2], 256:384] = False
    assert np.array_equal(got[:rows][keep], base[:rows][keep])

