"""GPU parity of the blockwise-scaled E4M3 product (gemm_run_blockscaled)
against the CPU oracle (oracle.gemm_e4m3_block_ref):
  D[i,j] = sum_b sa[i,b] sb[j/128,b] sum_{k in block b} A[i,k] B[j,k]
with E8M0 scale bytes, one per (row, 128-k block) of A and per (128
columns, 128-k block) of B, A [M][K] and B [N][K] E4M3 codes.

Integer-valued codes with scales 2^-2 .. 2^2 keep every partial and total
sum exact in fp32, so those cases are bit-exact.  Random codes are held to
a bound in three parts:
  * each v_mfma_scale_f32_16x16x128_f8f6f4 adds its 128 scaled products
    (and the incoming accumulator) inside its own reduction, whose width
    and rounding the ISA documentation does not state, so this part is
    bounded empirically, per instruction, against |C_b| + S_b (S_b the
    block's sum|s a b|, C_b what the earlier blocks carried in): measured,
    full 128-k blocks stay within 2^-15.2 of it, but a block with few
    nonzero products (the last block of K = 400 holds 16) reaches 2^-12.8
    of its own S_b -- with scales 2^-6 .. 2^6 such a block can carry most
    of an output, which no bound in the total sum|s a b| alone covers.  So
    this part is INSTR_S x sum_b (|C_b| + S_b) <= INSTR_S x sum_b (kb - b)
    S_b with INSTR_S = 2^-12;
  * one fp32 rounding per 128-k block when the result is stored: at most
    ceil(K/128) x 2^-24 of the total sum|s a b|;
  * the output rounding, 2^-22 (f32), 2^-8 (bf16) of |ref|.
Every random case logs its worst ratio to the bound.
"""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal, from_dev_bits, values
from test_gpu_fp8 import REL, TORCH_OUT, dev_u8, scalar

INSTR_S = 2.0 ** -12   # one scaled instruction, relative to |C| + its block's sum|s a b| (empirical)


def block_bound(A, B, sa, sb, ref, out):
    """(tolerance, total sum|s a b|): the three parts above, the per-block
    absolute sums S_b taken in float64 from the decoded codes."""
    M, K = A.shape
    N = B.shape[0]
    kb = -(-K // 128)
    a = np.abs(oracle.decode_e4m3(A))
    b = np.abs(oracle.decode_e4m3(B))
    ea = np.vectorize(oracle.e8m0)(sa[:, :kb])            # [M][kb]
    eb = np.vectorize(oracle.e8m0)(sb[:, :kb])            # [ceil(N/128)][kb]
    colblk = np.arange(N) // 128
    weighted = np.zeros((M, N))
    total = np.zeros((M, N))
    for blk in range(kb):
        ks = slice(128 * blk, min(128 * blk + 128, K))
        S = (a[:, ks] @ b[:, ks].T) * ea[:, blk][:, None] * eb[colblk, blk][None, :]
        total += S
        weighted += (kb - blk) * S
    return INSTR_S * weighted + kb * 2.0 ** -24 * total + REL[out] * np.abs(ref) + 1e-30, total

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def scales(rows, K, lo, hi, rs, ld=None):
    """E8M0 bytes [rows][ld] (ld even, at least ceil(K/128)); the padding
    holds NaN scales, which must never be used."""
    kb = -(-K // 128)
    ld = kb + (kb & 1) if ld is None else ld
    s = np.full((rows, ld), 255, dtype=np.uint8)   # slack: NaN scales, never read
    s[:, :kb] = rs.randint(127 + lo, 127 + hi + 1, size=(rows, kb))
    return s


def run(A, B, sa, sb, M, N, K, out):
    ldd = N if out == "f32" else -(-N // 8) * 8
    plan = mg.gemm_plan(M, N, K, a_type="e4m3", d_type=out, a_layout="row", b_layout="col", ldd=ldd)
    D = torch.full((M, ldd), float("nan"), dtype=TORCH_OUT[out], device="cuda")
    mg.gemm_run_blockscaled(plan, dev_u8(A), dev_u8(B), D, torch.from_numpy(sa).cuda(),
                            torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    assert torch.isnan(D[:, N:]).all(), "padding columns written"
    return plan, from_dev_bits(D[:, :N].contiguous())


def inputs(M, N, K, variant, seed):
    rs = np.random.RandomState(seed)
    dist = ("int", 3) if variant == "int" else ("normal", 100.0)
    A, B = datagen.matrix_e4m3((M, K), dist, rs), datagen.matrix_e4m3((N, K), dist, rs)
    lo, hi = (-2, 2) if variant == "int" else (-6, 6)
    kb = -(-K // 128)
    return A, B, scales(M, K, lo, hi, rs, ld=kb + (kb & 1) + 4), scales(-(-N // 128), K, lo, hi, rs)


# several tiles; ragged M, N and K (a last k block of 16 / 72 / 16); an odd
# number of k blocks (the step pairs end past K); one partial block only
SHAPES = [(512, 512, 1024), (300, 516, 400), (513, 260, 1040), (17, 36, 16), (256, 384, 896), (64, 1024, 4112)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["random", "int"])
def test_blockscaled_against_oracle(shape, out, variant):
    M, N, K = shape
    log(f"case e4m3 block {M}x{N}x{K} {out} {variant}")
    A, B, sa, sb = inputs(M, N, K, variant, seed=M + 3 * N + 7 * K)
    plan, got = run(A, B, sa, sb, M, N, K, out)
    ref = oracle.gemm_e4m3_block_ref(A, B, sa, sb)
    if variant == "int":
        assert_bits_equal(got, ref, out, plan.describe())
    else:
        tol, absum = block_bound(A, B, sa, sb, ref, out)
        err = np.abs(values(got, out) - ref)
        log(f"  max err / sum|s a b| = 2^{np.log2((err / (absum + 1e-300)).max() + 1e-300):.1f}, "
            f"max err / tol = {(err / tol).max():.3f}")
        assert np.all(err <= tol), f"{plan.describe()}: max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"


def test_unit_scales_equal_the_per_tensor_product():
    """Every scale 2^0: the bits of gemm_run_scaled with scales 1 (the
    scaled instruction with unit scales computes the unscaled one's sums)."""
    M, N, K = 512, 768, 2048
    rs = np.random.RandomState(3)
    A, B = datagen.matrix_e4m3((M, K), ("normal", 50.0), rs), datagen.matrix_e4m3((N, K), ("normal", 50.0), rs)
    sa = np.full((M, K // 128), 127, np.uint8)      # K // 128 = 16: even pitches
    sb = np.full((N // 128, K // 128), 127, np.uint8)
    _, got = run(A, B, sa, sb, M, N, K, "f32")
    plan = mg.gemm_plan(M, N, K, a_type="e4m3", d_type="f32", a_layout="row", b_layout="col")
    D = torch.empty(M, N, dtype=torch.float32, device="cuda")
    mg.gemm_run_scaled(plan, dev_u8(A), dev_u8(B), D, scalar(1.0), scalar(1.0))
    torch.cuda.synchronize()
    assert np.array_equal(got, from_dev_bits(D))


def test_scale_moves_only_its_block():
    """Raising one A scale byte by one doubles exactly that row's part from
    that k block; raising one B scale byte changes only its 128 columns."""
    M, N, K = 256, 512, 512
    A, B, sa, sb = inputs(M, N, K, "int", seed=21)
    _, base = run(A, B, sa, sb, M, N, K, "f32")
    # rows in each half of both wave rows of the tile (the kernel loads a
    # wave's 128 rows of scales as two halves of 64)
    for row, kb in ((37, 2), (100, 0), (131, 3), (250, 1)):
        sa2 = sa.copy()
        sa2[row, kb] += 1
        _, got = run(A, B, sa2, sb, M, N, K, "f32")
        assert_bits_equal(got, oracle.gemm_e4m3_block_ref(A, B, sa2, sb), "f32", f"A scale of row {row} raised")
        assert np.array_equal(np.delete(got, row, 0), np.delete(base, row, 0))
    sb2 = sb.copy()
    sb2[3, 1] -= 2
    _, got = run(A, B, sa, sb2, M, N, K, "f32")
    assert_bits_equal(got, oracle.gemm_e4m3_block_ref(A, B, sa, sb2), "f32", "B scale lowered")
    assert np.array_equal(got[:, :384], base[:, :384])


def test_blockscaled_full_size_sampled():
    """8192^3 with random codes and scales 2^-6 .. 2^6, bf16 out: 12 rows
    (first, last, a seeded sample) checked in full against the oracle."""
    M = N = K = 8192
    log("case e4m3 block 8192^3 sampled")
    rs = np.random.RandomState(8192)
    A = datagen.matrix_e4m3((M, K), ("normal", 100.0), rs)
    B = datagen.matrix_e4m3((N, K), ("normal", 100.0), rs)
    sa, sb = scales(M, K, -6, 6, rs), scales(N // 128, K, -6, 6, rs)
    plan, got = run(A, B, sa, sb, M, N, K, "bf16")
    rows = sorted({0, M - 1, *rs.randint(0, M, 10).tolist()})
    ref = oracle.gemm_e4m3_block_ref(A[rows], B, sa[rows], sb)
    tol, _ = block_bound(A[rows], B, sa[rows], sb, ref, "bf16")
    err = np.abs(values(got[rows], "bf16") - ref)
    log(f"  rows {rows}: max err / tol = {(err / tol).max():.3f}")
    assert np.all(err <= tol), f"{plan.describe()}: worst ratio {(err / tol).max():.3f}"
