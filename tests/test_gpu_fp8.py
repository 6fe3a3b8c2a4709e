"""GPU parity of the E4M3 dense product with per-tensor scales
(gemm_run_scaled) against the CPU oracle: D = scale_a * scale_b * (A x B),
A [M][K] and B [N][K] E4M3 codes, fp32 accumulate, one rounding to the
output type.

Integer-valued codes with power-of-two scales make every sum exact in fp32
(and in any accumulator of 24 bits or more), so those cases are bit-exact.
Random codes are held to a bound in the sum of absolute products, in two
parts:
  * each v_mfma_f32_16x16x128_f8f6f4 reduces its (up to) 128 exact products
    internally; the ISA documentation states the result (the sum added to
    the accumulator) but not the order, width or rounding of that
    reduction, so this part can only be bounded empirically: INSTR = 2^-13
    of scale * sum|a b| (the worst seen is 2^-15.2, at K = 16, one
    instruction with 16 nonzero products -- far above one fp32 rounding, so
    the reduction is narrower than an fp32 chain);
  * the ceil(K/128) instruction results are then added into the fp32
    accumulator, each addition rounding once: at most ceil(K/128) * 2^-24
    of scale * sum|a b| (the n*u bound of a recursive sum);
plus the final rounding to the output type, 2^-22 (f32: the scale multiply
and the store), 2^-8 (bf16) or 2^-10 (f16) of |ref|.  Every random case
logs its worst err / (scale * sum|a b|) and err / tolerance.
"""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal, from_dev_bits, sample_positions, values

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu

REL = {"f32": 2.0 ** -22, "bf16": 2.0 ** -8, "f16": 2.0 ** -10}
TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def dev_u8(a, ld=None):
    """[rows][K] codes on the device, rows ld bytes apart (slack holds NaN codes)."""
    rows, K = a.shape
    ld = K if ld is None else ld
    buf = np.full((rows, ld), 0x7F, dtype=np.uint8)
    buf[:, :K] = a
    return torch.from_numpy(buf).cuda()


def scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def run(A, B, M, N, K, out, sa, sb, lda=None, ldb=None, flags=0):
    """D's rows padded to 16 bytes (16-bit outputs: ldd a multiple of 8);
    the padding starts as NaN and must stay so."""
    ldd = N if out == "f32" else -(-N // 8) * 8
    plan = mg.gemm_plan(M, N, K, a_type="e4m3", d_type=out, a_layout="row", b_layout="col",
                        lda=lda or K, ldb=ldb or K, ldd=ldd, flags=flags)
    D = torch.full((M, ldd), float("nan"), dtype=TORCH_OUT[out], device="cuda")
    mg.gemm_run_scaled(plan, dev_u8(A, lda), dev_u8(B, ldb), D, scalar(sa), scalar(sb))
    torch.cuda.synchronize()
    assert torch.isnan(D[:, N:]).all(), "padding columns written"
    return plan, from_dev_bits(D[:, :N].contiguous())


INSTR = 2.0 ** -13     # one matrix instruction's internal reduction (empirical)


def rel_sum(K):
    """Bound on |err| / (scale * sum|a b|) before the output rounding."""
    return INSTR + -(-K // 128) * 2.0 ** -24


def bound(A, B, ref, out, s):
    """(tolerance, scale * sum|a b|)"""
    absum = abs(s) * oracle.gemm_e4m3_ref(A & 0x7F, B & 0x7F)
    return rel_sum(A.shape[1]) * absum + REL[out] * np.abs(ref) + 1e-30, absum


def inputs(M, N, K, variant, seed):
    rs = np.random.RandomState(seed)
    dist = ("int", 3) if variant == "int" else ("normal", 100.0)
    return datagen.matrix_e4m3((M, K), dist, rs), datagen.matrix_e4m3((N, K), dist, rs)


SHAPES = [(256, 256, 128), (300, 516, 400), (513, 260, 1040), (17, 36, 16), (1000, 772, 2064), (64, 1024, 4112)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("variant", ["random", "int"])
def test_against_oracle(shape, out, variant):
    M, N, K = shape
    log(f"case e4m3 {M}x{N}x{K} {out} {variant}")
    A, B = inputs(M, N, K, variant, seed=M + N + K)
    sa, sb = (0.5, 0.25) if variant == "int" else (0.0123, 0.75)
    plan, got = run(A, B, M, N, K, out, sa, sb)
    s = float(np.float32(sa)) * float(np.float32(sb))
    ref = oracle.gemm_e4m3_ref(A, B, float(np.float32(sa)), float(np.float32(sb)))
    if variant == "int":
        assert_bits_equal(got, ref, out, plan.describe())
    else:
        err = np.abs(values(got, out) - ref)
        tol, absum = bound(A, B, ref, out, s)
        log(f"  K={K}: max err / (scale * sum|ab|) = 2^{np.log2((err / absum).max() + 1e-300):.1f}, "
            f"max err / tol = {(err / tol).max():.3f}")
        assert np.all(err <= tol), f"{plan.describe()}: max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"


def test_wide_leading_dimensions_never_read_slack():
    M, N, K = 300, 260, 528
    A, B = inputs(M, N, K, "int", seed=4)
    plan, got = run(A, B, M, N, K, "f32", 1.0, 2.0, lda=K + 32, ldb=K + 48)
    assert_bits_equal(got, oracle.gemm_e4m3_ref(A, B, 1.0, 2.0), "f32", plan.describe())


def test_scales_read_when_the_kernel_runs():
    """One plan, the scale tensors rewritten on the device between runs; and
    gemm_run on an E4M3 plan is the product with both scales 1."""
    M, N, K = 256, 512, 256
    A, B = inputs(M, N, K, "int", seed=8)
    plan = mg.gemm_plan(M, N, K, a_type="e4m3", d_type="f32", a_layout="row", b_layout="col")
    dA, dB = dev_u8(A), dev_u8(B)
    s_a, s_b = scalar(1.0), scalar(1.0)
    D = torch.empty(M, N, dtype=torch.float32, device="cuda")
    base = oracle.gemm_e4m3_ref(A, B)
    for va, vb in [(1.0, 1.0), (4.0, 0.5), (-0.25, 8.0)]:
        s_a.fill_(va)
        s_b.fill_(vb)
        mg.gemm_run_scaled(plan, dA, dB, D, s_a, s_b)
        torch.cuda.synchronize()
        assert_bits_equal(from_dev_bits(D), base * (va * vb), "f32", f"scales {va} {vb}")
    D.fill_(float("nan"))
    mg.gemm_run(plan, dA, dB, D)
    torch.cuda.synchronize()
    assert_bits_equal(from_dev_bits(D), base, "f32", "gemm_run, unit scales")


def test_empty_and_zero_k():
    plan = mg.gemm_plan(0, 64, 64, a_type="e4m3", d_type="f32", a_layout="row", b_layout="col")
    mg.gemm_run_scaled(plan, None, None, torch.empty(0, device="cuda"), scalar(1.0), scalar(1.0))
    plan = mg.gemm_plan(40, 64, 0, a_type="e4m3", d_type="bf16", a_layout="row", b_layout="col", lda=16, ldb=16)
    D = torch.full((40, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    mg.gemm_run_scaled(plan, dev_u8(np.zeros((40, 16), np.uint8)), dev_u8(np.zeros((64, 16), np.uint8)), D,
                       scalar(3.0), scalar(3.0))
    torch.cuda.synchronize()
    assert (D == 0).all()


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_full_size_8192_sampled(out):
    """8192^3, the launch the bench times; sampled outputs (tile edges,
    borders and random positions) against the oracle element by element."""
    M = N = K = 8192
    log(f"case e4m3 8192^3 {out}")
    rs = np.random.RandomState(123)
    A = datagen.matrix_e4m3((M, K), ("normal", 100.0), rs)
    B = datagen.matrix_e4m3((N, K), ("normal", 100.0), rs)
    sa, sb = 0.01, 0.01
    plan, got = run(A, B, M, N, K, out, sa, sb)
    log("  " + plan.describe())
    r, c = sample_positions(M, N, 256, seed=5)
    fa, fb = float(np.float32(sa)), float(np.float32(sb))
    ref = oracle.gemm_e4m3_ref_sampled(A, B, r, c, fa, fb)
    absum = abs(fa * fb) * oracle.gemm_e4m3_ref_sampled(A & 0x7F, B & 0x7F, r, c)
    tol = rel_sum(K) * absum + REL[out] * np.abs(ref)
    err = np.abs(values(got[r, c], out) - ref)
    log(f"  K={K}: max err / (scale * sum|ab|) = 2^{np.log2((err / absum).max() + 1e-300):.1f}, "
        f"max err / tol = {(err / tol).max():.3f}")
    assert np.all(err <= tol), f"max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"
    # every output was written (no NaN fill left)
    assert not np.isnan(values(got, out)).any()
