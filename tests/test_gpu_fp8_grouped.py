"""GPU parity of the grouped E4M3 product (grouped_gemm_run_scaled) against
the CPU oracle: expert e's rows times its column-major weights, each sum
multiplied by scale_a * scale_b[e].  Integer codes with power-of-two scales
are bit-exact; random codes are held to the bound of the dense E4M3 tests
(test_gpu_fp8.rel_sum(K) of scale * sum|a b| -- the instruction's internal
reduction, bounded empirically, plus the fp32 chain over the K/128
instruction results -- and the output rounding)."""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal, from_dev_bits, values
from test_gpu_fp8 import rel_sum

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu

REL = {"f32": 2.0 ** -22, "bf16": 2.0 ** -8}
TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16}
COUNTS = [0, 1, 100, 256, 257, 600, 0, 33]


def log(*a):
    print(*a, flush=True, file=sys.stderr)


@pytest.mark.parametrize("K", [400, 1040])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["random", "int"])
def test_grouped_e4m3_against_oracle(K, out, variant):
    N, G = 512, len(COUNTS)
    log(f"case grouped e4m3 K={K} {out} {variant}")
    rs = np.random.RandomState(K + len(out))
    dist = ("int", 3) if variant == "int" else ("normal", 100.0)
    off = np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32)
    rows = int(off[-1])
    A = datagen.matrix_e4m3((rows + 5, K), dist, rs)  # 5 rows past off[G]: never written
    W = datagen.matrix_e4m3((G, N, K), dist, rs)
    sa = 0.5 if variant == "int" else 0.0123
    sb = (2.0 ** rs.randint(-3, 3, size=G)).astype(np.float32) if variant == "int" else \
        rs.uniform(0.5, 2.0, size=G).astype(np.float32)
    plan = mg.grouped_gemm_plan(G, rows + 5, N, K, a_type="e4m3", d_type=out, b_layout="col")
    D = torch.full((rows + 5, N), float("nan"), dtype=TORCH_OUT[out], device="cuda")
    mg.grouped_gemm_run_scaled(plan, torch.from_numpy(A).cuda(), torch.from_numpy(W).cuda(), D,
                               torch.from_numpy(off).cuda(), torch.tensor([sa], dtype=torch.float32).cuda(),
                               torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    got = from_dev_bits(D)
    assert np.isnan(values(got[rows:], out)).all(), "rows past off[G] written"
    fa = float(np.float32(sa))
    ref = oracle.grouped_e4m3_ref(A, W, off, fa, sb.astype(np.float64))[:rows]
    if variant == "int":
        assert_bits_equal(got[:rows], ref, out, plan.describe())
    else:
        absum = np.abs(oracle.grouped_e4m3_ref(A & 0x7F, W & 0x7F, off, fa, sb.astype(np.float64))[:rows])
        err = np.abs(values(got[:rows], out) - ref)
        tol = rel_sum(K) * absum + REL[out] * np.abs(ref)
        log(f"  K={K}: max err / (scale * sum|ab|) = 2^{np.log2((err / (absum + 1e-300)).max() + 1e-300):.1f}, "
            f"max err / tol = {(err / (tol + 1e-300)).max():.3f}")
        assert np.all(err <= tol), f"{plan.describe()}: max err {err.max():.3e}"


def test_grouped_e4m3_unit_scales_and_offsets_changed_on_device():
    """grouped_gemm_run (no scales) is the product with scales 1; one plan,
    the offsets rewritten on the device between runs."""
    G, N, K = 4, 256, 256
    rs = np.random.RandomState(3)
    A = datagen.matrix_e4m3((600, K), ("int", 2), rs)
    W = datagen.matrix_e4m3((G, N, K), ("int", 2), rs)
    plan = mg.grouped_gemm_plan(G, 600, N, K, a_type="e4m3", d_type="f32", b_layout="col")
    dA, dW = torch.from_numpy(A).cuda(), torch.from_numpy(W).cuda()
    offs = torch.zeros(G + 1, dtype=torch.int32, device="cuda")
    for counts in ([300, 0, 1, 299], [10, 256, 0, 100]):
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        offs.copy_(torch.from_numpy(off))
        D = torch.full((600, N), float("nan"), dtype=torch.float32, device="cuda")
        mg.grouped_gemm_run(plan, dA, dW, D, offs)
        torch.cuda.synchronize()
        ref = oracle.grouped_e4m3_ref(A, W, off, 1.0, np.ones(G))[:int(off[-1])]
        assert_bits_equal(from_dev_bits(D)[:int(off[-1])], ref, "f32", f"counts {counts}")
