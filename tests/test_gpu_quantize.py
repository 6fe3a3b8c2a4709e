"""GPU parity of the blockwise E4M3 quantisation (mgemm_quantize_e4m3_block)
against the CPU oracle (oracle.quantize_e4m3_block): codes and E8M0 scale
bytes bit for bit, with padded pitches whose padding must stay untouched,
and its output fed as A to the block-scaled product."""
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

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def source(rows, cols, dtype, seed):
    """Rows of normal values at magnitudes 2^-e .. 2^e (e = 20 for bf16, 6 for
    fp16), an all-zero block, negative zeros, one block with an infinity and
    one with a NaN; returned as the 16-bit values in float64."""
    rs = np.random.RandomState(seed)
    e = 20 if dtype == "bf16" else 6
    x = rs.standard_normal((rows, cols)) * 2.0 ** rs.randint(-e, e + 1, size=(rows, 1))
    x[1, 128:256] = 0.0                     # (when there is a second block)
    x[2, 7] = -0.0
    x[3, min(300, cols - 2)] = np.inf
    x[4, cols - 1] = np.nan
    x[5, ::3] = 0.0
    return torch.from_numpy(x).to(TDT[dtype]).to(torch.float64).numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("cols", [1000, 128, 2048, 998])   # 998: not a multiple of 8, the one-wave-per-block kernel
def test_quantize_against_oracle(dtype, cols):
    rows = 37
    log(f"case quantize {dtype} {rows}x{cols}")
    x = source(rows, cols, dtype, seed=cols + len(dtype))
    nb = -(-cols // 128)
    X = torch.zeros(rows, cols + 32, dtype=TDT[dtype], device="cuda")
    X[:, :cols] = torch.from_numpy(x).to(TDT[dtype]).cuda()
    Q = torch.full((rows, cols + 24), 0xAA, dtype=torch.uint8, device="cuda")
    S = torch.full((rows, nb + 3), 0xAA, dtype=torch.uint8, device="cuda")
    mg.quantize_e4m3_block(X[:, :cols], Q[:, :cols], S[:, :nb])
    torch.cuda.synchronize()
    q, s = Q.cpu().numpy(), S.cpu().numpy()
    assert (q[:, cols:] == 0xAA).all() and (s[:, nb:] == 0xAA).all(), "padding written"
    qr, sr = oracle.quantize_e4m3_block(x)
    assert np.array_equal(s[:, :nb], sr), "scales differ"
    bad = np.argwhere(q[:, :cols] != qr)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"
    bi = min(300, cols - 2) // 128
    assert s[3, bi] == 255 and (q[3, 128 * bi:min(128 * bi + 128, cols)] == 0x7F).all()
    if cols >= 256:
        assert s[1, 1] == 127 and not q[1, 128:256].any()


def test_quantize_empty_is_a_no_op():
    X = torch.zeros(0, 256, dtype=torch.bfloat16, device="cuda")
    Q = torch.zeros(0, 256, dtype=torch.uint8, device="cuda")
    S = torch.zeros(0, 2, dtype=torch.uint8, device="cuda")
    mg.quantize_e4m3_block(X, Q, S)
    torch.cuda.synchronize()


def test_quantized_rows_feed_the_block_scaled_product():
    """X quantised on the GPU is A of gemm_run_blockscaled (lda = ldq, lds_a =
    the scale pitch): the product matches the oracle's block-scaled product
    of the oracle's own quantisation of X, within the block-scaled bound."""
    M, N, K = 300, 260, 1040
    rs = np.random.RandomState(77)
    x = torch.from_numpy(rs.standard_normal((M, K)) * 4.0).to(torch.bfloat16)
    kb = -(-K // 128)
    X = x.cuda()
    Q = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    S = torch.full((M, kb + (kb & 1)), 255, dtype=torch.uint8, device="cuda")
    mg.quantize_e4m3_block(X, Q, S[:, :kb])
    B = datagen.matrix_e4m3((N, K), ("normal", 100.0), rs)
    sb = scales(-(-N // 128), K, -6, -4, rs)
    plan = mg.gemm_plan(M, N, K, a_type="e4m3", d_type="f32", a_layout="row", b_layout="col")
    D = torch.empty(M, N, dtype=torch.float32, device="cuda")
    mg.gemm_run_blockscaled(plan, Q, torch.from_numpy(B).cuda(), D, S, torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    qr, sr = oracle.quantize_e4m3_block(x.to(torch.float64).numpy())
    assert np.array_equal(Q.cpu().numpy(), qr) and np.array_equal(S[:, :kb].cpu().numpy(), sr)
    sa = np.full((M, kb + (kb & 1)), 255, np.uint8)
    sa[:, :kb] = sr
    ref = oracle.gemm_e4m3_block_ref(qr, B, sa, sb)
    tol, _ = block_bound(qr, B, sa, sb, ref, "f32")
    err = np.abs(values(from_dev_bits(D), "f32") - ref)
    log(f"  quantised product: max err / tol = {(err / tol).max():.3f}")
    assert np.all(err <= tol)


def test_quantized_h_feeds_the_grouped_block_scaled_fc2():
    """The FP8 form of an MoE layer's FC2 input: h (bf16, experts of 0-300
    rows) quantised on the GPU, then grouped_gemm_run_blockscaled with E4M3
    expert weights and their block scales; per expert within the
    block-scaled bound of the oracle's product of the oracle's own
    quantisation (which the GPU's codes and scales equal bit for bit)."""
    counts = [0, 37, 300, 1, 129, 0, 64]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows, G, I, H = int(off[-1]), len(counts), 768, 384
    rs = np.random.RandomState(78)
    h = torch.from_numpy(rs.standard_normal((rows, I)) * 0.5).to(torch.bfloat16)
    kb = I // 128
    hq = torch.empty(rows, I, dtype=torch.uint8, device="cuda")
    hs = torch.empty(rows, kb, dtype=torch.uint8, device="cuda")
    mg.quantize_e4m3_block(h.cuda(), hq, hs)
    W2 = datagen.matrix_e4m3((G, H, I), ("normal", 100.0), rs)
    sb = np.stack([scales(-(-H // 128), I, -8, -6, rs) for _ in range(G)])
    plan = mg.grouped_gemm_plan(G, rows, H, I, a_type="e4m3", d_type="f32", b_layout="col")
    Y = torch.full((rows, H), float("nan"), dtype=torch.float32, device="cuda")
    mg.grouped_gemm_run_blockscaled(plan, hq, torch.from_numpy(W2).cuda(), Y, torch.from_numpy(off).cuda(), hs,
                                    torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    qr, sr = oracle.quantize_e4m3_block(h.to(torch.float64).numpy())
    assert np.array_equal(hq.cpu().numpy(), qr) and np.array_equal(hs.cpu().numpy(), sr)
    ref = oracle.grouped_e4m3_block_ref(qr, W2, off, sr, sb)
    got = values(from_dev_bits(Y), "f32")
    for e in range(G):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            tol, _ = block_bound(qr[lo:hi], W2[e], sr[lo:hi], sb[e], ref[lo:hi], "f32")
            assert np.all(np.abs(got[lo:hi] - ref[lo:hi]) <= tol), f"expert {e}"
