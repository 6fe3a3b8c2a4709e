"""CPU pins of the FP8 (E4M3) oracle: the decoder against the format's own
constants and against torch's float8_e4m3fn conversion over all 256 codes,
the per-tensor-scaled product against exact rational brute force, and the
identities a transposed operand pair and the scales must satisfy."""
import math
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle

torch = pytest.importorskip("torch")


def test_decode_format_constants():
    """Values fixed by the E4M3 layout (bias 7, 3 fraction bits, subnormals
    below exponent field 1, no infinities, NaN only at S.1111.111)."""
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
            0x3C: 1.5, 0x40: 2.0, 0x44: 3.0, 0x4F: 7.5, 0x57: 15.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
            0xB8: -1.0, 0xFE: -448.0}
    got = oracle.decode_e4m3(np.array(list(want), dtype=np.uint8))
    assert got.tolist() == list(want.values())
    assert math.copysign(1.0, oracle.decode_e4m3(np.array([0x80], dtype=np.uint8))[0]) == -1.0
    assert np.isnan(oracle.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    assert np.isfinite(oracle.decode_e4m3(np.array([0x7E, 0xF8, 0x7D], dtype=np.uint8))).all()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def finite_codes(shape, rs):
    c = rs.randint(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


def test_product_against_rational_brute_force():
    rs = np.random.RandomState(5)
    M, N, K = 5, 4, 37
    A, B = finite_codes((M, K), rs), finite_codes((N, K), rs)
    sa, sb = 0.375, 1.0 / 1024
    val = lambda c: Fraction(torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn)
                             .to(torch.float64).item())
    got = oracle.gemm_e4m3_ref(A, B, sa, sb)
    for i in range(M):
        for j in range(N):
            exact = Fraction(sa) * Fraction(sb) * sum(val(A[i, k]) * val(B[j, k]) for k in range(K))
            # the double sum of at most 37 products of 4-bit significands is exact
            assert Fraction(got[i, j]) == exact, (i, j)


def test_transpose_and_scale_identities():
    rs = np.random.RandomState(9)
    A, B = finite_codes((24, 50), rs), finite_codes((17, 50), rs)
    base = oracle.gemm_e4m3_ref(A, B)
    assert np.array_equal(oracle.gemm_e4m3_ref(B, A), base.T)
    assert np.array_equal(oracle.gemm_e4m3_ref(A, B, 4.0, 0.125), base * 0.5)
    # a code's sign bit flips the sign of its row of the product
    An = A.copy()
    An[3] ^= 0x80
    neg = oracle.gemm_e4m3_ref(An, B)
    assert np.array_equal(neg[3], -base[3]) and np.array_equal(np.delete(neg, 3, 0), np.delete(base, 3, 0))


def test_special_case_identity_and_sampled():
    """One code per row of A at position i (the rest zero) picks row i of B:
    A x B = diag(values) selection; the sampled form agrees with the full one."""
    rs = np.random.RandomState(2)
    K = 16
    A = np.zeros((K, K), dtype=np.uint8)
    A[np.arange(K), np.arange(K)] = 0x38  # 1.0
    B = finite_codes((7, K), rs)
    got = oracle.gemm_e4m3_ref(A, B)
    assert np.array_equal(got, oracle.decode_e4m3(B).T)
    A2, B2 = finite_codes((33, 70), rs), finite_codes((29, 70), rs)
    full = oracle.gemm_e4m3_ref(A2, B2, 2.0, 3.0)
    r, c = rs.randint(0, 33, 40), rs.randint(0, 29, 40)
    assert np.array_equal(oracle.gemm_e4m3_ref_sampled(A2, B2, r, c, 2.0, 3.0), full[r, c])


def test_datagen_codes_are_finite_and_round_to_nearest():
    rs = np.random.RandomState(1)
    c = datagen.matrix_e4m3((64, 64), ("normal", 100.0), rs)
    v = oracle.decode_e4m3(c)
    assert np.isfinite(v).all() and np.abs(v).max() <= 448.0
    ci = datagen.matrix_e4m3((8, 8), ("int", 3), np.random.RandomState(2))
    vi = oracle.decode_e4m3(ci)
    assert np.array_equal(vi, np.round(vi)) and np.abs(vi).max() <= 3


def test_grouped_is_the_per_expert_product():
    """Each expert's rows equal the dense product of those rows and that
    expert's weights with its own scale; empty experts produce nothing and a
    one-row expert is one row of the dense product."""
    rs = np.random.RandomState(4)
    counts = [0, 1, 7, 0, 12]
    off = np.concatenate([[0], np.cumsum(counts)])
    K, N = 48, 20
    A = finite_codes((int(off[-1]) + 3, K), rs)
    W = finite_codes((len(counts), N, K), rs)
    sb = np.array([1.0, 0.5, 2.0, 4.0, 0.25])
    got = oracle.gemm_e4m3_ref  # the dense form, pinned above
    g = oracle.grouped_e4m3_ref(A, W, off, 0.75, sb)
    assert np.isnan(g[int(off[-1]):]).all()
    dense_all = {e: got(A, W[e]) for e in range(len(counts))}
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        assert np.array_equal(g[lo:hi], dense_all[e][lo:hi] * (0.75 * sb[e]))


# --- blockwise scales (E8M0 bytes: one per row of A and 128-k block, one per
# 128 output columns and 128-k block) ---

def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0(c) for c in codes])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert (oracle.e8m0(127), oracle.e8m0(128), oracle.e8m0(126)) == (1.0, 2.0, 0.5)


def unit_scales(M, N, K):
    return (np.full((M, -(-K // 128)), 127, np.uint8), np.full((-(-N // 128), -(-K // 128)), 127, np.uint8))


def test_block_unit_scales_are_the_per_tensor_product():
    rs = np.random.RandomState(11)
    M, N, K = 9, 200, 300   # two column blocks, three k blocks (the last one 44 long)
    A, B = finite_codes((M, K), rs), finite_codes((N, K), rs)
    sa, sb = unit_scales(M, N, K)
    assert np.array_equal(oracle.gemm_e4m3_block_ref(A, B, sa, sb), oracle.gemm_e4m3_ref(A, B))


def test_block_closed_form_all_ones():
    """A = B = 1.0 everywhere: block b's partial product is its length, so
    D[i, j] = sum_b len_b 2^(ea[i,b] + eb[j//128, b]) with len = 128, 128, 128, 72."""
    M, N, K = 6, 300, 456
    A = np.full((M, K), 0x38, np.uint8)
    B = np.full((N, K), 0x38, np.uint8)
    ea = np.array([[(i + b) % 3 - 1 for b in range(4)] for i in range(M)])
    eb = np.array([[(c + 2 * b) % 2 for b in range(4)] for c in range(3)])
    sa, sb = (ea + 127).astype(np.uint8), (eb + 127).astype(np.uint8)
    got = oracle.gemm_e4m3_block_ref(A, B, sa, sb)
    lens = [128, 128, 128, 72]
    for i in range(M):
        for j in range(N):
            assert got[i, j] == sum(lens[b] * 2.0 ** (ea[i, b] + eb[j // 128, b]) for b in range(4)), (i, j)


def test_block_rational_brute_force():
    """Exact rational arithmetic on torch's own decoders of both formats."""
    rs = np.random.RandomState(12)
    M, N, K = 3, 130, 150
    A, B = finite_codes((M, K), rs), finite_codes((N, K), rs)
    sa = rs.randint(120, 135, size=(M, 2)).astype(np.uint8)
    sb = rs.randint(120, 135, size=(2, 2)).astype(np.uint8)
    f8 = lambda c: Fraction(torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn)
                            .to(torch.float64).item())
    e8 = lambda c: Fraction(torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e8m0fnu)
                            .to(torch.float64).item())
    got = oracle.gemm_e4m3_block_ref(A, B, sa, sb)
    for i in range(M):
        for j in (0, 1, 64, 127, 128, 129):
            exact = Fraction(0)
            for k in range(K):
                exact += e8(sa[i, k // 128]) * e8(sb[j // 128, k // 128]) * f8(A[i, k]) * f8(B[j, k])
            assert Fraction(got[i, j]) == exact, (i, j)


def test_block_scale_pairs_with_its_own_block():
    """Raising scale (i, b) by one power of two equals doubling row i's codes
    in k block b (codes with exponent field <= 13 double exactly); raising
    (c, b) of B's scales changes only output columns [128 c, 128 c + 128)."""
    rs = np.random.RandomState(13)
    M, N, K = 5, 260, 330
    A = finite_codes((M, K), rs)
    A[((A >> 3) & 15) > 13] &= 0x87     # exponent field <= 13 everywhere (doubling stays finite)
    B = finite_codes((N, K), rs)
    sa = rs.randint(124, 131, size=(M, 3)).astype(np.uint8)
    sb = rs.randint(124, 131, size=(3, 3)).astype(np.uint8)
    base = oracle.gemm_e4m3_block_ref(A, B, sa, sb)
    for i, b in ((0, 0), (3, 2), (4, 1)):
        s2 = sa.copy()
        s2[i, b] += 1
        A2 = A.copy()
        ks = slice(128 * b, min(128 * b + 128, K))
        nz = (A2[i, ks] & 0x7F) != 0
        seg = A2[i, ks].copy()
        # doubling a code: exponent field + 1 (normal codes); subnormal codes
        # double by doubling their fraction when it stays below 8, else they
        # become the normal code with exponent 1
        out = []
        for c in seg:
            s, e, f = c & 0x80, (c >> 3) & 15, c & 7
            if e > 0:
                out.append(s | ((e + 1) << 3) | f)
            elif f < 4:
                out.append(s | (f * 2))
            else:
                out.append(s | (1 << 3) | ((f * 2 - 8)))
        A2[i, ks] = np.array(out, dtype=np.uint8)
        assert np.array_equal(oracle.decode_e4m3(A2[i, ks])[nz], 2 * oracle.decode_e4m3(seg)[nz])
        assert np.array_equal(oracle.gemm_e4m3_block_ref(A, B, s2, sb), oracle.gemm_e4m3_block_ref(A2, B, sa, sb))
    s3 = sb.copy()
    s3[1, 2] += 2
    moved = oracle.gemm_e4m3_block_ref(A, B, sa, s3)
    cols = np.arange(N)
    inside = (cols >= 128) & (cols < 256)
    assert np.array_equal(moved[:, ~inside], base[:, ~inside])
    assert not np.array_equal(moved[:, inside], base[:, inside])


def test_block_nan_scale():
    rs = np.random.RandomState(14)
    M, N, K = 4, 140, 200
    A, B = finite_codes((M, K), rs), finite_codes((N, K), rs)
    sa, sb = unit_scales(M, N, K)
    sa[2, 1] = 255
    sb[1, 0] = 255
    got = oracle.gemm_e4m3_block_ref(A, B, sa, sb)
    assert np.isnan(got[2]).all()
    assert np.isnan(got[:, 128:]).all()
    assert np.isfinite(np.delete(got, 2, 0)[:, :128]).all()


# --- grouped form with block scales ---

def test_grouped_block_unit_and_uniform_scales_are_the_per_tensor_grouped():
    """Unit block scales give the per-tensor grouped product with scales 1;
    scales uniform per expert (one byte u for all of A's, v_e for all of
    expert e's weight blocks) give it with scale_a = 2^(u-127), scale_b[e] =
    2^(v_e-127).  Empty experts produce nothing; rows past off[G] stay NaN."""
    rs = np.random.RandomState(12)
    counts = [0, 3, 9, 0, 14, 1]
    off = np.concatenate([[0], np.cumsum(counts)])
    rows, G, N, K = int(off[-1]), len(counts), 260, 300
    A = finite_codes((rows + 2, K), rs)
    W = finite_codes((G, N, K), rs)
    kb, nb = -(-K // 128), -(-N // 128)
    sa = np.full((rows + 2, kb + 1), 127, np.uint8)
    sb = np.full((G, nb, kb + 1), 127, np.uint8)
    g = oracle.grouped_e4m3_block_ref(A, W, off, sa, sb)
    assert np.isnan(g[rows:]).all()
    assert np.array_equal(g[:rows], oracle.grouped_e4m3_ref(A, W, off, 1.0, np.ones(G))[:rows])
    v = np.array([127, 125, 130, 127, 126, 129])
    sa[:] = 126
    for e in range(G):
        sb[e] = v[e]
    g = oracle.grouped_e4m3_block_ref(A, W, off, sa, sb)
    assert np.array_equal(g[:rows], oracle.grouped_e4m3_ref(A, W, off, 0.5, 2.0 ** (v - 127.0))[:rows])


def test_grouped_block_scale_moves_only_its_part():
    """Raising routed row r's scale of k block b by one adds exactly that
    row's block-b partial product (the per-tensor product over that k range,
    times the weight block's scale) once more; raising expert e's scale of
    column block c and k block b changes only e's rows in c's columns."""
    rs = np.random.RandomState(13)
    counts = [5, 0, 11, 6]
    off = np.concatenate([[0], np.cumsum(counts)])
    rows, G, N, K = int(off[-1]), len(counts), 200, 384
    A = finite_codes((rows, K), rs)
    W = finite_codes((G, N, K), rs)
    kb, nb = K // 128, -(-N // 128)
    sa = rs.randint(125, 130, size=(rows, kb)).astype(np.uint8)
    sb = rs.randint(125, 130, size=(G, nb, kb)).astype(np.uint8)
    base = oracle.grouped_e4m3_block_ref(A, W, off, sa, sb)
    r, b, e = 7, 1, 2                          # row 7 is expert 2's third row
    sa2 = sa.copy()
    sa2[r, b] += 1
    got = oracle.grouped_e4m3_block_ref(A, W, off, sa2, sb)
    part = oracle.gemm_e4m3_ref(A[r:r + 1, 128 * b:128 * (b + 1)], W[e][:, 128 * b:128 * (b + 1)])[0]
    wscale = np.array([oracle.e8m0(sb[e, j // 128, b]) for j in range(N)])
    assert np.array_equal(got[r], base[r] + part * oracle.e8m0(sa[r, b]) * wscale)
    assert np.array_equal(np.delete(got, r, 0), np.delete(base, r, 0))
    sb2 = sb.copy()
    sb2[3, 1, 2] -= 1
    got = oracle.grouped_e4m3_block_ref(A, W, off, sa, sb2)
    lo, hi = off[3], off[4]
    changed = np.zeros_like(got, dtype=bool)
    changed[lo:hi, 128:] = True
    assert np.array_equal(got[~changed], base[~changed])
    assert not np.array_equal(got[changed], base[changed])


# --- blockwise quantisation to E4M3 with E8M0 scales ---

def test_quantize_codes_are_torchs_conversion_of_the_scaled_block():
    """Each block's codes are torch's float8_e4m3fn conversion (round to
    nearest even) of x / 2^E, and 2^E is the smallest power of two that
    brings the block's largest magnitude to 448 or below: 224 < amax / 2^E
    <= 448.  Ragged last block (cols = 300), magnitudes from 2^-30 to 2^30,
    negative zeros."""
    rs = np.random.RandomState(21)
    rows, cols = 6, 300
    x = rs.standard_normal((rows, cols)) * 2.0 ** rs.randint(-30, 31, size=(rows, 1))
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    x[2, 5] = -0.0
    q, s = oracle.quantize_e4m3_block(x)
    assert s.shape == (rows, 3)
    for r in range(rows):
        for b in range(3):
            v = x[r, 128 * b:min(128 * b + 128, cols)]
            scale = 2.0 ** (int(s[r, b]) - 127)
            amax = np.abs(v).max()
            assert 224.0 < amax / scale <= 448.0, (r, b)
            want = torch.from_numpy(v / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[r, 128 * b:128 * b + v.size], want), (r, b)
    assert q[2, 5] == 0x80


def test_quantize_exact_values_round_trip_and_special_blocks():
    """Values that are E4M3 values times the block's power of two come back
    exactly; an all-zero block takes scale 2^0 and zero codes; a block with
    a NaN or an infinity takes the NaN scale byte and NaN codes; the largest
    magnitude 448 * 2^k maps to code 0x7E with scale 2^k."""
    rs = np.random.RandomState(22)
    codes = rs.randint(0, 127, size=(4, 256)).astype(np.uint8) | (rs.randint(0, 2, size=(4, 256)) << 7).astype(np.uint8)
    codes[:, 0] = 0x7E                                     # 448 in every block
    codes[:, 128] = 0xFE
    k = np.array([-20, 0, 7, 33])
    x = oracle.decode_e4m3(codes) * 2.0 ** k[:, None]
    q, s = oracle.quantize_e4m3_block(x)
    assert np.array_equal(s, np.repeat((k + 127)[:, None], 2, axis=1).astype(np.uint8))
    dec = oracle.decode_e4m3(q) * 2.0 ** (s.astype(np.int64).repeat(128, axis=1) - 127)
    assert np.array_equal(dec, x)
    z = np.zeros((2, 130))
    z[1, 129] = np.nan
    z[1, 3] = np.inf
    q, s = oracle.quantize_e4m3_block(z)
    assert list(s[0]) == [127, 127] and not q[0].any()
    assert list(s[1]) == [255, 255] and (q[1] == 0x7F).all()


def test_quantize_error_within_half_an_e4m3_step():
    """|decode(code) * 2^E - x| is at most half of the E4M3 spacing at x / 2^E
    (2^-10 below 2^-6, 2^(floor(log2|y|) - 4) above), times 2^E."""
    rs = np.random.RandomState(23)
    x = torch.from_numpy(rs.standard_normal((8, 512)) * 3.0).to(torch.bfloat16).to(torch.float64).numpy()
    q, s = oracle.quantize_e4m3_block(x)
    scale = 2.0 ** (s.astype(np.int64).repeat(128, axis=1) - 127)
    y = np.abs(x) / scale
    half = np.where(y < 2.0 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 4))
    assert np.all(np.abs(oracle.decode_e4m3(q) * scale - x) <= half * scale)
