"""Pins for the CPU oracle (no GPU).

The oracle is only trusted after these tests tie it to something other than
itself: exhaustive comparison of its 16-bit decoders with numpy / torch,
round-to-nearest-even checked against the definition with exact rationals,
the GEMM against exact rational arithmetic and against an independent
pure-Python ascending-k double sum on tiny shapes, and closed forms
(identity, all-ones, permutations, integer data).  A plausible slip in the
oracle -- a dropped term, a transposed operand, a wrong index or sign, a
truncating encoder -- fails at least one of them.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle

# ---------------------------------------------------------------- codecs


def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_exhaustive():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _sample_doubles(n, seed):
    rng = np.random.RandomState(seed)
    mags = rng.uniform(-140, 130, size=n)
    x = rng.uniform(1, 2, size=n) * np.exp2(np.floor(mags))
    x *= np.where(rng.rand(n) < 0.5, -1.0, 1.0)
    return x


def test_f16_encode_matches_numpy():
    # numpy rounds float64 -> float16 directly, to nearest even
    xs = _sample_doubles(200000, 3)
    xs = xs[np.abs(xs) < 1e6]
    # add exact ties and subnormal ties: midpoints between neighbouring halves
    h = np.arange(0, 0x7bff, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2.0
    xs = np.concatenate([xs, mids, -mids, [65504.0, 65519.99, 65520.0, 1e9, -1e9, 0.0, -0.0]])
    ours = oracle.encode(xs, "f16")
    ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f32_encode_matches_hardware_cast():
    xs = _sample_doubles(200000, 4)
    xs = np.concatenate([xs, [3.4028235677973366e38, 3.4028236e38, 1e-46, 7e-46, -0.0]])
    ours = oracle.encode(xs, "f32")
    ref = xs.astype(np.float32).view(np.uint32)
    assert np.array_equal(ours, ref)


def _bf16_value(b: int) -> Fraction:
    s = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if e == 0:
        return s * Fraction(f, 2 ** 133)
    return s * Fraction(128 + f) * (Fraction(2) ** (e - 134))


def test_bf16_encode_is_nearest_even_by_definition():
    """For every sample, no other finite bf16 is nearer; ties pick an even
    fraction field.  Exact rationals, so nothing here rounds."""
    xs = list(_sample_doubles(3000, 5)) + [257.0, 259.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8,
                                           1 + 2 ** -8 + 2 ** -30, 2.0 ** -133, 1.5 * 2.0 ** -133,
                                           2.0 ** -134, 0.75 * 2.0 ** -133]
    for x in xs:
        b = int(oracle.encode(np.array([x]), "bf16")[0])
        fx = Fraction(x)
        v = _bf16_value(b)
        d = abs(v - fx)
        for nb in (b - 1, b + 1):
            if nb < 0 or (nb & 0x7F80) == 0x7F80 or (nb ^ b) & 0x8000:
                continue
            dn = abs(_bf16_value(nb) - fx)
            assert d <= dn, (x, hex(b), hex(nb))
            if d == dn:
                assert b % 2 == 0, ("tie must go to even", x, hex(b))


def test_bf16_encode_printed_cases():
    enc = lambda x: int(oracle.encode(np.array([x]), "bf16")[0])
    assert oracle.decode(np.array([enc(257.0)], np.uint16), "bf16")[0] == 256.0
    assert oracle.decode(np.array([enc(259.0)], np.uint16), "bf16")[0] == 260.0
    assert enc(1 + 2 ** -8) == 0x3F80                      # tie -> even (1.0)
    assert enc(1 + 3 * 2 ** -8) == 0x3F82                  # tie -> even (1 + 2^-6)
    assert enc(1 + 2 ** -8 + 2 ** -30) == 0x3F81           # rounded once, from the double
    assert enc(3.4e38) == 0x7F80 and enc(-3.4e38) == 0xFF80  # overflow -> inf
    assert enc(-0.0) == 0x8000


# ---------------------------------------------------------------- GEMM

SIZES = [1, 2, 3, 5, 8, 13, 16, 17]


def _exact(Av, Bv):
    M, K = Av.shape
    N = Bv.shape[1]
    return [[sum((Fraction(Av[i, k]) * Fraction(Bv[k, j]) for k in range(K)), Fraction(0))
             for j in range(N)] for i in range(M)]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")])
def test_gemm_matches_exact_and_sequential_sum(dt, layout):
    rng = random.Random(11)
    al, bl = layout
    for _ in range(6):
        M, N, K = rng.choice(SIZES), rng.choice(SIZES), rng.choice(SIZES)
        rs = np.random.RandomState(rng.randrange(1 << 30))
        a = datagen.matrix((M, K), ("uniform", 1.0), dt, rs)
        b = datagen.matrix((K, N), ("normal", 3.0), dt, rs)
        ref = oracle.gemm_ref(datagen.store(a, al), datagen.store(b, bl), dt, dt, al, bl)
        Av, Bv = oracle.decode(a, dt), oracle.decode(b, dt)
        exact = _exact(Av, Bv)
        for i in range(M):
            for j in range(N):
                # the definition: one double addition per k, ascending
                s = 0.0
                for k in range(K):
                    s += float(Av[i, k]) * float(Bv[k, j])
                assert ref[i, j] == s
                bound = Fraction(K * 2 ** -52) * sum(abs(Fraction(Av[i, k]) * Fraction(Bv[k, j])) for k in range(K))
                assert abs(Fraction(ref[i, j]) - exact[i][j]) <= bound


def test_gemm_integer_exact():
    cfg = datagen.DENSE["gemm512_f16"]
    a, b = datagen.gemm_inputs(cfg, "int", M=33, N=31, K=40)
    ref = oracle.gemm_ref(a, b, "f16", "f16")
    Ai = oracle.decode(a, "f16").astype(np.int64)
    Bi = oracle.decode(b, "f16").astype(np.int64)
    assert np.array_equal(ref, (Ai @ Bi).astype(np.float64))


def _bits(x, dt):
    return datagen._to_bits(np.asarray(x, dtype=np.float32), dt)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_identity_and_all_ones(dt):
    rs = np.random.RandomState(5)
    B = datagen.matrix((24, 19), ("uniform", 1.0), dt, rs)
    I = _bits(np.eye(24), dt)
    ref = oracle.gemm_ref(I, B, dt, dt)
    assert np.array_equal(ref, oracle.decode(B, dt))
    A = datagen.matrix((7, 24), ("normal", 1.0), dt, rs)
    ref = oracle.gemm_ref(A, I, dt, dt)
    assert np.array_equal(ref, oracle.decode(A, dt))
    for K in (512, 2048, 7168):
        ones_a, ones_b = _bits(np.ones((3, K)), dt), _bits(np.ones((K, 5)), dt)
        ref = oracle.gemm_ref(ones_a, ones_b, dt, dt)
        assert np.all(ref == K)
        assert np.all(oracle.to_dtype_value(ref, "bf16") == K)


def test_permutation_columns_exact():
    rs = np.random.RandomState(9)
    A = datagen.matrix((11, 16), ("normal", 1.0), "bf16", rs)
    perm = rs.permutation(16)
    P = np.zeros((16, 16), dtype=np.float32)
    P[perm, np.arange(16)] = 1.0            # column j of A @ P is column perm[j] of A
    ref = oracle.gemm_ref(A, _bits(P, "bf16"), "bf16", "bf16")
    assert np.array_equal(ref, oracle.decode(A, "bf16")[:, perm])


def test_sampled_equals_full():
    rs = np.random.RandomState(3)
    A = datagen.matrix((20, 40), ("uniform", 1.0), "bf16", rs)
    B = datagen.matrix((40, 12), ("uniform", 1.0), "bf16", rs)
    full = oracle.gemm_ref(A, datagen.store(B, "col"), "bf16", "bf16", "row", "col")
    r = rs.randint(0, 20, 30)
    c = rs.randint(0, 12, 30)
    s = oracle.gemm_ref_sampled(A, datagen.store(B, "col"), r, c, "bf16", "bf16", "row", "col")
    assert np.array_equal(s, full[r, c])


def test_empty_k_gives_zero():
    A = np.zeros((4, 0), dtype=np.uint16)
    B = np.zeros((0, 3), dtype=np.uint16)
    assert np.array_equal(oracle.gemm_ref(A, B, "bf16", "bf16"), np.zeros((4, 3)))


# ---------------------------------------------------------------- SiLU gate


def test_silu_special_cases():
    scipy_special = pytest.importorskip("scipy.special")
    assert oracle.silu(0.0) == 0.0
    for x in np.linspace(-30, 30, 241):
        ref = x * scipy_special.expit(x)
        assert abs(oracle.silu(x) - ref) <= 4e-16 * max(1.0, abs(ref))
    assert oracle.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert abs(oracle.silu(-50.0)) < 1e-19


def test_silu_gate_pairs_interleaved_columns():
    """Build gate and up separately, lay them out with the 8-column
    interleave, and check h = SiLU(gate) * up column by column."""
    scipy_special = pytest.importorskip("scipy.special")
    rs = np.random.RandomState(2)
    gate = rs.standard_normal((5, 32))
    up = rs.standard_normal((5, 32))
    G = datagen.interleave_gate_up(gate, up, 8)
    h = oracle.silu_gate(G, 8)
    ref = gate * scipy_special.expit(gate) * up
    assert np.allclose(h, ref, rtol=1e-14, atol=1e-15)
    # zero gate or zero up -> zero output, exactly
    G0 = datagen.interleave_gate_up(np.zeros_like(gate), up, 8)
    assert np.all(oracle.silu_gate(G0) == 0.0)
    G1 = datagen.interleave_gate_up(gate, np.zeros_like(up), 8)
    assert np.all(oracle.silu_gate(G1) == 0.0)


# ---------------------------------------------------------------- grouped


def test_grouped_matches_dense_slices_and_handles_empty():
    cfg = datagen.MOE["moe_small"]
    r, A, W1, W2 = datagen.moe_inputs_host(cfg)
    assert (r.counts == 0).any(), "the small MoE stand-in must contain an empty expert"
    g = oracle.grouped_ref(A, W1, r.offsets)
    for e in range(cfg.num_experts):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            assert np.array_equal(g[lo:hi], oracle.gemm_ref(A[lo:hi], W1[e], "bf16", "bf16"))
    # reversing expert order reverses the output blocks
    order = list(range(cfg.num_experts))[::-1]
    A_rev = np.concatenate([A[r.offsets[e]:r.offsets[e + 1]] for e in order])
    counts_rev = r.counts[order]
    off_rev = np.concatenate([[0], np.cumsum(counts_rev)])
    g_rev = oracle.grouped_ref(A_rev, W1[order], off_rev)
    for i, e in enumerate(order):
        assert np.array_equal(g_rev[off_rev[i]:off_rev[i + 1]], g[r.offsets[e]:r.offsets[e + 1]])


def test_moe_integer_chain_exact():
    """Integer FC1 sums are exact; the chain's h is then the rounded SiLU
    gate of exact values, and FC2 on an integer h is exact again."""
    cfg = datagen.MOE["moe_small"]
    r, A, W1, W2 = datagen.moe_inputs_host(cfg, "int")
    g = oracle.grouped_ref(A, W1, r.offsets)
    Ai = oracle.decode(A, "bf16").astype(np.int64)
    for e in range(cfg.num_experts):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        W = oracle.decode(W1[e], "bf16").astype(np.int64)
        assert np.array_equal(g[lo:hi], (Ai[lo:hi] @ W).astype(np.float64))
    hint = datagen._to_bits(np.random.RandomState(0).randint(-2, 3, (A.shape[0], cfg.inter)).astype(np.float32), "bf16")
    y = oracle.grouped_ref(hint, W2, r.offsets)
    Hi = oracle.decode(hint, "bf16").astype(np.int64)
    for e in range(cfg.num_experts):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        W = oracle.decode(W2[e], "bf16").astype(np.int64)
        assert np.array_equal(y[lo:hi], (Hi[lo:hi] @ W).astype(np.float64))


def test_moe_ref_closed_form_with_saturated_gate():
    """moe_ref (FC1 -> SiLU gate -> bf16 h -> FC2 per expert) against a
    closed form worked out with Python integers.  Every routed row has
    A[r, 0] = 1 and every gate column of W1 is 64 at k = 0 and 0 elsewhere,
    so each gate sum is exactly 64; SiLU(64) = 64 / (1 + e^-64) is 64.0 in
    fp64 (e^-64 is below half an ulp of 1), so h = 64 * up, an integer that
    bf16 holds exactly (|up| <= 64 has at most 7 significant bits), and
    y = h . W2 is exact.  One row's first up sum is forced to 259, so its h
    (64 * 259) needs nine significant bits and bf16 must round it to nearest
    (64 * 260; truncation would give 64 * 258), and FC2 must take the
    rounded value.  Gate and up
    columns follow the interleave of eight columns, gate first.  A swapped
    gate/up order, a wrong expert's weights, an unrounded h fed to FC2, or a
    mis-walked (or empty) expert fails."""
    rs = np.random.RandomState(7)
    K1, I, H = 16, 16, 24          # hidden in, intermediate, hidden out
    offsets = [0, 3, 3, 7]         # three experts, the second empty
    G, rows = len(offsets) - 1, offsets[-1]
    A = rs.randint(-2, 3, (rows, K1))
    A[:, 0] = 1
    W1 = rs.randint(-2, 3, (G, K1, 2 * I))
    W2 = rs.randint(-2, 3, (G, I, H))
    for c in range(I):             # gate column of output c: 16 (c // 8) + c % 8
        jg = 16 * (c // 8) + c % 8
        W1[:, :, jg] = 0
        W1[:, 0, jg] = 64
    # row 0 (expert 0): up sum of output column 0 is 259
    ju0 = 8
    A[0, 1] = 1
    W1[0, :, ju0] = 0
    W1[0, 0, ju0], W1[0, 1, ju0] = 256, 3

    def bf16_int(v):
        """v rounded to 8 significant bits, ties to even (bf16 on integers)."""
        m, sign = abs(v), (-1 if v < 0 else 1)
        sh = max(m.bit_length() - 8, 0)
        q, rem = divmod(m, 1 << sh)
        half = 1 << sh >> 1
        if sh and (rem > half or (rem == half and q & 1)):
            q += 1
        return sign * (q << sh)

    bits = lambda x: (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.all((np.abs(W1) < 256) | (W1 == 256))   # every weight is exact in bf16
    h_ref, h_bits, y_ref = oracle.moe_ref(bits(A), bits(W1), bits(W2), offsets)
    for e in range(G):
        for r in range(offsets[e], offsets[e + 1]):
            up = [sum(int(A[r, k]) * int(W1[e, k, 16 * (c // 8) + c % 8 + 8]) for k in range(K1)) for c in range(I)]
            h = [64 * u for u in up]
            hb = [bf16_int(v) for v in h]
            y = [sum(hb[c] * int(W2[e, c, j]) for c in range(I)) for j in range(H)]
            assert h_ref[r].tolist() == [float(v) for v in h]
            assert oracle.decode(h_bits[r], "bf16").tolist() == [float(v) for v in hb]
            assert y_ref[r].tolist() == [float(v) for v in y]
    assert h_ref.shape == (rows, I) and y_ref.shape == (rows, H)
    assert h_ref[0, 0] == 64 * 259 and oracle.decode(h_bits[0, :1], "bf16")[0] == 64 * 260


def test_routing_pinned_counts():
    """The 64-expert routing reproduces the pinned seed-0 counts."""
    golden = np.loadtxt(datagen_golden("moe64_counts_seed0.txt"), dtype=np.int64)
    r = datagen.moe_route(datagen.MOE["moe64"])
    assert np.array_equal(r.counts, golden)
    assert r.counts.sum() == 4096 * 8 and r.counts.max() <= 4096
    assert int((r.counts == 0).sum()) == 5 and int((r.counts < 64).sum()) == 23
    # every token has top_k distinct experts
    assert all(len(set(row)) == 8 for row in r.top.tolist())


def datagen_golden(name):
    import os
    return os.path.join(os.path.dirname(__file__), "golden", name)
