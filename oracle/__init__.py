"""CPU oracle for the dense and grouped FP16/BF16 GEMM -- TEST INFRASTRUCTURE.

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``bf16_gemm_amd``)
never imports it, and this package never imports the product.

The arithmetic lives in ``oracle.c`` (plain fp64 sums, its own 16-bit
codecs, RNE output rounding); this module only marshals numpy arrays across
ctypes and walks experts in order for the grouped form.  What is computed,
and from which passage of the pages:

* ``gemm_ref`` -- each output element is the exact-product, ascending-k,
  double-precision sum that "B200 的 2CTA 怎样调优" (section 七, the
  accumulate-then-epilogue sketch) describes: accumulate A[i,k]*B[k,j] along
  all of K, then hand the finished sum to the epilogue.
* ``encode`` -- the epilogue's type conversion, read as IEEE
  round-to-nearest-even applied once to the double sum.
* ``silu_gate`` -- up x SiLU(gate) (same page, section 七, "Gate／SwiGLU"),
  with gate/up interleaved in blocks of eight output columns, gate first
  ("MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 10).
* ``decode_e4m3`` / ``gemm_e4m3_ref`` -- the FP8 form with one scale per
  tensor ("MegaMoE", Hopper section 04: per-tensor scales are applied once,
  in the epilogue): scale_a x scale_b x the ascending-k double sum of the
  decoded E4M3 products (E4M3 bits from the OCP 8-bit float layout).
* ``e8m0`` / ``gemm_e4m3_block_ref`` -- the blockwise FP8 form ("MegaMoE",
  Hopper section 04: activation scales per token and per 128-k block,
  weight scales per 128 x 128 block, each K block's partial product scaled
  before it is added): scales are E8M0 bytes (2^(v - 127), 255 NaN), the
  power-of-two scale format the pages name for MXFP8 blocks.
* ``grouped_e4m3_ref`` / ``grouped_e4m3_block_ref`` -- the per-expert FP8
  products (per-tensor scales with one weight scale per expert; block
  scales per routed row and per 128 x 128 block of each expert's weight).
* ``grouped_ref`` / ``moe_ref`` -- the per-expert form: expert e owns rows
  [off[e], off[e+1]) of the routed activations and multiplies them by its
  own weight matrix ("MegaMoE", Recap 1 on the MoE stages: FC1 -> activation
  -> FC2 per expert).  The intermediate h is rounded to bf16 before FC2.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle*.py`` (exhaustive codec checks, exact rational brute
force, closed forms, reductions to other pinned forms); none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

F16, BF16, F32, F64 = 1, 2, 3, 4
ROW, COL = 0, 1
_DT = {"f16": F16, "bf16": BF16, "f32": F32, "f64": F64}
_LAYOUT = {"row": ROW, "col": COL}

#: gate/up interleave granularity (output columns per block), gate first
GATE_UP_INTERLEAVE = 8

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(os.path.join(_HERE, "oracle.c")):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_SO)
    i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.oracle_double_to_f16.argtypes = [ctypes.c_double]
    lib.oracle_double_to_f16.restype = ctypes.c_uint16
    lib.oracle_double_to_f32_bits.argtypes = [ctypes.c_double]
    lib.oracle_double_to_f32_bits.restype = ctypes.c_uint32
    lib.oracle_decode.argtypes = [i32, vp, i64, dp]
    lib.oracle_encode.argtypes = [i32, dp, i64, vp]
    lib.oracle_gemm_ref.argtypes = [i64, i64, i64, i32, i32, vp, i64, i32, i32, vp, i64, dp]
    lib.oracle_gemm_ref.restype = i32
    lib.oracle_gemm_ref_sampled.argtypes = [i64, i32, i32, vp, i64, i32, i32, vp, i64, vp, vp, i64, dp]
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_silu_gate.argtypes = [i64, i64, i64, dp, dp]
    lib.oracle_silu_gate_weighted.argtypes = [i64, i64, i64, dp, dp, dp]
    lib.oracle_num_threads.restype = i32
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_decode_e4m3.argtypes = [vp, i64, dp]
    lib.oracle_gemm_e4m3_ref.argtypes = [i64, i64, i64, vp, i64, vp, i64, ctypes.c_double, ctypes.c_double, dp]
    lib.oracle_gemm_e4m3_ref.restype = i32
    lib.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_to_double.restype = ctypes.c_double
    lib.oracle_gemm_e4m3_block_ref.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, dp]
    lib.oracle_gemm_e4m3_block_ref.restype = i32
    lib.oracle_gemm_e4m3_ref_sampled.argtypes = [i64, vp, i64, vp, i64, ctypes.c_double, ctypes.c_double,
                                                 vp, vp, i64, dp]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact values (float64) of 16-bit ``dtype`` bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode(_DT[dtype], _p(b), b.size, _p(out))
    return out


def encode(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Round doubles to ``dtype`` (RNE).  Returns uint16 bits for f16/bf16,
    uint32 bits for f32."""
    r = np.ascontiguousarray(ref, dtype=np.float64)
    out = np.empty(r.shape, dtype=np.uint32 if dtype == "f32" else np.uint16)
    _load().oracle_encode(_DT[dtype], _p(r), r.size, _p(out))
    return out


def to_dtype_value(ref: np.ndarray, dtype: str) -> np.ndarray:
    """The value (float64) of ``ref`` after RNE rounding to ``dtype``."""
    bits = encode(ref, dtype)
    if dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    return decode(bits, dtype)


def _check2d(x: np.ndarray, name: str):
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 bit array, got {x.dtype} {x.shape}")


def gemm_ref(A: np.ndarray, B: np.ndarray, a_type: str, b_type: str,
             a_layout: str = "row", b_layout: str = "row") -> np.ndarray:
    """Unrounded fp64 product of the logical M x K matrix A and K x N matrix B.

    ``A``/``B`` are uint16 bit arrays in their storage layout: a row-major
    operand is stored [rows][cols], a column-major one [cols][rows].
    Returns an M x N float64 array (ascending-k double sums).
    """
    _check2d(A, "A")
    _check2d(B, "B")
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if a_layout == "row":
        M, K = A.shape
    else:
        K, M = A.shape
    if b_layout == "row":
        K2, N = B.shape
    else:
        N, K2 = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    lda, ldb = A.shape[1], B.shape[1]
    ref = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_ref(M, N, K, _DT[a_type], _LAYOUT[a_layout], _p(A), lda,
                                 _DT[b_type], _LAYOUT[b_layout], _p(B), ldb, _p(ref))
    if rc != 0:
        raise MemoryError("oracle_gemm_ref could not allocate its temporaries")
    return ref


def gemm_ref_sampled(A: np.ndarray, B: np.ndarray, rows, cols, a_type: str, b_type: str,
                     a_layout: str = "row", b_layout: str = "row") -> np.ndarray:
    """The fp64 sums of ``gemm_ref`` at the elements (rows[t], cols[t]) only."""
    _check2d(A, "A")
    _check2d(B, "B")
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    K = A.shape[1] if a_layout == "row" else A.shape[0]
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(r.shape, dtype=np.float64)
    _load().oracle_gemm_ref_sampled(K, _DT[a_type], _LAYOUT[a_layout], _p(A), A.shape[1],
                                    _DT[b_type], _LAYOUT[b_layout], _p(B), B.shape[1],
                                    _p(r), _p(c), r.size, _p(out))
    return out


def silu(x: float) -> float:
    return float(_load().oracle_silu(float(x)))


def silu_gate(G: np.ndarray, interleave: int = GATE_UP_INTERLEAVE, row_weight=None) -> np.ndarray:
    """h = SiLU(gate) * up (fp64, unrounded) from an rows x N fp64 GEMM output
    whose columns interleave gate and up in blocks of ``interleave``.

    ``row_weight``: None, or one weight per row, multiplied into that row's h
    after SwiGLU and before any rounding (the FC1 epilogue's optional routing
    weight, "MegaMoE：Blackwell 与 Hopper 的融合算子解读", Hopper section 09:
    taken into FC2's input, p(hW2) = (ph)W2)."""
    G = np.ascontiguousarray(G, dtype=np.float64)
    rows, N = G.shape
    if N % (2 * interleave):
        raise ValueError("N must be a multiple of twice the interleave")
    h = np.empty((rows, N // 2), dtype=np.float64)
    if row_weight is None:
        _load().oracle_silu_gate(rows, N, interleave, _p(G), _p(h))
    else:
        w = np.ascontiguousarray(row_weight, dtype=np.float64).reshape(-1)
        if w.size != rows:
            raise ValueError("one weight per row")
        _load().oracle_silu_gate_weighted(rows, N, interleave, _p(G), _p(w), _p(h))
    return h


def grouped_ref(A: np.ndarray, W: np.ndarray, offsets, a_type: str = "bf16",
                w_type: str = "bf16", w_layout: str = "row") -> np.ndarray:
    """Per-expert product: rows [off[e], off[e+1]) of A times W[e].

    ``A``: routed rows, [total_rows][K] uint16 (row-major).
    ``W``: [G][K][N] (row layout) or [G][N][K] (col layout) uint16.
    Returns [total_rows][N] float64; rows past off[G] are not produced.
    """
    off = [int(x) for x in offsets]
    G = len(off) - 1
    N = W.shape[2] if w_layout == "row" else W.shape[1]
    out = np.zeros((off[G], N), dtype=np.float64)
    for e in range(G):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            out[lo:hi] = gemm_ref(A[lo:hi], W[e], a_type, w_type, "row", w_layout)
    return out


def moe_ref(A: np.ndarray, W1: np.ndarray, W2: np.ndarray, offsets):
    """FC1 -> SiLU gate -> bf16 h -> FC2 for every expert.

    Returns (h_ref, h_bits, y_ref): the unrounded gated activations, their
    bf16 rounding (the FC2 input), and the unrounded FC2 sums on that input.
    """
    g = grouped_ref(A, W1, offsets)
    h_ref = silu_gate(g)
    h_bits = encode(h_ref, "bf16")
    y_ref = grouped_ref(h_bits, W2, offsets)
    return h_ref, h_bits, y_ref


def moe_combine_ref(Z: np.ndarray, pos, weights, dtype: str = "bf16") -> np.ndarray:
    """Top-k combine of the expert outputs ("MegaMoE：Blackwell 与 Hopper 的融合
    算子解读", Blackwell section 13: the top-k reduce reads every branch of a
    token and adds them into its output; Hopper section 09: the routing
    weight p scales an expert's contribution, p(hW2) = (ph)W2).

    ``Z``: [rows][H] 16-bit bits (expert outputs in expert order); ``pos``:
    [T][top_k] row of Z for each (token, choice); ``weights``: [T][top_k], or
    None for a plain sum (expert outputs that already carry their weights).
    Returns y[t] = sum_k weights[t, k] * Z[pos[t, k]] (fp64, unrounded); a
    position outside [0, rows) adds nothing.
    """
    z = decode(Z, dtype)
    pos = np.asarray(pos)
    w = np.ones(pos.shape, dtype=np.float64) if weights is None else np.asarray(weights, dtype=np.float64)
    y = np.zeros((pos.shape[0], z.shape[1]), dtype=np.float64)
    for k in range(pos.shape[1]):
        p = pos[:, k]
        ok = (p >= 0) & (p < z.shape[0])
        y[ok] += w[ok, k][:, None] * z[p[ok]]
    return y



def _check_u8(x: np.ndarray, name: str):
    if x.dtype != np.uint8 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint8 bit array, got {x.dtype} {x.shape}")


def decode_e4m3(bits: np.ndarray) -> np.ndarray:
    """Exact values (float64) of E4M3 bit patterns (NaN for 0x7F / 0xFF)."""
    b = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode_e4m3(_p(b), b.size, _p(out))
    return out


def gemm_e4m3_ref(A: np.ndarray, B: np.ndarray, scale_a: float = 1.0, scale_b: float = 1.0) -> np.ndarray:
    """Unrounded fp64 scale_a * scale_b * (A x B) of E4M3 operands.

    ``A``: [M][K] uint8 (k contiguous); ``B``: [N][K] uint8, the K x N
    operand stored column-major (k contiguous).  Returns M x N float64.
    """
    _check_u8(A, "A")
    _check_u8(B, "B")
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    (M, K), (N, K2) = A.shape, B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    ref = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_e4m3_ref(M, N, K, _p(A), K, _p(B), K, float(scale_a), float(scale_b), _p(ref))
    if rc != 0:
        raise MemoryError("oracle_gemm_e4m3_ref could not allocate its temporaries")
    return ref


def e8m0(v) -> float:
    """Value of an E8M0 scale byte: 2^(v - 127), NaN for 255."""
    return _load().oracle_e8m0_to_double(int(v))


def gemm_e4m3_block_ref(A: np.ndarray, B: np.ndarray, sa: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """Unrounded fp64 blockwise-scaled product of E4M3 operands ("MegaMoE：
    Blackwell 与 Hopper 的融合算子解读", Hopper section 04, the blockwise path).

    ``A``: [M][K] uint8; ``B``: [N][K] uint8 (the K x N operand, k
    contiguous); ``sa``: [M][ceil(K/128)] E8M0 bytes, one per row and 128-k
    block; ``sb``: [ceil(N/128)][ceil(K/128)] E8M0 bytes, one per 128 output
    columns and 128-k block.  Returns M x N float64:
    sum over blocks b of e8m0(sa[i,b]) e8m0(sb[j//128,b]) sum_{k in b} a b.
    """
    for x, n in ((A, "A"), (B, "B"), (sa, "sa"), (sb, "sb")):
        _check_u8(x, n)
    A, B, sa, sb = (np.ascontiguousarray(x) for x in (A, B, sa, sb))
    (M, K), (N, K2) = A.shape, B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    kb, nb = -(-K // 128), -(-N // 128)
    if sa.shape[0] != M or sa.shape[1] < kb or sb.shape[0] < nb or sb.shape[1] < kb:
        raise ValueError(f"scale shapes {sa.shape}, {sb.shape} do not cover M={M}, N={N}, K={K}")
    ref = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_e4m3_block_ref(M, N, K, _p(A), K, _p(B), K, _p(sa), sa.shape[1], _p(sb),
                                            sb.shape[1], _p(ref))
    if rc != 0:
        raise MemoryError("oracle_gemm_e4m3_block_ref could not allocate its temporaries")
    return ref


def gemm_e4m3_ref_sampled(A: np.ndarray, B: np.ndarray, rows, cols, scale_a: float = 1.0,
                          scale_b: float = 1.0) -> np.ndarray:
    """``gemm_e4m3_ref`` at the elements (rows[t], cols[t]) only."""
    _check_u8(A, "A")
    _check_u8(B, "B")
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(r.shape, dtype=np.float64)
    _load().oracle_gemm_e4m3_ref_sampled(A.shape[1], _p(A), A.shape[1], _p(B), B.shape[1], float(scale_a),
                                         float(scale_b), _p(r), _p(c), r.size, _p(out))
    return out


def grouped_e4m3_block_ref(A: np.ndarray, W: np.ndarray, offsets, sa: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """The per-expert blockwise-scaled E4M3 product ("MegaMoE：Blackwell 与
    Hopper 的融合算子解读", Recap 1: expert e multiplies its rows [off[e],
    off[e+1]) by its own weights; Hopper section 04, the blockwise path:
    activation scales per token and 128-k block, weight scales per 128 x 128
    block of the expert's weight).  ``A``: [rows][K] uint8; ``W``: [G][N][K]
    uint8; ``sa``: [rows][>= ceil(K/128)] E8M0 bytes (routed row r's scales);
    ``sb``: [G][ceil(N/128)][>= ceil(K/128)] E8M0 bytes.  Returns [rows][N]
    float64; rows past off[G] stay NaN (not produced)."""
    off = np.asarray(offsets, dtype=np.int64)
    G, N, K = W.shape
    if sb.ndim != 3 or sb.shape[0] != G:
        raise ValueError(f"sb must be [G][ceil(N/128)][kb], got {sb.shape}")
    out = np.full((A.shape[0], N), np.nan)
    for e in range(G):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            out[lo:hi] = gemm_e4m3_block_ref(np.ascontiguousarray(A[lo:hi]), np.ascontiguousarray(W[e]),
                                             np.ascontiguousarray(sa[lo:hi]), np.ascontiguousarray(sb[e]))
    return out


def grouped_e4m3_ref(A: np.ndarray, W: np.ndarray, offsets, scale_a: float, scale_b) -> np.ndarray:
    """The per-expert E4M3 product ("MegaMoE", Recap 1: expert e multiplies its
    rows [off[e], off[e+1]) by its own weights; Hopper section 04: one scale
    for the activations, one per expert for the weights).  ``A``: [rows][K]
    uint8; ``W``: [G][N][K] uint8 (each expert's K x N weight column-major);
    ``scale_b``: G floats.  Returns [rows][N] float64; rows past off[G] stay
    NaN (not produced)."""
    off = np.asarray(offsets, dtype=np.int64)
    G, N, K = W.shape
    out = np.full((A.shape[0], N), np.nan)
    for e in range(G):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            out[lo:hi] = gemm_e4m3_ref(np.ascontiguousarray(A[lo:hi]), np.ascontiguousarray(W[e]),
                                       scale_a, float(scale_b[e]))
    return out


def quantize_e4m3_block(x: np.ndarray, block: int = 128):
    """Blockwise FP8 quantisation of a [rows][cols] matrix ("MegaMoE：Blackwell
    与 Hopper 的融合算子解读", Hopper sections 04 and 09: after SwiGLU each
    block's absolute maximum gives a power-of-two (MXFP8, E8M0) scale, and
    the block is multiplied by the scale's reciprocal and converted to FP8).

    Blocks are ``block`` consecutive columns of one row (the last one may be
    shorter).  Scale of a block: the smallest power of two 2^E with
    amax <= 448 * 2^E (448: the largest finite E4M3 value), E clamped to the
    E8M0 range [-127, 127]; an all-zero block takes E = 0; a block holding a
    NaN or an infinity takes the NaN scale byte 255 and NaN codes.  Codes:
    x / 2^E rounded to the nearest E4M3 value, ties to the even code.
    Returns (codes uint8 [rows][cols], scale bytes uint8 [rows][ceil(cols /
    block)]), scale byte = E + 127."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    nblk = -(-cols // block)
    # every non-negative finite E4M3 value, in code order (codes 0 .. 126)
    grid = decode_e4m3(np.arange(127, dtype=np.uint8))
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, nblk), dtype=np.uint8)
    for r in range(rows):
        for b in range(nblk):
            v = x[r, block * b:min(block * b + block, cols)]
            if not np.all(np.isfinite(v)):
                scales[r, b] = 255
                codes[r, block * b:block * b + v.size] = 0x7F
                continue
            amax = float(np.max(np.abs(v))) if v.size else 0.0
            if amax == 0.0:
                E = 0
            else:
                E = math.frexp(amax)[1] - 1 - 8          # floor(log2 amax) - 8
                if amax > 448.0 * 2.0 ** E:
                    E += 1
                E = min(max(E, -127), 127)
            scales[r, b] = E + 127
            y = np.abs(v) * 2.0 ** -E                      # exact: a power-of-two scaling
            hi = np.searchsorted(grid, y, side="left")     # first grid value >= y
            hi = np.minimum(hi, 126)
            lo = np.maximum(hi - 1, 0)
            dlo, dhi = y - grid[lo], grid[hi] - y
            pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
            pick = np.where(grid[hi] == y, hi, pick)
            codes[r, block * b:block * b + v.size] = pick.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0)
    return codes, scales
