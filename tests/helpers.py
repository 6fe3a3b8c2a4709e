"""Shared helpers of the GPU parity tests: moving bit arrays to and from the
device, the acceptance rule, and sample selection for full-size cases.

Acceptance (floating point), with ref the unrounded fp64 oracle sum over K
terms:
  * fp32 output:  |D - ref| <= 1e-4 * sqrt(K)
  * bf16 output:  |D - ref| <= 2^-7 * |ref| + 1e-4 * sqrt(K)
  * fp16 output:  |D - ref| <= 2^-10 * |ref| + 1e-4 * sqrt(K)
The bf16 relative term is twice bf16's half-ulp (2^-8), the fp16 one twice
fp16's (2^-11); the absolute term covers fp32 accumulation in any order.
Integer-valued inputs must match the oracle's rounding bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}
TORCH_OUT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def to_dev(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """uint16 bit array -> device tensor of that 16-bit type (same shape)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(TORCH16[dtype])


def from_dev_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy bit array (uint16 for 16-bit, uint32 for fp32)."""
    c = t.detach().contiguous().cpu()
    if c.dtype == torch.float32:
        return c.numpy().view(np.uint32)
    return c.view(torch.int16).numpy().view(np.uint16)


def values(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    return oracle.decode(bits, dtype)


def tolerance(ref: np.ndarray, K: int, out: str) -> np.ndarray:
    absn = 1e-4 * math.sqrt(max(K, 1))
    rel = {"f32": 0.0, "bf16": 2.0 ** -7, "f16": 2.0 ** -10}[out]
    return rel * np.abs(ref) + absn


def assert_close(got_bits: np.ndarray, ref: np.ndarray, K: int, out: str, what: str = ""):
    got = values(got_bits, out)
    tol = tolerance(ref, K, out)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; max err {float(np.nanmax(err)):.3e}; "
            f"first {idx.tolist()}: got {got[tuple(idx[0])]!r} ref {ref[tuple(idx[0])]!r} tol {tol[tuple(idx[0])]!r}")
    return float(err.max()) if err.size else 0.0


# Chains of products (FC1 -> h -> FC2 -> combine).  The oracle runs its own
# chain on the inputs alone: its next stage takes its own rounding of the
# previous stage's exact result.  The GPU's next stage took the GPU's
# rounding, which may differ from the oracle's by the stage's acceptance
# rule plus the oracle's own rounding (at most half an ulp: 2^-8 relative in
# bf16, 2^-11 in fp16).  That difference is carried through the next
# product: |sum_k (x_gpu_k - x_oracle_k) w_kj| <= sum_k bound_k |w_kj|.
HALF_ULP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
RULE_REL = {"f32": 0.0, "bf16": 2.0 ** -7, "f16": 2.0 ** -10}


def stage_gap(x_ref: np.ndarray, K: int, dtype: str) -> np.ndarray:
    """Largest |GPU rounding - oracle rounding| of a stage output whose exact
    value is x_ref (a sum over K terms)."""
    return (RULE_REL[dtype] + HALF_ULP[dtype]) * np.abs(x_ref) + 1e-4 * math.sqrt(max(K, 1))


def assert_close_carried(got_bits: np.ndarray, ref: np.ndarray, K: int, out: str, carry: np.ndarray,
                         what: str = ""):
    """The acceptance rule for a stage fed the previous stage's GPU output,
    widened by the carried difference ``carry`` (same shape as ref)."""
    got = values(got_bits, out)
    tol = tolerance(ref, K, out) + carry
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the carried tolerance; first at "
                             f"{list(i)}: got {got[i]!r} ref {ref[i]!r} tol {tol[i]!r}")


def assert_bits_equal(got_bits: np.ndarray, ref: np.ndarray, out: str, what: str = ""):
    want = oracle.encode(ref, out)
    if not np.array_equal(got_bits, want):
        d = np.argwhere(got_bits != want)
        i = tuple(d[0])
        raise AssertionError(f"{what}: {len(d)} elements differ from the oracle; first at {list(i)}: "
                             f"got {values(got_bits, out)[i]!r} want {values(want, out)[i]!r}")


def sample_positions(M: int, N: int, n_random: int, tiles=(256, 256), seed: int = 0):
    """Rows/cols to check at full size: random ones plus tile edges and the
    matrix borders."""
    rs = np.random.RandomState(seed)
    r = list(rs.randint(0, M, n_random))
    c = list(rs.randint(0, N, n_random))
    edges_r = sorted({0, M - 1} | {min(M - 1, x) for t in range(tiles[0], M, tiles[0]) for x in (t - 1, t)})
    edges_c = sorted({0, N - 1} | {min(N - 1, x) for t in range(tiles[1], N, tiles[1]) for x in (t - 1, t)})
    for i in range(min(len(edges_r), 64)):
        r.append(edges_r[i])
        c.append(edges_c[rs.randint(len(edges_c))])
    for j in range(min(len(edges_c), 64)):
        r.append(edges_r[rs.randint(len(edges_r))])
        c.append(edges_c[j])
    return np.array(r, dtype=np.int64), np.array(c, dtype=np.int64)
