"""Seeded synthetic inputs for the dense and grouped GEMM workloads.

This module only draws random numbers and lays them out; it holds none of the
GEMM's arithmetic.  Both the CPU oracle and the HIP library receive exactly
the buffers produced here, as 16-bit bit patterns (numpy ``uint16``), so the
two sides never disagree about their inputs.

Workloads (shapes, dtypes, layouts and value distributions as the workload
list of this library states them; the pages themselves measure square
synthetic GEMMs only -- "使用 Warp Specialization 和 Cluster 扩展 GEMM",
完整优化结果 table at 4096^3, and "GEMM优化（三）", sections 3.1-3.5 at 4096^2
and 8192^2 -- so seeded synthetic matrices stand in for any real data):

=====================  ===============================================  =========================
name                   shape / dtypes / layout                          values
=====================  ===============================================  =========================
gemm512_f16            512^3, f16 in, f32 out, A and B row-major        uniform[-1,1]
gemm4096_bf16          4096^3, bf16 in, bf16 out, row-major             normal(0,1)
gemm8192_bf16_bcol     8192^3, bf16 in, f32 out, B column-major         uniform[-1,1]
ts16384x2048x7168      bf16 in/out, row-major                           A normal(0,1), B normal(0,.02)
decode128x7168x2048    bf16 in/out, row-major (small-M decode shape)     A normal(0,1), B normal(0,.02)
moe64                  64 experts, hidden 7168, inter 2048, 4096 tok    X normal(0,1), W normal(0,.02)
=====================  ===============================================  =========================

Every dense workload also has an integer-valued variant with entries drawn
uniformly from {-2,...,2}; its sums are exact in fp32 in any order.

Value draws: ``numpy.random.RandomState(seed)``; A is drawn first, then B,
each as its logical matrix (A: M x K, B: K x N).  A column-major B is then
stored transposed ([N][K], K contiguous).  Values are drawn in float32 and
rounded to the input type by numpy (f16) or torch (bf16), both RNE.

MoE routing: ``p ~ Dirichlet(0.3 * 1_E)`` and every token picks top_k
distinct experts by Gumbel-top-k on log p (sequential sampling without
replacement, proportional to p), from ``RandomState(routing_seed)``.  Rows are
grouped by expert, and by token id within an expert.  With the 64-expert
workload and seed 0 this gives ragged counts with many experts under 64 rows
and five empty experts.  The large MoE weights can be drawn on a torch device
(Philox) with a per-expert seed so that the full 5.6 GB set never has to be
made on the host; small variants use the host generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class GemmConfig:
    name: str
    M: int
    N: int
    K: int
    in_dtype: str          # "f16" | "bf16"
    out_dtype: str         # "f32" | "bf16" | "f16"
    a_layout: str = "row"
    b_layout: str = "row"
    a_dist: tuple = ("uniform", 1.0)   # ("uniform", half-width) | ("normal", std)
    b_dist: tuple = ("uniform", 1.0)
    seed: int = 0
    int_seed: int = 100

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


@dataclass(frozen=True)
class MoeConfig:
    name: str
    num_experts: int
    hidden: int            # FC1 K and FC2 N
    inter: int             # h width; FC1 N = 2 * inter (gate + up)
    num_tokens: int
    top_k: int
    dirichlet_alpha: float = 0.3
    routing_seed: int = 0
    x_seed: int = 51
    w1_seed: int = 52
    w2_seed: int = 53
    int_seeds: tuple = (151, 152, 153)
    x_std: float = 1.0
    w_std: float = 0.02


DENSE = {
    c.name: c for c in [
        GemmConfig("gemm512_f16", 512, 512, 512, "f16", "f32",
                   a_dist=("uniform", 1.0), b_dist=("uniform", 1.0), seed=1, int_seed=101),
        GemmConfig("gemm4096_bf16", 4096, 4096, 4096, "bf16", "bf16",
                   a_dist=("normal", 1.0), b_dist=("normal", 1.0), seed=2, int_seed=102),
        GemmConfig("gemm8192_bf16_bcol", 8192, 8192, 8192, "bf16", "f32", b_layout="col",
                   a_dist=("uniform", 1.0), b_dist=("uniform", 1.0), seed=3, int_seed=103),
        GemmConfig("ts16384x2048x7168", 16384, 2048, 7168, "bf16", "bf16",
                   a_dist=("normal", 1.0), b_dist=("normal", 0.02), seed=41, int_seed=141),
        GemmConfig("decode128x7168x2048", 128, 7168, 2048, "bf16", "bf16",
                   a_dist=("normal", 1.0), b_dist=("normal", 0.02), seed=42, int_seed=142),
    ]
}

MOE = {
    "moe64": MoeConfig("moe64", num_experts=64, hidden=7168, inter=2048, num_tokens=4096, top_k=8),
    # a CPU-sized stand-in with the same structure (ragged, empty and tiny experts)
    "moe_small": MoeConfig("moe_small", num_experts=8, hidden=256, inter=128, num_tokens=192, top_k=2,
                           routing_seed=7, x_seed=61, w1_seed=62, w2_seed=63, int_seeds=(161, 162, 163)),
}


def _to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> 16-bit patterns of ``dtype`` (RNE, by numpy / torch)."""
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def draw(rs: np.random.RandomState, shape, dist) -> np.ndarray:
    """float32 draws of a distribution ("uniform", w) on [-w, w] or ("normal", s)."""
    kind, p = dist
    if kind == "uniform":
        return rs.uniform(-p, p, size=shape).astype(np.float32)
    if kind == "normal":
        return (rs.standard_normal(size=shape) * p).astype(np.float32)
    if kind == "int":
        return rs.randint(-p, p + 1, size=shape).astype(np.float32)
    raise ValueError(kind)


def matrix(shape, dist, dtype: str, rs: np.random.RandomState) -> np.ndarray:
    return _to_bits(draw(rs, shape, dist), dtype)


def matrix_e4m3(shape, dist, rs: np.random.RandomState) -> np.ndarray:
    """uint8 E4M3 codes of float32 draws (RNE and saturation by torch's
    float8_e4m3fn cast; draws beyond +-448 are clipped first)."""
    import torch
    x = np.clip(draw(rs, shape, dist), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def gemm_inputs(cfg: GemmConfig, variant: str = "random", M: Optional[int] = None,
                N: Optional[int] = None, K: Optional[int] = None):
    """(A_storage, B_storage) uint16 bit arrays for a dense workload.

    ``variant``: "random" (the workload's distributions, ``cfg.seed``) or
    "int" (entries in {-2..2}, ``cfg.int_seed``).  M/N/K override the
    workload's sizes (same distributions and seeds) for scaled-down cases.
    A is stored [M][K] (row) or [K][M] (col); B is stored [K][N] (row) or
    [N][K] (col).
    """
    M = cfg.M if M is None else M
    N = cfg.N if N is None else N
    K = cfg.K if K is None else K
    if variant == "random":
        rs = np.random.RandomState(cfg.seed)
        da, db = cfg.a_dist, cfg.b_dist
    elif variant == "int":
        rs = np.random.RandomState(cfg.int_seed)
        da = db = ("int", 2)
    else:
        raise ValueError(variant)
    a = draw(rs, (M, K), da)
    b = draw(rs, (K, N), db)
    if cfg.a_layout == "col":
        a = np.ascontiguousarray(a.T)
    if cfg.b_layout == "col":
        b = np.ascontiguousarray(b.T)
    return _to_bits(a, cfg.in_dtype), _to_bits(b, cfg.in_dtype)


def store(x_logical_bits: np.ndarray, layout: str) -> np.ndarray:
    """Storage of a logical matrix in ``layout`` (col-major = transposed copy)."""
    return np.ascontiguousarray(x_logical_bits if layout == "row" else x_logical_bits.T)


# ---------------------------------------------------------------------------
# MoE routing and inputs
# ---------------------------------------------------------------------------

@dataclass
class Routing:
    top: np.ndarray              # [num_tokens, top_k] expert ids
    counts: np.ndarray           # [E] rows per expert
    offsets: np.ndarray          # [E + 1] prefix sums (int32)
    token_of_row: np.ndarray     # [total_rows] source token of each routed row
    expert_of_row: np.ndarray = field(default=None)
    pos: np.ndarray = field(default=None)     # [num_tokens, top_k] routed row of (token, choice)
    weight: np.ndarray = field(default=None)  # [num_tokens, top_k] fp32 routing weight (softmax of the scores)


def moe_routing(num_tokens: int, num_experts: int, top_k: int, alpha: float, seed: int) -> Routing:
    rs = np.random.RandomState(seed)
    p = rs.dirichlet([alpha] * num_experts)
    g = rs.gumbel(size=(num_tokens, num_experts))
    with np.errstate(divide="ignore"):
        score = np.log(p)[None, :] + g
    top = np.argsort(-score, axis=1, kind="stable")[:, :top_k]
    counts = np.bincount(top.ravel(), minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    rows = []
    experts = []
    for e in range(num_experts):
        toks = np.nonzero((top == e).any(axis=1))[0]   # ascending token id
        rows.append(toks)
        experts.append(np.full(toks.size, e, dtype=np.int32))
    token_of_row = np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)
    # the row each (token, choice) was routed to: expert e's rows hold its
    # tokens in ascending order
    pos = np.empty(top.shape, dtype=np.int32)
    for k in range(top_k):
        e = top[:, k]
        for ex in np.unique(e):
            sel = np.nonzero(e == ex)[0]
            pos[sel, k] = offsets[ex] + np.searchsorted(rows[ex], sel)
    s = np.take_along_axis(score, top, axis=1)
    s = np.exp(s - s.max(axis=1, keepdims=True))
    weight = (s / s.sum(axis=1, keepdims=True)).astype(np.float32)
    return Routing(top=top, counts=counts, offsets=offsets, token_of_row=token_of_row,
                   expert_of_row=np.concatenate(experts), pos=pos, weight=weight)


def moe_route(cfg: MoeConfig) -> Routing:
    return moe_routing(cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.dirichlet_alpha, cfg.routing_seed)


def interleave_gate_up(gate: np.ndarray, up: np.ndarray, il: int = 8) -> np.ndarray:
    """Lay out separate gate and up weight columns ([K][I] each) as one
    [K][2I] matrix whose columns alternate blocks of ``il``: gate[0:il],
    up[0:il], gate[il:2il], up[il:2il], ...  (pure data layout)."""
    K, I = gate.shape
    if I % il:
        raise ValueError("inter width must be a multiple of the interleave")
    g = gate.reshape(K, I // il, 1, il)
    u = up.reshape(K, I // il, 1, il)
    return np.concatenate([g, u], axis=2).reshape(K, 2 * I)


def moe_inputs_host(cfg: MoeConfig, variant: str = "random"):
    """Host-made MoE inputs: (routing, A_rows, W1, W2) as uint16 bit arrays.

    A_rows: [total_rows][hidden] -- X's rows gathered by expert.
    W1: [E][hidden][2*inter] with gate/up interleaved by 8; W2: [E][inter][hidden].
    Intended for CPU-sized configs; the 64-expert workload is ~5.6 GB.
    """
    r = moe_route(cfg)
    E, H, I = cfg.num_experts, cfg.hidden, cfg.inter
    if variant == "random":
        sx, s1, s2 = cfg.x_seed, cfg.w1_seed, cfg.w2_seed
        dx, dw = ("normal", cfg.x_std), ("normal", cfg.w_std)
    else:
        sx, s1, s2 = cfg.int_seeds
        dx = dw = ("int", 2)
    X = draw(np.random.RandomState(sx), (cfg.num_tokens, H), dx)
    rs1 = np.random.RandomState(s1)
    W1 = np.empty((E, H, 2 * I), dtype=np.float32)
    for e in range(E):
        gate = draw(rs1, (H, I), dw)
        up = draw(rs1, (H, I), dw)
        W1[e] = interleave_gate_up(gate, up)
    rs2 = np.random.RandomState(s2)
    W2 = draw(rs2, (E, I, H), dw)
    A = X[r.token_of_row]
    return r, _to_bits(A, "bf16"), _to_bits(W1, "bf16"), _to_bits(W2, "bf16")


def moe_inputs_device(cfg: MoeConfig, device, variant: str = "random"):
    """Device-made MoE inputs as torch bf16 tensors (A_rows, W1, W2) plus the
    routing.  Each expert's weights come from torch's generator on ``device``
    seeded with (w_seed * 1000 + e), so any one expert can be regenerated
    alone.  X is drawn on the host (RandomState) and gathered there."""
    import torch
    r = moe_route(cfg)
    E, H, I = cfg.num_experts, cfg.hidden, cfg.inter
    if variant == "random":
        sx, s1, s2 = cfg.x_seed, cfg.w1_seed, cfg.w2_seed
    else:
        sx, s1, s2 = cfg.int_seeds
    dx = ("normal", cfg.x_std) if variant == "random" else ("int", 2)
    X = draw(np.random.RandomState(sx), (cfg.num_tokens, H), dx)
    A = torch.from_numpy(_to_bits(X[r.token_of_row], "bf16").view(np.int16)).to(device).view(torch.bfloat16)
    W1 = torch.empty((E, H, 2 * I), dtype=torch.bfloat16, device=device)
    W2 = torch.empty((E, I, H), dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    for e in range(E):
        gen.manual_seed(s1 * 1000 + e)
        W1[e] = _device_draw(torch, (H, 2 * I), variant, cfg.w_std, gen, device)
        gen.manual_seed(s2 * 1000 + e)
        W2[e] = _device_draw(torch, (I, H), variant, cfg.w_std, gen, device)
    return r, A, W1, W2


def _device_draw(torch, shape, variant, std, gen, device):
    if variant == "random":
        return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
    return torch.randint(-2, 3, shape, generator=gen, device=device).to(torch.bfloat16)
