"""Python binding of the MI355X GEMM library (include/mgemm.h).

Argument marshalling only: every computation runs in the HIP kernels of
``libmgemm.so``.  torch supplies device memory and streams.  torch is
imported before the library is loaded so that both share torch's HIP
runtime.  If the library has not been built this module raises on import
-- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded first: one HIP runtime per process)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmgemm.so")

F16, BF16, F32 = 1, 2, 3
ROW_MAJOR, COL_MAJOR = 0, 1
EPI_NONE, EPI_SILU_GATE_I8 = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_NO_MEMORY, ERR_HIP = range(6)

PLAN_FORCE_TILE_256x256 = 0x1
PLAN_FORCE_TILE_128x128 = 0x2
PLAN_FORCE_TILE_32x256 = 0x4
PLAN_FORCE_TILE_64x256 = 0x8
PLAN_FORCE_TILE_256x256_DTL = 0x10
PLAN_FORCE_TILE_NARROW = 0x20
PLAN_FORCE_TILE_NARROW64 = 0x40
PLAN_FORCE_TILE_NARROW32 = 0x80
PLAN_NO_XCD_REMAP = 0x100


def PLAN_SPLIT_K(n: int) -> int:
    """Plan flag fixing the number of K ranges per output tile (1 = no split)."""
    return (int(n) & 0xFF) << 16

E4M3 = 4
DTYPE = {"f16": F16, "bf16": BF16, "f32": F32, "e4m3": E4M3}
TORCH_DTYPE = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
LAYOUT = {"row": ROW_MAJOR, "col": COL_MAJOR}


class Desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a_type", ctypes.c_int), ("b_type", ctypes.c_int), ("d_type", ctypes.c_int),
                ("a_layout", ctypes.c_int), ("b_layout", ctypes.c_int),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldd", ctypes.c_int64)]


class GroupedDesc(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("max_total_rows", ctypes.c_int64),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a_type", ctypes.c_int), ("b_type", ctypes.c_int), ("d_type", ctypes.c_int),
                ("b_layout", ctypes.c_int),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("stride_b", ctypes.c_int64),
                ("ldd", ctypes.c_int64), ("epilogue", ctypes.c_int)]


class MoeDesc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("max_total_rows", ctypes.c_int64),
                ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64), ("dtype", ctypes.c_int),
                ("lda", ctypes.c_int64), ("ldw1", ctypes.c_int64), ("stride_w1", ctypes.c_int64),
                ("ldw2", ctypes.c_int64), ("stride_w2", ctypes.c_int64),
                ("ldh", ctypes.c_int64), ("ldy", ctypes.c_int64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("waves_m", ctypes.c_int32), ("waves_n", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64),
                ("tiles", ctypes.c_int64), ("k_steps", ctypes.c_int64), ("coverage", ctypes.c_double),
                ("grid", ctypes.c_int32), ("group_m", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("splits", ctypes.c_int32)]


class Budget(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_int64), ("coverage", ctypes.c_double),
                ("lds_bytes", ctypes.c_int64), ("k_steps", ctypes.c_int64)]


#: every symbol include/mgemm.h declares
EXPORTS = ["gemm_plan", "grouped_gemm_plan", "gemm_plan_workspace_size", "gemm_run", "gemm_run_scaled",
           "grouped_gemm_run", "grouped_gemm_run_scaled",
           "gemm_plan_describe", "gemm_plan_info", "gemm_plan_destroy", "gemm_status_string",
           "gemm_last_error_message", "mgemm_tile_budget", "mgemm_group_working_set", "mgemm_round_tokens",
           "mgemm_version", "mgemm_moe_combine", "grouped_gemm_run_gather", "gemm_run_noalloc",
           "moe_fused_plan", "moe_fused_run", "gemm_run_blockscaled", "grouped_gemm_run_weighted",
           "moe_fused_run_weighted", "grouped_gemm_run_blockscaled", "mgemm_quantize_e4m3_block"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python bf16_gemm_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, u32, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int
    lib.gemm_plan.argtypes = [ctypes.POINTER(Desc), u32, ctypes.POINTER(vp)]
    lib.gemm_plan.restype = st
    lib.grouped_gemm_plan.argtypes = [ctypes.POINTER(GroupedDesc), u32, ctypes.POINTER(vp)]
    lib.grouped_gemm_plan.restype = st
    lib.gemm_plan_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.gemm_plan_workspace_size.restype = st
    lib.gemm_run.argtypes = [vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gemm_run.restype = st
    lib.gemm_run_noalloc.argtypes = [vp, vp, vp, vp, vp]
    lib.gemm_run_noalloc.restype = st
    lib.gemm_run_scaled.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gemm_run_scaled.restype = st
    lib.grouped_gemm_run_scaled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.grouped_gemm_run_scaled.restype = st
    lib.grouped_gemm_run.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.grouped_gemm_run.restype = st
    lib.gemm_plan_describe.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t]
    lib.gemm_plan_describe.restype = st
    lib.gemm_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.gemm_plan_info.restype = st
    lib.gemm_plan_destroy.argtypes = [vp]
    lib.gemm_plan_destroy.restype = None
    lib.gemm_status_string.argtypes = [st]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_last_error_message.argtypes = []
    lib.gemm_last_error_message.restype = ctypes.c_char_p
    lib.mgemm_tile_budget.argtypes = [i64, i64, i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(Budget)]
    lib.mgemm_tile_budget.restype = st
    lib.mgemm_group_working_set.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            i64, ctypes.c_int32]
    lib.mgemm_group_working_set.restype = i64
    lib.mgemm_round_tokens.argtypes = [i64, ctypes.c_int32]
    lib.mgemm_round_tokens.restype = i64
    lib.mgemm_version.restype = ctypes.c_char_p
    lib.grouped_gemm_run_gather.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.grouped_gemm_run_gather.restype = st
    lib.grouped_gemm_run_weighted.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.grouped_gemm_run_weighted.restype = st
    lib.gemm_run_blockscaled.argtypes = [vp, vp, vp, vp, vp, i64, vp, i64, vp, ctypes.c_size_t, vp]
    lib.grouped_gemm_run_blockscaled.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, i64, i64, vp, ctypes.c_size_t, vp]
    lib.grouped_gemm_run_blockscaled.restype = st
    lib.gemm_run_blockscaled.restype = st
    lib.moe_fused_plan.argtypes = [ctypes.POINTER(MoeDesc), u32, ctypes.POINTER(vp)]
    lib.moe_fused_plan.restype = st
    lib.moe_fused_run.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_fused_run.restype = st
    lib.moe_fused_run_weighted.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_fused_run_weighted.restype = st
    lib.mgemm_moe_combine.argtypes = [vp, i64, i64, vp, vp, vp, i64, i64, ctypes.c_int32, i64, ctypes.c_int, vp]
    lib.mgemm_moe_combine.restype = st
    lib.mgemm_quantize_e4m3_block.argtypes = [vp, i64, i64, i64, ctypes.c_int, vp, i64, vp, i64, vp]
    lib.mgemm_quantize_e4m3_block.restype = st
    return lib


lib = _load()


class MgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.gemm_last_error_message().decode(errors="replace")
        super().__init__(f"{where}: {lib.gemm_status_string(status).decode()}: {msg}")


def _check(status: int, where: str):
    if status != OK:
        raise MgemmError(status, where)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """An immutable plan (owns the C handle)."""

    def __init__(self, handle: int, desc):
        self.handle = handle
        self.desc = desc

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and lib is not None:
            lib.gemm_plan_destroy(h)

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(512)
        _check(lib.gemm_plan_describe(self.handle, buf, 512), "gemm_plan_describe")
        return buf.value.decode()

    def info(self) -> PlanInfo:
        inf = PlanInfo()
        _check(lib.gemm_plan_info(self.handle, ctypes.byref(inf)), "gemm_plan_info")
        return inf

    def workspace_size(self) -> int:
        n = ctypes.c_size_t(0)
        _check(lib.gemm_plan_workspace_size(self.handle, ctypes.byref(n)), "gemm_plan_workspace_size")
        return n.value


def gemm_plan(M, N, K, a_type="bf16", b_type=None, d_type="f32", a_layout="row", b_layout="row",
              lda=None, ldb=None, ldd=None, flags: int = 0) -> Plan:
    """Plan D[M,N] = A[M,K] x B[K,N].  Types "f16"/"bf16"/"f32", layouts
    "row"/"col"; leading dimensions default to the packed ones."""
    b_type = b_type or a_type
    d = Desc(M, N, K, DTYPE[a_type], DTYPE[b_type], DTYPE[d_type], LAYOUT[a_layout], LAYOUT[b_layout],
             lda if lda is not None else (K if a_layout == "row" else M),
             ldb if ldb is not None else (N if b_layout == "row" else K),
             ldd if ldd is not None else N)
    h = ctypes.c_void_p()
    _check(lib.gemm_plan(ctypes.byref(d), flags, ctypes.byref(h)), "gemm_plan")
    return Plan(h.value, d)


def grouped_gemm_plan(num_groups, max_total_rows, N, K, a_type="bf16", b_type=None, d_type="bf16",
                      b_layout="row", lda=None, ldb=None, stride_b=None, ldd=None,
                      epilogue: int = EPI_NONE, flags: int = 0) -> Plan:
    b_type = b_type or a_type
    ldb_v = ldb if ldb is not None else (N if b_layout == "row" else K)
    d = GroupedDesc(num_groups, max_total_rows, N, K, DTYPE[a_type], DTYPE[b_type], DTYPE[d_type],
                    LAYOUT[b_layout], lda if lda is not None else K, ldb_v,
                    stride_b if stride_b is not None else K * N,
                    ldd if ldd is not None else (N // 2 if epilogue == EPI_SILU_GATE_I8 else N), epilogue)
    h = ctypes.c_void_p()
    _check(lib.grouped_gemm_plan(ctypes.byref(d), flags, ctypes.byref(h)), "grouped_gemm_plan")
    return Plan(h.value, d)


def workspace_for(plan: Plan, device="cuda"):
    """A device buffer of the plan's workspace size (None if it needs none)."""
    n = plan.workspace_size()
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _nbytes(x, given: int) -> int:
    if given or x is None or isinstance(x, int):
        return given
    return x.numel() * x.element_size()


def gemm_run(plan: Plan, A, B, D, workspace=None, workspace_bytes: int = 0, stream=None):
    """Enqueue the planned product on ``stream`` (default: torch's current
    stream).  A, B, D: device tensors (or raw device addresses).  A plan that
    splits K needs a workspace (``workspace_for(plan)``); when none is given
    for such a plan, one is taken from torch's allocator on D's device."""
    if workspace is None and plan.workspace_size() and isinstance(D, torch.Tensor):
        workspace = workspace_for(plan, D.device)
    _check(lib.gemm_run(plan.handle, _ptr(A), _ptr(B), _ptr(D), _ptr(workspace), _nbytes(workspace, workspace_bytes),
                        _stream(stream)), "gemm_run")


#: scratch bytes per device behind gemm_run_noalloc (MGEMM_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


def gemm_run_noalloc(plan: Plan, A, B, D, stream=None):
    """Enqueue the planned product without a workspace: a plan's scratch
    comes from the library's own per-device array (no allocation).  Calls
    that overlap on one GPU race."""
    _check(lib.gemm_run_noalloc(plan.handle, _ptr(A), _ptr(B), _ptr(D), _stream(stream)), "gemm_run_noalloc")


def gemm_run_scaled(plan: Plan, A, B, D, scale_a, scale_b, stream=None):
    """Enqueue D = scale_a * scale_b * (A x B) for a plan with E4M3 inputs;
    ``scale_a`` / ``scale_b``: device float32 tensors of one element (read by
    the kernel when it runs).  A, B: uint8 (or float8_e4m3fn) device tensors
    holding the E4M3 codes."""
    _check(lib.gemm_run_scaled(plan.handle, _ptr(A), _ptr(B), _ptr(D), _ptr(scale_a), _ptr(scale_b), None, 0,
                               _stream(stream)), "gemm_run_scaled")


def gemm_run_blockscaled(plan: Plan, A, B, D, scale_a, scale_b, stream=None):
    """Enqueue the blockwise-scaled E4M3 product: ``scale_a`` a uint8 device
    tensor [M, >= ceil(K/128)] of E8M0 bytes (one per row and 128-k block),
    ``scale_b`` [ceil(N/128), >= ceil(K/128)] (one per 128 columns and 128-k
    block); their row pitches are taken from the tensors' strides."""
    _check(lib.gemm_run_blockscaled(plan.handle, _ptr(A), _ptr(B), _ptr(D), _ptr(scale_a), scale_a.stride(0),
                                    _ptr(scale_b), scale_b.stride(0), None, 0, _stream(stream)),
           "gemm_run_blockscaled")


def grouped_gemm_run_scaled(plan: Plan, A, B, D, row_offsets, scale_a, scale_b, stream=None):
    """Enqueue the grouped E4M3 product; ``scale_a``: device float32 tensor of
    one element, ``scale_b``: one float32 per expert (device)."""
    _check(lib.grouped_gemm_run_scaled(plan.handle, _ptr(A), _ptr(B), _ptr(D), _ptr(row_offsets), _ptr(scale_a),
                                       _ptr(scale_b), None, 0, _stream(stream)), "grouped_gemm_run_scaled")


def grouped_gemm_run_blockscaled(plan: Plan, A, B, D, row_offsets, scale_a, scale_b, stream=None):
    """Enqueue the grouped E4M3 product with E8M0 block scales: ``scale_a`` a
    uint8 device tensor [rows, >= ceil(K/128)] (one byte per routed row and
    128-k block), ``scale_b`` [G, ceil(N/128), >= ceil(K/128)] (one per
    expert, 128 columns and 128-k block); pitches from the tensors' strides."""
    _check(lib.grouped_gemm_run_blockscaled(plan.handle, _ptr(A), _ptr(B), _ptr(D), _ptr(row_offsets), _ptr(scale_a),
                                            scale_a.stride(0), _ptr(scale_b), scale_b.stride(1), scale_b.stride(0),
                                            None, 0, _stream(stream)), "grouped_gemm_run_blockscaled")


def grouped_gemm_run(plan: Plan, A, B, D, row_offsets, workspace=None, workspace_bytes: int = 0, stream=None):
    """Enqueue the planned grouped product; ``row_offsets`` is a device int32
    tensor of num_groups + 1 prefix sums."""
    _check(lib.grouped_gemm_run(plan.handle, _ptr(A), _ptr(B), _ptr(D), _ptr(row_offsets), _ptr(workspace),
                                _nbytes(workspace, workspace_bytes), _stream(stream)), "grouped_gemm_run")


def grouped_gemm_run_gather(plan: Plan, X, B, D, row_offsets, row_index, x_rows=None, stream=None):
    """Enqueue the planned grouped product with A's routed row r read from
    X[row_index[r]] (``row_index``: device int32 tensor, one entry per
    routed row)."""
    x_rows = X.shape[0] if x_rows is None else x_rows
    _check(lib.grouped_gemm_run_gather(plan.handle, _ptr(X), x_rows, _ptr(B), _ptr(D), _ptr(row_offsets),
                                       _ptr(row_index), None, 0, _stream(stream)), "grouped_gemm_run_gather")


def grouped_gemm_run_weighted(plan: Plan, A, B, D, row_offsets, row_weight, row_index=None, x_rows=None,
                              stream=None):
    """Enqueue the SiLU-gated grouped product with routed row r's h
    multiplied by ``row_weight[r]`` (float32 cuda tensor, one per routed row)
    before the rounding.  ``row_index``: None (A holds the routed rows) or the
    gathered form's int32 index into A = X."""
    if row_index is not None:
        x_rows = A.shape[0] if x_rows is None else x_rows
    _check(lib.grouped_gemm_run_weighted(plan.handle, _ptr(A), x_rows or 0, _ptr(B), _ptr(D), _ptr(row_offsets),
                                         _ptr(row_index), _ptr(row_weight), None, 0, _stream(stream)),
           "grouped_gemm_run_weighted")


def moe_fused_plan(num_experts, max_total_rows, hidden, inter, dtype="bf16", lda=None, ldw1=None,
                   stride_w1=None, ldw2=None, stride_w2=None, ldh=None, ldy=None, flags: int = 0) -> Plan:
    """Plan the fused MoE layer (FC1 with the SiLU gate, then FC2, one
    launch).  Leading dimensions default to the packed ones."""
    ldw1 = ldw1 if ldw1 is not None else 2 * inter
    ldw2 = ldw2 if ldw2 is not None else hidden
    d = MoeDesc(num_experts, max_total_rows, hidden, inter, DTYPE[dtype], lda if lda is not None else hidden,
                ldw1, stride_w1 if stride_w1 is not None else hidden * ldw1,
                ldw2, stride_w2 if stride_w2 is not None else inter * ldw2,
                ldh if ldh is not None else inter, ldy if ldy is not None else hidden)
    h = ctypes.c_void_p()
    _check(lib.moe_fused_plan(ctypes.byref(d), flags, ctypes.byref(h)), "moe_fused_plan")
    return Plan(h.value, d)


def moe_fused_run(plan: Plan, X, W1, W2, H, Y, row_offsets, workspace=None, row_index=None, x_rows=None,
                  workspace_bytes: int = 0, stream=None):
    """Enqueue the fused layer.  X: routed rows (or, with ``row_index``, the
    token rows that routed row r reads as X[row_index[r]]); H receives h and
    Y the FC2 output.  Without a workspace one is taken from torch's
    allocator on Y's device."""
    if workspace is None and isinstance(Y, torch.Tensor):
        workspace = workspace_for(plan, Y.device)
    if row_index is not None and x_rows is None:
        x_rows = X.shape[0]
    _check(lib.moe_fused_run(plan.handle, _ptr(X), x_rows or 0, _ptr(row_index), _ptr(W1), _ptr(W2), _ptr(H),
                             _ptr(Y), _ptr(row_offsets), _ptr(workspace), _nbytes(workspace, workspace_bytes),
                             _stream(stream)), "moe_fused_run")


def moe_fused_run_weighted(plan: Plan, X, W1, W2, H, Y, row_offsets, row_weight, workspace=None, row_index=None,
                           x_rows=None, workspace_bytes: int = 0, stream=None):
    """``moe_fused_run`` with routed row r's h multiplied by row_weight[r]
    (float32 cuda tensor, one entry per routed row) before its rounding."""
    if workspace is None and isinstance(Y, torch.Tensor):
        workspace = workspace_for(plan, Y.device)
    if row_index is not None and x_rows is None:
        x_rows = X.shape[0]
    _check(lib.moe_fused_run_weighted(plan.handle, _ptr(X), x_rows or 0, _ptr(row_index), _ptr(W1), _ptr(W2),
                                      _ptr(H), _ptr(Y), _ptr(row_offsets), _ptr(row_weight), _ptr(workspace),
                                      _nbytes(workspace, workspace_bytes), _stream(stream)), "moe_fused_run_weighted")


def moe_combine(Z, pos, weights, Y, top_k: int, z_rows=None, stream=None):
    """Enqueue Y[t] = sum_k weights[t, k] * Z[pos[t, k]] (fp32 accumulate,
    one rounding).  Z: [z_rows, H] and Y: [T, H] 16-bit cuda tensors with
    unit column stride; pos: int32 and weights: float32 cuda tensors of
    T * top_k entries; weights None: a plain sum (weights of 1)."""
    T, H = Y.shape
    z_rows = Z.shape[0] if z_rows is None else z_rows
    _check(lib.mgemm_moe_combine(_ptr(Z), z_rows, Z.stride(0), _ptr(pos), _ptr(weights), _ptr(Y), Y.stride(0), T,
                                 top_k, H, TORCH_DTYPE[Y.dtype], _stream(stream)), "mgemm_moe_combine")


def quantize_e4m3_block(X, Q, S, stream=None):
    """Enqueue the blockwise E4M3 quantisation of X (a 16-bit cuda tensor
    [rows, cols], unit column stride) into Q (uint8 [rows, >= cols]) and S
    (uint8 [rows, >= ceil(cols / 128)] E8M0 scales); pitches from strides."""
    rows, cols = X.shape
    _check(lib.mgemm_quantize_e4m3_block(_ptr(X), rows, cols, X.stride(0), TORCH_DTYPE[X.dtype], _ptr(Q), Q.stride(0),
                                         _ptr(S), S.stride(0), _stream(stream)), "mgemm_quantize_e4m3_block")


def tile_budget(M, N, K, BM, BN, BK, stages, elt_bytes) -> Budget:
    b = Budget()
    _check(lib.mgemm_tile_budget(M, N, K, BM, BN, BK, stages, elt_bytes, ctypes.byref(b)), "mgemm_tile_budget")
    return b


def group_working_set(group_m, group_n, BM, BN, K, elt_bytes) -> int:
    return int(lib.mgemm_group_working_set(group_m, group_n, BM, BN, K, elt_bytes))


def round_tokens(n, granule) -> int:
    return int(lib.mgemm_round_tokens(n, granule))


def version() -> str:
    return lib.mgemm_version().decode()
