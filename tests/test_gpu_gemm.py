"""GPU parity of the dense GEMM against the CPU oracle, through the C ABI.

Small and ragged shapes are compared element by element with the full
oracle; the full-size workloads are compared on sampled elements (random
ones plus every tile edge) in the same launch configuration the bench
times.  Integer-valued inputs must match bit for bit; random inputs must
meet the acceptance rule in helpers.py.
"""
import math
import sys
import zlib

import numpy as np
import pytest

import datagen
import oracle
from helpers import (TORCH_OUT, assert_bits_equal, assert_close, from_dev_bits, sample_positions, to_dev)

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu

TILES = {"auto": 0, "256": mg.PLAN_FORCE_TILE_256x256, "128": mg.PLAN_FORCE_TILE_128x128,
         "32n": mg.PLAN_FORCE_TILE_32x256, "64n": mg.PLAN_FORCE_TILE_64x256,
         "256d": mg.PLAN_FORCE_TILE_256x256_DTL, "nrw": mg.PLAN_FORCE_TILE_NARROW}


def tile_skip(tile, al, bl):
    if tile in ("32n", "64n", "nrw") and al == "col":
        pytest.skip("narrow-M tiles take a k-contiguous A only")
    if tile == "256d" and al != "row":
        pytest.skip("the direct-to-LDS tile takes a row-major (k-contiguous) A only")


def log(*a):
    print(*a, flush=True, file=sys.stderr)


ESIZE = {"f32": 4, "bf16": 2, "f16": 2}


def pad8(x: np.ndarray) -> np.ndarray:
    """Storage with its row length padded (with zeros) to a multiple of 8."""
    r, c = x.shape
    if c % 8 == 0:
        return x
    y = np.zeros((r, (c + 7) // 8 * 8), dtype=x.dtype)
    y[:, :c] = x
    return y


def run_dense(a_bits, b_bits, M, N, K, in_t, out_t, a_layout="row", b_layout="row", flags=0, ldd=None,
              sentinel=False, stream=None, workspace_fill=None):
    """Run the library on host bit arrays; returns (D bits [M][N], plan).

    With ``sentinel`` the output lives in a byte buffer pre-filled with 0xFF
    that extends three rows and 64 bytes past D; every byte outside the
    M x N window (the ldd padding and the tail) must still be 0xFF."""
    a_bits, b_bits = pad8(a_bits), pad8(b_bits)   # 16-byte aligned rows
    A = to_dev(a_bits, in_t)
    B = to_dev(b_bits, in_t)
    ldd = ldd or (N + 7) // 8 * 8
    es = ESIZE[out_t]
    nbytes = M * ldd * es + ((3 * ldd * es + 64) if sentinel else 0)
    raw = torch.full((max(nbytes, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    D = raw[: M * ldd * es].view(TORCH_OUT[out_t]).view(M, ldd)
    plan = mg.gemm_plan(M, N, K, in_t, d_type=out_t, a_layout=a_layout, b_layout=b_layout,
                        lda=a_bits.shape[1], ldb=b_bits.shape[1], ldd=ldd, flags=flags)
    ws = mg.workspace_for(plan)
    if ws is not None and workspace_fill is not None:
        ws.fill_(workspace_fill)   # stale scratch contents must not matter
    mg.gemm_run(plan, A, B, D, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    if sentinel:
        tail = raw[M * ldd * es:].cpu().numpy()
        assert np.all(tail == 0xFF), "write past the last row of D"
        if ldd > N and M > 0:
            pad = raw[: M * ldd * es].view(M, ldd * es)[:, N * es:].cpu().numpy()
            assert np.all(pad == 0xFF), "write into D's padding columns"
    return from_dev_bits(D[:, :N]), plan


COMBOS = [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"), ("f16", "f16")]
LAYOUTS = [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")]


@pytest.mark.parametrize("in_t,out_t", COMBOS)
@pytest.mark.parametrize("al,bl", LAYOUTS)
@pytest.mark.parametrize("tile", ["256", "128", "32n", "64n", "256d", "nrw"])
def test_ragged_random_and_integer(in_t, out_t, al, bl, tile):
    tile_skip(tile, al, bl)
    M, N, K = 300, 520, 200   # several tiles, ragged in M, N and K
    log(f"case ragged tile={tile} {in_t}->{out_t} {al}/{bl} M={M} N={N} K={K}")
    cfg = datagen.GemmConfig("t", M, N, K, in_t, out_t, al, bl, ("uniform", 1.0), ("normal", 1.0), seed=7, int_seed=8)
    a, b = datagen.gemm_inputs(cfg, "random")
    got, plan = run_dense(a, b, M, N, K, in_t, out_t, al, bl, TILES[tile], sentinel=True)
    ref = oracle.gemm_ref(a, b, in_t, in_t, al, bl)
    assert_close(got, ref, K, out_t, plan.describe())
    a, b = datagen.gemm_inputs(cfg, "int")
    got, plan = run_dense(a, b, M, N, K, in_t, out_t, al, bl, TILES[tile])
    assert_bits_equal(got, oracle.gemm_ref(a, b, in_t, in_t, al, bl), out_t, plan.describe())


@pytest.mark.parametrize("M,N,K", [(1, 4, 8), (7, 9, 16), (33, 3, 24), (64, 61, 64), (257, 255, 72), (5, 1030, 8),
                                   (2, 2, 512)])
@pytest.mark.parametrize("in_t,out_t", [("bf16", "f32"), ("f16", "f16")])
def test_tiny_and_ragged_shapes(M, N, K, in_t, out_t):
    log(f"case tiny {in_t}->{out_t} M={M} N={N} K={K}")
    cfg = datagen.GemmConfig("t", M, N, K, in_t, out_t, seed=M * 7 + N, int_seed=K)
    a, b = datagen.gemm_inputs(cfg, "int")
    ldd = (N + 7) // 8 * 8 + 8
    got, plan = run_dense(a, b, M, N, K, in_t, out_t, ldd=ldd, sentinel=True)
    assert_bits_equal(got, oracle.gemm_ref(a, b, in_t, in_t), out_t, plan.describe())


def test_empty_shapes():
    log("case empty shapes")
    D = torch.full((4, 8), 7.0, device="cuda")
    A = torch.zeros((4, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((0, 8), dtype=torch.bfloat16, device="cuda")
    plan = mg.gemm_plan(4, 8, 0, "bf16", d_type="f32", lda=8, ldb=8)
    mg.gemm_run(plan, torch.zeros(8, dtype=torch.bfloat16, device="cuda"),
                torch.zeros(8, dtype=torch.bfloat16, device="cuda"), D)
    torch.cuda.synchronize()
    assert torch.all(D == 0)           # the empty sum
    D.fill_(7.0)
    plan = mg.gemm_plan(0, 8, 16, "bf16", d_type="f32", lda=16)
    mg.gemm_run(plan, None, None, D)   # no-op: nothing touched, nulls allowed
    plan = mg.gemm_plan(4, 0, 16, "bf16", d_type="f32", lda=16, ldb=8, ldd=8)
    mg.gemm_run(plan, None, None, D)
    torch.cuda.synchronize()
    assert torch.all(D == 7.0)


@pytest.mark.parametrize("in_t", ["bf16", "f16"])
def test_identity_ones_permutation_exact(in_t):
    log(f"case identity/ones/permutation {in_t}")
    rs = np.random.RandomState(4)
    K = 320
    X = datagen.matrix((K, 272), ("normal", 1.0), in_t, rs)
    I = datagen._to_bits(np.eye(K, dtype=np.float32), in_t)
    got, _ = run_dense(I, X, K, 272, K, in_t, "f32")
    assert np.array_equal(got.view(np.float32).astype(np.float64), oracle.decode(X, in_t))
    ones_a = datagen._to_bits(np.ones((130, 4096), np.float32), in_t)
    ones_b = datagen._to_bits(np.ones((4096, 260), np.float32), in_t)
    got, _ = run_dense(ones_a, ones_b, 130, 260, 4096, in_t, in_t)
    assert np.all(oracle.decode(got, in_t) == 4096.0)
    # B a permutation: D is a column permutation of A, bit-exact for any values
    A = datagen.matrix((200, K), ("normal", 3.0), in_t, rs)
    perm = rs.permutation(K)
    P = np.zeros((K, K), np.float32)
    P[perm, np.arange(K)] = 1.0
    for bl in ("row", "col"):
        Pb = datagen.store(datagen._to_bits(P, in_t), bl)
        got, _ = run_dense(A, Pb, 200, K, K, in_t, "f32", "row", bl)
        assert np.array_equal(got.view(np.float32).astype(np.float64), oracle.decode(A, in_t)[:, perm])


def test_stream_and_event_ordering():
    log("case stream ordering")
    M = N = K = 512
    cfg = datagen.DENSE["gemm512_f16"]
    a, b = datagen.gemm_inputs(cfg, "int")
    A, B = to_dev(a, "f16"), to_dev(b, "f16")
    D = torch.empty((M, N), dtype=torch.float32, device="cuda")
    plan = mg.gemm_plan(M, N, K, "f16", d_type="f32")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ev = torch.cuda.Event()
    with torch.cuda.stream(s1):
        A2 = A * 1       # produced on s1
        ev.record(s1)
    s2.wait_event(ev)
    mg.gemm_run(plan, A2, B, D, stream=s2)
    with torch.cuda.stream(s2):
        D2 = D.clone()   # consumer on the same stream: ordered after the GEMM
    torch.cuda.synchronize()
    assert_bits_equal(from_dev_bits(D2), oracle.gemm_ref(a, b, "f16", "f16"), "f32", "stream")


def test_deterministic():
    log("case determinism")
    cfg = datagen.DENSE["gemm4096_bf16"]
    a, b = datagen.gemm_inputs(cfg, "random", M=1024, N=1024, K=2048)
    g1, _ = run_dense(a, b, 1024, 1024, 2048, "bf16", "bf16")
    g2, _ = run_dense(a, b, 1024, 1024, 2048, "bf16", "bf16")
    assert np.array_equal(g1, g2)


def test_run_errors():
    plan = mg.gemm_plan(64, 64, 64, "bf16", d_type="f32")
    A = torch.zeros(64 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    D = torch.zeros(64 * 64, dtype=torch.float32, device="cuda")
    st = mg.lib.gemm_run(plan.handle, A.data_ptr() + 2, A.data_ptr(), D.data_ptr(), None, 0, None)
    assert st == mg.ERR_UNSUPPORTED


# ------------------------------------------------------------------ split-K


@pytest.mark.parametrize("in_t,out_t", [("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("al,bl", LAYOUTS)
@pytest.mark.parametrize("tile", ["256", "128", "32n", "64n", "256d", "nrw"])
def test_split_k_random_and_integer(in_t, out_t, al, bl, tile):
    """K split into ranges whose fp32 partial tiles are added by the
    reduction (a second kernel; on the few-token tile, the last range in
    the same launch, with two m tiles of it here): ragged M, N (two edge
    columns) and K (a short last step); the workspace starts full of 0xFF."""
    tile_skip(tile, al, bl)
    M, N, K = 150, 302, 1000
    cfg = datagen.GemmConfig("t", M, N, K, in_t, out_t, al, bl, ("uniform", 1.0), ("normal", 1.0), seed=17,
                             int_seed=18)
    for S in (2, 3, 7):
        log(f"case split-K tile={tile} S={S} {in_t}->{out_t} {al}/{bl} M={M} N={N} K={K}")
        flags = TILES[tile] | mg.PLAN_SPLIT_K(S)
        a, b = datagen.gemm_inputs(cfg, "random")
        got, plan = run_dense(a, b, M, N, K, in_t, out_t, al, bl, flags, sentinel=True, workspace_fill=0xFF)
        assert plan.info().splits > 1, plan.describe()
        assert_close(got, oracle.gemm_ref(a, b, in_t, in_t, al, bl), K, out_t, plan.describe())
        a, b = datagen.gemm_inputs(cfg, "int")
        got, plan = run_dense(a, b, M, N, K, in_t, out_t, al, bl, flags)
        assert_bits_equal(got, oracle.gemm_ref(a, b, in_t, in_t, al, bl), out_t, plan.describe())


def test_split_k_workspace_checked_before_launch():
    log("case split-K workspace errors")
    plan = mg.gemm_plan(64, 256, 1024, "bf16", d_type="bf16", flags=mg.PLAN_SPLIT_K(4) | mg.PLAN_FORCE_TILE_NARROW)
    need = plan.workspace_size()
    # few-token tile: 2 output tiles (counters padded to 256 B), 4 slabs each
    assert "narrow128" in plan.describe() and need == 256 + 2 * 4 * 65536
    A = torch.zeros((64, 1024), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((1024, 256), dtype=torch.bfloat16, device="cuda")
    D = torch.full((64, 256), -1.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    h, a, b, d = plan.handle, A.data_ptr(), B.data_ptr(), D.data_ptr()
    assert mg.lib.gemm_run(h, a, b, d, None, 0, None) == mg.ERR_WORKSPACE
    assert mg.lib.gemm_run(h, a, b, d, ws.data_ptr(), need - 1, None) == mg.ERR_WORKSPACE
    assert mg.lib.gemm_run(h, a, b, d, ws.data_ptr() + 8, need, None) == mg.ERR_WORKSPACE
    assert b"workspace" in mg.lib.gemm_last_error_message()
    torch.cuda.synchronize()
    assert torch.all(D == -1.0)        # nothing was launched
    mg.gemm_run(plan, A, B, D, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(D == 0.0)


def test_split_k_deterministic():
    log("case split-K determinism")
    M, N, K = 128, 1024, 4096
    cfg = datagen.GemmConfig("t", M, N, K, "bf16", "bf16", seed=21, int_seed=22)
    a, b = datagen.gemm_inputs(cfg, "random")
    g1, p1 = run_dense(a, b, M, N, K, "bf16", "bf16", flags=mg.PLAN_SPLIT_K(8), workspace_fill=0)
    g2, _ = run_dense(a, b, M, N, K, "bf16", "bf16", flags=mg.PLAN_SPLIT_K(8), workspace_fill=0x7F)
    assert p1.info().splits == 8 and np.array_equal(g1, g2)


def embed(x: np.ndarray, cols: int, fill: int) -> np.ndarray:
    """x in the first columns of a wider array whose other entries are `fill`."""
    y = np.full((x.shape[0], cols), fill, dtype=x.dtype)
    y[:, :x.shape[1]] = x
    return y


@pytest.mark.parametrize("al,bl", LAYOUTS)
@pytest.mark.parametrize("tile", ["auto", "256", "128", "32n", "64n", "256d", "nrw"])
def test_wide_leading_dimensions(tile, al, bl):
    """Leading dimensions well past the matrix (lda = K+24 etc., in elements
    of the stored rows), the slack holding NaN bit patterns: any read of it
    shows up as NaN in D.  Integer inputs, bit-exact; D's padding must stay
    untouched."""
    tile_skip(tile, al, bl)
    M, N, K = 300, 520, 136
    log(f"case wide-ld tile={tile} {al}{bl}")
    cfg = datagen.GemmConfig("t", M, N, K, "bf16", "f32", al, bl, seed=21, int_seed=22)
    a, b = datagen.gemm_inputs(cfg, "int")
    nan16 = 0x7FC1
    a_w = embed(a, a.shape[1] + 24, nan16)
    b_w = embed(b, b.shape[1] + 40, nan16)
    ldd = N + 72
    got, plan = run_dense(a_w, b_w, M, N, K, "bf16", "f32", al, bl, TILES[tile], ldd=ldd, sentinel=True)
    ref = oracle.gemm_ref(a, b, "bf16", "bf16", al, bl)
    assert_bits_equal(got, ref, "f32", plan.describe())


DTL_SHORT_K = ([(K, bl, "bf16", "f32") for K in (8, 64, 72, 136, 200) for bl in ("row", "col")]
               + [(K, bl, "f16", "f16") for K in (72, 200) for bl in ("row", "col")])


@pytest.mark.parametrize("K,bl,in_t,out_t", DTL_SHORT_K)
def test_direct_to_lds_short_k_two_tiles_per_workgroup(K, bl, in_t, out_t):
    """The direct-to-LDS tile with one to four K steps (the prologue's second
    step and the ring's trailing loads fall past K) on 17 x 17 tiles, so 33
    of the 256 workgroups run a second tile in the LDS the first one left:
    every output element against the oracle, integer inputs, bit-exact."""
    M, N = 4300, 4100
    log(f"case dtl short-k M={M} N={N} K={K} {in_t}->{out_t} B {bl}")
    cfg = datagen.GemmConfig("t", M, N, K, in_t, out_t, "row", bl, seed=11, int_seed=K + 3)
    a, b = datagen.gemm_inputs(cfg, "int")
    got, plan = run_dense(a, b, M, N, K, in_t, out_t, "row", bl, TILES["256d"])
    assert "256x256dtl" in plan.describe() and "tiles=289" in plan.describe(), plan.describe()
    ref = oracle.gemm_ref(a, b, in_t, in_t, "row", bl)
    assert_bits_equal(got, ref, out_t, plan.describe())


@pytest.mark.parametrize("K", [1000, 2056])
@pytest.mark.parametrize("bl", ["row", "col"])
def test_direct_to_lds_long_k_ragged_tail(K, bl):
    """The direct-to-LDS tile over many K steps with a partial last one: the
    steps before the last take the unmasked loads, the last three the masked
    ones; ragged M and N (partial tiles at both edges).  Integer inputs
    bit-exact, random inputs within the tolerance."""
    M, N = 300, 520
    log(f"case dtl long-k M={M} N={N} K={K} B {bl}")
    cfg = datagen.GemmConfig("t", M, N, K, "bf16", "f32", "row", bl, ("uniform", 1.0), ("normal", 1.0),
                             seed=K, int_seed=K + 1)
    a, b = datagen.gemm_inputs(cfg, "int")
    got, plan = run_dense(a, b, M, N, K, "bf16", "f32", "row", bl, TILES["256d"], sentinel=True)
    assert "256x256dtl" in plan.describe() and "splits=1" in plan.describe(), plan.describe()
    assert_bits_equal(got, oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl), "f32", plan.describe())
    a, b = datagen.gemm_inputs(cfg, "random")
    got, plan = run_dense(a, b, M, N, K, "bf16", "f32", "row", bl, TILES["256d"])
    assert_close(got, oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl), K, "f32", plan.describe())


@pytest.mark.parametrize("bl,out_t", [("col", "f32"), ("row", "bf16")])
def test_direct_to_lds_steady_state_second_tile_full(bl, out_t):
    """The paired-step steady-state loop (unmasked loads, the 2-slot
    operand's slot fixed per step of a pair) on a workgroup's second tile:
    4352 x 4352 gives 17 x 17 = 289 tiles of 256 x 256 on 256 workgroups,
    K = 1024 gives 16 steps, 12 of them in unmasked pairs.  Every output
    element against the oracle, integer inputs, bit-exact."""
    M = N = 4352
    K = 1024
    log(f"case dtl steady-state second tile M={M} N={N} K={K} B {bl} -> {out_t}")
    cfg = datagen.GemmConfig("t", M, N, K, "bf16", out_t, "row", bl, seed=41, int_seed=43 + (bl == "row"))
    a, b = datagen.gemm_inputs(cfg, "int")
    got, plan = run_dense(a, b, M, N, K, "bf16", out_t, "row", bl, TILES["256d"])
    d = plan.describe()
    assert "256x256dtl" in d and "tiles=289" in d and "grid=256" in d and "splits=1" in d, d
    assert_bits_equal(got, oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl), out_t, d)


# --------------------------------------------------------------- full size

FULL = ["gemm512_f16", "gemm4096_bf16", "gemm8192_bf16_bcol", "ts16384x2048x7168", "decode128x7168x2048"]


@pytest.mark.parametrize("name,flags", [(n, 0) for n in FULL] +
                         [("gemm8192_bf16_bcol", mg.PLAN_FORCE_TILE_256x256),
                          ("gemm4096_bf16", mg.PLAN_FORCE_TILE_256x256)])
@pytest.mark.parametrize("variant", ["random", "int"])
def test_full_size_workloads(name, flags, variant):
    cfg = datagen.DENSE[name]
    log(f"case full {name} flags={flags:#x} {variant}")
    a, b = datagen.gemm_inputs(cfg, variant)
    A, B = to_dev(a, cfg.in_dtype), to_dev(b, cfg.in_dtype)
    D = torch.empty((cfg.M, cfg.N), dtype=TORCH_OUT[cfg.out_dtype], device="cuda")
    plan = mg.gemm_plan(cfg.M, cfg.N, cfg.K, cfg.in_dtype, d_type=cfg.out_dtype, a_layout=cfg.a_layout,
                        b_layout=cfg.b_layout, flags=flags)
    mg.gemm_run(plan, A, B, D)
    torch.cuda.synchronize()
    got = from_dev_bits(D)
    if cfg.M * cfg.N * cfg.K <= 512 ** 3:
        ref = oracle.gemm_ref(a, b, cfg.in_dtype, cfg.in_dtype, cfg.a_layout, cfg.b_layout)
        sel = (slice(None), slice(None))
        g = got
    else:
        inf = plan.info()
        seed = zlib.crc32(name.encode()) % 1000   # fixed per workload: a failure replays
        log(f"  sample seed {seed}")
        r, c = sample_positions(cfg.M, cfg.N, 3000, (inf.block_m, inf.block_n), seed=seed)
        ref = oracle.gemm_ref_sampled(a, b, r, c, cfg.in_dtype, cfg.in_dtype, cfg.a_layout, cfg.b_layout)
        g = got[r, c]
    if variant == "int":
        assert_bits_equal(g, ref, cfg.out_dtype, plan.describe())
    else:
        err = assert_close(g, ref, cfg.K, cfg.out_dtype, plan.describe())
        log(f"  max abs err {err:.3e} (tol base {1e-4 * math.sqrt(cfg.K):.3e})")
    # no NaN/Inf anywhere in the output
    vals = D.float()
    assert torch.isfinite(vals).all()


@pytest.mark.parametrize("tile", ["auto", "128", "256"])
@pytest.mark.parametrize("out_t", ["f32", "bf16"])
def test_col_major_a_odd_row_count(tile, out_t):
    """Column-major A with an odd M: the last row's last element shares a
    dword with the storage padding at the last k row, which must not be
    read as zero (every element, integer inputs, bit for bit)."""
    M, N, K = 431, 138, 320
    log(f"case col-major A odd M tile={tile} bf16->{out_t} M={M} N={N} K={K}")
    cfg = datagen.GemmConfig("t", M, N, K, "bf16", out_t, "col", "row", seed=11, int_seed=12)
    a, b = datagen.gemm_inputs(cfg, "int")
    got, plan = run_dense(a, b, M, N, K, "bf16", out_t, "col", "row", TILES[tile], sentinel=True)
    assert_bits_equal(got, oracle.gemm_ref(a, b, "bf16", "bf16", "col", "row"), out_t, plan.describe())


@pytest.mark.parametrize("M,N,K", [(64, 64, 65536), (1, 1, 8), (3, 2056, 32768), (700, 9, 4104)])
def test_extreme_aspect_ratios(M, N, K):
    """Very long K against tiny M and N (the planner's split and few-token
    choices), and one-element outputs; integer inputs (sums below 2^24, so
    exact in fp32), every element bit for bit."""
    log(f"case extreme M={M} N={N} K={K}")
    for bl in ("row", "col"):
        cfg = datagen.GemmConfig("t", M, N, K, "bf16", "f32", "row", bl, seed=21, int_seed=22)
        a, b = datagen.gemm_inputs(cfg, "int")
        got, plan = run_dense(a, b, M, N, K, "bf16", "f32", "row", bl, sentinel=True)
        log("  " + plan.describe())
        assert_bits_equal(got, oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl), "f32", plan.describe())


def test_largest_leading_dimension():
    """lda and ldb at the 2^20-element limit (rows 2 MiB apart), a few rows."""
    M, N, K, ld = 5, 24, 64, 1 << 20
    log(f"case largest leading dimension ld={ld}")
    cfg = datagen.GemmConfig("t", M, N, K, "bf16", "f32", "row", "col", seed=23, int_seed=24)
    a, b = datagen.gemm_inputs(cfg, "int")
    A = np.zeros((M, ld), dtype=np.uint16)
    A[:, :K] = a
    B = np.zeros((N, ld), dtype=np.uint16)
    B[:, :K] = b
    got, plan = run_dense(A, B, M, N, K, "bf16", "f32", "row", "col", sentinel=True)
    assert_bits_equal(got, oracle.gemm_ref(a, b, "bf16", "bf16", "row", "col"), "f32", plan.describe())
