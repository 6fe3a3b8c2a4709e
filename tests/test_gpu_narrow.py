"""GPU parity of the few-token tile against the CPU oracle: dense plans
with up to 128 rows (the decode shape among them) and the tile's split of K
with the reduction inside the launch.

The tile computes only a tile's valid tokens rounded up to 16 (one to
eight blocks of 16), so the cases cover every token-block count, ragged
column counts and K tails.  A split plan's ranges publish fp32 partial
tiles and the last range to arrive adds them in range order, so results
must not depend on timing: repeated runs are compared bit for bit, the
workspace is handed over full of 0xFF bytes, reused across plans, and the
launch is replayed from a captured HIP graph.  Integer-valued inputs are
bit-exact against the oracle; random inputs within the tolerance.
"""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import TORCH_OUT, assert_bits_equal, assert_close, from_dev_bits, to_dev

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def inputs(M, N, K, bl, variant, seed, in_t="bf16"):
    cfg = datagen.GemmConfig("narrow", M, N, K, in_t, "f32", "row", bl, ("normal", 1.0), ("normal", 0.02),
                             seed=seed, int_seed=seed + 1)
    return datagen.gemm_inputs(cfg, variant)


def ldd_for(N, out_t):
    return -(-N // 8) * 8 if out_t != "f32" else -(-N // 4) * 4


def pad8(x):
    """Storage rows padded (with zeros) to a multiple of 8 elements (16 bytes)."""
    r, c = x.shape
    if c % 8 == 0:
        return x
    y = np.zeros((r, -(-c // 8) * 8), dtype=x.dtype)
    y[:, :c] = x
    return y


def run(a, b, M, N, K, bl, in_t, out_t, flags=0, ws=None, plan=None):
    """(D bits [M][N], plan); D's padding columns start as NaN and must stay so."""
    a, b = pad8(a), pad8(b)
    ldd = ldd_for(N, out_t)
    plan = plan or mg.gemm_plan(M, N, K, in_t, d_type=out_t, b_layout=bl, lda=a.shape[1], ldb=b.shape[1],
                                ldd=ldd, flags=flags)
    D = torch.full((M, ldd), float("nan"), dtype=TORCH_OUT[out_t], device="cuda")
    if ws is None and plan.workspace_size():
        ws = torch.full((plan.workspace_size(),), 0xFF, dtype=torch.uint8, device="cuda")
    mg.gemm_run(plan, to_dev(a, in_t), to_dev(b, in_t), D, workspace=ws)
    torch.cuda.synchronize()
    if ldd > N:
        assert torch.isnan(D[:, N:].float()).all(), "padding columns written"
    return from_dev_bits(D[:, :N]), plan


SHAPES = [(1, 128, 64), (5, 260, 72), (16, 512, 136), (17, 1000, 520), (33, 384, 1024), (64, 256, 200),
          (100, 772, 2056), (128, 1024, 520), (127, 130, 8)]


WIDTHS = {128: mg.PLAN_FORCE_TILE_NARROW, 64: mg.PLAN_FORCE_TILE_NARROW64, 32: mg.PLAN_FORCE_TILE_NARROW32}


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("bl", ["row", "col"])
@pytest.mark.parametrize("variant", ["random", "int"])
@pytest.mark.parametrize("width", [128, 64, 32])
def test_narrow_dense(shape, bl, variant, width):
    """Every token-block count (1 .. 8), ragged N (an edge column included),
    K tails, on each width of the tile; the planner's split choice."""
    M, N, K = shape
    log(f"case narrow{width} {M}x{N}x{K} B {bl} {variant}")
    a, b = inputs(M, N, K, bl, variant, seed=M * 7 + K)
    got, plan = run(a, b, M, N, K, bl, "bf16", "bf16", flags=WIDTHS[width])
    d = plan.describe()
    assert f"tile=narrow{width}" in d and f"tokens={-(-M // 16) * 16} " in d, d
    ref = oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl)
    if variant == "int":
        assert_bits_equal(got, ref, "bf16", d)
    else:
        assert_close(got, ref, K, "bf16", d)


@pytest.mark.parametrize("in_t,out_t", [("f16", "f32"), ("f16", "f16"), ("bf16", "f32")])
def test_narrow_other_types(in_t, out_t):
    M, N, K = 40, 640, 400
    log(f"case narrow {in_t}->{out_t}")
    for variant in ("int", "random"):
        a, b = inputs(M, N, K, "row", variant, seed=9, in_t=in_t)
        got, plan = run(a, b, M, N, K, "row", in_t, out_t)
        ref = oracle.gemm_ref(a, b, in_t, in_t, "row", "row")
        if variant == "int":
            assert_bits_equal(got, ref, out_t, plan.describe())
        else:
            assert_close(got, ref, K, out_t, plan.describe())


@pytest.mark.parametrize("splits", [2, 3, 4, 7])
@pytest.mark.parametrize("bl", ["row", "col"])
@pytest.mark.parametrize("width", [128, 64, 32])
def test_narrow_split_fixed_order(splits, bl, width):
    """Forced K splits (7 ranges of 2 steps, the last one short): integer
    inputs bit-exact; random inputs within the tolerance and bit-identical
    over three runs on one 0xFF-filled workspace (the reduction order does not
    depend on which range finishes last)."""
    M, N, K = 100, 520, 840
    log(f"case narrow{width} split {splits} B {bl}")
    flags = mg.PLAN_SPLIT_K(splits) | WIDTHS[width]
    a, b = inputs(M, N, K, bl, "int", seed=splits)
    got, plan = run(a, b, M, N, K, bl, "bf16", "f32", flags=flags)
    assert f"splits={splits}" in plan.describe(), plan.describe()
    assert_bits_equal(got, oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl), "f32", plan.describe())
    a, b = inputs(M, N, K, bl, "random", seed=splits + 50)
    ws = torch.full((plan.workspace_size(),), 0xFF, dtype=torch.uint8, device="cuda")
    outs = [run(a, b, M, N, K, bl, "bf16", "f32", ws=ws, plan=plan)[0] for _ in range(3)]
    assert all(np.array_equal(o, outs[0]) for o in outs[1:]), "split results differ between runs"
    assert_close(outs[0], oracle.gemm_ref(a, b, "bf16", "bf16", "row", bl), K, "f32", plan.describe())


def test_narrow_split_workspace_shared_by_plans():
    """One workspace used by two split plans in turn, each run twice: the
    arrival counters of one plan are slab bytes of the other."""
    cases = [(128, 7168, 2048, 4), (64, 1536, 4096, 8), (128, 7168, 2048, 4)]
    size = max(mg.gemm_plan(M, N, K, "bf16", d_type="bf16", flags=mg.PLAN_SPLIT_K(S)).workspace_size()
               for M, N, K, S in cases)
    ws = torch.full((size,), 0xFF, dtype=torch.uint8, device="cuda")
    for i, (M, N, K, S) in enumerate(cases):
        log(f"case narrow shared workspace {M}x{N}x{K} splits {S}")
        a, b = inputs(M, N, K, "row", "int", seed=100 + i)
        plan = mg.gemm_plan(M, N, K, "bf16", d_type="bf16", flags=mg.PLAN_SPLIT_K(S))
        ref = oracle.gemm_ref(a, b, "bf16", "bf16", "row", "row")
        for _ in range(2):
            got, _ = run(a, b, M, N, K, "row", "bf16", "bf16", ws=ws, plan=plan)
            assert_bits_equal(got, ref, "bf16", plan.describe())


@pytest.mark.parametrize("variant", ["random", "int"])
def test_decode_shape_every_element(variant):
    """128 x 7168 x 2048 (row-major bf16 weights normal(0, 0.02), activations
    normal(0, 1)) in the bench's launch: every output element."""
    cfg = datagen.DENSE["decode128x7168x2048"]
    log(f"case decode full {variant}")
    a, b = datagen.gemm_inputs(cfg, variant)
    got, plan = run(a, b, cfg.M, cfg.N, cfg.K, cfg.b_layout, cfg.in_dtype, cfg.out_dtype)
    d = plan.describe()
    assert "tile=narrow" in d and "tokens=128" in d and plan.info().splits > 1, d
    ref = oracle.gemm_ref(a, b, cfg.in_dtype, cfg.in_dtype, cfg.a_layout, cfg.b_layout)
    if variant == "int":
        assert_bits_equal(got, ref, cfg.out_dtype, d)
    else:
        assert_close(got, ref, cfg.K, cfg.out_dtype, d)


def test_narrow_split_graph_replay():
    """The split launch captured in a HIP graph (the same run tag on every
    replay) and replayed three times, new inputs copied in and D refilled
    between replays by eager work; every replay against the oracle."""
    M, N, K = 96, 2048, 1536
    plan = mg.gemm_plan(M, N, K, "bf16", d_type="f32", flags=mg.PLAN_SPLIT_K(4))
    assert "narrow" in plan.describe() and "splits=4" in plan.describe()
    ws = torch.full((plan.workspace_size(),), 0xFF, dtype=torch.uint8, device="cuda")
    sets = [inputs(M, N, K, "row", "int", seed=300 + i) for i in range(3)]
    A = to_dev(sets[0][0], "bf16")
    B = to_dev(sets[0][1], "bf16")
    D = torch.empty((M, N), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mg.gemm_run(plan, A, B, D, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.gemm_run(plan, A, B, D, workspace=ws)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(sets):
        log(f"case narrow graph replay {i}")
        A.copy_(to_dev(a, "bf16"))
        B.copy_(to_dev(b, "bf16"))
        D.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(from_dev_bits(D), oracle.gemm_ref(a, b, "bf16", "bf16"), "f32", f"replay {i}")
