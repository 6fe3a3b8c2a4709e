"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
its planner reproduces the pages' worked budget numbers, and argument
errors are reported before anything is enqueued (no GPU needed)."""
import json
import os
import re

import pytest

import bf16_gemm_amd as mg

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "planner_pins.json")))
HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mgemm.h")


def test_exports_match_header():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)      # drop comments
    declared = set(re.findall(r"\b((?:gemm|grouped_gemm|mgemm|moe)_\w+)\s*\(", text))
    assert declared == set(mg.EXPORTS), declared ^ set(mg.EXPORTS)
    for name in declared:
        assert hasattr(mg.lib, name), name
    assert mg.version().startswith("mgemm")


def test_header_constants_match_binding():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    enums = dict((k, int(v)) for k, v in re.findall(r"\b(MGEMM_[A-Z0-9_]+)\s*=\s*(\d+)", text))
    flags = dict((k, int(v, 16)) for k, v in re.findall(r"#define\s+(MGEMM_PLAN_\w+)\s+0x([0-9a-fA-F]+)u", text))
    assert (enums["MGEMM_F16"], enums["MGEMM_BF16"], enums["MGEMM_F32"]) == (mg.F16, mg.BF16, mg.F32)
    assert (enums["MGEMM_ROW_MAJOR"], enums["MGEMM_COL_MAJOR"]) == (mg.ROW_MAJOR, mg.COL_MAJOR)
    assert (enums["MGEMM_EPI_NONE"], enums["MGEMM_EPI_SILU_GATE_I8"]) == (mg.EPI_NONE, mg.EPI_SILU_GATE_I8)
    assert [enums[k] for k in ("MGEMM_OK", "MGEMM_ERR_INVALID_ARG", "MGEMM_ERR_UNSUPPORTED", "MGEMM_ERR_WORKSPACE",
                               "MGEMM_ERR_NO_MEMORY", "MGEMM_ERR_HIP")] == [mg.OK, mg.ERR_INVALID_ARG,
                                                                            mg.ERR_UNSUPPORTED, mg.ERR_WORKSPACE,
                                                                            mg.ERR_NO_MEMORY, mg.ERR_HIP]
    assert len(flags) == 9
    for name, value in flags.items():
        assert getattr(mg, name[len("MGEMM_"):]) == value, name
    assert "((((uint32_t)(n)) & 0xFFu) << 16)" in text and mg.PLAN_SPLIT_K(5) == 5 << 16


def test_tile_calculator_pin():
    g = GOLD["tile_calculator"]
    b = mg.tile_budget(g["M"], g["N"], g["K"], g["BM"], g["BN"], g["BK"], g["stages"], g["elt_bytes"])
    assert b.tiles == g["tiles"]
    assert b.coverage == pytest.approx(g["coverage"])
    assert b.k_steps == g["k_steps"]
    # one CTA of the page's pair holds half of each tile side
    half = mg.tile_budget(g["M"], g["N"], g["K"], g["BM"] // 2, g["BN"] // 2, g["BK"], g["stages"], g["elt_bytes"])
    assert half.lds_bytes == g["per_cta_input_kib_with_pair_split"] * 1024
    assert b.lds_bytes == 2 * half.lds_bytes


def test_k_tile_doubling_pin():
    g = GOLD["k_tile_doubling"]
    for bk, kib in g["stage_kib"].items():
        b = mg.tile_budget(256, 256, 4096, g["BM_per_cta"], g["BN_per_cta"], int(bk), 1, 2)
        assert b.lds_bytes == kib * 1024
        b3 = mg.tile_budget(256, 256, 4096, g["BM_per_cta"], g["BN_per_cta"], int(bk), 3, 2)
        assert b3.lds_bytes == g["three_stage_kib"][bk] * 1024


def test_stage_cost_pin():
    g = GOLD["stage_cost"]
    b = mg.tile_budget(4096, 4096, 4096, g["BM"], g["BN"], g["BK"], 1, g["elt_bytes"])
    assert b.lds_bytes == g["stage_bytes"]
    for depth, kb in g["depth_total_kb"].items():
        tot = mg.tile_budget(4096, 4096, 4096, g["BM"], g["BN"], g["BK"], int(depth), 2).lds_bytes + g["writeback_bytes"]
        assert tot == kb * 1024


def test_supertile_working_set_pin():
    g = GOLD["supertile_working_set"]
    for c in g["cases"]:
        ws = mg.group_working_set(c["group_m"], c["group_n"], g["BM"], g["BN"], g["K"], g["elt_bytes"])
        assert ws == c["bytes"]
        if "a_part_bytes" in c:
            assert mg.group_working_set(c["group_m"], 0, g["BM"], g["BN"], g["K"], g["elt_bytes"]) == c["a_part_bytes"]
    p = g["b_reread_passes"]
    assert p["grid_m"] // p["super_m"] == p["passes"]


def test_dynamic_n_pin():
    g = GOLD["dynamic_n"]
    assert mg.round_tokens(g["tokens"], g["granule"]) == g["rounded"]
    assert g["static_n"] - g["tokens"] == g["padding_before"]
    assert g["rounded"] - g["tokens"] == g["padding_after"]
    assert mg.round_tokens(0, 16) == 0 and mg.round_tokens(16, 16) == 16 and mg.round_tokens(17, 16) == 32
    assert mg.round_tokens(5, 12) == -1


def test_plan_choices_for_workloads():
    p = mg.gemm_plan(8192, 8192, 8192, "bf16", d_type="f32", b_layout="col")
    i = p.info()
    assert (i.block_m, i.block_n, i.block_k) == (256, 256, 64)
    assert i.tiles == 1024 and i.coverage == 1.0 and i.lds_bytes <= 160 * 1024
    assert i.grid == min(1024, i.num_cus)
    # the decode shape: 128 tokens on the few-token tile; the planner's time
    # model takes 64 columns and two K ranges (112 tiles x 2 = 224 tasks)
    p = mg.gemm_plan(128, 7168, 2048, "bf16", d_type="bf16")
    i = p.info()
    assert "tile=narrow64 tokens=128" in p.describe() and (i.block_m, i.block_n) == (128, 64), p.describe()
    # two rings at 128 tokens: 8 token slots, 3 weight slots (the deeper one is info().stages)
    assert i.splits == 2 and i.tiles == 112 and i.grid == 224 and i.stages == 8, p.describe()
    assert "stages=8a/3b" in p.describe() and i.lds_bytes == 8 * 128 * 128 + 3 * 64 * 128, p.describe()
    p = mg.gemm_plan(128, 7168, 2048, "bf16", d_type="bf16", flags=mg.PLAN_SPLIT_K(1))
    assert "narrow" in p.describe() and p.info().splits == 1 and p.workspace_size() == 0, p.describe()
    # forced widths: 128 columns (six token slots, three weight slots), 32
    # columns (two waves; four token slots, the vmcnt bound of one token
    # wave's 16 loads a step, and sixteen weight slots)
    p = mg.gemm_plan(128, 7168, 2048, "bf16", d_type="bf16", flags=mg.PLAN_FORCE_TILE_NARROW)
    assert "tile=narrow128" in p.describe() and "stages=6a/3b" in p.describe() and p.info().splits == 4, \
        p.describe()
    p = mg.gemm_plan(128, 7168, 2048, "bf16", d_type="bf16", flags=mg.PLAN_FORCE_TILE_NARROW32)
    assert "tile=narrow32" in p.describe() and "waves=1x2" in p.describe() and p.info().stages == 16
    # fewer tokens: smaller token slots, more of them (up to eight), more weight slots
    p = mg.gemm_plan(16, 7168, 2048, "bf16", d_type="bf16", flags=mg.PLAN_FORCE_TILE_NARROW64)
    assert "stages=8a/16b" in p.describe() and p.info().lds_bytes == 8 * 16 * 128 + 16 * 64 * 128, p.describe()
    # the token width is the row count rounded up to 16 (mgemm_round_tokens)
    for M, w in [(1, 16), (16, 16), (17, 32), (100, 112), (128, 128)]:
        assert f"tokens={w} " in mg.gemm_plan(M, 4096, 1024, "bf16", d_type="bf16").describe()
    assert "narrow" not in mg.gemm_plan(129, 4096, 1024, "bf16", d_type="bf16").describe()
    p = mg.grouped_gemm_plan(64, 32768, 4096, 7168, epilogue=mg.EPI_SILU_GATE_I8)
    assert "[1,129)->narrow128" in p.describe() and "[129,inf)->256x256dtl" in p.describe()


def test_split_k_plans():
    # whole-chip shapes are never split and need no workspace
    for (M, N, K) in [(8192, 8192, 8192), (4096, 4096, 4096), (16384, 2048, 7168), (512, 512, 512)]:
        p = mg.gemm_plan(M, N, K, "bf16", d_type="bf16")
        assert p.info().splits == 1 and p.workspace_size() == 0 and "splits=1" in p.describe(), p.describe()
    # a split plan on the few-token tile needs one 8-byte arrival counter per
    # output tile (rounded up to 256 bytes), then a 64 KiB partial slab per
    # (tile, range)
    # (128 x block_n x 4 bytes)
    p = mg.gemm_plan(128, 7170, 2048, "bf16", d_type="bf16", ldb=7176, ldd=7176)
    i = p.info()
    assert i.splits > 1 and f"splits={i.splits}" in p.describe() and i.tiles == 112
    assert p.workspace_size() == 1024 + 112 * i.splits * 128 * 64 * 4
    # forced counts: K = 2048 is 32 steps; 3 ranges of 11 steps
    p = mg.gemm_plan(128, 7168, 2048, "bf16", d_type="bf16", flags=mg.PLAN_SPLIT_K(3) | mg.PLAN_FORCE_TILE_NARROW)
    assert p.info().splits == 3 and p.workspace_size() == 512 + 56 * 3 * 65536
    # other tiles split with fp32 slabs of M x (N rounded down to 4), added by a second kernel
    p = mg.gemm_plan(128, 7168, 2048, "bf16", d_type="bf16", flags=mg.PLAN_SPLIT_K(3) | mg.PLAN_FORCE_TILE_128x128)
    assert p.info().splits == 3 and p.workspace_size() == 3 * 128 * 7168 * 4
    p = mg.gemm_plan(64, 64, 128, "bf16", d_type="f32", flags=mg.PLAN_SPLIT_K(16))
    assert p.info().splits == 2   # never more ranges than K steps
    p = mg.gemm_plan(8192, 8192, 8192, "bf16", flags=mg.PLAN_SPLIT_K(2) | mg.PLAN_FORCE_TILE_256x256)
    assert p.info().splits == 2 and p.workspace_size() == 2 * 8192 * 8192 * 4
    with pytest.raises(mg.MgemmError) as e:
        mg.gemm_plan(128, 7168, 2048, "bf16", flags=mg.PLAN_SPLIT_K(65))
    assert e.value.status == mg.ERR_INVALID_ARG
    # K == 0 and empty shapes: nothing to split
    assert mg.gemm_plan(4, 8, 0, "bf16", lda=8, flags=mg.PLAN_SPLIT_K(4)).workspace_size() == 0
    assert mg.gemm_plan(0, 8, 64, "bf16", flags=mg.PLAN_SPLIT_K(4)).workspace_size() == 0


def test_stream_k_plans():
    """A partial last round of 256 x 256 tiles (at most half the CUs) with a
    long K is balanced by stream-K: the last tiles are cut into K ranges
    (at most four), the rest run whole; its workspace holds one 8-byte
    counter per cut tile (256-byte rounded) and one 256 x 256 fp32 partial
    per range."""
    p = mg.gemm_plan(5120, 4096, 8192, "bf16", d_type="bf16", b_layout="col")
    d = p.describe()
    assert "tile=256x256dtl" in d and "tiles=320" in d and "stream_k_tiles=64" in d and "splits=4" in d, d
    assert p.info().grid == 256 and p.workspace_size() == 512 + 64 * 4 * 256 * 256 * 4
    p = mg.gemm_plan(4352, 4352, 4096, "bf16", d_type="bf16")
    assert "stream_k_tiles=33" in p.describe() and p.workspace_size() == 512 + 33 * 4 * 256 * 256 * 4
    # whole rounds, short K, a mostly full last round, or a fixed split: no stream-K
    for (M, N, K, fl) in [(8192, 8192, 8192, 0), (4352, 4352, 1024, 0), (7936, 8192, 4096, 0),
                          (5120, 4096, 8192, mg.PLAN_SPLIT_K(1))]:
        p = mg.gemm_plan(M, N, K, "bf16", d_type="bf16", flags=fl)
        assert "stream_k" not in p.describe(), p.describe()


def test_direct_to_lds_tile_choice():
    # k-contiguous A and B: the planner's 256x256 tile runs on the direct-to-LDS engine
    p = mg.gemm_plan(8192, 8192, 8192, "bf16", d_type="f32", b_layout="col")
    i = p.info()
    # (four waves of 128x128; column-major B: the 3-slot ring on B)
    assert "tile=256x256dtl" in p.describe() and i.lds_bytes == 160 * 1024 and (i.waves_m, i.waves_n) == (2, 2)
    assert "waves=2x2" in p.describe() and "stages=2a/3b" in p.describe() and i.stages == 3
    # forcing the 256x256 tile keeps the register-staged engine
    p = mg.gemm_plan(8192, 8192, 8192, "bf16", d_type="f32", b_layout="col", flags=mg.PLAN_FORCE_TILE_256x256)
    assert "tile=256x256 " in p.describe() and p.info().lds_bytes == 128 * 1024
    # row-major B too (its fragments are read with LDS transpose reads); a
    # column-major A never
    p = mg.gemm_plan(4096, 4096, 4096, "bf16", d_type="bf16")
    assert "tile=256x256dtl waves=2x2" in p.describe() and "stages=3a/2b" in p.describe()
    assert (p.info().waves_m, p.info().waves_n) == (2, 2)
    assert "dtl" not in mg.gemm_plan(4096, 4096, 4096, "bf16", d_type="bf16", a_layout="col").describe()
    p = mg.gemm_plan(8192, 8192, 8192, "bf16", d_type="f32", b_layout="col", flags=mg.PLAN_FORCE_TILE_256x256_DTL)
    i = p.info()
    assert "tile=256x256dtl" in p.describe() and i.lds_bytes == 160 * 1024 and (i.block_m, i.block_n) == (256, 256)
    for kw in (dict(a_layout="col", b_layout="row"), dict(a_layout="col", b_layout="col")):
        with pytest.raises(mg.MgemmError) as e:
            mg.gemm_plan(512, 512, 512, "bf16", flags=mg.PLAN_FORCE_TILE_256x256_DTL, **kw)
        assert e.value.status == mg.ERR_UNSUPPORTED
    # grouped: the large-expert bucket runs on the direct-to-LDS tile (task
    # list in registers); forcing the 256x256 tile keeps the register engine
    g = mg.grouped_gemm_plan(64, 32768, 4096, 7168)
    assert "[129,inf)->256x256dtl" in g.describe() and "[1,129)->narrow128" in g.describe()
    # the few-token tile takes a row-major A only
    with pytest.raises(mg.MgemmError) as e:
        mg.gemm_plan(64, 512, 512, "bf16", a_layout="col", flags=mg.PLAN_FORCE_TILE_NARROW)
    assert e.value.status == mg.ERR_UNSUPPORTED
    for bl in ("row", "col"):
        g = mg.grouped_gemm_plan(4, 64, 256, 128, b_layout=bl, flags=mg.PLAN_FORCE_TILE_256x256_DTL)
        assert "->256x256dtl" in g.describe()
        g = mg.grouped_gemm_plan(4, 64, 256, 128, b_layout=bl, flags=mg.PLAN_FORCE_TILE_256x256)
        assert "->256x256 " in g.describe()


def test_lds_budget_rejects_three_stage_macro_tile():
    """The planner sizes each plan's ring with the stage budget and keeps it
    within a CU's 160 KiB: three stages of both 256x256 operands (192 KiB)
    do not fit, so the 256x256 plans give the deeper third stage to one
    operand only (3 + 2 stages = 160 KiB), A when B is row-major, B when it
    is column-major; two-stage tiles fit twice per CU."""
    assert mg.tile_budget(256, 256, 64, 256, 256, 64, 3, 2).lds_bytes == 192 * 1024 > 160 * 1024
    half = mg.tile_budget(256, 256, 64, 256, 256, 64, 1, 2).lds_bytes // 2   # one operand's stage
    for bl, deep in (("row", "3a/2b"), ("col", "2a/3b")):
        p = mg.gemm_plan(8192, 8192, 8192, "bf16", d_type="bf16", b_layout=bl)
        inf = p.info()
        assert "tile=256x256dtl" in p.describe() and f"stages={deep}" in p.describe()
        assert inf.stages == 3 and inf.lds_bytes == 5 * half == 160 * 1024
    p = mg.gemm_plan(2048, 2048, 512, "bf16")
    assert "tile=128x128" in p.describe()
    assert p.info().lds_bytes == mg.tile_budget(2048, 2048, 512, 128, 128, 64, 2, 2).lds_bytes == 64 * 1024
    assert p.info().grid == min(p.info().tiles, 2 * p.info().num_cus)   # two rings per CU


def test_group_m_from_working_set():
    """group_m: of the power-of-two blocks of tiles one XCD runs at once
    (its CUs x workgroups per CU), the one whose super-tile working set is
    smallest, fewer rows on a tie -- 4 x 8 for the 256x256 tile."""
    def expect(p, BM, BN, occ):
        inf = p.info()
        conc = inf.num_cus // 8 * occ
        best, best_ws, gm = 1, None, 1
        while gm <= conc and gm <= inf.tiles_m:
            ws = mg.group_working_set(gm, -(-conc // gm), BM, BN, p.desc.K, 2)
            if best_ws is None or ws < best_ws:
                best, best_ws = gm, ws
            gm *= 2
        return best
    p = mg.gemm_plan(8192, 8192, 8192, "bf16", d_type="bf16")
    assert p.info().group_m == expect(p, 256, 256, 1) == 4
    p = mg.gemm_plan(2048, 2048, 512, "bf16")
    assert p.info().group_m == expect(p, 128, 128, 2) == 8
    p = mg.gemm_plan(128, 7168, 2048, "bf16", d_type="bf16")
    assert p.info().group_m == 1   # one tile row


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1, N=4, K=8), mg.ERR_INVALID_ARG),
    (dict(M=4, N=8, K=12), mg.ERR_UNSUPPORTED),
    (dict(M=4, N=8, K=16, lda=8), mg.ERR_INVALID_ARG),
    (dict(M=4, N=8, K=8, lda=12), mg.ERR_UNSUPPORTED),
    (dict(M=4, N=8, K=8, ldd=10), mg.ERR_UNSUPPORTED),
    (dict(M=4, N=8, K=8, a_type="f16", b_type="bf16"), mg.ERR_UNSUPPORTED),
    (dict(M=4, N=8, K=8, a_type="bf16", d_type="f16"), mg.ERR_UNSUPPORTED),
])
def test_plan_argument_errors(kw, status):
    args = dict(M=4, N=8, K=8, a_type="bf16")
    args.update(kw)
    with pytest.raises(mg.MgemmError) as e:
        mg.gemm_plan(**args)
    assert e.value.status == status
    assert mg.lib.gemm_last_error_message().decode()


def test_grouped_plan_errors():
    with pytest.raises(mg.MgemmError) as e:
        mg.grouped_gemm_plan(0, 10, 32, 32)
    assert e.value.status == mg.ERR_INVALID_ARG
    with pytest.raises(mg.MgemmError) as e:
        mg.grouped_gemm_plan(4, 10, 40, 32, epilogue=mg.EPI_SILU_GATE_I8)
    assert e.value.status == mg.ERR_UNSUPPORTED
    with pytest.raises(mg.MgemmError):
        mg.grouped_gemm_plan(4, 10, 32, 32, stride_b=8)


def test_null_arguments_rejected():
    assert mg.lib.gemm_plan(None, 0, None) == mg.ERR_INVALID_ARG
    assert mg.lib.gemm_run(None, None, None, None, None, 0, None) == mg.ERR_INVALID_ARG
    p = mg.gemm_plan(4, 8, 8, "bf16")
    assert mg.lib.gemm_run(p.handle, None, None, None, None, 0, None) == mg.ERR_INVALID_ARG
    assert mg.lib.gemm_status_string(mg.ERR_HIP) == b"MGEMM_ERR_HIP"


def test_e4m3_plan_rules():
    """E4M3 plans: k-contiguous A and B only, 16-element alignment, no split
    of K; the grouped form takes column-major expert weights and no
    epilogue, and no gathered rows.  The run calls check the plan type, the
    scale pointers and the gather before anything is launched (the fake
    device addresses below are never touched: the calls return first)."""
    fake = 1 << 20
    ok = mg.gemm_plan(512, 512, 256, a_type="e4m3", d_type="bf16", a_layout="row", b_layout="col")
    assert "e4m3 NT->bf16 tile=256x256dtl" in ok.describe() and "bk=128" in ok.describe()
    assert "splits=1" in ok.describe()
    for kw in [dict(b_layout="row"), dict(a_layout="col", lda=512), dict(K=264), dict(N=514),
               dict(flags=mg.PLAN_FORCE_TILE_128x128), dict(flags=mg.PLAN_SPLIT_K(4))]:
        args = dict(M=512, N=512, K=256, a_type="e4m3", d_type="bf16", a_layout="row", b_layout="col")
        args.update(kw)
        with pytest.raises(mg.MgemmError) as e:
            mg.gemm_plan(**args)
        assert e.value.status == mg.ERR_UNSUPPORTED, kw
    g = mg.grouped_gemm_plan(4, 256, 256, 256, a_type="e4m3", d_type="bf16", b_layout="col")
    assert "e4m3 NT->bf16" in g.describe() and "256x256dtl" in g.describe()
    for kw in [dict(b_layout="row"), dict(b_layout="col", epilogue=mg.EPI_SILU_GATE_I8),
               dict(b_layout="col", stride_b=256 * 256 + 8)]:
        with pytest.raises(mg.MgemmError) as e:
            mg.grouped_gemm_plan(4, 256, 256, 256, a_type="e4m3", d_type="bf16", **kw)
        assert e.value.status == mg.ERR_UNSUPPORTED, kw
    with pytest.raises(mg.MgemmError) as e:
        mg.grouped_gemm_run_scaled(g, fake, fake, fake, fake, fake, None, stream=0)
    assert e.value.status == mg.ERR_INVALID_ARG
    # the E4M3 grouped kernel reads A in place: a gathered run is refused
    with pytest.raises(mg.MgemmError) as e:
        mg.grouped_gemm_run_gather(g, fake, fake, fake, fake, fake, x_rows=64, stream=0)
    assert e.value.status == mg.ERR_UNSUPPORTED
    assert "E4M3" in mg.lib.gemm_last_error_message().decode()
    fake = 1 << 20
    with pytest.raises(mg.MgemmError) as e:
        mg.gemm_run_scaled(ok, fake, fake, fake, None, fake, stream=0)
    assert e.value.status == mg.ERR_INVALID_ARG
    bf = mg.gemm_plan(512, 512, 256, a_type="bf16", d_type="bf16")
    with pytest.raises(mg.MgemmError) as e:
        mg.gemm_run_scaled(bf, fake, fake, fake, fake, fake, stream=0)
    assert e.value.status == mg.ERR_UNSUPPORTED


def test_moe_fused_plan_rules():
    """The fused MoE plan: shape and alignment rules, its workspace formula
    (6400 bytes of schedule, then one int32 counter per possible row block:
    ceil(rows / 256) + experts), and the run call's checks before any
    launch (the fake device addresses are never touched)."""
    p = mg.moe_fused_plan(64, 32768, 7168, 2048)
    assert p.workspace_size() == (6400 + 4 * (128 + 64) + 255) // 256 * 256
    assert "moe_fused G=64" in p.describe() and "largest-first" in p.describe()
    assert p.info().grid == p.info().num_cus
    q = mg.moe_fused_plan(8, 384, 256, 128, dtype="f16")
    assert q.workspace_size() == (6400 + 4 * (2 + 8) + 255) // 256 * 256
    bad = [
        (dict(num_experts=0), mg.ERR_INVALID_ARG),
        (dict(num_experts=257), mg.ERR_UNSUPPORTED),
        (dict(hidden=0), mg.ERR_INVALID_ARG),
        (dict(hidden=264), mg.ERR_UNSUPPORTED),        # hidden % 16
        (dict(inter=96), mg.ERR_UNSUPPORTED),          # inter % 64
        (dict(ldh=160), mg.ERR_UNSUPPORTED),           # ldh % 64
        (dict(lda=200), mg.ERR_INVALID_ARG),           # lda < hidden
        (dict(ldw1=200), mg.ERR_INVALID_ARG),          # ldw1 < 2 inter
        (dict(stride_w1=8), mg.ERR_INVALID_ARG),
        (dict(dtype="f32"), mg.ERR_UNSUPPORTED),
        (dict(flags=mg.PLAN_FORCE_TILE_NARROW), mg.ERR_UNSUPPORTED),
    ]
    for kw, status in bad:
        args = dict(num_experts=8, max_total_rows=384, hidden=256, inter=128)
        args.update(kw)
        with pytest.raises(mg.MgemmError) as e:
            mg.moe_fused_plan(**args)
        assert e.value.status == status, kw
    fake = 1 << 20
    ws_n = q.workspace_size()
    # no workspace, a short one, a misaligned H, a non-MoE plan, a null pointer
    with pytest.raises(mg.MgemmError) as e:
        mg.moe_fused_run(q, fake, fake, fake, fake, fake, fake, workspace=None, stream=0)
    assert e.value.status == mg.ERR_WORKSPACE
    with pytest.raises(mg.MgemmError) as e:
        mg.moe_fused_run(q, fake, fake, fake, fake, fake, fake, workspace=fake, workspace_bytes=ws_n - 256,
                         stream=0)
    assert e.value.status == mg.ERR_WORKSPACE
    with pytest.raises(mg.MgemmError) as e:
        mg.moe_fused_run(q, fake, fake, fake, fake + 64, fake, fake, workspace=fake, workspace_bytes=ws_n,
                         stream=0)
    assert e.value.status == mg.ERR_UNSUPPORTED
    with pytest.raises(mg.MgemmError) as e:
        mg.moe_fused_run(mg.gemm_plan(4, 8, 8, "bf16"), fake, fake, fake, fake, fake, fake, workspace=fake,
                         workspace_bytes=ws_n, stream=0)
    assert e.value.status == mg.ERR_INVALID_ARG
    with pytest.raises(mg.MgemmError) as e:
        mg.moe_fused_run(q, fake, fake, None, fake, fake, fake, workspace=fake, workspace_bytes=ws_n, stream=0)
    assert e.value.status == mg.ERR_INVALID_ARG
    with pytest.raises(mg.MgemmError) as e:
        mg.moe_fused_run(q, fake, fake, fake, fake, fake, fake, workspace=fake, workspace_bytes=ws_n,
                         row_index=fake, x_rows=1 << 23, stream=0)
    assert e.value.status == mg.ERR_INVALID_ARG
    # no rows: nothing to do, nothing touched
    mg.moe_fused_run(mg.moe_fused_plan(8, 0, 256, 128), fake, fake, fake, fake, fake, fake, workspace=None,
                     stream=0)


def test_weighted_run_rules():
    """grouped_gemm_run_weighted: only SiLU-gate plans, a non-null 4-byte
    aligned weight array; refused before anything is launched (the fake
    device addresses are never touched)."""
    fake = 1 << 20
    plain = mg.grouped_gemm_plan(4, 256, 256, 256)
    with pytest.raises(mg.MgemmError) as e:
        mg.grouped_gemm_run_weighted(plain, fake, fake, fake, fake, fake, stream=0)
    assert e.value.status == mg.ERR_UNSUPPORTED and "SiLU" in str(e.value)
    gated = mg.grouped_gemm_plan(4, 256, 256, 256, epilogue=mg.EPI_SILU_GATE_I8)
    for w in (None, fake + 2):
        with pytest.raises(mg.MgemmError) as e:
            mg.grouped_gemm_run_weighted(gated, fake, fake, fake, fake, w, stream=0)
        assert e.value.status == mg.ERR_INVALID_ARG, w


def test_fused_weighted_run_rules():
    """moe_fused_run_weighted: a non-null 4-byte aligned weight array, checked
    before anything else runs (the fake device addresses are never touched)."""
    fake = 1 << 20
    plan = mg.moe_fused_plan(8, 384, 256, 128)
    for w in (None, fake + 2):
        with pytest.raises(mg.MgemmError) as e:
            mg.moe_fused_run_weighted(plan, fake, fake, fake, fake, fake, fake, w, workspace=fake,
                                      workspace_bytes=1 << 20, stream=0)
        assert e.value.status == mg.ERR_INVALID_ARG and "weight" in str(e.value), w


def test_grouped_blockscaled_run_rules():
    """grouped_gemm_run_blockscaled refuses, before any launch: a non-E4M3
    plan; scale pitches below ceil(K/128), an expert stride below
    ceil(N/128) x lds_b (INVALID_ARG); an odd pitch (UNSUPPORTED)."""
    fake = 1 << 20

    def run(plan, lds_a, lds_b, stride_sb):
        st = mg.lib.grouped_gemm_run_blockscaled(plan.handle, fake, fake, fake, fake, fake, lds_a, fake, lds_b,
                                                 stride_sb, None, 0, None)
        return st, mg.lib.gemm_last_error_message().decode()

    st, msg = run(mg.grouped_gemm_plan(4, 256, 256, 512), 4, 4, 8)
    assert st == mg.ERR_UNSUPPORTED and "E4M3" in msg
    p = mg.grouped_gemm_plan(4, 256, 256, 512, a_type="e4m3", d_type="f32", b_layout="col")   # 4 k blocks, 2 column blocks
    for lds_a, lds_b, stride in ((2, 4, 8), (4, 2, 8), (4, 4, 7), (0, 4, 8)):
        st, msg = run(p, lds_a, lds_b, stride)
        assert st == mg.ERR_INVALID_ARG, (lds_a, lds_b, stride, msg)
    st, msg = run(p, 5, 4, 8)
    assert st == mg.ERR_UNSUPPORTED and "even" in msg


def test_quantize_rules():
    """mgemm_quantize_e4m3_block refuses, before any launch: odd cols or
    pitches, a misaligned X (UNSUPPORTED); short pitches, null pointers, a
    16-bit type other than BF16 / F16 (INVALID_ARG / UNSUPPORTED)."""
    fake = 1 << 20

    def run(X, rows, cols, ldx, t, Q, ldq, S, lds):
        st = mg.lib.mgemm_quantize_e4m3_block(X, rows, cols, ldx, t, Q, ldq, S, lds, None)
        return st, mg.lib.gemm_last_error_message().decode()

    assert run(fake, 4, 255, 256, mg.BF16, fake, 256, fake, 2)[0] == mg.ERR_UNSUPPORTED
    assert run(fake + 2, 4, 256, 256, mg.BF16, fake, 256, fake, 2)[0] == mg.ERR_UNSUPPORTED
    assert run(fake, 4, 256, 256, mg.F32, fake, 256, fake, 2)[0] == mg.ERR_UNSUPPORTED
    for args in ((fake, 4, 256, 200, mg.BF16, fake, 256, fake, 2), (fake, 4, 256, 256, mg.BF16, fake, 256, fake, 1),
                 (None, 4, 256, 256, mg.F16, fake, 256, fake, 2), (fake, -1, 256, 256, mg.F16, fake, 256, fake, 2)):
        assert run(*args)[0] == mg.ERR_INVALID_ARG, args
    assert run(None, 0, 256, 256, mg.BF16, None, 256, None, 2)[0] == mg.OK
