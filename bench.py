"""Throughput of the MI355X GEMM library on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over the workload's inputs, which are
resident in HBM before timing starts: for a dense workload one gemm_run, for
the MoE workload FC1 (SiLU-gated) plus FC2 over all experts.

Timing protocol ("B200 的 2CTA 怎样调优" section 十: warm up separately,
repeat, report the spread; hot and rotating input buffers):
  * warm-up: at least W untimed steps, and at least WARMUP_SECONDS of them.
    The engine clock idles low and takes tens of milliseconds of load to
    settle (1.7-2.0 GHz under sustained MFMA load), so five steps of 8192^3
    (4 ms) would time the clock's ramp, not the kernel; the line reports
    the W asked for and the steps actually run;
  * then exactly K steps, bracketed by device synchronisation, split into
    (up to) ten windows by events recorded on the stream the kernels are
    launched on: the value is K steps over the whole bracket, the windows
    give median / min / max per step;
  * the engine and memory clocks and the board power are sampled from
    sysfs while the timed steps run (and once before the warm-up), and the
    clock-adjusted MFMA peak is reported beside the nominal 2.4 GHz one;
  * workloads whose operands fit the 256 MB MALL (the decode shape) are also
    timed over rotating copies of their buffers (more bytes than the MALL
    holds), so every step reads its weights from HBM.

Prints one JSON line: the metric (TFLOPS of algorithmic work, 2*M*N*K per
GEMM, no padding), the roofline of the dominant kernel against MI355X's
dense MFMA peak, and the CPU oracle timed on a bounded sample of the same
workload (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense MFMA peak for 16-bit inputs: 256 CUs x 2.4 GHz x 4096 FLOP per
# clock per CU = 2516.6 TFLOP/s (AMD's "2.5 PFLOP/s" dense bf16/fp16 figure).
PEAK_TFLOPS = {"bf16": 256 * 2.4e9 * 4096 / 1e12, "f16": 256 * 2.4e9 * 4096 / 1e12,
               # E4M3 inputs: twice the FLOP per clock (AMD's "5.0 PFLOP/s" dense fp8 figure)
               "e4m3": 256 * 2.4e9 * 8192 / 1e12}
HBM_GBPS = 8000.0
METRIC = "GEMM TFLOPS and % of MI355X bf16 dense peak at 4096^3/8192^3 (1 GPU)"
DEFAULT_WORKLOAD = "gemm8192_bf16_bcol"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: as many as fill WARMUP_SECONDS, at least 10)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the second square size the metric is quoted at (4096^3 next to 8192^3) "
                         "and the E4M3 8192^3 line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 256 MiB device copy (the reference kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args()


# the kernels and the planner that picks their launch (tile, grid, tile order):
# a change to any of them makes stored traffic counts stale
KERNEL_SOURCES = ["bf16_gemm_amd/csrc/engine.hpp", "bf16_gemm_amd/csrc/kernels.hpp",
                  "bf16_gemm_amd/csrc/narrow.hpp", "bf16_gemm_amd/csrc/moe_fused.hpp",
                  "bf16_gemm_amd/csrc/tile_tables.hpp", "bf16_gemm_amd/csrc/plan.cpp"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments dropped and runs of white
    space collapsed, so that an edit of the comments alone keeps the recorded
    counters valid."""
    import hashlib
    import re
    tok = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        code = tok.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(workload: str):
    """HBM-side bytes per step (the step's kernels once each) measured with
    rocprofv3 (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on
    a plain copy), read from the workload's summary under profiles/; None
    unless that summary was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("source_hash", "traffic_bytes_per_step"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_hash") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_step"])
    except (KeyError, ValueError):
        return None


def calibrate_copy():
    import torch
    x = torch.empty(256 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4,
                      "launches": 3}), flush=True)


def dev16(torch, bits, dt):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(
        torch.bfloat16 if dt == "bf16" else torch.float16)


def dense_case(torch, mg, datagen, name, copies=1):
    """The workload's step; with copies > 1 a list of steps, one per copy of
    A, B and D (the rotating-buffer regime)."""
    cfg = datagen.DENSE[name]
    a, b = datagen.gemm_inputs(cfg, "random")
    A, B = dev16(torch, a, cfg.in_dtype), dev16(torch, b, cfg.in_dtype)
    out = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[cfg.out_dtype]
    plan = mg.gemm_plan(cfg.M, cfg.N, cfg.K, cfg.in_dtype, d_type=cfg.out_dtype, a_layout=cfg.a_layout,
                        b_layout=cfg.b_layout)
    ws = mg.workspace_for(plan)      # split-K scratch, allocated before timing
    sets = [(A, B, torch.empty((cfg.M, cfg.N), dtype=out, device="cuda"))]
    for _ in range(copies - 1):
        sets.append((A.clone(), B.clone(), torch.empty((cfg.M, cfg.N), dtype=out, device="cuda")))

    def make(Ai, Bi, Di):
        return lambda: mg.gemm_run(plan, Ai, Bi, Di, workspace=ws)
    step = make(*sets[0]) if copies == 1 else [make(*x) for x in sets]

    esz = 4 if cfg.out_dtype == "f32" else 2
    inf = plan.info()
    info = dict(flops=cfg.flops, bytes=2 * (cfg.M * cfg.K + cfg.K * cfg.N) + esz * cfg.M * cfg.N,
                plan=plan.describe(), dtype=cfg.in_dtype,
                config={"workload": name, "M": cfg.M, "N": cfg.N, "K": cfg.K, "in": cfg.in_dtype,
                        "out": cfg.out_dtype, "a_layout": cfg.a_layout, "b_layout": cfg.b_layout},
                launches_per_step=1 + (inf.splits > 1) + (cfg.N % 4 != 0))
    return step, info, (cfg, a, b)


def moe_case(torch, mg, datagen):
    cfg = datagen.MOE["moe64"]
    r, A, W1, W2 = datagen.moe_inputs_device(cfg, "cuda")
    rows = int(r.offsets[-1])
    H, I, E = cfg.hidden, cfg.inter, cfg.num_experts
    offs = torch.from_numpy(r.offsets).cuda()
    h = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    p1 = mg.grouped_gemm_plan(E, rows, 2 * I, H, stride_b=H * 2 * I, epilogue=mg.EPI_SILU_GATE_I8)
    p2 = mg.grouped_gemm_plan(E, rows, H, I, stride_b=I * H)

    def step():
        mg.grouped_gemm_run(p1, A, W1, h, offs)
        mg.grouped_gemm_run(p2, h, W2, y, offs)

    flops = 2.0 * rows * (2 * I) * H + 2.0 * rows * H * I
    active = int((r.counts > 0).sum())
    wbytes = active * (H * 2 * I + I * H) * 2
    abytes = rows * H * 2 + rows * I * 2 * 2 + rows * H * 2
    info = dict(flops=flops, bytes=wbytes + abytes, plan=p1.describe() + " | " + p2.describe(), dtype="bf16",
                config={"workload": "moe64", "experts": E, "hidden": H, "inter": I, "tokens": cfg.num_tokens,
                        "top_k": cfg.top_k, "routed_rows": rows, "active_experts": active},
                launches_per_step=len(p1.describe().split("grid=")) - 1 + len(p2.describe().split("grid=")) - 1)
    return step, info, None


def moe_fused_case(torch, mg, datagen):
    """The 64-expert layer's FC1 (SiLU gate) and FC2 in one persistent
    launch (moe_fused_run), on the same inputs as the moe64 workload."""
    cfg = datagen.MOE["moe64"]
    r, A, W1, W2 = datagen.moe_inputs_device(cfg, "cuda")
    rows = int(r.offsets[-1])
    H, I, E = cfg.hidden, cfg.inter, cfg.num_experts
    offs = torch.from_numpy(r.offsets).cuda()
    h = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    plan = mg.moe_fused_plan(E, rows, H, I)
    ws = mg.workspace_for(plan)

    def step():
        mg.moe_fused_run(plan, A, W1, W2, h, y, offs, workspace=ws)

    flops = 2.0 * rows * (2 * I) * H + 2.0 * rows * H * I
    active = int((r.counts > 0).sum())
    wbytes = active * (H * 2 * I + I * H) * 2
    abytes = rows * H * 2 + rows * I * 2 * 2 + rows * H * 2
    info = dict(flops=flops, bytes=wbytes + abytes, plan=plan.describe(), dtype="bf16",
                config={"workload": "moe64_fused", "experts": E, "hidden": H, "inter": I,
                        "tokens": cfg.num_tokens, "top_k": cfg.top_k, "routed_rows": rows,
                        "active_experts": active},
                launches_per_step=2)
    return step, info, None


def moe_layer_case(torch, mg, datagen, fold=False, fused=False):
    """The whole 64-expert layer: FC1 reading the routed rows of X through
    the routing's row index (the dispatch fused into its A loads), FC2, and
    the weighted top-k combine into each token's output row.  fold: the
    routing weights multiplied into FC1's SiLU-gate epilogue instead
    (p(hW2) = (ph)W2), the combine a plain sum.  fused: FC1 and FC2 in the
    one persistent launch (moe_fused_run / moe_fused_run_weighted)."""
    import numpy as np
    cfg = datagen.MOE["moe64"]
    r, A, W1, W2 = datagen.moe_inputs_device(cfg, "cuda")
    rows = int(r.offsets[-1])
    H, I, E, T = cfg.hidden, cfg.inter, cfg.num_experts, cfg.num_tokens
    first = np.full(T, -1, dtype=np.int64)
    first[r.token_of_row[::-1]] = np.arange(rows)[::-1]   # a routed row of each token
    X = A[torch.from_numpy(first).cuda()].contiguous()    # the token rows the dispatch reads
    del A
    offs = torch.from_numpy(r.offsets).cuda()
    idx = torch.from_numpy(r.token_of_row.astype(np.int32)).cuda()
    pos = torch.from_numpy(r.pos).cuda()
    wts = torch.from_numpy(r.weight).cuda()
    h = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    p1 = mg.grouped_gemm_plan(E, rows, 2 * I, H, stride_b=H * 2 * I, epilogue=mg.EPI_SILU_GATE_I8)
    p2 = mg.grouped_gemm_plan(E, rows, H, I, stride_b=I * H)
    w_row = np.empty(rows, dtype=np.float32)
    w_row[r.pos] = r.weight                               # each routed row's routing weight
    w_row = torch.from_numpy(w_row).cuda()
    pf = mg.moe_fused_plan(E, rows, H, I) if fused else None
    ws = mg.workspace_for(pf) if fused else None

    def step_fused():
        mg.moe_fused_run(pf, X, W1, W2, h, z, offs, workspace=ws, row_index=idx, x_rows=T)
        mg.moe_combine(z, pos, wts, y, cfg.top_k)

    def step_fused_fold():
        mg.moe_fused_run_weighted(pf, X, W1, W2, h, z, offs, w_row, workspace=ws, row_index=idx, x_rows=T)
        mg.moe_combine(z, pos, None, y, cfg.top_k)

    def step():
        mg.grouped_gemm_run_gather(p1, X, W1, h, offs, idx)
        mg.grouped_gemm_run(p2, h, W2, z, offs)
        mg.moe_combine(z, pos, wts, y, cfg.top_k)

    def step_fold():
        mg.grouped_gemm_run_weighted(p1, X, W1, h, offs, w_row, row_index=idx)
        mg.grouped_gemm_run(p2, h, W2, z, offs)
        mg.moe_combine(z, pos, None, y, cfg.top_k)

    flops = 2.0 * rows * (2 * I) * H + 2.0 * rows * H * I
    active = int((r.counts > 0).sum())
    wbytes = active * (H * 2 * I + I * H) * 2
    abytes = T * H * 2 + rows * I * 2 * 2 + rows * H * 2 * 2 + T * H * 2
    name = "moe64_layer" + ("_fused" if fused else "") + ("_fold" if fold else "")
    stages = ("gathered FC1 (SiLU gate x routing weight) + FC2 + plain top-k sum" if fold else
              "gathered FC1 (SiLU gate) + FC2 + weighted top-k combine")
    if fused:
        plan, launches = pf.describe() + " | combine", 3
        stages += ", FC1 and FC2 in one persistent launch"
    else:
        plan = p1.describe() + " | " + p2.describe() + " | combine"
        launches = len(p1.describe().split("grid=")) - 1 + len(p2.describe().split("grid=")) - 1 + 1
    info = dict(flops=flops, bytes=wbytes + abytes, plan=plan, dtype="bf16",
                config={"workload": name, "experts": E, "hidden": H,
                        "inter": I, "tokens": T, "top_k": cfg.top_k, "routed_rows": rows, "active_experts": active,
                        "stages": stages},
                launches_per_step=launches)
    steps = {(False, False): step, (True, False): step_fold, (False, True): step_fused,
             (True, True): step_fused_fold}
    return steps[(fold, fused)], info, None


# E4M3 workloads: per-tensor scales, B column-major, bf16 out
E4M3 = {"gemm8192_e4m3": (8192, 8192, 8192), "gemm8192_e4m3_block": (8192, 8192, 8192)}


def e4m3_case(torch, mg, datagen, name):
    import numpy as np
    M, N, K = E4M3[name]
    rs = np.random.RandomState(8192)
    # normal(0, 100) codes: a per-tensor-quantised tensor whose largest
    # magnitudes (4.5 sigma) reach the format's 448; the scales undo the 100
    a = datagen.matrix_e4m3((M, K), ("normal", 100.0), rs)
    b = datagen.matrix_e4m3((N, K), ("normal", 100.0), rs)
    A, B = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    sa = torch.tensor([0.01], dtype=torch.float32, device="cuda")
    sb = torch.tensor([0.01], dtype=torch.float32, device="cuda")
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    plan = mg.gemm_plan(M, N, K, "e4m3", d_type="bf16", a_layout="row", b_layout="col")
    block = name.endswith("_block")
    if block:
        # E8M0 block scales 2^-9 .. 2^-5 (one per row and 128-k block, one
        # per 128 x 128 weight block)
        kb = -(-K // 128)
        bsa = torch.from_numpy(rs.randint(118, 123, size=(M, kb + (kb & 1))).astype(np.uint8)).cuda()
        bsb = torch.from_numpy(rs.randint(118, 123, size=(-(-N // 128), kb + (kb & 1))).astype(np.uint8)).cuda()

        def step():
            mg.gemm_run_blockscaled(plan, A, B, D, bsa, bsb)
    else:
        def step():
            mg.gemm_run_scaled(plan, A, B, D, sa, sb)

    scale_bytes = (M + -(-N // 128)) * -(-K // 128) if block else 8
    info = dict(flops=2.0 * M * N * K, bytes=M * K + N * K + 2 * M * N + scale_bytes, plan=plan.describe(),
                dtype="e4m3",
                config={"workload": name, "M": M, "N": N, "K": K, "in": "e4m3", "out": "bf16",
                        "a_layout": "row", "b_layout": "col",
                        "scales": "E8M0 per (row, 128-k) and per 128x128 weight block" if block else "per-tensor"},
                launches_per_step=1)
    return step, info, ("e4m3", M, N, K, a, b)


def cpu_baseline_e4m3(case, target_s):
    import oracle
    _, M, N, K, a, b = case

    def timed(R):
        t0 = time.perf_counter()
        oracle.gemm_e4m3_ref(a[:R], b, 0.01, 0.01)
        return time.perf_counter() - t0
    r1, r2 = 4, 36
    t1, t2 = timed(r1), timed(r2)
    per_row = max((t2 - t1) / (r2 - r1), 1e-6)
    R2 = int(min(M, max(r2, (target_s - max(t1 - r1 * per_row, 0.0)) / per_row)))
    t = timed(R2)
    return {"value": 2.0 * R2 * N * K / t / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"first {R2} of {M} output rows (all {N} columns, full K={K}), {t:.1f} s incl. operand decode"}


def cpu_baseline(case, target_s):
    """The oracle, as it stands, on the first R rows of the same product."""
    import numpy as np

    import oracle
    if case is None:
        return None
    if case[0] == "e4m3":
        return cpu_baseline_e4m3(case, target_s)
    cfg, a, b = case
    a_rows = (lambda R: a[:R]) if cfg.a_layout == "row" else (lambda R: np.ascontiguousarray(a[:, :R]))
    # two calibration runs give the fixed cost (decoding B) and the per-row
    # cost; the timed run then covers about target_s seconds
    def timed(R):
        t0 = time.perf_counter()
        oracle.gemm_ref(a_rows(R), b, cfg.in_dtype, cfg.in_dtype, cfg.a_layout, cfg.b_layout)
        return time.perf_counter() - t0
    r1, r2 = 4, 36
    t1, t2 = timed(r1), timed(r2)
    per_row = max((t2 - t1) / (r2 - r1), 1e-6)
    R2 = int(min(cfg.M, max(r2, (target_s - max(t1 - r1 * per_row, 0.0)) / per_row)))
    t0 = time.perf_counter()
    oracle.gemm_ref(a_rows(R2), b, cfg.in_dtype, cfg.in_dtype, cfg.a_layout, cfg.b_layout)
    t = time.perf_counter() - t0
    flops = 2.0 * R2 * cfg.N * cfg.K
    return {"value": flops / t / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"first {R2} of {cfg.M} output rows (all {cfg.N} columns, full K={cfg.K}), "
                      f"{t:.1f} s incl. operand decode"}


# Last-level (MALL) cache of MI355X: a workload whose bytes fit in it is
# also timed over enough rotating copies of its buffers to exceed it.
MALL_BYTES = 256 << 20


def sub_line(info, t, tflops, peak, roof, pct_key="pct_of_peak"):
    return {"config": info["config"], "value": round(tflops, 2), "unit": "TFLOPS", "ms_per_step": round(t["ms"], 5),
            pct_key: round(100 * tflops / peak, 2), "windows": window_stats(t),
            "clocks": clock_report(t, tflops, info["dtype"]), "roofline": roof}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not "
              "supported by this benchmark", file=sys.stderr)
        sys.exit(2)
    import torch

    import bf16_gemm_amd as mg
    import datagen
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.workload == "moe64":
        step, info, case = moe_case(torch, mg, datagen)
    elif args.workload == "moe64_fused":
        step, info, case = moe_fused_case(torch, mg, datagen)
    elif args.workload in ("moe64_layer", "moe64_layer_fold", "moe64_layer_fused", "moe64_layer_fused_fold"):
        step, info, case = moe_layer_case(torch, mg, datagen, fold=args.workload.endswith("_fold"),
                                          fused="_fused" in args.workload)
    elif args.workload in E4M3:
        step, info, case = e4m3_case(torch, mg, datagen, args.workload)
    else:
        step, info, case = dense_case(torch, mg, datagen, args.workload)
    print(f"# plan: {info['plan']}", file=sys.stderr, flush=True)
    t = time_steps(torch, step, args.steps, args.warmup)
    roof, tflops, peak = roofline(info, t["ms"])
    hot = None
    if args.workload in datagen.DENSE and info["bytes"] < MALL_BYTES:
        # every step's buffers fit the MALL: the line's value is the
        # rotating regime (each step reads its own copy, from HBM), the hot
        # one is reported beside it
        del step
        copies = -(-(MALL_BYTES * 5 // 4) // info["bytes"])
        hot = sub_line(info, t, tflops, peak, roof)
        hot["regime"] = "hot (one set of buffers, MALL-resident)"
        step, info, _ = dense_case(torch, mg, datagen, args.workload, copies=copies)
        info["config"] = dict(info["config"], buffers=f"rotating x{copies}")
        print(f"# rotating over {copies} copies of A, B, D", file=sys.stderr, flush=True)
        t = time_steps(torch, step, args.steps, args.warmup)
        roof, tflops, peak = roofline(info, t["ms"])
    secondary = []
    e4m3_line = e4m3_block_line = None
    if args.workload == DEFAULT_WORKLOAD and not args.no_secondary:
        # the metric is quoted at 4096^3 as well: same timing, reported beside
        del step
        step2, info2, _ = dense_case(torch, mg, datagen, "gemm4096_bf16")
        print(f"# plan: {info2['plan']}", file=sys.stderr, flush=True)
        t2 = time_steps(torch, step2, args.steps, args.warmup)
        roof2, tflops2, peak2 = roofline(info2, t2["ms"])
        secondary.append(sub_line(info2, t2, tflops2, peak2, roof2))
        # the E4M3 product of the same size (per-tensor scales), priced
        # against the fp8 dense peak: reported beside, not the metric
        del step2
        step3, info3, _ = e4m3_case(torch, mg, datagen, "gemm8192_e4m3")
        print(f"# plan: {info3['plan']}", file=sys.stderr, flush=True)
        t3 = time_steps(torch, step3, args.steps, args.warmup)
        roof3, tflops3, peak3 = roofline(info3, t3["ms"])
        e4m3_line = sub_line(info3, t3, tflops3, peak3, roof3, "pct_of_fp8_peak")
        del step3
        # the same product with E8M0 block scales (the blockwise FP8 path)
        step4, info4, _ = e4m3_case(torch, mg, datagen, "gemm8192_e4m3_block")
        print(f"# plan: {info4['plan']} (block scales)", file=sys.stderr, flush=True)
        t4 = time_steps(torch, step4, args.steps, args.warmup)
        roof4, tflops4, peak4 = roofline(info4, t4["ms"])
        e4m3_block_line = sub_line(info4, t4, tflops4, peak4, roof4, "pct_of_fp8_peak")
        del step4
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, args.cpu_seconds)
    line = {"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
            "warmup": t["warmup_asked"], "ms_per_step": round(t["ms"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": info["dtype"], "data": "synthetic",
            "config": info["config"], "pct_of_peak": round(100 * tflops / peak, 2),
            "roofline": roof, "cpu_baseline": cpu,
            "warmup_run": {"steps": t["warmup_run"], "seconds": round(t["warmup_s"], 3),
                           "rule": f"at least --warmup steps and at least {WARMUP_SECONDS} s"},
            "windows": window_stats(t), "clocks": clock_report(t, tflops, info["dtype"]),
            "versions": versions(torch)}
    if hot:
        line["hot"] = hot
    if secondary:
        line["also"] = secondary
    if e4m3_line:
        line["e4m3"] = e4m3_line
        line["e4m3_block"] = e4m3_block_line
    print(json.dumps(line), flush=True)


def versions(torch):
    v = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            v["rocm"] = f.read().strip()
    except OSError:
        pass
    return v


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# MI355X's clocks take tens of milliseconds of load to settle: 4096^3 runs
# at ~121 us per step after 10 warmup steps and ~98 us after 400 (8192^3:
# 793 against 768 us after 100).  The untimed steps therefore fill at least
# this much time, and number at least --warmup (default 10).
WARMUP_SECONDS = 0.25
WINDOWS = 10


class ClockSampler:
    """Engine (sclk) and memory (mclk) clocks read from the GPU's sysfs
    performance-level files every ~2 ms in a background thread (the level
    marked current), and the board power the driver's hwmon reports
    (power1_input, else power1_average, in microwatts); None where the files
    are not visible."""

    def __init__(self):
        self.card = self._find_card()
        self.power_file = self._find_power(self.card)
        self.samples = []
        self._stop = None
        self._thread = None

    @staticmethod
    def _find_power(card):
        import glob
        if not card:
            return None
        for name in ("power1_input", "power1_average"):
            hits = sorted(glob.glob(os.path.join(card, "hwmon", "hwmon*", name)))
            if hits:
                return hits[0]
        return None

    def read_power_w(self):
        if not self.power_file:
            return None
        try:
            with open(self.power_file) as f:
                return int(f.read().strip()) / 1e6
        except (OSError, ValueError):
            return None

    @staticmethod
    def _find_card():
        import glob
        cards = sorted(os.path.dirname(p) for p in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if len(cards) == 1:
            return cards[0]
        try:   # several visible: the one on torch's device 0's PCI bus
            import torch
            bus = torch.cuda.get_device_properties(0).pci_bus_id
            for c in cards:
                slot = os.path.basename(os.path.realpath(c))   # e.g. 0000:75:00.0
                if int(slot.split(":")[1], 16) == bus:
                    return c
        except Exception:
            pass
        return None

    @staticmethod
    def _current_mhz(path):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        return float(line.split(":")[1].strip().split("Mhz")[0].strip("( )"))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def read(self):
        if not self.card:
            return None, None
        return (self._current_mhz(os.path.join(self.card, "pp_dpm_sclk")),
                self._current_mhz(os.path.join(self.card, "pp_dpm_mclk")))

    def start(self):
        import threading
        if not self.card:
            return self
        self.samples = []
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                sc, mc = self.read()
                if sc is not None:
                    self.samples.append((sc, mc, self.read_power_w()))
                self._stop.wait(0.002)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        if self._thread:
            self._stop.set()
            self._thread.join()
        return self

    def summary(self):
        if not self.samples:
            return None
        sc = sorted(x[0] for x in self.samples)
        mc = sorted(x[1] for x in self.samples if x[1] is not None)
        pw = sorted(x[2] for x in self.samples if x[2] is not None)
        return {"sclk_mhz": {"median": sc[len(sc) // 2], "min": sc[0], "max": sc[-1]},
                "mclk_mhz": mc[len(mc) // 2] if mc else None, "samples": len(sc),
                "power_w": {"median": pw[len(pw) // 2], "min": pw[0], "max": pw[-1]} if pw else None}


def time_steps(torch, step, steps, warmup):
    """Warm up, then time exactly `steps` steps (see the module docstring).
    `step` is a callable, or a list of callables run in rotation (one per
    copy of the buffers).  Returns a dict: ms (per step over the whole
    bracket), windows (per-step ms of each window), warmup_asked,
    warmup_run, warmup_s, clocks."""
    fns = step if isinstance(step, (list, tuple)) else [step]
    clk = ClockSampler()
    idle = clk.read()
    idle_w = clk.read_power_w()
    asked = 10 if warmup is None else warmup
    n, t0 = 0, time.perf_counter()
    t_end = t0 + WARMUP_SECONDS
    while n < asked or time.perf_counter() < t_end:
        fns[n % len(fns)]()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0
    stream = torch.cuda.current_stream()     # the stream every launch goes to
    nwin = min(WINDOWS, steps)
    bounds = [round(i * steps / nwin) for i in range(nwin + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nwin + 1)]
    clk.start()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for w in range(nwin):
        for i in range(bounds[w], bounds[w + 1]):
            fns[i % len(fns)]()
        ev[w + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clk.stop()
    ms = ev[0].elapsed_time(ev[nwin]) / steps
    win = [ev[w].elapsed_time(ev[w + 1]) / (bounds[w + 1] - bounds[w]) for w in range(nwin)]
    clocks = clk.summary()
    if clocks is not None:
        clocks["idle_before_mhz"] = {"sclk": idle[0], "mclk": idle[1]}
        clocks["idle_before_w"] = idle_w
    ws = sorted(win)
    print(f"# {steps} steps in {nwin} windows after {n} warmup steps ({warm_s:.2f} s): {ms * 1e3:.1f} us/step "
          f"(events; windows median {ws[len(ws) // 2] * 1e3:.1f}, min {ws[0] * 1e3:.1f}, max {ws[-1] * 1e3:.1f}), "
          f"wall {wall * 1e6 / steps:.1f} us/step; clocks {clocks}", file=sys.stderr, flush=True)
    return {"ms": ms, "windows": win, "warmup_asked": asked, "warmup_run": n, "warmup_s": warm_s,
            "clocks": clocks}


def window_stats(t):
    ws = sorted(t["windows"])
    return {"n": len(ws), "median_ms": round(ws[len(ws) // 2], 5), "min_ms": round(ws[0], 5),
            "max_ms": round(ws[-1], 5)}


def clock_report(t, tflops, dtype):
    """Clocks seen while the timed steps ran, and the MFMA peak at that
    engine clock (the nominal peak scaled by sclk / 2400 MHz)."""
    c = t["clocks"]
    if not c:
        return None
    out = dict(c)
    sclk = c["sclk_mhz"]["median"]
    if sclk:
        adj = PEAK_TFLOPS[dtype] * sclk / 2400.0
        out["adjusted_peak_tflops"] = round(adj, 1)
        out["frac_of_adjusted_peak"] = round(tflops / adj, 4)
    return out


def roofline(info, ms):
    tflops = info["flops"] / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[info["dtype"]]
    # the bound is the one the algorithmic intensity falls under: below the
    # ridge (peak FLOP/s over 8 TB/s, ~315 FLOP/B) a step is HBM-bound
    gbps = info["bytes"] / (ms * 1e-3) / 1e9
    hbm_bound = info["flops"] / info["bytes"] < peak * 1e12 / (HBM_GBPS * 1e9)
    roof = {"bound": "hbm" if hbm_bound else "mfma",
            "achieved": round(gbps, 1) if hbm_bound else round(tflops, 2),
            "peak": HBM_GBPS if hbm_bound else round(peak, 1),
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round(gbps / HBM_GBPS, 4) if hbm_bound else round(tflops / peak, 4),
            "traffic": profiled_traffic(info["config"]["workload"]),
            "kernel": info["plan"], "launches_per_step": info["launches_per_step"],
            "algorithmic_bytes_per_step": info["bytes"],
            "algorithmic_flops_per_step": info["flops"],
            "achieved_hbm_gbps_algorithmic": round(gbps, 1),
            "kernel_source_hash": kernel_source_hash()}
    return roof, tflops, peak


if __name__ == "__main__":
    main()
