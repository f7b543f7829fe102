#!/usr/bin/env python3
"""Benchmark of the MI355X MoE-layer hot path: one step = route -> dispatch -> expert MLP -> combine
over one batch of synthetic tokens, inputs resident in HBM, on one GPU.

Prints ONE JSON line: MoE-layer tokens/s (whole step), per-stage times, dispatch+combine GB/s against
the HBM peak, the roofline of the dominant stage (the expert-MLP grouped GEMM) and the CPU oracle timed
on a bounded sample of the same workload.

The K timed steps carry HIP events at every step boundary (per-step times: median and p90) and around the
expert-MLP call (its average duration gives the roofline); route, dispatch and combine are timed in a second,
instrumented pass of K steps, because every event record costs GPU time between kernels.

  python bench.py [--gpus 1] [--steps 32] [--warmup 16] [--workload large-skewed-prefill]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 MI355X; dispatch+combine GB/s and % HBM peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3
DEFAULT_WORKLOAD = "large-skewed-prefill"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default=None,
                    help="workload name, or its position (1-5) in moe_workloads.WORKLOADS "
                         "(default: large-skewed-prefill)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--fused-combine", action="store_true",
                    help="fuse the combine into the expert MLP's down GEMM (moe_expert_mlp_combine): the tile "
                         "that completes a token's column band combines it at once")
    ap.add_argument("--sender-accumulate", action="store_true",
                    help="combine with sender-side partial accumulation (moe_combine_send + moe_combine_recv): "
                         "one partial row per (destination rank, token) instead of one row per kept pair")
    ap.add_argument("--fp8-dispatch", action="store_true",
                    help="dispatch fp8 block-scaled rows (E4M3 codes, one power-of-two scale per 128 hidden "
                         "elements) and run the expert MLP on them; combine stays bf16 (bf16 workloads only)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times), the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters, and exit")
    ap.add_argument("--calibrate-gemm", action="store_true",
                    help="only time the vendor library's bf16 batched GEMM (hipBLASLt through torch.bmm, contiguous "
                         "operands) on the workload's expert-GEMM shapes and on an 8192^3 GEMM, and exit: the "
                         "practical MFMA ceiling of this machine, for context")
    return ap.parse_args()


MLP_SOURCES = ("combine_router_gemm_amd/csrc/mlp.hip", "combine_router_gemm_amd/csrc/common.h")


def mlp_source_digest() -> str:
    """sha256 over the expert-MLP kernel sources: counters taken on other sources no longer apply."""
    import hashlib
    h = hashlib.sha256()
    for rel in MLP_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per moe_expert_mlp call from the committed counter summary of this workload, or None
    if there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"expert_mlp_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                key, _, val = line[2:].partition(":")
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != mlp_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(mib: int) -> None:
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device-to-device copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": 3}), flush=True)


def calibrate_gemm(cfg, reps: int = 20) -> None:
    """Vendor-library reference: hipBLASLt bf16 GEMMs (torch.bmm / torch.mm, contiguous operands) with the
    shapes of the workload's two expert GEMMs, El experts x (capacity rows per local expert), without the
    row gather, the fused SwiGLU and the row scatter the expert MLP does."""
    import torch
    import moe_workloads as W

    dev = torch.device("cuda:0")
    C = W.capacity(cfg, cfg.T)
    M = max(1, W.rows_max(cfg.T, cfg.k, cfg.E, C) // cfg.El)
    El, H, F = cfg.El, cfg.H, cfg.F

    def timed(fn, flops, case):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        print(json.dumps({"calibration": "vendor bf16 GEMM", "case": case, "us": round(us, 1),
                          "TFLOP/s": round(flops / us / 1e6, 1),
                          "frac_of_peak": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}), flush=True)

    bf = torch.bfloat16
    a = torch.randn(El, M, H, device=dev, dtype=bf)
    wgu = torch.randn(El, H, 2 * F, device=dev, dtype=bf)
    h = torch.randn(El, M, F, device=dev, dtype=bf)
    wdn = torch.randn(El, F, H, device=dev, dtype=bf)
    o1 = torch.empty(El, M, 2 * F, device=dev, dtype=bf)
    o2 = torch.empty(El, M, H, device=dev, dtype=bf)
    timed(lambda: torch.bmm(a, wgu, out=o1), 2 * El * M * H * 2 * F, f"{cfg.name} gate/up {El}x[{M}x{H}]x[{H}x{2 * F}]")
    timed(lambda: torch.bmm(h, wdn, out=o2), 2 * El * M * F * H, f"{cfg.name} down {El}x[{M}x{F}]x[{F}x{H}]")
    del a, wgu, h, wdn, o1, o2
    x = torch.randn(8192, 8192, device=dev, dtype=bf)
    y = torch.randn(8192, 8192, device=dev, dtype=bf)
    timed(lambda: torch.mm(x, y), 2 * 8192 ** 3, "square 8192^3")


def pick_workload(name):
    import moe_workloads as W
    if name is None:
        return W.workload(DEFAULT_WORKLOAD)
    names = list(W.WORKLOADS)
    if name in W.WORKLOADS:
        return W.WORKLOADS[name]
    if name.isdigit() and 1 <= int(name) <= len(names):   # position in the listing, from 1
        return W.WORKLOADS[names[int(name) - 1]]
    raise SystemExit(f"unknown workload {name!r}; choose from {names}")


def algorithmic_bytes(cfg, C, counts, s, fp8=False, sender=False):
    """Bytes each stage must move (what the method needs, not what the kernels happen to move).

    fp8: the send rows are one byte per element plus a 4-byte scale per 128 elements.
    sender: combine writes one partial row per (rank, token) and reads it back, on top of the kept rows
    and the output."""
    T, H, E, k, F, El = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.El
    q = (H + 4 * (H // 128)) if fp8 else H * s       # bytes of one send row
    kept = counts["kept"]
    touched = counts["tokens_touched"]
    active_local = counts["active_local"]
    bias = 0 if counts["bias_stride"] is None else (E * 4 if counts["bias_stride"] == 0 else T * E * 4)
    route = T * H * s + E * H * 4 + bias + T * E * 4 + T * k * 8
    dispatch = touched * H * s + kept * q + kept * 8 + 2 * T * k * 4 + E * 16
    combine = kept * H * s + T * k * 8 + T * H * s
    if sender:
        combine += 2 * counts["partial_rows"] * H * s + T * k * 4
    mlp = active_local * 3 * H * F * s + kept * q + kept * H * s
    return dict(route=route, dispatch=dispatch, combine=combine, mlp=mlp,
                route_flops=2 * T * E * H, mlp_flops=6 * H * F * kept)


def cpu_baseline(cfg, inp_dev, fp8=False, min_seconds=10.0, max_seconds=30.0, max_mlp_experts=32):
    """Time the CPU oracle (as it stands) on the same workload, stage by stage.

    Route, dispatch and combine run on the whole batch, so the capacity, the drops and the rows are the
    workload's own. The expert MLP runs on every row of a sample of local experts (at most
    max_mlp_experts, evenly spaced; one expert's weights on the host at a time) and its time is scaled to
    all active local experts by the mean time per sampled expert. Combine reads the dispatched rows in
    place of expert outputs (its cost does not depend on the values). The whole sequence repeats until
    about min_seconds of measured oracle work (never past max_seconds)."""
    import numpy as np
    import torch

    import moe_workloads as W
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001 - report the affinity if the BLAS pool cannot be queried
        threads = len(os.sched_getaffinity(0))

    def host(t):
        if t is None:
            return None
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    T, E, k, R, El = cfg.T, cfg.E, cfg.k, cfg.R, cfg.El
    dt = cfg.dtype
    x = host(inp_dev["x"])
    bias = host(inp_dev["bias"])
    wr = host(inp_dev["w_router"])
    C = W.capacity(cfg, T)
    stages = {"route": 0.0, "dispatch": 0.0, "expert_mlp": 0.0, "combine": 0.0}
    runs, total, work = 0, 0.0, 0.0  # estimated layer seconds; measured oracle seconds
    while runs == 0 or (work < min_seconds and work * (runs + 1) / runs <= max_seconds):
        t0 = time.perf_counter()
        logits = oracle.router_logits(x, dt, wr, bias)
        ids, w = oracle.topk_softmax(logits, k)
        t1 = time.perf_counter()
        if fp8:
            lay, codes, scales = oracle.fp8.dispatch_fp8(x, ids, E, C, R)
        else:
            lay, sb = oracle.dispatch(x, dt, ids, E, C, R)
        t2 = time.perf_counter()
        rex = oracle.row_experts(lay.expert_offset, E)
        local = rex % El
        active = np.unique(local)
        picks = active[np.unique(np.linspace(0, len(active) - 1, min(max_mlp_experts, len(active))).round().astype(int))] \
            if len(active) else active
        mlp_s, mlp_rows = 0.0, 0
        for l in picks:
            rows = np.nonzero(local == l)[0]
            wgu = {int(l): host(inp_dev["w_gate_up"][int(l)])}
            wdn = {int(l): host(inp_dev["w_down"][int(l)])}
            a = oracle.fp8.dequantize_rows_bf16(codes[rows], scales[rows]) if fp8 else sb[rows]
            tm = time.perf_counter()
            oracle.expert_mlp(a, dt, rex[rows], El, wgu, wdn, cfg.F)
            mlp_s += time.perf_counter() - tm
            mlp_rows += len(rows)
            del wgu, wdn
        mlp_est = mlp_s * len(active) / max(len(picks), 1)
        t3 = time.perf_counter()
        stand_in = oracle.fp8.dequantize_rows_bf16(codes, scales) if fp8 else sb
        oracle.combine(stand_in, dt, lay.pair_row, w)
        t4 = time.perf_counter()
        stages["route"] += t1 - t0
        stages["dispatch"] += t2 - t1
        stages["expert_mlp"] += mlp_est
        stages["combine"] += t4 - t3
        total += (t1 - t0) + (t2 - t1) + mlp_est + (t4 - t3)
        work += (t1 - t0) + (t2 - t1) + mlp_s + (t4 - t3)
        runs += 1
    what = " with fp8 dispatch" if fp8 else ""
    sample = (f"the whole {cfg.name} batch ({T} tokens, capacity {C}, {lay.total} kept rows){what}: route, dispatch "
              f"and combine on every token; the expert MLP on all {mlp_rows} rows of {len(picks)} of the "
              f"{len(active)} active local experts (evenly spaced), scaled by the mean time per expert; "
              f"{runs} run{'s' if runs > 1 else ''}, {work:.1f} s of oracle work")
    return dict(value=T * runs / total, unit="tokens/s", cores=int(threads), kind="oracle", sample=sample,
                seconds_per_layer=round(total / runs, 3), oracle_seconds=round(work, 2),
                stages_s={n: round(v / runs, 3) for n, v in stages.items()}, runs=runs,
                mlp_sample={"experts": int(len(picks)), "rows": int(mlp_rows), "active_local_experts": int(len(active))})


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no collectives or "
              f"multi-GPU path; the single-GPU figure is the per-GPU share.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    if args.calibrate_gemm:
        import torch
        cfg = pick_workload(args.workload)
        torch.cuda.set_device(0)
        calibrate_gemm(cfg)
        return

    import torch

    import combine_router_gemm_amd as moe
    import moe_workloads as W

    cfg = pick_workload(args.workload)
    torch.cuda.set_device(0)
    moe.load_library()
    dev = torch.device("cuda:0")
    print(f"[bench] {W.describe(cfg)} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    inp = W.make_inputs(cfg, device=dev)
    T, H, E, k, R, F = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.F
    C = inp["C"]
    x = inp["x"]
    s = x.element_size()
    fp8 = args.fp8_dispatch
    sender = args.sender_accumulate
    fused = args.fused_combine
    if fused and (sender or fp8):
        raise SystemExit("--fused-combine runs the bf16/fp32 expert MLP with the receiver-side combine only")
    if fp8 and (x.dtype != torch.bfloat16 or H % moe.MOE_FP8_BLOCK):
        raise SystemExit(f"--fp8-dispatch needs bf16 activations and H % {moe.MOE_FP8_BLOCK} == 0")

    # every buffer and workspace is allocated once, outside the timed region
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    L = moe.Layout(T, k, E, R, C, H, device=dev)
    send_buf = torch.empty(L.rows_max, H, dtype=x.dtype, device=dev)
    out_buf = torch.empty_like(send_buf)
    if fp8:
        send_q = torch.empty(L.rows_max, H, dtype=torch.uint8, device=dev)
        send_scale = torch.empty(L.rows_max, H // moe.MOE_FP8_BLOCK, dtype=torch.float32, device=dev)
    y = torch.empty(T, H, dtype=x.dtype, device=dev)
    partial = torch.empty(R, T, H, dtype=x.dtype, device=dev) if sender else None
    xdt = moe.MOE_BF16 if x.dtype == torch.bfloat16 else moe.MOE_F32
    ws_route = torch.empty(max(1, moe.moe_route_workspace_bytes(T, H, E, xdt)), dtype=torch.uint8, device=dev)
    ws_disp = torch.empty(max(1, moe.moe_dispatch_workspace_bytes(T, k, E)), dtype=torch.uint8, device=dev)
    ws_mlp = torch.empty(max(1, moe.moe_expert_mlp_combine_workspace_bytes(T, k, E, R, C, H, F, xdt) if fused else
                             moe.moe_expert_mlp_workspace_bytes(T, k, E, R, C, F, xdt)), dtype=torch.uint8,
                         device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None, mlp_ev=None):
        """One step. ev: five events bracketing the four stages; mlp_ev: two events around the MLP only."""
        if ev is not None:
            ev[0].record(stream)
        moe.moe_route(x, inp["w_router"], inp["bias"], k, logits, ids, wts, workspace=ws_route)
        if ev is not None:
            ev[1].record(stream)
        if fp8:
            moe.moe_dispatch_fp8(x, ids, L, send_q, send_scale, workspace=ws_disp)
        else:
            moe.moe_dispatch(x, ids, L, send_buf, workspace=ws_disp)
        if ev is not None:
            ev[2].record(stream)
        if mlp_ev is not None:
            mlp_ev[0].record(stream)
        if fp8:
            moe.moe_expert_mlp_fp8(send_q, send_scale, L, inp["w_gate_up"], inp["w_down"], out_buf, workspace=ws_mlp)
        elif fused:
            moe.moe_expert_mlp_combine(send_buf, L, inp["w_gate_up"], inp["w_down"], wts, out_buf, y, workspace=ws_mlp)
        else:
            moe.moe_expert_mlp(send_buf, L, inp["w_gate_up"], inp["w_down"], out_buf, workspace=ws_mlp)
        if ev is not None:
            ev[3].record(stream)
        if mlp_ev is not None:
            mlp_ev[1].record(stream)
        if sender:
            moe.moe_combine_send(out_buf, L, wts, partial)
            moe.moe_combine_recv(partial, L, y)
        elif not fused:
            moe.moe_combine(out_buf, L, wts, y)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, bracketed by device synchronisation. Only the dominant stage (the
    # expert MLP) is bracketed by events here (each event record costs a few microseconds of GPU time
    # between kernels); the other stages are timed in a separate instrumented pass below.
    mlp_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    step_events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_events[i].record(stream)
        step(mlp_ev=mlp_events[i])
    step_events[args.steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mlp_us_timed = 1e3 * sum(ev[0].elapsed_time(ev[1]) for ev in mlp_events) / args.steps
    ms_per_step = 1e3 * wall / args.steps
    step_ms = sorted(step_events[i].elapsed_time(step_events[i + 1]) for i in range(args.steps))

    def pct(q):
        """q-quantile of the per-step times (linear interpolation)."""
        pos = q * (len(step_ms) - 1)
        lo = int(pos)
        hi = min(lo + 1, len(step_ms) - 1)
        return step_ms[lo] + (step_ms[hi] - step_ms[lo]) * (pos - lo)

    # instrumented pass (not part of the headline): every stage bracketed by events
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    stage = {"route": 0.0, "dispatch": 0.0, "expert_mlp": 0.0, "combine": 0.0}
    names = list(stage)
    for ev in events:
        for j, n in enumerate(names):
            stage[n] += ev[j].elapsed_time(ev[j + 1])
    stage_us = {n: 1e3 * v / args.steps for n, v in stage.items()}
    gpu_step_us = sum(stage_us.values())

    # routing outcome of the (deterministic) step, read back after the timed region
    kept = int(L.expert_kept.sum().item())
    kept_per_e = L.expert_kept.cpu()
    active_local = int((kept_per_e.view(R, cfg.El).sum(0) > 0).sum().item())
    pr = L.pair_row.cpu()
    touched = int((pr >= 0).any(dim=1).sum().item())
    # rows a combine exchange would carry back: one per kept pair, or one per (rank, token) with partials
    seg = L.expert_offset.cpu()[torch.arange(R + 1) * cfg.El]
    rank_of = torch.searchsorted(seg, pr.clamp(min=0).contiguous(), right=True) - 1
    rk = torch.where(pr >= 0, rank_of, torch.full_like(rank_of, -1)).sort(dim=1).values
    partial_rows = int((rk[:, :1] >= 0).sum().item() + ((rk[:, 1:] != rk[:, :-1]) & (rk[:, 1:] >= 0)).sum().item())
    counts = dict(kept=kept, tokens_touched=touched, active_local=active_local, partial_rows=partial_rows,
                  bias_stride=None if inp["bias"] is None else inp["bias_stride"])
    ab = algorithmic_bytes(cfg, C, counts, s, fp8, sender)
    if fused:  # the combine's bytes move inside the expert-MLP call
        ab["mlp"] += ab["combine"]

    mlp_s = mlp_us_timed * 1e-6
    mlp_ai = ab["mlp_flops"] / max(ab["mlp"], 1)
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if s == 2 else MFMA_F32_PEAK_TFLOPS
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mlp_ai >= ridge:
        achieved = ab["mlp_flops"] / mlp_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=mfma_peak, unit="TFLOP/s",
                    frac=round(achieved / mfma_peak, 4), traffic=None)
    else:
        achieved = ab["mlp"] / mlp_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None)
    roof["traffic"] = None if (fp8 or fused) else measured_traffic(cfg.name)
    roof["kernel"] = ("moe_expert_mlp_fp8" if fp8 else ("moe_expert_mlp_combine" if fused else "moe_expert_mlp")) + \
        (" (grouped GEMM: counter clear + gate/up + down-with-combine launches" if fused else
         " (grouped GEMM: gate/up + down launches") + \
        ", after a tile-plan launch when there are several ranks or the tiles are direct-to-LDS)"
    roof["algorithmic_bytes"] = ab["mlp"]
    roof["algorithmic_flops"] = ab["mlp_flops"]

    dc_s = (stage_us["dispatch"] + (0.0 if fused else stage_us["combine"])) * 1e-6
    dc_gbs = (ab["dispatch"] + (0 if fused else ab["combine"])) / dc_s / 1e9
    tokens_per_s = T / (ms_per_step * 1e-3)
    # the router's roofline: its fp32 dot products run as three exact bf16 products each on the matrix
    # cores, so its bound is the larger of its bytes at the HBM peak and 3 x its flops at the bf16 (or, for
    # fp32 activations, 1 x at the fp32) matrix peak
    route_s = stage_us["route"] * 1e-6
    route_mfma_flops = ab["route_flops"] * (3 if s == 2 else 1)
    route_bound_s = max(ab["route"] / (HBM_PEAK_GBS * 1e9), route_mfma_flops / (mfma_peak * 1e12))
    route_roof = {"TFLOP/s": round(ab["route_flops"] / route_s / 1e12, 3),
                  "GB/s": round(ab["route"] / route_s / 1e9, 1),
                  "bound": "mfma" if route_mfma_flops / (mfma_peak * 1e12) >= ab["route"] / (HBM_PEAK_GBS * 1e9)
                  else "hbm",
                  "roofline_us": round(route_bound_s * 1e6, 2),
                  "frac": round(route_bound_s / route_s, 4),
                  "frac_of_fp32_peak": round(ab["route_flops"] / route_s / 1e12 / MFMA_F32_PEAK_TFLOPS, 4)}

    def hbm_stage(name):
        gbs = ab[name] / (stage_us[name] * 1e-6) / 1e9
        return {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": ab[name]}

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(pct(0.5), 4), "p90": round(pct(0.9), 4), "min": round(step_ms[0], 4),
                    "max": round(step_ms[-1], 4), "source": "HIP events at every step boundary of the timed steps"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "experts": E, "top_k": k, "ffn": F,
                   "dest_ranks": R, "capacity": C, "routing": cfg.routing, "act_dtype": cfg.dtype,
                   "dispatch_payload": "fp8-e4m3-block128" if fp8 else cfg.dtype,
                   "combine": "sender-side partials" if sender else
                   ("fused into the down GEMM" if fused else "receiver-side")},
        "roofline": roof,
        "expert_mlp_us_timed": round(mlp_us_timed, 2),
        "stages_us": {n: round(v, 2) for n, v in stage_us.items()},
        "gpu_step_us_events": round(gpu_step_us, 2),
        "dispatch_combine": {"GB/s": round(dc_gbs, 1), "frac_hbm_peak": round(dc_gbs / HBM_PEAK_GBS, 4),
                             "bytes": ab["dispatch"] + (0 if fused else ab["combine"]),
                             "stages": "dispatch only (the combine runs inside the expert MLP)" if fused else
                             "dispatch + combine"},
        "route": route_roof,
        "dispatch": hbm_stage("dispatch"),
        "combine": None if fused else hbm_stage("combine"),
        "effective_assignments_per_s": round(kept / (ms_per_step * 1e-3), 1),
        "routing": {"kept_pairs": kept, "pairs": T * k, "dropped_pairs": T * k - kept,
                    "active_local_experts": active_local},
        "combine_link_rows": {"receiver_side": kept, "sender_side": partial_rows,
                              "bytes_per_row": H * s},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, inp, fp8)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
