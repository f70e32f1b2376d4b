"""Benchmark of the MoE FFN layer forward pass on one MI355X.

One step = one moe_forward call (router, permute, grouped SwiGLU FFN,
combine) over one batch of the Mixtral-8x7B-shaped workload (T=4096,
d_model=4096, E=8, top-2, d_ff=14336, bf16 with fp32 accumulation, router in
fp32), inputs resident in HBM.  Prints one JSON line.  After the headline
workload the other workloads run in the same process (`configs`: each one's
step time, grouped-FFN roofline fraction and stage rates).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-configs]
                    [--no-cpu-baseline] [--cpu-sample-tokens N]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 E4M3 expert weights with per-expert scales "
                         "(moe_forward_scaled) instead of bf16 weights")
    ap.add_argument("--router-stats", action="store_true",
                    help="also time moe_forward_stats (router statistics "
                         "computed in the routing step) against moe_forward")
    ap.add_argument("--shared-dff", type=int, default=0,
                    help="add a shared expert of this hidden size (the "
                         "DeepSeek-V3 layer form; moe_forward_shared)")
    ap.add_argument("--backward", action="store_true",
                    help="also time the training step (moe_forward_train + "
                         "moe_backward) and report the backward's GEMM rate")
    ap.add_argument("--library-loop", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the vendor-library form of the same FFN on "
                         "the same permuted rows: one hipBLASLt GEMM per expert "
                         "and projection (torch.nn.functional.linear) plus the "
                         "SwiGLU in torch; context for the grouped FFN only")
    ap.add_argument("--sample-power", action=argparse.BooleanOptionalAction, default=True,
                    help="also run the grouped FFN back to back for a few "
                         "seconds while amd-smi samples socket power and the "
                         "graphics clock; reports the MFMA peak at that clock")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the step captured once in a HIP graph and "
                         "replayed (the library allocates and synchronises "
                         "nothing, so a whole layer call can be captured)")
    ap.add_argument("--configs", action=argparse.BooleanOptionalAction, default=True,
                    help="after the headline workload, run every other workload "
                         "in the same process and report each one's step time, "
                         "grouped-FFN roofline fraction and stage rates (the "
                         "`configs` object)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def _calibrate_copy():
    """A plain device-to-device copy of 1 GiB, three times: the counter
    reference for HBM traffic (each copy reads and writes 1 GiB)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                      "bytes_written_per_copy": n, "copies": 3}), flush=True)


def _traffic(workload):
    """HBM traffic per grouped-FFN launch from the committed counter summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated), or None when there is
    none for this workload or the GEMM source changed since it was taken."""
    import hashlib
    f = os.path.join(ROOT, "profiles", f"grouped_ffn_{workload}_traffic.md")
    src = os.path.join(ROOT, "mixture_experts_layer_wavefront_amd", "csrc",
                       "grouped_gemm.hip")
    if not os.path.exists(f):
        return None
    vals = {}
    for line in open(f):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if vals.get("source_sha256") != sha:
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _time_loop(fn, steps, stream):
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(steps):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / steps  # ms per call


def _route_tflops(T, d, E, t_route_ms, x_bf16):
    tf = 2.0 * T * d * E / (t_route_ms * 1e-3) / 1e12
    if x_bf16:
        return {"route_logits": tf, "route_units": "bf16 mfma, three planes",
                "route_frac": 3.0 * tf / 2500.0}
    return {"route_logits": tf, "route_units": "fp32 vector fma", "route_frac": tf / 157.3}


def _progress(msg):
    """One line per finished stage on stderr (the JSON line stays alone on
    stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _graph_time(step, n, stream):
    """The step captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed n times; ms per replay, event-timed on the given stream."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ms = _time_loop(g.replay, n, stream)
    del g
    return ms


def _smi_sample():
    """One amd-smi reading: (socket power in W, mean graphics clock over the
    XCDs in MHz), or None where amd-smi is missing or prints no such field."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"],
                           capture_output=True, text=True, timeout=10)
        js = json.loads(r.stdout)
    except Exception:
        return None
    gpu = js[0] if isinstance(js, list) else js.get("gpu_data", [js])[0]
    try:
        watts = float(gpu["power"]["socket_power"]["value"])
        clk = [float(v["clk"]["value"]) for k, v in gpu["clock"].items()
               if k.startswith("gfx_") and isinstance(v, dict)
               and isinstance(v.get("clk"), dict) and v["clk"].get("value") not in (None, "N/A")]
    except (KeyError, TypeError, ValueError):
        return None
    return watts, (sum(clk) / len(clk) if clk else None)


def _sample_power(fn, flops, stream, secs=4.0):
    """Runs fn back to back for about `secs` seconds while a thread samples
    amd-smi every 0.2 s; reports the medians (the first two samples, taken
    while the clock ramps, are dropped), the event-timed rate and the bf16
    MFMA peak scaled to the sampled clock (the 2.5 PFLOP/s figure is quoted
    at 2400 MHz)."""
    import threading
    import torch
    samples, done = [], threading.Event()

    def sampler():
        while not done.is_set():
            v = _smi_sample()
            if v is not None:
                samples.append(v)
            done.wait(0.2)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    t0, n = time.perf_counter(), 0
    s.record(stream)
    while time.perf_counter() - t0 < secs:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    e.record(stream)
    e.synchronize()
    done.set()
    th.join()
    ms = s.elapsed_time(e) / n
    tflops = flops / (ms * 1e-3) / 1e12
    kept = samples[2:] or samples
    if not kept:
        return {"ms_per_call": ms, "tflops": tflops, "samples": 0}
    med = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731
    watts = med([w for w, _ in kept])
    clks = [c for _, c in kept if c is not None]
    clk = med(clks) if clks else None
    out = {"ms_per_call": ms, "tflops": tflops, "samples": len(kept),
           "socket_power_w": watts, "gfx_clock_mhz": clk}
    if clk:
        peak = PEAK_BF16_TFLOPS * clk / 2400.0
        out.update(mfma_peak_at_clock_tflops=peak, frac_at_clock=tflops / peak)
    return out


def _library_loop(wl, dev, perm, n, stream, flops, fns_only=False):
    """The grouped FFN's work done the plain way on the same permuted rows:
    per expert, one hipBLASLt GEMM for gate|up (the two weights stacked), the
    SwiGLU in torch, one GEMM for the down projection (bf16 out).  Expert
    boundaries are read to the host before timing.  Also the two GEMMs alone
    (down projection on a fixed H), the library's best case."""
    import torch
    import torch.nn.functional as F
    o = perm["offsets"].cpu().tolist()
    Xp, Wd, dff = perm["X_perm"], dev["W_down"], wl.d_ff
    if Xp is None:  # the forward's permute copies no rows: gather them here
        Xp = dev["X"].index_select(0, perm["row_token"][:o[-1]].long())
    Wgu = torch.cat([dev["W_gate"], dev["W_up"]], dim=1).contiguous()
    Hf = torch.empty((o[-1], dff), dtype=torch.bfloat16, device="cuda").normal_(0.0, 0.05)
    live = [e for e in range(wl.E) if o[e + 1] > o[e]]

    def ffn_loop():
        for e in live:
            gu = F.linear(Xp[o[e]:o[e + 1]], Wgu[e])
            F.linear(F.silu(gu[:, :dff]) * gu[:, dff:], Wd[e])

    def gemms_only():
        for e in live:
            F.linear(Xp[o[e]:o[e + 1]], Wgu[e])
            F.linear(Hf[o[e]:o[e + 1]], Wd[e])
    if fns_only:
        return gemms_only
    for _ in range(2):
        ffn_loop()
        gemms_only()
    t_loop = _time_loop(ffn_loop, n, stream)
    t_gemm = _time_loop(gemms_only, n, stream)
    del Wgu, Hf
    return {"what": "per-expert hipBLASLt GEMMs (torch.nn.functional.linear) on "
                    "the same permuted rows",
            "ms_ffn_loop": t_loop, "ms_gemms_only": t_gemm,
            "gemms_only_tflops": flops / (t_gemm * 1e-3) / 1e12}


def _cpu_baseline(wl, dev, ntok, min_s=10.0, max_s=30.0, shared=None, fp8_scales=None):
    """The CPU oracle (as it stands) on the first `ntok` tokens of the same
    batch with the same weights, repeated until at least `min_s` seconds of
    CPU work (stopping before `max_s`); returns the dict for the JSON line."""
    import torch
    from threadpoolctl import threadpool_info

    import oracle as O

    host = {k: (None if v is None else
                (v.cpu().numpy() if v.dtype == torch.uint8 else v.float().cpu().numpy()))
            for k, v in dev.items()}
    ntok = min(ntok, wl.T)
    X = host["X"][:ntok]
    cf = float(np.float32(wl.capacity_factor))
    runs, total = 0, 0.0
    while total < min_s:
        t0 = time.perf_counter()
        if fp8_scales is not None:
            O.moe_forward_fp8(X, host["W_r"], host["bias"], host["W_gate"], host["W_up"],
                              host["W_down"], fp8_scales, wl.top_k,
                              cf if cf > 0 else None, wl.gating)
        elif shared is None:
            O.moe_forward(X, host["W_r"], host["bias"], host["W_gate"], host["W_up"],
                          host["W_down"], wl.top_k, cf if cf > 0 else None, wl.gating)
        else:
            O.moe_forward_shared(X, host["W_r"], host["bias"], host["W_gate"],
                                 host["W_up"], host["W_down"], *shared, wl.top_k,
                                 cf if cf > 0 else None, wl.gating)
        dt = time.perf_counter() - t0
        runs += 1
        total += dt
        if total + dt > max_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": ntok * runs / total, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "host_cpus": os.cpu_count(), "cpu_model": model,
            "sample": f"first {ntok} of the {wl.T} tokens, all {wl.E} experts "
                      f"(full weights{', plus the shared expert' if shared is not None else ''}), "
                      f"fp64 NumPy per-expert loop, {runs} run(s), {total:.1f} s wall"}


def _layer_bytes(wl, N, active, a_b, w_b, gather):
    """Algorithmic HBM bytes of each stage (inputs read once, outputs written
    once): route reads X and W_r and writes ids and weights; the permute reads
    the ids and writes the index maps, and without `gather` also reads X and
    writes X_perm; the FFN reads the active experts' weights and each kept
    copy's input row (of X_perm, or gathered from X) and writes Y_perm
    (fp32); the combine reads Y_perm, the dest rows and weights and writes the
    fp32 output."""
    T, d, E, k, dff = wl.T, wl.d_model, wl.E, wl.top_k, wl.d_ff
    return {"route": T * d * a_b + E * d * 4 + T * k * 8,
            "permute": (0 if gather else T * d * a_b + N * d * a_b) + T * k * 24 + N * 4,
            "grouped_ffn": 3 * active * d * dff * w_b + N * d * a_b + N * d * 4,
            "combine": N * d * 4 + T * d * 4 + T * k * 8}


def _run_layer(wl, steps, warmup, fp8=False):
    """Inputs of workload `wl` on the device, `warmup` untimed then `steps`
    timed moe_forward calls (two events around them, one after each), then
    each stage through its own entry point.  Returns a dict of the timings,
    the routing outcome and the objects the optional extras reuse."""
    import torch

    import mixture_experts_layer_wavefront_amd as M
    from mixture_experts_layer_wavefront_amd import workloads as W

    w_scales = None
    if fp8:
        d8 = W.make_device_fp8(wl, "cuda")
        dev = dict(X=d8["X"], W_r=d8["W_r"], bias=d8["bias"], W_gate=d8["Q_gate"],
                   W_up=d8["Q_up"], W_down=d8["Q_down"])
        w_scales = d8["scales"]
    else:
        dev = W.make_device(wl, "cuda")
    p = M.problem(wl.T, wl.d_model, wl.E, wl.top_k, wl.d_ff,
                  wl.capacity_factor, wl.dtype, wl.gating, "f32",
                  w_dtype="fp8" if fp8 else None)
    ws = torch.empty(M.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.T, wl.d_model), dtype=torch.float32, device="cuda")
    stats = torch.empty(2 * wl.E + 2, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    a = (dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"])

    def step():
        if fp8:
            M.moe_forward_scaled(p, *a, w_scales, out=out, stats=stats, workspace=ws)
        else:
            M.moe_forward(p, *a, out=out, stats=stats, workspace=ws)

    for _ in range(warmup):
        step()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        step()
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = stats.cpu().numpy()
    N = int(st[2 * wl.E])                       # kept token copies
    counts = st[:wl.E]
    active = int(np.count_nonzero(st[wl.E + 1:2 * wl.E + 1] - st[wl.E:2 * wl.E]))

    # ---- per stage (same kernels, called through the stage entry points) ----
    # bf16 activations: the forward's permute copies no rows and its grouped
    # FFN reads them from X through row_token (moe_grouped_ffn_rows)
    gather = wl.dtype == W.BF16
    idx, w = M.moe_route(p, dev["X"], dev["W_r"], dev["bias"])
    perm = M.moe_permute(p, dev["X"], idx, copy_rows=not gather)
    if gather:
        ffn = lambda Yo=None, w=None: M.moe_grouped_ffn_rows(  # noqa: E731
            p, dev["X"], perm["row_token"], perm["offsets"], dev["W_gate"], dev["W_up"],
            dev["W_down"], Yo, w, w_scales=w_scales)
    else:
        ffn = lambda Yo=None, w=None: M.moe_grouped_ffn(  # noqa: E731
            p, perm["X_perm"], perm["offsets"], dev["W_gate"], dev["W_up"],
            dev["W_down"], Yo, w)
    Y = ffn()
    o2 = M.moe_combine(p, Y, perm["dest_row"], w)
    ffn_ws = torch.empty(M.grouped_ffn_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    perm_ws = torch.empty(M.permute_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    n = max(steps, 5)
    t_route = _time_loop(lambda: M.moe_route(p, dev["X"], dev["W_r"], dev["bias"], idx, w),
                         n, stream)
    t_perm = _time_loop(lambda: M.moe_permute(p, dev["X"], idx, perm_ws, out=perm), n, stream)
    t_ffn = _time_loop(lambda: ffn(Y, ffn_ws), n, stream)
    t_comb = _time_loop(lambda: M.moe_combine(p, Y, perm["dest_row"], w, o2), n, stream)
    torch.cuda.synchronize()

    a_b = 2 if wl.dtype == W.BF16 else 4
    w_b = 1 if fp8 else a_b
    by = _layer_bytes(wl, N, active, a_b, w_b, gather)
    ffn_flops = 6.0 * N * wl.d_model * wl.d_ff
    return dict(wl=wl, p=p, dev=dev, a=a, ws=ws, out=out, stats=stats, stream=stream,
                step=step, w_scales=w_scales, ms=ms, per_step=per_step, wall=wall, st=st,
                N=N, counts=counts, active=active, idx=idx, w=w, perm=perm, ffn=ffn, Y=Y,
                ffn_ws=ffn_ws, n=n, bytes=by, ffn_flops=ffn_flops,
                stages_ms={"route": t_route, "permute": t_perm, "grouped_ffn": t_ffn,
                           "combine": t_comb})


def _ffn_roofline(r):
    """The grouped FFN launch against its binding roofline: MFMA when its
    algorithmic flops per algorithmic HBM byte reach the machine balance (bf16
    MFMA peak / HBM peak), else HBM."""
    t_ffn = r["stages_ms"]["grouped_ffn"]
    flops, by = r["ffn_flops"], r["bytes"]["grouped_ffn"]
    if flops / by >= PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
        tf = flops / (t_ffn * 1e-3) / 1e12
        return dict(bound="mfma", achieved=tf, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=tf / PEAK_BF16_TFLOPS)
    gbs = by / (t_ffn * 1e6)
    return dict(bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s",
                frac=gbs / PEAK_HBM_GBS)


def _workload_text(wl):
    return (f"{wl.name}: one MoE FFN layer forward, T={wl.T}, d_model={wl.d_model}, "
            f"E={wl.E}, top-{wl.top_k}, SwiGLU d_ff={wl.d_ff}, {wl.dtype} "
            f"weights/activations, fp32 router and accumulation, fp32 output"
            + (f", capacity factor {wl.capacity_factor}" if wl.capacity_factor > 0 else "")
            + (f", Zipf({wl.zipf_s}) router bias" if wl.zipf_s > 0 else ""))


def _config_summary(r):
    """One workload's figures for the `configs` object of the JSON line."""
    from mixture_experts_layer_wavefront_amd import workloads as W
    wl, sm, by = r["wl"], r["stages_ms"], r["bytes"]
    step_bytes = sum(by.values())
    ffn = _ffn_roofline(r)
    return {
        "workload": _workload_text(wl),
        "ms_per_step": r["ms"], "ms_per_step_median": r["per_step"][len(r["per_step"]) // 2],
        "ms_per_step_min": r["per_step"][0],
        "tokens_per_s": wl.T / (r["ms"] * 1e-3),
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_frac": step_bytes / (r["ms"] * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "ffn": dict(ffn, ms=sm["grouped_ffn"], flops=r["ffn_flops"],
                    bytes=by["grouped_ffn"]),
        "stages_ms": sm,
        "stages_gbs": {k: by[k] / (sm[k] * 1e6) for k in ("route", "permute", "combine")},
        "routing": {"kept_copies": r["N"], "dropped": int(r["st"][-1]),
                    "active_experts": r["active"],
                    "max_over_mean_load": float(r["counts"].max() /
                                                max(r["counts"].mean(), 1e-9))},
    }


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the whole MoE layer runs on a single "
              "MI355X; multi-GPU runs are not supported (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        _calibrate_copy()
        return

    import mixture_experts_layer_wavefront_amd as M
    from mixture_experts_layer_wavefront_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.fp8 and (args.shared_dff or args.router_stats):
        sys.exit("--fp8 combines with neither --shared-dff nor --router-stats")
    r = _run_layer(wl, args.steps, args.warmup, fp8=args.fp8)
    _progress(f"{wl.name}: {r['ms']:.3f} ms per step")
    p, dev, a, ws, out, stats, stream = (r[k] for k in ("p", "dev", "a", "ws", "out",
                                                          "stats", "stream"))
    step, ms, per_step, n, N = r["step"], r["ms"], r["per_step"], r["n"], r["N"]
    ffn, Y, ffn_ws, perm, w_scales = r["ffn"], r["Y"], r["ffn_ws"], r["perm"], r["w_scales"]
    T, d, E, k, dff = wl.T, wl.d_model, wl.E, wl.top_k, wl.d_ff
    ffn_flops, by = r["ffn_flops"], r["bytes"]
    t_route = r["stages_ms"]["route"]

    roofline = dict(_ffn_roofline(r),
                    kernel="grouped SwiGLU FFN (gate/up GEMM + SwiGLU epilogue, down GEMM)",
                    traffic=None if args.fp8 else _traffic(args.workload),
                    flops_per_launch=ffn_flops, bytes_per_launch=by["grouped_ffn"],
                    ms_per_launch=r["stages_ms"]["grouped_ffn"])
    roofline = {k_: roofline[k_] for k_ in ("bound", "kernel", "achieved", "peak", "unit",
                                            "frac", "traffic", "flops_per_launch",
                                            "bytes_per_launch", "ms_per_launch")}

    line = {
        "metric": "MoE-layer tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak), "
                  "Mixtral shape",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": per_step[len(per_step) // 2],
        "ms_per_step_min": per_step[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 (fp8 e4m3 expert weights)" if args.fp8 else "bf16")
                 if wl.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded; random weights of the layer's shape)",
        "config": {"workload": _workload_text(wl),
                   "T": T, "d_model": d, "E": E, "top_k": k, "d_ff": dff,
                   "capacity_factor": wl.capacity_factor,
                   "gating": ["topk_then_softmax", "softmax_then_topk"][wl.gating]},
        "roofline": roofline,
        "stages_ms": r["stages_ms"],
        # router logits: 2 T d E algorithmic flops of fp32 logits per step
        # (route stage: logits, top-k and gate weights).  fp32 layers compute
        # them with fp32 vector FMAs (peak 157.3 TFLOP/s); bf16 layers as three
        # exact bf16 products on the matrix cores, 3x the flops against the
        # dense bf16 peak (2500 TFLOP/s)
        "stages_tflops": _route_tflops(T, d, E, t_route, wl.dtype == W.BF16),
        "stages_gbs": {"route": by["route"] / (t_route * 1e6),
                       "permute": by["permute"] / (r["stages_ms"]["permute"] * 1e6),
                       "combine": by["combine"] / (r["stages_ms"]["combine"] * 1e6),
                       "grouped_ffn_weights_and_rows":
                           by["grouped_ffn"] / (r["stages_ms"]["grouped_ffn"] * 1e6)},
        "routing": {"kept_copies": N, "dropped": int(r["st"][-1]),
                    "active_experts": r["active"],
                    "max_over_mean_load": float(r["counts"].max() /
                                                max(r["counts"].mean(), 1e-9))},
        "wall_s_timed": r["wall"],
    }
    shared = None
    if args.shared_dff > 0:
        S = W.make_shared_device(wl, args.shared_dff, "cuda")
        ws_sh = torch.empty(M.forward_shared_workspace_bytes(p, args.shared_dff),
                            dtype=torch.uint8, device="cuda")

        def step():  # noqa: F811 -- the headline step is the layer with the shared expert
            M.moe_forward_shared(p, args.shared_dff, *a, *S, out=out, stats=stats,
                                 workspace=ws_sh)

        def step_serial():
            M.moe_forward_shared(p, args.shared_dff, *a, *S, out=out, stats=stats,
                                 workspace=ws_sh, side_stream=None)
        shared = (S, ws_sh, step_serial)
        for _ in range(args.warmup):
            step()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
        evs[-1].synchronize()
        t_routed = ms
        ms = evs[0].elapsed_time(evs[-1]) / args.steps
        per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
        line.update(value=T / (ms * 1e-3), ms_per_step=ms,
                    ms_per_step_median=per_step[len(per_step) // 2],
                    ms_per_step_min=per_step[0])
        for _ in range(2):
            step_serial()
        t_serial = _time_loop(step_serial, n, stream)
        line["config"]["shared_d_ff"] = args.shared_dff
        line["config"]["workload"] += (f", plus a shared expert (SwiGLU d_ff="
                                       f"{args.shared_dff}) on every token")
        line["shared_expert"] = {
            "ms_per_step_side_stream": ms, "ms_per_step_one_stream": t_serial,
            "ms_routed_layer_alone": t_routed,
            "shared_ffn_flops": 6.0 * T * d * args.shared_dff}
    if args.router_stats:
        ws_st = torch.empty(M.forward_stats_workspace_bytes(p), dtype=torch.uint8,
                            device="cuda")
        rstats = torch.empty(2 * wl.E + 2, dtype=torch.float32, device="cuda")

        def step_stats():
            M.moe_forward_stats(p, *a, out=out, stats=stats, router_stats=rstats,
                                workspace=ws_st)
        for _ in range(2):
            step_stats()
        t_stats = _time_loop(step_stats, n, stream)
        t_plain = _time_loop(lambda: M.moe_forward(p, *a, out=out, stats=stats,
                                                   workspace=ws), n, stream)
        rs = rstats.cpu().numpy()
        line["router_stats"] = {"ms_per_step_with_stats": t_stats,
                                "ms_per_step_without": t_plain,
                                "aux_loss": float(rs[2 * wl.E]),
                                "z_loss": float(rs[2 * wl.E + 1])}
    if args.backward:
        if args.fp8 or wl.dtype != W.BF16:
            sys.exit("--backward needs a bf16 layer without --fp8")
        state = torch.empty(M.train_state_bytes(p), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(M.backward_workspace_bytes(p), dtype=torch.uint8,
                           device="cuda")
        dout = torch.from_numpy(W.make_dout(wl)).to("cuda")
        grads = None

        def fwd_train():
            M.moe_forward_train(p, *a, out=out, stats=stats, state=state, workspace=ws)

        def bwd():
            nonlocal grads
            grads = M.moe_backward(p, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                                   dev["W_down"], state, dout, grads=grads,
                                   with_dbias=dev["bias"] is not None, workspace=ws_b)

        for _ in range(2):
            fwd_train()
            bwd()
        t_ft = _time_loop(fwd_train, n, stream)
        fwd_train()
        t_bwd = _time_loop(bwd, n, stream)
        t_train = _time_loop(lambda: (fwd_train(), bwd()), n, stream)
        bwd_flops = 12.0 * N * d * dff   # dH, dX_perm (x2), dW_down, dW_gate + dW_up (x2)
        line["training"] = {
            "ms_forward_train": t_ft, "ms_backward": t_bwd,
            "ms_training_step": t_train,
            "tokens_per_s_training": T / (t_train * 1e-3),
            "backward_gemm_flops": bwd_flops,
            "backward_tflops": bwd_flops / (t_bwd * 1e-3) / 1e12,
            "backward_frac_of_bf16_peak": bwd_flops / (t_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    if args.graph and shared is None:
        try:
            line["graph"] = {"ms_per_step_replayed": _graph_time(step, n, stream),
                             "ms_per_step_eager": ms}
        except Exception as ex:  # capture unsupported: report, do not fail the line
            line["graph"] = {"error": repr(ex)[:200]}
    if args.sample_power:
        _progress("sampling socket power")
        line["power"] = _sample_power(lambda: ffn(Y, ffn_ws), ffn_flops, stream)
        if args.library_loop and not args.fp8 and wl.dtype == W.BF16:
            lib = _library_loop(wl, dev, perm, 1, stream, ffn_flops, fns_only=True)
            line["power_library_gemms"] = _sample_power(lib, ffn_flops, stream)
    if args.library_loop and not args.fp8 and wl.dtype == W.BF16:
        _progress("vendor-library loop")
        line["library_loop"] = _library_loop(wl, dev, perm, n, stream, ffn_flops)
    if not args.no_cpu_baseline:
        _progress("CPU baseline (the oracle on the host)")
        line["cpu_baseline"] = _cpu_baseline(
            wl, dev, args.cpu_sample_tokens,
            shared=None if shared is None else [t.float().cpu().numpy() for t in shared[0]],
            fp8_scales=w_scales.cpu().numpy() if args.fp8 else None)
    if args.configs:
        # the other workloads, one after the other in the same process (the
        # headline's tensors are released first)
        del r, dev, a, ws, out, stats, perm, Y, ffn, ffn_ws, shared, step
        line["configs"] = {}
        for name, cw in W.WORKLOADS.items():
            if name == wl.name:
                continue
            torch.cuda.empty_cache()
            rc = _run_layer(cw, args.steps, args.warmup)
            _progress(f"{name}: {rc['ms']:.3f} ms per step")
            line["configs"][name] = _config_summary(rc)
            del rc
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
