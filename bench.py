#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X, plus its roofline and a CPU baseline.

A step is one pass of the whole path -- route, permute, grouped GEMM 1 (gate/up + SwiGLU),
grouped GEMM 2 (down), combine -- over one batch of seeded synthetic inputs already in
HBM, through the library's C ABI on torch's current stream. The expert weights are resident
in the library's packed layout (moe_pack_expert_weight, run once when the layer is loaded,
outside the timed region, as an inference engine stores its weights); the same steps on
the plain row-major weights are timed beside them. HIP events recorded on the stream
between the stages give per-stage times; the dominant kernel (GEMM 1) is reported against
the bf16 dense MFMA peak. The CPU oracle is timed on a bounded token sample.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s at 1 GPU; grouped-GEMM % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_up_mixtral_traffic.txt")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=None,
                    help="token count of the headline workload (a batch sweep); the other "
                         "workloads keep theirs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--backward", action="store_true",
                    help="time a training step instead: moe_forward then moe_backward")
    ap.add_argument("--weights", choices=("packed", "plain"), default="packed",
                    help="expert weight layout of the timed forward (bf16)")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="time the headline workload only (and skip the vendor BLAS reference)")
    ap.add_argument("--extra-steps", type=int, default=20,
                    help="timed steps of each of the other workloads")
    ap.add_argument("--extra-warmup", type=int, default=5)
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock reading (a 1.6 s GEMM-1 loop per workload), e.g. "
                         "under a profiler")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


GEMM_SOURCES = ("gemm.hip", "packed_kloop.h", "kloop_model.h", "tile_order.h")


def kernel_source_digest(path: str | None = None) -> str:
    """Digest of the GEMM sources (gemm.hip and the k-loop and tile-order headers it
    includes, or the one file `path`) with comments and whitespace removed, so that an edit
    of comments alone keeps the committed counter summary valid."""
    csrc = os.path.join(ROOT, "mixture_experts_layer_37_amd", "csrc")
    paths = [path] if path else [os.path.join(csrc, f) for f in GEMM_SOURCES]
    h = hashlib.sha256()
    for p in paths:
        text = re.sub(r"//[^\n]*", "", open(p, encoding="utf-8").read())
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(per_launch_flops_unused=None):
    """HBM bytes per GEMM-1 launch from the committed rocprofv3 counter summary, or None when
    the summary is missing or was taken on a different GEMM source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        m = re.match(r"^\s*([a-z0-9_]+)\s*:\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("gemm_source_sha256_16") != kernel_source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


EXTRA_WORKLOADS = ("small", "cap32", "fine", "mixtral_threshold")


def step_stats(ms):
    """mean, median, min and p90 of per-step times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min()),
            "p90": float(np.percentile(a, 90))}


def gemm_clock(launch, seconds=1.6, settle=0.8):
    """The GPU's graphics clock while GEMM 1 runs back to back: `launch` is enqueued for
    `seconds` while a thread samples amdsmi's current per-XCD gfx clocks (the readings
    refresh a few times a second); samples from the first `settle` seconds are dropped.
    Returns the mean over samples and XCDs (MHz), the per-XCD means and the sample count, or
    None where amdsmi cannot read the device."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
        amdsmi.amdsmi_get_gpu_metrics_info(handle)
    except Exception:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            t = time.perf_counter()
            try:
                clks = amdsmi.amdsmi_get_gpu_metrics_info(handle).get("current_gfxclks")
                if isinstance(clks, list):
                    clks = [float(v) for v in clks if isinstance(v, (int, float))]
                    if clks:
                        samples.append((t, clks))
            except Exception:
                pass
            stop.wait(0.05)

    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        launch()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()   # keep the queue short so the loop ends on time
    torch.cuda.synchronize()
    stop.set()
    th.join()
    use = [c for t, c in samples if t - t0 >= settle]
    amdsmi.amdsmi_shut_down()
    if not use:
        return None
    nx = min(len(c) for c in use)
    per_xcd = [sum(c[i] for c in use) / len(use) for i in range(nx)]
    return {"mhz": sum(per_xcd) / nx, "per_xcd_mhz": [round(v) for v in per_xcd],
            "samples": len(use), "launches": n}


def add_measured(rec, peaks):
    """The record's fractions against what this device sustains (measured_peaks)."""
    if peaks is None:
        return
    rec["grouped_gemm_frac_of_measured"] = rec["_ffn_tflops"] / peaks["mfma_bf16_tflops"]
    rec["hbm_frac_of_measured"] = {n: v * PEAK_HBM_GBS / peaks["hbm_copy_gbs"]
                                   for n, v in rec["hbm_frac"].items()}
    if "materialised_permute" in rec:
        rec["materialised_permute"]["hbm_frac_of_measured"] = (
            rec["materialised_permute"]["hbm_frac"] * PEAK_HBM_GBS / peaks["hbm_copy_gbs"])


def run_workload(name, args, steps, warmup, headline, peaks=None):
    """Times `steps` forward steps of one workload (after `warmup`) and returns its record;
    the headline workload also carries the roofline, the plain-weight context, the
    materialised permute, the router against a one-pass read and the CPU baseline."""
    import numpy as np
    import torch

    from mixture_experts_layer_37_amd import _lib as L
    from mixture_experts_layer_37_amd import configs as C
    from mixture_experts_layer_37_amd.inputs import make_inputs
    from mixture_experts_layer_37_amd.layer import MoELayer, to_device

    cfg = C.get(name)
    if cfg.dtype == C.BF16:
        cfg = cfg.with_(weights=args.weights)
    if headline and args.tokens is not None:
        cfg = cfg.with_(tokens=args.tokens,
                        description=re.sub(r"^\d+ tokens( \([^)]*\))?", f"{args.tokens} tokens",
                                           cfg.description))
    T, H, I, E, k = cfg.tokens, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    inp = make_inputs(cfg, seed=args.seed, threads=16)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    dev = x.device
    c = layer.c
    ws = layer.ws
    edt = x.dtype
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    rt = torch.empty(T * k, dtype=torch.int32, device=dev)
    sr = torch.empty((T, k), dtype=torch.int32, device=dev)
    h = torch.empty((T * k, I), dtype=edt, device=dev)
    y = torch.empty((T * k, H), dtype=edt, device=dev)
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    names = ["route_permute", "gemm_up", "gemm_down", "combine"]
    packed = cfg.weights == "packed"

    def step(ev=None, plain=False):
        # the path moe_forward runs: route and the permutation's row maps in one call (the
        # count step inside the streaming router), then GEMM 1 reading the token rows in
        # place through the maps
        cw = layer.c_plain if plain else c
        wg, wu, wd = ((layer.w_gate, layer.w_up, layer.w_down) if plain or not packed
                      else (layer.fw_gate, layer.fw_up, layer.fw_down))
        if ev: ev[0].record(stream)
        L.moe_route_permute(cw, x, layer.w_router if plain else layer.fw_router, layer.bias,
                            logits, idx, w, counts, offs, rt, sr, ws, stream)
        if ev: ev[1].record(stream)
        L.moe_expert_up_rows(cw, x, rt, offs, wg, wu, h, stream)
        if ev: ev[2].record(stream)
        L.moe_expert_down(cw, h, offs, wd, y, ws, stream)
        if ev: ev[3].record(stream)
        L.moe_combine(cw, y, sr, w, out, stream)
        if ev: ev[4].record(stream)

    def timed_steps(n, plain=False):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(n):
            step(ev[s], plain=plain)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / n
        per_step = [e[0].elapsed_time(e[-1]) for e in ev]
        stages = {nm: float(np.median([e[i].elapsed_time(e[i + 1]) for e in ev])) * 1e3
                  for i, nm in enumerate(names)}
        return wall, per_step, stages

    def route_and_permute_alone(reps=7):
        """moe_route and moe_permute (row maps) as separate calls, each rep right after a
        full step (the cache state of the timed steps): median µs of each."""
        r_us, p_us = [], []
        for _ in range(reps):
            step()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            L.moe_route(c, x, layer.fw_router if packed else layer.w_router, layer.bias, logits,
                        idx, w, ws, stream)
            e[1].record(stream)
            L.moe_permute(c, x, idx, None, counts, offs, rt, sr, ws, stream)
            e[2].record(stream)
            torch.cuda.synchronize()
            r_us.append(e[0].elapsed_time(e[1]) * 1e3)
            p_us.append(e[1].elapsed_time(e[2]) * 1e3)
        return float(np.median(r_us)), float(np.median(p_us))

    if headline and args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    print(f"[bench] {cfg.name}: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: timing {steps} steps", file=sys.stderr, flush=True)
    wall_ms, per_step, stages_us = timed_steps(steps)
    stats = step_stats(per_step)
    # the router and the permutation each on its own (moe_route, moe_permute), for their
    # bandwidth figures; the step runs them as one call (stages_us.route_permute)
    stages_us["route"], stages_us["permute"] = route_and_permute_alone()

    n_kept = int(offs[-1].item())
    up_flops = (4 if cfg.activation == C.SWIGLU else 2) * n_kept * H * I
    down_flops = 2 * n_kept * H * I
    ffn_flops = up_flops + down_flops
    total_flops = 2 * T * H * E + ffn_flops
    up_tflops = up_flops / (stages_us["gemm_up"] * 1e-6) / 1e12
    ffn_tflops = ffn_flops / ((stages_us["gemm_up"] + stages_us["gemm_down"]) * 1e-6) / 1e12
    es = 2 if cfg.dtype == C.BF16 else 4
    # algorithmic bytes of the bandwidth-bound steps (the permute moves index data only: its
    # row gather is fused into GEMM 1)
    route_bytes = T * H * es + H * E * es + T * E * 4 + T * k * 8
    permute_bytes = T * k * 4 * 4
    combine_bytes = n_kept * H * es + T * H * es + T * k * 8
    hbm = {"route": route_bytes / (stages_us["route"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
           "permute_row_maps": permute_bytes / (stages_us["permute"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
           "combine": combine_bytes / (stages_us["combine"] * 1e-6) / 1e9 / PEAK_HBM_GBS}
    rec = {"workload": cfg.description, "tokens": T, "hidden": H, "inter": I, "experts": E,
           "top_k": k, "routing": cfg.routing, "capacity_factor": cfg.capacity_factor,
           "kept_rows": n_kept, "steps": steps, "warmup": warmup,
           "ms_per_step": stats, "ms_per_step_wall_mean": wall_ms,
           "tokens_per_s": T / (stats["median"] * 1e-3),
           "stages_us": stages_us,
           "gemm_up_frac_of_peak": up_tflops / PEAK_BF16_TFLOPS,
           "grouped_gemm_frac_of_peak": ffn_tflops / PEAK_BF16_TFLOPS,
           "layer_tflops": total_flops / (stats["median"] * 1e-3) / 1e12,
           "hbm_frac": hbm}
    rec["_ffn_tflops"] = ffn_tflops
    add_measured(rec, peaks)
    wg, wu = ((layer.fw_gate, layer.fw_up) if packed else (layer.w_gate, layer.w_up))
    rec["gemm_clock"] = None if args.no_clock else gemm_clock(
        lambda: L.moe_expert_up_rows(c, x, rt, offs, wg, wu, h, stream))
    if not headline:
        rec["device_flags"] = L.moe_read_device_status(c, ws, 3, stream)
        return rec

    # the headline's extras
    rec["_wall_ms"] = wall_ms
    rec["_up_flops"], rec["_up_tflops"] = up_flops, up_tflops
    rec["weights"] = ("packed once at load (moe_pack_expert_weight)" if packed
                      else "plain row-major")
    rec["activation"] = cfg.activation
    rec["threshold"] = ((cfg.threshold if cfg.threshold > 0 else 1.0 / E)
                        if cfg.routing == "threshold" else None)
    if packed:
        # context: the same steps on the plain row-major weights (bit-identical output)
        n_plain = max(2, steps // 2)
        for _ in range(2):
            step(plain=True)
        pw, pst, pstages = timed_steps(n_plain, plain=True)
        rec["plain_weights"] = {"ms_per_step": step_stats(pst), "steps": n_plain,
                                "stages_us": pstages}
        step()   # leave the packed step's results in place for the checks below
        torch.cuda.synchronize()
    rec["materialised_permute"] = materialised_permute(L, c, x, idx, counts, offs, rt, sr, ws,
                                                       stream, T, H, k, n_kept, es)
    rd = one_pass_read_us(stream, x, T * H * es, step)
    if rd is not None:
        # the router against a plain one-pass read of the same token matrix, each timed
        # right after a full step (the same cache state): 1.0 = as fast as reading x
        rec["route_vs_one_pass_read"] = {
            "read_us": rd, "route_us": stages_us["route"],
            "read_gbs": T * H * es / (rd * 1e-6) / 1e9, "frac": rd / stages_us["route"]}
    rec["device_flags"] = L.moe_read_device_status(c, ws, 3, stream)
    if not args.no_cpu_baseline:
        rec["_cpu_baseline"] = cpu_baseline(cfg, inp, out, logits, idx, args.cpu_sample_tokens,
                                            rec)
    return rec


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU layout "
              "is described in the design notes and is not run here.", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_37_amd import configs as C

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.backward:
        from mixture_experts_layer_37_amd.inputs import make_inputs
        from mixture_experts_layer_37_amd.layer import MoELayer, to_device
        cfg = C.get(args.config)
        inp = make_inputs(cfg, seed=args.seed, threads=16)
        layer = MoELayer(cfg, inp)
        return backward_bench(args, cfg, layer, to_device(cfg, inp["x"]))

    stream = torch.cuda.current_stream()
    head = run_workload(args.config, args, args.steps, args.warmup, True)
    torch.cuda.empty_cache()
    peaks = measured_peaks(stream)   # after the headline, so its load does not precede it
    add_measured(head, peaks)
    cfg = C.get(args.config)
    if args.tokens is not None:
        cfg = cfg.with_(tokens=args.tokens)
    # the headline: whole-step wall time over the K timed steps, as the step contract says
    ms_per_step = head.pop("_wall_ms")
    up_flops, up_tflops = head.pop("_up_flops"), head.pop("_up_tflops")
    cpu = head.pop("_cpu_baseline", None)
    # the committed counter summary covers GEMM 1 (packed weights) of the Mixtral top-2
    # workload only
    traffic = (measured_traffic() if cfg.name == "mixtral" and args.weights == "packed"
               and args.tokens in (None, C.get(args.config).tokens) else None)
    result = {
        "metric": METRIC,
        "value": cfg.tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_stats": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == C.BF16 else "f32",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": head["workload"], "tokens": head["tokens"],
                   "hidden": head["hidden"], "inter": head["inter"],
                   "experts": head["experts"], "top_k": head["top_k"],
                   "capacity_factor": head["capacity_factor"],
                   "activation": head["activation"], "routing": head["routing"],
                   "threshold": head["threshold"], "kept_rows": head["kept_rows"],
                   "weights": head["weights"]},
        "roofline": {"kernel": ("grouped_gemm_packed_kernel<SwiGLU> (moe_expert_up_rows)"
                                if args.weights == "packed" else
                                "grouped_gemm_bf16_kernel<SwiGLU> (moe_expert_up_rows)"),
                     "bound": "mfma", "achieved": up_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": up_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "algorithmic_flops": up_flops},
        "grouped_gemm_frac_of_peak": head["grouped_gemm_frac_of_peak"],
        "layer_tflops": head["layer_tflops"],
        "stages_us": head["stages_us"],
        "hbm_frac": head["hbm_frac"],
        "gemm_clock": head["gemm_clock"],
    }
    for key in ("plain_weights", "materialised_permute", "hbm_frac_of_measured",
                "grouped_gemm_frac_of_measured",
                "route_vs_one_pass_read", "device_flags", "parity"):
        if key in head:
            result[key] = head[key]
    result["measured_peaks"] = peaks
    if not args.no_extra_workloads and cfg.dtype == C.BF16:
        result["vendor_gemm"] = vendor_gemm_reference(cfg, stream, head["stages_us"])
        torch.cuda.empty_cache()
    if peaks is not None:
        result["roofline"]["peak_measured"] = peaks["mfma_bf16_tflops"]
        result["roofline"]["frac_of_measured"] = up_tflops / peaks["mfma_bf16_tflops"]
    # every workload of the layer, each timed on its own (the headline's entry repeats it)
    workloads = {cfg.name: {k: v for k, v in head.items()
                            if k not in ("plain_weights", "materialised_permute",
                                         "route_vs_one_pass_read", "parity")}}
    for rec in [head] + list(workloads.values()):
        rec.pop("_ffn_tflops", None)
    if not args.no_extra_workloads:
        for name in EXTRA_WORKLOADS:
            if name == cfg.name:
                continue
            rec = run_workload(name, args, args.extra_steps, args.extra_warmup, False, peaks)
            rec.pop("_ffn_tflops", None)
            workloads[name] = rec
            torch.cuda.empty_cache()
    result["workloads"] = workloads
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def backward_bench(args, cfg, layer, x):
    """One training step of the layer: moe_forward_train (the forward keeping GEMM 1's
    pre-activations), then moe_backward on a seeded dout. Reports tokens/s of the whole step,
    the forward and backward times (HIP events on the stream both run on), and the
    backward's GEMM rate: dh 2NHI, dx 4NHI and the three weight gradients 6NHI flops over the
    N kept rows (SwiGLU; GELU dh 2NHI, dx 2NHI, weight gradients 4NHI)."""
    import numpy as np
    import torch

    from mixture_experts_layer_37_amd import _lib as L
    from mixture_experts_layer_37_amd import configs as C
    from mixture_experts_layer_37_amd.inputs import f32_to_bf16_bits
    from mixture_experts_layer_37_amd.layer import to_device

    T, H, I = cfg.tokens, cfg.hidden, cfg.inter
    rng = np.random.default_rng(args.seed + 1)
    dout = to_device(cfg, f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        layer.forward_train(x, stream=stream)   # keeps GEMM 1's pre-activations
        if ev: ev[1].record(stream)
        g = layer.backward(x, dout, stream=stream)
        if ev: ev[2].record(stream)
        return g

    print(f"[bench] backward: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] backward: timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    n_kept = int(layer.view(L.MOE_WS_OFFSETS)[-1].item())
    per_row = 12 if cfg.activation == C.SWIGLU else 8
    bwd_flops = per_row * n_kept * H * I
    result = {
        "metric": "MoE layer training step (forward + backward) tokens/s at 1 GPU",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded inputs and dout)",
        "config": {"workload": cfg.description + "; forward + backward", "tokens": T,
                   "hidden": H, "inter": I, "experts": cfg.experts, "top_k": cfg.top_k,
                   "routing": cfg.routing, "kept_rows": n_kept},
        "forward_ms": fwd_ms, "backward_ms": bwd_ms,
        "backward_gemm_flops": bwd_flops,
        "backward_tflops": bwd_flops / (bwd_ms * 1e-3) / 1e12,
        "backward_frac_of_peak": bwd_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
    }
    print(json.dumps(result), flush=True)


def measured_peaks(stream):
    """What this device sustains, from the library's probes (libmoe_peaks.so): an MFMA-only
    loop (bf16 v_mfma_f32_32x32x16, no memory traffic) at the packed GEMMs' occupancy, one
    block of 4 waves per CU (one wave per SIMD; 4 blocks per CU sustain ~15% less), and a
    1 GiB device-to-device streaming copy (bytes read + written). None if not built."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "mixture_experts_layer_37_amd", "libmoe_peaks.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.moe_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.moe_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = cus, 16000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sh = stream.cuda_stream

    def timed(fn, reps=3):
        fn()
        best = None
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    ms_mfma = timed(lambda: lib.moe_peak_mfma(sink.data_ptr(), blocks, iters, sh))
    ms_copy = timed(lambda: lib.moe_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh))
    return {"mfma_bf16_tflops": blocks * 4 * iters * 8 * 32768 / (ms_mfma * 1e-3) / 1e12,
            "hbm_copy_gbs": 2 * nbytes / (ms_copy * 1e-3) / 1e9}


def vendor_gemm_reference(cfg, stream, stages_us, reps=7):
    """The ROCm BLAS (torch.bmm) on the same two expert products with the rows split evenly,
    T*k/E per expert, bf16, contiguous operands: GEMM 1's x_e [R, H] x [H, 2I] (gate and up
    side by side, no activation) and GEMM 2's h_e [R, I] x [I, H]. A reference beside the
    grouped GEMMs (which also gather x, apply SwiGLU and take the routed, uneven rows); the
    layer never calls it. Median of `reps` after two warm-up calls."""
    import torch
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    R = cfg.tokens * cfg.top_k // E
    gen = torch.Generator(device="cuda").manual_seed(0)

    def med_us(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return sorted(ts)[len(ts) // 2]

    out = {"library": "torch.bmm (ROCm BLAS)", "rows_per_expert": R}
    for key, K, N, stage in (("gemm_up", H, 2 * I, "gemm_up"), ("gemm_down", I, H, "gemm_down")):
        a = torch.randn(E, R, K, device="cuda", dtype=torch.bfloat16, generator=gen)
        b = torch.randn(E, K, N, device="cuda", dtype=torch.bfloat16, generator=gen) * K ** -0.5
        us = med_us(lambda: torch.bmm(a, b))
        del a, b
        tflops = 2.0 * E * R * K * N / (us * 1e-6) / 1e12
        out[key] = {"us": us, "tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS,
                    "grouped_us": stages_us[stage], "grouped_over_vendor": stages_us[stage] / us}
    return out


def one_pass_read_us(stream, buf, nbytes, step, reps=7):
    """Median time of one plain streaming read of `nbytes` of `buf` (libmoe_peaks.so's
    moe_peak_read, 2 blocks of 256 threads per CU), each rep right after a full forward step
    so that caches hold what they hold when the router runs. None if the probes are not
    built."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "mixture_experts_layer_37_amd", "libmoe_peaks.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.moe_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                  ctypes.c_int, ctypes.c_void_p]
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    times = []
    for _ in range(reps):
        step()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = lib.moe_peak_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks,
                               stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if rc != 0:
            return None
        times.append(e0.elapsed_time(e1) * 1e3)
    return float(sorted(times)[len(times) // 2])


def materialised_permute(L, c, x, idx, counts, offs, rt, sr, ws, stream, T, H, k, n_kept, es):
    """moe_permute writing x_perm (the standalone gather, not on the timed path): mean time
    over 10 calls and its HBM fraction for x read once + x_perm written + index arrays."""
    import torch
    xp = torch.empty((T * k, H), dtype=x.dtype, device=x.device)
    L.moe_permute(c, x, idx, xp, counts, offs, rt, sr, ws, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        L.moe_permute(c, x, idx, xp, counts, offs, rt, sr, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 10
    nbytes = T * H * es + n_kept * H * es + T * k * 4 * 4
    return {"us": us, "hbm_frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}


def cpu_baseline(cfg, inp, out_dev, logits_dev, idx_dev, n_tok, result):
    """The oracle, as it is, on the first n_tok tokens of the same layer (its expert weights
    widened to float64 one expert at a time). The same leg re-checks the timed outputs:
    routing bit-exact from the GPU's own logits on every token, and the sampled tokens'
    layer outputs against the oracle's."""
    import numpy as np

    import oracle as O
    from mixture_experts_layer_37_amd.inputs import ExpertView, as_float, bf16_bits_to_f32
    from mixture_experts_layer_37_amd.layer import from_device

    gl = logits_dev.cpu().numpy().astype(np.float64)
    if cfg.routing == "threshold":
        ridx, _ = O.threshold_select(gl, cfg.top_k, cfg.threshold)
        exact = O.threshold_margin(gl, cfg.threshold) >= 1e-12
    else:
        ridx, _ = O.select_experts(gl, cfg.top_k)
        exact = np.ones(len(ridx), dtype=bool)
    result["parity"] = {"routing_bit_exact": bool(np.array_equal(ridx[exact],
                                                                 idx_dev.cpu().numpy()[exact]))}
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    n_tok = min(n_tok, cfg.tokens)
    xs = as_float(cfg, inp["x"][:n_tok])
    wg = ExpertView(cfg, inp["w_gate"]) if cfg.activation == "swiglu" else None
    # repeat the whole sample until about 10 s of oracle time (at most 3 passes)
    times = []
    while len(times) < 3 and sum(times) < 10.0:
        t0 = time.perf_counter()
        ref = O.forward(xs, as_float(cfg, inp["w_router"]), inp["bias"], wg,
                        ExpertView(cfg, inp["w_up"]), ExpertView(cfg, inp["w_down"]),
                        top_k=cfg.top_k, activation=cfg.activation,
                        capacity_factor=cfg.capacity_factor, renormalize=cfg.renormalize,
                        routing=cfg.routing, threshold=cfg.threshold)
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    rep = {"value": n_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"first {n_tok} of {cfg.tokens} tokens of the same layer, all experts; "
                     f"{len(times)} pass(es), {dt:.1f} s each", "host_cpus": len(os.sched_getaffinity(0))}
    if cfg.capacity_factor <= 0:      # a token prefix routes exactly as in the full batch
        got = from_device(out_dev[:n_tok])
        got = (bf16_bits_to_f32(got) if got.dtype == np.uint16 else got).astype(np.float64)
        use = ref["margin"] >= 1e-4   # near ties (threshold routing: |p - delta| / delta)
        err = np.abs(got[use] - ref["out"][use])
        result["parity"]["sample_max_rel"] = float(err.max() / np.abs(ref["out"][use]).max())
        result["parity"]["sample_mean_rel"] = float(err.sum() / np.abs(ref["out"][use]).sum())
    return rep


if __name__ == "__main__":
    main()
