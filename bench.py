#!/usr/bin/env python3
"""Benchmark of one absorbed MLA decode step on one MI355X.

A step is the whole hot path on one batch through mla_decode_step, over inputs already resident
in HBM: one kernel launch for one bf16 sequence at the V3 head sizes (at most 4096 cached tokens),
otherwise mla_absorb_q -> mla_decode_partial -> mla_decode_combine_uv (the combine pass and
mla_uv_out; one kernel at batch <= 4).  Prints one JSON line.

Default workload: DeepSeek-V3-shape decode, B=1, H=128, d_c=512, d_R=64, N=4096 cached tokens,
bf16 caches and weights (``--config 3/4/5`` selects the other synthetic workloads).

Timing: inputs are replicated into enough copies that consecutive steps never find their
weights or cache in the 256 MB Infinity Cache (about 1 GB rotated); one HIP graph holds one step
per copy and is replayed, so host launch overhead is not timed.  Per-kernel durations come from HIP events recorded
on the launch stream around back-to-back launches of one kernel over the rotated copies, after
the stream has been primed so that the host runs ahead of the GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "cached latents/sec + achieved HBM TB/s, MLA absorbed decode (V3 shape)"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "k_absorb_bf16": "absorb_uv_mfma.hip",
    "k_absorb_gemv": "absorb_uv_mfma.hip",
    "k_uv_bf16": "absorb_uv_mfma.hip",
    "k_uv_gemv": "absorb_uv_mfma.hip",
    "k_partial_mfma": "decode_partial_mfma.hip",
    "k_partial_small": "decode_partial_small.hip",
    "k_combine_rows": "decode_generic.hip",
    "k_combine_heads": "decode_generic.hip",
    "k_combine_uv": "absorb_uv_mfma.hip",
    "k_step_b1": "decode_step.hip",
}


def fused_combine_uv(wl):
    """Whether mla_decode_combine_uv runs as one kernel for this workload (the library's rule)."""
    return wl.dtype != "f32" and wl.B <= 4 and wl.d_h == 128 and wl.d_c == 512


def kernel_names(wl):
    """Kernel that each pass launches for this workload (the library's own dispatch rules)."""
    small = wl.B <= 4
    tiles = wl.B * ((wl.n_max + 31) // 32)
    small_partial = wl.dtype == "bf16" and wl.B <= 256 and tiles <= 1024
    return {"absorb": "k_absorb_gemv" if small else "k_absorb_bf16",
            "partial": "k_partial_small" if small_partial else "k_partial_mfma",
            "combine": "k_combine_heads" if (wl.H // 32) * wl.B >= 256 else "k_combine_rows",
            "uv": "k_uv_gemv" if small else "k_uv_bf16", "combine_uv": "k_combine_uv"}


def one_launch_step(wl, num_splits):
    """Whether DecodeStep runs the one-launch form of mla_decode_step for this workload (the
    library's rule for aligned arguments on a GPU with at least 256 compute units)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return (num_splits == 0 and wl.dtype == "bf16" and wl.B == 1 and wl.H == 128 and wl.d_h == 128
            and wl.d_c == 512 and wl.d_R == 64 and wl.n_max <= 4096 and cus >= 256
            and (wl.layout != "paged" or wl.page_size % 32 == 0))


def environment():
    """GPU name, ROCm / HIP versions and the host CPU model of this run."""
    import torch
    env = {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip,
           "cus": torch.cuda.get_device_properties(0).multi_processor_count}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    env["cpu_model"] = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    env["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    env["host_cores"] = len(os.sched_getaffinity(0))
    return env


def sampled_parity(inp, got, n_extra=4, seed=0):
    """Worst relative L2 over sampled (sequence, head) pairs of the timed run's outputs (o and
    o_lat) against the oracle: heads 0, 31, 32, 63, 64, 95, 96, 127 (every 32-head block's edges)
    of the shortest, the longest, the first and a few random sequences."""
    import numpy as np
    import oracle
    wl = inp.wl
    rng = np.random.default_rng(seed)
    bs = {0, wl.B - 1, int(np.argmin(inp.lens)), int(np.argmax(inp.lens))}
    bs |= set(int(x) for x in rng.choice(wl.B, size=min(wl.B, n_extra), replace=False))
    heads = sorted({h for h in (0, 31, 32, 63, 64, 95, 96, 127) if h < wl.H} | {wl.H - 1})
    pairs = [(b, h) for b in sorted(bs) if inp.lens[b] > 0 for h in heads]
    ref = oracle.decode(inp, pairs=pairs)
    res = {"pairs": len(pairs)}
    for key in ("o", "o_lat"):
        res[key] = float(max(oracle.relative_l2(got[key][b, h], ref[key][b, h]) for b, h in pairs)) if pairs else None
    res["tolerance"] = 1e-5 if wl.dtype == "f32" else 1e-2
    return res


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400, help="timed steps (exactly this many)")
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--rotate-mb", type=float, default=1024.0, help="bytes of input copies rotated per pass")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle timing budget (0 = skip)")
    ap.add_argument("--kernel-reps", type=int, default=50, help="events-bracketed passes per kernel")
    ap.add_argument("--kernel-in-step", action="store_true",
                    help="also time each call of a several-call step inside whole steps (an event pair per call)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--row", choices=["decode", "append", "mha", "query", "out", "layer"], default="decode",
                    help="decode: the absorbed decode step (default); append: the cache write of one step; "
                         "mha: the same-dimension MHA decode beside the latent path's attention pass; "
                         "query: the query side (c_q, q_C, q_R, then q' unfolded or through the folded "
                         "W_UK^T W_UQ); out: the output side (W_UV then W_O, or the folded W_O W_UV); "
                         "layer: one whole attention layer's decode step (cache write, query side, "
                         "attention, W_UV, W_O)")
    ap.add_argument("--layer-context", type=int, default=4096,
                    help="--row layer: tokens per sequence after the new one is appended")
    ap.add_argument("--append-batch", type=int, default=1,
                    help="--row append / query / out: new tokens (sequences) per call")
    ap.add_argument("--shard", type=int, default=1, metavar="G",
                    help="decode row: one GPU's share of the workload split by token range over G GPUs "
                         "(every sequence keeps 1/G of its tokens); the exchange between GPUs is not run")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB",
                    help="only run 4 plain device copies and 4 read-only sums of MB megabytes (a reference for "
                         "HBM byte counters and the streaming ceiling)")
    return ap.parse_args()


def source_hash(fname: str) -> str:
    p = os.path.join(ROOT, "mla_latent_kv_attn_amd", "csrc", fname)
    with open(p, "rb") as f:
        h = hashlib.sha256(f.read())
    hdrs = ("mla_internal.h", "partial_common.h") + (("step_internal.h",) if fname == "decode_step.hip" else ())
    for hdr in hdrs:
        with open(os.path.join(ROOT, "mla_latent_kv_attn_amd", "csrc", hdr), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def alg_bytes(wl, sum_len):
    """Algorithmic HBM bytes per kernel launch (what the method must move)."""
    B, H, d_h, d_c, d_R = wl.B, wl.H, wl.d_h, wl.d_c, wl.d_R
    lat_b = {"bf16": 2, "fp8": 1, "f32": 4}[wl.dtype]
    rope_b = 4 if wl.dtype == "f32" else 2
    qb = 4 if wl.dtype == "f32" else 2
    per_tok = d_c * lat_b + d_R * rope_b + (4 if wl.dtype == "fp8" else 0)
    absorb = H * d_h * d_c * qb + B * H * d_h * qb + B * H * d_c * qb
    partial = sum_len * per_tok + B * H * (d_c + d_R) * qb
    combine = B * H * d_c * 4 + B * H * 4
    uv = H * d_h * d_c * qb + B * H * d_c * 4 + B * H * d_h * 4
    return {"absorb": absorb, "partial": partial, "combine": combine, "uv": uv, "combine_uv": combine + uv}, per_tok


def alg_flops(wl, sum_len):
    B, H, d_h, d_c, d_R = wl.B, wl.H, wl.d_h, wl.d_c, wl.d_R
    return {"absorb": 2 * B * H * d_h * d_c,
            "partial": sum_len * (2 * H * (d_c + d_R) + 2 * H * d_c),
            "combine": 0, "uv": 2 * B * H * d_h * d_c, "combine_uv": 2 * B * H * d_h * d_c}


def cpu_baseline(inp, budget_s):
    """The oracle as it stands, on this host's cores, timed on whole steps of the workload (or on
    a bounded sample of sequences when one step would exceed the budget)."""
    import numpy as np
    import threadpoolctl
    import oracle
    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(limits=cores):
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        wl = inp.wl
        # sample: all heads of a prefix of the sequences, grown until the budget is used
        order = list(range(wl.B))
        done_lat, t_used, reps = 0, 0.0, 0
        nb = 1
        while t_used < budget_s:
            bs = order[:nb]
            pairs = [(b, h) for b in bs for h in range(wl.H)]
            t0 = time.perf_counter()
            oracle.decode(inp, pairs=pairs, want_diag=False)
            dt = time.perf_counter() - t0
            t_used += dt
            done_lat += int(inp.lens[bs].astype(np.int64).sum())
            reps += 1
            if dt < budget_s / 8 and nb < wl.B:
                nb = min(wl.B, nb * 2)
        sample = (f"{reps} oracle runs over the first {nb} of {wl.B} sequences (all {wl.H} heads; explicit K/V "
                  f"rebuild, float64 numpy), {t_used:.1f} s")
        return {"value": done_lat / t_used, "unit": "latents/s", "cores": threads, "kind": "oracle",
                "sample": sample}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the absorbed decode kernel is measured "
                                   "on one MI355X; multi-GPU sharding is a design note, not built",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration > 0:
        # plain device-to-device copies of a buffer well above the 256 MB Infinity Cache: the
        # reference for the HBM byte counters, and the practical read+write bandwidth ceiling
        n = int(args.copy_calibration * 1e6) // 16 * 16
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ca.record()
        for _ in range(4):
            dst.copy_(src)
        cb.record()
        cb.synchronize()
        ms = ca.elapsed_time(cb) / 4
        # read-only stream: a float sum over the same bytes (the reduction writes one word)
        fv = src.view(torch.float32)
        _ = fv.sum()
        torch.cuda.synchronize()
        ra, rb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ra.record()
        for _ in range(4):
            _ = fv.sum()
        rb.record()
        rb.synchronize()
        rms = ra.elapsed_time(rb) / 4
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5, "copy_ms": round(ms, 4),
                          "read_plus_write_TBps": round(2 * n / (ms * 1e-3) / 1e12, 3),
                          "sums": 5, "sum_ms": round(rms, 4), "read_only_TBps": round(n / (rms * 1e-3) / 1e12, 3)}),
              flush=True)
        return

    if args.row == "append":
        main_append(args)
        return
    if args.row == "mha":
        main_mha(args)
        return
    if args.row in ("query", "out"):
        main_proj(args)
        return
    if args.row == "layer":
        main_layer(args)
        return

    from mla_latent_kv_attn_amd import ops
    from mla_latent_kv_attn_amd.step import DecodeStep
    from workloads import make_inputs
    from workloads.configs import WORKLOADS
    from workloads.device import device_cache, to_device

    wl = WORKLOADS[args.config]
    if args.shard > 1:
        G = args.shard
        wl = wl.with_(name=f"{wl.name}-shard{G}", n_max=wl.n_max // G, len_lo=max(1, wl.len_lo // G),
                      len_hi=wl.len_hi // G,
                      description=f"{wl.description}; one GPU's share of {G} by token range (tokens / {G})")
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    print(f"[bench] generating {wl.name}", file=sys.stderr, flush=True)
    inp = make_inputs(wl, poison=False)
    sum_len = inp.sum_len
    base = to_device(inp, dev)
    per_copy = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    R = max(1, min(64, math.ceil(args.rotate_mb * 1e6 / per_copy)))
    copies = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()} for _ in range(R - 1)]
    caches = [device_cache(inp, c) for c in copies]
    q_dtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    step = DecodeStep(wl.B, wl.H, wl.d_h, wl.d_c, wl.d_R, wl.n_max, q_dtype, dev, args.num_splits)
    W = args.num_splits or ops.mla_decode_auto_splits(wl.B, wl.H, wl.n_max)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    form = "one launch" if one_launch_step(wl, args.num_splits) else f"three or four calls, {W} splits"
    print(f"[bench] {R} input copies of {per_copy / 1e6:.1f} MB, {form}", file=sys.stderr, flush=True)

    def one(i):
        c = copies[i % R]
        step(c["q_C"], c["q_R"], c["W_UK"], c["W_UV"], caches[i % R], c["lens"])

    # ---------------- whole-step timing: exactly `steps` steps, as replays of a graph of R steps (one
    # per rotated copy) plus one replay of a graph holding the remaining steps % R
    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, R)):
            one(i)
    torch.cuda.synchronize()
    use_graph = not args.no_graph
    steps = args.steps
    spread = None
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(R):
                one(i)
        rem = steps % R
        g_rem = None
        if rem:
            g_rem = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_rem, stream=stream):
                for i in range(rem):
                    one(i)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(2):
                g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):          # replay() launches on the current stream
            e0.record(stream)
            for _ in range(steps // R):
                g.replay()
            if g_rem is not None:
                g_rem.replay()
            e1.record(stream)
        e1.synchronize()
        # spread: graph replays of R steps timed one by one (outside the timed region)
        per = []
        with torch.cuda.stream(stream):
            for _ in range(max(10, min(40, 4000 // R))):
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record(stream)
                g.replay()
                a1.record(stream)
                a1.synchronize()
                per.append(a0.elapsed_time(a1) / R)
        per = np.array(per)
        spread = {"replays": len(per), "steps_per_replay": R,
                  "ms_per_step_p10": round(float(np.percentile(per, 10)), 6),
                  "ms_per_step_median": round(float(np.median(per)), 6),
                  "ms_per_step_p90": round(float(np.percentile(per, 90)), 6)}
    else:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(steps):
                one(i)
            e1.record(stream)
        e1.synchronize()
    ms_per_step = e0.elapsed_time(e1) / steps
    torch.cuda.synchronize()
    got = {"o": step.out.cpu().numpy().astype(np.float64), "o_lat": step.o_latent.cpu().numpy().astype(np.float64)}

    # ---------------- per-kernel durations: HIP events around kernel_reps back-to-back launches of
    # one kernel (rotating input copies, so weights and caches stay cold), on the launch stream.
    # --kernel-in-step adds, for a step of several calls, kernel_reps whole steps in a row with an
    # event pair around each call: the chip holds its power limit during the large-batch steps,
    # and a loop of the partial pass alone runs it at a lower clock than the steps do (each event
    # pair adds a few microseconds of its own).
    single = one_launch_step(wl, args.num_splits)
    if single:
        names = ["step"]
    else:
        names = ["absorb", "partial", "combine_uv"] if fused_combine_uv(wl) else ["absorb", "partial", "combine", "uv"]
    reps = args.kernel_reps

    def launch(name, r):
        c = copies[r % R]
        if name == "step":
            ops.mla_decode_step(c["q_C"], c["q_R"], c["W_UK"], c["W_UV"], caches[r % R], c["lens"], wl.n_max,
                                step.workspace, out=step.out, q_abs=step.q_abs, o_latent=step.o_latent,
                                lse=step.lse, scale=step.scale, stream=stream)
        elif name == "absorb":
            ops.mla_absorb_q(c["q_C"], c["W_UK"], out=step.q_abs, stream=stream)
        elif name == "partial":   # as in the step: spare workgroups (small batch) warm W_UV
            ops.mla_decode_partial_warm(step.q_abs, c["q_R"], caches[r % R], c["lens"], wl.n_max, step.scale,
                                        pws, c["W_UV"], num_splits=args.num_splits, stream=stream)
        elif name == "combine":
            ops.mla_decode_combine(c["lens"], wl.n_max, wl.B, wl.H, wl.d_c, pws, step.o_latent,
                                   step.lse, num_splits=args.num_splits, stream=stream)
        elif name == "combine_uv":
            ops.mla_decode_combine_uv(c["lens"], wl.n_max, pws, c["W_UV"], step.o_latent, out=step.out,
                                      lse=step.lse, num_splits=args.num_splits, stream=stream)
        else:
            ops.mla_uv_out(step.o_latent, c["W_UV"], out=step.out, stream=stream)

    pws = None
    if not single:
        pws = torch.empty(max(1, ops.mla_decode_workspace_bytes(wl.B, wl.H, wl.d_c, wl.n_max, args.num_splits)),
                          dtype=torch.uint8, device=dev)
    def back_to_back(name):
        ka, kb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)  # keep the GPU busy while the host enqueues the launches
        ka.record(stream)
        for r in range(reps):
            launch(name, r)
        kb.record(stream)
        kb.synchronize()
        return ka.elapsed_time(kb) * 1e3 / reps

    kern_us, kern_in_step = {}, {}
    with torch.cuda.stream(stream):
        for name in names:
            kern_us[name] = back_to_back(name)
        if args.kernel_in_step and not single:
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(reps)]
            torch.cuda._sleep(20_000_000)
            for r in range(reps):
                ev[r][0].record(stream)
                for k, name in enumerate(names):
                    launch(name, r)
                    ev[r][k + 1].record(stream)
            ev[-1][-1].synchronize()
            for k, name in enumerate(names):
                kern_in_step[name] = float(np.mean([ev[r][k].elapsed_time(ev[r][k + 1]) for r in range(reps)])) * 1e3
    torch.cuda.synchronize()
    if single:
        err = int(step.workspace[:4].view(torch.int32)[0].item())
        if err:
            raise SystemExit(f"mla_decode_step: a wait between workgroups gave up (error word {err})")

    ab, per_tok = alg_bytes(wl, sum_len)
    af = alg_flops(wl, sum_len)
    step_bytes = ab["absorb"] + ab["partial"] + ab["combine"] + ab["uv"]
    step_flops = af["absorb"] + af["partial"] + af["uv"]
    ab["step"], af["step"] = step_bytes, step_flops
    value = sum_len / (ms_per_step * 1e-3)
    dom = max(names, key=lambda n: kern_us[n])
    kname = "k_step_b1" if single else kernel_names(wl)[dom]
    achieved_gbps = ab[dom] / (kern_us[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_profiles(kname, wl.name), "alg_bytes_per_launch": ab[dom],
                "avg_us": round(kern_us[dom], 3)}
    mfma_name = "step" if single else "partial"
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "latents/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else ("fp8-e4m3 latents, bf16 MFMA" if wl.dtype == "fp8" else "f32"),
        "data": "synthetic (seeded; random-init weights, no trained checkpoint)",
        "config": {"workload": wl.description, "B": wl.B, "H": wl.H, "d_c": wl.d_c, "d_R": wl.d_R,
                   "sum_len": sum_len, "layout": wl.layout,
                   "form": "one launch (mla_decode_step)" if single else "absorb, partial, combine(+uv)",
                   "num_splits": 32 if single else W, "graph": use_graph, "input_copies_rotated": R},
        "step_spread": spread,
        "hbm_TBps_step": round(step_bytes / (ms_per_step * 1e-3) / 1e12, 3),
        "step_alg_bytes": step_bytes,
        "kernels_us": {k: round(v, 3) for k, v in kern_us.items()},
        "kernels_frac_of_hbm_peak": {k: round(ab[k] / (kern_us[k] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4) for k in names},
        "mfma_util_algorithmic": {"kernel": kname,
                                  "frac_of_bf16_peak": round(af[mfma_name] / (kern_us[mfma_name] * 1e-6) / 1e12
                                                             / BF16_PEAK_TFLOPS, 4)},
        "roofline": roofline,
        "env": environment(),
    }
    if kern_in_step:
        out["kernels_us_in_step"] = {k: round(v, 3) for k, v in kern_in_step.items()}
    print("[bench] checking the timed run's outputs against the oracle", file=sys.stderr, flush=True)
    out["rel_l2_sampled"] = sampled_parity(inp, got)
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def main_append(args):
    """The cache write of one decode step (mla_cache_append) at the V3 shape: B new tokens, hidden
    size 7168, latent 512 and rope key 64 written as bf16 into a split cache.  Weights are rotated
    over enough copies to miss the 256 MB Infinity Cache; one HIP graph holds one call per copy."""
    import numpy as np
    import torch
    from mla_latent_kv_attn_amd import ops
    from workloads.append import make_append_inputs

    B, D, N = args.append_batch, 7168, 64
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    inp = make_append_inputs(B, D)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    base = {"h": bf16(inp.h), "W_DKV": bf16(inp.W_DKV), "W_KR": bf16(inp.W_KR)}
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    R = max(1, min(128, math.ceil(args.rotate_mb * 1e6 / per_copy)))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    pos = torch.from_numpy((np.arange(B) * 7 + 3).astype(np.int32) % N).to(dev)
    lat = torch.zeros((B, N, 512), dtype=torch.bfloat16, device=dev)
    rope = torch.zeros((B, N, 64), dtype=torch.bfloat16, device=dev)
    cache = ops.Cache.split(lat, rope)
    ws = torch.empty(ops.mla_cache_append_workspace_bytes(B, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def one(i):
        c = copies[i % R]
        ops.mla_cache_append(c["h"], c["W_DKV"], c["W_KR"], pos, cache, workspace=ws, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, R)):
            one(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(R):
            one(i)
    torch.cuda.synchronize()
    reps = max(1, math.ceil(args.steps / R))
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    calls = reps * R
    us = e0.elapsed_time(e1) * 1e3 / calls
    alg = 576 * D * 2 + B * D * 2 + B * 4 + B * (512 + 64) * 2     # weights, h, positions, the new rows
    achieved = alg / (us * 1e-6) / 1e9
    out = {
        "metric": "cache rows appended/sec (MLA cache write, V3 shape)",
        "value": round(B / (us * 1e-6), 1), "unit": "rows/s", "n_gpus": 1, "steps": calls, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; random-init weights, no trained checkpoint)",
        "config": {"workload": f"V3 cache write, B={B} new tokens, hidden 7168 -> latent 512 + rope 64, bf16 split cache",
                   "B": B, "D": D, "graph": True, "input_copies_rotated": R},
        "roofline": {"bound": "hbm", "kernel": "mla_cache_append (%s)"
                                                % ("k_proj_gemv, writing the cache row" if B <= 8 else
                                                   "k_append_proj + k_append_finalize"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "alg_bytes_per_launch": alg,
                     "avg_us": round(us, 3)},
    }
    if args.cpu_seconds > 0:
        import threadpoolctl
        from oracle import decode_bf16
        from oracle.cache_write import cache_row
        cores = len(os.sched_getaffinity(0))
        h, Wd, Wr = decode_bf16(inp.h), decode_bf16(inp.W_DKV), decode_bf16(inp.W_KR)
        pnp = pos.cpu().numpy()
        with threadpoolctl.threadpool_limits(limits=cores):
            info = threadpoolctl.threadpool_info()
            threads = max([i.get("num_threads", 1) for i in info] or [1])
            n, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < args.cpu_seconds:
                cache_row(h, Wd, Wr, pnp)
                n += 1
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n * B / dt, 1), "unit": "rows/s", "cores": threads, "kind": "oracle",
                               "sample": f"{n} oracle calls on the same {B} tokens (float64 numpy), {dt:.1f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def main_proj(args):
    """The projections around the attention core at the V3 shape (hidden 7168, d_q 1536, 128 heads,
    d_h 128, d_c 512, d_R 64), B new tokens, bf16 weights rotated over enough copies to miss the
    256 MB Infinity Cache, each call timed in a HIP graph.
      query: mla_query_proj (c_q = W_DQ h, q_C = W_UQ c_q, q_R = RoPE(W_QR c_q)) then mla_absorb_q
             (q' = W_UK^T q_C), beside mla_absorb_q_folded (q' = W_QK c_q with the folded weights);
      out:   mla_uv_out (o = W_UV o_lat) then mla_out_proj (W_O o), beside mla_out_proj with the
             folded W_OV = W_O W_UV applied to o_lat."""
    import numpy as np
    import torch
    from mla_latent_kv_attn_amd import ops
    from workloads.proj import make_output_inputs, make_query_inputs

    B = args.append_batch
    D, d_q, H, d_h, d_c, d_R = 7168, 1536, 128, 128, 512, 64
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def nbytes(ts):
        return sum(t.numel() * t.element_size() for t in ts)

    def rotated(base):
        R = max(1, min(64, math.ceil(args.rotate_mb * 1e6 / nbytes(base.values()))))
        return [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]

    def timed(copies, call):
        us, calls = _graph_time_us([lambda c=c: call(c) for c in copies], args.steps, stream)
        return us, calls

    if args.row == "query":
        inp = make_query_inputs(B)
        h, pos = bf16(inp.h), torch.from_numpy(inp.pos).to(dev)
        c_q = torch.empty(B, d_q, dtype=torch.bfloat16, device=dev)
        q_C = torch.empty(B, H, d_h, dtype=torch.bfloat16, device=dev)
        q_R = torch.empty(B, H, d_R, dtype=torch.bfloat16, device=dev)
        q_abs = torch.empty(B, H, d_c, dtype=torch.bfloat16, device=dev)
        wsz = max(ops.mla_query_workspace_bytes(B, D, d_q, H, d_h, d_R), ops.mla_proj_workspace_bytes(B, H * d_c, d_q))
        ws = torch.empty(max(wsz, 16), dtype=torch.uint8, device=dev)
        base = {"W_DQ": bf16(inp.W_DQ), "W_UQ": bf16(inp.W_UQ), "W_QR": bf16(inp.W_QR)}
        t_proj, calls = timed(rotated(base), lambda c: ops.mla_query_proj(
            h, c["W_DQ"], c["W_UQ"], c["W_QR"], pos, H, c_q=c_q, q_C=q_C, q_R=q_R, workspace=ws, stream=stream))
        uk = rotated({"W_UK": bf16(inp.W_UK)})
        t_abs, _ = timed(uk, lambda c: ops.mla_absorb_q(q_C, c["W_UK"], out=q_abs, stream=stream))
        W_QK = ops.mla_fold_q(base["W_UQ"], uk[0]["W_UK"])
        torch.cuda.synchronize()
        t_fold, _ = timed(rotated({"W_QK": W_QK}), lambda c: ops.mla_absorb_q_folded(
            c_q, c["W_QK"], out=q_abs, workspace=ws, stream=stream))
        w_main = nbytes(base.values())
        alg = w_main + B * D * 2 + B * d_q * 2 * 2 + B * H * (d_h + d_R) * 2 + B * 4
        achieved = alg / (t_proj * 1e-6) / 1e9
        step_us = t_proj + t_abs
        out = {
            "metric": "query-side tokens/sec (c_q, q_C, q_R and the absorbed q', V3 shape)",
            "value": round(B / (step_us * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": calls,
            "warmup": args.warmup, "ms_per_step": round(step_us / 1e3, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; random-init weights, no trained checkpoint)",
            "config": {"workload": f"V3 query side, B={B} new tokens, hidden 7168 -> c_q 1536 -> 128 x (128 + 64), "
                                   "then W_UK^T q_C", "B": B, "graph": True},
            "kernels_us": {"mla_query_proj": round(t_proj, 3), "mla_absorb_q": round(t_abs, 3),
                           "mla_absorb_q_folded": round(t_fold, 3)},
            "folded_variant": {"us": round(t_proj + t_fold, 3), "note": "the folded path still needs c_q and q_R "
                               "(timed here as the whole mla_query_proj); its own weight read is W_QK",
                               "weight_bytes_unfolded": w_main + H * d_h * d_c * 2,
                               "weight_bytes_folded": nbytes([base["W_DQ"], base["W_QR"], W_QK])},
            "roofline": {"bound": "hbm", "kernel": "mla_query_proj (%s)" % ("k_proj_gemv x2" if B <= 4 else
                                                                           "k_proj_gemv, k_proj_mfma + k_proj_reduce"
                                                                           if B <= 8 else
                                                                           "k_proj_mfma + k_proj_reduce, x2"),
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                         "alg_bytes_per_launch": alg, "avg_us": round(t_proj, 3)},
        }
    else:
        inp = make_output_inputs(B)
        o_lat = torch.from_numpy(inp.o_lat).to(dev)
        o = torch.empty(B, H, d_h, dtype=torch.float32, device=dev)
        y = torch.empty(B, D, dtype=torch.float32, device=dev)
        ws = torch.empty(max(ops.mla_proj_workspace_bytes(B, D, H * d_c), 16), dtype=torch.uint8, device=dev)
        base = {"W_O": bf16(inp.W_O), "W_UV": bf16(inp.W_UV)}
        copies = rotated(base)
        t_uv, calls = timed(copies, lambda c: ops.mla_uv_out(o_lat, c["W_UV"], out=o, stream=stream))
        t_o, _ = timed(copies, lambda c: ops.mla_out_proj(o, c["W_O"], out=y, workspace=ws, stream=stream))
        W_OV = ops.mla_fold_o(base["W_O"], base["W_UV"])
        torch.cuda.synchronize()
        t_fold, _ = timed(rotated({"W_OV": W_OV}), lambda c: ops.mla_out_proj(o_lat, c["W_OV"], out=y, workspace=ws,
                                                                             stream=stream))
        alg = nbytes([base["W_O"]]) + B * H * d_h * 4 + B * D * 4
        achieved = alg / (t_o * 1e-6) / 1e9
        step_us = t_uv + t_o
        out = {
            "metric": "output-side tokens/sec (W_UV then W_O, V3 shape)",
            "value": round(B / (step_us * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": calls,
            "warmup": args.warmup, "ms_per_step": round(step_us / 1e3, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; random-init weights, no trained checkpoint)",
            "config": {"workload": f"V3 output side, B={B} tokens, 128 x 512 latent outputs -> 128 x 128 -> 7168",
                       "B": B, "graph": True},
            "kernels_us": {"mla_uv_out": round(t_uv, 3), "mla_out_proj": round(t_o, 3),
                           "mla_out_proj_folded": round(t_fold, 3)},
            "folded_variant": {"us": round(t_fold, 3), "weight_bytes_unfolded": nbytes(base.values()),
                               "weight_bytes_folded": nbytes([W_OV])},
            "roofline": {"bound": "hbm", "kernel": "mla_out_proj (%s)" % ("k_proj_gemv" if B <= 8 else
                                                                         "k_proj_mfma + k_proj_reduce"),
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                         "alg_bytes_per_launch": alg, "avg_us": round(t_o, 3)},
        }
    if args.cpu_seconds > 0:
        import threadpoolctl
        import oracle.output as oo
        import oracle.query as oq
        from oracle import decode_bf16
        cores = len(os.sched_getaffinity(0))
        if args.row == "query":
            Wd, Wu, Wr, Wk = (decode_bf16(x) for x in (inp.W_DQ, inp.W_UQ, inp.W_QR, inp.W_UK))
            hh = decode_bf16(inp.h)

            def once():
                qc, _ = oq.q_up(Wu, Wr, oq.q_down(Wd, hh), inp.pos, H)
                oq.absorb(Wk, qc)
        else:
            Wo, Wv = decode_bf16(inp.W_O), decode_bf16(inp.W_UV)

            def once():
                oo.out_proj(Wo, np.einsum("hik,bhk->bhi", Wv, inp.o_lat.astype(np.float64)))
        with threadpoolctl.threadpool_limits(limits=cores):
            info = threadpoolctl.threadpool_info()
            threads = max([i.get("num_threads", 1) for i in info] or [1])
            n, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < args.cpu_seconds:
                once()
                n += 1
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n * B / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"{n} oracle passes over the same {B} tokens (float64 numpy), {dt:.1f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def main_layer(args):
    """One whole attention layer's decode step (DecodeLayer) at the V3 shape: B sequences of
    --layer-context tokens after the new token is appended; bf16 weights (373 MB per layer) and
    caches rotated over enough copies to miss the 256 MB Infinity Cache, the calls in a HIP graph."""
    import numpy as np
    import torch
    from mla_latent_kv_attn_amd import ops
    from mla_latent_kv_attn_amd.layer import DecodeLayer
    from workloads.layer import make_layer_inputs

    B, N = args.append_batch, args.layer_context
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    inp = make_layer_inputs([N - 1] * B, N)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    base_w = {k: bf16(v) for k, v in inp.weights.items()}
    w_bytes = sum(t.numel() * 2 for t in base_w.values())
    cache_bytes = B * N * (512 + 64) * 2
    R = max(1, min(16, math.ceil(args.rotate_mb * 1e6 / (w_bytes + cache_bytes))))
    layers = []
    for r in range(R):
        w = base_w if r == 0 else {k: v.clone() for k, v in base_w.items()}
        cache = ops.Cache.split(bf16(inp.latent), bf16(inp.rope))
        layers.append(DecodeLayer(w, cache, B, max_len=N))
    h = bf16(inp.h)
    pos = torch.from_numpy(inp.pos).to(dev)
    seq_lens = torch.from_numpy(inp.pos + 1).to(dev)
    us, calls = _graph_time_us([lambda L=L: L(h, pos, seq_lens, stream=stream) for L in layers], args.steps, stream)
    alg = w_bytes + cache_bytes + B * 7168 * 2 + B * 7168 * 4
    achieved = alg / (us * 1e-6) / 1e9
    out = {
        "metric": "attention-layer decode steps/sec x tokens (V3 shape, whole layer)",
        "value": round(B / (us * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": calls, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; random-init weights, no trained checkpoint)",
        "config": {"workload": f"V3 attention layer decode, B={B} sequences x {N} tokens: cache write, query side, "
                               "absorbed attention, W_UV, W_O", "B": B, "context": N, "graph": True,
                   "copies_rotated": R},
        "roofline": {"bound": "hbm", "kernel": "whole layer (11-14 kernels)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "alg_bytes_per_launch": alg, "avg_us": round(us, 3)},
    }
    if args.cpu_seconds > 0:
        import threadpoolctl
        import oracle
        import oracle.output as oo
        import oracle.query as oq
        from oracle import decode_bf16
        from oracle.cache_write import cache_row, encode_bf16
        from workloads.configs import Workload
        from workloads.gen import DecodeInputs
        cores = len(os.sched_getaffinity(0))
        W = {k: decode_bf16(v) for k, v in inp.weights.items()}
        hh = decode_bf16(inp.h)

        def held(x):
            return decode_bf16(encode_bf16(x))

        def once():
            row = cache_row(hh, W["W_DKV"], W["W_KR"], inp.pos)
            q_C, q_R = oq.q_up(W["W_UQ"], W["W_QR"], held(oq.q_down(W["W_DQ"], hh)), inp.pos, 128)
            lat = decode_bf16(inp.latent).astype(np.float32)
            rp = decode_bf16(inp.rope).astype(np.float32)
            lat[:, N - 1] = decode_bf16(row["c_bf16"])
            rp[:, N - 1] = decode_bf16(row["k_R_bf16"])
            wl = Workload("layer", seed=0, B=B, H=128, d_h=128, d_c=512, d_R=64, n_max=N, len_lo=N, len_hi=N,
                          dtype="f32", layout="split")
            d = DecodeInputs(wl=wl, lens=np.full(B, N, np.int32), q_C=held(q_C).astype(np.float32),
                             q_R=held(q_R).astype(np.float32), W_UK=W["W_UK"].astype(np.float32),
                             W_UV=W["W_UV"].astype(np.float32), latent=lat, rope=rp)
            oo.out_proj(W["W_O"], oracle.decode(d, want_diag=False)["o"])

        with threadpoolctl.threadpool_limits(limits=cores):
            info = threadpoolctl.threadpool_info()
            threads = max([i.get("num_threads", 1) for i in info] or [1])
            n, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < args.cpu_seconds:
                once()
                n += 1
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n * B / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"{n} oracle layer passes over the same {B} tokens (float64 numpy), {dt:.1f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def _graph_time_us(fns, steps, stream):
    """Average time of one call, over a graph holding the calls fns[0..n-1] (one per input copy)."""
    import torch
    with torch.cuda.stream(stream):
        for f in fns:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(steps / len(fns)))
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * len(fns)), reps * len(fns)


def main_mha(args):
    """Same-dimension comparison: plain MHA decode with explicit per-head K/V (keys 192, values 128
    per head, H = 128) on the lengths of a latent-path workload, timed beside that workload's
    attention pass (mla_decode_attn: partial + combine, q' and q_R in, o_latent out).  K/V and q are
    seeded normal bf16 tensors drawn on the device (the MHA cache of the paged 32k workload is 43 GB)."""
    import numpy as np
    import torch
    from mla_latent_kv_attn_amd import ops
    from workloads import make_inputs
    from workloads.configs import WORKLOADS
    from workloads.device import device_cache, to_device

    wl = WORKLOADS[args.config]
    if wl.dtype != "bf16":
        raise SystemExit("--row mha compares against a bf16 workload (configs 2-4)")
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    inp = make_inputs(wl, poison=False)
    lens_np = inp.lens.astype(np.int64)
    sum_len = int(lens_np.sum())
    B, H, N = wl.B, wl.H, wl.n_max
    # ---- MHA: K/V bytes per cached token 2 * H * (192 + 128)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    kv_bytes = B * H * N * (192 + 128) * 2
    R = max(1, min(4, math.ceil(args.rotate_mb * 1e6 / kv_bytes)))
    print(f"[bench] MHA caches {kv_bytes / 1e9:.2f} GB x {R}", file=sys.stderr, flush=True)
    mcopies = []
    for _ in range(R):
        K = torch.randn((B, H, N, 192), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        V = torch.randn((B, H, N, 128), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        mcopies.append((K, V))
    q = torch.randn((B, H, 192), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    lens = torch.from_numpy(inp.lens).to(dev)
    ws = torch.empty(ops.mla_mha_decode_workspace_bytes(B, H, N), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, 128), dtype=torch.float32, device=dev)
    mha_fns = [(lambda c=c: ops.mla_mha_decode(q, c[0], c[1], lens, N, workspace=ws, out=out, stream=stream))
               for c in mcopies]
    mha_us, calls = _graph_time_us(mha_fns, max(10, args.steps // 10), stream)
    del mcopies
    torch.cuda.empty_cache()
    # ---- the latent path's attention pass on the same lengths
    base = to_device(inp, dev)
    per_copy = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    RL = max(1, min(64, math.ceil(args.rotate_mb * 1e6 / per_copy)))
    copies = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()} for _ in range(RL - 1)]
    caches = [device_cache(inp, c) for c in copies]
    q_abs = [ops.mla_absorb_q(c["q_C"], c["W_UK"]) for c in copies]
    mws = torch.empty(ops.mla_decode_workspace_bytes(B, H, wl.d_c, N), dtype=torch.uint8, device=dev)
    o_lat = torch.empty((B, H, wl.d_c), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(wl.d_h + wl.d_R)
    mla_fns = [(lambda i=i: ops.mla_decode_attn(q_abs[i], copies[i]["q_R"], caches[i], copies[i]["lens"], N, scale=scale,
                                                workspace=mws, o_latent=o_lat, want_lse=False,
                                                stream=stream)) for i in range(RL)]
    mla_us, _ = _graph_time_us(mla_fns, args.steps, stream)
    mha_bytes = sum_len * H * (192 + 128) * 2 + B * H * (192 * 2 + 128 * 4)
    mla_bytes = sum_len * (wl.d_c + wl.d_R) * 2 + B * H * ((wl.d_c + wl.d_R) * 2 + wl.d_c * 4)
    ach = mha_bytes / (mha_us * 1e-6) / 1e9
    out_j = {
        "metric": "cached tokens/sec, same-dimension MHA decode (comparison with the latent path)",
        "value": round(sum_len / (mha_us * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": calls,
        "warmup": args.warmup, "ms_per_step": round(mha_us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded; device-drawn normal K/V and q)",
        "config": {"workload": f"MHA decode at V3 head sizes (H={H}, keys 192, values 128) on the lengths of "
                               f"{wl.description}", "B": B, "H": H, "sum_len": sum_len, "graph": True,
                   "input_copies_rotated": R},
        "roofline": {"bound": "hbm", "kernel": "mla_mha_decode (k_mha_partial + k_mha_combine)",
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None, "alg_bytes_per_launch": mha_bytes,
                     "avg_us": round(mha_us, 3)},
        "latent_path": {"call": "mla_decode_attn (partial + combine)", "us": round(mla_us, 3),
                        "alg_bytes": mla_bytes, "bytes_ratio_mha_over_mla": round(mha_bytes / mla_bytes, 2),
                        "time_ratio_mha_over_mla": round(mha_us / mla_us, 2)},
    }
    if args.cpu_seconds > 0:
        import threadpoolctl
        from oracle import attend
        cores = len(os.sched_getaffinity(0))
        L0 = int(inp.lens[0])
        rng = np.random.default_rng(0)
        Kh = rng.standard_normal((L0, 192))
        Vh = rng.standard_normal((L0, 128))
        qh = rng.standard_normal(192)
        with threadpoolctl.threadpool_limits(limits=cores):
            info = threadpoolctl.threadpool_info()
            threads = max([i.get("num_threads", 1) for i in info] or [1])
            n, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < args.cpu_seconds:
                attend(Kh, Vh, qh, 1.0 / math.sqrt(192))
                n += 1
            dt = time.perf_counter() - t0
        out_j["cpu_baseline"] = {"value": round(n * L0 / dt, 1), "unit": "tokens/s (one head)", "cores": threads,
                                 "kind": "oracle", "sample": f"{n} oracle attend calls, one head over {L0} tokens "
                                                             f"(float64 numpy), {dt:.1f} s"}
    else:
        out_j["cpu_baseline"] = None
    print(json.dumps(out_j), flush=True)


def traffic_from_profiles(kname: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if a committed measurement exists for
    this kernel, this workload and the current kernel source."""
    path = os.path.join(PROFILES, f"{kname}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash(KERNEL_SOURCES[kname]):
        return None
    return d.get("hbm_bytes_per_launch")


if __name__ == "__main__":
    main()
