"""Benchmark of the routed-expert MoE layer forward over 4-bit codebook experts on one MI355X.

One step = one pass of the whole hot path (route -> permute -> gate|up+SwiGLU -> down ->
unpermute/combine; routing and permutation as one launch for few tokens) over one batch of
synthetic tokens, with inputs resident in HBM.

Headline workload (the line's ``value``): the GLM-shaped single-layer decode (hidden 6144,
intermediate 2048, 256 experts, top-8, 8 tokens), HBM-bound. Every step routes a fresh batch
of tokens, and the steps rotate over several device copies of the layer's weights so that no
step reads weights that the previous steps left in the ~256 MB last-level cache (MALL).

Without ``--config`` the same run also measures the other four workloads, one after the other,
with the same step counts, and reports each in the line's ``configs`` block: the tiny layer,
the 2048-token Zipf prefill, the 32-layer decode stack (64 tokens) and the 8192-token Zipf
prefill with E2M1 experts and a channel permutation. ``--config N`` prints workload N alone.

Every workload reports:
* ``value``: tokens/s of the timed region (HIP events only at its two ends, K steps);
* ``step_ms`` / ``tokens_per_s_dist``: median, p10, p90 and n over the K steps of a second
  pass over the same batches with events at every step boundary and around the two
  projections (an event between two kernels idles the GPU for a few microseconds, which is why
  ``value`` comes from the first pass);
* ``roofline`` for the dominant kernel (the gate|up projection): algorithmic bytes (decode) or
  flops (prefill) per launch over its average duration from those events, against MI355X's
  published peak (8 TB/s HBM, 2.5 PFLOP/s dense bf16); where both bounds are close (the 2048-token
  prefill) the fraction is max(F/P, B/BW) / t; ``traffic`` is the kernel's HBM bytes per
  launch from the rocprofv3 counter summaries in ``profiles/`` (null when none matches the
  current kernel source);
* ``layer``: the same fractions for the whole step;
* ``cpu_baseline``: the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

METRIC = "routed-MoE layer tokens/s; decode HBM GB/s and prefill MFMA util vs peak"

HEADLINE = 2
OTHER_CONFIGS = (1, 3, 4, 5)


def expert_bytes(H, I):
    """Stored bytes of one expert: codes (4 bit/weight) + E8M0 scales (1 byte per 32)."""
    gate_up = 2 * (I * H // 2 + I * H // 32)
    down = H * I // 2 + H * I // 32
    return gate_up, down


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a decode step is ~0.25 ms, and the first steps after a synchronize run slower than the
    # steady state (8-token layer, GPU time per step over 20 / 100 / 400 back-to-back steps:
    # 245 / 223 / 217 us), so the defaults time enough steps for the steady state to dominate
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="measure this workload alone (default: the decode headline plus the "
                         "other four in the configs block)")
    ap.add_argument("--no-configs", action="store_true",
                    help="without --config: the headline workload only")
    ap.add_argument("--copies", type=int, default=4,
                    help="device copies of the weights rotated over the steps (MALL-cold reads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2,
                    help="tokens of the headline workload the CPU oracle is timed on")
    ap.add_argument("--fused", action="store_true",
                    help="decode workloads: the whole layer as one cooperative launch "
                         "(moeq_moe_decode) instead of the five per-step calls")
    ap.add_argument("--shared", action="store_true",
                    help="layer workloads: add a shared expert (the routed experts' shape and "
                         "format, every token, weight 1) on a side stream, summed in the combine")
    ap.add_argument("--encode", action="store_true",
                    help="time the on-GPU encoder instead: weighted grid fit, per-expert arm "
                         "choice and packing of one GLM-shaped layer of bf16 experts")
    ap.add_argument("--router", action="store_true",
                    help="stack: route every layer from its activations through a bf16 router "
                         "(logits = X . Wr^T, sigmoid gating) instead of pre-drawn logits")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    return ap.parse_args()


KERNEL_SOURCES = {
    "decode_kernel<true>": ["codebook_quantized_moe_amd/csrc/gemm_decode.hip",
                            "codebook_quantized_moe_amd/csrc/moeq_device.h"],
    "prefill_kernel<true>": ["codebook_quantized_moe_amd/csrc/gemm_prefill.hip",
                             "codebook_quantized_moe_amd/csrc/moeq_device.h"],
    "decode_layer_kernel": ["codebook_quantized_moe_amd/csrc/gemm_decode.hip",
                            "codebook_quantized_moe_amd/csrc/moeq_device.h",
                            "codebook_quantized_moe_amd/csrc/route_device.h",
                            "codebook_quantized_moe_amd/csrc/permute_device.h",
                            "codebook_quantized_moe_amd/csrc/combine_device.h"],
}


def source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled(tag, kernel, workload):
    """The `tag:` line of the rocprofv3 summaries in profiles/ for `kernel` on `workload`, as a
    dict, or None when there is none or the kernel's source has changed since the counters were
    taken (the summaries record the source hash)."""
    digest = source_digest(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                if not line.startswith(tag + ":"):
                    continue
                kv = dict(item.split("=", 1) for item in line.split()[1:])
                if kv.get("kernel") == kernel and kv.get("workload") == workload:
                    return kv if kv.get("source_sha256") == digest else None
    return None


def profiled_traffic(kernel, workload):
    """HBM bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, see the summary)."""
    kv = profiled("traffic", kernel, workload)
    return int(kv["total_bytes"]) if kv else None


def profiled_busy(kernel, workload):
    """MFMA and VALU busy fractions of the kernel from its counter summary, if current."""
    kv = profiled("busy", kernel, workload)
    if not kv:
        return None
    return {k: float(v) for k, v in kv.items() if k not in ("kernel", "workload", "source_sha256")}


def dist(values):
    a = np.asarray(values, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def tok_dist(T, step_ms):
    d = dist(step_ms)
    # tokens/s of the median / p10 / p90 step (a faster step is a higher rate: p10 <-> p90)
    return {"median": round(T / d["median"] * 1e3, 2), "p10": round(T / d["p90"] * 1e3, 2),
            "p90": round(T / d["p10"] * 1e3, 2), "n": d["n"]}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(cfg, lw, x, logits, n_tokens):
    """The fp64 oracle, as it stands, on the first n_tokens tokens of one batch."""
    import oracle
    threads = blas_threads()
    toks = list(range(min(n_tokens, cfg.T)))
    t0 = time.perf_counter()
    oracle.layer_forward(x, logits, cfg.k, lw, tokens=toks)
    dt = time.perf_counter() - t0
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(toks)} of the {cfg.T} tokens of one batch (all routing, the "
                      f"sampled tokens' experts), {dt:.1f} s, numpy fp64 "
                      f"(BLAS threads {threads}, os.cpu_count {os.cpu_count()})"}


def cpu_baseline_stack(cfg, w, x_bits, logits):
    """The fp64 oracle on token 0 through layer 0 of the stack (its 8 experts' bytes read back
    from the device), scaled to the stack: tokens/s = 1 / (layers x that time)."""
    import oracle
    import synth
    threads = blas_threads()
    ids = oracle.route_topk(logits, cfg.k)[0][0]
    E, H, I = cfg.E, cfg.H, cfg.I

    def host(t, e_list, shape):
        a = np.zeros(shape, np.uint8)           # untouched experts stay zero pages
        for e in e_list:
            a[e] = t[e].cpu().numpy()
        return a

    el = [int(e) for e in ids]
    lw = synth.LayerWeights(host(w.gate_codes, el, (E, I, H // 2)),
                            host(w.gate_scales, el, (E, I, H // 32)),
                            host(w.up_codes, el, (E, I, H // 2)),
                            host(w.up_scales, el, (E, I, H // 32)),
                            host(w.down_codes, el, (E, H, I // 2)),
                            host(w.down_scales, el, (E, H, I // 32)),
                            np.asarray(w.tables, np.float32), w.table_id.cpu().numpy())
    t0 = time.perf_counter()
    oracle.layer_forward(x_bits, logits, cfg.k, lw, tokens=[0])
    dt = time.perf_counter() - t0
    return {"value": 1.0 / (cfg.layers * dt), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"token 0 through layer 0 only ({dt:.1f} s, its 8 experts read back from "
                      f"the device), scaled to the {cfg.layers}-layer stack as 1 / "
                      f"({cfg.layers} x that time); numpy fp64 (BLAS threads {threads}, "
                      f"os.cpu_count {os.cpu_count()})"}


def roofline(kind, flops, nbytes, ms, kernel, traffic, busy=None):
    """Roofline figures of one launch (or step) of `ms` milliseconds. kind: "hbm", "mfma" or
    "both" (the larger of F/P and B/BW bounds it; frac = that bound / t)."""
    s = ms / 1e3
    gbs = nbytes / s / 1e9
    tfs = flops / s / 1e12
    hf, mf = gbs / HBM_PEAK_GBS, tfs / BF16_PEAK_TFLOPS
    if kind == "both":
        kind = "mfma" if flops / BF16_PEAK_TFLOPS >= nbytes / HBM_PEAK_GBS * 1e3 else "hbm"
    if kind == "hbm":
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(hf, 4)}
    else:
        r = {"bound": "mfma", "achieved": round(tfs, 1), "peak": BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(mf, 4)}
    r["traffic"] = traffic
    r["kernel"] = kernel
    r["hbm_frac"] = round(hf, 4)
    r["mfma_frac"] = round(mf, 4)
    if traffic is not None:
        r["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE, profiles/)"
        r["traffic_over_algorithmic"] = round(traffic / nbytes, 3)
    if busy is not None:
        r["counters"] = busy
    return r


def free_device():
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def measure_layer(args, cfg, cpu_tokens):
    """One single-layer workload; returns its record."""
    import torch
    import codebook_quantized_moe_amd as mq
    import synth

    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    dev = torch.device("cuda")
    print(f"bench: {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    t_gen = time.perf_counter()
    lw = synth.make_layer(cfg.cfg_id, E, H, I, e2m1_experts=cfg.e2m1, permute=cfg.permute)
    w0 = mq.DeviceWeights.from_host(lw)
    copies = [w0]
    # the library's choice of projection kernels: few rows per expert on average -> decode
    decode = T * k < 16 * E and T * k <= 4096
    ncopies = max(1, args.copies) if decode else 1
    for _ in range(ncopies - 1):
        copies.append(mq.DeviceWeights(*(t.clone() if torch.is_tensor(t) else t
                                         for t in (w0.gate_codes, w0.gate_scales, w0.up_codes,
                                                   w0.up_scales, w0.down_codes, w0.down_scales,
                                                   w0.tables, w0.table_id))))
    nb = args.warmup + args.steps
    # every step gets a fresh batch at decode sizes; the prefill workloads rotate over 4
    # batches (100 MB of activations each at 8k tokens: generating one per step would
    # dominate the run, and none of them fits in the MALL)
    nbd = nb if decode else min(nb, 4)
    xs, lgs = [], []
    for b in range(nbd):
        xs.append(synth.make_x(cfg.cfg_id, T, H, batch=b))
        lgs.append(synth.make_logits(cfg.cfg_id, T, E, zipf_s=cfg.zipf_s, batch=b))
    xd = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs]
    ld = [torch.from_numpy(l).to(dev) for l in lgs]
    sw = None
    if args.shared:
        sw = mq.DeviceWeights.from_host(synth.make_shared(cfg.cfg_id, H, I))
    L = mq.MoeLayer(T, H, I, E, k, shared_I=I if sw is not None else None)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    # touched experts of every batch, from the library's own routing
    touched_d = []
    for b in range(nbd):
        L.route(ld[b])
        L.permute()
        off = L.offsets.cpu().numpy()
        touched_d.append(int((np.diff(off) > 0).sum()))
    touched = [touched_d[b % nbd] for b in range(nb)]

    fused = args.fused and decode and sw is None

    def step(b, ev=None):
        """ev: events [step start, gate|up start, gate|up end (= down start), down end,
        step end, side start, side end] of this step, or None."""
        w = copies[b % ncopies]
        x, lg = xd[b % nbd], ld[b % nbd]
        if ev is not None:
            ev[0].record()
        if fused:
            if ev is not None:
                ev[1].record()
            L.forward_fused(x, lg, w)
            if ev is not None:
                ev[2].record()
                ev[3].record()
                ev[4].record()
            return
        if sw is not None:
            # the shared expert on the side stream, beside the routed path
            main = torch.cuda.current_stream()
            L.fork.record(main)
            L.side.wait_event(L.fork)
            if ev is not None:
                ev[5].record(L.side)
            L.shared_expert(x, sw, stream=L.side)
            if ev is not None:
                ev[6].record(L.side)
            L.join.record(L.side)
        L.route_permute(lg)
        if ev is not None:
            ev[1].record()
        L.gateup(x, w)
        if ev is not None:
            ev[2].record()
        L.down(w)
        if ev is not None:
            ev[3].record()
        if sw is not None:
            main.wait_event(L.join)
        L.combine(shared=sw is not None)
        if ev is not None:
            ev[4].record()

    # pass 1 (value): warmup, then the timed steps with events only around the whole region;
    # pass 2: the same steps again with events at the step boundaries and around the two
    # projections, for the per-step distribution and the kernels' durations
    print(f"bench: {cfg.name}: timing", file=sys.stderr, flush=True)
    for b in range(args.warmup):
        step(b)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for b in range(args.warmup, nb):
        step(b)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    timed = range(args.warmup, nb)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(nb)]
    for b in timed:
        step(b, ev[b])
    torch.cuda.synchronize()
    step_ms = [ev[b][0].elapsed_time(ev[b][4]) for b in timed]
    gu_ms = [ev[b][1].elapsed_time(ev[b][2]) for b in timed]
    dn_ms = [ev[b][2].elapsed_time(ev[b][3]) for b in timed]
    sh_ms = [ev[b][5].elapsed_time(ev[b][6]) for b in timed] if sw is not None else None

    gu_w, dn_w = expert_bytes(H, I)
    P = T * k
    gu_bytes = [touched[b] * gu_w + T * H * 2 + P * I * 2 for b in timed]
    dn_bytes = [touched[b] * dn_w + P * I * 2 + P * H * 4 + P * 4 for b in timed]
    step_bytes = [touched[b] * (gu_w + dn_w) + T * E * 4 + 2 * T * H * 2 for b in timed]
    flops_gu = 2.0 * P * 2 * I * H
    flops_dn = 2.0 * P * H * I
    step_flops = flops_gu + flops_dn
    if sw is not None:
        # the shared expert's weights, its intermediate out and in, z out and in
        sh_bytes = gu_w + dn_w + T * H * 2 + 2 * T * I * 2 + 2 * T * H * 4
        step_bytes = [sb + sh_bytes for sb in step_bytes]
        step_flops += 2.0 * T * 3 * H * I

    ms_per_step = total_ms / args.steps
    value = T * args.steps / (total_ms / 1e3)
    gu_avg = float(np.mean(gu_ms))
    dn_avg = float(np.mean(dn_ms))
    kind = "hbm" if decode else ("mfma" if cfg.T >= 4096 else "both")
    kernel = "decode_kernel<true>" if decode else "prefill_kernel<true>"
    if fused:
        # one kernel for the whole layer: its algorithmic bytes over its duration
        kernel = "decode_layer_kernel"
        roof = roofline("hbm", step_flops, float(np.mean(step_bytes)), gu_avg, kernel,
                        profiled_traffic(kernel, cfg.name), profiled_busy(kernel, cfg.name))
    else:
        roof = roofline(kind, flops_gu, float(np.mean(gu_bytes)), gu_avg, kernel,
                        profiled_traffic(kernel, cfg.name), profiled_busy(kernel, cfg.name))
    if cfg.name == "tiny":
        roof["note"] = ("launch-bound: a few microseconds per kernel launch dominate "
                        "(209 KB of weights, 6.3 MFLOP per step)")
    layer_roof = roofline(kind, step_flops, float(np.mean(step_bytes)), ms_per_step,
                          "whole step (all kernels and the gaps between them)", None)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "intermediate": I,
                   "experts": E, "top_k": k, "zipf_s": cfg.zipf_s,
                   "e2m1_experts": list(cfg.e2m1), "channel_permutation": cfg.permute,
                   "weight_copies": ncopies, "distinct_batches": nbd,
                   "shared_expert": sw is not None, "single_launch": fused},
        "roofline": roof,
        "step_ms": dist(step_ms),
        "tokens_per_s_dist": tok_dist(T, step_ms),
        "kernels": {"decode_layer": {"avg_us": round(gu_avg * 1e3, 2),
                                     "us": dist([m * 1e3 for m in gu_ms]),
                                     "bytes_per_launch": int(np.mean(step_bytes)),
                                     "GB_s": round(float(np.mean(step_bytes)) / gu_avg / 1e6, 1)}}
        if fused else {
            "gateup_swiglu": {"avg_us": round(gu_avg * 1e3, 2),
                              "us": dist([m * 1e3 for m in gu_ms]),
                              "bytes_per_launch": int(np.mean(gu_bytes)),
                              "GB_s": round(float(np.mean(gu_bytes)) / gu_avg / 1e6, 1),
                              "TFLOP_s": round(flops_gu / gu_avg / 1e9, 2)},
            "down": {"avg_us": round(dn_avg * 1e3, 2),
                     "us": dist([m * 1e3 for m in dn_ms]),
                     "bytes_per_launch": int(np.mean(dn_bytes)),
                     "GB_s": round(float(np.mean(dn_bytes)) / dn_avg / 1e6, 1),
                     "TFLOP_s": round(flops_dn / dn_avg / 1e9, 2)},
        },
        "layer": {"touched_experts_avg": round(float(np.mean([touched[b] for b in timed])), 2),
                  "algorithmic_bytes_per_step": int(np.mean(step_bytes)),
                  "algorithmic_flops_per_step": step_flops,
                  "step_GB_s": round(float(np.mean(step_bytes)) / ms_per_step / 1e6, 1),
                  "step_TFLOP_s": round(step_flops / ms_per_step / 1e9, 2),
                  "step_hbm_frac": layer_roof["hbm_frac"],
                  "step_mfma_frac": layer_roof["mfma_frac"],
                  "step_roofline_frac": layer_roof["frac"],
                  "step_bound": layer_roof["bound"]},
        "input_setup_s": round(t_gen, 1),
    }
    if sw is not None:
        sh_us = float(np.mean(sh_ms)) * 1e3
        rec["shared_expert"] = {"avg_us_on_side_stream": round(sh_us, 2),
                                "bytes_per_call": int(sh_bytes),
                                "GB_s": round(sh_bytes / sh_us / 1e3, 1),
                                "TFLOP_s": round(2.0 * T * 3 * H * I / sh_us / 1e6, 2)}

    # the router front end (logits = X . Wr^T, bf16 in, fp32 out) on the same batches, timed on
    # its own after the step: the workload's logits are drawn, so it is not part of the step
    wr = torch.from_numpy(synth.make_router(cfg.cfg_id, E, H).view(np.int16)).to(dev)
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nb)]
    for b in range(nb):
        rev[b][0].record()
        L.router(xd[b % nbd], wr)
        rev[b][1].record()
    torch.cuda.synchronize()
    r_us = float(np.mean([rev[b][0].elapsed_time(rev[b][1]) for b in timed])) * 1e3
    r_bytes = E * H * 2 + T * H * 2 + T * E * 4
    rec["router"] = {"avg_us": round(r_us, 2), "bytes_per_launch": r_bytes,
                     "GB_s": round(r_bytes / r_us / 1e3, 1),
                     "hbm_frac": round(r_bytes / r_us / 1e3 / HBM_PEAK_GBS, 4),
                     "TFLOP_s": round(2.0 * T * E * H / r_us / 1e6, 2)}

    if args.pmc_calibrate:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()
        rec["pmc_calibration_copy_bytes"] = 256 << 20

    del copies, w0, xd, ld, L, sw
    free_device()
    if not args.no_cpu_baseline:
        print(f"bench: {cfg.name}: cpu baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, lw, xs[0], lgs[0], cpu_tokens)
    else:
        rec["cpu_baseline"] = None
    return rec


def measure_stack(args, cfg):
    """The 32-layer stack decode (64 tokens): one step = the forward through every layer, the
    MoE output added to X in place. The layers' codes and scales are drawn on the device
    (uniform code bytes, scale bytes 119..123, i.e. the magnitude of N(0, 0.01..0.02) weights):
    the kernels' work does not depend on the weight values, and generating 32 distinct 5.1 GB
    layers on the host would take many minutes (their parity is checked against the oracle by
    the stack tests). Tables: each layer's own fitted grid and E2M1; router logits N(0, 1) per
    layer, as the workload defines them. With --router each layer instead routes from its own
    activations: a bf16 router N(0, 1/H) per layer (logits about N(0, 1)), sigmoid gating, and
    the router launch inside the step."""
    import torch
    import codebook_quantized_moe_amd as mq
    import synth

    T, H, I, E, k, L = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.layers
    dev = torch.device("cuda")
    print(f"bench: {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    t_gen = time.perf_counter()
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.key(cfg.cfg_id, 99))

    def codes(N, K):
        return torch.randint(0, 256, (E, N, K // 2), dtype=torch.uint8, device=dev, generator=gen)

    def scales(N, K):
        return torch.randint(119, 124, (E, N, K // 32), dtype=torch.uint8, device=dev,
                             generator=gen)

    layers = []
    logits_host = []
    for l in range(L):
        tables = np.stack([synth.lloyd_grid(cfg.cfg_id, l), synth.E2M1_GRID]).astype(np.float32)
        w = mq.DeviceWeights(codes(I, H), scales(I, H), codes(I, H), scales(I, H), codes(H, I),
                             scales(H, I), tables, torch.zeros(E, dtype=torch.uint8, device=dev))
        if args.router:
            lg = torch.from_numpy(synth.make_router(cfg.cfg_id, E, H, layer=l).view(np.int16))
        else:
            lgh = synth.make_logits(cfg.cfg_id, T, E, layer=l)
            logits_host.append(lgh)
            lg = torch.from_numpy(lgh)
        layers.append((w, lg.to(dev)))
    print(f"bench: {cfg.name}: {L} layers on the device", file=sys.stderr, flush=True)
    x0h = synth.make_x(cfg.cfg_id, T, H)
    x0 = torch.from_numpy(x0h.view(np.int16)).to(dev)
    X = torch.empty_like(x0)
    ML = mq.MoeLayer(T, H, I, E, k, gating=(mq.MOEQ_GATING_SIGMOID_TOPK if args.router
                                            else mq.MOEQ_GATING_SOFTMAX_TOPK))

    def route(lg):
        if args.router:
            ML.router(X, lg)
            ML.route_permute(ML.logits)
        else:
            ML.route_permute(lg)

    # touched experts per layer (with the router they follow the activations, which every
    # step starts again from x0, so one untimed pass gives them)
    touched = []
    X.copy_(x0)
    for w, lg in layers:
        route(lg)
        touched.append(int((np.diff(ML.offsets.cpu().numpy()) > 0).sum()))
        ML.gateup(X, w)
        ML.down(w)
        ML.combine(residual=X, out=X)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    nb = args.warmup + args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(L)] for _ in range(nb)]
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nb)]

    def step(b, timing=False):
        if timing:
            sev[b][0].record()
        X.copy_(x0)
        for l, (w, lg) in enumerate(layers):
            route(lg)
            if timing:
                ev[b][l][0].record()
            ML.gateup(X, w)
            if timing:
                ev[b][l][1].record()
            ML.down(w)
            ML.combine(residual=X, out=X)
        if timing:
            sev[b][1].record()

    # pass 1 (value) without events between kernels; pass 2 (distribution, gate|up durations)
    print(f"bench: {cfg.name}: timing", file=sys.stderr, flush=True)
    for b in range(args.warmup):
        step(b)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for b in range(args.warmup, nb):
        step(b)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    for b in range(args.warmup, nb):
        step(b, timing=True)
    torch.cuda.synchronize()
    ms_per_step = total_ms / args.steps
    value = T * args.steps / (total_ms / 1e3)
    gu_w, dn_w = expert_bytes(H, I)
    P = T * k
    timed = range(args.warmup, nb)
    step_ms = [sev[b][0].elapsed_time(sev[b][1]) for b in timed]
    gu_us = [ev[b][l][0].elapsed_time(ev[b][l][1]) * 1e3 for b in timed for l in range(L)]
    gu_bytes = [touched[l] * gu_w + T * H * 2 + P * I * 2 for l in range(L)]
    step_bytes = sum(touched[l] * (gu_w + dn_w) for l in range(L)) + L * (T * E * 4 + 3 * T * H * 2)
    step_flops = L * 2.0 * P * 3 * H * I
    if args.router:
        step_bytes += L * (E * H * 2 + T * H * 2 + T * E * 4)
        step_flops += L * 2.0 * T * E * H
    kernel = "decode_kernel<true>"
    roof = roofline("hbm", 2.0 * P * 2 * I * H, float(np.mean(gu_bytes)),
                    float(np.mean(gu_us)) / 1e3, kernel, profiled_traffic(kernel, cfg.name),
                    profiled_busy(kernel, cfg.name))
    layer_roof = roofline("hbm", step_flops, step_bytes, ms_per_step, "whole step", None)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (codes and scales drawn on the device)",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "intermediate": I,
                   "experts": E, "top_k": k, "layers": L, "residual": True,
                   "routing": "bf16 router, sigmoid" if args.router else "drawn logits"},
        "roofline": roof,
        "step_ms": dist(step_ms),
        "tokens_per_s_dist": tok_dist(T, step_ms),
        "kernels": {"gateup_swiglu": {"avg_us": round(float(np.mean(gu_us)), 2),
                                      "us": dist(gu_us),
                                      "bytes_per_launch": int(np.mean(gu_bytes))}},
        "layer": {"touched_experts_avg": round(float(np.mean(touched)), 2),
                  "algorithmic_bytes_per_step": int(step_bytes),
                  "algorithmic_flops_per_step": step_flops,
                  "step_GB_s": round(step_bytes / ms_per_step / 1e6, 1),
                  "step_TFLOP_s": round(step_flops / ms_per_step / 1e9, 2),
                  "step_hbm_frac": layer_roof["hbm_frac"],
                  "step_mfma_frac": layer_roof["mfma_frac"],
                  "step_roofline_frac": layer_roof["frac"],
                  "step_bound": "hbm"},
        "input_setup_s": round(t_gen, 1),
    }
    w_first = layers[0][0]
    del layers, ML, X, x0
    if not args.no_cpu_baseline and not args.router:
        print(f"bench: {cfg.name}: cpu baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline_stack(cfg, w_first, x0h, logits_host[0])
    else:
        rec["cpu_baseline"] = None
    del w_first
    free_device()
    return rec


def run_encode(args):
    """The on-GPU encoder on one GLM-shaped layer: 256 experts of bf16 N(0, 0.02) gate, up
    [2048, 6144] and down [6144, 2048] drawn on the device (19.3 GB). One step = two rounds of
    the weighted grid fit (moeq_lloyd_stats over the three matrices), the two error passes per
    matrix for the arm choice (moeq_quantize without output bytes, moeq_select_arms) and the
    packing pass (moeq_quantize with codes and scales): 5 passes over the layer's weights (each
    pass reads all three matrices once)."""
    import torch
    import codebook_quantized_moe_amd as mq
    from codebook_quantized_moe_amd import encode
    import synth

    E, H, I = 256, 6144, 2048
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.key(2, 98))
    mats = []
    for shape in ((E, I, H), (E, I, H), (E, H, I)):
        m = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        for e in range(E):
            m[e].normal_(0.0, 0.02, generator=gen)
        mats.append(m.view(torch.int16))
    wbytes = sum(m.numel() * 2 for m in mats)
    g0 = synth.lloyd_grid(2, 0)
    # warm-up on one expert
    encode.fit_grid([m[:1] for m in mats], g0, 1)
    encode.encode_layer(*[m[:1] for m in mats], g0)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    grid, dist_ = encode.fit_grid(mats, g0, 2)
    ev[1].record()
    enc = encode.encode_layer(*mats, grid)
    ev[2].record()
    torch.cuda.synchronize()
    fit_ms = ev[0].elapsed_time(ev[1])
    enc_ms = ev[1].elapsed_time(ev[2])
    total_ms = fit_ms + enc_ms
    # one packing pass alone, for the kernel's own rate
    q0 = torch.cuda.Event(enable_timing=True)
    q1 = torch.cuda.Event(enable_timing=True)
    m = mats[0]
    codes = torch.empty((E, I, H // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((E, I, H // 32), dtype=torch.uint8, device=dev)
    q0.record()
    mq.moeq_quantize(m, E, I, H, enc["tables"], enc["table_id"], codes, scales, None)
    q1.record()
    torch.cuda.synchronize()
    q_ms = q0.elapsed_time(q1)
    q_bytes = m.numel() * 2 + codes.numel() + scales.numel()
    ach = q_bytes / (q_ms / 1e3) / 1e9
    tid = enc["table_id"].cpu().numpy()
    out = {
        "metric": "layer encode: bf16 GB/s over the 5 passes (grid fit, arm choice, packing)",
        "value": round(5 * wbytes / (total_ms / 1e3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 1,
        "ms_per_step": round(total_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (N(0, 0.02) drawn on the device)",
        "config": {"workload": "glm_layer_encode", "experts": E, "hidden": H, "intermediate": I,
                   "weight_bytes": wbytes, "fit_rounds": 2},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "quantize_kernel (packing pass of the gate matrices)"},
        "encode": {"fit_ms": round(fit_ms, 2), "arms_and_pack_ms": round(enc_ms, 2),
                   "grid": [round(float(v), 5) for v in grid],
                   "fit_weighted_sq_error": dist_, "experts_on_e2m1": int(tid.sum())},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


# keys of the contract's top level that a configs-block entry does not repeat
_LINE_ONLY = ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "dtype", "data")


def block_entry(rec):
    return {k: v for k, v in rec.items() if k not in _LINE_ONLY}


def measure(args, cfg_id, cpu_tokens):
    import synth
    cfg = synth.CONFIGS[cfg_id]
    if cfg.layers > 1:
        return measure_stack(args, cfg)
    return measure_layer(args, cfg, cpu_tokens)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a run.", file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: F401
    import codebook_quantized_moe_amd as mq  # noqa: F401  (fails loudly when not built)

    if args.encode:
        return run_encode(args)
    if args.config is not None:
        print(json.dumps(measure(args, args.config, args.cpu_tokens)), flush=True)
        return
    line = measure(args, HEADLINE, args.cpu_tokens)
    variant = args.fused or args.shared or args.router
    if not args.no_configs and not variant:
        block = {}
        for c in OTHER_CONFIGS:
            # the CPU oracle on 1 token of the large workloads (about 10 s each), all 16 of tiny
            rec = measure(args, c, 16 if c == 1 else 1)
            block[rec["config"]["workload"]] = block_entry(rec)
        line["configs"] = block
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
