#!/usr/bin/env python3
"""Throughput of the block-diffusion denoising step on one MI355X.

Workload (default ``layer_bf16``): one MoE layer at the 16B-parameter /
~1B-active shape (hidden 2048, 16 heads x 128, 256 experts top-8 + 1 shared
expert, expert FFN 512, vocabulary 4096 + [MASK]), bf16, batch 1, a cached
prefix of 1024 tokens and a 32-token block with 16 [MASK] positions.  A step
is one call of dllm_denoise_step at t = 4 of an 8-step block (16 masked
remaining, 4 steps left: the linear schedule commits 4 tokens), so denoised
tokens/s = 4 x steps / time.  Weights are seeded synthetic N(0, 0.02); four
device copies of the layer (each with its own KV cache) are rotated so the
256 MB last-level cache cannot serve repeated weight reads.  The routed
experts' gate/up weights are repacked once at load (dllm_pack_gate_up) into
the fragment layout the expert kernels read contiguously.

Prints one JSON line (rank 0).  The roofline object covers the dominant
kernel (grouped expert gate/up): algorithmic bytes per launch (touched
experts' gate+up weights + shared expert + activations) over the mean launch
time from HIP events recorded on the library's stream around that launch in
every fourth step of the timed region (each event pair adds stream markers,
so timing every launch of every group would slow the step measurably).
The cpu_baseline leg times the float64 oracle on a bounded sample of the same
step (prefill untimed) on the host cores.  The prefill (dllm_block_init over
the 1024-token prefix, once per weight copy) is timed separately and reported
with its algorithmic flops.  A secondary object, batched_layer, measures one
layer of the batched thinking shape (16 sequences x 2048-token prefixes, fp8
experts), where attention streams enough cached K/V for its HBM roofline to
be meaningful and the LDS-tiled LM head covers 256 rows x 157,184 ids; a third,
understanding_layer, one layer of the understanding shape (one sequence,
4160-token prefix), where the streaming LM head covers 16 rows x 157,184 ids.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoised tokens/sec per MI355X + step latency; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
PROF_EVERY = 4   # timed-region steps per sampled gate/up launch timing


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


GATEUP_COUNTERS = "expert_gateup_layer_bf16_hbm_counters.txt"
BATCHED_COUNTERS = "attn_experts_head_think_fp8_layer_hbm_counters.txt"


def measured_traffic(kernel, summary=GATEUP_COUNTERS):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter
    summary under profiles/, or None when the kernel source changed since it
    was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    src = os.path.join(ROOT, "masked_block_diffusion_amd", "csrc", "dllm_kernels.hip")
    try:
        rec = {}
        for line in open(path):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") != sha:
            return None
        return int(rec[f"{kernel}_traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def prefill_flops(wl):
    """Algorithmic flops of appending the prefix (all layers): projections,
    router, k routed + shared SwiGLU experts per token, and attention over
    the keys each query sees under the block-wise mask (its own block and all
    earlier ones)."""
    m, g = wl.model, wl.gen
    D, HD, E, F, Fs = m.hidden, m.n_heads * m.head_dim, m.n_experts, m.expert_ffn, m.shared_ffn
    P, LB, R = wl.prefix_len, g.block_length, g.rows
    per_tok = 2 * (4 * HD * D) + 2 * D * E + 2 * 3 * D * (m.top_k * F + m.n_shared * Fs)
    keys = sum(min(P, (i // LB + 1) * LB) for i in range(P))
    attn = 4 * HD * keys
    return R * m.n_layers * (P * per_tok + attn)


def prefill_record(wl, ms_list):
    """Prefill (dllm_block_init over the prefix), timed with events around the
    call on the library's stream; the first copy's call is left out (first
    launches)."""
    ms = float(np.median(ms_list))
    fl = prefill_flops(wl)
    return {"tokens": wl.prefix_len * wl.gen.rows, "ms": round(ms, 3),
            "tokens_per_s": round(wl.prefix_len * wl.gen.rows / (ms * 1e-3), 1),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "flops": int(fl),
            "mfma_peak_tflops": 2500.0 if wl.model.act_dtype != "f32" else 157.3,
            "calls": len(ms_list)}


def batched_layer(torch, di, B, name="think_fp8_layer", copies=2, warmup=5, steps=30, counters=None):
    """The batched thinking shape, one layer: 16 sequences with 2048-token
    prefixes, fp8 experts, LM head over the 157,184-id text sub-vocabulary.
    At this shape attention streams 273 MB of cached K/V per layer step, the
    experts run in work-list mode and the head streams 644 MB for 256 head
    rows, so it is where those kernels' HBM rooflines mean something (at the
    single-sequence shape attention is latency-bound).  Reports the step rate
    and, from HIP events around the attention, expert and head launch groups
    on every step of a separate pass, each group's mean time, achieved GB/s
    and fraction of 8 TB/s."""
    wl = di.workload(name)
    m, g = wl.model, wl.gen
    t_step = g.steps // 2
    log("batched layer weights", wl.name)
    w = di.make_weights(m, 0)
    prefix, block = di.make_prefix(wl, 0), di.make_block(wl, 0)
    stream = torch.cuda.current_stream()
    ss = []
    for c in range(copies):
        dev = B.Session.upload(w, torch.device("cuda:0"))
        s = B.Session(wl, w, max_prefix=wl.prefix_len + g.block_length, max_clean=wl.prefix_len,
                      stream=stream, _device_weights=dev)
        s.block_init(prefix)
        ss.append(s)
    torch.cuda.synchronize()
    ids_in = ss[0].ids_tensor(block)
    outs = [torch.empty_like(ids_in) for _ in ss]

    def step(i):
        ss[i % copies].denoise_step(t_step, ids_in, outs[i % copies])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    committed = int(np.sum(block == m.mask_id)) - int(ss[0].remaining.cpu().numpy().sum())
    groups = sum(1 << B.PROF_GROUPS.index(k) for k in ("attention", "expert_gateup", "expert_down", "head"))
    for s in ss:
        B._check(B.dllm_profile_enable(s.ctx, groups), s.ctx, "profile")
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    prof = {}
    for s in ss:
        B.dllm_profile_enable(s.ctx, 0)
        st, d = B.dllm_profile_read(s.ctx)
        B._check(st, s.ctx, "profile read")
        for k, (msum, n) in d.items():
            a = prof.setdefault(k, [0.0, 0])
            a[0] += msum
            a[1] += n
    us = {k: v[0] / max(v[1], 1) * 1e3 for k, v in prof.items() if v[1]}
    R, H, dh, D, F = g.rows, m.n_heads, m.head_dim, m.hidden, m.expert_ffn
    route = ss[0].debug(B.DEBUG_ROUTE_IDX, 0, np.int32, (R * g.block_length, m.top_k))
    touched = len(np.unique(route))
    ees = {"f32": 4, "bf16": 2, "fp8": 1}[m.expert_dtype]
    aes = {"f32": 4, "bf16": 2}[m.act_dtype]
    M = R * g.block_length
    S = M * m.top_k
    head_rows = int(np.sum(block == m.mask_id))   # one head row per masked position (no guidance)
    nbytes = {
        # cached K and V of every row and head plus the block's own
        "attention": R * H * (wl.prefix_len + g.block_length) * dh * 2 * aes,
        "expert_gateup": touched * 2 * F * D * ees + m.n_shared * 2 * m.shared_ffn * D * aes + M * D * aes
        + (S + M * m.n_shared) * F * aes,
        "expert_down": touched * D * F * ees + m.n_shared * D * m.shared_ffn * aes
        + (S + M * m.n_shared) * (F * aes + D * 4),
        # vocabulary rows of the sub-vocabulary, the head rows read once
        "head": (g.vocab_hi - g.vocab_lo) * D * aes + head_rows * D * aes,
    }
    # the head launch holds n_seq x block_length rows (no guidance here): the
    # streaming head up to 32 rows, the LDS-tiled head above
    tiled_head = g.n_seq * g.block_length > 32
    kname = {"attention": "k_attn_stream", "expert_gateup": "k_expert_gateup", "expert_down": "k_expert_down",
             "head": "k_head_tiled" if tiled_head else "k_head_conf"}
    kern = {}
    for k, b in nbytes.items():
        gbs = b / (us[k] * 1e-6) / 1e9
        kern[k] = {"kernel": kname[k], "bytes_per_launch": int(b), "mean_launch_us": round(us[k], 2),
                   "achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                   "traffic": measured_traffic(kname[k], counters) if counters else None}
    for s in ss:
        s.close()
    return {"workload": wl.name, "description": wl.description, "ms_per_step": round(ms, 4),
            "denoised_tokens_per_s": round(committed * 1e3 / ms, 1), "committed_per_step": committed,
            "steps": steps, "weight_copies": copies, "touched_experts": touched,
            "kernels": kern,
            "head_rows": head_rows, "vocab": int(g.vocab_hi - g.vocab_lo),
            "note": "attention = all launches of the attention group (the streaming kernel, plus the merge "
                    "pass when the keys are split); head = " + ("LDS-tiled" if tiled_head else "streaming") +
                    " LM head + confidence partials; times from HIP events around each launch group on every "
                    "step of a separate pass" + ("" if counters else "; traffic: no counters taken for this "
                                                 "workload")}


def calibrate_copy(torch):
    """A 256 MiB elementwise copy (read 256 MiB, write 256 MiB), three times:
    the reference dispatch that scales the HBM byte counters."""
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(wl, weights, prefix, block, t_step, seconds):
    from oracle import dllm_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    m, g = wl.model, wl.gen
    model = O.Model(m, weights)
    cache = O.Cache.empty(m, g.rows)
    O.block_init(model, cache, prefix, g.block_length)        # untimed setup
    n = 0
    committed = 0
    t0 = time.perf_counter()
    while True:
        ids, rem, _ = O.denoise_step(model, cache, g, block, t_step)
        committed += int(np.sum(block == m.mask_id) - np.sum(rem))
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": committed / dt, "unit": "denoised tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} oracle denoising steps (t={t_step}) of the {wl.name} workload, "
                      f"{dt:.1f} s, prefill untimed"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="layer_bf16")
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the secondary batched-thinking layer measurement")
    ap.add_argument("--batched-only", action="store_true",
                    help="run only the batched-thinking layer measurement (for kernel profiles)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 256 MiB elementwise copy (256 MiB read + 256 MiB written) before "
                         "the timed region, as the reference kernel for HBM byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dllm_inputs as di
    from masked_block_diffusion_amd import binding as B

    if args.batched_only:
        if args.calibrate_copy:
            calibrate_copy(torch)
        print(json.dumps({"batched_layer": batched_layer(torch, di, B, counters=BATCHED_COUNTERS)}), flush=True)
        return
    wl = di.workload(args.workload)
    m, g = wl.model, wl.gen
    t_step = g.steps // 2
    log("weights", wl.name)
    weights = di.make_weights(m, 0)
    prefix = di.make_prefix(wl, 0)
    block = di.make_block(wl, 0)
    stream = torch.cuda.current_stream()
    sessions = []
    prefill_ms = []
    for c in range(args.copies):
        dev = B.Session.upload(weights, torch.device("cuda:0"))
        s = B.Session(wl, weights, max_prefix=wl.prefix_len + g.block_length,
                      max_clean=wl.prefix_len, stream=stream, _device_weights=dev)
        ids = s.ids_tensor(prefix)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        s.block_init(ids)
        e1.record(stream)
        torch.cuda.synchronize()
        prefill_ms.append(e0.elapsed_time(e1))
        sessions.append(s)
    torch.cuda.synchronize()
    ids_in = sessions[0].ids_tensor(block)
    outs = [torch.empty_like(ids_in) for _ in sessions]

    def step(i):
        s = sessions[i % len(sessions)]
        s.denoise_step(t_step, ids_in, outs[i % len(sessions)])

    if args.calibrate_copy:
        calibrate_copy(torch)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # touched experts of this input (same routing every step)
    M = g.rows * g.block_length
    route = sessions[0].debug(B.DEBUG_ROUTE_IDX, 0, np.int32, (M, m.top_k))
    touched = len(np.unique(route))
    committed = int(np.sum(block == m.mask_id)) - int(sessions[0].remaining.cpu().numpy().sum())

    def read_prof():
        prof = {}
        for s in sessions:
            st, d = B.dllm_profile_read(s.ctx)
            B._check(st, s.ctx, "profile read")
            for k, (ms, n) in d.items():
                a = prof.setdefault(k, [0.0, 0])
                a[0] += ms
                a[1] += n
        return prof

    # Timed region.  Every PROF_EVERY-th step records a HIP event pair around
    # the grouped expert gate/up launch (the roofline kernel) on the library's
    # stream; each pair adds two stream markers, so only a sample is timed.
    gateup_bit = 1 << B.PROF_GROUPS.index("expert_gateup")
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        sampled = i % PROF_EVERY == 0
        if sampled:
            B.dllm_profile_enable(sessions[i % len(sessions)].ctx, gateup_bit)
        step(i)
        if sampled:
            B.dllm_profile_enable(sessions[i % len(sessions)].ctx, 0)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    prof = read_prof()
    value = committed * args.steps / (ms_total / 1e3)
    # per-group launch times (informational) from an untimed pass with every group timed
    for s in sessions:
        B._check(B.dllm_profile_enable(s.ctx, B.PROF_ALL), s.ctx, "profile")
    for i in range(40):
        step(i)
    torch.cuda.synchronize()
    for s in sessions:
        B.dllm_profile_enable(s.ctx, 0)
    prof_all = read_prof()

    # algorithmic bytes of one grouped gate/up launch
    ees = {"f32": 4, "bf16": 2, "fp8": 1}[m.expert_dtype]
    aes = {"f32": 4, "bf16": 2}[m.act_dtype]
    D, F, Fs = m.hidden, m.expert_ffn, m.shared_ffn
    S = M * m.top_k
    gu_bytes = touched * 2 * F * D * ees + m.n_shared * 2 * Fs * D * aes + M * D * aes + \
        (S + M * m.n_shared) * F * aes
    dn_bytes = touched * D * F * ees + m.n_shared * D * Fs * aes + (S + M * m.n_shared) * (F * aes + D * 4)
    gu_ms = prof["expert_gateup"][0] / max(prof["expert_gateup"][1], 1)
    dn_ms = prof_all["expert_down"][0] / max(prof_all["expert_down"][1], 1)
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    kernels = {k: round(v[0] / max(v[1], 1) * 1e3, 2) for k, v in prof_all.items()}
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "denoised tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m.expert_dtype if m.expert_dtype != "f32" else "f32",
        "data": "synthetic (seeded N(0,0.02) weights, uniform random ids)",
        "config": {"workload": wl.name, "layers": m.n_layers, "hidden": m.hidden,
                   "heads": f"{m.n_heads}x{m.head_dim}",
                   "experts": f"{m.n_experts} top-{m.top_k} + {m.n_shared} shared",
                   "expert_ffn": F, "vocab": m.vocab, "prefix": wl.prefix_len,
                   "block": g.block_length, "masked_in_block": wl.masked_in_block,
                   "step": f"t={t_step} of {g.steps}", "committed_per_step": committed,
                   "batch": g.n_seq, "weight_copies": args.copies,
                   "expert_gate_up_layout": "packed fragments (dllm_pack_gate_up, once at load)"},
        "roofline": {"bound": "hbm", "kernel": "k_expert_gateup (grouped expert gate/up + SwiGLU)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("k_expert_gateup") if wl.name == "layer_bf16" else None,
                     "bytes_per_launch": int(gu_bytes), "mean_launch_us": round(gu_ms * 1e3, 2),
                     "timed_launches": int(prof["expert_gateup"][1]), "touched_experts": touched},
        "kernels_mean_us": kernels,
        "kernels_mean_us_note": "untimed pass of 40 steps with every kernel group timed",
        "expert_down": {"bytes_per_launch": int(dn_bytes), "mean_launch_us": round(dn_ms * 1e3, 2),
                        "achieved_GBs": round(dn_bytes / (dn_ms * 1e-3) / 1e9, 1)},
        "step_latency_ms": round(ms_per_step, 4),
        "prefill": prefill_record(wl, prefill_ms[1:] or prefill_ms),
        "wall_s_timed": round(wall, 3),
    }
    for s in sessions:
        s.close()
    del sessions
    torch.cuda.empty_cache()
    res["batched_layer"] = None if args.no_batched else batched_layer(torch, di, B, counters=BATCHED_COUNTERS)
    # one layer of the understanding shape: the streaming LM head over 157,184 ids (644 MB per step)
    res["understanding_layer"] = None if args.no_batched else batched_layer(torch, di, B, name="und_layer")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(wl, weights, prefix, block, t_step, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
