#!/usr/bin/env python3
"""Throughput of the block-diffusion denoising step on one MI355X.

Headline workload (``think_fp8``, the largest that fits one GPU): batched
thinking mode of the 20-layer 16B-parameter MoE backbone (hidden 2048, 16
heads x 128, 256 experts top-8 + 1 shared expert, expert width 512, routed
expert weights OCP E4M3FN with per-row float32 scales widened to bf16 for the
matrix cores; attention, shared expert, embeddings and head bf16), 16
sequences, 2048-token prompts, 4096 generated tokens per sequence in 128
blocks of 32, 32 steps per block with one commit per sequence and step, LM
head over the 157,184-id text sub-vocabulary.

A step is one dllm_denoise_step of all 20 layers for the 16 sequences (16
committed tokens).  The generation's steps differ only in the cached prefix
length P, which grows from 2048 (first block) to 6112 (last block); only
attention depends on P, linearly, so the mean step of the generation is the
mean of a first-block and a last-block step.  The timed region alternates
the two states (two contexts over the same weights, one with each cache),
so denoised tokens/s = 16 x steps / time is the generation's average step
rate with inputs resident in HBM; the block appends (one clean 32-token pass
per block) are timed separately and folded into an extrapolated
whole-generation rate, and the prompt prefill is reported on its own.

Weights are seeded synthetic values written on the GPU by the counter-based
generator of dllm_inputs (the same bits as its host twin); token ids are
uniform random.  The routed gate/up weights are repacked once at load
(dllm_pack_gate_up).

Prints one JSON line.  ``rooflines`` covers the two largest launch groups,
the streaming attention and the grouped fp8 expert gate/up: algorithmic bytes
(attention: the K/V of every cached and block position at each state's P;
gate/up: touched experts' codes and scales from each layer's routing, the
shared expert, activations) over the launch time from HIP events that the
library records on its stream around that launch group, in a sample of the
timed steps (both states).  ``roofline`` is the one with the larger share of
the mean step (``step_time_share``).  ``kernels`` gives every launch group's time and HBM fraction from a
separate untimed pass, at the first and the last block.  ``cpu_baseline``
times the float64 oracle on a sample of the same step (one layer and the head
at each state, extrapolated to 20 layers).  Secondary objects: one
``layer_bf16`` layer step (hidden 2048, 1024-token prefix, batch 1) and one
layer of the understanding shape (``und_layer``: 4160-token prefix, the
streaming head over 157,184 ids).
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoised tokens/sec per MI355X + step latency; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_TFLOPS = 2500.0
# of every PROF_PERIOD timed steps, the first four record event pairs: two
# (one per state) around the attention launches, two around the gate/up ones;
# the rest run unmarked (an event pair around each of a step's 20 launches of
# a group adds about 0.2 ms to that step)
PROF_PERIOD = 16

THINK_COUNTERS = "think_fp8_step_hbm_counters.txt"
THINK_MFMA = "think_fp8_step_mfma_counters.txt"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_sha():
    src = os.path.join(ROOT, "masked_block_diffusion_amd", "csrc", "dllm_kernels.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()


def measured_traffic(kernel, summary):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter
    summary under profiles/, or None when the kernel source changed since it
    was taken (or there is none)."""
    path = os.path.join(ROOT, "profiles", summary)
    try:
        rec = {}
        for line in open(path):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
        if rec.get("kernel_source_sha256") != kernel_sha():
            return None
        return int(rec[f"{kernel}_traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def prefill_flops(m, rows, P, LB):
    """Algorithmic flops of appending a P-token prefix to `rows` model rows
    (all layers): projections, router, k routed + shared SwiGLU experts per
    token, and attention over the keys each query sees under the block-wise
    mask (its own block and all earlier ones)."""
    D, HD, E, F, Fs = m.hidden, m.n_heads * m.head_dim, m.n_experts, m.expert_ffn, m.shared_ffn
    per_tok = 2 * (4 * HD * D) + 2 * D * E + 2 * 3 * D * (m.top_k * F + m.n_shared * Fs)
    keys = sum(min(P, (i // LB + 1) * LB) for i in range(P))
    return rows * m.n_layers * (P * per_tok + 4 * HD * keys)


def calibrate_copy(torch):
    """A 256 MiB elementwise copy (read 256 MiB, write 256 MiB), three times:
    the reference dispatch that scales the HBM byte counters."""
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def ev_pair(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def read_prof(B, sessions):
    prof = {}
    for s in sessions:
        st, d = B.dllm_profile_read(s.ctx)
        B._check(st, s.ctx, "profile read")
        for k, (ms, n) in d.items():
            a = prof.setdefault(k, [0.0, 0])
            a[0] += ms
            a[1] += n
    return prof


def group_bytes(m, g, P, touched, head_rows, vsub):
    """Algorithmic bytes of one launch of each group at prefix length P, for
    one layer whose routing touched `touched` experts (head: once per step)."""
    ees = {"f32": 4, "bf16": 2, "fp8": 1}[m.expert_dtype]
    aes = {"f32": 4, "bf16": 2}[m.act_dtype]
    sc = 4 if m.expert_dtype == "fp8" else 0          # float32 row scale per weight row
    R, H, dh, D, F, Fs = g.rows, m.n_heads, m.head_dim, m.hidden, m.expert_ffn, m.shared_ffn
    M = R * g.block_length
    S = M * m.top_k
    return {
        "expert_gateup": touched * 2 * F * (D * ees + sc) + m.n_shared * 2 * Fs * D * aes + M * D * aes
        + (S + M * m.n_shared) * F * aes,
        # output rows in the activation type (float32 or bf16)
        "expert_down": touched * D * (F * ees + sc) + m.n_shared * D * Fs * aes + (S + M * m.n_shared) * (F + D) * aes,
        # cached K and V of every row and head plus the block's own
        "attention": R * H * (P + g.block_length) * dh * 2 * aes,
        "qkv": 3 * H * dh * D * aes + M * D * aes + 3 * M * H * dh * aes,
        # vocabulary rows of the sub-vocabulary, the head rows read once
        "head": vsub * D * aes + head_rows * D * aes,
    }


def touched_per_layer(B, s, m, M):
    return [len(np.unique(s.debug(B.DEBUG_ROUTE_IDX, l, np.int32, (M, m.top_k)))) for l in range(m.n_layers)]


# ----------------------------------------------------------------------------
# headline: the 20-layer batched thinking step
# ----------------------------------------------------------------------------

def thinking_step(torch, di, B, DV, steps, warmup, calibrate=False):
    wl = di.workload("think_fp8")
    m, g = wl.model, wl.gen
    LB = g.block_length
    P0 = wl.prefix_len
    P1 = wl.prefix_len + (wl.n_blocks - 1) * LB         # cached prefix of the last block
    wl.masked_in_block = 16                             # mid-block: 16 [MASK] left, 16 steps left
    t_step = g.steps // 2
    stream = torch.cuda.current_stream()
    log("thinking model weights on the GPU", m.n_layers, "layers")
    t0 = time.perf_counter()
    dev = DV.make_weights_device(m, 0, "cuda:0", stream)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    prompt = di.make_prefix(wl, 0)                      # [16, 2048] uniform text ids
    rng = np.random.default_rng([0, 103])
    generated = rng.integers(g.vocab_lo, g.vocab_hi, size=(g.n_seq, P1 - P0)).astype(np.int32)
    block = di.make_block(wl, 0)
    # first block: P = 2048 (one append of 32 left for timing it); last block: P = 6112
    sA = B.Session(wl, None, max_prefix=P0 + 2 * LB, max_clean=P0, stream=stream, _device_weights=dev)
    sB = B.Session(wl, None, max_prefix=P1 + LB, max_clean=1024, stream=stream, _device_weights=dev)
    torch.cuda.synchronize()
    e0, e1 = ev_pair(torch)
    e0.record(stream)
    sA.block_init(sA.ids_tensor(prompt))
    e1.record(stream)
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    full = np.concatenate([prompt, generated], axis=1)
    for c0 in range(0, P1, 1024):
        sB.block_init(sB.ids_tensor(full[:, c0:c0 + 1024]))
    torch.cuda.synchronize()
    assert sA.prefix_length == P0 and sB.prefix_length == P1
    sess = [sA, sB]
    ids_in = sA.ids_tensor(block)
    outs = [torch.empty_like(ids_in) for _ in sess]

    def step(i):
        sess[i % 2].denoise_step(t_step, ids_in, outs[i % 2])

    if calibrate:
        calibrate_copy(torch)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    M = g.rows * LB

    # timed region: steps alternate first / last block; of every PROF_PERIOD
    # steps, two (one per state) record event pairs around each attention
    # launch, two around each gate/up launch, the others none
    gate_bit = 1 << B.PROF_GROUPS.index("expert_gateup")
    attn_bit = 1 << B.PROF_GROUPS.index("attention")
    torch.cuda.synchronize()
    ev0, ev1 = ev_pair(torch)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        ph = i % PROF_PERIOD
        B.dllm_profile_enable(sess[i % 2].ctx, attn_bit if ph < 2 else (gate_bit if ph < 4 else 0))
        step(i)
        B.dllm_profile_enable(sess[i % 2].ctx, 0)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    timed = [read_prof(B, [s]) for s in sess]
    gate_prof = [t.get("expert_gateup", [0.0, 0]) for t in timed]
    attn_prof = [t.get("attention", [0.0, 0]) for t in timed]

    # per-state step latency and every launch group (untimed pass)
    lat, groups = [], []
    for s in sess:
        for _ in range(3):
            s.denoise_step(t_step, ids_in, outs[0])
        torch.cuda.synchronize()
        a, b = ev_pair(torch)
        a.record(stream)
        for _ in range(10):
            s.denoise_step(t_step, ids_in, outs[0])
        b.record(stream)
        torch.cuda.synchronize()
        lat.append(a.elapsed_time(b) / 10)
        B._check(B.dllm_profile_enable(s.ctx, B.PROF_ALL), s.ctx, "profile")
        for _ in range(6):
            s.denoise_step(t_step, ids_in, outs[0])
        torch.cuda.synchronize()
        B.dllm_profile_enable(s.ctx, 0)
        groups.append(read_prof(B, [s]))
    # routing of the step (each context's last pass is the step just run,
    # whatever the warm-up and step counts)
    touched = [touched_per_layer(B, s, m, M) for s in sess]
    committed = int(np.sum(block == m.mask_id)) - int(sA.remaining.cpu().numpy().sum())
    # block appends (one clean 32-token pass) at each state
    app = []
    for s in sess:
        a, b = ev_pair(torch)
        clean = s.ids_tensor(rng.integers(g.vocab_lo, g.vocab_hi, size=(g.n_seq, LB)).astype(np.int32))
        torch.cuda.synchronize()
        a.record(stream)
        s.block_init(clean)
        b.record(stream)
        torch.cuda.synchronize()
        app.append(a.elapsed_time(b))

    vsub = g.vocab_hi - g.vocab_lo
    head_rows = int(np.sum(block == m.mask_id))
    # roofline: gate/up bytes of every timed launch over their summed time
    gu_bytes, gu_ms, gu_n = 0.0, 0.0, 0
    for si, s in enumerate(sess):
        ms, n = gate_prof[si]
        if n == 0:
            continue
        per_step = sum(group_bytes(m, g, s.prefix_length, u, head_rows, vsub)["expert_gateup"] for u in touched[si])
        gu_bytes += per_step * (n // m.n_layers)
        gu_ms += ms
        gu_n += n
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9 if gu_ms else 0.0   # no marked gate/up steps below 4 steps
    # attention: the same over both states (its bytes grow with P)
    at_bytes, at_ms, at_n = 0.0, 0.0, 0
    for si in range(2):
        ms, n = attn_prof[si]
        P = P0 if si == 0 else P1
        at_bytes += group_bytes(m, g, P, touched[si][0], head_rows, vsub)["attention"] * n
        at_ms += ms
        at_n += n
    at_achieved = at_bytes / (at_ms * 1e-3) / 1e9 if at_ms else 0.0
    kern = {}
    counters = {"expert_gateup": "k_expert_gateup", "expert_down": "k_expert_down",
                "attention": "k_attn_stream", "qkv": "k_qkv_rope_tiled", "head": "k_head_tiled"}
    for si, (name, s) in enumerate((("first_block", sess[0]), ("last_block", sess[1]))):
        # the profile pass ran after the append above for none of them: P as in the timed steps
        P = P0 if si == 0 else P1
        rec = {"prefix": P, "step_ms": round(lat[si], 4), "append_ms": round(app[si], 4)}
        for k, (msum, n) in groups[si].items():
            if not n:
                continue
            us = msum / n * 1e3
            nb = np.mean([group_bytes(m, g, P, u, head_rows, vsub)[k] for u in touched[si]])
            gbs = nb / (us * 1e-6) / 1e9
            rec[k] = {"kernel": counters[k], "mean_launch_us": round(us, 2), "launches_per_step": int(round(n / 6)),
                      "bytes_per_launch": int(nb), "achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
            # matrix-core work issued per launch (committed counter profile) over the live launch time
            fl = measured_mfma_flops(counters[k], THINK_MFMA)
            if fl:
                tf = fl / (us * 1e-6) / 1e12
                rec[k]["mfma_tflops"] = round(tf, 1)
                rec[k]["mfma_frac"] = round(tf / BF16_MFMA_TFLOPS, 4)
        rec["touched_experts_mean"] = round(float(np.mean(touched[si])), 1)
        kern[name] = rec
    rooflines = {
        "expert_gateup": {"bound": "hbm", "kernel": "k_expert_gateup (grouped fp8 expert gate/up + SwiGLU)",
                          "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBS, 4),
                          "traffic": measured_traffic("k_expert_gateup", THINK_COUNTERS),
                          "bytes_per_launch": int(gu_bytes / max(gu_n, 1)),
                          "mean_launch_us": round(gu_ms / max(gu_n, 1) * 1e3, 2), "timed_launches": gu_n,
                          "touched_experts_mean": round(float(np.mean(touched)), 1)},
        "attention": {"bound": "hbm", "kernel": "k_attn_stream (streaming block-wise attention; first- and "
                                                "last-block launches alike)",
                      "achieved": round(at_achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(at_achieved / HBM_PEAK_GBS, 4),
                      "traffic": measured_traffic("k_attn_stream", THINK_COUNTERS),
                      "bytes_per_launch": int(at_bytes / max(at_n, 1)),
                      "mean_launch_us": round(at_ms / max(at_n, 1) * 1e3, 2), "timed_launches": at_n},
    }
    # the dominant kernel: the largest share of the mean step (both states)
    share = {}
    for k in rooflines:
        per_state = [kern[st][k]["mean_launch_us"] * kern[st][k]["launches_per_step"] / 1e3 / lat[si]
                     for si, st in enumerate(("first_block", "last_block")) if k in kern[st]]
        share[k] = float(np.mean(per_state)) if per_state else 0.0
    dominant = max(share, key=share.get)
    ms_per_step = ms_total / steps
    value = committed * steps / (ms_total / 1e3)
    n_blocks = wl.n_blocks
    gen_ms = n_blocks * (g.steps * float(np.mean(lat)) + float(np.mean(app)))
    fl = prefill_flops(m, g.rows, P0, LB)
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "denoised tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based N(0,0.02)-shaped weights generated on the GPU, uniform random ids)",
        "config": {"workload": "think_fp8", "layers": m.n_layers, "hidden": m.hidden,
                   "heads": f"{m.n_heads}x{m.head_dim}",
                   "experts": f"{m.n_experts} top-{m.top_k} + {m.n_shared} shared", "expert_ffn": m.expert_ffn,
                   "expert_weights": "fp8 e4m3fn, per-row fp32 scales, widened to bf16 for the MFMA",
                   "batch": g.n_seq, "prompt": P0, "gen_length": n_blocks * LB, "block": LB,
                   "steps_per_block": g.steps, "committed_per_step": committed,
                   "vocab": f"{m.vocab_text} text + {m.vocab_image} visual (head over the text ids)",
                   "timed_states": f"alternating first block (P={P0}) and last block (P={P1}), "
                                   f"t={t_step} of {g.steps} with 16 [MASK] left"},
        "step_latency_ms": {"first_block": round(lat[0], 4), "last_block": round(lat[1], 4)},
        "roofline": rooflines[dominant],
        "rooflines": rooflines,
        "step_time_share": {k: round(v, 4) for k, v in share.items()},
        "kernels": kern,
        "kernels_note": "launch groups from HIP events around each group on every launch of a separate "
                        "6-step pass per state; attention = streaming kernel (one split per unit at this "
                        "batch); head = LDS-tiled LM head + confidence partials, once per step",
        "generation_extrapolated": {
            "tokens_per_s": round(g.n_seq * n_blocks * LB / (gen_ms / 1e3), 1),
            "ms": round(gen_ms, 1),
            "how": f"{n_blocks} blocks x ({g.steps} steps at the mean of the first- and last-block step "
                   "latencies + one block append at the mean of both), excluding the prompt prefill"},
        "prefill": {"tokens": P0 * g.rows, "ms": round(prefill_ms, 3),
                    "tokens_per_s": round(P0 * g.rows / (prefill_ms * 1e-3), 1),
                    "tflops": round(fl / (prefill_ms * 1e-3) / 1e12, 2), "flops": int(fl),
                    "mfma_peak_tflops": BF16_MFMA_TFLOPS,
                    "mfma_frac": round(fl / (prefill_ms * 1e-3) / 1e12 / BF16_MFMA_TFLOPS, 4)},
        "mfma": {"unit": "TFLOP/s", "peak": BF16_MFMA_TFLOPS,
                 "prefill_frac": round(fl / (prefill_ms * 1e-3) / 1e12 / BF16_MFMA_TFLOPS, 4),
                 "step_kernels": {f"{st}.{k}": {"tflops": v["mfma_tflops"], "frac": v["mfma_frac"]}
                                  for st, rec in kern.items() for k, v in rec.items()
                                  if isinstance(v, dict) and "mfma_frac" in v},
                 "how": "step kernels: bf16 MFMA flops issued per launch (rocprofv3 counter profile under "
                        "profiles/, valid for this kernel source) over the live mean launch time; prefill: "
                        "algorithmic flops over its event-timed duration"},
        "weights_on_gpu_s": round(gen_s, 2),
        "wall_s_timed": round(wall, 3),
    }
    host = {"wl": wl, "block": block, "t": t_step, "P": (P0, P1)}
    for s in sess:
        s.close()
    del dev
    return res, host


# ----------------------------------------------------------------------------
# secondary: single layer steps
# ----------------------------------------------------------------------------

def layer_step(torch, di, B, DV, name, copies, steps, warmup, counters=None, keep=None):
    """One layer of `name`: `copies` device copies of its weights (each with
    its own cache) rotate so the last-level cache cannot serve repeats.
    keep: SPRINT retention at this keep ratio (attention mass, one warm-up
    step): each context runs the block's step 0 first, which scores the
    prefix and selects the kept positions, and the timed steps attend over
    those."""
    wl = di.workload(name)
    m, g = wl.model, wl.gen
    if keep is not None:
        g.use_sprint, g.keep_ratio, g.cache_warmup_steps = True, keep, 1
    t_step = g.steps // 2
    stream = torch.cuda.current_stream()
    prefix, block = di.make_prefix(wl, 0), di.make_block(wl, 0)
    ss = []
    pre = []
    for c in range(copies):
        dev = DV.make_weights_device(m, c, "cuda:0", stream)
        s = B.Session(wl, None, max_prefix=wl.prefix_len + g.block_length, max_clean=min(wl.prefix_len, 1024),
                      stream=stream, _device_weights=dev)
        torch.cuda.synchronize()
        a, b = ev_pair(torch)
        a.record(stream)
        for c0 in range(0, wl.prefix_len, 1024):
            s.block_init(s.ids_tensor(prefix[:, c0:c0 + 1024]))
        b.record(stream)
        torch.cuda.synchronize()
        pre.append(a.elapsed_time(b))
        ss.append(s)
    ids_in = ss[0].ids_tensor(block)
    outs = [torch.empty_like(ids_in) for _ in ss]

    def step(i):
        ss[i % copies].denoise_step(t_step, ids_in, outs[i % copies])

    if keep is not None:
        for i in range(copies):
            ss[i].denoise_step(0, ids_in, outs[i])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = ev_pair(torch)
    a.record(stream)
    for i in range(steps):
        step(i)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    committed = int(np.sum(block == m.mask_id)) - int(ss[0].remaining.cpu().numpy().sum())
    for s in ss:
        B._check(B.dllm_profile_enable(s.ctx, B.PROF_ALL), s.ctx, "profile")
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    for s in ss:
        B.dllm_profile_enable(s.ctx, 0)
    prof = read_prof(B, ss)
    M = g.rows * g.block_length
    touched = [len(np.unique(s.debug(B.DEBUG_ROUTE_IDX, 0, np.int32, (M, m.top_k)))) for s in ss]
    # attention bytes: the retained prefix positions when retention is on
    p_att = int(ss[0].debug(B.DEBUG_NKEPT, 0, np.int32, (1,))[0]) if keep is not None else wl.prefix_len
    vsub = (g.vocab_hi or m.vocab) - g.vocab_lo
    head_rows = int(np.sum(block == m.mask_id))
    kern = {}
    for k, (msum, n) in prof.items():
        if not n:
            continue
        us = msum / n * 1e3
        nb = np.mean([group_bytes(m, g, p_att if k == "attention" else wl.prefix_len, u, head_rows, vsub)[k]
                      for u in touched])
        gbs = nb / (us * 1e-6) / 1e9
        kern[k] = {"mean_launch_us": round(us, 2), "bytes_per_launch": int(nb), "achieved_GBs": round(gbs, 1),
                   "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if counters:
        for k, kn in (("expert_gateup", "k_expert_gateup"), ("expert_down", "k_expert_down")):
            if k in kern:
                kern[k]["traffic"] = measured_traffic(kn, counters)
    fl = prefill_flops(m, g.rows, wl.prefix_len, g.block_length)
    pms = float(np.median(pre[1:] or pre))
    for s in ss:
        s.close()
    if keep is not None:
        return {"keep_ratio": keep, "kept_positions": p_att, "ms_per_step": round(ms, 4), "kernels": kern}
    return {"workload": wl.name, "description": wl.description, "ms_per_step": round(ms, 4),
            "denoised_tokens_per_s": round(committed * 1e3 / ms, 1), "committed_per_step": committed,
            "steps": steps, "weight_copies": copies, "touched_experts_mean": round(float(np.mean(touched)), 1),
            "kernels": kern,
            "prefill": {"tokens": wl.prefix_len * g.rows, "ms": round(pms, 3),
                        "tflops": round(fl / (pms * 1e-3) / 1e12, 2),
                        "mfma_frac": round(fl / (pms * 1e-3) / 1e12 / BF16_MFMA_TFLOPS, 4)},
            "note": "per-group times from HIP events around each launch group in a separate pass"}


# ----------------------------------------------------------------------------
# the other two 20-layer workloads: text-to-image with CFG, understanding with
# SPRINT (step latencies on the first block; secondary objects)
# ----------------------------------------------------------------------------

def stack_steps(torch, di, B, DV, name, steps, warmup, keeps=(None,)):
    """Step latencies of the 20-layer `name` workload on its first block: the
    prompt appended, then `steps` timed repetitions of a mid-block step (t =
    steps_per_block / 2) per retention setting in `keeps` (None: no
    retention; r: SPRINT keep r, whose warm-up step 0 is timed separately).
    Committed tokens per step follow the workload's own schedule."""
    wl = di.workload(name)
    m, g = wl.model, wl.gen
    LB = g.block_length
    stream = torch.cuda.current_stream()
    dev = DV.make_weights_device(m, 0, "cuda:0", stream)
    prompt = di.make_prefix(wl, 0)
    block0 = np.full((g.n_seq, LB), m.mask_id, np.int32)   # the block's first step
    t_mid = g.steps // 2
    wm = di.clone(wl)
    wm.masked_in_block = LB * (g.steps - t_mid) // g.steps   # [MASK] left at t_mid on the linear schedule
    block = di.make_block(wm, 0)
    out = {"workload": name, "description": wl.description, "layers": m.n_layers, "prefix": wl.prefix_len,
           "model_rows": g.rows, "vocab_sub": (g.vocab_hi or m.vocab) - g.vocab_lo}
    for keep in keeps:
        w2 = di.clone(wl)
        g2 = w2.gen
        g2.use_sprint = keep is not None
        if keep is not None:
            g2.keep_ratio, g2.cache_warmup_steps = keep, 1
        s = B.Session(w2, None, max_prefix=wl.prefix_len + LB, max_clean=min(wl.prefix_len, 1024), stream=stream,
                      _device_weights=dev)
        e0, e1 = ev_pair(torch)
        e0.record(stream)
        for c0 in range(0, wl.prefix_len, 1024):
            s.block_init(s.ids_tensor(prompt[:, c0:c0 + 1024]))
        e1.record(stream)
        torch.cuda.synchronize()
        pre_ms = e0.elapsed_time(e1)
        ids0 = s.ids_tensor(block0)
        ids_in = s.ids_tensor(block)
        o = torch.empty_like(ids_in)
        rec = {"prefill_ms": round(pre_ms, 3)}
        e0, e1 = ev_pair(torch)
        e0.record(stream)
        s.denoise_step(0, ids0, o)                      # the block's first step (SPRINT: the warm-up)
        e1.record(stream)
        torch.cuda.synchronize()
        rec["step0_ms"] = round(e0.elapsed_time(e1), 4)
        for _ in range(warmup):
            s.denoise_step(t_mid, ids_in, o)
        torch.cuda.synchronize()
        e0, e1 = ev_pair(torch)
        e0.record(stream)
        for _ in range(steps):
            s.denoise_step(t_mid, ids_in, o)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        committed = int(np.sum(block == m.mask_id)) - int(s.remaining.cpu().numpy().sum())
        # a whole block: its first step plus steps_per_block - 1 like the timed one
        # (every block position denoised: n_seq x block_length tokens)
        block_ms = rec["step0_ms"] + (g.steps - 1) * ms
        rec.update({"step_ms": round(ms, 4), "committed_per_step": committed,
                    "denoised_tokens_per_s": round(committed * 1e3 / ms, 1), "block_ms": round(block_ms, 3),
                    "block_tokens_per_s": round(g.n_seq * LB * 1e3 / block_ms, 1)})
        s.close()
        out["full_retention" if keep is None else f"sprint_keep_{keep}"] = rec
    del dev
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a sample of the thinking step
# ----------------------------------------------------------------------------

def cpu_info():
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(p.get("num_threads", 1) for p in info)
    except Exception:
        pass
    return model, blas, threads


def cpu_baseline(torch, host):
    """The oracle (float64 numpy, as it stands) on one layer of the thinking
    step at the first- and the last-block prefix, plus the head and the
    commit, extrapolated to 20 layers: time(step) = 20 x time(layer) +
    time(head and decisions).  The caches are seeded random K/V of the right
    size (the timing does not depend on their values); the weights are layer 0
    of the model the GPU ran (generated again on the GPU for a one-layer model,
    row-major, and copied to the host)."""
    from oracle import dllm_oracle as O
    import dllm_inputs as di
    from dllm_inputs import device as DV
    wl = di.clone(host["wl"])
    m, g = wl.model, wl.gen
    m.n_layers = 1
    dev = DV.make_weights_device(m, 0, "cuda:0")
    w = {"dtypes": {"dense": m.act_dtype, "expert": m.expert_dtype}}
    for k, t in dev.items():
        a = t.cpu().numpy()
        w[k] = a.view(np.uint16) if a.dtype == np.int16 else a
    del dev
    torch.cuda.empty_cache()
    model = O.Model(m, w)
    cpu, blas, threads = cpu_info()
    rng = np.random.default_rng(7)
    block, t_step = host["block"], host["t"]
    # tokens committed per step: the linear quota ceil(r / (T - t)) of each sequence
    rem = [int(np.sum(block[s] == m.mask_id)) for s in range(g.n_seq)]
    committed = sum(min(r, -(-r // (g.steps - t_step))) for r in rem)
    t_layer, t_rest, work = [], [], 0.0
    for P in host["P"]:
        cache = O.Cache.empty(m, g.rows)
        cache.K = [rng.standard_normal((g.rows, P, m.n_heads, m.head_dim))]
        cache.V = [rng.standard_normal((g.rows, P, m.n_heads, m.head_dim))]
        cache.P = P
        t0 = time.perf_counter()
        O.forward(model, block, cache, append=False, block_len=g.block_length)
        t1 = time.perf_counter()
        O.denoise_step(model, cache, g, block, t_step)
        t2 = time.perf_counter()
        t_layer.append(t1 - t0)
        t_rest.append(max((t2 - t1) - (t1 - t0), 0.0))
        work += t2 - t0
    steps_s = [20 * a + b for a, b in zip(t_layer, t_rest)]
    return {"value": round(committed / float(np.mean(steps_s)), 4), "unit": "denoised tokens/s",
            "cores": int(threads), "kind": "oracle", "cpu": cpu, "blas": blas,
            "sample": f"extrapolated from {work:.1f} s of CPU work: one oracle layer forward and one 1-layer "
                      f"oracle step (head over 157,184 ids, commit) of the 16-sequence thinking step at "
                      f"P={host['P'][0]} and P={host['P'][1]}; step = 20 x layer + head and decisions = "
                      f"{steps_s[0]:.2f} s / {steps_s[1]:.2f} s, {committed} tokens per step"}


# ----------------------------------------------------------------------------
# rocprofv3 summaries (for profiles/): per (kernel, grid) over every dispatch
# ----------------------------------------------------------------------------

def _short(name):
    n = name.replace("(anonymous namespace)::", "").split("(")[0]
    return n.replace("void ", "").replace("dllm::", "")


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        yield from csv.DictReader(f)


def summarize_trace(d):
    """Kernel durations of a `rocprofv3 --kernel-trace --output-format csv`
    run, grouped by (kernel, grid size): dispatches, median and mean in us."""
    groups = {}
    for r in _read_csv(os.path.join(d, "run_kernel_trace.csv")):
        k = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
        groups.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    print(f"# {'kernel':<52} {'grid':>9} {'calls':>6} {'median_us':>10} {'mean_us':>9} {'total_ms':>9}")
    for (k, grid), v in rows:
        print(f"# {k[:52]:<52} {grid:>9} {len(v):>6} {np.median(v):>10.2f} {np.mean(v):>9.2f} {sum(v) / 1e3:>9.2f}")
    print(f"kernel_source_sha256: {kernel_sha()}")


def summarize_counters(fetch_dir, write_dir, min_calls=1):
    """HBM bytes per dispatch from two `rocprofv3 --pmc FETCH_SIZE` /
    `--pmc WRITE_SIZE` runs of the same command, grouped by (kernel, grid):
    median KiB per dispatch (and the mean, for groups that mix two shapes of
    the same grid), scaled by what the counters read for the 256 MiB
    reference copy (torch elementwise multiply of 64M float32, read 256 MiB,
    write 256 MiB) that the command runs with --calibrate-copy."""
    cal = {}

    def load(d, counter):
        g = {}
        for r in _read_csv(os.path.join(d, "run_counter_collection.csv")):
            if r["Counter_Name"] != counter:
                continue
            if "MulFunctor<float>" in r["Kernel_Name"] and int(r["Grid_Size"]) * 4 == 64 << 20:
                cal.setdefault(counter, []).append(float(r["Counter_Value"]))   # the reference copy
                continue
            k = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
            g.setdefault(k, []).append(float(r["Counter_Value"]))
        return g
    fe, wr = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    f_cal = np.median(cal["FETCH_SIZE"]) if "FETCH_SIZE" in cal else None
    w_cal = np.median(cal["WRITE_SIZE"]) if "WRITE_SIZE" in cal else None
    fscale = (256 * 1024) / f_cal if f_cal else 1.0
    wscale = (256 * 1024) / w_cal if w_cal else 1.0
    print(f"# calibration: the 256 MiB copy reads FETCH_SIZE = {f_cal} KiB, WRITE_SIZE = {w_cal} KiB per dispatch")
    print(f"fetch_scale: {fscale:.4f}")
    print(f"write_scale: {wscale:.4f}")
    print(f"# {'kernel':<52} {'grid':>9} {'calls':>6} {'FETCH_KiB':>11} {'WRITE_KiB':>10} {'scaled_MB':>10} "
          f"{'mean_MB':>9}")
    out = {}
    for k in sorted(fe, key=lambda k: -np.median(fe[k]) * len(fe[k])):
        if len(fe[k]) < min_calls or k not in wr:
            continue
        f, w = float(np.median(fe[k])), float(np.median(wr[k]))
        b = (f * fscale + w * wscale) * 1024
        bm = (float(np.mean(fe[k])) * fscale + float(np.mean(wr[k])) * wscale) * 1024
        out[k] = b
        print(f"# {k[0][:52]:<52} {k[1]:>9} {len(fe[k]):>6} {f:>11.1f} {w:>10.1f} {b / 1e6:>10.2f} "
              f"{bm / 1e6:>9.2f}")
    print(f"kernel_source_sha256: {kernel_sha()}")
    return out


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def summarize_mfma(mfma_dir, trace_dir):
    """Matrix-core work per dispatch from a `rocprofv3 --pmc` run of the
    counters in MFMA_COUNTERS, grouped by (kernel, grid): the bf16 MFMA flops
    the kernel issued (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, one MOP being 512
    flops) and, with the median duration of the same (kernel, grid) in a
    kernel-trace run of the same command, the issued rate and its fraction of
    the dense bf16 peak; mfma_busy is SQ_VALU_MFMA_BUSY_CYCLES (summed over
    the SIMDs) over GRBM_GUI_ACTIVE per XCD (the csv sums it over the Num_Xcc
    XCDs) times Simd_Count: the share of SIMD cycles with a matrix op in
    flight while the kernel ran (the counter profiler's MfmaUtil)."""
    agent = [r for r in _read_csv(os.path.join(mfma_dir, "run_agent_info.csv")) if int(r.get("Simd_Count") or 0) > 0][0]
    n_xcc, n_simd = int(agent["Num_Xcc"]), int(agent["Simd_Count"])
    vals = {}
    for r in _read_csv(os.path.join(mfma_dir, "run_counter_collection.csv")):
        if r["Counter_Name"] not in MFMA_COUNTERS:
            continue
        k = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
        vals.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
    dur = {}
    for r in _read_csv(os.path.join(trace_dir, "run_kernel_trace.csv")):
        k = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
        dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"# {'kernel':<44} {'grid':>9} {'calls':>6} {'mfma_GFLOP':>10} {'trace_us':>9} {'TFLOP/s':>8} "
          f"{'of_peak':>7} {'mfma_busy':>9}")
    rows = []
    for k, d in vals.items():
        per = [x for x in d.values() if len(x) == len(MFMA_COUNTERS)]
        if not per:
            continue
        mops = float(np.median([x["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for x in per]))
        if mops == 0:
            continue
        util = float(np.median([x["SQ_VALU_MFMA_BUSY_CYCLES"] / (x["GRBM_GUI_ACTIVE"] / n_xcc * n_simd)
                                for x in per if x["GRBM_GUI_ACTIVE"] > 0]))
        fl = mops * 512
        us = float(np.median(dur[k])) if k in dur else float("nan")
        rows.append((fl * len(per), k, len(per), fl, us, util))
    for _, k, n, fl, us, bf in sorted(rows, key=lambda t: -t[0]):
        tf = fl / (us * 1e-6) / 1e12 if us == us else float("nan")
        print(f"# {k[0][:44]:<44} {k[1]:>9} {n:>6} {fl / 1e9:>10.3f} {us:>9.2f} {tf:>8.1f} "
              f"{tf / BF16_MFMA_TFLOPS:>7.3f} {bf:>9.3f}")
    print(f"kernel_source_sha256: {kernel_sha()}")


def measured_mfma_flops(kernel, summary):
    """bf16 MFMA flops per launch of `kernel` from a committed counter summary
    (None when the kernel source changed since it was taken, or there is none)."""
    path = os.path.join(ROOT, "profiles", summary)
    try:
        rec = {}
        for line in open(path):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
        if rec.get("kernel_source_sha256") != kernel_sha():
            return None
        return float(rec[f"{kernel}_mfma_flops_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


STALL_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_INST_LEVEL_VMEM")


def summarize_stalls(d):
    """Where the waves of each (kernel, grid) spend their cycles, from a
    `rocprofv3 --pmc` run of STALL_COUNTERS: each counter's median per
    dispatch over SQ_WAVE_CYCLES (wait_any: waiting on a memory or LDS
    counter; wait_inst_any: ready but not issued; active_*: issuing;
    inst_level_vmem: vector memory instructions in flight per wave)."""
    acc = {}
    for r in _read_csv(os.path.join(d, "run_counter_collection.csv")):
        k = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = [c for c in STALL_COUNTERS if c != "SQ_WAVE_CYCLES"]
    print(f"# {'kernel':<40} {'grid':>9} {'calls':>6} " + " ".join(f"{c[3:].lower():>16}" for c in names))
    for k in sorted(acc, key=lambda k: -sum(acc[k].get("SQ_WAVE_CYCLES", [0]))):
        cs = acc[k]
        if "SQ_WAVE_CYCLES" not in cs or len(cs["SQ_WAVE_CYCLES"]) < 20:
            continue
        wc = float(np.median(cs["SQ_WAVE_CYCLES"])) or 1.0
        print(f"# {k[0][:40]:<40} {k[1]:>9} {len(cs['SQ_WAVE_CYCLES']):>6} " +
              " ".join(f"{float(np.median(cs.get(c, [0]))) / wc:>16.3f}" for c in names))
    print(f"kernel_source_sha256: {kernel_sha()}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the single-layer objects")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 256 MiB elementwise copy (256 MiB read + 256 MiB written) before the timed "
                         "region, as the reference dispatch for HBM byte counters")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the per-kernel summary of a rocprofv3 --kernel-trace csv run and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the per-kernel HBM bytes of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-stalls", metavar="DIR",
                    help="print the wave-cycle breakdown of a rocprofv3 --pmc run of STALL_COUNTERS")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("MFMA_DIR", "TRACE_DIR"),
                    help="print the per-kernel matrix-core work of a rocprofv3 --pmc run of the MFMA counters "
                         "(durations from a kernel-trace run of the same command) and exit")
    args = ap.parse_args()
    if args.summarize_stalls:
        summarize_stalls(args.summarize_stalls)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 2:
        print("--steps must be >= 2 (the timed steps alternate two states)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dllm_inputs as di
    from dllm_inputs import device as DV
    from masked_block_diffusion_amd import binding as B

    res, host = thinking_step(torch, di, B, DV, args.steps, args.warmup, args.calibrate_copy)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(torch, host)
    else:
        res["cpu_baseline"] = None
    del host
    torch.cuda.empty_cache()
    if not args.no_secondary:
        log("layer_bf16")
        res["layer_bf16"] = layer_step(torch, di, B, DV, "layer_bf16", copies=4, steps=100, warmup=10,
                                       counters=None)
        torch.cuda.empty_cache()
        log("und_layer")
        und = layer_step(torch, di, B, DV, "und_layer", copies=2, steps=30, warmup=5)
        torch.cuda.empty_cache()
        log("und_layer, SPRINT keep 0.5")
        sp = layer_step(torch, di, B, DV, "und_layer", copies=2, steps=30, warmup=5, keep=0.5)
        att_full = und["kernels"].get("attention", {}).get("mean_launch_us")
        att_sp = sp["kernels"].get("attention", {}).get("mean_launch_us")
        und["sprint_keep_half"] = {
            "keep_ratio": 0.5, "kept_positions": sp["kept_positions"], "ms_per_step": sp["ms_per_step"],
            "step_speedup_vs_full_retention": round(und["ms_per_step"] / sp["ms_per_step"], 3),
            "attention_us": att_sp, "attention_us_full_retention": att_full,
            "attention_speedup": round(att_full / att_sp, 3) if att_full and att_sp else None,
            "kernels": sp["kernels"],
            "how": "the same layer and step with retention by attention mass (step 0 of the block scores the "
                   "prefix and keeps ceil(0.5 P) positions; the timed steps attend over them through the "
                   "kept-index gather kernel) against full retention"}
        res["understanding_layer"] = und
        torch.cuda.empty_cache()
        log("t2i_cfg, 20 layers")
        res["t2i_stack"] = stack_steps(torch, di, B, DV, "t2i_cfg", steps=10, warmup=2)
        log("und_sprint, 20 layers")
        res["und_stack"] = stack_steps(torch, di, B, DV, "und_sprint", steps=10, warmup=2, keeps=(None, 0.5))
        u = res["und_stack"]
        u["sprint_step_speedup"] = round(u["full_retention"]["step_ms"] / u["sprint_keep_0.5"]["step_ms"], 3)
        u["sprint_block_speedup"] = round(u["full_retention"]["block_ms"] / u["sprint_keep_0.5"]["block_ms"], 3)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
