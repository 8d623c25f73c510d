"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module only *produces* inputs: model shapes, generation knobs, weights
in their storage format (float32 bits, bfloat16 bits, OCP E4M3FN codes plus
per-row float32 scales) and token ids.  It holds none of the denoising step's
arithmetic; both the oracle and the GPU library consume what it returns and
decode it with code of their own.

Shapes follow the workloads described for the LLaDA2.0-Uni MoE backbone
(arXiv 2604.20796 paper review, "MoE backbone and block-wise attention";
model card, "Hardware requirements": 16B total / ~1B active parameters).  The
pages give no layer dimensions, so the 16B-scale shape below is a chosen
stand-in (hidden 2048, 16x128 heads, 256 experts top-8 + 1 shared, expert FFN
512), consistent with the stated totals.

Weights are N(0, 0.02) (drawn with numpy's PCG64 normal sampler), router
biases U(-0.1, 0.1) (the auxiliary-loss-free selection bias), norm gains 1.
Every tensor (every expert matrix, for the routed experts) has its own child
seed, so a tensor's values do not depend on which other tensors a
configuration contains.
"""
from __future__ import annotations

import copy
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, asdict

import numpy as np

# ----------------------------------------------------------------------------
# configuration records
# ----------------------------------------------------------------------------

DTYPES = ("f32", "bf16", "fp8")


@dataclass
class ModelConfig:
    n_layers: int
    hidden: int
    n_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    n_shared: int          # 0 or 1 shared expert
    expert_ffn: int
    shared_ffn: int
    vocab_text: int
    vocab_image: int
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    act_dtype: str = "bf16"     # dense weights / activations: "f32" | "bf16"
    expert_dtype: str = "bf16"  # routed expert weights: "f32" | "bf16" | "fp8"

    @property
    def vocab(self) -> int:
        return self.vocab_text + self.vocab_image

    @property
    def mask_id(self) -> int:
        # text ids [0, Vt), visual ids [Vt, Vt+Vv), then the [MASK] id
        return self.vocab_text + self.vocab_image


@dataclass
class GenParams:
    block_length: int = 32
    steps: int = 8
    n_seq: int = 1                # logical sequences (CFG doubles the rows)
    cfg_scale: float = 0.0        # <= 0: CFG off
    cfg_text_scale: float = 0.0   # > 0: three-way editing guidance (rows: full,
    cfg_image_scale: float = 1.0  # image-only, unconditional); cfg_scale must be off
    vocab_lo: int = 0
    vocab_hi: int = 0             # 0 -> full vocabulary
    confidence: int = 0           # 0 low_confidence, 1 top_k_margin, 2 neg_entropy
    use_threshold: bool = False
    threshold: float = 0.93
    use_sprint: bool = False
    keep_ratio: float = 1.0
    cache_warmup_steps: int = 1
    retention_score: int = 0      # 0 accumulated attention mass, 1 key norm + confidence
    retention_alpha: float = 0.5  # weight of the normalized key norm in score 1
    image_keep_ratio: float = 0.0  # > 0: visual prefix positions form their own pool
    text_keep_ratio: float = 0.0   # > 0: the other positions form their own pool

    @property
    def cfg_on(self) -> bool:
        return self.cfg_scale > 0.0

    @property
    def cfg3_on(self) -> bool:
        return self.cfg_text_scale > 0.0

    @property
    def group(self) -> int:
        """Model rows per sequence."""
        return 3 if self.cfg3_on else (2 if self.cfg_on else 1)

    @property
    def rows(self) -> int:
        return self.n_seq * self.group


@dataclass
class Workload:
    name: str
    model: ModelConfig
    gen: GenParams
    prefix_len: int               # cached prefix tokens per row
    n_blocks: int = 1             # blocks generated
    masked_in_block: int = 32     # [MASK] positions at the start of the block
    description: str = ""
    prefix_visual: int = 0        # leading visual ids in the prefix (rest text)

    def to_dict(self):
        d = asdict(self)
        return d


def _base_big(act="bf16", expert="bf16", layers=20, vt=157184, vv=16384):
    return ModelConfig(n_layers=layers, hidden=2048, n_heads=16, head_dim=128,
                       n_experts=256, top_k=8, n_shared=1, expert_ffn=512,
                       shared_ffn=512, vocab_text=vt, vocab_image=vv,
                       act_dtype=act, expert_dtype=expert)


def workload(name: str) -> Workload:
    """Named workloads.  The first five mirror the published problem set."""
    if name == "tiny_fp32":
        m = ModelConfig(n_layers=2, hidden=256, n_heads=8, head_dim=32,
                        n_experts=16, top_k=2, n_shared=1, expert_ffn=128,
                        shared_ffn=128, vocab_text=4096, vocab_image=0,
                        act_dtype="f32", expert_dtype="f32")
        g = GenParams(block_length=32, steps=8, n_seq=1)
        return Workload(name, m, g, prefix_len=64, masked_in_block=32,
                        description="2-layer fp32 plumbing model, 64-token prefix, "
                                    "one 32-token block in 8 steps")
    if name == "layer_bf16":
        m = _base_big(layers=1, vt=4096, vv=0)
        g = GenParams(block_length=32, steps=8, n_seq=1)
        return Workload(name, m, g, prefix_len=1024, masked_in_block=16,
                        description="one 16B-scale MoE layer, bf16, 1024-token cached "
                                    "prefix, 32-token block with 16 [MASK]")
    if name == "t2i_cfg":
        m = _base_big()
        g = GenParams(block_length=32, steps=8, n_seq=1, cfg_scale=2.0,
                      vocab_lo=157184, vocab_hi=157184 + 16384)
        return Workload(name, m, g, prefix_len=256, n_blocks=128,
                        description="text-to-image: 20 layers, CFG pair, 4096 visual "
                                    "tokens in 128 blocks x 8 steps")
    if name == "und_sprint":
        m = _base_big()
        g = GenParams(block_length=32, steps=32, n_seq=1, vocab_lo=0,
                      vocab_hi=157184, use_threshold=True, threshold=0.9,
                      use_sprint=True, keep_ratio=0.5, cache_warmup_steps=1)
        return Workload(name, m, g, prefix_len=4160, n_blocks=64,
                        prefix_visual=4096,
                        description="understanding with SPRINT: 4096 visual + 64 text "
                                    "prefix, 2048 generated, threshold 0.9, keep 0.5")
    if name == "think_fp8":
        m = _base_big(expert="fp8")
        g = GenParams(block_length=32, steps=32, n_seq=16, vocab_lo=0, vocab_hi=157184)
        return Workload(name, m, g, prefix_len=2048, n_blocks=128,
                        description="batched thinking: 16 sequences, fp8 experts, "
                                    "4096 generated in 128 blocks x 32 steps")
    if name == "think_fp8_layer":
        # one layer of the batched thinking workload: fp8 experts, 16
        # sequences, 2048-token prefixes, 16 [MASK] left in the block at step
        # 16 of 32 (one commit per sequence), LM head over the full text
        # sub-vocabulary (256 head rows x 157,184 ids)
        m = _base_big(expert="fp8", layers=1)
        g = GenParams(block_length=32, steps=32, n_seq=16, vocab_lo=0, vocab_hi=157184)
        return Workload(name, m, g, prefix_len=2048, masked_in_block=16,
                        description="one fp8-expert layer of the batched thinking shape: 16 "
                                    "sequences x 2048-token prefix, 32-token blocks")
    if name == "und_layer":
        # one layer of the understanding shape, without retention: one
        # sequence, 4096 visual + 64 text prefix ids, 16 [MASK] left in the
        # 32-token block, LM head over the full text sub-vocabulary (16 head
        # rows x 157,184 ids: the streaming head, 644 MB per step)
        m = _base_big(layers=1)
        g = GenParams(block_length=32, steps=32, n_seq=1, vocab_lo=0, vocab_hi=157184)
        return Workload(name, m, g, prefix_len=4160, masked_in_block=16, prefix_visual=4096,
                        description="one bf16 layer of the understanding shape: 4096 visual + 64 text "
                                    "prefix, 16 [MASK], LM head over 157,184 text ids")
    if name == "t2i_layer":
        # one layer of the text-to-image shape: a CFG pair (the unconditional
        # row's prompt is all [MASK]), 256-token prompt, an all-[MASK] block of
        # 32 in 8 steps of 4, LM head over the 16,384-id visual sub-vocabulary
        m = _base_big(layers=1)
        g = GenParams(block_length=32, steps=8, n_seq=1, cfg_scale=2.0,
                      vocab_lo=157184, vocab_hi=157184 + 16384)
        return Workload(name, m, g, prefix_len=256, masked_in_block=32,
                        description="one bf16 layer of the text-to-image shape: CFG pair, "
                                    "256-token prompt, visual sub-vocabulary")
    # reduced-size feature cases (same code paths, shapes the oracle finishes fast)
    if name == "small_bf16":
        m = ModelConfig(n_layers=2, hidden=256, n_heads=4, head_dim=64,
                        n_experts=32, top_k=4, n_shared=1, expert_ffn=128,
                        shared_ffn=128, vocab_text=1000, vocab_image=512,
                        act_dtype="bf16", expert_dtype="bf16")
        g = GenParams(block_length=32, steps=8, n_seq=1)
        return Workload(name, m, g, prefix_len=96, masked_in_block=32)
    if name == "small_cfg":
        w = workload("small_bf16")
        w.name = name
        w.gen.cfg_scale = 2.0
        w.gen.vocab_lo, w.gen.vocab_hi = 1000, 1512
        return w
    if name == "small_sprint":
        w = workload("small_bf16")
        w.name = name
        w.gen.use_sprint = True
        w.gen.keep_ratio = 0.5
        w.gen.use_threshold = True
        w.gen.threshold = 0.9
        w.gen.steps = 32
        w.gen.vocab_lo, w.gen.vocab_hi = 0, 1000
        w.prefix_visual = 64
        return w
    if name == "small_sprint_kc":
        # the review's SPRINT variant: key norm + confidence score, image pool
        # kept at 0.8 and text pool at 1.0
        w = workload("small_sprint")
        w.name = name
        w.gen.retention_score = 1
        w.gen.retention_alpha = 0.5
        w.gen.image_keep_ratio = 0.8
        w.gen.text_keep_ratio = 1.0
        return w
    if name == "small_edit":
        # editing: source image (64 visual ids) + instruction (32 text ids),
        # three-way guidance with the model card's text scale 4.0 (image scale
        # 1.5 is a chosen value; the pages give none); visual sub-vocabulary
        w = workload("small_bf16")
        w.name = name
        w.prefix_visual = 64
        w.gen.cfg_text_scale = 4.0
        w.gen.cfg_image_scale = 1.5
        w.gen.vocab_lo, w.gen.vocab_hi = 1000, 1512
        return w
    if name == "small_fp8":
        # fp8 expert fragments span 64 reduction elements: hidden a multiple
        # of 512 (8 wavefronts split it)
        w = workload("small_bf16")
        w.name = name
        w.model.expert_dtype = "fp8"
        w.model.hidden = 512
        w.gen.n_seq = 4
        w.gen.steps = 32
        w.gen.vocab_lo, w.gen.vocab_hi = 0, 1000
        return w
    raise KeyError(name)


PUBLISHED_WORKLOADS = ("tiny_fp32", "layer_bf16", "t2i_cfg", "und_sprint", "think_fp8")

# ----------------------------------------------------------------------------
# storage-format encoders (input preparation only)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def _e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """Encode float64 values that are already representable in OCP E4M3FN
    (|v| <= 448, on the format's grid) into their 8-bit codes."""
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    code = np.zeros(v.shape, dtype=np.uint8)
    nz = a > 0
    sub = nz & (a < 2.0 ** -6)
    nrm = nz & ~sub
    # subnormals: value = mant * 2^-9
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.uint8)
    _, ex = np.frexp(a[nrm])              # a = f * 2^ex, f in [0.5, 1)
    e = ex - 1                            # a = 1.m * 2^e
    mant = np.rint((a[nrm] / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    code[nrm] = (((e + 7) << 3) | mant).astype(np.uint8)
    return code | sign


def quantize_rows_e4m3fn(w: np.ndarray, chunk_rows: int = 1 << 14):
    """Per-output-row weight quantization to OCP E4M3FN.

    scale = amax(row) / 448 (float32); code = saturate(round-half-even(w/scale))
    on the E4M3FN grid.  Returns (uint8 codes, float32 scales[rows]).

    Bit-level form of quantize_rows_e4m3fn_reference (same codes): the
    quotient is formed in float64; normal magnitudes (>= 2^-6) are rounded to
    3 mantissa bits half-to-even on their float64 bits, subnormal ones to
    multiples of 2^-9; the code is read off the rounded exponent and
    mantissa.  Rows are processed in chunks to bound memory."""
    w = np.asarray(w, np.float32)
    shape = w.shape
    rows = w.reshape(-1, shape[-1])
    codes = np.empty(rows.shape, np.uint8)
    scales = np.empty(rows.shape[0], np.float32)
    for r0 in range(0, rows.shape[0], chunk_rows):
        blk = rows[r0: r0 + chunk_rows].astype(np.float64)
        amax = np.max(np.abs(blk), axis=-1)
        sc = (amax / 448.0).astype(np.float32)
        sc = np.where(sc == 0, np.float32(1.0), sc)
        x = blk / sc.astype(np.float64)[:, None]
        neg = np.signbit(x)
        a = np.minimum(np.abs(x), 448.0)
        u = a.view(np.uint64)
        lsb = (u >> np.uint64(49)) & np.uint64(1)
        ur = (u + np.uint64((1 << 48) - 1) + lsb) & ~np.uint64((1 << 49) - 1)
        e = ((ur >> np.uint64(52)).astype(np.int64) & 0x7FF) - 1023
        m = ((ur >> np.uint64(49)) & np.uint64(7)).astype(np.int64)
        normal = (e + 7) << 3 | m
        normal = np.minimum(normal, 0x7E)                       # saturate at 448
        sub = np.rint(a / 2.0 ** -9).astype(np.int64)            # half to even; 8 = smallest normal
        c = np.where(a >= 2.0 ** -6, normal, sub)
        codes[r0: r0 + chunk_rows] = (c | (neg.astype(np.int64) << 7)).astype(np.uint8)
        scales[r0: r0 + chunk_rows] = sc
    return codes.reshape(shape), scales.reshape(shape[:-1])


def quantize_rows_e4m3fn_reference(w: np.ndarray):
    """Per-output-row E4M3FN quantization written with frexp / ldexp (slow
    reference for quantize_rows_e4m3fn)."""
    w64 = w.astype(np.float64)
    amax = np.max(np.abs(w64), axis=-1)
    scale = (amax / 448.0).astype(np.float32)
    scale = np.where(scale == 0, np.float32(1.0), scale)
    x = w64 / scale.astype(np.float64)[..., None]
    a = np.minimum(np.abs(x), 448.0)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -10))
    e = np.maximum(ex - 1, -6)
    q = np.ldexp(1.0, e - 3)              # grid spacing in this binade
    v = np.minimum(np.rint(a / q) * q, 448.0)  # np.rint: half to even
    v = np.copysign(v, x)
    return _e4m3fn_encode(v), scale


# ----------------------------------------------------------------------------
# weights and token ids
# ----------------------------------------------------------------------------

_TAGS = {"embed": 1, "attn_norm": 2, "w_qkv": 3, "w_o": 4, "moe_norm": 5,
         "w_router": 6, "router_bias": 7, "w_gate": 8, "w_up": 9, "w_down": 10,
         "ws_gate": 11, "ws_up": 12, "ws_down": 13, "final_norm": 14, "lm_head": 15}


def _normal(seed, tag, layer, shape, std=0.02):
    rng = np.random.default_rng([seed, _TAGS[tag], layer])
    return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)


def _store(x, dt):
    if dt == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dt == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dt)


def make_weights(m: ModelConfig, seed: int = 0, layers=None) -> dict:
    """All weights in storage format (dense: m.act_dtype; experts: m.expert_dtype).

    Layout (row-major, output dimension first, reduction dimension contiguous):
      embed [V+1, D]; attn_norm/moe_norm [L, D] f32; w_qkv [L, 3*H*dh, D]
      (rows: q heads, then k heads, then v heads); w_o [L, D, H*dh];
      w_router [L, E, D]; router_bias [L, E] f32; w_gate/w_up [L, E, F, D];
      w_down [L, E, D, F]; (fp8: s_gate/s_up [L, E, F], s_down [L, E, D] f32);
      ws_gate/ws_up [L, Fs, D]; ws_down [L, D, Fs]; final_norm [D] f32;
      lm_head [V, D].
    ``layers`` restricts generation to a subset of layer indices (others are
    returned as None) for callers that only need some layers."""
    D, H, dh, E, F, Fs = m.hidden, m.n_heads, m.head_dim, m.n_experts, m.expert_ffn, m.shared_ffn
    L = m.n_layers
    ad, ed = m.act_dtype, m.expert_dtype
    want = range(L) if layers is None else layers
    w = {"dtypes": {"dense": ad, "expert": ed}}
    w["embed"] = _store(_normal(seed, "embed", 0, (m.vocab + 1, D)), ad)
    w["final_norm"] = np.ones(D, np.float32)
    w["lm_head"] = _store(_normal(seed, "lm_head", 0, (m.vocab, D)), ad)

    def stack(fn):
        out = [None] * L
        for l in want:
            out[l] = fn(l)
        if layers is None:
            return np.stack(out)
        return out

    w["attn_norm"] = stack(lambda l: np.ones(D, np.float32))
    w["moe_norm"] = stack(lambda l: np.ones(D, np.float32))
    w["w_qkv"] = stack(lambda l: _store(_normal(seed, "w_qkv", l, (3 * H * dh, D)), ad))
    w["w_o"] = stack(lambda l: _store(_normal(seed, "w_o", l, (D, H * dh)), ad))
    w["w_router"] = stack(lambda l: _store(_normal(seed, "w_router", l, (E, D)), ad))
    w["router_bias"] = stack(lambda l: np.random.default_rng([seed, _TAGS["router_bias"], l])
                             .uniform(-0.1, 0.1, size=E).astype(np.float32))

    def expert(tag, shape, l):
        # one child seed per expert; experts are drawn (and quantized) on a
        # thread pool, since numpy releases the interpreter lock in both
        n_e = shape[0]
        vals = np.empty(shape, np.uint8 if ed == "fp8" else (np.float32 if ed == "f32" else np.uint16))
        scales = np.empty(shape[:-1], np.float32) if ed == "fp8" else None

        def one(e):
            rng = np.random.default_rng([seed, _TAGS[tag], l, 1000 + e])
            x = rng.standard_normal(size=shape[1:], dtype=np.float32) * np.float32(0.02)
            if ed == "fp8":
                vals[e], scales[e] = quantize_rows_e4m3fn(x)
            else:
                vals[e] = _store(x, ed)

        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, range(n_e)))
        return vals, scales

    for tag, shape, stag in (("w_gate", (E, F, D), "s_gate"),
                             ("w_up", (E, F, D), "s_up"),
                             ("w_down", (E, D, F), "s_down")):
        vals = [None] * L
        scales = [None] * L
        for l in want:
            vals[l], scales[l] = expert(tag, shape, l)
        if layers is None:
            w[tag] = np.stack(vals)
            w[stag] = np.stack(scales) if ed == "fp8" else None
        else:
            w[tag] = vals
            w[stag] = scales if ed == "fp8" else None
    if m.n_shared:
        w["ws_gate"] = stack(lambda l: _store(_normal(seed, "ws_gate", l, (Fs, D)), ad))
        w["ws_up"] = stack(lambda l: _store(_normal(seed, "ws_up", l, (Fs, D)), ad))
        w["ws_down"] = stack(lambda l: _store(_normal(seed, "ws_down", l, (D, Fs)), ad))
    else:
        w["ws_gate"] = w["ws_up"] = w["ws_down"] = None
    return w


def make_prefix(wl: Workload, seed: int = 0) -> np.ndarray:
    """Prefix ids [rows, prefix_len].  The first ``prefix_visual`` positions are
    visual ids, the rest text ids; with CFG the unconditional row (odd rows)
    is the same prompt with every id replaced by [MASK].  With three-way
    guidance the rows of a sequence are (full prompt, the prompt with its text
    ids replaced by [MASK], all [MASK])."""
    m, g = wl.model, wl.gen
    rng = np.random.default_rng([seed, 101])
    ids = np.empty((g.n_seq, wl.prefix_len), np.int32)
    nv = wl.prefix_visual
    if nv:
        ids[:, :nv] = rng.integers(m.vocab_text, m.vocab_text + m.vocab_image, size=(g.n_seq, nv))
    ids[:, nv:] = rng.integers(0, m.vocab_text, size=(g.n_seq, wl.prefix_len - nv))
    if g.cfg3_on:
        rows = np.full((3 * g.n_seq, wl.prefix_len), m.mask_id, np.int32)
        rows[0::3] = ids
        rows[1::3, :nv] = ids[:, :nv]
        return rows
    if not g.cfg_on:
        return ids
    rows = np.empty((2 * g.n_seq, wl.prefix_len), np.int32)
    rows[0::2] = ids
    rows[1::2] = m.mask_id
    return rows


def make_block(wl: Workload, seed: int = 0) -> np.ndarray:
    """Block ids [n_seq, L_B]: ``masked_in_block`` positions (a seeded
    permutation) are [MASK]; the others are fixed random ids from the
    generation sub-vocabulary."""
    m, g = wl.model, wl.gen
    rng = np.random.default_rng([seed, 102])
    lo, hi = g.vocab_lo, (g.vocab_hi or m.vocab)
    ids = rng.integers(lo, hi, size=(g.n_seq, g.block_length)).astype(np.int32)
    for s in range(g.n_seq):
        pos = rng.permutation(g.block_length)[: wl.masked_in_block]
        ids[s, pos] = m.mask_id
    return ids


def clone(wl: Workload) -> Workload:
    return copy.deepcopy(wl)
