"""Oracle for the block-level masked-diffusion denoising step (TEST INFRASTRUCTURE).

This is a plain, slow, float64 CPU statement of what the GPU library computes.
It exists only to check the GPU path: nothing outside ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it, and it imports nothing from the GPU package.  It shares no
code with the HIP kernels; only the seeded input generators (``dllm_inputs``)
feed both sides.

Sources (the pages are the authority; where they are silent the reading taken
is stated next to the code):
  * P2 = arXiv 2604.20796 paper review (baba9811.github.io), sections
    "Diffusion LLM", "Block Diffusion Language Model (BDLM)", "Mixture-of-Experts",
    "MoE backbone and block-wise attention", "Positional embedding",
    "SPRINT - training-free inference acceleration", "BDLM loss",
    "Load balancing - auxiliary-loss-free MoE bias".
  * P4 = LLaDA2.0-Uni model card (ai.gitcode.com mirror), sections
    "SPRINT acceleration" and the understand_image / generate_image examples.

Every floating-point quantity is float64 except where a decision is defined in
the kernel's precision (router sigmoid rounded to float32 and the biased key
added in float32), because the pages fix no precision.

Pins: tests/test_oracle_*.py check each function here against brute force,
closed forms and special cases; the header of each function names its pin.
Parity unpinned: fidelity to the real LLaDA2.0-Uni weights/code (none exist
here).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------------------
# storage decoders
# ----------------------------------------------------------------------------


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float64 (exact: bfloat16 is the top half of float32)."""
    u32 = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3FN code -> float64.

    Definition (OCP 8-bit floating point spec, E4M3 variant): 1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent 0 encodes
    subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN; there are no
    infinities, so exponent 15 with mantissa 0..6 are normal numbers (max 448).
    Pin: exhaustive 256-code table built independently in the tests."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    v = np.where(e == 0, sub, nrm)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


_E4M3FN_TABLE = None


def decode(arr, dt: str) -> np.ndarray:
    """Storage format -> float64.  fp8 codes go through the 256-entry table of
    e4m3fn_to_f64 (the same definition, evaluated once per code)."""
    global _E4M3FN_TABLE
    if dt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dt == "bf16":
        return bf16_to_f64(arr)
    if dt == "fp8":
        if _E4M3FN_TABLE is None:
            _E4M3FN_TABLE = e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
        return _E4M3FN_TABLE[np.asarray(arr, dtype=np.uint8)]
    raise ValueError(dt)


# ----------------------------------------------------------------------------
# model weights (decoded lazily)
# ----------------------------------------------------------------------------


class Model:
    """Float64 view of a weight set produced by ``dllm_inputs.make_weights``."""

    def __init__(self, cfg, weights: dict, keep_experts=False):
        self.cfg = cfg
        self.w = weights
        self.ad = weights["dtypes"]["dense"]
        self.ed = weights["dtypes"]["expert"]
        self._dense = {}
        # keep_experts: remember decoded expert matrices (large models stepped
        # several times; memory 8 bytes per weight)
        self._experts = {} if keep_experts else None

    def dense(self, name, l=None):
        key = (name, l)
        if key not in self._dense:
            a = self.w[name] if l is None else self.w[name][l]
            dt = "f32" if a.dtype == np.float32 else self.ad
            self._dense[key] = decode(a, dt)
        return self._dense[key]

    def expert(self, name, l, e):
        """Routed expert matrix in float64; fp8 codes times their per-row scale."""
        key = (name, l, int(e))
        if self._experts is not None and key in self._experts:
            return self._experts[key]
        a = decode(self.w[name][l][e], self.ed)
        if self.ed == "fp8":
            sc = self.w["s" + name[1:]][l][e].astype(np.float64)
            a = a * sc[:, None]
        if self._experts is not None:
            self._experts[key] = a
        return a

    def embed(self, ids):
        return decode(self.w["embed"][np.asarray(ids)], self.ad)


# ----------------------------------------------------------------------------
# primitives
# ----------------------------------------------------------------------------


def rmsnorm(x, gain, eps):
    """RMSNorm with gains (reading: pre-norm RMSNorm, eps 1e-6; the pages name
    no normalisation).  Pin: unit-RMS output for gain 1, scale invariance."""
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * gain


def rope(x, pos, base):
    """1D rotary embedding (P2 "Positional embedding": 1D RoPE over the
    raster-flattened sequence).  Reading: rotate-half pairs (i, i+d/2),
    theta_i = base^(-2i/d), absolute 0-based positions.
    x: [n, H, d]; pos: [n].  Pins: norm preservation, position-shift
    invariance of q.k, identity at position 0."""
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def block_visible(qpos, kpos, block_len):
    """Block-wise attention mask (P2 "BDLM": diffusion inside a block, left to
    right across blocks; "MoE backbone and block-wise attention": the same
    pattern restricts attention).  Blocks are aligned from position 0.
    A key is visible iff its block index <= the query's block index.
    Pins: block length 1 gives the causal mask; one block over the whole
    sequence gives full bidirectional attention."""
    qb = np.asarray(qpos)[:, None] // block_len
    kb = np.asarray(kpos)[None, :] // block_len
    return kb <= qb


def attention(q, k, v, qpos, kpos, block_len):
    """softmax(q k^T / sqrt(d) + mask) v, written as the full score matrix.
    q: [nq, H, d]; k, v: [nk, H, d].  Returns (out [nq, H, d], probs [H, nq, nk]).
    Reading: multi-head attention with as many K/V heads as query heads, no
    biases, no QK-norm.  Pin: scalar-loop brute force; causal/bidirectional
    special cases; rows of probs sum to 1."""
    d = q.shape[-1]
    s = np.einsum("qhd,khd->hqk", q, k) / math.sqrt(d)
    vis = block_visible(qpos, kpos, block_len)
    s = np.where(vis[None], s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return np.einsum("hqk,khd->qhd", p, v), p


def sigmoid_f32(z):
    """Router score: sigmoid evaluated in float64 and rounded to float32
    (the kernel's precision for this decision)."""
    return (1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))).astype(np.float32)


def keys_from_logits(z, bias):
    """Scores s = sigmoid(z) (-> float32) and selection keys s + b added in
    float32, from router logits z [n, E]."""
    s = sigmoid_f32(z)
    key = s + np.asarray(bias, np.float32)[None, :]     # float32 + float32
    return s, key.astype(np.float32)


def route_keys(x, w_router, bias):
    """Router logits z = x W_r^T (float64), scores s = sigmoid (-> float32) and
    selection keys s + b added in float32 (P2 "Load balancing": the
    auxiliary-loss-free bias steers expert *selection*; P2 "Mixture-of-Experts":
    top-k experts per token)."""
    z = x @ w_router.T
    s, key = keys_from_logits(z, bias)
    return z, s, key


def topk_desc(key_row, k):
    """Indices of the k largest keys, ties to the lower index (stable order).
    Pin: equals a full stable sort."""
    order = np.lexsort((np.arange(len(key_row)), -np.asarray(key_row, np.float64)))
    return order[:k]


def gates_from(s_row, sel):
    """Gates = unbiased sigmoid scores of the selected experts normalised to sum
    1 (reading R6).  Pin: identical experts reproduce the dense FFN."""
    g = np.asarray(s_row, np.float64)[sel]
    return g / g.sum()


def swiglu(x, wg, wu, wd):
    """SwiGLU feed-forward W_d (silu(W_g x) * (W_u x)); matrices are
    [out, in].  Pin: hand-expanded scalar loop."""
    a = x @ wg.T
    b = x @ wu.T
    hmid = a / (1.0 + np.exp(-a)) * b
    return hmid @ wd.T


def cfg_mix(l_cond, l_uncond, w):
    """Classifier-free guidance l = l_u + w (l_c - l_u) (P4 generate_image
    cfg_scale; the formula is not printed, reading R10).  Pins: w=1 -> cond,
    w=0 -> uncond."""
    return l_uncond + w * (l_cond - l_uncond)


def cfg3_mix(l_full, l_image, l_uncond, s_text, s_image):
    """Three-way editing guidance (P4 edit_image cfg_text_scale; the note on
    SPRINT names cfg_text_scale / cfg_image_scale as three-way guidance; the
    formula is not printed).  Reading: the image scale moves from the
    unconditional to the image-only prediction, the text scale from the
    image-only to the full one:
        l = l_u + s_img (l_img - l_u) + s_txt (l_full - l_img).
    Pins: s_img = s_txt = 1 -> l_full; both 0 -> l_u; l_img = l_u reduces to
    two-way CFG with w = s_txt."""
    return l_uncond + s_image * (l_image - l_uncond) + s_text * (l_full - l_image)


def confidence(logits, strategy=0):
    """Per row: argmax (ties to the lower id) and confidence.
    strategy 0 low_confidence: c = max p = 1 / sum exp(l - l_max)
    (P2 SPRINT: c_i = max_v p(v|x_t)); 1 top_k_margin: p1 - p2;
    2 neg_entropy: sum p log p (P4 SPRINT strategies).
    Pins: np.argmax first occurrence; closed forms on crafted rows."""
    l = np.asarray(logits, np.float64)
    xhat = np.argmax(l, axis=-1)
    m = np.max(l, axis=-1, keepdims=True)
    e = np.exp(l - m)
    z = e.sum(axis=-1)
    if strategy == 0:
        c = 1.0 / z
    elif strategy == 1:
        p = e / z[:, None]
        ps = np.sort(p, axis=-1)
        c = ps[:, -1] - ps[:, -2]
    elif strategy == 2:
        p = e / z[:, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            c = np.sum(np.where(p > 0, p * np.log(p), 0.0), axis=-1)
    else:
        raise ValueError(strategy)
    return xhat, c


def quota(remaining, steps, t):
    """Per-step unmask count k_t = ceil(r_t / (T - t)) (P2 SPRINT: at least
    ceil(m/(T-t)) per step; P4: ceil(remaining_masked / steps_left)).
    Pin: m=32, T=8 gives 4 each step; r reaches 0 at the last step."""
    left = steps - t
    return -(-int(remaining) // left)


def select_commit(ids_row, mask_id, xhat, conf, steps, t, use_threshold, threshold,
                  order_hint=None, hint_conf=None):
    """Commit the quota of [MASK] positions with the highest confidence
    (P2 SPRINT "non-uniform token unmasking"; P4 "batch acceptance").
    Reading: n = ceil(r/(T-t)); threshold mode n = max(n, #{c > tau});
    order by (confidence desc, position asc); committed ids never change.
    ``xhat``/``conf`` are indexed by block position (only masked positions are
    read).  ``order_hint`` / ``hint_conf``: an alternative committed set and
    the confidences it was ranked by (see Hints): adopted only if it is
    exactly the set this rule picks under ``hint_conf`` and the oracle's own
    confidences separate it from the oracle's set by at most twice the largest
    confidence difference.
    Pins: commit count equals the schedule; no [MASK] after the last step."""
    ids = np.array(ids_row, copy=True)
    masked = np.nonzero(ids == mask_id)[0]
    r = len(masked)
    info = {"n": 0, "adopted": 0}
    if r == 0:
        return ids, info

    def count(c):
        n = quota(r, steps, t)
        if use_threshold:
            n = max(n, int(np.sum(c[masked] > threshold)))
        return min(n, r)

    def top(c, n):
        return np.sort(masked[np.lexsort((masked, -np.asarray(c)[masked]))][:n])

    n = count(conf)
    chosen = top(conf, n)
    if order_hint is not None and hint_conf is not None:
        hint = np.sort(np.asarray(order_hint))
        hc = np.asarray(hint_conf, np.float64)
        if not np.array_equal(hint, chosen) and len(hint) == n == count(hc) and np.array_equal(top(hc, n), hint):
            e = float(np.max(np.abs(hc[masked] - conf[masked])))
            rest = np.setdiff1d(masked, hint)
            gap = (np.max(conf[rest]) if len(rest) else -np.inf) - np.min(conf[hint])
            if gap <= 2 * e:
                chosen = hint
                info["adopted"] = 1
                info["gap"], info["window"] = float(gap), 2 * e
    ids[chosen] = xhat[chosen]
    info["n"] = int(len(chosen))
    info["chosen"] = chosen
    return ids, info


def n_keep(ratio, P):
    """Retained prefix length ceil(r P) (the understanding workload keeps the
    top 50 %).  The ratio is a float32 knob; a relative 1e-6 guard absorbs its
    binary representation so a decimal ratio such as 0.8 keeps ceil(0.8 P)."""
    r = float(np.float32(ratio))
    return int(min(P, max(0, math.ceil(r * P * (1.0 - 1e-6)))))


def retention_select(score, ratio, pool=None, pool_ratios=None):
    """Kept prefix positions: the top ceil(r P) by retention score, ties to the
    lower position, returned in ascending order (P2 SPRINT "sparse prefix
    retention", P4 "KV cache reuse and pruning").

    Modality-aware pruning (P2 SPRINT: images pruned harder than text; P4:
    image_keep_ratio / text_keep_ratio): with ``pool`` (0 text, 1 visual per
    position) and ``pool_ratios`` = (text ratio, image ratio), each pool keeps
    its own top ceil(r_p P_p) and the kept set is their union.  Pins: ratio 1
    keeps all; equals a brute-force sort per pool; |kept| = sum ceil(r_p P_p)."""
    score = np.asarray(score, np.float64)
    P = len(score)
    if pool is None or pool_ratios is None:
        pool = np.zeros(P, np.int64)
        pool_ratios = (ratio, ratio)
    pool = np.asarray(pool)
    kept = []
    for p in (0, 1):
        where = np.nonzero(pool == p)[0]
        n = n_keep(pool_ratios[p], len(where))
        order = np.lexsort((where, -score[where]))
        kept.append(where[order[:n]])
    return np.sort(np.concatenate(kept))


def modality_pool(ids, cfg):
    """Pool of each prefix position: 1 for visual ids [V_t, V_t + V_v), 0 for
    everything else (text ids and [MASK], e.g. the prompt of an unconditional
    CFG row); ids follow the model card's layout (visual id = code + offset)."""
    ids = np.asarray(ids)
    return ((ids >= cfg.vocab_text) & (ids < cfg.vocab_text + cfg.vocab_image)).astype(np.int64)


def pool_ratios_of(gen):
    """(text, image) keep ratios when modality pools are on, else None.  A pool
    whose own ratio is unset (<= 0) takes keep_ratio."""
    ri, rt = float(gen.image_keep_ratio), float(gen.text_keep_ratio)
    if ri <= 0 and rt <= 0:
        return None
    return (rt if rt > 0 else gen.keep_ratio, ri if ri > 0 else gen.keep_ratio)


def key_norms(cache, r):
    """l_i: the Euclidean norm of prefix position i's cached key, averaged over
    layers and heads (one value per position, the granularity at which the
    P2 SPRINT score prunes).  RoPE is a rotation, so post-RoPE keys give the
    same norms as pre-RoPE ones."""
    P = cache.P
    tot = np.zeros(P)
    n = 0
    for K in cache.K:
        tot += np.sqrt(np.sum(K[r, :P] ** 2, axis=-1)).sum(axis=-1)   # [P, H] -> [P]
        n += K.shape[2]
    return tot / max(n, 1)


def keynorm_conf_score(cache, r, alpha):
    """P2 SPRINT importance of prefix position i (the formula is lost in the
    page's text; reading from the surrounding definitions):
        s_i = alpha * l~_i + (1 - alpha) * c_i,
    l~_i = l_i / mean_j l_j (mean-normalized key norm over the row's prefix;
    0 when every key is zero), c_i = the top-1 probability the model assigns
    at position i (computed when the position was appended; the block-wise
    mask makes it the same at every later step)."""
    l = key_norms(cache, r)
    mu = float(np.mean(l)) if len(l) else 0.0
    lt = l / mu if mu > 0 else np.zeros_like(l)
    return alpha * lt + (1.0 - alpha) * cache.conf[r, : cache.P]


# ----------------------------------------------------------------------------
# KV cache and forward passes
# ----------------------------------------------------------------------------


@dataclass
class Cache:
    """Prefix K/V per layer and row, post-RoPE, float64: K[l] is [rows, P, H, d].
    ``ids`` [rows, P] are the prefix token ids (modality pools); ``conf``
    [rows, P] the top-1 probability at each prefix position (NaN where it was
    not computed)."""
    K: list
    V: list
    P: int = 0
    ids: np.ndarray | None = None
    conf: np.ndarray | None = None

    @staticmethod
    def empty(cfg, rows):
        H, d = cfg.n_heads, cfg.head_dim
        z = lambda: np.zeros((rows, 0, H, d))
        return Cache([z() for _ in range(cfg.n_layers)], [z() for _ in range(cfg.n_layers)], 0,
                     np.zeros((rows, 0), np.int32), np.zeros((rows, 0)))


@dataclass
class Hints:
    """Decisions another implementation of the step took, with the keys it
    took them from.  Where keys tie within rounding several decisions are
    correct (the order of equal keys is not unique), so an alternative
    decision replaces the oracle's own only when
      (1) it is exactly the decision its own keys imply under the oracle's
          rule for that decision (top-k with ties to the lower id, argmax,
          commit ranking and count, per-pool retention), and
      (2) the oracle's float64 keys separate the two decisions by at most
          2 e (+ slack for the argmax), e being the largest difference between
          the two sets of keys on that row: keys that move by at most e can
          swap two keys only when those lie within 2 e of each other.
    Given (1), (2) always holds; it is kept as a check, and the window it
    logs is how far the decisions may lie apart.  What bounds e is the
    difference of the two sets of keys itself, which callers compare against
    their tolerance.  ``log`` records every adoption as (kind, where..., gap,
    window).

    routing / router_z: layer -> expert ids [n, k] in rank order and the
    float32 router logits [n, E] they were ranked from.  xhat: absolute argmax
    ids [n_seq, L_B]; logits: per sequence, the guidance-mixed logits
    [n_masked, V_sub] of the alternative, which may differ from those its
    argmax was taken on by up to ``logit_slack`` times the row's largest
    magnitude (another summation order).  commit: per sequence the committed
    positions; conf: [n_seq, L_B] the confidences they were ranked by.  kept /
    score: per model row the kept prefix positions and [rows, >= P] the
    retention scores they were chosen by."""
    routing: dict = field(default_factory=dict)
    router_z: dict = field(default_factory=dict)
    xhat: np.ndarray | None = None
    logits: list | None = None
    logit_slack: float = 0.0
    commit: list | None = None
    conf: np.ndarray | None = None
    kept: list | None = None
    score: np.ndarray | None = None
    log: list = field(default_factory=list)


def _moe(model, l, x, hints=None, layer_tag=None):
    """Routed experts + shared expert for token rows x [n, D] (P2 "MoE": router
    picks top-k experts per token; spec: sigmoid-plus-bias top-k with a
    shared expert).  Returns (y, idx, gates, keys, router logits)."""
    cfg = model.cfg
    wr = model.dense("w_router", l)
    b = model.w["router_bias"][l]
    z, s, key = route_keys(x, wr, b)
    n = x.shape[0]
    k = cfg.top_k
    idx = np.stack([topk_desc(key[i], k) for i in range(n)]) if n else np.zeros((0, k), int)
    if hints is not None and layer_tag in hints.routing:
        alt = np.asarray(hints.routing[layer_tag])
        _, akey = keys_from_logits(np.asarray(hints.router_z[layer_tag], np.float32).astype(np.float64), b)
        k64, a64 = key.astype(np.float64), akey.astype(np.float64)
        for i in range(n):
            if np.array_equal(np.sort(alt[i]), np.sort(idx[i])):
                continue
            if not np.array_equal(alt[i], topk_desc(akey[i], k)):
                continue                                   # not what its own keys select
            e = float(np.max(np.abs(a64[i] - k64[i])))
            rest = np.setdiff1d(np.arange(cfg.n_experts), alt[i])
            gap = float(np.max(k64[i][rest]) - np.min(k64[i][alt[i]]))
            if gap <= 2 * e:
                idx[i] = alt[i]
                hints.log.append(("route", layer_tag, i, gap, 2 * e))
    gates = np.stack([gates_from(s[i], idx[i]) for i in range(n)]) if n else np.zeros((0, k))
    y = np.zeros_like(x)
    for e in np.unique(idx):
        rows, slot = np.nonzero(idx == e)
        wg = model.expert("w_gate", l, e)
        wu = model.expert("w_up", l, e)
        wd = model.expert("w_down", l, e)
        y[rows] += gates[rows, slot][:, None] * swiglu(x[rows], wg, wu, wd)
    if cfg.n_shared:
        y += swiglu(x, model.dense("ws_gate", l), model.dense("ws_up", l), model.dense("ws_down", l))
    return y, idx, gates, key, z


def layer_forward(model, l, h, cache, pos, append, kept=None, want_mass=False,
                  hints=None, block_len=32):
    """One transformer layer for rows h [R, n, D] at positions pos [n].

    Keys: the cached prefix of each row (all of it, or the ``kept`` positions)
    followed by this call's own tokens, under the block-wise mask.  With
    ``append`` the new K/V are written to the cache (a clean pass, P2 "BDLM":
    earlier blocks are always seen clean); otherwise they only serve this call
    (a noisy denoising step).  ``want_mass`` returns the attention probability
    mass on each prefix key summed over heads and queries."""
    cfg = model.cfg
    R, n, D = h.shape
    H, d = cfg.n_heads, cfg.head_dim
    wqkv = model.dense("w_qkv", l)
    wo = model.dense("w_o", l)
    x = rmsnorm(h, model.dense("attn_norm", l), cfg.rms_eps)
    qkv = x @ wqkv.T
    q = qkv[..., : H * d].reshape(R, n, H, d)
    k = qkv[..., H * d: 2 * H * d].reshape(R, n, H, d)
    v = qkv[..., 2 * H * d:].reshape(R, n, H, d)
    q = np.stack([rope(q[r], pos, cfg.rope_base) for r in range(R)])
    k = np.stack([rope(k[r], pos, cfg.rope_base) for r in range(R)])
    P = cache.P
    attn = np.zeros((R, n, H * d))
    mass = np.zeros((R, P)) if want_mass else None
    total_mass = 0.0
    for r in range(R):
        ppos = np.arange(P) if kept is None else np.asarray(kept[r])
        kk = np.concatenate([cache.K[l][r, ppos], k[r]], axis=0)
        vv = np.concatenate([cache.V[l][r, ppos], v[r]], axis=0)
        kpos = np.concatenate([ppos, pos])
        o, p = attention(q[r], kk, vv, pos, kpos, block_len)
        attn[r] = o.reshape(n, H * d)
        if want_mass:
            mass[r][ppos] += p[:, :, : len(ppos)].sum(axis=(0, 1))
            total_mass += p.sum()
    h = h + attn @ wo.T
    if append:
        cache.K[l] = np.concatenate([cache.K[l], k], axis=1)
        cache.V[l] = np.concatenate([cache.V[l], v], axis=1)
    x = rmsnorm(h, model.dense("moe_norm", l), cfg.rms_eps)
    y, idx, gates, key, z = _moe(model, l, x.reshape(R * n, D), hints, l)
    h = h + y.reshape(R, n, D)
    return h, {"mass": mass, "total_mass": total_mass, "route_idx": idx,
               "gates": gates, "route_key": key, "route_z": z}


def forward(model, ids, cache, append, kept=None, want_mass=False, hints=None, block_len=32):
    """All layers over ids [R, n] placed at positions cache.P .. cache.P+n-1."""
    cfg = model.cfg
    R, n = ids.shape
    pos = cache.P + np.arange(n)
    h = model.embed(ids)
    info = {"mass": np.zeros((R, cache.P)) if want_mass else None, "total_mass": 0.0,
            "route_idx": [], "route_key": [], "route_z": [], "gates": []}
    P0 = cache.P
    for l in range(cfg.n_layers):
        cache.P = P0        # appended K/V of earlier layers do not move positions
        h, li = layer_forward(model, l, h, cache, pos, append, kept, want_mass, hints, block_len)
        if want_mass:
            info["mass"] += li["mass"]
            info["total_mass"] += li["total_mass"]
        info["route_idx"].append(li["route_idx"])
        info["route_key"].append(li["route_key"])
        info["route_z"].append(li["route_z"])
        info["gates"].append(li["gates"])
    cache.P = P0 + (n if append else 0)
    return h, info


def block_init(model, cache, clean_ids, block_len=32, gen=None, hints=None):
    """Append clean tokens (the prompt, or a just-finished block) to the cache:
    a forward pass over the committed ids under the block-wise mask (reading
    R2: a finished block's K/V come from its clean ids, never from its last
    noisy step).  The cache length stays a multiple of the block length
    (reading R1: blocks are aligned from position 0).  With ``gen`` asking for
    the key-norm + confidence retention score, the top-1 probability of every
    appended position (LM head over the generation's sub-vocabulary, as for
    the block's own positions) is kept for it.  ``hints``: alternative router
    decisions for these tokens (see Hints).  Returns the final hidden states
    of the appended tokens [R, n, D] (None when nothing is appended)."""
    clean_ids = np.asarray(clean_ids)
    if clean_ids.shape[1] % block_len:
        raise ValueError("clean token count must be a multiple of the block length")
    if clean_ids.shape[1] == 0:
        return None
    R, n = clean_ids.shape
    h, _ = forward(model, clean_ids, cache, append=True, hints=hints, block_len=block_len)
    conf = np.full((R, n), np.nan)
    if gen is not None and gen.retention_score == 1:
        lo, hi = gen.vocab_lo, (gen.vocab_hi or model.cfg.vocab)
        for r in range(R):
            conf[r] = confidence(head_logits(model, h[r], lo, hi), 0)[1]
    cache.ids = np.concatenate([cache.ids, clean_ids.astype(np.int32)], axis=1)
    cache.conf = np.concatenate([cache.conf, conf], axis=1)
    return h


def head_logits(model, h_rows, lo, hi):
    """Final RMSNorm then LM-head logits over the sub-vocabulary [lo, hi)
    (reading R9: the softmax/argmax run over the restricted columns)."""
    cfg = model.cfg
    x = rmsnorm(h_rows, model.dense("final_norm"), cfg.rms_eps)
    w = model.dense("lm_head")[lo:hi]
    return x @ w.T


@dataclass
class BlockState:
    """Per-block SPRINT state: the kept prefix positions of each row."""
    kept: list | None = None


def denoise_step(model, cache, gen, block_ids, t, bstate=None, hints=None):
    """One denoising step on the open block.

    block_ids: [n_seq, L_B] with [MASK] at undecided positions.  Rows of the
    model batch are the sequences, (cond, uncond) pairs with CFG, or (full,
    image-only, uncond) triples with three-way editing guidance; all rows of
    a sequence see the same block ids.  Returns (new_ids, remaining, info).

    Steps: embed -> L x [RMSNorm, QKV, RoPE, block attention over the
    (retained) prefix + this block, O-proj + residual, RMSNorm, sigmoid+bias
    top-k routing, experts + shared expert, residual] -> final norm -> LM head
    on masked positions over the sub-vocab -> CFG mix -> confidence -> commit
    the quota.  SPRINT: steps t < cache_warmup_steps attend to the whole prefix;
    the last warm-up step scores the prefix (accumulated attention mass of
    this step, or key norm + confidence) and selects the kept set used by
    later steps of this block."""
    cfg = model.cfg
    mask_id = cfg.mask_id
    LB = gen.block_length
    block_ids = np.asarray(block_ids, np.int32)
    n_seq = block_ids.shape[0]
    G = gen.group
    rows_ids = np.repeat(block_ids, G, axis=0)
    R = rows_ids.shape[0]
    bstate = bstate if bstate is not None else BlockState()
    # the model card: with three-way editing guidance SPRINT falls back to the
    # baseline (no prefix retention)
    sprint = gen.use_sprint and not gen.cfg3_on
    warm = (not sprint) or t < gen.cache_warmup_steps
    if not warm and bstate.kept is None:
        raise RuntimeError("retained steps need a warm-up step first")
    kept = None if warm else bstate.kept
    select_now = sprint and t == gen.cache_warmup_steps - 1
    want_mass = select_now and gen.retention_score == 0
    h, info = forward(model, rows_ids, cache, append=False, kept=kept,
                      want_mass=want_mass, hints=hints, block_len=LB)
    lo, hi = gen.vocab_lo, (gen.vocab_hi or cfg.vocab)
    new = block_ids.copy()
    remaining = np.zeros(n_seq, np.int32)
    out = {"logits": [], "xhat": [], "conf": [], "commit": [], "info": info, "h": h}
    for s in range(n_seq):
        pos_m = np.nonzero(block_ids[s] == mask_id)[0]
        xh = np.zeros(LB, np.int64)
        cf = np.full(LB, -np.inf)
        if len(pos_m):
            if gen.cfg3_on:
                lf = head_logits(model, h[3 * s, pos_m], lo, hi)
                li = head_logits(model, h[3 * s + 1, pos_m], lo, hi)
                lu = head_logits(model, h[3 * s + 2, pos_m], lo, hi)
                lg = cfg3_mix(lf, li, lu, gen.cfg_text_scale, gen.cfg_image_scale)
            elif gen.cfg_on:
                lc = head_logits(model, h[2 * s, pos_m], lo, hi)
                lu = head_logits(model, h[2 * s + 1, pos_m], lo, hi)
                lg = cfg_mix(lc, lu, gen.cfg_scale)
            else:
                lg = head_logits(model, h[s, pos_m], lo, hi)
            xi, ci = confidence(lg, gen.confidence)
            if hints is not None and hints.xhat is not None and hints.logits is not None:
                la = np.asarray(hints.logits[s], np.float64)
                for j, p in enumerate(pos_m):
                    a = int(hints.xhat[s, p]) - lo
                    if a == xi[j] or not 0 <= a < lg.shape[1]:
                        continue
                    slack = hints.logit_slack * float(np.max(np.abs(la[j])))
                    if la[j, a] < np.max(la[j]) - slack:
                        continue                           # not a maximum of its own logits
                    e = float(np.max(np.abs(la[j] - lg[j])))
                    gap = float(lg[j, xi[j]] - lg[j, a])
                    if gap <= 2 * e + slack:
                        xi[j] = a
                        hints.log.append(("argmax", s, int(p), gap, 2 * e + slack))
            xh[pos_m] = xi + lo
            cf[pos_m] = ci
            out["logits"].append(lg)
        else:
            out["logits"].append(np.zeros((0, hi - lo)))
        hint = hc = None
        if hints is not None and hints.commit is not None and hints.conf is not None:
            hint, hc = hints.commit[s], hints.conf[s]
        ns, sinfo = select_commit(block_ids[s], mask_id, xh, cf, gen.steps, t,
                                  gen.use_threshold, gen.threshold, hint, hc)
        if sinfo["adopted"]:
            hints.log.append(("commit", s, sinfo["gap"], sinfo["window"]))
        new[s] = ns
        remaining[s] = int(np.sum(ns == mask_id))
        out["xhat"].append(xh)
        out["conf"].append(cf)
        out["commit"].append(sinfo.get("chosen", np.zeros(0, int)))
    if select_now:
        kept_rows, scores = [], []
        ratios = pool_ratios_of(gen)
        for r in range(R):
            if gen.retention_score == 0:
                sc = info["mass"][r]
            else:
                sc = keynorm_conf_score(cache, r, gen.retention_alpha)
            pool = modality_pool(cache.ids[r, : cache.P], cfg) if ratios else np.zeros(len(sc), np.int64)
            ks = retention_select(sc, gen.keep_ratio, pool, ratios)
            if hints is not None and hints.kept is not None and hints.score is not None:
                alt = np.sort(np.asarray(hints.kept[r]))
                if not np.array_equal(alt, ks):
                    ok, gap, win = _alt_kept_valid(sc, np.asarray(hints.score[r], np.float64)[: len(sc)], alt,
                                                   pool, ratios, gen.keep_ratio)
                    if ok:
                        ks = alt
                        hints.log.append(("kept", r, gap, win))
            kept_rows.append(ks)
            scores.append(sc)
        bstate.kept = kept_rows
        out["retention_score"] = scores
    return new, remaining, out


def _alt_kept_valid(score, alt_score, alt, pool, ratios, keep_ratio):
    """Whether ``alt`` may replace the oracle's kept set (see Hints): it must be
    exactly the per-pool selection of retention_select under ``alt_score``,
    and in every pool the oracle's own scores may rank a dropped position
    above a kept one by at most 2 e, e = max |alt_score - score| over the row.
    Returns (valid, largest gap, window)."""
    alt = np.asarray(alt)
    if not np.array_equal(retention_select(alt_score, keep_ratio, pool, ratios), alt):
        return False, np.inf, 0.0
    e = float(np.max(np.abs(alt_score - score))) if len(score) else 0.0
    worst = -np.inf
    for p in (0, 1):
        in_p = np.nonzero(pool == p)[0]
        a = np.intersect1d(alt, in_p)
        rest = np.setdiff1d(in_p, a)
        if len(a) and len(rest):
            worst = max(worst, float(np.max(score[rest]) - np.min(score[a])))
    return worst <= 2 * e, worst, 2 * e


def generate_block(model, cache, gen, block_ids, hints_per_step=None):
    """Run denoising steps until no [MASK] remains or the step budget is spent
    (P2 SPRINT: block diffusion costs B x T forward passes; threshold mode can
    finish early).  Returns (ids, steps_taken, per-step outputs)."""
    ids = np.asarray(block_ids, np.int32).copy()
    bstate = BlockState()
    steps = []
    for t in range(gen.steps):
        hints = None if hints_per_step is None else hints_per_step(t, ids)
        ids, rem, out = denoise_step(model, cache, gen, ids, t, bstate, hints)
        steps.append(out)
        if int(np.sum(rem)) == 0:
            return ids, t + 1, steps
    return ids, gen.steps, steps
