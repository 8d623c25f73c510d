"""Pins for the oracle: each check fixes a result by something other than the
oracle's own formula (brute force, closed forms, special cases that reduce to
textbook routines, invariants).  CPU only."""
import math
import os

import numpy as np
import pytest

import dllm_inputs as di
from oracle import dllm_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def test_e4m3fn_spot_values():
    """Spot values of the OCP E4M3FN format, derived by hand (golden file)."""
    rows = []
    for line in open(os.path.join(GOLDEN, "e4m3fn_spot.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), float(val)))
    codes = np.array([c for c, _ in rows], np.uint8)
    got = O.e4m3fn_to_f64(codes)
    for (c, v), g in zip(rows, got):
        if math.isnan(v):
            assert math.isnan(g), hex(c)
        else:
            assert g == v and math.copysign(1, g) == math.copysign(1, v), hex(c)


def test_e4m3fn_exhaustive_structure():
    """All 256 codes: positive codes 0..126 strictly increasing, negatives mirror,
    only 0x7f/0xff are NaN, every value is exactly representable in bfloat16,
    and the input-side encoder (independent code) round-trips every value."""
    codes = np.arange(256, dtype=np.uint8)
    v = O.e4m3fn_to_f64(codes)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2
    pos = v[:127]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[128:255], -v[:127])
    # exactly representable in bf16: 3 mantissa bits, exponents within range
    f32 = v[:127].astype(np.float32)
    bf = di.f32_to_bf16_bits(f32)
    assert np.array_equal(O.bf16_to_f64(bf), v[:127])
    # encoder round trip (encoder lives in the input module, written separately)
    grid = np.concatenate([v[:127], -v[1:127]])
    enc = di._e4m3fn_encode(grid)
    assert np.array_equal(O.e4m3fn_to_f64(enc), grid)


def test_e4m3fn_row_quantization_error_bound():
    """Quantize -> decode error is at most half a grid step times the row scale,
    and the row maximum maps to +-448 (saturation point)."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 200)) * 0.02).astype(np.float32)
    codes, scale = di.quantize_rows_e4m3fn(w)
    deq = O.e4m3fn_to_f64(codes) * scale[:, None].astype(np.float64)
    x = w.astype(np.float64) / scale[:, None]
    a = np.abs(x)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -10))
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    assert np.all(np.abs(deq - w) <= 0.5 * step * scale[:, None] * (1 + 1e-12))
    assert np.all(np.max(np.abs(O.e4m3fn_to_f64(codes)), axis=1) == 448.0)


def test_bf16_decode_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-30, 65280.0], np.float32)
    bits = di.f32_to_bf16_bits(x)
    assert np.array_equal(O.bf16_to_f64(bits), np.array([1.0, -2.5, 3.140625,
                                                         O.bf16_to_f64(bits)[3], 65280.0]))
    # round-to-nearest-even at a tie: 1 + 2^-8 is halfway between bf16 1 and 1+2^-7
    t = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)
    assert np.array_equal(O.bf16_to_f64(di.f32_to_bf16_bits(t)), [1.0, 1.0 + 2.0 ** -6])


# ----------------------------------------------------------------------------
# norm, rope, attention
# ----------------------------------------------------------------------------

def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    y = O.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0)
    assert np.allclose(O.rmsnorm(7.5 * x, np.ones(64), 0.0), y)


def test_rope_properties():
    rng = np.random.default_rng(1)
    n, H, d = 6, 3, 16
    q = rng.standard_normal((n, H, d))
    k = rng.standard_normal((n, H, d))
    pos = np.array([0, 1, 5, 9, 100, 1000])
    rq = O.rope(q, pos, 10000.0)
    # identity at position 0, norms preserved
    assert np.allclose(rq[0], q[0])
    assert np.allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1))
    # q.k depends only on the position difference
    a = np.einsum("hd,hd->h", O.rope(q[1:2], [7], 1e4)[0], O.rope(k[2:3], [3], 1e4)[0])
    b = np.einsum("hd,hd->h", O.rope(q[1:2], [507], 1e4)[0], O.rope(k[2:3], [503], 1e4)[0])
    assert np.allclose(a, b)
    # pair (i, i+d/2) is a 2-D rotation by pos * base^(-2i/d): check via complex numbers
    i = 3
    z = (q[4, 0, i] + 1j * q[4, 0, i + d // 2]) * np.exp(1j * 100 * 10000.0 ** (-2 * i / d))
    assert np.isclose(rq[4, 0, i], z.real) and np.isclose(rq[4, 0, i + d // 2], z.imag)


def _brute_attention(q, k, v, qpos, kpos, bl):
    """Scalar loops: scores, mask by block index, softmax, weighted sum."""
    nq, H, d = q.shape
    nk = k.shape[0]
    out = np.zeros((nq, H, d))
    for h in range(H):
        for i in range(nq):
            sc = []
            for j in range(nk):
                if kpos[j] // bl <= qpos[i] // bl:
                    sc.append((j, sum(q[i, h, t] * k[j, h, t] for t in range(d)) / math.sqrt(d)))
            mx = max(s for _, s in sc)
            ws = [(j, math.exp(s - mx)) for j, s in sc]
            z = sum(w for _, w in ws)
            for j, w in ws:
                out[i, h] += (w / z) * v[j, h]
    return out


@pytest.mark.parametrize("bl", [1, 3, 4, 64])
def test_attention_brute_force(bl):
    rng = np.random.default_rng(bl)
    nq, nk, H, d = 5, 12, 2, 4
    q = rng.standard_normal((nq, H, d))
    k = rng.standard_normal((nk, H, d))
    v = rng.standard_normal((nk, H, d))
    kpos = np.arange(nk)
    qpos = np.arange(nk - nq, nk)        # the last nq tokens query everything
    o, p = O.attention(q, k, v, qpos, kpos, bl)
    assert np.allclose(o, _brute_attention(q, k, v, qpos, kpos, bl))
    assert np.allclose(p.sum(-1), 1.0)


def test_attention_block1_is_causal_and_full_block_is_bidirectional():
    rng = np.random.default_rng(7)
    n, H, d = 9, 2, 8
    q, k, v = (rng.standard_normal((n, H, d)) for _ in range(3))
    pos = np.arange(n)

    def textbook(mask):
        s = np.einsum("qhd,khd->hqk", q, k) / math.sqrt(d)
        s = np.where(mask[None], s, -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        return np.einsum("hqk,khd->qhd", p, v)

    causal = np.tril(np.ones((n, n), bool))
    assert np.allclose(O.attention(q, k, v, pos, pos, 1)[0], textbook(causal))
    full = np.ones((n, n), bool)
    assert np.allclose(O.attention(q, k, v, pos, pos, n)[0], textbook(full))


# ----------------------------------------------------------------------------
# router, MoE
# ----------------------------------------------------------------------------

def test_topk_matches_full_sort_with_ties():
    rng = np.random.default_rng(2)
    for _ in range(50):
        key = rng.integers(0, 6, size=32).astype(np.float32)   # many exact ties
        k = int(rng.integers(1, 9))
        got = O.topk_desc(key, k)
        ref = sorted(range(32), key=lambda i: (-float(key[i]), i))[:k]
        assert list(got) == ref


def test_router_planted_bias_and_all_experts():
    rng = np.random.default_rng(4)
    n, D, E, k = 10, 16, 8, 3
    x = rng.standard_normal((n, D))
    wr = rng.standard_normal((E, D)) * 0.02
    b = np.zeros(E, np.float32)
    b[5] = 10.0
    _, s, key = O.route_keys(x, wr, b)
    for i in range(n):
        assert 5 in O.topk_desc(key[i], k)
        sel = O.topk_desc(key[i], E)
        assert sorted(sel) == list(range(E))
        g = O.gates_from(s[i], O.topk_desc(key[i], k))
        assert np.isclose(g.sum(), 1.0)
    # selection uses s + b but gates use the unbiased s
    sel = O.topk_desc(key[0], k)
    assert np.allclose(O.gates_from(s[0], sel), s[0][sel] / s[0][sel].sum())


def test_swiglu_hand_expanded():
    rng = np.random.default_rng(5)
    D, F = 6, 4
    x = rng.standard_normal((1, D))
    wg, wu = rng.standard_normal((F, D)), rng.standard_normal((F, D))
    wd = rng.standard_normal((D, F))
    hmid = []
    for f in range(F):
        a = sum(wg[f, i] * x[0, i] for i in range(D))
        b = sum(wu[f, i] * x[0, i] for i in range(D))
        hmid.append(a / (1 + math.exp(-a)) * b)
    y = [sum(wd[o, f] * hmid[f] for f in range(F)) for o in range(D)]
    assert np.allclose(O.swiglu(x, wg, wu, wd)[0], y)


def _tiny_model(expert_dtype="f32", act="f32", layers=1, E=4, k=2, seed=0, shared=1):
    m = di.ModelConfig(n_layers=layers, hidden=8, n_heads=2, head_dim=4, n_experts=E,
                       top_k=k, n_shared=shared, expert_ffn=4, shared_ffn=4,
                       vocab_text=20, vocab_image=6, act_dtype=act, expert_dtype=expert_dtype)
    return m, di.make_weights(m, seed)


def test_identical_experts_reproduce_dense_ffn():
    m, w = _tiny_model(E=6, k=3, shared=0)
    for name in ("w_gate", "w_up", "w_down"):
        w[name][:, :] = w[name][:, :1]          # every expert equals expert 0
    model = O.Model(m, w)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((7, m.hidden))
    y, idx, gates, _, _ = O._moe(model, 0, x)
    dense = O.swiglu(x, model.expert("w_gate", 0, 0), model.expert("w_up", 0, 0),
                     model.expert("w_down", 0, 0))
    assert np.allclose(y, dense)
    assert np.bincount(idx.ravel(), minlength=6).sum() == 7 * 3


def _scalar_layer(model, l, h, ck, cv, P, pos, bl):
    """A whole layer in plain Python loops over scalars (no matmul, no einsum):
    norm, q/k/v projections, rotary pairs, masked softmax attention, output
    projection, norm, sigmoid router with float32 keys, top-k, SwiGLU experts,
    shared expert.  Independent brute force for ``layer_forward``."""
    cfg = model.cfg
    D, H, d, E = cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.n_experts
    n = len(h)
    W = model.dense("w_qkv", l)
    Wo = model.dense("w_o", l)

    def norm(row):
        r = math.sqrt(sum(a * a for a in row) / len(row) + cfg.rms_eps)
        return [a / r for a in row]

    def rot(vec, p):
        half = d // 2
        out = list(vec)
        for i in range(half):
            ang = p * cfg.rope_base ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            out[i] = vec[i] * c - vec[i + half] * s
            out[i + half] = vec[i + half] * c + vec[i] * s
        return out

    qs, ks, vs = [], [], []
    for t in range(n):
        x = norm(h[t])
        proj = [sum(W[o, i] * x[i] for i in range(D)) for o in range(3 * H * d)]
        qs.append([rot(proj[hh * d:(hh + 1) * d], pos[t]) for hh in range(H)])
        ks.append([rot(proj[H * d + hh * d: H * d + (hh + 1) * d], pos[t]) for hh in range(H)])
        vs.append([proj[2 * H * d + hh * d: 2 * H * d + (hh + 1) * d] for hh in range(H)])
    out = []
    for t in range(n):
        att = []
        for hh in range(H):
            keys = [(j, list(ck[j, hh]), list(cv[j, hh])) for j in range(P)]
            keys += [(pos[u], ks[u][hh], vs[u][hh]) for u in range(n)]
            sc = [(kv, sum(a * b for a, b in zip(qs[t][hh], kk)) / math.sqrt(d))
                  for (kp, kk, kv) in keys if kp // bl <= pos[t] // bl]
            mx = max(s for _, s in sc)
            z = sum(math.exp(s - mx) for _, s in sc)
            acc = [0.0] * d
            for kv, s in sc:
                for i in range(d):
                    acc[i] += math.exp(s - mx) / z * kv[i]
            att += acc
        h1 = [h[t][o] + sum(Wo[o, i] * att[i] for i in range(H * d)) for o in range(D)]
        x = norm(h1)
        wr = model.dense("w_router", l)
        b = model.w["router_bias"][l]
        s = [np.float32(1.0 / (1.0 + math.exp(-sum(wr[e, i] * x[i] for i in range(D)))))
             for e in range(E)]
        key = [np.float32(s[e] + np.float32(b[e])) for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-float(key[e]), e))[: cfg.top_k]
        gs = sum(float(s[e]) for e in sel)
        y = [0.0] * D

        def ffn(wg, wu, wd, g):
            F = wg.shape[0]
            hm = []
            for f in range(F):
                a = sum(wg[f, i] * x[i] for i in range(D))
                c = sum(wu[f, i] * x[i] for i in range(D))
                hm.append(a / (1 + math.exp(-a)) * c)
            for o in range(D):
                y[o] += g * sum(wd[o, f] * hm[f] for f in range(F))

        for e in sel:
            ffn(model.expert("w_gate", l, e), model.expert("w_up", l, e),
                model.expert("w_down", l, e), float(s[e]) / gs)
        if cfg.n_shared:
            ffn(model.dense("ws_gate", l), model.dense("ws_up", l), model.dense("ws_down", l), 1.0)
        out.append([h1[o] + y[o] for o in range(D)])
    return np.array(out)


@pytest.mark.parametrize("edt", ["f32", "bf16", "fp8"])
def test_layer_matches_scalar_brute_force(edt):
    m, w = _tiny_model(expert_dtype=edt, act="f32" if edt == "f32" else "bf16", E=5, k=2)
    model = O.Model(m, w)
    bl = 4
    rng = np.random.default_rng(11)
    P, n = 8, 4
    cache = O.Cache.empty(m, 1)
    O.block_init(model, cache, rng.integers(0, m.vocab, size=(1, P)), block_len=bl)
    h = model.embed(rng.integers(0, m.vocab + 1, size=(1, n)))
    pos = np.arange(P, P + n)
    got, _ = O.layer_forward(model, 0, h, cache, pos, append=False, block_len=bl)
    ref = _scalar_layer(model, 0, h[0], cache.K[0][0], cache.V[0][0], P, pos, bl)
    assert np.allclose(got[0], ref, rtol=1e-10, atol=1e-12)


def test_prefill_layer_matches_scalar_brute_force():
    """Multi-block clean pass: the new tokens span blocks and see each other
    block-causally."""
    m, w = _tiny_model(E=4, k=2)
    model = O.Model(m, w)
    bl = 3
    rng = np.random.default_rng(12)
    cache = O.Cache.empty(m, 1)
    ids = rng.integers(0, m.vocab, size=(1, 9))
    h = model.embed(ids)
    got, _ = O.layer_forward(model, 0, h, cache, np.arange(9), append=True, block_len=bl)
    ref = _scalar_layer(model, 0, h[0], np.zeros((0, 2, 4)), np.zeros((0, 2, 4)), 0,
                        np.arange(9), bl)
    assert np.allclose(got[0], ref, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# cache equivalence, retention
# ----------------------------------------------------------------------------

def _small_wl(**kw):
    wl = di.workload("tiny_fp32")
    wl.model.n_layers = 2
    wl.model.hidden = 32
    wl.model.n_heads = 2
    wl.model.head_dim = 16
    wl.model.n_experts = 6
    wl.model.top_k = 2
    wl.model.expert_ffn = 16
    wl.model.shared_ffn = 16
    wl.model.vocab_text = 50
    wl.gen.block_length = 8
    wl.gen.steps = 4
    wl.prefix_len = 16
    for k, v in kw.items():
        setattr(wl.gen, k, v)
    return wl


def test_cached_step_equals_uncached_forward():
    """A denoising step over the cached prefix equals one uncached forward over
    [prefix; block] (the block's rows), and chunked prefill equals one-shot."""
    wl = _small_wl()
    m = wl.model
    model = O.Model(m, di.make_weights(m, 1))
    prefix = di.make_prefix(wl, 1)
    block = np.full((1, 8), m.mask_id, np.int32)
    block[0, [1, 4]] = [3, 7]
    c1 = O.Cache.empty(m, 1)
    O.block_init(model, c1, prefix, 8)
    h_step, _ = O.forward(model, block, c1, append=False, block_len=8)
    c0 = O.Cache.empty(m, 1)
    h_full, _ = O.forward(model, np.concatenate([prefix, block], 1), c0, append=False, block_len=8)
    assert np.allclose(h_step[0], h_full[0, 16:], atol=1e-12)
    c2 = O.Cache.empty(m, 1)
    O.block_init(model, c2, prefix[:, :8], 8)
    O.block_init(model, c2, prefix[:, 8:], 8)
    for l in range(m.n_layers):
        assert np.allclose(c2.K[l], c1.K[l], atol=1e-12)
        assert np.allclose(c2.V[l], c1.V[l], atol=1e-12)


def test_retention_invariants():
    wl = _small_wl(use_sprint=True, keep_ratio=0.5)
    m, g = wl.model, wl.gen
    model = O.Model(m, di.make_weights(m, 2))
    cache = O.Cache.empty(m, 1)
    O.block_init(model, cache, di.make_prefix(wl, 2), 8)
    block = np.full((1, 8), m.mask_id, np.int32)
    bs = O.BlockState()
    _, _, out = O.denoise_step(model, cache, g, block, 0, bs)
    info = out["info"]
    # probability mass over all keys = layers * heads * block queries
    assert np.isclose(info["total_mass"], m.n_layers * m.n_heads * 8)
    mass = info["mass"][0]
    assert np.all(mass > 0) and mass.sum() < m.n_layers * m.n_heads * 8
    kept = bs.kept[0]
    assert len(kept) == math.ceil(0.5 * 16)
    ref = sorted(range(16), key=lambda i: (-mass[i], i))[:8]
    assert list(kept) == sorted(ref)
    # keep ratio 1: identical to full retention at every later step
    g1 = di.clone(wl).gen
    g1.keep_ratio = 1.0
    bsa = O.BlockState()
    ids_a, _, _ = O.denoise_step(model, cache, g1, block, 0, bsa)
    ids_b, _, oa = O.denoise_step(model, cache, g1, ids_a, 1, bsa)
    g0 = di.clone(wl).gen
    g0.use_sprint = False
    ids_c, _, oc = O.denoise_step(model, cache, g0, ids_a, 1)
    assert np.array_equal(ids_b, ids_c)
    assert np.array_equal(oa["logits"][0], oc["logits"][0])


def _sprint_kc_wl(**kw):
    """Small model with a visual sub-vocabulary: 16-token prefix, the first 8
    ids visual, key norm + confidence score, image pool 0.8, text pool 1.0."""
    wl = _small_wl(use_sprint=True, keep_ratio=0.5, retention_score=1, retention_alpha=0.5,
                   image_keep_ratio=0.8, text_keep_ratio=1.0, vocab_lo=0, vocab_hi=50)
    wl.model.vocab_image = 30
    wl.prefix_visual = 8
    for k, v in kw.items():
        setattr(wl.gen, k, v)
    return wl


def test_keynorm_conf_score_closed_form():
    """With V and the expert down projections zeroed, every layer adds nothing
    to the residual, so each prefix hidden state stays its embedding row.  The
    key norm of position i is then, per layer and head, |W_k rms(e_i)| (RoPE
    rotates pairs and keeps norms, so it is left out here), and its top-1
    probability is max softmax(rms(e_i) . head) over the sub-vocabulary; both
    computed here directly from the weights, without the layer stack."""
    wl = _sprint_kc_wl()
    m, g = wl.model, wl.gen
    w = di.make_weights(m, 7)
    H, d = m.n_heads, m.head_dim
    w["w_qkv"][:, : H * d] = 0.0            # queries
    w["w_qkv"][:, 2 * H * d:] = 0.0         # values
    w["w_down"][:] = 0.0
    w["ws_down"][:] = 0.0
    model = O.Model(m, w)
    # distinct ids: equal ids would tie exactly in the direct computation but
    # differ by rounding after RoPE at different positions
    rng = np.random.default_rng(7)
    prefix = np.concatenate([rng.permutation(np.arange(50, 80))[:8],
                             rng.permutation(50)[:8]]).astype(np.int32)[None]
    cache = O.Cache.empty(m, 1)
    O.block_init(model, cache, prefix, 8, g)
    e = w["embed"][prefix[0]].astype(np.float64)
    x = e / np.sqrt(np.mean(e * e, axis=1, keepdims=True) + m.rms_eps)
    norms = []
    for l in range(m.n_layers):
        wk = w["w_qkv"][l, H * d: 2 * H * d].astype(np.float64).reshape(H, d, m.hidden)
        for hh in range(H):
            kv = x @ wk[hh].T
            norms.append(np.sqrt(np.sum(kv * kv, axis=1)))
    l_ref = np.mean(norms, axis=0)
    assert np.allclose(O.key_norms(cache, 0), l_ref, rtol=1e-12)
    logits = x @ w["lm_head"][g.vocab_lo: g.vocab_hi].astype(np.float64).T
    c_ref = np.array([1.0 / np.sum(np.exp(r - r.max())) for r in logits])
    assert np.allclose(cache.conf[0], c_ref, rtol=1e-12)
    s = O.keynorm_conf_score(cache, 0, 0.5)
    assert np.isclose(np.mean(s - 0.5 * c_ref), 0.5)       # the key-norm term has mean alpha
    # alpha = 1 ranks by key norm alone, alpha = 0 by confidence alone
    for alpha, key in ((1.0, l_ref), (0.0, c_ref)):
        got = O.retention_select(O.keynorm_conf_score(cache, 0, alpha), 0.5)
        assert list(got) == sorted(sorted(range(16), key=lambda i: (-key[i], i))[:8])


def test_keynorm_score_scale_invariance_and_prefix_chunking():
    """Scaling every cached key by a constant leaves the mean-normalized score
    unchanged; the prefix confidences do not depend on how the prefix was
    appended (the block-wise mask hides later blocks); without the score they
    are not computed."""
    wl = _sprint_kc_wl()
    m, g = wl.model, wl.gen
    model = O.Model(m, di.make_weights(m, 8))
    prefix = di.make_prefix(wl, 8)
    c1 = O.Cache.empty(m, 1)
    O.block_init(model, c1, prefix, 8, g)
    c2 = O.Cache.empty(m, 1)
    O.block_init(model, c2, prefix[:, :8], 8, g)
    O.block_init(model, c2, prefix[:, 8:], 8, g)
    assert np.allclose(c1.conf, c2.conf, rtol=1e-12)
    assert np.array_equal(c1.ids, prefix) and np.array_equal(c2.ids, prefix)
    s1 = O.keynorm_conf_score(c1, 0, 0.5)
    c1.K = [3.7 * K for K in c1.K]
    assert np.allclose(O.keynorm_conf_score(c1, 0, 0.5), s1, rtol=1e-12)
    c3 = O.Cache.empty(m, 1)
    O.block_init(model, c3, prefix, 8)
    assert np.all(np.isnan(c3.conf))


def _ceil_ratio(r, n):
    from fractions import Fraction
    return math.ceil(Fraction(str(r)) * n)


def test_retention_pools_brute_force():
    """Per-modality pools: each pool keeps its own top ceil(r_p P_p) (ties to
    the lower position), checked against a per-pool sort; a pool whose scores
    are all below the other pool's still keeps its share; both ratios 1 keep
    everything; one pool reproduces the single-pool selection."""
    rng = np.random.default_rng(21)
    for P in (7, 64, 301):
        score = np.round(rng.random(P) * 20) / 4          # many exact ties
        pool = (rng.random(P) < 0.6).astype(np.int64)
        for rt, ri in ((1.0, 0.8), (0.5, 0.5), (0.3, 1.0), (1.0, 1.0)):
            got = O.retention_select(score, 0.9, pool, (rt, ri))
            ref = []
            for p, r in ((0, rt), (1, ri)):
                where = [i for i in range(P) if pool[i] == p]
                ref += sorted(where, key=lambda i: (-score[i], i))[: _ceil_ratio(r, len(where))]
            assert list(got) == sorted(ref), (P, rt, ri)
        assert len(O.retention_select(score, 0.5, pool, (1.0, 1.0))) == P
        assert np.array_equal(O.retention_select(score, 0.4, np.zeros(P, np.int64), (0.4, 0.4)),
                              O.retention_select(score, 0.4))
    score = np.concatenate([np.full(10, 5.0), np.arange(10) * 0.1])
    pool = np.array([0] * 10 + [1] * 10)
    got = O.retention_select(score, 0.5, pool, (0.5, 0.5))
    assert list(got) == [0, 1, 2, 3, 4, 15, 16, 17, 18, 19]


def test_modality_pool_and_ratios():
    m = _sprint_kc_wl().model
    ids = np.array([0, 49, 50, 79, 80, -1])
    assert list(O.modality_pool(ids, m)) == [0, 0, 1, 1, 0, 0]   # [MASK] = 80 counts as text
    g = di.GenParams(keep_ratio=0.5)
    assert O.pool_ratios_of(g) is None
    g.image_keep_ratio = 0.8
    assert O.pool_ratios_of(g) == (0.5, 0.8)


def test_sprint_keynorm_step_pools():
    """A SPRINT step with the key-norm + confidence score: the text pool (ratio
    1) is kept whole, the image pool keeps ceil(0.8 * 8) = 7 of its 8
    positions, and ratios of 1 for both pools make later steps identical to
    full retention."""
    wl = _sprint_kc_wl()
    m, g = wl.model, wl.gen
    model = O.Model(m, di.make_weights(m, 9))
    prefix = di.make_prefix(wl, 9)
    assert np.all(prefix[0, :8] >= 50) and np.all(prefix[0, 8:] < 50)
    cache = O.Cache.empty(m, 1)
    O.block_init(model, cache, prefix, 8, g)
    block = np.full((1, 8), m.mask_id, np.int32)
    bs = O.BlockState()
    ids1, _, out = O.denoise_step(model, cache, g, block, 0, bs)
    kept = bs.kept[0]
    sc = out["retention_score"][0]
    assert len(kept) == 7 + 8 and set(range(8, 16)) <= set(kept)
    dropped = sorted(set(range(8)) - set(kept))
    assert len(dropped) == 1 and sc[dropped[0]] == min(sc[:8])
    assert out["info"]["mass"] is None                 # no attention mass needed
    g1 = di.clone(wl).gen
    g1.image_keep_ratio = 1.0
    bsa = O.BlockState()
    ids_a, _, _ = O.denoise_step(model, cache, g1, block, 0, bsa)
    ids_b, _, oa = O.denoise_step(model, cache, g1, ids_a, 1, bsa)
    g0 = di.clone(wl).gen
    g0.use_sprint = False
    ids_c, _, oc = O.denoise_step(model, cache, g0, ids_a, 1)
    assert np.array_equal(ids_b, ids_c)
    assert np.array_equal(oa["logits"][0], oc["logits"][0])


def test_retention_ties_and_count():
    mass = np.array([0.5, 0.2, 0.5, 0.1, 0.2, 0.2, 0.9])
    kept = O.retention_select(mass, 0.5)
    assert list(kept) == [0, 1, 2, 6]           # ceil(3.5)=4: 0.9,0.5,0.5, then 0.2 at pos 1
    assert len(O.retention_select(mass, 1.0)) == 7
    assert O.n_keep(0.8, 95) == 76 and O.n_keep(0.5, 4160) == 2080 and O.n_keep(0.3, 10) == 3


# ----------------------------------------------------------------------------
# head, CFG, confidence, schedule
# ----------------------------------------------------------------------------

def test_cfg_endpoints():
    rng = np.random.default_rng(6)
    lc, lu = rng.standard_normal((3, 10)), rng.standard_normal((3, 10))
    assert np.allclose(O.cfg_mix(lc, lu, 1.0), lc, rtol=0, atol=1e-15)
    assert np.array_equal(O.cfg_mix(lc, lu, 0.0), lu)
    assert np.allclose(O.cfg_mix(lc, lu, 2.0), 2 * lc - lu)


def test_confidence_closed_forms():
    V = 64
    l = np.zeros((1, V))
    x, c = O.confidence(l, 0)
    assert x[0] == 0 and np.isclose(c[0], 1.0 / V)
    assert np.isclose(O.confidence(l, 1)[1][0], 0.0)
    assert np.isclose(O.confidence(l, 2)[1][0], -math.log(V))
    l2 = np.full((1, V), -1e9)
    l2[0, 17] = 0.0
    l2[0, 40] = 0.0                               # exact tie: lower id wins
    x, c = O.confidence(l2, 0)
    assert x[0] == 17 and np.isclose(c[0], 0.5)
    rng = np.random.default_rng(8)
    l3 = rng.standard_normal((5, 100)) * 3
    p = np.exp(l3) / np.exp(l3).sum(1, keepdims=True)
    assert np.allclose(O.confidence(l3, 0)[1], p.max(1))
    ps = np.sort(p, 1)
    assert np.allclose(O.confidence(l3, 1)[1], ps[:, -1] - ps[:, -2])
    assert np.array_equal(O.confidence(l3, 0)[0], np.argmax(l3, 1))


def test_schedule_linear_32_in_8():
    mask = 99
    rng = np.random.default_rng(10)
    ids = np.full(32, mask)
    prev = ids.copy()
    for t in range(8):
        assert O.quota(int(np.sum(ids == mask)), 8, t) == 4
        xh = rng.integers(0, 50, size=32)
        cf = rng.random(32)
        ids, info = O.select_commit(ids, mask, xh, cf, 8, t, False, 0.9)
        assert info["n"] == 4
        keep = prev != mask
        assert np.array_equal(ids[keep], prev[keep])      # committed ids never change
        prev = ids.copy()
    assert not np.any(ids == mask)


def test_schedule_front_loads_remainder_and_threshold():
    assert [O.quota(r, 4, t) for r, t in ((10, 0), (7, 1), (4, 2), (2, 3))] == [3, 3, 2, 2]
    mask = 99
    ids = np.full(32, mask)
    cf = np.full(32, 0.1)
    cf[[3, 9, 20, 21, 30]] = 0.97                    # planted peaks above tau
    xh = np.arange(32)
    out, info = O.select_commit(ids, mask, xh, cf, 32, 0, True, 0.93)
    assert info["n"] == 5 and set(np.nonzero(out != mask)[0]) == {3, 9, 20, 21, 30}
    out, info = O.select_commit(ids, mask, xh, cf, 4, 0, True, 0.93)
    assert info["n"] == 8                            # quota ceil(32/4)=8 > 5 peaks
    # ties in confidence go to the lower position
    out, info = O.select_commit(ids, mask, xh, np.zeros(32), 8, 0, False, 0.9)
    assert list(np.nonzero(out != mask)[0]) == [0, 1, 2, 3]


def test_generate_block_end_to_end_tiny():
    """Free-running block generation: every step commits the schedule's count,
    ids land in the sub-vocabulary, no [MASK] remains."""
    wl = _small_wl()
    m, g = wl.model, wl.gen
    g.vocab_lo, g.vocab_hi = 10, 40
    model = O.Model(m, di.make_weights(m, 3))
    cache = O.Cache.empty(m, 1)
    O.block_init(model, cache, di.make_prefix(wl, 3), 8)
    ids, steps, outs = O.generate_block(model, cache, g, np.full((1, 8), m.mask_id, np.int32))
    assert steps == 4
    assert [len(o["commit"][0]) for o in outs] == [2, 2, 2, 2]
    assert np.all((ids >= 10) & (ids < 40))


def test_cfg3_mix_endpoints():
    """Three-way guidance: both scales 1 give the full-condition logits, both 0
    the unconditional ones, and an image-only prediction equal to the
    unconditional one reduces it to two-way CFG with w = text scale."""
    rng = np.random.default_rng(31)
    lf, li, lu = (rng.standard_normal((3, 50)) for _ in range(3))
    assert np.allclose(O.cfg3_mix(lf, li, lu, 1.0, 1.0), lf, rtol=0, atol=1e-14)
    assert np.array_equal(O.cfg3_mix(lf, li, lu, 0.0, 0.0), lu)
    assert np.array_equal(O.cfg3_mix(lf, lu, lu, 4.0, 1.5), O.cfg_mix(lf, lu, 4.0))
    # the image scale alone moves along (l_img - l_u): s_txt = 0
    assert np.allclose(O.cfg3_mix(lf, li, lu, 0.0, 2.0), lu + 2.0 * (li - lu), atol=1e-14)


def test_cfg3_step_without_image_is_two_way_cfg():
    """A prompt with no visual part makes the image-only row identical to the
    unconditional row (both all [MASK]), so a three-way step equals a two-way
    CFG step with cfg_scale = text scale: same ids, same mixed logits."""
    wl = _small_wl(cfg_text_scale=4.0, cfg_image_scale=1.5)
    m, g = wl.model, wl.gen
    model = O.Model(m, di.make_weights(m, 11))
    prefix3 = di.make_prefix(wl, 11)
    assert prefix3.shape[0] == 3 and np.array_equal(prefix3[1], prefix3[2])
    assert np.all(prefix3[2] == m.mask_id)
    c3 = O.Cache.empty(m, 3)
    O.block_init(model, c3, prefix3, 8)
    wl2 = _small_wl(cfg_scale=4.0)
    prefix2 = di.make_prefix(wl2, 11)
    assert np.array_equal(prefix2[0], prefix3[0])
    c2 = O.Cache.empty(m, 2)
    O.block_init(model, c2, prefix2, 8)
    block = np.full((1, 8), m.mask_id, np.int32)
    ids3, rem3, o3 = O.denoise_step(model, c3, g, block, 0)
    ids2, rem2, o2 = O.denoise_step(model, c2, wl2.gen, block, 0)
    assert np.array_equal(ids3, ids2) and np.array_equal(rem3, rem2)
    assert np.array_equal(o3["logits"][0], o2["logits"][0])


def test_cfg3_prompt_rows_and_sprint_fallback():
    """Rows per sequence: (full prompt, visual part only, all [MASK]).  With
    three-way guidance SPRINT falls back to the baseline: no kept set, later
    steps attend to the whole prefix."""
    wl = _sprint_kc_wl(cfg_text_scale=4.0, cfg_image_scale=1.5)
    m, g = wl.model, wl.gen
    p = di.make_prefix(wl, 12)
    assert p.shape == (3, 16)
    assert np.all(p[0, :8] >= 50) and np.all(p[0, 8:] < 50)
    assert np.array_equal(p[1, :8], p[0, :8]) and np.all(p[1, 8:] == m.mask_id)
    assert np.all(p[2] == m.mask_id)
    model = O.Model(m, di.make_weights(m, 12))
    cache = O.Cache.empty(m, 3)
    O.block_init(model, cache, p, 8, g)
    block = np.full((1, 8), m.mask_id, np.int32)
    bs = O.BlockState()
    ids1, _, out = O.denoise_step(model, cache, g, block, 0, bs)
    assert bs.kept is None and "retention_score" not in out
    ids2, _, o2 = O.denoise_step(model, cache, g, ids1, 1, bs)
    g0 = di.clone(wl).gen
    g0.use_sprint = False
    ids2b, _, o2b = O.denoise_step(model, cache, g0, ids1, 1)
    assert np.array_equal(ids2, ids2b)
    assert np.array_equal(o2["logits"][0], o2b["logits"][0])


def test_cfg_rows_share_block_and_mix():
    wl = _small_wl(cfg_scale=2.0)
    m, g = wl.model, wl.gen
    model = O.Model(m, di.make_weights(m, 4))
    prefix = di.make_prefix(wl, 4)
    assert prefix.shape[0] == 2 and np.all(prefix[1] == m.mask_id)
    cache = O.Cache.empty(m, 2)
    O.block_init(model, cache, prefix, 8)
    block = np.full((1, 8), m.mask_id, np.int32)
    _, _, out = O.denoise_step(model, cache, g, block, 0)
    h, _ = O.forward(model, np.repeat(block, 2, 0), cache, append=False, block_len=8)
    lc = O.head_logits(model, h[0], 0, m.vocab)
    lu = O.head_logits(model, h[1], 0, m.vocab)
    assert np.allclose(out["logits"][0], lu + 2.0 * (lc - lu))
