"""Pins for the oracle's near-tie rule (Hints): an alternative decision is
taken only when it is exactly what its own keys select, the log records it,
and the windows follow from the key differences.  Also the per-key attention
mass against scalar loops.  CPU only."""
import math

import numpy as np

import dllm_inputs as di
from oracle import dllm_oracle as O


def _model(E=6, k=2, D=8):
    m = di.ModelConfig(n_layers=1, hidden=D, n_heads=2, head_dim=4, n_experts=E, top_k=k,
                       n_shared=0, expert_ffn=4, shared_ffn=4, vocab_text=20, vocab_image=0,
                       act_dtype="f32", expert_dtype="f32")
    return m, O.Model(m, di.make_weights(m, 3))


def _route_inputs(model, n=5, seed=1):
    x = np.random.default_rng(seed).standard_normal((n, model.cfg.hidden))
    z = x @ model.dense("w_router", 0).T
    return x, z


def test_route_hint_inconsistent_with_its_keys_is_rejected():
    """Alternative experts that its own logits do not select (here: the
    oracle's own logits, with the k-th and (k+1)-th experts swapped) are not
    adopted, however close the keys."""
    m, model = _model()
    x, z = _route_inputs(model)
    _, idx, _, key, _ = O._moe(model, 0, x)
    alt = idx.copy()
    order = [O.topk_desc(key[i], m.n_experts) for i in range(len(x))]
    for i in range(len(x)):
        alt[i, -1] = order[i][m.top_k]            # the first expert left out
    h = O.Hints(routing={0: alt}, router_z={0: z.astype(np.float32)})
    _, idx2, _, _, _ = O._moe(model, 0, x, h, 0)
    assert np.array_equal(idx2, idx) and not h.log


def test_route_hint_inconsistent_is_rejected_in_a_wide_window():
    """The same inconsistent alternative with logits far from the oracle's (a
    window of twice the key difference wide enough to hold the gap): the
    consistency rule alone rejects it."""
    m, model = _model()
    x, z = _route_inputs(model)
    _, idx, _, key, _ = O._moe(model, 0, x)
    b = model.w["router_bias"][0]
    za = (z - 3.0 * np.sign(z)).astype(np.float32)     # keys move by up to ~0.5
    _, akey = O.keys_from_logits(za.astype(np.float64), b)
    alt = idx.copy()
    checked = 0
    for i in range(len(x)):
        cand = idx[i].copy()
        cand[-1] = O.topk_desc(key[i], m.n_experts)[m.top_k]   # k-th swapped for (k+1)-th
        if np.array_equal(cand, O.topk_desc(akey[i], m.top_k)):
            continue                                    # consistent under these logits: not this case
        e = float(np.max(np.abs(akey[i].astype(np.float64) - key[i].astype(np.float64))))
        rest = np.setdiff1d(np.arange(m.n_experts), cand)
        if float(np.max(key[i][rest]) - np.min(key[i][cand])) <= 2 * e:
            alt[i] = cand                               # the window alone would admit it
            checked += 1
    assert checked >= 1
    h = O.Hints(routing={0: alt}, router_z={0: za})
    _, idx2, _, _, _ = O._moe(model, 0, x, h, 0)
    assert np.array_equal(idx2, idx) and not h.log


def test_route_hint_consistent_near_tie_is_adopted_and_logged():
    """Logits moved just enough that the (k+1)-th expert overtakes the k-th:
    the alternative is the top-k of its own keys, so it is adopted, logged,
    and the oracle's gap lies inside the logged window (twice the key
    difference)."""
    m, model = _model()
    x, z = _route_inputs(model)
    _, idx, _, key, _ = O._moe(model, 0, x)
    i = 2
    order = O.topk_desc(key[i], m.n_experts)
    e_in, e_out = order[m.top_k - 1], order[m.top_k]
    za = z.copy()
    # raise e_out's logit until its float32 key passes e_in's
    s_in = float(O.keys_from_logits(z[i:i + 1], model.w["router_bias"][0])[1][0, e_in])
    lo, hi = z[i, e_out], z[i, e_out] + 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        za[i, e_out] = mid
        ka = O.keys_from_logits(za[i:i + 1].astype(np.float32).astype(np.float64),
                                model.w["router_bias"][0])[1][0]
        if ka[e_out] > s_in:
            hi = mid
        else:
            lo = mid
    za[i, e_out] = hi
    za = za.astype(np.float32)
    _, akey = O.keys_from_logits(za.astype(np.float64), model.w["router_bias"][0])
    alt = np.stack([O.topk_desc(akey[j], m.top_k) for j in range(len(x))])
    assert e_out in alt[i] and e_in not in alt[i]
    h = O.Hints(routing={0: alt}, router_z={0: za})
    _, idx2, _, _, _ = O._moe(model, 0, x, h, 0)
    assert np.array_equal(idx2[i], alt[i])
    assert [a[:3] for a in h.log] == [("route", 0, i)]
    gap, win = h.log[0][3], h.log[0][4]
    assert 0 <= gap <= win
    # other rows: same sets, nothing adopted
    for j in range(len(x)):
        if j != i:
            assert set(idx2[j]) == set(idx[j])


def test_argmax_hint_rules():
    """Argmax: an alternative id that is not a maximum of its own logits is
    rejected; one that is (a planted near-tie) is adopted with the gap inside
    twice the logit difference."""
    wl = di.workload("tiny_fp32")
    m = wl.model
    m.n_layers, m.hidden, m.n_heads, m.head_dim = 1, 16, 2, 8
    m.n_experts, m.top_k, m.expert_ffn, m.shared_ffn, m.vocab_text = 4, 2, 8, 8, 30
    g = wl.gen
    g.block_length, g.steps = 4, 4
    model = O.Model(m, di.make_weights(m, 5))
    cache = O.Cache.empty(m, 1)
    O.block_init(model, cache, np.arange(8, dtype=np.int32)[None] % 30, 4)
    block = np.full((1, 4), m.mask_id, np.int32)
    _, _, ref = O.denoise_step(model, cache, g, block, 0)
    lg = ref["logits"][0]                               # [4, 30] oracle logits
    xh = ref["xhat"][0]
    # alternative: position 1 takes its second-best id; its logits are the
    # oracle's with that id raised just above the best
    j = 1
    second = int(np.argsort(-lg[j], kind="stable")[1])
    la = lg.copy()
    la[j, second] = lg[j, xh[j]] + 1e-9
    alt_x = xh.copy()
    alt_x[j] = second
    h = O.Hints(xhat=alt_x[None], logits=[la], logit_slack=0.0)
    _, _, out = O.denoise_step(model, cache, g, block, 0, hints=h)
    assert out["xhat"][0][j] == second
    assert h.log and h.log[0][:3] == ("argmax", 0, j) and h.log[0][3] <= h.log[0][4]
    # the same alternative id without raised logits: not a maximum, rejected,
    # also when the logits differ a lot elsewhere in the row (a wide window)
    lfar = lg.copy()
    lfar[j, int(np.argsort(-lg[j], kind="stable")[-1])] -= 50.0
    for la2 in (lg, lfar):
        h2 = O.Hints(xhat=alt_x[None], logits=[la2], logit_slack=0.0)
        _, _, out2 = O.denoise_step(model, cache, g, block, 0, hints=h2)
        assert out2["xhat"][0][j] == xh[j] and not h2.log


def test_commit_hint_rules():
    ids = np.full(8, 99, np.int32)
    ids[[0, 3]] = [1, 2]                                # positions 0, 3 fixed
    conf = np.array([0, .5, .4, 0, .39999, .1, .2, .3])
    xhat = np.arange(8) + 10
    # quota ceil(6 / 2) = 3: the oracle takes 1, 2, 4 (0.5, 0.4, 0.39999)
    base, _ = O.select_commit(ids, 99, xhat, conf, 2, 0, False, 0.0)
    assert list(np.nonzero(base != ids)[0]) == [1, 2, 4]
    # an alternative set {1, 2, 7} with confidences that rank it on top
    hc = conf.copy()
    hc[7] = 0.41
    new, info = O.select_commit(ids, 99, xhat, conf, 2, 0, False, 0.0, [1, 2, 7], hc)
    assert info["adopted"] == 1 and list(info["chosen"]) == [1, 2, 7]
    assert info["gap"] <= info["window"] + 1e-15
    # the same set with confidences that do not rank it on top: rejected
    new, info = O.select_commit(ids, 99, xhat, conf, 2, 0, False, 0.0, [1, 2, 7], conf)
    assert info["adopted"] == 0 and list(info["chosen"]) == [1, 2, 4]
    # ... also when those confidences differ a lot elsewhere (a wide window)
    far = conf.copy()
    far[5] = -0.9
    new, info = O.select_commit(ids, 99, xhat, conf, 2, 0, False, 0.0, [1, 2, 7], far)
    assert info["adopted"] == 0 and list(info["chosen"]) == [1, 2, 4]
    # a set of the wrong size: rejected
    new, info = O.select_commit(ids, 99, xhat, conf, 2, 0, False, 0.0, [1, 2], hc)
    assert info["adopted"] == 0


def test_kept_hint_rules():
    """Kept sets: duplicates, wrong per-pool counts and sets that are not the
    selection of their own scores are rejected; a consistent near-tie is
    adopted."""
    rng = np.random.default_rng(4)
    score = rng.random(12)
    pool = np.array([1] * 6 + [0] * 6)
    ratios = (0.5, 0.5)
    ref = O.retention_select(score, 1.0, pool, ratios)
    assert len(ref) == 6
    ok, _, _ = O._alt_kept_valid(score, score, np.concatenate([ref[:-1], ref[:1]]), pool, ratios, 1.0)
    assert not ok                                       # duplicate entry
    in1 = [p for p in range(6) if p not in ref]
    in0 = [p for p in range(6, 12) if p not in ref]
    wrong = np.sort(np.concatenate([ref[ref < 6], [in1[0]], ref[ref >= 6][:-1]]))
    ok, _, _ = O._alt_kept_valid(score, score, wrong, pool, ratios, 1.0)
    assert not ok                                       # 4 visual + 2 text
    # swap the weakest kept text position with the strongest dropped one
    kt = [p for p in ref if p >= 6]
    weakest = min(kt, key=lambda p: score[p])
    strongest = max(in0, key=lambda p: score[p])
    alt = np.sort(np.array([p for p in ref if p != weakest] + [strongest]))
    ok, _, _ = O._alt_kept_valid(score, score, alt, pool, ratios, 1.0)
    assert not ok                                       # not what its scores select
    assert score[strongest] < score[weakest]
    sa = score.copy()                                   # scores under which alt is the selection
    sa[strongest] = score[weakest] + 1e-12
    ok, gap, win = O._alt_kept_valid(score, sa, alt, pool, ratios, 1.0)
    assert ok and gap <= win


def test_attention_mass_matches_scalar_loops():
    """Per-key attention mass at a warm-up step: for every prefix key, the
    softmax probability summed over layers, heads and the block's queries,
    recomputed here element by element from the cached keys with scalar
    loops, and the total over all keys (prefix + block) = L * H * L_B."""
    wl = di.workload("tiny_fp32")
    m = wl.model
    m.n_layers, m.hidden, m.n_heads, m.head_dim = 2, 16, 3, 8
    m.n_experts, m.top_k, m.expert_ffn, m.shared_ffn, m.vocab_text = 4, 2, 8, 8, 40
    g = wl.gen
    g.block_length, g.steps, g.use_sprint, g.keep_ratio = 4, 4, True, 0.5
    model = O.Model(m, di.make_weights(m, 7))
    cache = O.Cache.empty(m, 1)
    rng = np.random.default_rng(8)
    O.block_init(model, cache, rng.integers(0, 40, size=(1, 12)).astype(np.int32), 4)
    block = np.full((1, 4), m.mask_id, np.int32)
    block[0, 2] = 5
    _, _, out = O.denoise_step(model, cache, g, block, 0, O.BlockState())
    mass = out["info"]["mass"][0]
    # scalar recomputation: the block's q/k/v per layer from a forward over
    # the block ids with the same cache, layer inputs captured one at a time
    P, LB, H, d = cache.P, 4, m.n_heads, m.head_dim
    pos = np.arange(P, P + LB)
    ref = [0.0] * P
    total = 0.0
    h = model.embed(block)
    for l in range(m.n_layers):
        x = O.rmsnorm(h, model.dense("attn_norm", l), m.rms_eps)[0]
        W = model.dense("w_qkv", l)
        qkv = [[sum(W[o, i] * x[t, i] for i in range(m.hidden)) for o in range(3 * H * d)] for t in range(LB)]
        for hh in range(H):
            def rot(v, p):
                out_ = list(v)
                for i in range(d // 2):
                    a = p * m.rope_base ** (-2.0 * i / d)
                    out_[i] = v[i] * math.cos(a) - v[i + d // 2] * math.sin(a)
                    out_[i + d // 2] = v[i + d // 2] * math.cos(a) + v[i] * math.sin(a)
                return out_
            qs = [rot(qkv[t][hh * d:(hh + 1) * d], pos[t]) for t in range(LB)]
            ks = [rot(qkv[t][H * d + hh * d:H * d + (hh + 1) * d], pos[t]) for t in range(LB)]
            for t in range(LB):
                keys = [list(cache.K[l][0, j, hh]) for j in range(P)] + ks
                sc = [sum(a * b for a, b in zip(qs[t], kk)) / math.sqrt(d) for kk in keys]
                mx = max(sc)
                z = sum(math.exp(v - mx) for v in sc)
                for j in range(P):
                    ref[j] += math.exp(sc[j] - mx) / z
                total += sum(math.exp(v - mx) / z for v in sc)
        h, _ = O.layer_forward(model, l, h, cache, pos, append=False, block_len=LB)
    assert np.allclose(mass, ref, rtol=1e-10, atol=1e-13)
    assert math.isclose(total, m.n_layers * H * LB, rel_tol=1e-12)
