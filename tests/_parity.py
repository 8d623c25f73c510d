"""Shared driver for GPU-vs-oracle parity: runs the HIP library through the C
ABI and the oracle on the same seeded inputs, step by step.

Where both sides take a discrete decision on floating-point keys (router
top-k, argmax, commit ranking, retained set), the GPU decision is accepted
only if it is also a valid choice under the oracle's own float64 keys within
the stated tolerance (several results are correct when keys tie within
rounding); the oracle logs each such adoption and the tests bound their
number.  Everything else is compared value by value."""
from __future__ import annotations

import sys
import time

import numpy as np

import dllm_inputs as di
from oracle import dllm_oracle as O


def say(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


def max_abs_rel(x, y):
    """max |x - y| / max |y|  (y = oracle)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    den = np.max(np.abs(y)) if y.size else 1.0
    return float(np.max(np.abs(x - y)) / max(den, 1e-30)) if y.size else 0.0


TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


def tolerance(wl):
    m = wl.model
    if m.act_dtype == "f32":
        return TOL["f32"]
    return TOL["fp8"] if m.expert_dtype == "fp8" else TOL["bf16"]


def logit_slack(wl):
    """Allowed difference, relative to a row's largest logit magnitude, between
    the head logits the step's fused kernel decided on and the ones the
    inspection call recomputes from the same rows and weights with another
    kernel: the two float32 dot products of D terms differ only in summation
    order (about D * 2^-24 relative to the sum of |terms|, a few times the
    largest logit here)."""
    return 8.0 * wl.model.hidden * 2.0 ** -24


# Largest share of router and argmax decisions that may take the GPU's
# near-tie choice on the bf16 / fp8 paths (the float32 paths must agree on
# every decision).  Commit and kept sets are checked for validity only: the
# [MASK] positions of a block share one embedding, so their confidences agree
# to about 1e-6 relative, below bf16 resolution, and the retained set's cut
# falls where the masses are densest; there, most differences are ties.
# The prefix's append passes rank up to 256 experts for every clean token of
# a long prefix, where 3-4.5% of the top-k cuts fall inside the window at the
# full-size shapes.
ADOPT_FRAC = {"route": 0.05, "argmax": 0.15, "prefill_route": 0.08}


class Result:
    def __init__(self):
        self.hidden_err = []
        self.logit_err = []
        self.logit_abs_err = []      # max |logit difference| per step (absolute)
        self.conf_self_err = []     # fused confidences vs confidence() of the GPU's own logits
        self.conf_err = []          # fused confidences vs the oracle's (reported)
        self.mass_err = []
        self.route_z_err = []       # router logits the GPU ranked by vs the oracle's, per step
        self.pconf_err = []          # reported: prefix top-1 probabilities vs the oracle's
        self.prefix_x_err = None     # append pass's final-normed rows vs the oracle's
        self.prefix_conf_self_err = None
        self.adoptions = []
        self.decisions = {"route": 0, "argmax": 0, "commit": 0, "kept": 0, "prefill_route": 0}
        self.steps = 0
        self.plans = []
        self.append_plans = []
        self.self_checked = {"route": 0, "argmax": 0, "commit": 0, "kept": 0}

    def adopted(self, kind):
        return [a for a in self.adoptions if a[0] == kind]


def run(wl, weights=None, seed=0, max_steps=None, block=None, session=None, check=True, rows=None,
        prefix=None, keep_experts=False):
    """Run one block on the GPU and the oracle in lock step.  Returns Result.

    rows: optional list of sequences for the oracle to follow (sequences are
    independent: each has its own rows, cache and routing), for shapes where
    the oracle cannot run every sequence; the GPU runs all of them and is
    compared on these.  The prefix is appended in the GPU's append passes
    (see prefill)."""
    import torch
    from masked_block_diffusion_amd import binding as B

    m, g = wl.model, wl.gen
    if weights is None:
        weights = di.make_weights(m, seed)
    R = g.rows
    G = g.group
    LB = g.block_length
    mask = m.mask_id
    seqs = list(range(g.n_seq)) if rows is None else list(rows)
    orows = [s * G + j for s in seqs for j in range(G)]      # model rows the oracle follows
    og = di.clone(wl).gen
    og.n_seq = len(seqs)
    say(wl.name, "session", f"L={m.n_layers} D={m.hidden} E={m.n_experts} rows={R} P={wl.prefix_len}")
    sess = session or B.Session(wl, weights, inspect=True)
    prefix = di.make_prefix(wl, seed) if prefix is None else prefix
    model = O.Model(m, weights, keep_experts=keep_experts)
    cache = O.Cache.empty(m, len(orows))
    res = Result()
    prefill(res, wl, sess, model, cache, prefix, orows, og)
    ids = di.make_block(wl, seed) if block is None else np.asarray(block, np.int32)
    bstate = O.BlockState()
    M = R * LB
    Ro = len(orows)
    tok_rows = np.concatenate([np.arange(r * LB, (r + 1) * LB) for r in orows])   # GPU token rows followed
    T = g.steps if max_steps is None else min(max_steps, g.steps)
    vsub = (g.vocab_hi or m.vocab) - g.vocab_lo
    hpe = 4 if g.cfg3_on else G          # head rows per masked entry
    for t in range(T):
        ids_in = sess.ids_tensor(ids)
        ids_out = torch.empty_like(ids_in)
        say(wl.name, f"dllm_denoise_step t={t}")
        sess.denoise_step(t, ids_in, ids_out)
        torch.cuda.synchronize()
        res.plans.append(sess.attn_plan())
        gids = ids_out.cpu().numpy()
        grem = sess.remaining.cpu().numpy()
        routing_all = {l: sess.debug(B.DEBUG_ROUTE_IDX, l, np.int32, (M, m.top_k)) for l in range(m.n_layers)}
        router_z_all = {l: sess.debug(B.DEBUG_ROUTER_Z, l, np.float32, (M, m.n_experts)) for l in range(m.n_layers)}
        routing = {l: v[tok_rows] for l, v in routing_all.items()}
        router_z = {l: v[tok_rows] for l, v in router_z_all.items()}
        gconf = sess.debug(B.DEBUG_CONF, 0, np.float32, (g.n_seq, LB))
        gxhat = sess.debug(B.DEBUG_XHAT, 0, np.int32, (g.n_seq, LB))
        gh = sess.debug(B.DEBUG_HIDDEN, 0, np.float32, (M, m.hidden))[tok_rows]
        commits = [np.nonzero((ids[s] == mask) & (gids[s] != mask))[0] for s in seqs]
        # the GPU's head logits of every masked entry (recomputed from the
        # step's own final rows), guidance-mixed in float64, per sequence
        nm_seq = [int(np.sum(ids[s] == mask)) for s in range(g.n_seq)]
        glog_seq = [np.zeros((0, vsub))] * g.n_seq
        if sum(nm_seq):
            gl = sess.debug(B.DEBUG_LOGITS, 0, np.float32)[: sum(nm_seq) * hpe * vsub]
            gl = gl.reshape(-1, hpe, vsub).astype(np.float64)
            if g.cfg3_on:
                gl = O.cfg3_mix(gl[:, 0], gl[:, 1], gl[:, 2], g.cfg_text_scale, g.cfg_image_scale)
            elif g.cfg_on:
                gl = O.cfg_mix(gl[:, 0], gl[:, 1], g.cfg_scale)
            else:
                gl = gl[:, 0]
            off = np.concatenate([[0], np.cumsum(nm_seq)])
            glog_seq = [gl[off[s]:off[s + 1]] for s in range(g.n_seq)]
        select_now = g.use_sprint and not g.cfg3_on and t == g.cache_warmup_steps - 1
        kept = None
        gmass = None
        if select_now:
            P = sess.prefix_length
            nk = sess.debug(B.DEBUG_NKEPT, 0, np.int32, (R,))
            kept_all = sess.debug(B.DEBUG_KEPT, 0, np.int32, (R, sess.max_prefix))
            kept = [kept_all[r, : nk[r]] for r in orows]
            gmass_all = sess.debug(B.DEBUG_MASS, 0, np.float32, (R, sess.max_prefix))[:, :P]
            gmass = gmass_all[orows]
        self_consistent(res, wl, t, ids, gids, routing_all, router_z_all, weights["router_bias"], gxhat, gconf,
                        glog_seq,
                        kept_all if select_now else None, nk if select_now else None,
                        gmass_all if select_now else None, sess, P if select_now else 0)
        hints = O.Hints(routing=routing, router_z=router_z, xhat=gxhat[seqs],
                        logits=[glog_seq[s] for s in seqs], logit_slack=logit_slack(wl),
                        commit=commits, conf=gconf[seqs], kept=kept, score=gmass)
        t0 = time.time()
        oids, orem, out = O.denoise_step(model, cache, og, ids[seqs], t, bstate, hints)
        res.steps += 1
        res.adoptions += hints.log
        res.decisions["route"] += Ro * LB * m.n_layers
        res.decisions["argmax"] += int(np.sum(ids[seqs] == mask))
        res.decisions["commit"] += sum(1 for s in seqs if nm_seq[s])
        res.decisions["kept"] += Ro if select_now else 0
        # hidden state (followed model rows x block tokens)
        oh = out["h"].reshape(Ro * LB, m.hidden)
        res.hidden_err.append(max_abs_rel(gh, oh))
        res.route_z_err.append(max(max_abs_rel(router_z[l], out["info"]["route_z"][l]) for l in range(m.n_layers)))
        nm = sum(nm_seq[s] for s in seqs)
        if nm:
            glog = np.concatenate([glog_seq[s] for s in seqs if nm_seq[s]], 0)
            olog = np.concatenate([x for x in out["logits"] if len(x)], 0)
            res.logit_err.append(max_abs_rel(glog, olog))
            res.logit_abs_err.append(float(np.max(np.abs(glog - olog))))
            # the fused head's confidences against the confidence function of
            # the oracle applied to the GPU's own logits (checks the fused
            # reduction), and against the oracle's confidences (reported)
            _, cself = O.confidence(glog, g.confidence)
            gc = np.concatenate([gconf[s][ids[s] == mask] for s in seqs])
            oc = np.concatenate([out["conf"][i][ids[s] == mask] for i, s in enumerate(seqs)])
            res.conf_self_err.append(max_abs_rel(gc, cself))
            res.conf_err.append(max_abs_rel(gc, oc))
        if select_now:
            # the retention score (attention mass or key norm + confidence) and
            # the kept counts, which the oracle fixes per pool
            res.mass_err.append(max_abs_rel(gmass, np.stack(out["retention_score"])))
            ratios = O.pool_ratios_of(g)
            for i, r in enumerate(orows):
                pool = O.modality_pool(cache.ids[i, : cache.P], m) if ratios else np.zeros(P, np.int64)
                assert len(kept[i]) == len(O.retention_select(np.zeros(P), g.keep_ratio, pool, ratios)), r
            if g.retention_score == 1:
                gpc = sess.debug(B.DEBUG_PCONF, 0, np.float32, (R, sess.max_prefix))[orows, :P]
                res.pconf_err.append(max_abs_rel(gpc, cache.conf[:, :P]))
        if check:
            assert np.array_equal(gids[seqs], oids), f"t={t}: committed ids differ\nGPU {gids[seqs]}\nORC {oids}"
            assert np.array_equal(grem[seqs], orem), f"t={t}: remaining differ {grem[seqs]} vs {orem}"
        say(wl.name, f"t={t} hidden {res.hidden_err[-1]:.2e} logits "
                     f"{res.logit_err[-1] if res.logit_err else 0:.2e} router {res.route_z_err[-1]:.2e} conf(self) "
                     f"{res.conf_self_err[-1] if res.conf_self_err else 0:.2e} adoptions {len(hints.log)} "
                     f"plan {res.plans[-1]} oracle {time.time() - t0:.1f}s")
        ids = gids
        if int(np.sum(grem)) == 0:
            break
    res.final_ids = ids
    res.session = sess
    return res


def prefill(res, wl, sess, model, cache, prefix, orows, og):
    """The prefix, appended on both sides in the GPU's append-pass chunks
    (sess.append_tokens tokens per sequence): after each chunk the
    GPU's routing and router logits of that pass go to the oracle's append as
    near-tie hints (the same rule as in the steps), and the chunk's
    final-normed rows (LM-head input) are compared; with the key-norm +
    confidence score, the stored top-1 probabilities are compared with the
    confidence function of those GPU rows times the head (the fused head's
    reduction, up to summation order)."""
    import torch
    from masked_block_diffusion_amd import binding as B
    m, g = wl.model, wl.gen
    R, LB, D = g.rows, g.block_length, m.hidden
    P = prefix.shape[1]
    tok = sess.append_tokens
    lo, hi = g.vocab_lo, (g.vocab_hi or m.vocab)
    wh = model.dense("lm_head")[lo:hi] if g.retention_score == 1 else None
    t0 = time.time()
    say(wl.name, "dllm_block_init", prefix.shape, f"in passes of {tok}")
    if P == 0:   # an empty prefix: the call opens the block with nothing cached
        sess.block_init(prefix)
        O.block_init(model, cache, prefix[orows], LB, og)
    for c0 in range(0, P, tok):
        n = min(tok, P - c0)
        sess.block_init(prefix[:, c0:c0 + n])
        torch.cuda.synchronize()
        res.append_plans.append(sess.attn_plan())
        tr = np.concatenate([np.arange(r * n, (r + 1) * n) for r in orows])
        hints = O.Hints(routing={l: sess.debug(B.DEBUG_ROUTE_IDX, l, np.int32, (R * n, m.top_k))[tr]
                                 for l in range(m.n_layers)},
                        router_z={l: sess.debug(B.DEBUG_ROUTER_Z, l, np.float32, (R * n, m.n_experts))[tr]
                                  for l in range(m.n_layers)})
        h = O.block_init(model, cache, prefix[orows, c0:c0 + n], LB, og, hints)
        res.adoptions += [("prefill_" + a[0],) + a[1:] for a in hints.log]
        res.decisions["prefill_route"] += len(tr) * m.n_layers
        raw = sess.debug(B.DEBUG_NORMED, 0, np.uint16 if m.act_dtype == "bf16" else np.float32, (R * n, D))
        xg = O.decode(raw, m.act_dtype).reshape(R, n, D)[orows]
        xo = O.rmsnorm(h, model.dense("final_norm"), m.rms_eps)
        res.prefix_x_err = max(res.prefix_x_err or 0.0, max_abs_rel(xg, xo))
        if wh is not None:
            gpc = sess.debug(B.DEBUG_PCONF, 0, np.float32, (R, sess.max_prefix))[orows, c0:c0 + n]
            cself = np.stack([O.confidence(xg[i] @ wh.T, 0)[1] for i in range(len(orows))])
            res.prefix_conf_self_err = max(res.prefix_conf_self_err or 0.0, max_abs_rel(gpc, cself))
    say(wl.name, f"prefill {time.time() - t0:.1f}s: rows {res.prefix_x_err or 0:.2e} conf(self) "
                 f"{res.prefix_conf_self_err if res.prefix_conf_self_err is not None else 0:.2e} "
                 f"route adoptions {len(res.adopted('prefill_route'))}")


def self_consistent(res, wl, t, ids, gids, routing, router_z, bias, gxhat, gconf, glog_seq, kept_all, n_kept,
                    gmass, sess, P):
    """Every decision the GPU took in this step is exactly the one its own
    keys imply under the oracle's rules, on every row and sequence (not only
    the ones the oracle follows): router top-k of its float32 keys (ties to
    the lower id), argmax of its logits (up to the summation-order slack),
    the commit of its confidences and argmax ids, the retained set of its
    scores."""
    m, g = wl.model, wl.gen
    mask = m.mask_id
    for l, idx in routing.items():
        _, key = O.keys_from_logits(router_z[l].astype(np.float64), bias[l])
        for i in range(len(idx)):
            assert np.array_equal(idx[i], O.topk_desc(key[i], m.top_k)), ("route", t, l, i)
        res.self_checked["route"] += len(idx)
    slack = logit_slack(wl)
    for s in range(g.n_seq):
        pos = np.nonzero(ids[s] == mask)[0]
        lg = glog_seq[s]
        for j, p in enumerate(pos):
            a = int(gxhat[s, p]) - g.vocab_lo
            assert lg[j, a] >= np.max(lg[j]) - slack * np.max(np.abs(lg[j])), ("argmax", t, s, p)
        res.self_checked["argmax"] += len(pos)
        new, _ = O.select_commit(ids[s], mask, gxhat[s], gconf[s].astype(np.float64), g.steps, t,
                                 g.use_threshold, g.threshold)
        assert np.array_equal(new, gids[s]), ("commit", t, s, new, gids[s])
        res.self_checked["commit"] += 1
    if kept_all is not None:
        ratios = O.pool_ratios_of(g)
        from masked_block_diffusion_amd import binding as B
        pids = sess.debug(B.DEBUG_PIDS, 0, np.int32, (g.rows, sess.max_prefix))[:, :P] if ratios else None
        for r in range(g.rows):
            pool = O.modality_pool(pids[r], m) if ratios else np.zeros(P, np.int64)
            ref = O.retention_select(gmass[r].astype(np.float64), g.keep_ratio, pool, ratios)
            assert np.array_equal(kept_all[r, : n_kept[r]], ref), ("kept", t, r)
        res.self_checked["kept"] += g.rows


def check(res, wl, adopt_frac=None):
    """Tolerances of every compared quantity, and the adoption bound per
    decision type."""
    tol = tolerance(wl)
    assert max(res.hidden_err) <= tol, res.hidden_err
    # the router keys the GPU decided on: every near-tie window is twice
    # their measured difference, so that difference is held to the tolerance
    assert max(res.route_z_err) <= tol, res.route_z_err
    if res.logit_err:
        assert max(res.logit_err) <= tol, res.logit_err
        # the fused reduction against the same function on the GPU's own logits
        ctol = 1e-5 if wl.model.act_dtype == "f32" else 1e-4
        assert max(res.conf_self_err) <= ctol, res.conf_self_err
    if res.mass_err:
        assert max(res.mass_err) <= tol, res.mass_err
    if res.prefix_x_err is not None:
        # the appended tokens' final-normed rows within the tolerance, and the
        # fused head's prefix probabilities equal to the confidence function
        # of those rows
        assert res.prefix_x_err <= tol, res.prefix_x_err
    if res.prefix_conf_self_err is not None:
        ctol = 1e-5 if wl.model.act_dtype == "f32" else 1e-4
        assert res.prefix_conf_self_err <= ctol, res.prefix_conf_self_err
    assert all(res.self_checked[k] > 0 for k in ("route", "commit")), res.self_checked
    f32 = wl.model.act_dtype == "f32"
    for kind, n in res.decisions.items():
        got = res.adopted(kind)
        for a in got:                       # every adoption lies inside its window
            assert a[-2] <= a[-1], a
        if f32 or adopt_frac == 0.0:
            assert not got, (kind, got)
        elif kind in ADOPT_FRAC:
            frac = ADOPT_FRAC[kind] if adopt_frac is None else adopt_frac
            assert len(got) <= int(frac * n) + 1, (kind, n, got)
    say("decisions", res.decisions, "adopted", {k: len(res.adopted(k)) for k in res.decisions},
        "self-checked", res.self_checked)
