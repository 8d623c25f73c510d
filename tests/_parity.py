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


def guidance_gain(g):
    """Worst-case growth of a per-row logit error through the guidance mix: the
    L1 norm of the mix coefficients on the model rows (1 without guidance;
    |1 - w| + |w| for CFG; |1 - s_img| + |s_img - s_txt| + |s_txt| for
    three-way guidance)."""
    if g.cfg3_on:
        si, st = g.cfg_image_scale, g.cfg_text_scale
        return abs(1 - si) + abs(si - st) + abs(st)
    if g.cfg_on:
        return abs(1 - g.cfg_scale) + abs(g.cfg_scale)
    return 1.0


def eps_for(wl):
    """Tie tolerances for discrete decisions, from the arithmetic: float32
    paths agree to ~1e-6 relative, bf16 paths to the 2e-2 tolerance.  The
    argmax and commit decisions sit after the guidance mix, which scales the
    per-row logit errors by up to ``guidance_gain``."""
    amp = guidance_gain(wl.gen)
    if wl.model.act_dtype == "f32":
        return dict(route=2e-5, logit=1e-4 * amp, conf=1e-4 * amp, mass=1e-4)
    big = 6e-2 if wl.model.expert_dtype == "fp8" else 2e-2
    return dict(route=5e-3 if big < 5e-2 else 1e-2, logit=big * amp, conf=big * amp, mass=big)


class Result:
    def __init__(self):
        self.hidden_err = []
        self.logit_err = []
        self.conf_err = []
        self.mass_err = []
        self.pconf_err = []
        self.adoptions = []
        self.decisions = 0
        self.steps = 0


def run(wl, weights=None, seed=0, max_steps=None, block=None, session=None, check=True):
    """Run one block on the GPU and the oracle in lock step.  Returns Result."""
    import torch
    from masked_block_diffusion_amd import binding as B

    m, g = wl.model, wl.gen
    if weights is None:
        weights = di.make_weights(m, seed)
    R = g.rows
    LB = g.block_length
    mask = m.mask_id
    say(wl.name, "session", f"L={m.n_layers} D={m.hidden} E={m.n_experts} rows={R} P={wl.prefix_len}")
    sess = session or B.Session(wl, weights)
    prefix = di.make_prefix(wl, seed)
    say(wl.name, "dllm_block_init", prefix.shape)
    sess.block_init(prefix)
    torch.cuda.synchronize()
    model = O.Model(m, weights)
    cache = O.Cache.empty(m, R)
    t0 = time.time()
    O.block_init(model, cache, prefix, LB, g)
    say(wl.name, f"oracle prefill {time.time() - t0:.1f}s")
    ids = di.make_block(wl, seed) if block is None else np.asarray(block, np.int32)
    bstate = O.BlockState()
    eps = eps_for(wl)
    res = Result()
    M = R * LB
    T = g.steps if max_steps is None else min(max_steps, g.steps)
    for t in range(T):
        ids_in = sess.ids_tensor(ids)
        ids_out = torch.empty_like(ids_in)
        say(wl.name, f"dllm_denoise_step t={t}")
        sess.denoise_step(t, ids_in, ids_out)
        torch.cuda.synchronize()
        gids = ids_out.cpu().numpy()
        grem = sess.remaining.cpu().numpy()
        routing = {l: sess.debug(B.DEBUG_ROUTE_IDX, l, np.int32, (M, m.top_k)) for l in range(m.n_layers)}
        gconf = sess.debug(B.DEBUG_CONF, 0, np.float32, (g.n_seq, LB))
        gxhat = sess.debug(B.DEBUG_XHAT, 0, np.int32, (g.n_seq, LB))
        gh = sess.debug(B.DEBUG_HIDDEN, 0, np.float32, (M, m.hidden))
        commits = [np.nonzero((ids[s] == mask) & (gids[s] != mask))[0] for s in range(g.n_seq)]
        select_now = g.use_sprint and not g.cfg3_on and t == g.cache_warmup_steps - 1
        kept = None
        gmass = None
        if select_now:
            P = sess.prefix_length
            nk = sess.debug(B.DEBUG_NKEPT, 0, np.int32, (R,))
            kept_all = sess.debug(B.DEBUG_KEPT, 0, np.int32, (R, sess.max_prefix))
            kept = [kept_all[r, : nk[r]] for r in range(R)]
            gmass = sess.debug(B.DEBUG_MASS, 0, np.float32, (R, sess.max_prefix))[:, :P]
        hints = O.Hints(routing=routing, route_eps=eps["route"], xhat=gxhat,
                        logit_eps=eps["logit"], commit=commits, conf_eps=eps["conf"], kept=kept,
                        mass_eps=eps["mass"])
        t0 = time.time()
        oids, orem, out = O.denoise_step(model, cache, g, ids, t, bstate, hints)
        res.steps += 1
        res.adoptions += hints.log
        res.decisions += M * m.n_layers + int(np.sum(ids == mask))
        # hidden state (model rows x block tokens)
        oh = out["h"].reshape(M, m.hidden)
        res.hidden_err.append(max_abs_rel(gh, oh))
        # logits of masked positions, CFG-mixed
        glog = sess.debug(B.DEBUG_LOGITS, 0, np.float32)
        vsub = (g.vocab_hi or m.vocab) - g.vocab_lo
        nm = int(np.sum(ids == mask))
        if nm:
            hpe = 4 if g.cfg3_on else g.group          # head rows per masked entry
            glog = glog[: nm * hpe * vsub].reshape(-1, hpe, vsub)
            if g.cfg3_on:
                glog = O.cfg3_mix(glog[:, 0], glog[:, 1], glog[:, 2], g.cfg_text_scale, g.cfg_image_scale)
            elif g.cfg_on:
                glog = glog[:, 1] + g.cfg_scale * (glog[:, 0] - glog[:, 1])
            else:
                glog = glog[:, 0]
            olog = np.concatenate([x for x in out["logits"] if len(x)], 0)
            res.logit_err.append(max_abs_rel(glog, olog))
            oc = np.concatenate([out["conf"][s][ids[s] == mask] for s in range(g.n_seq)])
            gc = np.concatenate([gconf[s][ids[s] == mask] for s in range(g.n_seq)])
            res.conf_err.append(max_abs_rel(gc, oc))
        if select_now:
            # the retention score (attention mass or key norm + confidence) and
            # the kept counts, which the oracle fixes per pool
            res.mass_err.append(max_abs_rel(gmass, np.stack(out["retention_score"])))
            ratios = O.pool_ratios_of(g)
            for r in range(R):
                pool = O.modality_pool(cache.ids[r, : cache.P], m) if ratios else np.zeros(P, np.int64)
                assert len(kept[r]) == len(O.retention_select(np.zeros(P), g.keep_ratio, pool, ratios)), r
            if g.retention_score == 1:
                gpc = sess.debug(B.DEBUG_PCONF, 0, np.float32, (R, sess.max_prefix))[:, :P]
                res.pconf_err.append(max_abs_rel(gpc, cache.conf[:, :P]))
        if check:
            assert np.array_equal(gids, oids), f"t={t}: committed ids differ\nGPU {gids}\nORC {oids}"
            assert np.array_equal(grem, orem), f"t={t}: remaining differ {grem} vs {orem}"
        say(wl.name, f"t={t} hidden {res.hidden_err[-1]:.2e} logits "
                     f"{res.logit_err[-1] if res.logit_err else 0:.2e} adoptions {len(hints.log)} "
                     f"oracle {time.time() - t0:.1f}s")
        ids = gids
        if int(np.sum(grem)) == 0:
            break
    res.final_ids = ids
    res.session = sess
    return res
