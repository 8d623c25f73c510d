"""Whole-step parity of the HIP library (through the C ABI) against the
oracle on seeded inputs: hidden states and logits within the stated
tolerance, committed ids / remaining counts exact (GPU near-tie decisions
accepted only when valid under the oracle's keys, and counted)."""
import numpy as np
import pytest

import dllm_inputs as di
from masked_block_diffusion_amd import binding as B
from tests import _parity as PA

pytestmark = pytest.mark.gpu


def _check(res, wl, max_adopt_frac=None):
    PA.check(res, wl, max_adopt_frac)


def test_tiny_fp32_free_running_generation():
    """2-layer fp32 model, 64-token prefix, one all-[MASK] block of 32 in 8
    steps, 4 per step: every committed id matches the oracle."""
    wl = di.workload("tiny_fp32")
    block = np.full((1, 32), wl.model.mask_id, np.int32)
    res = PA.run(wl, seed=0, block=block)
    _check(res, wl, max_adopt_frac=0.0)
    assert res.steps == 8
    assert not np.any(res.final_ids == wl.model.mask_id)


def test_small_bf16_block():
    wl = di.workload("small_bf16")
    res = PA.run(wl, seed=1, block=np.full((1, 32), wl.model.mask_id, np.int32))
    _check(res, wl)
    assert not np.any(res.final_ids == wl.model.mask_id)


def test_small_cfg_block():
    wl = di.workload("small_cfg")
    res = PA.run(wl, seed=2, block=np.full((1, 32), wl.model.mask_id, np.int32), max_steps=3)
    _check(res, wl)


def test_small_sprint_threshold_block():
    wl = di.workload("small_sprint")
    res = PA.run(wl, seed=3, block=np.full((1, 32), wl.model.mask_id, np.int32), max_steps=4)
    _check(res, wl)
    assert res.mass_err


def test_small_sprint_keynorm_conf_pools():
    """SPRINT with the review's score (key norm + top-1 probability, alpha 0.5)
    and modality pools (image 0.8, text 1.0) over a 64-visual + 32-text prefix:
    prefix confidences, scores and per-pool kept sets match the oracle, and the
    later steps attend to the kept set only."""
    wl = di.workload("small_sprint_kc")
    res = PA.run(wl, seed=5, block=np.full((1, 32), wl.model.mask_id, np.int32), max_steps=3)
    _check(res, wl)
    assert res.mass_err and res.pconf_err
    n_kept = res.session.debug(B.DEBUG_NKEPT, 0, np.int32, (1,))
    assert n_kept[0] == 52 + 32          # ceil(0.8 * 64) + 32


def test_small_sprint_keynorm_conf_f32_cfg():
    """The same score in float32 (tight tolerance) with a CFG pair: each model
    row (conditional, unconditional) scores and prunes its own prefix; the
    unconditional row's [MASK] prompt falls in the text pool."""
    wl = di.workload("small_sprint_kc")
    wl.model.act_dtype = wl.model.expert_dtype = "f32"
    wl.gen.cfg_scale = 2.0
    wl.gen.use_threshold = False
    wl.gen.steps = 8
    res = PA.run(wl, seed=6, block=np.full((1, 32), wl.model.mask_id, np.int32), max_steps=3)
    _check(res, wl)
    n_kept = res.session.debug(B.DEBUG_NKEPT, 0, np.int32, (2,))
    assert list(n_kept) == [52 + 32, 96]


def test_small_edit_three_way_guidance():
    """Editing with three-way guidance (text scale 4.0, image scale 1.5): model
    rows (full prompt, image-only prompt, unconditional) each with their own
    cache; the fused head mixes each 4-row group before the confidence."""
    wl = di.workload("small_edit")
    res = PA.run(wl, seed=7, block=np.full((1, 32), wl.model.mask_id, np.int32), max_steps=3)
    _check(res, wl)
    assert res.logit_err


def test_small_edit_f32_batch_sprint_fallback():
    """Float32 three-way guidance over 2 sequences (6 model rows) with SPRINT
    requested: SPRINT falls back to the baseline on both sides (no retention),
    every committed id matches."""
    wl = di.workload("small_edit")
    wl.model.act_dtype = wl.model.expert_dtype = "f32"
    wl.gen.n_seq = 2
    wl.gen.use_sprint = True
    wl.gen.keep_ratio = 0.5
    res = PA.run(wl, seed=8, max_steps=3)
    _check(res, wl, max_adopt_frac=0.0)
    assert not res.mass_err
    assert np.all(res.session.debug(B.DEBUG_NKEPT, 0, np.int32, (6,)) == 0)


@pytest.mark.parametrize("name,prefix,n_seq", [("small_bf16", 512, 1), ("small_fp8", 256, 4),
                                              ("tiny_fp32", 256, 1)])
def test_long_prefill_expert_items(name, prefix, n_seq):
    """Prefixes long enough that the append pass runs the work-list expert
    path with many rows per expert (>= 24 slots per expert on average, several
    32-row items for most experts): the cached K/V it produces drive the
    following steps, which match the oracle."""
    wl = di.workload(name)
    wl.prefix_len = prefix
    wl.gen.n_seq = n_seq
    m = wl.model
    assert n_seq * min(prefix, 1024 // n_seq) * m.top_k >= 24 * m.n_experts
    res = PA.run(wl, seed=9, max_steps=2)
    _check(res, wl)


@pytest.mark.parametrize("name,steps", [("small_bf16", 2), ("small_fp8", 2), ("tiny_fp32", 2),
                                        ("layer_bf16", 1)])
def test_packed_gate_up_bit_identical(name, steps):
    """Gate/up weights in the packed fragment layout (dllm_pack_gate_up) give
    bit-identical steps to the row-major layout: only addresses change."""
    import torch
    wl = di.workload(name)
    m, g = wl.model, wl.gen
    w = di.make_weights(m, 3)
    prefix, block = di.make_prefix(wl, 3), di.make_block(wl, 3)
    out = []
    for pack in (False, True):
        s = B.Session(wl, w, pack_gate_up=pack)
        assert s.w.gate_up_packed == int(pack)
        s.block_init(prefix)
        ids = s.ids_tensor(block)
        hs = []
        for t in range(steps):
            nxt = torch.empty_like(ids)
            s.denoise_step(t, ids, nxt)
            hs.append(s.debug(B.DEBUG_HIDDEN, 0, np.float32))
            ids = nxt
        out.append((ids.cpu().numpy(), hs))
        s.close()
    assert np.array_equal(out[0][0], out[1][0])
    for a, b in zip(out[0][1], out[1][1]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name,n_seq", [("small_bf16", 4), ("small_cfg", 2), ("small_edit", 1)])
def test_large_vocab_tiled_head(name, n_seq):
    """128 head rows over a 40,960-id sub-vocabulary (one row per entry, CFG
    pairs, three-way groups): enough 128 x 128 tiles for the LDS-tiled LM head
    with 128-column confidence partials."""
    wl = di.workload(name)
    m, g = wl.model, wl.gen
    g.n_seq = n_seq
    if g.vocab_hi and g.vocab_lo >= m.vocab_text:   # image sub-vocabulary
        m.vocab_image = 40960
        g.vocab_lo, g.vocab_hi = m.vocab_text, m.vocab_text + 40960
    else:
        m.vocab_text = 40960
        g.vocab_lo, g.vocab_hi = 0, 40960
    rows = n_seq * 32 * (4 if g.cfg_text_scale > 0 else (2 if g.cfg_scale > 0 else 1))
    assert rows == 128 and (g.vocab_hi - g.vocab_lo) // 128 >= 256
    res = PA.run(wl, seed=6, block=np.full((n_seq, 32), m.mask_id, np.int32), max_steps=2)
    _check(res, wl)


@pytest.mark.parametrize("name,n_seq", [("small_bf16", 6), ("small_bf16", 2), ("small_cfg", 3), ("small_edit", 2),
                                        ("small_bf16", 8)])
def test_ragged_vocab_tiled_head(name, n_seq):
    """LDS-tiled LM head over a 41,037-id sub-vocabulary (the last 128-column
    tile holds 77 ids): 192 or 256 head rows (two 128-row tiles, the second
    partial at 192; CFG pairs for small_cfg, three-way groups for small_edit)
    or 64 rows (the 64-row tile).  The second step has fewer head rows than
    the launch's capacity, so only the live row tiles run.  With 8 sequences
    (8 x 32 entries x 321 partials) the confidence merge runs one workgroup
    per entry, then the per-sequence commit."""
    wl = di.workload(name)
    m, g = wl.model, wl.gen
    g.n_seq = n_seq
    m.vocab_text = 41037
    g.vocab_lo, g.vocab_hi = 0, 41037
    rows = n_seq * 32 * (4 if g.cfg_text_scale > 0 else (2 if g.cfg_scale > 0 else 1))
    assert rows in (64, 192, 256) and (g.vocab_hi - g.vocab_lo) % 128 == 77
    res = PA.run(wl, seed=8, block=np.full((n_seq, 32), m.mask_id, np.int32), max_steps=2)
    _check(res, wl)


@pytest.mark.parametrize("prefix", [48, 64])
def test_block16_partial_attention_tiles(prefix):
    """16-token blocks: every append pass ends its key range inside a 32-key
    attention tile, and with a 64-token prefix the block's own keys fill half
    a tile in each step (the streaming kernel reads the last valid row for the
    rest, with weight 0); a 48-token prefix is not a multiple of 32, so steps
    take the 128-key kernel."""
    wl = di.workload("small_bf16")
    wl.gen.block_length = 16
    wl.gen.steps = 4
    wl.prefix_len = prefix
    wl.masked_in_block = 16
    res = PA.run(wl, seed=11, block=np.full((1, 16), wl.model.mask_id, np.int32))
    _check(res, wl)
    assert not np.any(res.final_ids == wl.model.mask_id)


def test_small_fp8_batch():
    wl = di.workload("small_fp8")
    res = PA.run(wl, seed=4, max_steps=3)
    _check(res, wl)


def test_layer_bf16_full_size_step():
    """One 16B-scale MoE layer (hidden 2048, 256 experts top-8 + shared) over a
    1024-token prefix; a 32-token block with 16 [MASK]."""
    wl = di.workload("layer_bf16")
    res = PA.run(wl, seed=0, max_steps=2)
    _check(res, wl)


def test_t2i_layer_full_size_cfg_block():
    """One layer at the text-to-image shape (hidden 2048, 256 experts top-8 +
    shared): the conditional / unconditional row pair of one sequence (the
    unconditional prompt all [MASK]) over a 256-token prompt, CFG scale 2.0
    mixed on the head's logit tiles over the 16,384-id visual sub-vocabulary,
    an all-[MASK] block of 32 finished in 8 steps of 4 commits."""
    wl = di.workload("t2i_layer")
    res = PA.run(wl, seed=3, block=np.full((1, 32), wl.model.mask_id, np.int32), keep_experts=True)
    _check(res, wl)
    assert res.steps == 8
    assert not np.any(res.final_ids == wl.model.mask_id)
    lo, hi = wl.gen.vocab_lo, wl.gen.vocab_hi
    assert np.all((res.final_ids >= lo) & (res.final_ids < hi))


def _bf16_to_f64(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _f32_to_bf16(x):
    """Round-to-nearest-even float32 -> bf16 bits (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_think_fp8_layer_full_size_head_sampled():
    """The batched thinking layer at full size, in the launch configuration the
    bench times (16 sequences x 2048-token prefix, fp8 experts, the LDS-tiled
    LM head over the 157,184-id text sub-vocabulary: 256 head rows of 512 in
    the launch): for sampled masked positions, the step's confidence and
    argmax against an fp64 head over all 157,184 ids, fed with the step's own
    final hidden state (RMSNorm in float32, rounded to bf16 like the head's
    input).  Low-confidence score c = 1 / sum exp(l - max l)."""
    torch = pytest.importorskip("torch")
    wl = di.workload("think_fp8_layer")
    m, g = wl.model, wl.gen
    assert g.confidence == 0 and not g.cfg_on
    w = di.make_weights(m, 0)
    prefix, block = di.make_prefix(wl, 0), di.make_block(wl, 0)
    s = B.Session(wl, w, max_prefix=wl.prefix_len + g.block_length, max_clean=wl.prefix_len)
    s.block_init(prefix)
    ids_in = s.ids_tensor(block)
    ids_out = torch.empty_like(ids_in)
    s.denoise_step(g.steps // 2, ids_in, ids_out)
    LB, D = g.block_length, m.hidden
    h = s.debug(B.DEBUG_HIDDEN, shape=(g.n_seq * LB, D))
    conf = s.debug(B.DEBUG_CONF, shape=(g.n_seq, LB))
    xhat = s.debug(B.DEBUG_XHAT, dtype=np.int32, shape=(g.n_seq, LB))
    masked = np.argwhere(block == m.mask_id)
    assert len(masked) == 256 and np.all(np.isfinite(conf[block == m.mask_id]))
    picks = masked[np.linspace(0, len(masked) - 1, 6).astype(int)]
    rows = picks[:, 0] * LB + picks[:, 1]
    hr = h[rows].astype(np.float32)
    inv = np.float32(1.0) / np.sqrt(np.mean(hr * hr, axis=1, dtype=np.float32) + np.float32(m.rms_eps))
    x = _bf16_to_f64(_f32_to_bf16(hr * inv[:, None] * w["final_norm"][None, :]))
    lo, hi = g.vocab_lo, g.vocab_hi
    logits = np.empty((len(rows), hi - lo))
    for c0 in range(lo, hi, 16384):
        c1 = min(hi, c0 + 16384)
        logits[:, c0 - lo:c1 - lo] = x @ _bf16_to_f64(w["lm_head"][c0:c1]).T
    ref_idx = np.argmax(logits, axis=1)
    ref_max = logits[np.arange(len(rows)), ref_idx]
    ref_conf = 1.0 / np.sum(np.exp(logits - ref_max[:, None]), axis=1)
    got_conf = conf[picks[:, 0], picks[:, 1]].astype(np.float64)
    got_idx = xhat[picks[:, 0], picks[:, 1]] - lo
    PA.say("sampled head rows", rows.tolist(), "conf", got_conf.tolist(), "ref", ref_conf.tolist())
    np.testing.assert_allclose(got_conf, ref_conf, rtol=2e-3)
    for i in range(len(rows)):   # argmax: equal, or a near-tie of the fp64 logits
        assert got_idx[i] == ref_idx[i] or ref_max[i] - logits[i, got_idx[i]] <= 2e-3, (i, got_idx[i], ref_idx[i])


def test_router_column_tiles_256_experts():
    """256 experts and 4 sequences (128 model rows): the router's 64-row tiles
    take 4 column tiles per workgroup, sharing the normalized rows; two layers,
    so layer 0's routing reaches the compared hidden states and ids."""
    wl = di.workload("small_bf16")
    wl.model.n_experts = 256
    wl.gen.n_seq = 4
    res = PA.run(wl, seed=12, block=np.full((4, 32), wl.model.mask_id, np.int32), max_steps=2)
    _check(res, wl)


def _oracle_generate(wl, weights, prefix, blocks):
    """Free-running oracle generation of len(blocks) blocks after `prefix`."""
    from oracle import dllm_oracle as O
    m, g = wl.model, wl.gen
    model = O.Model(m, weights)
    cache = O.Cache.empty(m, g.rows)
    O.block_init(model, cache, prefix, g.block_length, g)
    out = []
    for b in blocks:
        ids, n, _ = O.generate_block(model, cache, g, b)
        out.append((ids, n))
        O.block_init(model, cache, np.repeat(ids, g.group, axis=0), g.block_length, g)
    return out


def test_generate_block_two_blocks_tiny_fp32():
    """dllm_generate_block through the C ABI: an all-[MASK] block runs its 8
    steps (4 commits each) and every committed id equals the oracle's
    free-running generation; the finished block is then appended with
    dllm_block_init and the next block generated the same way."""
    torch = pytest.importorskip("torch")
    wl = di.workload("tiny_fp32")
    m, g = wl.model, wl.gen
    w = di.make_weights(m, 0)
    prefix = di.make_prefix(wl, 0)
    s = B.Session(wl, w, max_prefix=wl.prefix_len + 2 * g.block_length)
    s.block_init(prefix)
    blocks = [np.full((1, g.block_length), m.mask_id, np.int32)] * 2
    got = []
    for b in blocks:
        ids = s.ids_tensor(b)
        n = s.generate_block(ids)
        torch.cuda.synchronize()
        got.append((ids.cpu().numpy(), n))
        s.block_init(ids)
    assert s.prefix_length == wl.prefix_len + 2 * g.block_length
    ref = _oracle_generate(wl, w, prefix, blocks)
    for (gi, gn), (oi, on) in zip(got, ref):
        assert gn == on == 8
        assert np.array_equal(gi, oi), (gi, oi)
        assert not np.any(gi == m.mask_id)
    s.close()


def test_generate_block_threshold_zero_one_step():
    """Threshold mode with threshold 0: every masked position has c > 0, so the
    first step commits all of them and the block loop stops after one step;
    the committed ids equal the oracle's."""
    torch = pytest.importorskip("torch")
    wl = di.workload("tiny_fp32")
    m, g = wl.model, wl.gen
    g.use_threshold, g.threshold = True, 0.0
    w = di.make_weights(m, 1)
    prefix = di.make_prefix(wl, 1)
    s = B.Session(wl, w)
    s.block_init(prefix)
    block = np.full((1, g.block_length), m.mask_id, np.int32)
    ids = s.ids_tensor(block)
    n = s.generate_block(ids)
    torch.cuda.synchronize()
    (oi, on), = _oracle_generate(wl, w, prefix, [block])
    assert n == on == 1
    assert np.array_equal(ids.cpu().numpy(), oi)
    s.close()


@pytest.mark.parametrize("strategy,n_seq,vocab", [(1, 1, 0), (2, 1, 0), (1, 4, 41037), (2, 4, 41037)])
def test_confidence_strategies_fused_head(strategy, n_seq, vocab):
    """top_k_margin (p1 - p2) and neg_entropy (sum p log p) through the fused
    head of a whole step: the streaming head (32 head rows) and, over a
    41,037-id sub-vocabulary with 4 sequences, the LDS-tiled head (128 rows,
    128-column partials); confidences, commits and hidden states against the
    oracle."""
    wl = di.workload("small_bf16")
    m, g = wl.model, wl.gen
    g.confidence = strategy
    g.n_seq = n_seq
    if vocab:
        m.vocab_text = vocab
        g.vocab_lo, g.vocab_hi = 0, vocab
    res = PA.run(wl, seed=13 + strategy, block=np.full((n_seq, 32), m.mask_id, np.int32), max_steps=3)
    _check(res, wl)
    assert res.conf_self_err


def test_streaming_attention_multi_tile_and_append_passes():
    """16 sequences over 1024-token prefixes: 64 (row, head) units, so the
    streaming attention plan gives each workgroup a range of more than 128
    keys (several 32-key tiles per wavefront with the online-softmax rescale)
    and merges 3 splits; the prefill goes in as 16 append passes of 64 tokens,
    all but the first at P > 0."""
    wl = di.workload("small_bf16")
    wl.gen.n_seq = 16
    wl.prefix_len = 1024
    res = PA.run(wl, seed=14, max_steps=2)
    _check(res, wl)
    kind, split, n_splits = res.plans[0]
    assert kind == B.ATTN_STREAM and split > 128 and n_splits > 1, res.plans


def test_prefill_pass_items_dealt_per_xcd():
    """One append pass of 4096 token rows (8 sequences x 512-token prefixes):
    in passes of 2048 rows or more the work-list expert kernels deal the
    items to the XCDs in turn (here at most 352 items of 2 gate/up and 4
    down column blocks, on grids sized for 353 items, so the layout fits);
    the pass's final-normed rows and the following steps match the
    oracle."""
    wl = di.workload("small_bf16")
    wl.gen.n_seq = 8
    wl.prefix_len = 512
    res = PA.run(wl, seed=31, max_steps=2)
    assert res.session.append_tokens * wl.gen.rows >= 2048 and len(res.append_plans) == 1, \
        (res.session.append_tokens, res.append_plans)
    _check(res, wl)


@pytest.mark.parametrize("hidden,ffn", [(1024, 512), (2048, 256)])
def test_fp8_experts_multi_chunk(hidden, ffn):
    """fp8 experts with several 64-wide chunks per wavefront: hidden 1024 gives
    each gate/up wavefront 2 chunks, expert width 512 gives the down kernel 8
    chunks (4 batches of 2); hidden 2048 gives gate/up 4 chunks.  Batch 4 with
    a 256-token prefix (work-list items in the append passes)."""
    wl = di.workload("small_fp8")
    wl.model.hidden = hidden
    wl.model.expert_ffn = ffn
    wl.prefix_len = 256
    res = PA.run(wl, seed=15, max_steps=2)
    _check(res, wl)


def test_tiled_qkv_paired_tiles_head128():
    """The tiled QKV projection with head width 128 takes paired 64-column
    tiles (columns j0..j0+31 and j0+64..j0+95 of a head, the two halves of 32
    rotation pairs): 4 sequences (128-row steps) with 2 heads of 128 and
    1024-row append passes."""
    wl = di.workload("small_fp8")
    wl.model.n_heads = 2
    wl.model.head_dim = 128
    wl.prefix_len = 256
    res = PA.run(wl, seed=17, max_steps=2)
    _check(res, wl)


@pytest.mark.parametrize("heads,dh,prefix", [(4, 64, 480), (8, 32, 512)])
def test_append_pass_shared_key_tiles(heads, dh, prefix):
    """Append passes of 4+ query blocks (enough workgroups) take the kernel in
    which 4 query blocks of one (row, head) share each K/V tile: 4 sequences
    with a 15-block prefix at head width 64 (the last group of query blocks
    has an idle wavefront) and a 16-block prefix at head width 32, one pass
    each; the pass's final-normed rows and the later steps are compared with
    the oracle."""
    from masked_block_diffusion_amd import binding as B
    wl = di.workload("small_fp8")
    wl.model.n_heads = heads
    wl.model.head_dim = dh
    wl.prefix_len = prefix
    res = PA.run(wl, seed=23, max_steps=2)
    assert [p[0] for p in res.append_plans] == [B.ATTN_APPEND], res.append_plans
    _check(res, wl)


@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16"])
def test_empty_prefix(name):
    """No cached prefix (the block is the whole context): the block's queries
    attend to the block alone; float32 decisions match exactly.  The block
    holds some fixed ids: an all-[MASK] block without context has positions
    that differ only by RoPE, whose confidences tie to 1e-18 in float64."""
    wl = di.workload(name)
    wl.prefix_len = 0
    wl.prefix_visual = 0
    wl.masked_in_block = 20
    res = PA.run(wl, seed=19, max_steps=3)
    _check(res, wl, max_adopt_frac=0.0 if wl.model.act_dtype == "f32" else None)


def test_block_without_mask_and_single_mask():
    """Degenerate blocks: with no [MASK] a step commits nothing and leaves the
    ids unchanged; with one [MASK] the step commits exactly that position."""
    import torch
    wl = di.workload("tiny_fp32")
    m = wl.model
    block = di.make_block(wl, 21)
    full = np.where(block == m.mask_id, 7, block).astype(np.int32)
    res = PA.run(wl, seed=21, block=full, max_steps=1)
    _check(res, wl, max_adopt_frac=0.0)
    assert np.array_equal(res.final_ids, full)
    one = full.copy()
    one[0, 13] = m.mask_id
    res = PA.run(wl, seed=21, block=one, max_steps=1)
    _check(res, wl, max_adopt_frac=0.0)
    assert res.final_ids[0, 13] != m.mask_id
    assert np.array_equal(np.delete(res.final_ids[0], 13), np.delete(one[0], 13))
