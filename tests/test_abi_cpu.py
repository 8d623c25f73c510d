"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, sizes workspaces, and rejects bad calls
before any launch."""
import ctypes as C
import os
import re

import pytest

import dllm_inputs as di

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dllm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dllm_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    from masked_block_diffusion_amd import binding as B
    lib = B.load_library()
    names = _declared()
    assert "dllm_denoise_step" in names and "dllm_block_init" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTED)


def _structs(name="layer_bf16", **over):
    from masked_block_diffusion_amd import binding as B
    wl = di.workload(name)
    for k, v in over.items():
        setattr(wl.gen, k, v)
    return wl, B.model_config_struct(wl.model), B.gen_params_struct(wl.gen, 2048, 1024)


def test_workspace_sizes():
    from masked_block_diffusion_amd import binding as B
    wl, c, g = _structs()
    ws = B.dllm_workspace_bytes(c, g)
    kv = B.dllm_kv_bytes(c, g)
    assert ws > 0 and ws % 256 == 0
    assert kv == 1 * 1 * 16 * 2048 * 128 * 2
    # append passes: whole blocks up to 4096 model-row tokens, capped by max_clean
    R, LB = wl.gen.rows, g.block_length
    assert B.dllm_append_tokens(c, g) == min(max(1, 4096 // (R * LB)) * LB, 1024)
    g.max_clean_tokens = 0
    assert B.dllm_append_tokens(c, g) == max(1, 4096 // (R * LB)) * LB
    g.max_clean_tokens = 1024
    c.hidden = 100                                       # not a multiple of 128
    assert B.dllm_workspace_bytes(c, g) == 0
    assert B.dllm_append_tokens(c, g) == 0


def _fake_weights(B, fp8=False):
    w = B.dllm_weights()
    for i, (n, _) in enumerate(B.dllm_weights._fields_):
        setattr(w, n, 0x10000000 + 0x1000 * i)
    return w


def test_create_and_call_order_errors_without_gpu():
    """Every error here is raised on the host before any HIP call."""
    from masked_block_diffusion_amd import binding as B
    wl, c, g = _structs()
    w = _fake_weights(B)
    kv = B.dllm_kv_cache(0x20000000, 0x30000000)
    ws = B.dllm_workspace_bytes(c, g)
    st, ctx = B.dllm_create(c, g, w, kv, 0x40000000, ws - 1, 0)
    assert st == B.DLLM_ERR_OUT_OF_MEMORY
    st, ctx = B.dllm_create(c, g, w, kv, 0x40000001, ws, 0)   # misaligned workspace
    assert st == B.DLLM_ERR_INVALID_ARG
    w2 = _fake_weights(B)
    w2.w_qkv = None
    assert B.dllm_create(c, g, w2, kv, 0x40000000, ws, 0)[0] == B.DLLM_ERR_INVALID_ARG
    st, ctx = B.dllm_create(c, g, w, kv, 0x40000000, ws, 0)
    assert st == B.DLLM_OK
    assert B.dllm_prefix_length(ctx) == 0
    assert B.dllm_denoise_step(ctx, 0, 0x1000, 0x1000, 0x2000) == B.DLLM_ERR_BAD_STATE
    assert "block_init" in B.dllm_last_error(ctx)
    assert B.dllm_denoise_step(ctx, -1, 0x1000, 0x1000, 0x2000) == B.DLLM_ERR_INVALID_ARG
    assert B.dllm_denoise_step(ctx, 0, 0, 0x1000, 0x2000) == B.DLLM_ERR_INVALID_ARG
    assert B.dllm_block_init(ctx, 0x1000, 33) == B.DLLM_ERR_INVALID_ARG
    assert B.dllm_block_init(ctx, 0x1000, 2048 + 32) == B.DLLM_ERR_INVALID_ARG   # > max_clean
    B.dllm_destroy(ctx)


def test_shape_validation_messages():
    from masked_block_diffusion_amd import binding as B
    wl, c, g = _structs()
    g.block_length = 65
    assert B.dllm_workspace_bytes(c, g) == 0
    wl, c, g = _structs()
    c.expert_dtype = B.DLLM_F32                 # bf16 activations need bf16/fp8 experts
    assert B.dllm_workspace_bytes(c, g) == 0
    wl, c, g = _structs()
    g.vocab_lo, g.vocab_hi = 10, 5
    assert B.dllm_workspace_bytes(c, g) == 0
    # fp8 expert fragments span 64 reduction elements, split over 8 wavefronts
    wl, c, g = _structs()
    c.expert_dtype = B.DLLM_FP8_E4M3
    assert B.dllm_workspace_bytes(c, g) > 0
    c.hidden = 768
    assert B.dllm_workspace_bytes(c, g) == 0
    c.hidden, c.expert_ffn = 2048, 96
    assert B.dllm_workspace_bytes(c, g) == 0


def test_retention_knob_validation():
    """Retention score knobs are checked on the host: unknown score, alpha
    outside [0, 1], pool ratios above 1; the key-norm + confidence score adds
    the LM-head partials of an append chunk to the workspace, and one-pool
    retention a compacted copy of the retained K/V; the retention check
    rejects pools without both ratios before any launch."""
    from masked_block_diffusion_amd import binding as B
    _, c, g = _structs(use_sprint=True, keep_ratio=0.5)
    base = B.dllm_workspace_bytes(c, g)
    assert base > 0
    g.retention_score = 2
    assert B.dllm_workspace_bytes(c, g) == 0
    g.retention_score = B.DLLM_RETAIN_KEYNORM_CONF
    g.retention_alpha = 1.5
    assert B.dllm_workspace_bytes(c, g) == 0
    g.retention_alpha = 0.5
    ws_kc = B.dllm_workspace_bytes(c, g)
    assert ws_kc > base
    g.image_keep_ratio = 1.5
    assert B.dllm_workspace_bytes(c, g) == 0
    g.image_keep_ratio, g.text_keep_ratio = 0.8, 1.0
    # per-modality pools keep different counts per row and gather them by
    # index: no compacted copy of the retained K/V, which one pool holds
    assert 0 < B.dllm_workspace_bytes(c, g) < ws_kc
    assert B.dllm_debug_retention(0x1000, 1, 10, 0.5, 0x2000, 0, 5, 0.0, 1.0, 0x3000, 0x4000, 0) == \
        B.DLLM_ERR_INVALID_ARG
    assert B.dllm_debug_retention(0x1000, 1, 10, 0.0, 0, 0, 5, 0.8, 1.0, 0x3000, 0x4000, 0) == \
        B.DLLM_ERR_INVALID_ARG


def test_three_way_guidance_validation():
    """Three-way guidance triples the model rows (KV cache), excludes two-way CFG and needs a finite image scale >= 0."""
    from masked_block_diffusion_amd import binding as B
    _, c, g = _structs()
    kv1 = B.dllm_kv_bytes(c, g)
    g.cfg_text_scale, g.cfg_image_scale = 4.0, 1.5
    assert B.dllm_kv_bytes(c, g) == 3 * kv1
    assert B.dllm_workspace_bytes(c, g) > 0      # append chunks shrink to R x tokens <= 512
    g.cfg_scale = 2.0
    assert B.dllm_workspace_bytes(c, g) == 0
    g.cfg_scale = 0.0
    g.cfg_image_scale = -1.0
    assert B.dllm_workspace_bytes(c, g) == 0
    g.cfg_image_scale = float("inf")
    assert B.dllm_workspace_bytes(c, g) == 0


def test_pack_gate_up_validation():
    """The repack call checks its pointers (null, aliasing or overlapping
    buffers) and the shape on the host."""
    from masked_block_diffusion_amd import binding as B
    _, c, g = _structs()
    nbytes = c.n_layers * c.n_experts * c.expert_ffn * c.hidden * 2
    assert B.dllm_pack_gate_up(c, 0, 0x2000, 0) == B.DLLM_ERR_INVALID_ARG
    assert B.dllm_pack_gate_up(c, 0x1000, 0x1000, 0) == B.DLLM_ERR_INVALID_ARG
    assert B.dllm_pack_gate_up(c, 0x100000, 0x100000 + nbytes // 2, 0) == B.DLLM_ERR_INVALID_ARG
    c.expert_ffn = 40
    assert B.dllm_pack_gate_up(c, 0x100000, 0x100000 + 4 * nbytes, 0) == B.DLLM_ERR_INVALID_ARG
    c.expert_ffn, c.hidden, c.expert_dtype = 512, 96, B.DLLM_FP8_E4M3   # fp8 fragments: 64-wide
    assert B.dllm_pack_gate_up(c, 0x100000, 0x100000 + 4 * nbytes, 0) == B.DLLM_ERR_INVALID_ARG
