"""dllm_create_static (workspace in the library's static device array, for
callers that cannot allocate) against dllm_create with a caller workspace:
the same steps through the C ABI give the same outputs, on two contexts in a
row, the second with a smaller input (its state must not leak from the first
one's contents of the shared array)."""
import numpy as np
import pytest

import dllm_inputs as di
from masked_block_diffusion_amd import binding as B

pytestmark = pytest.mark.gpu


def _run(wl, w, prefix, block, steps, static):
    import torch
    s = B.Session(wl, w, static_scratch=static)
    assert (s.ws is None) == static
    s.block_init(prefix)
    ids = s.ids_tensor(block)
    hs, confs = [], []
    for t in range(steps):
        nxt = torch.empty_like(ids)
        s.denoise_step(t, ids, nxt)
        torch.cuda.synchronize()
        hs.append(s.debug(B.DEBUG_HIDDEN, 0, np.float32))
        confs.append(s.debug(B.DEBUG_CONF, 0, np.float32))
        ids = nxt
    out = (ids.cpu().numpy(), s.remaining.cpu().numpy(), hs, confs)
    s.close()
    return out


@pytest.mark.parametrize("name,n_seq,prefix_len,steps", [("small_sprint", 4, 256, 3), ("small_sprint", 1, 64, 3)])
def test_static_scratch_matches_caller_workspace(name, n_seq, prefix_len, steps):
    """SPRINT retention and threshold mode (state kept in the workspace across
    steps), batch 4 with a 256-token prefix, then batch 1 with a 64-token one:
    committed ids, remaining counts, hidden states and confidences are
    bit-identical to the caller-workspace path (same kernels, same order)."""
    wl = di.workload(name)
    wl.gen.n_seq = n_seq
    wl.prefix_len = prefix_len
    w = di.make_weights(wl.model, 21)
    prefix, block = di.make_prefix(wl, 21), di.make_block(wl, 21)
    ref = _run(wl, w, prefix, block, steps, static=False)
    got = _run(wl, w, prefix, block, steps, static=True)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    for a, b in zip(got[2] + got[3], ref[2] + ref[3]):
        assert np.array_equal(a, b)


def test_static_scratch_rejects_large_shapes():
    """A 1024-token prefill chunk at hidden 2048 needs 248 MiB of workspace:
    rejected before any HIP call with DLLM_ERR_OUT_OF_MEMORY."""
    wl = di.workload("layer_bf16")
    c = B.model_config_struct(wl.model)
    g = B.gen_params_struct(wl.gen, 1056, 1024)
    assert B.dllm_workspace_bytes(c, g) > 64 << 20
    st, ctx = B.dllm_create_static(c, g, B.dllm_weights(), B.dllm_kv_cache(), 0)
    assert st == B.DLLM_ERR_OUT_OF_MEMORY and not ctx.value
