"""C-ABI behaviour on the GPU: call order, capacity errors, determinism."""
import numpy as np
import pytest

import dllm_inputs as di

pytestmark = pytest.mark.gpu


def test_errors_and_determinism():
    import torch
    from masked_block_diffusion_amd import binding as B
    wl = di.workload("small_sprint")
    w = di.make_weights(wl.model, 5)
    s = B.Session(wl, w, max_prefix=wl.prefix_len + 32)
    ids = s.ids_tensor(np.full((1, 32), wl.model.mask_id, np.int32))
    with pytest.raises(B.DllmError) as e:
        s.denoise_step(0, ids)
    assert e.value.status == B.DLLM_ERR_BAD_STATE
    with pytest.raises(B.DllmError) as e:
        s.block_init(di.make_prefix(wl, 5)[:, :40])
    assert e.value.status == B.DLLM_ERR_INVALID_ARG
    s.block_init(di.make_prefix(wl, 5))
    with pytest.raises(B.DllmError) as e:
        s.denoise_step(1, ids)                 # retained step before the warm-up step
    assert e.value.status == B.DLLM_ERR_BAD_STATE
    with pytest.raises(B.DllmError) as e:
        s.denoise_step(wl.gen.steps, ids)
    assert e.value.status == B.DLLM_ERR_INVALID_ARG
    a = s.denoise_step(0, ids, torch.empty_like(ids)).cpu().numpy()
    h1 = s.debug(B.DEBUG_HIDDEN)
    b = s.denoise_step(0, ids, torch.empty_like(ids)).cpu().numpy()
    h2 = s.debug(B.DEBUG_HIDDEN)
    assert np.array_equal(a, b) and np.array_equal(h1, h2)     # bit-identical reruns
    s.block_init(np.zeros((1, 32), np.int32))
    with pytest.raises(B.DllmError) as e:
        s.block_init(np.zeros((1, 32), np.int32))   # capacity exceeded
    assert e.value.status == B.DLLM_ERR_OUT_OF_MEMORY
    s.close()
