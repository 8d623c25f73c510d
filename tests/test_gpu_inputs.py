"""The GPU input generator (libdllm_inputs.so) writes the same bits as its
host twin (dllm_inputs.counter): whole small models, and sampled matrices of
the 20-layer thinking model the bench runs."""
import numpy as np
import pytest

import dllm_inputs as di
from dllm_inputs import counter as CT

pytestmark = pytest.mark.gpu


def _host_view(t):
    import torch
    a = t.cpu()
    return a.numpy().view(np.uint16) if a.dtype == torch.int16 else a.numpy()


@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16", "small_fp8"])
def test_device_weights_equal_host_twin(name):
    from dllm_inputs import device as DV
    m = di.workload(name).model
    dev = DV.make_weights_device(m, 5)
    host = CT.make_weights_counter(m, 5)
    for k, v in host.items():
        if k == "dtypes" or v is None:
            continue
        assert np.array_equal(_host_view(dev[k]), v), k


def test_device_weights_thinking_model_sampled():
    """The 20-layer fp8-expert thinking model (17 GB): embedding and head rows,
    a dense tensor of the first and last layer, and expert matrices (codes
    and row scales) of experts 0 and 255 in layers 0 and 19."""
    import torch
    from dllm_inputs import device as DV
    m = di.workload("think_fp8").model
    dev = DV.make_weights_device(m, 0)
    torch.cuda.synchronize()
    D = m.hidden
    for tag, rows in (("embed", [0, 12345, m.vocab]), ("lm_head", [1, 157183, m.vocab - 1])):
        for r in rows:
            want = di.f32_to_bf16_bits(CT.normal(0, tag, 0, 0, D, start=r * D))
            assert np.array_equal(_host_view(dev[tag][r]), want), (tag, r)
    for l in (0, m.n_layers - 1):
        want = di.f32_to_bf16_bits(CT.normal(0, "w_o", l, 0, D * D).reshape(D, D))
        assert np.array_equal(_host_view(dev["w_o"][l]), want)
        assert np.array_equal(dev["router_bias"][l].cpu().numpy(), CT.uniform(0, "router_bias", l, m.n_experts, 0.1))
        for e in (0, m.n_experts - 1):
            for tag, stag, rows, cols in (("w_gate", "s_gate", m.expert_ffn, D), ("w_down", "s_down", D, m.expert_ffn)):
                codes, sc = di.quantize_rows_e4m3fn(CT.normal(0, tag, l, e, rows * cols).reshape(rows, cols))
                assert np.array_equal(dev[tag][l, e].cpu().numpy(), codes), (tag, l, e)
                assert np.array_equal(dev[stag][l, e].cpu().numpy(), sc), (stag, l, e)
