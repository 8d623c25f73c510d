"""The counter streams of ``dllm_inputs.counter`` generated on the GPU
(libdllm_inputs.so, built from ``dllm_inputs/csrc/gen_inputs.hip``): a whole
model's seeded weights written straight into device memory, the same bits as
``counter.make_weights_counter`` on the host.  torch provides the memory."""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from dllm_inputs import counter as CT

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdllm_inputs.so")
_lib = None
ABI_VERSION = 2      # the entry points' signatures below; bumped with every change to them


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not built: run masked_block_diffusion_amd/build.py")
    lib = C.CDLL(path)
    if not hasattr(lib, "dllm_inputs_abi_version") or lib.dllm_inputs_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} was built from other sources than this module: rebuild it "
                          "(masked_block_diffusion_amd/build.py)")
    lib.dllm_inputs_normal.restype = C.c_int
    lib.dllm_inputs_normal.argtypes = [C.c_void_p, C.c_int, C.c_longlong, C.c_uint32, C.c_uint32, C.c_uint32,
                                       C.c_uint32, C.c_float, C.c_void_p]
    lib.dllm_inputs_normal_fp8.restype = C.c_int
    lib.dllm_inputs_normal_fp8.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_uint32,
                                           C.c_uint32, C.c_uint32, C.c_uint32, C.c_float, C.c_void_p]
    lib.dllm_inputs_uniform.restype = C.c_int
    lib.dllm_inputs_uniform.argtypes = [C.c_void_p, C.c_longlong, C.c_uint32, C.c_uint32, C.c_uint32, C.c_float,
                                        C.c_void_p]
    _lib = lib
    return lib


def _ok(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed ({st})")


def make_weights_device(m, seed: int = 0, device="cuda:0", stream=None) -> dict:
    """All weights of model m on `device`, as torch tensors named and laid out
    like ``Session.upload`` makes them (bfloat16 bits as int16, E4M3FN codes
    as uint8 with float32 row scales)."""
    import torch
    lib = load_library()
    dev = torch.device(device)
    st = (stream or torch.cuda.current_stream(dev)).cuda_stream
    D, H, dh, E, F, Fs, L = m.hidden, m.n_heads, m.head_dim, m.n_experts, m.expert_ffn, m.shared_ffn, m.n_layers
    k = float(CT.scale_for(0.02))
    ad, ed = m.act_dtype, m.expert_dtype
    tdt = {"f32": torch.float32, "bf16": torch.int16}

    def normal_into(t, tag, layer, expert):
        _ok(lib.dllm_inputs_normal(t.data_ptr(), 0 if t.dtype == torch.float32 else 1, t.numel(), seed,
                                   CT.TAGS[tag], layer, expert, k, st), tag)

    def dense(tag, per_layer_shape, layered=True):
        if not layered:
            t = torch.empty(per_layer_shape, dtype=tdt[ad], device=dev)
            normal_into(t, tag, 0, 0)
            return t
        t = torch.empty((L,) + per_layer_shape, dtype=tdt[ad], device=dev)
        for l in range(L):
            normal_into(t[l], tag, l, 0)
        return t

    w = {}
    w["embed"] = dense("embed", (m.vocab + 1, D), layered=False)
    w["lm_head"] = dense("lm_head", (m.vocab, D), layered=False)
    w["final_norm"] = torch.ones(D, dtype=torch.float32, device=dev)
    w["attn_norm"] = torch.ones((L, D), dtype=torch.float32, device=dev)
    w["moe_norm"] = torch.ones((L, D), dtype=torch.float32, device=dev)
    w["w_qkv"] = dense("w_qkv", (3 * H * dh, D))
    w["w_o"] = dense("w_o", (D, H * dh))
    w["w_router"] = dense("w_router", (E, D))
    rb = torch.empty((L, E), dtype=torch.float32, device=dev)
    for l in range(L):
        _ok(lib.dllm_inputs_uniform(rb[l].data_ptr(), E, seed, CT.TAGS["router_bias"], l,
                                    float(np.float32(0.1 / 2 ** 23)), st), "router_bias")
    w["router_bias"] = rb
    for tag, rows, cols, stag in (("w_gate", F, D, "s_gate"), ("w_up", F, D, "s_up"), ("w_down", D, F, "s_down")):
        if ed == "fp8":
            codes = torch.empty((L, E, rows, cols), dtype=torch.uint8, device=dev)
            scales = torch.empty((L, E, rows), dtype=torch.float32, device=dev)
            for l in range(L):
                _ok(lib.dllm_inputs_normal_fp8(codes[l].data_ptr(), scales[l].data_ptr(), rows, cols, E,
                                               seed, CT.TAGS[tag], l, 0, k, st), tag)
            w[tag], w[stag] = codes, scales
        else:
            t = torch.empty((L, E, rows, cols), dtype=tdt[ed], device=dev)
            for l in range(L):
                for e in range(E):
                    normal_into(t[l, e], tag, l, e)
            w[tag] = t
    if m.n_shared:
        w["ws_gate"] = dense("ws_gate", (Fs, D))
        w["ws_up"] = dense("ws_up", (Fs, D))
        w["ws_down"] = dense("ws_down", (D, Fs))
    return w
