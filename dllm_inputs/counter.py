"""Counter-based seeded weights (input preparation only; none of the
denoising step's arithmetic).

The generator is Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror,
D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten
rounds of two 32x32 -> 64-bit products on a 128-bit counter under a 64-bit
key that is advanced by a Weyl sequence between rounds.  Every value is a
pure function of (seed, tensor tag, layer, expert, element index), so a large
model can be generated on the GPU (``dllm_inputs/csrc/gen_inputs.hip``) and
any part of it again on the host, bit for bit, with this module.

Streams: key = (seed, tag * 65536 + layer); counter = (j mod 2^32, j div 2^32,
expert, 0) for the j-th pair of elements of one matrix (one matrix per
(tag, layer, expert); dense tensors use expert 0).  Output words (w0, w1)
give element 2j, (w2, w3) element 2j + 1.

Values: a weight is the sum of four 16-bit uniforms centred on zero (the
Irwin-Hall distribution of order 4: bell-shaped, variance 4 (2^32 - 1) / 12,
bounded at 3.46 standard deviations), times one float32 constant that sets
the standard deviation (0.02); the integer is exact in float32 and the product
is one rounding, so every platform produces the same bits.  A uniform value
in [-h, h) is (w0 >> 8) - 2^23 times h / 2^23 in float32.  Storage formats
(float32, bfloat16, E4M3FN codes with per-row scales) are those of
``dllm_inputs``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint32(0x9E3779B9), np.uint32(0xBB67AE85)
_LO32 = np.uint64(0xFFFFFFFF)

TAGS = {"embed": 1, "w_qkv": 3, "w_o": 4, "w_router": 6, "router_bias": 7, "w_gate": 8, "w_up": 9,
        "w_down": 10, "ws_gate": 11, "ws_up": 12, "ws_down": 13, "lm_head": 15}

# standard deviation of the centred sum of four 16-bit uniforms
IH_SD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on uint32 counter arrays (broadcast) and a scalar key."""
    c0, c1, c2, c3 = (np.asarray(x, np.uint32) for x in (c0, c1, c2, c3))
    k0, k1 = np.uint32(k0), np.uint32(k1)
    for _ in range(10):
        p0 = c0.astype(np.uint64) * _M0
        p1 = c2.astype(np.uint64) * _M1
        hi0, lo0 = (p0 >> np.uint64(32)).astype(np.uint32), (p0 & _LO32).astype(np.uint32)
        hi1, lo1 = (p1 >> np.uint64(32)).astype(np.uint32), (p1 & _LO32).astype(np.uint32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = np.uint32((int(k0) + int(_W0)) & 0xFFFFFFFF)
        k1 = np.uint32((int(k1) + int(_W1)) & 0xFFFFFFFF)
    return c0, c1, c2, c3


def scale_for(std: float) -> np.float32:
    """The float32 factor that gives the Irwin-Hall sums standard deviation std."""
    return np.float32(std / IH_SD)


def _ih(a, b):
    s = (a & np.uint32(0xFFFF)).astype(np.int32) + (a >> np.uint32(16)).astype(np.int32)
    s += (b & np.uint32(0xFFFF)).astype(np.int32) + (b >> np.uint32(16)).astype(np.int32)
    return s - np.int32(131070)


def normal(seed, tag, layer, expert, n, std=0.02, start=0):
    """Elements [start, start + n) of the (seed, tag, layer, expert) stream as
    float32 (start even)."""
    assert start % 2 == 0
    j = np.arange(start // 2, (start + n + 1) // 2, dtype=np.uint64)
    w0, w1, w2, w3 = philox4x32_10((j & _LO32).astype(np.uint32), (j >> np.uint64(32)).astype(np.uint32),
                                   np.uint32(expert), np.uint32(0), seed, TAGS[tag] * 65536 + layer)
    out = np.empty(2 * len(j), np.float32)
    k = scale_for(std)
    out[0::2] = _ih(w0, w1).astype(np.float32) * k
    out[1::2] = _ih(w2, w3).astype(np.float32) * k
    return out[:n]


def uniform(seed, tag, layer, n, half):
    """n float32 values in [-half, half) of the (seed, tag, layer, 0) stream,
    one per counter."""
    j = np.arange(n, dtype=np.uint64)
    w0, _, _, _ = philox4x32_10((j & _LO32).astype(np.uint32), (j >> np.uint64(32)).astype(np.uint32),
                                np.uint32(0), np.uint32(0), seed, TAGS[tag] * 65536 + layer)
    return ((w0 >> np.uint32(8)).astype(np.int32) - np.int32(1 << 23)).astype(np.float32) * np.float32(half / 2 ** 23)


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def make_weights_counter(m, seed: int = 0, layers=None) -> dict:
    """All weights of model m in storage format, from the counter streams: the
    same dictionary layout as ``dllm_inputs.make_weights`` (see there), and
    the same bits as the GPU generator.  ``layers`` restricts the per-layer
    tensors to those layer indices (others None)."""
    from dllm_inputs import f32_to_bf16_bits, quantize_rows_e4m3fn
    D, H, dh, E, F, Fs = m.hidden, m.n_heads, m.head_dim, m.n_experts, m.expert_ffn, m.shared_ffn
    L = m.n_layers
    ad, ed = m.act_dtype, m.expert_dtype
    want = list(range(L)) if layers is None else list(layers)

    def store(x, dt):
        return np.ascontiguousarray(x, np.float32) if dt == "f32" else f32_to_bf16_bits(x)

    def dense(tag, l, shape):
        return store(normal(seed, tag, l, 0, int(np.prod(shape))).reshape(shape), ad)

    w = {"dtypes": {"dense": ad, "expert": ed}}
    w["embed"] = dense("embed", 0, (m.vocab + 1, D))
    w["lm_head"] = dense("lm_head", 0, (m.vocab, D))
    w["final_norm"] = np.ones(D, np.float32)

    def per_layer(fn):
        out = [None] * L
        for l in want:
            out[l] = fn(l)
        return np.stack(out) if layers is None else out

    w["attn_norm"] = per_layer(lambda l: np.ones(D, np.float32))
    w["moe_norm"] = per_layer(lambda l: np.ones(D, np.float32))
    w["w_qkv"] = per_layer(lambda l: dense("w_qkv", l, (3 * H * dh, D)))
    w["w_o"] = per_layer(lambda l: dense("w_o", l, (D, H * dh)))
    w["w_router"] = per_layer(lambda l: dense("w_router", l, (E, D)))
    w["router_bias"] = per_layer(lambda l: uniform(seed, "router_bias", l, E, 0.1))

    def experts(tag, rows, cols, l):
        vals = np.empty((E, rows, cols), np.uint8 if ed == "fp8" else (np.float32 if ed == "f32" else np.uint16))
        scales = np.empty((E, rows), np.float32) if ed == "fp8" else None

        def one(e):
            x = normal(seed, tag, l, e, rows * cols).reshape(rows, cols)
            if ed == "fp8":
                vals[e], scales[e] = quantize_rows_e4m3fn(x)
            else:
                vals[e] = store(x, ed)

        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(one, range(E)))
        return vals, scales

    for tag, rows, cols, stag in (("w_gate", F, D, "s_gate"), ("w_up", F, D, "s_up"), ("w_down", D, F, "s_down")):
        vals, scales = [None] * L, [None] * L
        for l in want:
            vals[l], scales[l] = experts(tag, rows, cols, l)
        if layers is None:
            w[tag] = np.stack(vals)
            w[stag] = np.stack(scales) if ed == "fp8" else None
        else:
            w[tag], w[stag] = vals, (scales if ed == "fp8" else None)
    if m.n_shared:
        w["ws_gate"] = per_layer(lambda l: dense("ws_gate", l, (Fs, D)))
        w["ws_up"] = per_layer(lambda l: dense("ws_up", l, (Fs, D)))
        w["ws_down"] = per_layer(lambda l: dense("ws_down", l, (D, Fs)))
    else:
        w["ws_gate"] = w["ws_up"] = w["ws_down"] = None
    return w
