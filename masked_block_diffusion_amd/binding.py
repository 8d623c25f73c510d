"""ctypes binding of libdllm.so (include/dllm.h), same names as the C ABI.

Argument marshalling only.  ``Session`` below is a convenience that places the
seeded synthetic weights in device memory with torch (plumbing: allocation,
host->device copies, streams) and drives the library; every step of the
denoising path runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdllm.so")

DLLM_OK = 0
DLLM_ERR_INVALID_ARG = -1
DLLM_ERR_OUT_OF_MEMORY = -2
DLLM_ERR_HIP = -3
DLLM_ERR_BAD_STATE = -4
DLLM_ERR_UNSUPPORTED = -5
DLLM_F32, DLLM_BF16, DLLM_FP8_E4M3 = 0, 1, 2
DTYPE_CODE = {"f32": DLLM_F32, "bf16": DLLM_BF16, "fp8": DLLM_FP8_E4M3}

DEBUG_ROUTE_IDX, DEBUG_GATES, DEBUG_CONF, DEBUG_XHAT, DEBUG_MASS, DEBUG_KEPT, DEBUG_NKEPT, \
    DEBUG_HIDDEN, DEBUG_LOGITS, DEBUG_KNORM, DEBUG_PCONF, DEBUG_PIDS, DEBUG_ROUTER_Z, DEBUG_NORMED = range(14)
ATTN_FLOAT, ATTN_MFMA, ATTN_STREAM, ATTN_APPEND = 0, 1, 2, 3
DLLM_RETAIN_MASS, DLLM_RETAIN_KEYNORM_CONF = 0, 1


class dllm_model_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "hidden", "n_heads", "head_dim", "n_experts", "top_k", "n_shared",
        "expert_ffn", "shared_ffn", "vocab_text", "vocab_image")] + [
        ("rope_base", C.c_float), ("rms_eps", C.c_float),
        ("act_dtype", C.c_int32), ("expert_dtype", C.c_int32)]


class dllm_gen_params(C.Structure):
    _fields_ = [("block_length", C.c_int32), ("steps", C.c_int32), ("n_seq", C.c_int32),
                ("cfg_scale", C.c_float), ("vocab_lo", C.c_int32), ("vocab_hi", C.c_int32),
                ("confidence", C.c_int32), ("use_threshold", C.c_int32), ("threshold", C.c_float),
                ("use_sprint", C.c_int32), ("keep_ratio", C.c_float),
                ("cache_warmup_steps", C.c_int32), ("max_prefix", C.c_int32),
                ("max_clean_tokens", C.c_int32), ("retention_score", C.c_int32),
                ("retention_alpha", C.c_float), ("image_keep_ratio", C.c_float),
                ("text_keep_ratio", C.c_float), ("cfg_text_scale", C.c_float),
                ("cfg_image_scale", C.c_float)]


WEIGHT_NAMES = ("embed", "attn_norm", "w_qkv", "w_o", "moe_norm", "w_router", "router_bias", "w_gate",
                "w_up", "w_down", "s_gate", "s_up", "s_down", "ws_gate", "ws_up", "ws_down",
                "final_norm", "lm_head")


class dllm_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_NAMES] + [("gate_up_packed", C.c_int32)]


class dllm_kv_cache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p)]


_lib = None

_SIGS = {
    "dllm_workspace_bytes": (C.c_size_t, [C.POINTER(dllm_model_config), C.POINTER(dllm_gen_params)]),
    "dllm_kv_bytes": (C.c_size_t, [C.POINTER(dllm_model_config), C.POINTER(dllm_gen_params)]),
    "dllm_append_tokens": (C.c_int, [C.POINTER(dllm_model_config), C.POINTER(dllm_gen_params)]),
    "dllm_create": (C.c_int, [C.POINTER(C.c_void_p), C.POINTER(dllm_model_config),
                              C.POINTER(dllm_gen_params), C.POINTER(dllm_weights),
                              C.POINTER(dllm_kv_cache), C.c_void_p, C.c_size_t, C.c_void_p]),
    "dllm_create_static": (C.c_int, [C.POINTER(C.c_void_p), C.POINTER(dllm_model_config),
                                     C.POINTER(dllm_gen_params), C.POINTER(dllm_weights),
                                     C.POINTER(dllm_kv_cache), C.c_void_p]),
    "dllm_block_init": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32]),
    "dllm_denoise_step": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dllm_generate_block": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(C.c_int32)]),
    "dllm_prefix_length": (C.c_int32, [C.c_void_p]),
    "dllm_destroy": (None, [C.c_void_p]),
    "dllm_last_error": (C.c_char_p, [C.c_void_p]),
    "dllm_status_string": (C.c_char_p, [C.c_int]),
    "dllm_debug_buffer": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_void_p),
                                    C.POINTER(C.c_size_t)]),
    "dllm_debug_bytes": (C.c_size_t, [C.POINTER(dllm_model_config), C.POINTER(dllm_gen_params)]),
    "dllm_debug_attach": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t]),
    "dllm_debug_attn_plan": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32)]),
    "dllm_debug_block_attention": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                             C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                             C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                             C.c_void_p, C.POINTER(C.c_int32), C.c_void_p]),
    "dllm_debug_route": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                   C.c_void_p, C.c_void_p, C.c_void_p]),
    "dllm_debug_unmask": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                    C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                    C.c_int32, C.c_float, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_void_p]),
    "dllm_debug_retention": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_float, C.c_void_p,
                                       C.c_int32, C.c_int32, C.c_float, C.c_float, C.c_void_p,
                                       C.c_void_p, C.c_void_p]),
    "dllm_debug_decode_fp8": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]),
    "dllm_pack_gate_up": (C.c_int, [C.POINTER(dllm_model_config), C.c_void_p, C.c_void_p, C.c_void_p]),
    "dllm_profile_enable": (C.c_int, [C.c_void_p, C.c_int32]),
    "dllm_profile_read": (C.c_int, [C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_longlong)]),
}

PROF_GROUPS = ("expert_gateup", "expert_down", "attention", "qkv", "head")
PROF_ALL = (1 << len(PROF_GROUPS)) - 1

EXPORTED = tuple(_SIGS)


def load_library(path: str = LIB_PATH):
    """Load libdllm.so; raises if it is missing (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not built: run masked_block_diffusion_amd/build.py "
                          "(the HIP library is the only compute path)")
    lib = C.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


class DllmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _check(st, ctx=None, what=""):
    if st != DLLM_OK:
        lib = load_library()
        detail = lib.dllm_last_error(ctx).decode() if ctx else lib.dllm_status_string(st).decode()
        raise DllmError(st, f"{what}: {detail}")


# ---- thin wrappers with the ABI's names -----------------------------------

def dllm_workspace_bytes(cfg, gp):
    return load_library().dllm_workspace_bytes(C.byref(cfg), C.byref(gp))


def dllm_kv_bytes(cfg, gp):
    return load_library().dllm_kv_bytes(C.byref(cfg), C.byref(gp))


def dllm_append_tokens(cfg, gp):
    return load_library().dllm_append_tokens(C.byref(cfg), C.byref(gp))


def dllm_create(cfg, gp, w, kv, ws_ptr, ws_bytes, stream):
    out = C.c_void_p()
    st = load_library().dllm_create(C.byref(out), C.byref(cfg), C.byref(gp), C.byref(w),
                                    C.byref(kv), C.c_void_p(ws_ptr), ws_bytes, C.c_void_p(stream))
    return st, out


def dllm_create_static(cfg, gp, w, kv, stream):
    out = C.c_void_p()
    st = load_library().dllm_create_static(C.byref(out), C.byref(cfg), C.byref(gp), C.byref(w),
                                           C.byref(kv), C.c_void_p(stream))
    return st, out


def dllm_block_init(ctx, ids_ptr, n_clean):
    return load_library().dllm_block_init(ctx, C.c_void_p(ids_ptr), n_clean)


def dllm_denoise_step(ctx, t, ids_in, ids_out, remaining):
    return load_library().dllm_denoise_step(ctx, t, C.c_void_p(ids_in), C.c_void_p(ids_out),
                                            C.c_void_p(remaining))


def dllm_generate_block(ctx, ids_ptr):
    n = C.c_int32(0)
    st = load_library().dllm_generate_block(ctx, C.c_void_p(ids_ptr), C.byref(n))
    return st, n.value


def dllm_prefix_length(ctx):
    return load_library().dllm_prefix_length(ctx)


def dllm_destroy(ctx):
    load_library().dllm_destroy(ctx)


def dllm_last_error(ctx):
    return load_library().dllm_last_error(ctx).decode()


def dllm_status_string(st):
    return load_library().dllm_status_string(st).decode()


def dllm_debug_buffer(ctx, which, layer=0):
    p, n = C.c_void_p(), C.c_size_t()
    st = load_library().dllm_debug_buffer(ctx, which, layer, C.byref(p), C.byref(n))
    return st, p.value, n.value


def dllm_debug_bytes(cfg, gp):
    return load_library().dllm_debug_bytes(C.byref(cfg), C.byref(gp))


def dllm_debug_attach(ctx, buf_ptr, nbytes):
    return load_library().dllm_debug_attach(ctx, C.c_void_p(buf_ptr), nbytes)


def dllm_debug_attn_plan(ctx):
    a = (C.c_int32 * 3)()
    st = load_library().dllm_debug_attn_plan(ctx, a)
    return st, (a[0], a[1], a[2])


def dllm_debug_block_attention(act_dtype, q, kc, vc, cap, bk, bv, kept, n_kept, rows, n_heads, head_dim,
                               block_length, P, out, lse, stream):
    """Device pointers as ints (0 for NULL); returns (status, plan)."""
    a = (C.c_int32 * 3)()
    st = load_library().dllm_debug_block_attention(
        act_dtype, C.c_void_p(q), C.c_void_p(kc or None), C.c_void_p(vc or None), cap, C.c_void_p(bk),
        C.c_void_p(bv), C.c_void_p(kept or None), C.c_void_p(n_kept or None), rows, n_heads, head_dim,
        block_length, P, C.c_void_p(out), C.c_void_p(lse or None), a, C.c_void_p(stream))
    return st, (a[0], a[1], a[2])


def dllm_debug_route(logits_ptr, bias_ptr, n, E, k, idx_ptr, gates_ptr, stream):
    return load_library().dllm_debug_route(C.c_void_p(logits_ptr), C.c_void_p(bias_ptr), n, E, k,
                                           C.c_void_p(idx_ptr), C.c_void_p(gates_ptr),
                                           C.c_void_p(stream))


def dllm_debug_unmask(ids_in, logits, n_seq, LB, v_sub, vocab_lo, mask_id, steps, t, conf_strategy,
                      use_threshold, threshold, ids_out, remaining, conf, xhat, stream):
    return load_library().dllm_debug_unmask(
        C.c_void_p(ids_in), C.c_void_p(logits), n_seq, LB, v_sub, vocab_lo, mask_id, steps, t,
        conf_strategy, use_threshold, threshold, C.c_void_p(ids_out), C.c_void_p(remaining),
        C.c_void_p(conf), C.c_void_p(xhat), C.c_void_p(stream))


def dllm_debug_retention(score_ptr, rows, P, keep_ratio, ids_ptr, vis_lo, vis_hi,
                         image_keep_ratio, text_keep_ratio, kept_ptr, count_ptr, stream):
    return load_library().dllm_debug_retention(C.c_void_p(score_ptr), rows, P, keep_ratio,
                                               C.c_void_p(ids_ptr), vis_lo, vis_hi,
                                               image_keep_ratio, text_keep_ratio,
                                               C.c_void_p(kept_ptr), C.c_void_p(count_ptr),
                                               C.c_void_p(stream))


def dllm_pack_gate_up(cfg, src_ptr, dst_ptr, stream):
    return load_library().dllm_pack_gate_up(C.byref(cfg), C.c_void_p(src_ptr), C.c_void_p(dst_ptr),
                                            C.c_void_p(stream))


def dllm_debug_decode_fp8(codes_ptr, n, out_ptr, stream):
    return load_library().dllm_debug_decode_fp8(C.c_void_p(codes_ptr), n, C.c_void_p(out_ptr),
                                                C.c_void_p(stream))


def dllm_profile_enable(ctx, groups):
    """groups: bit mask over PROF_GROUPS (PROF_ALL for every group, 0 off)."""
    return load_library().dllm_profile_enable(ctx, int(groups))


def dllm_profile_read(ctx):
    n = len(PROF_GROUPS)
    ms = (C.c_double * n)()
    cnt = (C.c_longlong * n)()
    st = load_library().dllm_profile_read(ctx, ms, cnt)
    return st, {g: (ms[i], cnt[i]) for i, g in enumerate(PROF_GROUPS)}


# ---- structs from the seeded workload records ------------------------------

def model_config_struct(m) -> dllm_model_config:
    return dllm_model_config(m.n_layers, m.hidden, m.n_heads, m.head_dim, m.n_experts, m.top_k,
                             m.n_shared, m.expert_ffn, m.shared_ffn, m.vocab_text, m.vocab_image,
                             float(m.rope_base), float(m.rms_eps), DTYPE_CODE[m.act_dtype],
                             DTYPE_CODE[m.expert_dtype])


def gen_params_struct(g, max_prefix, max_clean) -> dllm_gen_params:
    return dllm_gen_params(g.block_length, g.steps, g.n_seq, float(g.cfg_scale), g.vocab_lo,
                           g.vocab_hi, g.confidence, int(g.use_threshold), float(g.threshold),
                           int(g.use_sprint), float(g.keep_ratio), g.cache_warmup_steps,
                           max_prefix, max_clean, int(g.retention_score), float(g.retention_alpha),
                           float(g.image_keep_ratio), float(g.text_keep_ratio),
                           float(g.cfg_text_scale), float(g.cfg_image_scale))


class Session:
    """Device-resident weights, KV cache and workspace for one workload, plus a
    library context.  torch provides the device memory and the stream."""

    def __init__(self, wl, weights: dict, max_prefix=None, max_clean=None, device="cuda:0",
                 stream=None, _device_weights=None, pack_gate_up=True, inspect=False,
                 static_scratch=False):
        import torch
        self.torch = torch
        self.wl = wl
        m, g = wl.model, wl.gen
        self.device = torch.device(device)
        bl = g.block_length
        self.max_prefix = max_prefix if max_prefix is not None else \
            wl.prefix_len + wl.n_blocks * bl
        self.max_clean = max_clean if max_clean is not None else max(wl.prefix_len, bl)
        self.cfg = model_config_struct(m)
        self.gp = gen_params_struct(g, self.max_prefix, self.max_clean)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.dev = _device_weights if _device_weights is not None else self.upload(weights, self.device)
        if pack_gate_up and not self.dev.get("_gate_up_packed"):
            # load-time repack of the routed gate/up weights (library kernel)
            for name in ("w_gate", "w_up"):
                src = self.dev[name]
                dst = torch.empty_like(src)
                _check(dllm_pack_gate_up(self.cfg, src.data_ptr(), dst.data_ptr(), self.stream.cuda_stream),
                       None, "dllm_pack_gate_up")
                self.stream.synchronize()
                self.dev[name] = dst
            self.dev["_gate_up_packed"] = True
        w = dllm_weights()
        for name in WEIGHT_NAMES:
            t = self.dev.get(name)
            setattr(w, name, t.data_ptr() if t is not None else None)
        w.gate_up_packed = 1 if self.dev.get("_gate_up_packed") else 0
        self.w = w
        kvb = dllm_kv_bytes(self.cfg, self.gp)
        wsb = dllm_workspace_bytes(self.cfg, self.gp)
        if wsb == 0:
            raise DllmError(DLLM_ERR_INVALID_ARG, "workspace size query rejected the shape")
        self.k_cache = torch.zeros(max(kvb, 1), dtype=torch.uint8, device=self.device)
        self.v_cache = torch.zeros(max(kvb, 1), dtype=torch.uint8, device=self.device)
        self.kv = dllm_kv_cache(self.k_cache.data_ptr(), self.v_cache.data_ptr())
        if static_scratch:
            # the library's static scratch (no workspace allocation)
            self.ws = None
            st, ctx = dllm_create_static(self.cfg, self.gp, self.w, self.kv, self.stream.cuda_stream)
            _check(st, None, "dllm_create_static")
        else:
            self.ws = torch.zeros(wsb + 256, dtype=torch.uint8, device=self.device)
            base = self.ws.data_ptr()
            self.ws_ptr = (base + 255) // 256 * 256
            st, ctx = dllm_create(self.cfg, self.gp, self.w, self.kv, self.ws_ptr, wsb,
                                  self.stream.cuda_stream)
            _check(st, None, "dllm_create")
        self.ctx = ctx
        self.remaining = torch.zeros(g.n_seq, dtype=torch.int32, device=self.device)
        self.dbg = None
        if inspect:
            # caller-owned inspection buffer: router logits of every layer and
            # the recomputed head logits (test support)
            nb = dllm_debug_bytes(self.cfg, self.gp)
            self.dbg = torch.zeros(nb + 256, dtype=torch.uint8, device=self.device)
            p = (self.dbg.data_ptr() + 255) // 256 * 256
            _check(dllm_debug_attach(self.ctx, p, nb), self.ctx, "dllm_debug_attach")

    @staticmethod
    def upload(weights: dict, device):
        import torch
        dev = {}
        for name, a in weights.items():
            if name == "dtypes" or a is None:
                continue
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                t = torch.from_numpy(a.view(np.int16))
            else:
                t = torch.from_numpy(a)
            dev[name] = t.to(device)
        return dev

    def close(self):
        if getattr(self, "ctx", None):
            dllm_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- calls --
    def ids_tensor(self, ids):
        return self.torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(self.device)

    def block_init(self, clean_ids):
        t = clean_ids if hasattr(clean_ids, "data_ptr") else self.ids_tensor(clean_ids)
        n = t.shape[1] if t.dim() == 2 else 0
        _check(dllm_block_init(self.ctx, t.data_ptr() if n else 0, n), self.ctx, "dllm_block_init")
        self._keep = t

    def denoise_step(self, t, ids_in, ids_out=None):
        ids_out = ids_in if ids_out is None else ids_out
        _check(dllm_denoise_step(self.ctx, t, ids_in.data_ptr(), ids_out.data_ptr(),
                                 self.remaining.data_ptr()), self.ctx, "dllm_denoise_step")
        return ids_out

    def generate_block(self, ids):
        st, n = dllm_generate_block(self.ctx, ids.data_ptr())
        _check(st, self.ctx, "dllm_generate_block")
        return n

    @property
    def append_tokens(self):
        return dllm_append_tokens(self.cfg, self.gp)

    @property
    def prefix_length(self):
        return dllm_prefix_length(self.ctx)

    def attn_plan(self):
        """(kernel, keys per workgroup, workgroups per unit) of the last pass."""
        st, p = dllm_debug_attn_plan(self.ctx)
        _check(st, self.ctx, "dllm_debug_attn_plan")
        return p

    def debug(self, which, layer=0, dtype=np.float32, shape=None):
        """Copy an internal buffer to the host (synchronises the stream)."""
        st, ptr, n = dllm_debug_buffer(self.ctx, which, layer)
        _check(st, self.ctx, "dllm_debug_buffer")
        self.stream.synchronize()
        out = np.empty(n, dtype=np.uint8)
        if n:
            rc = _hip().hipMemcpy(C.c_void_p(out.ctypes.data), C.c_void_p(ptr), n, 2)
            if rc != 0:
                raise DllmError(DLLM_ERR_HIP, f"hipMemcpy failed ({rc})")
        a = out.view(dtype)
        return a if shape is None else a.reshape(shape)


_hiplib = None


def _hip():
    global _hiplib
    if _hiplib is None:
        _hiplib = C.CDLL("libamdhip64.so")
        _hiplib.hipMemcpy.restype = C.c_int
        _hiplib.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]
    return _hiplib
