"""ctypes binding of libswiftkv (include/swiftkv.h): argument marshalling only.

Every computation runs in the HIP library.  If the library has not been
built this module raises on first use; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_float, c_int32, c_int64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libswiftkv.so")

SKV_OK, SKV_ERR_INVALID_ARG, SKV_ERR_OOM, SKV_ERR_HIP, SKV_ERR_UNSUPPORTED = 0, -1, -2, -3, -4
SKV_BF16, SKV_FP32, SKV_FP8_E4M3 = 0, 1, 2
SKV_KV_MODEL, SKV_KV_FP8 = 0, 1
(SKV_K_GEMM_QKV, SKV_K_ATTN_PREFILL, SKV_K_GEMM_O, SKV_K_GEMM_GATEUP, SKV_K_GEMM_DOWN, SKV_K_GEMM_KVSKIP,
 SKV_K_RMSNORM, SKV_K_LAST_TOKEN, SKV_K_ATTN_PREFILL_SPLIT) = range(9)
KERNEL_CLASS_NAMES = ["gemm_qkv", "attn_prefill", "gemm_o", "gemm_gateup", "gemm_down", "gemm_kvskip", "rmsnorm",
                      "last_token", "attn_prefill_split"]


class skv_model_config(Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn_dim", c_int32), ("vocab", c_int32), ("rope_theta", c_float),
                ("rms_eps", c_float), ("swiftkv_l", c_int32), ("acrosskv_g", c_int32), ("dtype", c_int32),
                ("max_tokens", c_int32), ("max_batch", c_int32), ("max_seqlen", c_int32), ("kv_dtype", c_int32)]


class skv_layer_weights(Structure):
    _fields_ = [(n, c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up",
                                         "w_down")]


class skv_tensor_view(Structure):
    _fields_ = [("data", c_void_p), ("dtype", c_int32), ("ndim", c_int32), ("shape", c_int64 * 4),
                ("stride", c_int64 * 4)]


class skv_batch(Structure):
    _fields_ = [("batch", c_int32), ("total_tokens", c_int32), ("max_seqlen", c_int32),
                ("max_blocks_per_seq", c_int32), ("cu_seqlens_host", c_void_p), ("block_tables_host", c_void_p),
                ("token_ids", c_void_p), ("cu_seqlens", c_void_p), ("block_tables", c_void_p)]


class skv_step_batch(Structure):
    _fields_ = [("tokens", skv_batch), ("ctx_lens_host", c_void_p), ("ctx_lens", c_void_p),
                ("need_logits_host", c_void_p)]


EXPORTED = ["skv_model_create", "skv_model_load_globals", "skv_model_load_layer", "skv_model_destroy",
            "skv_kv_cache_create", "skv_kv_cache_destroy", "skv_num_kv_slots", "skv_kv_cache_view", "skv_kv_cache_scales", "skv_prefill",
            "skv_step", "skv_step_noalloc",
            "skv_flops", "skv_profile_enable", "skv_profile_read", "skv_mfma_probe", "skv_last_error"]

_lib = None


class SkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"skv status {status}: {msg}")
        self.status = status


def lib():
    """Load libswiftkv.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m swiftkv_prefill_skipping_amd.build`")
        # One HIP runtime per process: the torch wheel bundles its own
        # libamdhip64.so.7 under the same soname as the system one this
        # library links, and whichever is mapped first serves both.  Torch
        # finds no device on a runtime other than its own, so it is loaded
        # first whenever it is installed.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        vp = c_void_p
        L.skv_model_create.argtypes = [POINTER(skv_model_config), POINTER(c_void_p)]
        L.skv_model_load_globals.argtypes = [vp, vp, vp, vp]
        L.skv_model_load_layer.argtypes = [vp, c_int32, POINTER(skv_layer_weights)]
        L.skv_model_destroy.argtypes = [vp]
        L.skv_model_destroy.restype = None
        L.skv_kv_cache_create.argtypes = [vp, c_int32, c_int32, POINTER(c_void_p)]
        L.skv_kv_cache_destroy.argtypes = [vp]
        L.skv_kv_cache_destroy.restype = None
        L.skv_num_kv_slots.argtypes = [vp]
        L.skv_num_kv_slots.restype = c_int32
        L.skv_kv_cache_view.argtypes = [vp, c_int32, POINTER(skv_tensor_view), POINTER(skv_tensor_view)]
        L.skv_kv_cache_scales.argtypes = [vp, c_int32, POINTER(skv_tensor_view), POINTER(skv_tensor_view)]
        L.skv_prefill.argtypes = [vp, vp, POINTER(skv_batch), vp, vp]
        L.skv_step.argtypes = [vp, vp, POINTER(skv_step_batch), vp, vp]
        L.skv_step_noalloc.argtypes = [vp, vp, POINTER(skv_step_batch), vp, vp]
        L.skv_flops.argtypes = [POINTER(skv_model_config), vp, c_int32, POINTER(c_double), POINTER(c_double)]
        L.skv_profile_enable.argtypes = [vp, c_int32, c_int32]
        L.skv_profile_read.argtypes = [vp, POINTER(c_double), POINTER(c_int64), POINTER(c_double), POINTER(c_double)]
        L.skv_mfma_probe.argtypes = [c_int32, c_int32, vp, POINTER(c_double), POINTER(c_double), POINTER(c_int32),
                                     POINTER(c_double)]
        L.skv_last_error.argtypes = []
        L.skv_last_error.restype = c_char_p
        for name in EXPORTED:
            f = getattr(L, name)
            if name not in ("skv_model_destroy", "skv_kv_cache_destroy", "skv_num_kv_slots", "skv_last_error"):
                f.restype = c_int32
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != SKV_OK:
        raise SkvError(status, lib().skv_last_error().decode())


def _ptr(a) -> int:
    """Address of a numpy array or torch tensor (host or device); None -> 0."""
    if a is None:
        return 0
    if hasattr(a, "data_ptr"):
        return a.data_ptr()
    return a.ctypes.data


def make_config(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, rope_theta, rms_eps, swiftkv_l,
                acrosskv_g, dtype, max_tokens, max_batch, max_seqlen, kv_dtype=SKV_KV_MODEL) -> skv_model_config:
    return skv_model_config(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, rope_theta, rms_eps,
                            swiftkv_l, acrosskv_g, dtype, max_tokens, max_batch, max_seqlen, kv_dtype)


def skv_model_create(cfg: skv_model_config) -> int:
    h = c_void_p()
    check(lib().skv_model_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h.value


def skv_model_load_globals(model: int, embed, final_norm, lm_head) -> None:
    check(lib().skv_model_load_globals(model, _ptr(embed), _ptr(final_norm), _ptr(lm_head)))


def skv_model_load_layer(model: int, layer: int, w: dict) -> None:
    s = skv_layer_weights(*[_ptr(w.get(n)) for n, _ in skv_layer_weights._fields_])
    check(lib().skv_model_load_layer(model, layer, ctypes.byref(s)))


def skv_model_destroy(model: int) -> None:
    lib().skv_model_destroy(model)


def skv_kv_cache_create(model: int, num_blocks: int, block_size: int = 16) -> int:
    h = c_void_p()
    check(lib().skv_kv_cache_create(model, num_blocks, block_size, ctypes.byref(h)))
    return h.value


def skv_kv_cache_destroy(cache: int) -> None:
    lib().skv_kv_cache_destroy(cache)


def skv_num_kv_slots(model: int) -> int:
    return lib().skv_num_kv_slots(model)


def skv_kv_cache_view(cache: int, layer: int):
    k, v = skv_tensor_view(), skv_tensor_view()
    check(lib().skv_kv_cache_view(cache, layer, ctypes.byref(k), ctypes.byref(v)))
    return k, v


def skv_kv_cache_scales(cache: int, layer: int):
    k, v = skv_tensor_view(), skv_tensor_view()
    check(lib().skv_kv_cache_scales(cache, layer, ctypes.byref(k), ctypes.byref(v)))
    return k, v


def skv_prefill(model: int, cache: int, batch: skv_batch, logits_ptr: int, stream: int = 0) -> None:
    check(lib().skv_prefill(model, cache, ctypes.byref(batch), logits_ptr, stream))


def skv_step(model: int, cache: int, batch: skv_step_batch, logits_ptr: int, stream: int = 0) -> None:
    check(lib().skv_step(model, cache, ctypes.byref(batch), logits_ptr, stream))


def skv_step_noalloc(model: int, cache: int, batch: skv_step_batch, logits_ptr: int, stream: int = 0) -> None:
    check(lib().skv_step_noalloc(model, cache, ctypes.byref(batch), logits_ptr, stream))


def skv_flops(cfg: skv_model_config, seqlens) -> tuple:
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    full, swift = c_double(), c_double()
    check(lib().skv_flops(ctypes.byref(cfg), arr.ctypes.data if arr.size else 0, int(arr.size), ctypes.byref(full),
                          ctypes.byref(swift)))
    return full.value, swift.value


def skv_profile_enable(model: int, kernel_class: int, enable: bool = True) -> None:
    check(lib().skv_profile_enable(model, kernel_class, 1 if enable else 0))


def skv_mfma_probe(random_operands: bool, iters: int, stream: int) -> dict:
    tf, mhz, cus, mx = c_double(), c_double(), c_int32(), c_double()
    check(lib().skv_mfma_probe(1 if random_operands else 0, iters, stream, ctypes.byref(tf), ctypes.byref(mhz),
                               ctypes.byref(cus), ctypes.byref(mx)))
    return {"tflops": tf.value, "clock_mhz": mhz.value, "cus": cus.value, "max_clock_mhz": mx.value}


def skv_profile_read(model: int) -> dict:
    t, n, fl, by = c_double(), c_int64(), c_double(), c_double()
    check(lib().skv_profile_read(model, ctypes.byref(t), ctypes.byref(n), ctypes.byref(fl), ctypes.byref(by)))
    return {"total_ms": t.value, "launches": n.value, "flops": fl.value, "bytes": by.value}
