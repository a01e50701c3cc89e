"""Python-side plumbing around libswiftkv: build a model from seeded weights,
put a batch in device memory, call skv_prefill, read the paged KV cache back
in logical order.  PyTorch provides device memory and streams only; all
arithmetic of the path runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from . import _lib as L

_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        # by soname, so the runtime already mapped (torch's, see _lib.lib)
        # is the one returned rather than a second copy
        L.lib()
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    return _hip


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("no HIP device visible to torch")
    return torch


def config_from(shape, dtype: str, l: int, g: int, max_tokens: int, max_batch: int, max_seqlen: int,
                kv_fp8: bool = False):
    return L.make_config(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                         shape.ffn_dim, shape.vocab, shape.rope_theta, shape.rms_eps, l, g,
                         L.SKV_BF16 if dtype == "bf16" else L.SKV_FP32, max_tokens, max_batch, max_seqlen,
                         L.SKV_KV_FP8 if kv_fp8 else L.SKV_KV_MODEL)


class Model:
    """Owns an skv_model handle."""

    def __init__(self, cfg: L.skv_model_config):
        self.cfg = cfg
        self.handle = L.skv_model_create(cfg)

    def load_globals(self, embed, final_norm, lm_head):
        L.skv_model_load_globals(self.handle, embed, final_norm, lm_head)

    def load_layer(self, layer: int, w: Dict[str, np.ndarray]):
        L.skv_model_load_layer(self.handle, layer, w)

    @property
    def num_kv_slots(self) -> int:
        return L.skv_num_kv_slots(self.handle)

    def close(self):
        if self.handle:
            L.skv_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def load_seeded_model(workload, max_tokens: int, max_batch: int, max_seqlen: int, layer_hook=None,
                      kv_fp8: bool = False) -> Model:
    """Create a model for `workload` and load its seeded weights layer by layer.

    layer_hook(i, weights) (optional) sees each layer's host arrays after
    they were loaded (used to stream the same arrays to the oracle).
    """
    import skv_inputs as si
    s = workload.shape
    cfg = config_from(s, workload.dtype, workload.swiftkv_l, workload.acrosskv_g, max_tokens, max_batch, max_seqlen,
                      kv_fp8)
    m = Model(cfg)
    gw = si.global_weights(s, workload.dtype)
    m.load_globals(gw["embed"], gw["final_norm"], gw["lm_head"])
    del gw
    for i in range(1, s.n_layers + 1):
        w = si.layer_weights(s, i, workload.dtype)
        m.load_layer(i, w)
        if layer_hook is not None:
            layer_hook(i, w)
    return m


class Cache:
    """Owns an skv_kv_cache handle."""

    def __init__(self, model: Model, num_blocks: int, block_size: int = 16):
        self.model = model
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.handle = L.skv_kv_cache_create(model.handle, num_blocks, block_size)

    def view(self, layer: int):
        return L.skv_kv_cache_view(self.handle, layer)

    def _copy_view(self, v: L.skv_tensor_view):
        torch = _torch()
        shape = tuple(v.shape[i] for i in range(v.ndim))
        dt = {L.SKV_BF16: torch.uint16, L.SKV_FP32: torch.float32, L.SKV_FP8_E4M3: torch.uint8}[v.dtype]
        t = torch.empty(shape, dtype=dt, device="cuda")
        nbytes = t.numel() * t.element_size()
        torch.cuda.synchronize()
        rc = _hiprt().hipMemcpy(t.data_ptr(), v.data, nbytes, 3)  # device to device
        if rc != 0:
            raise RuntimeError(f"hipMemcpy failed ({rc})")
        return t.view(torch.bfloat16) if v.dtype == L.SKV_BF16 else t

    def read_layer(self, layer: int):
        """Device copies of (K, V) of a layer, each [num_blocks, hkv, block_size, dh]; an FP8 cache's values are
        decoded (code value times the position's scale, fp32)."""
        k, v = self.view(layer)
        kt, vt = self._copy_view(k), self._copy_view(v)
        if k.dtype != L.SKV_FP8_E4M3:
            return kt, vt
        torch = _torch()
        ks, vs = (self._copy_view(x) for x in L.skv_kv_cache_scales(self.handle, layer))

        def dec(codes, sc):
            val = codes.cpu().view(torch.float8_e4m3fn).float()              # E4M3 values (host conversion)
            return (val * sc.cpu()[:, None, :, None]).to(codes.device)
        return dec(kt, ks), dec(vt, vs)

    def read_codes(self, layer: int):
        """Host copies of an FP8 cache layer: (K codes, V codes) uint8 [num_blocks, hkv, block_size, dh] and
        (K scales, V scales) fp32 [num_blocks, block_size]."""
        k, v = self.view(layer)
        ks, vs = L.skv_kv_cache_scales(self.handle, layer)
        return tuple(self._copy_view(x).cpu().numpy() for x in (k, v, ks, vs))

    def close(self):
        if self.handle:
            L.skv_kv_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def logical_kv(kt, vt, block_row: np.ndarray, n: int):
    """Gather one prompt's K/V in position order: ([n, hkv, dh], [n, hkv, dh]) fp32 on the host."""
    torch = _torch()
    bs = kt.shape[2]
    nb = -(-n // bs)
    idx = torch.as_tensor(np.asarray(block_row[:nb], dtype=np.int64), device=kt.device)
    k = kt.index_select(0, idx).permute(0, 2, 1, 3).reshape(nb * bs, kt.shape[1], kt.shape[3])[:n]
    v = vt.index_select(0, idx).permute(0, 2, 1, 3).reshape(nb * bs, vt.shape[1], vt.shape[3])[:n]
    return k.float().cpu().numpy(), v.float().cpu().numpy()


@dataclass
class DeviceBatch:
    batch: object                 # skv_inputs.Batch
    token_ids: object             # torch int32 cuda
    cu_dev: object
    bt_dev: object
    cu_host: np.ndarray
    bt_host: np.ndarray
    struct: L.skv_batch


def device_batch(batch) -> DeviceBatch:
    torch = _torch()
    cu = np.ascontiguousarray(batch.cu_seqlens, dtype=np.int32)
    bt = np.ascontiguousarray(batch.block_tables, dtype=np.int32)
    tok = torch.as_tensor(batch.token_ids, dtype=torch.int32).cuda()
    cu_d = torch.as_tensor(cu).cuda()
    bt_d = torch.as_tensor(bt.reshape(-1)).cuda()
    st = L.skv_batch(len(batch.lengths), batch.total_tokens, batch.max_seqlen, bt.shape[1], cu.ctypes.data,
                     bt.ctypes.data, tok.data_ptr(), cu_d.data_ptr(), bt_d.data_ptr())
    return DeviceBatch(batch, tok, cu_d, bt_d, cu, bt, st)


def prefill(model: Model, cache: Cache, db: DeviceBatch, logits=None, stream=None):
    """Enqueue skv_prefill on `stream` (torch stream; default = current) and return the logits tensor."""
    torch = _torch()
    B = db.struct.batch
    if logits is None:
        logits = torch.empty((B, model.cfg.vocab), dtype=torch.float32, device="cuda")
    s = stream if stream is not None else torch.cuda.current_stream()
    L.skv_prefill(model.handle, cache.handle, db.struct, logits.data_ptr(), s.cuda_stream)
    return logits


@dataclass
class DeviceStep:
    """A mixed batch in device memory: new tokens per sequence plus cached lengths."""
    tokens: DeviceBatch
    ctx_dev: object
    ctx_host: np.ndarray
    struct: L.skv_step_batch
    need_host: object = None


def device_step(token_ids, new_lens, ctx_lens, block_tables, need_logits=None) -> DeviceStep:
    """Device copies of a step batch: sequence b brings new_lens[b] of the
    packed token_ids after ctx_lens[b] cached positions; block_tables [B, m].
    need_logits (optional, [B]): 0 for a prompt chunk that more chunks follow;
    a call with no nonzero entry writes no logits."""
    torch = _torch()
    new_lens = np.asarray(new_lens, dtype=np.int32)
    cu = np.zeros(len(new_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(new_lens)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    tok = torch.as_tensor(np.asarray(token_ids, dtype=np.int32)).cuda()
    cu_d = torch.as_tensor(cu).cuda()
    bt_d = torch.as_tensor(bt.reshape(-1)).cuda()
    ctx_d = torch.as_tensor(ctx).cuda()
    inner = L.skv_batch(len(new_lens), int(cu[-1]), int(new_lens.max()), bt.shape[1], cu.ctypes.data, bt.ctypes.data,
                        tok.data_ptr(), cu_d.data_ptr(), bt_d.data_ptr())
    db = DeviceBatch(None, tok, cu_d, bt_d, cu, bt, inner)
    need = None if need_logits is None else np.ascontiguousarray(need_logits, dtype=np.int32)
    st = L.skv_step_batch(inner, ctx.ctypes.data, ctx_d.data_ptr(), need.ctypes.data if need is not None else None)
    return DeviceStep(db, ctx_d, ctx, st, need)


def step(model: Model, cache: Cache, ds: DeviceStep, logits=None, stream=None):
    """Enqueue skv_step on `stream` (torch stream; default = current) and return the logits tensor."""
    torch = _torch()
    B = ds.struct.tokens.batch
    if logits is None:
        logits = torch.empty((B, model.cfg.vocab), dtype=torch.float32, device="cuda")
    s = stream if stream is not None else torch.cuda.current_stream()
    L.skv_step(model.handle, cache.handle, ds.struct, logits.data_ptr(), s.cuda_stream)
    return logits
