"""Seeded synthetic inputs for the SwiftKV prefill: weights, prompts, paged block tables.

This module is shared by the oracle tests and by the HIP path's harness
(tests, ``bench.py``, ``__graft_entry__.smoke``).  It holds no part of the
method's arithmetic: it only produces numbers from seeds and describes the
workload shapes.  Both sides receive identical arrays from it.

Random numbers come from ``philox.c`` (Philox4x32-10 + Box-Muller), compiled
into ``libskv_inputs.so`` next to this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libskv_inputs.so")
_SRC_PATH = os.path.join(_HERE, "philox.c")
_lib = None


def build_lib(force: bool = True) -> str:
    """Compile philox.c into libskv_inputs.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", _SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, f64 = ctypes.c_uint64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.skvin_normal_f32.argtypes = [u64, u64, u64, f64, f64, vp]
        lib.skvin_normal_bf16.argtypes = [u64, u64, u64, f64, f64, vp]
        lib.skvin_uniform_f32.argtypes = [u64, u64, u64, f64, f64, vp]
        lib.skvin_uniform_bf16.argtypes = [u64, u64, u64, f64, f64, vp]
        lib.skvin_randint.argtypes = [u64, u64, u64, u64, vp]
        lib.skvin_raw.argtypes = [u64, u64, u64, vp]
        lib.skvin_philox4x32_10.argtypes = [vp, vp, vp]
        for f in (lib.skvin_normal_f32, lib.skvin_normal_bf16, lib.skvin_uniform_f32,
                  lib.skvin_uniform_bf16, lib.skvin_randint, lib.skvin_raw, lib.skvin_philox4x32_10):
            f.restype = None
        _lib = lib
    return _lib


# ----------------------------------------------------------------------------
# raw draws
# ----------------------------------------------------------------------------

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _load().skvin_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def normal(seed: int, stream: int, shape, mean: float = 0.0, std: float = 1.0, dtype: str = "fp32") -> np.ndarray:
    """N(mean, std) draws; dtype "fp32" -> float32, "bf16" -> uint16 bf16 bit patterns (RNE)."""
    n = int(np.prod(shape))
    if dtype == "fp32":
        out = np.empty(n, dtype=np.float32)
        _load().skvin_normal_f32(seed, stream, n, mean, std, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        _load().skvin_normal_bf16(seed, stream, n, mean, std, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def uniform(seed: int, stream: int, shape, lo: float, hi: float, dtype: str = "fp32") -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == "fp32":
        out = np.empty(n, dtype=np.float32)
        _load().skvin_uniform_f32(seed, stream, n, lo, hi, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        _load().skvin_uniform_bf16(seed, stream, n, lo, hi, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def randint(seed: int, stream: int, n: int, high: int) -> np.ndarray:
    """n integers uniform in [0, high)."""
    out = np.empty(n, dtype=np.int64)
    if n:
        _load().skvin_randint(seed, stream, n, high, out.ctypes.data)
    return out


def raw_words(seed: int, stream: int, index: int) -> np.ndarray:
    out = np.zeros(4, dtype=np.uint32)
    _load().skvin_raw(seed, stream, index, out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns, nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


# ----------------------------------------------------------------------------
# model / workload descriptions
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rope_theta: float
    rms_eps: float = 1e-5
    weight_seed: int = 1
    init_std: float = 0.02
    gain: str = "normal"          # "normal": 1 + N(0, init_std); "uniform": U(0.5, 1.5)

    @property
    def dq(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def dkv(self) -> int:
        return self.n_kv_heads * self.head_dim


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    dtype: str                    # "fp32" | "bf16"
    swiftkv_l: int
    acrosskv_g: int
    n_prompts: int
    len_lo: int
    len_hi: int
    input_seed: int
    shuffle_blocks: bool = False
    block_size: int = 16
    fixed_lengths: Optional[tuple] = None

    @property
    def n_groups(self) -> int:
        return -(-(self.shape.n_layers - self.swiftkv_l) // self.acrosskv_g)


TINY = ModelShape("tiny", 4, 256, 4, 2, 64, 688, 1024, 10000.0, weight_seed=1)
LLAMA8B = ModelShape("llama-3.1-8b-shape", 32, 4096, 32, 8, 128, 14336, 128256, 500000.0, weight_seed=8)
LLAMA70B = ModelShape("llama-3.1-70b-shape", 80, 8192, 64, 8, 128, 28672, 128256, 500000.0, weight_seed=70)

# The five workloads: tiny fp32 parity model; 8B-shape l=16 over 16 prompts of
# 500-1000 tokens; 8B-shape l=24 with 4-way AcrossKV over 32x1000; 70B-shape
# l=40 over 32x1000; 8B-shape l=16 over one 32768-token prompt in a shuffled
# paged cache.
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32_l2": Workload("tiny_fp32_l2", TINY, "fp32", 2, 1, 1, 128, 128, input_seed=1),
    "llama8b_l16_b16": Workload("llama8b_l16_b16", LLAMA8B, "bf16", 16, 1, 16, 500, 1000, input_seed=2),
    "llama8b_l24_g4_b32": Workload("llama8b_l24_g4_b32", LLAMA8B, "bf16", 24, 4, 32, 1000, 1000, input_seed=3),
    "llama70b_l40_b32": Workload("llama70b_l40_b32", LLAMA70B, "bf16", 40, 1, 32, 1000, 1000, input_seed=4),
    "llama8b_l16_long32k": Workload("llama8b_l16_long32k", LLAMA8B, "bf16", 16, 1, 1, 32768, 32768, input_seed=5,
                                    shuffle_blocks=True),
}
WORKLOAD_ORDER = ["tiny_fp32_l2", "llama8b_l16_b16", "llama8b_l24_g4_b32", "llama70b_l40_b32", "llama8b_l16_long32k"]

# stream ids: layer * 16 + kind; layer 0 holds the model-global tensors
K_ATTN_NORM, K_WQ, K_WK, K_WV, K_WO, K_FFN_NORM, K_WGATE, K_WUP, K_WDOWN = range(9)
K_EMBED, K_FINAL_NORM, K_LM_HEAD = 9, 10, 11
S_LENGTHS, S_TOKENS, S_BLOCKS = 1, 2, 3

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def layer_tensor_shapes(s: ModelShape) -> Dict[str, tuple]:
    d = s.d_model
    return {
        "attn_norm": (d,), "wq": (s.dq, d), "wk": (s.dkv, d), "wv": (s.dkv, d), "wo": (d, s.dq),
        "ffn_norm": (d,), "w_gate": (s.ffn_dim, d), "w_up": (s.ffn_dim, d), "w_down": (d, s.ffn_dim),
    }


def _gain(s: ModelShape, stream: int, n: int, dtype: str) -> np.ndarray:
    if s.gain == "normal":
        return normal(s.weight_seed, stream, (n,), 1.0, s.init_std, dtype)
    if s.gain == "uniform":
        return uniform(s.weight_seed, stream, (n,), 0.5, 1.5, dtype)
    raise ValueError(s.gain)


def layer_weights(s: ModelShape, layer: int, dtype: str) -> Dict[str, np.ndarray]:
    """Weights of 1-based ``layer`` in torch Linear layout [out, in].

    dtype "bf16" returns uint16 bit patterns, "fp32" returns float32.  Linear
    weights ~ N(0, init_std); RMSNorm gains per ``s.gain``.
    """
    if not 1 <= layer <= s.n_layers:
        raise ValueError(f"layer {layer} outside 1..{s.n_layers}")
    shapes = layer_tensor_shapes(s)
    out = {}
    for kind, name in enumerate(LAYER_TENSORS):
        stream = layer * 16 + kind
        shp = shapes[name]
        if name.endswith("norm"):
            out[name] = _gain(s, stream, shp[0], dtype)
        else:
            out[name] = normal(s.weight_seed, stream, shp, 0.0, s.init_std, dtype)
    return out


def global_weights(s: ModelShape, dtype: str) -> Dict[str, np.ndarray]:
    """Embedding [V, d], final norm gain [d], untied LM head [V, d]."""
    return {
        "embed": normal(s.weight_seed, K_EMBED, (s.vocab, s.d_model), 0.0, s.init_std, dtype),
        "final_norm": _gain(s, K_FINAL_NORM, s.d_model, dtype),
        "lm_head": normal(s.weight_seed, K_LM_HEAD, (s.vocab, s.d_model), 0.0, s.init_std, dtype),
    }


def as_f32(a: np.ndarray) -> np.ndarray:
    return bf16_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


class CachedLayers:
    """Keeps each layer's generated arrays (bf16 bits or fp32) as a loader hands them over, and widens them to fp32
    on request, so a second consumer of the same seeded weights need not generate them again."""

    def __init__(self):
        self.layers = {}

    def hook(self, i, w):
        self.layers[i] = w

    def make(self, i):
        return {k: as_f32(v) for k, v in self.layers[i].items()}


@dataclass
class Batch:
    lengths: np.ndarray            # int64 [B]
    tokens: List[np.ndarray]       # B arrays of int64 token ids
    block_size: int
    block_tables: np.ndarray       # int32 [B, max_blocks]; -1 padding
    num_blocks: int

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    @property
    def token_ids(self) -> np.ndarray:
        return np.concatenate(self.tokens).astype(np.int32) if self.tokens else np.zeros(0, np.int32)

    @property
    def total_tokens(self) -> int:
        return int(self.lengths.sum())

    @property
    def max_seqlen(self) -> int:
        return int(self.lengths.max()) if len(self.lengths) else 0


def make_block_tables(lengths, block_size: int, seed: int, shuffle: bool, extra_blocks: int = 0):
    """Paged layout: prompt b owns ceil(N_b / block_size) physical blocks.

    With ``shuffle`` the physical block ids are a seeded permutation of
    0..num_blocks-1; otherwise they are assigned in order.
    """
    nbs = [-(-int(n) // block_size) for n in lengths]
    total = sum(nbs) + extra_blocks
    if shuffle:
        keys = randint(seed, S_BLOCKS, total, 1 << 53)
        perm = np.argsort(keys, kind="stable").astype(np.int32)
    else:
        perm = np.arange(total, dtype=np.int32)
    maxb = max(nbs) if nbs else 1
    bt = np.full((len(nbs), max(maxb, 1)), -1, dtype=np.int32)
    off = 0
    for b, nb in enumerate(nbs):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    return bt, total


def make_batch(w: Workload, lengths: Optional[List[int]] = None, shuffle: Optional[bool] = None) -> Batch:
    """Seeded prompts: lengths uniform in [len_lo, len_hi] (inclusive), ids uniform in [0, V)."""
    if lengths is None:
        if w.fixed_lengths is not None:
            lengths = list(w.fixed_lengths)
        else:
            span = w.len_hi - w.len_lo + 1
            lengths = [w.len_lo + int(v) for v in randint(w.input_seed, S_LENGTHS, w.n_prompts, span)]
    lengths = np.asarray(lengths, dtype=np.int64)
    ids = randint(w.input_seed, S_TOKENS, int(lengths.sum()), w.shape.vocab)
    toks, off = [], 0
    for n in lengths:
        toks.append(ids[off:off + int(n)].copy())
        off += int(n)
    sh = w.shuffle_blocks if shuffle is None else shuffle
    bt, nblk = make_block_tables(lengths, w.block_size, w.input_seed, sh)
    return Batch(lengths, toks, w.block_size, bt, nblk)


def small_workload(name: str, *, n_layers=4, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn_dim=1536,
                   vocab=2048, rope_theta=500000.0, dtype="bf16", l=2, g=1, lengths=(100,), seed=11,
                   shuffle=False, gain="normal", weight_seed=101) -> Workload:
    """A small model for parity tests that still spans several kernel tiles."""
    shape = ModelShape(name, n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, rope_theta,
                       weight_seed=weight_seed, gain=gain)
    return Workload(name, shape, dtype, l, g, len(lengths), min(lengths) if lengths else 0,
                    max(lengths) if lengths else 0, seed, shuffle_blocks=shuffle, fixed_lengths=tuple(lengths))


__all__ = [n for n in dir() if not n.startswith("_")]
