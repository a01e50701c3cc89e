"""Plain CPU oracle for the SwiftKV prefill.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.  The HIP library never calls it, and it shares no
code with the HIP path.

Source: "SwiftKV: Fast Prefill-Optimized Inference with Knowledge-Preserving
Model Transformation" (Qiao, Yao, Rajbhandari, He; arXiv 2410.03960), read
from two pages:
  [P1] the paper-graph summary page, section 3.4 "Detailed, Sentence-Based
       Technical Breakdown" (Eq. 2, "What operations are skipped",
       Table 1, AcrossKV and its memory formula) and "Inference
       Implementation in Production Serving Frameworks";
  [P2] the AI_PARSE_DOCUMENT documentation page, whose example output
       quotes the paper's abstract, section 1, section 3.4 "Efficient
       Distillation" and section 3.5 "Optimized Implementation for Inference".

What it computes, for every prompt independently (1-based layers, x_i is the
input of layer i, l = number of unskipped layers, g = AcrossKV group size):
  1. x_1 = E[tokens].
  2. layers 1..l run normally on every prompt token; their K/V are kept
     ([P1] 3.4 "Inference Implementation": early-layer KV populated normally).
  3. boundary, Eq. 2 ([P1] 3.4 "The SwiftKV Rewiring Mechanism"; [P2] section
     1 "Model transformation"): for each skipped layer j > l,
     KV_j = W_KV^j applied to x_{l+1}.  The projection is applied after layer
     j's input RMSNorm (pre-norm Llama block; the pages place the KV
     projections after layer norm).  RoPE is applied to K at each token's
     position.  With AcrossKV ([P1] 3.4 AcrossKV, Eq. KV_group) consecutive
     groups of g skipped layers share one KV computed with the first layer of
     the group as representative.
  4. only the last prompt token continues through layers l+1..L ([P1] 3.4
     "What the first generated token does differently"), attending to the
     SwiftKV cache of each layer (all N positions, its own included).
  5. logits = RMSNorm(y; final gain) @ W_lm^T for that last token.

swiftkv_step extends this to a mixed batch ([P1] "Inference Implementation
in Production Serving Frameworks"; [P2] section 3.5): each sequence may hold
cached positions already (a prompt chunk after earlier chunks, a decode
token); its new tokens run steps 2-3 attending to the cache as well, and its
last new token runs step 4 and 5.

Readings where the pages are silent:
  * Llama block: pre-norm RMSNorm, GQA attention with RoPE (rotate-half,
    inv_freq_i = theta^(-2i/dh), no frequency scaling), SwiGLU MLP
    W_d(silu(W_g a) * W_u a), no biases, untied LM head.
  * q-head h reads kv-head floor(h / (hq/hkv)); scale 1/sqrt(dh); causal mask
    within a prompt; max-subtracted softmax.
  * the last token's own K/V at layers > l is the SwiftKV value (from
    x_{l+1}), like every other prompt token's.
  * AcrossKV representative = lowest layer of each group; a short last
    group is allowed when g does not divide L - l.

FLOP counting (for the closed-form check): every matmul of an [m,k] by a
[k,n] operand adds 2*m*n*k; attention adds 4*ctx*dh per query per head with
ctx = number of keys attended.  Norms, RoPE, softmax, gathers are not
counted.

Parity of this oracle is pinned by tests/test_oracle_pins.py against an
independent library Llama (l = L), an incremental one-token-at-a-time decode,
the pages' printed FLOP (Table 1) and KV-memory figures, and closed-form
identities; the step by tests/test_oracle_step_pins.py (chunked = one-shot
prefill, decode at l = L = standard decode, batch independence, FLOPs).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class Dims:
    """Decoder dimensions (no weights)."""
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rope_theta: float
    rms_eps: float = 1e-5

    @property
    def dq(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def dkv(self) -> int:
        return self.n_kv_heads * self.head_dim


class FlopCounter:
    def __init__(self) -> None:
        self.total = 0

    def add(self, n: int) -> None:
        self.total += int(n)


# ----------------------------------------------------------------------------
# textbook pieces of a Llama-style pre-norm decoder layer
# ----------------------------------------------------------------------------

def matmul_wt(a: np.ndarray, w: np.ndarray, fc: Optional[FlopCounter]) -> np.ndarray:
    """a @ w.T for a Linear weight w stored [out, in]."""
    if fc is not None:
        fc.add(2 * a.shape[0] * w.shape[0] * w.shape[1])
    return a @ w.T


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + eps).astype(x.dtype)) * gamma


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float, dtype) -> Tuple[np.ndarray, np.ndarray]:
    """cos/sin tables [n, head_dim/2]; angles pos * theta^(-2i/head_dim) in float64."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE on x [n, heads, head_dim]: pairs (i, i + head_dim/2)."""
    dh = x.shape[-1]
    half = dh // 2
    cos, sin = rope_cos_sin(positions, dh, theta, x.dtype)
    cos = cos[:, None, :]
    sin = sin[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, fc: Optional[FlopCounter],
                         q_chunk: int = 2048) -> np.ndarray:
    """softmax(q k^T / sqrt(dh), causal) v per head; q [n,hq,dh], k/v [n,hkv,dh] -> [n, hq*dh].

    Query rows are processed in chunks only to bound memory; each row is the
    plain formula.
    """
    n, hq, dh = q.shape
    hkv = k.shape[1]
    rep = hq // hkv
    scale = 1.0 / math.sqrt(dh)
    out = np.empty((n, hq, dh), dtype=q.dtype)
    for h in range(hq):
        g = h // rep
        kh, vh = k[:, g, :], v[:, g, :]
        for s0 in range(0, n, q_chunk):
            s1 = min(n, s0 + q_chunk)
            s = (q[s0:s1, h, :] @ kh[:s1].T) * q.dtype.type(scale)
            qi = np.arange(s0, s1)[:, None]
            kj = np.arange(s1)[None, :]
            s = np.where(kj <= qi, s, -np.inf)
            out[s0:s1, h, :] = softmax_rows(s) @ vh[:s1]
    if fc is not None:
        fc.add(4 * dh * hq * (n * (n + 1) // 2))
    return out.reshape(n, hq * dh)


def single_query_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, fc: Optional[FlopCounter]) -> np.ndarray:
    """One query position per head attending to every row of k/v: q [hq,dh], k/v [n,hkv,dh] -> [hq*dh]."""
    hq, dh = q.shape
    n, hkv, _ = k.shape
    rep = hq // hkv
    scale = q.dtype.type(1.0 / math.sqrt(dh))
    out = np.empty((hq, dh), dtype=q.dtype)
    for h in range(hq):
        g = h // rep
        s = (k[:, g, :] @ q[h]) * scale
        out[h] = softmax_rows(s[None, :])[0] @ v[:, g, :]
    if fc is not None:
        fc.add(4 * n * dh * hq)
    return out.reshape(hq * dh)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1 + np.exp(-x))


def swiglu_mlp(m: np.ndarray, W: Dict[str, np.ndarray], fc: Optional[FlopCounter]) -> np.ndarray:
    h = silu(matmul_wt(m, W["w_gate"], fc)) * matmul_wt(m, W["w_up"], fc)
    return matmul_wt(h, W["w_down"], fc)


def _keep(t: np.ndarray) -> np.ndarray:
    return t


def qkv_projection(x: np.ndarray, W: Dict[str, np.ndarray], pos: np.ndarray, dims: Dims,
                   fc: Optional[FlopCounter], store: Callable = _keep):
    """RMSNorm then q/k/v projections, RoPE on q and k.  Returns q [n,hq,dh], k, v [n,hkv,dh]."""
    n = x.shape[0]
    a = store(rmsnorm(x, W["attn_norm"], dims.rms_eps))
    q = matmul_wt(a, W["wq"], fc).reshape(n, dims.n_q_heads, dims.head_dim)
    k = matmul_wt(a, W["wk"], fc).reshape(n, dims.n_kv_heads, dims.head_dim)
    v = matmul_wt(a, W["wv"], fc).reshape(n, dims.n_kv_heads, dims.head_dim)
    return store(rope(q, pos, dims.rope_theta)), store(rope(k, pos, dims.rope_theta)), store(v)


def mlp_residual(x: np.ndarray, W: Dict[str, np.ndarray], dims: Dims, fc: Optional[FlopCounter],
                 store: Callable = _keep) -> np.ndarray:
    """x + W_d(silu(W_g m) * W_u m) with m = RMSNorm(x; ffn gain)."""
    m = store(rmsnorm(x, W["ffn_norm"], dims.rms_eps))
    h = store(silu(matmul_wt(m, W["w_gate"], fc)) * matmul_wt(m, W["w_up"], fc))
    return x + matmul_wt(h, W["w_down"], fc)


def decoder_layer(x: np.ndarray, W: Dict[str, np.ndarray], pos: np.ndarray, dims: Dims,
                  fc: Optional[FlopCounter], store: Callable = _keep, kv_cache: Callable = _keep):
    """Standard pre-norm layer over all n positions of one prompt.  Returns (x_next, K, V).

    ``kv_cache`` maps K and V to what the cache holds (identity, or the FP8
    round trip); attention reads the cached values."""
    q, k, v = qkv_projection(x, W, pos, dims, fc, store)
    k, v = kv_cache(k), kv_cache(v)
    o = store(causal_gqa_attention(q, k, v, fc))
    x = x + matmul_wt(o, W["wo"], fc)
    return mlp_residual(x, W, dims, fc, store), k, v


# ----------------------------------------------------------------------------
# FP8 KV cache (per-token scale), [S] "Complementarity with KV quantization"
# (Appendix B.1, Table B.1)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent 0 is subnormal, m * 2^-9; no infinities;
    S.1111.111 is NaN) as float32."""
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag).astype(np.float32)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """E4M3 code nearest to each float32 value, ties to even; |y| <= 448."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)                 # exact
    if np.any(a > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    sub = np.rint(a * 512.0)                          # subnormal step 2^-9; 8 = the smallest normal's code
    mant, ex = np.frexp(a)                            # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                                        # a = (2 mant) 2^e
    m = np.rint((2.0 * mant - 1.0) * 8.0)             # exact products; rint rounds ties to even
    up = m == 8
    e = np.where(up, e + 1, e)
    m = np.where(up, 0, m)
    normal = (e + 7) * 8 + m
    code = np.where(a < 2.0 ** -6, sub, normal).astype(np.int64)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def fp8_quantize_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token FP8: each row (one token's K or V over all kv heads) gets
    scale = max|row| / 448 and codes = E4M3(row * (1 / scale)), every step a
    single float32 operation (division, reciprocal, product, clamp to +-448),
    so the code decisions are those of float32 arithmetic.  A zero row has
    scale 0 and zero codes."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    scale = amax / np.float32(E4M3_MAX)
    inv = np.where(scale > 0, np.float32(1.0) / np.where(scale > 0, scale, np.float32(1.0)), np.float32(0.0))
    y = np.clip(x * inv.astype(np.float32)[:, None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return e4m3_encode(y), scale.astype(np.float32)


def fp8_dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes * scale per row, float32."""
    return (e4m3_decode(codes) * np.asarray(scale, dtype=np.float32)[:, None]).astype(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), returned as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).reshape(np.shape(x))


def fp8_kv_roundtrip(t: np.ndarray) -> np.ndarray:
    """What a per-token FP8 cache hands back for K or V [n, hkv, dh].

    The quantiser takes the values a bf16 inference path holds (the pages
    serve in bf16), so each K/V value is rounded to bf16 first; the code
    decisions are then float32 arithmetic on bf16 inputs."""
    n = t.shape[0]
    flat = bf16_round(np.asarray(t, dtype=np.float32).reshape(n, -1))
    c, sc = fp8_quantize_rows(flat)
    return fp8_dequantize_rows(c, sc).reshape(t.shape).astype(t.dtype)


# ----------------------------------------------------------------------------
# SwiftKV structure
# ----------------------------------------------------------------------------

def n_groups(L: int, l: int, g: int) -> int:
    """Number of KV tensors for the skipped layers: ceil((L - l) / g)."""
    return -(-(L - l) // g)


def kv_slots(L: int, l: int, g: int) -> int:
    """KV tensors held in total: l unskipped layers + one per AcrossKV group."""
    return l + n_groups(L, l, g)


def slot_of_layer(j: int, L: int, l: int, g: int) -> int:
    """0-based KV slot read by 1-based layer j."""
    if not 1 <= j <= L:
        raise ValueError(j)
    return j - 1 if j <= l else l + (j - l - 1) // g


def representative(j: int, l: int, g: int) -> int:
    """First (lowest) layer of the AcrossKV group holding skipped layer j."""
    return l + 1 + g * ((j - l - 1) // g)


class WeightSource:
    """Interface the oracle reads weights through (arrays already in the oracle's float type).

    ``layer(i)`` returns the 1-based layer's dict with keys attn_norm, wq, wk,
    wv, wo, ffn_norm, w_gate, w_up, w_down (Linear weights [out, in]).
    """
    embed: np.ndarray
    final_norm: np.ndarray
    lm_head: np.ndarray

    def layer(self, i: int) -> Dict[str, np.ndarray]:  # pragma: no cover - interface
        raise NotImplementedError


class DictWeights(WeightSource):
    def __init__(self, embed, final_norm, lm_head, layers: Sequence[Dict[str, np.ndarray]], dtype=np.float32):
        self.dtype = dtype
        self.embed = np.asarray(embed, dtype=dtype)
        self.final_norm = np.asarray(final_norm, dtype=dtype)
        self.lm_head = np.asarray(lm_head, dtype=dtype)
        self._layers = [{k: np.asarray(v, dtype=dtype) for k, v in W.items()} for W in layers]

    def layer(self, i: int) -> Dict[str, np.ndarray]:
        return self._layers[i - 1]


class LazyWeights(WeightSource):
    """Layers produced on demand by a callable (used to stream large models)."""

    def __init__(self, embed, final_norm, lm_head, make_layer: Callable[[int], Dict[str, np.ndarray]],
                 dtype=np.float32):
        self.dtype = dtype
        self.embed = np.asarray(embed, dtype=dtype)
        self.final_norm = np.asarray(final_norm, dtype=dtype)
        self.lm_head = np.asarray(lm_head, dtype=dtype)
        self._make = make_layer

    def layer(self, i: int) -> Dict[str, np.ndarray]:
        return {k: np.asarray(v, dtype=self.dtype) for k, v in self._make(i).items()}


@dataclass
class OracleResult:
    kv: List[Dict[int, Tuple[np.ndarray, np.ndarray]]]   # per prompt: slot -> (K [n,hkv,dh], V [n,hkv,dh])
    logits: np.ndarray                                    # [B, vocab]
    flops: int
    x_boundary: List[np.ndarray]                          # per prompt x_{l+1} [n, d]


def swiftkv_prefill(dims: Dims, weights: WeightSource, prompts: Sequence[np.ndarray], l: int, g: int = 1,
                    dtype=np.float32, store: Optional[Callable] = None, kv_fp8: bool = False) -> OracleResult:
    """SwiftKV prefill of a batch of independent prompts (steps 1-5 of the module docstring).

    Layers are visited in increasing order exactly once (layer-major), so a
    streaming WeightSource can generate each layer when it is asked for.

    ``store`` (default: keep values as computed) is applied where a reduced-
    precision inference path stores a tensor: the RMSNorm outputs fed to the
    projections, q / k / v after RoPE, the attention output, the SwiGLU
    output.  With a bf16 rounding function this evaluates the same definition
    with bf16 storage (the precision the pages serve in), which measures how
    far bf16 storage alone moves each output from the plain evaluation.

    ``kv_fp8``: the cache holds per-token FP8 K and V (fp8_kv_roundtrip);
    every attention reads those values and ``kv`` returns them.
    """
    st = store if store is not None else _keep
    kq = fp8_kv_roundtrip if kv_fp8 else _keep
    L = dims.n_layers
    if not 0 <= l <= L:
        raise ValueError(f"swiftkv l={l} outside 0..{L}")
    if g < 1:
        raise ValueError("acrosskv group size must be >= 1")
    if any(len(p) < 1 for p in prompts):
        raise ValueError("every prompt needs at least one token")
    fc = FlopCounter()
    eps = dims.rms_eps
    xs = [weights.embed[np.asarray(p)].astype(dtype) for p in prompts]          # step 1
    pos = [np.arange(len(p)) for p in prompts]
    kv: List[Dict[int, Tuple[np.ndarray, np.ndarray]]] = [dict() for _ in prompts]

    for i in range(1, l + 1):                                                     # step 2
        W = weights.layer(i)
        for b in range(len(prompts)):
            xs[b], k, v = decoder_layer(xs[b], W, pos[b], dims, fc, st, kq)
            kv[b][i - 1] = (k, v)

    ys = [x[-1:].copy() for x in xs]                                              # last token rows
    for j in range(l + 1, L + 1):
        W = weights.layer(j)
        s = slot_of_layer(j, L, l, g)
        if representative(j, l, g) == j:                                          # step 3 (Eq. 2)
            for b in range(len(prompts)):
                n = xs[b].shape[0]
                a = st(rmsnorm(xs[b], W["attn_norm"], eps))
                k = matmul_wt(a, W["wk"], fc).reshape(n, dims.n_kv_heads, dims.head_dim)
                v = matmul_wt(a, W["wv"], fc).reshape(n, dims.n_kv_heads, dims.head_dim)
                kv[b][s] = (kq(st(rope(k, pos[b], dims.rope_theta))), kq(st(v)))
        for b in range(len(prompts)):                                             # step 4
            n = xs[b].shape[0]
            K, V = kv[b][s]
            a = st(rmsnorm(ys[b], W["attn_norm"], eps))
            q = matmul_wt(a, W["wq"], fc).reshape(1, dims.n_q_heads, dims.head_dim)
            q = st(rope(q, np.array([n - 1]), dims.rope_theta))
            o = st(single_query_attention(q[0], K, V, fc)[None, :])
            y = ys[b] + matmul_wt(o, W["wo"], fc)
            ys[b] = mlp_residual(y, W, dims, fc, st)

    logits = np.concatenate(                                                      # step 5
        [matmul_wt(st(rmsnorm(y, weights.final_norm, eps)), weights.lm_head, fc) for y in ys], axis=0)
    return OracleResult(kv, logits, fc.total, xs)


def attention_with_past(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
                        fc: Optional[FlopCounter]) -> np.ndarray:
    """GQA attention of queries at absolute positions q_pos over cached keys/values.

    q [n,hq,dh]; k/v [m,hkv,dh] hold positions 0..m-1.  Query row i sees the
    keys at positions 0..q_pos[i] (causal, earlier calls' positions
    included).  Returns [n, hq*dh].
    """
    n, hq, dh = q.shape
    rep = hq // k.shape[1]
    scale = q.dtype.type(1.0 / math.sqrt(dh))
    visible = np.arange(k.shape[0])[None, :] <= np.asarray(q_pos)[:, None]
    out = np.empty((n, hq, dh), dtype=q.dtype)
    for h in range(hq):
        g = h // rep
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        out[:, h, :] = softmax_rows(np.where(visible, s, -np.inf)) @ v[:, g, :]
    if fc is not None:
        fc.add(4 * dh * hq * int(np.sum(np.asarray(q_pos) + 1)))
    return out.reshape(n, hq * dh)


@dataclass
class StepResult:
    kv: List[Dict[int, Tuple[np.ndarray, np.ndarray]]]   # per sequence: slot -> (K, V) over all ctx + n positions
    logits: np.ndarray                                    # [B, vocab], after each sequence's last new token
    flops: int


def swiftkv_step(dims: Dims, weights: WeightSource, past: Sequence[Dict[int, Tuple[np.ndarray, np.ndarray]]],
                 new_tokens: Sequence[np.ndarray], l: int, g: int = 1, dtype=np.float32,
                 kv_fp8: bool = False, store: Optional[Callable] = None) -> StepResult:
    """One forward pass over a mixed batch of prompt chunks and decode tokens.

    Source: [P1] "Inference Implementation in Production Serving Frameworks"
    (mixed batches, chunked prefill) and [P2] section 3.5: every token of
    the batch, prefill chunk or decode token, runs layers 1..l with its
    early-layer KV stored normally; right after layer l the KV of every
    skipped layer is computed from x_{l+1} of every new token; only the
    tokens that continue (the decode tokens; here the last new token of
    every sequence, which also yields a finished prompt's first logits) run
    layers l+1..L, attending to the cache.

    ``past[b]`` maps each KV slot to sequence b's cached (K, V) over
    positions 0..C_b-1 (an empty dict: C_b = 0); ``new_tokens[b]`` are its
    new tokens at positions C_b, C_b+1, ...  Returns the extended caches
    (new arrays; ``past`` is not modified) and the logits after each
    sequence's last new token.  ``kv_fp8``: the cache holds per-token FP8
    values (fp8_kv_roundtrip of each new token's K and V); ``past`` then
    holds such values too.  ``store``: as in swiftkv_prefill (the stored
    tensors rounded, e.g. to bf16).
    """
    L, eps = dims.n_layers, dims.rms_eps
    kq = fp8_kv_roundtrip if kv_fp8 else _keep
    st = store if store is not None else _keep
    if not 0 <= l <= L or g < 1:
        raise ValueError("bad l or g")
    if len(past) != len(new_tokens) or any(len(t) < 1 for t in new_tokens):
        raise ValueError("one non-empty token run per sequence")
    fc = FlopCounter()
    nslot = kv_slots(L, l, g)
    empty = np.zeros((0, dims.n_kv_heads, dims.head_dim), dtype)
    kv = [{s: past[b].get(s, (empty, empty)) for s in range(nslot)} for b in range(len(past))]
    ctx = [kv[b][0][0].shape[0] for b in range(len(past))]
    for b in range(len(past)):
        if any(kv[b][s][0].shape[0] != ctx[b] for s in range(nslot)):
            raise ValueError("every slot of a sequence must hold the same positions")
    xs = [weights.embed[np.asarray(t)].astype(dtype) for t in new_tokens]
    pos = [ctx[b] + np.arange(len(new_tokens[b])) for b in range(len(past))]

    for i in range(1, l + 1):                      # layers 1..l: every new token
        W = weights.layer(i)
        for b in range(len(past)):
            q, k, v = qkv_projection(xs[b], W, pos[b], dims, fc, st)
            K = np.concatenate([kv[b][i - 1][0], kq(k)], axis=0)
            V = np.concatenate([kv[b][i - 1][1], kq(v)], axis=0)
            kv[b][i - 1] = (K, V)
            x = xs[b] + matmul_wt(st(attention_with_past(q, K, V, pos[b], fc)), W["wo"], fc)
            xs[b] = mlp_residual(x, W, dims, fc, st)

    ys = [x[-1:].copy() for x in xs]
    for j in range(l + 1, L + 1):
        W = weights.layer(j)
        s = slot_of_layer(j, L, l, g)
        if representative(j, l, g) == j:           # KV of the skipped layers from x_{l+1}
            for b in range(len(past)):
                n = xs[b].shape[0]
                a = st(rmsnorm(xs[b], W["attn_norm"], eps))
                k = matmul_wt(a, W["wk"], fc).reshape(n, dims.n_kv_heads, dims.head_dim)
                v = matmul_wt(a, W["wv"], fc).reshape(n, dims.n_kv_heads, dims.head_dim)
                kv[b][s] = (np.concatenate([kv[b][s][0], kq(st(rope(k, pos[b], dims.rope_theta)))], axis=0),
                            np.concatenate([kv[b][s][1], kq(st(v))], axis=0))
        for b in range(len(past)):                 # the continuing token
            K, V = kv[b][s]
            p_last = int(pos[b][-1])
            a = st(rmsnorm(ys[b], W["attn_norm"], eps))
            q = matmul_wt(a, W["wq"], fc).reshape(1, dims.n_q_heads, dims.head_dim)
            q = st(rope(q, np.array([p_last]), dims.rope_theta))
            o = st(attention_with_past(q, K, V, np.array([p_last]), fc))
            y = ys[b] + matmul_wt(o, W["wo"], fc)
            ys[b] = mlp_residual(y, W, dims, fc, st)

    logits = np.concatenate(
        [matmul_wt(st(rmsnorm(y, weights.final_norm, eps)), weights.lm_head, fc) for y in ys], axis=0)
    return StepResult(kv, logits, fc.total)


def standard_incremental_decode(dims: Dims, weights: WeightSource, prompt: np.ndarray, dtype=np.float32):
    """Unmodified model run one token at a time with a growing KV cache.

    Returns (K list per layer [n,hkv,dh], V list, logits of the last token).
    A second, independent route to the l = L prefill result: no causal mask,
    each position is a single query over the cache built so far.
    """
    L, eps = dims.n_layers, dims.rms_eps
    Ks = [np.zeros((0, dims.n_kv_heads, dims.head_dim), dtype) for _ in range(L)]
    Vs = [np.zeros((0, dims.n_kv_heads, dims.head_dim), dtype) for _ in range(L)]
    Ws = [weights.layer(i) for i in range(1, L + 1)]
    y = None
    for t, tok in enumerate(np.asarray(prompt)):
        y = weights.embed[tok][None, :].astype(dtype)
        for i in range(L):
            W = Ws[i]
            q, k, v = qkv_projection(y, W, np.array([t]), dims, None)
            Ks[i] = np.concatenate([Ks[i], k], axis=0)
            Vs[i] = np.concatenate([Vs[i], v], axis=0)
            o = single_query_attention(q[0], Ks[i], Vs[i], None)[None, :]
            y = y + matmul_wt(o, W["wo"], None)
            y = y + swiglu_mlp(rmsnorm(y, W["ffn_norm"], eps), W, None)
    logits = matmul_wt(rmsnorm(y, weights.final_norm, eps), weights.lm_head, None)[0]
    return Ks, Vs, logits


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def prefill_flops(dims: Dims, l: int, g: int, lengths: Sequence[int]) -> Tuple[int, int]:
    """(full-depth FLOPs, SwiftKV FLOPs) of a prefill over prompts of the given lengths.

    Full depth = the unmodified model (every layer, every token; LM head on
    the last token).  SwiftKV = layers 1..l for every token, one K/V
    projection per AcrossKV group for every token, layers l+1..L for the
    last token only (its attention spans all N positions).
    """
    d, dq, dkv, f, V, L = dims.d_model, dims.dq, dims.dkv, dims.ffn_dim, dims.vocab, dims.n_layers
    hq, dh = dims.n_q_heads, dims.head_dim
    G = n_groups(L, l, g)
    lin = 2 * d * dq + 2 * dq * d + 6 * d * f + 4 * d * dkv
    full = swift = 0
    for n in lengths:
        n = int(n)
        layer_full = n * lin + 2 * n * (n + 1) * dh * hq
        full += L * layer_full + 2 * d * V
        swift += (l * layer_full + G * n * 4 * d * dkv
                  + (L - l) * (2 * d * dq + 2 * dq * d + 6 * d * f + 4 * n * dh * hq) + 2 * d * V)
    return full, swift


def step_flops(dims: Dims, l: int, g: int, ctx: Sequence[int], new: Sequence[int]) -> int:
    """SwiftKV FLOPs of one mixed-batch step: sequence b holds ctx[b] cached
    positions and brings new[b] tokens.  Layers 1..l for every new token
    (token at position p attends p+1 keys), one K/V projection per AcrossKV
    group for every new token, layers l+1..L and the LM head for the last
    new token (attending ctx + new keys)."""
    d, dq, dkv, f, V, L = dims.d_model, dims.dq, dims.dkv, dims.ffn_dim, dims.vocab, dims.n_layers
    hq, dh = dims.n_q_heads, dims.head_dim
    G = n_groups(L, l, g)
    total = 0
    for c, n in zip(ctx, new):
        c, n = int(c), int(n)
        t = c + n
        keys = (t * (t + 1) - c * (c + 1)) // 2          # sum of p + 1 over the new positions
        total += l * (n * (2 * d * dq + 2 * dq * d + 6 * d * f + 4 * d * dkv) + 4 * dh * hq * keys)
        total += G * n * 4 * d * dkv
        total += (L - l) * (2 * d * dq + 2 * dq * d + 6 * d * f + 4 * t * dh * hq) + 2 * d * V
    return total


def per_token_breakdown(dims: Dims, l: int, g: int, attn_per_layer_flops: float = 0.0) -> Dict[str, float]:
    """Per-prefill-token FLOPs by operation, in the style of the paper's Table 1.

    vocab counts the embedding lookup and the LM head as two d x V products
    (the way the page's Table 1 lists "Vocabulary projection");
    ``attn_per_layer_flops`` supplies the attention cost per layer, whose
    sequence length the table does not print.
    """
    d, dq, dkv, f, V, L = dims.d_model, dims.dq, dims.dkv, dims.ffn_dim, dims.vocab, dims.n_layers
    G = n_groups(L, l, g)
    return {
        "vocab": 2 * 2 * d * V,
        "kv": (l + G) * 4 * d * dkv,
        "qo": l * (2 * d * dq + 2 * dq * d),
        "mlp": l * 6 * d * f,
        "attention": l * attn_per_layer_flops,
    }


def kv_memory_fraction(L: int, l: int, g: int, kv_bits: int = 16) -> float:
    """KV memory relative to the unmodified model with a 16-bit cache:
    (l + (L-l)/g) / L (AcrossKV memory formula) times kv_bits / 16 (an FP8
    cache halves every entry; the per-token scales are not counted, as in
    the pages' figures)."""
    return kv_slots(L, l, g) / L * kv_bits / 16
