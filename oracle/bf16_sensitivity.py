"""Where bf16 storage moves the SwiftKV prefill: the oracle with bf16 rounding at chosen points only.

    python oracle/bf16_sensitivity.py [N_TOKENS] [VARIANT ...]

TEST INFRASTRUCTURE (CPU only, like the rest of oracle/): it evaluates
oracle.swiftkv_oracle.swiftkv_prefill on the 8B-shaped model (seeded weights,
the first N_TOKENS of the shortest prompt of the 16-prompt batch, l = 16) once
plainly and once per variant with a ``store`` hook that rounds to bf16 only
at selected (layer, point) pairs, and prints, per variant, the max-relative
and Frobenius distance from the plain evaluation of slot 0, 3, 7, 11 and 15's
K, the first and last skipped slot's K, and the logits.

The points are where a bf16 inference path stores a tensor (the oracle's
``store=`` points): a = the attention RMSNorm output, q / k / v after RoPE,
o = the attention output, m = the MLP RMSNorm output, h = the SwiGLU output
(layers <= l); ba / bk / bv at the boundary; la, lq, lo, lm, lh for the
last token's layers; fa = the final norm.  The hook identifies a point by
the order in which swiftkv_prefill calls it for a single prompt.

Variants: all (every point), noL1 (every point but layer 1's), noL1_<p>+<p>
(every point but the listed points of layer 1), only_<p>+<p> (the listed
points in every layer), no_last (every point but the last token's).
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import skv_inputs as si  # noqa: E402
from oracle import swiftkv_oracle as O  # noqa: E402


def schedule(L: int, l: int):
    """(layer, point) of each store call, in swiftkv_prefill's order for one prompt, g = 1."""
    s = []
    for i in range(1, l + 1):
        s += [(i, t) for t in ("a", "q", "k", "v", "o", "m", "h")]
    for j in range(l + 1, L + 1):
        s += [(j, t) for t in ("ba", "bk", "bv")]
        s += [(j, t) for t in ("la", "lq", "lo", "lm", "lh")]
    return s + [(L + 1, "fa")]


def selector(variant: str):
    if variant == "all":
        return lambda i, t: True
    if variant == "noL1":
        return lambda i, t: i > 1
    if variant == "no_last":
        return lambda i, t: not t.startswith("l") and t != "fa"
    if variant.startswith("noL1_"):
        pts = set(variant[5:].split("+"))
        return lambda i, t: not (i == 1 and t in pts)
    if variant.startswith("only_"):
        pts = set(variant[5:].split("+"))
        return lambda i, t: t in pts
    raise ValueError(variant)


class Store:
    def __init__(self, sched, pick):
        self.sched, self.pick, self.n = sched, pick, 0

    def __call__(self, x):
        layer, point = self.sched[self.n]
        self.n += 1
        return O.bf16_round(np.asarray(x, dtype=np.float32)).reshape(np.shape(x)) if self.pick(layer, point) else x


def max_rel(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.max(np.abs(g - o)) / np.max(np.abs(o)))


def frob(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.linalg.norm(g - o) / np.linalg.norm(o))


def main():
    n = int(sys.argv[1]) if len(sys.argv) > 1 else 128
    variants = sys.argv[2:] or ["all", "noL1", "noL1_a", "noL1_a+q+k+v+o", "noL1_m", "noL1_h", "no_last"]
    w = si.WORKLOADS["llama8b_l16_b16"]
    s = w.shape
    batch = si.make_batch(w)
    toks = [batch.tokens[int(np.argmin(batch.lengths))][:n]]
    dims = O.Dims(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn_dim, s.vocab, s.rope_theta,
                  s.rms_eps)
    gw = si.global_weights(s, w.dtype)
    cache = {}

    def make(i):
        if i not in cache:
            cache[i] = {k: si.as_f32(v) for k, v in si.layer_weights(s, i, w.dtype).items()}
        return cache[i]
    W = O.LazyWeights(si.as_f32(gw["embed"]), si.as_f32(gw["final_norm"]), si.as_f32(gw["lm_head"]), make)
    sched = schedule(s.n_layers, w.swiftkv_l)
    ref = O.swiftkv_prefill(dims, W, toks, w.swiftkv_l, 1)
    slots = [0, 3, 7, 11, 15, 16, 31]
    print(f"{n} tokens; columns: K of slots {slots}, then logits; max-relative / Frobenius distance from plain")
    for v in variants:
        st = Store(sched, selector(v))
        r = O.swiftkv_prefill(dims, W, toks, w.swiftkv_l, 1, store=st)
        assert st.n == len(sched), "store calls do not follow the expected schedule"
        mr = [max_rel(r.kv[0][k][0], ref.kv[0][k][0]) for k in slots] + [max_rel(r.logits[0], ref.logits[0])]
        fr = [frob(r.kv[0][k][0], ref.kv[0][k][0]) for k in slots] + [frob(r.logits[0], ref.logits[0])]
        print(f"{v:18s} max  " + " ".join(f"{x:.1e}" for x in mr))
        print(f"{'':18s} frob " + " ".join(f"{x:.1e}" for x in fr), flush=True)


if __name__ == "__main__":
    main()
