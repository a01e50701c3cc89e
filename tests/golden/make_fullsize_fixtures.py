"""Write the full-size parity fixtures from the CPU oracle.

    python tests/golden/make_fullsize_fixtures.py [WORKLOAD ...]

For each full-size workload this evaluates the oracle (oracle/swiftkv_oracle)
twice on a seeded set of its prompts, on the CPU:
  * plainly (fp32 NumPy): the expected values;
  * with bf16 storage (``store=`` rounding to bf16 at every point where a bf16
    inference path hands a tensor to the next operation: RMSNorm outputs,
    q / k / v after RoPE, attention outputs, SwiGLU outputs): how far bf16
    storage alone moves each output from the plain evaluation (the "floor").
and writes ``tests/golden/fullsize/<workload>.npz`` holding
  * the plain last-token logits of every selected prompt (float16),
  * the plain K and V of every cache slot at seeded positions of some prompts
    (float16; positions 0 and N-1 always included),
  * per compared tensor the floor: max |bf16-storage - plain| / max |plain|
    and the Frobenius ratio, over exactly the elements the GPU test compares,
  * for the prompts whose whole K/V the GPU test checks against a live run of
    the oracle, the same floors over positions 0..full_npos-1.
Stored values are float16: the storage rounding (at most 2^-11 of a value)
moves a measured max-relative error by at most 4.9e-4.

Inputs come from skv_inputs (the seeded generator shared with the GPU side);
nothing here reads a GPU result.  Prompts are independent (the oracle's
batch-independence pin), so a subset of a batch is evaluated alone.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import skv_inputs as si  # noqa: E402
from oracle import swiftkv_oracle as O  # noqa: E402

OUT_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fullsize")
S_POSITIONS = 9   # skv_inputs stream of the sampled K/V positions (per workload input seed)

# prompts: every prompt with a stored logits row; kv: prompts with stored K/V samples and how many positions;
# full: prompts (and how many leading positions) whose whole K/V the GPU test compares with a live oracle run
SPEC = {
    "llama8b_l16_b16": dict(prompts="all", kv=[], npos=0, full="shortest_longest", full_npos=None),
    "llama8b_l24_g4_b32": dict(prompts=[0, 11, 20, 31], kv=[11, 20], npos=8, full=[0, 31], full_npos=None),
    "llama70b_l40_b32": dict(prompts=[0, 5, 19, 31], kv=[0, 5, 19, 31], npos=4, full=[], full_npos=None),
    "llama8b_l16_long32k": dict(prompts=[0], kv=[0], npos=24, full=[0], full_npos=1024),
}


def dims_of(shape: si.ModelShape) -> O.Dims:
    return O.Dims(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim,
                  shape.vocab, shape.rope_theta, shape.rms_eps)


def round_bf16(x):
    return O.bf16_round(np.asarray(x, dtype=np.float32)).reshape(np.shape(x))


def max_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got)))


def frob_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def sample_positions(w: si.Workload, b: int, n: int, count: int) -> np.ndarray:
    """Seeded K/V positions of prompt b (length n): 0 and n-1, the first and last position of a 16-token block
    where the prompt has one, the rest uniform."""
    fixed = [0, n - 1] + ([15, 16] if n > 17 else [])
    draws = si.randint(w.input_seed, S_POSITIONS * 1000 + b, 4 * count, n)
    pos = []
    for p in fixed + [int(v) for v in draws]:
        if p not in pos:
            pos.append(p)
        if len(pos) == count:
            break
    return np.array(sorted(pos), dtype=np.int32)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Layers:
    """The workload's seeded layers in fp32, generated when the oracle asks (layer-major, one pass)."""

    def __init__(self, w: si.Workload, tag: str):
        self.w, self.tag, self.t0 = w, tag, time.time()

    def make(self, i):
        if i % 8 == 0:
            say(f"  [{self.tag}] layer {i} of {self.w.shape.n_layers} ({time.time() - self.t0:.0f} s)")
        return {k: si.as_f32(v) for k, v in si.layer_weights(self.w.shape, i, self.w.dtype).items()}


def evaluate(w: si.Workload, toks, store, tag):
    gw = si.global_weights(w.shape, w.dtype)
    W = O.LazyWeights(si.as_f32(gw["embed"]), si.as_f32(gw["final_norm"]), si.as_f32(gw["lm_head"]),
                      Layers(w, tag).make)
    del gw
    kw = {} if store is None else {"store": store}
    return O.swiftkv_prefill(dims_of(w.shape), W, toks, w.swiftkv_l, w.acrosskv_g, **kw)


def pick(spec_val, batch, all_count):
    if spec_val == "all":
        return list(range(all_count))
    if spec_val == "shortest_longest":
        return [int(np.argmin(batch.lengths)), int(np.argmax(batch.lengths))]
    return list(spec_val)


def build(name: str) -> str:
    w = si.WORKLOADS[name]
    spec = SPEC[name]
    batch = si.make_batch(w)
    prompts = pick(spec["prompts"], batch, len(batch.lengths))
    full = pick(spec["full"], batch, len(batch.lengths))
    kvp = list(spec["kv"])
    evalp = sorted(set(prompts) | set(full) | set(kvp))
    lengths = [int(batch.lengths[b]) for b in evalp]
    say(f"[{name}] prompts {evalp} (lengths {lengths}); logits of {prompts}, K/V samples of {kvp}, whole K/V of {full}")
    toks = [batch.tokens[b] for b in evalp]
    L, l, g = w.shape.n_layers, w.swiftkv_l, w.acrosskv_g
    nslots = O.kv_slots(L, l, g)
    at = {b: i for i, b in enumerate(evalp)}
    pos = {b: sample_positions(w, b, int(batch.lengths[b]), spec["npos"]) for b in kvp}
    fnp = {b: (spec["full_npos"] or int(batch.lengths[b])) for b in full}

    t0 = time.time()
    ref = evaluate(w, toks, None, f"{name} plain")
    say(f"[{name}] plain evaluation {time.time() - t0:.0f} s")
    ref_logits = {b: ref.logits[at[b]].astype(np.float32) for b in prompts}
    ref_kv = {b: np.stack([np.stack([ref.kv[at[b]][s][t][pos[b]] for t in (0, 1)]) for s in range(nslots)])
              for b in kvp}
    ref_full = {b: [[ref.kv[at[b]][s][t][:fnp[b]].copy() for t in (0, 1)] for s in range(nslots)] for b in full}
    del ref

    t1 = time.time()
    st = evaluate(w, toks, round_bf16, f"{name} bf16 storage")
    say(f"[{name}] bf16-storage evaluation {time.time() - t1:.0f} s")
    logits_floor = np.array([[max_rel(st.logits[at[b]], ref_logits[b]), frob_rel(st.logits[at[b]], ref_logits[b])]
                             for b in prompts], dtype=np.float32).reshape(len(prompts), 2)
    kv_floor = np.zeros((len(kvp), nslots, 2, 2), dtype=np.float32)
    for qi, b in enumerate(kvp):
        for s in range(nslots):
            for t in (0, 1):
                got = st.kv[at[b]][s][t][pos[b]]
                kv_floor[qi, s, t] = (max_rel(got, ref_kv[b][s, t]), frob_rel(got, ref_kv[b][s, t]))
    full_floor = np.zeros((len(full), nslots, 2, 2), dtype=np.float32)
    for ri, b in enumerate(full):
        for s in range(nslots):
            for t in (0, 1):
                got = st.kv[at[b]][s][t][:fnp[b]]
                full_floor[ri, s, t] = (max_rel(got, ref_full[b][s][t]), frob_rel(got, ref_full[b][s][t]))
    del st

    for v in list(ref_logits.values()) + list(ref_kv.values()):
        assert np.all(np.abs(v) < 6.0e4), "value outside the float16 range"
    hkv, dh = w.shape.n_kv_heads, w.shape.head_dim
    npos = spec["npos"]
    osha = hashlib.sha256(open(os.path.join(ROOT, "oracle", "swiftkv_oracle.py"), "rb").read()).hexdigest()
    meta = {
        "workload": name, "oracle_sha256": osha, "written": time.strftime("%Y-%m-%d"),
        "stored_dtype": "float16", "floor": "bf16 storage at the oracle's store= points vs the plain evaluation",
        "logits_prompts": prompts, "kv_prompts": kvp, "full_prompts": full,
        "full_npos": [fnp[b] for b in full], "lengths": {str(b): int(batch.lengths[b]) for b in evalp},
    }
    os.makedirs(OUT_DIR, exist_ok=True)
    path = os.path.join(OUT_DIR, f"{name}.npz")
    np.savez_compressed(
        path,
        meta=np.array(json.dumps(meta)),
        prompts=np.array(prompts, dtype=np.int32),
        logits=np.stack([ref_logits[b] for b in prompts]).astype(np.float16),
        logits_floor=logits_floor,
        kv_prompts=np.array(kvp, dtype=np.int32),
        kv_pos=np.stack([pos[b] for b in kvp]).astype(np.int32) if kvp else np.zeros((0, npos), np.int32),
        kv=(np.stack([ref_kv[b] for b in kvp]).astype(np.float16) if kvp
            else np.zeros((0, nslots, 2, npos, hkv, dh), np.float16)),
        kv_floor=kv_floor,
        full_prompts=np.array(full, dtype=np.int32),
        full_npos=np.array([fnp[b] for b in full], dtype=np.int32),
        full_floor=full_floor,
    )
    say(f"[{name}] wrote {path} ({os.path.getsize(path) / 1e6:.1f} MB, {time.time() - t0:.0f} s)")
    return path


if __name__ == "__main__":
    names = sys.argv[1:] or list(SPEC)
    for n in names:
        build(n)
