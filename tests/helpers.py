"""Shared helpers of the tests: seeded inputs -> oracle inputs, error metrics."""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

import skv_inputs as si
from oracle import swiftkv_oracle as O


def dims_of(shape: si.ModelShape) -> O.Dims:
    return O.Dims(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim,
                  shape.vocab, shape.rope_theta, shape.rms_eps)


CachedLayers = si.CachedLayers


def oracle_weights(w: si.Workload, cached: CachedLayers = None) -> O.WeightSource:
    """The oracle's view of the seeded weights: the exact stored values in fp32."""
    gw = si.global_weights(w.shape, w.dtype)
    if cached is None:
        make = lambda i: {k: si.as_f32(v) for k, v in si.layer_weights(w.shape, i, w.dtype).items()}
    else:
        make = cached.make
    return O.LazyWeights(si.as_f32(gw["embed"]), si.as_f32(gw["final_norm"]), si.as_f32(gw["lm_head"]), make)


def max_rel(got, ref) -> float:
    """max |got - ref| / max |ref| over one tensor (the parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / den)


# pytest's capture manager (set by conftest.py): progress lines bypass output
# capture, so a long GPU test shows it is alive while it runs
CAPMAN = None


def say(*a):
    """Print a progress line to the real stderr, past pytest's capture."""
    if CAPMAN is not None:
        with CAPMAN.global_and_fixture_disabled():
            print(*a, file=sys.stderr, flush=True)
    else:
        print(*a, file=sys.stderr, flush=True)


def oracle_code_sha256(source: bytes) -> str:
    """SHA-256 of a Python module's code: its syntax tree with every docstring removed (comments never reach
    the tree), so edits to comments and docstrings leave it unchanged."""
    import ast
    tree = ast.parse(source)
    for node in ast.walk(tree):
        body = getattr(node, "body", None)
        if (isinstance(node, (ast.Module, ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)) and body
                and isinstance(body[0], ast.Expr) and isinstance(body[0].value, ast.Constant)
                and isinstance(body[0].value.value, str)):
            node.body = body[1:] or [ast.Pass()]
    return hashlib.sha256(ast.dump(tree, include_attributes=False).encode()).hexdigest()


FULLSIZE_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize")


def fullsize_fixture(name: str):
    """The stored oracle results of one full-size workload (tests/golden/make_fullsize_fixtures.py), or None.

    Returns a dict with: meta; prompts / logits (float64 from the stored float16)
    / logits_floor; kv_prompts / kv_pos / kv [Q, slots, 2, S, hkv, dh] /
    kv_floor [Q, slots, 2, 2]; full_prompts / full_npos / full_floor
    [R, slots, 2, 2].  Floors are (max-relative, Frobenius) of the oracle's
    bf16-storage evaluation against its plain one over the same elements."""
    path = os.path.join(FULLSIZE_DIR, f"{name}.npz")
    if not os.path.exists(path):
        return None
    z = np.load(path, allow_pickle=False)
    out = {k: z[k] for k in z.files if k != "meta"}
    out["meta"] = json.loads(str(z["meta"]))
    out["logits"] = out["logits"].astype(np.float64)
    out["kv"] = out["kv"].astype(np.float64)
    return out
