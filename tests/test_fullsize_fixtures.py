"""The stored full-size oracle results (tests/golden/fullsize/*.npz) against the oracle itself, on the CPU.

Structure: every stored file matches the seeded batch it claims (prompt
lengths, positions inside each prompt, 0 and N-1 among them), was written by
the current oracle (its source hash), holds finite values and floors.

Pin (slow): the shortest prompt of the 8B l=16 batch is evaluated again by
the oracle, plainly and with bf16 storage.  Its stored logits row must match
the plain evaluation to the float16 storage rounding, its stored floors (the
bf16-storage evaluation's distance from the plain one, per K/V tensor over
every position and for the logits) must match the recomputed ones, and the
set of tensors whose floor reaches the 2e-2 bar - the only tensors the GPU
tests allow above the bar - must be the same."""
import hashlib
import json
import os

import numpy as np
import pytest

import skv_inputs as si
from oracle import swiftkv_oracle as O
from tests.helpers import FULLSIZE_DIR, dims_of, fullsize_fixture, max_rel, oracle_code_sha256

NAMES = ["llama8b_l16_b16", "llama8b_l24_g4_b32", "llama70b_l40_b32", "llama8b_l16_long32k"]
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _present():
    return [n for n in NAMES if os.path.exists(os.path.join(FULLSIZE_DIR, f"{n}.npz"))]


def frob_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


@pytest.mark.parametrize("name", NAMES)
def test_fixture_structure(name):
    fx = fullsize_fixture(name)
    if fx is None:
        pytest.skip(f"{name}: no stored oracle results yet")
    w = si.WORKLOADS[name]
    batch = si.make_batch(w)
    meta = fx["meta"]
    src = open(os.path.join(ROOT, "oracle", "swiftkv_oracle.py"), "rb").read()
    # written by this oracle source, or by an earlier one whose code (docstrings and comments aside) is this one's,
    # as tests/golden/record_oracle_equivalence.py checked and recorded
    equiv_path = os.path.join(FULLSIZE_DIR, "oracle_equivalents.json")
    equiv = json.load(open(equiv_path)) if os.path.exists(equiv_path) else {}
    assert (meta["oracle_sha256"] == hashlib.sha256(src).hexdigest()
            or equiv.get(meta["oracle_sha256"]) == oracle_code_sha256(src)), \
        "the oracle changed since these results were written: regenerate them"
    assert meta["workload"] == name
    for b, n in meta["lengths"].items():
        assert int(batch.lengths[int(b)]) == n
    nslots = O.kv_slots(w.shape.n_layers, w.swiftkv_l, w.acrosskv_g)
    P = len(fx["prompts"])
    assert fx["logits"].shape == (P, w.shape.vocab) and np.isfinite(fx["logits"]).all()
    assert fx["logits_floor"].shape == (P, 2) and (fx["logits_floor"] > 0).all()
    Q = len(fx["kv_prompts"])
    if Q:
        S = fx["kv_pos"].shape[1]
        assert fx["kv"].shape == (Q, nslots, 2, S, w.shape.n_kv_heads, w.shape.head_dim)
        assert np.isfinite(fx["kv"]).all() and (fx["kv_floor"] > 0).all()
        for qi, b in enumerate(fx["kv_prompts"]):
            pos = fx["kv_pos"][qi]
            n = int(batch.lengths[int(b)])
            assert np.all(np.diff(pos) > 0) and pos[0] == 0 and pos[-1] == n - 1
    R = len(fx["full_prompts"])
    assert fx["full_floor"].shape == (R, nslots, 2, 2)
    for ri, b in enumerate(fx["full_prompts"]):
        assert 1 <= int(fx["full_npos"][ri]) <= int(batch.lengths[int(b)])


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_floor_of_the_shortest_8b_prompt_recomputed():
    name = "llama8b_l16_b16"
    fx = fullsize_fixture(name)
    if fx is None:
        pytest.skip(f"{name}: no stored oracle results yet")
    w = si.WORKLOADS[name]
    batch = si.make_batch(w)
    b = int(np.argmin(batch.lengths))
    ri = [int(x) for x in fx["full_prompts"]].index(b)
    pi = [int(x) for x in fx["prompts"]].index(b)
    gw = si.global_weights(w.shape, w.dtype)
    res = {}
    for mode, store in (("plain", None), ("bf16", lambda x: O.bf16_round(x).reshape(np.shape(x)))):
        W = O.LazyWeights(si.as_f32(gw["embed"]), si.as_f32(gw["final_norm"]), si.as_f32(gw["lm_head"]),
                          lambda i: {k: si.as_f32(v) for k, v in si.layer_weights(w.shape, i, w.dtype).items()})
        kw = {} if store is None else {"store": store}
        res[mode] = O.swiftkv_prefill(dims_of(w.shape), W, [batch.tokens[b]], w.swiftkv_l, w.acrosskv_g, **kw)
    plain, st = res["plain"], res["bf16"]
    # stored logits row = the plain evaluation, to the float16 storage rounding
    ref = plain.logits[0].astype(np.float64)
    assert np.all(np.abs(fx["logits"][pi] - ref) <= 2.0 ** -11 * np.abs(ref) + 1e-7)
    # floors recomputed
    got_floor = {("logits",): (max_rel(st.logits[0], plain.logits[0]), frob_rel(st.logits[0], plain.logits[0]))}
    want_floor = {("logits",): tuple(fx["logits_floor"][pi])}
    nslots = O.kv_slots(w.shape.n_layers, w.swiftkv_l, w.acrosskv_g)
    for s in range(nslots):
        for t in (0, 1):
            got_floor[(s, t)] = (max_rel(st.kv[0][s][t], plain.kv[0][s][t]), frob_rel(st.kv[0][s][t], plain.kv[0][s][t]))
            want_floor[(s, t)] = tuple(fx["full_floor"][ri, s, t])
    for k in got_floor:
        for a, e in zip(got_floor[k], want_floor[k]):
            assert abs(a - e) <= 1e-3 * e, (k, a, e)
    above_got = {k for k, v in got_floor.items() if v[0] >= 2e-2}
    above_want = {k for k, v in want_floor.items() if v[0] >= 2e-2}
    assert above_got == above_want
    # the regime the GPU tests allow exists only on the deep side: layer 1's slot is below the bar
    assert (0, 0) not in above_got and (0, 1) not in above_got


def test_oracle_code_hash_ignores_docstrings_and_comments_only():
    """The code hash behind oracle_equivalents.json: equal across docstring and comment edits, different when a
    single constant of the code changes."""
    a = b'"""module"""\ndef f(x):\n    """doc"""\n    return x + 1\n'
    b = b'"""other module text"""\ndef f(x):\n    """other doc"""\n    # a note\n    return x + 1\n'
    c = b'"""module"""\ndef f(x):\n    """doc"""\n    return x + 2\n'
    assert oracle_code_sha256(a) == oracle_code_sha256(b)
    assert oracle_code_sha256(a) != oracle_code_sha256(c)
