"""Pins of the oracle's mixed-batch step (prompt chunks and decode tokens), CPU only.

The step has no printed values on the pages; what fixes it is the method's
structure ("Inference Implementation in Production Serving Frameworks",
section 3.5 "Optimized Implementation for Inference"): chunk boundaries need
no special handling, so

* feeding a prompt in chunks, one step per chunk, must give the cache and the
  final logits of a one-shot SwiftKV prefill of the whole prompt, and each
  chunk's logits those of the prefill of the prompt up to that chunk's end;
* at l = L (no skipped layers) a decode token is an ordinary decode step:
  the logits match one-token-at-a-time decoding of the unmodified model,
  itself pinned to a library Llama;
* sequences of one batch do not interact;
* the FLOP counter matches the closed form.
"""
import numpy as np
import pytest

from oracle import swiftkv_oracle as O
from tests.test_oracle_pins import prompts_for, rel, tiny_dims, tiny_weights

TIGHT = 1e-10  # float64 evaluations of the same function in different orders


def run_chunks(dims, W, prompt, chunks, l, g):
    """Feed `prompt` in the given chunk sizes; returns (final kv, logits after every chunk)."""
    past, logits, off = {}, [], 0
    for n in chunks:
        r = O.swiftkv_step(dims, W, [past], [prompt[off:off + n]], l, g, dtype=np.float64)
        past = r.kv[0]
        logits.append(r.logits[0])
        off += n
    assert off == len(prompt)
    return past, logits


@pytest.mark.parametrize("l,g", [(0, 1), (2, 1), (1, 3), (4, 1), (2, 2)])
def test_chunked_prefill_equals_one_shot_prefill(l, g):
    dims = tiny_dims()
    W = tiny_weights(dims)
    prompt = prompts_for(dims, [29])[0]
    chunks = [7, 1, 13, 8]
    kv, logits = run_chunks(dims, W, prompt, chunks, l, g)
    full = O.swiftkv_prefill(dims, W, [prompt], l, g, dtype=np.float64)
    assert set(kv) == set(full.kv[0]) == set(range(O.kv_slots(dims.n_layers, l, g)))
    for s in kv:
        assert rel(kv[s][0], full.kv[0][s][0]) < TIGHT, f"K slot {s}"
        assert rel(kv[s][1], full.kv[0][s][1]) < TIGHT, f"V slot {s}"
    end = 0
    for n, lg in zip(chunks, logits):
        end += n
        ref = O.swiftkv_prefill(dims, W, [prompt[:end]], l, g, dtype=np.float64).logits[0]
        assert rel(lg, ref) < TIGHT, f"logits after {end} tokens"


def test_decode_at_full_depth_equals_standard_decode():
    dims = tiny_dims()
    W = tiny_weights(dims)
    prompt = prompts_for(dims, [12])[0]
    L = dims.n_layers
    r = O.swiftkv_step(dims, W, [{}], [prompt[:5]], L, 1, dtype=np.float64)
    past = r.kv[0]
    for t in range(5, len(prompt)):
        r = O.swiftkv_step(dims, W, [past], [prompt[t:t + 1]], L, 1, dtype=np.float64)
        past = r.kv[0]
        _, _, ref = O.standard_incremental_decode(dims, W, prompt[:t + 1], dtype=np.float64)
        assert rel(r.logits[0], ref) < TIGHT, f"decode of token {t}"


def test_decode_token_after_swiftkv_prefill_is_the_next_prefill_position():
    """With skipped layers: decode token N after a prefill of N tokens gives the
    KV and logits of the prefill of N + 1 tokens (its own KV at j > l comes
    from its x_{l+1}, like a prompt token's)."""
    dims = tiny_dims()
    W = tiny_weights(dims)
    l, g = 2, 2
    prompt = prompts_for(dims, [17])[0]
    pre = O.swiftkv_prefill(dims, W, [prompt[:16]], l, g, dtype=np.float64)
    r = O.swiftkv_step(dims, W, [pre.kv[0]], [prompt[16:]], l, g, dtype=np.float64)
    full = O.swiftkv_prefill(dims, W, [prompt], l, g, dtype=np.float64)
    assert rel(r.logits[0], full.logits[0]) < TIGHT
    for s in full.kv[0]:
        assert rel(r.kv[0][s][0], full.kv[0][s][0]) < TIGHT
        assert rel(r.kv[0][s][1], full.kv[0][s][1]) < TIGHT


def test_mixed_batch_sequences_do_not_interact():
    dims = tiny_dims()
    W = tiny_weights(dims)
    l, g = 2, 1
    ps = prompts_for(dims, [9, 14, 6], seed=11)
    # sequence 0: a prompt chunk with 4 cached positions; 1: a decode token
    # after 13; 2: a fresh prompt
    past0 = O.swiftkv_prefill(dims, W, [ps[0][:4]], l, g, dtype=np.float64).kv[0]
    past1 = O.swiftkv_prefill(dims, W, [ps[1][:13]], l, g, dtype=np.float64).kv[0]
    pasts, news = [past0, past1, {}], [ps[0][4:], ps[1][13:], ps[2]]
    both = O.swiftkv_step(dims, W, pasts, news, l, g, dtype=np.float64)
    for b in range(3):
        solo = O.swiftkv_step(dims, W, [pasts[b]], [news[b]], l, g, dtype=np.float64)
        assert np.array_equal(both.logits[b], solo.logits[0])
        for s in solo.kv[0]:
            assert np.array_equal(both.kv[b][s][0], solo.kv[0][s][0])
            assert np.array_equal(both.kv[b][s][1], solo.kv[0][s][1])


def test_attention_with_past_is_single_query_attention_per_row():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((5, 4, 8))
    k = rng.standard_normal((11, 2, 8))
    v = rng.standard_normal((11, 2, 8))
    pos = np.array([6, 7, 8, 9, 10])
    got = O.attention_with_past(q, k, v, pos, None)
    for i, p in enumerate(pos):
        ref = O.single_query_attention(q[i], k[:p + 1], v[:p + 1], None)
        assert rel(got[i], ref) < 1e-13


@pytest.mark.parametrize("l,g", [(0, 1), (2, 1), (1, 2), (4, 1)])
def test_step_flop_counter_matches_closed_form(l, g):
    dims = tiny_dims()
    W = tiny_weights(dims)
    ps = prompts_for(dims, [10, 7], seed=2)
    past0 = O.swiftkv_prefill(dims, W, [ps[0][:6]], l, g, dtype=np.float64).kv[0]
    r = O.swiftkv_step(dims, W, [past0, {}], [ps[0][6:], ps[1]], l, g, dtype=np.float64)
    assert r.flops == O.step_flops(dims, l, g, [6, 0], [4, 7])
    # without cached positions the step is a prefill
    assert O.step_flops(dims, l, g, [0, 0], [10, 7]) == O.prefill_flops(dims, l, g, [10, 7])[1]


def test_step_storage_hook_identity_is_plain():
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float32)
    ps = prompts_for(dims, [11, 5], seed=13)
    past = O.swiftkv_prefill(dims, W, [ps[0][:8]], 2, 1).kv[0]
    a = O.swiftkv_step(dims, W, [past, {}], [ps[0][8:], ps[1]], 2, 1)
    b = O.swiftkv_step(dims, W, [past, {}], [ps[0][8:], ps[1]], 2, 1, store=lambda t: t)
    assert np.array_equal(a.logits, b.logits)
