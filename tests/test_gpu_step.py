"""Mixed-batch steps on the GPU (skv_step) against the oracle's swiftkv_step.

A schedule is a list of calls; each call brings, for some sequences, their
next n tokens after what earlier calls cached (a prompt chunk, a whole
prompt, or a single decode token).  The GPU and the oracle run the same
schedule in lockstep; every call's logits rows and, at the end, every KV
slot of every sequence (all positions) are compared with the parity metric
max |gpu - oracle| / max |oracle|: 1e-4 for fp32 models, 2e-2 for bf16.

Batches of at most 32 new tokens (bf16) take the row path through layers
1..l; larger ones the tiled GEMMs and the MFMA attention with cached
prefixes.  The schedules below exercise both, chunk starts that are not
multiples of the 16-token block or the 64-key tile, single-token rows inside
large batches, and AcrossKV / l = 0 / l = L.
"""
import sys

import numpy as np
import pytest

import skv_inputs as si
from oracle import swiftkv_oracle as O
from tests.helpers import CachedLayers, dims_of, max_rel, oracle_weights, say

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def _say(*a):
    say(*a)


def fp8_kv_check(got, ref, tol=2e-2):
    """K/V of an FP8 cache against the oracle's FP8 values.  Bound per element:
    one E4M3 step (at the larger of the two values, in the scale of the token's row) + 2 tol max|oracle|.
    Derivation: the GPU's values before quantisation differ from the oracle's by at most the bf16 bar,
    e <= tol max|oracle| (the 16-bit cache's parity).  Quantisation then adds at most one step where the two
    land on neighbouring codes, and the row scale (row max / 448) moves by the row maximum's own error, which
    changes every dequantised element of the row by at most e as well.  The codes themselves are checked bit
    for bit against the oracle's quantiser separately.  Returns (ok, worst error / bound, max-relative error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = ref.shape[0]
    r = ref.reshape(n, -1)
    g = got.reshape(n, -1)
    sc = np.max(np.abs(r), axis=1, keepdims=True) / 448.0
    y = np.maximum(np.abs(r), np.abs(g)) / np.where(sc > 0, sc, 1.0)    # the larger binade of the two
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3)) * sc
    amax = float(np.max(np.abs(r))) if r.size else 0.0
    err = np.abs(g - r)
    worst = float(np.max(err / (step + 2 * tol * amax + 1e-30))) if r.size else 0.0
    return worst <= 1.0, worst, max_rel(got, ref)


# Logits with an FP8 cache: the bf16 bar plus one E4M3 step of the largest cached value (32 of 448, 1/14 of the
# row maximum), which a single key passes straight to the attention output when its code lands on the
# neighbouring value (the GPU quantises bf16 values computed in another order, so neighbouring codes occur).
FP8_LOGITS_TOL = 2e-2 + 1.0 / 14


def run_schedule(w, final_lengths, schedule, shuffle=True, label="", kv_fp8=False):
    import torch
    from swiftkv_prefill_skipping_amd import runner
    from tests.test_gpu_parity import gpu_kv
    batch = si.make_batch(w, lengths=list(final_lengths), shuffle=shuffle)
    B = len(final_lengths)
    max_new = max(sum(n for _, n in call) for call in schedule)
    cached = CachedLayers()
    model = runner.load_seeded_model(w, max_new, max(len(c) for c in schedule), int(max(final_lengths)),
                                     layer_hook=cached.hook, kv_fp8=kv_fp8)
    cache = runner.Cache(model, batch.num_blocks)
    W = oracle_weights(w, cached)
    dims = dims_of(w.shape)
    tol = TOL[w.dtype]
    ctx = [0] * B
    past = [{} for _ in range(B)]
    worst = 0.0
    logit_errs = []
    for ci, call in enumerate(schedule):
        seqs = [s for s, _ in call]
        runs = [batch.tokens[s][ctx[s]:ctx[s] + n] for s, n in call]
        assert all(len(r) == n for r, (_, n) in zip(runs, call)), "schedule runs past a prompt"
        _say(f"[step] {label} call {ci}: " + ", ".join(f"seq {s} ctx {ctx[s]} +{n}" for s, n in call))
        ds = runner.device_step(np.concatenate(runs), [n for _, n in call], [ctx[s] for s in seqs],
                                batch.block_tables[seqs])
        lg = runner.step(model, cache, ds)
        torch.cuda.synchronize()
        lg = lg.cpu().numpy()
        r = O.swiftkv_step(dims, W, [past[s] for s in seqs], runs, w.swiftkv_l, w.acrosskv_g, kv_fp8=kv_fp8)
        for i, (s, n) in enumerate(call):
            e = max_rel(lg[i], r.logits[i])
            worst = max(worst, e)
            logit_errs.append(e)
            assert e < (FP8_LOGITS_TOL if kv_fp8 else tol), f"{label} call {ci} seq {s} logits: {e:.3e}"
            past[s] = r.kv[i]
            ctx[s] += n
    assert ctx == [int(n) for n in final_lengths], "schedule must cover every prompt"
    for b in range(B):
        gkv = gpu_kv(cache, w, batch, b)
        assert set(gkv) == set(past[b])
        for s in gkv:
            for t, name in ((0, "K"), (1, "V")):
                if kv_fp8:
                    ok, e, mr = fp8_kv_check(gkv[s][t], past[b][s][t])
                    worst = max(worst, mr)
                    assert ok, f"{label} seq {b} slot {s} {name}: {e:.2f} of the bound (max-rel {mr:.3e})"
                    continue
                e = max_rel(gkv[s][t], past[b][s][t])
                worst = max(worst, e)
                assert e < tol, f"{label} seq {b} slot {s} {name}: {e:.3e}"
    _say(f"[step] {label}: worst max-rel error {worst:.3e} (bar {FP8_LOGITS_TOL if kv_fp8 else tol} on logits); "
         f"logits " + " ".join(f"{e:.1e}" for e in logit_errs))
    return model, cache


def test_chunked_prefill_large_batches_bf16():
    """Chunks of 40..150 tokens after cached prefixes of 0, 40, 100, 101 and 251 positions (tiled path), with a
    single-token row and a fresh prompt riding in one batch."""
    w = si.small_workload("step_chunks", l=2, g=1, lengths=(300, 77, 5), seed=41)
    sched = [[(0, 100), (1, 40)],
             [(0, 1), (1, 37), (2, 5)],
             [(0, 150)],
             [(0, 49)]]
    run_schedule(w, (300, 77, 5), sched, label="chunks")


@pytest.mark.parametrize("l,g", [(2, 1), (1, 2), (0, 1), (4, 1)], ids=["l2", "l1_g2", "l0", "lL"])
def test_decode_steps_bf16(l, g):
    """A prefill, then five decode steps of one token per sequence (row path through layers 1..l)."""
    w = si.small_workload(f"step_decode_{l}_{g}", l=l, g=g, lengths=(205, 134, 69), seed=43)
    sched = [[(0, 200), (1, 129), (2, 64)]] + [[(0, 1), (1, 1), (2, 1)]] * 5
    run_schedule(w, (205, 134, 69), sched, label=f"decode l={l} g={g}")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (8, 1)], ids=["rep4", "rep8"])
def test_decode_rows_either_side_of_the_single_pass_threshold(hq, hkv):
    """Decode rows whose contexts reach 1023 and 1024 keys (the longest the single-pass row attention takes) and
    then 1025 (the chunked kernel and its combine pass), with 4 or 8 query heads per kv head (one or two head
    groups per workgroup), against the oracle at every call."""
    w = si.small_workload(f"step_dec1_{hq}_{hkv}", n_layers=3, n_q_heads=hq, n_kv_heads=hkv, l=1, g=1,
                          lengths=(1025, 300), seed=53)
    sched = [[(0, 1022), (1, 297)]] + [[(0, 1), (1, 1)]] * 3
    run_schedule(w, (1025, 300), sched, label=f"single-pass threshold hq={hq} hkv={hkv}")


def test_row_path_chunks_and_decode_bf16():
    """Small mixed batches: a 20-token chunk with two decode tokens, a 32-token chunk (the largest row-path batch),
    then 33 tokens (the smallest tiled batch) after a cached prefix."""
    w = si.small_workload("step_rows", l=2, g=1, lengths=(135, 81, 34), seed=47)
    sched = [[(0, 50), (1, 80), (2, 33)],
             [(0, 20), (1, 1), (2, 1)],
             [(0, 32)],
             [(0, 33)]]
    run_schedule(w, (135, 81, 34), sched, label="rows")


def test_chunks_and_decode_fp32():
    w = si.small_workload("step_fp32", n_layers=5, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn_dim=176,
                          vocab=512, dtype="fp32", l=2, g=2, lengths=(90, 41), seed=49)
    sched = [[(0, 30), (1, 40)],
             [(0, 55), (1, 1)],
             [(0, 1)],
             [(0, 4)]]
    run_schedule(w, (90, 41), sched, label="fp32")


def test_step_host_side_errors():
    import torch
    from swiftkv_prefill_skipping_amd import _lib as L, runner
    w = si.small_workload("step_errs", l=1, g=1, lengths=(40, 20), seed=53)
    batch = si.make_batch(w)
    model = runner.load_seeded_model(w, 64, 2, 48)
    cache = runner.Cache(model, batch.num_blocks)
    logits = torch.empty((2, w.shape.vocab), dtype=torch.float32, device="cuda")
    toks = np.zeros(2, dtype=np.int32)

    def call(ctx, bt=batch.block_tables):
        ds = runner.device_step(toks, [1, 1], ctx, bt)
        L.skv_step(model.handle, cache.handle, ds.struct, logits.data_ptr(), 0)
        return ds

    with pytest.raises(L.SkvError):
        call([48, 0])                          # position 48 is past max_seqlen 48
    with pytest.raises(L.SkvError):
        call([-1, 0])                          # negative cached length
    with pytest.raises(L.SkvError):
        call([0, 32])                          # sequence 1 would need a third block; its table has two
    ds = runner.device_step(toks, [1, 1], [3, 3], batch.block_tables)
    half = L.skv_step_batch(ds.struct.tokens, ds.ctx_host.ctypes.data, 0)
    with pytest.raises(L.SkvError):            # only one of the two ctx arrays
        L.skv_step(model.handle, cache.handle, half, logits.data_ptr(), 0)
    call([3, 3])                               # a good call still works
    torch.cuda.synchronize()


@pytest.mark.parametrize("l,g,kv_fp8", [(2, 2, False), (1, 1, True)])
def test_unfinished_chunks_skip_the_deep_layers(l, g, kv_fp8):
    """A call whose sequences are all prompt chunks that more chunks follow (need_logits_host all 0) stops
    after layer l and writes no logits: only a prompt's last token runs the layers past l.  The same chunk
    schedule with and without the marks leaves a bitwise-identical cache and bitwise-identical logits in
    the calls that end prompts, and the all-unfinished call leaves its logits buffer untouched."""
    import torch
    from swiftkv_prefill_skipping_amd import runner
    from tests.test_gpu_parity import gpu_kv
    lengths = (300, 170, 150)  # chunks of 100: the first call ends no prompt
    w = si.small_workload(f"unfinished_l{l}_g{g}", l=l, g=g, lengths=lengths, seed=61)
    batch = si.make_batch(w, shuffle=True)
    chunk = 100
    model = runner.load_seeded_model(w, chunk * len(lengths), len(lengths), max(lengths), kv_fp8=kv_fp8)
    caches, ended = [], []
    skipped = 0
    for marked in (False, True):
        cache = runner.Cache(model, batch.num_blocks)
        ctx = np.zeros(len(lengths), dtype=np.int64)
        rows = {}
        while (ctx < batch.lengths).any():
            live = [b for b in range(len(lengths)) if ctx[b] < batch.lengths[b]]
            ns = [int(min(chunk, batch.lengths[b] - ctx[b])) for b in live]
            toks = np.concatenate([batch.tokens[b][ctx[b]:ctx[b] + n] for b, n in zip(live, ns)])
            ends = [int(ctx[b] + n == batch.lengths[b]) for b, n in zip(live, ns)]
            ds = runner.device_step(toks, ns, ctx[live], batch.block_tables[live], ends if marked else None)
            lg = torch.full((len(live), w.shape.vocab), 7.0, dtype=torch.float32, device="cuda")
            runner.step(model, cache, ds, lg)
            torch.cuda.synchronize()
            if marked and not any(ends):
                skipped += 1
                assert bool((lg == 7.0).all()), "a call of unfinished chunks wrote logits"
            for i, (b, e) in enumerate(zip(live, ends)):
                if e:
                    rows[b] = lg[i].clone()
            ctx[live] += ns
        caches.append(cache)
        ended.append(rows)
    assert skipped == 1
    _say(f"[case] unfinished chunks l={l} g={g} fp8={kv_fp8}")
    for b in range(len(lengths)):
        assert torch.equal(ended[0][b], ended[1][b]), b
        k0 = gpu_kv(caches[0], w, batch, b)
        k1 = gpu_kv(caches[1], w, batch, b)
        for s_ in k0:
            assert np.array_equal(k0[s_][0], k1[s_][0]) and np.array_equal(k0[s_][1], k1[s_][1]), (b, s_)


def test_need_logits_host_rules():
    """Some sequence needing logits with a NULL logits pointer is an argument error, checked before any work."""
    import torch
    from swiftkv_prefill_skipping_amd import _lib as L, runner
    w = si.small_workload("need_rules", l=1, g=1, lengths=(40, 20), seed=67)
    batch = si.make_batch(w)
    model = runner.load_seeded_model(w, 64, 2, 48)
    cache = runner.Cache(model, batch.num_blocks)
    toks = np.zeros(2, dtype=np.int32)
    ds = runner.device_step(toks, [1, 1], [3, 3], batch.block_tables, [0, 1])
    with pytest.raises(L.SkvError) as e:
        L.skv_step(model.handle, cache.handle, ds.struct, 0, 0)
    assert e.value.status == L.SKV_ERR_INVALID_ARG
    ds0 = runner.device_step(toks, [1, 1], [3, 3], batch.block_tables, [0, 0])
    L.skv_step(model.handle, cache.handle, ds0.struct, 0, 0)
    torch.cuda.synchronize()
