"""HIP path vs oracle at the workloads' full sizes (needs a gfx950 GPU).

The GPU runs each whole batch in the launch configuration bench.py times.
Expected values come from two sources, both the CPU oracle:
  * tests/golden/fullsize/<workload>.npz, written on the CPU by
    tests/golden/make_fullsize_fixtures.py (calls oracle/ only): last-token
    logits of a seeded set of prompts (all 16 of the 8B l=16 batch), K/V of
    every slot at seeded positions (the 32768-token prompt: 24 positions from
    0 to 32767; the 70B batch: 4 prompts), and for every compared tensor its
    floor (how far the oracle's bf16-storage evaluation is from its plain
    one over the same elements);
  * a live run of the plain oracle here on a few prompts (every slot, every
    position) where it finishes in seconds.
Bar per tensor (tests/test_gpu_parity.judge): max |gpu - oracle| / max
|oracle| < 2e-2, or, where the tensor's own CPU floor is at least 2e-2 (deep
layers of these random-init models), within 1.2x of that floor (and 1.1x +
1e-3 on the Frobenius ratio).  Prompts are independent, so the oracle runs
on a subset of a batch alone.
"""
import time

import numpy as np
import pytest

import skv_inputs as si
from oracle import swiftkv_oracle as O
from tests.helpers import CachedLayers, dims_of, fullsize_fixture, max_rel, oracle_weights, say
from tests.test_gpu_parity import Tally, compare, frob_rel, gpu_kv, judge, run_gpu

pytestmark = pytest.mark.gpu

TOL = 2e-2


def round_bf16(x):
    return si.bf16_to_f32(si.f32_to_bf16(np.ascontiguousarray(x, dtype=np.float32))).reshape(x.shape)


def _say(*a):
    say(*a)


def _fixture(name):
    fx = fullsize_fixture(name)
    assert fx is not None, f"tests/golden/fullsize/{name}.npz is missing (tests/golden/make_fullsize_fixtures.py)"
    return fx


def _full_floors(fx, nslots):
    """(prompt, slot, t) -> floor over the leading positions a live oracle run compares, plus logits floors."""
    fl = {}
    for ri, b in enumerate(fx["full_prompts"]):
        for s in range(nslots):
            for t in (0, 1):
                fl[(int(b), s, t)] = fx["full_floor"][ri, s, t]
    for pi, b in enumerate(fx["prompts"]):
        fl[(int(b), "logits")] = fx["logits_floor"][pi]
    return fl


def check_against_fixture(w, batch, logits, cache, fx, label):
    """Every stored logits row and every stored K/V sample against the GPU's."""
    from swiftkv_prefill_skipping_amd import runner
    tally = Tally(f"{label} (stored oracle results)", TOL)
    lines = []
    lg = logits.float().cpu().numpy()
    row = []
    for pi, b in enumerate(fx["prompts"]):
        row.append(f"{int(b)}:" + tally.check(lg[int(b)], fx["logits"][pi], fx["logits_floor"][pi],
                                                f"prompt {int(b)} logits"))
    lines.append("  logits by prompt: " + " ".join(row))
    L_, l, g = w.shape.n_layers, w.swiftkv_l, w.acrosskv_g
    if len(fx["kv_prompts"]):
        layer_of_slot = {}
        for j in range(1, L_ + 1):
            layer_of_slot.setdefault(O.slot_of_layer(j, L_, l, g), j)
        tables = {s: cache.read_layer(j) for s, j in layer_of_slot.items()}
        for qi, b in enumerate(fx["kv_prompts"]):
            b = int(b)
            pos = fx["kv_pos"][qi]
            n = int(batch.lengths[b])
            assert pos.max() < n
            row = []
            for s in sorted(tables):
                kt, vt = tables[s]
                k, v = runner.logical_kv(kt, vt, batch.block_tables[b], n)
                ek = tally.check(k[pos], fx["kv"][qi, s, 0], fx["kv_floor"][qi, s, 0], f"prompt {b} slot {s} K")
                ev = tally.check(v[pos], fx["kv"][qi, s, 1], fx["kv_floor"][qi, s, 1], f"prompt {b} slot {s} V")
                row.append(f"{s}:{ek}/{ev}")
            lines.append(f"  prompt {b} K/V at positions {list(pos)}: " + " ".join(row))
    return tally.finish(lines)


def _run_full(name, live_prompts):
    import torch
    w = si.WORKLOADS[name]
    batch = si.make_batch(w)
    fx = _fixture(name)
    assert [int(b) for b in fx["full_prompts"]] == list(live_prompts)
    t0 = time.time()
    cached = CachedLayers()
    model, cache, db, logits = run_gpu(w, batch, cached=cached)
    assert torch.isfinite(logits).all()
    _say(f"[full] {name}: GPU prefill of {batch.total_tokens} tokens done ({time.time() - t0:.1f} s); live oracle on "
         f"prompts {list(live_prompts)} (lengths {[int(batch.lengths[b]) for b in live_prompts]})")
    check_against_fixture(w, batch, logits, cache, fx, name)
    if live_prompts:
        t1 = time.time()
        toks = [batch.tokens[b] for b in live_prompts]
        ores = O.swiftkv_prefill(dims_of(w.shape), oracle_weights(w, cached), toks, w.swiftkv_l, w.acrosskv_g)
        _say(f"[full] live oracle done ({time.time() - t1:.1f} s)")
        nslots = O.kv_slots(w.shape.n_layers, w.swiftkv_l, w.acrosskv_g)
        compare(w, batch, logits, cache, ores, list(live_prompts), tol=TOL, label=f"{name} (live oracle)",
                floors=_full_floors(fx, nslots))
    return model, cache, batch


def test_llama8b_l16_b16():
    """8B shape, l=16, 16 prompts of 500-1000 tokens (the bench workload): every prompt's logits and, for the
    shortest and the longest prompt, every slot's K/V at every position."""
    _run_full("llama8b_l16_b16", [3, 12])


def test_llama8b_l24_acrosskv4_b32():
    """8B shape, l=24 with 4-way AcrossKV (2 shared KV tensors for layers 25-32), 32 x 1000 tokens: logits of
    prompts 0, 11, 20 and 31, every slot's whole K/V of prompts 0 and 31, K/V samples of prompts 11 and 20."""
    _run_full("llama8b_l24_g4_b32", [0, 31])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_llama70b_l40_b32():
    """70B shape (80 layers, d=8192, 64/8 heads, f=28672) on one GPU, l=40, 32 prompts x 1000 tokens: logits of
    prompts 0, 5, 19 and 31 and every slot's K/V at 4 positions of each (stored oracle results)."""
    _run_full("llama70b_l40_b32", [])


def _logical_device(kt, vt, block_row, n):
    """One prompt's K and V in position order, on the device (no host copy)."""
    import torch
    bs = kt.shape[2]
    nb = -(-n // bs)
    idx = torch.as_tensor(np.asarray(block_row[:nb], dtype=np.int64), device=kt.device)
    k = kt.index_select(0, idx).permute(0, 2, 1, 3).reshape(nb * bs, kt.shape[1], kt.shape[3])[:n]
    v = vt.index_select(0, idx).permute(0, 2, 1, 3).reshape(nb * bs, vt.shape[1], vt.shape[3])[:n]
    return k, v


def test_llama8b_l16_long32k():
    """8B shape, l=16, one 32768-token prompt in shuffled 16-token blocks: its logits and every slot's K/V at 24
    positions from 0 to 32767 against the stored oracle results, positions < 1024 of every slot against a live
    oracle run on the 1024-token prefix, and the paging bitwise against an identity block order."""
    import torch
    from swiftkv_prefill_skipping_amd import runner
    name = "llama8b_l16_long32k"
    w = si.WORKLOADS[name]
    batch = si.make_batch(w)
    assert w.shuffle_blocks and batch.total_tokens == 32768
    fx = _fixture(name)
    t0 = time.time()
    cached = CachedLayers()
    model, cache, db, logits = run_gpu(w, batch, cached=cached)
    _say(f"[full] {name}: GPU prefill of {batch.total_tokens} tokens done ({time.time() - t0:.1f} s)")
    assert torch.isfinite(logits).all()
    check_against_fixture(w, batch, logits, cache, fx, name)

    # the same prompt in identity block order: bitwise the same logical KV and logits
    batch_id = si.make_batch(w, shuffle=False)
    assert not np.array_equal(batch_id.block_tables, batch.block_tables)
    cache_id = runner.Cache(model, batch_id.num_blocks)
    logits_id = runner.prefill(model, cache_id, runner.device_batch(batch_id))
    torch.cuda.synchronize()
    assert torch.equal(logits, logits_id), "logits depend on the physical block order"
    n = int(batch.lengths[0])
    seen = set()
    for j in range(1, w.shape.n_layers + 1):
        s_ = O.slot_of_layer(j, w.shape.n_layers, w.swiftkv_l, w.acrosskv_g)
        if s_ in seen:
            continue
        seen.add(s_)
        ka, va = _logical_device(*cache.read_layer(j), batch.block_tables[0], n)
        kb, vb = _logical_device(*cache_id.read_layer(j), batch_id.block_tables[0], n)
        assert torch.equal(ka, kb) and torch.equal(va, vb), f"slot {s_}: KV depends on the physical block order"
        assert torch.isfinite(ka.float()).all() and torch.isfinite(va.float()).all()
    _say(f"[full] {name}: shuffled and identity paging agree bitwise on {len(seen)} slots and the logits")
    del cache_id

    P = int(fx["full_npos"][0])
    t1 = time.time()
    ores = O.swiftkv_prefill(dims_of(w.shape), oracle_weights(w, cached), [batch.tokens[0][:P]], w.swiftkv_l,
                             w.acrosskv_g)
    _say(f"[full] live oracle on the {P}-token prefix done ({time.time() - t1:.1f} s)")
    nslots = O.kv_slots(w.shape.n_layers, w.swiftkv_l, w.acrosskv_g)
    compare(w, batch, logits, cache, ores, [0], tol=TOL, label=f"{name} (positions < {P})",
            floors=_full_floors(fx, nslots), npos=P)


def test_llama8b_decode_step_and_fp8_cache_sampled():
    """The bench workload's decode step and FP8 cache at full size: the whole batch prefilled on the GPU, one
    decode token per prompt (skv_step); the shortest prompt's decode logits against the oracle's step after its
    prefill.  Then the same batch with the per-token FP8 cache: that prompt's prefill logits and the K/V of four
    slots against the oracle with the FP8 cache.  The floors (the oracle's bf16-storage evaluations of the same
    step and of the FP8 prefill) are computed here on the host."""
    import torch
    from swiftkv_prefill_skipping_amd import runner
    from tests.test_gpu_step import FP8_LOGITS_TOL, fp8_kv_check
    w = si.WORKLOADS["llama8b_l16_b16"]
    batch = si.make_batch(w)
    B = len(batch.lengths)
    b = int(np.argmin(batch.lengths))
    extra = 2
    bt = np.full((B, batch.block_tables.shape[1] + extra), -1, dtype=np.int32)
    for i, ln in enumerate(batch.lengths):
        nb = -(-int(ln) // 16)
        bt[i, :nb] = batch.block_tables[i, :nb]
        bt[i, nb:nb + extra] = batch.num_blocks + i * extra + np.arange(extra)
    nxt = si.randint(w.input_seed, 7, B, w.shape.vocab)
    dims = dims_of(w.shape)
    t0 = time.time()
    cached = CachedLayers()
    model = runner.load_seeded_model(w, batch.total_tokens, B, batch.max_seqlen + 16 * extra, layer_hook=cached.hook)
    cache = runner.Cache(model, batch.num_blocks + B * extra)
    db = runner.device_batch(batch)
    ds = runner.device_step(nxt, [1] * B, batch.lengths, bt)
    runner.prefill(model, cache, db)
    lg = runner.step(model, cache, ds)
    torch.cuda.synchronize()
    lg = lg.cpu().numpy()
    assert np.isfinite(lg).all()
    _say(f"[full] decode step of {B} tokens after the prefill done ({time.time() - t0:.1f} s); oracle on prompt {b}")
    W = oracle_weights(w, cached)
    res = {}
    for mode, store in (("fp32", None), ("bf16-storage", round_bf16)):
        kw = {} if store is None else {"store": store}
        pre = O.swiftkv_prefill(dims, W, [batch.tokens[b]], w.swiftkv_l, w.acrosskv_g, **kw)
        res[mode] = O.swiftkv_step(dims, W, [pre.kv[0]], [nxt[b:b + 1]], w.swiftkv_l, w.acrosskv_g, **kw)
    ref, st = res["fp32"].logits[0], res["bf16-storage"].logits[0]
    floor = (max_rel(st, ref), frob_rel(st, ref))
    e, fg = max_rel(lg[b], ref), frob_rel(lg[b], ref)
    verdict = judge(e, fg, floor, TOL)
    _say(f"[full] decode logits of prompt {b}: {e:.3e} (floor {floor[0]:.3e}; frob {fg:.3e} vs {floor[1]:.3e}): "
         f"{verdict}")
    assert verdict != "fail", (e, fg, floor)
    model.close()
    cache.close()

    t1 = time.time()
    m8 = runner.load_seeded_model(w, batch.total_tokens, B, batch.max_seqlen, kv_fp8=True)
    c8 = runner.Cache(m8, batch.num_blocks)
    lg8 = runner.prefill(m8, c8, db)
    torch.cuda.synchronize()
    lg8 = lg8.cpu().numpy()
    _say(f"[full] FP8-cache prefill done ({time.time() - t1:.1f} s)")
    o8 = O.swiftkv_prefill(dims, W, [batch.tokens[b]], w.swiftkv_l, w.acrosskv_g, kv_fp8=True)
    o8b = O.swiftkv_prefill(dims, W, [batch.tokens[b]], w.swiftkv_l, w.acrosskv_g, kv_fp8=True, store=round_bf16)
    floor8 = (max_rel(o8b.logits[0], o8.logits[0]), frob_rel(o8b.logits[0], o8.logits[0]))
    e8, f8 = max_rel(lg8[b], o8.logits[0]), frob_rel(lg8[b], o8.logits[0])
    verdict8 = judge(e8, f8, floor8, FP8_LOGITS_TOL)
    _say(f"[full] FP8 prefill logits of prompt {b}: {e8:.3e} (floor {floor8[0]:.3e}; frob {f8:.3e} vs "
         f"{floor8[1]:.3e}; bar {FP8_LOGITS_TOL:.3e}): {verdict8}")
    assert verdict8 != "fail", (e8, f8, floor8)
    gkv = gpu_kv(c8, w, batch, b)
    for s in (0, w.swiftkv_l - 1, w.swiftkv_l, max(gkv)):
        for t, name in ((0, "K"), (1, "V")):
            # the per-element FP8 bound is built on the bf16 bar; where the tensor's own bf16-storage floor is above
            # the bar, the floor takes its place
            fl = max_rel(o8b.kv[0][s][t], o8.kv[0][s][t])
            tol = fl if fl >= TOL else TOL
            ok, r, mr = fp8_kv_check(gkv[s][t], o8.kv[0][s][t], tol=tol)
            _say(f"[full] FP8 slot {s} {name}: {r:.2f} of the bound (max-rel {mr:.2e}, floor {fl:.2e}, tol {tol:.2e})")
            assert ok, (s, name, r, mr)


def test_small_model_long_context():
    """Attention over long prompts against the full oracle: a 3-layer model (d=512, 8/2 heads of 128, l=2) on an
    8192-token and a 3000-token prompt; every KV slot and both logits rows (the last token attends over all keys of
    the skipped layer)."""
    w = si.small_workload("long8k", n_layers=3, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn_dim=512,
                          vocab=1024, l=2, g=1, lengths=(8192, 3000), seed=31, weight_seed=131)
    batch = si.make_batch(w)
    model, cache, db, logits = run_gpu(w, batch)
    ores = O.swiftkv_prefill(dims_of(w.shape), oracle_weights(w), batch.tokens, w.swiftkv_l, w.acrosskv_g)
    compare(w, batch, logits, cache, ores, [0, 1], tol=TOL, label=w.name)


def test_attention_forms_either_side_of_the_short_prompt_threshold():
    """Prompt attention has a 4-wave form for batches whose sequences bring at most 2048 new tokens and the
    8-wave form above that: a batch at the threshold (2048 and 700 tokens) and one just past it (2049 and
    700), each against the oracle, every KV slot and the logits, on the 3-layer model with 128-dim heads."""
    for lengths in ((2048, 700), (2049, 700)):
        w = si.small_workload(f"attn_forms_{lengths[0]}", n_layers=3, d_model=512, n_q_heads=8, n_kv_heads=2,
                              head_dim=128, ffn_dim=512, vocab=1024, l=2, g=1, lengths=lengths, seed=41,
                              weight_seed=141)
        batch = si.make_batch(w)
        model, cache, db, logits = run_gpu(w, batch)
        ores = O.swiftkv_prefill(dims_of(w.shape), oracle_weights(w), batch.tokens, w.swiftkv_l, w.acrosskv_g)
        compare(w, batch, logits, cache, ores, [0, 1], tol=TOL, label=w.name)


def test_midsize_split_tail_gemms():
    """d_model 4096 over 5000 tokens: the O, gate/up and down GEMMs have 320 tiles on 256 CUs, so their
    last wave runs as K-split partial tiles plus the fixed-order reduction."""
    w = si.small_workload("midsize", n_layers=2, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                          ffn_dim=2048, vocab=2048, l=1, g=1, lengths=(500,) * 10, seed=21, weight_seed=121)
    batch = si.make_batch(w)
    model, cache, db, logits = run_gpu(w, batch)
    ores = O.swiftkv_prefill(dims_of(w.shape), oracle_weights(w), [batch.tokens[b] for b in (0, 7)], w.swiftkv_l,
                             w.acrosskv_g)
    compare(w, batch, logits, cache, ores, [0, 7], tol=TOL, label=w.name)
