"""Throughput of the SwiftKV prefill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-full-depth]
                    [--no-decode] [--no-fp8] [--no-mfma-probe] [--no-vendor-gemm]
    python bench.py --copy-calibration MIB   # plain device copy of known size, for HBM counter scaling

One step = one skv_prefill call over the whole batch (every row of the hot
path: layers 1..l for all prompt tokens, the fused skipped-layer KV GEMM,
the last-token path through layers l+1..L and the LM head), inputs and
weights already resident in HBM.  Prints one JSON line.  The same batch is
then also timed through the unmodified model (l = L, same kernels), so the
line carries the SwiftKV / full-depth wall-clock ratio next to the FLOP ratio,
and (bf16) through skv_step: one decode token per prompt after its prefill
(weight-streaming, HBM-bound) and the same prompts prefilled in chunks of 256
tokens per prompt per call; finally prefill and decode with a per-token FP8
KV cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tok/s + normalized TFLOPs (full-depth FLOPs/s), 8B & 70B SwiftKV-50%"
MI355X_BF16_DENSE_TFLOPS = 2500.0   # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU (dense, no sparsity)
MI355X_HBM_GBS = 8000.0


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemm_bf16_hbm_traffic_llama8b_l16_b16.md")


def measured_traffic(kernel_key: str):
    """HBM-side bytes per launch of one GEMM kernel from the committed counter record, or None.

    The record holds FETCH_SIZE / WRITE_SIZE per dispatch scaled by a copy
    kernel of known size; it is used only while the GEMM sources still hash to
    the value it was taken with.
    """
    import hashlib
    try:
        text = open(TRAFFIC_RECORD).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        csrc = os.path.join(ROOT, "swiftkv_prefill_skipping_amd", "csrc")
        sha = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in rec["files"])).hexdigest()
        if sha != rec["source_sha256"]:
            return None
        k = rec["kernels"][kernel_key]
        return {"read_bytes": k["read_bytes_per_launch"], "write_bytes": k["write_bytes_per_launch"],
                "bytes": k["read_bytes_per_launch"] + k["write_bytes_per_launch"], "unit": "bytes/launch"}
    except (OSError, IndexError, KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(workload, batch, cached, n_prompts=3):
    """Time the oracle on the host cores over the batch's three shortest prompts (10-15 s of work at the 8B shape)."""
    from threadpoolctl import threadpool_info
    import skv_inputs as si
    from oracle import swiftkv_oracle as O
    sel = [int(b) for b in np.argsort(batch.lengths, kind="stable")[:n_prompts]]
    s = workload.shape
    dims = O.Dims(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn_dim, s.vocab, s.rope_theta,
                  s.rms_eps)
    gw = si.global_weights(s, workload.dtype)
    W = O.LazyWeights(si.as_f32(gw["embed"]), si.as_f32(gw["final_norm"]), si.as_f32(gw["lm_head"]), cached.make)
    t0 = time.perf_counter()
    r = O.swiftkv_prefill(dims, W, [batch.tokens[b] for b in sel], workload.swiftkv_l, workload.acrosskv_g)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    n = int(sum(int(batch.lengths[b]) for b in sel))
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "flops": r.flops, "gflops_per_s": round(r.flops / dt / 1e9, 1),
            "sample": f"prompts {sel} of the batch ({n} tokens) through the whole path, fp32 NumPy oracle, "
                      f"{dt:.1f} s wall, {r.flops / 1e12:.2f} TFLOP counted by the oracle"}


def copy_calibration(mib: int):
    """Three launches of one elementwise kernel that reads and writes `mib` MiB each."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"launches": 3, "bytes_read_per_launch": n * 4,
                                           "bytes_written_per_launch": n * 4}}), flush=True)


def decode_tables(batch, extra: int):
    """Block tables of the batch with `extra` fresh blocks appended to every prompt's row (ids after the
    prefill's), so decode tokens after the prompts have room."""
    B = len(batch.lengths)
    bs = batch.block_size
    width = max(-(-int(n) // bs) for n in batch.lengths) + extra
    bt = np.full((B, width), -1, dtype=np.int32)
    for b, n in enumerate(batch.lengths):
        nb = -(-int(n) // bs)
        bt[b, :nb] = batch.block_tables[b, :nb]
        bt[b, nb:nb + extra] = batch.num_blocks + b * extra + np.arange(extra)
    return bt


def decode_bytes(cfg, ctx_lens) -> float:
    """Algorithmic HBM bytes of one SwiftKV decode step (bf16): every weight read once (layers 1..l with their
    K/V rows, layers l+1..L with Q only, the folded skipped-layer K/V rows, the LM head) plus every cached K/V
    row the new tokens attend to."""
    d, dh, hq, hkv, f, V = cfg.d_model, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.ffn_dim, cfg.vocab
    L, l, g = cfg.n_layers, cfg.swiftkv_l, cfg.acrosskv_g
    dq, dkv = hq * dh, hkv * dh
    G = -(-(L - l) // g)
    w = l * d * (dq + 2 * dkv) + (L - l) * d * dq + G * 2 * dkv * d + L * (dq * d + 3 * d * f) + V * d
    kv = L * sum(int(c) + 1 for c in ctx_lens) * 2 * dkv
    return 2.0 * (w + kv)


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def vendor_gemm(M, N, K, ours_ms, reps=10):
    """The vendor library's bf16 GEMM (torch.matmul -> hipBLASLt, plain bf16 output) on the dominant GEMM's
    shape, next to the library's own call of that GEMM (with its fused epilogue), on the same GPU: context for
    the roofline fraction, not part of the timed step."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(11)
    a = ((torch.rand(M, K, device="cuda", generator=g) - 0.5) * 0.07).to(torch.bfloat16)
    b = ((torch.rand(N, K, device="cuda", generator=g) - 0.5) * 0.07).to(torch.bfloat16)
    bt = b.t()
    for _ in range(3):
        c = a @ bt
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ bt
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, bt, c
    torch.cuda.empty_cache()
    tf = 2.0 * M * N * K / (ms / 1e3) / 1e12
    return {"library": "hipBLASLt (torch.matmul, bf16 in and out, no epilogue)", "M": M, "N": N, "K": K,
            "ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / MI355X_BF16_DENSE_TFLOPS, 4),
            "ours_ms_with_epilogue": round(ours_ms, 4), "ours_vs_vendor_time": round(ours_ms / ms, 4)}


def measure_decode(model, cache, w, batch, extra, logits, stream, args):
    """One decode token per prompt at position N_b (context N_b + 1), the same step repeated."""
    import skv_inputs as si
    from swiftkv_prefill_skipping_amd import runner
    B = len(batch.lengths)
    dbt = decode_tables(batch, extra)
    nxt = si.randint(w.input_seed, 7, B, w.shape.vocab)
    ds = runner.device_step(nxt, [1] * B, batch.lengths, dbt)
    ms_dec = time_calls(lambda: runner.step(model, cache, ds, logits, stream), args.steps, args.warmup, stream)
    by = decode_bytes(model.cfg, batch.lengths)
    log(f"[bench] decode step ({B} tokens): {ms_dec:.3f} ms")
    return {"tokens": B, "context_tokens": int(sum(batch.lengths)) + B, "ms_per_step": round(ms_dec, 4),
            "tokens_per_s": round(B / (ms_dec / 1e3), 1), "bound": "hbm", "algorithmic_bytes": by,
            "achieved_GBs": round(by / (ms_dec / 1e3) / 1e9, 1), "peak_GBs": MI355X_HBM_GBS,
            "frac": round(by / (ms_dec / 1e3) / 1e9 / MI355X_HBM_GBS, 4)}


def measure_chunked(model, cache, w, batch, stream, args, ms_one_shot, swift_flops, chunk=256):
    """The batch's prompts prefilled through skv_step, at most `chunk` tokens per prompt per call."""
    import torch
    from swiftkv_prefill_skipping_amd import runner
    B, T = len(batch.lengths), batch.total_tokens
    calls, ctx = [], np.zeros(B, dtype=np.int64)
    while (ctx < batch.lengths).any():
        live = [b for b in range(B) if ctx[b] < batch.lengths[b]]
        ns = [int(min(chunk, batch.lengths[b] - ctx[b])) for b in live]
        toks = np.concatenate([batch.tokens[b][ctx[b]:ctx[b] + n] for b, n in zip(live, ns)])
        # logits only where the chunk ends its prompt: a call of unfinished chunks alone stops after layer l
        need = [int(ctx[b] + n == batch.lengths[b]) for b, n in zip(live, ns)]
        calls.append(runner.device_step(toks, ns, ctx[live], batch.block_tables[live], need))
        ctx[live] += ns
    lgc = [torch.empty((c.struct.tokens.batch, w.shape.vocab), dtype=torch.float32, device="cuda") for c in calls]

    def chunked():
        for c, lg in zip(calls, lgc):
            runner.step(model, cache, c, lg, stream)
    ms_ch = time_calls(chunked, args.steps, args.warmup, stream)
    log(f"[bench] chunked prefill ({len(calls)} calls of <= {chunk} tokens per prompt): {ms_ch:.3f} ms")
    return {"chunk_tokens_per_prompt": chunk, "calls": len(calls), "ms_per_prefill": round(ms_ch, 4),
            "tokens_per_s": round(T / (ms_ch / 1e3), 1), "time_vs_one_shot": round(ms_ch / ms_one_shot, 4),
            "actual_tflops": round(swift_flops / (ms_ch / 1e3) / 1e12, 2)}


def measure_fp8(w, batch, db, logits, stream, args, extra, ms_bf16, dec_bf16):
    """The same batch with a per-token FP8 KV cache: prefill and decode step times, KV bytes."""
    import torch
    from swiftkv_prefill_skipping_amd import runner
    T, B = batch.total_tokens, len(batch.lengths)
    t0 = time.time()
    m8 = runner.load_seeded_model(w, T, B, batch.max_seqlen + extra * batch.block_size, kv_fp8=True)
    c8 = runner.Cache(m8, batch.num_blocks + B * extra)
    log(f"[bench] FP8-cache model loaded in {time.time() - t0:.1f} s")
    ms8 = time_calls(lambda: runner.prefill(m8, c8, db, logits, stream), args.steps, args.warmup, stream)
    log(f"[bench] FP8 KV cache: prefill {ms8:.3f} ms/step")
    out = {"ms_per_step": round(ms8, 4), "tokens_per_s": round(T / (ms8 / 1e3), 1),
           "time_vs_bf16_cache": round(ms8 / ms_bf16, 4)}
    if dec_bf16 is not None:
        runner.prefill(m8, c8, db, logits, stream)
        d8 = measure_decode(m8, c8, w, batch, extra, logits, stream, args)
        out["decode_ms_per_step"] = d8["ms_per_step"]
        out["decode_time_vs_bf16_cache"] = round(d8["ms_per_step"] / dec_bf16["ms_per_step"], 4)
    s = w.shape
    slots = w.swiftkv_l + -(-(s.n_layers - w.swiftkv_l) // w.acrosskv_g)
    per_tok_bf16 = slots * 2 * s.n_kv_heads * s.head_dim * 2
    per_tok_fp8 = slots * 2 * (s.n_kv_heads * s.head_dim + 4)
    out["kv_bytes_per_token"] = {"bf16": per_tok_bf16, "fp8_with_scales": per_tok_fp8,
                                 "full_model_bf16": s.n_layers * 2 * s.n_kv_heads * s.head_dim * 2}
    c8.close()
    m8.close()
    return out


# dominant kernel class of each workload's step (the one its roofline object covers)
DOMINANT = {"llama8b_l16_b16": "gemm_gateup", "llama8b_l24_g4_b32": "gemm_gateup", "llama70b_l40_b32": "gemm_gateup",
            "llama8b_l16_long32k": "attn_prefill", "tiny_fp32_l2": "gemm_gateup"}
KERNEL_TEXT = {"gemm_gateup": "gemm_gateup (bf16 MFMA GEMM + SwiGLU epilogue)",
               "attn_prefill": "attn_prefill8 (causal GQA flash attention, bf16 MFMA; plain form: every layer but layer 1)"}


def measure_workload(name, steps, warmup, stream):
    """Load one workload's model, time `steps` prefill steps of its batch (after `warmup`), with HIP events on the
    launch stream around every launch of its dominant kernel class.  Returns its sub-object of the JSON line."""
    import torch
    import skv_inputs as si
    from swiftkv_prefill_skipping_amd import _lib as L, runner
    w = si.WORKLOADS[name]
    batch = si.make_batch(w)
    T, B = batch.total_tokens, len(batch.lengths)
    t0 = time.time()
    model = runner.load_seeded_model(w, T, B, batch.max_seqlen)
    cache = runner.Cache(model, batch.num_blocks)
    db = runner.device_batch(batch)
    logits = torch.empty((B, w.shape.vocab), dtype=torch.float32, device="cuda")
    log(f"[bench] {name}: {B} prompts, {T} tokens; model loaded in {time.time() - t0:.1f} s")
    for _ in range(warmup):
        runner.prefill(model, cache, db, logits, stream)
    torch.cuda.synchronize()
    dom = DOMINANT[name]
    L.skv_profile_enable(model.handle, L.KERNEL_CLASS_NAMES.index(dom), True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        runner.prefill(model, cache, db, logits, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    prof = L.skv_profile_read(model.handle)
    L.skv_profile_enable(model.handle, L.KERNEL_CLASS_NAMES.index(dom), False)
    ms = e0.elapsed_time(e1) / steps
    assert torch.isfinite(logits).all()
    full, swift = L.skv_flops(model.cfg, batch.lengths)
    t = ms / 1e3
    avg = prof["total_ms"] / max(prof["launches"], 1)
    fpl = prof["flops"] / max(prof["launches"], 1)
    ach = fpl / (avg / 1e3) / 1e12
    log(f"[bench] {name}: {ms:.2f} ms/step, {T / t:.0f} tokens/s; {dom} {ach:.0f} TFLOP/s")
    split_form = None
    if dom == "attn_prefill" and model.cfg.dtype == L.SKV_BF16:
        # layer 1's split-bf16 attention is its own kernel instance (three products per block, same
        # algorithmic FLOPs): timed apart, over one more step, so the roofline above covers the plain form only
        cls = L.KERNEL_CLASS_NAMES.index("attn_prefill_split")
        L.skv_profile_enable(model.handle, cls, True)
        runner.prefill(model, cache, db, logits, stream)
        torch.cuda.synchronize()
        sp = L.skv_profile_read(model.handle)
        L.skv_profile_enable(model.handle, cls, False)
        if sp["launches"]:
            sms = sp["total_ms"] / sp["launches"]
            split_form = {"kernel": "attn_prefill8, split-bf16 form (layer 1)", "launches": sp["launches"],
                          "avg_launch_ms": round(sms, 4),
                          "algorithmic_tflops": round(sp["flops"] / sp["launches"] / (sms / 1e3) / 1e12, 2),
                          "time_vs_plain_form": round(sms / avg, 3)}
            log(f"[bench] {name}: split-form attention {sms:.3f} ms per launch ({sms / avg:.2f}x the plain form)")
    cache.close()
    model.close()
    out = {"workload": name, "prompts": B, "prompt_tokens": T, "swiftkv_l": w.swiftkv_l, "acrosskv_g": w.acrosskv_g,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 3), "tokens_per_s": round(T / t, 1),
            "normalized_tflops": round(full / t / 1e12, 2), "actual_tflops": round(swift / t / 1e12, 2),
            "normalized_frac_of_bf16_peak": round(full / t / 1e12 / MI355X_BF16_DENSE_TFLOPS, 4),
            "actual_frac_of_bf16_peak": round(swift / t / 1e12 / MI355X_BF16_DENSE_TFLOPS, 4),
            "flops_full_depth": full, "flops_swiftkv": swift,
            "roofline": {"kernel": KERNEL_TEXT[dom], "bound": "mfma", "achieved": round(ach, 2),
                         "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / MI355X_BF16_DENSE_TFLOPS, 4), "traffic": None,
                         "avg_launch_ms": round(avg, 4), "launches": prof["launches"], "flops_per_launch": fpl,
                         "algorithmic_bytes_per_launch": prof["bytes"] / max(prof["launches"], 1)}}
    if split_form is not None:
        out["roofline"]["split_form"] = split_form
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_l16_b16")
    ap.add_argument("--other-workloads", default="llama8b_l24_g4_b32,llama70b_l40_b32,llama8b_l16_long32k",
                    help="comma-separated workloads also timed (a sub-object each in 'workloads'); empty = none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the pure-MFMA throughput probe (random and constant operands)")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip timing the vendor library's GEMM on the dominant GEMM's shape")
    ap.add_argument("--no-full-depth", action="store_true",
                    help="skip timing the same batch through all layers (l = L) with the same kernels")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip timing a decode step and a chunked prefill over the same prompts")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip timing the same batch with a per-token FP8 KV cache")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time decode steps (for kernel traces of the decode path)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 fp32 device copies of MIB MiB each (reference for FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import skv_inputs as si
    from swiftkv_prefill_skipping_amd import _lib as L, runner

    w = si.WORKLOADS[args.workload]
    batch = si.make_batch(w)
    T, B = batch.total_tokens, len(batch.lengths)
    log(f"[bench] workload {w.name}: {B} prompts, {T} tokens, lengths {list(batch.lengths)}")
    cached = si.CachedLayers() if not args.no_cpu_baseline else None
    t0 = time.time()
    extra = 4  # blocks per prompt beyond its prefill, for the decode measurement
    model = runner.load_seeded_model(w, T, B, batch.max_seqlen + extra * batch.block_size,
                                     layer_hook=cached.hook if cached else None)
    log(f"[bench] weights generated and loaded in {time.time() - t0:.1f} s")
    cache = runner.Cache(model, batch.num_blocks + B * extra)
    db = runner.device_batch(batch)
    logits = torch.empty((B, w.shape.vocab), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    if args.decode_only:
        # decode steps alone, over the cache as created (zero K/V: the same work as after a prefill)
        print(json.dumps({"workload": w.name, "decode_step": measure_decode(model, cache, w, batch, extra, logits,
                                                                            stream, args)}), flush=True)
        return

    for i in range(args.warmup):
        runner.prefill(model, cache, db, logits, stream)
    torch.cuda.synchronize()
    log("[bench] warmup done")

    dom_name = DOMINANT.get(w.name, "gemm_gateup")
    dominant = L.KERNEL_CLASS_NAMES.index(dom_name)
    L.skv_profile_enable(model.handle, dominant, True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # one event between consecutive steps as well, for the per-step spread
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps - 1)]
    ev0.record(stream)
    for i in range(args.steps):
        runner.prefill(model, cache, db, logits, stream)
        if i < args.steps - 1:
            evs[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prof = L.skv_profile_read(model.handle)
    L.skv_profile_enable(model.handle, dominant, False)
    ms = ev0.elapsed_time(ev1) / args.steps
    marks = [ev0] + evs + [ev1]
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step (events), {wall / args.steps * 1e3:.3f} ms/step (wall)")

    full, swift = L.skv_flops(model.cfg, batch.lengths)
    t = ms / 1e3
    tok_s = T / t
    norm_tf = full / t / 1e12
    act_tf = swift / t / 1e12
    avg_launch_ms = prof["total_ms"] / max(prof["launches"], 1)
    flops_per_launch = prof["flops"] / max(prof["launches"], 1)
    achieved = flops_per_launch / (avg_launch_ms / 1e3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": {"min": round(step_ms[0], 4), "median": round(float(np.median(step_ms)), 4),
                    "max": round(step_ms[-1], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "description": "Llama-3.1-8B-shaped decoder (random init), SwiftKV l=16 of "
                   "32 layers, 16 prompts with lengths uniform in [500,1000], uniform random token ids"
                   if w.name == "llama8b_l16_b16" else w.name,
                   "prompts": B, "prompt_tokens": T, "swiftkv_l": w.swiftkv_l, "acrosskv_g": w.acrosskv_g},
        "normalized_tflops": round(norm_tf, 2),
        "actual_tflops": round(act_tf, 2),
        "normalized_frac_of_bf16_peak": round(norm_tf / MI355X_BF16_DENSE_TFLOPS, 4),
        "actual_frac_of_bf16_peak": round(act_tf / MI355X_BF16_DENSE_TFLOPS, 4),
        "flops_full_depth": full,
        "flops_swiftkv": swift,
        "roofline": {"kernel": KERNEL_TEXT[dom_name], "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MI355X_BF16_DENSE_TFLOPS, 4),
                     "traffic": (measured_traffic("EpiSwiGLUPanel") or {}).get("bytes") if w.name == "llama8b_l16_b16"
                     else None,
                     "traffic_detail": measured_traffic("EpiSwiGLUPanel") if w.name == "llama8b_l16_b16" else None,
                     "algorithmic_bytes_per_launch": prof["bytes"] / max(prof["launches"], 1),
                     "avg_launch_ms": round(avg_launch_ms, 4), "launches": prof["launches"],
                     "flops_per_launch": flops_per_launch},
    }
    if not args.no_vendor_gemm and w.dtype == "bf16" and dom_name == "gemm_gateup":
        res["vendor_gemm"] = vendor_gemm(T, 2 * w.shape.ffn_dim, w.shape.d_model, avg_launch_ms)
        log(f"[bench] vendor GEMM: {res['vendor_gemm']}")
    if not args.no_decode and w.dtype == "bf16":
        runner.prefill(model, cache, db, logits, stream)
        res["decode_step"] = measure_decode(model, cache, w, batch, extra, logits, stream, args)
        res["chunked_prefill"] = measure_chunked(model, cache, w, batch, stream, args, ms, swift)
    if not args.no_fp8 and w.dtype == "bf16":
        model.close()
        cache.close()
        res["fp8_kv_cache"] = measure_fp8(w, batch, db, logits, stream, args, extra, ms, res.get("decode_step"))
    if not args.no_full_depth and w.swiftkv_l < w.shape.n_layers:
        # the unmodified model (every layer for every prompt token), same weights, batch and kernels: the
        # wall-clock ratio to compare with the FLOP ratio
        import dataclasses
        model.close()
        cache.close()
        wf = dataclasses.replace(w, name=w.name + "_full_depth", swiftkv_l=w.shape.n_layers, acrosskv_g=1)
        t0 = time.time()
        mf = runner.load_seeded_model(wf, T, B, batch.max_seqlen)
        cf = runner.Cache(mf, batch.num_blocks)
        log(f"[bench] full-depth model loaded in {time.time() - t0:.1f} s")
        for i in range(args.warmup):
            runner.prefill(mf, cf, db, logits, stream)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            runner.prefill(mf, cf, db, logits, stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_full = ev0.elapsed_time(ev1) / args.steps
        full_f, _ = L.skv_flops(mf.cfg, batch.lengths)
        log(f"[bench] full depth: {ms_full:.3f} ms/step")
        res["full_depth_baseline"] = {
            "ms_per_step": round(ms_full, 4), "tokens_per_s": round(T / (ms_full / 1e3), 1),
            "tflops": round(full_f / (ms_full / 1e3) / 1e12, 2),
            "swiftkv_time_ratio": round(ms / ms_full, 4), "swiftkv_flops_ratio": round(swift / full, 4)}
        cf.close()
        mf.close()
    if not args.no_mfma_probe:
        # the matrix cores alone, no memory traffic: what dense bf16 sustains on this GPU with random operands
        # (the power limit of data like these weights) and with constant ones
        pr = {k: L.skv_mfma_probe(k == "random_operands", 20000, stream.cuda_stream)
              for k in ("random_operands", "constant_operands")}
        res["mfma_probe"] = {
            "kernel": "v_mfma_f32_16x16x32_bf16 (the GEMMs' instruction), 64 independent accumulators per wave, "
                      "4 waves per CU, no memory",
            "cus": pr["random_operands"]["cus"], "max_clock_mhz": pr["random_operands"]["max_clock_mhz"],
            **{k: {"tflops": round(v["tflops"], 1), "clock_mhz": round(v["clock_mhz"], 0),
                   "frac_of_bf16_peak": round(v["tflops"] / MI355X_BF16_DENSE_TFLOPS, 4)} for k, v in pr.items()},
            f"{dom_name}_frac_of_random_operand_probe": round(achieved / pr["random_operands"]["tflops"], 4)}
        log(f"[bench] MFMA probe: {res['mfma_probe']}")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(w, batch, cached)
    del cached
    others = [n for n in args.other_workloads.split(",") if n and n != w.name]
    if others:
        model.close()
        cache.close()
        res["workloads"] = {n: measure_workload(n, min(args.steps, 5), min(args.warmup, 2), stream) for n in others}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
