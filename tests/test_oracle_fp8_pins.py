"""Pins of the oracle's per-token FP8 KV cache ([S] "Complementarity with KV
quantization", Appendix B.1 / Table B.1), CPU only.

* the E4M3 codec against an independent library implementation (torch's
  float8_e4m3fn): every one of the 256 codes decodes the same, and encoding
  agrees on every representable value, every midpoint (ties to even), the
  values just either side of the midpoints and the subnormal range;
* the half-ulp error bound of the per-token quantizer, and its scale
  (the row maximum lands exactly on +-448);
* the pages' printed KV-memory reductions with FP8 (tests/golden/);
* the cache stays chunk-invariant: a prompt fed in chunks with an FP8 cache
  equals the one-shot FP8 prefill, and a decode token is the next prefill
  position.
"""
import json
import os

import numpy as np
import pytest

from oracle import swiftkv_oracle as O
from tests.test_oracle_pins import GOLDEN, prompts_for, rel, tiny_dims, tiny_weights


def torch_e4m3(values: np.ndarray) -> np.ndarray:
    torch = pytest.importorskip("torch")
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_every_code_matches_library():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], lib[ok])
    assert np.sum(np.isnan(ours)) == 2                     # S.1111.111 only
    assert O.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0


def test_encode_matches_library_on_values_midpoints_and_neighbours():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    pos = np.unique(vals[(vals >= 0) & ~np.isnan(vals)]).astype(np.float64)   # 0 .. 448, sorted
    mids = (pos[:-1] + pos[1:]) / 2
    probe = np.concatenate([pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                            np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float32)
    rng = np.random.default_rng(7)
    probe = np.concatenate([probe, rng.uniform(0, 448, 20000).astype(np.float32),
                            (rng.uniform(0, 1, 5000) * 2.0 ** -6).astype(np.float32)])
    probe = np.concatenate([probe, -probe])
    assert np.array_equal(O.e4m3_encode(probe), torch_e4m3(probe))


def test_roundtrip_of_representable_values_is_exact():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    back = O.e4m3_encode(vals)
    assert np.array_equal(O.e4m3_decode(back), vals)


def test_per_token_quantizer_error_bound_and_scale():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 4, (64, 1)))).astype(np.float32)
    x[5] = 0.0
    codes, scale = O.fp8_quantize_rows(x)
    assert scale[5] == 0 and not codes[5].any()
    deq = O.fp8_dequantize_rows(codes, scale)
    for r in range(x.shape[0]):
        if scale[r] == 0:
            continue
        y = x[r].astype(np.float64) / scale[r]
        ay = np.abs(y)
        half_ulp = np.where(ay < 2.0 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(ay, 2.0 ** -6))) - 4))
        err = np.abs(deq[r].astype(np.float64) - x[r]) / scale[r]
        assert np.all(err <= half_ulp * (1 + 1e-5) + 1e-6), r
        assert np.max(np.abs(O.e4m3_decode(codes[r]))) == 448.0     # the row maximum maps to +-448


def test_bf16_rounding_matches_library():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-30, 30, 50000))).astype(np.float32)
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)   # exact halfway cases
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1.0])])
    lib = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.bf16_round(x).view(np.uint32), lib.view(np.uint32))


def test_fp8_kv_memory_reductions_printed_by_the_pages():
    gold = json.load(open(os.path.join(GOLDEN, "fp8_kv_memory.json")))
    L, l = gold["n_layers"], gold["l"]
    for c in gold["cases"]:
        frac = O.kv_memory_fraction(L, l, c["g"], kv_bits=8 if c["fp8"] else 16)
        assert abs((1 - frac) * 100 - c["reduction_pct"]) < 1e-12


@pytest.mark.parametrize("l,g", [(2, 1), (1, 2), (0, 1)])
def test_fp8_cache_chunked_equals_one_shot(l, g):
    dims = tiny_dims()
    W = tiny_weights(dims)
    prompt = prompts_for(dims, [25])[0]
    past, off = {}, 0
    for n in (9, 1, 15):
        r = O.swiftkv_step(dims, W, [past], [prompt[off:off + n]], l, g, dtype=np.float64, kv_fp8=True)
        past = r.kv[0]
        off += n
    full = O.swiftkv_prefill(dims, W, [prompt], l, g, dtype=np.float64, kv_fp8=True)
    assert rel(r.logits[0], full.logits[0]) < 1e-10
    for s in full.kv[0]:
        assert rel(past[s][0], full.kv[0][s][0]) < 1e-10
        assert rel(past[s][1], full.kv[0][s][1]) < 1e-10


def test_fp8_cache_values_are_codes_times_token_scale():
    """Every cached K/V row is (E4M3 code) x (one scale per token), and the FP8 path differs from the 16-bit one
    by about the FP8 resolution, not more."""
    dims = tiny_dims()
    W = tiny_weights(dims)
    prompt = prompts_for(dims, [20])[0]
    q = O.swiftkv_prefill(dims, W, [prompt], 2, 1, dtype=np.float64, kv_fp8=True)
    p = O.swiftkv_prefill(dims, W, [prompt], 2, 1, dtype=np.float64)
    for s, (K, V) in q.kv[0].items():
        for t in (K, V):
            # values on a per-token E4M3 grid come back from a second round trip up to float32 rounding of the
            # scale (values off the grid would move by up to half an E4M3 step, ~6%)
            again = O.fp8_kv_roundtrip(t.astype(np.float32))
            assert np.max(np.abs(again - t) / np.maximum(np.abs(t), 1e-30)) < 1e-6
            assert rel(t, p.kv[0][s][0 if t is K else 1]) < 0.1
    assert 1e-3 < rel(q.logits[0], p.logits[0]) < 0.2
