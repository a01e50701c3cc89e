"""CPU-only checks of the C ABI: the library loads, exports every declared
symbol, and its host-side logic (config validation, closed-form FLOPs)
behaves without touching a GPU."""
import os
import re

import numpy as np
import pytest

import skv_inputs as si
from oracle import swiftkv_oracle as O
from tests.helpers import dims_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from swiftkv_prefill_skipping_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        from swiftkv_prefill_skipping_amd import build
        build.build(verbose=False)
    return L


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "swiftkv.h")).read()
    return sorted(set(re.findall(r"\b(skv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = _lib()
    import ctypes
    so = ctypes.CDLL(L.LIB_PATH)
    syms = declared_symbols()
    assert len(syms) >= 13
    for s in syms:
        assert hasattr(so, s), s
    assert set(syms) == set(L.EXPORTED)


def cfg_for(w, **over):
    L = _lib()
    s = w.shape
    args = dict(n_layers=s.n_layers, d_model=s.d_model, n_q_heads=s.n_q_heads, n_kv_heads=s.n_kv_heads,
                head_dim=s.head_dim, ffn_dim=s.ffn_dim, vocab=s.vocab, rope_theta=s.rope_theta, rms_eps=s.rms_eps,
                swiftkv_l=w.swiftkv_l, acrosskv_g=w.acrosskv_g, dtype=L.SKV_BF16 if w.dtype == "bf16" else L.SKV_FP32,
                max_tokens=40000, max_batch=32, max_seqlen=40000)
    args.update(over)
    return L.make_config(**args)


@pytest.mark.parametrize("name", si.WORKLOAD_ORDER)
def test_flops_closed_form_matches_oracle(name):
    L = _lib()
    w = si.WORKLOADS[name]
    lengths = si.make_batch(w).lengths
    full, swift = L.skv_flops(cfg_for(w), lengths)
    of, osw = O.prefill_flops(dims_of(w.shape), w.swiftkv_l, w.acrosskv_g, lengths)
    assert full == pytest.approx(of, rel=1e-12)
    assert swift == pytest.approx(osw, rel=1e-12)


@pytest.mark.parametrize("over,status", [
    (dict(swiftkv_l=33), -1), (dict(swiftkv_l=-1), -1), (dict(acrosskv_g=0), -1), (dict(n_kv_heads=3), -1),
    (dict(head_dim=64), -4), (dict(max_batch=33), -4), (dict(max_tokens=0), -1), (dict(vocab=1000), -4),
])
def test_config_validation_rejects_before_any_device_call(over, status):
    L = _lib()
    w = si.WORKLOADS["llama8b_l16_b16"]
    with pytest.raises(L.SkvError) as e:
        L.skv_model_create(cfg_for(w, **over))
    assert e.value.status == status
    assert L.lib().skv_last_error().decode()


def test_fp32_validation():
    L = _lib()
    w = si.WORKLOADS["tiny_fp32_l2"]
    with pytest.raises(L.SkvError):
        L.skv_model_create(cfg_for(w, head_dim=48))
    full, swift = L.skv_flops(cfg_for(w), [128])
    assert swift < full


def test_step_rejects_null_arguments_without_a_device():
    L = _lib()
    import ctypes
    with pytest.raises(L.SkvError) as e:
        L.check(L.lib().skv_step(None, None, None, None, None))
    assert e.value.status == L.SKV_ERR_INVALID_ARG


def test_mfma_probe_rejects_bad_arguments_before_any_device_call():
    L = _lib()
    with pytest.raises(L.SkvError) as e:
        L.skv_mfma_probe(True, 0, 0)
    assert e.value.status == -1
    assert "iters" in L.lib().skv_last_error().decode()
