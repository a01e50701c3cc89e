"""Pins of the CPU oracle against things other than itself (CPU only).

* an independent library implementation of a standard Llama decoder
  (transformers' LlamaForCausalLM / its modules) -- the l = L special case,
  the skipped-layer KV of Eq. 2 and the last-token path;
* brute force: one-token-at-a-time decode of the unmodified model;
* the pages' printed numbers: Table 1 FLOPs per prefill token (Llama-3.1-70B)
  and the AcrossKV KV-memory reductions (tests/golden/);
* closed forms and invariants: RoPE relative-position invariance, attention
  special cases, causality, prompt independence, the gain-fold identity, and
  the exact FLOP count.
"""
import json
import math
import os

import numpy as np
import pytest

import skv_inputs as si
from oracle import swiftkv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_dims(**kw):
    base = dict(n_layers=4, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn_dim=96, vocab=97,
                rope_theta=10000.0, rms_eps=1e-5)
    base.update(kw)
    return O.Dims(**base)


def tiny_weights(dims, seed=5, dtype=np.float64, gain="uniform"):
    shape = si.ModelShape("pin", dims.n_layers, dims.d_model, dims.n_q_heads, dims.n_kv_heads, dims.head_dim,
                          dims.ffn_dim, dims.vocab, dims.rope_theta, dims.rms_eps, weight_seed=seed, init_std=0.08,
                          gain=gain)
    gw = si.global_weights(shape, "fp32")
    layers = [si.layer_weights(shape, i, "fp32") for i in range(1, dims.n_layers + 1)]
    return O.DictWeights(gw["embed"], gw["final_norm"], gw["lm_head"], layers, dtype=dtype)


def prompts_for(dims, lengths, seed=3):
    ids = si.randint(seed, 2, int(sum(lengths)), dims.vocab)
    out, off = [], 0
    for n in lengths:
        out.append(ids[off:off + n])
        off += n
    return out


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------
# library Llama (transformers), fp64
# ----------------------------------------------------------------------------

def hf_model(dims, W):
    torch = pytest.importorskip("torch")
    tf = pytest.importorskip("transformers")
    cfg = tf.LlamaConfig(vocab_size=dims.vocab, hidden_size=dims.d_model, intermediate_size=dims.ffn_dim,
                         num_hidden_layers=dims.n_layers, num_attention_heads=dims.n_q_heads,
                         num_key_value_heads=dims.n_kv_heads, head_dim=dims.head_dim, rope_theta=dims.rope_theta,
                         rms_norm_eps=dims.rms_eps, tie_word_embeddings=False, attention_bias=False, mlp_bias=False,
                         max_position_embeddings=4096, hidden_act="silu")
    cfg._attn_implementation = "eager"
    m = tf.LlamaForCausalLM(cfg).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64).copy())
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(t(W.embed))
        m.model.norm.weight.copy_(t(W.final_norm))
        m.lm_head.weight.copy_(t(W.lm_head))
        for i, layer in enumerate(m.model.layers):
            Li = W.layer(i + 1)
            layer.input_layernorm.weight.copy_(t(Li["attn_norm"]))
            layer.self_attn.q_proj.weight.copy_(t(Li["wq"]))
            layer.self_attn.k_proj.weight.copy_(t(Li["wk"]))
            layer.self_attn.v_proj.weight.copy_(t(Li["wv"]))
            layer.self_attn.o_proj.weight.copy_(t(Li["wo"]))
            layer.post_attention_layernorm.weight.copy_(t(Li["ffn_norm"]))
            layer.mlp.gate_proj.weight.copy_(t(Li["w_gate"]))
            layer.mlp.up_proj.weight.copy_(t(Li["w_up"]))
            layer.mlp.down_proj.weight.copy_(t(Li["w_down"]))
    return m


def hf_cache_kv(pkv, layer):
    """(K, V) of one layer from a transformers cache as [n, hkv, dh] numpy."""
    lay = pkv.layers[layer]
    k, v = lay.keys, lay.values
    return k[0].permute(1, 0, 2).numpy(), v[0].permute(1, 0, 2).numpy()


# the library computes its norms in float32, so agreement is at float32 level
HF_TOL = 2e-5


def test_full_depth_equals_library_llama():
    """l = L is a standard prefill: every layer's KV and the last logits match the library model."""
    torch = pytest.importorskip("torch")
    dims = tiny_dims()
    W = tiny_weights(dims)
    prompt = prompts_for(dims, [23])[0]
    res = O.swiftkv_prefill(dims, W, [prompt], l=dims.n_layers, dtype=np.float64)
    m = hf_model(dims, W)
    with torch.no_grad():
        out = m(torch.from_numpy(prompt[None, :].astype(np.int64)), use_cache=True)
    assert rel(res.logits[0], out.logits[0, -1].numpy()) < HF_TOL
    for i in range(dims.n_layers):
        k, v = hf_cache_kv(out.past_key_values, i)
        assert rel(res.kv[0][i][0], k) < HF_TOL, f"K layer {i + 1}"
        assert rel(res.kv[0][i][1], v) < HF_TOL, f"V layer {i + 1}"


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_skipped_layer_kv_equals_library_projection_of_boundary_state(l):
    """Eq. 2: KV_j = layer j's K/V projection (after its input norm, K rotated) fed x_{l+1}."""
    torch = pytest.importorskip("torch")
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    dims = tiny_dims()
    W = tiny_weights(dims)
    prompt = prompts_for(dims, [19])[0]
    res = O.swiftkv_prefill(dims, W, [prompt], l=l, dtype=np.float64)
    m = hf_model(dims, W)
    n = len(prompt)
    with torch.no_grad():
        out = m(torch.from_numpy(prompt[None, :].astype(np.int64)), output_hidden_states=True, use_cache=True)
        x_b = out.hidden_states[l]                      # input of layer l+1
        assert rel(res.x_boundary[0], x_b[0].numpy()) < HF_TOL
        pos_ids = torch.arange(n)[None, :]
        cos, sin = m.model.rotary_emb(x_b, pos_ids)
        for j in range(l + 1, dims.n_layers + 1):
            layer = m.model.layers[j - 1]
            a = layer.input_layernorm(x_b)
            k = layer.self_attn.k_proj(a).view(1, n, dims.n_kv_heads, dims.head_dim).transpose(1, 2)
            v = layer.self_attn.v_proj(a).view(1, n, dims.n_kv_heads, dims.head_dim).transpose(1, 2)
            _, k = apply_rotary_pos_emb(k, k, cos, sin)
            K, V = res.kv[0][O.slot_of_layer(j, dims.n_layers, l, 1)]
            assert rel(K, k[0].permute(1, 0, 2).numpy()) < HF_TOL, f"K j={j}"
            assert rel(V, v[0].permute(1, 0, 2).numpy()) < HF_TOL, f"V j={j}"
        for i in range(l):                               # layers <= l: populated normally
            k, v = hf_cache_kv(out.past_key_values, i)
            assert rel(res.kv[0][i][0], k) < HF_TOL
            assert rel(res.kv[0][i][1], v) < HF_TOL


class _FixedKV:
    """Cache stand-in for the library attention: returns the stored SwiftKV K/V of every position."""

    def __init__(self, kv_by_layer):
        self.kv = kv_by_layer

    def update(self, key_states, value_states, layer_idx, cache_kwargs=None):
        return self.kv[layer_idx]


@pytest.mark.parametrize("l,g", [(1, 1), (2, 1), (0, 1), (1, 2), (2, 2)])
def test_last_token_path_equals_library_layers(l, g):
    """The last prompt token runs layers l+1..L (library modules) over the SwiftKV cache, then norm + LM head."""
    torch = pytest.importorskip("torch")
    dims = tiny_dims()
    W = tiny_weights(dims)
    prompt = prompts_for(dims, [17])[0]
    n = len(prompt)
    res = O.swiftkv_prefill(dims, W, [prompt], l=l, g=g, dtype=np.float64)
    m = hf_model(dims, W)
    kv = {}
    for j in range(l + 1, dims.n_layers + 1):
        K, V = res.kv[0][O.slot_of_layer(j, dims.n_layers, l, g)]
        kv[j - 1] = (torch.from_numpy(K).permute(1, 0, 2)[None].contiguous(),
                     torch.from_numpy(V).permute(1, 0, 2)[None].contiguous())
    with torch.no_grad():
        out = m(torch.from_numpy(prompt[None, :].astype(np.int64)), output_hidden_states=True)
        y = out.hidden_states[l][:, -1:, :]
        pos = torch.tensor([[n - 1]])
        cos, sin = m.model.rotary_emb(y, pos)
        cache = _FixedKV(kv)
        for j in range(l + 1, dims.n_layers + 1):
            layer = m.model.layers[j - 1]
            r = layer(y, attention_mask=None, position_ids=pos, past_key_values=cache,
                      position_embeddings=(cos, sin))
            y = r[0] if isinstance(r, tuple) else r
        logits = m.lm_head(m.model.norm(y))[0, 0].numpy()
    assert rel(res.logits[0], logits) < HF_TOL


# ----------------------------------------------------------------------------
# brute force and structural invariants
# ----------------------------------------------------------------------------

def test_full_depth_equals_incremental_decode():
    dims = tiny_dims(n_layers=3)
    W = tiny_weights(dims, seed=9)
    prompt = prompts_for(dims, [21], seed=8)[0]
    res = O.swiftkv_prefill(dims, W, [prompt], l=dims.n_layers, dtype=np.float64)
    Ks, Vs, logits = O.standard_incremental_decode(dims, W, prompt, dtype=np.float64)
    assert rel(res.logits[0], logits) < 1e-12
    for i in range(dims.n_layers):
        assert rel(res.kv[0][i][0], Ks[i]) < 1e-12
        assert rel(res.kv[0][i][1], Vs[i]) < 1e-12


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_unskipped_layers_kv_bitwise_equal_unmodified_model(l):
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float32)
    ps = prompts_for(dims, [9, 14])
    full = O.swiftkv_prefill(dims, W, ps, l=dims.n_layers)
    sk = O.swiftkv_prefill(dims, W, ps, l=l)
    for b in range(2):
        for i in range(l):
            assert np.array_equal(full.kv[b][i][0], sk.kv[b][i][0])
            assert np.array_equal(full.kv[b][i][1], sk.kv[b][i][1])


@pytest.mark.parametrize("g", [2, 3])
def test_acrosskv_equals_no_merging_with_representative_weights(g):
    """AcrossKV (g) == no merging (g = 1) on a model whose skipped layers carry their representative's W_K, W_V.

    The skipped layers share one input-norm gain so that the substitution
    leaves their query side untouched; then every KV tensor and the logits
    must agree bitwise.
    """
    dims = tiny_dims(n_layers=6)
    W = tiny_weights(dims, dtype=np.float64)
    l = 1
    ps = prompts_for(dims, [11, 6])
    shared_gain = W.layer(l + 1)["attn_norm"]
    base_layers = [dict(W.layer(j), attn_norm=(shared_gain if j > l else W.layer(j)["attn_norm"]))
                   for j in range(1, dims.n_layers + 1)]
    Wm = O.DictWeights(W.embed, W.final_norm, W.lm_head, base_layers, dtype=np.float64)
    rep_layers = []
    for j in range(1, dims.n_layers + 1):
        Lj = dict(base_layers[j - 1])
        if j > l:
            R = base_layers[O.representative(j, l, g) - 1]
            Lj["wk"], Lj["wv"] = R["wk"], R["wv"]
        rep_layers.append(Lj)
    W2 = O.DictWeights(W.embed, W.final_norm, W.lm_head, rep_layers, dtype=np.float64)
    merged = O.swiftkv_prefill(dims, Wm, ps, l=l, g=g, dtype=np.float64)
    unmerged = O.swiftkv_prefill(dims, W2, ps, l=l, g=1, dtype=np.float64)
    assert len(merged.kv[0]) == O.kv_slots(dims.n_layers, l, g) == l + math.ceil((dims.n_layers - l) / g)
    for b in range(2):
        for j in range(l + 1, dims.n_layers + 1):
            K1, V1 = merged.kv[b][O.slot_of_layer(j, dims.n_layers, l, g)]
            K2, V2 = unmerged.kv[b][O.slot_of_layer(j, dims.n_layers, l, 1)]
            assert np.array_equal(K1, K2) and np.array_equal(V1, V2)
    assert np.array_equal(merged.logits, unmerged.logits)
    # without the substitution the two differ (the merge is not a no-op)
    plain = O.swiftkv_prefill(dims, Wm, ps, l=l, g=1, dtype=np.float64)
    assert not np.allclose(plain.logits, merged.logits)


def test_acrosskv_group_size_one_is_no_merging():
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float32)
    ps = prompts_for(dims, [12])
    a = O.swiftkv_prefill(dims, W, ps, l=2, g=1)
    assert len(a.kv[0]) == dims.n_layers
    for j in range(3, dims.n_layers + 1):
        assert O.representative(j, 2, 1) == j
        assert O.slot_of_layer(j, dims.n_layers, 2, 1) == j - 1


def test_prompts_are_independent():
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float32)
    ps = prompts_for(dims, [7, 13, 5])
    together = O.swiftkv_prefill(dims, W, ps, l=2)
    for b, p in enumerate(ps):
        alone = O.swiftkv_prefill(dims, W, [p], l=2)
        assert np.array_equal(alone.logits[0], together.logits[b])
        for s in alone.kv[0]:
            assert np.array_equal(alone.kv[0][s][0], together.kv[b][s][0])


@pytest.mark.parametrize("l", [0, 2, 4])
def test_causality_of_kv(l):
    """Changing token p leaves every slot's KV at positions < p unchanged and changes position p."""
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float64)
    p0 = prompts_for(dims, [15])[0]
    p1 = p0.copy()
    p1[9] = (p1[9] + 1) % dims.vocab
    a = O.swiftkv_prefill(dims, W, [p0], l=l, dtype=np.float64)
    b = O.swiftkv_prefill(dims, W, [p1], l=l, dtype=np.float64)
    for s in a.kv[0]:
        for t in range(2):
            assert np.array_equal(a.kv[0][s][t][:9], b.kv[0][s][t][:9])
            assert not np.allclose(a.kv[0][s][t][9], b.kv[0][s][t][9])


def test_rope_properties():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 1, 32))
    theta = 500000.0
    # position 0 is the identity, rotation preserves the norm
    assert np.allclose(O.rope(q, np.array([0]), theta), q, atol=0, rtol=0)
    r = O.rope(q, np.array([37]), theta)
    assert abs(np.linalg.norm(r) - np.linalg.norm(q)) < 1e-12
    # relative-position invariance of the score
    for (p, pp, s) in [(3, 1, 5), (100, 7, 900), (0, 0, 12345)]:
        a = np.sum(O.rope(q, np.array([p + s]), theta) * O.rope(k, np.array([pp + s]), theta))
        b = np.sum(O.rope(q, np.array([p]), theta) * O.rope(k, np.array([pp]), theta))
        assert abs(a - b) < 1e-9
    # pair i rotates by angle pos * theta^(-2i/dh): check one coordinate pair by hand
    dh, i, pos = 32, 5, 11
    x = np.zeros((1, 1, dh))
    x[0, 0, i] = 1.0
    y = O.rope(x, np.array([pos]), theta)
    ang = pos * theta ** (-2.0 * i / dh)
    assert abs(y[0, 0, i] - math.cos(ang)) < 1e-12
    assert abs(y[0, 0, i + dh // 2] - math.sin(ang)) < 1e-12


def test_attention_special_cases():
    rng = np.random.default_rng(1)
    n, hq, hkv, dh = 6, 4, 2, 8
    q = rng.standard_normal((n, hq, dh))
    k = rng.standard_normal((n, hkv, dh))
    v = rng.standard_normal((n, hkv, dh))
    o = O.causal_gqa_attention(q, k, v, None).reshape(n, hq, dh)
    # the first position attends only to itself
    for h in range(hq):
        assert np.allclose(o[0, h], v[0, h // 2], atol=1e-14)
    # identical keys -> uniform weights -> running mean of values
    kk = np.repeat(k[:1], n, axis=0)
    o2 = O.causal_gqa_attention(q, kk, v, None).reshape(n, hq, dh)
    for p in range(n):
        for h in range(hq):
            assert np.allclose(o2[p, h], v[:p + 1, h // 2].mean(axis=0), atol=1e-13)
    # GQA head map: heads 0,1 read kv head 0; heads 2,3 read kv head 1
    vv = v.copy()
    vv[:, 1] += 100.0
    o3 = O.causal_gqa_attention(q, k, vv, None).reshape(n, hq, dh)
    assert np.allclose(o3[:, :2], o[:, :2]) and not np.allclose(o3[:, 2:], o[:, 2:])
    # single-query form equals the last causal row
    s = O.single_query_attention(q[-1], k, v, None).reshape(hq, dh)
    assert np.allclose(s, o[-1], atol=1e-14)


def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0]])
    g = np.array([2.0, 0.5])
    y = O.rmsnorm(x, g, 0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(y, [[2 * 3 / r, 0.5 * 4 / r]], rtol=1e-15)
    assert np.allclose(O.rmsnorm(7 * x, g, 0.0), y, rtol=1e-14)   # scale invariance


def test_gain_fold_identity_fp64():
    """r * (x @ (W diag(gamma))^T) == RMSNorm(x; gamma) @ W^T, r = 1/sqrt(mean x^2 + eps)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 64))
    W = rng.standard_normal((32, 64))
    gam = rng.uniform(0.5, 1.5, 64)
    eps = 1e-5
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    lhs = r * (x @ (W * gam[None, :]).T)
    rhs = O.rmsnorm(x, gam, eps) @ W.T
    assert rel(lhs, rhs) < 1e-12


# ----------------------------------------------------------------------------
# FLOP accounting and the pages' printed figures
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("l,g,lengths", [(2, 1, [5]), (0, 1, [3, 8]), (4, 1, [6]), (1, 2, [4, 9]), (1, 3, [10])])
def test_flop_counter_equals_closed_form(l, g, lengths):
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float32)
    ps = prompts_for(dims, lengths)
    res = O.swiftkv_prefill(dims, W, ps, l=l, g=g)
    full, swift = O.prefill_flops(dims, l, g, lengths)
    assert res.flops == swift
    if l == dims.n_layers:
        assert full == swift
    base = O.swiftkv_prefill(dims, W, ps, l=dims.n_layers)
    assert base.flops == full


def test_table1_llama70b_flops_per_token():
    gold = json.load(open(os.path.join(GOLDEN, "table1_llama70b_flops.json")))
    m = gold["model"]
    dims = O.Dims(m["n_layers"], m["d_model"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"], m["ffn_dim"],
                  m["vocab"], 500000.0)
    L = dims.n_layers
    tol = gold["row_tolerance_gflops"]
    attn_per_layer = gold["baseline"]["attention"] * 1e9 / L
    base = {k: v / 1e9 for k, v in O.per_token_breakdown(dims, L, 1, attn_per_layer).items()}
    for k in ("vocab", "kv", "qo", "mlp"):
        assert abs(base[k] - gold["baseline"][k]) <= tol[k], k
    assert abs(sum(base.values()) - gold["baseline"]["total"]) <= tol["total"]
    for key in ("swiftkv_25", "swiftkv_50", "swiftkv_50_acrosskv4"):
        case = gold[key]
        br = {k: v / 1e9 for k, v in O.per_token_breakdown(dims, case["l"], case["g"], attn_per_layer).items()}
        for k in ("qo", "mlp", "attention", "kv"):
            if k in case:
                assert abs(br[k] - case[k]) <= tol[k], (key, k)
        assert abs(sum(br.values()) - case["total"]) <= tol["total"], key
    # the skipped share of per-layer (non-KV) work is (L - l) / L
    for l in (60, 40):
        b0 = O.per_token_breakdown(dims, L, 1, attn_per_layer)
        b1 = O.per_token_breakdown(dims, l, 1, attn_per_layer)
        for k in ("qo", "mlp", "attention"):
            assert abs(b1[k] / b0[k] - l / L) < 1e-12


def test_acrosskv_memory_reductions():
    gold = json.load(open(os.path.join(GOLDEN, "acrosskv_kv_memory.json")))
    L, l = gold["n_layers"], gold["l"]
    for c in gold["cases"]:
        assert O.kv_slots(L, l, c["g"]) == c["kv_layers"]
        assert abs((1 - O.kv_memory_fraction(L, l, c["g"])) * 100 - c["reduction_pct"]) < 1e-12


def test_full_depth_flops_closed_form_matches_hand_count():
    """F_full = L [N (2 d dq + 2 dq d + 6 d f + 4 d dkv) + 2 N (N+1) dh hq] + 2 d V for one prompt."""
    dims = O.Dims(32, 4096, 32, 8, 128, 14336, 128256, 500000.0)
    N = 1000
    full, swift = O.prefill_flops(dims, 16, 1, [N])
    d, f = 4096, 14336
    per_layer = N * (2 * d * d * 2 + 6 * d * f + 4 * d * 1024) + 2 * N * (N + 1) * 128 * 32
    assert full == 32 * per_layer + 2 * d * 128256
    skip_layer = 2 * d * d * 2 + 6 * d * f + 4 * N * 128 * 32
    assert swift == 16 * per_layer + 16 * N * 4 * d * 1024 + 16 * skip_layer + 2 * d * 128256


def test_invalid_arguments_rejected():
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float32)
    with pytest.raises(ValueError):
        O.swiftkv_prefill(dims, W, [np.array([1, 2])], l=5)
    with pytest.raises(ValueError):
        O.swiftkv_prefill(dims, W, [np.array([1, 2])], l=1, g=0)
    with pytest.raises(ValueError):
        O.swiftkv_prefill(dims, W, [np.array([], dtype=np.int64)], l=1)


def _round_bf16(x):
    return si.bf16_to_f32(si.f32_to_bf16(np.ascontiguousarray(x, dtype=np.float32))).reshape(x.shape)


def test_storage_mode_identity_is_plain_evaluation():
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float32)
    ps = prompts_for(dims, [13, 6])
    a = O.swiftkv_prefill(dims, W, ps, l=2, g=1)
    b = O.swiftkv_prefill(dims, W, ps, l=2, g=1, store=lambda t: t)
    assert np.array_equal(a.logits, b.logits)
    for i in range(2):
        for s in a.kv[i]:
            assert np.array_equal(a.kv[i][s][0], b.kv[i][s][0]) and np.array_equal(a.kv[i][s][1], b.kv[i][s][1])


def test_bf16_storage_mode_rounds_what_it_stores():
    """With bf16 storage every K/V tensor is bf16-representable and the outputs move by bf16-sized amounts."""
    dims = tiny_dims()
    W = tiny_weights(dims, dtype=np.float32)
    ps = prompts_for(dims, [17])
    ref = O.swiftkv_prefill(dims, W, ps, l=2, g=2)
    emu = O.swiftkv_prefill(dims, W, ps, l=2, g=2, store=_round_bf16)
    for s, (k, v) in emu.kv[0].items():
        assert np.array_equal(k, _round_bf16(k)) and np.array_equal(v, _round_bf16(v))
        e = rel(k, ref.kv[0][s][0])
        assert 0 < e < 0.05, (s, e)
    e = rel(emu.logits, ref.logits)
    assert 0 < e < 0.05
