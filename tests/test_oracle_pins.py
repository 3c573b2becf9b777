"""Pins of the CPU oracle against what the pages and mathematics fix.

Every check here is independent of the oracle's own code path: worked values
printed on the pages, closed forms, invariants, library routines (NumPy's
binary16, torch's rms_norm and scaled_dot_product_attention) and a
brute-force full-sequence model written differently (dense causal mask, no
cache, complex-number rotation).
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch

import qwen2_synth as syn
from oracle import qwen2_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paper_worked_values.json")


def golden():
    with open(GOLDEN) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def f16(bits):
    """Independent binary16 decode: NumPy's own float16."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def tiny_variant(**kw):
    return dataclasses.replace(syn.MODELS["tiny"], name="tiny-" + "-".join(f"{k}{v}" for k, v in kw.items()), **kw)


# ---------------------------------------------------------------- f16 decode
def test_f16_decoder_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = O.decode_f16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # subnormals are kept, not flushed
    assert O.decode_f16(np.array([1], np.uint16))[0] == 2.0 ** -24


# ---------------------------------------------------------------- worked values
def test_shapes_and_sizes_match_pages():
    g = golden()
    m = syn.MODELS["qwen2.5-0.5b"]
    c = g["config_0_5b"]
    assert (m.n_layer, m.n_embd, m.n_head, m.n_head_kv, m.n_ff, m.n_vocab) == (
        c["n_layer"], c["n_embd"], c["n_head"], c["n_head_kv"], c["n_ff"], c["n_vocab"])
    assert m.rope_theta == c["rope_theta"] and m.rms_eps == c["rms_eps"] and m.tied == c["tied"]
    assert m.n_embd // m.n_head == g["head_dim_0_5b"] == m.head_dim
    assert m.n_head_kv * m.head_dim == g["kv_width_0_5b"]
    assert m.n_head // m.n_head_kv == g["gqa_group_0_5b"]
    sh = m.shapes()
    for name, shape in g["shapes_0_5b"].items():
        if name == "tok_embd":
            assert [m.n_vocab, m.n_embd] == shape
        else:
            assert list(sh[name]) == shape, name
    emb = m.n_vocab * m.n_embd * 2
    assert emb == g["embed_f16_bytes_0_5b"]
    assert round(emb / 2 ** 20) == g["embed_f16_mib_approx_0_5b"]
    wb = syn.weight_bytes(m)
    assert wb["f16"] == 987_922_432
    assert round(wb["f16"] / 2 ** 20) == g["resident_f16_weights_mib_approx_0_5b"]
    assert syn.MODELS["qwen2-hd128"].head_dim == g["head_dim_large"]


def test_kv_bytes_per_position_match_pages():
    g = golden()
    m = syn.MODELS["qwen2.5-0.5b"]
    hp = O.hparams_for(m, n_ctx=4096)
    orc = O.Qwen2Oracle(hp, {"layers": []})
    K, V = orc._cache(0)
    per_pos = (K.nbytes + V.nbytes) // hp.n_ctx
    assert per_pos == g["kv_bytes_per_position_kb_0_5b"] * 1024 == 24_576
    assert (K.nbytes + V.nbytes) == g["kv_mb_approx_at_n_ctx_4096_0_5b"] * 2 ** 20


# ---------------------------------------------------------------- single ops
def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    for H in (64, 896, 3584):
        h = (rng.standard_normal((5, H)) * 3).astype(np.float32)
        w = (1 + 0.02 * rng.standard_normal(H)).astype(np.float32)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(h).double(), (H,),
                                           torch.from_numpy(w).double(), eps=1e-6)
        got = O.rms_norm(h, w, 1e-6)
        assert got.dtype == np.float32
        np.testing.assert_allclose(got, ref.numpy().astype(np.float32), rtol=2e-7, atol=0)


def test_rope_identity_at_position_zero():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 3, 64)).astype(np.float32)
    phi = O.rope_angles(np.array([0]), 64, 1e6)
    assert np.array_equal(O.rope_rotate_half(x, phi), x)


def test_rope_preserves_pair_norms_and_uses_half_split_pairs():
    rng = np.random.default_rng(2)
    hd = 64
    x = rng.standard_normal((4, 2, hd)).astype(np.float32)
    pos = np.array([1, 17, 1000, 8191])
    phi = O.rope_angles(pos, hd, 1e6)
    y = O.rope_rotate_half(x, phi).astype(np.float64)
    x64 = x.astype(np.float64)
    n0 = np.hypot(x64[..., :hd // 2], x64[..., hd // 2:])
    n1 = np.hypot(y[..., :hd // 2], y[..., hd // 2:])
    np.testing.assert_allclose(n1, n0, rtol=3e-7)
    # closed form with complex numbers: z = a + i b rotates by exp(i phi)
    inv = 1e6 ** (-np.arange(0, hd, 2) / hd)
    z = (x64[..., :hd // 2] + 1j * x64[..., hd // 2:]) * np.exp(1j * pos[:, None, None] * inv)
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-6)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(3)
    hd = 64
    q = rng.standard_normal((1, 1, hd)).astype(np.float32)
    k = rng.standard_normal((1, 1, hd)).astype(np.float32)

    def score(m, n):
        qm = O.rope_rotate_half(q, O.rope_angles(np.array([m]), hd, 1e6)).astype(np.float64)
        kn = O.rope_rotate_half(k, O.rope_angles(np.array([n]), hd, 1e6)).astype(np.float64)
        return float(np.sum(qm * kn))

    base = score(7, 3)
    for m, n in [(4, 0), (104, 100), (4099, 4095)]:
        assert abs(score(m, n) - base) < 2e-5 * abs(base) + 1e-5
    assert abs(score(8, 3) - base) > 1e-3


def test_interleaved_rope_differs():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 2, 16)).astype(np.float32)
    phi = O.rope_angles(np.array([3, 9]), 16, 1e6)
    assert np.max(np.abs(O.rope_interleaved(x, phi) - O.rope_rotate_half(x, phi))) > 1e-2


def test_interleaved_rope_closed_form_and_pair_order():
    """Interleaved RoPE turns each pair (x[2d], x[2d+1]) by phi[d] (the 2-D
    rotation written out), and equals rotate_half applied after moving
    dimension 2d to d and 2d+1 to d + hd/2, then moved back."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 2, 8)).astype(np.float32)
    phi = O.rope_angles(np.array([0, 5, 77]), 8, 1e4)
    got = O.rope_interleaved(x, phi)
    for n in range(3):
        for d in range(4):
            c, s = np.cos(phi[n, d]), np.sin(phi[n, d])
            a, b = x[n, :, 2 * d].astype(np.float64), x[n, :, 2 * d + 1].astype(np.float64)
            np.testing.assert_allclose(got[n, :, 2 * d], a * c - b * s, rtol=1e-6, atol=1e-7)
            np.testing.assert_allclose(got[n, :, 2 * d + 1], b * c + a * s, rtol=1e-6, atol=1e-7)
    perm = np.concatenate([np.arange(0, 8, 2), np.arange(1, 8, 2)])  # new dim j <- old perm[j]
    back = np.argsort(perm)
    np.testing.assert_array_equal(O.rope_rotate_half(x[..., perm], phi)[..., back], got)


def test_softmax_rows_sum_to_one_and_mask():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((6, 100)) * 30
    s[:, 50:] = -np.inf
    p = O.softmax(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=100 * np.finfo(np.float64).eps)
    assert np.all(p[:, 50:] == 0)


def test_next_token_probs_closed_forms():
    """Two logits give the logistic function of their difference; equal
    logits give the uniform distribution; adding a constant changes nothing;
    the largest logit keeps the largest probability; torch's softmax (an
    independent routine) agrees."""
    d = np.array([-4.0, -0.5, 0.0, 2.0, 30.0])
    two = np.stack([d, np.zeros_like(d)], -1)
    p = O.next_token_probs(two)
    np.testing.assert_allclose(p[:, 0], 1 / (1 + np.exp(-d)), rtol=2e-7)
    np.testing.assert_allclose(O.next_token_probs(np.full((1, 7), 3.5)), 1 / 7, rtol=1e-7)
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((3, 1000)) * 8).astype(np.float32)
    np.testing.assert_array_equal(O.next_token_probs(x), O.next_token_probs(x.astype(np.float64) + 1e3))
    assert np.array_equal(np.argmax(O.next_token_probs(x), -1), np.argmax(x, -1))
    ref = torch.softmax(torch.tensor(x, dtype=torch.float64), -1).numpy()
    np.testing.assert_allclose(O.next_token_probs(x), ref, rtol=1e-6, atol=1e-30)


def test_stop_positions_brute_force():
    """The earliest read-out position per slot whose id is a stop id,
    against a scan over every (slot, position) on small random histories."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        n_seq = int(rng.integers(1, 4))
        stop = list(rng.integers(0, 6, rng.integers(0, 3)))
        reads = [(int(rng.integers(0, n_seq)), int(rng.integers(0, 20)), int(rng.integers(0, 6)))
                 for _ in range(rng.integers(0, 12))]
        got = O.stop_positions(n_seq, reads, stop)
        for s_ in range(n_seq):
            hits = [p for p in range(20) for (q, pp, t) in reads if q == s_ and pp == p and t in stop]
            assert got[s_] == (min(hits) if hits else -1)
    assert list(O.stop_positions(2, [(0, 5, 9), (0, 3, 9), (1, 4, 8)], [9])) == [3, -1]


def test_silu_closed_form():
    z = np.array([-3.0, 0.0, 1.5])
    np.testing.assert_allclose(O.silu(z), z * (1 / (1 + np.exp(-z))), rtol=1e-15)
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(torch.tensor(z)).numpy(), rtol=1e-15)


def test_argmax_ties_and_nan():
    v = np.array([1.0, 3.0, np.nan, 3.0, -1.0], np.float32)
    assert O.argmax_lowest(v) == 1
    assert O.argmax_lowest(np.array([np.nan, np.nan], np.float32)) == 0
    assert O.argmax_lowest(np.array([-np.inf, -5.0], np.float32)) == 1


# ---------------------------------------------------------------- model-level
def build(shape, n_ctx=64, n_seq=1):
    w = syn.make_weights(shape)
    return O.Qwen2Oracle(O.hparams_for(shape, n_ctx, n_seq), w), w


def brute_force(shape, w, tokens, interleaved=False):
    """Full-sequence forward with a dense causal mask, no cache, all float64.
    Returns (logits of every row, list of layer outputs)."""
    H, nh, nkv, hd, eps = shape.n_embd, shape.n_head, shape.n_head_kv, shape.head_dim, shape.rms_eps
    n = len(tokens)
    h = f16(w["tok_embd"])[tokens]
    pos = np.arange(n)
    inv = shape.rope_theta ** (-np.arange(0, hd, 2) / hd)
    rot = np.exp(1j * pos[:, None] * inv[None, :])[:, None, :]

    def rope(x):
        if interleaved:
            z = (x[..., 0::2] + 1j * x[..., 1::2]) * rot
            out = np.empty_like(x)
            out[..., 0::2], out[..., 1::2] = z.real, z.imag
            return out
        z = (x[..., :hd // 2] + 1j * x[..., hd // 2:]) * rot
        return np.concatenate([z.real, z.imag], -1)

    def norm(x, g):
        return x / np.sqrt((x ** 2).mean(-1, keepdims=True) + eps) * g

    causal = np.tril(np.ones((n, n), dtype=bool))
    outs = []
    for L in w["layers"]:
        x = norm(h, L["attn_norm"].astype(np.float64))
        q = rope((x @ f16(L["wq"]).T + L["bq"]).reshape(n, nh, hd))
        k = rope((x @ f16(L["wk"]).T + L["bk"]).reshape(n, nkv, hd))
        v = (x @ f16(L["wv"]).T + L["bv"]).reshape(n, nkv, hd)
        k = np.repeat(k, nh // nkv, axis=1)
        v = np.repeat(v, nh // nkv, axis=1)
        s = np.einsum("ihd,jhd->hij", q, k) / math.sqrt(hd)
        s = np.where(causal[None], s, -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        o = np.einsum("hij,jhd->ihd", p, v).reshape(n, nh * hd)
        h = h + o @ f16(L["wo"]).T
        x = norm(h, L["ffn_norm"].astype(np.float64))
        gt = x @ f16(L["w_gate"]).T
        up = x @ f16(L["w_up"]).T
        h = h + (gt / (1 + np.exp(-gt)) * up) @ f16(L["w_down"]).T
        outs.append(h)
    y = norm(h, w["out_norm"].astype(np.float64))
    lm = w["tok_embd"] if shape.tied else w["lm_head"]
    return y @ f16(lm).T, outs


def rel_err(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.max(np.abs(ref)))


@pytest.mark.parametrize("kv", [2, 4, 1])
def test_oracle_matches_brute_force(kv):
    shape = syn.MODELS["tiny"] if kv == 2 else tiny_variant(n_head_kv=kv)
    orc, w = build(shape)
    toks = syn.make_prompt(shape, 16)
    ref, outs = brute_force(shape, w, toks)
    # prefill the first 8, then decode the other 8 one by one
    r = orc.prefill(0, toks[:8], np.arange(8))
    assert rel_err(r.logits[0], ref[7]) < 1e-6
    assert rel_err(r.layer_output[0], outs[-1][7]) < 1e-6
    for i in range(8, 16):
        r = orc.decode([0], [toks[i]], [i])
        assert rel_err(r.logits[0], ref[i]) < 1e-6, i
        assert r.argmax[0] == int(np.argmax(ref[i]))


@pytest.mark.parametrize("kv", [2, 4, 1])
def test_interleaved_model_matches_brute_force(kv):
    """The model-level Interleaved flag (minfer page, section 3) wired through
    the whole oracle: q and k both rotated in 2d / 2d+1 pairs, v not at all,
    on GQA, MHA and MQA layouts, prefill then cached decode steps."""
    shape = syn.MODELS["tiny"] if kv == 2 else tiny_variant(n_head_kv=kv)
    w = syn.make_weights(shape)
    orc = O.Qwen2Oracle(O.hparams_for(shape, 64, 1, rope_style=1), w)
    toks = syn.make_prompt(shape, 14, 9)
    ref, outs = brute_force(shape, w, toks, interleaved=True)
    r = orc.prefill(0, toks[:9], np.arange(9))
    assert rel_err(r.logits[0], ref[8]) < 1e-6
    assert rel_err(r.layer_output[0], outs[-1][8]) < 1e-6
    for i in range(9, 14):
        r = orc.decode([0], [toks[i]], [i])
        assert rel_err(r.logits[0], ref[i]) < 1e-6, i
        assert r.argmax[0] == int(np.argmax(ref[i]))
    # and the flag matters: the NonInterleaved brute force disagrees
    ref_ni, _ = brute_force(shape, w, toks, interleaved=False)
    assert rel_err(r.logits[0], ref_ni[13]) > 1e-3


def test_interleaved_pin_catches_a_half_wired_flag(monkeypatch):
    """Planted mistake: the Interleaved pairing applied to q but the
    NonInterleaved one to k.  The model-level pin above must reject it."""
    shape = syn.MODELS["tiny"]
    w = syn.make_weights(shape)
    toks = syn.make_prompt(shape, 10, 9)
    ref, _ = brute_force(shape, w, toks, interleaved=True)
    calls = {"n": 0}
    real = O.rope_interleaved

    def q_only(x, phi):
        calls["n"] += 1
        return real(x, phi) if calls["n"] % 2 == 1 else O.rope_rotate_half(x, phi)

    monkeypatch.setattr(O, "rope_interleaved", q_only)
    orc = O.Qwen2Oracle(O.hparams_for(shape, 64, 1, rope_style=1), w)
    r = orc.prefill(0, toks, np.arange(10))
    assert calls["n"] == 2 * shape.n_layer
    assert rel_err(r.logits[0], ref[9]) > 1e-3


def test_wrong_rope_style_is_detected_by_brute_force():
    shape = syn.MODELS["tiny"]
    orc, w = build(shape)
    toks = syn.make_prompt(shape, 12)
    ref_bad, _ = brute_force(shape, w, toks, interleaved=True)
    r = orc.prefill(0, toks, np.arange(12))
    assert rel_err(r.logits[0], ref_bad[-1]) > 1e-3


def test_single_key_attention_returns_v():
    shape = syn.MODELS["tiny"]
    orc, w = build(shape)
    r = orc.prefill(0, syn.make_prompt(shape, 1), [0], taps=True)
    for lt in r.taps["layers"]:
        o = lt["attention_head_outputs"][0]            # [nh, hd]
        v = lt["attention_values"][:, 0]               # [nkv, hd]
        for h in range(shape.n_head):
            assert np.array_equal(o[h], v[h // (shape.n_head // shape.n_head_kv)])


def test_mha_special_case_equals_torch_sdpa():
    shape = tiny_variant(n_head_kv=4)
    orc, w = build(shape)
    r = orc.prefill(0, syn.make_prompt(shape, 10), np.arange(10), taps=True)
    for lt in r.taps["layers"]:
        q = torch.from_numpy(lt["attention_queries"]).double()[None]   # [1, nh, n, hd]
        k = torch.from_numpy(lt["attention_keys"]).double()[None]
        v = torch.from_numpy(lt["attention_values"]).double()[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
        got = np.transpose(lt["attention_head_outputs"], (1, 0, 2))
        np.testing.assert_allclose(got, ref[0].numpy(), rtol=0, atol=2e-7 * float(ref.abs().max()) + 1e-12)


def test_gqa_mapping_kv_head_j_reaches_group_j_only():
    # 14 query heads over 2 KV heads, as on the 0.5B shape (group 7).
    shape = tiny_variant(n_embd=224, n_head=14, n_head_kv=2, head_dim=16)
    w = syn.make_weights(shape)
    hp = O.hparams_for(shape, 32)
    toks = syn.make_prompt(shape, 6)
    base = O.Qwen2Oracle(hp, w).prefill(0, toks, np.arange(6), taps=True)
    for j in range(2):
        w2 = dict(w)
        w2["layers"] = [dict(L) for L in w["layers"]]
        wk = w2["layers"][0]["wk"].copy()
        wk[j * 16:(j + 1) * 16] ^= np.uint16(0x0400)  # perturb every row of KV head j
        w2["layers"][0]["wk"] = wk
        pert = O.Qwen2Oracle(hp, w2).prefill(0, toks, np.arange(6), taps=True)
        a = base.taps["layers"][0]["attention_head_outputs"]
        b = pert.taps["layers"][0]["attention_head_outputs"]
        for h in range(14):
            changed = not np.array_equal(a[:, h], b[:, h])
            assert changed == (7 * j <= h <= 7 * j + 6), (j, h)


def test_bias_is_added_before_rope_zero_input():
    shape = syn.MODELS["tiny"]
    w = syn.make_weights(shape)
    w["layers"] = [dict(L) for L in w["layers"]]
    w["layers"][0]["attn_norm"] = np.zeros_like(w["layers"][0]["attn_norm"])
    hp = O.hparams_for(shape, 64)
    orc = O.Qwen2Oracle(hp, w)
    pos = np.array([0, 3, 5, 20, 63])
    r = orc.prefill(0, syn.make_prompt(shape, 5), pos, taps=True)
    L0 = w["layers"][0]
    hd, nkv = shape.head_dim, shape.n_head_kv
    bk = L0["bk"].astype(np.float64).reshape(nkv, hd)
    bv = L0["bv"].astype(np.float64).reshape(nkv, hd)
    inv = shape.rope_theta ** (-np.arange(0, hd, 2) / hd)
    K, V = orc.k_cache[0][0], orc.v_cache[0][0]
    for p in pos:
        z = (bk[:, :hd // 2] + 1j * bk[:, hd // 2:]) * np.exp(1j * p * inv)
        np.testing.assert_allclose(K[:, p], np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-7)
        np.testing.assert_array_equal(V[:, p], L0["bv"].reshape(nkv, hd))
    # With contiguous positions every visible slot holds the same value
    # vector per KV head, so attention_output = Wo . bv at every position.
    orc2 = O.Qwen2Oracle(hp, w)
    r = orc2.prefill(0, syn.make_prompt(shape, 7), np.arange(7), taps=True)
    o = np.repeat(bv, shape.n_head // nkv, axis=0).reshape(-1)
    ref = f16(L0["wo"]) @ o
    got = r.taps["layers"][0]["attention_output"]
    for i in range(7):
        np.testing.assert_allclose(got[i], ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def test_residual_identity_and_readout():
    shape = syn.MODELS["tiny"]
    orc, w = build(shape)
    r = orc.prefill(0, syn.make_prompt(shape, 9), np.arange(9), taps=True)
    for lt in r.taps["layers"]:
        lhs = lt["layer_input"].astype(np.float64) + lt["attention_output"] + lt["mlp_output"]
        np.testing.assert_allclose(lhs, lt["layer_output"], rtol=0,
                                   atol=4 * np.finfo(np.float32).eps * np.abs(lhs).max())
    last = torch.from_numpy(r.taps["layers"][-1]["layer_output"][-1:]).double()
    y = torch.nn.functional.rms_norm(last, (shape.n_embd,), torch.from_numpy(w["out_norm"]).double(), eps=1e-6)
    logits = y.numpy() @ f16(w["tok_embd"]).T
    np.testing.assert_allclose(r.logits, logits, rtol=0, atol=1e-6 * np.abs(logits).max())
    assert r.argmax[0] == int(np.argmax(r.logits[0]))


def test_full_causal_first_token_reaches_last_row_and_future_is_invisible():
    shape = syn.MODELS["tiny"]
    w = syn.make_weights(shape)
    hp = O.hparams_for(shape, 64)
    toks = syn.make_prompt(shape, 48)
    a = O.Qwen2Oracle(hp, w).prefill(0, toks, np.arange(48), taps=True)
    t2 = toks.copy()
    t2[0] = (t2[0] + 1) % shape.n_vocab
    b = O.Qwen2Oracle(hp, w).prefill(0, t2, np.arange(48))
    assert np.max(np.abs(a.logits - b.logits)) > 0
    t3 = toks.copy()
    t3[30] = (t3[30] + 1) % shape.n_vocab
    c = O.Qwen2Oracle(hp, w).prefill(0, t3, np.arange(48), taps=True)
    for la, lc in zip(a.taps["layers"], c.taps["layers"]):
        assert np.array_equal(la["layer_output"][:30], lc["layer_output"][:30])
        assert not np.array_equal(la["layer_output"][30:], lc["layer_output"][30:])


def test_prefill_equals_prefill_then_decode():
    shape = syn.MODELS["tiny"]
    w = syn.make_weights(shape)
    hp = O.hparams_for(shape, 64)
    toks = syn.make_prompt(shape, 20)
    a = O.Qwen2Oracle(hp, w).prefill(0, toks, np.arange(20))
    o2 = O.Qwen2Oracle(hp, w)
    o2.prefill(0, toks[:19], np.arange(19))
    b = o2.decode([0], toks[19:], [19])
    np.testing.assert_allclose(a.logits, b.logits, rtol=0, atol=2 * np.finfo(np.float32).eps * np.abs(a.logits).max())
    assert a.argmax[0] == b.argmax[0]


def test_sequences_do_not_interact():
    shape = syn.MODELS["tiny"]
    w = syn.make_weights(shape)
    hp = O.hparams_for(shape, 64, n_seq=3)
    t0, t1 = syn.make_prompt(shape, 6, 0), syn.make_prompt(shape, 9, 1)
    o = O.Qwen2Oracle(hp, w)
    o.prefill(0, t0, np.arange(6))
    o.prefill(2, t1, np.arange(9))
    r = o.decode([2, 0], [5, 7], [9, 6])
    s0 = O.Qwen2Oracle(hp, w)
    s0.prefill(0, t0, np.arange(6))
    r0 = s0.decode([0], [7], [6])
    np.testing.assert_allclose(r.logits[1], r0.logits[0], rtol=0, atol=1e-6 * np.abs(r0.logits).max())


# ---------------------------------------------------------------- validation
def test_hard_errors_leave_cache_untouched():
    shape = syn.MODELS["tiny"]
    orc, w = build(shape, n_ctx=16, n_seq=2)
    orc.prefill(0, [1, 2, 3], [0, 1, 2])
    K0, V0 = orc.k_cache[0].copy(), orc.v_cache[0].copy()
    cases = [
        ("E_POS", lambda: orc.prefill(0, [4, 5], [3, 16])),       # position == n_ctx
        ("E_POS", lambda: orc.prefill(0, [4], [-1])),
        ("E_TOKEN", lambda: orc.prefill(0, [4, shape.n_vocab], [3, 4])),
        ("E_SEQ", lambda: orc.prefill(2, [4], [3])),
        ("E_SEQ", lambda: orc.decode([0, 0], [1, 2], [3, 4])),
        ("E_ORDER", lambda: orc.prefill(0, [4, 5, 6], [3, 5, 4])),
        ("E_ORDER", lambda: orc.prefill(0, [4, 5], [3, 3])),
        ("E_ARG", lambda: orc.prefill(0, [], [])),
        ("E_POS", lambda: orc.decode([0, 1], [1, 2], [3, 16])),
    ]
    for code, call in cases:
        with pytest.raises(O.OracleError) as e:
            call()
        assert e.value.code == code
        assert np.array_equal(orc.k_cache[0], K0) and np.array_equal(orc.v_cache[0], V0)
    with pytest.raises(O.OracleError) as e:
        O.Qwen2Oracle(dataclasses.replace(orc.hp, n_head_kv=3), w)
    assert e.value.code == "E_HPARAMS"
