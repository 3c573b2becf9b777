"""Pin the oracle to an independent library implementation of the same model:
Hugging Face ``transformers``' Qwen2ForCausalLM (the module tree the nnterp
Qwen2 encyclopedia page documents), run on the CPU in float64 with the same
binary16 weights.  Then plant plausible mistakes in the oracle and check that
this pin catches each one.

The library computes its rotary angles and its softmax in float32 even in a
float64 model, so agreement is bounded by float32 rounding (a few 1e-6
relative), far below what any planted mistake produces.
"""
import dataclasses

import numpy as np
import pytest
import torch

import qwen2_synth as syn
from oracle import qwen2_oracle as O

transformers = pytest.importorskip("transformers")

TOL = 2e-5  # max-abs error / max |ref|


def f16t(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.float16).astype(np.float64))


def hf_model(shape, w):
    cfg = transformers.Qwen2Config(
        vocab_size=shape.n_vocab, hidden_size=shape.n_embd, intermediate_size=shape.n_ff,
        num_hidden_layers=shape.n_layer, num_attention_heads=shape.n_head,
        num_key_value_heads=shape.n_head_kv, rope_theta=shape.rope_theta,
        rms_norm_eps=shape.rms_eps, tie_word_embeddings=shape.tied,
        max_position_embeddings=8192, use_sliding_window=False)
    cfg._attn_implementation = "eager"
    torch.manual_seed(0)
    m = transformers.Qwen2ForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": f16t(w["tok_embd"]),
          "model.norm.weight": torch.from_numpy(w["out_norm"]).double(),
          "lm_head.weight": f16t(w["tok_embd"] if shape.tied else w["lm_head"])}
    for i, L in enumerate(w["layers"]):
        p = f"model.layers.{i}."
        sd[p + "input_layernorm.weight"] = torch.from_numpy(L["attn_norm"]).double()
        sd[p + "post_attention_layernorm.weight"] = torch.from_numpy(L["ffn_norm"]).double()
        for ours, theirs in (("wq", "q_proj"), ("wk", "k_proj"), ("wv", "v_proj"), ("wo", "o_proj")):
            sd[p + f"self_attn.{theirs}.weight"] = f16t(L[ours])
        for b, theirs in (("bq", "q_proj"), ("bk", "k_proj"), ("bv", "v_proj")):
            sd[p + f"self_attn.{theirs}.bias"] = torch.from_numpy(L[b]).double()
        for ours, theirs in (("w_gate", "gate_proj"), ("w_up", "up_proj"), ("w_down", "down_proj")):
            sd[p + f"mlp.{theirs}.weight"] = f16t(L[ours])
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in k for k in missing), (missing, unexpected)
    return m


def hf_run(m, tokens):
    with torch.no_grad():
        out = m(torch.from_numpy(np.asarray(tokens, np.int64))[None], output_hidden_states=True)
    return out.logits[0].numpy(), [h[0].numpy() for h in out.hidden_states]


def rel(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.max(np.abs(ref)))


def oracle_run(shape, w, tokens, n_ctx=256):
    orc = O.Qwen2Oracle(O.hparams_for(shape, n_ctx), w)
    return orc.prefill(0, tokens, np.arange(len(tokens)), taps=True)


def compare(shape, w, tokens, hf):
    logits, hs = hf
    r = oracle_run(shape, w, tokens)
    errs = [rel(r.taps["token_embeddings"], hs[0])]
    for l in range(shape.n_layer - 1):
        errs.append(rel(r.taps["layers"][l]["layer_output"], hs[l + 1]))
    errs.append(rel(r.final_norm_output[0], hs[-1][-1]))
    errs.append(rel(r.logits[0], logits[-1]))
    return max(errs), r, logits


SHAPES = {
    "tiny": syn.MODELS["tiny"],
    # the 0.5B shape (hd 64, group 7, full vocabulary), 2 layers
    "0.5b-L2": syn.model_shape("qwen2.5-0.5b", n_layer=2),
    # hd 128, group 7, untied head, reduced width so the test stays fast
    "hd128-narrow": dataclasses.replace(syn.MODELS["qwen2-hd128"], name="hd128-narrow", n_layer=2,
                                        n_embd=896, n_head=7, n_head_kv=1, n_ff=640, n_vocab=4096),
    "mha": dataclasses.replace(syn.MODELS["tiny"], name="tiny-mha", n_head_kv=4),
}


@pytest.fixture(scope="module")
def cases():
    out = {}
    for name, shape in SHAPES.items():
        w = syn.make_weights(shape)
        n = 24 if name != "tiny" else 40
        toks = syn.make_prompt(shape, n)
        out[name] = (shape, w, toks, hf_run(hf_model(shape, w), toks))
    return out


@pytest.mark.parametrize("name", list(SHAPES))
def test_oracle_matches_transformers_qwen2(cases, name):
    shape, w, toks, hf = cases[name]
    err, r, logits = compare(shape, w, toks, hf)
    assert err < TOL, err
    assert r.argmax[0] == int(np.argmax(logits[-1]))


MUTATIONS = {
    "interleaved rope": ("rope_rotate_half", lambda orig: O.rope_interleaved),
    "gqa mapping h % n_kv": ("kv_head_of", lambda orig: (lambda h, nh, nkv: h % nkv)),
    "bias dropped": ("linear", lambda orig: (lambda x, wb, b=None, w64=None: orig(x, wb, None, w64))),
    "scale 1/head_dim": ("attention_scale", lambda orig: (lambda hd: 1.0 / hd)),
    "norm with mean subtracted": ("rms_norm", lambda orig: (
        lambda h, w, eps: orig(np.asarray(h, np.float64) - np.mean(h, -1, keepdims=True), w, eps))),
    "silu replaced by sigmoid": ("silu", lambda orig: (lambda z: 1 / (1 + np.exp(-np.asarray(z, np.float64))))),
    "rope sign flipped": ("rope_angles", lambda orig: (lambda p, hd, th, fs=1.0: -orig(p, hd, th, fs))),
}


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_planted_oracle_mistake_is_caught(cases, monkeypatch, mutation):
    attr, make = MUTATIONS[mutation]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    shape, w, toks, hf = cases["0.5b-L2"]
    err, _, _ = compare(shape, w, toks, hf)
    assert err > 50 * TOL, (mutation, err)
