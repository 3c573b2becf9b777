"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and its host-side validation (which runs before anything is
enqueued) agrees with the oracle's error codes.  No GPU call is made."""
import dataclasses
import os
import re

import numpy as np
import pytest

import qwen2_synth as syn
from oracle import qwen2_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qwen2.h")

q = pytest.importorskip("qwen2_decoder_forward_amd")
if not os.path.exists(q.LIB_PATH):
    pytest.skip("library not built", allow_module_level=True)


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwen2_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = q.lib()
    names = declared()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(L, n), n


def test_struct_sizes_match_header_layout():
    import ctypes
    assert ctypes.sizeof(q.Hparams) == 11 * 4 + 3 * 4
    assert ctypes.sizeof(q.LayerWeights) == 12 * 8
    assert ctypes.sizeof(q.Weights) == 4 * 8


def test_strerror_names():
    for code, name in q.CODES.items():
        assert q.qwen2_strerror(code)
    assert "n_ctx" in q.qwen2_strerror(-3)


def hp_for(shape, n_ctx=16, n_seq=2):
    return q.make_hparams(shape, n_ctx, n_seq)


def oracle_code(fn):
    try:
        fn()
    except O.OracleError as e:
        return e.code
    return "OK"


def test_validation_matches_oracle():
    shape = syn.MODELS["tiny"]
    hp = hp_for(shape)
    ohp = O.hparams_for(shape, 16, 2)
    orc = O.Qwen2Oracle(ohp, syn.make_weights(shape))
    V = shape.n_vocab
    prefill_cases = [
        (0, [1, 2], [0, 1]), (0, [1, 2], [3, 16]), (0, [4], [-1]), (0, [4, V], [3, 4]),
        (0, [-1], [0]), (2, [4], [3]), (-1, [4], [3]), (0, [4, 5, 6], [3, 5, 4]),
        (0, [4, 5], [3, 3]), (0, [], []), (1, [V, 1], [99, 0]),  # token checked before position
        (0, list(range(16)), list(range(16))),
    ]
    for seq, toks, pos in prefill_cases:
        got = q.CODES[q.qwen2_check_prefill(hp, seq, toks, pos)]
        want = oracle_code(lambda: orc._validate([seq] * len(toks), toks, pos, prefill=True)
                           if toks else orc.prefill(seq, toks, pos))
        assert got == want, (seq, toks, pos, got, want)
    decode_cases = [
        ([0, 1], [3, 4]), ([0, 0], [3, 4]), ([0, 2], [3, 4]), ([1], [16]), ([1], [-5]),
        ([1, 0], [15, 0]), ([], []),
    ]
    for seqs, pos in decode_cases:
        got = q.CODES[q.qwen2_check_decode(hp, seqs, pos)]
        want = oracle_code(lambda: orc._validate(seqs, [0] * len(seqs), pos, prefill=False))
        assert got == want, (seqs, pos, got, want)


def test_batch_validation():
    """A batched prefill is valid exactly when its slots are distinct and each
    sequence would pass qwen2_check_prefill on its own; errors report in the
    header's order (arguments, slots, then sequence by sequence)."""
    shape = syn.MODELS["tiny"]
    hp = hp_for(shape)  # n_ctx 16, n_seq 2
    V = shape.n_vocab
    cases = [
        (([0, 1], [[1, 2], [3]], [[0, 1], [5]]), "OK"),
        (([1], [[1]], [[15]]), "OK"),
        (([], [], []), "E_ARG"),
        (([0, 1], [[1], []], [[0], []]), "E_ARG"),          # an empty sequence
        (([0, 0], [[1], [2]], [[0], [1]]), "E_SEQ"),        # repeated slot
        (([0, 2], [[1], [2]], [[0], [1]]), "E_SEQ"),        # slot out of range
        (([0, 0], [[V], [2]], [[0], [1]]), "E_SEQ"),        # slots before tokens
        (([0, 1], [[1], [V]], [[0], [1]]), "E_TOKEN"),
        (([0, 1], [[1], [2]], [[0], [16]]), "E_POS"),
        (([0, 1], [[1, 2], [2]], [[3, 3], [1]]), "E_ORDER"),
        (([1, 0], [[1, V], [2]], [[0, 1], [-1]]), "E_TOKEN"),  # the first bad sequence reports
        (([1, 0], [[1, 2], [V]], [[1, 0], [1]]), "E_ORDER"),
    ]
    for (seqs, toks, pos), want in cases:
        got = q.CODES[q.qwen2_check_prefill_batch(hp, seqs, toks, pos)]
        assert got == want, (seqs, toks, pos, got, want)
    # when every slot is distinct, the batch's verdict is that of the first
    # failing sequence checked alone
    rng = np.random.default_rng(5)
    for _ in range(200):
        nb = int(rng.integers(1, 3))
        seqs = list(rng.permutation(2)[:nb])
        toks = [list(rng.integers(-1, V + 1, rng.integers(1, 4))) for _ in range(nb)]
        pos = [sorted(rng.integers(-1, 17, len(t))) for t in toks]
        singles = [q.CODES[q.qwen2_check_prefill(hp, s, t, p)] for s, t, p in zip(seqs, toks, pos)]
        want = next((c for c in singles if c != "OK"), "OK")
        assert q.CODES[q.qwen2_check_prefill_batch(hp, seqs, toks, pos)] == want


@pytest.mark.parametrize("change,ok", [
    ({}, True),
    ({"n_head_kv": 3}, False),             # n_head % n_head_kv
    ({"head_dim": 32, "n_embd": 128}, False),  # head_dim not in {16, 64, 128}
    ({"n_embd": 80, "n_head": 5}, False),  # n_embd % 64
    ({"n_embd": 128}, False),              # n_embd != n_head * head_dim
    ({"n_head": 36, "n_head_kv": 4, "n_embd": 576}, False),  # group 9 > 8
    ({"n_head_kv": 4}, True),              # MHA
    ({"n_head_kv": 1}, True),              # MQA, group 4
    ({"n_embd": 8192, "n_head": 64, "n_head_kv": 8, "head_dim": 128}, True),   # 64/8 heads (72B)
    ({"n_embd": 8320, "n_head": 65, "n_head_kv": 5, "head_dim": 128}, False),  # n_embd > 8192
])
def test_hparams_checks(change, ok):
    shape = dataclasses.replace(syn.MODELS["tiny"], **change)
    hp = hp_for(shape)
    assert (q.qwen2_check_hparams(hp) == 0) == ok


def test_rope_style_and_bad_scalars_rejected():
    hp = hp_for(syn.MODELS["tiny"])
    hp.rope_style = 1  # Interleaved: a model-level flag
    assert q.CODES[q.qwen2_check_hparams(hp)] == "OK"
    for bad in (2, -1):
        hp.rope_style = bad
        assert q.CODES[q.qwen2_check_hparams(hp)] == "E_HPARAMS"
    hp = hp_for(syn.MODELS["tiny"])
    hp.rope_theta = 0.0
    assert q.CODES[q.qwen2_check_hparams(hp)] == "E_HPARAMS"
    hp = hp_for(syn.MODELS["tiny"])
    hp.n_ctx = 0
    assert q.CODES[q.qwen2_check_hparams(hp)] == "E_HPARAMS"


def test_real_shapes_are_accepted():
    for name in syn.MODELS:
        assert q.qwen2_check_hparams(hp_for(syn.MODELS[name], 4096, 1)) == 0, name


def test_probe_arguments_rejected_before_any_launch():
    """The ceiling probes check their arguments on the host (no device is
    touched for a rejected call) and report through qwen2_last_error(NULL)."""
    L = q.lib()
    out = 4096  # (a non-null stand-in address; never dereferenced here)
    for buf, nbytes, nb in ((None, 1 << 20, 64), (out, 15, 64), (out, 0, 64), (out, 1 << 20, 0),
                            (out, 1 << 20, 65537)):
        assert L.qwen2_probe_read(buf, nbytes, nb, out, None) == -1
        assert b"qwen2_probe_read" in L.qwen2_last_error(None)
    for iters, nb, o in ((0, 64, out), (10, 0, out), (10, 64, None), (10, 70000, out)):
        assert L.qwen2_probe_mfma(iters, nb, o, None) == -1
        assert b"qwen2_probe_mfma" in L.qwen2_last_error(None)
