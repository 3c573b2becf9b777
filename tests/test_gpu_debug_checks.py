"""Debug checks (QWEN2_DEBUG_CHECKS=1 at load; the GPU guards of the minfer
page, section 7, that fail with the offending values).

* Valid calls (prefill with a gapped continuation, one- and two-row decode, a
  batched prefill) pass every check, and give the logits and ids of a context
  without the checks (to rounding: the residual adds are float atomics).
* Non-finite logits (binary16 NaN lm_head rows) and non-finite K (a NaN K
  bias) are reported as QWEN2_E_DEBUG with their place and value.
"""
import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import qwen2_decoder_forward_amd as q  # noqa: E402
import qwen2_synth as syn  # noqa: E402
from gpu_common import DEV, say  # noqa: E402

pytestmark = pytest.mark.gpu

SHAPE = dataclasses.replace(syn.MODELS["tiny"], name="tiny-untied", tied=False)
F16_NAN = 0x7E00


def model(w, debug, n_seq=4):
    if debug:
        os.environ["QWEN2_DEBUG_CHECKS"] = "1"
    try:
        return q.Model(SHAPE, w, n_ctx=64, n_seq=n_seq)
    finally:
        os.environ.pop("QWEN2_DEBUG_CHECKS", None)


def run_calls(m):
    """A fixed sequence of valid calls; returns every logits row and id."""
    V = SHAPE.n_vocab
    outs = []
    lg = torch.zeros(V, device=DEV)
    ids = torch.zeros(4, dtype=torch.int32, device=DEV)
    p0 = syn.make_prompt(SHAPE, 9, 1)
    m.prefill(0, p0, np.arange(9), lg, ids[0:1])
    outs.append((lg.clone(), ids[0:1].clone()))
    m.prefill(0, syn.make_prompt(SHAPE, 3, 2), np.array([12, 13, 20]), lg, ids[0:1])  # gapped
    outs.append((lg.clone(), ids[0:1].clone()))
    m.decode([0], ids[0:1], [21], lg, ids[1:2])
    outs.append((lg.clone(), ids[1:2].clone()))
    lg2 = torch.zeros((3, V), device=DEV)
    toks = [syn.make_prompt(SHAPE, n, 3 + n) for n in (5, 11, 2)]
    m.prefill_batch([1, 2, 3], toks, [np.arange(len(t)) for t in toks], lg2, ids[0:3])
    outs.append((lg2.clone(), ids[0:3].clone()))
    m.decode([1, 3], ids[0:2], [5, 2], lg2[:2], ids[2:4])
    outs.append((lg2[:2].clone(), ids[2:4].clone()))
    torch.cuda.synchronize()
    return outs


def test_valid_calls_pass_and_match_unchecked():
    w = syn.make_weights(SHAPE)
    say("[debug-checks] valid calls with and without the checks")
    ref = run_calls(model(w, False))
    got = run_calls(model(w, True))
    # (float atomics order the residual adds differently from run to run,
    # so the two contexts agree to rounding, not bit for bit)
    for (a, ia), (b, ib) in zip(ref, got):
        a, b = a.cpu().numpy().reshape(len(ia), -1), b.cpu().numpy().reshape(len(ia), -1)
        assert np.max(np.abs(a - b)) <= 1e-4 * np.max(np.abs(a))
        for r in range(len(ia)):
            top2 = np.sort(a[r])[-2:]
            if top2[1] - top2[0] > 1e-3:
                assert int(ia[r]) == int(ib[r])


def test_nonfinite_logits_reported():
    w = syn.make_weights(SHAPE)
    lm = w["lm_head"].copy()
    lm[[3, 77]] = F16_NAN
    w["lm_head"] = lm
    m = model(w, True)
    lg = torch.zeros(SHAPE.n_vocab, device=DEV)
    ids = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("[debug-checks] NaN lm_head rows")
    with pytest.raises(q.Qwen2Error) as e:
        m.prefill(0, syn.make_prompt(SHAPE, 4, 5), np.arange(4), lg, ids)
    assert e.value.code == -9
    assert "logit" in str(e.value) and "id 3" in str(e.value) and "nan" in str(e.value).lower()
    with pytest.raises(q.Qwen2Error) as e:
        m.decode([0], ids, [4], lg, ids)
    assert e.value.code == -9 and "id 3" in str(e.value)


def test_nonfinite_k_reported():
    w = syn.make_weights(SHAPE)
    bk = w["layers"][1]["bk"].copy()
    bk[5] = np.nan
    w["layers"][1]["bk"] = bk
    m = model(w, True)
    lg = torch.zeros(SHAPE.n_vocab, device=DEV)
    ids = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("[debug-checks] NaN K bias of layer 1")
    with pytest.raises(q.Qwen2Error) as e:
        m.prefill(0, syn.make_prompt(SHAPE, 6, 6), np.arange(6), lg, ids)
    msg = str(e.value)
    assert e.value.code == -9 and "non-finite K" in msg and "layer 1" in msg, msg
