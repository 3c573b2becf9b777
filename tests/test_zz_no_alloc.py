"""The allocation-free entry point qwen2_next_token_probs_static against the
context form qwen2_next_token_probs on the same logits: two calls in a row
(the second with fewer rows, so the fixed scratch holds the first call's
partials when the second starts), each compared with the context form to the
softmax bar of the next_token_probs tests (|p - ref| <= 1e-5 ref + 1e-38,
rows summing to 1 within 1e-5) and with the oracle's softmax; then a call
over a shorter vocabulary than the model's, against the oracle."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import qwen2_decoder_forward_amd as q  # noqa: E402
import qwen2_synth as syn  # noqa: E402
from gpu_common import DEV, check_probs, say  # noqa: E402

pytestmark = pytest.mark.gpu


def test_static_probs_match_context_probs_twice():
    shape = dataclasses.replace(syn.MODELS["tiny"], name="tiny-V151936", n_vocab=151936)
    w = syn.make_weights(shape)
    m = q.Model(shape, w, n_ctx=64, n_seq=64)
    rng = np.random.default_rng(11)
    # two calls compared with the context form (the second on fewer rows),
    # then one with a shorter vocabulary than the model's, against the oracle
    for rows, V in ((64, 151936), (3, 151936), (5, 40000)):
        say(f"[no-alloc] rows {rows}, vocabulary {V}")
        lg = (rng.standard_normal((rows, V)) * 4).astype(np.float32)
        lg[0, 5] = 60.0  # a dominant entry: its probability is close to 1
        logits = torch.from_numpy(lg).to(DEV)
        ref_probs = torch.empty_like(logits)
        got = torch.full_like(logits, float("nan"))
        if V == shape.n_vocab:
            m.next_token_probs(logits, rows, ref_probs)
        q.qwen2_next_token_probs_static(logits, rows, V, got)
        torch.cuda.synchronize()
        g = got.cpu().numpy()
        check_probs(g, lg, f"static rows {rows} V {V}")
        if V == shape.n_vocab:
            r = ref_probs.cpu().numpy()
            assert np.max(np.abs(g - r) - 1e-5 * r) <= 1e-38, "static vs context form"
    m.close()


def test_static_probs_rejects_bad_sizes():
    lg = torch.zeros((2, 8), device=DEV)
    pr = torch.empty_like(lg)
    for rows, V in ((0, 8), (65, 8), (2, 0)):
        with pytest.raises(q.Qwen2Error) as e:
            q.qwen2_next_token_probs_static(lg, rows, V, pr)
        assert e.value.name == "E_ARG"
    assert "rows" in q.qwen2_last_error(None)
