"""GPU read-out edge cases: ties and NaN in the greedy argmax.

The reading of the pages used here (they are silent on it): the greedy id is
the lowest index of the largest logit, and a NaN logit never wins.  The
lm_head rows are crafted so that these cases happen by construction, on each
of the three read-out kernels: the persistent one-row kernel (a prefill
read-out), the 2..8-row GEMV (a decode batch of 5) and the MFMA lm_head of
more than 8 rows (a decode batch of 12).

Crafted untied lm_head (tiny model width, the full 151,936-entry vocabulary
so that ties fall in different blocks and the persistent kernel loops):
  * rows 0 and 5: binary16 NaN, so logits 0 and 5 are NaN;
  * rows 7 and 150,001: one identical vector r, so logits 7 and 150,001 are
    equal (the same sums in the same order on both sides);
  * every other row zero, so every other logit is exactly 0.
r is 0.25 * sign(y) for the final-norm output y of the first read-out row
of each call, so that row's largest logit is the 7 / 150,001 tie (answer 7);
a row with y . r < 0 has its largest logit 0 shared by every zero row, and
its answer is 1 (the lowest index that is not NaN).
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import qwen2_synth as syn  # noqa: E402
from gpu_common import DEV, Pair, say  # noqa: E402
from oracle import qwen2_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu

SHAPE = dataclasses.replace(syn.MODELS["tiny"], name="tiny-untied-V151936", n_vocab=151936,
                            tied=False)
NAN_ROWS = (0, 5)
TIE_ROWS = (7, 150001)
F16_NAN = 0x7E00


def crafted(w, y0):
    lm = np.zeros((SHAPE.n_vocab, SHAPE.n_embd), np.uint16)
    lm[list(NAN_ROWS)] = F16_NAN
    r = (0.25 * np.where(np.asarray(y0) >= 0, 1.0, -1.0)).astype(np.float16).view(np.uint16)
    lm[list(TIE_ROWS)] = r
    out = dict(w)
    out["lm_head"] = lm
    return out


def run_calls(pair, B):
    """Prefill every slot with a short prompt, then (B > 1) one decode step of
    B rows.  Returns (GPU logits, GPU ids, oracle result) of the last call."""
    for s in range(B):
        toks = syn.make_prompt(SHAPE, 6 + s, 70 + s)
        lg, gid, r = pair.prefill(s, toks, np.arange(len(toks)))
    if B == 1:
        return lg[None], np.array([gid]), r
    seqs = list(range(B))
    toks = [int(t) for t in syn.make_prompt(SHAPE, B, 99)]
    pos = [6 + s for s in range(B)]
    return pair.decode(seqs, toks, pos)


def first_row_y(w, B):
    """Final-norm output of the first read-out row of the last call (the
    lm_head does not change it)."""
    o = O.Qwen2Oracle(O.hparams_for(SHAPE, 64, max(B, 1)), w)
    r = None
    for s in range(B):
        toks = syn.make_prompt(SHAPE, 6 + s, 70 + s)
        r = o.prefill(s, toks, np.arange(len(toks)))
    if B > 1:
        r = o.decode(list(range(B)), [int(t) for t in syn.make_prompt(SHAPE, B, 99)],
                     [6 + s for s in range(B)])
    return r.final_norm_output[0]


@pytest.fixture(scope="module")
def base_w():
    return syn.make_weights(SHAPE)


@pytest.mark.parametrize("B,kernel", [(1, "k_lmhead"), (5, "GEMV lm_head"),
                                      (12, "MFMA lm_head")])
def test_argmax_ties_lowest_index_and_nan_never_wins(base_w, B, kernel):
    w = crafted(base_w, first_row_y(base_w, B))
    say(f"[readout-edges] {kernel}: {B} read-out row(s)")
    p = Pair(SHAPE, w, n_ctx=64, n_seq=max(B, 1))
    lg, ids, r = run_calls(p, B)
    tol = 1e-4 if B <= 8 else 1e-2  # f32 GEMV rows; f16 MFMA operands above 8 rows
    answers = []
    for b in range(B):
        ref = r.logits[b]
        got = lg[b]
        nan = np.isnan(ref)
        assert np.array_equal(np.flatnonzero(nan), list(NAN_ROWS)), "oracle NaN rows"
        assert np.array_equal(np.isnan(got), nan), f"{kernel} row {b}: NaN logits differ"
        # the crafted tie is exact on both sides
        assert got[TIE_ROWS[0]] == got[TIE_ROWS[1]], f"{kernel} row {b}: tie rows differ"
        # The only non-zero logits are y . r, a sum of terms of both signs
        # that may nearly cancel; its rounding error scales with the sum of
        # the terms' magnitudes 0.25 * sum|y|, which is the scale used here.
        ok = ~nan
        scale = max(np.max(np.abs(ref[ok])), 0.25 * float(np.sum(np.abs(r.final_norm_output[b]))))
        err = np.max(np.abs(got[ok] - ref[ok])) / scale
        assert err <= tol, f"{kernel} row {b}: logits error {err:.3e}"
        expect = int(r.argmax[b])
        assert expect in (TIE_ROWS[0], 1), expect
        assert int(ids[b]) == expect, f"{kernel} row {b}: id {int(ids[b])} != {expect}"
        answers.append(expect)
    assert answers[0] == TIE_ROWS[0], "the first row's largest logit is the crafted tie"
    say(f"[readout-edges] {kernel}: ids {answers}")
    p.close()


def test_all_nan_logits_give_id_zero(base_w):
    """Every lm_head row NaN: all logits rank equally (below every number),
    so the lowest index wins and the id is 0 (the oracle's reading for an
    all-NaN row)."""
    w = dict(base_w)
    w["lm_head"] = np.full((SHAPE.n_vocab, SHAPE.n_embd), F16_NAN, np.uint16)
    p = Pair(SHAPE, w, n_ctx=64, n_seq=12)
    for B in (1, 5, 12):
        lg, ids, r = run_calls(p, B)
        assert np.all(np.isnan(lg[:B]))
        assert list(r.argmax[:B]) == [0] * B
        assert [int(i) for i in ids[:B]] == [0] * B, f"{B} rows: ids {ids[:B]}"
        p.o.reset()  # (the next prefills rewrite the same GPU slots)
    p.close()
