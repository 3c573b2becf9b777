"""Shared helpers of the GPU parity tests (HIP path vs the CPU oracle)."""
import sys

import numpy as np
import torch

import qwen2_decoder_forward_amd as q
import qwen2_synth as syn
from oracle import qwen2_oracle as O

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def check(got, ref, tol, what):
    e = rel_err(got, ref)
    assert e <= tol, f"{what}: max-abs error / max|ref| = {e:.3e} > {tol}"
    return e


def top2_margin(logits) -> float:
    s = np.sort(np.asarray(logits, np.float32))
    return float(s[-1] - s[-2])


def check_id(gpu_id, ref_logits, ref_id, what):
    """Greedy ids must agree wherever the oracle's top-2 margin exceeds 1e-2."""
    if top2_margin(ref_logits) > 1e-2:
        assert int(gpu_id) == int(ref_id), f"{what}: id {int(gpu_id)} != oracle {int(ref_id)}"
        return True
    return False


def check_probs(got, logits, what):
    """next_token_probs against the oracle's softmax of the same logits:
    |p - ref| <= 1e-5 ref + 1e-38 element by element (f32 exponentials of
    arguments down to about -100), and each row sums to 1 within 1e-5."""
    ref = O.next_token_probs(logits).astype(np.float64)
    got = np.asarray(got, np.float64)
    bad = np.abs(got - ref) > 1e-5 * ref + 1e-38
    assert not bad.any(), f"{what}: {int(bad.sum())} probabilities off, e.g. {got[bad][:3]} vs {ref[bad][:3]}"
    assert np.all(np.abs(got.sum(-1) - 1) < 1e-5), f"{what}: rows sum to {got.sum(-1)}"


class Pair:
    """A GPU context and an oracle over the same weights."""

    def __init__(self, shape, weights, n_ctx, n_seq=1, cache_decoded=False, rope_style=0):
        self.shape = shape
        self.w = weights
        self.m = q.Model(shape, weights, n_ctx, n_seq, rope_style=rope_style)
        self.o = O.Qwen2Oracle(O.hparams_for(shape, n_ctx, n_seq, rope_style), weights,
                               cache_decoded)
        self.V, self.H = shape.n_vocab, shape.n_embd
        self.logits = torch.empty((max(n_seq, 1), self.V), dtype=torch.float32, device=DEV)
        self.ids = torch.zeros(max(n_seq, 1), dtype=torch.int32, device=DEV)
        self.hid = torch.empty((max(n_seq, 1), self.H), dtype=torch.float32, device=DEV)

    def hidden(self, which, rows):
        self.m.read_hidden(which, self.hid)
        torch.cuda.synchronize()
        return self.hid[:rows].cpu().numpy()

    def prefill(self, seq, toks, pos):
        self.m.prefill(seq, toks, pos, self.logits[0], self.ids[:1])
        r = self.o.prefill(seq, toks, pos)
        torch.cuda.synchronize()
        return self.logits[0].cpu().numpy(), int(self.ids[0].item()), r

    def prefill_batch(self, seqs, toks, poss):
        """One batched call on the GPU; the oracle runs each sequence's prefill
        on its own (a batch is defined as those independent prefills)."""
        B = len(seqs)
        self.m.prefill_batch(seqs, toks, poss, self.logits[:B], self.ids[:B])
        rs = [self.o.prefill(s, t, p) for s, t, p in zip(seqs, toks, poss)]
        torch.cuda.synchronize()
        return self.logits[:B].cpu().numpy(), self.ids[:B].cpu().numpy(), rs

    def decode(self, seqs, toks, pos):
        B = len(seqs)
        tdev = torch.tensor(np.asarray(toks, np.int32), device=DEV)
        self.m.decode(seqs, tdev, pos, self.logits[:B], self.ids[:B])
        r = self.o.decode(seqs, toks, pos)
        torch.cuda.synchronize()
        # the device-side bad-token flag must be clear
        assert self.m.sync_status() == 0
        return self.logits[:B].cpu().numpy(), self.ids[:B].cpu().numpy(), r

    def close(self):
        self.m.close()


def run_chain(pair, prompt, steps, tol, label, seq=0, pos0=0, hidden_tol=None):
    """Prefill then `steps` teacher-forced greedy decode steps, each checked."""
    hidden_tol = tol if hidden_tol is None else hidden_tol
    n = len(prompt)
    pos = np.arange(pos0, pos0 + n)
    say(f"[{label}] prefill n={n}")
    lg, gid, r = pair.prefill(seq, prompt, pos)
    errs = [check(lg, r.logits[0], tol, f"{label} prefill logits")]
    check(pair.hidden(0, 1), r.layer_output, hidden_tol, f"{label} prefill layer_output")
    check(pair.hidden(1, 1), r.final_norm_output, hidden_tol, f"{label} prefill final_norm_output")
    n_ids = int(check_id(gid, r.logits[0], r.argmax[0], f"{label} prefill"))
    tok = int(r.argmax[0])
    for s in range(steps):
        p = pos0 + n + s
        lg, gids, r = pair.decode([seq], [tok], [p])
        errs.append(check(lg[0], r.logits[0], tol, f"{label} decode step {s} logits"))
        if s % 8 == 0 or s == steps - 1:
            check(pair.hidden(0, 1), r.layer_output, hidden_tol, f"{label} step {s} layer_output")
        n_ids += int(check_id(gids[0], r.logits[0], r.argmax[0], f"{label} step {s}"))
        tok = int(r.argmax[0])
    say(f"[{label}] max rel err {max(errs):.3e}, ids checked {n_ids}/{steps + 1}")
    return errs
