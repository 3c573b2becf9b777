"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: max-abs error <= 1e-4 * max|ref| on the tiny (f32-activation) path,
<= 1e-2 * max|ref| for hidden states and logits elsewhere, greedy ids
bit-exact wherever the oracle's top-2 logit margin exceeds 1e-2 (teacher
forcing: both sides are fed the oracle's id).
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import qwen2_synth as syn  # noqa: E402
from gpu_common import DEV, Pair, check, check_id, check_probs, run_chain, say  # noqa: E402

pytestmark = pytest.mark.gpu

TINY = syn.MODELS["tiny"]
TOL_F32 = 1e-4
TOL = 1e-2


@pytest.fixture(scope="module")
def tiny_w():
    return syn.make_weights(TINY)


def test_tiny_prefill_and_greedy_decode(tiny_w):
    """The tiny configuration: prompt 8 (GEMV path), 8 greedy steps, n_ctx 64."""
    p = Pair(TINY, tiny_w, n_ctx=64)
    run_chain(p, syn.make_prompt(TINY, 8), 8, TOL_F32, "tiny")
    p.close()


def test_tiny_kv_cache_matches_oracle(tiny_w):
    p = Pair(TINY, tiny_w, n_ctx=64)
    toks = syn.make_prompt(TINY, 8)
    p.prefill(0, toks, np.arange(8))
    nkv, hd = TINY.n_head_kv, TINY.head_dim
    for l in range(TINY.n_layer):
        k = torch.empty((nkv, 8, hd), device=DEV)
        v = torch.empty((nkv, 8, hd), device=DEV)
        p.m.kv_read(l, 0, 0, 8, k, v)
        torch.cuda.synchronize()
        check(k.cpu().numpy(), p.o.k_cache[0][l][:, :8], TOL_F32, f"K layer {l}")
        check(v.cpu().numpy(), p.o.v_cache[0][l][:, :8], TOL_F32, f"V layer {l}")
    p.close()


@pytest.mark.parametrize("n", [9, 40, 100, 600, 1100, 2100])
def test_tiny_mfma_prefill_path(tiny_w, n):
    """Prompts longer than 8 rows take the MFMA GEMM + flash-attention path
    (f16 operands): ragged 32-row tiles, hd = 16; from 512 rows on the
    large-tile GEMM (128-row tiles, a ragged last band at 1100); at 2100 rows
    the attention splits its longest query tiles' key ranges over two blocks
    and merges their softmax states."""
    p = Pair(TINY, tiny_w, n_ctx=max(128, n + 8))
    run_chain(p, syn.make_prompt(TINY, n, 3), 3, TOL, f"tiny-mfma-{n}")
    p.close()


def test_tiny_positions_with_gaps_and_continuation(tiny_w):
    """Positions are data: a continuation prefill and gapped positions (unwritten
    slots read as zero on both sides)."""
    p = Pair(TINY, tiny_w, n_ctx=64)
    lg, _, r = p.prefill(0, [5, 6, 7], [0, 2, 5])
    check(lg, r.logits[0], TOL_F32, "gapped prefill")
    lg, _, r = p.prefill(0, [8, 9], [6, 7])
    check(lg, r.logits[0], TOL_F32, "continuation prefill")
    lg, _, r = p.decode([0], [10], [20])
    check(lg[0], r.logits[0], TOL_F32, "decode after a gap")
    p.close()


def test_mfma_prefill_rows_far_apart(tiny_w):
    """One prefill pass (MFMA path) whose rows 0..30 sit at positions 0..30
    and whose last row sits at position 4000: the attention's second key
    half (keys from 2048 on) is invisible to the first 31 rows, which must
    contribute zero weight there (not NaN)."""
    p = Pair(TINY, tiny_w, n_ctx=4200)
    pos = list(range(31)) + [4000]
    lg, _, r = p.prefill(0, syn.make_prompt(TINY, 32, 11), pos)
    assert np.all(np.isfinite(lg))
    check(lg, r.logits[0], TOL, "prefill with rows 0..30 and 4000")
    check(p.hidden(0, 1), r.layer_output, TOL, "layer_output")
    p.close()


def test_hard_error_at_n_ctx_leaves_cache_unchanged(tiny_w):
    import qwen2_decoder_forward_amd as q
    p = Pair(TINY, tiny_w, n_ctx=16)
    toks = syn.make_prompt(TINY, 6)
    p.prefill(0, toks, np.arange(6))
    nkv, hd = TINY.n_head_kv, TINY.head_dim

    def snapshot():
        out = []
        for l in range(TINY.n_layer):
            k = torch.empty((nkv, 16, hd), device=DEV)
            v = torch.empty((nkv, 16, hd), device=DEV)
            p.m.kv_read(l, 0, 0, 16, k, v)
            out += [k, v]
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in out]

    before = snapshot()
    for call, code in [
        (lambda: p.m.prefill(0, [1, 2], [6, 16]), "E_POS"),
        (lambda: p.m.prefill(0, [1], [-1]), "E_POS"),
        (lambda: p.m.prefill(0, [TINY.n_vocab], [6]), "E_TOKEN"),
        (lambda: p.m.prefill(0, [1, 2], [7, 7]), "E_ORDER"),
        (lambda: p.m.prefill(1, [1], [6]), "E_SEQ"),
        (lambda: p.m.decode([0], torch.zeros(1, dtype=torch.int32, device=DEV), [16]), "E_POS"),
    ]:
        with pytest.raises(q.Qwen2Error) as e:
            call()
        assert e.value.name == code
    after = snapshot()
    for a, b in zip(before, after):
        assert np.array_equal(a, b)
    # a valid call after the errors behaves as if they never happened
    lg, _, r = p.decode([0], [3], [6])
    check(lg[0], r.logits[0], TOL_F32, "decode after rejected calls")
    p.close()


def test_device_token_out_of_range_is_latched(tiny_w):
    import qwen2_decoder_forward_amd as q
    p = Pair(TINY, tiny_w, n_ctx=16)
    bad = torch.tensor([TINY.n_vocab + 3], dtype=torch.int32, device=DEV)
    p.m.decode([0], bad, [0], p.logits[:1], p.ids[:1])
    assert q.CODES[p.m.sync_status()] == "E_TOKEN"
    assert p.m.sync_status() == 0
    p.close()


@pytest.mark.parametrize("B", [3, 12])
def test_batched_decode(tiny_w, B):
    """Several sequences in one decode call: B <= 8 on the GEMV path, B > 8 on
    the MFMA path; prefixes of different lengths."""
    p = Pair(TINY, tiny_w, n_ctx=64, n_seq=16)
    # B <= 8: prefixes of at most 8 rows keep the whole chain on the f32 path
    lens = [2 + (5 * s) % 7 for s in range(B)] if B <= 8 else [3 + (7 * s) % 11 for s in range(B)]
    for s in range(B):
        p.prefill(s, syn.make_prompt(TINY, lens[s], 10 + s), np.arange(lens[s]))
    seqs = list(range(B))[::-1]
    toks = [int(t) for t in syn.make_prompt(TINY, B, 99)]
    pos = [lens[s] for s in seqs]
    lg, ids, r = p.decode(seqs, toks, pos)
    tol = TOL_F32 if B <= 8 else TOL
    for b in range(B):
        check(lg[b], r.logits[b], tol, f"batched B={B} row {b}")
        check_id(ids[b], r.logits[b], r.argmax[b], f"batched row {b}")
    h = p.hidden(0, B)
    check(h, r.layer_output, tol, "batched layer_output")
    p.close()


def test_multi_pass_prefill(tiny_w):
    """A prompt longer than the 4096-row pass is processed in passes."""
    p = Pair(TINY, tiny_w, n_ctx=8192)
    toks = syn.make_prompt(TINY, 4100, 5)
    lg, gid, r = p.prefill(0, toks, np.arange(4100))
    check(lg, r.logits[0], TOL, "multi-pass prefill logits")
    check_id(gid, r.logits[0], r.argmax[0], "multi-pass prefill")
    p.close()


@pytest.mark.parametrize("case", ["continuation", "gapped"])
def test_split_prefill_dispatch_orders(tiny_w, case):
    """A 2048-row pass splits its longest query tiles (64 tiles x 2 KV heads:
    128 blocks before the split) and dispatches its work longest first.
    continuation: the rows follow a 100-row prefill (positions 100..2147), so
    the closed-form item order starts at position 100; gapped: positions
    0..1023 and 1124..2147, not contiguous, so the pieces-first order serves
    (the gap's slots are unwritten and read as zero on both sides)."""
    p = Pair(TINY, tiny_w, n_ctx=4096)
    if case == "continuation":
        p.prefill(0, syn.make_prompt(TINY, 100, 8), np.arange(100))
        pos = np.arange(100, 2148)
    else:
        pos = np.concatenate([np.arange(1024), np.arange(1124, 2148)])
    lg, gid, r = p.prefill(0, syn.make_prompt(TINY, 2048, 9), pos)
    check(lg, r.logits[0], TOL, f"split prefill ({case}) logits")
    check_id(gid, r.logits[0], r.argmax[0], f"split prefill ({case})")
    h = p.hidden(0, 1)
    check(h[0], r.layer_output[-1], TOL, f"split prefill ({case}) last hidden row")
    p.close()


def _check_batch(p, seqs, toks, poss, tol, what):
    lg, ids, rs = p.prefill_batch(seqs, toks, poss)
    h = p.hidden(0, len(seqs))
    for b, r in enumerate(rs):
        check(lg[b], r.logits[0], tol, f"{what}: logits of sequence {seqs[b]}")
        check_id(ids[b], r.logits[0], r.argmax[0], f"{what}: id of sequence {seqs[b]}")
        check(h[b], r.layer_output[0], tol, f"{what}: layer_output of sequence {seqs[b]}")


def test_prefill_batch_gemv_rows(tiny_w):
    """A batched prefill of 6 rows in all (the f32 GEMV path and a 3-row
    read-out): a continuation after an earlier prefill, gapped positions and
    a one-row sequence, in an order unlike the slot order."""
    p = Pair(TINY, tiny_w, n_ctx=64, n_seq=4)
    p.prefill(2, syn.make_prompt(TINY, 5, 21), np.arange(5))
    seqs = [2, 0, 3]
    toks = [syn.make_prompt(TINY, 2, 22), syn.make_prompt(TINY, 3, 23), [7]]
    poss = [[5, 6], [0, 3, 9], [0]]
    _check_batch(p, seqs, toks, poss, TOL_F32, "batch-gemv")
    # the cache now continues with a decode of every sequence
    lg, ids, r = p.decode(seqs, [1, 2, 3], [7, 10, 1])
    for b in range(3):
        check(lg[b], r.logits[b], TOL_F32, f"decode after the batch, row {b}")
    p.close()


@pytest.mark.parametrize("lens", [[1, 40, 2, 33, 9, 1, 64, 5, 17, 3, 8, 31],
                                  [300, 1, 700, 45]])
def test_prefill_batch_mfma_rows(tiny_w, lens):
    """Batched prefills on the MFMA path: one-row, ragged and multi-tile
    sequences sharing each GEMM; 12 read-out rows take the MFMA read-out,
    4 the GEMV one; some sequences continue an earlier prefill."""
    B = len(lens)
    p = Pair(TINY, tiny_w, n_ctx=1024, n_seq=16)
    start = [0] * B
    for b in range(0, B, 3):
        start[b] = 11 + b
        p.prefill(b, syn.make_prompt(TINY, start[b], 40 + b), np.arange(start[b]))
    seqs = list(range(B))[::-1]
    toks = [syn.make_prompt(TINY, lens[s], 60 + s) for s in seqs]
    poss = [np.arange(start[s], start[s] + lens[s]) for s in seqs]
    _check_batch(p, seqs, toks, poss, TOL, f"batch-mfma-{B}")
    p.close()


def test_prefill_batch_straddles_passes(tiny_w):
    """9,030 rows in all: the 8,192-row first pass of a multi-sequence
    context ends inside the second sequence, whose rows continue in the next
    pass."""
    p = Pair(TINY, tiny_w, n_ctx=8192, n_seq=3)
    lens = [6000, 3000, 30]
    seqs = [1, 0, 2]
    toks = [syn.make_prompt(TINY, n, 80 + i) for i, n in enumerate(lens)]
    poss = [np.arange(n) for n in lens]
    _check_batch(p, seqs, toks, poss, TOL, "batch-passes")
    p.close()


def test_prefill_batch_rejects_before_any_work(tiny_w):
    """A repeated slot or a bad position anywhere in the batch fails the whole
    call before anything is enqueued: the cache keeps its contents."""
    import qwen2_decoder_forward_amd as q
    p = Pair(TINY, tiny_w, n_ctx=64, n_seq=3)
    p.prefill(0, [1, 2, 3], [0, 1, 2])
    nkv, hd = TINY.n_head_kv, TINY.head_dim
    k0 = torch.empty((nkv, 64, hd), device=DEV)
    v0 = torch.empty((nkv, 64, hd), device=DEV)
    p.m.kv_read(0, 0, 0, 64, k0, v0)
    for seqs, toks, poss, code in [([0, 0], [[4], [5]], [[3], [4]], "E_SEQ"),
                                   ([0, 1], [[4], [5, 6]], [[3], [0, 64]], "E_POS")]:
        with pytest.raises(q.Qwen2Error) as ei:
            p.m.prefill_batch(seqs, toks, poss, p.logits[:2], p.ids[:2])
        assert ei.value.name == code
    k1 = torch.empty_like(k0)
    v1 = torch.empty_like(v0)
    p.m.kv_read(0, 0, 0, 64, k1, v1)
    torch.cuda.synchronize()
    assert torch.equal(k0, k1) and torch.equal(v0, v1)
    p.close()


def test_interleaved_rope_model(tiny_w):
    """rope_style 1 (Interleaved, a model-level flag): prompt 8 and greedy
    steps on the f32 path, a 40-row MFMA prefill, and the K cache read back
    in natural dimension order, all against the oracle run with the same
    flag (whose interleaved rotation differs from the default one)."""
    p = Pair(TINY, tiny_w, n_ctx=64, rope_style=1)
    run_chain(p, syn.make_prompt(TINY, 8, 4), 4, TOL_F32, "interleaved")
    nkv, hd = TINY.n_head_kv, TINY.head_dim
    for l in range(TINY.n_layer):
        k = torch.empty((nkv, 12, hd), device=DEV)
        v = torch.empty((nkv, 12, hd), device=DEV)
        p.m.kv_read(l, 0, 0, 12, k, v)
        torch.cuda.synchronize()
        check(k.cpu().numpy(), p.o.k_cache[0][l][:, :12], TOL_F32, f"interleaved K layer {l}")
        check(v.cpu().numpy(), p.o.v_cache[0][l][:, :12], TOL_F32, f"interleaved V layer {l}")
        # a write of what was read leaves the cache (and the next step) unchanged
        p.m.kv_write(l, 0, 0, 12, k, v)
    lg, _, r = p.decode([0], [3], [12])
    check(lg[0], r.logits[0], TOL_F32, "interleaved decode after a K round trip")
    p.close()
    p = Pair(TINY, tiny_w, n_ctx=128, rope_style=1)
    lg, gid, r = p.prefill(0, syn.make_prompt(TINY, 40, 6), np.arange(40))
    check(lg, r.logits[0], TOL, "interleaved 40-row prefill")
    p.close()


def test_next_token_probs(tiny_w):
    """Softmax of the read-out logits: one row after a prefill, 12 after a
    batched decode, and rows of wide-range logits written directly (large
    negative gaps, ties)."""
    p = Pair(TINY, tiny_w, n_ctx=64, n_seq=12)
    V = TINY.n_vocab
    probs = torch.empty((12, V), dtype=torch.float32, device=DEV)
    lg, _, r = p.prefill(0, syn.make_prompt(TINY, 6, 3), np.arange(6))
    p.m.next_token_probs(p.logits, 1, probs)
    torch.cuda.synchronize()
    check_probs(probs[:1].cpu().numpy(), lg[None], "after a prefill")
    seqs = list(range(12))
    for s_ in seqs[1:]:
        p.prefill(s_, syn.make_prompt(TINY, 3, 30 + s_), np.arange(3))
    lg, _, r = p.decode(seqs, list(range(12)), [6] + [3] * 11)
    p.m.next_token_probs(p.logits, 12, probs)
    torch.cuda.synchronize()
    check_probs(probs.cpu().numpy(), lg, "after a 12-row decode")
    x = torch.randn((5, V), generator=torch.Generator().manual_seed(9)) * 40
    x[1] = 0.0
    x[2, ::3] = -200.0
    x[3, 7] = 500.0
    p.logits[:5].copy_(x.to(DEV))
    p.m.next_token_probs(p.logits, 5, probs)
    torch.cuda.synchronize()
    check_probs(probs[:5].cpu().numpy(), x.numpy(), "direct logits")
    import qwen2_decoder_forward_amd as q
    for rows in (0, 13):  # rows must be in [1, max(n_seq, 8)] = [1, 12]
        with pytest.raises(q.Qwen2Error) as e:
            p.m.next_token_probs(p.logits, rows, probs)
        assert e.value.name == "E_ARG"
    p.close()


def test_stop_ids_latch_earliest_position(tiny_w):
    """Stop ids are data: every greedy read-out (decode on both paths, prefill,
    batched prefill) whose id is a stop id marks its slot; the earliest
    read-out position is kept, compared exactly with the oracle's definition
    applied to the ids this run produced."""
    import qwen2_decoder_forward_amd as q
    from oracle import qwen2_oracle as O
    p = Pair(TINY, tiny_w, n_ctx=64, n_seq=12)
    m = p.m
    stops_out = torch.empty(12, dtype=torch.int32, device=DEV)
    # a first greedy chain without stop ids, to pick ids that will recur
    ids = torch.zeros(13, dtype=torch.int32, device=DEV)
    m.prefill(0, syn.make_prompt(TINY, 5, 8), np.arange(5), None, ids[0:1])
    for k in range(12):
        m.decode([0], ids[k:k + 1], [5 + k], None, ids[k + 1:k + 2])
    first = ids.cpu().numpy()
    stop = [int(first[4]), int(first[9]), TINY.n_vocab - 1]
    m.set_stop_ids(stop)
    m.read_stops(stops_out, clear=True)
    reads = []
    # slot 1: the same prompt, a greedy chain on the GEMV path
    ids.zero_()
    m.prefill(1, syn.make_prompt(TINY, 5, 8), np.arange(5), None, ids[0:1])
    for k in range(12):
        m.decode([1], ids[k:k + 1], [5 + k], None, ids[k + 1:k + 2])
    got = ids.cpu().numpy()
    reads += [(1, 4 + k, int(got[k])) for k in range(13)]
    # a batched prefill of 10 slots (MFMA read-out), then a 10-row decode step
    slots = list(range(2, 12))
    toks = [syn.make_prompt(TINY, 2 + j % 3, 50 + j) for j in range(10)]
    poss = [np.arange(len(t)) for t in toks]
    bids = torch.zeros(10, dtype=torch.int32, device=DEV)
    m.prefill_batch(slots, toks, poss, None, bids)
    b0 = bids.cpu().numpy()
    reads += [(s_, len(t) - 1, int(b0[j])) for j, (s_, t) in enumerate(zip(slots, toks))]
    m.decode(slots, bids, [len(t) for t in toks], None, bids)
    b1 = bids.cpu().numpy()
    reads += [(s_, len(t), int(b1[j])) for j, (s_, t) in enumerate(zip(slots, toks))]
    m.read_stops(stops_out)
    torch.cuda.synchronize()
    want = O.stop_positions(12, reads, stop)
    assert list(stops_out.cpu().numpy()) == list(want), (list(stops_out.cpu().numpy()), list(want))
    assert (want >= 0).any()  # the chain repeats its first run, so a stop id recurs
    m.read_stops(stops_out, clear=True)
    m.read_stops(stops_out)
    torch.cuda.synchronize()
    assert (stops_out.cpu().numpy() == -1).all()
    with pytest.raises(q.Qwen2Error):
        m.set_stop_ids([TINY.n_vocab])
    with pytest.raises(q.Qwen2Error):
        m.set_stop_ids(list(range(9)))
    # no stop ids: nothing latches
    m.set_stop_ids([])
    ids.zero_()
    for k in range(4):
        m.decode([1], ids[k:k + 1], [20 + k], None, ids[k + 1:k + 2])
    m.read_stops(stops_out)
    torch.cuda.synchronize()
    assert (stops_out.cpu().numpy() == -1).all()
    p.close()


HD128 = dataclasses.replace(syn.MODELS["qwen2-hd128"], name="hd128-narrow", n_layer=2,
                            n_embd=896, n_head=7, n_head_kv=1, n_ff=640, n_vocab=4096)


@pytest.mark.parametrize("n", [5, 70])
def test_hd128_untied_group7(n):
    """head_dim 128, group 7, untied lm_head (the large shape's kernels) at a
    narrow width."""
    w = syn.make_weights(HD128)
    p = Pair(HD128, w, n_ctx=256)
    run_chain(p, syn.make_prompt(HD128, n), 4, TOL if n > 8 else TOL_F32 * 10, f"hd128-{n}")
    p.close()


# Head layouts of the family at their real widths (two layers, a small FFN
# and vocabulary): 12/2 and 16/2 heads of 128 (groups 6 and 8), 40/8 (group
# 5, the widest hidden size whose normed row the decode GEMVs keep in
# registers), 64/8 (hidden 8192: the decode GEMVs norm the row in a
# separate kernel first), multi-head attention (n_head_kv = n_head, Qwen1.5)
# and the two other RoPE bases.
FAMILY = {
    "heads12-2": dict(n_embd=1536, n_head=12, n_head_kv=2, head_dim=128),
    "heads16-2": dict(n_embd=2048, n_head=16, n_head_kv=2, head_dim=128),
    "heads40-8": dict(n_embd=5120, n_head=40, n_head_kv=8, head_dim=128),
    "heads64-8": dict(n_embd=8192, n_head=64, n_head_kv=8, head_dim=128),
    "mha8-theta1e4": dict(n_embd=512, n_head=8, n_head_kv=8, head_dim=64, rope_theta=1e4),
    "theta1e7": dict(n_embd=896, n_head=14, n_head_kv=2, head_dim=64, rope_theta=1e7),
}


@pytest.mark.parametrize("name", list(FAMILY))
def test_family_head_shapes(name):
    """Prompt 5 (f32 path) with greedy steps, then a 40-row prompt (MFMA
    path), against the oracle."""
    shape = dataclasses.replace(syn.MODELS["qwen2-hd128"], name=name, n_layer=2, n_ff=512,
                                n_vocab=2048, **FAMILY[name])
    w = syn.make_weights(shape)
    p = Pair(shape, w, n_ctx=128)
    run_chain(p, syn.make_prompt(shape, 5), 3, TOL_F32 * 10, f"{name}-5")
    p.close()
    p = Pair(shape, w, n_ctx=128)
    lg, gid, r = p.prefill(0, syn.make_prompt(shape, 40, 2), np.arange(40))
    check(lg, r.logits[0], TOL, f"{name} 40-row prefill")
    check_id(gid, r.logits[0], r.argmax[0], f"{name} 40-row prefill")
    p.close()


def test_graph_replay_matches_direct_launches(tiny_w, monkeypatch):
    """Decode steps replayed from captured graphs (different pointers and
    positions on every replay, eager prefills and host syncs in between) give
    the same ids and logits as the same kernels launched directly (up to the
    float-atomic summation order of the fused attention + WO: 1e-6)."""
    import qwen2_decoder_forward_amd as q
    toks = syn.make_prompt(TINY, 8)

    def chain():
        m = q.Model(TINY, tiny_w, n_ctx=64)
        lg = torch.empty((6, TINY.n_vocab), device=DEV)
        ids = torch.zeros(7, dtype=torch.int32, device=DEV)
        m.prefill(0, toks, np.arange(8), lg[0], ids[0:1])
        for s in range(5):
            m.decode([0], ids[s:s + 1], [8 + s], lg[s + 1], ids[s + 1:s + 2])
            torch.cuda.synchronize()
        assert m.sync_status() == 0
        out = lg.cpu().numpy(), ids.cpu().numpy()
        m.close()
        return out

    lg_graph, ids_graph = chain()
    monkeypatch.setenv("QWEN2_NO_GRAPH", "1")
    lg_direct, ids_direct = chain()
    assert np.array_equal(ids_graph, ids_direct)
    check(lg_graph, lg_direct, 1e-6, "graph vs direct logits")


def test_attention_reference_moves_mid_row(tiny_w):
    """Keys planted in the cache (qwen2_kv_write on the GPU, directly on the
    oracle side) at positions 0..127, those of the second 64-key tile 20
    times larger than the first's: their scores exceed the first tile's
    maximum by far more than the 2^10 (base-2) margin within which the
    prefill attention keeps its per-row reference maximum, so the reference
    moves in the middle of each row and the output accumulated so far is
    rescaled.  A 40-row continuation prefill at positions 128..167 (MFMA
    attention), then one 12-row decode step over 12 sequences with the same
    planted keys (chunked decode attention, its chunk records merged), each
    against the oracle."""
    n_seq = 12
    p = Pair(TINY, tiny_w, n_ctx=256, n_seq=n_seq)
    nkv, hd, L = TINY.n_head_kv, TINY.head_dim, TINY.n_layer
    rng = np.random.default_rng(11)
    k = rng.standard_normal((nkv, 128, hd)).astype(np.float32)
    k[:, 64:] *= 20.0
    v = rng.standard_normal((nkv, 128, hd)).astype(np.float32)
    kd, vd = torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV)
    for s_ in range(n_seq):
        Kc, Vc = p.o._cache(s_)
        for l in range(L):
            p.m.kv_write(l, s_, 0, 128, kd, vd)
            Kc[l][:, :128] = k
            Vc[l][:, :128] = v
    torch.cuda.synchronize()
    lg, gid, r = p.prefill(0, syn.make_prompt(TINY, 40, 12), np.arange(128, 168))
    check(lg, r.logits[0], TOL, "40-row prefill over planted keys")
    check(p.hidden(0, 1), r.layer_output, TOL, "40-row prefill layer_output")
    check_id(gid, r.logits[0], r.argmax[0], "40-row prefill over planted keys")
    for s_ in range(1, n_seq):
        p.prefill(s_, syn.make_prompt(TINY, 3, 60 + s_), np.arange(128, 131))
    seqs = list(range(n_seq))
    toks = [int(t) for t in syn.make_prompt(TINY, n_seq, 13)]
    lg, ids, r = p.decode(seqs, toks, [168] + [131] * (n_seq - 1))
    for b in range(n_seq):
        check(lg[b], r.logits[b], TOL, f"12-row decode over planted keys, row {b}")
        check_id(ids[b], r.logits[b], r.argmax[b], f"12-row decode over planted keys, row {b}")
    p.close()


def test_one_row_decode_across_slots_and_graph_eviction(tiny_w):
    """One-row decode steps address their slot's K/V from the host, and each
    (slot, chunk count) gets its own captured step: 40 slots decoded one row
    at a time, in an interleaved order, twice over (more distinct steps than
    the 32 graphs a context keeps, so evicted graphs are captured again), each
    step against the oracle.  Before the prompts, every slot's cache is
    filled with large values at positions 0..63 (through qwen2_kv_write on
    the GPU and directly on the oracle side): slots past a row's position
    hold data the attention must mask out, not zeros."""
    n_slots = 40
    p = Pair(TINY, tiny_w, n_ctx=64, n_seq=n_slots)
    nkv, hd, L = TINY.n_head_kv, TINY.head_dim, TINY.n_layer
    rng = np.random.default_rng(5)
    junk_k = (rng.standard_normal((nkv, 64, hd)) * 50).astype(np.float32)
    junk_v = (rng.standard_normal((nkv, 64, hd)) * 50).astype(np.float32)
    kd, vd = torch.from_numpy(junk_k).to(DEV), torch.from_numpy(junk_v).to(DEV)
    for s in range(n_slots):
        Kc, Vc = p.o._cache(s)
        for l in range(L):
            p.m.kv_write(l, s, 0, 64, kd, vd)
            Kc[l][:, :64] = junk_k
            Vc[l][:, :64] = junk_v
    torch.cuda.synchronize()
    lens = [1 + (3 * s) % 6 for s in range(n_slots)]
    for s in range(n_slots):
        p.prefill(s, syn.make_prompt(TINY, lens[s], 500 + s), np.arange(lens[s]))
    order = [(7 * i) % n_slots for i in range(n_slots)]
    step = 0
    for rnd in range(2):
        for s in order:
            pos = lens[s] + rnd
            lg, ids, r = p.decode([s], [int(syn.make_prompt(TINY, 1, 900 + step)[0])], [pos])
            check(lg[0], r.logits[0], TOL_F32, f"slot {s} round {rnd}")
            check_id(ids[0], r.logits[0], r.argmax[0], f"slot {s} round {rnd}")
            step += 1
    p.close()
