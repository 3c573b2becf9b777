"""GPU parity on the full-size workloads (besides the benchmark's own):

* 0.5B shape, 4096-token prompt (n_ctx 8192), then decode steps past 4096
  (chunked attention with the merge kernel);
* 0.5B shape, 64 sequences with 1024-token prefixes, one batched decode step
  at position 1024 (MFMA path): the oracle prefills sequences 0 and 63 itself
  and, for the others, decodes from the GPU's KV cache read back;
* the hd-128 / group-7 / untied shape at full width (2 layers) with a
  2048-token prompt against the oracle, and the full 28-layer model checked
  for properties that hold at any size (prefill of n+1 tokens = prefill of n
  then one decode step; argmax = lowest index of the largest logit);
* the 1.5B head layout (12/2 heads of 128) at full width (2 layers) with the
  512-token workload prompt against the oracle;
* the hd-128 model at its full depth of 28 layers against the oracle: a
  128-row prompt on the MFMA path, teacher-forced steps, and a step at a
  gapped position past 512 (chunked attention and the merge + WO kernel at
  head_dim 128);
* batched prefill at full width: the 0.5B shape with nine sequences whose
  first 8,192-row pass holds eight of them (one attention launch of 512
  blocks, no causal split), one sequence straddling two passes and one
  continuing an earlier prefill; and an hd-128 batch large enough for the
  large-tile GEMMs.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import qwen2_synth as syn  # noqa: E402
from gpu_common import DEV, Pair, check, check_id, run_chain, say  # noqa: E402

pytestmark = pytest.mark.gpu

S = syn.MODELS["qwen2.5-0.5b"]
TOL = 1e-2


@pytest.fixture(scope="module")
def w05():
    say("[workloads] drawing 0.5B weights")
    return syn.make_weights(S)


@pytest.fixture(scope="module")
def hd128_w():
    say("[workloads] drawing the 28-layer hd-128 weights")
    return syn.make_weights(syn.MODELS["qwen2-hd128"])


def test_long_context_prompt_4096_then_decode(w05):
    p = Pair(S, w05, n_ctx=8192, cache_decoded=True)
    run_chain(p, syn.make_prompt(S, 4096, 7), 4, TOL, "0.5b-long")
    p.close()


def test_batched_decode_64_sequences_at_1024(w05):
    B, n = 64, 1024
    p = Pair(S, w05, n_ctx=2048, n_seq=B, cache_decoded=True)
    prompts = [syn.make_prompt(S, n, 100 + j) for j in range(B)]
    say("[batched] GPU prefill of 64 x 1024")
    for j in range(B):
        p.m.prefill(j, prompts[j], np.arange(n), None, None)
    torch.cuda.synchronize()
    L, nkv, hd = S.n_layer, S.n_head_kv, S.head_dim
    k = torch.empty((nkv, n, hd), device=DEV)
    v = torch.empty((nkv, n, hd), device=DEV)
    for j in (0, B - 1):
        say(f"[batched] oracle prefill of sequence {j}")
        p.o.prefill(j, prompts[j], np.arange(n))
        for l in range(L):
            p.m.kv_read(l, j, 0, n, k, v)
            torch.cuda.synchronize()
            check(k.cpu().numpy(), p.o.k_cache[j][l][:, :n], TOL, f"seq {j} layer {l} K")
            check(v.cpu().numpy(), p.o.v_cache[j][l][:, :n], TOL, f"seq {j} layer {l} V")
    say("[batched] handing the GPU cache of sequences 1..62 to the oracle")
    for j in range(1, B - 1):
        Kc, Vc = p.o._cache(j)
        for l in range(L):
            p.m.kv_read(l, j, 0, n, k, v)
            torch.cuda.synchronize()
            Kc[l][:, :n] = k.cpu().numpy()
            Vc[l][:, :n] = v.cpu().numpy()
    seqs = list(range(B))
    toks = [int(t) for t in syn.make_prompt(S, B, 999)]
    say("[batched] decode step of 64 rows")
    lg, ids, r = p.decode(seqs, toks, [n] * B)
    n_ids = 0
    for b in range(B):
        check(lg[b], r.logits[b], TOL, f"batched row {b} logits")
        n_ids += int(check_id(ids[b], r.logits[b], r.argmax[b], f"batched row {b}"))
    check(p.hidden(0, B), r.layer_output, TOL, "batched layer_output")
    check(p.hidden(1, B), r.final_norm_output, TOL, "batched final_norm_output")
    say(f"[batched] ids checked {n_ids}/{B}")
    p.close()


@pytest.mark.parametrize("n", [2048, 2100])
def test_hd128_full_width_two_layers_prompt(n):
    """The 2048-token workload prompt, and 2100 rows: a ragged last row tile
    (52 of 256 rows) in the 256 x 256 GEMM tiles of WO / down (two K splits)
    and gate/up."""
    G2 = syn.model_shape("qwen2-hd128", n_layer=2)
    say(f"[hd128-L2-{n}] drawing weights")
    w = syn.make_weights(G2)
    p = Pair(G2, w, n_ctx=4096)
    run_chain(p, syn.make_prompt(G2, n), 2, TOL, f"hd128-L2-{n}")
    p.close()


@pytest.mark.parametrize("n", [512, 530])
def test_1_5b_layout_full_width_two_layers_prompt(n):
    """The 1.5B head layout (12/2 heads of 128, hidden 1536, FFN 8960, the
    151,936-entry tied vocabulary) at two layers: the 512-token workload
    prompt on the large-tile GEMMs and 530 rows (a ragged last row tile),
    then greedy steps on the 4-chunk decode GEMVs."""
    S15 = syn.model_shape("qwen2.5-1.5b-heads", n_layer=2)
    say(f"[1.5b-L2-{n}] drawing weights")
    w = syn.make_weights(S15)
    p = Pair(S15, w, n_ctx=1024)
    run_chain(p, syn.make_prompt(S15, n), 2, TOL, f"1.5b-L2-{n}")
    p.close()


@pytest.mark.timeout(600)
def test_hd128_full_model_properties(hd128_w):
    """28 layers, hidden 3584, at the workload's 2048-token prompt: properties
    that hold at any size, checked on the GPU path itself (an extra beside
    the oracle comparison of the full-depth model below)."""
    import qwen2_decoder_forward_amd as q
    G = syn.MODELS["qwen2-hd128"]
    w = hd128_w
    m = q.Model(G, w, n_ctx=4096)
    info = m.info()
    assert info.weight_bytes_f16 == syn.weight_bytes(G)["f16"]
    prompt = syn.make_prompt(G, 2048)
    V = G.n_vocab
    lg_a = torch.empty(V, device=DEV)
    id_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("[hd128] prefill 2048")
    m.prefill(0, prompt, np.arange(2048), lg_a, id_a)
    lg_b = torch.empty(V, device=DEV)
    id_b = torch.zeros(1, dtype=torch.int32, device=DEV)
    m2 = q.Model(G, w, n_ctx=4096)
    say("[hd128] prefill 2047 + decode 1")
    m2.prefill(0, prompt[:2047], np.arange(2047), None, None)
    m2.decode([0], torch.tensor(prompt[2047:], dtype=torch.int32, device=DEV), [2047], lg_b, id_b)
    torch.cuda.synchronize()
    a, b = lg_a.cpu().numpy(), lg_b.cpu().numpy()
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    check(b, a, TOL, "hd128: prefill(n) vs prefill(n-1) + decode")
    assert int(id_a.item()) == int(np.argmax(a))
    assert int(id_b.item()) == int(np.argmax(b))
    m.close()
    m2.close()


def _check_batch(p, seqs, toks, poss, what):
    lg, ids, rs = p.prefill_batch(seqs, toks, poss)
    hid = p.hidden(0, len(seqs))
    fin = p.hidden(1, len(seqs))
    n_ids = 0
    for b, r in enumerate(rs):
        check(lg[b], r.logits[0], TOL, f"{what}: logits of sequence {seqs[b]}")
        n_ids += int(check_id(ids[b], r.logits[0], r.argmax[0], f"{what}: id of sequence {seqs[b]}"))
        check(hid[b], r.layer_output[0], TOL, f"{what}: layer_output of sequence {seqs[b]}")
        check(fin[b], r.final_norm_output[0], TOL, f"{what}: final_norm_output of sequence {seqs[b]}")
    say(f"[{what}] ids checked {n_ids}/{len(seqs)}")


@pytest.mark.timeout(600)
def test_prefill_batch_0_5b_shape_full_pass(w05):
    """Two layers of the 0.5B shape (full width and vocabulary).  Nine
    sequences: the first 8,192-row pass holds sequences 0..7 (8 segments,
    256 query tiles x 2 KV heads = 512 attention blocks: the unsplit branch of
    the multi-sequence launch); sequence 7 straddles into the second pass;
    sequence 0 continues an earlier 100-token prefill (its rows sit at
    positions 100..1123)."""
    S2 = syn.model_shape("qwen2.5-0.5b", n_layer=2)
    p = Pair(S2, w05, n_ctx=2048, n_seq=9, cache_decoded=True)
    say("[batch-0.5b] continuation base: 100 tokens on slot 0")
    p.prefill(0, syn.make_prompt(S2, 100, 200), np.arange(100))
    lens = [1024] * 7 + [1100, 500]
    seqs = [0, 3, 1, 2, 6, 4, 5, 7, 8]
    start = {0: 100}
    toks = [syn.make_prompt(S2, n, 210 + i) for i, n in enumerate(lens)]
    poss = [np.arange(start.get(s, 0), start.get(s, 0) + n) for s, n in zip(seqs, lens)]
    say("[batch-0.5b] batched prefill of 9 sequences, 9,824 rows")
    _check_batch(p, seqs, toks, poss, "batch-0.5b")
    # the cache then serves a decode step of every sequence
    last = [int(ps[-1]) for ps in poss]
    lg, ids, r = p.decode(seqs, list(range(1, 10)), [x + 1 for x in last])
    for b in range(9):
        check(lg[b], r.logits[b], TOL, f"decode after the batch, row {b}")
    p.close()


def test_prefill_batch_hd128_full_width():
    """Two hd-128 layers (group 7, untied): four sequences, 1,230 rows in one
    pass, enough for the large-tile GEMMs, one a continuation."""
    G2 = syn.model_shape("qwen2-hd128", n_layer=2)
    say("[batch-hd128] drawing weights")
    w = syn.make_weights(G2)
    p = Pair(G2, w, n_ctx=1024, n_seq=4, cache_decoded=True)
    p.prefill(2, syn.make_prompt(G2, 60, 300), np.arange(60))
    lens = [600, 257, 40, 333]
    seqs = [1, 2, 0, 3]
    start = {2: 60}
    toks = [syn.make_prompt(G2, n, 310 + i) for i, n in enumerate(lens)]
    poss = [np.arange(start.get(s, 0), start.get(s, 0) + n) for s, n in zip(seqs, lens)]
    say("[batch-hd128] batched prefill of 4 sequences, 1,230 rows")
    _check_batch(p, seqs, toks, poss, "batch-hd128")
    p.close()


@pytest.mark.timeout(900)
def test_hd128_full_depth_against_oracle(hd128_w):
    """The hd-128 workload model at its full 28 layers against the oracle:
    a 128-row prompt (MFMA path), three teacher-forced greedy steps (f32
    GEMV path, fused attention + WO), then one step at position 600 after a
    gap (chunked attention over 10 chunks and the merge + WO kernel at
    head_dim 128; the unwritten slots read as zero on both sides)."""
    G = syn.MODELS["qwen2-hd128"]
    p = Pair(G, hd128_w, n_ctx=4096, cache_decoded=True)
    say("[hd128-L28] prefill 128 + 3 steps (the oracle decodes its weights first)")
    prompt = syn.make_prompt(G, 128, 5)
    run_chain(p, prompt, 3, TOL, "hd128-L28")
    say("[hd128-L28] gapped step at position 600")
    lg, ids, r = p.decode([0], [int(prompt[1])], [600])
    check(lg[0], r.logits[0], TOL, "hd128-L28 step at 600 logits")
    check(p.hidden(0, 1), r.layer_output, TOL, "hd128-L28 step at 600 layer_output")
    check(p.hidden(1, 1), r.final_norm_output, TOL, "hd128-L28 step at 600 final_norm_output")
    check_id(ids[0], r.logits[0], r.argmax[0], "hd128-L28 step at 600")
    p.close()
