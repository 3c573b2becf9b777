"""GPU parity on the Qwen2.5-0.5B shape (24 layers, hidden 896, 14/2 heads,
hd 64, FFN 4864, vocab 151936, tied): the benchmark's workload, checked
against the CPU oracle under the 1e-2 * max|ref| bar with greedy ids exact
where the oracle's top-2 margin exceeds 1e-2."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import qwen2_synth as syn  # noqa: E402
from gpu_common import DEV, Pair, check, check_id, check_probs, run_chain, say  # noqa: E402

pytestmark = pytest.mark.gpu

S = syn.MODELS["qwen2.5-0.5b"]
TOL = 1e-2


@pytest.fixture(scope="module")
def w05():
    say("[0.5b] drawing weights")
    return syn.make_weights(S)


def test_0_5b_weight_store_and_kv_sizes(w05):
    import qwen2_decoder_forward_amd as q
    m = q.Model(S, w05, n_ctx=4096)
    info = m.info()
    assert info.weight_bytes_f16 == 987_922_432          # ~942 MiB of f16 weights
    assert info.kv_bytes_per_pos == 24_576               # 24 KB of f32 K/V per position
    assert info.kv_bytes == 96 * 2 ** 20                 # n_ctx 4096 -> 96 MiB
    m.close()


def test_0_5b_next_token_probs_and_stop_ids(w05):
    """The 151,936-entry distribution of a prefill read-out and of a 3-row
    decode against the oracle's softmax of the same logits; the eos / im_end
    ids as stop ids (a random-init model rarely produces them: the latch must
    then stay at -1, else hold the read-out position)."""
    import qwen2_decoder_forward_amd as q
    from oracle import qwen2_oracle as O
    m = q.Model(S, w05, n_ctx=256, n_seq=3)
    m.set_stop_ids([151643, 151645])
    V = S.n_vocab
    logits = torch.empty((3, V), dtype=torch.float32, device=DEV)
    probs = torch.empty((3, V), dtype=torch.float32, device=DEV)
    ids = torch.zeros(3, dtype=torch.int32, device=DEV)
    for s_ in range(3):
        m.prefill(s_, syn.make_prompt(S, 16, 70 + s_), np.arange(16), logits[s_], ids[s_:s_ + 1])
    m.next_token_probs(logits, 3, probs)
    torch.cuda.synchronize()
    check_probs(probs.cpu().numpy(), logits.cpu().numpy(), "0.5B prefill read-outs")
    first = ids.cpu().numpy().copy()
    m.decode([2, 0, 1], ids[[2, 0, 1]].contiguous(), [16, 16, 16], logits, ids)
    m.next_token_probs(logits, 3, probs)
    stops = torch.empty(3, dtype=torch.int32, device=DEV)
    m.read_stops(stops)
    torch.cuda.synchronize()
    check_probs(probs.cpu().numpy(), logits.cpu().numpy(), "0.5B 3-row decode")
    dec = ids.cpu().numpy()
    reads = [(s_, 15, int(first[s_])) for s_ in range(3)]
    reads += [(s_, 16, int(dec[b])) for b, s_ in enumerate([2, 0, 1])]
    assert list(stops.cpu().numpy()) == list(O.stop_positions(3, reads, [151643, 151645]))
    m.close()


def test_0_5b_prompt_128_then_greedy_decode(w05):
    """Prompt 128 (MFMA path), then teacher-forced greedy decode steps (GEMV
    path), every step's logits and the hidden states checked."""
    p = Pair(S, w05, n_ctx=4096, cache_decoded=True)
    run_chain(p, syn.make_prompt(S, 128), 24, TOL, "0.5b")
    p.close()


def test_0_5b_free_running_greedy_chain(w05):
    """The benchmark's loop: argmax feeds the next token on the device.  The
    GPU chain must equal the oracle's free-running chain up to the first step
    whose oracle top-2 margin is <= 1e-2 (after that they may diverge)."""
    import qwen2_decoder_forward_amd as q
    p = Pair(S, w05, n_ctx=4096, cache_decoded=True)
    prompt = syn.make_prompt(S, 128)
    steps = 16
    ids = torch.zeros(steps + 1, dtype=torch.int32, device=DEV)
    p.m.prefill(0, prompt, np.arange(128), None, ids[0:1])
    for s in range(steps):
        p.m.decode([0], ids[s:s + 1], [128 + s], None, ids[s + 1:s + 2])
    torch.cuda.synchronize()
    gpu = ids.cpu().numpy()
    r = p.o.prefill(0, prompt, np.arange(128))
    chain, margins = [int(r.argmax[0])], [r.logits[0]]
    for s in range(steps):
        r = p.o.decode([0], [chain[-1]], [128 + s])
        chain.append(int(r.argmax[0]))
        margins.append(r.logits[0])
    agreed = 0
    for s in range(steps + 1):
        if not check_id(gpu[s], margins[s], chain[s], f"free-running step {s}"):
            break
        agreed += 1
    say(f"[0.5b free-running] {agreed}/{steps + 1} ids agree before any low-margin step")
    assert agreed >= 1
    p.close()
