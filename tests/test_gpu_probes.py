"""The device-ceiling probes do the work their rates are computed from.

qwen2_probe_read: every 32-bit word of the buffer is read exactly once, so the
XOR of all per-wavefront folds equals the XOR of the buffer's words.
qwen2_probe_mfma: each wavefront adds the same four 32 x 32 x 16 products
`iters` times, so the sum of its accumulators has a closed form: for
C = A B, sum_ij C_ij = sum_k (sum_i A_ik)(sum_j B_kj), with the fragments'
values as the kernel builds them from the lane index (lane l holds row l % 32
of A at k = 8 (l / 32) .. + 7, and column l % 32 of B at the same k)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import qwen2_decoder_forward_amd as q  # noqa: E402
from gpu_common import DEV, say  # noqa: E402

pytestmark = pytest.mark.gpu


def test_read_probe_reads_every_word_once():
    rng = np.random.default_rng(5)
    for nbytes, nb in ((16 * 1000003, 64), (64 << 20, 1024), (16, 1)):
        words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
        buf = torch.from_numpy(words.view(np.int32)).to(DEV)
        out = torch.zeros(4 * nb, dtype=torch.int32, device=DEV)
        say(f"[probes] read {nbytes} bytes with {nb} blocks")
        q.qwen2_probe_read(buf, nbytes, nb, out)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(words), (nbytes, nb)


def frag(lane, j, mul, add, mod, off):
    # (f32 arithmetic, then one rounding to binary16, as in the kernel)
    return np.float16(np.float32(0.001) * np.float32((lane * mul + j * add) % mod) - np.float32(off))


def test_mfma_probe_sum_matches_closed_form():
    iters, nb = 200, 8
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    Aa = np.zeros((16, 32))  # a used as the B operand
    Bb = np.zeros((32, 16))  # b used as the A operand
    for lane in range(64):
        r, k0 = lane % 32, 8 * (lane // 32)
        for j in range(8):
            a = float(frag(lane, j, 7, 3, 17, 0.008))
            b = float(frag(lane, j, 5, 11, 13, 0.006))
            A[r, k0 + j], Bb[r, k0 + j] = a, b
            B[k0 + j, r], Aa[k0 + j, r] = b, a
    s = lambda X, Y: float((X @ Y).sum())  # noqa: E731
    want = iters * (s(A, B) + s(Bb, Aa) + s(A, Aa) + s(Bb, B))
    out = torch.zeros(4 * nb, dtype=torch.float32, device=DEV)
    say(f"[probes] mfma {iters} iterations, {nb} blocks")
    q.qwen2_probe_mfma(iters, nb, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.allclose(got, want, rtol=1e-4, atol=1e-6), (got[:4], want)


def test_probe_rates_are_physical():
    """Rates within what the device can do (guards against work the
    compiler could have dropped)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    nbytes = 1 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.empty(4 * 2048, dtype=torch.int32, device=DEV)
    q.qwen2_probe_read(buf, nbytes, 2048, out)
    ev[0].record()
    q.qwen2_probe_read(buf, nbytes, 2048, out)
    ev[1].record()
    torch.cuda.synchronize()
    gbs = nbytes / (ev[0].elapsed_time(ev[1]) / 1e3) / 1e9
    fo = torch.empty(4 * 1024, dtype=torch.float32, device=DEV)
    q.qwen2_probe_mfma(2000, 1024, fo)
    ev[0].record()
    q.qwen2_probe_mfma(2000, 1024, fo)
    ev[1].record()
    torch.cuda.synchronize()
    tfs = 1024 * 4 * 2000 * 4 * 2 * 32 * 32 * 16 / (ev[0].elapsed_time(ev[1]) / 1e3) / 1e12
    say(f"[probes] read {gbs:.0f} GB/s, f16 MFMA {tfs:.0f} TFLOP/s")
    assert 1000 < gbs <= 8000, gbs
    assert 200 < tfs <= 2500, tfs
