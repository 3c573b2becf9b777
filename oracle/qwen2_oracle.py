"""CPU oracle of the Qwen2 / Qwen2.5 decoder forward pass.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run this module; the GPU library
never does, and this module imports nothing from it.

What it computes (plain definition, written out step by step):

* The decoder layer dataflow of the minfer "Qwen2 / Qwen2.5 Architecture
  Support" page, section 1: RMSNorm, WQ/WK/WV projections plus bias, RoPE on
  Q and K, KV store, grouped-query attention (Q K^T scale, softmax, times V),
  WO plus residual, RMSNorm, gate/up, SiLU(gate) * up, down plus residual.
* Biases on q/k/v only, added before the rotary embedding; no bias on o_proj
  or the MLP (nnterp Qwen2 encyclopedia page, Notes, the subsection on the
  q/k/v biases).
* RoPE in the NonInterleaved / GPT-NeoX rotate_half pairing (minfer page,
  section 3; xinfer Module 7, section 7.2 table): dimension d pairs with
  d + head_dim/2.
* Query head h reads KV head floor(h / (n_head / n_head_kv)), i.e. KV head j
  serves query heads 7j..7j+6 on the 0.5B shape; score scale head_dim^-0.5
  (nnterp page, "Grouped-query attention").
* Full causal attention, no sliding window (nnterp page, Notes, the
  subsection on the sliding-window config keys).
* Positions are data: a row at position p attends to its sequence's KV slots
  0..p; a position >= n_ctx is a hard error that leaves the cache untouched
  (minfer page, section 6 and troubleshooting item 5).
* Readout: final RMSNorm, then lm_head (the token embedding when tied), with
  nothing applied after it (nnterp page, Notes, the readout subsection;
  xinfer Module 7, section 7.3), and greedy argmax on the device side of the
  pages' engines (xinfer 7.3) taken here as the lowest index of the largest
  logit.
* next_token_probs: the next-token distribution at a read-out position, the
  softmax of that row's logits (nnterp page, standardized tap list).
* Stop ids are data (eos and im_end, minfer page, section 5): a greedy
  read-out whose id is one of them marks its sequence as stopped at that
  read-out position; the earliest such position is kept.

Precision: activations are stored as float32 between operations (the CPU
reference and activations are f32 in the xinfer Module 7, section 7.4 dtype
table); every dot product, sum and transcendental is evaluated in float64 and
rounded to float32 once per operation output.  Weights are the same binary16
bit patterns the GPU library receives, decoded by this module's own decoder.

Readings where the pages are silent (each also listed in the design notes):
RMSNorm is w * x / sqrt(mean(x^2) + eps); RoPE angle is
pos * freq_scale * theta^(-2d/head_dim) with freq_scale = 1, evaluated in
float64; softmax subtracts the row maximum; every row of a call stores its
K/V before any row attends; KV slots never written read as zero; positions
within one prefill must be strictly increasing; the argmax ignores NaN and
takes the lowest index on ties.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

f32 = np.float32
f64 = np.float64


# --------------------------------------------------------------------------
# binary16 decoding (own decoder; pinned against NumPy's float16 in tests)
# --------------------------------------------------------------------------
def _build_f16_table() -> np.ndarray:
    """Value of every binary16 bit pattern, as float64.

    IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
    bits.  Exponent 0 encodes zero and subnormals f * 2^-24; exponent 31
    encodes infinities (f = 0) and NaNs.
    """
    bits = np.arange(65536, dtype=np.int64)
    sign = np.where((bits >> 15) & 1, -1.0, 1.0)
    e = (bits >> 10) & 0x1F
    f = (bits & 0x3FF).astype(f64)
    normal = np.ldexp(1024.0 + f, (e - 25).astype(np.int32))  # (1 + f/1024) 2^(e-15)
    sub = np.ldexp(f, -24)
    mag = np.where(e == 0, sub, normal)
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


F16_TABLE = _build_f16_table()


def decode_f16(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns (uint16) -> float64 values."""
    return F16_TABLE[np.asarray(bits, dtype=np.uint16)]


# --------------------------------------------------------------------------
# hyperparameters and errors
# --------------------------------------------------------------------------
class OracleError(ValueError):
    """A rejected call.  ``code`` is one of E_ARG, E_HPARAMS, E_SEQ, E_TOKEN,
    E_POS, E_ORDER."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


@dataclasses.dataclass(frozen=True)
class Hparams:
    n_layer: int
    n_embd: int
    n_head: int
    n_head_kv: int
    head_dim: int
    n_ff: int
    n_vocab: int
    n_ctx: int
    n_seq: int
    tied: bool
    rope_theta: float
    rms_eps: float
    rope_freq_scale: float = 1.0
    # RoPE pairing is a model-level flag (minfer page, section 3): 0 =
    # NonInterleaved (the Qwen2 family), 1 = Interleaved (Llama style)
    rope_style: int = 0

    def validate(self) -> None:
        if min(self.n_layer, self.n_embd, self.n_head, self.n_head_kv,
               self.head_dim, self.n_ff, self.n_vocab, self.n_ctx,
               self.n_seq) <= 0:
            raise OracleError("E_HPARAMS", "every size must be positive")
        # head_dim = hidden / n_heads (xinfer Module 7, section 7.1).
        if self.n_embd != self.n_head * self.head_dim:
            raise OracleError("E_HPARAMS", "n_embd != n_head * head_dim")
        # each KV head serves a whole group of query heads (nnterp, GQA).
        if self.n_head % self.n_head_kv:
            raise OracleError("E_HPARAMS", "n_head % n_head_kv != 0")
        if self.head_dim % 2:
            raise OracleError("E_HPARAMS", "RoPE pairs need an even head_dim")
        if self.rope_style not in (0, 1):
            raise OracleError("E_HPARAMS", "rope_style is 0 (NonInterleaved) or 1 (Interleaved)")


# --------------------------------------------------------------------------
# the operations, one function each
# --------------------------------------------------------------------------
def rms_norm(h: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Pre-norm RMSNorm without mean subtraction or bias (xinfer 7.2 table):
    y = w * x / sqrt(mean(x^2) + eps).  Rows are the last axis."""
    x = np.asarray(h, dtype=f64)
    inv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return (x * inv * np.asarray(w, dtype=f64)).astype(f32)


def linear(x: np.ndarray, w_bits: np.ndarray, bias: Optional[np.ndarray] = None,
           w64: Optional[np.ndarray] = None) -> np.ndarray:
    """y = x W^T (+ b) for a [out, in] binary16 weight, float64 sum, f32 out."""
    W = decode_f16(w_bits) if w64 is None else w64
    y = np.asarray(x, dtype=f64) @ W.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=f64)
    return y.astype(f32)


def rope_angles(positions: np.ndarray, head_dim: int, theta: float,
                freq_scale: float = 1.0) -> np.ndarray:
    """phi[i, d] = pos_i * freq_scale * theta^(-2d/head_dim), d < head_dim/2."""
    d = np.arange(head_dim // 2, dtype=f64)
    inv_freq = theta ** (-2.0 * d / head_dim)
    return np.asarray(positions, dtype=f64)[:, None] * freq_scale * inv_freq[None, :]


def rope_rotate_half(x: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """NonInterleaved RoPE: dimension d pairs with d + head_dim/2.

    x: [n, heads, head_dim] float32, phi: [n, head_dim/2].  For each pair
    (a, b) = (x[d], x[d + hd/2]) the result is (a cos - b sin, b cos + a sin).
    """
    x = np.asarray(x, dtype=f64)
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1).astype(f32)


def rope_interleaved(x: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Llama-style Interleaved RoPE: dimension 2d pairs with 2d + 1, rotated
    by phi[:, d].  Not the Qwen2 family's convention, but a model-level flag
    (minfer page, section 3)."""
    x = np.asarray(x, dtype=f64)
    a, b = x[..., 0::2], x[..., 1::2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out.astype(f32)


def softmax(s: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis, in float64, max subtracted first.
    Entries equal to -inf (masked keys) get probability 0."""
    s = np.asarray(s, dtype=f64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def next_token_probs(logits: np.ndarray) -> np.ndarray:
    """The next-token distribution of each read-out row: softmax over the
    vocabulary of its logits (float64, rounded to float32)."""
    return softmax(logits).astype(f32)


def stop_positions(n_seq: int, readouts, stop_ids) -> np.ndarray:
    """readouts: (sequence slot, read-out position, greedy id) triples in any
    order.  Returns, per slot, the smallest read-out position whose id is a
    stop id, or -1 when there is none."""
    stops = set(int(t) for t in stop_ids)
    out = np.full(n_seq, -1, dtype=np.int64)
    for seq, pos, tok in readouts:
        if int(tok) in stops and (out[seq] < 0 or pos < out[seq]):
            out[seq] = pos
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=f64)
    return z / (1.0 + np.exp(-z))


def attention_scale(head_dim: int) -> float:
    """Score scale head_dim^-0.5 (nnterp Qwen2 page, Grouped-query attention)."""
    return head_dim ** -0.5


def kv_head_of(h: int, n_head: int, n_head_kv: int) -> int:
    """KV head read by query head h: contiguous groups of n_head/n_head_kv
    query heads share one KV head (KV head j serves 7j..7j+6 on 14/2)."""
    return h // (n_head // n_head_kv)


def argmax_lowest(logits: np.ndarray) -> int:
    """Index of the largest logit; ties go to the lowest index; NaN never
    wins (all-NaN rows give 0)."""
    v = np.asarray(logits, dtype=f32)
    ok = ~np.isnan(v)
    if not ok.any():
        return 0
    m = np.max(v[ok])
    return int(np.flatnonzero(ok & (v == m))[0])


# --------------------------------------------------------------------------
# the model
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Result:
    logits: np.ndarray            # [n_out, V] float32
    argmax: np.ndarray            # [n_out] int32
    layer_output: np.ndarray      # [n_out, H] last layer's output rows
    final_norm_output: np.ndarray  # [n_out, H]
    taps: Optional[dict] = None


class Qwen2Oracle:
    """Plain forward pass with a per-sequence KV cache.

    ``weights`` uses the layout of ``qwen2_synth.make_weights``: binary16
    bit patterns (uint16) for matrices, float32 for biases and norms.
    """

    def __init__(self, hp: Hparams, weights: dict, cache_decoded: bool = False):
        hp.validate()
        self.hp = hp
        self.w = weights
        self.cache_decoded = cache_decoded
        self._dec: Dict[tuple, np.ndarray] = {}
        # K and V cache per sequence: [n_layer, n_head_kv, n_ctx, head_dim]
        # float32, zero until written (KV slots never written read as zero).
        self.k_cache: Dict[int, np.ndarray] = {}
        self.v_cache: Dict[int, np.ndarray] = {}

    # ---- weights -----------------------------------------------------------
    def _w64(self, key: tuple, bits: np.ndarray) -> Optional[np.ndarray]:
        if not self.cache_decoded:
            return None
        if key not in self._dec:
            self._dec[key] = decode_f16(bits)
        return self._dec[key]

    def lm_head_bits(self) -> np.ndarray:
        # W_lm = E when tied (xinfer 7.3; nnterp Notes, readout subsection).
        return self.w["tok_embd"] if self.hp.tied else self.w["lm_head"]

    # ---- cache -------------------------------------------------------------
    def _cache(self, seq: int):
        if seq not in self.k_cache:
            hp = self.hp
            shape = (hp.n_layer, hp.n_head_kv, hp.n_ctx, hp.head_dim)
            self.k_cache[seq] = np.zeros(shape, dtype=f32)
            self.v_cache[seq] = np.zeros(shape, dtype=f32)
        return self.k_cache[seq], self.v_cache[seq]

    def reset(self) -> None:
        self.k_cache.clear()
        self.v_cache.clear()

    # ---- validation --------------------------------------------------------
    def _validate(self, seqs, tokens, positions, prefill: bool) -> None:
        hp = self.hp
        n = len(tokens)
        if n <= 0 or len(seqs) != n or len(positions) != n:
            raise OracleError("E_ARG", "empty call or mismatched lengths")
        for s in seqs:
            if not 0 <= int(s) < hp.n_seq:
                raise OracleError("E_SEQ", f"sequence {int(s)} not in [0, {hp.n_seq})")
        if not prefill and len(set(int(s) for s in seqs)) != n:
            raise OracleError("E_SEQ", "a sequence appears twice in one decode batch")
        for t in tokens:
            if not 0 <= int(t) < hp.n_vocab:
                raise OracleError("E_TOKEN", f"token {int(t)} not in [0, {hp.n_vocab})")
        for p in positions:
            if not 0 <= int(p) < hp.n_ctx:
                raise OracleError("E_POS", f"position {int(p)} not in [0, {hp.n_ctx})")
        if prefill:
            p = np.asarray(positions, dtype=np.int64)
            if np.any(p[1:] <= p[:-1]):
                raise OracleError("E_ORDER", "positions of one prefill must increase")

    # ---- public calls ------------------------------------------------------
    def prefill(self, seq: int, tokens: Sequence[int], positions: Sequence[int],
                taps: bool = False) -> Result:
        """One prompt (or continuation) of one sequence; reads out the last row."""
        n = len(tokens)
        seqs = [seq] * n
        self._validate(seqs, tokens, positions, prefill=True)
        return self._forward(np.asarray(seqs), np.asarray(tokens), np.asarray(positions),
                             out_rows=[n - 1], taps=taps)

    def decode(self, seq_ids: Sequence[int], tokens: Sequence[int],
               positions: Sequence[int], taps: bool = False) -> Result:
        """One token for each of several distinct sequences."""
        self._validate(seq_ids, tokens, positions, prefill=False)
        n = len(tokens)
        return self._forward(np.asarray(seq_ids), np.asarray(tokens),
                             np.asarray(positions), out_rows=list(range(n)), taps=taps)

    # ---- the forward pass --------------------------------------------------
    def _attention(self, l: int, seqs, positions, q: np.ndarray) -> tuple:
        """Causal GQA attention of every row against its sequence's cache.

        q: [n, n_head, hd] float32 (already rotated).  Returns the head
        outputs [n, n_head, hd] float32 and, per row group, scores/probs.
        """
        hp = self.hp
        n = q.shape[0]
        scale = attention_scale(hp.head_dim)
        out = np.zeros((n, hp.n_head, hp.head_dim), dtype=f32)
        scores_all = {}
        for s in sorted(set(int(x) for x in seqs)):
            rows = np.flatnonzero(seqs == s)
            pos = positions[rows].astype(np.int64)
            P = int(pos.max()) + 1
            Kc, Vc = self._cache(s)
            mask = np.arange(P)[None, :] > pos[:, None]   # key j visible iff j <= pos
            for h in range(hp.n_head):
                g = kv_head_of(h, hp.n_head, hp.n_head_kv)
                K = Kc[l, g, :P].astype(f64)
                V = Vc[l, g, :P].astype(f64)
                sc = (q[rows, h].astype(f64) @ K.T) * scale
                sc[mask] = -np.inf
                p = softmax(sc)
                out[rows, h] = (p @ V).astype(f32)
                scores_all[(s, h)] = (rows, sc, p)
        return out, scores_all

    def _forward(self, seqs, tokens, positions, out_rows: List[int], taps: bool) -> Result:
        hp, w = self.hp, self.w
        n = len(tokens)
        nh, nkv, hd, H = hp.n_head, hp.n_head_kv, hp.head_dim, hp.n_embd
        T: Optional[dict] = {"layers": []} if taps else None

        # Embedding lookup, no scaling.
        h = decode_f16(w["tok_embd"][tokens]).astype(f32)
        if taps:
            T["token_embeddings"] = h.copy()
        phi = rope_angles(positions, hd, hp.rope_theta, hp.rope_freq_scale)

        for l in range(hp.n_layer):
            L = w["layers"][l]
            lt: dict = {}
            if taps:
                lt["layer_input"] = h.copy()
            x = rms_norm(h, L["attn_norm"], hp.rms_eps)
            q = linear(x, L["wq"], L["bq"], self._w64((l, "wq"), L["wq"]))
            k = linear(x, L["wk"], L["bk"], self._w64((l, "wk"), L["wk"]))
            v = linear(x, L["wv"], L["bv"], self._w64((l, "wv"), L["wv"]))
            rope = rope_interleaved if self.hp.rope_style == 1 else rope_rotate_half
            q = rope(q.reshape(n, nh, hd), phi)
            k = rope(k.reshape(n, nkv, hd), phi)
            v = v.reshape(n, nkv, hd)
            # KV store of every row first, then attention.
            for i in range(n):
                Kc, Vc = self._cache(int(seqs[i]))
                Kc[l, :, positions[i]] = k[i]
                Vc[l, :, positions[i]] = v[i]
            o, sc = self._attention(l, seqs, positions, q)
            attn_out = linear(o.reshape(n, nh * hd), L["wo"], None,
                              self._w64((l, "wo"), L["wo"]))
            h_mid = (h.astype(f64) + attn_out.astype(f64)).astype(f32)
            x2 = rms_norm(h_mid, L["ffn_norm"], hp.rms_eps)
            gate = linear(x2, L["w_gate"], None, self._w64((l, "w_gate"), L["w_gate"]))
            up = linear(x2, L["w_up"], None, self._w64((l, "w_up"), L["w_up"]))
            act = silu(gate)
            a = (act * up.astype(f64)).astype(f32)
            mlp_out = linear(a, L["w_down"], None, self._w64((l, "w_down"), L["w_down"]))
            h_out = (h_mid.astype(f64) + mlp_out.astype(f64)).astype(f32)
            if taps:
                lt.update(
                    attention_norm_output=x,
                    attention_queries=np.transpose(q, (1, 0, 2)).copy(),
                    attention_keys=np.transpose(k, (1, 0, 2)).copy(),
                    attention_values=np.transpose(v, (1, 0, 2)).copy(),
                    attention_scores=sc, attention_head_outputs=o,
                    attention_premix=o.reshape(n, nh * hd).copy(),
                    attention_output=attn_out, layer_mid=h_mid,
                    mlp_norm_output=x2, mlp_input=x2,
                    mlp_activation=act.astype(f32), mlp_neurons=a,
                    mlp_output=mlp_out, layer_output=h_out)
                T["layers"].append(lt)
            h = h_out

        rows = np.asarray(out_rows)
        y = rms_norm(h[rows], w["out_norm"], hp.rms_eps)
        W_lm = self.lm_head_bits()
        logits = linear(y, W_lm, None, self._w64(("lm_head",), W_lm))
        ids = np.array([argmax_lowest(r) for r in logits], dtype=np.int32)
        if taps:
            T["final_norm_output"] = y
            T["logits"] = logits
        return Result(logits=logits, argmax=ids, layer_output=h[rows].copy(),
                      final_norm_output=y, taps=T)


def hparams_for(shape, n_ctx: int, n_seq: int = 1, rope_style: int = 0) -> Hparams:
    """Hparams from a ``qwen2_synth.ModelShape`` plus the cache sizes."""
    return Hparams(n_layer=shape.n_layer, n_embd=shape.n_embd, n_head=shape.n_head,
                   n_head_kv=shape.n_head_kv, head_dim=shape.head_dim, n_ff=shape.n_ff,
                   n_vocab=shape.n_vocab, n_ctx=n_ctx, n_seq=n_seq, tied=shape.tied,
                   rope_theta=shape.rope_theta, rms_eps=shape.rms_eps, rope_style=rope_style)
