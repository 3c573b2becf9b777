"""Python binding of libqwen2_mi355x.so (the MI355X Qwen2 decoder forward).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI declared in include/qwen2.h.  Device buffers are
passed as torch tensors on the ROCm device (or raw integer addresses); the
stream defaults to torch's current stream.  There is no CPU fallback: if the
library is missing, importing a call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

__all__ = [
    "Hparams", "LayerWeights", "Weights", "Info", "Qwen2Error", "CODES", "lib", "LIB_PATH",
    "qwen2_check_hparams", "qwen2_check_prefill", "qwen2_check_prefill_batch",
    "qwen2_check_decode", "qwen2_load", "qwen2_prefill", "qwen2_prefill_batch", "qwen2_decode",
    "qwen2_read_hidden", "qwen2_kv_read", "qwen2_kv_write", "qwen2_next_token_probs",
    "qwen2_next_token_probs_static",
    "qwen2_set_stop_ids", "qwen2_read_stops",
    "qwen2_sync_status", "qwen2_info", "qwen2_last_error", "qwen2_strerror", "qwen2_free",
    "qwen2_prof_enable", "qwen2_prof_read", "qwen2_prof_repeat", "qwen2_probe_read",
    "qwen2_probe_mfma", "OPS", "make_hparams", "Model",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqwen2_mi355x.so")

CODES = {0: "OK", -1: "E_ARG", -2: "E_HPARAMS", -3: "E_POS", -4: "E_TOKEN", -5: "E_SEQ",
         -6: "E_ORDER", -7: "E_HIP", -8: "E_OOM", -9: "E_DEBUG"}

# op kinds of qwen2_prof_enable / qwen2_prof_read (QWEN2_OP_* in the header)
OPS = {"embed": 0, "qkv": 1, "attn": 2, "wo": 3, "gateup": 4, "down": 5, "lmhead": 6, "norm": 7}

i32, f32, u16 = C.c_int32, C.c_float, C.c_uint16
PF, PU16, PI32 = C.POINTER(C.c_float), C.POINTER(C.c_uint16), C.POINTER(C.c_int32)


class Hparams(C.Structure):
    _fields_ = [("n_layer", i32), ("n_embd", i32), ("n_head", i32), ("n_head_kv", i32),
                ("head_dim", i32), ("n_ff", i32), ("n_vocab", i32), ("n_ctx", i32),
                ("n_seq", i32), ("tied", i32), ("rope_style", i32), ("rope_theta", f32),
                ("rope_freq_scale", f32), ("rms_eps", f32)]


class LayerWeights(C.Structure):
    _fields_ = [("attn_norm", PF), ("bq", PF), ("bk", PF), ("bv", PF), ("ffn_norm", PF),
                ("wq", PU16), ("wk", PU16), ("wv", PU16), ("wo", PU16), ("w_gate", PU16),
                ("w_up", PU16), ("w_down", PU16)]


class Weights(C.Structure):
    _fields_ = [("tok_embd", PU16), ("lm_head", PU16), ("out_norm", PF),
                ("layers", C.POINTER(LayerWeights))]


class Info(C.Structure):
    _fields_ = [("weight_bytes_f16", C.c_uint64), ("weight_bytes_f32", C.c_uint64),
                ("weight_bytes_alloc", C.c_uint64), ("kv_bytes_per_pos", C.c_uint64),
                ("kv_bytes", C.c_uint64), ("scratch_bytes", C.c_uint64), ("n_ctx", i32),
                ("n_seq", i32), ("max_rows", i32)]


class Qwen2Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        self.code = code
        self.name = CODES.get(code, str(code))
        super().__init__(f"{self.name} ({code}): {msg}")


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m qwen2_decoder_forward_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        vp = C.c_void_p
        sig = {
            "qwen2_check_hparams": (i32, [C.POINTER(Hparams)]),
            "qwen2_check_prefill": (i32, [C.POINTER(Hparams), i32, PI32, PI32, i32]),
            "qwen2_check_prefill_batch": (i32, [C.POINTER(Hparams), i32, PI32, PI32, PI32, PI32]),
            "qwen2_check_decode": (i32, [C.POINTER(Hparams), i32, PI32, PI32]),
            "qwen2_load": (i32, [C.POINTER(Hparams), C.POINTER(Weights), vp, C.POINTER(vp)]),
            "qwen2_prefill": (i32, [vp, i32, PI32, PI32, i32, vp, vp, vp]),
            "qwen2_prefill_batch": (i32, [vp, i32, PI32, PI32, PI32, PI32, vp, vp, vp]),
            "qwen2_decode": (i32, [vp, i32, PI32, vp, PI32, vp, vp, vp]),
            "qwen2_read_hidden": (i32, [vp, i32, vp, vp]),
            "qwen2_next_token_probs": (i32, [vp, vp, i32, vp, vp]),
            "qwen2_next_token_probs_static": (i32, [vp, i32, i32, vp, vp]),
            "qwen2_set_stop_ids": (i32, [vp, PI32, i32]),
            "qwen2_read_stops": (i32, [vp, vp, i32, vp]),
            "qwen2_kv_read": (i32, [vp, i32, i32, i32, i32, vp, vp, vp]),
            "qwen2_kv_write": (i32, [vp, i32, i32, i32, i32, vp, vp, vp]),
            "qwen2_sync_status": (i32, [vp, vp]),
            "qwen2_info": (i32, [vp, C.POINTER(Info)]),
            "qwen2_last_error": (C.c_char_p, [vp]),
            "qwen2_strerror": (C.c_char_p, [i32]),
            "qwen2_free": (None, [vp]),
            "qwen2_prof_enable": (i32, [vp, C.c_uint32]),
            "qwen2_prof_read": (i32, [vp, i32, PI32, C.POINTER(C.c_double)]),
            "qwen2_prof_repeat": (i32, [vp, i32, i32, i32, vp]),
            "qwen2_probe_read": (i32, [vp, C.c_size_t, i32, vp, vp]),
            "qwen2_probe_mfma": (i32, [i32, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


# ---------------------------------------------------------------- marshalling
def _ptr(x) -> Optional[int]:
    """Device address of a torch tensor / integer, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _check(rc: int, ctx=None):
    if rc != 0:
        msg = lib().qwen2_last_error(ctx)
        raise Qwen2Error(rc, (msg or b"").decode() or lib().qwen2_strerror(rc).decode())


def make_hparams(shape, n_ctx: int, n_seq: int = 1, rope_style: int = 0) -> Hparams:
    """Hparams from any object with the qwen2_synth.ModelShape fields."""
    return Hparams(shape.n_layer, shape.n_embd, shape.n_head, shape.n_head_kv, shape.head_dim,
                   shape.n_ff, shape.n_vocab, n_ctx, n_seq, int(shape.tied), rope_style,
                   shape.rope_theta, 1.0, shape.rms_eps)


# ---------------------------------------------------------------- the C calls
def qwen2_check_hparams(hp: Hparams) -> int:
    return lib().qwen2_check_hparams(C.byref(hp))


def qwen2_check_prefill(hp: Hparams, seq: int, tokens, positions) -> int:
    t, p = _i32(tokens), _i32(positions)
    return lib().qwen2_check_prefill(C.byref(hp), seq, _p(t, PI32), _p(p, PI32), len(t))


def _batch(seq_ids, tokens, positions):
    """Flattens per-sequence lists into (seq_ids, lens, tokens, positions)."""
    s = _i32(seq_ids)
    if len(tokens) != len(s) or len(positions) != len(s):
        raise ValueError("one token list and one position list per sequence")
    t = [_i32(x) for x in tokens]
    p = [_i32(x) for x in positions]
    if any(len(a) != len(b) for a, b in zip(t, p)):
        raise ValueError("tokens and positions of a sequence differ in length")
    lens = np.array([len(a) for a in t], dtype=np.int32)
    cat = lambda xs: np.ascontiguousarray(np.concatenate(xs) if xs else np.zeros(0, np.int32))
    return s, lens, cat(t), cat(p)


def qwen2_check_prefill_batch(hp: Hparams, seq_ids, tokens, positions) -> int:
    """tokens, positions: one array per sequence."""
    s, n, t, p = _batch(seq_ids, tokens, positions)
    return lib().qwen2_check_prefill_batch(C.byref(hp), len(s), _p(s, PI32), _p(n, PI32),
                                           _p(t, PI32), _p(p, PI32))


def qwen2_check_decode(hp: Hparams, seq_ids, positions) -> int:
    s, p = _i32(seq_ids), _i32(positions)
    return lib().qwen2_check_decode(C.byref(hp), len(s), _p(s, PI32), _p(p, PI32))


def qwen2_load(hp: Hparams, weights: dict, stream=None) -> int:
    """Copies host weights (layout of qwen2_synth.make_weights) to the device."""
    keep = []

    def f(a):
        a = np.ascontiguousarray(a, dtype=np.float32)
        keep.append(a)
        return _p(a, PF)

    def h(a):
        a = np.ascontiguousarray(a, dtype=np.uint16)
        keep.append(a)
        return _p(a, PU16)

    layers = (LayerWeights * hp.n_layer)()
    for i, L in enumerate(weights["layers"][:hp.n_layer]):
        layers[i] = LayerWeights(f(L["attn_norm"]), f(L["bq"]), f(L["bk"]), f(L["bv"]),
                                 f(L["ffn_norm"]), h(L["wq"]), h(L["wk"]), h(L["wv"]), h(L["wo"]),
                                 h(L["w_gate"]), h(L["w_up"]), h(L["w_down"]))
    lm = weights.get("lm_head")
    w = Weights(h(weights["tok_embd"]), h(lm) if lm is not None else None,
                f(weights["out_norm"]), layers)
    ctx = C.c_void_p()
    _check(lib().qwen2_load(C.byref(hp), C.byref(w), _stream(stream), C.byref(ctx)))
    return ctx.value


def qwen2_prefill(ctx: int, seq: int, tokens, positions, logits=None, argmax=None,
                  stream=None) -> None:
    t, p = _i32(tokens), _i32(positions)
    _check(lib().qwen2_prefill(ctx, seq, _p(t, PI32), _p(p, PI32), len(t), _ptr(logits),
                               _ptr(argmax), _stream(stream)), ctx)


def qwen2_prefill_batch(ctx: int, seq_ids, tokens, positions, logits=None, argmax=None,
                        stream=None) -> None:
    """tokens, positions: one array per sequence; logits [len(seq_ids), V]."""
    s, n, t, p = _batch(seq_ids, tokens, positions)
    _check(lib().qwen2_prefill_batch(ctx, len(s), _p(s, PI32), _p(n, PI32), _p(t, PI32),
                                     _p(p, PI32), _ptr(logits), _ptr(argmax), _stream(stream)),
           ctx)


def qwen2_decode(ctx: int, seq_ids, tokens_dev, positions, logits=None, argmax=None,
                 stream=None) -> None:
    s, p = _i32(seq_ids), _i32(positions)
    _check(lib().qwen2_decode(ctx, len(s), _p(s, PI32), _ptr(tokens_dev), _p(p, PI32),
                              _ptr(logits), _ptr(argmax), _stream(stream)), ctx)


def qwen2_read_hidden(ctx: int, which: int, out, stream=None) -> None:
    _check(lib().qwen2_read_hidden(ctx, which, _ptr(out), _stream(stream)), ctx)


def qwen2_next_token_probs(ctx: int, logits, rows: int, probs, stream=None) -> None:
    _check(lib().qwen2_next_token_probs(ctx, _ptr(logits), rows, _ptr(probs), _stream(stream)),
           ctx)


def qwen2_next_token_probs_static(logits, rows: int, n_vocab: int, probs, stream=None) -> None:
    """The allocation-free form (no context; the library's fixed scratch)."""
    _check(lib().qwen2_next_token_probs_static(_ptr(logits), rows, n_vocab, _ptr(probs),
                                               _stream(stream)))


def qwen2_probe_read(buf, nbytes: int, n_blocks: int, out, stream=None) -> None:
    """Streaming read of nbytes at buf (device ceiling probe; out: [4 n_blocks] int32)."""
    _check(lib().qwen2_probe_read(_ptr(buf), nbytes, n_blocks, _ptr(out), _stream(stream)))


def qwen2_probe_mfma(iters: int, n_blocks: int, out, stream=None) -> None:
    """Register-only f16 MFMA loop (device ceiling probe; out: [4 n_blocks] f32)."""
    _check(lib().qwen2_probe_mfma(iters, n_blocks, _ptr(out), _stream(stream)))


def qwen2_set_stop_ids(ctx: int, ids) -> None:
    a = _i32(ids)
    _check(lib().qwen2_set_stop_ids(ctx, _p(a, PI32), len(a)), ctx)


def qwen2_read_stops(ctx: int, out, clear: bool = False, stream=None) -> None:
    _check(lib().qwen2_read_stops(ctx, _ptr(out), int(bool(clear)), _stream(stream)), ctx)


def qwen2_kv_read(ctx: int, layer: int, seq: int, pos0: int, n: int, k, v, stream=None) -> None:
    _check(lib().qwen2_kv_read(ctx, layer, seq, pos0, n, _ptr(k), _ptr(v), _stream(stream)), ctx)


def qwen2_kv_write(ctx: int, layer: int, seq: int, pos0: int, n: int, k, v, stream=None) -> None:
    _check(lib().qwen2_kv_write(ctx, layer, seq, pos0, n, _ptr(k), _ptr(v), _stream(stream)), ctx)


def qwen2_sync_status(ctx: int, stream=None) -> int:
    return lib().qwen2_sync_status(ctx, _stream(stream))


def qwen2_info(ctx: int) -> Info:
    out = Info()
    _check(lib().qwen2_info(ctx, C.byref(out)), ctx)
    return out


def qwen2_last_error(ctx: Optional[int] = None) -> str:
    return (lib().qwen2_last_error(ctx) or b"").decode()


def qwen2_strerror(code: int) -> str:
    return lib().qwen2_strerror(code).decode()


def qwen2_prof_enable(ctx: int, ops) -> None:
    """Time every launch of the given op kinds (names of OPS) with HIP events."""
    mask = 0
    for o in ops:
        mask |= 1 << OPS[o]
    _check(lib().qwen2_prof_enable(ctx, mask), ctx)


def qwen2_prof_read(ctx: int, op: str):
    """(launches, total milliseconds) of one op kind since the last read."""
    n, ms = C.c_int32(), C.c_double()
    _check(lib().qwen2_prof_read(ctx, OPS[op], C.byref(n), C.byref(ms)), ctx)
    return n.value, ms.value


def qwen2_prof_repeat(ctx: int, op: str, rows: int, iters: int, stream=None) -> None:
    """Enqueue `iters` back-to-back launches of one op (layer i % n_layer)."""
    _check(lib().qwen2_prof_repeat(ctx, OPS[op], rows, iters, _stream(stream)), ctx)


def qwen2_free(ctx: int) -> None:
    lib().qwen2_free(ctx)


class Model:
    """A loaded context with its hparams (convenience over the calls above)."""

    def __init__(self, shape, weights: dict, n_ctx: int, n_seq: int = 1, stream=None,
                 rope_style: int = 0):
        self.hp = make_hparams(shape, n_ctx, n_seq, rope_style)
        self.ctx = qwen2_load(self.hp, weights, stream)

    def prefill(self, seq, tokens, positions, logits=None, argmax=None, stream=None):
        qwen2_prefill(self.ctx, seq, tokens, positions, logits, argmax, stream)

    def prefill_batch(self, seq_ids, tokens, positions, logits=None, argmax=None, stream=None):
        qwen2_prefill_batch(self.ctx, seq_ids, tokens, positions, logits, argmax, stream)

    def decode(self, seq_ids, tokens_dev, positions, logits=None, argmax=None, stream=None):
        qwen2_decode(self.ctx, seq_ids, tokens_dev, positions, logits, argmax, stream)

    def read_hidden(self, which, out, stream=None):
        qwen2_read_hidden(self.ctx, which, out, stream)

    def next_token_probs(self, logits, rows, probs, stream=None):
        qwen2_next_token_probs(self.ctx, logits, rows, probs, stream)

    def set_stop_ids(self, ids):
        qwen2_set_stop_ids(self.ctx, ids)

    def read_stops(self, out, clear=False, stream=None):
        qwen2_read_stops(self.ctx, out, clear, stream)

    def kv_read(self, layer, seq, pos0, n, k, v, stream=None):
        qwen2_kv_read(self.ctx, layer, seq, pos0, n, k, v, stream)

    def kv_write(self, layer, seq, pos0, n, k, v, stream=None):
        qwen2_kv_write(self.ctx, layer, seq, pos0, n, k, v, stream)

    def sync_status(self, stream=None) -> int:
        return qwen2_sync_status(self.ctx, stream)

    def info(self) -> Info:
        return qwen2_info(self.ctx)

    def close(self):
        if self.ctx:
            qwen2_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
