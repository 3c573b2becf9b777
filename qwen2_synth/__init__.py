"""Seeded synthetic inputs for the Qwen2 decoder forward pass.

This module only draws numbers: model shapes, random-init weights and
uniform-random prompt ids.  It holds none of the forward pass's arithmetic and
is the one module that both the CPU oracle and the GPU path's tests/benchmarks
import.

Recipe (shared by every consumer):

* Every tensor has its own NumPy PCG64 stream, seeded by
  ``SeedSequence(master, spawn_key=(0, idx))``.  ``idx`` is 0 for the token
  embedding, 1 for the final norm, 2 for an untied lm_head and
  ``3 + 12*layer + t`` for the layer tensors, ``t`` running over
  attn_norm, wq, bq, wk, bk, wv, bv, wo, ffn_norm, w_gate, w_up, w_down.
  A model with fewer layers therefore shares its first layers bit for bit
  with the deeper one.
* Projection and embedding matrices: ``0.02 * N(0, 1)`` drawn in float32,
  rounded to IEEE binary16 (round to nearest even, subnormals kept) and
  stored as their uint16 bit patterns, row-major ``[out, in]`` (the layout of
  a PyTorch ``Linear`` weight, as in the Qwen2.5-0.5B module printout of the
  nnterp Qwen2 encyclopedia page).
* Biases: ``0.02 * N(0, 1)`` float32.  Norm weights: ``1 + 0.02 * N(0, 1)``
  float32.
* Prompts: ``integers(0, vocab)`` int32, stream ``SeedSequence(master,
  spawn_key=(1, j))`` for the j-th prompt (one per sequence slot).

The model shapes follow the Qwen2.5-0.5B config (nnterp Qwen2 page, "Config";
xinfer Module 7, section 7.1) and a Qwen2-7B-like hd=128 shape.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "ModelShape", "Workload", "MODELS", "WORKLOADS", "model_shape",
    "make_weights", "make_prompt", "weight_bytes", "LAYER_TENSORS",
]

LAYER_TENSORS = ("attn_norm", "wq", "bq", "wk", "bk", "wv", "bv", "wo",
                 "ffn_norm", "w_gate", "w_up", "w_down")


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layer: int
    n_embd: int
    n_head: int
    n_head_kv: int
    head_dim: int
    n_ff: int
    n_vocab: int
    tied: bool
    rope_theta: float
    rms_eps: float
    master: int  # seed of every stream of this model

    def with_layers(self, n_layer: int) -> "ModelShape":
        return dataclasses.replace(self, n_layer=n_layer,
                                   name=f"{self.name}-L{n_layer}")

    def shapes(self) -> Dict[str, tuple]:
        """Shape of every per-layer tensor ([out, in] for matrices)."""
        H, hd, nh, nkv, I = (self.n_embd, self.head_dim, self.n_head,
                             self.n_head_kv, self.n_ff)
        return {
            "attn_norm": (H,), "wq": (nh * hd, H), "bq": (nh * hd,),
            "wk": (nkv * hd, H), "bk": (nkv * hd,),
            "wv": (nkv * hd, H), "bv": (nkv * hd,),
            "wo": (H, nh * hd), "ffn_norm": (H,),
            "w_gate": (I, H), "w_up": (I, H), "w_down": (H, I),
        }


MODELS: Dict[str, ModelShape] = {
    # 2 layers, hidden 64, 4/2 heads, hd 16, FFN 172, vocab 512, tied.
    "tiny": ModelShape("tiny", 2, 64, 4, 2, 16, 172, 512, True, 1e6, 1e-6, 1),
    # Qwen2.5-0.5B shape, tied lm_head.
    "qwen2.5-0.5b": ModelShape("qwen2.5-0.5b", 24, 896, 14, 2, 64, 4864,
                               151936, True, 1e6, 1e-6, 2),
    # Qwen2-7B-like shape: hd 128, group 7, untied lm_head.
    "qwen2-hd128": ModelShape("qwen2-hd128", 28, 3584, 28, 4, 128, 18944,
                              152064, False, 1e6, 1e-6, 3),
    # The 12-over-2 head layout of 1.5B (nnterp page, "Grouped-query
    # attention": head_dim 128, so hidden 1536); the pages give no layer count
    # or FFN width for it: 28 layers and FFN 8960, tied lm_head.
    "qwen2.5-1.5b-heads": ModelShape("qwen2.5-1.5b-heads", 28, 1536, 12, 2, 128, 8960,
                                     151936, True, 1e6, 1e-6, 4),
}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: str
    prompt_len: int
    decode_steps: int
    n_ctx: int
    n_seq: int
    description: str


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", "tiny", 8, 8, 64, 1,
                     "tiny Qwen2-shaped decoder: prompt 8, 8 greedy steps, n_ctx 64"),
    "0.5b": Workload("0.5b", "qwen2.5-0.5b", 128, 128, 4096, 1,
                     "Qwen2.5-0.5B shape, batch 1: prompt 128, 128 greedy steps, n_ctx 4096"),
    "0.5b-long": Workload("0.5b-long", "qwen2.5-0.5b", 4096, 256, 8192, 1,
                          "Qwen2.5-0.5B shape: prompt 4096, 256 greedy steps, n_ctx 8192"),
    "0.5b-batched": Workload("0.5b-batched", "qwen2.5-0.5b", 1024, 1, 2048, 64,
                             "Qwen2.5-0.5B shape: 64 sequences with a 1024-token prefix, one decode step each"),
    "hd128": Workload("hd128", "qwen2-hd128", 2048, 128, 4096, 1,
                      "Qwen2-7B-like shape (hd 128, untied): prompt 2048, 128 greedy steps, n_ctx 4096"),
    "1.5b-heads": Workload("1.5b-heads", "qwen2.5-1.5b-heads", 512, 128, 4096, 1,
                           "12/2 heads of 128 (the 1.5B layout), 28 layers, FFN 8960: prompt 512, "
                           "128 greedy steps, n_ctx 4096"),
}


def model_shape(name: str, n_layer: Optional[int] = None) -> ModelShape:
    m = MODELS[name]
    return m if n_layer is None else m.with_layers(n_layer)


def _rng(master: int, kind: int, idx: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(master, spawn_key=(kind, idx))))


def _draw(master: int, idx: int, shape: tuple, kind: str) -> np.ndarray:
    g = _rng(master, 0, idx)
    a = g.standard_normal(shape, dtype=np.float32)
    a *= np.float32(0.02)
    if kind == "matrix":
        return a.astype(np.float16).view(np.uint16)
    if kind == "norm":
        a += np.float32(1.0)
    return a


def _kind(tname: str) -> str:
    if tname.endswith("norm"):
        return "norm"
    if tname in ("bq", "bk", "bv"):
        return "bias"
    return "matrix"


def make_weights(m: ModelShape, threads: Optional[int] = None) -> dict:
    """Draw every weight of model ``m``.

    Returns ``{"tok_embd": u16[V,H], "out_norm": f32[H], "lm_head": u16[V,H]
    or None (tied), "layers": [dict per layer]}``.
    """
    H, V = m.n_embd, m.n_vocab
    shapes = m.shapes()
    jobs = [("tok_embd", None, 0, (V, H), "matrix"),
            ("out_norm", None, 1, (H,), "norm")]
    if not m.tied:
        jobs.append(("lm_head", None, 2, (V, H), "matrix"))
    for l in range(m.n_layer):
        for t, tname in enumerate(LAYER_TENSORS):
            jobs.append((tname, l, 3 + 12 * l + t, shapes[tname], _kind(tname)))
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    out: dict = {"lm_head": None, "layers": [dict() for _ in range(m.n_layer)]}

    def run(job):
        tname, l, idx, shape, kind = job
        return tname, l, _draw(m.master, idx, shape, kind)

    with _cf.ThreadPoolExecutor(max(1, threads)) as ex:
        for tname, l, arr in ex.map(run, jobs):
            if l is None:
                out[tname] = arr
            else:
                out["layers"][l][tname] = arr
    return out


def make_prompt(m: ModelShape, n: int, j: int = 0) -> np.ndarray:
    """The j-th uniform-random prompt of ``n`` token ids in [0, vocab)."""
    return _rng(m.master, 1, j).integers(0, m.n_vocab, size=n, dtype=np.int32)


def weight_bytes(m: ModelShape) -> Dict[str, int]:
    """Bytes of the f16 matrices and f32 vectors of a model."""
    s = m.shapes()
    f16 = sum(int(np.prod(s[t])) for t in LAYER_TENSORS if _kind(t) == "matrix")
    f32 = sum(int(np.prod(s[t])) for t in LAYER_TENSORS if _kind(t) != "matrix")
    f16 = 2 * (m.n_layer * f16 + m.n_vocab * m.n_embd * (1 if m.tied else 2))
    f32 = 4 * (m.n_layer * f32 + m.n_embd)
    return {"f16": f16, "f32": f32}
