#!/usr/bin/env python3
"""Benchmark: Qwen2.5-0.5B-shaped decoder forward on one MI355X.

One step is one pass of the whole hot path over the 0.5B workload: a
128-token uniform-random prompt is prefilled (positions 0..127) and then 128
greedy decode steps run at positions 128..255, each step's argmax feeding the
next step's token on the device (no host round trip).  Weights are seeded
random-init f16 (the model has no trained checkpoint here), resident in HBM
before the timed region starts.

Prints one JSON line.  `value` is decode tokens/s at batch 1; prefill
tokens/s, the HBM fractions and the roofline of the dominant kernel (the
fused RMSNorm + gate/up + SwiGLU GEMV, timed per launch with HIP events on
the stream it runs on) sit beside it, with the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0  # MI355X dense f16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(shape, pos: int, wb: dict) -> int:
    """Algorithmic bytes of one batch-1 decode token at position `pos`: every
    weight once (f16 matrices incl. the tied lm_head, f32 biases and norms)
    plus the K/V of positions 0..pos read and one position written (f32)."""
    kv_pos = shape.n_layer * 2 * shape.n_head_kv * shape.head_dim * 4
    return wb["f16"] + wb["f32"] + kv_pos * (pos + 1) + kv_pos


def gateup_bytes(shape) -> int:
    """Algorithmic bytes of one decode launch of the fused gate/up GEMV:
    2*I*H f16 weights, the f32 residual row and norm weight in, I f32 out."""
    H, I = shape.n_embd, shape.n_ff
    return 2 * I * H * 2 + H * 4 + H * 4 + I * 4


def cpu_baseline(shape, weights, prompt, n_ctx, budget_s):
    """The CPU oracle as it stands, on a bounded sample of the workload: the
    128-token prefill, then greedy decode steps until about budget_s seconds
    have passed (at least two)."""
    from threadpoolctl import threadpool_info

    from oracle import qwen2_oracle as O
    orc = O.Qwen2Oracle(O.hparams_for(shape, n_ctx), weights)
    n = len(prompt)
    t0 = time.perf_counter()
    r = orc.prefill(0, prompt, np.arange(n))
    t1 = time.perf_counter()
    tok, steps = int(r.argmax[0]), 0
    while steps < 2 or time.perf_counter() - t1 < budget_s:
        r = orc.decode([0], [tok], [n + steps])
        tok = int(r.argmax[0])
        steps += 1
    t2 = time.perf_counter()
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": steps / (t2 - t1), "unit": "tok/s", "cores": int(threads), "kind": "oracle",
        "sample": f"NumPy oracle (f32 storage, f64 sums) on the 0.5B workload: prefill of the "
                  f"{n}-token prompt then {steps} greedy decode steps at positions {n}..{n + steps - 1}",
        "prefill_tok_s": n / (t1 - t0), "seconds": t2 - t0,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import qwen2_decoder_forward_amd as q
    import qwen2_synth as syn

    wl = syn.WORKLOADS["0.5b"]
    shape = syn.MODELS[wl.model]
    n, steps_dec, n_ctx = wl.prompt_len, wl.decode_steps, wl.n_ctx
    t = time.perf_counter()
    weights = syn.make_weights(shape)
    prompt = syn.make_prompt(shape, n)
    log(f"weights drawn in {time.perf_counter() - t:.1f} s")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = q.Model(shape, weights, n_ctx=n_ctx)
    info = model.info()
    wb = syn.weight_bytes(shape)
    assert info.weight_bytes_f16 == wb["f16"] and info.weight_bytes_f32 == wb["f32"]
    stream = torch.cuda.current_stream()
    logits = torch.empty(shape.n_vocab, dtype=torch.float32, device=dev)
    ids = torch.zeros(steps_dec + 1, dtype=torch.int32, device=dev)
    pos_prompt = np.arange(n, dtype=np.int32)

    def one_step(ev=None):
        if ev:
            ev[0].record(stream)
        model.prefill(0, prompt, pos_prompt, logits, ids[0:1])
        if ev:
            ev[1].record(stream)
        for s in range(steps_dec):
            model.decode([0], ids[s:s + 1], [n + s], logits, ids[s + 1:s + 2])
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prefill_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    decode_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    step_ms = sum(e[0].elapsed_time(e[2]) for e in evs) / args.steps
    if model.sync_status() != 0:
        raise RuntimeError("device-side error flag set during the benchmark")

    # dominant kernel: fused RMSNorm + gate/up + SwiGLU GEMV (24 launches per
    # decode token).  Its average duration is measured with HIP events on the
    # stream it runs on, around 480 back-to-back launches that cycle through
    # the 24 layers (418 MB of weights, more than the 256 MB Infinity Cache,
    # so every launch streams its weights from HBM as in the decode loop).
    reps = 20 * shape.n_layer
    q.qwen2_prof_repeat(model.ctx, "gateup", 1, shape.n_layer)  # warm the launch path
    ev_k = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev_k[0].record(stream)
    q.qwen2_prof_repeat(model.ctx, "gateup", 1, reps)
    ev_k[1].record(stream)
    torch.cuda.synchronize()
    dl = reps
    gu_avg_s = ev_k[0].elapsed_time(ev_k[1]) / reps / 1e3
    gu_bytes = gateup_bytes(shape)
    achieved = gu_bytes / gu_avg_s / 1e9

    dec_bytes = sum(decode_bytes(shape, n + s, wb) for s in range(steps_dec))
    dec_gbs = dec_bytes / (decode_ms / 1e3) / 1e9
    prefill_flops = 2 * n * (shape.n_layer * (shape.n_embd * (shape.n_head + 2 * shape.n_head_kv) *
                                             shape.head_dim + shape.n_head * shape.head_dim *
                                             shape.n_embd + 3 * shape.n_embd * shape.n_ff))
    prefill_flops += 4 * shape.n_layer * shape.n_head * shape.head_dim * n * (n + 1) // 2
    prefill_flops += 2 * shape.n_vocab * shape.n_embd
    prefill_bytes = wb["f16"] + wb["f32"] + n * shape.n_layer * 2 * shape.n_head_kv * shape.head_dim * 4

    out = {
        "metric": "decode tok/s (batch 1) + prefill tok/s, 0.5B shape; % HBM/MFMA peak",
        "value": steps_dec / (decode_ms / 1e3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 weights, f32 activations and accumulation",
        "data": "synthetic",
        "config": {"workload": "Qwen2.5-0.5B shape (24 layers, hidden 896, 14/2 heads, hd 64, "
                               "FFN 4864, vocab 151936, tied), batch 1: 128-token random prompt "
                               "prefilled, then 128 greedy decode steps, n_ctx 4096",
                   "prompt": n, "decode_steps": steps_dec, "n_ctx": n_ctx, "batch": 1},
        "decode_tok_s": steps_dec / (decode_ms / 1e3),
        "decode_ms_per_token": decode_ms / steps_dec,
        "decode_hbm_gbs": dec_gbs,
        "decode_hbm_frac": dec_gbs / HBM_PEAK_GBS,
        "prefill_tok_s": n / (prefill_ms / 1e3),
        "prefill_ms": prefill_ms,
        "prefill_hbm_frac": prefill_bytes / (prefill_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "prefill_mfma_frac": prefill_flops / (prefill_ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFS,
        "wall_s_timed": wall,
        "roofline": {
            "kernel": "k_gemv<1,4,EPI_SWIGLU> (RMSNorm + gate/up + SwiGLU, decode M=1)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": None,
            "bytes_per_launch": gu_bytes, "avg_launch_us": gu_avg_s * 1e6, "launches_timed": dl,
            "timing": "HIP events around back-to-back launches cycling through the 24 layers",
        },
        "cpu_baseline": None,
    }
    log(f"prefill {out['prefill_tok_s']:.0f} tok/s ({prefill_ms:.3f} ms), decode "
        f"{out['decode_tok_s']:.1f} tok/s ({decode_ms / steps_dec * 1e3:.1f} us/token, "
        f"{dec_gbs:.0f} GB/s), gate/up GEMV {gu_avg_s * 1e6:.2f} us = {achieved:.0f} GB/s")
    model.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, weights, prompt, n_ctx, args.cpu_seconds)
        log(f"cpu oracle: {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
