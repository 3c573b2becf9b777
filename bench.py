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

`--workload` selects one of the other workloads of the same model family
(4096-token prompt, 64 sequences decoded together, the hd-128 shape); for
those the line also carries per-projection MFMA fractions of the prefill.
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

# HBM bytes per launch of the 0.5B gate/up GEMV from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes, scaled by what the counters read for a 256 MiB copy
# (profiles/qwen2.5-0.5b_gateup_gemv_hbm_traffic.md); valid only while the
# kernel source is the one the counters were taken on.
GATEUP_TRAFFIC_BYTES = 17580542
GATEUP_TRAFFIC_SRC_SHA = "27ab86829299411f"


def gateup_traffic(shape):
    import hashlib
    h = hashlib.sha256()
    for name in ("k_gemv.hip", "q2_device.h"):  # the kernel and the device helpers it inlines
        src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "qwen2_decoder_forward_amd",
                           "csrc", name)
        with open(src, "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()[:16]
    if sha != GATEUP_TRAFFIC_SRC_SHA or shape.name != "qwen2.5-0.5b":
        return None
    return GATEUP_TRAFFIC_BYTES


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def streamed_f16(shape, wb: dict, rows: int) -> int:
    """binary16 bytes a pass over `rows` token rows reads: every matrix once
    (the lm_head included), plus the `rows` gathered embedding rows.  An
    untied model's embedding table is not streamed, only its rows are
    gathered, so its V x H table is not counted."""
    table = 0 if shape.tied else shape.n_vocab * shape.n_embd * 2
    return wb["f16"] - table + rows * shape.n_embd * 2


# Decode positions from which one row's attention runs chunked, reading the
# binary16 mirror of the cache (below it: the fused kernel reads the f32 cache)
FUSED_KEYS = 512


def kv_read_bytes(shape, positions: int, rows: int, chunked: bool) -> int:
    """K/V bytes an attention reads for `rows` rows over `positions` slots
    each: binary16 mirror on the chunked path, f32 cache on the fused one."""
    el = 2 if chunked else 4
    return rows * positions * shape.n_layer * 2 * shape.n_head_kv * shape.head_dim * el


def decode_bytes(shape, pos: int, wb: dict) -> int:
    """Bytes of one batch-1 decode token at position `pos`: every streamed
    weight once (f16 matrices incl. the lm_head, the token's embedding row,
    f32 biases and norms), the K/V of positions 0..pos as the attention reads
    them (f32 cache below FUSED_KEYS positions, binary16 mirror from there),
    and one position written (f32 cache and binary16 mirror)."""
    kv_w = shape.n_layer * 2 * shape.n_head_kv * shape.head_dim * (4 + 2)
    chunked = pos + 1 > FUSED_KEYS
    return streamed_f16(shape, wb, 1) + wb["f32"] + kv_read_bytes(shape, pos + 1, 1, chunked) + kv_w


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
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {
        "value": steps / (t2 - t1), "unit": "tok/s", "cores": int(threads), "kind": "oracle",
        "cpu_model": cpu,
        "sample": f"NumPy oracle (f32 storage, f64 sums) on the 0.5B workload: prefill of the "
                  f"{n}-token prompt then {steps} greedy decode steps at positions {n}..{n + steps - 1}",
        "prefill_tok_s": n / (t1 - t0), "seconds": t2 - t0,
    }


def measure_ceilings(torch, q, dev, stream) -> dict:
    """What this device reaches, timed with HIP events in this job: a plain
    streaming read of an 8 GiB buffer (past the 256 MB Infinity Cache, so HBM;
    best of three grid sizes, three reads each; a 2 GiB buffer reads about 8 %
    slower) and a register-only f16 MFMA loop (best of three grid sizes)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps / 1e3

    nbytes = 8 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    best_read = (0.0, 0)
    for nb in (4096, 8192, 16384):
        out = torch.empty(4 * nb, dtype=torch.int32, device=dev)
        t = timed(lambda: q.qwen2_probe_read(buf, nbytes, nb, out, stream=stream.cuda_stream), 3)
        best_read = max(best_read, (nbytes / t / 1e9, nb))
    del buf
    iters = 4000
    best_mfma = (0.0, 0)
    for nb in (512, 2048, 4096):
        out = torch.empty(4 * nb, dtype=torch.float32, device=dev)
        t = timed(lambda: q.qwen2_probe_mfma(iters, nb, out, stream=stream.cuda_stream), 3)
        flops = nb * 4 * iters * 4 * 2 * 32 * 32 * 16
        best_mfma = max(best_mfma, (flops / t / 1e12, nb))
    return {
        "hbm_read_gbs": best_read[0], "hbm_read_frac_of_peak": best_read[0] / HBM_PEAK_GBS,
        "hbm_read_blocks": best_read[1], "hbm_read_bytes": nbytes,
        "mfma_f16_tflops": best_mfma[0], "mfma_frac_of_peak": best_mfma[0] / MFMA_F16_PEAK_TFS,
        "mfma_blocks": best_mfma[1],
        "how": "qwen2_probe_read (non-temporal 16-byte loads, 8 in flight per thread) and "
               "qwen2_probe_mfma (v_mfma_f32_32x32x16_f16, four accumulators per wavefront), "
               "timed with HIP events in this job",
    }


def prefill_gemm_flops(shape, n: int) -> dict:
    """Dense flops of each projection of a prefill of n rows (the last layer's
    FFN runs on the last row only) and of the lm_head on that row."""
    H, I, hd = shape.n_embd, shape.n_ff, shape.head_dim
    nq, nkv, L = shape.n_head * hd, shape.n_head_kv * hd, shape.n_layer
    return {
        "qkv": 2 * n * L * H * (nq + 2 * nkv),
        "wo": 2 * n * L * nq * H,
        "gateup": 2 * (n * (L - 1) + 1) * 2 * I * H,
        "down": 2 * (n * (L - 1) + 1) * I * H,
        "lmhead": 2 * shape.n_vocab * H,
    }


def attn_prefill_flops(shape, n: int) -> int:
    """QK^T and PV flops of causal attention over positions 0..n-1."""
    return 4 * shape.n_layer * shape.n_head * shape.head_dim * n * (n + 1) // 2


def prefill_op_fractions(q, model, shape, prompt, n_ctx):
    """Per-op MFMA fractions of one prefill, timed per launch with HIP events
    (qwen2_prof_*) in a separate untimed pass."""
    ops = ["qkv", "attn", "wo", "gateup", "down", "lmhead"]
    n = len(prompt)
    q.qwen2_prof_enable(model.ctx, ops)
    model.prefill(0, prompt, np.arange(n, dtype=np.int32), None, None)
    out = {}
    fl = prefill_gemm_flops(shape, n)
    fl["attn"] = attn_prefill_flops(shape, n)
    for op in ops:
        cnt, ms = q.qwen2_prof_read(model.ctx, op)
        if cnt:
            out[op] = {"launches": cnt, "ms": ms,
                       "tflops": fl[op] / (ms / 1e3) / 1e12,
                       "mfma_frac": fl[op] / (ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFS}
    q.qwen2_prof_enable(model.ctx, [])
    gem = [o for o in ("qkv", "wo", "gateup", "down") if o in out]
    tot_fl = sum(fl[o] for o in gem)
    tot_ms = sum(out[o]["ms"] for o in gem)
    out["linear_aggregate"] = {"ms": tot_ms, "tflops": tot_fl / (tot_ms / 1e3) / 1e12,
                               "mfma_frac": tot_fl / (tot_ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFS}
    return out


def trace_summary(path: str) -> None:
    """Prints, from a rocprofv3 kernel trace (CSV) of a bench.py run, every
    kernel's average duration over the decode steps' graph replays and, for
    a kernel also launched back to back (the roofline loop), its average
    there: a launch whose predecessor and successor are the same kernel
    belongs to the loop, any other one runs between different kernels."""
    import csv
    import statistics as st
    with open(path) as f:
        rows = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                      for r in csv.DictReader(f))
    loop, seq = {}, {}
    for i, (s0, e0, name) in enumerate(rows):
        key = name.split("(")[0].replace("void ", "")
        same = (0 < i < len(rows) - 1 and rows[i - 1][2] == name and rows[i + 1][2] == name)
        (loop if same else seq).setdefault(key, []).append((e0 - s0) / 1e3)
    print(f"{'kernel':52s} {'in sequence':>22s} {'back to back':>22s}")
    for k in sorted(seq, key=lambda k: -sum(seq[k])):
        a = seq[k]
        b = loop.get(k, [])
        bb = f"{len(b):6d} x {st.mean(b):7.2f} us" if b else ""
        print(f"{k[:52]:52s} {len(a):6d} x {st.mean(a):7.2f} us {bb:>22s}")


def counter_summary(path: str, simds: int = 1024, xcds: int = 8) -> None:
    """Prints, from a rocprofv3 --pmc counter CSV, per kernel: dispatches, the
    mean of every collected counter per dispatch and, when
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE were collected, the MFMA
    busy fraction = busy cycles summed over the SIMDs / (GUI-active cycles of
    one XCD x SIMD count; 256 CUs x 4 SIMDs on the MI355X).  rocprofv3 sums
    GRBM_GUI_ACTIVE over the 8 XCDs, so one XCD's count is that sum / 8 (the
    vendor's MfmaUtil metric takes the largest XCD's).  The f16 MFMA flop
    count is SQ_INSTS_VALU_MFMA_MOPS_F16 x 512."""
    import csv
    import collections
    per = collections.defaultdict(dict)
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = r["Dispatch_Id"]
            per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            names[d] = r["Kernel_Name"].split("(")[0].replace("void ", "")
    groups = collections.defaultdict(list)
    for d, c in per.items():
        groups[names[d]].append(c)
    counters = sorted({k for c in per.values() for k in c})
    print(f"{'kernel':48s} {'disp':>5s} " + " ".join(f"{c[:26]:>26s} {'(max)':>12s}" for c in counters)
          + f" {'MFMA busy':>9s} {'f16 MFMA GFLOP':>14s}")
    for k in sorted(groups, key=lambda k: -sum(c.get("GRBM_GUI_ACTIVE", 0) for c in groups[k])):
        g = groups[k]
        mean = {c: sum(x.get(c, 0.0) for x in g) / len(g) for c in counters}
        mx = {c: max(x.get(c, 0.0) for x in g) for c in counters}
        util = ""
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("GRBM_GUI_ACTIVE"):
            util = (f"{100 * mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (mean['GRBM_GUI_ACTIVE'] / xcds * simds):8.1f}%")
        fl = ""
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in mean:
            fl = f"{mean['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512 / 1e9:14.2f}"
        print(f"{k[:48]:48s} {len(g):5d} " + " ".join(f"{mean[c]:26.6g} {mx[c]:12.6g}" for c in counters)
              + f" {util:>9s} {fl:>14s}")


def pmc_pass(torch, q, syn):
    """Launches for the HBM traffic counters: torch's copy of a 256 MiB tensor
    (every byte read once and written once: the calibration of FETCH_SIZE and
    WRITE_SIZE), then 48 launches of the decode gate/up GEMV on the 0.5B shape
    (two per layer, so 418 MB of weights > the 256 MB Infinity Cache)."""
    shape = syn.MODELS["qwen2.5-0.5b"]
    torch.cuda.set_device(0)
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    weights = syn.make_weights(shape)
    model = q.Model(shape, weights, n_ctx=256)
    q.qwen2_prof_repeat(model.ctx, "gateup", 1, 2 * shape.n_layer)
    torch.cuda.synchronize()
    model.close()
    log(f"pmc pass: copy of {src.numel() * 4} bytes, {2 * shape.n_layer} gate/up launches "
        f"of {gateup_bytes(shape)} algorithmic bytes")


def library_gemms(torch, syn, wl_name: str) -> None:
    """For comparison only: the prefill projections of a workload as plain
    library products (torch.matmul through hipBLASLt, f16 operands, no fused
    bias / RoPE / SwiGLU / residual epilogues), timed with HIP events; prints
    each shape's time and its share of the 2.5 PFLOP/s dense f16 peak."""
    wl = syn.WORKLOADS[wl_name]
    shape = syn.MODELS[wl.model]
    M, H, I = wl.prompt_len, shape.n_embd, shape.n_ff
    nq, nkv = shape.n_head * shape.head_dim, shape.n_head_kv * shape.head_dim
    shapes = {"qkv": (M, nq + 2 * nkv, H), "wo": (M, H, nq), "gateup": (M, 2 * I, H), "down": (M, H, I)}
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda").manual_seed(0)
    tot_fl = tot_us = 0.0
    for name, (m, n, k) in shapes.items():
        a = torch.randn(m, k, device="cuda", dtype=torch.float16, generator=g)
        w = torch.randn(n, k, device="cuda", dtype=torch.float16, generator=g)
        wt = w.t()
        for _ in range(3):
            c = a @ wt
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            c = a @ wt
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        fl = 2.0 * m * n * k
        tot_fl += fl
        tot_us += us
        log(f"[{wl_name}] library {name} {m} x {n} x {k}: {us:.1f} us, "
            f"{fl / us / 1e6:.0f} TFLOP/s = {100 * fl / us / 1e6 / MFMA_F16_PEAK_TFS:.1f} % of peak")
        del a, w, wt, c
    log(f"[{wl_name}] library projections together: {tot_us:.1f} us, "
        f"{100 * tot_fl / tot_us / 1e6 / MFMA_F16_PEAK_TFS:.1f} % of peak")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="0.5b",
                    help="0.5b (the benchmark line, default), 0.5b-long, 0.5b-batched, hd128, 1.5b-heads, tiny")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarise a rocprofv3 kernel trace of this script (no GPU use)")
    ap.add_argument("--counter-summary", metavar="CSV",
                    help="summarise a rocprofv3 --pmc counter CSV of this script (no GPU use)")
    ap.add_argument("--library-gemms", action="store_true",
                    help="only time the workload's prefill projections as plain torch.matmul "
                         "products (hipBLASLt), for comparison")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="only the launches a rocprofv3 --pmc counter pass reads: a plain 256 MiB "
                         "device copy (calibration), then 48 launches of the gate/up GEMV")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this implementation runs on one GPU; --gpus must be 1 "
                                   "(figures for several GPUs are not produced)"}))
        sys.exit(2)

    import torch

    import qwen2_decoder_forward_amd as q
    import qwen2_synth as syn

    if args.pmc_pass:
        pmc_pass(torch, q, syn)
        return
    if args.library_gemms:
        library_gemms(torch, syn, args.workload)
        return

    wl = syn.WORKLOADS[args.workload]
    shape = syn.MODELS[wl.model]
    n, steps_dec, n_ctx, n_seq = wl.prompt_len, wl.decode_steps, wl.n_ctx, wl.n_seq
    batched = n_seq > 1
    t = time.perf_counter()
    weights = syn.make_weights(shape)
    prompt = syn.make_prompt(shape, n)
    log(f"[{wl.name}] weights drawn in {time.perf_counter() - t:.1f} s")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = q.Model(shape, weights, n_ctx=n_ctx, n_seq=n_seq)
    info = model.info()
    wb = syn.weight_bytes(shape)
    assert info.weight_bytes_f16 == wb["f16"] and info.weight_bytes_f32 == wb["f32"]
    stream = torch.cuda.current_stream()
    V = shape.n_vocab
    pos_prompt = np.arange(n, dtype=np.int32)

    if batched:
        # setup (outside the decode timing): every sequence slot holds a
        # prefix of n tokens, written one sequence per call and by one
        # batched call, each twice (the same values, up to rounding order)
        prompts = [syn.make_prompt(shape, n, 100 + j) for j in range(n_seq)]
        seqs = list(range(n_seq))
        setup = {}
        for kind in ("per_sequence", "batched") * 2:  # the second round counts
            torch.cuda.synchronize()
            t_setup = time.perf_counter()
            if kind == "batched":
                model.prefill_batch(seqs, prompts, [pos_prompt] * n_seq)
            else:
                for j in range(n_seq):
                    model.prefill(j, prompts[j], pos_prompt, None, None)
            torch.cuda.synchronize()
            setup[kind] = n_seq * n / (time.perf_counter() - t_setup)
        log(f"[{wl.name}] {n_seq} prefixes of {n} tokens prefilled: "
            f"{setup['per_sequence']:.0f} tok/s one sequence per call, "
            f"{setup['batched']:.0f} tok/s in one batched call")
        toks = torch.tensor(syn.make_prompt(shape, n_seq, 999), dtype=torch.int32, device=dev)
        logits = torch.empty((n_seq, V), dtype=torch.float32, device=dev)
        ids = torch.zeros(n_seq, dtype=torch.int32, device=dev)

        def one_step(ev=None):
            if ev:
                ev[0].record(stream)
                ev[1].record(stream)
            model.decode(seqs, toks, [n] * n_seq, logits, ids)
            if ev:
                ev[2].record(stream)
    else:
        logits = torch.empty(V, dtype=torch.float32, device=dev)
        ids = torch.zeros(steps_dec + 1, dtype=torch.int32, device=dev)

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

    if batched:  # (more than 8 rows: the chunked attention over the binary16 mirror)
        dec_tokens = n_seq
        kv_w = shape.n_layer * 2 * shape.n_head_kv * shape.head_dim * (4 + 2)
        dec_bytes = (streamed_f16(shape, wb, n_seq) + wb["f32"] +
                     kv_read_bytes(shape, n + 1, n_seq, True) + n_seq * kv_w)
    else:
        dec_tokens = steps_dec
        dec_bytes = sum(decode_bytes(shape, n + s, wb) for s in range(steps_dec))
    dec_gbs = dec_bytes / (decode_ms / 1e3) / 1e9
    dec_tok_s = dec_tokens / (decode_ms / 1e3)

    # dominant decode kernel: fused RMSNorm + gate/up + SwiGLU GEMV (one launch
    # per layer and token).  Its average duration is measured live with HIP
    # events on the stream it runs on, around 20 back-to-back launches per
    # layer that cycle through the layers (on the 0.5B shape 418 MB of
    # weights, more than the 256 MB Infinity Cache, so every launch streams
    # its weights from HBM).  Inside the decode graph the same kernel runs
    # between other kernels; HIP events cannot bracket a node of a graph
    # replay (an event pair around every direct launch adds its own cost),
    # so that figure comes from a rocprofv3 kernel trace of this command,
    # split by `--trace-summary` into the graph replays and this loop.
    reps = 20 * shape.n_layer
    q.qwen2_prof_repeat(model.ctx, "gateup", 1, shape.n_layer)  # warm the launch path
    ev_k = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev_k[0].record(stream)
    q.qwen2_prof_repeat(model.ctx, "gateup", 1, reps)
    ev_k[1].record(stream)
    torch.cuda.synchronize()
    gu_avg_s = ev_k[0].elapsed_time(ev_k[1]) / reps / 1e3
    gu_bytes = gateup_bytes(shape)
    achieved = gu_bytes / gu_avg_s / 1e9
    kc = -(-shape.n_embd // 512)
    kb = 2 if kc <= 2 else 4 if kc <= 4 else 8 if kc <= 8 else 10

    # next_token_probs of the read-out rows (softmax over the vocabulary):
    # average of 100 back-to-back calls on the last step's logits
    prob_rows = n_seq if batched else 1
    probs = torch.empty((prob_rows, V), dtype=torch.float32, device=dev)
    model.next_token_probs(logits, prob_rows, probs)
    torch.cuda.synchronize()
    ev_k[0].record(stream)
    for _ in range(100):
        model.next_token_probs(logits, prob_rows, probs)
    ev_k[1].record(stream)
    torch.cuda.synchronize()
    probs_us = ev_k[0].elapsed_time(ev_k[1]) / 100 * 1e3

    ceil = measure_ceilings(torch, q, dev, stream)

    fl = prefill_gemm_flops(shape, n)
    prefill_flops = sum(fl.values()) + attn_prefill_flops(shape, n)
    # (weights once, the prompt's K/V written: f32 cache and binary16 mirror)
    prefill_bytes = (streamed_f16(shape, wb, n) + wb["f32"] +
                     n * shape.n_layer * 2 * shape.n_head_kv * shape.head_dim * (4 + 2))

    desc = (f"{wl.description}; model {shape.name}: {shape.n_layer} layers, hidden "
            f"{shape.n_embd}, {shape.n_head}/{shape.n_head_kv} heads, hd {shape.head_dim}, "
            f"FFN {shape.n_ff}, vocab {shape.n_vocab}, {'tied' if shape.tied else 'untied'}")
    out = {
        "metric": "decode tok/s (batch 1) + prefill tok/s, 0.5B shape; % HBM/MFMA peak",
        "value": dec_tok_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f16 weights; decode (rows <= 8): f32 activations, accumulation and KV "
                  "cache, except that attention from position 512 on reads the binary16 K/V "
                  "mirror (binary16 query and softmax-weight MFMA operands, f32 accumulation); "
                  "prefill and batched decode (rows > 8): f16 activation, K/V-mirror and "
                  "softmax-weight MFMA operands with f32 accumulation, f32 residual stream and "
                  "KV cache"),
        "data": "synthetic",
        "config": {"workload": desc, "prompt": n, "decode_steps": steps_dec, "n_ctx": n_ctx,
                   "batch": n_seq},
        "decode_tok_s": dec_tok_s,
        "decode_ms_per_step": decode_ms / (1 if batched else steps_dec),
        "decode_hbm_gbs": dec_gbs,
        "decode_hbm_frac": dec_gbs / HBM_PEAK_GBS,
        "decode_hbm_frac_of_ceiling": dec_gbs / ceil["hbm_read_gbs"],
        "wall_s_timed": wall,
        "next_token_probs_us": probs_us,
        "next_token_probs_rows": prob_rows,
        "roofline": {
            "kernel": f"k_gemv1<2, {kb}, 2> (RMSNorm + gate/up + SwiGLU, decode M=1)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": gateup_traffic(shape),
            "measured_ceiling": ceil["hbm_read_gbs"],
            "frac_of_ceiling": achieved / ceil["hbm_read_gbs"],
            "bytes_per_launch": gu_bytes, "avg_launch_us": gu_avg_s * 1e6, "launches_timed": reps,
            "timing": "HIP events around back-to-back launches cycling through the layers "
                      "(the in-graph duration: rocprofv3 trace, bench.py --trace-summary)",
        },
        "ceilings": ceil,
        "cpu_baseline": None,
    }
    if batched:
        out["setup_prefill_tok_s"] = setup
    if not batched:
        out["prefill_tok_s"] = n / (prefill_ms / 1e3)
        out["prefill_ms"] = prefill_ms
        out["prefill_hbm_frac"] = prefill_bytes / (prefill_ms / 1e3) / 1e9 / HBM_PEAK_GBS
        out["prefill_mfma_frac"] = prefill_flops / (prefill_ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFS
        out["prefill_mfma_frac_of_ceiling"] = (prefill_flops / (prefill_ms / 1e3) / 1e12 /
                                               ceil["mfma_f16_tflops"])
        if n > 8:
            # a fresh context, so the prefill runs on an empty cache as above
            model.close()
            model = q.Model(shape, weights, n_ctx=n_ctx, n_seq=n_seq)
            out["prefill_ops"] = prefill_op_fractions(q, model, shape, prompt, n_ctx)
        log(f"[{wl.name}] prefill {out['prefill_tok_s']:.0f} tok/s ({prefill_ms:.3f} ms, "
            f"{out['prefill_mfma_frac'] * 100:.1f}% MFMA)")
    log(f"[{wl.name}] decode {dec_tok_s:.1f} tok/s ({decode_ms:.3f} ms, {dec_gbs:.0f} GB/s), "
        f"gate/up GEMV {gu_avg_s * 1e6:.2f} us = {achieved:.0f} GB/s")
    log(f"[{wl.name}] ceilings: HBM read {ceil['hbm_read_gbs']:.0f} GB/s "
        f"({ceil['hbm_read_frac_of_peak'] * 100:.1f}% of peak), f16 MFMA "
        f"{ceil['mfma_f16_tflops']:.0f} TFLOP/s ({ceil['mfma_frac_of_peak'] * 100:.1f}% of peak)")
    log(f"[{wl.name}] next_token_probs of {prob_rows} row(s) x {V}: {probs_us:.2f} us "
        f"({8 * V * prob_rows / (probs_us * 1e3):.0f} GB/s of logits in + probabilities out)")
    if "prefill_ops" in out:
        log(f"[{wl.name}] prefill ops: " + ", ".join(
            f"{k} {v['mfma_frac'] * 100:.1f}%" for k, v in out["prefill_ops"].items()))
    model.close()
    if not args.no_cpu_baseline and wl.name == "0.5b":
        out["cpu_baseline"] = cpu_baseline(shape, weights, prompt, n_ctx, args.cpu_seconds)
        log(f"cpu oracle: {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
