#!/usr/bin/env python3
"""Benchmark of the Maglev attention + recurrent K/V injection path on one MI355X.

One step = one lifted-training pass of one d20 decoder-P layer over the batch
(B=8, T=2048, W=512, d=1280, 10 heads x 128, bf16, fp32 accumulation):
memory projection of the shifted targets -> injected sliding-window attention
forward -> memory-consistency loss (lambda 0.1) -> backward of the whole layer
path (dq, dk, dv, dm', dW_Km, dW_Vm, dgate). Inputs are synthetic, seeded and
resident in HBM before the timed region. The recurrent decode of the same
stack shape (64 streams x 20 layers, W=512 ring, 4096 steps, one HIP graph per
step) is measured in the same run and reported in its own object.

Prints ONE JSON line. `--gpus N` with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import recurrent_memory_sliding_amd as rms  # noqa: E402
import workloads as wl  # noqa: E402
from recurrent_memory_sliding_amd.decode import DecodeStack  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def layer_flops(sh: wl.LayerShape) -> dict:
    """Algorithmic FLOPs of one layer pass: in-window (i, j) pairs only, the
    projection GEMMs counted, elementwise work not counted; the attention
    backward counts 4 contractions (dV, dP, dQ, dK)."""
    T, W, B, H, Dh, d = sh.T, sh.W, sh.B, sh.H, sh.Dh, sh.d
    pairs = sum(min(i + 1, W) for i in range(T))           # per (b, h)
    attn_unit = 2.0 * pairs * Dh * B * H                     # one contraction
    proj_unit = 2.0 * B * T * d * (2 * H * Dh)               # one [N x d] x [d x 2HD] product
    return {
        "project_fwd": proj_unit,
        "attn_fwd": 2 * attn_unit,
        "attn_bwd": 4 * attn_unit,
        "project_bwd": 2 * proj_unit,
    }


def decode_bytes(sh: wl.DecodeShape) -> float:
    """Algorithmic HBM bytes of one decode step (all layers): the W-1 older ring
    slots of K and V read, the new slot written, projection weights read,
    q/k/v read, kmem/vmem written and read, memory read, output written."""
    e = 2 if sh.dtype == wl.BF16 else 4
    Bs, H, Dh, W, d = sh.Bs, sh.H, sh.Dh, sh.W, sh.d
    per_layer = (2 * Bs * H * (W - 1) * Dh * e          # ring reads
                 + 2 * Bs * H * Dh * e                   # new-slot writes
                 + 2 * H * Dh * d * e                    # W_Km, W_Vm
                 + 3 * Bs * H * Dh * e                   # q, k, v
                 + 4 * Bs * H * Dh * e                   # kmem, vmem write + read
                 + Bs * d * e                            # memory read by the projection
                 + Bs * H * Dh * e)                      # output
    return float(per_layer * sh.layers)


class Timer:
    """HIP events around each call on the launching stream."""

    def __init__(self):
        self.ev = {}

    def mark(self, name):
        s = torch.cuda.Event(enable_timing=True)
        s.record(torch.cuda.current_stream())
        return s

    def add(self, name, start):
        e = torch.cuda.Event(enable_timing=True)
        e.record(torch.cuda.current_stream())
        self.ev.setdefault(name, []).append((start, e))

    def avg_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.ev.items()}


def train_setup(sh, seed=2):
    inp = wl.layer_inputs(sh, seed, grads=True)
    g = {k: v.cuda() for k, v in inp.items()}
    dev = "cuda"
    B, T, H, Dh, d = sh.B, sh.T, sh.H, sh.Dh, sh.d
    bf = torch.bfloat16
    f32 = torch.float32
    buf = {
        "km": torch.empty((B, T, H, Dh), dtype=bf, device=dev),
        "vm": torch.empty((B, T, H, Dh), dtype=bf, device=dev),
        "kx": torch.empty((B, T, H, Dh), dtype=bf, device=dev),
        "vx": torch.empty((B, T, H, Dh), dtype=bf, device=dev),
        "o": torch.empty((B, T, H, Dh), dtype=bf, device=dev),
        "lse": torch.empty((B, H, T), dtype=f32, device=dev),
        "loss": torch.empty((1,), dtype=f32, device=dev),
        "dm": torch.empty((B, T, d), dtype=f32, device=dev),
        "grads": {
            "dq": torch.empty((B, T, H, Dh), dtype=bf, device=dev),
            "dk": torch.empty((B, T, H, Dh), dtype=bf, device=dev),
            "dv": torch.empty((B, T, H, Dh), dtype=bf, device=dev),
            "dm_prime": torch.empty((B, T, d), dtype=f32, device=dev),
            "dW_Km": torch.empty((H * Dh, d), dtype=f32, device=dev),
            "dW_Vm": torch.empty((H * Dh, d), dtype=f32, device=dev),
            "dgate": torch.empty((H,), dtype=f32, device=dev),
        },
    }
    buf["ws_bwd"] = torch.empty((rms.maglev_swa_inject_bwd_workspace(B, T, H, Dh, d, sh.W),),
                                dtype=torch.uint8, device=dev)
    buf["ws_loss"] = torch.empty((rms.maglev_consistency_loss_workspace(B * T, d),),
                                 dtype=torch.uint8, device=dev)
    rms.maglev_prepare(Dh, sh.rope_base, T)
    return g, buf


def train_step(sh, g, buf, timer=None):
    def run(name, fn):
        if timer is None:
            fn()
        else:
            s = timer.mark(name)
            fn()
            timer.add(name, s)

    run("maglev_mem_project", lambda: rms.maglev_mem_project(
        g["m_prime"], g["W_Km"], g["W_Vm"], sh.H, sh.Dh, shift=1, kmem=buf["km"], vmem=buf["vm"],
        k=g["k"], v=g["v"], gate_logit=g["gate_logit"], kmix=buf["kx"], vmix=buf["vx"],
        pos0=sh.pos0, rope_base=sh.rope_base))
    run("maglev_swa_inject_fwd", lambda: rms.maglev_swa_inject_fwd(
        g["q"], buf["kx"], buf["vx"], sh.W, pos0=sh.pos0, rope_base=sh.rope_base, d=sh.d,
        o=buf["o"], lse=buf["lse"]))
    # the backward writes dm'; the loss then adds its own term (accumulate bit 1)
    run("maglev_swa_inject_bwd", lambda: rms.maglev_swa_inject_bwd(
        g["q"], buf["kx"], buf["vx"], buf["km"], buf["vm"], g["gate_logit"], buf["o"], buf["lse"],
        g["dO"], g["m_prime"], g["W_Km"], g["W_Vm"], sh.W, pos0=sh.pos0, rope_base=sh.rope_base,
        accumulate=0, out=buf["grads"], workspace=buf["ws_bwd"]))
    run("maglev_consistency_loss", lambda: rms.maglev_consistency_loss(
        g["m"], g["m_prime"], sh.lam, loss=buf["loss"], dm=buf["dm"],
        dm_prime=buf["grads"]["dm_prime"], accumulate=2, workspace=buf["ws_loss"]))


def bench_train(sh, steps, warmup):
    g, buf = train_setup(sh)
    for _ in range(warmup):
        train_step(sh, g, buf)
    torch.cuda.synchronize()
    timer = Timer()
    t0 = time.perf_counter()
    for _ in range(steps):
        train_step(sh, g, buf, timer)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    calls = timer.avg_ms()
    del g, buf
    torch.cuda.empty_cache()
    return ms, calls


def bench_decode(sh, steps, warmup, seed=4):
    params = [wl.decode_layer_params(sh, seed, l) for l in range(sh.layers)]
    weights = [{"W_Km": p["W_Km"].cuda(), "W_Vm": p["W_Vm"].cuda(),
                "gate_logit": p["gate_logit"].cuda()} for p in params]
    kc = [p["kcache"].cuda() for p in params]
    vc = [p["vcache"].cuda() for p in params]
    pools = [(p["q_pool"].cuda(), p["k_pool"].cuda(), p["v_pool"].cuda()) for p in params]
    del params
    stack = DecodeStack(weights, kc, vc, torch.full((sh.Bs,), sh.W, dtype=torch.int64, device="cuda"),
                        wl.decode_initial_memory(sh, seed).cuda(), rope_base=sh.rope_base)
    # one graph per pool entry: step t replays graph t mod 16, bound to that entry's q/k/v
    def qkv(e):
        return ([p[0][e] for p in pools], [p[1][e] for p in pools], [p[2][e] for p in pools])

    stack.step(*qkv(0))               # eager step: initialises everything before capture
    for e in range(sh.pool):
        stack.capture(e, *qkv(e))
    t_step = 1
    for _ in range(warmup):
        stack.replay(t_step % sh.pool); t_step += 1
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        stack.replay(t_step % sh.pool); t_step += 1
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del stack, weights, kc, vc, pools
    torch.cuda.empty_cache()
    return ms


def cpu_baseline(sh):
    """The oracle, as it stands, on a bounded slice of the training workload:
    sequences 0-3 of 8, all heads, full T. The slice is half of the layer's
    attention pairs and projection rows, so the full-step time is scaled by 2."""
    import oracle

    oracle.build(force=False)
    inp = wl.layer_inputs(sh, 2, grads=True)
    nb = 4
    nh = sh.H
    Dh = sh.Dh
    sl = {n: inp[n][:nb, :, :nh].contiguous() for n in ("q", "k", "v", "dO")}
    sl["m_prime"] = inp["m_prime"][:nb].contiguous()
    sl["m"] = inp["m"][:nb].contiguous()
    sl["W_Km"] = inp["W_Km"][: nh * Dh].contiguous()
    sl["W_Vm"] = inp["W_Vm"][: nh * Dh].contiguous()
    sl["gate_logit"] = inp["gate_logit"][:nh].contiguous()
    t0 = time.perf_counter()
    km, vm = oracle.mem_project(sl["m_prime"], sl["W_Km"], sl["W_Vm"], nh, Dh, shift=1)
    oracle.swa_inject_fwd(sl["q"], sl["k"], sl["v"], km, vm, sl["gate_logit"], sh.W)
    oracle.consistency_loss(sl["m"], sl["m_prime"], sh.lam)
    oracle.swa_inject_bwd(sl["q"], sl["k"], sl["v"], sl["m_prime"], sl["W_Km"], sl["W_Vm"],
                          sl["gate_logit"], sl["dO"], sh.W)
    dt = time.perf_counter() - t0
    factor = sh.B * sh.H / (nb * nh)
    full_s = dt * factor
    return {
        "value": sh.B * sh.T / full_s,
        "unit": "tokens/s",
        "cores": oracle.omp_threads(),
        "kind": "oracle",
        "sample": "sequences 0-3 (all heads) of the d20 layer fwd+bwd+loss (T=2048, W=512): "
                  "%.1f s, scaled by %g to the full batch" % (dt, factor),
        "sample_seconds": round(dt, 2),
        "cpu": platform.processor() or platform.machine(),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=wl.D20_DECODE.steps)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    rms.lib()   # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)

    sh = wl.D20_LAYER
    flops = layer_flops(sh)
    total_flops = sum(flops.values())
    ms, calls = bench_train(sh, args.steps, args.warmup)
    tokens = sh.B * sh.T
    value = tokens / (ms / 1e3)
    path_tflops = total_flops / (ms / 1e3) / 1e12

    # roofline of the single-kernel call with the largest time
    per_call_flops = {"maglev_mem_project": flops["project_fwd"],
                      "maglev_swa_inject_fwd": flops["attn_fwd"]}
    dom = max(per_call_flops, key=lambda k: calls.get(k, 0.0))
    dom_tflops = per_call_flops[dom] / (calls[dom] / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(dom_tflops, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None}

    result = {
        "metric": "SWA+KV-inject fwd+bwd tokens/s & %bf16 MFMA peak (d20,T=2048,W=512); decode GB/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/d) weights)",
        "config": {"workload": "d20 decoder-P layer fwd+bwd + consistency loss",
                   "B": sh.B, "T": sh.T, "W": sh.W, "d_model": sh.d, "heads": sh.H,
                   "head_dim": sh.Dh, "lambda": sh.lam, "global_batch": sh.B, "seq_len": sh.T,
                   "parallelism": "single GPU"},
        "path": {"algorithmic_TFLOP_per_step": round(total_flops / 1e12, 4),
                 "TFLOP/s": round(path_tflops, 1),
                 "frac_bf16_peak": round(path_tflops / PEAK_BF16_TFLOPS, 4),
                 "calls_ms": {k: round(v, 4) for k, v in calls.items()}},
        "roofline": roofline,
    }
    if not args.no_decode:
        dsh = wl.D20_DECODE
        dms = bench_decode(dsh, args.decode_steps, 5)
        dbytes = decode_bytes(dsh)
        gbs = dbytes / (dms / 1e3) / 1e9
        result["decode"] = {
            "workload": "recurrent decode, 20 layers, 64 streams, W=512 bf16 ring, 10x128 heads",
            "steps": args.decode_steps, "ms_per_step": round(dms, 4),
            "tokens/s": round(dsh.Bs / (dms / 1e3), 1),
            "algorithmic_GB_per_step": round(dbytes / 1e9, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
            "graph": "one HIP graph per step (20 x (projection + decode + combine) + advance)",
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sh)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
