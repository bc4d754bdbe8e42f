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
import hashlib
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


def kernel_work(sh: wl.LayerShape, mix: str = "sigma") -> dict:
    """Algorithmic work of one launch of each kernel of the training step:
    {timing name: (FLOPs, HBM bytes)}. FLOPs count in-window pairs and the
    projection products only; bytes count each tensor the kernel must read or
    write once (bf16 activations, fp32 lse/D/gradients). mix = "gated": the
    gated form's kernels (dK/dV then writes the entry gradients only)."""
    T, W, B, H, Dh, d = sh.T, sh.W, sh.B, sh.H, sh.Dh, sh.d
    N, HD = B * T, H * Dh
    pairs = sum(min(i + 1, W) for i in range(T))
    attn = 2.0 * pairs * Dh * B * H          # one contraction over the band
    proj = 2.0 * N * d * 2 * HD              # one [N x d] x [d x 2HD] product
    act = 2.0 * N * HD                       # one bf16 activation tensor [B,T,H,Dh]
    rowf = 4.0 * N * H                       # one fp32 [B,H,T] vector
    mem = 2.0 * N * d                        # one bf16 [B,T,d] tensor
    wts = 2.0 * 2 * HD * d                   # W_Km and W_Vm, bf16
    f32nd = 4.0 * N * d
    gblocks = max(1, -(-N // max(8, -(-N // 512))))
    gpart = 4.0 * gblocks * 4 * HD                         # fp32 gate partials
    # dQ from the dS tiles the dK/dV pass stores (Dh = 128): the band of dS
    # (bf16), K~ and dq; else the recomputing pass (q^, dO, K~, V~ -> dq)
    dq_bytes = (2 * act + 2.0 * pairs * B * H) if Dh == 128 else (5 * act + 2 * rowf)
    if mix == "gated":
        return {
            "proj_fwd": (proj, mem + wts + 2 * act),
            "gated_mix": (0.0, 6 * act),                       # k v kp vm -> kmix vmix
            "attn_fwd": (2 * attn, 4 * act + rowf),
            "attn_bwd_prep": (0.0, 4 * act + 3 * rowf),
            "attn_bwd_dkdv": (3 * attn, 6 * act + 2 * rowf),   # q^ dO kmix vmix -> dk~ dv~
            "attn_bwd_dq": (attn, dq_bytes),
            "gated_mix_bwd": (0.0, 10 * act + gpart),          # dk~ dv~ k v kp vm -> dk dv dkp dvm
            "gate_grad_reduce": (0.0, gpart + 2 * 4.0 * 4 * HD),
            "proj_bwd_scale_w": (0.0, 2 * wts),
            "proj_bwd_dm": (proj, 2 * act + wts + f32nd),
            "proj_bwd_dw": (proj, 2 * act + mem),
            "proj_bwd_dw_reduce": (0.0, 4.0 * 2 * HD * d * 2),
            "loss_partial": (0.0, 2 * mem + f32nd + 2 * f32nd),
        }
    return {
        "proj_fwd": (proj, mem + wts + 2 * act),
        "mix": (0.0, 6 * act),                                  # k v kmem vmem -> kmix vmix
        "attn_fwd": (2 * attn, 4 * act + rowf),                 # q kmix vmix -> o, lse
        "attn_bwd_prep": (0.0, 4 * act + 3 * rowf),             # o dO q lse -> D, qr, lse2
        "attn_bwd_dkdv": (3 * attn, 6 * act + 2 * rowf),       # q^ dO kmix vmix -> dk dv
        "attn_bwd_dq": (attn, dq_bytes),
        "proj_bwd_scale_w": (0.0, 2 * wts),
        "proj_bwd_dm": (proj, 2 * act + wts + f32nd),           # dk dv Ws -> dm'
        "proj_bwd_dw": (proj, 2 * act + mem),                   # partials counted separately
        "proj_bwd_dw_reduce": (0.0, 4.0 * 2 * HD * d * 2 + wts),  # G -> dW, row dots with W
        "loss_partial": (0.0, 2 * mem + f32nd + 2 * f32nd),     # m m' -> dm, dm' +=
    }


CALL_KERNELS = {
    "maglev_mem_project": ("proj_fwd", "mix"),
    "maglev_swa_inject_fwd": ("attn_fwd",),
    "maglev_swa_inject_bwd": ("attn_bwd_prep", "attn_bwd_dkdv", "attn_bwd_dq", "dgate_reduce",
                              "zero_last_rows", "proj_bwd_scale_w", "proj_bwd_dm", "proj_bwd_dw",
                              "proj_bwd_dw_reduce"),
    "maglev_consistency_loss": ("loss_partial", "loss_final"),
}
CALL_KERNELS_GATED = {
    "maglev_mem_project_gated": ("proj_fwd", "gated_mix"),
    "maglev_swa_inject_fwd": ("attn_fwd",),
    "maglev_swa_inject_bwd_gated": ("attn_bwd_prep", "attn_bwd_dkdv", "attn_bwd_dq",
                                    "gated_mix_bwd", "gate_grad_reduce", "proj_bwd_scale_w",
                                    "proj_bwd_dm", "proj_bwd_dw", "proj_bwd_dw_reduce"),
    "maglev_consistency_loss": ("loss_partial", "loss_final"),
}


def roofline_of(flops, nbytes, seconds):
    """Roofline record of one kernel: bound by whichever of MFMA time and HBM
    time is larger at peak, achieved rate in that unit."""
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        a = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(a, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / PEAK_BF16_TFLOPS, 4)}
    a = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBS, 4)}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` (or per step, for a record that spans
    several kernels) from the committed counter runs
    (profiles/pmc_traffic.json), or None when they are missing or were taken
    on a different source of any kernel the record covers."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][kernel]
        sources = rec["sources"] if "sources" in rec else [rec["source"]]
        want = rec["source_sha256"] if "sources" in rec else [rec["source_sha256"]]
        for name, sha_rec in zip(sources, want):
            src = os.path.join(ROOT, "recurrent_memory_sliding_amd", "csrc", name)
            with open(src, "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != sha_rec:
                    return None
    except (OSError, KeyError, ValueError, TypeError):
        return None
    return float(rec["fetch_bytes"]) + float(rec["write_bytes"])


def train_setup(sh, seed=2, mix="sigma"):
    inp = wl.layer_inputs(sh, seed, grads=True)
    g = {k: v.cuda() for k, v in inp.items()}
    if mix == "gated":
        gv = wl.gate_vectors(sh.H, sh.Dh, seed)
        g["gates"] = torch.stack([gv[n] for n in rms.GATE_NAMES]).float().cuda()
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
    wsq = (rms.maglev_swa_inject_bwd_gated_workspace if mix == "gated"
           else rms.maglev_swa_inject_bwd_workspace)
    buf["ws_bwd"] = torch.empty((wsq(B, T, H, Dh, d, sh.W),), dtype=torch.uint8, device=dev)
    if mix == "gated":
        del buf["grads"]["dgate"]
        buf["grads"]["dgates"] = torch.empty((4, H * Dh), dtype=f32, device=dev)
    buf["ws_loss"] = torch.empty((rms.maglev_consistency_loss_workspace(B * T, d),),
                                 dtype=torch.uint8, device=dev)
    rms.maglev_prepare(Dh, sh.rope_base, T)
    return g, buf


def train_step_gated(sh, g, buf):
    """The same step with the gated form (channel-wise 2 sigmoid gates, RMSNorm
    on the projected memory key)."""
    rms.maglev_mem_project_gated(
        g["m_prime"], g["W_Km"], g["W_Vm"], sh.H, sh.Dh, g["k"], g["v"], g["gates"],
        pos0=sh.pos0, rope_base=sh.rope_base, kproj=buf["km"], vmem=buf["vm"], kmix=buf["kx"],
        vmix=buf["vx"])
    rms.maglev_swa_inject_fwd(
        g["q"], buf["kx"], buf["vx"], sh.W, pos0=sh.pos0, rope_base=sh.rope_base, d=sh.d,
        o=buf["o"], lse=buf["lse"])
    rms.maglev_swa_inject_bwd_gated(
        g["q"], buf["kx"], buf["vx"], g["k"], g["v"], buf["km"], buf["vm"], g["gates"], buf["o"],
        buf["lse"], g["dO"], g["m_prime"], g["W_Km"], g["W_Vm"], sh.W, pos0=sh.pos0,
        rope_base=sh.rope_base, accumulate=0, out=buf["grads"], workspace=buf["ws_bwd"])
    rms.maglev_consistency_loss(
        g["m"], g["m_prime"], sh.lam, loss=buf["loss"], dm=buf["dm"],
        dm_prime=buf["grads"]["dm_prime"], accumulate=2, workspace=buf["ws_loss"])


def train_step(sh, g, buf):
    rms.maglev_mem_project(
        g["m_prime"], g["W_Km"], g["W_Vm"], sh.H, sh.Dh, shift=1, kmem=buf["km"], vmem=buf["vm"],
        k=g["k"], v=g["v"], gate_logit=g["gate_logit"], kmix=buf["kx"], vmix=buf["vx"],
        pos0=sh.pos0, rope_base=sh.rope_base)
    rms.maglev_swa_inject_fwd(
        g["q"], buf["kx"], buf["vx"], sh.W, pos0=sh.pos0, rope_base=sh.rope_base, d=sh.d,
        o=buf["o"], lse=buf["lse"])
    # the backward writes dm'; the loss then adds its own term (accumulate bit 1)
    rms.maglev_swa_inject_bwd(
        g["q"], buf["kx"], buf["vx"], buf["km"], buf["vm"], g["gate_logit"], buf["o"], buf["lse"],
        g["dO"], g["m_prime"], g["W_Km"], g["W_Vm"], sh.W, pos0=sh.pos0, rope_base=sh.rope_base,
        accumulate=0, out=buf["grads"], workspace=buf["ws_bwd"])
    rms.maglev_consistency_loss(
        g["m"], g["m_prime"], sh.lam, loss=buf["loss"], dm=buf["dm"],
        dm_prime=buf["grads"]["dm_prime"], accumulate=2, workspace=buf["ws_loss"])


def bench_train(sh, steps, warmup, mix="sigma"):
    """Wall time per step over the timed steps. Every kernel is timed with HIP
    events during the warmup steps after the first (the per-kernel table); the
    timed steps then time the kernel with the most time only (with events the
    library binds to that kernel's dispatch, on its launch stream)."""
    g, buf = train_setup(sh, mix=mix)
    step = train_step_gated if mix == "gated" else train_step
    step(sh, g, buf)
    torch.cuda.synchronize()
    rms.maglev_profile_enable(True)
    for _ in range(max(warmup - 1, 1)):
        step(sh, g, buf)
    torch.cuda.synchronize()
    rms.maglev_profile_enable(False)
    survey = rms.maglev_profile_read()
    work = kernel_work(sh, mix)
    dom = max((k for k in survey if k in work), key=lambda k: survey[k][1] / survey[k][0])
    rms.maglev_profile_enable(True, only=dom)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(sh, g, buf)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rms.maglev_profile_enable(False)
    timed = rms.maglev_profile_read()
    ms = (t1 - t0) * 1e3 / steps
    del g, buf
    torch.cuda.empty_cache()
    return ms, survey, dom, timed[dom]


def bench_decode(sh, steps, warmup, seed=4, mix="sigma"):
    params = [wl.decode_layer_params(sh, seed, l) for l in range(sh.layers)]
    weights = [{"W_Km": p["W_Km"].cuda(), "W_Vm": p["W_Vm"].cuda(),
                "gate_logit": p["gate_logit"].cuda()} for p in params]
    if mix == "gated":
        for l, w in enumerate(weights):
            gv = wl.gate_vectors(sh.H, sh.Dh, seed * 100 + l)
            w["gates"] = torch.stack([gv[n] for n in rms.GATE_NAMES]).float().cuda()
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


def bench_prefiller(sh, steps, warmup):
    """Attention layers of the causal prefiller (no injection) at the layer
    shape: a sliding-window layer (W = 512) and a full-attention layer (W = T),
    forward (rotate keys + attention) and backward, timed with HIP events."""
    inp = wl.layer_inputs(sh, 5, grads=True)
    g = {n: inp[n].cuda() for n in ("q", "k", "v", "dO")}
    B, T, H, Dh = sh.B, sh.T, sh.H, sh.Dh
    out = {}
    for name, W in (("sliding_window_layer", sh.W), ("full_attention_layer", T)):
        kr = torch.empty_like(g["k"])
        o = torch.empty_like(g["q"])
        lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        dq, dk, dv = (torch.empty_like(g["q"]) for _ in range(3))
        ws = torch.empty((rms.maglev_attn_bwd_workspace(B, T, H, Dh, W),), dtype=torch.uint8,
                         device="cuda")

        def step():
            rms.maglev_attn_fwd(g["q"], g["k"], g["v"], W, rope_base=sh.rope_base, krot=kr, o=o,
                                lse=lse)
            rms.maglev_attn_bwd(g["q"], kr, g["v"], o, lse, g["dO"], W, rope_base=sh.rope_base,
                                dq=dq, dk=dk, dv=dv, workspace=ws)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        pairs = sum(min(i + 1, W) for i in range(T))
        flops = 6.0 * 2.0 * pairs * Dh * B * H      # 2 forward + 4 backward contractions
        out[name] = {"W": W, "ms_per_layer_fwd_bwd": round(ms, 4),
                     "tokens/s": round(B * T / (ms / 1e3), 1),
                     "algorithmic_TFLOP": round(flops / 1e12, 4),
                     "TFLOP/s": round(flops / (ms / 1e3) / 1e12, 1),
                     "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del g
    torch.cuda.empty_cache()
    return out


def bench_stack(sh, layers, steps, warmup):
    """One lifted pass through a stack of `layers` injected layers at the
    stack shape (forward of every layer, the consistency loss, backward of
    every layer), two ways:
      shared: one memory projection of m' shared by all layers (per-layer
        mix and gates), its backward once from the summed memory gradients;
      per_layer: every layer with its own m' and projection weights (its own
        projection forward and backward);
      gated_shared: the gated mix (channel-wise 2 sigmoid gates, RMSNorm on
        the recurrent key) over one shared projection, its backward once from
        the summed gradients of the pre-norm projections.
    Inputs are drawn on the device from a seeded generator (no parity is
    checked here). Timed with HIP events around whole passes."""
    dev, bf, f32 = "cuda", torch.bfloat16, torch.float32
    B, T, H, Dh, d, W = sh.B, sh.T, sh.H, sh.Dh, sh.d, sh.W
    HD = H * Dh
    gen = torch.Generator(device=dev).manual_seed(11)

    def rnd(*shape, std=1.0, dt=bf):
        return (torch.randn(*shape, generator=gen, device=dev) * std).to(dt)

    act = (B, T, H, Dh)
    L = [{"q": rnd(*act), "k": rnd(*act), "v": rnd(*act), "dO": rnd(*act),
          "gate": rnd(H, dt=f32), "mp": rnd(B, T, d), "WK": rnd(HD, d, std=d ** -0.5),
          "WV": rnd(HD, d, std=d ** -0.5), "kx": torch.empty(act, dtype=bf, device=dev),
          "vx": torch.empty(act, dtype=bf, device=dev), "km": torch.empty(act, dtype=bf, device=dev),
          "vm": torch.empty(act, dtype=bf, device=dev), "o": torch.empty(act, dtype=bf, device=dev),
          "lse": torch.empty((B, H, T), dtype=f32, device=dev),
          "dgate": torch.empty((H,), dtype=f32, device=dev),
          "gates": rnd(4, HD, std=0.7, dt=f32),
          "dgates": torch.empty((4, HD), dtype=f32, device=dev)} for _ in range(layers)]
    m = rnd(B, T, d)
    km, vm = (torch.empty(act, dtype=bf, device=dev) for _ in range(2))
    dkm, dvm = (torch.empty(act, dtype=f32, device=dev) for _ in range(2))
    dq, dk, dv = (torch.empty(act, dtype=bf, device=dev) for _ in range(3))
    dmp = torch.empty((B, T, d), dtype=f32, device=dev)
    dm = torch.empty((B, T, d), dtype=f32, device=dev)
    dWk, dWv = (torch.empty((HD, d), dtype=f32, device=dev) for _ in range(2))
    loss = torch.empty((1,), dtype=f32, device=dev)
    ws_sh = torch.empty((rms.maglev_swa_inject_bwd_shared_workspace(B, T, H, Dh, W),),
                        dtype=torch.uint8, device=dev)
    ws_sg = torch.empty((rms.maglev_swa_inject_bwd_shared_gated_workspace(B, T, H, Dh, W),),
                        dtype=torch.uint8, device=dev)
    ws_pb = torch.empty((rms.maglev_mem_project_bwd_workspace(B, T, H, Dh, d),), dtype=torch.uint8,
                        device=dev)
    ws_bw = torch.empty((rms.maglev_swa_inject_bwd_workspace(B, T, H, Dh, d, W),),
                        dtype=torch.uint8, device=dev)
    ws_ls = torch.empty((rms.maglev_consistency_loss_workspace(B * T, d),), dtype=torch.uint8,
                        device=dev)
    grads = {"dq": dq, "dk": dk, "dv": dv, "dm_prime": dmp, "dW_Km": dWk, "dW_Vm": dWv}
    mp, WK, WV = L[0]["mp"], L[0]["WK"], L[0]["WV"]

    def shared_pass():
        rms.maglev_mem_project(mp, WK, WV, H, Dh, shift=1, kmem=km, vmem=vm)
        for x in L:
            rms.maglev_mix_entries(x["k"], x["v"], km, vm, x["gate"], kmix=x["kx"], vmix=x["vx"])
            rms.maglev_swa_inject_fwd(x["q"], x["kx"], x["vx"], W, o=x["o"], lse=x["lse"])
        for i, x in enumerate(reversed(L)):
            rms.maglev_swa_inject_bwd_shared(x["q"], x["kx"], x["vx"], km, vm, x["gate"], x["o"],
                                             x["lse"], x["dO"], dkm, dvm, W,
                                             accumulate=1 if i else 0, dq=dq, dk=dk, dv=dv,
                                             dgate=x["dgate"], workspace=ws_sh)
        rms.maglev_mem_project_bwd(dkm, dvm, mp, WK, WV, dm_prime=dmp, dW_Km=dWk, dW_Vm=dWv,
                                   workspace=ws_pb)
        rms.maglev_consistency_loss(m, mp, sh.lam, loss=loss, dm=dm, dm_prime=dmp, accumulate=2,
                                    workspace=ws_ls)

    def gated_shared_pass():
        rms.maglev_mem_project(mp, WK, WV, H, Dh, shift=1, kmem=km, vmem=vm)
        for x in L:
            rms.maglev_mix_entries_gated(x["k"], x["v"], km, vm, x["gates"], kmix=x["kx"],
                                         vmix=x["vx"])
            rms.maglev_swa_inject_fwd(x["q"], x["kx"], x["vx"], W, o=x["o"], lse=x["lse"])
        for i, x in enumerate(reversed(L)):
            rms.maglev_swa_inject_bwd_shared_gated(x["q"], x["kx"], x["vx"], x["k"], x["v"], km, vm,
                                                   x["gates"], x["o"], x["lse"], x["dO"], dkm, dvm,
                                                   W, accumulate=1 if i else 0, dq=dq, dk=dk,
                                                   dv=dv, dgates=x["dgates"], workspace=ws_sg)
        rms.maglev_mem_project_bwd(dkm, dvm, mp, WK, WV, dm_prime=dmp, dW_Km=dWk, dW_Vm=dWv,
                                   workspace=ws_pb)
        rms.maglev_consistency_loss(m, mp, sh.lam, loss=loss, dm=dm, dm_prime=dmp, accumulate=2,
                                    workspace=ws_ls)

    def per_layer_pass():
        for x in L:
            rms.maglev_mem_project(x["mp"], x["WK"], x["WV"], H, Dh, shift=1, kmem=x["km"],
                                   vmem=x["vm"], k=x["k"], v=x["v"], gate_logit=x["gate"],
                                   kmix=x["kx"], vmix=x["vx"])
            rms.maglev_swa_inject_fwd(x["q"], x["kx"], x["vx"], W, o=x["o"], lse=x["lse"])
        grads["dgate"] = L[0]["dgate"]
        for x in reversed(L):
            grads["dgate"] = x["dgate"]
            rms.maglev_swa_inject_bwd(x["q"], x["kx"], x["vx"], x["km"], x["vm"], x["gate"], x["o"],
                                      x["lse"], x["dO"], x["mp"], x["WK"], x["WV"], W, out=grads,
                                      workspace=ws_bw)
        rms.maglev_consistency_loss(m, L[-1]["mp"], sh.lam, loss=loss, dm=dm, dm_prime=dmp,
                                    accumulate=2, workspace=ws_ls)

    pairs = sum(min(i + 1, W) for i in range(T))
    attn = 2.0 * pairs * Dh * B * H
    proj = 2.0 * B * T * d * 2 * HD
    out = {}
    for name, fn, flops in (("shared_projection", shared_pass, layers * 6 * attn + 3 * proj),
                            ("projection_per_layer", per_layer_pass, layers * (6 * attn + 3 * proj)),
                            ("gated_shared_projection", gated_shared_pass,
                             layers * 6 * attn + 3 * proj)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[name] = {"ms_per_pass": round(ms, 3), "tokens/s": round(B * T / (ms / 1e3), 1),
                     "algorithmic_TFLOP": round(flops / 1e12, 4),
                     "TFLOP/s": round(flops / (ms / 1e3) / 1e12, 1),
                     "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del L
    torch.cuda.empty_cache()
    return out


def bench_loss_head(N, d, V, steps, warmup):
    """The loss head at the last hidden state of a batch: final RMSNorm,
    soft-capped LM head (V entries), mean cross-entropy, consistency term
    (lambda 0.5) and the gradients w.r.t. h and U, one C-ABI call per step,
    timed with HIP events; a second timed pass records each kernel's average
    duration for its roofline."""
    x = wl.head_inputs(N, d, V, 12, wl.BF16)
    g = {n: t.cuda() for n, t in x.items()}
    m = torch.empty_like(g["h"])
    loss = torch.empty((1,), dtype=torch.float32, device="cuda")
    dh = torch.empty(g["h"].shape, dtype=torch.float32, device="cuda")
    dU = torch.empty(g["U"].shape, dtype=torch.float32, device="cuda")
    ws = torch.empty((rms.maglev_lm_head_workspace(N, d, V),), dtype=torch.uint8, device="cuda")

    def step():
        rms.maglev_lm_head(g["h"], g["U"], g["targets"], m_prime=g["m_prime"], lam=0.5, m=m,
                           loss=loss, dh=dh, dU=dU, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    rms.maglev_profile_enable(True)
    for _ in range(max(steps // 2, 2)):
        step()
    torch.cuda.synchronize()
    rms.maglev_profile_enable(False)
    survey = rms.maglev_profile_read()
    gemm = 2.0 * N * V * d
    nd = 2.0 * N * d   # one bf16 [N, d] tensor
    work = {  # (algorithmic flops, algorithmic bytes) per launch
        "lm_logits": (gemm, nd + 2.0 * V * d + 4.0 * N * V),
        "head_ce": (0.0, 4.0 * N * V + 2.0 * N * V + 8.0 * N),
        "lm_dm": (gemm, 2.0 * N * V + 2.0 * V * d + 4.0 * N * d),
        "lm_dm_transpose": (0.0, 4.0 * V * d),
        "lm_du": (gemm, 2.0 * N * V + nd + 4.0 * V * d),
        "head_norm": (0.0, 2.0 * nd + 4.0 * N),
        "head_norm_bwd": (0.0, nd + 8.0 * N * d + 4.0 * N),
    }
    kernels = {}
    for name, (n, tot) in sorted(survey.items(), key=lambda kv: -kv[1][1]):
        rec = {"launches": n, "avg_us": round(tot * 1e3 / n, 2)}
        if name in work:
            rec["roofline"] = roofline_of(work[name][0], work[name][1], tot / n / 1e3)
        kernels[name] = rec
    flops = 3.0 * gemm
    del g, ws
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "tokens/s": round(N / (ms / 1e3), 1),
            "algorithmic_TFLOP": round(flops / 1e12, 4),
            "TFLOP/s": round(flops / (ms / 1e3) / 1e12, 1),
            "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": kernels}


def cpu_baseline(sh):
    """The oracle, as it stands, on a bounded slice of the training workload:
    sequences 0-5 of 8, all heads, full T. The slice holds 6/8 of the layer's
    attention pairs and projection rows, so the full-step time is scaled by 8/6."""
    import oracle

    oracle.build(force=False)
    inp = wl.layer_inputs(sh, 2, grads=True)
    nb = 6
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
        "sample": "sequences 0-%d (all heads) of the d20 layer fwd+bwd+loss (T=2048, W=512): "
                  "%.1f s, scaled by %.4g to the full batch" % (nb - 1, dt, factor),
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
    ap.add_argument("--no-prefiller", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-head", action="store_true")
    ap.add_argument("--mix", choices=("sigma", "gated"), default="sigma",
                    help="mixing form: per-head sigma gate (default) or the gated form with "
                         "channel-wise 2 sigmoid gates and the normalised memory key")
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
    ms, survey, dom, (n_dom, t_dom) = bench_train(sh, args.steps, args.warmup, args.mix)
    tokens = sh.B * sh.T
    value = tokens / (ms / 1e3)
    path_tflops = total_flops / (ms / 1e3) / 1e12

    # per-kernel averages over the warmup steps; live roofline of the dominant kernel
    work = kernel_work(sh, args.mix)
    per_kernel = {}
    for name, (n, tot) in sorted(survey.items(), key=lambda kv: -kv[1][1]):
        rec = {"launches": n, "avg_us": round(tot * 1e3 / n, 2)}
        if name in work:
            rec["roofline"] = roofline_of(work[name][0], work[name][1], tot / n / 1e3)
        per_kernel[name] = rec
    call_kernels = CALL_KERNELS_GATED if args.mix == "gated" else CALL_KERNELS
    calls = {c: round(sum(survey[k][1] / survey[k][0] for k in ks if k in survey), 4)
             for c, ks in call_kernels.items()}
    roofline = roofline_of(work[dom][0], work[dom][1], t_dom / n_dom / 1e3)
    roofline["traffic"] = measured_traffic(dom)
    roofline["kernel"] = dom
    roofline["avg_us"] = round(t_dom * 1e3 / n_dom, 2)
    roofline["launches"] = n_dom
    roofline["algorithmic_per_launch"] = (work[dom][0] if roofline["bound"] == "mfma" else work[dom][1])

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
        "config": {"workload": "d20 decoder-P layer fwd+bwd + consistency loss"
                               + (", gated mix (2 sigmoid channel gates, RMSNorm memory key)"
                                  if args.mix == "gated" else ""),
                   "mix": args.mix,
                   "B": sh.B, "T": sh.T, "W": sh.W, "d_model": sh.d, "heads": sh.H,
                   "head_dim": sh.Dh, "lambda": sh.lam, "global_batch": sh.B, "seq_len": sh.T,
                   "parallelism": "single GPU"},
        "path": {"algorithmic_TFLOP_per_step": round(total_flops / 1e12, 4),
                 "TFLOP/s": round(path_tflops, 1),
                 "frac_bf16_peak": round(path_tflops / PEAK_BF16_TFLOPS, 4),
                 "calls_ms": calls, "kernels_warmup": per_kernel},
        "roofline": roofline,
    }
    if not args.no_decode:
        dsh = wl.D20_DECODE
        dms = bench_decode(dsh, args.decode_steps, 5, mix=args.mix)
        dbytes = decode_bytes(dsh)
        gbs = dbytes / (dms / 1e3) / 1e9
        result["decode"] = {
            "workload": "recurrent decode, 20 layers, 64 streams, W=512 bf16 ring, 10x128 heads",
            "steps": args.decode_steps, "ms_per_step": round(dms, 4),
            "tokens/s": round(dsh.Bs / (dms / 1e3), 1),
            "algorithmic_GB_per_step": round(dbytes / 1e9, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode_step") if args.mix == "sigma" else None},
            "graph": "one HIP graph per step: one projection of m_{t-1} by all layers' stacked weights, 20 decode steps, advance",
        }
    if not args.no_prefiller:
        result["prefiller"] = {
            "workload": "causal prefiller attention without injection, B=8, T=2048, 10x128 "
                        "heads, bf16: SLSL layers' sliding-window (W=512) and full (W=T) kinds",
            **bench_prefiller(sh, max(args.steps // 2, 5), 3)}
    if not args.no_stack:
        ssh = wl.D20_STACK
        result["stack"] = {
            "workload": "one lifted pass through %d injected layers, B=%d, T=%d, W=%d, d=%d, "
                        "10x128 heads, bf16, consistency loss at the end"
                        % (wl.D20_STACK_LAYERS, ssh.B, ssh.T, ssh.W, ssh.d),
            "layers": wl.D20_STACK_LAYERS,
            **bench_stack(ssh, wl.D20_STACK_LAYERS, 3, 1)}
    if not args.no_head:
        N, d, V = sh.B * sh.T, sh.d, wl.D20_VOCAB
        result["loss_head"] = {
            "workload": "loss head over %d positions (B=%d x T=%d), d=%d, V=%d, bf16: final "
                        "RMSNorm, 15-capped LM head, mean CE + consistency, dh and dU"
                        % (N, sh.B, sh.T, d, V),
            **bench_loss_head(N, d, V, max(args.steps // 2, 5), 2)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sh)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
