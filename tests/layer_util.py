"""Shared helpers of the GPU parity tests: run one layer through the C ABI
(via the binding) and through the CPU oracle on the same seeded inputs, and
compare with the stated tolerances.

Tolerances (max-abs error <= tol * scale):
  tol = 1e-4 for float32 workloads, 2e-2 for bf16 workloads.
  scale for activations (kmem, vmem, o, lse, dq, dk, dv, dm') = 1 on the named
    bf16 workloads (the stated bar), and max(1, max|ref|) on the extra shape
    and edge cases: a bf16 value of magnitude a carries a rounding step of up
    to a * 2^-8 and every MFMA operand (rotated q, mixed k/v, probabilities,
    dS, dO) is rounded once, so beyond magnitude 1 the bar scales with the
    tensor's largest value.
  scale for dW_Km, dW_Vm = max(1, max|ref|): sums over every token.
  scale for dgate[h] = max(1, ||terms_h||_2), the L2 norm of the summed terms
    s(1-s) (kmem*dk + vmem*dv) of that head: the error of a long sum of
    independently rounded terms grows with that norm, while a dropped or
    mis-signed term moves the sum by about the norm itself (50x the bar).
"""
import math

import numpy as np
import torch

import oracle
import recurrent_memory_sliding_amd as rms

TOL = {"f32": 1e-4, "bf16": 2e-2}


def flush(msg):
    print(msg, flush=True)


def gpu(d):
    return {k: v.cuda() for k, v in d.items()}


def maxabs(got, ref):
    g = got.detach().to("cpu", torch.float64).numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    return float(np.max(np.abs(g - ref))) if np.size(ref) else 0.0


def check(name, got, ref, tol, scale=1.0):
    ref = np.asarray(ref, dtype=np.float64)
    err = maxabs(got, ref)
    assert np.isfinite(err), "%s: non-finite values" % name
    assert err <= tol * scale, "%s: max-abs err %.3e > tol %.1e x scale %.3g" % (name, err, tol, scale)
    return err / scale


def max_scale(ref):
    ref = np.asarray(ref)
    return max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0


def dgate_scale(inp, sh, ref_grads, kmem, vmem):
    """Per-head L2 norm of the terms s(1-s)(kmem*dk + vmem*dv) summed into dgate."""
    s = 1.0 / (1.0 + np.exp(-oracle.f64(inp["gate_logit"])))
    tk = kmem * ref_grads["dk"]
    tv = vmem * ref_grads["dv"]
    norms = np.sqrt(np.sum(tk * tk + tv * tv, axis=(0, 1, 3)))
    return np.maximum(1.0, s * (1.0 - s) * norms)


def gpu_project(g, sh):
    """Memory projection with the mix: stores the mixed entries as g["kx"], g["vx"]."""
    km, vm, g["kx"], g["vx"] = rms.maglev_mem_project(
        g["m_prime"], g["W_Km"], g["W_Vm"], sh.H, sh.Dh, shift=1, k=g["k"], v=g["v"],
        gate_logit=g["gate_logit"], pos0=sh.pos0, rope_base=sh.rope_base)
    return km, vm


def gpu_forward(inp, sh):
    g = gpu(inp)
    km, vm = gpu_project(g, sh)
    o, lse = rms.maglev_swa_inject_fwd(g["q"], g["kx"], g["vx"], sh.W, pos0=sh.pos0,
                                       rope_base=sh.rope_base, d=sh.d)
    return g, km, vm, o, lse


def gpu_backward(g, km, vm, o, lse, sh, accumulate=0, out=None):
    return rms.maglev_swa_inject_bwd(g["q"], g["kx"], g["vx"], km, vm, g["gate_logit"], o, lse,
                                     g["dO"], g["m_prime"], g["W_Km"], g["W_Vm"], sh.W,
                                     pos0=sh.pos0, rope_base=sh.rope_base, accumulate=accumulate,
                                     out=out)


def oracle_forward(inp, sh):
    km, vm = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], sh.H, sh.Dh, shift=1)
    o, lse = oracle.swa_inject_fwd(inp["q"], inp["k"], inp["v"], km, vm, inp["gate_logit"], sh.W,
                                   pos0=sh.pos0, rope_base=sh.rope_base)
    return km, vm, o, lse


def oracle_backward(inp, sh):
    return oracle.swa_inject_bwd(inp["q"], inp["k"], inp["v"], inp["m_prime"], inp["W_Km"],
                                 inp["W_Vm"], inp["gate_logit"], inp["dO"], sh.W, pos0=sh.pos0,
                                 rope_base=sh.rope_base)


def check_forward(sh, inp, res_gpu, res_ref, strict=False):
    """strict: the named-workload bar (absolute) for the activations; float32
    workloads are always judged absolutely."""
    tol = TOL[sh.dtype]
    strict = strict or sh.dtype == "f32"
    g, km, vm, o, lse = res_gpu
    rkm, rvm, ro, rlse = res_ref
    rkx, rvx = oracle.mixed_entries(inp["k"], inp["v"], rkm, rvm, inp["gate_logit"], sh.pos0,
                                    sh.rope_base)
    errs = {}
    for name, got, ref in (("kmem", km, rkm), ("vmem", vm, rvm), ("o", o, ro), ("lse", lse, rlse)):
        errs[name] = check(name, got, ref, tol, 1.0 if strict else max_scale(ref))
    # the mixed entries are a stored intermediate whose magnitude exceeds 4 (bf16
    # half-ulp 1.6e-2 there): always judged relative to max(1, max|ref|)
    for name, got, ref in (("kmix", g["kx"], rkx), ("vmix", g["vx"], rvx)):
        errs[name] = check(name, got, ref, tol, max_scale(ref))
    return errs


def check_backward(sh, inp, grads, ref, kmem_ref, vmem_ref, strict=False):
    tol = TOL[sh.dtype]
    strict = strict or sh.dtype == "f32"
    errs = {}
    for n in ("dq", "dk", "dv", "dm_prime"):
        errs[n] = check(n, grads[n], ref[n], tol, 1.0 if strict else max_scale(ref[n]))
    for n in ("dW_Km", "dW_Vm"):
        errs[n] = check(n, grads[n], ref[n], tol, max_scale(ref[n]))
    sc = dgate_scale(inp, sh, ref, kmem_ref, vmem_ref)
    got = grads["dgate"].detach().cpu().double().numpy()
    err = np.abs(got - ref["dgate"])
    assert np.all(err <= tol * sc), "dgate: err %s > tol x scale %s" % (err, tol * sc)
    errs["dgate"] = float(np.max(err / sc))
    return errs
