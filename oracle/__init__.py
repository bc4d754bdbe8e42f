"""CPU oracle for the Maglev attention + recurrent K/V injection path.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product library never does.

The arithmetic lives in `maglev_oracle.c` (plain C, double precision, OpenMP),
compiled by `build()` with gcc. This module only marshals arrays: every input
is converted to float64 holding exactly the stored value (bf16 or fp32), and
every result comes back as float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "maglev_oracle.c")
_LIB = os.path.join(_HERE, "libmaglev_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics kept: no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(ctypes.c_double)
        I64 = ctypes.c_int64
        I32 = ctypes.c_int
        D = ctypes.c_double
        PI64 = ctypes.POINTER(ctypes.c_int64)
        L.oracle_round_bf16.argtypes = [D]
        L.oracle_round_bf16.restype = D
        L.oracle_mem_project.argtypes = [I64, I64, I32, I32, I32, I32, P, P, P, P, P]
        L.oracle_mem_project.restype = None
        L.oracle_swa_inject_fwd.argtypes = [I64, I64, I32, I32, I64, I64, D, D,
                                            P, P, P, P, P, P, P, P]
        L.oracle_swa_inject_fwd.restype = None
        L.oracle_swa_inject_bwd.argtypes = [I64, I64, I32, I32, I32, I64, I64, D, D,
                                            P, P, P, P, P, P, P, P,
                                            P, P, P, P, P, P, P]
        L.oracle_swa_inject_bwd.restype = None
        L.oracle_consistency_loss.argtypes = [I64, I32, D, P, P, P, P]
        L.oracle_consistency_loss.restype = D
        L.oracle_decode_step.argtypes = [I64, I32, I32, I64, D, D, I32,
                                         P, P, P, P, P, P, P, P, PI64, P]
        L.oracle_decode_step.restype = None
        L.oracle_swa_inject_fwd_rows.argtypes = [I64, I64, I32, I32, I64, I64, D, D,
                                                 P, P, P, P, P, P, I64, PI64, P, P]
        L.oracle_swa_inject_fwd_rows.restype = None
        L.oracle_mixed_entries.argtypes = [I64, I64, I32, I32, I64, D, P, P, P, P, P, P, P]
        L.oracle_mixed_entries.restype = None
        L.oracle_gated_entries.argtypes = [I64, I64, I32, I32, I64, D, D,
                                           P, P, P, P, P, P, P, P, P, P]
        L.oracle_gated_entries.restype = None
        L.oracle_swa_attend_fwd.argtypes = [I64, I64, I32, I32, I64, I64, D, D, P, P, P, P, P]
        L.oracle_swa_attend_fwd.restype = None
        L.oracle_swa_inject_bwd_gated.argtypes = [I64, I64, I32, I32, I32, I64, I64, D, D, D,
                                                  P, P, P, P, P, P, P, P, P, P, P,
                                                  P, P, P, P, P, P, P, P, P, P]
        L.oracle_swa_inject_bwd_gated.restype = None
        L.oracle_decode_step_gated.argtypes = [I64, I32, I32, I64, D, D, D, I32,
                                               P, P, P, P, P, P, P, P, P, P, P, PI64, P]
        L.oracle_decode_step_gated.restype = None
        L.oracle_lm_head.argtypes = [I64, I32, I64, D, D, D, P, P, PI64, P, P, P, P]
        L.oracle_lm_head.restype = D
        L.oracle_lm_head_rows.argtypes = [I64, PI64, I32, I64, D, D, I64, P, P, PI64, P, P, P]
        L.oracle_lm_head_rows.restype = None
        _lib = L
    return _lib


def f64(x) -> np.ndarray:
    """Exact float64 copy of a torch tensor (any float dtype) or array-like."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def round_bf16(x: float) -> float:
    return float(_load().oracle_round_bf16(float(x)))


def mem_project(m, W_Km, W_Vm, H: int, Dh: int, shift: int = 1):
    """kmem, vmem [B,T,H,Dh] from m [B,T,d] (shift=1: row t reads m[t-1], row 0 is zero)."""
    m, WK, WV = f64(m), f64(W_Km), f64(W_Vm)
    B, T, d = m.shape
    kmem = np.empty((B, T, H, Dh))
    vmem = np.empty((B, T, H, Dh))
    _load().oracle_mem_project(B, T, H, Dh, d, int(shift), _p(m), _p(WK), _p(WV), _p(kmem), _p(vmem))
    return kmem, vmem


def mixed_entries(k, v, kmem, vmem, gate_logit, pos0: int = 0, rope_base: float = 10000.0):
    """kmix = R k + s R kmem, vmix = v + s vmem, both [B,T,H,Dh] (s = sigmoid(gate))."""
    k, v, km, vm, g = (f64(a) for a in (k, v, kmem, vmem, gate_logit))
    B, T, H, Dh = k.shape
    if Dh > 512:
        raise ValueError("Dh above 512")
    kx = np.empty((B, T, H, Dh))
    vx = np.empty((B, T, H, Dh))
    _load().oracle_mixed_entries(B, T, H, Dh, int(pos0), float(rope_base), _p(k), _p(v), _p(km),
                                 _p(vm), _p(g), _p(kx), _p(vx))
    return kx, vx


def swa_inject_fwd(q, k, v, kmem, vmem, gate_logit, W: int, pos0: int = 0,
                   rope_base: float = 10000.0, scale: float = 0.0):
    """O [B,T,H,Dh] and lse [B,H,T]."""
    q, k, v, km, vm, g = (f64(a) for a in (q, k, v, kmem, vmem, gate_logit))
    B, T, H, Dh = q.shape
    o = np.empty((B, T, H, Dh))
    lse = np.empty((B, H, T))
    _load().oracle_swa_inject_fwd(B, T, H, Dh, int(W), int(pos0), float(rope_base), float(scale),
                                  _p(q), _p(k), _p(v), _p(km), _p(vm), _p(g), _p(o), _p(lse))
    return o, lse


def swa_inject_fwd_rows(q, k, v, kmem, vmem, gate_logit, W: int, rows, pos0: int = 0,
                        rope_base: float = 10000.0, scale: float = 0.0):
    """O and lse of selected queries; rows is an [n,3] array of (b, h, i)."""
    q, k, v, km, vm, g = (f64(a) for a in (q, k, v, kmem, vmem, gate_logit))
    B, T, H, Dh = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    o = np.empty((n, Dh))
    lse = np.empty((n,))
    _load().oracle_swa_inject_fwd_rows(B, T, H, Dh, int(W), int(pos0), float(rope_base),
                                       float(scale), _p(q), _p(k), _p(v), _p(km), _p(vm), _p(g),
                                       n, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                       _p(o), _p(lse))
    return o, lse


def swa_inject_bwd(q, k, v, m_prime, W_Km, W_Vm, gate_logit, dO, W: int, pos0: int = 0,
                   rope_base: float = 10000.0, scale: float = 0.0):
    """Gradients of the whole layer path (shift, projection, mix, attention).

    Returns dict with dq, dk, dv [B,T,H,Dh], dm_prime [B,T,d], dW_Km, dW_Vm [H*Dh,d], dgate [H].
    """
    q, k, v, mp, WK, WV, g, dO = (f64(a) for a in (q, k, v, m_prime, W_Km, W_Vm, gate_logit, dO))
    B, T, H, Dh = q.shape
    d = mp.shape[-1]
    out = {
        "dq": np.empty_like(q), "dk": np.empty_like(q), "dv": np.empty_like(q),
        "dm_prime": np.empty((B, T, d)), "dW_Km": np.empty((H * Dh, d)),
        "dW_Vm": np.empty((H * Dh, d)), "dgate": np.empty((H,)),
    }
    _load().oracle_swa_inject_bwd(B, T, H, Dh, d, int(W), int(pos0), float(rope_base), float(scale),
                                  _p(q), _p(k), _p(v), _p(mp), _p(WK), _p(WV), _p(g), _p(dO),
                                  _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dm_prime"]),
                                  _p(out["dW_Km"]), _p(out["dW_Vm"]), _p(out["dgate"]))
    return out


def swa_inject_bwd_shared(layers, m_prime, W_Km, W_Vm, W: int, pos0: int = 0,
                          rope_base: float = 10000.0, scale: float = 0.0):
    """Gradients of a stack of layers that share one memory projection
    (W_Km, W_Vm applied to the same shifted m') and each have their own
    q, k, v, gate logits and upstream gradient dO: layers is a list of dicts
    with those keys. The stack's objective is the sum over layers, so by the
    chain rule each layer contributes its single-layer gradient and the
    shared parameters and m' collect the sum of the contributions.
    Returns (per_layer, shared): per_layer[l] holds dq, dk, dv, dgate;
    shared holds dm_prime, dW_Km, dW_Vm."""
    per_layer, shared = [], None
    for x in layers:
        g = swa_inject_bwd(x["q"], x["k"], x["v"], m_prime, W_Km, W_Vm, x["gate_logit"], x["dO"],
                           W, pos0=pos0, rope_base=rope_base, scale=scale)
        per_layer.append({n: g[n] for n in ("dq", "dk", "dv", "dgate")})
        part = {n: g[n] for n in ("dm_prime", "dW_Km", "dW_Vm")}
        shared = part if shared is None else {n: shared[n] + part[n] for n in part}
    return per_layer, shared


def consistency_loss(m, m_prime, lam: float):
    """(loss, dm, dm_prime) for L = lam/(N sqrt d) * sum (m - m')^2 over N rows of width d."""
    m, mp = f64(m), f64(m_prime)
    d = m.shape[-1]
    N = m.size // d
    dm = np.empty_like(m)
    dmp = np.empty_like(m)
    loss = _load().oracle_consistency_loss(N, d, float(lam), _p(m), _p(mp), _p(dm), _p(dmp))
    return float(loss), dm, dmp


def decode_step(q, k, v, kmem, vmem, gate_logit, kcache: np.ndarray, vcache: np.ndarray, pos,
                rope_base: float = 10000.0, scale: float = 0.0, ring_bf16: bool = True):
    """One decode step; kcache/vcache (float64 [Bs,H,W,Dh]) are updated in place. Returns o."""
    q, k, v, km, vm, g = (f64(a) for a in (q, k, v, kmem, vmem, gate_logit))
    assert kcache.dtype == np.float64 and kcache.flags.c_contiguous
    assert vcache.dtype == np.float64 and vcache.flags.c_contiguous
    Bs, H, W, Dh = kcache.shape
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64).reshape(Bs))
    o = np.empty((Bs, H, Dh))
    _load().oracle_decode_step(Bs, H, Dh, W, float(rope_base), float(scale), int(bool(ring_bf16)),
                               _p(q), _p(k), _p(v), _p(km), _p(vm), _p(g), _p(kcache), _p(vcache),
                               pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _p(o))
    return o


# ----------------------------------------------------------------------------
# gated variant: k~ = g_kl R k + g_kr R RMSNorm(W_Km m'), v~ = g_vl v + g_vr W_Vm m',
# g = 2 sigmoid(a), four channel-wise logit vectors [H*Dh] in the order
# (a_kl, a_kr, a_vl, a_vr).
# ----------------------------------------------------------------------------
GATE_NAMES = ("a_kl", "a_kr", "a_vl", "a_vr")
RMS_EPS = 1e-6


def _gates(gates, HD: int):
    if isinstance(gates, dict):
        gates = [gates[n] for n in GATE_NAMES]
    out = [f64(g).reshape(-1) for g in gates]
    if len(out) != 4 or any(g.size != HD for g in out):
        raise ValueError("four gate logit vectors of H*Dh entries expected")
    return out


def gated_entries(k, v, kproj, vmem, gates, pos0: int = 0, rope_base: float = 10000.0,
                  eps: float = RMS_EPS):
    """Gated mixed entries kmix, vmix [B,T,H,Dh] from the pre-norm key projection."""
    k, v, kp, vm = (f64(a) for a in (k, v, kproj, vmem))
    B, T, H, Dh = k.shape
    if Dh > 512 or H * Dh > 4096:
        raise ValueError("Dh above 512 or H*Dh above 4096")
    g = _gates(gates, H * Dh)
    kx = np.empty((B, T, H, Dh))
    vx = np.empty((B, T, H, Dh))
    _load().oracle_gated_entries(B, T, H, Dh, int(pos0), float(rope_base), float(eps), _p(k),
                                 _p(v), _p(kp), _p(vm), *(_p(a) for a in g), _p(kx), _p(vx))
    return kx, vx


def swa_attend_fwd(q, kmix, vmix, W: int, pos0: int = 0, rope_base: float = 10000.0,
                   scale: float = 0.0):
    """O [B,T,H,Dh] and lse [B,H,T] of the rotated queries over given mixed entries."""
    q, kx, vx = (f64(a) for a in (q, kmix, vmix))
    B, T, H, Dh = q.shape
    o = np.empty((B, T, H, Dh))
    lse = np.empty((B, H, T))
    _load().oracle_swa_attend_fwd(B, T, H, Dh, int(W), int(pos0), float(rope_base),
                                  float(scale), _p(q), _p(kx), _p(vx), _p(o), _p(lse))
    return o, lse


def swa_inject_fwd_gated(q, k, v, m_prime, W_Km, W_Vm, gates, W: int, pos0: int = 0,
                         rope_base: float = 10000.0, scale: float = 0.0, eps: float = RMS_EPS):
    """Forward of the gated layer path: projection of the shifted memory, the
    gated mix, attention. Returns (o, lse)."""
    H, Dh = q.shape[2], q.shape[3]
    kp, vm = mem_project(m_prime, W_Km, W_Vm, H, Dh, shift=1)
    kx, vx = gated_entries(k, v, kp, vm, gates, pos0=pos0, rope_base=rope_base, eps=eps)
    return swa_attend_fwd(q, kx, vx, W, pos0=pos0, rope_base=rope_base, scale=scale)


def swa_inject_bwd_gated(q, k, v, m_prime, W_Km, W_Vm, gates, dO, W: int, pos0: int = 0,
                         rope_base: float = 10000.0, scale: float = 0.0,
                         eps: float = RMS_EPS):
    """Gradients of the gated layer path. Returns dict with dq, dk, dv,
    dm_prime, dW_Km, dW_Vm and the four gate-logit gradients (a_* names)."""
    q, k, v, mp, WK, WV, dO = (f64(a) for a in (q, k, v, m_prime, W_Km, W_Vm, dO))
    B, T, H, Dh = q.shape
    d = mp.shape[-1]
    if Dh > 512 or H * Dh > 4096:
        raise ValueError("Dh above 512 or H*Dh above 4096")
    g = _gates(gates, H * Dh)
    out = {
        "dq": np.empty_like(q), "dk": np.empty_like(q), "dv": np.empty_like(q),
        "dm_prime": np.empty((B, T, d)), "dW_Km": np.empty((H * Dh, d)),
        "dW_Vm": np.empty((H * Dh, d)),
    }
    for n in GATE_NAMES:
        out["d" + n] = np.empty((H * Dh,))
    _load().oracle_swa_inject_bwd_gated(
        B, T, H, Dh, d, int(W), int(pos0), float(rope_base), float(scale), float(eps),
        _p(q), _p(k), _p(v), _p(mp), _p(WK), _p(WV), *(_p(a) for a in g), _p(dO),
        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dm_prime"]), _p(out["dW_Km"]),
        _p(out["dW_Vm"]), *(_p(out["d" + n]) for n in GATE_NAMES))
    return out


def swa_inject_bwd_shared_gated(layers, m_prime, W_Km, W_Vm, W: int, pos0: int = 0,
                                rope_base: float = 10000.0, scale: float = 0.0,
                                eps: float = RMS_EPS):
    """Gradients of a stack of gated layers that share one projection of the
    shifted memory (the same m', W_Km, W_Vm for every layer) and each have
    their own q, k, v, four gate-logit vectors ("gates") and upstream
    gradient dO. The stack's objective is the sum over layers, so each layer
    contributes its single-layer gradient (swa_inject_bwd_gated) and the
    shared parameters and m' collect the sum.
    Returns (per_layer, shared): per_layer[l] holds dq, dk, dv and the four
    d<gate name> vectors; shared holds dm_prime, dW_Km, dW_Vm."""
    per_layer, shared = [], None
    for x in layers:
        g = swa_inject_bwd_gated(x["q"], x["k"], x["v"], m_prime, W_Km, W_Vm, x["gates"], x["dO"],
                                 W, pos0=pos0, rope_base=rope_base, scale=scale, eps=eps)
        per_layer.append({n: g[n] for n in ("dq", "dk", "dv") + tuple("d" + a for a in GATE_NAMES)})
        part = {n: g[n] for n in ("dm_prime", "dW_Km", "dW_Vm")}
        shared = part if shared is None else {n: shared[n] + part[n] for n in part}
    return per_layer, shared


def decode_step_gated(q, k, v, kproj, vmem, gates, kcache: np.ndarray, vcache: np.ndarray,
                      pos, rope_base: float = 10000.0, scale: float = 0.0,
                      eps: float = RMS_EPS, ring_bf16: bool = True):
    """One gated decode step (kproj is W_Km m_{t-1} before the norm); the
    float64 caches [Bs,H,W,Dh] are updated in place. Returns o [Bs,H,Dh]."""
    q, k, v, kp, vm = (f64(a) for a in (q, k, v, kproj, vmem))
    assert kcache.dtype == np.float64 and kcache.flags.c_contiguous
    assert vcache.dtype == np.float64 and vcache.flags.c_contiguous
    Bs, H, W, Dh = kcache.shape
    if Dh > 512 or H * Dh > 4096:
        raise ValueError("Dh above 512 or H*Dh above 4096")
    g = _gates(gates, H * Dh)
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64).reshape(Bs))
    o = np.empty((Bs, H, Dh))
    _load().oracle_decode_step_gated(Bs, H, Dh, W, float(rope_base), float(scale), float(eps),
                                     int(bool(ring_bf16)), _p(q), _p(k), _p(v), _p(kp), _p(vm),
                                     *(_p(a) for a in g), _p(kcache), _p(vcache),
                                     pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _p(o))
    return o


LM_CAP = 15.0


def lm_head(h, U, targets, m_prime=None, lam: float = 0.0, cap: float = LM_CAP,
            eps: float = RMS_EPS, grads: bool = True):
    """Loss head: m = RMSNorm(h), capped logits cap tanh(U m / cap), mean CE over
    all positions (targets outside [0, V) ignored) + lam / (N sqrt d) sum ||m - m'||^2.
    Returns dict with loss, m [N,d] and (grads) dh [N,d], dU [V,d]."""
    h, U = f64(h), f64(U)
    d = h.shape[-1]
    hs = h.reshape(-1, d)
    N, V = hs.shape[0], U.shape[0]
    tg = np.ascontiguousarray(np.asarray(targets, dtype=np.int64).reshape(N))
    mp = f64(m_prime).reshape(N, d) if m_prime is not None else None
    out = {"m": np.empty((N, d))}
    if grads:
        out["dh"] = np.empty((N, d))
        out["dU"] = np.empty((V, d))
    PI = ctypes.POINTER(ctypes.c_int64)
    out["loss"] = float(_load().oracle_lm_head(
        N, d, V, float(cap), float(eps), float(lam), _p(hs), _p(U), tg.ctypes.data_as(PI),
        _p(mp) if mp is not None else None, _p(out["m"]), _p(out["dh"]) if grads else None,
        _p(out["dU"]) if grads else None))
    return out


def lm_head_rows(h, U, targets, rows, cap: float = LM_CAP, eps: float = RMS_EPS):
    """(lse, ce, dm_head) of the listed rows only: log-sum-exp, CE term and
    U^T dz of each row (dz already carrying 1/N)."""
    h, U = f64(h), f64(U)
    d = h.shape[-1]
    hs = h.reshape(-1, d)
    N, V = hs.shape[0], U.shape[0]
    tg = np.ascontiguousarray(np.asarray(targets, dtype=np.int64).reshape(N))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    n = rows.size
    lse, ce, dm = np.empty(n), np.empty(n), np.empty((n, d))
    PI = ctypes.POINTER(ctypes.c_int64)
    _load().oracle_lm_head_rows(n, rows.ctypes.data_as(PI), d, V, float(cap), float(eps), N,
                                _p(hs), _p(U), tg.ctypes.data_as(PI), _p(lse), _p(ce), _p(dm))
    return lse, ce, dm


def omp_threads() -> int:
    """Threads the oracle's OpenMP regions use (OMP_NUM_THREADS or all cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.strip().isdigit():
        return int(env)
    return os.cpu_count() or 1
