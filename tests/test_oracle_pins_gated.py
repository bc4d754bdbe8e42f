"""Pins for the oracle's gated variant (channel-wise 2*sigmoid gates on the
local and recurrent terms, RMSNorm on the projected memory key), each against
something other than the oracle itself: numpy's complex arithmetic and
reductions, torch's scaled_dot_product_attention, the ungated oracle in the
special case where both forms coincide (itself pinned in test_oracle_pins),
an invariance of the norm, central finite differences, torch fp64 autograd
through a dense formulation, and the lifted pass replayed by the decode step.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import workloads as wl
from test_oracle_pins import band_mask, project, rope_complex, sdpa_reference

NAMES = oracle.GATE_NAMES


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def numpy_gated(k, v, kproj, vmem, gates, pos, base, eps):
    """Gated entries from numpy routines: the norm divides each [H*Dh] row by
    sqrt(mean of squares + eps); rotation is complex multiplication."""
    B, T, H, Dh = k.shape
    ms = np.mean(kproj.reshape(B, T, H * Dh) ** 2, axis=-1)[:, :, None, None]
    kn = kproj / np.sqrt(ms + eps)
    g = {n: 2.0 * expit(np.asarray(gates[n], dtype=np.float64)).reshape(H, Dh) for n in NAMES}
    kx = g["a_kl"] * rope_complex(k, pos, base) + g["a_kr"] * rope_complex(kn, pos, base)
    vx = g["a_vl"] * v + g["a_vr"] * vmem
    return kx, vx


def f64_inputs(raw, names=("q", "k", "v", "m_prime", "W_Km", "W_Vm")):
    return {n: oracle.f64(raw[n]) for n in names}


@pytest.mark.parametrize("pos0,base,eps", [(0, 10000.0, 1e-6), (1000, 10000.0, 1e-6),
                                           (3, 0.0, 1e-30), (0, 100.0, 0.25)])
def test_gated_entries_match_numpy(pos0, base, eps):
    sh = wl.LayerShape(B=2, T=11, W=4, d=16, H=3, Dh=8, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=41)
    x = f64_inputs(raw)
    gates = {n: oracle.f64(a) for n, a in wl.gate_vectors(sh.H, sh.Dh, 41, std=1.5).items()}
    kp = project(x["m_prime"], x["W_Km"], sh.H, sh.Dh)
    vm = project(x["m_prime"], x["W_Vm"], sh.H, sh.Dh)
    # heads of very different magnitude: a per-head norm would differ from the row norm
    kp = kp * np.array([0.1, 1.0, 30.0])[None, None, :, None]
    kx, vx = oracle.gated_entries(x["k"], x["v"], kp, vm, gates, pos0=pos0, rope_base=base,
                                  eps=eps)
    rk, rv = numpy_gated(x["k"], x["v"], kp, vm, gates, np.arange(sh.T) + pos0, base, eps)
    np.testing.assert_allclose(kx, rk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(vx, rv, rtol=1e-13, atol=1e-13)


def test_gated_zero_logits_unit_rms_equals_ungated_sigma_one():
    """a = 0 gives every gate the neutral value 1; with each projected row
    scaled to mean square 1 - eps the norm is the identity, so the entries and
    the forward equal the ungated form with s = 1 (gate logit +inf)."""
    sh = wl.LayerShape(B=2, T=19, W=5, d=16, H=2, Dh=8, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=42)
    x = f64_inputs(raw)
    eps = 1e-6
    kp = project(x["m_prime"], x["W_Km"], sh.H, sh.Dh)
    vm = project(x["m_prime"], x["W_Vm"], sh.H, sh.Dh)
    rows = kp.reshape(sh.B, sh.T, -1)
    ms = np.mean(rows ** 2, axis=-1, keepdims=True)
    factor = np.sqrt((1.0 - eps) / np.where(ms > 0, ms, 1.0))  # row t = 0 is zero (m'_0 = 0)
    kp = (rows * factor).reshape(kp.shape)
    zero = {n: np.zeros(sh.H * sh.Dh) for n in NAMES}
    kx, vx = oracle.gated_entries(x["k"], x["v"], kp, vm, zero, eps=eps)
    inf = np.full(sh.H, np.inf)
    ux, uv = oracle.mixed_entries(x["k"], x["v"], kp, vm, inf)
    np.testing.assert_allclose(kx, ux, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(vx, uv, rtol=1e-15, atol=0)
    o, lse = oracle.swa_attend_fwd(x["q"], kx, vx, sh.W)
    uo, ulse = oracle.swa_inject_fwd(x["q"], x["k"], x["v"], kp, vm, inf, sh.W)
    np.testing.assert_allclose(o, uo, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ulse, rtol=1e-12)


def test_gated_recurrent_gates_off_is_plain_swa():
    """a_kr = a_vr = -inf removes the memory; a_kl = a_vl = 0 keeps k, v as they are."""
    sh = wl.LayerShape(B=2, T=30, W=7, d=16, H=2, Dh=8, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=43)
    x = f64_inputs(raw)
    HD = sh.H * sh.Dh
    gates = {"a_kl": np.zeros(HD), "a_kr": np.full(HD, -np.inf),
             "a_vl": np.zeros(HD), "a_vr": np.full(HD, -np.inf)}
    o, lse = oracle.swa_inject_fwd_gated(x["q"], x["k"], x["v"], x["m_prime"], x["W_Km"],
                                         x["W_Vm"], gates, sh.W)
    pos = np.arange(sh.T)
    ro, rlse = sdpa_reference(rope_complex(x["q"], pos, 10000.0),
                              rope_complex(x["k"], pos, 10000.0), x["v"], sh.W)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=1e-11)


@pytest.mark.parametrize("T,W", [(29, 6), (16, 1), (20, 40)])
def test_attend_forward_matches_sdpa(T, W):
    """Attention over arbitrary given entries is torch SDPA with the band mask
    on the rotated queries."""
    rng = np.random.default_rng(44)
    B, H, Dh = 2, 3, 8
    q, kx, vx = (rng.standard_normal((B, T, H, Dh)) for _ in range(3))
    o, lse = oracle.swa_attend_fwd(q, kx, vx, W, pos0=7)
    ro, rlse = sdpa_reference(rope_complex(q, np.arange(T) + 7, 10000.0), kx, vx, W)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=1e-12)


def test_memory_key_scale_invariance():
    """With eps -> 0 the norm removes any per-row scale of the key projection:
    scaling W_Km leaves the output unchanged, while scaling W_Vm changes it."""
    sh = wl.LayerShape(B=1, T=17, W=5, d=16, H=2, Dh=8, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=45)
    x = f64_inputs(raw)
    gates = wl.gate_vectors(sh.H, sh.Dh, 45)
    run = lambda WK, WV: oracle.swa_inject_fwd_gated(x["q"], x["k"], x["v"], x["m_prime"], WK,
                                                     WV, gates, sh.W, eps=1e-30)[0]
    base = run(x["W_Km"], x["W_Vm"])
    np.testing.assert_allclose(run(37.0 * x["W_Km"], x["W_Vm"]), base, rtol=1e-11, atol=1e-12)
    assert np.max(np.abs(run(x["W_Km"], 3.0 * x["W_Vm"]) - base)) > 1e-3


def _gated_objective(x, gates, dO, W, pos0, base, eps):
    o, _ = oracle.swa_inject_fwd_gated(x["q"], x["k"], x["v"], x["m_prime"], x["W_Km"],
                                       x["W_Vm"], gates, W, pos0=pos0, rope_base=base, eps=eps)
    return float(np.sum(o * dO))


@pytest.mark.parametrize("W,pos0,base,eps", [(4, 0, 10000.0, 1e-6), (3, 5, 100.0, 0.5),
                                             (16, 0, 0.0, 1e-6)])
def test_gated_backward_matches_finite_differences(W, pos0, base, eps):
    sh = wl.LayerShape(B=1, T=12, W=W, d=8, H=2, Dh=4, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=46, grads=True)
    x = f64_inputs(raw)
    gates = {n: oracle.f64(a) for n, a in wl.gate_vectors(sh.H, sh.Dh, 46, std=1.0).items()}
    dO = oracle.f64(raw["dO"])
    g = oracle.swa_inject_bwd_gated(x["q"], x["k"], x["v"], x["m_prime"], x["W_Km"], x["W_Vm"],
                                    gates, dO, W, pos0=pos0, rope_base=base, eps=eps)
    h = 1e-6
    targets = [(x, n, "d" + n if n in ("q", "k", "v") else
                {"m_prime": "dm_prime", "W_Km": "dW_Km", "W_Vm": "dW_Vm"}[n])
               for n in ("q", "k", "v", "m_prime", "W_Km", "W_Vm")]
    targets += [(gates, n, "d" + n) for n in NAMES]
    for store, name, gname in targets:
        flat = store[name].reshape(-1)
        fd = np.empty(flat.size)
        for idx in range(flat.size):
            keep = flat[idx]
            flat[idx] = keep + h
            fp = _gated_objective(x, gates, dO, W, pos0, base, eps)
            flat[idx] = keep - h
            fm = _gated_objective(x, gates, dO, W, pos0, base, eps)
            flat[idx] = keep
            fd[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g[gname].reshape(-1), fd, rtol=1e-6, atol=1e-7, err_msg=gname)
    assert not g["dm_prime"][0, -1].any()


def _gated_stack_objective(layers, shared, W, eps):
    H, Dh = layers[0]["q"].shape[2], layers[0]["q"].shape[3]
    kp, vm = oracle.mem_project(shared["m_prime"], shared["W_Km"], shared["W_Vm"], H, Dh, shift=1)
    tot = 0.0
    for x in layers:
        kx, vx = oracle.gated_entries(x["k"], x["v"], kp, vm, x["gates"], eps=eps)
        o, _ = oracle.swa_attend_fwd(x["q"], kx, vx, W)
        tot += float(np.sum(o * x["dO"]))
    return tot


def test_gated_shared_projection_stack_matches_finite_differences():
    """Two gated layers over one projection of the same m' by the same
    weights, each with its own q, k, v, gates and dO: every gradient of the
    summed objective, the forward composed from the projection, the gated mix
    and the attention oracle (not from the backward's own composition)."""
    sh = wl.LayerShape(B=1, T=10, W=3, d=8, H=2, Dh=4, dtype=wl.F32)
    eps = 1e-6
    raws = [wl.layer_inputs(sh, seed=70 + l, grads=True) for l in range(2)]
    layers = []
    for l, r in enumerate(raws):
        x = {n: oracle.f64(r[n]) for n in ("q", "k", "v", "dO")}
        x["gates"] = {n: oracle.f64(a) for n, a in wl.gate_vectors(sh.H, sh.Dh, 70 + l, std=1.0).items()}
        layers.append(x)
    shared = {n: oracle.f64(raws[0][n]) for n in ("m_prime", "W_Km", "W_Vm")}
    per, sg = oracle.swa_inject_bwd_shared_gated(layers, shared["m_prime"], shared["W_Km"],
                                                 shared["W_Vm"], sh.W, eps=eps)
    h = 1e-6

    def fd(store, name):
        flat = store[name].reshape(-1)
        out = np.empty(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + h
            fp = _gated_stack_objective(layers, shared, sh.W, eps)
            flat[i] = keep - h
            fm = _gated_stack_objective(layers, shared, sh.W, eps)
            flat[i] = keep
            out[i] = (fp - fm) / (2 * h)
        return out.reshape(store[name].shape)

    for name, gname in (("m_prime", "dm_prime"), ("W_Km", "dW_Km"), ("W_Vm", "dW_Vm")):
        np.testing.assert_allclose(sg[gname], fd(shared, name), rtol=1e-6, atol=1e-7, err_msg=gname)
    for l in range(2):
        for name in ("q", "k", "v"):
            np.testing.assert_allclose(per[l]["d" + name], fd(layers[l], name), rtol=1e-6,
                                       atol=1e-7, err_msg="layer %d d%s" % (l, name))
        for n in NAMES:
            np.testing.assert_allclose(per[l]["d" + n], fd(layers[l]["gates"], n), rtol=1e-6,
                                       atol=1e-7, err_msg="layer %d d%s" % (l, n))
    # both layers really reach the shared parameters
    _, first = oracle.swa_inject_bwd_shared_gated(layers[:1], shared["m_prime"], shared["W_Km"],
                                                  shared["W_Vm"], sh.W, eps=eps)
    assert np.max(np.abs(sg["dW_Km"] - first["dW_Km"])) > 1e-3


def test_gated_backward_matches_torch_autograd_dense():
    """Torch fp64 autograd through a dense masked-softmax layer with the gated
    mix written from library ops (torch.rsqrt, complex rotation, sigmoid)."""
    sh = wl.LayerShape(B=2, T=21, W=6, d=12, H=3, Dh=4, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=47, grads=True)
    gv = wl.gate_vectors(sh.H, sh.Dh, 47, std=1.0)
    eps = 1e-6
    t = {n: raw[n].to(torch.float64).clone().requires_grad_(True)
         for n in ("q", "k", "v", "m_prime", "W_Km", "W_Vm")}
    for n in NAMES:
        t[n] = gv[n].to(torch.float64).clone().requires_grad_(True)
    dO = raw["dO"].to(torch.float64)
    B, T, H, Dh, d = sh.B, sh.T, sh.H, sh.Dh, sh.d
    half = Dh // 2
    inv = 10000.0 ** (-torch.arange(half, dtype=torch.float64) * 2.0 / Dh)
    rot = torch.polar(torch.ones(T, half, dtype=torch.float64),
                      torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :])

    def rope(x):
        z = torch.complex(x[..., :half], x[..., half:]) * rot[None, :, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    mprev = torch.cat([torch.zeros(B, 1, d, dtype=torch.float64), t["m_prime"][:, :-1]], dim=1)
    kp = mprev @ t["W_Km"].T                                    # [B,T,H*Dh]
    kn = (kp * torch.rsqrt(kp.pow(2).mean(-1, keepdim=True) + eps)).reshape(B, T, H, Dh)
    vm = (mprev @ t["W_Vm"].T).reshape(B, T, H, Dh)
    g = {n: (2 * torch.sigmoid(t[n])).reshape(H, Dh) for n in NAMES}
    Q = rope(t["q"]).permute(0, 2, 1, 3)
    K = (g["a_kl"] * rope(t["k"]) + g["a_kr"] * rope(kn)).permute(0, 2, 1, 3)
    V = (g["a_vl"] * t["v"] + g["a_vr"] * vm).permute(0, 2, 1, 3)
    S = (Q @ K.transpose(-1, -2)) / math.sqrt(Dh)
    S = S.masked_fill(~band_mask(T, sh.W), float("-inf"))
    O = torch.softmax(S, dim=-1) @ V
    (O.permute(0, 2, 1, 3) * dO).sum().backward()
    r = oracle.swa_inject_bwd_gated(raw["q"], raw["k"], raw["v"], raw["m_prime"], raw["W_Km"],
                                    raw["W_Vm"], gv, raw["dO"], sh.W, eps=eps)
    pairs = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("m_prime", "dm_prime"),
             ("W_Km", "dW_Km"), ("W_Vm", "dW_Vm")] + [(n, "d" + n) for n in NAMES]
    for name, gname in pairs:
        np.testing.assert_allclose(r[gname], t[name].grad.numpy(), rtol=1e-10, atol=1e-11,
                                   err_msg=gname)


def test_gated_backward_value_gates_closed_form():
    """W = 1: O = v~ exactly, so dv = g_vl dO, dq = dk = 0, and
    d/da_vl = 2 s (1 - s) sum_t dO (.) v per channel."""
    sh = wl.LayerShape(B=2, T=9, W=1, d=8, H=2, Dh=4, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=48, grads=True)
    gates = {n: oracle.f64(a) for n, a in wl.gate_vectors(sh.H, sh.Dh, 48).items()}
    r = oracle.swa_inject_bwd_gated(raw["q"], raw["k"], raw["v"], raw["m_prime"], raw["W_Km"],
                                    raw["W_Vm"], gates, raw["dO"], 1)
    dO, v = oracle.f64(raw["dO"]), oracle.f64(raw["v"])
    s = expit(gates["a_vl"]).reshape(sh.H, sh.Dh)
    np.testing.assert_allclose(r["dv"], 2 * s * dO, rtol=1e-14)
    assert not r["dq"].any() and not r["dk"].any()
    want = (2 * s * (1 - s) * np.sum(dO * v, axis=(0, 1))).reshape(-1)
    np.testing.assert_allclose(r["da_vl"], want, rtol=1e-12, atol=1e-14)


def test_gated_decode_from_empty_ring_equals_lifted_pass():
    """Decoding positions 0..T-1 from an empty ring with the same shifted
    memory reproduces the gated parallel pass row by row (exact ring)."""
    sh = wl.LayerShape(B=2, T=21, W=6, d=16, H=2, Dh=8, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=49)
    x = f64_inputs(raw)
    gates = wl.gate_vectors(sh.H, sh.Dh, 49, std=1.0)
    o_par, _ = oracle.swa_inject_fwd_gated(x["q"], x["k"], x["v"], x["m_prime"], x["W_Km"],
                                           x["W_Vm"], gates, sh.W)
    kp, vm = oracle.mem_project(x["m_prime"], x["W_Km"], x["W_Vm"], sh.H, sh.Dh, shift=1)
    kc = np.zeros((sh.B, sh.H, sh.W, sh.Dh))
    vc = np.zeros_like(kc)
    for t in range(sh.T):
        o_t = oracle.decode_step_gated(x["q"][:, t], x["k"][:, t], x["v"][:, t], kp[:, t],
                                       vm[:, t], gates, kc, vc, np.full(sh.B, t),
                                       ring_bf16=False)
        np.testing.assert_allclose(o_t, o_par[:, t], rtol=1e-12, atol=1e-13)


def test_gated_decode_ring_entry_matches_numpy_and_rounds():
    """The entry written to slot pos mod W is the numpy gated mix at that
    position, rounded to bf16 by torch's conversion when the ring is bf16."""
    Bs, H, Dh, W = 3, 2, 8, 5
    rng = np.random.default_rng(50)
    q, k, v, kp, vm = (rng.standard_normal((Bs, H, Dh)) for _ in range(5))
    gates = {n: rng.standard_normal(H * Dh) for n in NAMES}
    pos = np.array([0, 7, 123])
    kc = np.zeros((Bs, H, W, Dh))
    vc = np.zeros_like(kc)
    oracle.decode_step_gated(q, k, v, kp, vm, gates, kc, vc, pos)
    for b in range(Bs):
        rk, rv = numpy_gated(k[b][None, None], v[b][None, None], kp[b][None, None],
                             vm[b][None, None], gates, np.array([pos[b]]), 10000.0, 1e-6)
        want_k = torch.from_numpy(rk[0, 0]).to(torch.bfloat16).double().numpy()
        want_v = torch.from_numpy(rv[0, 0]).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(kc[b, :, pos[b] % W], want_k)
        np.testing.assert_array_equal(vc[b, :, pos[b] % W], want_v)
