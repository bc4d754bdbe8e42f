"""Pins for the CPU oracle: each check compares it with something other than
itself -- a library routine (torch's scaled_dot_product_attention, numpy's
complex arithmetic and matmul, torch.logsumexp, torch's bf16 conversion), a
closed form, an invariant the pages state, or central finite differences.

The pages print no worked numerical example for this path, so no pin uses
printed values; the choice of RoPE pairing/sign and softmax scale is a stated
convention that only the oracle and the kernels share (pages-unpinned).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import workloads as wl


# ----------------------------------------------------------------------------
# independent helpers built from library routines
# ----------------------------------------------------------------------------
def rope_complex(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotation as complex multiplication: channel pair (i, i+Dh/2) is the
    complex number x_i + 1j*x_{i+Dh/2}, multiplied by exp(1j*pos*base^(-2i/Dh)).
    x: [..., T, H, Dh]; pos: [T]."""
    if base <= 0:
        return x.copy()
    Dh = x.shape[-1]
    half = Dh // 2
    z = x[..., :half] + 1j * x[..., half:]
    inv = np.power(float(base), -np.arange(half) * 2.0 / Dh)
    ang = np.exp(1j * np.outer(pos.astype(np.float64), inv))  # [T, half]
    z = z * ang[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def shifted(m: np.ndarray) -> np.ndarray:
    out = np.zeros_like(m)
    out[:, 1:] = m[:, :-1]
    return out


def project(m, W, H, Dh, shift=1):
    x = shifted(m) if shift else m
    B, T, _ = x.shape
    return (x @ W.T).reshape(B, T, H, Dh)


def band_mask(T, W):
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    return (j <= i) & (i - j < W)


def sdpa_reference(qh, kt, vt, W, scale=None):
    """torch SDPA over [B,T,H,Dh] float64 inputs with the sliding band mask."""
    B, T, H, Dh = qh.shape
    Q = torch.from_numpy(qh).permute(0, 2, 1, 3)
    K = torch.from_numpy(kt).permute(0, 2, 1, 3)
    V = torch.from_numpy(vt).permute(0, 2, 1, 3)
    mask = band_mask(T, W)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    s = (Q @ K.transpose(-1, -2)) * (scale if scale else 1.0 / math.sqrt(Dh))
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)  # [B,H,T]
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


def mixed_reference(inp, W, pos0=0, base=10000.0):
    q, k, v = (oracle.f64(inp[n]) for n in ("q", "k", "v"))
    mp, WK, WV = (oracle.f64(inp[n]) for n in ("m_prime", "W_Km", "W_Vm"))
    g = oracle.f64(inp["gate_logit"])
    B, T, H, Dh = q.shape
    s = expit(g)[None, None, :, None]
    pos = np.arange(T) + pos0
    kmem = project(mp, WK, H, Dh)
    vmem = project(mp, WV, H, Dh)
    qh = rope_complex(q, pos, base)
    kt = rope_complex(k, pos, base) + s * rope_complex(kmem, pos, base)
    vt = v + s * vmem
    return qh, kt, vt, kmem, vmem


def small_shape(B=2, T=37, W=5, d=24, H=2, Dh=8, dtype=wl.F32):
    return wl.LayerShape(B=B, T=T, W=W, d=d, H=H, Dh=Dh, dtype=dtype)


def run_oracle_fwd(inp, W, pos0=0, base=10000.0, H=None, Dh=None):
    q = inp["q"]
    H, Dh = q.shape[2], q.shape[3]
    kmem, vmem = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], H, Dh, shift=1)
    return oracle.swa_inject_fwd(q, inp["k"], inp["v"], kmem, vmem, inp["gate_logit"], W,
                                 pos0=pos0, rope_base=base), kmem, vmem


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ----------------------------------------------------------------------------
# projection and shift
# ----------------------------------------------------------------------------
def test_projection_matches_numpy_matmul():
    sh = small_shape()
    inp = wl.layer_inputs(sh, seed=11)
    km, vm = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], sh.H, sh.Dh, shift=1)
    mp, WK, WV = (oracle.f64(inp[n]) for n in ("m_prime", "W_Km", "W_Vm"))
    np.testing.assert_allclose(km, project(mp, WK, sh.H, sh.Dh), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(vm, project(mp, WV, sh.H, sh.Dh), rtol=1e-12, atol=1e-12)
    km0, _ = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], sh.H, sh.Dh, shift=0)
    np.testing.assert_allclose(km0, project(mp, WK, sh.H, sh.Dh, shift=0), rtol=1e-12, atol=1e-12)


def test_one_hot_memory_injects_only_into_next_key():
    """m' = e_r at row t0 only: the shift moves it to key t0+1, where kmem
    equals column r of W_Km; every other row is exactly zero, row 0 included."""
    B, T, d, H, Dh = 1, 12, 16, 2, 8
    t0, r = 5, 3
    m = np.zeros((B, T, d))
    m[0, t0, r] = 1.0
    rng = np.random.default_rng(0)
    WK = rng.standard_normal((H * Dh, d))
    WV = rng.standard_normal((H * Dh, d))
    km, vm = oracle.mem_project(m, WK, WV, H, Dh, shift=1)
    for t in range(T):
        if t == t0 + 1:
            np.testing.assert_array_equal(km[0, t].reshape(-1), WK[:, r])
            np.testing.assert_array_equal(vm[0, t].reshape(-1), WV[:, r])
        else:
            assert not km[0, t].any() and not vm[0, t].any()


# ----------------------------------------------------------------------------
# forward against torch SDPA with an independent rotation
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,W", [(37, 5), (64, 1), (50, 50), (50, 200), (33, 2)])
def test_forward_matches_sdpa_with_band_mask(T, W):
    sh = small_shape(T=T, W=W)
    inp = wl.layer_inputs(sh, seed=100 + T + W)
    (o, lse), _, _ = run_oracle_fwd(inp, W)
    qh, kt, vt, _, _ = mixed_reference(inp, W)
    o_ref, lse_ref = sdpa_reference(qh, kt, vt, W)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-10, atol=1e-11)


def test_gate_minus_inf_is_plain_swa():
    """s = 0: the memory path vanishes and the layer is plain RoPE SWA."""
    sh = small_shape(T=40, W=7)
    inp = wl.layer_inputs(sh, seed=5)
    inp["gate_logit"] = torch.full((sh.H,), float("-inf"))
    (o, lse), _, _ = run_oracle_fwd(inp, sh.W)
    q, k, v = (oracle.f64(inp[n]) for n in ("q", "k", "v"))
    pos = np.arange(sh.T)
    o_ref, lse_ref = sdpa_reference(rope_complex(q, pos, 1e4), rope_complex(k, pos, 1e4), v, sh.W)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-10, atol=1e-11)


def test_window_covering_sequence_is_full_causal():
    sh = small_shape(T=30, W=30)
    inp = wl.layer_inputs(sh, seed=6)
    (o, _), _, _ = run_oracle_fwd(inp, sh.W)
    qh, kt, vt, _, _ = mixed_reference(inp, sh.W)
    Q, K, V = (torch.from_numpy(a).permute(0, 2, 1, 3) for a in (qh, kt, vt))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    (o_big, _), _, _ = run_oracle_fwd(inp, 10 * sh.T)
    np.testing.assert_array_equal(o, o_big)


def test_window_one_returns_mixed_value():
    """W = 1: softmax over one key, so O = v + s*vmem exactly and lse = S_ii."""
    sh = small_shape(T=20, W=1)
    inp = wl.layer_inputs(sh, seed=7)
    (o, lse), kmem, vmem = run_oracle_fwd(inp, 1)
    s = expit(oracle.f64(inp["gate_logit"]))[None, None, :, None]
    np.testing.assert_allclose(o, oracle.f64(inp["v"]) + s * vmem, rtol=1e-14, atol=1e-14)
    qh, kt, _, _, _ = mixed_reference(inp, 1)
    sii = np.einsum("bthc,bthc->bht", qh, kt) / math.sqrt(sh.Dh)
    np.testing.assert_allclose(lse, sii, rtol=1e-11, atol=1e-11)


def test_rope_closed_form_two_channels():
    """Dh = 2, q = k = (1, 0), no memory: theta_0 = 1 so S_ij = cos(i - j)/sqrt(2)."""
    T, W = 3, 2
    q = np.zeros((1, T, 1, 2)); q[..., 0] = 1.0
    k = q.copy()
    v = np.zeros((1, T, 1, 2)); v[0, :, 0, 0] = [1.0, 2.0, 3.0]
    zeros = np.zeros_like(q)
    o, lse = oracle.swa_inject_fwd(q, k, v, zeros, zeros, np.array([0.0]), W, rope_base=10000.0)
    sc = 1.0 / math.sqrt(2.0)
    a, b = math.exp(sc * math.cos(1.0)), math.exp(sc * math.cos(0.0))
    assert o[0, 1, 0, 0] == pytest.approx((1.0 * a + 2.0 * b) / (a + b), rel=1e-14)
    assert o[0, 2, 0, 0] == pytest.approx((2.0 * a + 3.0 * b) / (a + b), rel=1e-14)
    assert lse[0, 0, 2] == pytest.approx(math.log(a + b), rel=1e-14)
    assert o[0, 0, 0, 0] == 1.0


@pytest.mark.parametrize("c", [1, 97, 4096])
def test_relative_position_invariance(c):
    """Scores depend only on the offset i - j, so shifting every position by c
    leaves the outputs unchanged (to fp64 round-off of the angles)."""
    sh = small_shape(T=29, W=6)
    inp = wl.layer_inputs(sh, seed=8)
    (o0, l0), _, _ = run_oracle_fwd(inp, sh.W, pos0=0)
    (o1, l1), _, _ = run_oracle_fwd(inp, sh.W, pos0=c)
    np.testing.assert_allclose(o1, o0, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(l1, l0, rtol=1e-9, atol=1e-9)


def test_memory_key_rotated_at_local_key_position():
    """k = v = 0 and s = 1: attention runs over memories only, and must equal
    SDPA on (R_i q, R_j kmem_j, vmem_j) -- the memory key is rotated at the
    position of the key it joins, not at the position it was produced."""
    sh = small_shape(T=24, W=6)
    inp = wl.layer_inputs(sh, seed=9)
    inp["k"] = torch.zeros_like(inp["k"])
    inp["v"] = torch.zeros_like(inp["v"])
    inp["gate_logit"] = torch.full((sh.H,), 40.0)  # sigma = 1 in fp64
    assert expit(40.0) == 1.0
    (o, _), kmem, vmem = run_oracle_fwd(inp, sh.W)
    pos = np.arange(sh.T)
    q = oracle.f64(inp["q"])
    o_ref, _ = sdpa_reference(rope_complex(q, pos, 1e4), rope_complex(kmem, pos, 1e4), vmem, sh.W)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-11)
    # rotating the memory at its source position (j - 1) would give a different answer
    shifted_pos = np.maximum(pos - 1, 0)
    o_bad, _ = sdpa_reference(rope_complex(q, pos, 1e4), rope_complex(kmem, shifted_pos, 1e4), vmem, sh.W)
    assert np.abs(o - o_bad).max() > 1e-3


# ----------------------------------------------------------------------------
# mixed cache entries
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("pos0,base", [(0, 10000.0), (1000, 10000.0), (5, 0.0)])
def test_mixed_entries_match_complex_rotation(pos0, base):
    """k~ = R k + s R kmem and v~ = v + s vmem against numpy's complex rotation."""
    sh = small_shape(T=23, W=5)
    inp = wl.layer_inputs(sh, seed=12)
    km, vm = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], sh.H, sh.Dh, shift=1)
    kx, vx = oracle.mixed_entries(inp["k"], inp["v"], km, vm, inp["gate_logit"], pos0, base)
    pos = np.arange(sh.T) + pos0
    s = expit(oracle.f64(inp["gate_logit"]))[None, None, :, None]
    k, v = oracle.f64(inp["k"]), oracle.f64(inp["v"])
    np.testing.assert_allclose(kx, rope_complex(k, pos, base) + s * rope_complex(km, pos, base),
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(vx, v + s * vm, rtol=1e-14, atol=1e-15)


def test_mixed_entries_gate_limits():
    """s = 0 leaves the rotated local entry; s = 1 with k = v = 0 leaves the
    rotated memory entry."""
    sh = small_shape(T=17, W=5)
    inp = wl.layer_inputs(sh, seed=13)
    km, vm = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], sh.H, sh.Dh, shift=1)
    pos = np.arange(sh.T)
    kx, vx = oracle.mixed_entries(inp["k"], inp["v"], km, vm, np.full(sh.H, -np.inf))
    np.testing.assert_allclose(kx, rope_complex(oracle.f64(inp["k"]), pos, 1e4), rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(vx, oracle.f64(inp["v"]))
    z = np.zeros((sh.B, sh.T, sh.H, sh.Dh))
    kx, vx = oracle.mixed_entries(z, z, km, vm, np.full(sh.H, 40.0))
    np.testing.assert_allclose(kx, rope_complex(km, pos, 1e4), rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(vx, vm)


def test_forward_is_attention_over_mixed_entries():
    """The forward equals band-masked SDPA of (R q, k~, v~) with k~, v~ taken
    from the mixed-entries function: the two oracle functions agree."""
    sh = small_shape(T=31, W=6)
    inp = wl.layer_inputs(sh, seed=14)
    (o, lse), km, vm = run_oracle_fwd(inp, sh.W, pos0=7)
    kx, vx = oracle.mixed_entries(inp["k"], inp["v"], km, vm, inp["gate_logit"], 7)
    qh = rope_complex(oracle.f64(inp["q"]), np.arange(sh.T) + 7, 1e4)
    o_ref, lse_ref = sdpa_reference(qh, kx, vx, sh.W)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-10, atol=1e-11)


def test_fwd_rows_equal_full_forward():
    sh = small_shape(T=45, W=9)
    inp = wl.layer_inputs(sh, seed=10)
    (o, lse), kmem, vmem = run_oracle_fwd(inp, sh.W, pos0=3)
    rows = np.array([[0, 0, 0], [1, 1, 44], [0, 1, 8], [1, 0, 9], [1, 1, 20]])
    orow, lrow = oracle.swa_inject_fwd_rows(inp["q"], inp["k"], inp["v"], kmem, vmem,
                                            inp["gate_logit"], sh.W, rows, pos0=3)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(orow[n], o[b, i, h], rtol=1e-13, atol=1e-14)
        assert lrow[n] == pytest.approx(lse[b, h, i], rel=1e-13)


# ----------------------------------------------------------------------------
# backward: central finite differences of the whole layer path
# ----------------------------------------------------------------------------
def _layer_objective(x, dO, W, pos0, base):
    H, Dh = x["q"].shape[2], x["q"].shape[3]
    km, vm = oracle.mem_project(x["m_prime"], x["W_Km"], x["W_Vm"], H, Dh, shift=1)
    o, _ = oracle.swa_inject_fwd(x["q"], x["k"], x["v"], km, vm, x["gate_logit"], W,
                                 pos0=pos0, rope_base=base)
    return float(np.sum(o * dO))


@pytest.mark.parametrize("W,pos0,base", [(4, 0, 10000.0), (3, 5, 100.0), (16, 0, 0.0)])
def test_backward_matches_finite_differences(W, pos0, base):
    sh = wl.LayerShape(B=1, T=16, W=W, d=16, H=2, Dh=8, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=21, grads=True)
    x = {n: oracle.f64(raw[n]) for n in ("q", "k", "v", "m_prime", "W_Km", "W_Vm", "gate_logit")}
    dO = oracle.f64(raw["dO"])
    g = oracle.swa_inject_bwd(x["q"], x["k"], x["v"], x["m_prime"], x["W_Km"], x["W_Vm"],
                              x["gate_logit"], dO, W, pos0=pos0, rope_base=base)
    names = {"q": "dq", "k": "dk", "v": "dv", "m_prime": "dm_prime", "W_Km": "dW_Km",
             "W_Vm": "dW_Vm", "gate_logit": "dgate"}
    eps = 1e-6
    for name, gname in names.items():
        fd = np.empty_like(x[name])
        flat = x[name].reshape(-1)
        for idx in range(flat.size):
            keep = flat[idx]
            flat[idx] = keep + eps
            fp = _layer_objective(x, dO, W, pos0, base)
            flat[idx] = keep - eps
            fm = _layer_objective(x, dO, W, pos0, base)
            flat[idx] = keep
            fd.reshape(-1)[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-7, err_msg=gname)
    assert not g["dm_prime"][0, -1].any()  # m'_T is never consumed


def test_backward_matches_torch_autograd_dense():
    """A second, structurally different check: torch fp64 autograd through a
    dense masked-softmax layer built from library ops."""
    sh = wl.LayerShape(B=2, T=23, W=6, d=12, H=3, Dh=4, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=22, grads=True)
    t = {n: raw[n].to(torch.float64).clone().requires_grad_(True)
         for n in ("q", "k", "v", "m_prime", "W_Km", "W_Vm", "gate_logit")}
    dO = raw["dO"].to(torch.float64)
    B, T, H, Dh, d = sh.B, sh.T, sh.H, sh.Dh, sh.d
    pos = torch.arange(T, dtype=torch.float64)
    half = Dh // 2
    inv = 10000.0 ** (-torch.arange(half, dtype=torch.float64) * 2.0 / Dh)
    rot = torch.polar(torch.ones(T, half, dtype=torch.float64), pos[:, None] * inv[None, :])

    def rope(x):
        z = torch.complex(x[..., :half], x[..., half:]) * rot[None, :, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    mprev = torch.cat([torch.zeros(B, 1, d, dtype=torch.float64), t["m_prime"][:, :-1]], dim=1)
    km = (mprev @ t["W_Km"].T).reshape(B, T, H, Dh)
    vm = (mprev @ t["W_Vm"].T).reshape(B, T, H, Dh)
    s = torch.sigmoid(t["gate_logit"])[None, None, :, None]
    Q = rope(t["q"]).permute(0, 2, 1, 3)
    K = (rope(t["k"]) + s * rope(km)).permute(0, 2, 1, 3)
    V = (t["v"] + s * vm).permute(0, 2, 1, 3)
    S = (Q @ K.transpose(-1, -2)) / math.sqrt(Dh)
    S = S.masked_fill(~band_mask(T, sh.W), float("-inf"))
    O = torch.softmax(S, dim=-1) @ V
    (O.permute(0, 2, 1, 3) * dO).sum().backward()
    g = oracle.swa_inject_bwd(raw["q"], raw["k"], raw["v"], raw["m_prime"], raw["W_Km"],
                              raw["W_Vm"], raw["gate_logit"], raw["dO"], sh.W)
    for name, gname in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("m_prime", "dm_prime"),
                        ("W_Km", "dW_Km"), ("W_Vm", "dW_Vm"), ("gate_logit", "dgate")]:
        np.testing.assert_allclose(g[gname], t[name].grad.numpy(), rtol=1e-10, atol=1e-11,
                                   err_msg=gname)


def test_backward_window_one_closed_form():
    """W = 1: O = v~, so dq = dk = 0 and dv = dO exactly."""
    sh = wl.LayerShape(B=1, T=10, W=1, d=8, H=2, Dh=4, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=23, grads=True)
    g = oracle.swa_inject_bwd(raw["q"], raw["k"], raw["v"], raw["m_prime"], raw["W_Km"],
                              raw["W_Vm"], raw["gate_logit"], raw["dO"], 1)
    assert np.abs(g["dq"]).max() < 1e-13 and np.abs(g["dk"]).max() < 1e-13
    np.testing.assert_array_equal(g["dv"], oracle.f64(raw["dO"]))


def test_backward_gate_minus_inf_has_no_memory_gradient():
    sh = wl.LayerShape(B=1, T=12, W=4, d=8, H=2, Dh=4, dtype=wl.F32)
    raw = wl.layer_inputs(sh, seed=24, grads=True)
    raw["gate_logit"] = torch.full((2,), float("-inf"))
    g = oracle.swa_inject_bwd(raw["q"], raw["k"], raw["v"], raw["m_prime"], raw["W_Km"],
                              raw["W_Vm"], raw["gate_logit"], raw["dO"], 4)
    for n in ("dm_prime", "dW_Km", "dW_Vm", "dgate"):
        assert not g[n].any(), n


# ----------------------------------------------------------------------------
# consistency loss
# ----------------------------------------------------------------------------
def test_loss_zero_when_memories_agree():
    m = np.random.default_rng(1).standard_normal((3, 7, 16))
    L, dm, dmp = oracle.consistency_loss(m, m.copy(), 0.7)
    assert L == 0.0 and not dm.any() and not dmp.any()


def test_loss_constant_offset_closed_form():
    """m - m' = c everywhere: L = lam * N * d * c^2 / (N sqrt d) = lam c^2 sqrt(d)."""
    rng = np.random.default_rng(2)
    mp = rng.standard_normal((2, 9, 64))
    c, lam = 0.375, 0.1
    L, dm, dmp = oracle.consistency_loss(mp + c, mp, lam)
    assert L == pytest.approx(lam * c * c * 8.0, rel=1e-13)
    np.testing.assert_allclose(dm, 2 * lam * c / (18 * 8.0), rtol=1e-12)
    np.testing.assert_array_equal(dmp, -dm)


def test_loss_gradient_finite_differences():
    rng = np.random.default_rng(3)
    m = rng.standard_normal((1, 5, 6))
    mp = rng.standard_normal((1, 5, 6))
    lam = 1.3
    _, dm, _ = oracle.consistency_loss(m, mp, lam)
    eps = 1e-6
    fd = np.empty_like(m)
    for idx in np.ndindex(m.shape):
        a = m.copy(); a[idx] += eps
        b = m.copy(); b[idx] -= eps
        fd[idx] = (oracle.consistency_loss(a, mp, lam)[0] - oracle.consistency_loss(b, mp, lam)[0]) / (2 * eps)
    np.testing.assert_allclose(dm, fd, rtol=1e-6, atol=1e-8)  # central-difference round-off ~1e-9


def test_loss_expectation_for_independent_normals():
    """For independent N(0,1) m, m': E[(m - m')^2] = 2, so E[L] = 2 lam sqrt(d)
    (statistical, loose): 16.0 for the tiny fp32 workload."""
    sh = wl.TINY_FP32
    inp = wl.layer_inputs(sh, seed=0)
    L, _, _ = oracle.consistency_loss(inp["m"], inp["m_prime"], sh.lam)
    assert abs(L - 2 * sh.lam * math.sqrt(sh.d)) < 0.5


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def test_decode_from_empty_ring_equals_lifted_pass():
    """Decoding positions 0..T-1 from an empty ring, fed the same shifted
    memory, reproduces the parallel pass row by row (exact ring, no rounding)."""
    sh = small_shape(B=2, T=21, W=6, d=16, H=2, Dh=8)
    inp = wl.layer_inputs(sh, seed=30)
    (o_par, _), kmem, vmem = run_oracle_fwd(inp, sh.W)
    kc = np.zeros((sh.B, sh.H, sh.W, sh.Dh))
    vc = np.zeros_like(kc)
    q, k, v = (oracle.f64(inp[n]) for n in ("q", "k", "v"))
    for t in range(sh.T):
        o_t = oracle.decode_step(q[:, t], k[:, t], v[:, t], kmem[:, t], vmem[:, t],
                                 inp["gate_logit"], kc, vc, np.full(sh.B, t), ring_bf16=False)
        np.testing.assert_allclose(o_t, o_par[:, t], rtol=1e-12, atol=1e-13)


def test_decode_ring_slot_is_position_mod_W():
    """No rotation, s = 0: entries are copied verbatim, so after n steps slot
    p mod W holds exactly the marker of the newest position p with that residue."""
    Bs, H, Dh, W = 2, 2, 8, 5
    kc = np.full((Bs, H, W, Dh), -7.0)
    vc = np.full((Bs, H, W, Dh), -7.0)
    z = np.zeros((Bs, H, Dh))
    gate = np.full(H, -np.inf)
    n = 3 * W + 2
    for p in range(n):
        mk = wl.marker_values(torch.full((Bs * H,), p), Dh, tag=1.0).numpy().reshape(Bs, H, Dh)
        oracle.decode_step(z, mk, mk, z, z, gate, kc, vc, np.full(Bs, p), rope_base=0.0)
    for s in range(W):
        newest = max(p for p in range(n) if p % W == s)
        want = wl.marker_values(torch.tensor([newest]), Dh, tag=1.0).numpy()[0]
        np.testing.assert_array_equal(kc[:, :, s], np.broadcast_to(want, (Bs, H, Dh)))


def test_decode_first_steps_ignore_invalid_slots():
    """At position p < W-1 only slots 0..p are valid: garbage in later slots
    must not leak into the output, which is then the average-free softmax of
    the valid entries (checked against SDPA on those entries)."""
    Bs, H, Dh, W = 1, 1, 4, 8
    rng = np.random.default_rng(4)
    kc = rng.standard_normal((Bs, H, W, Dh)) * 50
    vc = rng.standard_normal((Bs, H, W, Dh)) * 50
    kc_valid = []
    for p in range(3):
        q, k, v = (rng.standard_normal((Bs, H, Dh)) for _ in range(3))
        z = np.zeros_like(q)
        o = oracle.decode_step(q, k, v, z, z, np.array([-np.inf]), kc, vc, [p], rope_base=0.0,
                               ring_bf16=False)
        Q = torch.from_numpy(q[:, :, None, :])
        K = torch.from_numpy(kc[:, :, : p + 1])
        V = torch.from_numpy(vc[:, :, : p + 1])
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[:, :, 0]
        np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_round_bf16_matches_torch_conversion():
    x = torch.randn(20000, generator=torch.Generator().manual_seed(5)) * 3.0
    x = torch.cat([x, torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, 1e-40])])
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_bf16(float(a)) for a in x.to(torch.float64)])
    np.testing.assert_array_equal(got, ref)


def test_golden_tiny_fp32_unchanged():
    """The oracle still reproduces the stored tiny-workload values (written by
    tests/golden/make_golden.py from the oracle alone)."""
    import json
    import os
    import sys

    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, here)
    try:
        import make_golden
    finally:
        sys.path.remove(here)
    with open(os.path.join(here, "tiny_fp32_seed0.json")) as f:
        stored = json.load(f)
    now = make_golden.compute()
    np.testing.assert_allclose(now["lse"], stored["lse"], rtol=1e-12, atol=1e-12)
    for t, row in stored["o_rows"].items():
        np.testing.assert_allclose(now["o_rows"][t], row, rtol=1e-12, atol=1e-12)
    assert now["loss"] == pytest.approx(stored["loss"], rel=1e-12)


# ----------------------------------------------------------------------------
# layers sharing one memory projection
# ----------------------------------------------------------------------------
def _stack_objective(layers, shared, W):
    H, Dh = layers[0]["q"].shape[2], layers[0]["q"].shape[3]
    km, vm = oracle.mem_project(shared["m_prime"], shared["W_Km"], shared["W_Vm"], H, Dh, shift=1)
    tot = 0.0
    for x in layers:
        o, _ = oracle.swa_inject_fwd(x["q"], x["k"], x["v"], km, vm, x["gate_logit"], W)
        tot += float(np.sum(o * x["dO"]))
    return tot


def test_shared_projection_stack_matches_finite_differences():
    """Two layers, one projection of the same m' by the same weights, their
    own q, k, v, gates and dO: every gradient of the summed objective."""
    sh = wl.LayerShape(B=1, T=10, W=3, d=8, H=2, Dh=4, dtype=wl.F32)
    raws = [wl.layer_inputs(sh, seed=60 + l, grads=True) for l in range(2)]
    layers = [{n: oracle.f64(r[n]) for n in ("q", "k", "v", "gate_logit", "dO")} for r in raws]
    shared = {n: oracle.f64(raws[0][n]) for n in ("m_prime", "W_Km", "W_Vm")}
    per, sg = oracle.swa_inject_bwd_shared(layers, shared["m_prime"], shared["W_Km"],
                                           shared["W_Vm"], sh.W)
    h = 1e-6

    def fd(store, name):
        flat = store[name].reshape(-1)
        out = np.empty(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + h
            fp = _stack_objective(layers, shared, sh.W)
            flat[i] = keep - h
            fm = _stack_objective(layers, shared, sh.W)
            flat[i] = keep
            out[i] = (fp - fm) / (2 * h)
        return out.reshape(store[name].shape)

    for name, gname in (("m_prime", "dm_prime"), ("W_Km", "dW_Km"), ("W_Vm", "dW_Vm")):
        np.testing.assert_allclose(sg[gname], fd(shared, name), rtol=1e-6, atol=1e-7, err_msg=gname)
    for l in range(2):
        for name in ("q", "k", "v", "gate_logit"):
            gname = "dgate" if name == "gate_logit" else "d" + name
            np.testing.assert_allclose(per[l][gname], fd(layers[l], name), rtol=1e-6, atol=1e-7,
                                       err_msg="layer %d %s" % (l, gname))


def test_nonfinite_value_reaches_exactly_the_band():
    """The oracle's reading of the band: query i attends to keys
    i-W+1..i only, so a NaN in value row j reaches exactly the outputs of
    rows j..j+W-1 (and of no other head); the other rows are what they are
    with that value row zeroed."""
    sh = wl.LayerShape(B=1, T=40, W=6, d=8, H=2, Dh=4, dtype=wl.F32)
    raw = wl.layer_inputs(sh, 81)
    q, k, v = (oracle.f64(raw[n]) for n in ("q", "k", "v"))
    zero = np.zeros_like(q)
    off = np.full(sh.H, -np.inf)
    j = 17
    bad = v.copy()
    bad[0, j, 1, 2] = np.nan
    o, _ = oracle.swa_inject_fwd(q, k, bad, zero, zero, off, sh.W)
    clean = v.copy()
    clean[0, j, 1, :] = 0.0
    oc, _ = oracle.swa_inject_fwd(q, k, clean, zero, zero, off, sh.W)
    hit = ~np.isfinite(o[0, :, 1, :]).all(axis=-1)
    assert np.array_equal(np.nonzero(hit)[0], np.arange(j, j + sh.W))
    assert np.isfinite(o[0, :, 0, :]).all()
    rest = np.ones(sh.T, bool)
    rest[j:j + sh.W] = False
    np.testing.assert_array_equal(o[0, rest], oc[0, rest])
