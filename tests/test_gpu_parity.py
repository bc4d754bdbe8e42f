"""GPU parity of the training-pass entry points against the CPU oracle, at
sizes the oracle finishes in seconds that still span several tiles and ragged
tails, plus the method's degenerate cases. Every call goes through the C ABI
(libmaglev.so) via the binding; the oracle sees the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import (TOL, check, check_backward, check_forward, flush, gpu, gpu_backward,
                        gpu_forward, gpu_project, oracle_backward, oracle_forward)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()          # raises if the HIP library is missing: no silent fallback
    oracle.build(force=False)


def shape(**kw):
    base = dict(B=2, T=300, W=70, d=256, H=2, Dh=128, dtype=wl.BF16, lam=0.1)
    base.update(kw)
    return wl.LayerShape(**base)


def run_fwd_case(sh, seed, grads=False, mutate=None):
    flush("case %s seed %d grads %s" % (sh, seed, grads))
    inp = wl.layer_inputs(sh, seed, grads=grads)
    if mutate:
        mutate(inp)
    res = gpu_forward(inp, sh)
    torch.cuda.synchronize()
    ref = oracle_forward(inp, sh)
    errs, op = check_forward(sh, inp, res, ref)
    if grads:
        g, km, vm, o, lse = res
        gr = gpu_backward(g, km, vm, o, lse, sh)
        torch.cuda.synchronize()
        errs.update(check_backward(sh, inp, gr, oracle_backward(inp, sh), ref[0], ref[1], op))
    flush("  errors %s" % {k: "%.2e" % v for k, v in errs.items()})
    return inp, res, errs


def test_tiny_fp32_forward_and_loss():
    """The tiny fp32 workload: B=1, T=256, W=32, d=64, one head of 64."""
    sh = wl.TINY_FP32
    inp, _, _ = run_fwd_case(sh, 0)
    g = gpu(inp)
    loss, dm, dmp = rms.maglev_consistency_loss(g["m"], g["m_prime"], sh.lam)
    torch.cuda.synchronize()
    rl, rdm, rdmp = oracle.consistency_loss(inp["m"], inp["m_prime"], sh.lam)
    assert abs(loss.item() - rl) <= 1e-4 * max(1.0, abs(rl))
    check("dm", dm, rdm, 1e-4)
    check("dm'", dmp, rdmp, 1e-4)
    assert np.max(np.abs(dm.cpu().double().numpy() - rdm)) <= 1e-3 * np.max(np.abs(rdm))


def test_bf16_ragged_forward_backward_dh128():
    run_fwd_case(shape(), 1, grads=True)


def test_bf16_ragged_forward_backward_dh64():
    run_fwd_case(shape(B=1, T=200, W=33, H=3, Dh=64, d=192), 2, grads=True)


def test_fp32_backward_exact_algebra():
    run_fwd_case(shape(B=2, T=150, W=40, H=2, Dh=64, d=128, dtype=wl.F32), 3, grads=True)


def test_fp32_backward_dh128():
    run_fwd_case(shape(B=1, T=97, W=30, H=2, Dh=128, d=64, dtype=wl.F32), 4, grads=True)


@pytest.mark.parametrize("T,W", [(130, 500), (257, 1), (1, 512), (64, 64), (129, 2), (640, 512),
                                 (575, 512), (96, 96)])
def test_bf16_window_edges(T, W):
    """Window covering the sequence (full causal), a single key, one token,
    a window equal to one tile, two keys, the d20 window over T a multiple of
    the 32-row tiles and one short of one (the last tile of a sequence is
    loaded with rows past T read as zeros, the others whole), and a window
    covering three whole tiles."""
    run_fwd_case(shape(B=1, T=T, W=W, H=2, Dh=128, d=128), 10 + T + W, grads=True)


def test_bf16_position_offset():
    run_fwd_case(shape(B=1, T=200, W=50, d=128, pos0=1000), 5, grads=True)


@pytest.mark.parametrize("logit", [float("-inf"), 40.0, -3.0])
def test_bf16_gate_extremes(logit):
    def mut(inp):
        inp["gate_logit"] = torch.full_like(inp["gate_logit"], logit)
    _, res, _ = run_fwd_case(shape(B=1, T=150, W=40, d=128), 6, grads=True, mutate=mut)


def test_rope_disabled():
    run_fwd_case(shape(B=1, T=100, W=30, d=128, rope_base=0.0), 7, grads=True)


def test_empty_batch_backward_zeroes_parameter_gradients():
    sh = shape(B=0, T=64)
    inp = wl.layer_inputs(shape(B=1, T=64), 8, grads=True)
    g = gpu({k: v[:0] if v.dim() >= 3 else v for k, v in inp.items()})
    km, vm = gpu_project(g, sh)
    o, lse = rms.maglev_swa_inject_fwd(g["q"], g["kx"], g["vx"], sh.W)
    out = {"dW_Km": torch.full((sh.H * sh.Dh, sh.d), 5.0, device="cuda"),
           "dW_Vm": torch.full((sh.H * sh.Dh, sh.d), 5.0, device="cuda"),
           "dgate": torch.full((sh.H,), 5.0, device="cuda")}
    gr = gpu_backward(g, km, vm, o, lse, sh, out=out)
    torch.cuda.synchronize()
    assert gr["dW_Km"].abs().max().item() == 0.0 and gr["dgate"].abs().max().item() == 0.0


def test_backward_accumulate_flags():
    sh = shape(B=1, T=140, W=40, d=128)
    inp = wl.layer_inputs(sh, 9, grads=True)
    g, km, vm, o, lse = gpu_forward(inp, sh)
    first = gpu_backward(g, km, vm, o, lse, sh)
    base = {k: v.clone() for k, v in first.items()}
    second = gpu_backward(g, km, vm, o, lse, sh, accumulate=7,
                          out={k: v.clone() for k, v in first.items()})
    torch.cuda.synchronize()
    for n in ("dm_prime", "dW_Km", "dW_Vm", "dgate"):
        torch.testing.assert_close(second[n], 2 * base[n], rtol=1e-5, atol=1e-6)
    for n in ("dq", "dk", "dv"):   # activation gradients are always overwritten
        assert torch.equal(second[n], base[n])


def test_backward_is_deterministic():
    sh = shape(B=2, T=333, W=100)
    inp = wl.layer_inputs(sh, 11, grads=True)
    g, km, vm, o, lse = gpu_forward(inp, sh)
    a = gpu_backward(g, km, vm, o, lse, sh)
    b = gpu_backward(g, km, vm, o, lse, sh)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_debug_mode_gives_the_same_results():
    """Debug mode (a synchronisation and an error check after every launch)
    returns OK and changes no result: forward, backward and loss bit-equal."""
    sh = shape(B=2, T=333, W=100)
    inp = wl.layer_inputs(sh, 12, grads=True)

    def run():
        g, km, vm, o, lse = gpu_forward(inp, sh)
        gr = gpu_backward(g, km, vm, o, lse, sh)
        loss, dm, dmp = rms.maglev_consistency_loss(g["m"], g["m_prime"], sh.lam)
        torch.cuda.synchronize()
        return dict(gr, o=o, lse=lse, loss=loss, dm=dm, dmp=dmp)

    plain = run()
    rms.maglev_debug_enable(True)
    try:
        assert rms.maglev_debug_enabled()
        dbg = run()
    finally:
        rms.maglev_debug_enable(False)
    for n in plain:
        assert torch.equal(plain[n], dbg[n]), n


def test_profiling_gives_the_same_results_and_times_every_kernel():
    """Per-kernel timing (events bound to the attention and GEMM dispatches,
    event records around the other kernels) changes no result, times each
    kernel of the pass once per launch, and with a name times only that one."""
    sh = shape(B=2, T=333, W=100)
    inp = wl.layer_inputs(sh, 13, grads=True)

    def run():
        g, km, vm, o, lse = gpu_forward(inp, sh)
        gr = gpu_backward(g, km, vm, o, lse, sh)
        loss, dm, dmp = rms.maglev_consistency_loss(g["m"], g["m_prime"], sh.lam)
        torch.cuda.synchronize()
        return dict(gr, o=o, lse=lse, loss=loss, dm=dm, dmp=dmp)

    plain = run()
    try:
        rms.maglev_profile_enable(True)
        timed = run()
        rms.maglev_profile_enable(False)
        every = rms.maglev_profile_read()
        rms.maglev_profile_enable(True, only="attn_bwd_dkdv")
        run()
        rms.maglev_profile_enable(False)
        one = rms.maglev_profile_read()
    finally:
        rms.maglev_profile_enable(False)
    for n in plain:
        assert torch.equal(plain[n], timed[n]), n
    flush("  timed %s" % {k: "%d x %.3f ms" % v for k, v in every.items()})
    for k in ("attn_fwd", "attn_bwd_prep", "attn_bwd_dkdv", "attn_bwd_dq", "mix", "loss_partial",
              "loss_final"):
        assert k in every, k
    for k, (n, ms) in every.items():
        assert n >= 1 and 0.0 < ms < 1000.0 * n, (k, n, ms)
    assert list(one) == ["attn_bwd_dkdv"] and one["attn_bwd_dkdv"][0] == 1, one


def test_loss_bf16_and_accumulate():
    sh = shape(B=3, T=500, d=1280)
    inp = wl.layer_inputs(sh, 12)
    g = gpu(inp)
    loss, dm, dmp = rms.maglev_consistency_loss(g["m"], g["m_prime"], sh.lam)
    torch.cuda.synchronize()
    rl, rdm, rdmp = oracle.consistency_loss(inp["m"], inp["m_prime"], sh.lam)
    assert abs(loss.item() - rl) <= 1e-4 * abs(rl)
    assert np.max(np.abs(dm.cpu().double().numpy() - rdm)) <= 1e-3 * np.max(np.abs(rdm))
    assert torch.equal(dmp, -dm)
    loss2, dm2, dmp2 = rms.maglev_consistency_loss(g["m"], g["m_prime"], sh.lam, loss=loss.clone(),
                                                   dm=dm.clone(), dm_prime=dmp.clone(), accumulate=7)
    torch.cuda.synchronize()
    torch.testing.assert_close(loss2, 2 * loss, rtol=1e-6, atol=0)
    torch.testing.assert_close(dm2, 2 * dm, rtol=1e-6, atol=0)
    # m == m': zero loss and gradients
    l0, d0, _ = rms.maglev_consistency_loss(g["m"], g["m"].clone(), sh.lam)
    torch.cuda.synchronize()
    assert l0.item() == 0.0 and d0.abs().max().item() == 0.0
