"""GPU parity of a stack of gated layers sharing one memory projection against
the CPU oracle: one projection of the shifted m' per pass (the pre-norm key
projection and the value projection), each layer's own gated mix, forward and
backward (summing the projections' gradients in float32), then one projection
backward. Checks every layer's o, dq, dk, dv and four gate-logit gradients,
and the shared dm', dW_Km, dW_Vm. Every call goes through the C ABI via the
binding."""
import math

import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import TOL, check, check_act, check_dw, flush, max_scale, operand_scale
from test_gpu_gated import EPS, NAMES, gate_grad_scale, gate_stack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def run_gpu(sh, raws, gates):
    """The pass on the GPU; returns per-layer host tensors and the shared grads."""
    gs = {n: raws[0][n].cuda() for n in ("m_prime", "W_Km", "W_Vm")}
    kp, vm = rms.maglev_mem_project(gs["m_prime"], gs["W_Km"], gs["W_Vm"], sh.H, sh.Dh, shift=1,
                                    pos0=sh.pos0, rope_base=sh.rope_base)
    dkp = torch.empty(kp.shape, dtype=torch.float32, device="cuda")
    dvm = torch.empty_like(dkp)
    got = []
    for l, r in enumerate(raws):
        x = {n: r[n].cuda() for n in ("q", "k", "v", "dO")}
        gt = gate_stack(gates[l]).cuda()
        kx, vx = rms.maglev_mix_entries_gated(x["k"], x["v"], kp, vm, gt, EPS, pos0=sh.pos0,
                                              rope_base=sh.rope_base)
        o, lse = rms.maglev_swa_inject_fwd(x["q"], kx, vx, sh.W, pos0=sh.pos0,
                                           rope_base=sh.rope_base)
        dq, dk, dv, dg = rms.maglev_swa_inject_bwd_shared_gated(
            x["q"], kx, vx, x["k"], x["v"], kp, vm, gt, o, lse, x["dO"], dkp, dvm, sh.W, EPS,
            pos0=sh.pos0, rope_base=sh.rope_base, accumulate=1 if l else 0)
        got.append({"o": o.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu(), "dgates": dg.cpu()})
    dm, dWk, dWv = rms.maglev_mem_project_bwd(dkp, dvm, gs["m_prime"], gs["W_Km"], gs["W_Vm"])
    torch.cuda.synchronize()
    return got, {"dm_prime": dm.cpu(), "dW_Km": dWk.cpu(), "dW_Vm": dWv.cpu()}


def compare(sh, raws, gates, got, shared_got):
    """Every element against the oracle's composition of the gated layer."""
    L = len(raws)
    shared = {n: raws[0][n] for n in ("m_prime", "W_Km", "W_Vm")}
    layers = []
    for l, r in enumerate(raws):
        x = {n: oracle.f64(r[n]) for n in ("q", "k", "v", "dO")}
        x["gates"] = gates[l]
        layers.append(x)
    per, sg = oracle.swa_inject_bwd_shared_gated(layers, shared["m_prime"], shared["W_Km"],
                                                 shared["W_Vm"], sh.W, pos0=sh.pos0,
                                                 rope_base=sh.rope_base, eps=EPS)
    rkp, rvm = oracle.mem_project(shared["m_prime"], shared["W_Km"], shared["W_Vm"], sh.H, sh.Dh)
    tol = TOL[sh.dtype]
    errs = {}
    op_max = 1.0
    for l in range(L):
        rkx, rvx = oracle.gated_entries(layers[l]["k"], layers[l]["v"], rkp, rvm, gates[l],
                                        pos0=sh.pos0, rope_base=sh.rope_base, eps=EPS)
        ro, _ = oracle.swa_attend_fwd(layers[l]["q"], rkx, rvx, sh.W, pos0=sh.pos0,
                                      rope_base=sh.rope_base)
        op = operand_scale(sh, rkx, rvx)
        op_max = max(op_max, op)
        errs["o%d" % l] = check_act("o layer %d" % l, got[l]["o"], ro, sh.dtype, op)
        for n in ("dq", "dk", "dv"):
            errs["%s%d" % (n, l)] = check_act("%s layer %d" % (n, l), got[l][n], per[l][n],
                                              sh.dtype, op)
        inp = dict(raws[l])
        inp.update(shared)
        sc = gate_grad_scale(sh, inp, gates[l], per[l], rkp)
        g = got[l]["dgates"].double().numpy()
        for i, n in enumerate(NAMES):
            err = np.abs(g[i] - per[l]["d" + n])
            flush("    d%s layer %d max-abs %.3e, largest error/scale %.3e"
                  % (n, l, err.max(), np.max(err / sc[n])))
            assert np.all(err <= tol * sc[n]), "d%s layer %d: worst err/scale %.3e" % (
                n, l, np.max(err / sc[n]))
    # dm' sums L layers' norm backwards over all H*Dh channels of both
    # projections: relative to max(1, max|ref|), sqrt(L) for the L roundings
    errs["dm_prime"] = check("dm_prime", shared_got["dm_prime"], sg["dm_prime"], tol,
                             math.sqrt(L) * max_scale(sg["dm_prime"]))
    for n in ("dW_Km", "dW_Vm"):
        errs[n] = check_dw(n, shared_got[n], sg[n], sh.dtype)
    flush("  errors %s" % {k: "%.2e" % v for k, v in errs.items()})
    return errs


def run_stack(sh, L, seed0, gate_std=0.7):
    flush("gated shared stack %s layers %d seed %d" % (sh, L, seed0))
    raws = [wl.layer_inputs(sh, seed0 + l, grads=True) for l in range(L)]
    gates = [wl.gate_vectors(sh.H, sh.Dh, seed0 + l, std=gate_std) for l in range(L)]
    got, shared_got = run_gpu(sh, raws, gates)
    return compare(sh, raws, gates, got, shared_got)


def test_gated_shared_stack_bf16_three_layers():
    run_stack(wl.LayerShape(B=2, T=200, W=50, d=128, H=2, Dh=128, dtype=wl.BF16), 3, 120)


def test_gated_shared_stack_bf16_dh64_pos0():
    run_stack(wl.LayerShape(B=1, T=160, W=33, d=192, H=3, Dh=64, dtype=wl.BF16, pos0=300), 2, 123)


def test_gated_shared_stack_fp32():
    run_stack(wl.LayerShape(B=2, T=90, W=20, d=64, H=2, Dh=64, dtype=wl.F32), 2, 125)


def test_gated_shared_stack_one_layer_equals_gated_layer():
    """A one-layer stack is the gated layer path: the same dm', dW and dgates
    as maglev_swa_inject_bwd_gated on the same inputs (float32, tight)."""
    sh = wl.LayerShape(B=2, T=70, W=16, d=64, H=2, Dh=64, dtype=wl.F32)
    raw = wl.layer_inputs(sh, 127, grads=True)
    gates = wl.gate_vectors(sh.H, sh.Dh, 127, std=0.7)
    got, shared_got = run_gpu(sh, [raw], [gates])
    g = {n: t.cuda() for n, t in raw.items()}
    gt = gate_stack(gates).cuda()
    kp, vm, kx, vx = rms.maglev_mem_project_gated(g["m_prime"], g["W_Km"], g["W_Vm"], sh.H, sh.Dh,
                                                  g["k"], g["v"], gt, EPS)
    o, lse = rms.maglev_swa_inject_fwd(g["q"], kx, vx, sh.W)
    ref = rms.maglev_swa_inject_bwd_gated(g["q"], kx, vx, g["k"], g["v"], kp, vm, gt, o, lse,
                                          g["dO"], g["m_prime"], g["W_Km"], g["W_Vm"], sh.W, EPS)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv"):
        check(n, got[0][n], ref[n].cpu().double().numpy(), 1e-6)
    check("dgates", got[0]["dgates"], ref["dgates"].cpu().double().numpy(), 1e-6)
    for n in ("dm_prime", "dW_Km", "dW_Vm"):
        check(n, shared_got[n], ref[n].cpu().double().numpy(), 1e-6,
              max_scale(ref[n].cpu().double().numpy()))
