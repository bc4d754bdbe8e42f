"""GPU parity of a stack of layers sharing one memory projection against the
CPU oracle: one projection of the shifted m' per pass, each layer's own mix,
forward and backward (summing the memory gradients in float32), then one
projection backward. Checks every layer's outputs and gradients and the
shared ones (dm', dW). Every call goes through the C ABI via the binding."""
import math

import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import DGATE_TOL, TOL, check, check_act, check_dw, dgate_scale, flush, operand_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def run_stack(sh, L, seed0):
    flush("shared stack %s layers %d seed %d" % (sh, L, seed0))
    raws = [wl.layer_inputs(sh, seed0 + l, grads=True) for l in range(L)]
    shared = {n: raws[0][n] for n in ("m_prime", "W_Km", "W_Vm")}
    gs = {n: t.cuda() for n, t in shared.items()}
    km, vm = rms.maglev_mem_project(gs["m_prime"], gs["W_Km"], gs["W_Vm"], sh.H, sh.Dh, shift=1,
                                    pos0=sh.pos0, rope_base=sh.rope_base)
    dkm = torch.empty(km.shape, dtype=torch.float32, device="cuda")
    dvm = torch.empty_like(dkm)
    got = []
    for l, r in enumerate(raws):
        x = {n: r[n].cuda() for n in ("q", "k", "v", "gate_logit", "dO")}
        kx, vx = rms.maglev_mix_entries(x["k"], x["v"], km, vm, x["gate_logit"], pos0=sh.pos0,
                                        rope_base=sh.rope_base)
        o, lse = rms.maglev_swa_inject_fwd(x["q"], kx, vx, sh.W, pos0=sh.pos0,
                                           rope_base=sh.rope_base)
        dq, dk, dv, dgate = rms.maglev_swa_inject_bwd_shared(
            x["q"], kx, vx, km, vm, x["gate_logit"], o, lse, x["dO"], dkm, dvm, sh.W,
            pos0=sh.pos0, rope_base=sh.rope_base, accumulate=1 if l else 0)
        got.append({"o": o, "dq": dq, "dk": dk, "dv": dv, "dgate": dgate})
    dm, dWk, dWv = rms.maglev_mem_project_bwd(dkm, dvm, gs["m_prime"], gs["W_Km"], gs["W_Vm"])
    torch.cuda.synchronize()

    layers = [{n: oracle.f64(r[n]) for n in ("q", "k", "v", "gate_logit", "dO")} for r in raws]
    per, sg = oracle.swa_inject_bwd_shared(layers, shared["m_prime"], shared["W_Km"],
                                           shared["W_Vm"], sh.W, pos0=sh.pos0,
                                           rope_base=sh.rope_base)
    rkm, rvm = oracle.mem_project(shared["m_prime"], shared["W_Km"], shared["W_Vm"], sh.H, sh.Dh)
    tol = TOL[sh.dtype]
    errs = {}
    op_max = 1.0
    for l in range(L):
        ro, _ = oracle.swa_inject_fwd(layers[l]["q"], layers[l]["k"], layers[l]["v"], rkm, rvm,
                                      layers[l]["gate_logit"], sh.W, pos0=sh.pos0,
                                      rope_base=sh.rope_base)
        rkx, rvx = oracle.mixed_entries(layers[l]["k"], layers[l]["v"], rkm, rvm,
                                        layers[l]["gate_logit"], sh.pos0, sh.rope_base)
        op = operand_scale(sh, rkx, rvx)
        op_max = max(op_max, op)
        errs["o%d" % l] = check_act("o layer %d" % l, got[l]["o"], ro, sh.dtype, op)
        for n in ("dq", "dk", "dv"):
            errs["%s%d" % (n, l)] = check_act("%s layer %d" % (n, l), got[l][n], per[l][n],
                                              sh.dtype, op)
        sc = DGATE_TOL[sh.dtype] / tol * dgate_scale(raws[l], sh, per[l], rkm, rvm)
        err = np.abs(got[l]["dgate"].cpu().double().numpy() - per[l]["dgate"])
        assert np.all(err <= tol * sc), "dgate layer %d: %s > %s" % (l, err, tol * sc)
    # the sum of L layers' contributions, each carrying its layer's rounding
    errs["dm_prime"] = check("dm_prime", dm, sg["dm_prime"], tol, math.sqrt(L) * op_max)
    for n, t in (("dW_Km", dWk), ("dW_Vm", dWv)):
        errs[n] = check_dw(n, t, sg[n], sh.dtype)
    flush("  errors %s" % {k: "%.2e" % v for k, v in errs.items()})


def test_shared_stack_bf16_three_layers():
    run_stack(wl.LayerShape(B=2, T=200, W=50, d=128, H=2, Dh=128, dtype=wl.BF16), 3, 90)


def test_shared_stack_bf16_dh64_pos0():
    run_stack(wl.LayerShape(B=1, T=160, W=33, d=192, H=3, Dh=64, dtype=wl.BF16, pos0=300), 2, 93)


def test_shared_stack_fp32():
    run_stack(wl.LayerShape(B=2, T=90, W=20, d=64, H=2, Dh=64, dtype=wl.F32), 2, 95)
