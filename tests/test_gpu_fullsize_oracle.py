"""Whole-tensor parity at the full workload sizes: every element of every
output of the d20 layer (B=8, T=2048, W=512, d=1280, 10x128 heads, lambda
0.1), of a layer of the 20-layer pass (B=4), of a two-layer stack sharing one
projection (B=4) and of the prefiller's full-attention layer (W = T = 2048),
each in the launch configuration the benchmark times, against the CPU oracle
run on the same seeded inputs. Also decode steps at the positions the decode
benchmark reaches (p up to W + 4095) and beyond, at the full head shape.

Bars (see layer_util): kmem, vmem, lse, dm' absolutely at 2e-2; o, dq, dk,
dv at 2e-2 but for a fraction 3e-5 of the elements (none above 6e-2); the
stored mixed entries relative to max(1, max|ref|); dW against its rms plus a
relative Frobenius error; dgate per head relative to the L2 norm of its
terms. Every check prints its raw max-abs. The oracle needs about 30 s of 16
host threads for the whole d20 backward."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import (DGATE_TOL, TOL, check, check_act, check_backward, check_dw,
                        check_forward, dgate_scale, flush, gpu_backward, gpu_forward, max_scale,
                        oracle_backward, oracle_forward, rms_scale)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def whole_layer(sh, seed):
    """GPU forward + backward of one layer, then the oracle's, every element."""
    flush("whole layer %s seed %d: GPU" % (sh, seed))
    inp = wl.layer_inputs(sh, seed, grads=True)
    res = gpu_forward(inp, sh)
    g, km, vm, o, lse = res
    gr = gpu_backward(g, km, vm, o, lse, sh)
    torch.cuda.synchronize()
    flush("  oracle forward")
    ref = oracle_forward(inp, sh)
    errs, _ = check_forward(sh, inp, res, ref, named=True)
    flush("  oracle backward")
    rg = oracle_backward(inp, sh)
    errs.update(check_backward(sh, inp, gr, rg, ref[0], ref[1]))
    for n in ("dW_Km", "dW_Vm"):
        flush("    %s rms(ref) %.3e, max|ref| %.3e" % (n, rms_scale(rg[n]), max_scale(rg[n])))
    flush("  errors/bar %s" % {k: "%.2f" % v for k, v in errs.items()})
    return inp, g


def test_d20_layer_every_element():
    """The benchmark's step: projection with the mix, attention forward, the
    whole backward and the consistency loss, at B=8, T=2048, W=512."""
    sh = wl.D20_LAYER
    inp, g = whole_layer(sh, 2)
    loss, dm, dmp = rms.maglev_consistency_loss(g["m"], g["m_prime"], sh.lam)
    torch.cuda.synchronize()
    rl, rdm, rdmp = oracle.consistency_loss(inp["m"], inp["m_prime"], sh.lam)
    flush("    loss %.8e vs %.8e" % (loss.item(), rl))
    assert abs(loss.item() - rl) <= 1e-4 * abs(rl)
    # dm ~ 1e-6: relative to its own largest magnitude (an absolute 2e-2 says nothing)
    check("dm", dm, rdm, 1e-3, float(np.max(np.abs(rdm))))
    check("dm'", dmp, rdmp, 1e-3, float(np.max(np.abs(rdmp))))


def test_d20_stack_layer_every_element():
    """The last layer (seed 3019) of the 20-layer pass, B=4."""
    whole_layer(wl.D20_STACK, 3000 + wl.D20_STACK_LAYERS - 1)


def test_d20_shared_projection_stack_every_element():
    """Two d20 layers (B=4) sharing one projection of the shifted m': every
    layer's o, dq, dk, dv, dgate and the shared dm', dW_Km, dW_Vm."""
    sh = wl.D20_STACK
    L = 2
    flush("shared-projection stack, %d layers at %s" % (L, sh))
    raws = [wl.layer_inputs(sh, 3100 + l, grads=True) for l in range(L)]
    shared = {n: raws[0][n] for n in ("m_prime", "W_Km", "W_Vm")}
    gs = {n: t.cuda() for n, t in shared.items()}
    km, vm = rms.maglev_mem_project(gs["m_prime"], gs["W_Km"], gs["W_Vm"], sh.H, sh.Dh, shift=1)
    dkm = torch.empty(km.shape, dtype=torch.float32, device="cuda")
    dvm = torch.empty_like(dkm)
    got = []
    for l, r in enumerate(raws):
        x = {n: r[n].cuda() for n in ("q", "k", "v", "gate_logit", "dO")}
        kx, vx = rms.maglev_mix_entries(x["k"], x["v"], km, vm, x["gate_logit"])
        o, lse = rms.maglev_swa_inject_fwd(x["q"], kx, vx, sh.W)
        dq, dk, dv, dgate = rms.maglev_swa_inject_bwd_shared(
            x["q"], kx, vx, km, vm, x["gate_logit"], o, lse, x["dO"], dkm, dvm, sh.W,
            accumulate=1 if l else 0)
        got.append({"o": o.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu(),
                    "dgate": dgate.cpu()})
    dm, dWk, dWv = rms.maglev_mem_project_bwd(dkm, dvm, gs["m_prime"], gs["W_Km"], gs["W_Vm"])
    torch.cuda.synchronize()
    flush("  oracle")
    layers = [{n: oracle.f64(r[n]) for n in ("q", "k", "v", "gate_logit", "dO")} for r in raws]
    per, sg = oracle.swa_inject_bwd_shared(layers, shared["m_prime"], shared["W_Km"],
                                           shared["W_Vm"], sh.W)
    rkm, rvm = oracle.mem_project(shared["m_prime"], shared["W_Km"], shared["W_Vm"], sh.H, sh.Dh)
    tol = TOL[sh.dtype]
    for l in range(L):
        ro, _ = oracle.swa_inject_fwd(layers[l]["q"], layers[l]["k"], layers[l]["v"], rkm, rvm,
                                      layers[l]["gate_logit"], sh.W)
        check_act("o layer %d" % l, got[l]["o"], ro, sh.dtype)
        for n in ("dq", "dk", "dv"):
            check_act("%s layer %d" % (n, l), got[l][n], per[l][n], sh.dtype)
        sc = DGATE_TOL[sh.dtype] / tol * dgate_scale(raws[l], sh, per[l], rkm, rvm)
        err = np.abs(got[l]["dgate"].double().numpy() - per[l]["dgate"])
        flush("    dgate layer %d max-abs %.3e (smallest bar %.3e)" % (l, err.max(), (tol * sc).min()))
        assert np.all(err <= tol * sc), "dgate layer %d: %s > %s" % (l, err, tol * sc)
    check("dm_prime", dm, sg["dm_prime"], tol)
    for n, t in (("dW_Km", dWk), ("dW_Vm", dWv)):
        check_dw(n, t, sg[n], sh.dtype)


def test_d20_gated_shared_projection_stack_every_element():
    """Two gated d20 layers (B=4) over one projection of the shifted m': every
    layer's o, dq, dk, dv and four gate-logit gradients, and the shared dm',
    dW_Km, dW_Vm, with the bars of the small gated stacks."""
    from test_gpu_shared_gated import compare, run_gpu
    sh = wl.D20_STACK
    L = 2
    flush("gated shared-projection stack, %d layers at %s" % (L, sh))
    raws = [wl.layer_inputs(sh, 3200 + l, grads=True) for l in range(L)]
    gates = [wl.gate_vectors(sh.H, sh.Dh, 3200 + l, std=0.7) for l in range(L)]
    got, shared_got = run_gpu(sh, raws, gates)
    flush("  oracle")
    compare(sh, raws, gates, got, shared_got)


def test_d20_full_attention_layer_backward_every_element():
    """The prefiller's full-attention layer (no injection) at B=8, T=W=2048:
    the GPU runs the whole batch; sequences are independent, so the oracle
    runs sequences 0 and 7 and every element of theirs is compared."""
    sh = wl.LayerShape(B=8, T=2048, W=2048, d=1280, H=10, Dh=128, dtype=wl.BF16)
    flush("full-attention layer B=8 T=W=2048")
    inp = wl.layer_inputs(sh, 87, grads=True)
    g = {n: inp[n].cuda() for n in ("q", "k", "v", "dO")}
    o, lse, kr = rms.maglev_attn_fwd(g["q"], g["k"], g["v"], sh.W)
    dq, dk, dv = rms.maglev_attn_bwd(g["q"], kr, g["v"], o, lse, g["dO"], sh.W)
    torch.cuda.synchronize()
    seqs = [0, 7]
    sub = {n: oracle.f64(inp[n][seqs]) for n in ("q", "k", "v", "dO")}
    zero = np.zeros_like(sub["q"])
    off = np.full(sh.H, -np.inf)
    flush("  oracle")
    ro, rlse = oracle.swa_inject_fwd(sub["q"], sub["k"], sub["v"], zero, zero, off, sh.W)
    Wz = np.zeros((sh.H * sh.Dh, sh.d))
    rg = oracle.swa_inject_bwd(sub["q"], sub["k"], sub["v"], np.zeros((2, sh.T, sh.d)), Wz, Wz,
                               off, sub["dO"], sh.W)
    check("lse", lse[seqs], rlse, TOL[sh.dtype])
    for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        check_act(n, t[seqs], rg[n] if n != "o" else ro, sh.dtype)


def test_decode_at_far_positions_full_head_shape():
    """Teacher-forced decode steps with RoPE on, 10 heads of 128, W=512, at the
    positions the 4096-step decode benchmark ends on (W + 4095), at W - 1
    (ring not yet full), at 4095 and at a position far beyond (10^6 + 3),
    whose rotation angle the kernel reduces in double precision: o every
    step, the rings at the end."""
    H, Dh, W = 10, 128, 512
    starts = [W + 4095, W - 1, 4095, 1_000_003]
    Bs = len(starts)
    gen = torch.Generator().manual_seed(4607)
    rnd = lambda *s: torch.randn(*s, generator=gen).bfloat16()
    kc0, vc0 = rnd(Bs, H, W, Dh), rnd(Bs, H, W, Dh)
    gate = torch.randn(H, generator=gen)
    kc, vc = kc0.cuda(), vc0.cuda()
    okc, ovc = oracle.f64(kc0), oracle.f64(vc0)
    pos = torch.tensor(starts, dtype=torch.int64).cuda()
    for step in range(4):
        q, k, v, km, vm = (rnd(Bs, H, Dh) for _ in range(5))
        o = rms.maglev_decode_step(q.cuda(), k.cuda(), v.cuda(), km.cuda(), vm.cuda(), gate.cuda(),
                                   kc, vc, pos)
        rms.maglev_decode_advance(pos)
        ro = oracle.decode_step(q, k, v, km, vm, gate, okc, ovc,
                                np.asarray(starts, dtype=np.int64) + step)
        torch.cuda.synchronize()
        check("o step %d" % step, o, ro, TOL[wl.BF16])
    # new entries may differ by one rounding step of bf16 (2^-7 relative)
    for name, got, ref in (("kcache", kc, okc), ("vcache", vc, ovc)):
        diff = np.abs(got.cpu().double().numpy() - ref)
        flush("    %s max-abs %.3e" % (name, diff.max()))
        assert np.all(diff <= 2.0 ** -7 * np.abs(ref) + 1e-5), name
