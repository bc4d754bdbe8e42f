"""Parity at the full workload sizes, in the launch configuration the benchmark
times: the d20 layer forward (B=8, T=2048, W=512, d=1280, 10x128 heads), the
same layer's forward+backward with the consistency loss (lambda 0.1), a layer
of the 20-layer pass (B=4) and the 64-stream, 20-layer decode.

The oracle computes sampled outputs one at a time on exact slices of the same
inputs (a query's output needs only its W keys and the memory row before them;
a key's gradient needs only the W queries after it and their windows), at the
named-workload bar: 2e-2 max-abs for the activations. Gradients that sum over
every token (dm', dW, dgate) are also checked through identities that hold at
any size, computed in float64 on the CPU from the GPU's own dk/dv, over every
row and column; so are the memory projections (kmem, vmem) of the forward."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from recurrent_memory_sliding_amd.decode import DecodeStack
from layer_util import check, check_act, flush, gpu, gpu_project, max_scale

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def head_slice(inp, sh, b, h, s0, s1):
    """Inputs of sequence b, head h, positions [s0, s1) (as a B=1, H=1 layer)."""
    Dh = sh.Dh
    sl = {n: inp[n][b:b + 1, s0:s1, h:h + 1].contiguous() for n in ("q", "k", "v")}
    if "dO" in inp:
        sl["dO"] = inp["dO"][b:b + 1, s0:s1, h:h + 1].contiguous()
    sl["m_prime"] = inp["m_prime"][b:b + 1, s0:s1].contiguous()
    sl["W_Km"] = inp["W_Km"][h * Dh:(h + 1) * Dh].contiguous()
    sl["W_Vm"] = inp["W_Vm"][h * Dh:(h + 1) * Dh].contiguous()
    sl["gate_logit"] = inp["gate_logit"][h:h + 1].contiguous()
    return sl


def oracle_query_row(inp, sh, b, h, i):
    """O, lse of query i and kmem/vmem of its window, from the oracle on the
    slice [i-W, i] (the extra first row only feeds the shifted memory)."""
    s0 = max(0, i - sh.W)
    sl = head_slice(inp, sh, b, h, s0, i + 1)
    km, vm = oracle.mem_project(sl["m_prime"], sl["W_Km"], sl["W_Vm"], 1, sh.Dh, shift=1)
    o, lse = oracle.swa_inject_fwd(sl["q"], sl["k"], sl["v"], km, vm, sl["gate_logit"], sh.W,
                                   pos0=s0, rope_base=sh.rope_base)
    kx, vx = oracle.mixed_entries(sl["k"], sl["v"], km, vm, sl["gate_logit"], s0, sh.rope_base)
    first = 1 if s0 > 0 else 0   # slice row 0 lacks its memory row when s0 > 0
    return (o[0, -1, 0], lse[0, 0, -1], km[0, first:, 0], vm[0, first:, 0], kx[0, first:, 0],
            vx[0, first:, 0], s0 + first)


def oracle_key_grads(inp, sh, b, h, j):
    """dq, dk, dv at position j from the oracle on the slice [j-W, j+W)."""
    s0, s1 = max(0, j - sh.W), min(sh.T, j + sh.W)
    sl = head_slice(inp, sh, b, h, s0, s1)
    g = oracle.swa_inject_bwd(sl["q"], sl["k"], sl["v"], sl["m_prime"], sl["W_Km"], sl["W_Vm"],
                              sl["gate_logit"], sl["dO"], sh.W, pos0=s0, rope_base=sh.rope_base)
    return g["dq"][0, j - s0, 0], g["dk"][0, j - s0, 0], g["dv"][0, j - s0, 0]


def sample_queries(sh):
    pts = [0, 1, 63, 64, 127, 128, sh.W - 1, sh.W, sh.W + 1, 1000, sh.T - 129, sh.T - 1]
    rng = np.random.default_rng(7)
    return [(int(rng.integers(sh.B)), int(rng.integers(sh.H)), p) for p in pts if p < sh.T]


def run_forward_fullsize(sh, inp):
    g = gpu(inp)
    km, vm = gpu_project(g, sh)
    o, lse = rms.maglev_swa_inject_fwd(g["q"], g["kx"], g["vx"], sh.W, d=sh.d)
    torch.cuda.synchronize()
    return g, km, vm, o, lse


def check_forward_samples(sh, inp, g, km, vm, o, lse):
    worst = 0.0
    for b, h, i in sample_queries(sh):
        ro, rl, rkm, rvm, rkx, rvx, t0 = oracle_query_row(inp, sh, b, h, i)
        worst = max(worst, check_act("o[%d,%d,%d]" % (b, i, h), o[b, i, h], ro, sh.dtype))
        check("lse", lse[b, h, i], rl, TOL)
        check("kmem rows", km[b, t0:i + 1, h], rkm, TOL)
        check("vmem rows", vm[b, t0:i + 1, h], rvm, TOL)
        # stored bf16 entries of magnitude above 4: judged relative to max(1, max|ref|)
        check("kmix rows", g["kx"][b, t0:i + 1, h], rkx, TOL, max_scale(rkx))
        check("vmix rows", g["vx"][b, t0:i + 1, h], rvx, TOL, max_scale(rvx))
    return worst


def shifted_projection(inp, sh):
    """kmem, vmem [B,T,H,Dh] of the whole batch in float64 (row t from m'[t-1],
    row 0 zero): the definition the projection product computes."""
    mp = inp["m_prime"].double()
    prev = torch.zeros_like(mp)
    prev[:, 1:] = mp[:, :-1]
    shape = (sh.B, sh.T, sh.H, sh.Dh)
    return ((prev @ inp["W_Km"].double().T).reshape(shape).numpy(),
            (prev @ inp["W_Vm"].double().T).reshape(shape).numpy())


def test_d20_layer_forward_fullsize():
    """Sampled outputs against the oracle, and every kmem/vmem entry (the
    256 x 320-tile projection this size launches) against the float64 product."""
    sh = wl.D20_LAYER
    flush("d20 layer forward, B=8 T=2048 W=512")
    inp = wl.layer_inputs(sh, 1)
    g, km, vm, o, lse = run_forward_fullsize(sh, inp)
    flush("  worst o error %.3e" % check_forward_samples(sh, inp, g, km, vm, o, lse))
    rk, rv = shifted_projection(inp, sh)
    check("kmem (all)", km, rk, TOL, max_scale(rk))
    check("vmem (all)", vm, rv, TOL, max_scale(rv))


def backward_fullsize(sh, seed, keys):
    inp = wl.layer_inputs(sh, seed, grads=True)
    g, km, vm, o, lse = run_forward_fullsize(sh, inp)
    gr = rms.maglev_swa_inject_bwd(g["q"], g["kx"], g["vx"], km, vm, g["gate_logit"], o, lse,
                                   g["dO"], g["m_prime"], g["W_Km"], g["W_Vm"], sh.W)
    torch.cuda.synchronize()
    for b, h, j in keys:
        rdq, rdk, rdv = oracle_key_grads(inp, sh, b, h, j)
        check_act("dq[%d,%d,%d]" % (b, j, h), gr["dq"][b, j, h], rdq, sh.dtype)
        check_act("dk[%d,%d,%d]" % (b, j, h), gr["dk"][b, j, h], rdk, sh.dtype)
        check_act("dv[%d,%d,%d]" % (b, j, h), gr["dv"][b, j, h], rdv, sh.dtype)
    # identities of the projection backward, from the GPU's own dk, dv (float64, CPU)
    dk = gr["dk"].cpu().double()
    dv = gr["dv"].cpu().double()
    s = torch.sigmoid(inp["gate_logit"].double())
    WK, WV = inp["W_Km"].double(), inp["W_Vm"].double()
    mp = inp["m_prime"].double()
    HD = sh.H * sh.Dh
    # every row of dm' and every entry of dW (the products this size launches)
    sk = (dk[:, 1:] * s[None, None, :, None]).reshape(sh.B, sh.T - 1, HD)
    sv = (dv[:, 1:] * s[None, None, :, None]).reshape(sh.B, sh.T - 1, HD)
    want = (sk @ WK + sv @ WV).numpy()
    check("dm' (all rows)", gr["dm_prime"][:, :-1], want, TOL, max_scale(want))
    del sk, sv, want
    assert gr["dm_prime"][:, -1].abs().max().item() == 0.0
    prev = torch.zeros_like(mp)
    prev[:, 1:] = mp[:, :-1]
    X = prev.reshape(-1, sh.d)                                   # [N, d]
    for name, grad in (("dW_Km", dk), ("dW_Vm", dv)):
        G = (grad * s[None, None, :, None]).reshape(-1, HD)      # [N, HD]
        want = (G.T @ X).numpy()
        check(name + " (all)", gr[name], want, TOL, max_scale(want))
    kmc, vmc = km.cpu().double(), vm.cpu().double()
    terms = (kmc * dk + vmc * dv).sum(dim=(0, 1, 3))
    want = (s * (1 - s) * terms).numpy()
    sq = ((kmc * dk) ** 2 + (vmc * dv) ** 2).sum(dim=(0, 1, 3)).sqrt()
    scale = np.maximum(1.0, (s * (1 - s) * sq).numpy())
    err = np.abs(gr["dgate"].cpu().double().numpy() - want)
    assert np.all(err <= TOL * scale), (err, scale)
    return inp, g


def test_d20_layer_forward_backward_fullsize():
    sh = wl.D20_LAYER
    flush("d20 layer forward+backward, B=8 T=2048 W=512, lambda 0.1")
    keys = [(0, 0, 0), (3, 4, 511), (5, 9, 512), (7, 2, 1000), (2, 6, 2047), (6, 1, 1536)]
    inp, g = backward_fullsize(sh, 2, keys)
    loss, dm, dmp = rms.maglev_consistency_loss(g["m"], g["m_prime"], sh.lam)
    torch.cuda.synchronize()
    rl, rdm, _ = oracle.consistency_loss(inp["m"], inp["m_prime"], sh.lam)
    assert abs(loss.item() - rl) <= 1e-4 * abs(rl)
    assert np.max(np.abs(dm.cpu().double().numpy() - rdm)) <= 1e-3 * np.max(np.abs(rdm))
    assert torch.equal(dmp, -dm)


def test_d20_stack_layer_fullsize():
    """One layer (the last, seed 3019) of the 20-layer pass at B=4."""
    sh = wl.D20_STACK
    flush("d20 stack layer 19, B=4 T=2048")
    backward_fullsize(sh, 3000 + wl.D20_STACK_LAYERS - 1, [(0, 3, 5), (3, 8, 1300), (2, 0, 2047)])


def test_d20_decode_fullsize_sampled_streams():
    """64 streams x 20 layers, rings prefilled for positions 0..511; three
    closed-loop steps (the memory is the last layer's output). The oracle runs
    streams 0 and 63 through all layers from the same initial state."""
    sh = wl.D20_DECODE
    Bs, H, Dh, W, L = sh.Bs, sh.H, sh.Dh, sh.W, sh.layers
    seed = 4
    flush("d20 decode, 64 streams x 20 layers, W=512")
    params = [wl.decode_layer_params(sh, seed, l) for l in range(L)]
    m0 = wl.decode_initial_memory(sh, seed)
    streams = [0, Bs - 1]
    ork = [oracle.f64(p["kcache"][streams]) for p in params]
    orv = [oracle.f64(p["vcache"][streams]) for p in params]
    weights = [{"W_Km": p["W_Km"].cuda(), "W_Vm": p["W_Vm"].cuda(),
                "gate_logit": p["gate_logit"].cuda()} for p in params]
    stack = DecodeStack(weights, [p["kcache"].cuda() for p in params],
                        [p["vcache"].cuda() for p in params],
                        torch.full((Bs,), W, dtype=torch.int64, device="cuda"), m0.cuda())
    om = oracle.f64(m0[streams])
    for step in range(3):
        e = step % sh.pool
        q = [p["q_pool"][e].cuda() for p in params]
        k = [p["k_pool"][e].cuda() for p in params]
        v = [p["v_pool"][e].cuda() for p in params]
        outs = stack.step(q, k, v)
        outs = [o.clone() for o in outs]
        torch.cuda.synchronize()
        for l in range(L):
            p = params[l]
            km, vm = oracle.mem_project(om[:, None, :], p["W_Km"], p["W_Vm"], H, Dh, shift=0)
            ro = oracle.decode_step(p["q_pool"][e][streams], p["k_pool"][e][streams],
                                    p["v_pool"][e][streams], km[:, 0], vm[:, 0], p["gate_logit"],
                                    ork[l], orv[l], np.full(2, W + step))
            check("decode step %d layer %d" % (step, l), outs[l][streams], ro, TOL)
            if l == L - 1:
                om = ro.reshape(2, H * Dh)
        flush("  step %d ok" % step)
