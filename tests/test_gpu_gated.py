"""GPU parity of the gated mixing form (channel-wise 2*sigmoid gates, RMSNorm
on the projected memory key) against the CPU oracle: projection and gated mix,
attention over the gated entries, the full backward including the four gate
vectors, the gated decode step, degenerate gates and windows, accumulation,
an empty batch, and sampled rows of the d20 layer at full size. Every call
goes through the C ABI via the binding."""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import TOL, check, check_act, check_dw, flush, gpu, max_scale, operand_scale

pytestmark = pytest.mark.gpu
NAMES = oracle.GATE_NAMES
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def shape(**kw):
    base = dict(B=2, T=300, W=70, d=256, H=2, Dh=128, dtype=wl.BF16)
    base.update(kw)
    return wl.LayerShape(**base)


def gate_stack(gates):
    return torch.stack([gates[n] for n in NAMES]).float()


def rope_np(x, pos, base):
    """Complex-rotation form of the rotation, for tolerance scales only."""
    if base <= 0:
        return x.copy()
    half = x.shape[-1] // 2
    z = x[..., :half] + 1j * x[..., half:]
    inv = np.power(float(base), -np.arange(half) * 2.0 / x.shape[-1])
    z = z * np.exp(1j * np.outer(pos.astype(np.float64), inv))[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def gate_grad_scale(sh, inp, gates, ref, kp):
    """Scale of the bar for each gate-logit gradient 2 s (1 - s) sum_n e_n x_n
    (e = dk~ or dv~, the gradient of a mixed entry; x = R k, R kn, v or vmem):
    2 s (1 - s) times the larger of
      ||e_c (.) x_c||_2            -- terms rounded independently, and
      max|e| * ||x_c||_2           -- every e_n held to the per-element bar of
                                      the entry gradients (tol * max|e|), in
                                      quadrature over the tokens; an entry
                                      gradient is a sum over a whole window
                                      whose cancellation leaves its rounding
                                      error near the bar even where e_n is small.
    A dropped, mis-indexed or mis-signed gate moves the sum by about the first
    norm itself. The entry gradients follow from the oracle's dk, dv:
    dk~ = R dk / g_kl, dv~ = dv / g_vl."""
    B, T, H, Dh = sh.B, sh.T, sh.H, sh.Dh
    pos = np.arange(T) + sh.pos0
    a = {n: oracle.f64(gates[n]).reshape(H, Dh) for n in NAMES}
    g = {n: 2 * expit(a[n]) for n in NAMES}
    dkt = rope_np(ref["dk"], pos, sh.rope_base) / g["a_kl"]
    dvt = ref["dv"] / g["a_vl"]
    rows = kp.reshape(B, T, H * Dh)
    kn = (rows / np.sqrt(np.mean(rows ** 2, axis=-1, keepdims=True) + EPS)).reshape(kp.shape)
    k, v = oracle.f64(inp["k"]), oracle.f64(inp["v"])
    _, vm = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], H, Dh, shift=1)
    xs = {"a_kl": rope_np(k, pos, sh.rope_base), "a_kr": rope_np(kn, pos, sh.rope_base),
          "a_vl": v, "a_vr": vm}
    es = {"a_kl": dkt, "a_kr": dkt, "a_vl": dvt, "a_vr": dvt}
    out = {}
    for n in NAMES:
        s = expit(a[n])
        l2 = lambda x: np.sqrt(np.sum(x ** 2, axis=(0, 1)))
        norm = np.maximum(l2(es[n] * xs[n]), np.max(np.abs(es[n])) * l2(xs[n]))
        out[n] = np.maximum(1.0, (2 * s * (1 - s) * norm).reshape(-1))
    return out


def run_case(sh, seed, grads=True, gate_std=0.7, gates=None, accumulate=False):
    flush("gated case %s seed %d" % (sh, seed))
    inp = wl.layer_inputs(sh, seed, grads=grads)
    gates = gates if gates is not None else wl.gate_vectors(sh.H, sh.Dh, seed, std=gate_std)
    tol = TOL[sh.dtype]
    g = gpu(inp)
    gt = gate_stack(gates).cuda()
    kp, vm, kx, vx = rms.maglev_mem_project_gated(g["m_prime"], g["W_Km"], g["W_Vm"], sh.H, sh.Dh,
                                                  g["k"], g["v"], gt, EPS, pos0=sh.pos0,
                                                  rope_base=sh.rope_base)
    o, lse = rms.maglev_swa_inject_fwd(g["q"], kx, vx, sh.W, pos0=sh.pos0, rope_base=sh.rope_base)
    torch.cuda.synchronize()
    rkp, rvm = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], sh.H, sh.Dh, shift=1)
    rkx, rvx = oracle.gated_entries(inp["k"], inp["v"], rkp, rvm, gates, pos0=sh.pos0,
                                    rope_base=sh.rope_base, eps=EPS)
    ro, rlse = oracle.swa_attend_fwd(inp["q"], rkx, rvx, sh.W, pos0=sh.pos0,
                                     rope_base=sh.rope_base)
    errs = {}
    # the stored gated entries relative to max(1, max|ref|); everything else absolutely
    for name, got, ref, sc in (("kproj", kp, rkp, 1.0), ("vmem", vm, rvm, 1.0),
                               ("kmix", kx, rkx, max_scale(rkx)), ("vmix", vx, rvx, max_scale(rvx)),
                               ("lse", lse, rlse, 1.0)):
        errs[name] = check(name, got, ref, tol, sc)
    # the gates (up to 2 on both terms) enlarge the stored entries
    op = operand_scale(sh, rkx, rvx)
    errs["o"] = check_act("o", o, ro, sh.dtype, op)
    if not grads:
        flush("  errors %s" % {k: "%.2e" % v for k, v in errs.items()})
        return errs
    out = None
    acc = 0
    if accumulate:   # start from known values: every += must land on them
        dev = "cuda"
        out = {"dm_prime": torch.full((sh.B, sh.T, sh.d), 0.5, device=dev),
               "dW_Km": torch.full((sh.H * sh.Dh, sh.d), -0.25, device=dev),
               "dW_Vm": torch.full((sh.H * sh.Dh, sh.d), 0.125, device=dev),
               "dgates": torch.full((4, sh.H * sh.Dh), 1.5, device=dev)}
        acc = 7
    gr = rms.maglev_swa_inject_bwd_gated(g["q"], kx, vx, g["k"], g["v"], kp, vm, gt, o, lse,
                                         g["dO"], g["m_prime"], g["W_Km"], g["W_Vm"], sh.W, EPS,
                                         pos0=sh.pos0, rope_base=sh.rope_base, accumulate=acc,
                                         out=out)
    torch.cuda.synchronize()
    ref = oracle.swa_inject_bwd_gated(inp["q"], inp["k"], inp["v"], inp["m_prime"], inp["W_Km"],
                                      inp["W_Vm"], gates, inp["dO"], sh.W, pos0=sh.pos0,
                                      rope_base=sh.rope_base, eps=EPS)
    off = {"dm_prime": 0.5, "dW_Km": -0.25, "dW_Vm": 0.125, "dgates": 1.5} if accumulate else {}
    for n in ("dq", "dk", "dv"):
        errs[n] = check_act(n, gr[n], ref[n], sh.dtype, op)
    # dm' of the gated form: every one of its rows sums the norm's backward over
    # all H*Dh channels of both projections (the norm couples the heads), so it
    # is judged relative to max(1, max|ref|)
    errs["dm_prime"] = check("dm_prime", gr["dm_prime"], ref["dm_prime"] + off.get("dm_prime", 0.0),
                             tol, max_scale(ref["dm_prime"]))
    for n in ("dW_Km", "dW_Vm"):
        errs[n] = check_dw(n, gr[n], ref[n] + off.get(n, 0.0), sh.dtype)
    sc = gate_grad_scale(sh, inp, gates, ref, rkp)
    got = gr["dgates"].cpu().double().numpy()
    for i, n in enumerate(NAMES):
        err = np.abs(got[i] - (ref["d" + n] + off.get("dgates", 0.0)))
        assert np.all(err <= tol * sc[n]), "d%s: worst err/scale %.3e" % (n, np.max(err / sc[n]))
        errs["d" + n] = float(np.max(err / sc[n]))
    flush("  errors %s" % {k: "%.2e" % v for k, v in errs.items()})
    return errs


def test_gated_bf16_dh128_ragged():
    run_case(shape(), 61)


def test_gated_bf16_dh64_three_heads():
    run_case(shape(B=1, T=200, W=33, H=3, Dh=64, d=192), 62)


def test_gated_bf16_ten_heads_two_waves_per_row():
    """H*Dh = 1280 (the d20 row): 80 chunk pairs, so each row's norm and
    backward reductions span two waves."""
    run_case(shape(B=1, T=130, W=40, H=10, Dh=128, d=256), 63)


def test_gated_bf16_wide_rows_one_group_per_workgroup():
    """H*Dh = 2560: a row takes 192 threads, so the mix kernels run one row
    group a workgroup (narrower rows run two); 41 rows leave a ragged block."""
    run_case(shape(B=1, T=41, W=20, H=20, Dh=128, d=64), 70)


def test_gated_fp32_wide_rows_one_group_per_workgroup():
    run_case(shape(B=1, T=37, W=16, H=18, Dh=128, d=64, dtype=wl.F32), 71)


def test_gated_fp32_exact_algebra():
    run_case(shape(B=2, T=150, W=40, H=2, Dh=64, d=128, dtype=wl.F32), 64)


def test_gated_fp32_dh128_pos0_and_accumulate():
    run_case(shape(B=1, T=97, W=30, H=2, Dh=128, d=64, dtype=wl.F32, pos0=1000), 65,
             accumulate=True)


def test_gated_bf16_accumulate():
    run_case(shape(B=1, T=160, W=50, H=2, Dh=128, d=128), 66, accumulate=True)


@pytest.mark.parametrize("W", [1, 512])
def test_gated_window_one_and_window_covering_sequence(W):
    run_case(shape(B=1, T=140, W=W, H=2, Dh=64, d=128), 67)


def test_gated_rope_off():
    run_case(shape(B=1, T=120, W=33, H=2, Dh=128, d=128, rope_base=0.0), 68)


def test_gated_extreme_gates():
    """Recurrent gates at -inf (exactly 0) and local gates at +inf (exactly 2)
    on some channels, large logits elsewhere."""
    sh = shape(B=1, T=100, W=30, H=2, Dh=64, d=128, dtype=wl.F32)
    gates = wl.gate_vectors(sh.H, sh.Dh, 69, std=4.0)
    gates["a_kr"][:40] = float("-inf")
    gates["a_vr"][10:70] = float("-inf")
    gates["a_kl"][5:20] = float("inf")
    # an infinite logit has a zero gate derivative in both the oracle and the kernels
    run_case(sh, 69, gates=gates)


def test_gated_empty_batch_zeroes_parameter_gradients():
    dev = "cuda"
    H, Dh, d = 2, 64, 128
    z = torch.zeros((0, 5, H, Dh), dtype=torch.bfloat16, device=dev)
    m = torch.zeros((0, 5, d), dtype=torch.bfloat16, device=dev)
    W_ = torch.randn(H * Dh, d, device=dev).bfloat16()
    gates = torch.zeros(4, H * Dh, device=dev)
    lse = torch.zeros((0, H, 5), device=dev)
    out = {"dW_Km": torch.full((H * Dh, d), 3.0, device=dev),
           "dW_Vm": torch.full((H * Dh, d), 3.0, device=dev),
           "dgates": torch.full((4, H * Dh), 3.0, device=dev)}
    rms.maglev_swa_inject_bwd_gated(z, z, z, z, z, z, z, gates, z, lse, z, m, W_, W_, 8, out=out)
    torch.cuda.synchronize()
    for n in ("dW_Km", "dW_Vm", "dgates"):
        assert not out[n].any(), n


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,Dh", [(wl.BF16, 128), (wl.BF16, 64), (wl.F32, 128)])
def test_gated_decode_teacher_forced_steps(dtype, Dh):
    Bs, H, W = 4, 3, 40
    tol = TOL[dtype]
    tdt = wl.torch_dtype(dtype)
    gen = torch.Generator().manual_seed(70 + Dh)
    rnd = lambda *s: torch.randn(*s, generator=gen).to(tdt)
    kc0, vc0 = rnd(Bs, H, W, Dh), rnd(Bs, H, W, Dh)
    gates = wl.gate_vectors(H, Dh, 70 + Dh, std=1.0)
    gt = gate_stack(gates).cuda()
    kc, vc = kc0.cuda(), vc0.cuda()
    okc, ovc = oracle.f64(kc0), oracle.f64(vc0)
    pos = torch.full((Bs,), W, dtype=torch.int64).cuda()
    for step in range(2 * W + 3):
        q, k, v, kp, vm = (rnd(Bs, H, Dh) for _ in range(5))
        kp = kp * (1.0 + step % 5)   # the norm must remove this scale
        o = rms.maglev_decode_step_gated(q.cuda(), k.cuda(), v.cuda(), kp.cuda(), vm.cuda(), gt,
                                         kc, vc, pos, eps=EPS)
        rms.maglev_decode_advance(pos)
        ro = oracle.decode_step_gated(q, k, v, kp, vm, gates, okc, ovc, np.full(Bs, W + step),
                                      eps=EPS, ring_bf16=(dtype == wl.BF16))
        torch.cuda.synchronize()
        check("o step %d" % step, o, ro, tol)
    # the newest entries may differ by one rounding step of the storage type
    check("kcache", kc, okc, tol, max_scale(okc))
    check("vcache", vc, ovc, tol, max_scale(ovc))


def test_gated_decode_strided_memory_equals_packed():
    """A stacked projection row (stride above H*Dh) gives the same step as the
    packed layout: the norm reads the layer's own slice only."""
    Bs, H, Dh, W, L = 5, 2, 64, 24, 3
    dev = "cuda"
    gen = torch.Generator().manual_seed(71)
    rnd = lambda *s: torch.randn(*s, generator=gen).bfloat16().to(dev)
    q, k, v = rnd(Bs, H, Dh), rnd(Bs, H, Dh), rnd(Bs, H, Dh)
    stack_k, stack_v = rnd(Bs, L * H * Dh), rnd(Bs, L * H * Dh)
    layer = 1
    kp = stack_k[:, layer * H * Dh:(layer + 1) * H * Dh].contiguous().reshape(Bs, H, Dh)
    vm = stack_v[:, layer * H * Dh:(layer + 1) * H * Dh].contiguous().reshape(Bs, H, Dh)
    gt = gate_stack(wl.gate_vectors(H, Dh, 71)).to(dev)
    kc0, vc0 = rnd(Bs, H, W, Dh), rnd(Bs, H, W, Dh)
    pos = torch.arange(Bs, dtype=torch.int64, device=dev) * 7 + 3
    kc1, vc1 = kc0.clone(), vc0.clone()
    o1 = rms.maglev_decode_step_gated(q, k, v, kp, vm, gt, kc1, vc1, pos)
    kc2, vc2 = kc0.clone(), vc0.clone()
    sk = stack_k[:, layer * H * Dh:]
    sv = stack_v[:, layer * H * Dh:]
    o2 = rms.maglev_decode_step_gated(q, k, v, sk, sv, gt, kc2, vc2, pos, mem_stride=L * H * Dh)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)


# ----------------------------------------------------------------------------
# d20 layer at full size, sampled rows
# ----------------------------------------------------------------------------
def test_d20_layer_gated_forward_fullsize_sampled():
    """B=8, T=2048, W=512, d=1280, 10 heads of 128: every kproj/vmem row the
    oracle recomputes for the sampled rows, their gated entries, and the
    outputs of sampled queries (the oracle attends over the W entries in the
    query's window, each computed from its own full row)."""
    sh = wl.D20_LAYER
    inp = wl.layer_inputs(sh, 72)
    gates = wl.gate_vectors(sh.H, sh.Dh, 72, std=0.7)
    g = gpu(inp)
    flush("d20 gated forward, full size")
    kp, vm, kx, vx = rms.maglev_mem_project_gated(g["m_prime"], g["W_Km"], g["W_Vm"], sh.H, sh.Dh,
                                                  g["k"], g["v"], gate_stack(gates).cuda(), EPS)
    o, lse = rms.maglev_swa_inject_fwd(g["q"], kx, vx, sh.W)
    torch.cuda.synchronize()
    tol = TOL[sh.dtype]
    rng = np.random.default_rng(72)
    m_prime, WK, WV = (oracle.f64(inp[n]) for n in ("m_prime", "W_Km", "W_Vm"))
    for b, i in [(0, 0), (3, 1), (7, 2047), (5, 511), (2, 512)] + \
            [(int(rng.integers(sh.B)), int(rng.integers(sh.T))) for _ in range(3)]:
        lo = max(0, i - sh.W + 1)
        # projection input rows lo-1 .. i-1 (row t reads m'[t-1], row 0 is zero)
        src = np.zeros((i - lo + 1, sh.d))
        for r, t in enumerate(range(lo, i + 1)):
            if t > 0:
                src[r] = m_prime[b, t - 1]
        rkp = (src @ WK.T).reshape(1, -1, sh.H, sh.Dh)
        rvm = (src @ WV.T).reshape(1, -1, sh.H, sh.Dh)
        sl = lambda n: oracle.f64(inp[n][b:b + 1, lo:i + 1])
        rkx, rvx = oracle.gated_entries(sl("k"), sl("v"), rkp, rvm, gates, pos0=lo, eps=EPS)
        ro, rlse = oracle.swa_attend_fwd(sl("q"), rkx, rvx, sh.W, pos0=lo)
        check("kproj row", kp[b, i], rkp[0, -1], tol)
        # the stored gated entries relative to max(1, max|ref|)
        check("kmix row", kx[b, i], rkx[0, -1], tol, max_scale(rkx[0, -1]))
        check("vmix row", vx[b, i], rvx[0, -1], tol, max_scale(rvx[0, -1]))
        check_act("o row", o[b, i], ro[0, -1], sh.dtype, operand_scale(sh, rkx, rvx))
        check("lse row", lse[b, :, i], rlse[0, :, -1], tol)
        flush("  row (%d, %d) ok" % (b, i))
