"""GPU parity of the recurrent decode step (W-slot ring cache) against the CPU
oracle: ring indexing bit-exact with integer markers, teacher-forced steps
against the oracle's own decode, decode from an empty ring against the lifted
parallel pass, invalid slots never read, and a bit-identical resume."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import check, flush

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def markers(Bs, H, Dh, p, tag):
    rows = torch.full((Bs * H,), p, dtype=torch.int64)
    x = wl.marker_values(rows, Dh, tag=tag)
    x[:, 3] = torch.arange(Bs * H, dtype=torch.float32)   # stream/head id, exact
    return x.reshape(Bs, H, Dh)


@pytest.mark.parametrize("W,Dh", [(16, 128), (512, 128), (24, 64)])
def test_ring_indexing_bit_exact(W, Dh):
    """No rotation, gate -inf (s = 0): each step copies its marker verbatim into
    slot p mod W; after n steps the GPU ring equals the oracle ring bitwise."""
    Bs, H = 3, 2
    dev = "cuda"
    kc = torch.full((Bs, H, W, Dh), -7.0, dtype=torch.bfloat16, device=dev)
    vc = kc.clone()
    okc = np.full((Bs, H, W, Dh), -7.0)
    ovc = okc.copy()
    gate = torch.full((H,), float("-inf"), device=dev)
    pos = torch.zeros(Bs, dtype=torch.int64, device=dev)
    zero = torch.zeros((Bs, H, Dh), dtype=torch.bfloat16, device=dev)
    checkpoints = {1, W - 1, W, W + 1, 3 * W + 5}
    for p in range(max(checkpoints)):
        mk = markers(Bs, H, Dh, p, 1.0).to(torch.bfloat16)
        mv = markers(Bs, H, Dh, p, 2.0).to(torch.bfloat16)
        rms.maglev_decode_step(zero, mk.to(dev), mv.to(dev), zero, zero, gate, kc, vc, pos,
                               rope_base=0.0)
        rms.maglev_decode_advance(pos)
        oracle.decode_step(np.zeros((Bs, H, Dh)), mk, mv, np.zeros((Bs, H, Dh)),
                           np.zeros((Bs, H, Dh)), gate.cpu(), okc, ovc, np.full(Bs, p),
                           rope_base=0.0)
        if p + 1 in checkpoints:
            torch.cuda.synchronize()
            flush("W=%d Dh=%d after %d steps" % (W, Dh, p + 1))
            assert np.array_equal(kc.cpu().double().numpy(), okc)
            assert np.array_equal(vc.cpu().double().numpy(), ovc)
    assert torch.equal(pos.cpu(), torch.full((Bs,), max(checkpoints), dtype=torch.int64))


@pytest.mark.parametrize("dtype,Dh", [(wl.BF16, 128), (wl.BF16, 64), (wl.F32, 128)])
def test_teacher_forced_steps_match_oracle(dtype, Dh):
    """Prefilled ring (positions 0..W-1), then 2W+3 steps from p = W with fresh
    q, k, v, kmem, vmem per step; o checked every step, the ring at the end
    (new entries may differ by one rounding step of the storage type)."""
    Bs, H, W = 4, 3, 40
    tol = 2e-2 if dtype == wl.BF16 else 1e-4
    tdt = wl.torch_dtype(dtype)
    gen = torch.Generator().manual_seed(40 + Dh)
    rnd = lambda *s: torch.randn(*s, generator=gen).to(tdt)
    kc0, vc0 = rnd(Bs, H, W, Dh), rnd(Bs, H, W, Dh)
    gate = torch.randn(H, generator=gen)
    kc, vc = kc0.cuda(), vc0.cuda()
    okc, ovc = oracle.f64(kc0), oracle.f64(vc0)
    pos = torch.full((Bs,), W, dtype=torch.int64).cuda()
    for step in range(2 * W + 3):
        q, k, v, km, vm = (rnd(Bs, H, Dh) for _ in range(5))
        o = rms.maglev_decode_step(q.cuda(), k.cuda(), v.cuda(), km.cuda(), vm.cuda(), gate.cuda(),
                                   kc, vc, pos)
        rms.maglev_decode_advance(pos)
        ro = oracle.decode_step(q, k, v, km, vm, gate, okc, ovc, np.full(Bs, W + step),
                                ring_bf16=(dtype == wl.BF16))
        torch.cuda.synchronize()
        check("o step %d" % step, o, ro, tol)
    # one rounding step of the storage type (bf16: 2^-7 relative), or float32 round-off
    rel = 2.0 ** -7 if dtype == wl.BF16 else 1e-6
    for name, got, ref in (("kcache", kc, okc), ("vcache", vc, ovc)):
        diff = np.abs(got.cpu().double().numpy() - ref)
        assert np.all(diff <= rel * np.abs(ref) + 1e-5), name


def test_decode_from_empty_ring_equals_lifted_pass():
    """Positions 0..T-1 decoded one at a time from a NaN-filled ring (slots not
    yet written are never read), fed the same shifted memory projection as the
    parallel pass, reproduce the oracle's lifted-pass output at every t."""
    sh = wl.LayerShape(B=2, T=100, W=32, d=256, H=2, Dh=128, dtype=wl.BF16)
    inp = wl.layer_inputs(sh, 50)
    g = {k: v.cuda() for k, v in inp.items()}
    km, vm = rms.maglev_mem_project(g["m_prime"], g["W_Km"], g["W_Vm"], sh.H, sh.Dh, shift=1)
    kc = torch.full((sh.B, sh.H, sh.W, sh.Dh), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = kc.clone()
    pos = torch.zeros(sh.B, dtype=torch.int64, device="cuda")
    outs = []
    for t in range(sh.T):
        sl = lambda x: x[:, t].contiguous()
        outs.append(rms.maglev_decode_step(sl(g["q"]), sl(g["k"]), sl(g["v"]), sl(km), sl(vm),
                                           g["gate_logit"], kc, vc, pos))
        rms.maglev_decode_advance(pos)
    torch.cuda.synchronize()
    rkm, rvm = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], sh.H, sh.Dh)
    ro, _ = oracle.swa_inject_fwd(inp["q"], inp["k"], inp["v"], rkm, rvm, inp["gate_logit"], sh.W)
    check("decode vs lifted pass", torch.stack(outs, dim=1), ro, 2e-2)


def test_memory_projection_of_one_row():
    """shift = 0, T = 1: the decode step's kmem/vmem for m_{t-1}."""
    Bs, d, H, Dh = 64, 1280, 10, 128
    gen = torch.Generator().manual_seed(60)
    m = torch.randn(Bs, 1, d, generator=gen).bfloat16()
    WK = (torch.randn(H * Dh, d, generator=gen) / d ** 0.5).bfloat16()
    WV = (torch.randn(H * Dh, d, generator=gen) / d ** 0.5).bfloat16()
    km, vm = rms.maglev_mem_project(m.cuda(), WK.cuda(), WV.cuda(), H, Dh, shift=0)
    torch.cuda.synchronize()
    rkm, rvm = oracle.mem_project(m, WK, WV, H, Dh, shift=0)
    check("kmem", km, rkm, 2e-2)
    check("vmem", vm, rvm, 2e-2)


def test_wide_projection_of_few_rows():
    """Few rows against many output columns (the per-step projection of every
    layer's stacked weights): 5 rows x 2 x 40 heads x 128."""
    Bs, d, H, Dh = 5, 256, 40, 128
    gen = torch.Generator().manual_seed(61)
    m = torch.randn(Bs, 1, d, generator=gen).bfloat16()
    WK = (torch.randn(H * Dh, d, generator=gen) / d ** 0.5).bfloat16()
    WV = (torch.randn(H * Dh, d, generator=gen) / d ** 0.5).bfloat16()
    km, vm = rms.maglev_mem_project(m.cuda(), WK.cuda(), WV.cuda(), H, Dh, shift=0)
    torch.cuda.synchronize()
    rkm, rvm = oracle.mem_project(m, WK, WV, H, Dh, shift=0)
    check("kmem", km, rkm, 2e-2)
    check("vmem", vm, rvm, 2e-2)


def test_strided_memory_equals_packed():
    """Reading one layer's slice of a stacked projection through mem_stride
    gives bit-identical steps to the same values packed."""
    Bs, H, Dh, W, L, d = 3, 2, 128, 24, 3, 256
    gen = torch.Generator().manual_seed(62)
    rnd = lambda *s: torch.randn(*s, generator=gen).bfloat16().cuda()
    kall, vall = rnd(Bs, L * H * Dh), rnd(Bs, L * H * Dh)
    gate = torch.randn(H, generator=gen).cuda()
    q, k, v = rnd(Bs, H, Dh), rnd(Bs, H, Dh), rnd(Bs, H, Dh)
    kc0, vc0 = rnd(Bs, H, W, Dh), rnd(Bs, H, W, Dh)
    pos = torch.tensor([W + 3, 5, 1000], dtype=torch.int64, device="cuda")
    for l in range(L):
        sk, sv = kall[:, l * H * Dh:(l + 1) * H * Dh], vall[:, l * H * Dh:(l + 1) * H * Dh]
        kc1, vc1, kc2, vc2 = kc0.clone(), vc0.clone(), kc0.clone(), vc0.clone()
        o1 = rms.maglev_decode_step(q, k, v, sk, sv, gate, kc1, vc1, pos, mem_stride=L * H * Dh)
        o2 = rms.maglev_decode_step(q, k, v, sk.contiguous().view(Bs, H, Dh),
                                    sv.contiguous().view(Bs, H, Dh), gate, kc2, vc2, pos)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(kc1, kc2) and torch.equal(vc1, vc2), l


def test_snapshot_restore_is_bit_identical():
    """The whole recurrent state of a stream is (ring, position, memory):
    copying it out and back in gives a bit-identical continuation."""
    Bs, H, Dh, W, d = 2, 2, 128, 24, 256
    gen = torch.Generator().manual_seed(70)
    rnd = lambda *s: torch.randn(*s, generator=gen).bfloat16().cuda()
    WK, WV = rnd(H * Dh, d) * 0.06, rnd(H * Dh, d) * 0.06
    gate = torch.randn(H, generator=gen).cuda()
    steps = [tuple(rnd(Bs, H, Dh) for _ in range(3)) for _ in range(40)]
    kc, vc = rnd(Bs, H, W, Dh), rnd(Bs, H, W, Dh)
    pos = torch.full((Bs,), W, dtype=torch.int64, device="cuda")
    m = rnd(Bs, 1, d)

    def run(state, lo, hi):
        kc, vc, pos, m = state
        outs = []
        for t in range(lo, hi):
            km, vm = rms.maglev_mem_project(m, WK, WV, H, Dh, shift=0)
            q, k, v = steps[t]
            o = rms.maglev_decode_step(q, k, v, km.view(Bs, H, Dh), vm.view(Bs, H, Dh), gate, kc,
                                       vc, pos)
            rms.maglev_decode_advance(pos)
            m = o.reshape(Bs, 1, d).contiguous()   # stand-in memory: the layer output
            outs.append(o.clone())
        return (kc, vc, pos, m), outs

    state, _ = run((kc, vc, pos, m), 0, 15)
    snap = tuple(x.cpu().clone() for x in state)
    state, a = run(state, 15, 40)
    state[0].fill_(0.0); state[1].fill_(0.0); state[2].fill_(0)
    restored = tuple(x.cuda() for x in snap)
    _, b = run(restored, 15, 40)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_graph_replay_matches_eager_steps():
    """Two identical stacks: one stepped eagerly, one by replaying captured HIP
    graphs (one per q/k/v set), with eager work and synchronisation between the
    replays. Every replay's outputs, rings and positions equal the eager ones bitwise."""
    from recurrent_memory_sliding_amd.decode import DecodeStack

    L, Bs, H, Dh, W = 2, 4, 2, 128, 24
    d = H * Dh
    gen = torch.Generator().manual_seed(80)
    rnd = lambda *s: torch.randn(*s, generator=gen).bfloat16()
    weights = [{"W_Km": (rnd(H * Dh, d) * 0.06).cuda(), "W_Vm": (rnd(H * Dh, d) * 0.06).cuda(),
                "gate_logit": torch.randn(H, generator=gen).cuda()} for _ in range(L)]
    rings = [(rnd(Bs, H, W, Dh), rnd(Bs, H, W, Dh)) for _ in range(L)]
    m0 = rnd(Bs, d)
    pool = [[tuple(rnd(Bs, H, Dh).cuda() for _ in range(3)) for _ in range(L)] for _ in range(3)]

    def make():
        return DecodeStack(weights, [r[0].cuda() for r in rings], [r[1].cuda() for r in rings],
                           torch.full((Bs,), W, dtype=torch.int64, device="cuda"), m0.cuda())

    eager, graphed = make(), make()
    qkv = lambda e: ([x[0] for x in pool[e]], [x[1] for x in pool[e]], [x[2] for x in pool[e]])
    for e in range(3):
        graphed.capture(e, *qkv(e))
    for t in range(12):
        a = [o.clone() for o in eager.step(*qkv(t % 3))]
        junk = torch.randn(1000, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        b = [o.clone() for o in graphed.replay(t % 3)]
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), t
        for l in range(L):
            assert torch.equal(eager.kcache[l], graphed.kcache[l])
        assert torch.equal(eager.pos, graphed.pos)


def test_negative_position_stream_is_skipped():
    """A stream whose position is negative writes nothing (ring and o keep
    their contents); the other streams of the same call are unaffected."""
    Bs, H, Dh, W = 3, 2, 128, 24
    gen = torch.Generator().manual_seed(90)
    rnd = lambda *s: torch.randn(*s, generator=gen).bfloat16()
    q, k, v, km, vm = (rnd(Bs, H, Dh) for _ in range(5))
    kc0, vc0 = rnd(Bs, H, W, Dh), rnd(Bs, H, W, Dh)
    gate = torch.randn(H, generator=gen)
    kc, vc = kc0.cuda(), vc0.cuda()
    o = torch.full((Bs, H, Dh), 7.0, dtype=torch.bfloat16, device="cuda")
    pos = torch.tensor([W + 5, -1, 3], dtype=torch.int64, device="cuda")
    rms.maglev_decode_step(q.cuda(), k.cuda(), v.cuda(), km.cuda(), vm.cuda(), gate.cuda(), kc,
                           vc, pos, o=o)
    torch.cuda.synchronize()
    assert torch.equal(kc[1].cpu(), kc0[1]) and torch.equal(vc[1].cpu(), vc0[1])
    assert torch.all(o[1].cpu() == 7.0)
    okc, ovc = oracle.f64(kc0[[0, 2]]), oracle.f64(vc0[[0, 2]])
    ro = oracle.decode_step(q[[0, 2]], k[[0, 2]], v[[0, 2]], km[[0, 2]], vm[[0, 2]], gate, okc,
                            ovc, np.array([W + 5, 3]))
    check("o of the other streams", o[[0, 2]], ro, 2e-2)
