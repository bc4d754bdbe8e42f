"""GPU parity of attention without injection -- the layers of the causal
prefiller (sliding-window layers with W = 512 and full-attention layers,
W >= T) -- against the CPU oracle. The oracle side is the layer path with the
gate at -inf and a zero memory, which its pins tie to plain sliding-window
attention; every GPU call goes through the C ABI via the binding."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import TOL, check, check_act, flush, max_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def plain_oracle(inp, sh, grads):
    """Forward (o, lse) and, with grads, (dq, dk, dv) of attention without
    injection: gate -inf (s = 0) and zero projection weights."""
    H = sh.H
    q, k, v = (oracle.f64(inp[n]) for n in ("q", "k", "v"))
    zero = np.zeros_like(q)
    off = np.full(H, -np.inf)
    o, lse = oracle.swa_inject_fwd(q, k, v, zero, zero, off, sh.W, pos0=sh.pos0,
                                   rope_base=sh.rope_base)
    kr, _ = oracle.mixed_entries(k, v, zero, zero, off, sh.pos0, sh.rope_base)
    if not grads:
        return o, lse, kr, None
    Wz = np.zeros((H * sh.Dh, sh.d))
    g = oracle.swa_inject_bwd(q, k, v, oracle.f64(inp["m_prime"]), Wz, Wz, off,
                              oracle.f64(inp["dO"]), sh.W, pos0=sh.pos0, rope_base=sh.rope_base)
    return o, lse, kr, g


def run_case(sh, seed):
    flush("prefiller case %s seed %d" % (sh, seed))
    inp = wl.layer_inputs(sh, seed, grads=True)
    g = {n: inp[n].cuda() for n in ("q", "k", "v", "dO")}
    o, lse, kr = rms.maglev_attn_fwd(g["q"], g["k"], g["v"], sh.W, pos0=sh.pos0,
                                     rope_base=sh.rope_base)
    dq, dk, dv = rms.maglev_attn_bwd(g["q"], kr, g["v"], o, lse, g["dO"], sh.W, pos0=sh.pos0,
                                     rope_base=sh.rope_base)
    torch.cuda.synchronize()
    ro, rlse, rkr, rg = plain_oracle(inp, sh, True)
    tol = TOL[sh.dtype]
    errs = {}
    # the stored rotated keys relative to max(1, max|ref|); the outputs absolutely
    errs["krot"] = check("krot", kr, rkr, tol, max_scale(rkr))
    errs["lse"] = check("lse", lse, rlse, tol)
    for name, got, ref in (("o", o, ro), ("dq", dq, rg["dq"]), ("dk", dk, rg["dk"]),
                           ("dv", dv, rg["dv"])):
        errs[name] = check_act(name, got, ref, sh.dtype)
    flush("  errors %s" % {k: "%.2e" % v for k, v in errs.items()})


def shape(**kw):
    base = dict(B=2, T=300, W=70, d=256, H=2, Dh=128, dtype=wl.BF16)
    base.update(kw)
    return wl.LayerShape(**base)


def test_sliding_window_layer_bf16():
    run_case(shape(), 81)


def test_full_attention_layer_bf16():
    """W >= T: every earlier position is in the window (a full causal layer)."""
    run_case(shape(B=1, T=333, W=333), 82)


def test_full_attention_layer_window_beyond_sequence_dh64():
    run_case(shape(B=2, T=200, W=4096, H=3, Dh=64, d=192), 83)


def test_sliding_window_layer_fp32_pos0():
    run_case(shape(B=1, T=150, W=37, H=2, Dh=64, d=128, dtype=wl.F32, pos0=777), 84)


def test_full_attention_layer_fp32_dh128():
    run_case(shape(B=1, T=120, W=120, H=2, Dh=128, d=128, dtype=wl.F32), 85)


def test_d20_full_attention_layer_fullsize_sampled():
    """B=8, T=2048, 10 heads of 128, W = T (the prefiller's full layers):
    sampled query rows against the oracle's row-sampled forward."""
    sh = wl.LayerShape(B=8, T=2048, W=2048, d=1280, H=10, Dh=128, dtype=wl.BF16)
    inp = wl.layer_inputs(sh, 86)
    g = {n: inp[n].cuda() for n in ("q", "k", "v")}
    flush("d20 full-attention layer, full size")
    o, lse, _ = rms.maglev_attn_fwd(g["q"], g["k"], g["v"], sh.W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(86)
    rows = [(0, 0, 0), (7, 9, 2047), (3, 4, 1024), (5, 1, 511)] + \
        [(int(rng.integers(8)), int(rng.integers(10)), int(rng.integers(2048))) for _ in range(4)]
    q, k, v = (oracle.f64(inp[n]) for n in ("q", "k", "v"))
    zero = np.zeros_like(q)
    ro, rlse = oracle.swa_inject_fwd_rows(q, k, v, zero, zero, np.full(sh.H, -np.inf), sh.W, rows)
    tol = TOL[sh.dtype]
    for n, (b, h, i) in enumerate(rows):
        check_act("o(%d,%d,%d)" % (b, h, i), o[b, i, h], ro[n], sh.dtype)
        check("lse(%d,%d,%d)" % (b, h, i), lse[b, h, i:i + 1], rlse[n:n + 1], tol)


def test_full_attention_beyond_stored_score_tiles_dh128():
    """T = W = 2600 (82 query tiles a key tile, above the 80 whose dS the
    dK/dV pass stores): the dQ pass recomputes the scores instead."""
    run_case(shape(B=1, T=2600, W=2600, H=1, Dh=128, d=128), 88)


# Reach of a non-finite entry in the bf16 path beyond the band's edges: waves of
# 32 queries take whole key tiles of at most 64 keys, and the scores are masked
# (not the value operands), so 0 * NaN reaches at most 31 + 63 rows further.
NONFINITE_REACH_BF16 = 94


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_nonfinite_value_reach(dtype):
    """A NaN in one value row j of one head: every row whose band holds j is
    non-finite (as in the oracle); in bf16 no row further than
    NONFINITE_REACH_BF16 beyond the band's edges is, in float32 (one key at a
    time) exactly the band; every finite row matches the oracle run with that
    value row zeroed, and the other head is untouched."""
    sh = shape(B=1, T=700, W=100, H=2, Dh=128, dtype=dtype)
    flush("non-finite value row, %s" % (sh,))
    inp = wl.layer_inputs(sh, 83)
    j, hb = 350, 1
    v = inp["v"].clone()
    v[0, j, hb, 5] = float("nan")
    g = {n: inp[n].cuda() for n in ("q", "k")}
    o, _, _ = rms.maglev_attn_fwd(g["q"], g["k"], v.cuda(), sh.W)
    torch.cuda.synchronize()
    o = o.cpu().double().numpy()
    hit = np.nonzero(~np.isfinite(o[0, :, hb, :]).all(axis=-1))[0]
    band = np.arange(j, j + sh.W)
    assert np.isin(band, hit).all()
    reach = NONFINITE_REACH_BF16 if dtype == wl.BF16 else 0
    assert hit.min() >= j - reach and hit.max() <= j + sh.W - 1 + reach, (hit.min(), hit.max())
    flush("  non-finite rows %d..%d, band %d..%d" % (hit.min(), hit.max(), band[0], band[-1]))
    assert np.isfinite(o[0, :, 1 - hb, :]).all()
    clean = dict(inp)
    vc = inp["v"].clone()
    vc[0, j, hb, :] = 0
    clean["v"] = vc
    ro, _, _, _ = plain_oracle(clean, sh, False)
    ok = np.ones(sh.T, bool)
    ok[hit] = False
    check_act("o (finite rows)", o[0][ok][None], ro[0][ok][None], dtype)
