"""GPU parity of the loss head (final RMSNorm, soft-capped LM head, mean
cross-entropy, consistency term, and the gradients w.r.t. h and U) against
the CPU oracle. Every GPU call goes through the C ABI via the binding.

Gradients carry the 1/N of the mean, so they are judged relative to their own
largest magnitude (tol x max|ref|), and so is the loss; m, a unit-RMS state,
against max(1, |ref|)."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import TOL, check, flush, max_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def rel_scale(ref):
    ref = np.asarray(ref)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    return m if m > 0 else 1.0


def gpu_head(x, lam, with_mp, want_grads=True):
    g = {n: t.cuda() for n, t in x.items()}
    loss, m, dh, dU = rms.maglev_lm_head(g["h"], g["U"], g["targets"],
                                         m_prime=g["m_prime"] if with_mp else None, lam=lam,
                                         want_grads=want_grads)
    torch.cuda.synchronize()
    return loss, m, dh, dU


def run_case(N, d, V, dtype, seed, lam=0.0, with_mp=False, ignore=()):
    flush("loss head N=%d d=%d V=%d %s seed %d lambda %g m' %s" % (N, d, V, dtype, seed, lam,
                                                                  with_mp))
    x = wl.head_inputs(N, d, V, seed, dtype)
    for i, t in ignore:
        x["targets"][i] = t
    loss, m, dh, dU = gpu_head(x, lam, with_mp)
    ref = oracle.lm_head(oracle.f64(x["h"]), oracle.f64(x["U"]), x["targets"].numpy(),
                         m_prime=oracle.f64(x["m_prime"]) if with_mp else None, lam=lam)
    tol = TOL[dtype]
    errs = {"loss": check("loss", loss, [ref["loss"]], tol, rel_scale(ref["loss"])),
            "m": check("m", m, ref["m"], tol, max_scale(ref["m"]))}
    for n, t in (("dh", dh), ("dU", dU)):
        errs[n] = check(n, t, ref[n], tol, rel_scale(ref[n]))
    flush("  errors %s" % {k: "%.2e" % v for k, v in errs.items()})
    return x, ref


def test_head_bf16_ragged_tiles_with_consistency():
    """N and V span several GEMM tiles with ragged tails; d = 192 leaves a K
    tail in the logits product; some targets are out of range (ignored)."""
    run_case(300, 192, 1000, wl.BF16, 1, lam=0.7, with_mp=True,
             ignore=[(0, -1), (17, 1000), (299, -100)])


def test_head_bf16_no_consistency():
    run_case(257, 128, 520, wl.BF16, 2)


def test_head_fp32_ragged():
    run_case(130, 64, 264, wl.F32, 3, lam=0.3, with_mp=True, ignore=[(5, 264)])


def test_head_fp32_smallest():
    """N = 1, the smallest d and V the call accepts."""
    run_case(1, 16, 16, wl.F32, 4, lam=1.0, with_mp=True)


def test_head_bf16_smallest_single_row():
    run_case(1, 16, 16, wl.BF16, 5)


def test_head_all_targets_ignored():
    """Every target outside [0, V): the cross-entropy and its gradients vanish
    and only the consistency term remains."""
    N, d, V = 70, 64, 128
    x, ref = run_case(N, d, V, wl.F32, 6, lam=0.5, with_mp=True,
                      ignore=[(i, -1) for i in range(N)])
    assert not np.any(ref["dU"])


def test_head_accumulate_and_forward_only():
    """accumulate bits add into dh, dU and loss; with no gradient outputs the
    call gives the same loss and m."""
    N, d, V = 200, 128, 384
    x = wl.head_inputs(N, d, V, 7, wl.BF16)
    g = {n: t.cuda() for n, t in x.items()}
    flush("loss head accumulate N=%d d=%d V=%d" % (N, d, V))
    loss, m, dh, dU = rms.maglev_lm_head(g["h"], g["U"], g["targets"], m_prime=g["m_prime"],
                                         lam=0.4)
    l1, dh1, dU1 = loss.clone(), dh.clone(), dU.clone()
    rms.maglev_lm_head(g["h"], g["U"], g["targets"], m_prime=g["m_prime"], lam=0.4, loss=loss,
                       dh=dh, dU=dU, accumulate=7)
    l0, m0, dh0, dU0 = rms.maglev_lm_head(g["h"], g["U"], g["targets"], m_prime=g["m_prime"],
                                          lam=0.4, want_grads=False)
    torch.cuda.synchronize()
    assert dh0 is None and dU0 is None
    assert torch.equal(l0, l1) and torch.equal(m0, m)
    # loss += (CE mean) then += (consistency): rounding order differs from 2 x
    assert torch.allclose(loss, 2 * l1, rtol=1e-6, atol=0)
    assert torch.equal(dh, 2 * dh1) and torch.equal(dU, 2 * dU1)


def test_head_is_deterministic():
    N, d, V = 512, 256, 2048
    x = wl.head_inputs(N, d, V, 8, wl.BF16)
    flush("loss head determinism N=%d d=%d V=%d" % (N, d, V))
    a = gpu_head(x, 0.2, True)
    b = gpu_head(x, 0.2, True)
    for s, t in zip(a, b):
        assert torch.equal(s, t)


def test_head_full_size_sampled():
    """N = 16384 positions (8 x 2048), d = 1280, V = 65536: the launch the
    benchmark times. Two properties make it checkable row by row:
    (1) with every target valid, dh of row n depends on row n and on N only
        through the factor 1/N, so dh_n = (S/N) dh_n(oracle over the S sampled
        rows alone), also with the consistency term; m_n is row-local;
    (2) with every target but the sampled ones ignored, the cross-entropy
        and dU come from the sampled rows only: loss = (S/N) loss(oracle on
        those rows) and dU = (S/N) dU(oracle), and dh vanishes elsewhere."""
    N, d, V = 16384, 1280, 65536
    x = wl.head_inputs(N, d, V, 9, wl.BF16)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 8191, N - 1], rng.integers(0, N, 12)]))
    S = rows.size
    tol = TOL[wl.BF16]
    sub = {n: oracle.f64(x[n])[rows] for n in ("h", "m_prime")}
    U = oracle.f64(x["U"])

    flush("loss head full size, all targets valid, lambda 0.5")
    loss, m, dh, dU = gpu_head(x, 0.5, True)
    ref = oracle.lm_head(sub["h"], U, x["targets"].numpy()[rows], m_prime=sub["m_prime"],
                         lam=0.5)
    f = S / N
    check("m rows", m[torch.as_tensor(rows)], ref["m"], tol, max_scale(ref["m"]))
    for i, n in enumerate(rows):
        check("dh row %d" % n, dh[int(n)], f * ref["dh"][i], tol, rel_scale(f * ref["dh"][i]))

    flush("loss head full size, only the sampled targets valid")
    tg = torch.full((N,), -1, dtype=torch.int64)
    tg[torch.as_tensor(rows)] = x["targets"][torch.as_tensor(rows)]
    y = dict(x, targets=tg)
    loss, m, dh, dU = gpu_head(y, 0.0, False)
    ref = oracle.lm_head(sub["h"], U, tg.numpy()[rows])
    check("loss", loss, [f * ref["loss"]], tol, rel_scale(f * ref["loss"]))
    check("dU", dU, f * ref["dU"], tol, rel_scale(f * ref["dU"]))
    mask = torch.ones(N, dtype=torch.bool)
    mask[torch.as_tensor(rows)] = False
    assert not torch.any(dh.cpu()[mask])


def test_head_transposed_dm_path_ragged():
    """N = 16400 (a ragged last row tile of 256), d = 1280, V = 1000 (not a
    multiple of the transpose's 64-row blocks): sizes that take the dm
    product on 256 x 320 tiles over U transposed. Every target valid, so
    dh of each sampled row is (S/N) times the oracle's over the sampled rows
    alone (property (1) of the full-size test), the last row included."""
    N, d, V = 16400, 1280, 1000
    x = wl.head_inputs(N, d, V, 13, wl.BF16)
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, 255, 16383, 16384, N - 1], rng.integers(0, N, 8)]))
    S = rows.size
    tol = TOL[wl.BF16]
    flush("loss head transposed dm path N=%d d=%d V=%d" % (N, d, V))
    loss, m, dh, dU = gpu_head(x, 0.5, True)
    ref = oracle.lm_head(oracle.f64(x["h"])[rows], oracle.f64(x["U"]), x["targets"].numpy()[rows],
                         m_prime=oracle.f64(x["m_prime"])[rows], lam=0.5)
    f = S / N
    for i, n in enumerate(rows):
        check("dh row %d" % n, dh[int(n)], f * ref["dh"][i], tol, rel_scale(f * ref["dh"][i]))
