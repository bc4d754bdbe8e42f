"""Pins for the oracle's loss head (final RMSNorm, soft-capped LM head, mean
cross-entropy, consistency term) against things other than itself: closed
forms, torch's cross_entropy and rms_norm in fp64, torch autograd through a
dense formulation, central finite differences, and an invariance of the norm."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def small(N=9, d=8, V=13, seed=1):
    x = wl.head_inputs(N, d, V, seed, dtype=wl.F32)
    return {k: (oracle.f64(v) if k != "targets" else v.numpy()) for k, v in x.items()}


def test_zero_head_gives_log_vocab():
    """U = 0: every capped logit is 0, so each CE term is log V and dh, dU come
    only from the uniform softmax (dU = sum_n (1/V - onehot)/N m_n)."""
    x = small()
    U = np.zeros_like(x["U"])
    r = oracle.lm_head(x["h"], U, x["targets"])
    assert r["loss"] == pytest.approx(math.log(U.shape[0]), rel=1e-14)
    assert not np.any(r["dh"])
    N, V = x["h"].shape[0], U.shape[0]
    onehot = np.zeros((N, V))
    onehot[np.arange(N), x["targets"]] = 1.0
    np.testing.assert_allclose(r["dU"], ((1.0 / V - onehot) / N).T @ r["m"], atol=1e-15)


def test_large_cap_is_plain_cross_entropy():
    """cap -> infinity removes the soft cap: the loss equals torch's
    cross_entropy of U rms_norm(h), in fp64."""
    x = small(N=17, d=16, V=40, seed=2)
    r = oracle.lm_head(x["h"], x["U"], x["targets"], cap=1e9, grads=False)
    h = torch.from_numpy(x["h"])
    m = torch.nn.functional.rms_norm(h, (h.shape[-1],), eps=1e-6)
    ref = torch.nn.functional.cross_entropy(m @ torch.from_numpy(x["U"]).T,
                                            torch.from_numpy(x["targets"]))
    assert r["loss"] == pytest.approx(ref.item(), rel=1e-12)
    np.testing.assert_allclose(r["m"], m.numpy(), rtol=1e-13)


def test_matches_torch_autograd_with_softcap_and_consistency():
    x = small(N=11, d=8, V=21, seed=3)
    lam = 0.7
    t = {k: torch.from_numpy(x[k].copy()).requires_grad_(True) for k in ("h", "U")}
    m = torch.nn.functional.rms_norm(t["h"], (8,), eps=1e-6)
    z = 15.0 * torch.tanh(m @ t["U"].T / 15.0)
    loss = torch.nn.functional.cross_entropy(z, torch.from_numpy(x["targets"]))
    mp = torch.from_numpy(x["m_prime"])
    loss = loss + lam / (11 * math.sqrt(8)) * ((m - mp) ** 2).sum()
    loss.backward()
    r = oracle.lm_head(x["h"], x["U"], x["targets"], m_prime=x["m_prime"], lam=lam)
    assert r["loss"] == pytest.approx(loss.item(), rel=1e-12)
    np.testing.assert_allclose(r["dh"], t["h"].grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(r["dU"], t["U"].grad.numpy(), rtol=1e-10, atol=1e-13)


def test_finite_differences_with_ignored_target():
    x = small(N=6, d=4, V=7, seed=4)
    x["targets"][2] = -1           # ignored position: no CE term, still counted in N
    lam, cap = 0.3, 2.0            # a small cap makes tanh's curvature matter
    f = lambda: oracle.lm_head(x["h"], x["U"], x["targets"], m_prime=x["m_prime"], lam=lam,
                               cap=cap, grads=False)["loss"]
    r = oracle.lm_head(x["h"], x["U"], x["targets"], m_prime=x["m_prime"], lam=lam, cap=cap)
    eps = 1e-6
    for name, gname in (("h", "dh"), ("U", "dU")):
        flat = x[name].reshape(-1)
        fd = np.empty(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + eps
            fp = f()
            flat[i] = keep - eps
            fm = f()
            flat[i] = keep
            fd[i] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(r[gname].reshape(-1), fd, rtol=1e-6, atol=1e-9, err_msg=gname)


def test_norm_removes_row_scale():
    x = small(seed=5)
    a = oracle.lm_head(x["h"], x["U"], x["targets"], eps=0.0, grads=False)["loss"]
    b = oracle.lm_head(x["h"] * np.linspace(0.5, 9.0, x["h"].shape[0])[:, None], x["U"],
                       x["targets"], eps=0.0, grads=False)["loss"]
    assert a == pytest.approx(b, rel=1e-13)


def test_rows_equal_full():
    x = small(N=10, d=8, V=15, seed=6)
    r = oracle.lm_head(x["h"], x["U"], x["targets"])
    rows = [0, 3, 9]
    lse, ce, dm = oracle.lm_head_rows(x["h"], x["U"], x["targets"], rows)
    # dh from the head part alone must equal the norm backward of dm
    for i, n in enumerate(rows):
        m = r["m"][n]
        rr = 1.0 / math.sqrt(np.mean(x["h"][n] ** 2) + 1e-6)
        dh = rr * (dm[i] - m * np.mean(dm[i] * m))
        np.testing.assert_allclose(dh, r["dh"][n], rtol=1e-12, atol=1e-15)
    assert ce.sum() > 0 and np.all(lse > ce - 50)
