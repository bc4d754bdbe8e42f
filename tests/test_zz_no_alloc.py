"""The allocation-free consistency loss (maglev_consistency_loss_noalloc)
against the entry point with a caller workspace (maglev_consistency_loss),
through the C ABI: two calls in a row, the second on a smaller input, each
compared bit for bit with the workspace call on the same inputs (same
kernels, same partial-sum order) and with the oracle (loss relative 1e-4,
dm and dm' relative to their largest magnitude at 1e-3, as for the
workspace entry point). Accumulate bits are exercised on the second call."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_sliding_amd as rms
import workloads as wl
from layer_util import flush

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rms.lib()
    oracle.build(force=False)


def one_call(N, d, lam, seed, acc):
    flush("no-alloc loss: N=%d d=%d lambda=%g accumulate=%d" % (N, d, lam, acc))
    gen = torch.Generator().manual_seed(seed)
    m = torch.randn(N, d, generator=gen).bfloat16()
    mp = torch.randn(N, d, generator=gen).bfloat16()
    gm, gmp = m.cuda(), mp.cuda()
    start = {"loss": 0.75, "dm": 0.5, "dmp": -0.25} if acc else {"loss": 0.0, "dm": 0.0, "dmp": 0.0}
    outs = []
    for fn in ("workspace", "noalloc"):
        loss = torch.full((1,), start["loss"], dtype=torch.float32, device="cuda")
        dm = torch.full((N, d), start["dm"], dtype=torch.float32, device="cuda")
        dmp = torch.full((N, d), start["dmp"], dtype=torch.float32, device="cuda")
        if fn == "workspace":
            rms.maglev_consistency_loss(gm, gmp, lam, loss=loss, dm=dm, dm_prime=dmp,
                                        accumulate=acc)
        else:
            rms.maglev_consistency_loss_noalloc(gm, gmp, lam, loss, dm, dmp, accumulate=acc)
        torch.cuda.synchronize()
        outs.append((loss.cpu(), dm.cpu(), dmp.cpu()))
    (l0, dm0, dp0), (l1, dm1, dp1) = outs
    assert torch.equal(l0, l1) and torch.equal(dm0, dm1) and torch.equal(dp0, dp1)
    rl, rdm, rdmp = oracle.consistency_loss(m, mp, lam)
    got = float(l1.item()) - start["loss"]
    flush("    loss %.8e vs oracle %.8e" % (got, rl))
    assert abs(got - rl) <= 1e-4 * abs(rl)
    for name, t, ref, s0 in (("dm", dm1, rdm, start["dm"]), ("dm'", dp1, rdmp, start["dmp"])):
        err = float(np.max(np.abs(t.double().numpy() - s0 - ref)))
        flush("    %s max-abs %.3e (bar %.3e)" % (name, err, 1e-3 * np.max(np.abs(ref))))
        assert err <= 1e-3 * np.max(np.abs(ref)), name


def test_no_alloc_loss_matches_workspace_entry_point_twice():
    """Call 1 at the d20 shape's per-sequence size (2048 x 1280: the grid
    fills the whole scratch), call 2 smaller (300 x 64, ragged against the
    256-thread workgroups), accumulating into preset outputs."""
    one_call(2048, 1280, 0.1, 11, 0)
    one_call(300, 64, 1.0, 12, 7)
