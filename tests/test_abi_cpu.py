"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/maglev.h declares, sizes its workspaces, and rejects
invalid arguments with the documented status before anything is enqueued.
No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import recurrent_memory_sliding_amd as rms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "maglev.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP = range(6)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rms.library_path()):
        pytest.skip("libmaglev.so not built")
    return rms.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(maglev_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["maglev_mem_project", "maglev_swa_inject_fwd", "maglev_swa_inject_bwd",
              "maglev_decode_step", "maglev_consistency_loss", "maglev_mem_project_gated",
              "maglev_swa_inject_bwd_gated", "maglev_decode_step_gated", "maglev_lm_head"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_library_exports_nothing_else():
    """The dynamic symbol table holds the declared C functions and nothing of
    the library's internals (kernels, launchers, helpers)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", rms.library_path()], capture_output=True,
                         text=True, check=True).stdout
    names = {l.split()[-1] for l in out.splitlines() if l.strip()}
    ours = {n for n in names if "maglev" in n}
    assert ours == set(declared_functions()), sorted(ours ^ set(declared_functions()))


def test_abi_version_and_status_strings(L):
    assert L.maglev_abi_version() == 6
    assert L.maglev_status_string(OK) == b"MAGLEV_OK"
    assert L.maglev_status_string(WORKSPACE) == b"MAGLEV_ERR_WORKSPACE"
    assert L.maglev_status_string(99) == b"MAGLEV_ERR_UNKNOWN"


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: every case below fails validation
FAKE_ODD = ctypes.c_void_p(0x10008)  # 8-byte aligned only


def geom(**kw):
    base = dict(B=2, T=64, H=2, Dh=128, d=256, W=16, pos0=0, rope_base=1e4, scale=0.0, dtype=1)
    base.update(kw)
    return rms.Geom(**base)


NO_MIX = [FAKE] * 3 + [None] * 3 + [FAKE] * 2 + [None] * 2   # m W_Km W_Vm | k v gate | kmem vmem | kmix vmix


def project(L, g, shift=1, ptrs=None):
    p = ptrs or NO_MIX
    return L.maglev_mem_project(ctypes.byref(g) if g is not None else None, shift, *p, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Dh=96), UNSUPPORTED), (dict(Dh=32), UNSUPPORTED), (dict(H=0), INVALID),
    (dict(d=100), INVALID), (dict(d=0), INVALID), (dict(W=0), INVALID), (dict(B=-1), INVALID),
    (dict(T=-5), INVALID), (dict(pos0=-1), INVALID), (dict(dtype=7), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(H=513, Dh=128), UNSUPPORTED),
])
def test_projection_rejects_bad_geometry(L, kw, status):
    assert project(L, geom(**kw)) == status


def test_projection_rejects_null_geometry_shift_and_pointers(L):
    assert project(L, None) == INVALID
    assert project(L, geom(), shift=2) == INVALID
    bad = list(NO_MIX); bad[1] = None   # W_Km
    assert project(L, geom(), ptrs=bad) == INVALID
    bad = list(NO_MIX); bad[6] = FAKE_ODD   # kmem
    assert project(L, geom(), ptrs=bad) == MISALIGNED
    assert b"aligned" in L.maglev_last_error()


@pytest.mark.parametrize("present", [(3,), (3, 4, 5), (3, 4, 5, 8), (8, 9), (5,)])
def test_projection_mixing_arguments_come_together(L, present):
    """k, v, gate, kmix, vmix (positions 3, 4, 5, 8, 9) are all given or all null."""
    p = list(NO_MIX)
    for i in present:
        p[i] = FAKE
    assert project(L, geom(), ptrs=p) == INVALID


def test_empty_batch_is_a_no_op(L):
    # B = 0 returns OK without touching any pointer or the device.
    assert project(L, geom(B=0)) == OK
    assert L.maglev_swa_inject_fwd(ctypes.byref(geom(T=0)), *([FAKE] * 5), None) == OK


def test_forward_validation(L):
    g = geom()
    args = [FAKE] * 5   # q kmix vmix o lse
    assert L.maglev_swa_inject_fwd(ctypes.byref(geom(Dh=80)), *args, None) == UNSUPPORTED
    bad = list(args); bad[1] = None  # kmix
    assert L.maglev_swa_inject_fwd(ctypes.byref(g), *bad, None) == INVALID
    bad = list(args); bad[4] = FAKE_ODD  # lse misaligned
    assert L.maglev_swa_inject_fwd(ctypes.byref(g), *bad, None) == MISALIGNED


def test_backward_workspace_query_and_validation(L):
    g = geom(B=8, T=2048, H=10, Dh=128, d=1280, W=512)
    need = L.maglev_swa_inject_bwd_workspace(ctypes.byref(g))
    # row-dot + gate partials (B*H*T floats each) + scaled weights + split-K partials
    assert need >= 2 * 8 * 10 * 2048 * 4 + 2 * 1280 * 1280 * 2
    assert L.maglev_swa_inject_bwd_workspace(ctypes.byref(geom(Dh=96))) == 0
    ptrs = [FAKE] * 19
    assert L.maglev_swa_inject_bwd(ctypes.byref(g), *ptrs, 0, None, 0, None) == WORKSPACE
    assert L.maglev_swa_inject_bwd(ctypes.byref(g), *ptrs, 0, FAKE, need - 1, None) == WORKSPACE
    assert L.maglev_swa_inject_bwd(ctypes.byref(g), *ptrs, 8, FAKE, need, None) == INVALID
    bad = list(ptrs); bad[12] = None  # dq
    assert L.maglev_swa_inject_bwd(ctypes.byref(g), *bad, 0, FAKE, need, None) == INVALID


def test_loss_validation(L):
    need = L.maglev_consistency_loss_workspace(16384, 1280)
    assert need > 0
    assert L.maglev_consistency_loss_workspace(10, 12) == 0
    base = [FAKE, FAKE, FAKE, None, None, 0, FAKE, need, None]
    assert L.maglev_consistency_loss(-1, 64, 1.0, 1, *base) == INVALID
    assert L.maglev_consistency_loss(4, 12, 1.0, 1, *base) == INVALID
    assert L.maglev_consistency_loss(4, 64, 1.0, 5, *base) == INVALID
    assert L.maglev_consistency_loss(4, 64, float("nan"), 1, *base) == INVALID
    nows = list(base); nows[6] = None
    assert L.maglev_consistency_loss(4, 64, 1.0, 1, *nows) == WORKSPACE
    noloss = list(base); noloss[2] = None
    assert L.maglev_consistency_loss(4, 64, 1.0, 1, *noloss) == INVALID


def test_decode_validation(L):
    need = L.maglev_decode_workspace(64, 10, 128, 512)
    assert need == 0                                     # the step needs no scratch
    head = [FAKE] * 5                                    # q k v kmem vmem
    tail = [FAKE] * 5                                    # gate kcache vcache pos o
    args = lambda **kw: [kw.get("Bs", 64), 10, kw.get("Dh", 128), kw.get("W", 512), 1e4, 0.0,
                         kw.get("dtype", 1)]
    step = lambda a, stride=0, t=tail, ws=FAKE, n=need: L.maglev_decode_step(*a, *head, stride, *t,
                                                                             ws, n, None)
    assert step(args(Dh=48)) == UNSUPPORTED
    assert step(args(W=0)) == INVALID
    bad = list(tail); bad[3] = None  # pos
    assert step(args(), t=bad) == INVALID
    assert step(args(), stride=10 * 128 - 8) == INVALID   # below H*Dh
    assert step(args(), stride=10 * 128 + 4) == INVALID   # not a multiple of 8
    assert step(args(Bs=2 ** 30, W=1)) == INVALID        # Bs*H at or above 2^31 workgroups
    assert step(args(Bs=0)) == OK
    assert step(args(Bs=0), stride=20 * 10 * 128) == OK
    assert L.maglev_decode_advance(5, None, None) == INVALID
    assert L.maglev_decode_advance(0, FAKE, None) == OK


# ---- gated form -------------------------------------------------------------
def project_gated(L, g, shift=1, eps=1e-6, ptrs=None, gates=FAKE):
    p = ptrs or [FAKE] * 5            # m W_Km W_Vm k v
    out = [FAKE] * 4                  # kproj vmem kmix vmix
    return L.maglev_mem_project_gated(ctypes.byref(g) if g is not None else None, shift, *p,
                                      gates, eps, *out, None)


def test_gated_projection_validation(L):
    assert project_gated(L, None) == INVALID
    assert project_gated(L, geom(), shift=3) == INVALID
    assert project_gated(L, geom(), gates=None) == INVALID
    assert project_gated(L, geom(), eps=-1.0) == INVALID
    assert project_gated(L, geom(), eps=float("nan")) == INVALID
    assert project_gated(L, geom(), eps=float("inf")) == INVALID
    assert project_gated(L, geom(H=40, Dh=128)) == UNSUPPORTED     # H*Dh above 4096
    assert project_gated(L, geom(Dh=96)) == UNSUPPORTED
    bad = [FAKE] * 5; bad[3] = None                                   # k
    assert project_gated(L, geom(), ptrs=bad) == INVALID
    bad = [FAKE] * 5; bad[4] = FAKE_ODD                               # v
    assert project_gated(L, geom(), ptrs=bad) == MISALIGNED
    assert project_gated(L, geom(B=0)) == OK                          # empty: nothing read


def test_gated_backward_workspace_and_validation(L):
    g = geom(B=8, T=2048, H=10, Dh=128, d=1280, W=512)
    base = L.maglev_swa_inject_bwd_workspace(ctypes.byref(g))
    need = L.maglev_swa_inject_bwd_gated_workspace(ctypes.byref(g))
    # the two projection gradients (bf16) and the gate partials come on top
    assert need >= base + 2 * 8 * 2048 * 1280 * 2 + 4 * 1280 * 4
    assert L.maglev_swa_inject_bwd_gated_workspace(ctypes.byref(geom(H=40))) == 0
    head = [FAKE] * 8                 # q kmix vmix k v kproj vmem gates
    tail = [FAKE] * 13                # o lse dO m' W_Km W_Vm dq dk dv dm' dWk dWv dgates
    call = lambda g, h=head, eps=1e-6, t=tail, acc=0, ws=FAKE, n=need: \
        L.maglev_swa_inject_bwd_gated(ctypes.byref(g), *h, eps, *t, acc, ws, n, None)
    assert call(g, ws=None) == WORKSPACE
    assert call(g, n=need - 1) == WORKSPACE
    assert call(g, acc=8) == INVALID
    assert call(g, eps=-1e-3) == INVALID
    bad = list(head); bad[7] = None   # gates
    assert call(g, h=bad) == INVALID
    bad = list(tail); bad[12] = None  # dgates
    assert call(g, t=bad) == INVALID
    bad = list(tail); bad[7] = FAKE_ODD  # dk
    assert call(g, t=bad) == MISALIGNED


def test_gated_decode_validation(L):
    head = [FAKE] * 5                 # q k v kproj vmem
    tail = [FAKE] * 4                 # kcache vcache pos o
    a = lambda **kw: [kw.get("Bs", 64), 10, kw.get("Dh", 128), kw.get("W", 512), 1e4, 0.0,
                      kw.get("dtype", 1)]
    step = lambda args, stride=0, gates=FAKE, eps=1e-6, t=tail: L.maglev_decode_step_gated(
        *args, *head, stride, gates, eps, *t, FAKE, 0, None)
    assert step(a(Dh=48)) == UNSUPPORTED
    assert step(a(), gates=None) == INVALID
    assert step(a(), eps=-1.0) == INVALID
    assert step(a(), stride=10 * 128 - 8) == INVALID
    bad = list(tail); bad[2] = None   # pos
    assert step(a(), t=bad) == INVALID
    assert step(a(Bs=2 ** 30, W=1)) == INVALID   # Bs*H at or above 2^31 workgroups
    assert step(a(Bs=0)) == OK


def test_attention_only_validation(L):
    g = geom(B=8, T=2048, H=10, Dh=128, d=1280, W=2048)
    need = L.maglev_attn_bwd_workspace(ctypes.byref(g))
    # rotated queries (bf16) and the padded lse / D rows; no projection scratch
    assert 8 * 2048 * 1280 * 2 <= need < L.maglev_swa_inject_bwd_workspace(ctypes.byref(g))
    assert L.maglev_attn_bwd_workspace(ctypes.byref(geom(Dh=96))) == 0
    assert L.maglev_rope_keys(ctypes.byref(geom(Dh=96)), FAKE, FAKE, None) == UNSUPPORTED
    assert L.maglev_rope_keys(ctypes.byref(geom()), FAKE, FAKE, None) == INVALID   # aliasing
    assert L.maglev_rope_keys(ctypes.byref(geom()), FAKE_ODD, FAKE, None) == MISALIGNED
    assert L.maglev_rope_keys(ctypes.byref(geom(T=0)), None, None, None) == OK
    ptrs = [FAKE] * 9                 # q krot v o lse dO dq dk dv
    assert L.maglev_attn_bwd(ctypes.byref(g), *ptrs, None, 0, None) == WORKSPACE
    assert L.maglev_attn_bwd(ctypes.byref(g), *ptrs, FAKE, need - 1, None) == WORKSPACE
    assert L.maglev_attn_bwd(ctypes.byref(g), *ptrs, FAKE_ODD, need, None) == MISALIGNED
    bad = list(ptrs); bad[4] = None   # lse
    assert L.maglev_attn_bwd(ctypes.byref(g), *bad, FAKE, need, None) == INVALID
    assert L.maglev_attn_bwd(ctypes.byref(geom(B=0)), *([None] * 9), None, 0, None) == OK


def test_shared_projection_validation(L):
    g = geom(B=4, T=2048, H=10, Dh=128, d=1280, W=512)
    args = [FAKE] * 7                 # k v kmem vmem gate kmix vmix
    assert L.maglev_mix_entries(ctypes.byref(geom(Dh=96)), *args, None) == UNSUPPORTED
    bad = list(args); bad[4] = None   # gate
    assert L.maglev_mix_entries(ctypes.byref(g), *bad, None) == INVALID
    bad = list(args); bad[2] = FAKE_ODD
    assert L.maglev_mix_entries(ctypes.byref(g), *bad, None) == MISALIGNED
    need = L.maglev_swa_inject_bwd_shared_workspace(ctypes.byref(g))
    assert need >= L.maglev_attn_bwd_workspace(ctypes.byref(g))
    ptrs = [FAKE] * 15                # q kmix vmix kmem vmem gate o lse dO dq dk dv dkmem dvmem dgate
    call = lambda p=ptrs, acc=0, ws=FAKE, n=need: L.maglev_swa_inject_bwd_shared(
        ctypes.byref(g), *p, acc, ws, n, None)
    assert call(acc=2) == INVALID     # only bits 0 and 2
    assert call(ws=None) == WORKSPACE
    assert call(n=need - 1) == WORKSPACE
    bad = list(ptrs); bad[12] = None  # dkmem
    assert call(p=bad) == INVALID
    pneed = L.maglev_mem_project_bwd_workspace(ctypes.byref(g))
    assert pneed >= 2 * 4 * 2048 * 1280 * 2   # the bf16 roundings of dkmem, dvmem
    pp = [FAKE] * 8                   # dkmem dvmem m' W_Km W_Vm dm' dWk dWv
    assert L.maglev_mem_project_bwd(ctypes.byref(g), *pp, 4, FAKE, pneed, None) == INVALID
    assert L.maglev_mem_project_bwd(ctypes.byref(g), *pp, 0, None, 0, None) == WORKSPACE
    bad = list(pp); bad[2] = None     # m'
    assert L.maglev_mem_project_bwd(ctypes.byref(g), *bad, 0, FAKE, pneed, None) == INVALID


def test_gated_shared_projection_validation(L):
    g = geom(B=4, T=2048, H=10, Dh=128, d=1280, W=512)
    ff, vp = ctypes.c_float, ctypes.c_void_p
    mix = lambda g, a=(FAKE,) * 5, eps=1e-6, out=(FAKE, FAKE): L.maglev_mix_entries_gated(
        ctypes.byref(g), *a, ff(eps), *out, None)     # k v kproj vmem gates | kmix vmix
    assert mix(geom(Dh=96)) == UNSUPPORTED
    assert mix(geom(H=40)) == UNSUPPORTED              # H*Dh above 4096
    assert mix(g, eps=-1.0) == INVALID
    assert mix(g, a=(FAKE,) * 4 + (None,)) == INVALID  # gates
    assert mix(g, out=(FAKE, FAKE_ODD)) == MISALIGNED
    assert mix(geom(B=0)) == OK
    need = L.maglev_swa_inject_bwd_shared_gated_workspace(ctypes.byref(g))
    # the attention scratch and the gate partials, no projection scratch
    assert L.maglev_attn_bwd_workspace(ctypes.byref(g)) < need
    assert need < L.maglev_swa_inject_bwd_gated_workspace(ctypes.byref(g))
    assert L.maglev_swa_inject_bwd_shared_gated_workspace(ctypes.byref(geom(H=40))) == 0
    head = [FAKE] * 8                 # q kmix vmix k v kproj vmem gates
    tail = [FAKE] * 9                 # o lse dO dq dk dv dkproj dvmem dgates
    call = lambda h=head, eps=1e-6, t=tail, acc=0, ws=FAKE, n=need: \
        L.maglev_swa_inject_bwd_shared_gated(ctypes.byref(g), *h, ff(eps), *t, acc, ws, n, None)
    assert call(acc=2) == INVALID     # only bits 0 and 2
    assert call(eps=float("nan")) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(n=need - 1) == WORKSPACE
    assert call(ws=FAKE_ODD) == MISALIGNED
    bad = list(head); bad[7] = None   # gates
    assert call(h=bad) == INVALID
    bad = list(tail); bad[8] = None   # dgates
    assert call(t=bad) == INVALID
    bad = list(tail); bad[6] = None   # dkproj
    assert call(t=bad) == INVALID
    assert L.maglev_swa_inject_bwd_shared_gated(ctypes.byref(geom(B=0)), *([None] * 7), FAKE,
                                                ff(1e-6), *([None] * 8), FAKE, 4, None, 0,
                                                None) == OK   # dgates kept (bit 2), nothing read


def test_loss_head_workspace_and_validation(L):
    need = L.maglev_lm_head_workspace(16384, 1280, 65536, 1)
    # float32 logits and bf16 dz dominate: 6 N V bytes
    assert need >= 6 * 16384 * 65536
    assert L.maglev_lm_head_workspace(16384, 1280, 65536, 0) > need
    for bad in [(0, 64, 64, 1), (4, 40, 64, 1), (4, 64, 12, 1), (4, 64, 8, 1), (4, 64, 64, 3)]:
        assert L.maglev_lm_head_workspace(*bad) == 0
    w = L.maglev_lm_head_workspace(4, 64, 64, 1)
    # h U targets m_prime m loss dh dU
    ptrs = [FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None]

    def call(N=4, d=64, V=64, cap=15.0, eps=1e-6, lam=0.0, dtype=1, p=None, acc=0, ws=FAKE,
             wsb=None):
        return L.maglev_lm_head(N, d, V, cap, eps, lam, dtype, *(p or ptrs), acc, ws,
                                w if wsb is None else wsb, None)

    assert call(N=0) == INVALID
    assert call(d=40) == INVALID
    assert call(V=12) == INVALID
    assert call(V=8) == INVALID
    assert call(cap=0.0) == INVALID
    assert call(cap=float("inf")) == INVALID
    assert call(cap=64.5) == INVALID
    assert call(cap=float("nan")) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(lam=float("nan")) == INVALID
    assert call(dtype=4) == INVALID
    assert call(acc=8) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(wsb=w - 1) == WORKSPACE
    assert call(ws=FAKE_ODD) == MISALIGNED
    for i, status in [(0, INVALID), (1, INVALID), (2, INVALID), (4, INVALID), (5, INVALID)]:
        bad = list(ptrs); bad[i] = None
        assert call(p=bad) == status, i
    for i in (0, 1, 3, 4, 6, 7):
        bad = list(ptrs); bad[i] = FAKE_ODD
        assert call(p=bad) == MISALIGNED, i


def test_prepare_validation(L):
    assert L.maglev_prepare(100, 1e4, 10) == UNSUPPORTED
    assert L.maglev_prepare(128, 1e4, -1) == INVALID
    # rope_base <= 0 disables the rotation: nothing to allocate; the set-up
    # still looks up the allocation-free loss's scratch on the current
    # device, which a host without a GPU does not have
    import torch
    assert L.maglev_prepare(128, 0.0, 1000) == (OK if torch.cuda.device_count() > 0 else HIP)


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    x = torch.zeros(2, 4, 64)
    with pytest.raises(rms.MaglevError):
        rms.maglev_mem_project(x, torch.zeros(64, 64), torch.zeros(64, 64), 1, 64)


def test_decode_binding_checks_every_shape_the_kernel_assumes():
    """The decode binding's shape checks (pure host logic, run before any
    launch): rings alike, q/k/v/o [Bs,H,Dh], gate logits [H] or [4,H*Dh]."""
    import torch

    chk = rms._decode_shapes
    Bs, H, W, Dh = 3, 2, 8, 64
    ring = torch.zeros(Bs, H, W, Dh)
    row = torch.zeros(Bs, H, Dh)
    gate = torch.zeros(H)
    chk(ring, ring, row, row, row, None, gate, False)                  # valid
    chk(ring, ring, row, row, row, row, torch.zeros(4, H * Dh), True)  # valid, gated
    bad = [
        (ring, torch.zeros(Bs, H, W + 1, Dh), row, row, row, None, gate, False),
        (torch.zeros(Bs, H, W), ring, row, row, row, None, gate, False),
        (ring, ring, torch.zeros(Bs, H, Dh + 1), row, row, None, gate, False),
        (ring, ring, row, torch.zeros(Bs + 1, H, Dh), row, None, gate, False),
        (ring, ring, row, row, torch.zeros(Bs * H * Dh), None, gate, False),
        (ring, ring, row, row, row, torch.zeros(Bs, H, 2 * Dh), gate, False),
        (ring, ring, row, row, row, None, torch.zeros(H + 1), False),
        (ring, ring, row, row, row, None, gate, True),
    ]
    for args in bad:
        with pytest.raises(rms.MaglevError):
            chk(*args)


def test_no_alloc_loss_validation(L):
    """The allocation-free loss rejects what the workspace call rejects,
    before any device work (the scratch address is only looked up after)."""
    f = L.maglev_consistency_loss_noalloc
    f.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_int32] + \
        [ctypes.c_void_p] * 5 + [ctypes.c_uint, ctypes.c_void_p]
    f.restype = ctypes.c_int32
    ok = dict(N=4, d=64, lam=0.1, dtype=1, m=FAKE, mp=FAKE, loss=FAKE, dm=None, dmp=None, acc=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["N"], a["d"], a["lam"], a["dtype"], a["m"], a["mp"], a["loss"], a["dm"],
                 a["dmp"], a["acc"], None)

    assert call(N=-1) == INVALID
    assert call(d=12) == INVALID
    assert call(lam=float("nan")) == INVALID
    assert call(dtype=7) == INVALID
    assert call(m=None) == INVALID
    assert call(loss=None) == INVALID
    assert call(mp=FAKE_ODD) == MISALIGNED
    assert call(dm=FAKE_ODD) == MISALIGNED
    assert call(acc=8) == INVALID


def test_debug_mode_switch(L):
    """maglev_debug_enable switches the debug mode without touching a GPU;
    MAGLEV_DEBUG in the environment sets it at load (checked in a child)."""
    import subprocess
    import sys
    before = L.maglev_debug_enabled()
    try:
        assert L.maglev_debug_enable(1) == 0 and L.maglev_debug_enabled() == 1
        assert L.maglev_debug_enable(0) == 0 and L.maglev_debug_enabled() == 0
    finally:
        L.maglev_debug_enable(before)
    code = ("import ctypes, sys; L = ctypes.CDLL(sys.argv[1]); "
            "print(L.maglev_debug_enabled())")
    for env, want in (("1", "1"), ("0", "0"), ("", "0")):
        out = subprocess.run([sys.executable, "-c", code, rms.library_path()],
                             env=dict(os.environ, MAGLEV_DEBUG=env), capture_output=True,
                             text=True, check=True).stdout.strip()
        assert out == want, (env, out)
