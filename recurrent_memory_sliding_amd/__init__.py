"""Python binding of libmaglev.so, the MI355X (gfx950) library for the Maglev
decoder-P attention path with recurrent K/V injection.

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks their dtype/shape/contiguity, and calls the C entry
point of the same name on the current torch stream. All arithmetic runs in
the library's HIP kernels; there is no other code path. If the library has
not been built, every call raises MaglevError.

Build:  python -m recurrent_memory_sliding_amd.build
C ABI:  include/maglev.h
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "MaglevError", "MAGLEV_F32", "MAGLEV_BF16", "lib", "library_path",
    "maglev_mem_project", "maglev_swa_inject_fwd", "maglev_swa_inject_bwd",
    "maglev_swa_inject_bwd_workspace", "maglev_consistency_loss",
    "maglev_consistency_loss_noalloc",
    "maglev_consistency_loss_workspace", "maglev_decode_step", "maglev_decode_workspace",
    "maglev_decode_advance", "maglev_prepare", "maglev_abi_version", "maglev_profile_enable",
    "maglev_debug_enable", "maglev_debug_enabled",
    "maglev_profile_read", "maglev_lm_head", "maglev_lm_head_workspace", "LM_CAP",
]

MAGLEV_F32 = 0
MAGLEV_BF16 = 1
_DT = {torch.float32: MAGLEV_F32, torch.bfloat16: MAGLEV_BF16}
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmaglev.so")
_lib = None


class MaglevError(RuntimeError):
    pass


class Geom(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64),
        ("H", ctypes.c_int32), ("Dh", ctypes.c_int32), ("d", ctypes.c_int32), ("W", ctypes.c_int32),
        ("pos0", ctypes.c_int64), ("rope_base", ctypes.c_float), ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded library (raises MaglevError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MaglevError("libmaglev.so is not built; run: python -m recurrent_memory_sliding_amd.build")
        L = ctypes.CDLL(_LIB_PATH)
        vp, sz, i32, i64, f32, u32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                      ctypes.c_int64, ctypes.c_float, ctypes.c_uint)
        G = ctypes.POINTER(Geom)
        sig = {
            "maglev_mem_project": ([G, ctypes.c_int] + [vp] * 10 + [vp], i32),
            "maglev_swa_inject_fwd": ([G, vp, vp, vp, vp, vp, vp], i32),
            "maglev_swa_inject_bwd_workspace": ([G], sz),
            "maglev_swa_inject_bwd": ([G] + [vp] * 19 + [u32, vp, sz, vp], i32),
            "maglev_consistency_loss_workspace": ([i64, i32], sz),
            "maglev_consistency_loss": ([i64, i32, f32, i32, vp, vp, vp, vp, vp, u32, vp, sz, vp], i32),
            "maglev_consistency_loss_noalloc": ([i64, i32, f32, i32, vp, vp, vp, vp, vp, u32, vp],
                                                i32),
            "maglev_decode_workspace": ([i32, i32, i32, i32], sz),
            "maglev_decode_step": ([i32, i32, i32, i32, f32, f32, i32] + [vp] * 5 + [i64]
                                   + [vp] * 5 + [vp, sz, vp], i32),
            "maglev_decode_advance": ([i32, vp, vp], i32),
            "maglev_mem_project_gated": ([G, ctypes.c_int] + [vp] * 6 + [f32] + [vp] * 4 + [vp],
                                         i32),
            "maglev_swa_inject_bwd_gated_workspace": ([G], sz),
            "maglev_swa_inject_bwd_gated": ([G] + [vp] * 8 + [f32] + [vp] * 13 + [u32, vp, sz, vp],
                                            i32),
            "maglev_mix_entries": ([G] + [vp] * 7 + [vp], i32),
            "maglev_swa_inject_bwd_shared_workspace": ([G], sz),
            "maglev_swa_inject_bwd_shared": ([G] + [vp] * 15 + [u32, vp, sz, vp], i32),
            "maglev_mix_entries_gated": ([G] + [vp] * 5 + [f32, vp, vp, vp], i32),
            "maglev_swa_inject_bwd_shared_gated_workspace": ([G], sz),
            "maglev_swa_inject_bwd_shared_gated": ([G] + [vp] * 8 + [f32] + [vp] * 9
                                                   + [u32, vp, sz, vp], i32),
            "maglev_mem_project_bwd_workspace": ([G], sz),
            "maglev_mem_project_bwd": ([G] + [vp] * 8 + [u32, vp, sz, vp], i32),
            "maglev_rope_keys": ([G, vp, vp, vp], i32),
            "maglev_attn_bwd_workspace": ([G], sz),
            "maglev_attn_bwd": ([G] + [vp] * 9 + [vp, sz, vp], i32),
            "maglev_decode_step_gated": ([i32, i32, i32, i32, f32, f32, i32] + [vp] * 5 + [i64]
                                         + [vp, f32] + [vp] * 4 + [vp, sz, vp], i32),
            "maglev_lm_head_workspace": ([i64, i32, i64, i32], sz),
            "maglev_lm_head": ([i64, i32, i64, f32, f32, f32, i32] + [vp] * 8 + [u32, vp, sz, vp],
                               i32),
            "maglev_prepare": ([i32, f32, i64], i32),
            "maglev_status_string": ([i32], ctypes.c_char_p),
            "maglev_last_error": ([], ctypes.c_char_p),
            "maglev_abi_version": ([], ctypes.c_int),
            "maglev_profile_enable": ([ctypes.c_int, ctypes.c_char_p], i32),
            "maglev_debug_enable": ([ctypes.c_int], i32),
            "maglev_debug_enabled": ([], ctypes.c_int),
            "maglev_profile_count": ([], ctypes.c_int),
            "maglev_profile_entry": ([ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                      ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise MaglevError("%s failed: %s (%s)" % (what, L.maglev_status_string(status).decode(),
                                                  L.maglev_last_error().decode()))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise MaglevError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise MaglevError("tensors must be contiguous")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise MaglevError("dtype must be float32 or bfloat16, got %s" % t.dtype)
    return _DT[t.dtype]


def _same(ref: torch.Tensor, *ts):
    for t in ts:
        if t is not None and t.dtype != ref.dtype:
            raise MaglevError("mixed activation dtypes")


def _decode_shapes(kcache, vcache, q, k, v, o, gate, gated):
    """Shapes one decode step's kernel assumes: rings [Bs,H,W,Dh] alike,
    q/k/v/o [Bs,H,Dh], gate logits [H] (sigma form) or [4,H*Dh] (gated)."""
    if kcache.dim() != 4 or tuple(vcache.shape) != tuple(kcache.shape):
        raise MaglevError("kcache and vcache must both be [Bs,H,W,Dh]")
    Bs, H, _, Dh = kcache.shape
    gate_numel = 4 * H * Dh if gated else H
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t is not None and tuple(t.shape) != (Bs, H, Dh):
            raise MaglevError("%s must be [Bs,H,Dh] = %s" % (name, (Bs, H, Dh)))
    if gate.numel() != gate_numel:
        raise MaglevError("gate logits must have %d entries" % gate_numel)


def make_geom(B, T, H, Dh, d, W, pos0=0, rope_base=10000.0, scale=0.0, dtype=MAGLEV_BF16) -> Geom:
    return Geom(B, T, H, Dh, d, W, pos0, rope_base, scale, dtype)


def maglev_abi_version() -> int:
    return lib().maglev_abi_version()


def maglev_debug_enable(on: bool = True) -> None:
    """Debug mode: every launch is followed by a stream synchronisation and an
    error check; a failure is reported by the launching call with the
    kernel's name. Also switched on at load by MAGLEV_DEBUG=1."""
    _check(lib().maglev_debug_enable(1 if on else 0), "maglev_debug_enable")


def maglev_debug_enabled() -> bool:
    return bool(lib().maglev_debug_enabled())


def maglev_profile_enable(on: bool = True, only: Optional[str] = None):
    """Switch per-kernel event timing on (clearing earlier totals; every kernel,
    or only the one named `only`) or off."""
    _check(lib().maglev_profile_enable(1 if on else 0, only.encode() if only else None),
           "maglev_profile_enable")


def maglev_profile_read() -> dict:
    """{kernel name: (launches, total milliseconds)} of the events recorded so far
    (waits for them)."""
    L = lib()
    out = {}
    for i in range(L.maglev_profile_count()):
        name = ctypes.c_char_p()
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(L.maglev_profile_entry(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)),
               "maglev_profile_entry")
        out[name.value.decode()] = (int(n.value), float(ms.value))
    return out


def maglev_prepare(Dh: int, rope_base: float, max_pos: int):
    """Make the RoPE table cover positions [0, max_pos) (call before graph capture)."""
    _check(lib().maglev_prepare(Dh, rope_base, max_pos), "maglev_prepare")


def maglev_mem_project(m, W_Km, W_Vm, H: int, Dh: int, shift: int = 1, kmem=None, vmem=None,
                       k=None, v=None, gate_logit=None, kmix=None, vmix=None, pos0: int = 0,
                       rope_base: float = 10000.0, stream=None):
    """kmem, vmem [B,T,H,Dh] = (m shifted by `shift` rows) projected by W_Km, W_Vm.

    With k, v [B,T,H,Dh] and gate_logit [H] (float32) it also writes the mixed
    entries kmix = R(k + s kmem), vmix = v + s vmem (s = sigmoid(gate_logit),
    R the rotation at position pos0 + t) and returns (kmem, vmem, kmix, vmix).
    """
    mixing = k is not None or v is not None or gate_logit is not None
    if mixing and (k is None or v is None or gate_logit is None):
        raise MaglevError("k, v and gate_logit come together")
    _dev(m, W_Km, W_Vm, kmem, vmem, k, v, gate_logit, kmix, vmix)
    _same(m, W_Km, W_Vm, kmem, vmem, k, v, kmix, vmix)
    B, T, d = m.shape
    if tuple(W_Km.shape) != (H * Dh, d) or tuple(W_Vm.shape) != (H * Dh, d):
        raise MaglevError("W_Km / W_Vm must be [H*Dh, d]")
    shp = (B, T, H, Dh)
    kmem = torch.empty(shp, dtype=m.dtype, device=m.device) if kmem is None else kmem
    vmem = torch.empty(shp, dtype=m.dtype, device=m.device) if vmem is None else vmem
    if mixing:
        if tuple(k.shape) != shp or tuple(v.shape) != shp:
            raise MaglevError("k / v must be [B,T,H,Dh]")
        if gate_logit.dtype != torch.float32 or gate_logit.numel() != H:
            raise MaglevError("gate_logit must be float32 [H]")
        kmix = torch.empty(shp, dtype=m.dtype, device=m.device) if kmix is None else kmix
        vmix = torch.empty(shp, dtype=m.dtype, device=m.device) if vmix is None else vmix
    else:
        kmix = vmix = None
    g = make_geom(B, T, H, Dh, d, 1, pos0, rope_base, 0.0, _dtype_code(m))
    _check(lib().maglev_mem_project(ctypes.byref(g), shift, _ptr(m), _ptr(W_Km), _ptr(W_Vm),
                                    _ptr(k), _ptr(v), _ptr(gate_logit), _ptr(kmem), _ptr(vmem),
                                    _ptr(kmix), _ptr(vmix), _stream(stream)),
           "maglev_mem_project")
    if mixing:
        return kmem, vmem, kmix, vmix
    return kmem, vmem


def maglev_swa_inject_fwd(q, kmix, vmix, W: int, pos0: int = 0, rope_base: float = 10000.0,
                          scale: float = 0.0, d: int = 0, o=None, lse=None,
                          need_lse: bool = True, stream=None):
    """O [B,T,H,Dh] and lse [B,H,T] (float32; None when need_lse is False)."""
    _dev(q, kmix, vmix, o, lse)
    _same(q, kmix, vmix, o)
    B, T, H, Dh = q.shape
    if tuple(kmix.shape) != tuple(q.shape) or tuple(vmix.shape) != tuple(q.shape):
        raise MaglevError("kmix / vmix must match q")
    o = torch.empty_like(q) if o is None else o
    if need_lse and lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    g = make_geom(B, T, H, Dh, d or H * Dh, W, pos0, rope_base, scale, _dtype_code(q))
    _check(lib().maglev_swa_inject_fwd(ctypes.byref(g), _ptr(q), _ptr(kmix), _ptr(vmix), _ptr(o),
                                       _ptr(lse) if need_lse else None, _stream(stream)),
           "maglev_swa_inject_fwd")
    return o, lse


def maglev_swa_inject_bwd_workspace(B, T, H, Dh, d, W, dtype=MAGLEV_BF16) -> int:
    g = make_geom(B, T, H, Dh, d, W, dtype=dtype)
    return int(lib().maglev_swa_inject_bwd_workspace(ctypes.byref(g)))


def maglev_swa_inject_bwd(q, kmix, vmix, kmem, vmem, gate_logit, o, lse, dO, m_prime, W_Km,
                          W_Vm, W: int, pos0: int = 0, rope_base: float = 10000.0,
                          scale: float = 0.0, accumulate: int = 0, out: Optional[dict] = None,
                          workspace=None, stream=None) -> dict:
    """Gradients dq, dk, dv (activation dtype), dm_prime, dW_Km, dW_Vm, dgate (float32).

    dk, dv are the gradients of the token's own k, v (before mixing)."""
    _dev(q, kmix, vmix, kmem, vmem, gate_logit, o, lse, dO, m_prime, W_Km, W_Vm, workspace)
    _same(q, kmix, vmix, kmem, vmem, o, dO, m_prime, W_Km, W_Vm)
    B, T, H, Dh = q.shape
    d = m_prime.shape[-1]
    dev = q.device
    if out is None:
        out = {}
    f32 = torch.float32
    out.setdefault("dq", torch.empty_like(q))
    out.setdefault("dk", torch.empty_like(q))
    out.setdefault("dv", torch.empty_like(q))
    out.setdefault("dm_prime", torch.empty((B, T, d), dtype=f32, device=dev))
    out.setdefault("dW_Km", torch.empty((H * Dh, d), dtype=f32, device=dev))
    out.setdefault("dW_Vm", torch.empty((H * Dh, d), dtype=f32, device=dev))
    out.setdefault("dgate", torch.empty((H,), dtype=f32, device=dev))
    _dev(*out.values())
    g = make_geom(B, T, H, Dh, d, W, pos0, rope_base, scale, _dtype_code(q))
    need = int(lib().maglev_swa_inject_bwd_workspace(ctypes.byref(g)))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(lib().maglev_swa_inject_bwd(
        ctypes.byref(g), _ptr(q), _ptr(kmix), _ptr(vmix), _ptr(kmem), _ptr(vmem), _ptr(gate_logit),
        _ptr(o), _ptr(lse), _ptr(dO), _ptr(m_prime), _ptr(W_Km), _ptr(W_Vm), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dm_prime"]), _ptr(out["dW_Km"]),
        _ptr(out["dW_Vm"]), _ptr(out["dgate"]), accumulate, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "maglev_swa_inject_bwd")
    return out


def maglev_consistency_loss_workspace(N: int, d: int) -> int:
    return int(lib().maglev_consistency_loss_workspace(N, d))


def maglev_consistency_loss(m, m_prime, lam: float, loss=None, dm=None, dm_prime=None,
                            want_grads: bool = True, accumulate: int = 0, workspace=None,
                            stream=None):
    """(loss [1] float32, dm, dm_prime [..., d] float32)."""
    _dev(m, m_prime, loss, dm, dm_prime, workspace)
    _same(m, m_prime)
    d = m.shape[-1]
    N = m.numel() // d
    dev = m.device
    loss = torch.empty((1,), dtype=torch.float32, device=dev) if loss is None else loss
    if want_grads:
        dm = torch.empty(m.shape, dtype=torch.float32, device=dev) if dm is None else dm
        dm_prime = torch.empty(m.shape, dtype=torch.float32, device=dev) if dm_prime is None else dm_prime
    need = int(lib().maglev_consistency_loss_workspace(N, d))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(lib().maglev_consistency_loss(N, d, lam, _dtype_code(m), _ptr(m), _ptr(m_prime),
                                         _ptr(loss), _ptr(dm), _ptr(dm_prime), accumulate,
                                         _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(stream)), "maglev_consistency_loss")
    return loss, dm, dm_prime


def maglev_consistency_loss_noalloc(m, m_prime, lam: float, loss, dm=None, dm_prime=None,
                                    accumulate: int = 0, stream=None):
    """The consistency loss with the library's device scratch instead of a
    workspace: the caller passes every output (loss [1] float32; dm,
    dm_prime [..., d] float32 or None) and nothing is allocated."""
    _dev(m, m_prime, loss, dm, dm_prime)
    _same(m, m_prime)
    d = m.shape[-1]
    N = m.numel() // d
    for t in (dm, dm_prime):
        if t is not None and (t.dtype != torch.float32 or t.shape != m.shape):
            raise MaglevError("dm / dm_prime must be float32 with m's shape")
    if loss.dtype != torch.float32 or loss.numel() < 1:
        raise MaglevError("loss must be a float32 tensor of at least one element")
    _check(lib().maglev_consistency_loss_noalloc(N, d, lam, _dtype_code(m), _ptr(m),
                                                 _ptr(m_prime), _ptr(loss), _ptr(dm),
                                                 _ptr(dm_prime), accumulate, _stream(stream)),
           "maglev_consistency_loss_noalloc")
    return loss, dm, dm_prime


LM_CAP = 15.0   # soft cap of the LM head's logits


def maglev_lm_head_workspace(N: int, d: int, V: int, dtype=torch.bfloat16) -> int:
    return int(lib().maglev_lm_head_workspace(N, d, V, _DT[dtype]))


def maglev_lm_head(h, U, targets, m_prime=None, lam: float = 0.0, cap: float = LM_CAP,
                   eps: float = 1e-6, want_grads: bool = True, m=None, loss=None, dh=None,
                   dU=None, accumulate: int = 0, workspace=None, stream=None):
    """Loss head: (loss [1] float32, m = RMSNorm(h) [..., d] dtype, dh [..., d]
    float32 or None, dU [V, d] float32 or None). targets: int64, h's leading
    shape; entries outside [0, V) are ignored."""
    _dev(h, U, targets, m_prime, m, loss, dh, dU, workspace)
    _same(h, U, m_prime, m)
    d = h.shape[-1]
    N = h.numel() // d
    V = U.shape[0]
    if U.dim() != 2 or U.shape[1] != d:
        raise MaglevError("U must be [V, d]")
    if targets.dtype != torch.int64 or targets.numel() != N or not targets.is_contiguous():
        raise MaglevError("targets must be contiguous int64 with one entry per row of h")
    if m_prime is not None and m_prime.shape != h.shape:
        raise MaglevError("m_prime must have h's shape")
    dev = h.device
    m = torch.empty_like(h) if m is None else m
    loss = torch.empty((1,), dtype=torch.float32, device=dev) if loss is None else loss
    if want_grads:
        dh = torch.empty(h.shape, dtype=torch.float32, device=dev) if dh is None else dh
        dU = torch.empty(U.shape, dtype=torch.float32, device=dev) if dU is None else dU
    need = int(lib().maglev_lm_head_workspace(N, d, V, _dtype_code(h)))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(lib().maglev_lm_head(N, d, V, cap, eps, lam, _dtype_code(h), _ptr(h), _ptr(U),
                                _ptr(targets), _ptr(m_prime), _ptr(m), _ptr(loss), _ptr(dh),
                                _ptr(dU), accumulate, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
           "maglev_lm_head")
    return loss, m, dh, dU


def maglev_decode_workspace(Bs: int, H: int, Dh: int, W: int) -> int:
    return int(lib().maglev_decode_workspace(Bs, H, Dh, W))


def maglev_decode_step(q, k, v, kmem, vmem, gate_logit, kcache, vcache, pos, o=None,
                       rope_base: float = 10000.0, scale: float = 0.0, workspace=None,
                       mem_stride: int = 0, stream=None):
    """One decode step; kcache/vcache [Bs,H,W,Dh] are updated in place. Returns o [Bs,H,Dh].

    kmem/vmem hold stream b's [H,Dh] block at element b*mem_stride (0: packed
    [Bs,H,Dh]; a larger stride reads one layer's slice of a stacked projection).
    A workspace passed in must be zero-filled before its first use (calls
    leave it so)."""
    _dev(q, k, v, gate_logit, kcache, vcache, pos, o, workspace)
    _same(q, k, v, kmem, vmem, kcache, vcache, o)
    _decode_shapes(kcache, vcache, q, k, v, o, gate_logit, False)
    if gate_logit.dtype != torch.float32:
        raise MaglevError("gate_logit must be float32")
    Bs, H, W, Dh = kcache.shape
    if pos.dtype != torch.int64 or pos.numel() != Bs:
        raise MaglevError("pos must be int64 [Bs]")
    stride = mem_stride or H * Dh
    for t in (kmem, vmem):   # may be strided views into a stacked projection
        if not t.is_cuda:
            raise MaglevError("tensors must be on the GPU")
        span = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
        if Bs > 0 and span < (Bs - 1) * stride + H * Dh:
            raise MaglevError("kmem/vmem too small for Bs x mem_stride")
    o = torch.empty_like(q) if o is None else o
    if workspace is None:
        need = int(lib().maglev_decode_workspace(Bs, H, Dh, W))
        workspace = torch.zeros((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().maglev_decode_step(Bs, H, Dh, W, rope_base, scale, _dtype_code(q), _ptr(q),
                                    _ptr(k), _ptr(v), _ptr(kmem), _ptr(vmem), int(mem_stride),
                                    _ptr(gate_logit), _ptr(kcache), _ptr(vcache), _ptr(pos),
                                    _ptr(o), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "maglev_decode_step")
    return o


# ----------------------------------------------------------------------------
# Gated form: k~ = g_kl R k + g_kr R RMSNorm(W_Km m'), v~ = g_vl v + g_vr W_Vm m',
# g = 2 sigmoid(a); gates are float32 [4, H*Dh] logits (a_kl, a_kr, a_vl, a_vr).
# ----------------------------------------------------------------------------
GATE_NAMES = ("a_kl", "a_kr", "a_vl", "a_vr")
RMS_EPS = 1e-6


def gate_tensor(gates, HD: int, device) -> torch.Tensor:
    """The [4, HD] float32 logit tensor the gated calls take, from a tensor or
    a mapping of the four names."""
    if not isinstance(gates, torch.Tensor):
        gates = torch.stack([torch.as_tensor(gates[n], dtype=torch.float32).reshape(-1)
                             for n in GATE_NAMES])
    gates = gates.to(device=device, dtype=torch.float32).reshape(4, HD).contiguous()
    return gates


def maglev_mem_project_gated(m, W_Km, W_Vm, H: int, Dh: int, k, v, gates, eps: float = RMS_EPS,
                             shift: int = 1, pos0: int = 0, rope_base: float = 10000.0,
                             kproj=None, vmem=None, kmix=None, vmix=None, stream=None):
    """(kproj, vmem, kmix, vmix): the projections of the shifted memory before
    the norm, and the gated mixed entries, all [B,T,H,Dh]."""
    B, T, d = m.shape
    gates = gate_tensor(gates, H * Dh, m.device)
    _dev(m, W_Km, W_Vm, k, v, gates, kproj, vmem, kmix, vmix)
    _same(m, W_Km, W_Vm, k, v, kproj, vmem, kmix, vmix)
    if tuple(W_Km.shape) != (H * Dh, d) or tuple(W_Vm.shape) != (H * Dh, d):
        raise MaglevError("W_Km / W_Vm must be [H*Dh, d]")
    shp = (B, T, H, Dh)
    if tuple(k.shape) != shp or tuple(v.shape) != shp:
        raise MaglevError("k / v must be [B,T,H,Dh]")
    new = lambda t: torch.empty(shp, dtype=m.dtype, device=m.device) if t is None else t
    kproj, vmem, kmix, vmix = new(kproj), new(vmem), new(kmix), new(vmix)
    g = make_geom(B, T, H, Dh, d, 1, pos0, rope_base, 0.0, _dtype_code(m))
    _check(lib().maglev_mem_project_gated(ctypes.byref(g), shift, _ptr(m), _ptr(W_Km), _ptr(W_Vm),
                                          _ptr(k), _ptr(v), _ptr(gates), float(eps), _ptr(kproj),
                                          _ptr(vmem), _ptr(kmix), _ptr(vmix), _stream(stream)),
           "maglev_mem_project_gated")
    return kproj, vmem, kmix, vmix


def maglev_swa_inject_bwd_gated_workspace(B, T, H, Dh, d, W, dtype=MAGLEV_BF16) -> int:
    g = make_geom(B, T, H, Dh, d, W, dtype=dtype)
    return int(lib().maglev_swa_inject_bwd_gated_workspace(ctypes.byref(g)))


def maglev_swa_inject_bwd_gated(q, kmix, vmix, k, v, kproj, vmem, gates, o, lse, dO, m_prime,
                                W_Km, W_Vm, W: int, eps: float = RMS_EPS, pos0: int = 0,
                                rope_base: float = 10000.0, scale: float = 0.0,
                                accumulate: int = 0, out: Optional[dict] = None, workspace=None,
                                stream=None) -> dict:
    """Gradients dq, dk, dv (activation dtype), dm_prime, dW_Km, dW_Vm and
    dgates [4, H*Dh] (float32) of the gated layer path."""
    B, T, H, Dh = q.shape
    d = m_prime.shape[-1]
    dev = q.device
    gates = gate_tensor(gates, H * Dh, dev)
    _dev(q, kmix, vmix, k, v, kproj, vmem, gates, o, lse, dO, m_prime, W_Km, W_Vm, workspace)
    _same(q, kmix, vmix, k, v, kproj, vmem, o, dO, m_prime, W_Km, W_Vm)
    if out is None:
        out = {}
    f32 = torch.float32
    out.setdefault("dq", torch.empty_like(q))
    out.setdefault("dk", torch.empty_like(q))
    out.setdefault("dv", torch.empty_like(q))
    out.setdefault("dm_prime", torch.empty((B, T, d), dtype=f32, device=dev))
    out.setdefault("dW_Km", torch.empty((H * Dh, d), dtype=f32, device=dev))
    out.setdefault("dW_Vm", torch.empty((H * Dh, d), dtype=f32, device=dev))
    out.setdefault("dgates", torch.empty((4, H * Dh), dtype=f32, device=dev))
    _dev(*out.values())
    g = make_geom(B, T, H, Dh, d, W, pos0, rope_base, scale, _dtype_code(q))
    need = int(lib().maglev_swa_inject_bwd_gated_workspace(ctypes.byref(g)))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(lib().maglev_swa_inject_bwd_gated(
        ctypes.byref(g), _ptr(q), _ptr(kmix), _ptr(vmix), _ptr(k), _ptr(v), _ptr(kproj),
        _ptr(vmem), _ptr(gates), float(eps), _ptr(o), _ptr(lse), _ptr(dO), _ptr(m_prime),
        _ptr(W_Km), _ptr(W_Vm), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
        _ptr(out["dm_prime"]), _ptr(out["dW_Km"]), _ptr(out["dW_Vm"]), _ptr(out["dgates"]),
        accumulate, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)), "maglev_swa_inject_bwd_gated")
    return out


def maglev_decode_step_gated(q, k, v, kproj, vmem, gates, kcache, vcache, pos, o=None,
                             eps: float = RMS_EPS, rope_base: float = 10000.0, scale: float = 0.0,
                             workspace=None, mem_stride: int = 0, stream=None):
    """One decode step of the gated form (kproj = W_Km m_{t-1} before the norm);
    kcache/vcache are updated in place. Returns o [Bs,H,Dh]."""
    if kcache.dim() != 4:
        raise MaglevError("kcache must be [Bs,H,W,Dh]")
    Bs, H, W, Dh = kcache.shape
    gates = gate_tensor(gates, H * Dh, q.device)
    _dev(q, k, v, gates, kcache, vcache, pos, o, workspace)
    _same(q, k, v, kproj, vmem, kcache, vcache, o)
    _decode_shapes(kcache, vcache, q, k, v, o, gates, True)
    if pos.dtype != torch.int64 or pos.numel() != Bs:
        raise MaglevError("pos must be int64 [Bs]")
    stride = mem_stride or H * Dh
    for t in (kproj, vmem):
        if not t.is_cuda:
            raise MaglevError("tensors must be on the GPU")
        span = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
        if Bs > 0 and span < (Bs - 1) * stride + H * Dh:
            raise MaglevError("kproj/vmem too small for Bs x mem_stride")
    o = torch.empty_like(q) if o is None else o
    if workspace is None:
        need = int(lib().maglev_decode_workspace(Bs, H, Dh, W))
        workspace = torch.zeros((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().maglev_decode_step_gated(Bs, H, Dh, W, rope_base, scale, _dtype_code(q), _ptr(q),
                                          _ptr(k), _ptr(v), _ptr(kproj), _ptr(vmem),
                                          int(mem_stride), _ptr(gates), float(eps), _ptr(kcache),
                                          _ptr(vcache), _ptr(pos), _ptr(o), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream)), "maglev_decode_step_gated")
    return o


# ----------------------------------------------------------------------------
# Layers sharing one memory projection: mem_project once per pass, then per
# layer mix_entries / swa_inject_fwd / swa_inject_bwd_shared (summing the
# memory gradients), then mem_project_bwd once.
# ----------------------------------------------------------------------------
def maglev_mix_entries(k, v, kmem, vmem, gate_logit, pos0: int = 0, rope_base: float = 10000.0,
                       kmix=None, vmix=None, stream=None):
    """(kmix, vmix) of one layer from the given (shared) memory terms."""
    _dev(k, v, kmem, vmem, gate_logit, kmix, vmix)
    _same(k, v, kmem, vmem, kmix, vmix)
    B, T, H, Dh = k.shape
    for t in (v, kmem, vmem):
        if tuple(t.shape) != tuple(k.shape):
            raise MaglevError("k, v, kmem, vmem must all be [B,T,H,Dh]")
    if gate_logit.dtype != torch.float32 or gate_logit.numel() != H:
        raise MaglevError("gate_logit must be float32 [H]")
    kmix = torch.empty_like(k) if kmix is None else kmix
    vmix = torch.empty_like(k) if vmix is None else vmix
    g = make_geom(B, T, H, Dh, H * Dh, 1, pos0, rope_base, 0.0, _dtype_code(k))
    _check(lib().maglev_mix_entries(ctypes.byref(g), _ptr(k), _ptr(v), _ptr(kmem), _ptr(vmem),
                                    _ptr(gate_logit), _ptr(kmix), _ptr(vmix), _stream(stream)),
           "maglev_mix_entries")
    return kmix, vmix


def maglev_swa_inject_bwd_shared_workspace(B, T, H, Dh, W, dtype=MAGLEV_BF16) -> int:
    g = make_geom(B, T, H, Dh, H * Dh, W, dtype=dtype)
    return int(lib().maglev_swa_inject_bwd_shared_workspace(ctypes.byref(g)))


def maglev_swa_inject_bwd_shared(q, kmix, vmix, kmem, vmem, gate_logit, o, lse, dO, dkmem, dvmem,
                                 W: int, pos0: int = 0, rope_base: float = 10000.0,
                                 scale: float = 0.0, accumulate: int = 0, dq=None, dk=None,
                                 dv=None, dgate=None, workspace=None, stream=None):
    """One layer's backward with shared memory terms: returns (dq, dk, dv, dgate);
    dkmem/dvmem (float32 [B,T,H,Dh]) receive s dk, s dv (added with bit 0)."""
    _dev(q, kmix, vmix, kmem, vmem, gate_logit, o, lse, dO, dkmem, dvmem, dq, dk, dv, dgate,
         workspace)
    _same(q, kmix, vmix, kmem, vmem, o, dO, dq, dk, dv)
    B, T, H, Dh = q.shape
    for t in (dkmem, dvmem):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(q.shape):
            raise MaglevError("dkmem / dvmem must be float32 [B,T,H,Dh]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    dgate = torch.empty((H,), dtype=torch.float32, device=q.device) if dgate is None else dgate
    g = make_geom(B, T, H, Dh, H * Dh, W, pos0, rope_base, scale, _dtype_code(q))
    if workspace is None:
        need = int(lib().maglev_swa_inject_bwd_shared_workspace(ctypes.byref(g)))
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().maglev_swa_inject_bwd_shared(
        ctypes.byref(g), _ptr(q), _ptr(kmix), _ptr(vmix), _ptr(kmem), _ptr(vmem), _ptr(gate_logit),
        _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkmem), _ptr(dvmem),
        _ptr(dgate), accumulate, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)), "maglev_swa_inject_bwd_shared")
    return dq, dk, dv, dgate


# Gated form over one shared projection: mem_project (no mixing arguments)
# once per pass gives the pre-norm kproj and vmem; per layer
# mix_entries_gated / swa_inject_fwd / swa_inject_bwd_shared_gated (summing
# the projections' gradients in float32); then mem_project_bwd once.
def maglev_mix_entries_gated(k, v, kproj, vmem, gates, eps: float = RMS_EPS, pos0: int = 0,
                             rope_base: float = 10000.0, kmix=None, vmix=None, stream=None):
    """(kmix, vmix) of one gated layer from the shared pre-norm projections."""
    B, T, H, Dh = k.shape
    gates = gate_tensor(gates, H * Dh, k.device)
    _dev(k, v, kproj, vmem, gates, kmix, vmix)
    _same(k, v, kproj, vmem, kmix, vmix)
    for t in (v, kproj, vmem):
        if tuple(t.shape) != tuple(k.shape):
            raise MaglevError("k, v, kproj, vmem must all be [B,T,H,Dh]")
    kmix = torch.empty_like(k) if kmix is None else kmix
    vmix = torch.empty_like(k) if vmix is None else vmix
    g = make_geom(B, T, H, Dh, H * Dh, 1, pos0, rope_base, 0.0, _dtype_code(k))
    _check(lib().maglev_mix_entries_gated(ctypes.byref(g), _ptr(k), _ptr(v), _ptr(kproj),
                                          _ptr(vmem), _ptr(gates), float(eps), _ptr(kmix),
                                          _ptr(vmix), _stream(stream)), "maglev_mix_entries_gated")
    return kmix, vmix


def maglev_swa_inject_bwd_shared_gated_workspace(B, T, H, Dh, W, dtype=MAGLEV_BF16) -> int:
    g = make_geom(B, T, H, Dh, H * Dh, W, dtype=dtype)
    return int(lib().maglev_swa_inject_bwd_shared_gated_workspace(ctypes.byref(g)))


def maglev_swa_inject_bwd_shared_gated(q, kmix, vmix, k, v, kproj, vmem, gates, o, lse, dO,
                                       dkproj, dvmem, W: int, eps: float = RMS_EPS, pos0: int = 0,
                                       rope_base: float = 10000.0, scale: float = 0.0,
                                       accumulate: int = 0, dq=None, dk=None, dv=None,
                                       dgates=None, workspace=None, stream=None):
    """One gated layer's backward over shared projections: returns
    (dq, dk, dv, dgates [4, H*Dh] float32); dkproj/dvmem (float32 [B,T,H,Dh])
    receive the layer's share of the projections' gradients (added with bit 0)."""
    B, T, H, Dh = q.shape
    gates = gate_tensor(gates, H * Dh, q.device)
    _dev(q, kmix, vmix, k, v, kproj, vmem, gates, o, lse, dO, dkproj, dvmem, dq, dk, dv, dgates,
         workspace)
    _same(q, kmix, vmix, k, v, kproj, vmem, o, dO, dq, dk, dv)
    for t in (dkproj, dvmem):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(q.shape):
            raise MaglevError("dkproj / dvmem must be float32 [B,T,H,Dh]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    if dgates is None:
        dgates = torch.empty((4, H * Dh), dtype=torch.float32, device=q.device)
    g = make_geom(B, T, H, Dh, H * Dh, W, pos0, rope_base, scale, _dtype_code(q))
    if workspace is None:
        need = int(lib().maglev_swa_inject_bwd_shared_gated_workspace(ctypes.byref(g)))
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().maglev_swa_inject_bwd_shared_gated(
        ctypes.byref(g), _ptr(q), _ptr(kmix), _ptr(vmix), _ptr(k), _ptr(v), _ptr(kproj),
        _ptr(vmem), _ptr(gates), float(eps), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dkproj), _ptr(dvmem), _ptr(dgates), accumulate, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)),
        "maglev_swa_inject_bwd_shared_gated")
    return dq, dk, dv, dgates


def maglev_mem_project_bwd_workspace(B, T, H, Dh, d, dtype=MAGLEV_BF16) -> int:
    g = make_geom(B, T, H, Dh, d, 1, dtype=dtype)
    return int(lib().maglev_mem_project_bwd_workspace(ctypes.byref(g)))


def maglev_mem_project_bwd(dkmem, dvmem, m_prime, W_Km, W_Vm, accumulate: int = 0, dm_prime=None,
                           dW_Km=None, dW_Vm=None, workspace=None, stream=None):
    """(dm_prime, dW_Km, dW_Vm), all float32, from float32 dkmem, dvmem [B,T,H,Dh]."""
    _dev(dkmem, dvmem, m_prime, W_Km, W_Vm, dm_prime, dW_Km, dW_Vm, workspace)
    _same(m_prime, W_Km, W_Vm)
    B, T, H, Dh = dkmem.shape
    d = m_prime.shape[-1]
    dev = m_prime.device
    f32 = torch.float32
    dm_prime = torch.empty((B, T, d), dtype=f32, device=dev) if dm_prime is None else dm_prime
    dW_Km = torch.empty((H * Dh, d), dtype=f32, device=dev) if dW_Km is None else dW_Km
    dW_Vm = torch.empty((H * Dh, d), dtype=f32, device=dev) if dW_Vm is None else dW_Vm
    g = make_geom(B, T, H, Dh, d, 1, 0, 0.0, 0.0, _dtype_code(m_prime))
    if workspace is None:
        need = int(lib().maglev_mem_project_bwd_workspace(ctypes.byref(g)))
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(lib().maglev_mem_project_bwd(
        ctypes.byref(g), _ptr(dkmem), _ptr(dvmem), _ptr(m_prime), _ptr(W_Km), _ptr(W_Vm),
        _ptr(dm_prime), _ptr(dW_Km), _ptr(dW_Vm), accumulate, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "maglev_mem_project_bwd")
    return dm_prime, dW_Km, dW_Vm


# ----------------------------------------------------------------------------
# Attention without injection (the prefiller's sliding-window and full layers)
# ----------------------------------------------------------------------------
def maglev_rope_keys(k, pos0: int = 0, rope_base: float = 10000.0, krot=None, stream=None):
    """krot = R_{pos0+t} k for k [B,T,H,Dh]."""
    _dev(k, krot)
    _same(k, krot)
    B, T, H, Dh = k.shape
    krot = torch.empty_like(k) if krot is None else krot
    g = make_geom(B, T, H, Dh, H * Dh, 1, pos0, rope_base, 0.0, _dtype_code(k))
    _check(lib().maglev_rope_keys(ctypes.byref(g), _ptr(k), _ptr(krot), _stream(stream)),
           "maglev_rope_keys")
    return krot


def maglev_attn_fwd(q, k, v, W: int, pos0: int = 0, rope_base: float = 10000.0,
                    scale: float = 0.0, krot=None, o=None, lse=None, stream=None):
    """Causal attention of window W without injection (W >= T: full causal).
    Returns (o, lse, krot); krot is what the backward takes."""
    krot = maglev_rope_keys(k, pos0, rope_base, krot=krot, stream=stream)
    o, lse = maglev_swa_inject_fwd(q, krot, v, W, pos0=pos0, rope_base=rope_base, scale=scale,
                                   o=o, lse=lse, stream=stream)
    return o, lse, krot


def maglev_attn_bwd_workspace(B, T, H, Dh, W, dtype=MAGLEV_BF16) -> int:
    g = make_geom(B, T, H, Dh, H * Dh, W, dtype=dtype)
    return int(lib().maglev_attn_bwd_workspace(ctypes.byref(g)))


def maglev_attn_bwd(q, krot, v, o, lse, dO, W: int, pos0: int = 0, rope_base: float = 10000.0,
                    scale: float = 0.0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """(dq, dk, dv) of attention without injection; dk is w.r.t. the unrotated k."""
    _dev(q, krot, v, o, lse, dO, dq, dk, dv, workspace)
    _same(q, krot, v, o, dO, dq, dk, dv)
    B, T, H, Dh = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    g = make_geom(B, T, H, Dh, H * Dh, W, pos0, rope_base, scale, _dtype_code(q))
    if workspace is None:
        need = int(lib().maglev_attn_bwd_workspace(ctypes.byref(g)))
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().maglev_attn_bwd(ctypes.byref(g), _ptr(q), _ptr(krot), _ptr(v), _ptr(o), _ptr(lse),
                                 _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "maglev_attn_bwd")
    return dq, dk, dv


def maglev_decode_advance(pos, stream=None):
    _dev(pos)
    _check(lib().maglev_decode_advance(pos.numel(), _ptr(pos), _stream(stream)), "maglev_decode_advance")


def default_scale(Dh: int) -> float:
    return 1.0 / math.sqrt(Dh)
