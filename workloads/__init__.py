"""Seeded synthetic inputs for the Maglev attention + recurrent K/V injection path.

This module only draws random numbers, rounds them to the storage dtype and
arranges them in the documented layouts. It holds none of the method's
arithmetic (no shift, projection, rotation, mixing, softmax or loss), so both
the CPU oracle and the HIP path can take their inputs from here without
sharing any computation.

Shapes follow the nanochat d20 decoder used by the Maglev experiments
(20 layers, width 1280, 10 heads of 128, context 2048, window 512), as given
in the experiments section of the Maglev summary on paper.rainbus.top
("Maglev：滑动窗口循环记忆", section 实验结果).

Layouts (row-major):
  q, k, v, dO      [B, T, H, Dh]
  m, m_prime       [B, T, d]
  W_Km, W_Vm       [H*Dh, d]
  gate_logit       [H]            (always float32)
  ring caches      [Bs, H, W, Dh]
"""
from __future__ import annotations

import dataclasses
import math

import torch

F32 = "f32"
BF16 = "bf16"

_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Geometry of one decoder-P attention layer."""

    B: int
    T: int
    W: int
    d: int
    H: int
    Dh: int
    dtype: str = BF16
    rope_base: float = 10000.0
    pos0: int = 0
    lam: float = 0.1

    @property
    def N(self) -> int:
        return self.B * self.T


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    """Geometry of the recurrent decode workload (ring cache of W slots)."""

    layers: int
    Bs: int
    W: int
    d: int
    H: int
    Dh: int
    steps: int
    dtype: str = BF16
    rope_base: float = 10000.0
    pool: int = 16


# The five workloads. Names say what they are.
TINY_FP32 = LayerShape(B=1, T=256, W=32, d=64, H=1, Dh=64, dtype=F32, lam=1.0)
D20_LAYER = LayerShape(B=8, T=2048, W=512, d=1280, H=10, Dh=128, dtype=BF16, lam=0.1)
D20_STACK = LayerShape(B=4, T=2048, W=512, d=1280, H=10, Dh=128, dtype=BF16, lam=0.1)
D20_STACK_LAYERS = 20
# LM-head vocabulary: the pages build on the nanochat stack and its tokenizer
# without printing a size; 2^16 entries is that tokenizer's default.
D20_VOCAB = 65536
D20_DECODE = DecodeShape(layers=20, Bs=64, W=512, d=1280, H=10, Dh=128, steps=4096)


def _normal(gen: torch.Generator, shape, std: float = 1.0) -> torch.Tensor:
    x = torch.empty(shape, dtype=torch.float32)
    x.normal_(mean=0.0, std=std, generator=gen)
    return x


def layer_inputs(shape: LayerShape, seed: int, grads: bool = False) -> dict:
    """Draw one layer's inputs on the CPU in the storage dtype.

    q, k, v, m_prime, m, dO ~ N(0, 1); W_Km, W_Vm ~ N(0, 1/d);
    gate logits ~ N(0, 1) in float32. The draw order is fixed so a seed
    always yields the same tensors whatever is requested afterwards.
    """
    g = torch.Generator().manual_seed(int(seed))
    dt = torch_dtype(shape.dtype)
    B, T, H, Dh, d = shape.B, shape.T, shape.H, shape.Dh, shape.d
    out = {}
    out["q"] = _normal(g, (B, T, H, Dh)).to(dt)
    out["k"] = _normal(g, (B, T, H, Dh)).to(dt)
    out["v"] = _normal(g, (B, T, H, Dh)).to(dt)
    out["m_prime"] = _normal(g, (B, T, d)).to(dt)
    std_w = 1.0 / math.sqrt(d)
    out["W_Km"] = _normal(g, (H * Dh, d), std_w).to(dt)
    out["W_Vm"] = _normal(g, (H * Dh, d), std_w).to(dt)
    out["gate_logit"] = _normal(g, (H,))
    out["m"] = _normal(g, (B, T, d)).to(dt)
    if grads:
        out["dO"] = _normal(g, (B, T, H, Dh)).to(dt)
    return out


def stack_inputs(shape: LayerShape, layers: int, seed0: int = 3000, grads: bool = True):
    """Per-layer inputs for the multi-layer lifted pass: layer l uses seed seed0+l."""
    return [layer_inputs(shape, seed0 + l, grads=grads) for l in range(layers)]


def decode_layer_params(shape: DecodeShape, seed: int, layer: int) -> dict:
    """Weights, gate logits, the q/k/v pool and the prefilled ring of one layer.

    The ring holds already-mixed, already-rotated N(0,1) entries for the
    positions 0..W-1 (slot s holds position s), drawn in the storage dtype.
    The pool holds `shape.pool` N(0,1) sets of (q, k, v) per layer; decode
    step t uses entry t mod pool.
    """
    g = torch.Generator().manual_seed(int(seed) * 1000 + int(layer))
    dt = torch_dtype(shape.dtype)
    Bs, H, Dh, W, d = shape.Bs, shape.H, shape.Dh, shape.W, shape.d
    std_w = 1.0 / math.sqrt(d)
    p = {}
    p["W_Km"] = _normal(g, (H * Dh, d), std_w).to(dt)
    p["W_Vm"] = _normal(g, (H * Dh, d), std_w).to(dt)
    p["gate_logit"] = _normal(g, (H,))
    p["q_pool"] = _normal(g, (shape.pool, Bs, H, Dh)).to(dt)
    p["k_pool"] = _normal(g, (shape.pool, Bs, H, Dh)).to(dt)
    p["v_pool"] = _normal(g, (shape.pool, Bs, H, Dh)).to(dt)
    p["kcache"] = _normal(g, (Bs, H, W, Dh)).to(dt)
    p["vcache"] = _normal(g, (Bs, H, W, Dh)).to(dt)
    return p


def decode_initial_memory(shape: DecodeShape, seed: int) -> torch.Tensor:
    """m_{-1} ~ N(0, 1) for every stream, [Bs, d]."""
    g = torch.Generator().manual_seed(int(seed) * 1000 + 999)
    return _normal(g, (shape.Bs, shape.d)).to(torch_dtype(shape.dtype))


def head_inputs(N: int, d: int, V: int, seed: int, dtype: str = BF16) -> dict:
    """Loss-head inputs: the decoder's last hidden state h ~ N(0, 1) [N, d],
    the targets m' ~ N(0, 1) [N, d] (unit RMS, like a final-RMSNorm state),
    the head U ~ N(0, 1/d) [V, d] and next-token targets uniform in [0, V)."""
    g = torch.Generator().manual_seed(int(seed) * 104729 + 5)
    dt = torch_dtype(dtype)
    out = {"h": _normal(g, (N, d)).to(dt), "m_prime": _normal(g, (N, d)).to(dt),
           "U": _normal(g, (V, d), 1.0 / math.sqrt(d)).to(dt)}
    out["targets"] = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    return out


def gate_vectors(H: int, Dh: int, seed: int, std: float = 0.5) -> dict:
    """Four channel-wise gate logit vectors [H*Dh] ~ N(0, std^2) in float32,
    named a_kl, a_kr, a_vl, a_vr (local/recurrent key, local/recurrent value)."""
    g = torch.Generator().manual_seed(int(seed) * 7919 + 17)
    return {n: _normal(g, (H * Dh,), std) for n in ("a_kl", "a_kr", "a_vl", "a_vr")}


def marker_values(rows: torch.Tensor, Dh: int, tag: float = 0.0) -> torch.Tensor:
    """Integer-valued markers [len(rows), Dh], exact in bf16 (every value is
    below 256): row i encodes rows[i] in base 64 (channel 0 = high digit + 1,
    channel 1 = low digit) and carries `tag` in channel 2; zeros elsewhere."""
    r = rows.to(torch.int64)
    x = torch.zeros((r.numel(), Dh), dtype=torch.float32)
    x[:, 0] = (r // 64).to(torch.float32) + 1.0
    x[:, 1] = (r % 64).to(torch.float32)
    if Dh > 2:
        x[:, 2] = float(tag)
    return x
