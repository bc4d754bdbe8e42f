"""Recurrent decode of a stack of injected sliding-window attention layers.

The state of every stream is exactly what the method keeps at inference
(Maglev summary on paper.rainbus.top, "Maglev：滑动窗口循环记忆", section
方法步骤详情; gist.science summary, section Inferentiemechanisme): one W-slot
K/V ring per layer holding mixed entries, the stream's absolute position, and
the previous step's memory m_{t-1}. Every layer of a step injects the same
m_{t-1}, so one step runs a single memory projection of m_{t-1} by all layers'
stacked weights (shift 0), then the decode step on each layer's ring, which
reads its layer's slice of that projection; the memory of the next step is
then taken from the last layer's output (the attention path stands in for the
rest of the decoder block, which is outside this library). All work is issued
through the C ABI on one stream, and a step can be captured once as a HIP
graph and replayed.
"""
from __future__ import annotations

from typing import List

import torch

from . import (RMS_EPS, maglev_decode_advance, maglev_decode_step, maglev_decode_step_gated,
               maglev_decode_workspace, maglev_mem_project, maglev_prepare)


class DecodeStack:
    """Ring caches, positions and memory of `Bs` streams through `layers` layers.

    weights: per layer dict with W_Km, W_Vm [H*Dh, d] and either gate_logit [H]
      (sigma-gated form) or gates [4, H*Dh] float32 (the gated form with the
      normalised memory key, maglev_decode_step_gated);
    kcache/vcache: per layer [Bs, H, W, Dh] tensors (updated in place);
    pos: int64 [Bs]; m: [Bs, d] memory of the previous step.
    """

    def __init__(self, weights: List[dict], kcache: List[torch.Tensor], vcache: List[torch.Tensor],
                 pos: torch.Tensor, m: torch.Tensor, rope_base: float = 10000.0):
        self.weights = weights
        self.kcache = kcache
        self.vcache = vcache
        self.pos = pos
        self.L = len(weights)
        Bs, H, W, Dh = kcache[0].shape
        self.Bs, self.H, self.W, self.Dh = Bs, H, W, Dh
        self.d = m.shape[-1]
        if self.d != H * Dh:
            raise ValueError("the stand-in memory is the last layer's output: d must equal H*Dh")
        dev, dt = m.device, m.dtype
        self.m = m.reshape(Bs, 1, self.d).clone()
        self.rope_base = rope_base
        # all layers' projection weights stacked along the output rows: one GEMM per step
        self.Wk_all = torch.cat([w["W_Km"] for w in weights], dim=0).contiguous()
        self.Wv_all = torch.cat([w["W_Vm"] for w in weights], dim=0).contiguous()
        self.HD = H * Dh
        self.kmem_all = torch.empty((Bs, 1, self.L * H, Dh), dtype=dt, device=dev)
        self.vmem_all = torch.empty((Bs, 1, self.L * H, Dh), dtype=dt, device=dev)
        flat_k = self.kmem_all.view(Bs, self.L * self.HD)
        flat_v = self.vmem_all.view(Bs, self.L * self.HD)
        self.kmem = [flat_k[:, l * self.HD:(l + 1) * self.HD] for l in range(self.L)]
        self.vmem = [flat_v[:, l * self.HD:(l + 1) * self.HD] for l in range(self.L)]
        # The last layer writes its output straight into the memory buffer: the
        # step's projection has read m before that write is issued.
        self.out = [torch.empty((Bs, H, Dh), dtype=dt, device=dev) for _ in range(self.L - 1)]
        self.out.append(self.m.view(Bs, H, Dh))
        need = maglev_decode_workspace(Bs, H, Dh, W)
        self.ws = torch.zeros((max(need, 1),), dtype=torch.uint8, device=dev)
        self.graphs = {}

    def _issue(self, q: List[torch.Tensor], k: List[torch.Tensor], v: List[torch.Tensor]):
        """Enqueue one step; q/k/v are per-layer [Bs, H, Dh] tensors."""
        maglev_mem_project(self.m, self.Wk_all, self.Wv_all, self.L * self.H, self.Dh, shift=0,
                           kmem=self.kmem_all, vmem=self.vmem_all)
        stride = self.L * self.HD
        for l in range(self.L):
            w = self.weights[l]
            if "gates" in w:
                maglev_decode_step_gated(q[l], k[l], v[l], self.kmem[l], self.vmem[l], w["gates"],
                                         self.kcache[l], self.vcache[l], self.pos, o=self.out[l],
                                         eps=w.get("eps", RMS_EPS), rope_base=self.rope_base,
                                         workspace=self.ws, mem_stride=stride)
            else:
                maglev_decode_step(q[l], k[l], v[l], self.kmem[l], self.vmem[l], w["gate_logit"],
                                   self.kcache[l], self.vcache[l], self.pos, o=self.out[l],
                                   rope_base=self.rope_base, workspace=self.ws,
                                   mem_stride=stride)
        maglev_decode_advance(self.pos)

    def step(self, q, k, v):
        """Run one step eagerly. Returns the per-layer outputs (views, overwritten next step)."""
        self._issue(q, k, v)
        return self.out

    def capture(self, key, q, k, v):
        """Capture one step reading these q/k/v buffers as a HIP graph under `key`."""
        maglev_prepare(self.Dh, self.rope_base, 1)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self._issue(q, k, v)
        torch.cuda.current_stream().wait_stream(s)
        self.graphs[key] = g

    def replay(self, key):
        self.graphs[key].replay()
        return self.out
