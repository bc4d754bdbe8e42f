"""Writes tests/golden/tiny_fp32_seed0.json from the CPU oracle alone.

Workload: the tiny fp32 forward (B=1, T=256, W=32, d=64, one head of 64,
RoPE base 10000, lambda=1, seed 0). Stored: every lse value, four full output
rows (t = 0, 31, 32, 255) and the consistency loss. The file anchors the
oracle's arithmetic: a later change to it must regenerate this file and say,
in its commit message, which passage of the pages justifies the change.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402

ROWS = [0, 31, 32, 255]


def compute():
    sh = wl.TINY_FP32
    inp = wl.layer_inputs(sh, seed=0)
    kmem, vmem = oracle.mem_project(inp["m_prime"], inp["W_Km"], inp["W_Vm"], sh.H, sh.Dh, shift=1)
    o, lse = oracle.swa_inject_fwd(inp["q"], inp["k"], inp["v"], kmem, vmem, inp["gate_logit"],
                                   sh.W, rope_base=sh.rope_base)
    loss, _, _ = oracle.consistency_loss(inp["m"], inp["m_prime"], sh.lam)
    return {
        "workload": "tiny fp32 forward: B=1 T=256 W=32 d=64 H=1 Dh=64 base=1e4 lambda=1 seed=0",
        "lse": lse[0, 0].tolist(),
        "o_rows": {str(t): o[0, t, 0].tolist() for t in ROWS},
        "loss": loss,
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_seed0.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", out)
