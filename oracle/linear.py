"""fp64 token-batch linear layer (oracle; test infrastructure only).

"Sarathi-Serve：以 chunked-prefills 与 stall-free batching 驯服 LLM 推理的吞吐—延迟权衡",
section 端到端文字序列 step ④: every layer of the forward pass runs the
hybrid batch through linear-layer GEMMs and the attention kernel; section
两阶段天然不对称: those linear layers take most of the time of both phases;
section 3 · token 预算的三个约束: GPU matrices are computed in tiles, so the
token count of a batch (the GEMM's row count) meets tile quantisation.

What is computed is the plain definition of a linear layer over a batch of
token rows: y[t, n] = sum_k x[t, k] * w[n, k] (the weight stored one output
feature per row, as in the usual linear-layer layout), no bias.  Inputs are
bf16 bit patterns widened exactly; the sum is an fp64 matrix product.
"""
from __future__ import annotations

import numpy as np


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x: [M, K] token rows, w: [N, K] weight rows -> y = x w^T as [M, N] float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("shape mismatch: x [M, K], w [N, K]")
    return x @ w.T
