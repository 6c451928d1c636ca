"""fp64 softmax attention for the rows of a hybrid batch (oracle).

What is computed (and why it is the plain definition):
  * "Sarathi-Serve：以 chunked-prefills 与 stall-free batching 驯服 LLM 推理的吞吐—延迟权衡",
    section GPU / 系统数据路径, step ⑤: a prefill chunk appends its new K/V and
    attends to the earlier chunks of its own prompt; a decode reads all of its
    history.
  * "Sarathi-Serve: Chunked Prefills for Stall-Free LLM Inference", sections
    intro and "What to notice when reading": chunking is a scheduling change,
    not a change of model math -- every prompt token is still paid for.  So
    a chunk row at absolute position p is ordinary causal attention over keys
    0..p of its request, and a decode row is the same with p = its position.
  * "In-flight Batching", section 技术原理: decode reads the whole KV cache.

Readings where the pages are silent: keys 0..p inclusive (the row's own key
included); softmax scale passed explicitly (1/sqrt(d) by default); grouped-query
heads map q head h to kv head h // (Hq / Hkv); no positional encoding here.

Sliding-window attention ("Sarathi-Serve: Chunked Prefills for Stall-Free LLM
Inference", Results and evidence: the evaluated models include sliding-window
variants; the pages give no window rule).  Reading taken: with a window of w
keys, the row at position p sees keys max(0, p - w + 1) .. p -- its own key
and the w - 1 before it; w = 0 means no window.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def causal_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, ctx: int, scale: float,
                window: int = 0) -> np.ndarray:
    """Attention of ``n`` consecutive query rows of one request.

    q: [n, Hq, d] rows at absolute positions ctx .. ctx+n-1.
    k, v: [ctx+n, Hkv, d] -- the request's whole contiguous K/V (history first,
    then this step's rows).  Row at position p sees keys 0..p, or with a
    window w > 0 only keys p-w+1 .. p.
    Returns [n, Hq, d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, Hq, d = q.shape
    total, Hkv, dk = k.shape
    if total != ctx + n or dk != d or v.shape != k.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    if window < 0:
        raise ValueError("window must be >= 0")
    group = Hq // Hkv
    pos = ctx + np.arange(n)
    keys = np.arange(total)[None, :]
    visible = keys <= pos[:, None]                                # [n, total]
    if window:
        visible &= keys > pos[:, None] - window
    out = np.empty((n, Hq, d), dtype=np.float64)
    for h in range(Hq):
        kh = h // group
        s = scale * (q[:, h, :] @ k[:, kh, :].T)                   # [n, total]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[:, h, :] = (w @ v[:, kh, :]) / w.sum(axis=1, keepdims=True)
    return out


def attend(seqs, q: np.ndarray, kv, scale: float, window: int = 0) -> np.ndarray:
    """All rows of a hybrid batch.

    seqs: list of (context_len, q_len) in batch order (decodes have q_len 1).
    q: [T, Hq, d] packed rows, sequence s occupying rows
       sum(q_len[:s]) .. +q_len[s].
    kv: per sequence, (k_s, v_s) each [context_len + q_len, Hkv, d].
    window: sliding window in keys (0: none), the same for every sequence.
    Returns [T, Hq, d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    out = np.empty(q.shape, dtype=np.float64)
    row = 0
    for (ctx, n), (k_s, v_s) in zip(seqs, kv):
        out[row:row + n] = causal_rows(q[row:row + n], k_s, v_s, ctx, scale, window)
        row += n
    if row != q.shape[0]:
        raise ValueError("q rows do not match the sequences")
    return out
