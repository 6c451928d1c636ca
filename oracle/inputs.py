"""The oracle's view of a seeded workload (oracle side -- TEST INFRASTRUCTURE ONLY).

Turns an instance of ``workloads`` plus the generators' bf16 tensors into the
arguments of ``attention.attend``: each sequence's (context length, query
rows) comes from the ORACLE's own batch builder (``scheduler``), and each
sequence's K/V is its request's contiguous rows -- history first, then this
step's rows -- taken from the generators' tensors, never from the GPU.  No
arithmetic of the method happens here; it only gathers inputs.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from oracle import scheduler as OS


def load_scheduler(inst, free_pages=None) -> OS.Scheduler:
    """An oracle scheduler holding the instance's running and waiting requests."""
    pages = inst.free_pages if free_pages is None else free_pages
    s = OS.Scheduler(inst.token_budget, inst.max_blocks_per_seq, np.asarray(pages).tolist())
    for r in inst.injected:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens, r.num_computed, r.num_generated)
    for r in inst.waiting:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
    return s


def f32(t) -> np.ndarray:
    """bf16 torch tensor -> float32 numpy (exact), on the CPU."""
    import torch
    return t.detach().to("cpu", torch.float32).numpy()


class LazyKV:
    """Per-sequence (K, V) of a batch, gathered one sequence at a time (so
    that a large batch's fp64 copies are never all in memory at once)."""

    def __init__(self, parts):
        self.parts = parts          # per sequence: list of (k, v) tensor pieces, in position order

    def __len__(self):
        return len(self.parts)

    def __getitem__(self, i):
        ks = [f32(k) for k, _ in self.parts[i]]
        vs = [f32(v) for _, v in self.parts[i]]
        return np.concatenate(ks), np.concatenate(vs)

    def __iter__(self):
        for i in range(len(self.parts)):
            yield self[i]


def attention_inputs(batch: OS.Batch, q, k_new, v_new, rows_of: Dict[int, list],
                     seq_subset: Optional[Sequence[int]] = None):
    """Arguments of attention.attend for the sequences of an oracle batch.

    q, k_new, v_new: this step's generated rows (bf16 tensors, batch order).
    rows_of: request id -> list of (k, v) pieces of its cached rows, in
    position order (its history before this step).
    Returns (seqs, q rows as float32, per-sequence K/V, packed row indices)."""
    cu = batch.cu_seqlens_q
    idx = range(len(batch.req_ids)) if seq_subset is None else seq_subset
    seqs, qs, parts, rows = [], [], [], []
    for s in idx:
        rid, ctx, n = batch.req_ids[s], batch.context_lens[s], batch.q_lens[s]
        hist = rows_of.get(rid, [])
        assert sum(int(k.shape[0]) for k, _ in hist) == ctx, "history rows do not match the context length"
        seqs.append((ctx, n))
        parts.append(list(hist) + [(k_new[cu[s]:cu[s + 1]], v_new[cu[s]:cu[s + 1]])])
        qs.append(f32(q[cu[s]:cu[s + 1]]))
        rows.extend(range(cu[s], cu[s + 1]))
    q_rows = np.concatenate(qs) if qs else np.zeros((0,) + tuple(q.shape[1:]), np.float32)
    return seqs, q_rows, LazyKV(parts), rows


def step_inputs(inst, hist: Dict[int, Tuple], q, k_new, v_new, free_pages=None,
                seq_subset: Optional[Sequence[int]] = None):
    """attention_inputs for the first batch of an instance (the oracle's
    builder on the instance's state); hist: request id -> (k, v) history."""
    ob = load_scheduler(inst, free_pages).build_batch()
    rows_of = {rid: [kv] for rid, kv in hist.items()}
    return attention_inputs(ob, q, k_new, v_new, rows_of, seq_subset)
