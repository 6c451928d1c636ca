"""Test plumbing: the oracle's expectations for a GPU step.

The GPU side (``chunked_prefill_decode_amd.runner``) uses only the library;
the oracle side uses only ``oracle/`` plus the shared input generators.  The
two meet only in the generators' bf16 tensors.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

import workloads as W
from chunked_prefill_decode_amd.runner import (ChunkingStudy, GpuStep, ScheduleRun, batch_from_arrays,  # noqa: F401
                                               load_scheduler as load_native_sched, slots_view)
from oracle import inputs as OI
from oracle import kvcache as OK
from oracle import scheduler as OS


def load_oracle_sched(inst: W.Instance, free_pages=None) -> OS.Scheduler:
    return OI.load_scheduler(inst, free_pages)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_inputs(inst: W.Instance, step: GpuStep, seq_subset=None):
    """(seqs, q rows, per-sequence K/V, packed row indices) of the step's
    first batch as the ORACLE builds it, from the generators' tensors."""
    return OI.step_inputs(inst, step.hist, step.q_gen, step.k_new_gen, step.v_new_gen, step.free_pages, seq_subset)


def expected_cache_bits(fill: float, num_pages: int, Hkv: int, d: int, writes):
    """The oracle's after-image of a cache filled with `fill` that then took
    the writes [(slots, k rows, v rows), ...] in order: uint16 [slots, Hkv, d]
    for K and for V."""
    fill_bits = bf16_bits(torch.tensor([fill], dtype=torch.bfloat16))[0]
    out = []
    for which in (1, 2):
        cache = np.full((num_pages * 16, Hkv, d), fill_bits, np.uint16)
        slots = [s for w in writes for s in w[0]]
        rows = np.concatenate([bf16_bits(w[which]).reshape(-1, Hkv, d) for w in writes]) if writes else None
        if slots:
            cache = OK.append_expected(cache, rows, slots)
        out.append(cache)
    return out[0], out[1]


def kv_bit_exact(step: GpuStep) -> bool:
    """After step.run(): the whole cache equals the oracle's expectation --
    the fill value everywhere, each request's history at the slots the
    ORACLE's builder gives its positions, then this step's rows at the
    oracle's slot mapping."""
    inst = step.inst
    ob = load_oracle_sched(inst, step.free_pages).build_batch()
    hslots, hk, hv = [], [], []
    for rid, ctx, bt in zip(ob.req_ids, ob.context_lens, ob.block_tables):
        if ctx == 0:
            continue
        k, v = step.hist[rid]
        hslots += OS.slots_of(bt, range(ctx))
        hk.append(k.cpu())
        hv.append(v.cpu())
    writes = []
    if hslots:
        writes.append((hslots, torch.cat(hk), torch.cat(hv)))
    writes.append((ob.slot_mapping, step.k_new_gen.cpu(), step.v_new_gen.cpu()))
    ke, ve = expected_cache_bits(step.fill, inst.num_pages, inst.num_kv_heads, inst.head_dim, writes)
    kg, vg = slots_view(step.k_cache, step.v_cache)
    ok = np.array_equal(bf16_bits(kg), ke)
    del ke
    return ok and np.array_equal(bf16_bits(vg), ve)
