"""What a paged KV append leaves in the cache (oracle).

"In-flight Batching", section KV Cache 管理的协同优化: the cache is cut into
16-token pages reached through a per-request block table, and the pages of a
request need not be physically contiguous.  "Sarathi-Serve：以 chunked-prefills
与 stall-free batching 驯服 LLM 推理的吞吐—延迟权衡", section GPU / 系统数据路径,
step ⑤: a prefill chunk appends its new K/V; a decode writes the slot of its
one new token (and reads the rest).

The oracle speaks of a cache only through logical slots (slot = page * 16 +
offset) and per-slot token vectors; the physical byte layout is the library's
business.  A negative slot means "do not store".
"""
from __future__ import annotations

import numpy as np


def append_expected(cache_slots: np.ndarray, new_rows: np.ndarray, slot_mapping) -> np.ndarray:
    """cache_slots: [num_slots, ...] before-image (any dtype, compared bitwise).
    new_rows: [T, ...] rows of this step.  Returns the after-image."""
    out = np.array(cache_slots, copy=True)
    for t, s in enumerate(slot_mapping):
        if s >= 0:
            out[int(s)] = new_rows[t]
    return out
