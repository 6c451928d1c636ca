"""ctypes binding of libsarathi_attn (argument marshalling only).

Every function here has the name of the C entry point it calls
(include/sarathi_attn.h) and only converts arguments: numpy arrays and torch
tensors become pointers, the current torch stream becomes a hipStream_t.
All computation happens in the library; if the library is missing this
module raises at import time -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SARATHI_ATTN_LIB") or os.path.join(_HERE, "libsarathi_attn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_BUDGET, SA_ERR_NO_PAGES, SA_ERR_CAPACITY = 0, 1, 2, 3, 4
SA_ERR_UNKNOWN_REQUEST, SA_ERR_HIP, SA_ERR_UNSUPPORTED, SA_ERR_STATE = 5, 6, 7, 8
SA_PLAN_STREAM_KV = 1
STATUS_NAMES = {0: "SA_OK", 1: "SA_ERR_INVALID_ARG", 2: "SA_ERR_BUDGET", 3: "SA_ERR_NO_PAGES",
                4: "SA_ERR_CAPACITY", 5: "SA_ERR_UNKNOWN_REQUEST", 6: "SA_ERR_HIP",
                7: "SA_ERR_UNSUPPORTED", 8: "SA_ERR_STATE"}

EXPORTED = [
    "sa_last_error", "sa_version", "sa_sched_create", "sa_sched_destroy", "sa_sched_clone", "sa_sched_set_policy",
    "sa_sched_add_request", "sa_sched_stats", "sa_build_batch", "sa_sched_commit", "sa_history_slots",
    "sa_batch_upload_size", "sa_batch_pack", "sa_batch_upload", "sa_batch_upload_append", "sa_kv_append",
    "sa_hybrid_attn_workspace_size",
    "sa_hybrid_attn", "sa_hybrid_attn_noalloc", "sa_linear_workspace_size", "sa_linear",
]
SA_NOALLOC_WORKSPACE_BYTES = 64 << 20


class SarathiError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libsarathi_attn.so is not built ({LIB_PATH}); run __graft_entry__.build()")
# torch is loaded first so that the library binds to the HIP runtime torch
# already holds (same soname), the one that owns the device memory and the
# streams passed in.  Loaded the other way round, the library would pull in
# the system's runtime as a second HIP/HSA instance in the process, and its
# calls would then find no device.
import torch  # noqa: E402,F401
_lib = ctypes.CDLL(LIB_PATH)

i32, i64, vp, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
P_i32, P_i64, P_sz = ctypes.POINTER(i32), ctypes.POINTER(i64), ctypes.POINTER(sz)


class sa_sched_config(ctypes.Structure):
    _fields_ = [("token_budget", i32), ("page_size", i32), ("max_blocks_per_seq", i32), ("num_pages", i32)]


class sa_batch(ctypes.Structure):
    _fields_ = [("cap_seqs", i32), ("cap_tokens", i32), ("num_seqs", i32), ("num_decodes", i32),
                ("num_prefill_chunks", i32), ("num_tokens", i32), ("max_blocks_per_seq", i32),
                ("max_kv_len", i32), ("req_ids", P_i64), ("cu_seqlens_q", P_i32), ("context_lens", P_i32),
                ("block_tables", P_i32), ("slot_mapping", P_i32)]


class sa_batch_dev(ctypes.Structure):
    _fields_ = [("cu_seqlens_q", vp), ("context_lens", vp), ("slot_mapping", vp), ("block_table_offsets", vp),
                ("block_tables", vp),
                ("work", vp), ("combine", vp),
                ("num_seqs", i32), ("num_decodes", i32), ("num_tokens", i32), ("bt_stride", i32),
                ("num_q_heads", i32), ("num_kv_heads", i32), ("head_dim", i32), ("num_pages", i32),
                ("num_work_items", i32), ("num_combine_groups", i32), ("num_partials", i32), ("sliding_window", i32),
                ("plan_flags", i32), ("reserved", i32)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib_sa_last_error = _sig("sa_last_error", ctypes.c_char_p, [])
_lib_sa_version = _sig("sa_version", ctypes.c_char_p, [])
_lib_sa_sched_create = _sig("sa_sched_create", i32, [ctypes.POINTER(sa_sched_config), P_i32, ctypes.POINTER(vp)])
_lib_sa_sched_destroy = _sig("sa_sched_destroy", None, [vp])
_lib_sa_sched_clone = _sig("sa_sched_clone", i32, [vp, ctypes.POINTER(vp)])
_lib_sa_sched_set_policy = _sig("sa_sched_set_policy", i32, [vp, i32, i32])
_lib_sa_sched_add_request = _sig("sa_sched_add_request", i32, [vp, i64, i32, i32, i32, i32])
_lib_sa_sched_stats = _sig("sa_sched_stats", i32, [vp, P_i32, P_i32, P_i32])
_lib_sa_build_batch = _sig("sa_build_batch", i32, [vp, ctypes.POINTER(sa_batch)])
_lib_sa_sched_commit = _sig("sa_sched_commit", i32, [vp, ctypes.POINTER(sa_batch), P_i64, i32, P_i32])
_lib_sa_history_slots = _sig("sa_history_slots", i32, [ctypes.POINTER(sa_batch), P_i32, i64, P_i64])
_lib_sa_batch_upload_size = _sig("sa_batch_upload_size", i32, [ctypes.POINTER(sa_batch), i32, i32, i32, i32, P_sz])
_lib_sa_batch_pack = _sig("sa_batch_pack", i32, [ctypes.POINTER(sa_batch), i32, i32, i32, i32, i32, vp, vp, sz,
                                                 ctypes.POINTER(sa_batch_dev)])
_lib_sa_batch_upload = _sig("sa_batch_upload", i32, [ctypes.POINTER(sa_batch), i32, i32, i32, i32, i32, vp, vp, sz,
                                                     vp, ctypes.POINTER(sa_batch_dev)])
_lib_sa_batch_upload_append = _sig("sa_batch_upload_append", i32, [ctypes.POINTER(sa_batch), i32, i32, i32, i32, i32,
                                                                   vp, vp, sz, vp, vp, vp, vp, vp,
                                                                   ctypes.POINTER(sa_batch_dev)])
_lib_sa_kv_append = _sig("sa_kv_append", i32, [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp])
_lib_sa_hybrid_attn_workspace_size = _sig("sa_hybrid_attn_workspace_size", i32, [ctypes.POINTER(sa_batch_dev), P_sz])
_lib_sa_hybrid_attn = _sig("sa_hybrid_attn", i32, [vp, vp, vp, ctypes.POINTER(sa_batch_dev), f32, vp, vp, sz, vp])
_lib_sa_hybrid_attn_noalloc = _sig("sa_hybrid_attn_noalloc", i32, [vp, vp, vp, ctypes.POINTER(sa_batch_dev), f32, vp, vp])
_lib_sa_linear_workspace_size = _sig("sa_linear_workspace_size", i32, [i32, i32, i32, P_sz])
_lib_sa_linear = _sig("sa_linear", i32, [vp, vp, vp, i32, i32, i32, vp, sz, vp])


def _check(st: int, where: str) -> None:
    if st != SA_OK:
        raise SarathiError(st, where, sa_last_error())


def _ptr(x) -> int:
    """Device or host address of a tensor/array, or an int passed through."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def sa_last_error() -> str:
    return _lib_sa_last_error().decode()


def sa_version() -> str:
    return _lib_sa_version().decode()


# ------------------------------------------------------------- scheduler ---
class HostBatch:
    """Caller-owned host arrays of one batch (numpy), plus the C struct."""

    def __init__(self, cap_seqs: int, cap_tokens: int, max_blocks_per_seq: int):
        self.req_ids = np.zeros(cap_seqs, np.int64)
        self.cu_seqlens_q = np.zeros(cap_seqs + 1, np.int32)
        self.context_lens = np.zeros(cap_seqs, np.int32)
        self.block_tables = np.full((cap_seqs, max_blocks_per_seq), -1, np.int32)
        self.slot_mapping = np.zeros(max(cap_tokens, 1), np.int32)
        self.c = sa_batch()
        self.c.cap_seqs = cap_seqs
        self.c.cap_tokens = cap_tokens
        self.c.max_blocks_per_seq = max_blocks_per_seq
        self.c.req_ids = self.req_ids.ctypes.data_as(P_i64)
        self.c.cu_seqlens_q = self.cu_seqlens_q.ctypes.data_as(P_i32)
        self.c.context_lens = self.context_lens.ctypes.data_as(P_i32)
        self.c.block_tables = self.block_tables.ctypes.data_as(P_i32)
        self.c.slot_mapping = self.slot_mapping.ctypes.data_as(P_i32)

    # views of the filled part
    @property
    def num_seqs(self): return self.c.num_seqs
    @property
    def num_decodes(self): return self.c.num_decodes
    @property
    def num_tokens(self): return self.c.num_tokens

    def view(self):
        S, T = self.c.num_seqs, self.c.num_tokens
        return dict(req_ids=self.req_ids[:S].tolist(), cu_seqlens_q=self.cu_seqlens_q[:S + 1].tolist(),
                    context_lens=self.context_lens[:S].tolist(), block_tables=self.block_tables[:S].tolist(),
                    slot_mapping=self.slot_mapping[:T].tolist(), num_decodes=self.c.num_decodes)


def sa_sched_create(token_budget: int, max_blocks_per_seq: int, free_pages, page_size: int = 16) -> int:
    fp = np.ascontiguousarray(free_pages, dtype=np.int32)
    cfg = sa_sched_config(token_budget, page_size, max_blocks_per_seq, len(fp))
    h = vp()
    _check(_lib_sa_sched_create(ctypes.byref(cfg), fp.ctypes.data_as(P_i32), ctypes.byref(h)), "sa_sched_create")
    return h.value


def sa_sched_destroy(h: int) -> None:
    _lib_sa_sched_destroy(h)


def sa_sched_clone(h: int) -> int:
    out = vp()
    _check(_lib_sa_sched_clone(h, ctypes.byref(out)), "sa_sched_clone")
    return out.value


def sa_sched_add_request(h: int, req_id: int, prompt_len: int, max_new_tokens: int,
                         num_computed: int = 0, num_generated: int = 0) -> None:
    _check(_lib_sa_sched_add_request(h, req_id, prompt_len, max_new_tokens, num_computed, num_generated),
           "sa_sched_add_request")


def sa_sched_stats(h: int):
    a, b, c = i32(), i32(), i32()
    _check(_lib_sa_sched_stats(h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "sa_sched_stats")
    return a.value, b.value, c.value


def sa_build_batch(h: int, batch: HostBatch) -> HostBatch:
    _check(_lib_sa_build_batch(h, ctypes.byref(batch.c)), "sa_build_batch")
    return batch


def sa_sched_commit(h: int, batch: HostBatch, cap: int = 4096) -> List[int]:
    fin = np.zeros(max(cap, 1), np.int64)
    n = i32()
    _check(_lib_sa_sched_commit(h, ctypes.byref(batch.c), fin.ctypes.data_as(P_i64), cap, ctypes.byref(n)),
           "sa_sched_commit")
    return fin[:n.value].tolist()


def sa_history_slots(batch: HostBatch) -> np.ndarray:
    n = i64()
    st = _lib_sa_history_slots(ctypes.byref(batch.c), None, 0, ctypes.byref(n))
    if st not in (SA_OK, SA_ERR_CAPACITY):
        _check(st, "sa_history_slots")
    out = np.zeros(max(n.value, 1), np.int32)
    _check(_lib_sa_history_slots(ctypes.byref(batch.c), out.ctypes.data_as(P_i32), n.value, ctypes.byref(n)),
           "sa_history_slots")
    return out[:n.value]


class Scheduler:
    """Owning wrapper of an sa_sched handle."""

    def __init__(self, token_budget: int, max_blocks_per_seq: int, free_pages, handle: Optional[int] = None):
        self.B, self.W = token_budget, max_blocks_per_seq
        self.h = handle if handle is not None else sa_sched_create(token_budget, max_blocks_per_seq, free_pages)

    def __del__(self):
        # At interpreter exit the module's globals may already be gone; the
        # process ends anyway, so the handle is simply left to it.
        h = getattr(self, "h", None)
        if h and _lib_sa_sched_destroy is not None:
            try:
                _lib_sa_sched_destroy(h)
            except Exception:
                pass
            self.h = None

    def clone(self) -> "Scheduler":
        return Scheduler(self.B, self.W, None, handle=sa_sched_clone(self.h))

    STALL_FREE, PREFILL_FIRST, DECODE_FIRST = 0, 1, 2

    def set_policy(self, policy: int, prefill_token_limit: int = 0) -> None:
        _check(_lib_sa_sched_set_policy(self.h, policy, prefill_token_limit), "sa_sched_set_policy")

    def add_request(self, req_id, prompt_len, max_new_tokens, num_computed=0, num_generated=0):
        sa_sched_add_request(self.h, req_id, prompt_len, max_new_tokens, num_computed, num_generated)

    def stats(self):
        return sa_sched_stats(self.h)

    def build_batch(self, cap_seqs: int = 1024, cap_tokens: Optional[int] = None) -> HostBatch:
        b = HostBatch(cap_seqs, self.B if cap_tokens is None else cap_tokens, self.W)
        return sa_build_batch(self.h, b)

    def commit(self, batch: HostBatch) -> List[int]:
        return sa_sched_commit(self.h, batch)


# ------------------------------------------------------------------ device ---
def sa_batch_upload_size(batch: HostBatch, Hq: int, Hkv: int, d: int, window: int = 0) -> int:
    n = sz()
    _check(_lib_sa_batch_upload_size(ctypes.byref(batch.c), Hq, Hkv, d, window, ctypes.byref(n)),
           "sa_batch_upload_size")
    return n.value


def sa_batch_pack(batch: HostBatch, Hq: int, Hkv: int, d: int, num_pages: int, staging: np.ndarray,
                  dev_address: int, window: int = 0) -> sa_batch_dev:
    """Host-only packing into a numpy buffer (16-byte aligned); the layout
    refers to device address `dev_address`, which is never touched."""
    out = sa_batch_dev()
    _check(_lib_sa_batch_pack(ctypes.byref(batch.c), Hq, Hkv, d, window, num_pages, staging.ctypes.data,
                              dev_address, staging.nbytes, ctypes.byref(out)), "sa_batch_pack")
    return out


def sa_batch_upload(batch: HostBatch, Hq: int, Hkv: int, d: int, num_pages: int, staging, dev_buf,
                    stream=None, window: int = 0) -> sa_batch_dev:
    """staging: pinned host tensor (uint8/int32), dev_buf: device tensor; both >= upload size bytes.
    window: sliding window in keys (0: none)."""
    out = sa_batch_dev()
    nbytes = min(staging.numel() * staging.element_size(), dev_buf.numel() * dev_buf.element_size())
    _check(_lib_sa_batch_upload(ctypes.byref(batch.c), Hq, Hkv, d, window, num_pages, _ptr(staging), _ptr(dev_buf),
                                nbytes, _stream(stream), ctypes.byref(out)), "sa_batch_upload")
    return out


def sa_batch_upload_append(batch: HostBatch, Hq: int, Hkv: int, d: int, num_pages: int, staging, dev_buf,
                           k_new, v_new, k_cache, v_cache, stream=None, window: int = 0) -> sa_batch_dev:
    """sa_batch_upload + sa_kv_append as one kernel; staging must be a pinned host tensor."""
    out = sa_batch_dev()
    nbytes = min(staging.numel() * staging.element_size(), dev_buf.numel() * dev_buf.element_size())
    _check(_lib_sa_batch_upload_append(ctypes.byref(batch.c), Hq, Hkv, d, window, num_pages, _ptr(staging),
                                       _ptr(dev_buf), nbytes, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                       _stream(stream), ctypes.byref(out)), "sa_batch_upload_append")
    return out


def sa_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens: int, num_kv_heads: int, head_dim: int,
                 num_pages: int, stream=None) -> None:
    _check(_lib_sa_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), num_tokens,
                             num_kv_heads, head_dim, num_pages, _stream(stream)), "sa_kv_append")


def sa_hybrid_attn_workspace_size(dev: sa_batch_dev) -> int:
    n = sz()
    _check(_lib_sa_hybrid_attn_workspace_size(ctypes.byref(dev), ctypes.byref(n)), "sa_hybrid_attn_workspace_size")
    return n.value


def sa_hybrid_attn(q, k_cache, v_cache, dev: sa_batch_dev, softmax_scale: float, out, workspace,
                   workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib_sa_hybrid_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(dev), softmax_scale, _ptr(out),
                               _ptr(workspace), workspace_bytes, _stream(stream)), "sa_hybrid_attn")


def sa_hybrid_attn_noalloc(q, k_cache, v_cache, dev: sa_batch_dev, softmax_scale: float, out, stream=None) -> None:
    _check(_lib_sa_hybrid_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(dev), softmax_scale,
                                       _ptr(out), _stream(stream)), "sa_hybrid_attn_noalloc")


def sa_linear_workspace_size(M: int, N: int, K: int) -> int:
    n = sz()
    _check(_lib_sa_linear_workspace_size(M, N, K, ctypes.byref(n)), "sa_linear_workspace_size")
    return n.value


def sa_linear(x, w, y, M: int, N: int, K: int, workspace=None, workspace_bytes: Optional[int] = None,
              stream=None) -> None:
    """y[M, N] = x[M, K] w[N, K]^T (bf16 device tensors); the workspace needs no initialisation."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib_sa_linear(_ptr(x), _ptr(w), _ptr(y), M, N, K, _ptr(workspace), workspace_bytes, _stream(stream)),
           "sa_linear")


def kv_cache_shapes(num_pages: int, num_kv_heads: int, head_dim: int):
    """Shapes of the K and V cache tensors in the library's layout."""
    return (num_pages, num_kv_heads, 16, head_dim), (num_pages, num_kv_heads, head_dim, 16)
