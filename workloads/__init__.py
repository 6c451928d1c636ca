"""Seeded synthetic inputs for the hybrid-batch paged-attention step.

This module only *draws* inputs: request lengths and progress, the order of the
physical page pool, Poisson arrivals, and bf16 Q/K/V values.  It holds none of
the method's arithmetic -- no batch building, no paging/slot arithmetic, no
attention -- so that both the CPU oracle (through the tests) and the HIP path
(through the tests and the benchmark) can consume the very same bits.

Workload shapes follow the pages:
  * token budgets 256 / 512 / 1536 / 2048 and the GQA layer shapes are the
    deployments evaluated in "Sarathi-Serve：以 chunked-prefills 与 stall-free
    batching 驯服 LLM 推理的吞吐—延迟权衡" (sections 3 分钟速读 and 核心机制-3);
  * prompt/output medians 1730/415 (openchat_sharegpt4) and 7059/208
    (arxiv_summarization), total length truncated at 8192 (same page, section
    实验与指标, "测试床与负载").  The datasets themselves are not available; these
    lognormal draws with the pages' medians stand in for them.  The lognormal
    sigma (0.6) is our own choice because the pages give no spread.
  * Q/K/V are N(0, 1) fp32 rounded once to bf16 (round-to-nearest-even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

PAGE_SIZE = 16          # tokens per KV page ("In-flight Batching", KV Cache 管理的协同优化)
MAX_MODEL_LEN = 8192    # truncation length of the workloads
LN_SIGMA = 0.6


@dataclass(frozen=True)
class Req:
    """A request as the scheduler receives it.

    ``num_computed`` prompt tokens are already in the KV cache and
    ``num_generated`` output tokens have been produced.  (0, 0) is a new
    request that waits for admission.
    """
    req_id: int
    prompt_len: int
    max_new_tokens: int
    num_computed: int = 0
    num_generated: int = 0

    @property
    def is_new(self) -> bool:
        return self.num_computed == 0 and self.num_generated == 0

    @property
    def cached_tokens(self) -> int:
        """Tokens whose K/V sit in the cache before the next step."""
        if self.num_computed < self.prompt_len:
            return self.num_computed
        return self.prompt_len + self.num_generated - 1


@dataclass
class Instance:
    name: str
    seed: int
    token_budget: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_blocks_per_seq: int
    num_pages: int
    free_pages: np.ndarray                    # int32 permutation: initial free-page FIFO order
    injected: List[Req] = field(default_factory=list)   # running requests, in injection order
    waiting: List[Req] = field(default_factory=list)    # new requests, FIFO order

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_budget(self, token_budget: int) -> "Instance":
        return replace(self, token_budget=token_budget, name=f"{self.name}-B{token_budget}")


def _lognormal_int(rng: np.random.Generator, median: float, lo: int, hi: int, size=None):
    x = np.rint(np.exp(rng.normal(math.log(median), LN_SIGMA, size=size)))
    return np.clip(x, lo, hi).astype(np.int64)


def _pages_for(tokens: int) -> int:
    return -(-tokens // PAGE_SIZE)


def _decode_reqs(rng, contexts, first_id: int, max_len: int) -> List[Req]:
    """Running decodes with the given number of cached tokens.

    A decode with ``ctx`` cached tokens has generated g tokens of a prompt of
    length ctx - g + 1; g ~ U{1..min(64, ctx)} and 1..80 more outputs remain.
    """
    out = []
    for i, ctx in enumerate(contexts):
        ctx = int(ctx)
        g = int(rng.integers(1, min(64, ctx) + 1))
        L = ctx - g + 1
        room = max_len - ctx            # positions still free for new tokens
        remaining = int(rng.integers(1, 81))
        remaining = max(1, min(remaining, room))
        out.append(Req(first_id + i, L, g + remaining, L, g))
    return out


def _finish(name, seed, B, Hq, Hkv, d, injected, waiting, rng, num_pages=None,
            max_len=MAX_MODEL_LEN) -> Instance:
    W = _pages_for(max_len)
    if num_pages is None:
        need = sum(_pages_for(r.cached_tokens + 1) for r in injected if r.num_computed == r.prompt_len)
        need += sum(_pages_for(r.prompt_len) for r in injected if r.num_computed < r.prompt_len)
        need += sum(_pages_for(r.prompt_len) for r in waiting)
        num_pages = int(math.ceil(1.25 * need))
    free = rng.permutation(num_pages).astype(np.int32)
    return Instance(name, seed, B, Hq, Hkv, d, W, num_pages, free, list(injected), list(waiting))


def make_config(n: int, token_budget: Optional[int] = None) -> Instance:
    """The five layer workloads.  ``token_budget`` overrides B (config-5 sweep)."""
    seed = 1000 + n
    rng = np.random.default_rng(seed)
    if n == 1:
        # Tiny: 4 q heads / 1 kv head / d 64; decodes with 40 and 70 cached
        # tokens; a 128-token prompt with 64 tokens done; B = 34; 64 pages.
        injected = [Req(1, 40, 4, 40, 1), Req(2, 70, 4, 70, 1), Req(3, 128, 1, 64, 0)]
        inst = _finish("tiny", seed, 34, 4, 1, 64, injected, [], rng, num_pages=64, max_len=128)
    elif n == 2:
        ctx = _lognormal_int(rng, 1700, 1, MAX_MODEL_LEN - 1, size=64)
        dec = _decode_reqs(rng, ctx, 1, MAX_MODEL_LEN)
        L = int(_lognormal_int(rng, 1730, 192, MAX_MODEL_LEN))
        o = int(rng.integers(0, L - 192 + 1))
        O = int(_lognormal_int(rng, 415, 1, MAX_MODEL_LEN - L + 1))
        p = Req(100, L, O, o, 0)
        inj, wait = (dec + [p], []) if o > 0 else (dec, [p])
        inst = _finish("mistral7b", seed, 256, 32, 8, 128, inj, wait, rng)
    elif n == 3:
        ctx = _lognormal_int(rng, 2000, 1, MAX_MODEL_LEN - 1, size=128)
        dec = _decode_reqs(rng, ctx, 1, MAX_MODEL_LEN)
        p = Req(1000, 7059, 208, 3072, 0)
        inst = _finish("yi34b", seed, 512, 56, 8, 128, dec + [p], [], rng)
    elif n == 4:
        ctx = rng.integers(512, MAX_MODEL_LEN, size=256)      # U{512..8191}
        dec = _decode_reqs(rng, ctx, 1, MAX_MODEL_LEN)
        L1 = int(_lognormal_int(rng, 1730, 2, MAX_MODEL_LEN))
        c1 = int(rng.integers(1, min(1279, L1 - 1) + 1))
        O1 = int(_lognormal_int(rng, 415, 1, MAX_MODEL_LEN - L1 + 1))
        L2 = int(_lognormal_int(rng, 1730, 1280 - c1, MAX_MODEL_LEN))
        O2 = int(_lognormal_int(rng, 415, 1, MAX_MODEL_LEN - L2 + 1))
        p1 = Req(1000, L1, O1, L1 - c1, 0)
        p2 = Req(1001, L2, O2, 0, 0)
        inst = _finish("llama2-70b", seed, 1536, 64, 8, 128, dec + [p1], [p2], rng)
    elif n == 5:
        ctx = rng.integers(3584, 4609, size=32)                # ~4k: U{3584..4608}
        dec = _decode_reqs(rng, ctx, 1, MAX_MODEL_LEN)
        p = Req(1000, 8192, 1, 2048, 0)
        inst = _finish("falcon180b-tp4", seed, 2048, 58, 2, 64, dec + [p], [], rng)
    else:
        raise ValueError(f"no config {n}")
    if token_budget is not None:
        inst = inst.with_budget(token_budget)
    return inst


def decode_batch_instance(seed: int, num_decodes: int, median_ctx: float, Hq: int, Hkv: int, d: int,
                          token_budget: int) -> Instance:
    """Decodes only: ``num_decodes`` running requests with lognormal contexts
    (median ``median_ctx``, sigma LN_SIGMA), as many as the budget takes."""
    rng = np.random.default_rng(seed)
    ctx = _lognormal_int(rng, median_ctx, 1, MAX_MODEL_LEN - 1, size=num_decodes)
    dec = _decode_reqs(rng, ctx, 1, MAX_MODEL_LEN)
    return _finish(f"decodes{num_decodes}-s{seed}", seed, token_budget, Hq, Hkv, d, dec, [], rng)


def long_context_instance(seed: int = 2101) -> Instance:
    """Decodes far longer than the evaluated models' 8k window (100 000,
    65 537 and 3 000 cached tokens) beside one 128-row prefill chunk, in
    Falcon-180B's TP-4 head shape (58 q heads, 2 kv heads, d 64): the blocks
    of the longest decodes are split over the most workgroups."""
    rng = np.random.default_rng(seed)
    contexts = [100_000, 65_537, 3_000]
    max_len = 100_160
    dec = _decode_reqs(rng, contexts, 1, max_len)
    chunk = Req(100, 2_048, 16, 512, 0)
    return _finish("long-context", seed, len(contexts) + 128, 58, 2, 64, dec + [chunk], [], rng, max_len=max_len)


SWEEP_BUDGETS = (256, 257, 512, 1024, 2048)
SWEEP_DIAGNOSTIC = (288, 289)


def poisson_arrivals(iterations: int, first_id: int, seed: int = 2004, rate: float = 0.5) -> List[List[Req]]:
    """New requests arriving at each iteration (sharegpt-like medians 1730/415)."""
    rng = np.random.default_rng(seed)
    out, rid = [], first_id
    for _ in range(iterations):
        k = int(rng.poisson(rate))
        batch = []
        for _ in range(k):
            L = int(_lognormal_int(rng, 1730, 1, MAX_MODEL_LEN - 1))
            O = int(_lognormal_int(rng, 415, 1, MAX_MODEL_LEN - L + 1))
            batch.append(Req(rid, L, O))
            rid += 1
        out.append(batch)
    return out


def random_small_instance(seed: int, max_reqs: int = 6, max_len: int = 96) -> Instance:
    """A tiny random state (few requests, short prompts) for property tests."""
    rng = np.random.default_rng(seed)
    W = _pages_for(max_len)
    injected, waiting, rid = [], [], 1
    for _ in range(int(rng.integers(0, max_reqs + 1))):
        kind = int(rng.integers(0, 3))
        L = int(rng.integers(1, max_len // 2 + 1))
        O = int(rng.integers(1, max_len - L + 2))
        if kind == 0:
            waiting.append(Req(rid, L, O))
        elif kind == 1 and L > 1:
            injected.append(Req(rid, L, O, int(rng.integers(1, L)), 0))
        elif O > 1:
            injected.append(Req(rid, L, O, L, int(rng.integers(1, O))))
        else:
            waiting.append(Req(rid, L, O))
        rid += 1
    B = int(rng.integers(max(1, len(injected)), 3 * max_len))
    need = sum(_pages_for(r.prompt_len + r.max_new_tokens) for r in injected + waiting)
    num_pages = int(rng.integers(max(1, need // 2), need + 4))
    free = rng.permutation(num_pages).astype(np.int32)
    return Instance(f"small{seed}", seed, B, 4, 2, 16, W, num_pages, free, injected, waiting)


# ---------------------------------------------------------------- values ---
def _torch():
    import torch
    return torch


def _gen(device, seed: int):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal_bf16(shape, seed: int, device="cpu"):
    """N(0,1) fp32 draws rounded once to bf16 (RNE)."""
    torch = _torch()
    g = _gen(device, seed)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def history_kv(inst: Instance, req: Req, device="cpu"):
    """K and V rows for the cached positions 0..cached-1 of ``req``: [cached, Hkv, d] bf16."""
    n = req.cached_tokens
    base = inst.seed * 1_000_003 + req.req_id * 7919
    k = normal_bf16((n, inst.num_kv_heads, inst.head_dim), base + 1, device)
    v = normal_bf16((n, inst.num_kv_heads, inst.head_dim), base + 2, device)
    return k, v


def step_qkv(inst: Instance, num_tokens: int, step: int = 0, device="cpu"):
    """This step's packed rows: q [T, Hq, d], k_new / v_new [T, Hkv, d], all bf16."""
    base = inst.seed * 7_000_003 + step * 104_729
    q = normal_bf16((num_tokens, inst.num_q_heads, inst.head_dim), base + 11, device)
    k = normal_bf16((num_tokens, inst.num_kv_heads, inst.head_dim), base + 12, device)
    v = normal_bf16((num_tokens, inst.num_kv_heads, inst.head_dim), base + 13, device)
    return q, k, v


# --------------------------------------------------------- linear layers ---
# Projection shapes of one decoder layer, (name, N, K) with y[B, N] = x[B, K] w[N, K]^T.
# The pages name the models and their attention head shapes; the hidden and
# MLP widths below are those models' published configurations (not on the
# pages).  Falcon-180B is one GPU's share under 4-way tensor parallelism
# (column-parallel QKV and MLP-up, row-parallel O and MLP-down), as for its
# attention layer.
LINEAR_LAYERS = {
    "mistral7b": [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336)],
    "yi34b": [("qkv", 9216, 7168), ("o", 7168, 7168), ("gate_up", 40960, 7168), ("down", 7168, 20480)],
    "llama2-70b": [("qkv", 10240, 8192), ("o", 8192, 8192), ("gate_up", 57344, 8192), ("down", 8192, 28672)],
    "falcon180b-tp4": [("qkv", 3968, 14848), ("o", 14848, 3712), ("up", 14848, 14848), ("down", 14848, 14848)],
}


def linear_weight_bf16(N: int, K: int, seed: int, device="cpu"):
    """Random-init weight [N, K]: N(0, 1/K) fp32 draws rounded once to bf16,
    so that outputs of N(0, 1) token rows are about unit size."""
    torch = _torch()
    g = _gen(device, seed)
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32)
    return (w * (1.0 / math.sqrt(K))).to(torch.bfloat16)
