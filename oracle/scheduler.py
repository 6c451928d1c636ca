"""Stall-free batch builder with a paged KV pool (oracle).

The iteration is the one the pages give for stall-free batching
("Sarathi-Serve：以 chunked-prefills 与 stall-free batching 驯服 LLM 推理的吞吐—延迟权衡",
section 核心机制-2, Algorithm 3; "Sarathi-Serve: Chunked Prefills for Stall-Free
LLM Inference", sections "The mechanism" and "Algorithm / figure walkthrough"):

  1. every running decode contributes its one token;
  2. unfinished prefills continue with a chunk that fills the remaining
     budget (chunk ~ B - n_decode);
  3. while budget remains, new requests are admitted (when KV memory allows)
     and get a first chunk cut to the remaining budget;
  4. the batch runs; afterwards progress advances and finished requests leave.

The invariant (same page, 核心机制-2): decodes are always in the batch and the
batch never exceeds B tokens.  Pages hold 16 tokens and a per-request block
table maps logical to physical pages ("In-flight Batching", KV Cache 管理的协同优化);
a request whose chunk is unfinished returns to the prefill state, and after its
last chunk it decodes until EOS / max length (same page, 调度状态机).

Readings taken where the pages are silent:
  * decodes are taken in running (admission) order; if there are more than B
    of them the invariant cannot hold and the builder reports a budget error;
  * chunk size is greedy: min(prompt tokens left, B - tokens so far); any number
    of chunks may share an iteration;
  * admission is FCFS with head-of-line blocking; a new request reserves
    ceil(L/16) pages for its whole prompt when admitted; a decode takes one
    more page when its new token starts a page; the free pool is a FIFO whose
    initial order is an input and freed pages return to its tail in logical
    order; there is no preemption, so an empty pool is an error;
  * the iteration that runs the last chunk yields the first output token, so
    the request has generated 1 token and decodes from the next iteration; a
    request finishes once it has generated max_new_tokens tokens, and the K/V
    of its last token is never appended;
  * a decode's context length is the number of tokens already in the cache
    before the step; its new token is at position prompt_len + generated - 1.

Baseline policies (set_policy), the two schedules the pages set stall-free
batching against ("Sarathi-Serve：以 chunked-prefills 与 stall-free batching
驯服 LLM 推理的吞吐—延迟权衡", 问题背景; "Sarathi-Serve: Chunked Prefills for
Stall-Free LLM Inference", the scheduling taxonomy):
  * prefill-prioritizing (vLLM / Orca): new prompts are admitted eagerly,
    whenever KV memory allows, and a prompt runs whole in one iteration, so a
    long prefill holds back every running decode (a generation stall);
  * decode-prioritizing (request-level batching): new requests are admitted
    only after every request of the batch has finished, so the batch shrinks
    as its requests end.
Readings taken: an iteration of a baseline is either prompts only or decodes
only; unfinished prompts (injected mid-flight) come first, then admissions
FCFS; prompts are taken whole while the iteration stays within a prefill
token limit (the first prompt is always taken); when no prompt can run, every
running decode runs (more decodes than the limit is a budget error).
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional

PAGE_SIZE = 16


class SchedError(Exception):
    pass


class BudgetError(SchedError):
    pass


class NoPagesError(SchedError):
    pass


STALL_FREE, PREFILL_FIRST, DECODE_FIRST = 0, 1, 2


class InvalidRequest(SchedError):
    pass


def pages_for(tokens: int) -> int:
    return -(-tokens // PAGE_SIZE)


def slots_of(pages, positions) -> List[int]:
    """Physical slot of each logical position: page pages[pos // 16], offset pos % 16."""
    return [int(pages[pos // PAGE_SIZE]) * PAGE_SIZE + pos % PAGE_SIZE for pos in positions]


@dataclass
class Request:
    req_id: int
    prompt_len: int          # L
    max_new_tokens: int      # O
    computed: int = 0        # c: prompt tokens whose K/V is in the cache
    generated: int = 0       # g: output tokens produced so far
    pages: List[int] = field(default_factory=list)

    @property
    def decoding(self) -> bool:
        return self.computed == self.prompt_len


@dataclass
class Batch:
    req_ids: List[int]
    q_lens: List[int]
    context_lens: List[int]
    block_tables: List[List[int]]     # each padded with -1 to max_blocks_per_seq
    slot_mapping: List[int]
    num_decodes: int

    @property
    def cu_seqlens_q(self) -> List[int]:
        out = [0]
        for n in self.q_lens:
            out.append(out[-1] + n)
        return out

    @property
    def num_tokens(self) -> int:
        return sum(self.q_lens)


class Scheduler:
    def __init__(self, token_budget: int, max_blocks_per_seq: int, free_pages):
        if token_budget < 1 or max_blocks_per_seq < 1:
            raise InvalidRequest("bad config")
        self.B = token_budget
        self.W = max_blocks_per_seq
        self.free = deque(int(p) for p in free_pages)
        self.running: List[Request] = []
        self.waiting: deque = deque()
        self._ids = set()
        self._pending: Optional[Batch] = None
        self.policy, self.limit = STALL_FREE, 0

    def set_policy(self, policy: int, prefill_token_limit: int = 0) -> None:
        if policy not in (STALL_FREE, PREFILL_FIRST, DECODE_FIRST):
            raise InvalidRequest("policy")
        if policy != STALL_FREE and prefill_token_limit < 1:
            raise InvalidRequest("prefill token limit")
        self.policy, self.limit = policy, prefill_token_limit
        self._pending = None

    # ------------------------------------------------------------------ add
    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int,
                    computed: int = 0, generated: int = 0) -> None:
        L, O, c, g = prompt_len, max_new_tokens, computed, generated
        if req_id in self._ids:
            raise InvalidRequest("duplicate id")
        if L < 1 or O < 1 or L + O - 1 > PAGE_SIZE * self.W:
            raise InvalidRequest("lengths")
        r = Request(req_id, L, O, c, g)
        if c == 0 and g == 0:
            self.waiting.append(r)
        elif 0 < c < L and g == 0:
            self._inject(r, pages_for(L))            # whole prompt reserved
        elif c == L and 1 <= g < O:
            self._inject(r, pages_for(L + g - 1))    # the tokens in the cache
        else:
            raise InvalidRequest("progress")
        self._ids.add(req_id)
        self._pending = None

    def _inject(self, r: Request, n: int) -> None:
        if n > len(self.free):
            raise NoPagesError("pool")
        r.pages = [self.free.popleft() for _ in range(n)]
        self.running.append(r)

    # ---------------------------------------------------------------- build
    def build_batch(self) -> Batch:
        """One iteration of the builder (stall-free unless a baseline policy is
        set).  On error nothing changes."""
        if self.policy != STALL_FREE:
            return self._build_baseline()
        decodes = [r for r in self.running if r.decoding]
        if len(decodes) > self.B:
            raise BudgetError("more decodes than budget")
        grow = [r for r in decodes if r.prompt_len + r.generated - 1 == PAGE_SIZE * len(r.pages)]
        if len(grow) > len(self.free):
            raise NoPagesError("decode growth")

        # Everything below mutates; the checks above guarantee it succeeds.
        seqs = []                                   # (request, context_len, q_len)
        for r in decodes:                           # step 1: every decode, one token
            pos = r.prompt_len + r.generated - 1
            if pos == PAGE_SIZE * len(r.pages):
                r.pages.append(self.free.popleft())
            seqs.append((r, pos, 1))
        n = len(decodes)
        for r in self.running:                      # step 2: continue unfinished prefills
            if r.decoding:
                continue
            if n == self.B:
                break
            chunk = min(r.prompt_len - r.computed, self.B - n)
            seqs.append((r, r.computed, chunk))
            n += chunk
        while self.waiting and n < self.B:          # step 3: admit new requests
            r = self.waiting[0]
            need = pages_for(r.prompt_len)
            if need > len(self.free):
                break                               # FCFS: nobody skips the head
            self.waiting.popleft()
            r.pages = [self.free.popleft() for _ in range(need)]
            self.running.append(r)
            chunk = min(r.prompt_len, self.B - n)
            seqs.append((r, 0, chunk))
            n += chunk

        return self._emit(seqs, len(decodes))

    def _build_baseline(self) -> Batch:
        """Prefill-prioritizing or decode-prioritizing iteration: prompts only,
        or decodes only."""
        seqs, n = [], 0
        for r in self.running:                      # unfinished prompts, whole
            if r.decoding:
                continue
            chunk = r.prompt_len - r.computed
            if n > 0 and n + chunk > self.limit:
                break
            seqs.append((r, r.computed, chunk))
            n += chunk
        may_admit = self.policy == PREFILL_FIRST or not self.running
        admit, free = [], len(self.free)
        for r in self.waiting:                      # eager (or cohort) admission, FCFS
            if not may_admit:
                break
            need = pages_for(r.prompt_len)
            if need > free or (n > 0 and n + r.prompt_len > self.limit):
                break
            free -= need
            admit.append(r)
            n += r.prompt_len
        if n == 0:                                  # no prompt can run: all decodes
            decodes = [r for r in self.running if r.decoding]
            if len(decodes) > self.limit:
                raise BudgetError("more decodes than the token limit")
            grow = [r for r in decodes if r.prompt_len + r.generated - 1 == PAGE_SIZE * len(r.pages)]
            if len(grow) > len(self.free):
                raise NoPagesError("decode growth")
            for r in decodes:
                pos = r.prompt_len + r.generated - 1
                if pos == PAGE_SIZE * len(r.pages):
                    r.pages.append(self.free.popleft())
                seqs.append((r, pos, 1))
            return self._emit(seqs, len(decodes))
        for r in admit:
            self.waiting.popleft()
            r.pages = [self.free.popleft() for _ in range(pages_for(r.prompt_len))]
            self.running.append(r)
            seqs.append((r, 0, r.prompt_len))
        return self._emit(seqs, 0)

    def _emit(self, seqs, num_decodes) -> Batch:
        slots = []
        for r, ctx, qn in seqs:
            slots += slots_of(r.pages, range(ctx, ctx + qn))
        batch = Batch(
            req_ids=[r.req_id for r, _, _ in seqs],
            q_lens=[qn for _, _, qn in seqs],
            context_lens=[ctx for _, ctx, _ in seqs],
            block_tables=[r.pages + [-1] * (self.W - len(r.pages)) for r, _, _ in seqs],
            slot_mapping=slots,
            num_decodes=num_decodes,
        )
        self._pending = batch
        return batch

    # --------------------------------------------------------------- commit
    def commit(self, batch: Batch) -> List[int]:
        """Advance progress after the batch ran; return finished ids in batch order."""
        if batch is not self._pending:
            raise InvalidRequest("commit of a batch that was not the last one built")
        by_id: Dict[int, Request] = {r.req_id: r for r in self.running}
        finished = []
        for i, (rid, qn) in enumerate(zip(batch.req_ids, batch.q_lens)):
            r = by_id[rid]
            if i < batch.num_decodes:
                r.generated += 1
            else:
                r.computed += qn
                if r.computed == r.prompt_len:
                    r.generated = 1                 # the last chunk yields the first token
            if r.generated == r.max_new_tokens:
                finished.append(rid)
        for rid in finished:
            r = by_id[rid]
            self.running.remove(r)
            self.free.extend(r.pages)
            self._ids.discard(rid)
        self._pending = None
        return finished
