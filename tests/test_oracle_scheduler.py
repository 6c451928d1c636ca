"""Pins for oracle.scheduler (the stall-free batch builder).

  * a hand-derived golden batch for the tiny workload (tests/golden);
  * the closed form C = B - n_decode for every workload and the budget sweep
    ("Sarathi-Serve: Chunked Prefills for Stall-Free LLM Inference", The mechanism);
  * the invariant: every running decode is in the batch and the batch holds at
    most B tokens ("Sarathi-Serve：以 chunked-prefills 与 stall-free batching 驯服
    LLM 推理的吞吐—延迟权衡", 核心机制-2), checked on thousands of random schedules;
  * chunks partition each prompt in order; a request decodes only after its
    last chunk ("In-flight Batching", 调度状态机);
  * an independent token-at-a-time formulation of the same greedy fill;
  * page conservation, error paths that leave the state unchanged.
"""
import copy
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import scheduler as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make_sched(inst):
    s = S.Scheduler(inst.token_budget, inst.max_blocks_per_seq, inst.free_pages.tolist())
    for r in inst.injected:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens, r.num_computed, r.num_generated)
    for r in inst.waiting:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
    return s


def test_golden_tiny_batch():
    gold = json.load(open(os.path.join(GOLDEN, "config1_batch.json")))
    inst = W.make_config(1)
    free = inst.free_pages.tolist()
    sched = make_sched(inst)
    b = sched.build_batch()
    exp = gold["expected"]
    assert b.req_ids == exp["req_ids"]
    assert b.num_decodes == exp["num_decodes"]
    assert b.cu_seqlens_q == exp["cu_seqlens_q"]
    assert b.context_lens == exp["context_lens"]
    first = 0
    owned = []
    for r in gold["requests_in_injection_order"]:
        owned.append(free[first:first + r["pages_reserved"]])
        first += r["pages_reserved"]
    slots = []
    for s_idx, (lp, off) in enumerate(zip(exp["slot_pages_logical"], exp["slot_offsets"])):
        assert b.block_tables[s_idx] == owned[s_idx] + [-1] * (8 - len(owned[s_idx]))
        slots += [owned[s_idx][p] * 16 + o for p, o in zip(lp, off)]
    assert b.slot_mapping == slots
    fin = sched.commit(b)
    assert fin == exp["after_commit"]["finished"]
    assert [r.generated for r in sched.running] == exp["after_commit"]["generated"]
    assert [r.computed for r in sched.running] == exp["after_commit"]["computed"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_chunk_is_budget_minus_decodes(n):
    inst = W.make_config(n)
    b = make_sched(inst).build_batch()
    D = sum(1 for r in inst.injected if r.num_computed == r.prompt_len)
    assert b.num_decodes == D
    assert b.num_tokens == inst.token_budget
    chunks = b.q_lens[D:]
    if n == 4:
        p1 = [r for r in inst.injected if r.num_computed < r.prompt_len][0]
        c1 = p1.prompt_len - p1.num_computed
        assert chunks == [c1, 1280 - c1]
    else:
        assert chunks == [inst.token_budget - D]


@pytest.mark.parametrize("B", W.SWEEP_BUDGETS + W.SWEEP_DIAGNOSTIC)
def test_sweep_chunks(B):
    b = make_sched(W.make_config(5, B)).build_batch()
    assert b.q_lens[32:] == [B - 32]
    assert b.context_lens[32] == 2048


def token_level_fill(running, waiting, free_count, B):
    """Independent formulation: hand out the budget one token at a time.

    Returns [(req_id, ctx, q_len)] in batch order or None if the decode
    growth needs more pages than exist."""
    out, budget = [], B
    grow = 0
    for r in running:
        if r.computed == r.prompt_len:
            pos = r.prompt_len + r.generated - 1
            grow += pos % 16 == 0 and pos // 16 == len(r.pages)
            out.append([r.req_id, pos, 1])
            budget -= 1
    if grow > free_count:
        return None
    free_count -= grow
    cands = [[r.req_id, r.computed, r.prompt_len - r.computed] for r in running if r.computed < r.prompt_len]
    for c in cands:
        given = 0
        while budget > 0 and given < c[2]:
            given += 1
            budget -= 1
        if given:
            out.append([c[0], c[1], given])
    for w in waiting:
        if budget == 0:
            break
        need = -(-w.prompt_len // 16)
        if need > free_count:
            break
        free_count -= need
        given = 0
        while budget > 0 and given < w.prompt_len:
            given += 1
            budget -= 1
        out.append([w.req_id, 0, given])
    return out


def check_invariants(sched_before, b, B):
    decoding = [r.req_id for r in sched_before.running if r.computed == r.prompt_len]
    assert b.req_ids[:b.num_decodes] == decoding          # every decode, in order, first
    assert all(q == 1 for q in b.q_lens[:b.num_decodes])
    assert b.num_tokens <= B
    assert len(set(b.req_ids)) == len(b.req_ids)
    assert all(q >= 1 for q in b.q_lens)
    assert len(b.slot_mapping) == b.num_tokens
    assert len(set(b.slot_mapping)) == len(b.slot_mapping)    # no slot written twice


@pytest.mark.parametrize("seed", range(40))
def test_random_schedules(seed):
    inst = W.random_small_instance(seed)
    try:
        sched = make_sched(inst)
    except S.NoPagesError:
        return
    arrivals = W.poisson_arrivals(30, 10_000, seed=seed, rate=0.7)
    total_pages = inst.num_pages
    progress = {r.req_id: r.computed for r in sched.running}
    for it in range(30):
        for r in arrivals[it]:
            L = min(r.prompt_len, 40)
            O = min(r.max_new_tokens, inst.max_blocks_per_seq * 16 - L + 1)
            sched.add_request(r.req_id, L, O)
        before = copy.deepcopy(sched)
        brute = token_level_fill(before.running, list(before.waiting), len(before.free), inst.token_budget)
        try:
            b = sched.build_batch()
        except S.BudgetError:
            assert sum(r.decoding for r in before.running) > inst.token_budget
            return
        except S.NoPagesError:
            assert brute is None
            # transactional: nothing changed
            assert [(r.req_id, r.computed, r.generated, r.pages) for r in sched.running] == \
                   [(r.req_id, r.computed, r.generated, r.pages) for r in before.running]
            assert list(sched.free) == list(before.free)
            return
        assert [list(x) for x in zip(b.req_ids, b.context_lens, b.q_lens)] == brute
        check_invariants(before, b, inst.token_budget)
        # chunks continue exactly where the previous one ended
        for rid, ctx, qn in zip(b.req_ids[b.num_decodes:], b.context_lens[b.num_decodes:], b.q_lens[b.num_decodes:]):
            assert progress.get(rid, 0) == ctx
            progress[rid] = ctx + qn
        # the decode token sits right after everything in the cache
        for rid, ctx in zip(b.req_ids[:b.num_decodes], b.context_lens[:b.num_decodes]):
            r = next(x for x in before.running if x.req_id == rid)
            assert ctx == r.prompt_len + r.generated - 1
        fin = sched.commit(b)
        for rid in fin:
            assert all(r.req_id != rid for r in sched.running)
        owned = [p for r in sched.running for p in r.pages]
        assert len(owned) + len(sched.free) == total_pages
        assert sorted(owned + list(sched.free)) == list(range(total_pages))


def test_request_lifecycle_and_page_return():
    sched = S.Scheduler(8, 4, list(range(10)))
    sched.add_request(7, 20, 3)             # new: waits
    b = sched.build_batch()
    assert (b.req_ids, b.context_lens, b.q_lens, b.num_decodes) == ([7], [0], [8], 0)
    assert b.block_tables[0] == [0, 1, -1, -1]        # ceil(20/16) = 2 pages reserved at admission
    sched.commit(b)
    b = sched.build_batch()
    assert (b.context_lens, b.q_lens) == ([8], [8])
    sched.commit(b)
    b = sched.build_batch()
    assert (b.context_lens, b.q_lens) == ([16], [4])  # last chunk
    assert sched.commit(b) == []
    r = sched.running[0]
    assert (r.computed, r.generated) == (20, 1)       # the last chunk yields the first token
    b = sched.build_batch()
    assert (b.num_decodes, b.context_lens, b.q_lens) == (1, [20], [1])
    assert b.slot_mapping == [1 * 16 + 4]
    assert sched.commit(b) == []
    b = sched.build_batch()
    assert b.context_lens == [21]
    assert sched.commit(b) == [7]                     # generated == max_new_tokens
    assert list(sched.free) == [2, 3, 4, 5, 6, 7, 8, 9, 0, 1]


def test_decode_takes_a_page_at_a_boundary():
    sched = S.Scheduler(4, 4, [9, 8, 7, 6])
    sched.add_request(1, 16, 5, 16, 1)                # 16 tokens cached: one full page
    b = sched.build_batch()
    assert b.block_tables[0][:2] == [9, 8] and b.slot_mapping == [8 * 16]
    assert list(sched.free) == [7, 6]


def test_budget_error_when_decodes_exceed_budget():
    sched = S.Scheduler(2, 4, list(range(8)))
    for i in range(3):
        sched.add_request(i, 5, 4, 5, 1)
    with pytest.raises(S.BudgetError):
        sched.build_batch()


def test_no_pages_error_leaves_state_unchanged():
    sched = S.Scheduler(8, 4, [0, 1])
    sched.add_request(1, 16, 5, 16, 1)
    sched.add_request(2, 16, 5, 16, 1)
    with pytest.raises(S.NoPagesError):
        sched.build_batch()
    assert [r.pages for r in sched.running] == [[0], [1]]
    assert list(sched.free) == []


def test_fcfs_head_of_line_blocks_admission():
    sched = S.Scheduler(64, 8, list(range(3)))
    sched.add_request(1, 60, 2)   # needs 4 pages: does not fit
    sched.add_request(2, 10, 2)   # would fit, but may not skip the head
    b = sched.build_batch()
    assert b.req_ids == [] and b.num_tokens == 0


def test_invalid_requests_rejected():
    sched = S.Scheduler(8, 2, list(range(4)))
    with pytest.raises(S.InvalidRequest):
        sched.add_request(1, 30, 4)          # 30 + 4 - 1 > 32 tokens of table
    with pytest.raises(S.InvalidRequest):
        sched.add_request(1, 10, 2, 10, 0)   # prompt done but nothing generated
    with pytest.raises(S.InvalidRequest):
        sched.add_request(1, 10, 2, 10, 2)   # already finished
    sched.add_request(1, 10, 2)
    with pytest.raises(S.InvalidRequest):
        sched.add_request(1, 10, 2)          # duplicate id


def test_commit_requires_the_last_built_batch():
    sched = S.Scheduler(8, 4, list(range(8)))
    sched.add_request(1, 10, 2)
    b = sched.build_batch()
    sched.add_request(2, 10, 2)
    with pytest.raises(S.InvalidRequest):
        sched.commit(b)
