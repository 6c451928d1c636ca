"""The C++ batch builder (through the C ABI) against the oracle, bit for bit.

Runs on the CPU: the scheduler is host code of libsarathi_attn and makes no
HIP call.  Covers the five workloads and the budget sweep, thousands of
random schedules with arrivals and commits, and every error path forced from
the host (state unchanged afterwards)."""
import numpy as np
import pytest

import workloads as W
from oracle import scheduler as OS
from tests.harness import batch_from_arrays, load_native_sched, load_oracle_sched

N = pytest.importorskip("chunked_prefill_decode_amd.native")


def same_batch(nb, ob):
    v = nb.view()
    assert v["req_ids"] == ob.req_ids
    assert v["cu_seqlens_q"] == ob.cu_seqlens_q
    assert v["context_lens"] == ob.context_lens
    assert v["block_tables"] == ob.block_tables
    assert v["slot_mapping"] == ob.slot_mapping
    assert v["num_decodes"] == ob.num_decodes
    assert nb.c.num_prefill_chunks == len(ob.req_ids) - ob.num_decodes
    assert nb.c.max_kv_len == max([c + q for c, q in zip(ob.context_lens, ob.q_lens)] or [0])


@pytest.mark.parametrize("n,B", [(1, None), (2, None), (3, None), (4, None), (5, None)]
                         + [(5, b) for b in W.SWEEP_BUDGETS + W.SWEEP_DIAGNOSTIC])
def test_workload_batches_bit_exact(n, B):
    inst = W.make_config(n, B)
    ns, os_ = load_native_sched(inst), load_oracle_sched(inst)
    nb = ns.build_batch(cap_seqs=400)
    ob = os_.build_batch()
    same_batch(nb, ob)
    assert ns.commit(nb) == os_.commit(ob)
    assert ns.stats() == (len(os_.running), len(os_.waiting), len(os_.free))


def history_slots_oracle(ob):
    out = []
    for bt, ctx in zip(ob.block_tables, ob.context_lens):
        out += OS.slots_of(bt, range(ctx))
    return out


@pytest.mark.parametrize("n", [1, 2, 3])
def test_history_slots(n):
    inst = W.make_config(n)
    nb = load_native_sched(inst).build_batch(cap_seqs=400)
    ob = load_oracle_sched(inst).build_batch()
    assert N.sa_history_slots(nb).tolist() == history_slots_oracle(ob)


def run_trace(inst, iters, arrivals, clamp_len=None):
    ns, os_ = load_native_sched(inst), load_oracle_sched(inst)
    steps = 0
    for it in range(iters):
        for r in arrivals[it]:
            L, O = r.prompt_len, r.max_new_tokens
            if clamp_len:
                L = min(L, clamp_len)
                O = min(O, inst.max_blocks_per_seq * 16 - L + 1)
            ns.add_request(r.req_id, L, O)
            os_.add_request(r.req_id, L, O)
        try:
            ob = os_.build_batch()
        except OS.BudgetError:
            with pytest.raises(N.SarathiError) as e:
                ns.build_batch(cap_seqs=512)
            assert e.value.status == N.SA_ERR_BUDGET
            break
        except OS.NoPagesError:
            with pytest.raises(N.SarathiError) as e:
                ns.build_batch(cap_seqs=512)
            assert e.value.status == N.SA_ERR_NO_PAGES
            break
        nb = ns.build_batch(cap_seqs=512, cap_tokens=inst.token_budget)
        same_batch(nb, ob)
        assert ns.commit(nb) == os_.commit(ob)
        assert ns.stats() == (len(os_.running), len(os_.waiting), len(os_.free))
        steps += 1
    return steps


@pytest.mark.parametrize("seed", range(300))
def test_random_schedules_bit_exact(seed):
    inst = W.random_small_instance(seed)
    try:
        load_oracle_sched(inst)
    except OS.NoPagesError:
        with pytest.raises(N.SarathiError) as e:
            load_native_sched(inst)
        assert e.value.status == N.SA_ERR_NO_PAGES
        return
    run_trace(inst, 40, W.poisson_arrivals(40, 10_000, seed=seed, rate=0.7), clamp_len=40)


def test_forty_iteration_trace_large_workload():
    """The LLaMA2-70B-shaped state driven by Poisson arrivals for 40 iterations."""
    inst = W.make_config(4)
    arrivals = W.poisson_arrivals(40, 5000)
    assert run_trace(inst, 40, arrivals) == 40


# ---------------------------------------------------------------- errors ---
def test_budget_error():
    s = N.Scheduler(2, 4, np.arange(8))
    for i in range(3):
        s.add_request(i, 5, 4, 5, 1)
    with pytest.raises(N.SarathiError) as e:
        s.build_batch()
    assert e.value.status == N.SA_ERR_BUDGET


def test_no_pages_is_transactional():
    s = N.Scheduler(8, 4, np.array([0, 1], np.int32))
    s.add_request(1, 16, 5, 16, 1)
    s.add_request(2, 16, 5, 16, 1)
    with pytest.raises(N.SarathiError) as e:
        s.build_batch()
    assert e.value.status == N.SA_ERR_NO_PAGES
    assert s.stats() == (2, 0, 0)
    with pytest.raises(N.SarathiError) as e:
        s.add_request(3, 16, 5, 16, 1)          # injection needing a page
    assert e.value.status == N.SA_ERR_NO_PAGES
    assert s.stats() == (2, 0, 0)


def test_capacity_reports_required_sizes():
    inst = W.make_config(2)
    s = load_native_sched(inst)
    b = N.HostBatch(10, 256, inst.max_blocks_per_seq)
    with pytest.raises(N.SarathiError) as e:
        N.sa_build_batch(s.h, b)
    assert e.value.status == N.SA_ERR_CAPACITY
    assert (b.c.num_seqs, b.c.num_tokens) == (65, 256)
    nb = s.build_batch(cap_seqs=65)             # state untouched: a full-size build works
    same_batch(nb, load_oracle_sched(inst).build_batch())


def test_invalid_requests():
    s = N.Scheduler(8, 2, np.arange(4))
    bad = [(1, 30, 4, 0, 0), (1, 10, 2, 10, 0), (1, 10, 2, 10, 2), (1, 0, 2, 0, 0), (1, 5, 0, 0, 0), (1, 10, 2, 11, 0)]
    for args in bad:
        with pytest.raises(N.SarathiError) as e:
            s.add_request(*args)
        assert e.value.status == N.SA_ERR_INVALID_ARG
    s.add_request(1, 10, 2)
    with pytest.raises(N.SarathiError) as e:
        s.add_request(1, 10, 2)
    assert e.value.status == N.SA_ERR_INVALID_ARG


def test_create_rejects_bad_pool_and_page_size():
    with pytest.raises(N.SarathiError) as e:
        N.sa_sched_create(8, 4, np.array([0, 0, 1], np.int32))
    assert e.value.status == N.SA_ERR_INVALID_ARG
    with pytest.raises(N.SarathiError) as e:
        N.sa_sched_create(8, 4, np.arange(4), page_size=32)
    assert e.value.status == N.SA_ERR_UNSUPPORTED
    with pytest.raises(N.SarathiError) as e:
        N.sa_sched_create(0, 4, np.arange(4))
    assert e.value.status == N.SA_ERR_INVALID_ARG


def test_commit_of_stale_batch_is_state_error():
    s = N.Scheduler(8, 4, np.arange(8))
    s.add_request(1, 10, 2)
    b = s.build_batch()
    s.add_request(2, 10, 2)
    with pytest.raises(N.SarathiError) as e:
        s.commit(b)
    assert e.value.status == N.SA_ERR_STATE
    b2 = s.build_batch()
    s.commit(b2)
    with pytest.raises(N.SarathiError) as e:
        s.commit(b2)                             # already committed
    assert e.value.status == N.SA_ERR_STATE


def test_rebuild_before_commit_gives_the_same_batch():
    inst = W.make_config(4)
    s = load_native_sched(inst)
    a = s.build_batch(cap_seqs=300).view()
    b = s.build_batch(cap_seqs=300).view()
    assert a == b


def test_clone_is_independent():
    inst = W.make_config(2)
    s = load_native_sched(inst)
    before = s.stats()
    c = s.clone()
    b = s.build_batch(cap_seqs=100)
    s.commit(b)
    assert c.stats() == before                  # the clone saw none of it
    bc = c.build_batch(cap_seqs=100)
    same_batch(bc, load_oracle_sched(inst).build_batch())
    o = load_oracle_sched(inst)                 # the original moved on to the second batch
    o.commit(o.build_batch())
    same_batch(s.build_batch(cap_seqs=100), o.build_batch())


def test_upload_size_checks_shapes():
    inst = W.make_config(1)
    b = load_native_sched(inst).build_batch(cap_seqs=8)
    assert N.sa_batch_upload_size(b, 4, 1, 64) > 0
    with pytest.raises(N.SarathiError) as e:
        N.sa_batch_upload_size(b, 4, 1, 96)
    assert e.value.status == N.SA_ERR_UNSUPPORTED
    with pytest.raises(N.SarathiError) as e:
        N.sa_batch_upload_size(b, 6, 4, 64)
    assert e.value.status == N.SA_ERR_INVALID_ARG
    bad = batch_from_arrays([2, 1], [3, 4], np.zeros((2, 8), np.int32), [0, 1, 2], num_decodes=1)
    with pytest.raises(N.SarathiError) as e:
        N.sa_batch_upload_size(bad, 4, 1, 64)     # a decode with two query rows
    assert e.value.status == N.SA_ERR_INVALID_ARG
