"""GPU: a 40-iteration stall-free schedule through the whole path on one
persistent paged cache.

The LLaMA2-70B-shaped state (64 q heads, 8 kv heads, d 128, B = 1536: 256
running decodes, one prompt mid-prefill, one waiting) takes Poisson(0.5)
arrivals per iteration (sharegpt-like lengths, seed 2004).  Every iteration
runs sa_build_batch -> sa_batch_upload -> sa_kv_append -> sa_hybrid_attn ->
sa_sched_commit, the way the serving iteration of "Sarathi-Serve：以
chunked-prefills 与 stall-free batching 驯服 LLM 推理的吞吐—延迟权衡" (核心机制-2:
build the batch, run it, drop finished requests, next iteration) and the
request state machine of "In-flight Batching" (调度状态机) describe it; pages
freed by finished requests are handed out again with their stale contents.

Checked against the oracle, mirrored step by step on the CPU:
  * metadata bit-exact every iteration (oracle/scheduler.py), finished ids
    equal at every commit;
  * the whole KV cache bit-exact every iteration: at iteration 0 all of it
    against oracle/kvcache.py's after-image (fill + history + the step's
    rows); from then on by induction -- the pages that differ from the
    previous (verified) cache must be among the pages the oracle's slot
    mapping touches, and those pages must equal append_expected applied to
    their previous contents;
  * attention, every row, at iterations 0, 9, 19, 29 and 39, against the
    fp64 oracle over each request's contiguous rows (max abs <= 2e-2, mean
    abs <= 2e-3).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import inputs as OI
from oracle import kvcache as OK
from oracle import scheduler as OS
from tests.harness import ScheduleRun, bf16_bits, expected_cache_bits, load_oracle_sched, slots_view
from tests.test_native_sched import same_batch

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3
ITERS = 40
CHECK_ATTENTION = (0, 9, 19, 29, 39)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_prefill_decode_amd import native  # noqa: F401


def page_images(k_cache, v_cache, pages):
    """Bits of the given physical pages as logical slots [len(pages) * 16, Hkv, d]."""
    idx = torch.from_numpy(pages).to(k_cache.device)
    k, v = slots_view(k_cache[idx], v_cache[idx])
    return bf16_bits(k), bf16_bits(v)


@pytest.mark.timeout(900)
def test_forty_iteration_schedule_through_the_whole_path():
    inst = W.make_config(4)
    arrivals = W.poisson_arrivals(ITERS, 5000)
    run = ScheduleRun(inst, arrivals, gen_device="cuda")
    osched = load_oracle_sched(inst)
    P, Hkv, d = inst.num_pages, inst.num_kv_heads, inst.head_dim
    rows_of = {}            # request id -> its cached (k, v) rows on the CPU, in position order
    snap = None             # verified cache of the previous iteration
    errors = []
    for it in range(ITERS):
        for r in arrivals[it]:
            osched.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
        x = run.iteration()
        ob = osched.build_batch()
        same_batch(x.batch, ob)
        assert sum(ob.q_lens) <= inst.token_budget
        torch.cuda.synchronize()
        k_new, v_new = x.k_new_gen.cpu(), x.v_new_gen.cpu()

        if it == 0:
            assert set(run.hist) == {r.req_id for r in inst.injected if r.cached_tokens > 0}
            rows_of = {rid: [(k.cpu(), v.cpu())] for rid, (k, v) in run.hist.items()}
            hslots, hk, hv = [], [], []
            for rid, ctx, bt in zip(ob.req_ids, ob.context_lens, ob.block_tables):
                if ctx:
                    hslots += OS.slots_of(bt, range(ctx))
                    hk.append(rows_of[rid][0][0])
                    hv.append(rows_of[rid][0][1])
            writes = [(hslots, torch.cat(hk), torch.cat(hv)), (ob.slot_mapping, k_new, v_new)]
            ke, ve = expected_cache_bits(run.fill, P, Hkv, d, writes)
            kg, vg = slots_view(run.k_cache, run.v_cache)
            assert np.array_equal(bf16_bits(kg), ke), "iteration 0: K cache differs from the oracle"
            del ke, kg
            assert np.array_equal(bf16_bits(vg), ve), "iteration 0: V cache differs from the oracle"
            del ve, vg
            snap = (run.k_cache.clone(), run.v_cache.clone())
        else:
            slots = np.asarray(ob.slot_mapping, np.int64)
            pages = np.unique(slots // 16)
            diff = (run.k_cache.view(torch.int16) != snap[0].view(torch.int16)).view(P, -1).any(dim=1)
            diff |= (run.v_cache.view(torch.int16) != snap[1].view(torch.int16)).view(P, -1).any(dim=1)
            changed = torch.nonzero(diff).flatten().cpu().numpy()
            assert np.isin(changed, pages).all(), f"iteration {it}: pages outside the slot mapping changed"
            where = {int(p): i for i, p in enumerate(pages)}
            local = [where[int(s) // 16] * 16 + int(s) % 16 for s in slots]
            kb, vb = page_images(snap[0], snap[1], pages)
            ka, va = page_images(run.k_cache, run.v_cache, pages)
            assert np.array_equal(ka, OK.append_expected(kb, bf16_bits(k_new), local)), f"iteration {it}: K"
            assert np.array_equal(va, OK.append_expected(vb, bf16_bits(v_new), local)), f"iteration {it}: V"
            snap[0].copy_(run.k_cache)
            snap[1].copy_(run.v_cache)

        if it in CHECK_ATTENTION:
            seqs, q, kv, rows = OI.attention_inputs(ob, x.q_gen, k_new, v_new, rows_of)
            want = OA.attend(seqs, q, kv, inst.softmax_scale)
            got = x.out.float().cpu().numpy().astype(np.float64)[rows]
            assert len(rows) == x.T and np.isfinite(got).all()
            err = np.abs(got - want)
            nd = ob.num_decodes
            errors.append((it, err.max(), err.mean()))
            print(f"iteration {it}: T={x.T} decodes={nd} chunks={len(ob.req_ids) - nd} "
                  f"max_abs={err.max():.3e} mean_abs={err.mean():.3e} "
                  f"(decode rows max {err[:nd].max() if nd else 0:.3e}, "
                  f"chunk rows max {err[nd:].max() if x.T > nd else 0:.3e})", flush=True)
            assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS

        cu = ob.cu_seqlens_q
        for s, rid in enumerate(ob.req_ids):
            rows_of.setdefault(rid, []).append((k_new[cu[s]:cu[s + 1]], v_new[cu[s]:cu[s + 1]]))
        fin = run.commit(x)
        assert fin == osched.commit(ob)
        for rid in fin:
            rows_of.pop(rid, None)
        print(f"iteration {it}: T={x.T} S={len(ob.req_ids)} decodes={ob.num_decodes} finished={len(fin)} "
              f"kv bit-exact", flush=True)
    assert len(errors) == len(CHECK_ATTENTION)
