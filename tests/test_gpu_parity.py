"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: metadata and KV append bit-exact; attention max |err| <= 2e-2 and mean
|err| <= 2e-3 against the oracle (bf16 inputs, fp32 accumulation, bf16
output).  Invariances: the physical page order and repeated runs give
bit-identical outputs; NaN in unused cache slots changes nothing; closed-form
cases are exact.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests.harness import GpuStep, batch_from_arrays, kv_bit_exact, load_native_sched, oracle_inputs

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_prefill_decode_amd import native  # noqa: F401  (fails loudly if the library is missing)


def report(tag, got, want):
    err = np.abs(got - want)
    print(f"{tag}: rows={got.shape[0]} max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    return err.max(), err.mean()


def check_parity(inst, step):
    """Every row of the step against the oracle; returns (max, mean) abs error."""
    assert step.T > 0
    out = step.out.float().cpu().numpy().astype(np.float64)
    seqs, q, kv, rows = oracle_inputs(inst, step, list(range(step.S)))
    want = OA.attend(seqs, q, kv, inst.softmax_scale, step.window)
    got = out[rows]
    assert len(rows) == step.T
    assert np.isfinite(got).all()
    nd = step.D
    if nd:
        report(f"{inst.name} decode rows", got[:nd], want[:nd])
    if len(rows) > nd:
        report(f"{inst.name} chunk rows", got[nd:], want[nd:])
    mx, mean = report(f"{inst.name} all rows", got, want)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
    return mx, mean


@pytest.mark.parametrize("n", [1, 2, 4])
def test_upload_copies_the_packed_bytes(n):
    """sa_batch_upload from pinned staging (the copy kernel reading it over
    PCIe) and from pageable staging (hipMemcpyAsync) leave the same bytes on
    the device: exactly what the packer wrote into the staging buffer."""
    from chunked_prefill_decode_amd import native as N
    inst = W.make_config(n)
    batch = load_native_sched(inst).build_batch(cap_seqs=len(inst.injected) + len(inst.waiting) + 1)
    Hq, Hkv, d, P = inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages
    nbytes = N.sa_batch_upload_size(batch, Hq, Hkv, d, 0)
    # zero-filled: the packer leaves the padding between 16-byte sections alone
    pinned = torch.zeros(nbytes, dtype=torch.uint8, pin_memory=True)
    pageable = torch.zeros(nbytes, dtype=torch.uint8)
    assert pinned.is_pinned() and not pageable.is_pinned()
    dev_a = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    dev_b = torch.full((nbytes,), 0xCD, dtype=torch.uint8, device="cuda")
    a = N.sa_batch_upload(batch, Hq, Hkv, d, P, pinned, dev_a)
    b = N.sa_batch_upload(batch, Hq, Hkv, d, P, pageable, dev_b)
    torch.cuda.synchronize()
    assert torch.equal(pinned, pageable)
    assert torch.equal(dev_a.cpu(), pinned) and torch.equal(dev_b.cpu(), pinned)
    assert a.num_work_items == b.num_work_items and a.num_combine_groups == b.num_combine_groups
    print(f"{inst.name}: {nbytes} bytes uploaded identically from pinned and pageable staging", flush=True)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_fused_upload_append_matches_the_two_calls(n):
    """sa_batch_upload_append (one kernel: metadata copy + K/V append with the
    slot mapping read from the pinned staging) leaves the caches bit-identical
    to sa_batch_upload + sa_kv_append, the device metadata equal to the
    staging bytes, and the attention over it bit-identical."""
    from chunked_prefill_decode_amd import native as N
    inst = W.make_config(n)
    step = GpuStep(inst, gen_device="cuda")
    Hq, Hkv, d, P = inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages
    kc, vc = step.k_cache.clone(), step.v_cache.clone()
    nbytes = step.staging.numel()
    staging = torch.zeros(nbytes, dtype=torch.uint8, pin_memory=True)
    meta = torch.full((nbytes,), 0xEE, dtype=torch.uint8, device="cuda")
    dev = N.sa_batch_upload_append(step.batch, Hq, Hkv, d, P, staging, meta, step.k_new, step.v_new, kc, vc)
    step.run()
    out = torch.empty_like(step.out)
    N.sa_hybrid_attn(step.q, kc, vc, dev, inst.softmax_scale, out, step.ws)
    torch.cuda.synchronize()
    assert torch.equal(meta.cpu(), staging)
    assert (dev.num_work_items, dev.num_combine_groups, dev.num_partials, dev.plan_flags) == \
        (step.dev.num_work_items, step.dev.num_combine_groups, step.dev.num_partials, step.dev.plan_flags)
    assert torch.equal(kc.view(torch.int16), step.k_cache.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), step.v_cache.view(torch.int16))
    assert torch.equal(out.view(torch.int16), step.out.view(torch.int16))
    print(f"{inst.name}: fused upload + append ({step.T} tokens, {nbytes} bytes) bit-identical", flush=True)


@pytest.mark.parametrize("n", [2, 4])
def test_step_loop_repeats_the_step_bit_for_bit(n):
    """The benchmark's serving loop (each step rebuilt from a copy of the
    scheduler state, packed into a ring of staging / metadata buffers,
    uploaded with the append in one kernel, attended, committed), run past
    two wraps of its ring with the sampled timing events: every step
    leaves the caches and the output bit-identical to one plain step."""
    from chunked_prefill_decode_amd.runner import StepLoop
    inst = W.make_config(n)
    step = GpuStep(inst, gen_device="cuda")
    want = step.run().clone()
    kc, vc = step.k_cache.clone(), step.v_cache.clone()
    steps = 2 * StepLoop.RING + 3
    loop = StepLoop(step, steps)
    for i in range(steps):
        step.out.fill_(0)
        tokens, ev, end = loop.run(i, timing=i % StepLoop.SAMPLE == 0)
        assert tokens == step.T and (ev is not None) == (i % StepLoop.SAMPLE == 0)
        torch.cuda.synchronize()
        assert torch.equal(step.out.view(torch.int16), want.view(torch.int16)), i
    loop = StepLoop(step, steps)                    # pipelined: the host runs ahead, guarded by the ring
    step.out.fill_(0)
    for i in range(steps):
        loop.run(i, timing=i % StepLoop.SAMPLE == 0)
    torch.cuda.synchronize()
    assert torch.equal(step.out.view(torch.int16), want.view(torch.int16))
    assert torch.equal(step.k_cache.view(torch.int16), kc.view(torch.int16))
    assert torch.equal(step.v_cache.view(torch.int16), vc.view(torch.int16))
    print(f"{inst.name}: {steps} loop steps bit-identical to one step", flush=True)


def test_fused_upload_append_refuses_pageable_staging():
    from chunked_prefill_decode_amd import native as N
    inst = W.make_config(1)
    step = GpuStep(inst)
    Hq, Hkv, d, P = inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages
    pageable = torch.zeros(step.staging.numel(), dtype=torch.uint8)
    with pytest.raises(N.SarathiError) as e:
        N.sa_batch_upload_append(step.batch, Hq, Hkv, d, P, pageable, step.meta, step.k_new, step.v_new,
                                 step.k_cache, step.v_cache)
    assert e.value.status == 1 and "pinned" in e.value.message
    torch.cuda.synchronize()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_kv_append_bit_exact(n):
    """The whole cache after history placement and the step's append, bit
    for bit against the oracle, at every workload's full size."""
    inst = W.make_config(n)
    print(f"kv_append bit-exact: {inst.name}", flush=True)
    step = GpuStep(inst, gen_device="cuda" if n > 2 else "cpu")
    step.run()
    torch.cuda.synchronize()
    assert kv_bit_exact(step)


@pytest.mark.parametrize("seed", range(6))
def test_kv_append_bit_exact_small_random(seed):
    inst = W.random_small_instance(seed)
    inst = W.Instance(inst.name, inst.seed, inst.token_budget, 8, 2, 64 if seed % 2 else 128,
                      inst.max_blocks_per_seq, inst.num_pages + 64,
                      np.random.default_rng(seed).permutation(inst.num_pages + 64).astype(np.int32),
                      inst.injected, inst.waiting)
    step = GpuStep(inst, gen_device="cpu")
    assert step.T > 0
    step.run()
    torch.cuda.synchronize()
    assert kv_bit_exact(step)


def test_tiny_parity():
    inst = W.make_config(1)
    step = GpuStep(inst)
    step.run()
    torch.cuda.synchronize()
    check_parity(inst, step)


@pytest.mark.parametrize("seed", range(12))
def test_small_random_parity(seed):
    """Ragged small batches: several chunks, odd offsets, pages shuffled."""
    base = W.random_small_instance(seed, max_reqs=8, max_len=160)
    Hq, Hkv, d = [(8, 2, 64), (8, 8, 128), (12, 2, 64), (28, 4, 128), (40, 2, 128), (58, 2, 64)][seed % 6]
    P = base.num_pages + 64
    inst = W.Instance(base.name, base.seed, base.token_budget, Hq, Hkv, d, base.max_blocks_per_seq, P,
                      np.random.default_rng(seed).permutation(P).astype(np.int32), base.injected, base.waiting)
    step = GpuStep(inst)
    assert step.T > 0
    step.run()
    torch.cuda.synchronize()
    check_parity(inst, step)


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_workload_parity_full_size(n):
    """Every row of the full-size batch (decodes of every plan item kind,
    chunk rows) against the oracle."""
    inst = W.make_config(n)
    print(f"full-size parity: {inst.name}", flush=True)
    step = GpuStep(inst, gen_device="cuda")
    step.run()
    torch.cuda.synchronize()
    check_parity(inst, step)


@pytest.mark.parametrize("seed", [1, 2, 5])
def test_decode_batch_parity(seed):
    """Decode-only batches whose one-round plans fill every slot by cutting
    packs and splitting keys (seeds 1, 5) or split long decodes of a wide
    kv group (seed 2): every row against the oracle."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, d = [(32, 8, 128), (28, 4, 128), (58, 2, 64), (64, 8, 128)][seed % 4]
    nd = int(rng.integers(40, 111))
    inst = W.decode_batch_instance(300 + seed, nd, float(rng.integers(800, 3000)), Hq, Hkv, d, 512)
    print(f"decode batch: seed {seed}, {nd} decodes, heads {Hq}/{Hkv}/{d}", flush=True)
    step = GpuStep(inst, gen_device="cuda")
    step.run()
    torch.cuda.synchronize()
    check_parity(inst, step)


def test_long_context_decodes_parity():
    """Decodes of 100 000 and 65 537 keys beside a prefill chunk: their
    blocks are split 64 ways, the most the merge takes."""
    inst = W.long_context_instance()
    step = GpuStep(inst, gen_device="cuda")
    assert step.dev.num_combine_groups > 0
    step.run()
    torch.cuda.synchronize()
    check_parity(inst, step)


@pytest.mark.parametrize("B", [256, 257, 512, 1024])
def test_budget_sweep_parity(B):
    inst = W.make_config(5, B)
    step = GpuStep(inst, gen_device="cuda")
    step.run()
    torch.cuda.synchronize()
    check_parity(inst, step)


def test_page_permutation_and_repeat_are_bit_identical():
    inst = W.make_config(3)
    a = GpuStep(inst, gen_device="cuda")
    out_a = a.run().clone()
    out_a2 = a.run().clone()
    perm = np.random.default_rng(77).permutation(inst.num_pages).astype(np.int32)
    b = GpuStep(inst, gen_device="cuda", free_pages=perm)
    out_b = b.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_a2.view(torch.int16))
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))


def test_nan_in_unused_slots_changes_nothing():
    inst = W.make_config(2)
    a = GpuStep(inst, gen_device="cuda", fill=1024.0)
    b = GpuStep(inst, gen_device="cuda", fill=float("nan"))
    oa, ob = a.run().clone(), b.run().clone()
    torch.cuda.synchronize()
    assert torch.isfinite(ob.float()).all()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_closed_form_cases_exact():
    """First prompt token returns V0 exactly; constant V rows return that row."""
    from chunked_prefill_decode_amd import native as N
    Hq, Hkv, d, P = 8, 2, 128, 32
    dev = "cuda:0"
    rng = np.random.default_rng(5)
    pages = rng.permutation(P).astype(np.int32)
    # sequence 0: decode, 37 cached keys + its own, all V rows equal per kv head
    # sequence 1: a 20-token chunk starting at position 0
    ctx = [37, 0]
    qn = [1, 20]
    bt = np.full((2, 8), -1, np.int32)
    bt[0, :3] = pages[:3]
    bt[1, :2] = pages[3:5]
    slots_all, rows_k, rows_v = [], [], []
    const = W.normal_bf16((Hkv, d), 1)
    k0 = W.normal_bf16((38, Hkv, d), 2)
    v0 = const.unsqueeze(0).expand(38, Hkv, d).contiguous()
    k1 = W.normal_bf16((20, Hkv, d), 3)
    v1 = W.normal_bf16((20, Hkv, d), 4)
    for s, (k, v) in enumerate([(k0, v0), (k1, v1)]):
        for pos in range(k.shape[0]):
            slots_all.append(int(bt[s, pos // 16]) * 16 + pos % 16)
    kall = torch.cat([k0, k1]).to(dev)
    vall = torch.cat([v0, v1]).to(dev)
    kc = torch.full((P, Hkv, 16, d), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full((P, Hkv, d, 16), float("nan"), dtype=torch.bfloat16, device=dev)
    sl = torch.tensor(slots_all, dtype=torch.int32, device=dev)
    N.sa_kv_append(kall, vall, kc, vc, sl, len(slots_all), Hkv, d, P)
    new_slots = [slots_all[37]] + slots_all[38:58]
    batch = batch_from_arrays(qn, ctx, bt, new_slots, num_decodes=1)
    q = W.normal_bf16((21, Hq, d), 6).to(dev)
    nbytes = N.sa_batch_upload_size(batch, Hq, Hkv, d)
    staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    meta = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    bd = N.sa_batch_upload(batch, Hq, Hkv, d, P, staging, meta)
    ws = torch.zeros(max(N.sa_hybrid_attn_workspace_size(bd), 256), dtype=torch.uint8, device=dev)
    out = torch.empty(21, Hq, d, dtype=torch.bfloat16, device=dev)
    N.sa_hybrid_attn(q, kc, vc, bd, 1 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    o = out.cpu()
    g = Hq // Hkv
    for h in range(Hq):
        assert torch.equal(o[0, h].view(torch.int16), const[h // g].view(torch.int16))      # constant V
        assert torch.equal(o[1, h].view(torch.int16), v1[0, h // g].view(torch.int16))      # one visible key
    assert torch.isfinite(o.float()).all()


def test_empty_batch_is_a_no_op():
    from chunked_prefill_decode_amd import native as N
    batch = batch_from_arrays([], [], np.zeros((0, 4), np.int32), [], num_decodes=0)
    nbytes = N.sa_batch_upload_size(batch, 4, 1, 64)
    staging = torch.empty(max(nbytes, 16), dtype=torch.uint8, pin_memory=True)
    meta = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda:0")
    bd = N.sa_batch_upload(batch, 4, 1, 64, 4, staging, meta)
    assert bd.num_work_items == 0
    N.sa_hybrid_attn(None, None, None, bd, 0.125, None, None)
    torch.cuda.synchronize()


@pytest.mark.parametrize("n", [2, 3])
def test_streamed_and_cached_kv_loads_are_bit_identical(n):
    """plan_flags only picks the cache policy of the decode path's K/V loads
    (non-temporal or cached); the arithmetic is the same, so the outputs must
    be identical bit for bit either way."""
    from chunked_prefill_decode_amd import native as N
    inst = W.make_config(n)
    step = GpuStep(inst, gen_device="cuda")
    outs = []
    for flags in (0, N.SA_PLAN_STREAM_KV):
        step.dev.plan_flags = flags
        outs.append(step.run().clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("lead", [32, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_scores_far_above_the_first_tile_stay_exact(d, lead):
    """Keys after the first `lead` keys score hundreds of log2 units above
    them, so a walk that keeps the running max of its first tiles overflows;
    the kernel must notice and produce the oracle's result anyway (the softmax
    here is nearly one-hot, which bf16 carries well).  lead = 256 puts the
    rise past the first group of tiles of the chunk walk at d = 64."""
    from chunked_prefill_decode_amd import native as N
    Hq, Hkv, P, L, ctx = 8, 2, 64, 300, 100
    dev = "cuda:0"
    pages = np.random.default_rng(11).permutation(P).astype(np.int32)
    npg = -(-(ctx + L) // 16)
    bt = np.full((1, npg), -1, np.int32)
    bt[0] = pages[:npg]
    k = W.normal_bf16((ctx + L, Hkv, d), 21).float()
    k[:lead] *= 0.01                               # the leading keys: scores near 0
    k[lead:] *= 6.0
    k = k.to(torch.bfloat16)
    v = W.normal_bf16((ctx + L, Hkv, d), 22)
    q = (W.normal_bf16((L, Hq, d), 23).float() * 6.0).to(torch.bfloat16)
    slots = [int(bt[0, p // 16]) * 16 + p % 16 for p in range(ctx + L)]
    kc = torch.full((P, Hkv, 16, d), 1024.0, dtype=torch.bfloat16, device=dev)
    vc = torch.full((P, Hkv, d, 16), 1024.0, dtype=torch.bfloat16, device=dev)
    N.sa_kv_append(k.to(dev), v.to(dev), kc, vc, torch.tensor(slots, dtype=torch.int32, device=dev), ctx + L, Hkv,
                   d, P)
    batch = batch_from_arrays([L], [ctx], bt, slots[ctx:], num_decodes=0)
    nbytes = N.sa_batch_upload_size(batch, Hq, Hkv, d)
    staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    meta = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    bd = N.sa_batch_upload(batch, Hq, Hkv, d, P, staging, meta)
    ws = torch.full((max(N.sa_hybrid_attn_workspace_size(bd), 256),), 0xFF, dtype=torch.uint8, device=dev)
    out = torch.empty(L, Hq, d, dtype=torch.bfloat16, device=dev)
    scale = 1 / math.sqrt(d)
    N.sa_hybrid_attn(q.to(dev), kc, vc, bd, scale, out, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    want = OA.attend([(ctx, L)], f64(q), [(f64(k), f64(v))], scale)
    assert np.isfinite(got).all()
    mx, mean = report(f"large scores d={d} lead={lead}", got, want)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
