"""GPU: the allocation-free attention entry point (library-owned static
workspace) against sa_hybrid_attn with a caller workspace.

Two calls in a row on one GPU, the second with a smaller batch: the static
array keeps the first call's partials, which the second must not read.  Both
outputs must equal sa_hybrid_attn's bit for bit (same plan, same kernels)."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.harness import GpuStep, load_native_sched

@pytest.fixture
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_prefill_decode_amd import native  # noqa: F401


@pytest.mark.gpu
def test_noalloc_matches_caller_workspace_on_two_calls(need_gpu):
    from chunked_prefill_decode_amd import native as N
    cases = [W.make_config(5, 1024), W.make_config(2)]     # many split partials, then fewer
    steps = []
    for inst in cases:
        print(f"no-alloc: {inst.name}", flush=True)
        step = GpuStep(inst, gen_device="cuda")
        assert 0 < N.sa_hybrid_attn_workspace_size(step.dev) <= N.SA_NOALLOC_WORKSPACE_BYTES
        steps.append(step)
    sizes = [N.sa_hybrid_attn_workspace_size(s.dev) for s in steps]
    assert sizes[1] < sizes[0]
    for step in steps:
        ref = step.run().clone()
        out = torch.empty_like(ref)
        N.sa_hybrid_attn_noalloc(step.q, step.k_cache, step.v_cache, step.dev, step.inst.softmax_scale, out)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), step.inst.name


def test_noalloc_rejects_a_plan_beyond_its_workspace():
    """A plan whose split partials need more than the static array is refused
    on the host, before anything is enqueued or any HIP call is made (the
    planner keeps real plans far below the limit, so the count is raised by
    hand in the batch descriptor)."""
    from chunked_prefill_decode_amd import native as N
    inst = W.make_config(2)
    batch = load_native_sched(inst).build_batch(cap_seqs=len(inst.injected) + len(inst.waiting) + 1)
    Hq, Hkv, d = inst.num_q_heads, inst.num_kv_heads, inst.head_dim
    nbytes = N.sa_batch_upload_size(batch, Hq, Hkv, d)
    buf = np.zeros(nbytes // 4 + 8, np.int32)
    off = (-buf.ctypes.data) % 16 // 4
    dev = N.sa_batch_pack(batch, Hq, Hkv, d, inst.num_pages, buf[off: off + nbytes // 4], 1 << 20)
    per_partial = N.sa_hybrid_attn_workspace_size(dev) // max(dev.num_partials, 1)
    dev.num_partials = N.SA_NOALLOC_WORKSPACE_BYTES // per_partial + 1
    assert N.sa_hybrid_attn_workspace_size(dev) > N.SA_NOALLOC_WORKSPACE_BYTES
    with pytest.raises(N.SarathiError) as e:
        N.sa_hybrid_attn_noalloc(None, None, None, dev, 0.1, None, stream=0)
    assert e.value.status == N.SA_ERR_CAPACITY
