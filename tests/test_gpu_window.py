"""GPU: sliding-window attention through the C ABI against the fp64 oracle.

A window of w keys lets the row at position p see keys p-w+1 .. p (the
sliding-window model variants of "Sarathi-Serve: Chunked Prefills for
Stall-Free LLM Inference", Results and evidence; the rule is the oracle's
reading).  Same bar as the other parity tests; in addition a window that
covers every sequence must reproduce the unwindowed output bit for bit, and
w = 1 must return each row's own V exactly.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.harness import GpuStep
from tests.test_gpu_parity import check_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_prefill_decode_amd import native  # noqa: F401


def run(inst, window, **kw):
    print(f"{inst.name} window={window}", flush=True)
    step = GpuStep(inst, gen_device="cuda", window=window, **kw)
    step.run()
    torch.cuda.synchronize()
    return step


@pytest.mark.parametrize("n,window", [(2, 4096), (2, 700), (4, 4096), (5, 1024), (5, 100)])
def test_workload_parity_with_window(n, window):
    """Mistral-7B shape with its 4096-key window, LLaMA-2-70B / Falcon-180B
    shapes with windows that cut decodes and chunk rows mid-tile."""
    inst = W.make_config(n)
    step = run(inst, window)
    check_parity(inst, step)


@pytest.mark.parametrize("seed", range(12))
def test_small_random_parity_with_window(seed):
    base = W.random_small_instance(seed, max_reqs=8, max_len=160)
    Hq, Hkv, d = [(8, 2, 64), (8, 8, 128), (12, 2, 64), (28, 4, 128), (40, 2, 128), (58, 2, 64)][seed % 6]
    w = [1, 2, 17, 32, 33, 95][seed % 6]
    P = base.num_pages + 64
    inst = W.Instance(base.name, base.seed, base.token_budget, Hq, Hkv, d, base.max_blocks_per_seq, P,
                      np.random.default_rng(seed).permutation(P).astype(np.int32), base.injected, base.waiting)
    step = GpuStep(inst, window=w)
    assert step.T > 0
    step.run()
    torch.cuda.synchronize()
    check_parity(inst, step)


@pytest.mark.parametrize("n", [2, 5])
def test_window_longer_than_every_sequence_is_bit_identical(n):
    inst = W.make_config(n)
    a = run(inst, 0).out.clone()
    b = run(inst, 1 << 20).out.clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_window_of_one_returns_own_value():
    inst = W.make_config(2)
    step = run(inst, 1)
    g = inst.num_q_heads // inst.num_kv_heads
    want = step.v_new_gen.to(step.device).repeat_interleave(g, dim=1)     # [T, Hq, d]
    assert torch.equal(step.out.view(torch.int16), want.view(torch.int16))
