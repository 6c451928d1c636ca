"""GPU parity over a randomised sweep of small hybrid batches: head shapes
from MHA to 96/4 GQA (d 64 and 128), token budgets from 32 to 1024 (tile
multiples and ragged), sliding windows from 1 key to 500, prompts and decodes
up to 3000 tokens, pages shuffled.  Every row is checked against the fp64
oracle to the same bar as the other parity tests."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests.harness import GpuStep, load_oracle_sched, oracle_inputs

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3
SHAPES = [(8, 2, 64), (8, 8, 128), (12, 2, 64), (28, 4, 128), (40, 2, 128), (58, 2, 64), (32, 8, 128),
          (56, 8, 128), (64, 8, 128), (4, 1, 64), (16, 1, 128), (48, 1, 64), (96, 4, 128), (7, 7, 64)]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_prefill_decode_amd import native  # noqa: F401


def instance(seed):
    """The seed's random batch; a draw whose first batch would be empty (no
    request fits) is replaced by the next draw, so every case has work."""
    for attempt in range(50):
        rng = np.random.default_rng(10_000 + seed + 100_000 * attempt)
        max_len = int(rng.choice([96, 400, 1200, 3000]))
        base = W.random_small_instance(seed + 100_000 * attempt, max_reqs=int(rng.integers(1, 12)), max_len=max_len)
        Hq, Hkv, d = SHAPES[seed % len(SHAPES)]
        B = int(rng.choice([base.token_budget, 32, 64, 257, 512, 1024]))
        P = base.num_pages + 64
        inst = W.Instance(base.name, base.seed, B, Hq, Hkv, d, base.max_blocks_per_seq, P,
                          rng.permutation(P).astype(np.int32), base.injected, base.waiting)
        window = int(rng.choice([0, 0, 0, 1, 17, 64, 100, 500]))
        if load_oracle_sched(inst).build_batch().num_tokens > 0:
            return inst, window
    raise AssertionError("no non-empty draw")


@pytest.mark.parametrize("seed", range(0, 84, 3))
def test_random_sweep_parity(seed):
    inst, window = instance(seed)
    step = GpuStep(inst, window=window)
    assert step.T > 0
    step.run()
    torch.cuda.synchronize()
    out = step.out.float().cpu().numpy().astype(np.float64)
    seqs, q64, kv, rows = oracle_inputs(inst, step, list(range(step.S)))
    want = OA.attend(seqs, q64, kv, inst.softmax_scale, window)
    got = out[rows]
    err = np.abs(got - want)
    print(f"seed {seed} Hq/Hkv/d {inst.num_q_heads}/{inst.num_kv_heads}/{inst.head_dim} B {inst.token_budget} "
          f"window {window} T {step.T}: max {err.max():.2e} mean {err.mean():.2e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
