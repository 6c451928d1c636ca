"""GPU: one prompt prefilled unchunked and in chunks through the paged path.

Chunking changes the schedule, not the result ("Sarathi-Serve" pages, the
chunked-prefills mechanism: a chunk attends to its prompt's earlier chunks
through the KV cache): the prompt's output rows must agree between schedules
and with the fp64 oracle, to the same bar as the other parity tests, and the
decodes riding in every chunk's iteration must match the oracle too.
"""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests.harness import ChunkingStudy

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_prefill_decode_amd import native  # noqa: F401


def run(study, its):
    for it in its:
        study.append(it)
        study.attend(it)
    torch.cuda.synchronize()


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 2, 128), (12, 2, 64), (58, 2, 64)])
def test_chunked_equals_unchunked_and_oracle(Hq, Hkv, d):
    L = 650                                            # ragged: not a multiple of any chunk or tile
    study = ChunkingStudy(L, Hq, Hkv, d, decodes=3, dec_ctx=300, seed=77)
    full = study.schedule(L, with_decodes=False)
    run(study, full)
    ref = f64(study.prompt_rows(full))
    want = OA.attend([(0, L)], f64(study.q), [(f64(study.k), f64(study.v))], study.scale)
    err = np.abs(ref - want)
    print(f"unchunked vs oracle: max {err.max():.3e} mean {err.mean():.3e}", flush=True)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
    for C in (128, 200, 512):
        its = study.schedule(C, with_decodes=True)
        run(study, its)
        got = f64(study.prompt_rows(its))
        e1, e2 = np.abs(got - ref), np.abs(got - want)
        print(f"C={C}: vs unchunked max {e1.max():.3e}; vs oracle max {e2.max():.3e} mean {e2.mean():.3e}", flush=True)
        assert e2.max() <= MAX_ABS and e2.mean() <= MEAN_ABS and e1.max() <= MAX_ABS
        # the decodes of the first iteration, against the oracle
        it = its[0]
        dec = f64(it.out[:it.D])
        seqs = [(study.dec_ctx, 1)] * it.D
        kv = [(f64(study.dk[j]), f64(study.dv[j])) for j in range(it.D)]
        wd = OA.attend(seqs, f64(study.dq[:it.D]), kv, study.scale)
        assert np.abs(dec - wd).max() <= MAX_ABS
