"""GPU: the token-batch linear layer (sa_linear, y = x w^T) against the fp64
oracle.

Bar: max |err| <= 2e-2 and mean |err| <= 2e-3 with bf16 inputs, fp32
accumulation and bf16 output -- the outputs are about unit size (weights
N(0, 1/K)), so bf16 rounding of y contributes at most ~2^-9 |y| and fp32
accumulation over K <= 28672 terms far less.  Split-K results must be
bit-identical across repeats whatever the workspace held before, and
identity weights copy x exactly.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import linear as OL

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_prefill_decode_amd import native  # noqa: F401


def run(x, w, M, N, K, ws=None):
    from chunked_prefill_decode_amd import native as Nn
    need = Nn.sa_linear_workspace_size(M, N, K)
    if ws is None:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    Nn.sa_linear(x, w, y, M, N, K, ws)
    torch.cuda.synchronize()
    return y, ws, need


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(tag, got, want):
    err = np.abs(got - want)
    print(f"{tag}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (33, 136, 128), (128, 256, 256), (257, 264, 192), (130, 1000, 640),
                                   (256, 6144, 4096), (300, 2048, 1024), (1024, 512, 3072)])
def test_parity_small_and_ragged(M, N, K):
    print(f"linear M={M} N={N} K={K}", flush=True)
    x = W.normal_bf16((M, K), 11 + M, DEV)
    w = W.linear_weight_bf16(N, K, 12 + N, DEV)
    y, _, _ = run(x, w, M, N, K)
    check(f"M={M} N={N} K={K}", f64(y), OL.linear(f64(x), f64(w)))


@pytest.mark.parametrize("model", sorted(W.LINEAR_LAYERS))
def test_model_projections_sampled_rows(model):
    """Every projection of a layer at full size, at M = 256, 257 and 2048
    token rows; the oracle computes a sample of 32 rows (all columns)."""
    for i, (name, N, K) in enumerate(W.LINEAR_LAYERS[model]):
        w = W.linear_weight_bf16(N, K, 200 + i, DEV)
        w64 = f64(w)
        for M in (256, 257, 2048):
            print(f"{model} {name} M={M} N={N} K={K}", flush=True)
            x = W.normal_bf16((M, K), 100 + i + M, DEV)
            y, _, _ = run(x, w, M, N, K)
            rows = np.linspace(0, M - 1, 32).round().astype(int)
            check(f"{model} {name} M={M}", f64(y[rows]), OL.linear(f64(x[rows]), w64))
            del x, y
        del w, w64


@pytest.mark.parametrize("M,N,K,part_bytes", [
    (1000, 14856, 1024, 0),                                  # 256 x 256 tiles, ragged M and N
    (700, 4104, 512, 0),                                     # 192 x 256 tiles, ragged M and N
    (3000, 28680, 512, 0),                                   # 128 x 288 tiles unsplit, ragged M and N
    (300, 4104, 512, 2 * 33 * 2 * 128 * 256 * 4),            # 128 x 256 tiles, K split 2 ways
    (520, 2056, 4096, 2 * 17 * 7 * 128 * 288 * 4),           # 128 x 288 tiles, K split 7 ways
    (257, 8200, 4096, 1 * 65 * 3 * 128 * 288 * 4),           # 128 x 288 tiles (256 < M <= 288), K split 3 ways
    (300, 2056, 1024, 3 * 17 * 4 * 128 * 128 * 4),           # 128 x 128 tiles, K split 4 ways
    (2100, 8200, 512, 0)])                                   # 128 x 128 tiles unsplit
def test_each_tile_shape_on_ragged_edges(M, N, K, part_bytes):
    """One case per tile shape of sa_linear, each with a partial last tile
    in both M and N; 32 sampled rows, among them the last, against the oracle.
    Where K is split the workspace size pins the shape and the split; the
    unsplit cases are the shapes the tile estimate picks for those sizes,
    which a zero workspace does not tell apart."""
    from chunked_prefill_decode_amd import native as Nn
    print(f"linear M={M} N={N} K={K}", flush=True)
    assert Nn.sa_linear_workspace_size(M, N, K) == part_bytes
    x = W.normal_bf16((M, K), 31 + M, DEV)
    w = W.linear_weight_bf16(N, K, 32 + N, DEV)
    y, _, _ = run(x, w, M, N, K)
    rows = np.linspace(0, M - 1, 32).round().astype(int)
    check(f"M={M} N={N} K={K}", f64(y[rows]), OL.linear(f64(x[rows]), f64(w)))


def test_split_k_is_deterministic_with_a_dirty_workspace():
    M, N, K = 256, 6144, 4096                       # few tiles: K is split
    x = W.normal_bf16((M, K), 1, DEV)
    w = W.linear_weight_bf16(N, K, 2, DEV)
    y1, ws, need = run(x, w, M, N, K)
    assert need > 0
    for fill in (0x7F, 0xFF, 0x00):                 # the workspace needs no initialisation
        ws.fill_(fill)
        y2, ws, _ = run(x, w, M, N, K, ws)
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("M,K", [(64, 512), (256, 4096)])
def test_identity_weight_copies_rows_exactly(M, K):
    x = W.normal_bf16((M, K), 5, DEV)
    w = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    y, _, _ = run(x, w, M, K, K)
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))


def test_matches_oracle_on_budget_sweep():
    """The Falcon-180B share's QKV projection over the token-budget sweep."""
    name, N, K = W.LINEAR_LAYERS["falcon180b-tp4"][0]
    w = W.linear_weight_bf16(N, K, 7, DEV)
    for M in (224, 225, 256, 257, 480, 992, 2016):
        x = W.normal_bf16((M, K), M, DEV)
        y, _, _ = run(x, w, M, N, K)
        rows = np.linspace(0, M - 1, 16).round().astype(int)
        check(f"falcon qkv M={M}", f64(y[rows]), OL.linear(f64(x[rows]), f64(w)))
