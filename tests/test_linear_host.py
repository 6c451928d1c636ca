"""sa_linear on the host: argument checks and workspace sizing (no kernel is
launched: every call here fails or returns before the launch)."""
import pytest

N = pytest.importorskip("chunked_prefill_decode_amd.native")


def test_ragged_budgets_take_the_288_row_tiles():
    """Just past a multiple of 256 token rows, the 288-row token tiles cover
    the extra rows in the same tile (no second, nearly empty token tile)."""
    assert N.sa_linear_workspace_size(257, 14848, 14848) == 1 * 116 * 2 * 128 * 288 * 4
    assert N.sa_linear_workspace_size(288, 14848, 14848) == 1 * 116 * 2 * 128 * 288 * 4
    assert N.sa_linear_workspace_size(257, 28672, 4096) == 0        # 224 tiles fill the chip unsplit
    assert N.sa_linear_workspace_size(256, 14848, 14848) == 1 * 116 * 2 * 128 * 256 * 4
    assert N.sa_linear_workspace_size(2049, 14848, 14848) == 0      # large M: enough tiles unsplit
    # 1025 tokens: four 288-row tiles (not five of 256) x 32 weight tiles, K split in two
    assert N.sa_linear_workspace_size(1025, 4096, 14336) == 4 * 32 * 2 * 128 * 288 * 4


def test_workspace_size():
    assert N.sa_linear_workspace_size(0, 128, 64) == 0
    big = N.sa_linear_workspace_size(4096, 8192, 4096)        # enough tiles: no split, no workspace
    assert big == 0
    small = N.sa_linear_workspace_size(256, 6144, 4096)       # few tiles: K is split
    assert small >= 2 * 256 * 6144 * 4                       # at least two fp32 partial products


@pytest.mark.parametrize("M,Nn,K,status", [(4, 128, 100, "SA_ERR_UNSUPPORTED"), (4, 130, 64, "SA_ERR_UNSUPPORTED"),
                                           (-1, 128, 64, "SA_ERR_INVALID_ARG"), (4, 0, 64, "SA_ERR_INVALID_ARG")])
def test_bad_shapes(M, Nn, K, status):
    with pytest.raises(N.SarathiError) as e:
        N.sa_linear(16, 16, 16, M, Nn, K, stream=0)
    assert e.value.status == getattr(N, status)


def test_null_and_misaligned_pointers():
    with pytest.raises(N.SarathiError) as e:
        N.sa_linear(0, 16, 16, 4, 128, 64, stream=0)
    assert e.value.status == N.SA_ERR_INVALID_ARG
    with pytest.raises(N.SarathiError) as e:
        N.sa_linear(8, 16, 16, 4, 128, 64, stream=0)
    assert e.value.status == N.SA_ERR_INVALID_ARG


def test_workspace_too_small():
    need = N.sa_linear_workspace_size(256, 6144, 4096)
    with pytest.raises(N.SarathiError) as e:
        N.sa_linear(1 << 20, 1 << 20, 1 << 20, 256, 6144, 4096, workspace=1 << 20, workspace_bytes=need - 1, stream=0)
    assert e.value.status == N.SA_ERR_CAPACITY


def test_empty_batch_is_a_no_op():
    N.sa_linear(0, 0, 0, 0, 128, 64, stream=0)
