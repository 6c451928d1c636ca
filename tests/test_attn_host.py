"""sa_kv_append, sa_hybrid_attn and sa_hybrid_attn_noalloc on the host: argument
checks and workspace sizing.  Every call here fails or returns before any HIP
call, so the addresses are stand-ins that nothing dereferences."""
import math

import pytest

N = pytest.importorskip("chunked_prefill_decode_amd.native")

A = 1 << 20                     # a 16-byte-aligned stand-in address


def dev(d=128, hq=64, hkv=8, items=4, partials=8, window=0):
    b = N.sa_batch_dev()
    b.cu_seqlens_q = b.context_lens = b.block_table_offsets = b.block_tables = A
    b.work = b.combine = A
    b.num_seqs, b.num_decodes, b.num_tokens, b.bt_stride = 4, 4, 4, 8
    b.num_q_heads, b.num_kv_heads, b.head_dim, b.num_pages = hq, hkv, d, 64
    b.num_work_items, b.num_combine_groups, b.num_partials = items, 1, partials
    b.sliding_window = window
    return b


def attn(b, scale=0.125, q=A, k=A, v=A, out=A, ws=A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = N.sa_hybrid_attn_workspace_size(b)
    with pytest.raises(N.SarathiError) as e:
        N.sa_hybrid_attn(q, k, v, b, scale, out, ws, ws_bytes, stream=0)
    return e.value.status


@pytest.mark.parametrize("d", [64, 128])
def test_workspace_size_is_one_fp32_row_per_partial_and_column(d):
    # per partial: 32 query columns x (running max, running sum, d output sums) in fp32
    assert N.sa_hybrid_attn_workspace_size(dev(d=d, partials=0)) == 0
    assert N.sa_hybrid_attn_workspace_size(dev(d=d, partials=8)) == 8 * 32 * (2 + d) * 4


@pytest.mark.parametrize("d", [0, 32, 96, 256])
def test_attn_head_dims_other_than_64_and_128_are_unsupported(d):
    assert attn(dev(d=d), ws_bytes=1 << 30) == N.SA_ERR_UNSUPPORTED


@pytest.mark.parametrize("hq,hkv", [(0, 8), (64, 0), (64, 7), (-8, 8)])
def test_attn_heads_must_group_evenly(hq, hkv):
    assert attn(dev(hq=hq, hkv=hkv)) == N.SA_ERR_INVALID_ARG


def test_attn_empty_plan_is_a_no_op():
    N.sa_hybrid_attn(0, 0, 0, dev(items=0), 0.125, 0, 0, 0, stream=0)


@pytest.mark.parametrize("which", ["q", "k", "v", "out"])
def test_attn_null_and_misaligned_tensors(which):
    assert attn(dev(), **{which: 0}) == N.SA_ERR_INVALID_ARG
    assert attn(dev(), **{which: A + 8}) == N.SA_ERR_INVALID_ARG


@pytest.mark.parametrize("field", ["work", "cu_seqlens_q", "block_table_offsets"])
def test_attn_null_plan_arrays(field):
    b = dev()
    setattr(b, field, 0)
    assert attn(b) == N.SA_ERR_INVALID_ARG


def test_attn_workspace_too_small_or_missing():
    b = dev(partials=8)
    need = N.sa_hybrid_attn_workspace_size(b)
    assert attn(b, ws_bytes=need - 1) == N.SA_ERR_CAPACITY
    assert attn(b, ws=0, ws_bytes=need) == N.SA_ERR_CAPACITY


def test_attn_negative_window():
    assert attn(dev(window=-1)) == N.SA_ERR_INVALID_ARG


@pytest.mark.parametrize("scale", [0.0, -0.125, math.nan, math.inf])
def test_attn_scale_must_be_positive_and_finite(scale):
    assert attn(dev(), scale=scale) == N.SA_ERR_INVALID_ARG


def test_noalloc_checks_its_static_workspace_limit():
    with pytest.raises(N.SarathiError) as e:      # 2^20 partials x 32 x 130 x 4 B = 17 GB > 64 MiB
        N.sa_hybrid_attn_noalloc(A, A, A, dev(partials=1 << 20), 0.125, A, stream=0)
    assert e.value.status == N.SA_ERR_CAPACITY
    with pytest.raises(N.SarathiError) as e:
        N.sa_hybrid_attn_noalloc(A, A, A, dev(partials=-1), 0.125, A, stream=0)
    assert e.value.status == N.SA_ERR_INVALID_ARG
    N.sa_hybrid_attn_noalloc(0, 0, 0, dev(items=0), 0.125, 0, stream=0)


def append(T=4, hkv=8, d=128, pages=64, k_new=A, v_new=A, k_cache=A, v_cache=A, slots=A):
    with pytest.raises(N.SarathiError) as e:
        N.sa_kv_append(k_new, v_new, k_cache, v_cache, slots, T, hkv, d, pages, stream=0)
    return e.value.status


@pytest.mark.parametrize("kw", [dict(T=-1), dict(hkv=0), dict(pages=0)])
def test_append_bad_sizes(kw):
    assert append(**kw) == N.SA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(hkv=70000)])
def test_append_unsupported_shapes(kw):
    assert append(**kw) == N.SA_ERR_UNSUPPORTED


def test_append_no_tokens_is_a_no_op():
    N.sa_kv_append(0, 0, 0, 0, 0, 0, 8, 128, 64, stream=0)


@pytest.mark.parametrize("which", ["k_new", "v_new", "k_cache", "v_cache"])
def test_append_null_and_misaligned_tensors(which):
    assert append(**{which: 0}) == N.SA_ERR_INVALID_ARG
    assert append(**{which: A + 2}) == N.SA_ERR_INVALID_ARG


def test_append_null_slot_mapping():
    assert append(slots=0) == N.SA_ERR_INVALID_ARG
