"""The attention work plan, checked on the host (no GPU): sa_batch_pack's
output is decoded and every column block must have each of its visible keys
covered exactly once.

Column blocks: a decode's q heads of one kv head (split into 16- or 32-wide
blocks) see keys [0, ctx + 1); chunk column block i (row block i / g, q head
i % g) sees keys [0, ctx + row0 + nrows).  A block is covered either by items
whose key ranges partition that interval (split pieces start on 32-key tile
boundaries and share one combine group), or -- whole decodes only -- by
exactly one entry of a packed decode item whose waves form a consecutive run.
With a sliding window w the interval starts instead at the 32-key tile of
the first key the block's earliest row sees (p - w + 1): no earlier tile is
walked, and no visible key is skipped.
"""
import numpy as np
import pytest

import workloads as W
from chunked_prefill_decode_amd import native as N
from tests.harness import batch_from_arrays, load_native_sched

ITEM, GROUP = 12, 8
DECODE, CHUNK, PACK = 0, 1, 2
DEV = 1 << 20                      # any 16-byte aligned address: never touched
SLOTS = 512


def build(inst):
    return load_native_sched(inst).build_batch(cap_seqs=len(inst.injected) + len(inst.waiting) + 1)


def pack(batch, Hq, Hkv, d, num_pages, window=0):
    nbytes = N.sa_batch_upload_size(batch, Hq, Hkv, d, window)
    buf = np.zeros(max(nbytes, 16) // 4 + 8, np.int32)
    off = (-buf.ctypes.data) % 16 // 4
    staging = buf[off: off + max(nbytes, 16) // 4]
    dev = N.sa_batch_pack(batch, Hq, Hkv, d, num_pages, staging, DEV, window)
    assert dev.sliding_window == window
    words = lambda p: (p - DEV) // 4 if p else 0
    items = staging[words(dev.work): words(dev.work) + dev.num_work_items * ITEM].reshape(-1, ITEM)
    groups = staging[words(dev.combine): words(dev.combine) + dev.num_combine_groups * GROUP].reshape(-1, GROUP)
    return dev, items.copy(), groups.copy()


def walk_start(p, window):
    return max(0, p - window + 1) // 32 * 32 if window else 0


def check_plan(batch, Hq, Hkv, d, num_pages, window=0):
    dev, items, groups = pack(batch, Hq, Hkv, d, num_pages, window)
    v = batch.view()
    cu, ctx = v["cu_seqlens_q"], v["context_lens"]
    S, D = len(ctx), batch.num_decodes
    g = Hq // Hkv
    dec_cols = 16 if g <= 16 else 32
    per_item = 8 if d == 64 else 4
    assert dev.num_work_items == len(items)
    cover = {}                                  # block -> list of (k0, k1, split, group)

    def add(key, k0, k1, split, grp):
        cover.setdefault(key, []).append((k0, k1, split, grp))

    for it in items:
        kind = it[0]
        if kind == DECODE:
            s, kh, head0, nh, row0, nrows, k0, k1, split, g0 = it[1:11]
            assert 0 <= s < D and 0 <= kh < Hkv and row0 == 0 and nrows == 1
            assert (head0 - kh * g) % dec_cols == 0 and kh * g <= head0 < (kh + 1) * g
            assert nh == min(dec_cols, (kh + 1) * g - head0)
            assert k0 % 32 == 0 and 0 <= k0 < k1 <= ctx[s] + 1
            add(("d", s, kh, head0), k0, k1, split, g0)
        elif kind == CHUNK:
            s, kh, i0, cnt = it[1:5]
            k0, k1, split, g0 = it[7:11]
            assert D <= s < S and 0 <= kh < Hkv and 1 <= cnt <= per_item
            q = cu[s + 1] - cu[s]
            nblk = -(-q // 32) * g
            assert 0 <= i0 and i0 + cnt <= nblk and k0 % 32 == 0 and 0 <= k0 < k1
            for j in range(cnt):
                i = i0 + j
                row0 = 32 * (i // g)
                end = ctx[s] + row0 + min(32, q - row0)
                if k0 < end:                    # the block sees keys of this piece
                    add(("c", s, kh, i), k0, min(k1, end), split, -1 if g0 < 0 else g0 + j)
        else:
            assert kind == PACK and g <= dec_cols
            m = int(it[1])
            js = [(m >> (4 * w)) & 15 for w in range(4)]
            assert js == sorted(js) and js[0] == 0, js          # consecutive runs, starting at decode 0
            nb = js[-1] + 1
            assert set(js) == set(range(nb))
            for j in range(nb):
                s, kh = it[2 + 2 * j], it[3 + 2 * j]
                assert 0 <= s < D and 0 <= kh < Hkv
                add(("d", s, kh, kh * g), walk_start(ctx[s], window), ctx[s] + 1, -1, -1)
            assert all(it[2 + 2 * j] == -1 for j in range(nb, 4))
    # every block present, its pieces partition [0, keys)
    expected = set()
    for s in range(D):
        for kh in range(Hkv):
            for h in range(0, g, dec_cols):
                expected.add(("d", s, kh, kh * g + h))
    for s in range(D, S):
        q = cu[s + 1] - cu[s]
        for kh in range(Hkv):
            for i in range(-(-q // 32) * g):
                expected.add(("c", s, kh, i))
    assert set(cover) == expected
    parts_seen = set()
    for key, pieces in cover.items():
        pieces.sort()
        if key[0] == "d":
            end = ctx[key[1]] + 1
            first = walk_start(ctx[key[1]], window)      # the tile of the decode's first visible key
            assert pieces[0][0] == first, (key, pieces)
        else:
            s, i = key[1], key[3]
            q = cu[s + 1] - cu[s]
            row0 = 32 * (i // g)
            end = ctx[s] + row0 + min(32, q - row0)
            # the item's walk starts at or before the block's first visible key, and
            # at most one item row block (8 column blocks) earlier
            assert pieces[0][0] % 32 == 0 and pieces[0][0] <= walk_start(ctx[s] + row0, window), (key, pieces)
            assert pieces[0][0] >= walk_start(ctx[s] + max(0, row0 - 32 * (-(-per_item // g))), window)
        assert pieces[-1][1] == end, (key, pieces)
        for a, b in zip(pieces, pieces[1:]):
            assert a[1] == b[0], (key, pieces)
        if len(pieces) == 1:
            assert pieces[0][2] == -1 and pieces[0][3] == -1
        else:
            grp = {p[3] for p in pieces}
            assert len(grp) == 1 and -1 not in grp
            gi = grp.pop()
            p0, ns = groups[gi][0], groups[gi][1]
            assert ns == len(pieces) and sorted(p[2] for p in pieces) == list(range(ns))
            assert groups[gi][2] == key[1]
            for k in range(ns):
                assert (p0 + k) not in parts_seen
                parts_seen.add(p0 + k)
    assert parts_seen == set(range(dev.num_partials))
    return dev


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload_plans_cover_every_key_once(n):
    inst = W.make_config(n)
    batch = build(inst)
    dev = check_plan(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    _, items, _ = pack(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    if n in (2, 5):          # a little over one round otherwise: packed into one round
        assert dev.num_work_items <= SLOTS
    if n in (3, 4):          # several rounds (LLaMA: 640 chunk items alone): average-cost splits
        assert dev.num_work_items > SLOTS and not (items[:, 0] == PACK).any()


@pytest.mark.parametrize("n,window", [(2, 4096), (2, 1000), (3, 4096), (4, 4096), (4, 33), (5, 1024), (5, 1)])
def test_windowed_plans_skip_tiles_outside_the_window(n, window):
    inst = W.make_config(n)
    batch = build(inst)
    dev = check_plan(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages, window)
    full = check_plan(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    if max(batch.view()["context_lens"]) >= window:
        assert dev.num_work_items <= full.num_work_items or dev.num_partials < full.num_partials


@pytest.mark.parametrize("seed", range(20))
def test_random_windowed_plans(seed):
    inst = W.random_small_instance(seed, max_reqs=10, max_len=400)
    try:
        batch = build(inst)
    except N.SarathiError:
        pytest.skip("state cannot be scheduled")
    w = [1, 2, 31, 32, 33, 64, 100, 257, 10 ** 6][seed % 9]
    for Hq, Hkv, d in [(4, 1, 64), (32, 8, 128), (58, 2, 64), (64, 1, 128)]:
        check_plan(batch, Hq, Hkv, d, inst.num_pages, w)


def test_negative_window_rejected():
    inst = W.make_config(1)
    with pytest.raises(N.SarathiError) as e:
        N.sa_batch_upload_size(build(inst), 4, 1, 64, -1)
    assert e.value.status == N.SA_ERR_INVALID_ARG


@pytest.mark.parametrize("B", list(W.SWEEP_BUDGETS) + list(W.SWEEP_DIAGNOSTIC))
def test_budget_sweep_plans(B):
    inst = W.make_config(5, B)
    check_plan(build(inst), inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)


@pytest.mark.parametrize("seed", range(40))
def test_random_plans_any_head_shape(seed):
    """Small random batches under head shapes with and without decode packing
    (g > 32 puts two column blocks in a kv group)."""
    inst = W.random_small_instance(seed, max_reqs=10, max_len=400)
    try:
        batch = build(inst)
    except N.SarathiError:
        pytest.skip("state cannot be scheduled")
    for Hq, Hkv, d in [(4, 1, 64), (32, 8, 128), (58, 2, 64), (64, 1, 128), (40, 1, 64), (8, 8, 128)]:
        check_plan(batch, Hq, Hkv, d, inst.num_pages)


def test_long_decodes_split_and_short_ones_pack():
    """Many decodes of mixed length: long ones are split, short ones share
    workgroups, and the plan still fits one round."""
    rng = np.random.default_rng(9)
    ctx = np.concatenate([rng.integers(1, 200, 40), rng.integers(6000, 8000, 8)]).astype(np.int32)
    W_ = 512
    bt = np.full((len(ctx), W_), -1, np.int32)
    P = 0
    for s, c in enumerate(ctx):
        n = -(-(int(c) + 1) // 16)
        bt[s, :n] = np.arange(P, P + n)
        P += n
    slots = [int(bt[s, c // 16]) * 16 + int(c) % 16 for s, c in enumerate(ctx)]
    batch = batch_from_arrays([1] * len(ctx), ctx.tolist(), bt, slots, num_decodes=len(ctx))
    dev, items, _ = pack(batch, 32, 8, 128, P)
    check_plan(batch, 32, 8, 128, P)
    kinds = items[:, 0]
    assert (kinds == PACK).any() and dev.num_combine_groups > 0
    assert dev.num_work_items <= SLOTS


def test_very_long_decodes_split_at_most_64_ways():
    """A 100k-key decode of a 2-kv-head model would take about 100 splits at
    the plan's smallest tile target; the merge holds 64 split weights per
    column, so the plan caps the splits (longer per-split walks instead)."""
    inst = W.long_context_instance()
    batch = build(inst)
    dev, items, groups = pack(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    check_plan(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    assert dev.num_combine_groups > 0 and groups[:, 1].max() == 64
    assert dev.num_work_items <= SLOTS


def item_reads_and_walk(items, ctx):
    """Per item: key tiles its workgroup reads, and tiles each wave walks."""
    reads, walk = [], []
    for it in items:
        if it[0] == CHUNK:
            t = -(-(it[8] - it[7]) // 32)
            reads.append(t); walk.append(t)
        elif it[0] == DECODE:
            t = -(-(it[8] - it[7]) // 32)
            reads.append(t); walk.append(-(-t // 4))
        else:
            m = int(it[1])
            js = [(m >> (4 * w)) & 15 for w in range(4)]
            ts = {j: -(-(int(ctx[it[2 + 2 * j]]) + 1) // 32) for j in set(js)}
            reads.append(sum(ts.values()))
            walk.append(max(-(-ts[j] // js.count(j)) for j in ts))
    return np.array(reads), np.array(walk)


@pytest.mark.parametrize("n,key", [(2, "reads"), (5, "walk")])
def test_one_round_plans_pair_long_with_short_items(n, key):
    """A one-round plan puts workgroups h and h + 256 (same CU) together: the
    first half is emitted longest first, the second half shortest first, by
    tiles read when the batch is HBM-bound (Mistral-7B) and by tiles walked
    per wave when it is bound by the matrix cores (Falcon-180B share)."""
    inst = W.make_config(n)
    batch = build(inst)
    dev, items, _ = pack(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    assert 256 < len(items) <= SLOTS
    reads, walk = item_reads_and_walk(items, batch.view()["context_lens"])
    c = reads if key == "reads" else walk
    assert (np.diff(c[:256]) <= 0).all() and (np.diff(c[256:]) >= 0).all()
    assert c[0] == c.max() and c[256] == c.min()   # the longest and the shortest share a CU


@pytest.mark.parametrize("B,last", [(896, True), (1024, True), (1280, True), (1536, True), (2048, True),
                                    (512, False), (768, False)])
def test_chunk_items_last_when_they_fill_the_chip(B, last):
    """LLaMA2-70B-shaped batches (256 decodes, several rounds, decode-dominated):
    the chunk items go after the decode items when, by themselves, they keep
    at least 27% of the 512 workgroup slots busy over their longest walk
    (B = 896: 0.28, 1024: 0.31, 1280: 0.40, 1536: 0.51, 2048: 0.84) -- the
    longer half of them right after the first 85% of the decodes, the rest
    after the last decode; with fewer chunk rows (B = 512: 0.24, 768: 0.26)
    they stay mixed in the longest-first order.  Within each class the order
    is longest first."""
    inst = W.make_config(4, token_budget=B)
    batch = build(inst)
    dev, items, _ = pack(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    reads, walk = item_reads_and_walk(items, batch.view()["context_lens"])
    chunk = items[:, 0] == CHUNK
    assert len(items) > SLOTS and chunk.any() and reads[~chunk].sum() >= 9 * reads[chunk].sum()
    fill = walk[chunk].sum() / (SLOTS * walk[chunk].max())
    assert (fill >= 0.27) == last
    if last:
        nd, nc = int((~chunk).sum()), int(chunk.sum())
        pos, move = nd * 85 // 100, nc // 2
        expect = np.r_[np.zeros(pos, bool), np.ones(move, bool), np.zeros(nd - pos, bool), np.ones(nc - move, bool)]
        assert (chunk == expect).all()
        assert (np.diff(walk[~chunk]) <= 0).all() and (np.diff(walk[chunk]) <= 0).all()
    else:
        assert (np.diff(walk) <= 0).all()
        assert chunk[: len(items) // 2].any()


def test_one_round_decode_plans_use_every_slot():
    """A decode-dominated batch whose plan fits one round with slots to spare
    (Mistral-7B-shaped: 492 items before) gets the spare slots: the packs
    that read the most are cut in two, one-decode packs split their keys,
    until all 512 are used; the heaviest CU (workgroups h and h + 256) reads
    no more than 3% above the average."""
    inst = W.make_config(2)
    batch = build(inst)
    dev, items, _ = pack(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    check_plan(batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages)
    assert len(items) == SLOTS
    reads, _ = item_reads_and_walk(items, batch.view()["context_lens"])
    per_cu = reads[: SLOTS // 2] + reads[SLOTS // 2:]
    assert per_cu.max() <= 1.03 * reads.sum() / (SLOTS // 2)


@pytest.mark.parametrize("seed", range(8))
def test_decode_batches_fill_the_round(seed):
    """Decode-only batches of 40-110 decodes over several head shapes: every
    key of every block is covered once; a one-round plan past half a round
    ends with all 512 slots used or no pack left to cut."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, d = [(32, 8, 128), (28, 4, 128), (58, 2, 64), (64, 8, 128)][seed % 4]
    nd = int(rng.integers(40, 111))
    inst = W.decode_batch_instance(300 + seed, nd, float(rng.integers(800, 3000)), Hq, Hkv, d, 512)
    batch = build(inst)
    dev = check_plan(batch, Hq, Hkv, d, inst.num_pages)
    _, items, _ = pack(batch, Hq, Hkv, d, inst.num_pages)
    assert len(items) == dev.num_work_items
    if SLOTS // 2 < len(items) < SLOTS:
        assert not (items[:, 0] == 2).any(), "a pack was left uncut below a full round"


@pytest.mark.parametrize("n", [1, 2, 4, 5])
def test_packed_metadata_round_trips(n):
    """The uploaded buffer holds cu_seqlens, context lengths, the slot mapping
    and each sequence's pages (ragged, logical order) exactly as the batch."""
    inst = W.make_config(n)
    batch = build(inst)
    Hq, Hkv, d = inst.num_q_heads, inst.num_kv_heads, inst.head_dim
    nbytes = N.sa_batch_upload_size(batch, Hq, Hkv, d, 0)
    buf = np.zeros(nbytes // 4 + 8, np.int32)
    off = (-buf.ctypes.data) % 16 // 4
    staging = buf[off: off + nbytes // 4]
    dev = N.sa_batch_pack(batch, Hq, Hkv, d, inst.num_pages, staging, DEV, 0)
    at = lambda p: (p - DEV) // 4
    v = batch.view()
    S, T = batch.num_seqs, batch.num_tokens
    assert staging[at(dev.cu_seqlens_q): at(dev.cu_seqlens_q) + S + 1].tolist() == v["cu_seqlens_q"]
    assert staging[at(dev.context_lens): at(dev.context_lens) + S].tolist() == v["context_lens"]
    assert staging[at(dev.slot_mapping): at(dev.slot_mapping) + T].tolist() == v["slot_mapping"]
    offs = staging[at(dev.block_table_offsets): at(dev.block_table_offsets) + S]
    widest = 0
    for s in range(S):
        n_pages = -(-(v["context_lens"][s] + v["cu_seqlens_q"][s + 1] - v["cu_seqlens_q"][s]) // 16)
        widest = max(widest, n_pages)
        row = staging[at(dev.block_tables) + offs[s]: at(dev.block_tables) + offs[s] + n_pages]
        assert row.tolist() == v["block_tables"][s][:n_pages]
        if s + 1 < S:
            assert offs[s + 1] == offs[s] + n_pages
    assert dev.bt_stride == widest
