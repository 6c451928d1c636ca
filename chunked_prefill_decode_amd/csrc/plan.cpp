// Metadata upload and the attention work plan (host side of libsarathi_attn).
//
// One upload per iteration: the batch metadata and the work plan are packed
// into a caller-provided (pinned) staging buffer and moved with a single copy
// (a kernel reading the pinned buffer, or hipMemcpyAsync for pageable
// memory), so the device sees everything the kernels need.
//
// Work plan.  Every work item is one workgroup of four wavefronts (see
// common.h for the item layout):
//   * decode items -- one decode, one kv head, the q heads of its group as
//     the columns (grouped-query heads share every K/V load); the four waves
//     split the item's keys and merge through LDS;
//   * chunk items -- 32 query rows of a prefill chunk for four q heads of one
//     kv-head group; the four waves walk the same keys, so every K/V tile is
//     fetched once per workgroup.
// With a sliding window a block's walk starts at the 32-key tile holding the
// first key any of its rows sees, so tiles wholly outside every row's window
// are never read.
// The cost of an item is counted in 32-key tiles per wave.  Items much longer
// than the average are split over several workgroups (their partial results
// are merged by a second kernel), and items are emitted longest first so the
// hardware's in-order dispatch balances the tail.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "common.h"

namespace {

constexpr int64_t kTargetItems = 512;   // one round of 2 workgroups per CU on 256 CUs (measured best)
constexpr int64_t kMinTarget = 8;       // tiles per wave below which no item is split

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline size_t pad4(size_t w) { return (w + 3) & ~size_t(3); }   // 16-byte sections

// A column block before splitting.
struct Block {
  int kind, s, kh, head0, nheads, row0, nrows;
  int64_t keys;    // one past the last key any row of the block sees
  int64_t lo;      // first key walked: a multiple of 32, at or below the block's first visible key
  int64_t span() const { return keys - lo; }
};

// Whole decodes packed into one workgroup: block indices and their waves.
struct Pack {
  int n = 0;
  int blk[sa::kWaves];
  int waves[sa::kWaves];
};

struct Plan {
  int S = 0, D = 0, T = 0, Hq = 0, Hkv = 0, d = 0, group = 0, dec_cols = 0;
  int window = 0;                // sliding window in keys, 0 = none
  int bt_stride = 1;              // pages of the widest sequence
  int64_t bt_total = 0;          // pages of all sequences
  int64_t target = kMinTarget;
  std::vector<Block> blocks;
  std::vector<int64_t> splits;   // per block: number of items (0: the block is in a pack)
  std::vector<int64_t> lens;     // per block: keys per item (multiple of 32)
  std::vector<Pack> packs;
  std::vector<int> by_length;    // block indices, longest first
  int64_t n_items = 0, n_groups = 0, n_partials = 0;
  size_t words_cu = 0, words_ctx = 0, words_slots = 0, words_btoff = 0, words_bt = 0, words_items = 0, words_groups = 0;
  size_t total_words() const {
    return words_cu + words_ctx + words_slots + words_btoff + words_bt + words_items + words_groups;
  }
};

int64_t block_cost(const Block& b) {   // 32-key tiles per wave
  return b.kind == sa::kDecodeItem ? ceil_div(b.span(), int64_t(sa::kKeyTile) * sa::kWaves)
                                   : ceil_div(b.span(), sa::kKeyTile);
}

// First key walked by a block whose earliest row sits at absolute position p:
// the tile holding key p - window + 1 (key 0 without a window).
int64_t walk_start(int64_t p, int window) {
  return window > 0 ? std::max<int64_t>(0, p - window + 1) / sa::kKeyTile * sa::kKeyTile : 0;
}

sa_status check_batch(const sa_batch* b, int Hq, int Hkv, int d, int window, int num_pages, Plan* x) {
  if (!b) return sa::fail(SA_ERR_INVALID_ARG, "batch: null pointer");
  if (window < 0) return sa::fail(SA_ERR_INVALID_ARG, "batch: sliding window %d", window);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv)
    return sa::fail(SA_ERR_INVALID_ARG, "batch: q heads %d must be a positive multiple of kv heads %d", Hq, Hkv);
  if (d != 64 && d != 128) return sa::fail(SA_ERR_UNSUPPORTED, "batch: head_dim %d (64 or 128 supported)", d);
  const int S = b->num_seqs, D = b->num_decodes;
  if (S < 0 || D < 0 || D > S) return sa::fail(SA_ERR_INVALID_ARG, "batch: %d sequences, %d decodes", S, D);
  if (!b->cu_seqlens_q) return sa::fail(SA_ERR_INVALID_ARG, "batch: null cu_seqlens_q");
  if (S > 0 && (!b->context_lens || !b->block_tables))
    return sa::fail(SA_ERR_INVALID_ARG, "batch: null context_lens / block_tables");
  const int W = b->max_blocks_per_seq;
  if (S > 0 && W < 1) return sa::fail(SA_ERR_INVALID_ARG, "batch: max_blocks_per_seq %d", W);
  if (b->cu_seqlens_q[0] != 0) return sa::fail(SA_ERR_INVALID_ARG, "batch: cu_seqlens_q[0] = %d", b->cu_seqlens_q[0]);
  int bt_stride = 1;
  int64_t bt_total = 0;
  for (int s = 0; s < S; ++s) {
    const int q = b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s];
    const int ctx = b->context_lens[s];
    if (q < 1) return sa::fail(SA_ERR_INVALID_ARG, "batch: sequence %d has q_len %d", s, q);
    if (s < D && q != 1) return sa::fail(SA_ERR_INVALID_ARG, "batch: decode %d has q_len %d", s, q);
    if (ctx < 0) return sa::fail(SA_ERR_INVALID_ARG, "batch: sequence %d has context %d", s, ctx);
    const int64_t kv = int64_t(ctx) + q;
    const int64_t np = ceil_div(kv, sa::kPageSize);
    if (np > W) return sa::fail(SA_ERR_INVALID_ARG, "batch: sequence %d needs %lld pages > W %d", s, (long long)np, W);
    const int32_t* row = b->block_tables + size_t(s) * size_t(W);
    for (int64_t j = 0; j < np; ++j)
      if (row[j] < 0 || row[j] >= num_pages)
        return sa::fail(SA_ERR_INVALID_ARG, "batch: sequence %d block %lld = page %d outside [0, %d)", s, (long long)j,
                        row[j], num_pages);
    bt_stride = std::max<int>(bt_stride, int(np));
    bt_total += np;
  }
  const int T = b->cu_seqlens_q[S];
  if (b->num_tokens != T) return sa::fail(SA_ERR_INVALID_ARG, "batch: num_tokens %d != cu_seqlens_q[S] %d", b->num_tokens, T);
  if (T > 0 && !b->slot_mapping) return sa::fail(SA_ERR_INVALID_ARG, "batch: null slot_mapping");
  x->S = S; x->D = D; x->T = T; x->Hq = Hq; x->Hkv = Hkv; x->d = d; x->window = window;
  x->group = Hq / Hkv;
  x->dec_cols = x->group <= 16 ? 16 : 32;
  x->bt_stride = bt_stride;
  x->bt_total = bt_total;
  return SA_OK;
}

int64_t decode_tiles(const Block& b) { return ceil_div(b.span(), sa::kKeyTile); }   // one wave's walk

// Items for per-wave tile target t.  Chunk blocks split when longer than 2t
// (their partials are several column blocks wide).  With `pack`, a decode
// block needs ceil(tiles / t) waves: up to 4 it is packed with other whole
// decodes into a workgroup (best fit over the free wave slots of the open
// workgroups); beyond 4 (or without `pack`) it takes whole workgroups of 4
// waves over equal key ranges.  With `assign`, the splits and packs are
// recorded in x.
// Split count of a block for target t (tile-aligned equal key ranges; at most
// kMaxSplits, the merge kernel's table of split weights).
int64_t split_count(const Block& k, int64_t t) {
  int64_t ns = k.kind == sa::kDecodeItem ? ceil_div(decode_tiles(k), sa::kWaves * t) : ceil_div(block_cost(k), 2 * t);
  ns = std::max<int64_t>(1, std::min<int64_t>({ns, ceil_div(k.span(), sa::kKeyTile), int64_t(sa::kMaxSplits)}));
  return ceil_div(k.span(), round_up(ceil_div(k.span(), ns), sa::kKeyTile));   // no empty split
}

// The number of items plan_items(x, t, pack, true) would make, without
// building anything.  Best fit over 4-wave workgroups of blocks needing
// 4, 3, 2, then 1 waves fills every 3-wave workgroup's last slot and the
// odd 2-wave workgroup's two slots with 1-wave blocks before opening new
// workgroups.
int64_t count_items(const Plan& x, int64_t t, bool pack) {
  const bool can_pack = pack && x.group <= x.dec_cols;
  int64_t items = 0, n[sa::kWaves + 1] = {0, 0, 0, 0, 0};
  for (const Block& k : x.blocks) {
    if (can_pack && k.kind == sa::kDecodeItem) {
      const int64_t w = ceil_div(decode_tiles(k), t);
      if (w <= sa::kWaves) {
        ++n[w];
        continue;
      }
    }
    items += split_count(k, t);
  }
  const int64_t free_slots = n[3] + (n[2] % 2 ? 2 : 0);
  return items + n[4] + n[3] + ceil_div(n[2], 2) + std::max<int64_t>(0, ceil_div(n[1] - free_slots, sa::kWaves));
}

// A pack's wave slots beyond those its decodes were given go, one at a time,
// to the decode with the longest walk per wave.
void spread_waves(const Plan& x, Pack& p) {
  int used = 0;
  for (int j = 0; j < p.n; ++j) used += p.waves[j];
  for (; used < sa::kWaves; ++used) {
    int best = 0;
    int64_t best_t = -1;
    for (int j = 0; j < p.n; ++j) {
      const int64_t tw = ceil_div(decode_tiles(x.blocks[size_t(p.blk[j])]), p.waves[j]);
      if (tw > best_t) { best_t = tw; best = j; }
    }
    ++p.waves[best];
  }
}

int64_t plan_items(Plan* x, int64_t t, bool pack, bool assign) {
  const bool can_pack = pack && x->group <= x->dec_cols;   // one column block covers a kv group
  int64_t items = 0;
  std::vector<int> open[sa::kWaves];               // packs by free wave slots (1..3)
  std::vector<Pack> packs;
  if (assign) {
    x->splits.assign(x->blocks.size(), 0);
    x->lens.assign(x->blocks.size(), 0);
  }
  // packed blocks in decreasing order of waves: first the ones needing 4, then 3, 2, 1;
  // blocks are visited longest first, so each class is in that order too
  std::vector<int> by_waves[sa::kWaves + 1];
  for (int i : x->by_length) {
    const Block& k = x->blocks[size_t(i)];
    int64_t ns;
    if (k.kind == sa::kDecodeItem) {
      const int64_t w = ceil_div(decode_tiles(k), t);
      if (can_pack && w <= sa::kWaves) {
        by_waves[w].push_back(int(i));
        continue;
      }
      ns = ceil_div(decode_tiles(k), sa::kWaves * t);
    } else {
      ns = ceil_div(block_cost(k), 2 * t);
    }
    ns = std::max<int64_t>(1, std::min<int64_t>({ns, ceil_div(k.span(), sa::kKeyTile), int64_t(sa::kMaxSplits)}));
    const int64_t len = round_up(ceil_div(k.span(), ns), sa::kKeyTile);   // split starts stay tile aligned
    ns = ceil_div(k.span(), len);                                        // no empty split
    items += ns;
    if (assign) {
      x->splits[i] = ns;
      x->lens[i] = len;
    }
  }
  for (int w = sa::kWaves; w >= 1; --w) {
    for (int i : by_waves[w]) {                    // longest first: a workgroup's decodes have similar walks
      int f = w;                                   // best fit: the fullest open pack with room
      while (f < sa::kWaves && open[f].empty()) ++f;
      int pk;
      if (f < sa::kWaves) {
        pk = open[f].back();
        open[f].pop_back();
      } else {
        pk = int(packs.size());
        packs.push_back(Pack{});
        f = sa::kWaves;
      }
      Pack& p = packs[size_t(pk)];
      p.blk[p.n] = i;
      p.waves[p.n] = w;
      ++p.n;
      if (f - w > 0) open[f - w].push_back(pk);
    }
  }
  items += int64_t(packs.size());
  if (assign) {
    for (Pack& p : packs) spread_waves(*x, p);
    x->packs = std::move(packs);
  }
  return items;
}

// A one-round plan with fewer items than resident workgroup slots leaves
// some CUs a single workgroup while the others run two, and in an HBM-bound
// (decode-dominated) batch what a CU reads sets when it finishes: on the
// Mistral-7B-shaped step (492 items) 20 CUs ended at ~39 us and the rest at
// 73-78, their end tracking the key tiles their two workgroups read
// (correlation 0.97).  So the free slots go to the packs that read the most:
// a pack of several whole decodes is cut in two (decodes alternately to the
// lighter half), a pack of one decode becomes a two-way split of its keys.
// Mistral-7B: 512 items, the heaviest CU reads 119 instead of 126 key tiles,
// attention 87.7 -> 86.3 us (the rest of the chip keeps HBM busy while a
// CU idles, so the end moves less than the reads).
void fill_round(Plan* x) {
  int64_t n = int64_t(x->packs.size()), dec = 0, chk = 0;
  for (size_t i = 0; i < x->blocks.size(); ++i) {
    n += x->splits[i];
    (x->blocks[i].kind == sa::kDecodeItem ? dec : chk) += ceil_div(x->blocks[i].span(), sa::kKeyTile);
  }
  if (dec < 9 * chk) return;                       // the emitted order balances walks, not reads
  if (n <= kTargetItems / 2) return;               // every CU runs at most one item: no CU waits on a partner
  for (; n < kTargetItems; ++n) {
    int best = -1;
    int64_t best_r = 0;
    for (size_t p = 0; p < x->packs.size(); ++p) {
      int64_t r = 0;
      for (int j = 0; j < x->packs[p].n; ++j) r += decode_tiles(x->blocks[size_t(x->packs[p].blk[j])]);
      if (r > best_r) { best_r = r; best = int(p); }
    }
    if (best < 0) return;
    const Pack pk = x->packs[size_t(best)];
    if (pk.n >= 2) {
      Pack h[2];
      int64_t r[2] = {0, 0};
      for (int j = 0; j < pk.n; ++j) {               // members are longest first
        const int s = r[0] <= r[1] ? 0 : 1;
        h[s].blk[h[s].n] = pk.blk[j];
        h[s].waves[h[s].n] = 1;
        ++h[s].n;
        r[s] += decode_tiles(x->blocks[size_t(pk.blk[j])]);
      }
      spread_waves(*x, h[0]);
      spread_waves(*x, h[1]);
      x->packs[size_t(best)] = h[0];
      x->packs.push_back(h[1]);
    } else {
      const size_t i = size_t(pk.blk[0]);
      const Block& k = x->blocks[i];
      const int64_t len = round_up(ceil_div(k.span(), 2), sa::kKeyTile);
      if (ceil_div(k.span(), len) < 2) return;       // a single tile: nothing left worth splitting
      x->splits[i] = ceil_div(k.span(), len);
      x->lens[i] = len;
      x->packs.erase(x->packs.begin() + best);
    }
  }
}

void make_blocks(const sa_batch* b, Plan* x) {
  x->blocks.clear();
  const int g = x->group;
  const int per_item = sa::chunk_blocks_per_item(x->d);
  {
    int64_t n = int64_t(x->D) * x->Hkv * ceil_div(g, x->dec_cols);
    for (int s = x->D; s < x->S; ++s)
      n += x->Hkv * ceil_div(ceil_div(b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s], sa::kCols) * g, per_item);
    x->blocks.reserve(size_t(n));
  }
  for (int s = x->D; s < x->S; ++s) {             // chunk items: 4 or 8 consecutive column blocks
    const int q = b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s];
    const int ctx = b->context_lens[s];
    const int nblk = int(ceil_div(q, sa::kCols)) * g;   // block i: row block i / g, q head i % g
    for (int kh = 0; kh < x->Hkv; ++kh)
      for (int i0 = 0; i0 < nblk; i0 += per_item) {
        const int cnt = std::min(per_item, nblk - i0);
        const int r_last = sa::kCols * ((i0 + cnt - 1) / g);
        x->blocks.push_back({sa::kChunkItem, s, kh, i0, cnt, 0, 0,
                             int64_t(ctx) + r_last + std::min(sa::kCols, q - r_last),
                             walk_start(int64_t(ctx) + sa::kCols * (i0 / g), x->window)});
      }
  }
  for (int s = 0; s < x->D; ++s)                  // decode blocks: the heads of one kv group
    for (int kh = 0; kh < x->Hkv; ++kh)
      for (int h = 0; h < g; h += x->dec_cols)
        x->blocks.push_back({sa::kDecodeItem, s, kh, kh * g + h, std::min(x->dec_cols, g - h), 0, 1,
                             int64_t(b->context_lens[s]) + 1, walk_start(b->context_lens[s], x->window)});
  x->by_length.resize(x->blocks.size());
  for (size_t i = 0; i < x->blocks.size(); ++i) x->by_length[i] = int(i);
  std::sort(x->by_length.begin(), x->by_length.end(), [&](int a, int c) {
    const int64_t ka = x->blocks[size_t(a)].span(), kc = x->blocks[size_t(c)].span();
    return ka != kc ? ka > kc : a < c;
  });
  // The plain plan splits at the average cost and lets the longest-first
  // order balance the rounds.  When that plan runs a little over one round
  // (at most 1.5), the last workgroups start late and finish alone; if some
  // plan fits in one round, take instead the smallest per-wave tile target
  // that does: every wave then walks at most that many tiles and no
  // workgroup waits for a slot.
  int64_t hi = kMinTarget, total = 0;
  for (const Block& k : x->blocks) {
    hi = std::max(hi, k.kind == sa::kDecodeItem ? decode_tiles(k) : block_cost(k));
    total += block_cost(k);
  }
  const int64_t avg = std::max<int64_t>(kMinTarget, ceil_div(total, kTargetItems));
  const int64_t rounds_x2 = 2 * count_items(*x, avg, false);   // the average-cost plan, in half rounds
  if (rounds_x2 <= 3 * kTargetItems && count_items(*x, hi, true) <= kTargetItems) {
    int64_t lo = kMinTarget;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (count_items(*x, mid, true) <= kTargetItems) hi = mid;
      else lo = mid + 1;
    }
    x->target = lo;
    plan_items(x, lo, true, true);
    fill_round(x);
  } else {
    x->target = avg;
    plan_items(x, avg, false, true);
  }
  int64_t items = int64_t(x->packs.size()), groups = 0, partials = 0;
  for (size_t i = 0; i < x->blocks.size(); ++i) {
    const int64_t ns = x->splits[i];
    items += ns;
    if (ns > 1) {
      const int64_t nb = x->blocks[i].kind == sa::kDecodeItem ? 1 : x->blocks[i].nheads;
      groups += nb;
      partials += nb * ns;
    }
  }
  x->n_items = items; x->n_groups = groups; x->n_partials = partials;
}

sa_status shape(const sa_batch* b, int Hq, int Hkv, int d, int window, int num_pages, Plan* x) {
  sa_status st = check_batch(b, Hq, Hkv, d, window, num_pages, x);
  if (st != SA_OK) return st;
  make_blocks(b, x);
  if (x->bt_total > (int64_t(1) << 30)) return sa::fail(SA_ERR_INVALID_ARG, "batch: block tables too large");
  if (x->n_items > (int64_t(1) << 30)) return sa::fail(SA_ERR_INVALID_ARG, "batch: work plan too large");
  x->words_cu = pad4(size_t(x->S) + 1);
  x->words_ctx = pad4(size_t(x->S));
  x->words_slots = pad4(size_t(x->T));
  x->words_btoff = pad4(size_t(x->S));
  x->words_bt = pad4(size_t(x->bt_total));
  x->words_items = size_t(x->n_items) * sa::kItemWords;
  x->words_groups = size_t(x->n_groups) * sa::kGroupWords;
  return SA_OK;
}

// Writes the items and split groups.  Returns the decode-path cache policy:
// stream (non-temporal) when the batch is decode-dominated -- decode items
// read at least 90% of the key tiles the plan reads (chunk items re-read
// their prompt's prefix, mostly from cache) -- and the decode K/V it reads
// is well beyond the 256 MB Infinity Cache.  Measured on decode-only batches
// of 16-256 decodes: streaming is ~10% faster from ~450 MB of K/V per step
// up, and up to ~10% slower below ~260 MB, where the cached loads find much
// of the previous step's K/V still in the Infinity Cache.
bool emit_plan(const sa_batch* b, const Plan& x, int32_t* items, int32_t* groups) {
  auto b_qlen = [&](int s) { return b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s]; };
  // Items are emitted longest first (counting sort over their cost).  The
  // cost is the item's walk in key tiles per wave, or -- in a one-round plan
  // of a decode-dominated batch, which HBM bandwidth bounds -- the key tiles
  // its workgroup reads (a chunk item's four waves share each tile they
  // read, a decode item's waves each read their own), which is what the
  // pairing of items on a CU below has to even out there.
  struct It { int64_t cost, read; bool chunk; int32_t w[sa::kItemWords]; };
  std::vector<It> all;
  all.reserve(size_t(x.n_items));
  int64_t gi = 0, part = 0;
  for (size_t i = 0; i < x.blocks.size(); ++i) {
    const Block& k = x.blocks[i];
    const int64_t ns = x.splits[i];
    const int64_t len = x.lens[i];
    if (ns == 0) continue;                         // in a pack
    int32_t g0 = -1;
    if (ns > 1) {
      g0 = int32_t(gi);
      const int nb = k.kind == sa::kDecodeItem ? 1 : k.nheads;
      for (int w = 0; w < nb; ++w) {
        int32_t* g = groups + gi * sa::kGroupWords;
        g[0] = int32_t(part); g[1] = int32_t(ns); g[2] = k.s;
        if (k.kind == sa::kDecodeItem) {
          g[3] = k.head0; g[4] = k.nheads; g[5] = k.row0; g[6] = k.nrows;
        } else {                                   // column block head0 + w of the chunk
          const int blk = k.head0 + w;
          const int q = b_qlen(k.s);
          g[3] = k.kh * x.group + blk % x.group; g[4] = 1;
          g[5] = sa::kCols * (blk / x.group); g[6] = std::min(sa::kCols, q - g[5]);
        }
        g[7] = 0;
        ++gi;
        part += ns;
      }
    }
    for (int64_t j = 0; j < ns; ++j) {
      It it;
      const int64_t k0 = k.lo + j * len, k1 = std::min<int64_t>(k.keys, k.lo + (j + 1) * len);   // k0 < k1
      Block piece = k;
      piece.lo = k0;
      piece.keys = k1;
      it.cost = block_cost(piece);
      it.read = ceil_div(piece.span(), sa::kKeyTile);
      it.chunk = k.kind == sa::kChunkItem;
      int32_t* w = it.w;
      w[0] = k.kind; w[1] = k.s; w[2] = k.kh; w[3] = k.head0; w[4] = k.nheads; w[5] = k.row0; w[6] = k.nrows;
      w[7] = int32_t(k0); w[8] = int32_t(k1);
      w[9] = ns > 1 ? int32_t(j) : -1;
      w[10] = g0;
      w[11] = 0;
      all.push_back(it);
    }
  }
  for (const Pack& p : x.packs) {
    It it;
    int32_t* w = it.w;
    w[0] = sa::kDecodeGroupItem;
    int32_t map = 0;
    int wave = 0;
    it.cost = 0;
    it.read = 0;
    it.chunk = false;
    for (int j = 0; j < sa::kWaves; ++j) {
      w[2 + 2 * j] = j < p.n ? x.blocks[size_t(p.blk[j])].s : -1;
      w[3 + 2 * j] = j < p.n ? x.blocks[size_t(p.blk[j])].kh : -1;
    }
    for (int j = 0; j < p.n; ++j) {
      for (int u = 0; u < p.waves[j]; ++u, ++wave) map |= j << (4 * wave);
      it.cost = std::max(it.cost, ceil_div(decode_tiles(x.blocks[size_t(p.blk[j])]), p.waves[j]));   // tiles per wave
      it.read += decode_tiles(x.blocks[size_t(p.blk[j])]);
    }
    w[1] = map;
    w[10] = -1;
    w[11] = 0;
    all.push_back(it);
  }
  int64_t decode_read = 0, chunk_read = 0;
  for (const It& it : all) (it.chunk ? chunk_read : decode_read) += it.read;
  const bool decode_dominated = decode_read >= 9 * chunk_read;
  if (int64_t(all.size()) <= kTargetItems && decode_dominated)
    for (It& it : all) it.cost = it.read;
  constexpr int64_t kStreamBytes = int64_t(320) << 20;   // 1.25 x the Infinity Cache
  const bool stream = decode_dominated && decode_read * 128 * x.d >= kStreamBytes;   // 128 d bytes per K+V tile
  int64_t maxc = 0;
  for (const It& it : all) maxc = std::max(maxc, it.cost);
  // A decode-dominated batch of more than one round: the decode items
  // first, the chunk items last (each class longest first; the longer half
  // of the chunk items moves in among the last decodes, below), when the
  // chunk items alone keep at least 27% of the resident workgroup slots busy
  // over their longest walk.  A chunk item that shares a CU with streaming
  // decodes waits behind their HBM misses for each key tile it loads
  // (per-workgroup timestamps: ~2.4 us per tile, against ~1.3 us once the
  // decodes are done), so mixing the two stretches the chunk items; but a
  // chunk phase too thin to fill the chip ends in a tail of long walks.
  // LLaMA2-70B-shaped steps (256 decodes of 0.5k-8k keys), attention us,
  // mixed -> chunk-last with the placement below: B = 512 (fill 0.24) 738
  // -> 767; 640 (0.24) 744 -> 766; 768 (0.26) 751 -> 750; 896 (0.28) 753
  // -> 751; 1024 (0.31) 759 -> 751; 1152 (0.35) 769 -> 751; 1280 (0.40)
  // 780 -> 753.  (Before that placement, with every chunk item after the
  // decodes: 1536 (0.51) 803 -> 788, 2048 (0.84) 860 -> 802.)
  int64_t chunk_walks = 0, chunk_longest = 0;
  for (const It& it : all)
    if (it.chunk) {
      chunk_walks += it.cost;
      chunk_longest = std::max(chunk_longest, it.cost);
    }
  const bool chunks_last = int64_t(all.size()) > kTargetItems && decode_dominated && chunk_longest > 0 &&
                           100 * chunk_walks >= 27 * kTargetItems * chunk_longest;
  if (chunks_last) {
    const int64_t shift = maxc + 1;
    for (It& it : all)
      if (!it.chunk) it.cost += shift;
    maxc += shift;
  }
  std::vector<int64_t> start(size_t(maxc) + 2, 0);
  for (const It& it : all) ++start[size_t(maxc - it.cost) + 1];
  for (size_t c = 1; c < start.size(); ++c) start[c] += start[c - 1];
  for (const It& it : all) {
    const int64_t pos = start[size_t(maxc - it.cost)]++;
    std::memcpy(items + pos * sa::kItemWords, it.w, sizeof(it.w));
  }
  constexpr int64_t kHalf = kTargetItems / 2;
  const int64_t n = int64_t(all.size());
  if (chunks_last) {
    // Sorted: the decode items, then the chunk items, each longest first.
    // The longer half of the chunk items goes in after 85% of the decode
    // items: their long walks then start while the last decodes stream and
    // end with the shorter chunk items that follow the decodes, instead of
    // setting the kernel's tail.  LLaMA2-70B-shaped step, attention us (the
    // longest fraction f of the chunk items moved to position p of the decode
    // list): none 771.5; f 0.5 at p 0.85: 756.8; 0.4 / 0.6 at 0.85: 760.2 /
    // 758.1; 0.5 at 0.80 / 0.88: 768.5 / 757.9; every chunk item at 0.85:
    // 773.3.  B = 2048: 793.7 -> 781.6.
    int64_t nd = 0;
    for (const It& it : all) nd += !it.chunk;
    const int64_t nc = n - nd, move = nc / 2, pos = nd * 85 / 100;
    std::vector<int32_t> sorted(items, items + n * sa::kItemWords);
    int64_t o = 0;
    auto put = [&](int64_t i, int64_t cnt) {
      std::memcpy(items + o * sa::kItemWords, sorted.data() + i * sa::kItemWords,
                  sizeof(int32_t) * size_t(cnt) * sa::kItemWords);
      o += cnt;
    };
    put(0, pos);                                   // decodes, longest first
    put(nd, move);                                 // the longer half of the chunk items
    put(pos, nd - pos);                            // the last 15% of the decodes
    put(nd + move, nc - move);                     // the shorter chunk items
  }
  // One round (every workgroup resident at once, two per CU): workgroups
  // h and h + 256 share a CU, so give the second half ascending cost, pairing
  // the k-th longest item with the k-th shortest and evening out the CUs.
  if (n > kHalf && n <= kTargetItems)
    for (int64_t a = kHalf, b = n - 1; a < b; ++a, --b)
      for (int wd = 0; wd < sa::kItemWords; ++wd) std::swap(items[a * sa::kItemWords + wd], items[b * sa::kItemWords + wd]);
  return stream;
}

}  // namespace

extern "C" {

sa_status sa_batch_upload_size(const sa_batch* b, int32_t Hq, int32_t Hkv, int32_t d, int32_t window,
                               size_t* bytes) {
  if (!bytes) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload_size: null bytes");
  Plan x;
  // page ids are checked at upload time; here any id is accepted
  sa_status st = shape(b, Hq, Hkv, d, window, 0x7fffffff, &x);
  if (st != SA_OK) return st;
  *bytes = x.total_words() * sizeof(int32_t);
  return SA_OK;
}

sa_status sa_batch_pack(const sa_batch* b, int32_t Hq, int32_t Hkv, int32_t d, int32_t window, int32_t num_pages,
                        void* host_staging, const void* dev_buf, size_t bytes, sa_batch_dev* out) {
  if (!out) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_pack: null out");
  if (num_pages < 1) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_pack: num_pages %d", num_pages);
  Plan x;
  sa_status st = shape(b, Hq, Hkv, d, window, num_pages, &x);
  if (st != SA_OK) return st;
  const size_t need = x.total_words() * sizeof(int32_t);
  if (bytes < need) return sa::fail(SA_ERR_CAPACITY, "sa_batch_pack: needs %zu bytes, got %zu", need, bytes);
  if (!host_staging || !dev_buf) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_pack: null buffer");
  if ((reinterpret_cast<uintptr_t>(dev_buf) & 15) || (reinterpret_cast<uintptr_t>(host_staging) & 15))
    return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_pack: buffers must be 16-byte aligned");

  int32_t* h = static_cast<int32_t*>(host_staging);
  int32_t* cu = h;
  int32_t* ctx = cu + x.words_cu;
  int32_t* slots = ctx + x.words_ctx;
  int32_t* bt_off = slots + x.words_slots;
  int32_t* bt = bt_off + x.words_btoff;
  int32_t* items = bt + x.words_bt;
  int32_t* groups = items + x.words_items;
  std::memcpy(cu, b->cu_seqlens_q, sizeof(int32_t) * size_t(x.S + 1));
  if (x.S) std::memcpy(ctx, b->context_lens, sizeof(int32_t) * size_t(x.S));
  if (x.T) std::memcpy(slots, b->slot_mapping, sizeof(int32_t) * size_t(x.T));
  // block tables, ragged: each sequence's pages in logical order, no padding
  int64_t off = 0;
  for (int s = 0; s < x.S; ++s) {
    const int32_t* row = b->block_tables + size_t(s) * size_t(b->max_blocks_per_seq);
    const int kv = b->context_lens[s] + b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s];
    const int np = (kv + sa::kPageSize - 1) / sa::kPageSize;
    bt_off[s] = int32_t(off);
    std::memcpy(bt + off, row, sizeof(int32_t) * size_t(np));
    off += np;
  }
  const bool stream_kv = emit_plan(b, x, items, groups);

  const int32_t* dv = static_cast<const int32_t*>(dev_buf);
  out->cu_seqlens_q = dv;
  out->context_lens = dv + x.words_cu;
  out->slot_mapping = out->context_lens + x.words_ctx;
  out->block_table_offsets = out->slot_mapping + x.words_slots;
  out->block_tables = out->block_table_offsets + x.words_btoff;
  out->work = out->block_tables + x.words_bt;
  out->combine = out->work + x.words_items;
  out->num_seqs = x.S;
  out->num_decodes = x.D;
  out->num_tokens = x.T;
  out->bt_stride = x.bt_stride;
  out->num_q_heads = Hq;
  out->num_kv_heads = Hkv;
  out->head_dim = d;
  out->num_pages = num_pages;
  out->num_work_items = int32_t(x.n_items);
  out->num_combine_groups = int32_t(x.n_groups);
  out->num_partials = int32_t(x.n_partials);
  out->sliding_window = window;
  // Decode K/V is read once per step: non-temporal loads stream it faster
  // (Mistral-7B and LLaMA-2-70B batches, 95% decode reads, 0.47 and 4.5 GB:
  // -7% and -3%), but measured slower once the chunk items' cached prefix
  // reads take a larger share (Yi-34B at 80%: +1%; Falcon-180B share at 16%:
  // +4%) or the K/V nearly fits the Infinity Cache (see emit_plan).
  out->plan_flags = stream_kv ? SA_PLAN_STREAM_KV : 0;
  out->reserved = 0;
  return SA_OK;
}

sa_status sa_batch_upload(const sa_batch* b, int32_t Hq, int32_t Hkv, int32_t d, int32_t window, int32_t num_pages,
                          void* host_staging, void* dev_buf, size_t bytes, void* stream, sa_batch_dev* out) {
  sa_batch_dev dev;
  const sa_status st = sa_batch_pack(b, Hq, Hkv, d, window, num_pages, host_staging, dev_buf, bytes, &dev);
  if (st != SA_OK) return st;
  const size_t need = size_t(reinterpret_cast<const char*>(dev.combine) - static_cast<const char*>(dev_buf)) +
                      size_t(dev.num_combine_groups) * sa::kGroupWords * sizeof(int32_t);
  // Pinned staging has a device address: a copy kernel on `stream` reads it
  // over PCIe.  Pageable staging has none (the failed lookup's error is
  // cleared) and goes through hipMemcpyAsync.  `need` is a multiple of 16:
  // every section of the packed buffer is a multiple of 4 words.
  void* src_dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&src_dev, host_staging, 0);
  if (e == hipSuccess && src_dev) {
    e = sa::copy_pinned_to_device(src_dev, dev_buf, need, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sa::fail(SA_ERR_HIP, "sa_batch_upload: copy kernel: %s", hipGetErrorString(e));
  } else {
    (void)hipGetLastError();
    e = hipMemcpyAsync(dev_buf, host_staging, need, hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sa::fail(SA_ERR_HIP, "sa_batch_upload: hipMemcpyAsync: %s", hipGetErrorString(e));
  }
  *out = dev;
  return SA_OK;
}

sa_status sa_batch_upload_append(const sa_batch* b, int32_t Hq, int32_t Hkv, int32_t d, int32_t window,
                                 int32_t num_pages, void* host_staging, void* dev_buf, size_t bytes, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache, void* stream, sa_batch_dev* out) {
  if (b && b->num_tokens > 0) {
    if (!k_new || !v_new || !k_cache || !v_cache) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload_append: null tensor");
    for (const void* p : {k_new, v_new, static_cast<const void*>(k_cache), static_cast<const void*>(v_cache)})
      if (reinterpret_cast<uintptr_t>(p) & 15)
        return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload_append: tensors must be 16-byte aligned");
  }
  sa_batch_dev dev;
  const sa_status st = sa_batch_pack(b, Hq, Hkv, d, window, num_pages, host_staging, dev_buf, bytes, &dev);
  if (st != SA_OK) return st;
  const size_t need = size_t(reinterpret_cast<const char*>(dev.combine) - static_cast<const char*>(dev_buf)) +
                      size_t(dev.num_combine_groups) * sa::kGroupWords * sizeof(int32_t);
  void* src_dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&src_dev, host_staging, 0);
  if (e != hipSuccess || !src_dev) {
    (void)hipGetLastError();
    return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload_append: host_staging is not pinned host memory");
  }
  const int32_t* slots_dev = static_cast<const int32_t*>(src_dev) + (dev.slot_mapping - static_cast<const int32_t*>(dev_buf));
  e = sa::upload_append(src_dev, dev_buf, need, slots_dev, k_new, v_new, k_cache, v_cache, dev.num_tokens, Hkv, d,
                        num_pages, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return sa::fail(SA_ERR_HIP, "sa_batch_upload_append: launch: %s", hipGetErrorString(e));
  *out = dev;
  return SA_OK;
}

}  // extern "C"
