// Metadata upload and the attention work plan (host side of libsarathi_attn).
//
// One upload per iteration: the batch metadata and the work plan are packed
// into a caller-provided (pinned) staging buffer and moved with a single
// hipMemcpyAsync, so the device sees everything the kernels need.
//
// Work plan.  A work item is one wavefront's job: up to 32 columns, each a
// (query row, q head) pair of one sequence sharing one kv head, against a key
// range.  Decodes put the q heads of one kv-head group in the columns
// (grouped-query heads share every K/V load); prefill chunks put 32
// consecutive query rows of one q head in the columns.  Long key ranges are
// split so that enough items exist to fill the chip; splits write partial
// (max, sum, unnormalised output) results that a combine pass merges.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "common.h"

namespace {

constexpr int kTargetItems = 4096;      // about 4 wavefronts per SIMD on 256 CUs
constexpr int kMinSplit = 256;          // keys; multiple of the 32-key tile

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

struct Shape {
  int S, D, T, Hq, Hkv, d, group, head_blocks;
  int64_t split_dec, split_chunk;
  int64_t n_items, n_groups, n_partials;
  int bt_stride;
  size_t words_cu, words_ctx, words_slots, words_bt, words_items, words_groups;
  size_t total_words() const {
    return words_cu + words_ctx + words_slots + words_bt + words_items + words_groups;
  }
};

inline size_t pad4(size_t w) { return (w + 3) & ~size_t(3); }   // 16-byte sections

sa_status check_and_shape(const sa_batch* b, int Hq, int Hkv, int d, int num_pages, Shape* sh) {
  if (!b) return sa::fail(SA_ERR_INVALID_ARG, "batch: null pointer");
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
  }
  const int T = b->cu_seqlens_q[S];
  if (b->num_tokens != T) return sa::fail(SA_ERR_INVALID_ARG, "batch: num_tokens %d != cu_seqlens_q[S] %d", b->num_tokens, T);
  if (T > 0 && !b->slot_mapping) return sa::fail(SA_ERR_INVALID_ARG, "batch: null slot_mapping");

  Shape& x = *sh;
  x.S = S; x.D = D; x.T = T; x.Hq = Hq; x.Hkv = Hkv; x.d = d;
  x.group = Hq / Hkv;
  x.head_blocks = int(ceil_div(x.group, sa::kCols));
  x.bt_stride = bt_stride;

  // split lengths: enough items to fill the chip, not so many that partial
  // results cost real traffic
  int64_t dec_keys = 0;
  for (int s = 0; s < D; ++s) dec_keys += int64_t(b->context_lens[s]) + 1;
  dec_keys *= int64_t(Hkv) * x.head_blocks;
  x.split_dec = std::max<int64_t>(kMinSplit, round_up(ceil_div(dec_keys, kTargetItems), kMinSplit));
  int64_t chunk_blocks = 0, chunk_keys = 0;
  for (int s = D; s < S; ++s) {
    const int q = b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s];
    const int ctx = b->context_lens[s];
    for (int r0 = 0; r0 < q; r0 += sa::kCols) {
      const int nr = std::min(sa::kCols, q - r0);
      chunk_blocks += Hq;
      chunk_keys += int64_t(Hq) * (int64_t(ctx) + r0 + nr);
    }
  }
  if (chunk_blocks >= kTargetItems / 2)
    x.split_chunk = int64_t(1) << 40;   // enough column blocks already: no split
  else
    x.split_chunk = std::max<int64_t>(kMinSplit, round_up(ceil_div(chunk_keys, kTargetItems / 2), kMinSplit));

  int64_t items = 0, groups = 0, partials = 0;
  auto count = [&](int64_t keys, int64_t split) {
    const int64_t ns = ceil_div(keys, split);
    items += ns;
    if (ns > 1) { ++groups; partials += ns; }
  };
  for (int s = D; s < S; ++s) {
    const int q = b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s];
    const int ctx = b->context_lens[s];
    for (int h = 0; h < Hq; ++h)
      for (int r0 = 0; r0 < q; r0 += sa::kCols) count(int64_t(ctx) + r0 + std::min(sa::kCols, q - r0), x.split_chunk);
  }
  for (int s = 0; s < D; ++s)
    for (int kh = 0; kh < Hkv; ++kh)
      for (int hb = 0; hb < x.head_blocks; ++hb) count(int64_t(b->context_lens[s]) + 1, x.split_dec);
  if (items > (int64_t(1) << 30)) return sa::fail(SA_ERR_INVALID_ARG, "batch: work plan too large");
  x.n_items = items; x.n_groups = groups; x.n_partials = partials;
  x.words_cu = pad4(size_t(S) + 1);
  x.words_ctx = pad4(size_t(S));
  x.words_slots = pad4(size_t(T));
  x.words_bt = pad4(size_t(S) * size_t(bt_stride));
  x.words_items = size_t(items) * sa::kItemWords;
  x.words_groups = size_t(groups) * sa::kGroupWords;
  return SA_OK;
}

void emit_plan(const sa_batch* b, const Shape& x, int32_t* items, int32_t* groups) {
  int64_t it = 0, gi = 0, part = 0;
  auto emit = [&](int s, int kh, int head0, int nrows, int nheads, int row0, int64_t keys, int64_t split) {
    const int64_t ns = (keys + split - 1) / split;
    for (int64_t k = 0; k < ns; ++k) {
      int32_t* w = items + it * sa::kItemWords;
      w[0] = s; w[1] = kh; w[2] = head0; w[3] = nrows | (nheads << 16); w[4] = row0;
      w[5] = int32_t(k * split);
      w[6] = int32_t(std::min<int64_t>(keys, (k + 1) * split));
      w[7] = ns > 1 ? int32_t(part + k) : -1;
      w[8] = ns > 1 ? int32_t(gi) : -1;
      w[9] = w[10] = w[11] = 0;
      ++it;
    }
    if (ns > 1) {
      int32_t* g = groups + gi * sa::kGroupWords;
      g[0] = int32_t(part); g[1] = int32_t(ns); g[2] = g[3] = 0;
      ++gi;
      part += ns;
    }
  };
  // prefill chunks first: their items are the longest
  for (int s = x.D; s < x.S; ++s) {
    const int q = b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s];
    const int ctx = b->context_lens[s];
    for (int h = 0; h < x.Hq; ++h)
      for (int r0 = 0; r0 < q; r0 += sa::kCols) {
        const int nr = std::min(sa::kCols, q - r0);
        emit(s, h / x.group, h, nr, 1, r0, int64_t(ctx) + r0 + nr, x.split_chunk);
      }
  }
  for (int s = 0; s < x.D; ++s)
    for (int kh = 0; kh < x.Hkv; ++kh)
      for (int hb = 0; hb < x.head_blocks; ++hb) {
        const int h0 = hb * sa::kCols;
        emit(s, kh, kh * x.group + h0, 1, std::min(sa::kCols, x.group - h0), 0, int64_t(b->context_lens[s]) + 1,
             x.split_dec);
      }
}

}  // namespace

extern "C" {

sa_status sa_batch_upload_size(const sa_batch* b, int32_t Hq, int32_t Hkv, int32_t d, size_t* bytes) {
  if (!bytes) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload_size: null bytes");
  Shape x;
  // page ids are checked at upload time; here any id is accepted
  sa_status st = check_and_shape(b, Hq, Hkv, d, 0x7fffffff, &x);
  if (st != SA_OK) return st;
  *bytes = x.total_words() * sizeof(int32_t);
  return SA_OK;
}

sa_status sa_batch_upload(const sa_batch* b, int32_t Hq, int32_t Hkv, int32_t d, int32_t num_pages,
                          void* host_staging, void* dev_buf, size_t bytes, void* stream, sa_batch_dev* out) {
  if (!out) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload: null out");
  if (num_pages < 1) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload: num_pages %d", num_pages);
  Shape x;
  sa_status st = check_and_shape(b, Hq, Hkv, d, num_pages, &x);
  if (st != SA_OK) return st;
  const size_t need = x.total_words() * sizeof(int32_t);
  if (bytes < need) return sa::fail(SA_ERR_CAPACITY, "sa_batch_upload: needs %zu bytes, got %zu", need, bytes);
  if (!host_staging || !dev_buf) return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload: null buffer");
  if ((reinterpret_cast<uintptr_t>(dev_buf) & 15) || (reinterpret_cast<uintptr_t>(host_staging) & 15))
    return sa::fail(SA_ERR_INVALID_ARG, "sa_batch_upload: buffers must be 16-byte aligned");

  int32_t* h = static_cast<int32_t*>(host_staging);
  int32_t* cu = h;
  int32_t* ctx = cu + x.words_cu;
  int32_t* slots = ctx + x.words_ctx;
  int32_t* bt = slots + x.words_slots;
  int32_t* items = bt + x.words_bt;
  int32_t* groups = items + x.words_items;
  std::memcpy(cu, b->cu_seqlens_q, sizeof(int32_t) * size_t(x.S + 1));
  if (x.S) std::memcpy(ctx, b->context_lens, sizeof(int32_t) * size_t(x.S));
  if (x.T) std::memcpy(slots, b->slot_mapping, sizeof(int32_t) * size_t(x.T));
  for (int s = 0; s < x.S; ++s) {
    const int32_t* row = b->block_tables + size_t(s) * size_t(b->max_blocks_per_seq);
    int32_t* dst = bt + size_t(s) * size_t(x.bt_stride);
    const int kv = b->context_lens[s] + b->cu_seqlens_q[s + 1] - b->cu_seqlens_q[s];
    const int np = (kv + sa::kPageSize - 1) / sa::kPageSize;
    std::memcpy(dst, row, sizeof(int32_t) * size_t(np));
    std::fill(dst + np, dst + x.bt_stride, 0);   // never read by the kernels
  }
  emit_plan(b, x, items, groups);

  hipError_t e = hipMemcpyAsync(dev_buf, host_staging, need, hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return sa::fail(SA_ERR_HIP, "sa_batch_upload: hipMemcpyAsync: %s", hipGetErrorString(e));

  const int32_t* dv = static_cast<const int32_t*>(dev_buf);
  out->cu_seqlens_q = dv;
  out->context_lens = dv + x.words_cu;
  out->slot_mapping = out->context_lens + x.words_ctx;
  out->block_tables = out->slot_mapping + x.words_slots;
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
  out->reserved = 0;
  return SA_OK;
}

}  // extern "C"
