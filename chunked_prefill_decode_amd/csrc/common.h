// Internal helpers shared by the host translation units of libsarathi_attn.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "sarathi_attn.h"

namespace sa {

// Thread-local text of the last failure, returned by sa_last_error().
std::string& last_error();

// Records a failure message and returns the status, so call sites can write
// `return fail(SA_ERR_INVALID_ARG, "...", ...)`.
inline sa_status fail(sa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error() = buf;
  return st;
}

constexpr int kPageSize = 16;

// Work plan packed after the metadata in the uploaded buffer.  One work item
// is one workgroup (4 wavefronts) of the attention kernel.  A "column" is a
// (query row, q head) pair; every column of an item reads the same kv head.
//   [0] kind: kDecodeItem -- one query row; the columns are q heads
//           head0 .. head0+nheads-1 of one kv-head group and the 4 waves
//           split the key range, merging through LDS;
//         kChunkItem -- column blocks [3] .. [3]+[4]-1 of a prefill chunk
//           and kv head: block i is the 32 query rows of row block i / g of
//           q head kvhead*g + i % g (g = Hq / Hkv); wave w serves block
//           [3] + w, and all waves walk the same keys, so they share every
//           K/V tile.
//   [1] sequence index   [2] kv head   [3] head0 / first block   [4] nheads / blocks
//   [5] row0             [6] nrows     [7] k0 (multiple of 32)   [8] k1
//   [9] split index k, or -1 when the item covers every visible key and
//       writes the final bf16 output itself
//   [10] first split group of the item (decode: 1 group; chunk: one group
//        per column block, consecutive), or -1   [11] unused
//   kDecodeGroupItem -- up to 4 whole decodes whose column block covers
//           their kv group (g <= 32): bits 4w .. 4w+3 of [1] name the decode j
//           that wave w serves (a decode's waves are consecutive); decode j
//           is sequence [2 + 2j], kv head [3 + 2j]; never split.
constexpr int kItemWords = 12;
constexpr int kDecodeItem = 0;
constexpr int kChunkItem = 1;
constexpr int kDecodeGroupItem = 2;
// Split group: one column block whose keys are split over several items.
//   [0] first partial index  [1] number of splits  [2] sequence index
//   [3] head0  [4] nh  [5] row0  [6] nrows  [7] unused
// Column c of the block is query row row0 + c / nh of the sequence, q head
// head0 + c % nh (decode blocks: nh heads of one row; chunk blocks: nh = 1).
constexpr int kGroupWords = 8;
// Most splits of one column block: the merge kernel keeps one weight per split
// and column in LDS (its table has this many rows).
constexpr int kMaxSplits = 64;
constexpr int kCols = 32;                 // max columns per column block
constexpr int kKeyTile = 32;              // keys per inner step
constexpr int kWaves = 4;                 // wavefronts per workgroup
// Column blocks per wavefront of a chunk item (two at d = 64, one at d = 128)
// and per chunk item.
constexpr int chunk_blocks_per_wave(int head_dim) { return head_dim == 64 ? 2 : 1; }
constexpr int chunk_blocks_per_item(int head_dim) { return kWaves * chunk_blocks_per_wave(head_dim); }

// Workspace of sa_hybrid_attn: partial results of split column blocks,
//   float ml[num_partials][32][2]        (running max in log2 units, sum)
//   float o [num_partials][32][head_dim] (unnormalised output)
inline size_t workspace_bytes(int64_t num_partials, int head_dim) {
  return size_t(num_partials) * kCols * (2 + head_dim) * sizeof(float);
}

// Enqueues on `st` a kernel copying `bytes` (a multiple of 16; both ends
// 16-byte aligned) from pinned host memory, given by its device address, to
// device memory (kernels.hip).
hipError_t copy_pinned_to_device(const void* src_dev, void* dst, size_t bytes, hipStream_t st);

// Enqueues on `st` one kernel doing copy_pinned_to_device(src_dev, dst,
// bytes) and the K/V append of sa_kv_append with the slot mapping read from
// slots_dev (device address of pinned host memory); d is 64 or 128, the
// tensors 16-byte aligned (kernels.hip).
hipError_t upload_append(const void* src_dev, void* dst, size_t bytes, const int32_t* slots_dev, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache, int T, int Hkv, int d, int num_pages,
                         hipStream_t st);

}  // namespace sa
