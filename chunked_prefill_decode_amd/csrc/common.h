// Internal helpers shared by the host translation units of libsarathi_attn.
#pragma once

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
// is one wavefront's job: a block of up to 32 "columns" (query row, q head)
// of one sequence that share one kv head, against the key range [k0, k1).
//   [0] sequence index            [1] kv head
//   [2] q head of column 0        [3] nrows | (nheads << 16); column c is
//                                     row row0 + c / nheads, head head0 + c % nheads
//   [4] row0 (offset inside the sequence's q rows)
//   [5] k0 (multiple of 32)       [6] k1 (exclusive)
//   [7] partial index, or -1 when the item covers every visible key and
//       writes the final bf16 output itself
//   [8] split group index, or -1  [9..11] unused
constexpr int kItemWords = 12;
// Split group: [0] first partial index [1] number of splits [2..3] unused.
constexpr int kGroupWords = 4;
constexpr int kCols = 32;                 // columns per work item (MFMA N = 32)
constexpr int kKeyTile = 32;              // keys per inner step

// Workspace of sa_hybrid_attn:
//   int32 counters[num_groups] (padded to 256 bytes): split arrivals; zero
//         before the first call, and every completed call leaves them zero
//   float ml[num_partials][32][2]        (running max in log2 units, sum)
//   float o [num_partials][32][head_dim] (unnormalised output)
inline size_t counter_bytes(int64_t num_groups) { return size_t((num_groups * 4 + 255) / 256 * 256); }
inline size_t workspace_bytes(int64_t num_groups, int64_t num_partials, int head_dim) {
  return counter_bytes(num_groups) + size_t(num_partials) * kCols * (2 + head_dim) * sizeof(float);
}

}  // namespace sa
