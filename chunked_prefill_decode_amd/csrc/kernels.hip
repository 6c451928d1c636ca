// gfx950 kernels of libsarathi_attn: paged KV append and hybrid-batch attention.
//
// Attention of a hybrid batch ("Sarathi-Serve：以 chunked-prefills 与 stall-free
// batching 驯服 LLM 推理的吞吐—延迟权衡", GPU / 系统数据路径 steps ③-⑤): single-token
// decodes and prefill chunks run in one step; a chunk row at absolute position
// p attends to keys 0..p of its own prompt (earlier chunks are re-read from the
// paged cache) and a decode attends to its whole history ("In-flight
// Batching", 技术原理).  All K/V reads go through 16-token pages.
//
// A wavefront owns a column block: up to 32 (or 16) columns, each a (query
// row, q head) pair that reads one kv head.  Per 32-key tile it computes
// S^T = K * Q^T on the bf16 matrix cores (rows = keys, columns = the block's
// columns), an online softmax in fp32 (running max in log2 units, exp2), and
// O^T += V^T * P^T on the matrix cores.  S^T keeps a column's scores inside
// one lane and its twins, so the softmax reductions need one or two
// cross-lane exchanges.  The K rows fed to the first product are permuted so
// that each lane ends up holding 8 *consecutive* keys of its column, which is
// exactly the B-operand layout of the second product; V is stored dim-major
// inside a page, so its A operand is one 16-byte load.  The online softmax is
// the published streaming-softmax method (Milakov & Gimelshein, 2018) as used
// by tiled attention kernels.
//
// Workgroups (4 wavefronts) run the items of the host plan:
//   decode items -- the 4 waves take interleaved key tiles of one
//     (decode, kv head) column block and merge their softmax states in LDS;
//   decode-group items -- up to 4 whole decodes, each served by a run of
//     consecutive waves and merged the same way;
//   chunk items -- each wave serves one (d = 128) or two (d = 64) column
//     blocks of a prefill chunk (32 query rows of one q head) over the same
//     keys; every K/V tile is staged once per workgroup in an LDS ring by
//     direct global->LDS loads and read by all four waves.
// Column blocks split over several items leave partial states that
// merge_kernel combines.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>
#include <vector>

#include "common.h"

// Workspace of sa_hybrid_attn_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends (split partials only; no initialisation).
static constexpr size_t kStaticWorkspaceBytes = SA_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }
// K/V loads of the decode path read each cache byte once per step.  With NT
// they are non-temporal, which streams from HBM markedly faster on this chip
// than loads that allocate in the caches (a plain streaming kernel: ~7.0
// against ~4.7 TB/s); the plan turns it on for HBM-bound batches.
template <bool NT>
__device__ __forceinline__ bf16x8 load8_kv(const uint16_t* p) {
  if (NT) return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  return load8(p);
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read-only metadata (block tables, work plan, sequence offsets) is never
// written while a kernel runs, so it is read through the constant address
// space: wave-uniform reads become scalar loads, which do not wait on the
// vector-memory counter that tracks the K/V loads in flight.
typedef __attribute__((address_space(4))) const int32_t cint;
__device__ __forceinline__ int ld_meta(const int32_t* p, int64_t i) { return ((cint*)p)[i]; }

// Zero the bf16 elements of a V^T fragment whose keys (first + e) are at or
// past kv_len: cache slots past the sequence end may hold anything (NaN).
__device__ __forceinline__ bf16x8 clip_keys(bf16x8 v, int first, int kv_len) {
  if (first + 8 <= kv_len) return v;
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (first + e >= kv_len) u[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
  return __builtin_bit_cast(bf16x8, u);
}

// 4 floats -> 4 bf16 (round to nearest even), packed in 8 bytes.
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  f32x8 t{};
  t[0] = a; t[1] = b; t[2] = c; t[3] = d;
  const u32x4 u = __builtin_bit_cast(u32x4, __builtin_convertvector(t, bf16x8));
  return u32x2{u[0], u[1]};
}

// ---------------------------------------------------------------- append ---
// One workgroup per (16 consecutive tokens, kv head).  K rows are copied as
// 16-byte pieces (token-major in the page, like the input).  V goes through
// LDS and leaves dim-major: the 16 lanes of a quarter-wave take the 16 tokens
// of one dim, so when those tokens fill consecutive slots of a page (a
// prefill chunk) their 2-byte stores form whole 32-byte rows of the page.
// The 16 slots are fetched once into LDS, so slot_mapping may also be host
// memory read through its device address (the fused upload + append).
constexpr int kAppendTokens = 16;
template <int D>
struct AppendLds {
  uint16_t vt[kAppendTokens * (D + 8)];   // padded rows
  int32_t slot[kAppendTokens];
};

template <int D>
__device__ __forceinline__ void append_rows(int t0, int kh, const uint16_t* __restrict__ k_new,
                                            const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_cache,
                                            uint16_t* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping,
                                            int T, int Hkv, int64_t num_slots, AppendLds<D>& sh) {
  constexpr int G = D / 8;                             // 16-byte pieces per row
  constexpr int LD = D + 8;
  static_assert(kAppendTokens * G <= 256, "one K/V piece per thread");
  if (threadIdx.x < kAppendTokens) {
    const int t = t0 + threadIdx.x;
    sh.slot[threadIdx.x] = t < T ? slot_mapping[t] : -1;
  }
  const int tok = threadIdx.x / G, grp = threadIdx.x - tok * G, t = t0 + tok;
  const bool piece = threadIdx.x < kAppendTokens * G && t < T;
  u32x4 kp = u32x4{0u, 0u, 0u, 0u};
  if (piece) {
    const int64_t src = (int64_t(t) * Hkv + kh) * D + grp * 8;
    *reinterpret_cast<u32x4*>(sh.vt + tok * LD + grp * 8) = *reinterpret_cast<const u32x4*>(v_new + src);
    kp = *reinterpret_cast<const u32x4*>(k_new + src);
  }
  __syncthreads();
  if (piece) {
    const int32_t slot = sh.slot[tok];
    if (slot >= 0 && int64_t(slot) < num_slots)
      *reinterpret_cast<u32x4*>(k_cache + ((int64_t(slot >> 4) * Hkv + kh) * 16 + (slot & 15)) * D + grp * 8) = kp;
  }
  const int vtok = threadIdx.x & (kAppendTokens - 1);
  const int32_t slot = sh.slot[vtok];
  if (slot < 0 || int64_t(slot) >= num_slots) return;
  uint16_t* dst = v_cache + ((int64_t(slot >> 4) * Hkv + kh) * D) * 16 + (slot & 15);
  for (int dim = threadIdx.x / kAppendTokens; dim < D; dim += 256 / kAppendTokens) dst[dim * 16] = sh.vt[vtok * LD + dim];
}

template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new,
                                                        uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                                        const int32_t* __restrict__ slot_mapping, int T, int Hkv,
                                                        int64_t num_slots) {
  __shared__ __attribute__((aligned(16))) AppendLds<D> sh;
  append_rows<D>(blockIdx.x * kAppendTokens, blockIdx.y, k_new, v_new, k_cache, v_cache, slot_mapping, T, Hkv,
                 num_slots, sh);
}

// ------------------------------------------------------------- attention ---
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* cu_q;
  const int32_t* ctx_lens;
  const int32_t* bt;
  const int32_t* bt_off;
  const int32_t* items;
  const int32_t* groups;
  uint16_t* out;
  float* part_ml;
  float* part_o;
  int Hq;
  int Hkv;
  int group;          // Hq / Hkv
  int window;         // sliding window in keys (the row at p sees p-window+1 .. p); 0 = none
  float scale_log2;   // softmax_scale * log2(e)
};

// Paged K/V of one (sequence, kv head).
struct KvView {
  const uint16_t* k;       // k_cache + kv-head offset
  const uint16_t* v;       // v_cache + kv-head offset
  const int32_t* bt;       // the sequence's block-table row
  int64_t pstride;         // elements per page (all kv heads)
  int kv_len;              // keys that exist: context + q_len
};

// Physical pages of the two 16-key halves of the tile at kt (wave-uniform,
// scalar loads); a half past the sequence end gets page 0 and is never read.
struct Pages { int p0, p1; };
__device__ __forceinline__ Pages tile_pages(const KvView& kv, int kt) {
  Pages p;
  p.p0 = kt < kv.kv_len ? ld_meta(kv.bt, kt >> 4) : 0;
  p.p1 = kt + 16 < kv.kv_len ? ld_meta(kv.bt, (kt >> 4) + 1) : 0;
  return p;
}

// Cross-lane reductions over lanes l and l^32 / l^16.  (The gfx950 lane-swap
// instructions gave wrong reductions inside this kernel although a stand-alone
// check matched their documented semantics, so the LDS-crossbar shuffle is
// used instead.)
__device__ __forceinline__ float max_x32(float v) { return fmaxf(v, __shfl_xor(v, 32)); }
__device__ __forceinline__ float max_x16(float v) { return fmaxf(v, __shfl_xor(v, 16)); }
__device__ __forceinline__ float sum_x32(float v) { return v + __shfl_xor(v, 32); }
__device__ __forceinline__ float sum_x16(float v) { return v + __shfl_xor(v, 16); }

// Q enters the matrix cores with its own bf16 bits; the scores are scaled by
// c = softmax_scale * log2(e) in fp32 (one multiply per score), so that the
// softmax runs in log2 units.  (Rounding Q * c to bf16 instead would put a
// relative error of 2^-9 on every score, which ruins rows whose scores span
// hundreds of log2 units.)

template <int LO, int N, int M>
__device__ __forceinline__ float tree_sum_part(const float (&v)[M]) {
  if constexpr (N == 1) return v[LO];
  else return tree_sum_part<LO, N / 2>(v) + tree_sum_part<LO + N / 2, N - N / 2>(v);
}
template <int N>
__device__ __forceinline__ float tree_sum(const float (&v)[N]) { return tree_sum_part<0, N>(v); }
template <int N>
__device__ __forceinline__ float tree_max(const float (&v)[N]) {
  float r = fmaxf(fmaxf(v[0], v[1]), v[2]);
#pragma unroll
  for (int j = 3; j + 1 < N; j += 2) r = fmaxf(fmaxf(r, v[j]), v[j + 1]);
  if (N % 2 == 0) r = fmaxf(r, v[N - 1]);
  return r;
}

// Online softmax state of one column, lazily rescaled.  A lane turns its
// unscaled scores r into s - m = r * c - m (log2 units) with one fused
// multiply-add each.
// The running max m (log2 units) is raised only when a tile's score exceeds
// it by more than 2^8 in the exp2 domain: the weights then stay below 256,
// which fp32 accumulation and bf16 weights hold with full relative precision,
// and almost every tile skips the cross-lane max and the accumulator rescale.
// Until a column has seen a visible key, m = 0 and the column is not started.
constexpr float kLazyLog2 = 8.f;

// Per-column softmax state: thr is the score (minus m) above which m must be
// raised: kLazyLog2 once the column has started, -inf before.
struct SoftmaxState {
  float m, l, thr;
  __device__ __forceinline__ void init() { m = 0.f; l = 0.f; thr = -INFINITY; }
  __device__ __forceinline__ bool started() const { return thr != -INFINITY; }
  __device__ __forceinline__ float log2_max() const { return started() ? m : -INFINITY; }
};

// Handles a tile whose scores (minus m) are sv: if any column of the wave must
// raise its max, the column max is taken across the lanes holding the column
// (colmax), m and the accumulators are rescaled and sv is shifted to the new m.
// The rescale itself, given the lane's max of sv (the rare path).
template <int NV, class Acc, int NA, class ColMax>
__device__ __forceinline__ void rescale(float (&sv)[NV], float lmax, SoftmaxState& st, Acc (&o)[NA],
                                        ColMax colmax) {
  const float cmax = colmax(lmax);
  const bool need = st.started() ? cmax > 0.f : cmax > -INFINITY;
  const float delta = need ? cmax : 0.f;
  const float alpha = __builtin_amdgcn_exp2f(-delta);
  st.m += delta;
  if (need) st.thr = kLazyLog2;
  st.l *= alpha;
#pragma unroll
  for (int i = 0; i < NA; ++i) o[i] *= alpha;
#pragma unroll
  for (int j = 0; j < NV; ++j) sv[j] -= delta;
}
template <int NV, class Acc, int NA, class ColMax>
__device__ __forceinline__ void lazy_rescale(float (&sv)[NV], SoftmaxState& st, Acc (&o)[NA], ColMax colmax) {
  const float lmax = tree_max(sv);
  if (__builtin_amdgcn_ballot_w64(lmax > st.thr)) rescale(sv, lmax, st, o, colmax);
}

// ---- 32-column block: v_mfma_f32_32x32x16_bf16 ----
// Output register j of lane l (h = l / 32) is row 8(j/4) + 4h + j%4 of the
// S^T tile; K row r = 8a + 4h + b is fed key 16(a/2) + 8h + 4(a%2) + b, so that
// register j holds key 16(j/8) + 8h + j%8: keys 8h..8h+7 in registers 0..7 and
// 16+8h..16+8h+7 in registers 8..15.
__device__ __forceinline__ int key_of_row32(int r) {
  const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

template <int D>
struct Block32 {
  static constexpr int KB = D / 16;   // k-blocks of the S product
  static constexpr int DB = D / 32;   // 32-dim output blocks
  struct Frag {
    bf16x8 kf[KB];
    bf16x8 vf[2][DB];
  };
  bf16x8 qf[KB];
  f32x16 o[DB];
  SoftmaxState sm;
  float c;       // softmax_scale * log2(e)
  int col, hi, krow;

  __device__ __forceinline__ void init(int lane, const uint16_t* qrow, bool valid, float scale_log2) {
    col = lane & 31;
    hi = lane >> 5;
    krow = key_of_row32(col);
    c = scale_log2;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qf[kb] = valid ? load8(qrow + 16 * kb + 8 * hi) : zero8();
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    sm.init();
  }
  __device__ __forceinline__ float log2_max() const { return sm.log2_max(); }

  // Issue the loads of the 32-key tile at kt (a multiple of 32).
  template <bool NT>
  __device__ __forceinline__ void load(const KvView& kv, int kt, Pages pg, Frag& f) const {
    const int key = kt + krow;
    if (key < kv.kv_len) {
      const uint16_t* kp = kv.k + int64_t(krow >= 16 ? pg.p1 : pg.p0) * kv.pstride + (key & 15) * D + 8 * hi;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) f.kf[kb] = load8_kv<NT>(kp + 16 * kb);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) f.kf[kb] = zero8();
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kb0 = kt + 16 * ks;   // page-aligned half tile; this lane's keys kb0+8hi .. +7
      if (kb0 < kv.kv_len) {
        const uint16_t* vp = kv.v + int64_t(ks ? pg.p1 : pg.p0) * kv.pstride + col * 16 + 8 * hi;
#pragma unroll
        for (int db = 0; db < DB; ++db) f.vf[ks][db] = clip_keys(load8_kv<NT>(vp + 32 * 16 * db), kb0 + 8 * hi, kv.kv_len);
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) f.vf[ks][db] = zero8();
      }
    }
  }

  // Consume a loaded tile; unless the tile is full, keys >= kend (and with a
  // sliding window, keys < kbeg) are masked.
  // Phases of a tile: the S product (scores minus m), the causal /
  // sequence-end / window mask, the (rare) rescale, and the weights with the
  // P.V product.
  __device__ __forceinline__ f32x16 scores(const Frag& f) const {
    f32x16 sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.kf[0], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int kb = 1; kb < KB; ++kb) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.kf[kb], qf[kb], sacc, 0, 0, 0);
    return sacc;
  }
  template <bool WIN>
  __device__ __forceinline__ void mask(float (&sv)[16], int kt, int kbeg, int kend) const {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = kt + 16 * (j >> 3) + 8 * hi + (j & 7);
      if (key >= kend || (WIN && key < kbeg)) sv[j] = -INFINITY;
    }
  }
  template <bool WIN>
  __device__ __forceinline__ void compute(const Frag& f, int kt, int kbeg, int kend, bool full) {
    const f32x16 sacc = scores(f);
    float sv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) sv[j] = __builtin_fmaf(sacc[j], c, -sm.m);
    if (!full) mask<WIN>(sv, kt, kbeg, kend);
    lazy_rescale(sv, sm, o, [](float v) { return max_x32(v); });
    accumulate(sv, f);
  }
  __device__ __forceinline__ void accumulate(const float (&sv)[16], const Frag& f) {
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) p[j] = __builtin_amdgcn_exp2f(sv[j]);
    sm.l += tree_sum(p);
    f32x8 p0, p1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p0[j] = p[j];
      p1[j] = p[8 + j];
    }
    const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
    const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.vf[0][db], pb0, o[db], 0, 0, 0);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.vf[1][db], pb1, o[db], 0, 0, 0);
    }
  }

  __device__ __forceinline__ float column_sum() const { return sum_x32(sm.l); }
  // The lane's output values come in groups of 4 consecutive dims:
  // group gi = db*4 + jj covers dims 32db + 8jj + 4hi .. +3.
  static constexpr int NG = DB * 4;
  __device__ __forceinline__ int group_dim(int gi) const { return 32 * (gi >> 2) + 8 * (gi & 3) + 4 * hi; }
  __device__ __forceinline__ f32x4 group(int gi) const {
    const int db = gi >> 2, jj = gi & 3;
    return f32x4{o[db][4 * jj], o[db][4 * jj + 1], o[db][4 * jj + 2], o[db][4 * jj + 3]};
  }
  __device__ __forceinline__ bool column_writer() const { return hi == 0; }
};

// ---- 16-column block: v_mfma_f32_16x16x32_bf16 ----
// Output register j of lane l (q = l / 16) is row 4q + j of an S^T tile; two
// tiles t = 0, 1 cover 32 keys, and K row r of tile t is fed key
// 8(r/4) + 4t + r%4, so lane l holds keys 8q .. 8q+7 (tile 0: 8q+j, tile 1:
// 8q+4+j) -- the B-operand layout of the P*V product.
template <int D>
struct Block16 {
  static constexpr int KB = D / 32;   // k-blocks of the S product (32 dims)
  static constexpr int DB = D / 16;   // 16-dim output blocks
  struct Frag {
    bf16x8 kf[2][KB];
    bf16x8 vf[DB];
  };
  bf16x8 qf[KB];
  f32x4 o[DB];
  SoftmaxState sm;
  float c;       // softmax_scale * log2(e)
  int col, qd;

  __device__ __forceinline__ void init(int lane, const uint16_t* qrow, bool valid, float scale_log2) {
    col = lane & 15;
    qd = lane >> 4;
    c = scale_log2;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qf[kb] = valid ? load8(qrow + 32 * kb + 8 * qd) : zero8();
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    sm.init();
  }
  __device__ __forceinline__ float log2_max() const { return sm.log2_max(); }

  template <bool NT>
  __device__ __forceinline__ void load(const KvView& kv, int kt, Pages pg, Frag& f) const {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kin = 8 * (col >> 2) + 4 * t + (col & 3);   // key inside the tile
      if (kt + kin < kv.kv_len) {
        const uint16_t* kp = kv.k + int64_t(kin >= 16 ? pg.p1 : pg.p0) * kv.pstride + (kin & 15) * D + 8 * qd;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) f.kf[t][kb] = load8_kv<NT>(kp + 32 * kb);
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) f.kf[t][kb] = zero8();
      }
    }
    const int kfirst = kt + 8 * qd;   // this lane's keys kfirst .. kfirst+7
    if (kfirst < kv.kv_len) {
      const uint16_t* vp = kv.v + int64_t(qd >= 2 ? pg.p1 : pg.p0) * kv.pstride + col * 16 + 8 * (qd & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) f.vf[db] = clip_keys(load8_kv<NT>(vp + 16 * 16 * db), kfirst, kv.kv_len);
    } else {
#pragma unroll
      for (int db = 0; db < DB; ++db) f.vf[db] = zero8();
    }
  }

  template <bool WIN>
  __device__ __forceinline__ void compute(const Frag& f, int kt, int kbeg, int kend, bool full) {
    f32x4 s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.kf[0][0], qf[0], f32x4{}, 0, 0, 0);
    f32x4 s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.kf[1][0], qf[0], f32x4{}, 0, 0, 0);
#pragma unroll
    for (int kb = 1; kb < KB; ++kb) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.kf[0][kb], qf[kb], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.kf[1][kb], qf[kb], s1, 0, 0, 0);
    }
    float sv[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = __builtin_fmaf(s0[j], c, -sm.m);
      sv[4 + j] = __builtin_fmaf(s1[j], c, -sm.m);
    }
    if (!full) {
      const int kfirst = kt + 8 * qd;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (kfirst + j >= kend || (WIN && kfirst + j < kbeg)) sv[j] = -INFINITY;
    }
    lazy_rescale(sv, sm, o, [](float v) { return max_x32(max_x16(v)); });
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(sv[j]);
    sm.l += tree_sum(p);
    f32x8 pv;
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = p[j];
    const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.vf[db], pb, o[db], 0, 0, 0);
  }

  __device__ __forceinline__ float column_sum() const { return sum_x32(sum_x16(sm.l)); }
  // group gi = db covers dims 16db + 4qd .. +3.
  static constexpr int NG = DB;
  __device__ __forceinline__ int group_dim(int gi) const { return 16 * gi + 4 * qd; }
  __device__ __forceinline__ f32x4 group(int gi) const { return o[gi]; }
  __device__ __forceinline__ bool column_writer() const { return qd == 0; }
};

// Walks tiles kt = first, first + step, ... < end with the next tile's loads
// in flight while the current one is computed (two alternating fragments),
// and the page ids two tiles ahead.  A tile inside [full_beg, full_end) needs
// no mask; others mask keys outside [kbeg, kend) (kbeg only with WIN).
// Without PF (register budget too small for two fragments) each tile is
// loaded and consumed in turn.
template <bool PF, bool WIN, bool NT, class Blk>
__device__ __forceinline__ void walk(Blk& b, const KvView& kv, int first, int end, int step, int kbeg, int kend,
                                     int full_beg, int full_end) {
  if (first >= end) return;
  auto full = [&](int kt) { return (!WIN || kt >= full_beg) && kt + 32 <= full_end; };
  if (!PF) {
    for (int kt = first; kt < end; kt += step) {
      typename Blk::Frag f;
      b.template load<NT>(kv, kt, tile_pages(kv, kt), f);
      b.template compute<WIN>(f, kt, kbeg, kend, full(kt));
    }
    return;
  }
  typename Blk::Frag fa, fb;
  Pages pn = tile_pages(kv, first + step);
  b.template load<NT>(kv, first, tile_pages(kv, first), fa);
  for (int kt = first;;) {
    int kn = kt + step;
    Pages pnn = tile_pages(kv, kn + step);
    if (kn < end) b.template load<NT>(kv, kn, pn, fb);
    b.template compute<WIN>(fa, kt, kbeg, kend, full(kt));
    kt = kn;
    if (kt >= end) break;
    kn = kt + step;
    pn = tile_pages(kv, kn + step);
    if (kn < end) b.template load<NT>(kv, kn, pnn, fa);
    b.template compute<WIN>(fb, kt, kbeg, kend, full(kt));
    kt = kn;
    if (kt >= end) break;
  }
}

template <int D>
__device__ __forceinline__ KvView kv_view(const AttnArgs& A, int s, int kh, int kv_len) {
  KvView kv;
  kv.pstride = int64_t(A.Hkv) * 16 * D;
  kv.k = A.k_cache + int64_t(kh) * 16 * D;
  kv.v = A.v_cache + int64_t(kh) * D * 16;
  kv.bt = A.bt + ld_meta(A.bt_off, s);
  kv.kv_len = kv_len;
  return kv;
}

// Writes a finished block's columns: bf16 output, or a partial state.
template <class Blk, int D>
__device__ __forceinline__ void store_block(const AttnArgs& A, const Blk& b, float lsum, bool valid, int64_t out_row,
                                            int head, int part) {
  if (!valid) return;
  if (part < 0) {
    const float inv = 1.f / lsum;
    uint16_t* op = A.out + (out_row * A.Hq + head) * D;
#pragma unroll
    for (int gi = 0; gi < Blk::NG; ++gi) {
      const f32x4 v = b.group(gi);
      *reinterpret_cast<u32x2*>(op + b.group_dim(gi)) = pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    }
  } else {
    float* po = A.part_o + (int64_t(part) * sa::kCols + b.col) * D;
#pragma unroll
    for (int gi = 0; gi < Blk::NG; ++gi) *reinterpret_cast<f32x4*>(po + b.group_dim(gi)) = b.group(gi);
    if (b.column_writer()) {
      float* pm = A.part_ml + (int64_t(part) * sa::kCols + b.col) * 2;
      pm[0] = b.log2_max();
      pm[1] = lsum;
    }
  }
}

// Decode item.  kDecodeItem: the 4 waves split the keys [k0, k1) of one
// column block.  kDecodeGroupItem: up to 4 whole decodes (column blocks
// covering a kv group), each served by a run of consecutive waves.  Each
// block's waves take interleaved key tiles and merge their softmax states in
// LDS.  With a sliding window (WIN) the decode at position ctx sees keys
// ctx-window+1 .. ctx; a whole decode's walk starts at that key's tile.
template <int D, int NCOL, bool WIN, bool NT>
__device__ __forceinline__ void decode_item(const AttnArgs& A, const int32_t* w, float* lds) {
  using Blk = typename std::conditional<NCOL == 16, Block16<D>, Block32<D>>::type;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  int s, kh, head0, nheads, k0, k1, split, g0, wpb, w_first;
  if (ld_meta(w, 0) == sa::kDecodeItem) {
    s = ld_meta(w, 1); kh = ld_meta(w, 2); head0 = ld_meta(w, 3); nheads = ld_meta(w, 4);
    k0 = ld_meta(w, 7); k1 = ld_meta(w, 8); split = ld_meta(w, 9); g0 = ld_meta(w, 10);
    wpb = sa::kWaves;
    w_first = 0;
  } else {
    const int map = ld_meta(w, 1);                // 4 bits per wave: its decode in the item
    const int j = (map >> (4 * wave)) & 15;
    wpb = 0;
    int sub = 0;
#pragma unroll
    for (int i = 0; i < sa::kWaves; ++i)
      if (((map >> (4 * i)) & 15) == j) {
        sub += i < wave;
        ++wpb;
      }
    w_first = wave - sub;                         // a decode's waves are consecutive
    s = ld_meta(w, 2 + 2 * j); kh = ld_meta(w, 3 + 2 * j);
    head0 = kh * A.group; nheads = A.group;
    k0 = 0; k1 = -1; split = -1; g0 = -1;
  }
  const int sub = wave - w_first;                 // this wave's place among its block's waves
  const int ctx = ld_meta(A.ctx_lens, s);
  const int kbeg = WIN ? max(0, ctx - A.window + 1) : 0;   // first visible key
  if (k1 < 0) {
    k0 = kbeg & ~(sa::kKeyTile - 1);
    k1 = ctx + 1;
  }
  const int64_t qrow = ld_meta(A.cu_q, s);
  const KvView kv = kv_view<D>(A, s, kh, ctx + 1);

  Blk b;
  const int c = lane % NCOL;
  const bool valid = c < nheads;
  b.init(lane, A.q + (qrow * A.Hq + head0 + (valid ? c : 0)) * D, valid, A.scale_log2);
  const int kend = valid ? k1 : k0;
  // each wave keeps the next tile's loads in flight (a second register
  // fragment), except for 32-wide blocks at d = 128, where those registers
  // would cost the chunk path, which shares the kernel, occupancy
  walk<NCOL == 16 || D == 64, WIN, NT>(b, kv, k0 + sa::kKeyTile * sub, k1, sa::kKeyTile * wpb, kbeg, kend, kbeg, k1);

  // merge the states of the block's waves: M = max m_w, out = sum 2^(m_w - M) o_w / sum 2^(m_w - M) l_w
  constexpr int LD = D + 4;                        // padded row of the LDS tile
  float* lm = lds;                                 // [4][NCOL]
  float* ll = lm + sa::kWaves * NCOL;              // [4][NCOL]
  float* lo = ll + sa::kWaves * NCOL;              // [4][NCOL][LD]
  const int w0 = w_first;                         // the block's first wave
  const float lsum = b.column_sum();
  const float m2 = b.log2_max();                  // log2 units
  if (b.column_writer()) lm[wave * NCOL + b.col] = m2;
  __syncthreads();
  float M = -INFINITY;
  for (int i = w0; i < w0 + wpb; ++i) M = fmaxf(M, lm[i * NCOL + b.col]);
  const float f = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
  if (b.column_writer()) ll[wave * NCOL + b.col] = lsum * f;
  if (valid) {                                     // padding columns are never read back
    float* my = lo + (wave * NCOL + b.col) * LD;
#pragma unroll
    for (int gi = 0; gi < Blk::NG; ++gi) *reinterpret_cast<f32x4*>(my + b.group_dim(gi)) = b.group(gi) * f;
  }
  __syncthreads();

  constexpr int Q4 = D / 4;
  const int part = split < 0 ? -1 : ld_meta(A.groups, int64_t(g0) * sa::kGroupWords) + split;
  for (int idx = threadIdx.x - 64 * w0; idx < nheads * Q4; idx += 64 * wpb) {
    const int cc = idx / Q4, d4 = (idx - cc * Q4) * 4;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    float L = 0.f, Mc = -INFINITY;
    for (int i = w0; i < w0 + wpb; ++i) {
      acc += *reinterpret_cast<const f32x4*>(lo + (i * NCOL + cc) * LD + d4);
      L += ll[i * NCOL + cc];
      Mc = fmaxf(Mc, lm[i * NCOL + cc]);
    }
    if (part < 0) {
      const float inv = 1.f / L;
      *reinterpret_cast<u32x2*>(A.out + (qrow * A.Hq + head0 + cc) * D + d4) =
          pack4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    } else {
      *reinterpret_cast<f32x4*>(A.part_o + (int64_t(part) * sa::kCols + cc) * D + d4) = acc;
      if (d4 == 0) {
        float* pm = A.part_ml + (int64_t(part) * sa::kCols + cc) * 2;
        pm[0] = Mc;
        pm[1] = L;
      }
    }
  }
}

// ---- chunk workgroups: K/V tiles staged in LDS by direct global->LDS loads ----
// One 32-key tile in LDS (unpadded, XOR-swizzled so that the 16-byte fragment
// reads of 16 consecutive lanes hit distinct banks):
//   K   : 32 rows (keys) x D; 16-byte chunk c of row r sits at c ^ swz_k(r);
//   V^T : two halves (keys 0-15, 16-31), each D rows (dims) x 16 keys; chunk
//         c (8 keys) of dim row d sits at c ^ ((d >> 3) & 1).
// A direct load instruction fills 1 KB (64 lanes x 16 bytes, lane i at byte
// 16 i) and the layout puts every instruction's 1 KB inside one page half, so
// the page base is wave-uniform and each lane's offset is the same for every
// tile.
template <int D>
struct ChunkTile {
  static constexpr int CPR = D / 8;              // 16-byte chunks per K row
  static constexpr int K_ELEMS = 32 * D;
  static constexpr int V_ELEMS = 32 * D;          // two halves of D x 16
  static constexpr int ELEMS = K_ELEMS + V_ELEMS; // one stage (bf16 elements)
  static constexpr int HALF_INSTS = D / 32;       // 1 KB instructions per page half of K (and of V)
  // Tiles computed between two barriers, and tiles resident in the ring (the
  // group being computed plus STAGES - GROUP in flight).  At d = 64 a barrier
  // every 4 tiles with 8 stages (64 KB, still two workgroups per CU) measured
  // 2-4% faster than one per tile with 4 stages on the Falcon-180B TP4 share
  // at B = 1024-2048; at d = 128 the 16 KB tiles leave room for 4 stages only.
  static constexpr int GROUP = D == 64 ? 4 : 1;
  static constexpr int STAGES = D == 64 ? 8 : 4;
  __device__ static __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  // element offset of K row r, logical chunk c
  __device__ static __forceinline__ int k_at(int r, int c) { return r * D + ((c ^ swz_k(r)) << 3); }
  // element offset of V^T half h, dim d, logical chunk c (keys 8c .. 8c+7 of the half)
  __device__ static __forceinline__ int v_at(int h, int d, int c) {
    return K_ELEMS + h * (D * 16) + d * 16 + ((c ^ ((d >> 3) & 1)) << 3);
  }
};

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// Issues this wave's direct loads of the tile at kt into one stage.  The
// workgroup has 4 * HALF_INSTS instructions per tile (K and V, two halves);
// wave w issues the ones numbered w, w+4, ... .  A half past the sequence end
// re-reads the tile's first page instead (those keys are masked; their V
// entries are zeroed before use when the page is the last one), so every tile
// costs every wave the same number of loads.
template <int D>
struct DmaLoader {
  using T = ChunkTile<D>;
  static constexpr int N_INST = 4 * T::HALF_INSTS;      // per tile, whole workgroup
  static constexpr int PER_WAVE = N_INST / sa::kWaves;  // 2 (d=64) or 4 (d=128)
  int lane_off[PER_WAVE];   // element offset inside the page block (K or V) for this lane
  int lds_off[PER_WAVE];    // element offset of the instruction's 1 KB inside a stage
  int half[PER_WAVE];
  bool is_v[PER_WAVE];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int j = wave + sa::kWaves * i;                 // instruction number
      is_v[i] = j >= 2 * T::HALF_INSTS;
      const int jj = is_v[i] ? j - 2 * T::HALF_INSTS : j;  // within K or within V
      half[i] = jj / T::HALF_INSTS;
      const int pos = 64 * (jj % T::HALF_INSTS) + lane;    // chunk position inside the half
      if (!is_v[i]) {
        // K half h = rows 16h .. 16h+15: position -> (row, physical chunk)
        const int r = 16 * half[i] + pos / T::CPR, phys = pos % T::CPR;
        const int c = phys ^ T::swz_k(r);
        lane_off[i] = (r & 15) * D + c * 8;                 // row of the page, logical chunk
        lds_off[i] = 64 * 8 * jj;                            // K half blocks are contiguous
      } else {
        const int d = pos / 2, phys = pos & 1;
        const int c = phys ^ ((d >> 3) & 1);
        lane_off[i] = d * 16 + c * 8;                        // V^T page: dim row, 8 keys
        lds_off[i] = T::K_ELEMS + 64 * 8 * jj;
      }
    }
  }
  __device__ __forceinline__ void issue(const KvView& kv, int kt, Pages pg, uint16_t* stage) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int page = (half[i] == 0 || kt + 16 >= kv.kv_len) ? pg.p0 : pg.p1;
      const uint16_t* src = (is_v[i] ? kv.v : kv.k) + int64_t(page) * kv.pstride + lane_off[i];
      __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)(stage + lds_off[i]), 16, 0, 0);
    }
  }
};

// Waits until at most N direct loads of this wave are outstanding (vmcnt),
// leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier for the direct-load rings: waits for this wave's LDS
// reads and writes only.  __syncthreads() would also wait for every global
// load in flight (its fence covers the direct loads' LDS writes), which
// would leave a single step of loads in flight however deep the ring; the
// wait_vmcnt before the barrier decides which steps must have landed.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__device__ __forceinline__ void read_frag(const uint16_t* stage, const Block32<D>& b, typename Block32<D>::Frag& f) {
  using T = ChunkTile<D>;
#pragma unroll
  for (int kb = 0; kb < Block32<D>::KB; ++kb) f.kf[kb] = load8(stage + T::k_at(b.krow, 2 * kb + b.hi));
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < Block32<D>::DB; ++db) f.vf[ks][db] = load8(stage + T::v_at(ks, 32 * db + b.col, b.hi));
}

// Zero the V^T entries of keys >= kv_len in a staged tile (the sequence's
// last page may hold anything past its end).
template <int D>
__device__ __forceinline__ void clip_stage(uint16_t* stage, int kt, int kv_len) {
  using T = ChunkTile<D>;
  for (int e = threadIdx.x; e < 2 * D * 2; e += 256) {   // (half, dim, chunk) triples
    const int h = e / (2 * D), d = (e / 2) % D, c = e & 1;
    const int first = kt + 16 * h + 8 * c;
    if (first + 8 > kv_len) {
      uint16_t* p = stage + T::v_at(h, d, c);
      *reinterpret_cast<u32x4*>(p) =
          __builtin_bit_cast(u32x4, clip_keys(load8(p), first, kv_len));
    }
  }
}

// Chunk item: column blocks i0 .. i0+cnt-1 of one (sequence, kv head); block
// i is the 32 query rows of row block i / g for q head i % g, and wave w
// serves blocks i0 + BPW*w .. i0 + BPW*w + BPW-1 (BPW = 2 at d = 64, where the
// registers allow it: the two blocks share every K/V fragment, and their
// independent products and softmaxes interleave in the wave).  The workgroup
// walks the keys tile by tile through an LDS ring (d = 128: 4 stages, 3 tiles
// of loads in flight, one barrier per tile; d = 64: 8 stages, a barrier per
// group of 4 tiles, the next 4 in flight); every tile is fetched once and
// read by all four waves.  With a sliding window (WIN) the row at position p sees
// keys p-window+1 .. p: a block computes only the tiles that meet its rows'
// windows, and masks the tiles at either edge of the band.
template <int D, int BPW, bool WIN>
__device__ __forceinline__ void chunk_item(const AttnArgs& A, const int32_t* w, uint16_t* lds) {
  using T = ChunkTile<D>;
  using DL = DmaLoader<D>;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int s = ld_meta(w, 1), kh = ld_meta(w, 2), i0 = ld_meta(w, 3), cnt = ld_meta(w, 4);
  const int k0 = ld_meta(w, 7), k1 = ld_meta(w, 8), split = ld_meta(w, 9), g0 = ld_meta(w, 10);
  const int ctx = ld_meta(A.ctx_lens, s);
  const int64_t qbeg = ld_meta(A.cu_q, s);
  const int qlen = ld_meta(A.cu_q, s + 1) - int(qbeg);
  const KvView kv = kv_view<D>(A, s, kh, ctx + qlen);

  const int last = i0 + cnt - 1;
  const int row0_last = sa::kCols * (last / A.group);
  const int kend_wg = min(k1, ctx + row0_last + min(sa::kCols, qlen - row0_last));
  const int c = lane & 31;

  Block32<D> b[BPW];
  int head[BPW], kend_blk[BPW], kend_col[BPW], full_end[BPW];
  int kbeg_blk[BPW], kbeg_col[BPW], full_beg[BPW];  // window edges (WIN only)
  bool valid[BPW];
  int64_t qrow[BPW];
  int kend_w = k0;                                   // this wave's last visible key + 1
  int kbeg_w = k1;                                   // this wave's first visible key (WIN only)
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int bi = BPW * wave + j;                   // block number inside the item
    const bool active = bi < cnt;
    const int blk = i0 + (active ? bi : 0);
    const int row0 = sa::kCols * (blk / A.group);
    const int nrows = min(sa::kCols, qlen - row0);
    head[j] = kh * A.group + blk % A.group;
    valid[j] = active && c < nrows;
    qrow[j] = qbeg + row0 + (valid[j] ? c : 0);
    b[j].init(lane, A.q + (qrow[j] * A.Hq + head[j]) * D, valid[j], A.scale_log2);
    kend_blk[j] = active ? min(k1, ctx + row0 + nrows) : k0;
    kend_col[j] = valid[j] ? min(k1, ctx + row0 + c + 1) : k0;   // row at position p sees keys <= p
    full_end[j] = min(k1, ctx + row0 + 1);                        // every row of the block sees keys below
    kend_w = max(kend_w, kend_blk[j]);
    if (WIN) {
      kbeg_blk[j] = max(0, ctx + row0 - A.window + 1);            // the block's first row sees keys from here
      kbeg_col[j] = max(0, ctx + row0 + c - A.window + 1);
      full_beg[j] = max(0, ctx + row0 + nrows - A.window);       // every row of the block sees keys from here
      if (active) kbeg_w = min(kbeg_w, kbeg_blk[j]);
    } else {
      kbeg_blk[j] = kbeg_col[j] = full_beg[j] = 0;
    }
  }

  DmaLoader<D> ld;
  ld.init(wave, lane);
  // stale LDS may hold any bits: V of halves never loaded must read as zeros
  for (int e = threadIdx.x * 8; e < T::STAGES * T::ELEMS; e += 256 * 8)
    *reinterpret_cast<u32x4*>(lds + e) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  if constexpr (T::GROUP == 1) {
    constexpr int AHEAD = T::STAGES - 1;                          // tiles in flight
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      const int kt = k0 + 32 * i;
      if (kt < kend_wg) ld.issue(kv, kt, tile_pages(kv, kt), lds + i * T::ELEMS);
    }
    typename Block32<D>::Frag f;
    int st = 0;
    // page ids of the next refill, fetched one tile ahead (at the end of the
    // previous tile's products) so that their scalar loads are off the issue path
    Pages pg_next = k0 + 32 * AHEAD < kend_wg ? tile_pages(kv, k0 + 32 * AHEAD) : Pages{0, 0};
    for (int kt = k0; kt < kend_wg; kt += 32) {
      // this tile's loads were issued AHEAD-1 tiles before the most recent ones
      if (kt + 32 * (AHEAD - 1) < kend_wg) wait_vmcnt<DL::PER_WAVE * (AHEAD - 1)>();
      else wait_vmcnt<0>();
      lds_barrier();
      uint16_t* stage = lds + st * T::ELEMS;
      if (kt + 32 > kv.kv_len) {               // the sequence ends inside this tile
        clip_stage<D>(stage, kt, kv.kv_len);
        __syncthreads();
      }
      // refill the stage computed in the previous step (every wave is past it)
      const int kn = kt + 32 * AHEAD;
      if (kn < kend_wg) ld.issue(kv, kn, pg_next, lds + ((st + AHEAD) % T::STAGES) * T::ELEMS);
      if (kt < kend_w && (!WIN || kt + 32 > kbeg_w)) {
        read_frag<D>(stage, b[0], f);          // fragment layout depends on the lane only
#pragma unroll
        for (int j = 0; j < BPW; ++j)
          if (kt < kend_blk[j] && (!WIN || kt + 32 > kbeg_blk[j]))
            b[j].template compute<WIN>(f, kt, kbeg_col[j], kend_col[j],
                                       (!WIN || kt >= full_beg[j]) && kt + 32 <= full_end[j]);
      }
      if (kn + 32 < kend_wg) pg_next = tile_pages(kv, kn + 32);
      st = (st + 1) % T::STAGES;
    }
  } else {
    // Groups of G tiles between barriers: at a group's start every wave's loads
    // of the group's tiles have landed (the vmcnt wait, then the barrier), and
    // every wave is past the previous group, whose stages are refilled.
    constexpr int G = T::GROUP;
    constexpr int AHEAD = T::STAGES - G;                        // tiles in flight beyond the group
    static_assert(AHEAD >= G, "a refill must land beyond the group being computed");
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      const int kt = k0 + 32 * i;
      if (kt < kend_wg) ld.issue(kv, kt, tile_pages(kv, kt), lds + i * T::ELEMS);
    }
    typename Block32<D>::Frag f;
    int st = 0;
    Pages pg_next[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
      pg_next[g] = k0 + 32 * (AHEAD + g) < kend_wg ? tile_pages(kv, k0 + 32 * (AHEAD + g)) : Pages{0, 0};
    for (int kt = k0; kt < kend_wg; kt += 32 * G) {
      // loads issued after the group's tiles: those of AHEAD - G tiles, when all exist
      if (kt + 32 * (AHEAD - 1) < kend_wg) wait_vmcnt<DL::PER_WAVE * (AHEAD - G)>();
      else wait_vmcnt<0>();
      lds_barrier();
      bool clipped = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int t = kt + 32 * g;
        if (t < kend_wg && t + 32 > kv.kv_len) {   // the sequence ends inside this tile
          clip_stage<D>(lds + ((st + g) % T::STAGES) * T::ELEMS, t, kv.kv_len);
          clipped = true;
        }
      }
      if (clipped) __syncthreads();
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int kn = kt + 32 * (AHEAD + g);
        if (kn < kend_wg) ld.issue(kv, kn, pg_next[g], lds + ((st + AHEAD + g) % T::STAGES) * T::ELEMS);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int t = kt + 32 * g;
        if (t < kend_wg && t < kend_w && (!WIN || t + 32 > kbeg_w)) {
          read_frag<D>(lds + ((st + g) % T::STAGES) * T::ELEMS, b[0], f);
#pragma unroll
          for (int j = 0; j < BPW; ++j)
            if (t < kend_blk[j] && (!WIN || t + 32 > kbeg_blk[j]))
              b[j].template compute<WIN>(f, t, kbeg_col[j], kend_col[j],
                                         (!WIN || t >= full_beg[j]) && t + 32 <= full_end[j]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int kn = kt + 32 * (AHEAD + G + g);
        if (kn < kend_wg) pg_next[g] = tile_pages(kv, kn);
      }
      st = (st + G) % T::STAGES;
    }
  }
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int bi = BPW * wave + j;
    if (bi >= cnt) break;
    const float lsum = b[j].column_sum();
    const int part = split < 0 ? -1 : ld_meta(A.groups, int64_t(g0 + bi) * sa::kGroupWords) + split;
    store_block<Block32<D>, D>(A, b[j], lsum, valid[j], qrow[j], head[j], part);
  }
}

template <int D, int NCOL, bool WIN, bool NT>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs A) {
  constexpr int kMergeBytes = (2 * sa::kWaves * NCOL + sa::kWaves * NCOL * (D + 4)) * 4;
  constexpr int kChunkBytes = ChunkTile<D>::STAGES * ChunkTile<D>::ELEMS * 2;
  __shared__ __attribute__((aligned(16))) char lds[kMergeBytes > kChunkBytes ? kMergeBytes : kChunkBytes];
  const int32_t* w = A.items + int64_t(blockIdx.x) * sa::kItemWords;
  if (ld_meta(w, 0) != sa::kChunkItem)
    decode_item<D, NCOL, WIN, NT>(A, w, reinterpret_cast<float*>(lds));
  else
    chunk_item<D, sa::chunk_blocks_per_wave(D), WIN>(A, w, reinterpret_cast<uint16_t*>(lds));
}

// --------------------------------------------------------------- merge ---
// One workgroup per split group: with M the largest running max,
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i.  The splits' (m, l)
// are fetched in one step into LDS and turned into weights there, and the
// loop over splits is unrolled so that the partial loads of several splits
// are in flight together.
constexpr int kMergeMaxSplits = sa::kMaxSplits;   // the plan never splits a block more
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const int32_t* __restrict__ groups,
                                                    const int32_t* __restrict__ cu_q,
                                                    const float* __restrict__ part_ml,
                                                    const float* __restrict__ part_o, uint16_t* __restrict__ out,
                                                    int Hq) {
  __shared__ float ms[kMergeMaxSplits][sa::kCols];    // m_i per split and column
  __shared__ float wgt[kMergeMaxSplits][sa::kCols];   // l_i, then 2^(m_i - M) / L
  const int32_t* g = groups + int64_t(blockIdx.x) * sa::kGroupWords;
  const int p0 = g[0], ns = g[1], s = g[2], head0 = g[3], nh = g[4], row0 = g[5], nrows = g[6];
  const int ncols = nrows * nh;
  const int t = threadIdx.x;
  // every split's (m, l) of every column in one step of independent loads
  for (int e = t; e < ns * sa::kCols; e += 256) {
    const int i = e / sa::kCols, c = e - i * sa::kCols;
    if (c < ncols) {
      const float* pm = part_ml + (int64_t(p0 + i) * sa::kCols + c) * 2;
      ms[i][c] = pm[0];
      wgt[i][c] = pm[1];
    }
  }
  __syncthreads();
  if (t < ncols) {
    float M = -INFINITY, L = 0.f;
    for (int i = 0; i < ns; ++i) M = fmaxf(M, ms[i][t]);
    for (int i = 0; i < ns; ++i) {
      const float f = ms[i][t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[i][t] - M);
      L += f * wgt[i][t];
      ms[i][t] = f;
    }
    const float inv = 1.f / L;
    for (int i = 0; i < ns; ++i) wgt[i][t] = ms[i][t] * inv;
  }
  __syncthreads();
  constexpr int Q4 = D / 4;
  const int64_t qbeg = cu_q[s];
  for (int idx = t; idx < ncols * Q4; idx += 256) {
    const int c = idx / Q4, d4 = (idx - c * Q4) * 4;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* po = part_o + (int64_t(p0) * sa::kCols + c) * D + d4;
#pragma unroll 8
    for (int i = 0; i < ns; ++i) acc += wgt[i][c] * *reinterpret_cast<const f32x4*>(po + int64_t(i) * sa::kCols * D);
    const int ri = c / nh, head = head0 + (c - ri * nh);
    *reinterpret_cast<u32x2*>(out + ((qbeg + row0 + ri) * Hq + head) * D + d4) = pack4(acc[0], acc[1], acc[2], acc[3]);
  }
}

sa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sa::fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SA_OK;
}

template <int D, bool WIN, bool NT>
void launch_attn(const AttnArgs& a, int n_items, bool wide_decode, hipStream_t st) {
  if (wide_decode)
    hipLaunchKernelGGL((attn_kernel<D, 32, WIN, NT>), dim3(unsigned(n_items)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, 16, WIN, NT>), dim3(unsigned(n_items)), dim3(256), 0, st, a);
}
template <int D, bool WIN>
void launch_attn(const AttnArgs& a, int n_items, bool wide_decode, bool stream_kv, hipStream_t st) {
  if (stream_kv) launch_attn<D, WIN, true>(a, n_items, wide_decode, st);
  else launch_attn<D, WIN, false>(a, n_items, wide_decode, st);
}

// The device address of `scratch` on each GPU, resolved once per device with
// hipGetSymbolAddress: host code never passes the array's name itself to a
// kernel (on the host it only stands in for the symbol).
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_addr;   // per device ordinal; null until resolved

sa_status scratch_address(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return sa::fail(SA_ERR_HIP, "sa_hybrid_attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (size_t(dev) >= g_scratch_addr.size()) g_scratch_addr.resize(size_t(dev) + 1, nullptr);
  if (!g_scratch_addr[size_t(dev)]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return sa::fail(SA_ERR_HIP, "sa_hybrid_attn_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_addr[size_t(dev)] = p;
  }
  *addr = g_scratch_addr[size_t(dev)];
  return SA_OK;
}

}  // namespace

// ---------------------------------------------------------- upload copy ---
// The metadata upload: copies n16 16-byte words from pinned host memory,
// read through its device address over PCIe, into device memory.  On the
// compute stream this costs one short kernel; a copy-engine transfer of the
// same bytes pays a hand-off between the copy and compute queues on either
// side (~25 us between kernels even for 56 KB).
__global__ __launch_bounds__(256) void meta_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n16) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += int64_t(gridDim.x) * 256)
    dst[i] = __builtin_nontemporal_load(src + i);
}

// Upload + append in one launch: workgroups [0, copy_wgs) copy the packed
// metadata (as meta_copy_kernel), the rest append the step's K/V rows (as
// kv_append_kernel, workgroup copy_wgs + b taking token block b / Hkv and kv
// head b % Hkv), reading the slot mapping from the pinned staging buffer.
// The two parts touch disjoint memory, so no ordering between them is needed.
template <int D>
__global__ __launch_bounds__(256) void upload_append_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t n16, int copy_wgs, const uint16_t* __restrict__ k_new,
                                                            const uint16_t* __restrict__ v_new,
                                                            uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                                            const int32_t* __restrict__ slot_mapping, int T, int Hkv,
                                                            int64_t num_slots) {
  __shared__ __attribute__((aligned(16))) AppendLds<D> sh;
  if (int(blockIdx.x) < copy_wgs) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += int64_t(copy_wgs) * 256)
      dst[i] = __builtin_nontemporal_load(src + i);
    return;
  }
  const int b = int(blockIdx.x) - copy_wgs;
  append_rows<D>((b / Hkv) * kAppendTokens, b % Hkv, k_new, v_new, k_cache, v_cache, slot_mapping, T, Hkv, num_slots,
                 sh);
}

namespace sa {
hipError_t copy_pinned_to_device(const void* src_dev, void* dst, size_t bytes, hipStream_t st) {
  const int64_t n16 = int64_t(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t g = std::min<int64_t>((n16 + 255) / 256, 1024);   // one 16-byte word per thread and pass
  hipLaunchKernelGGL(meta_copy_kernel, dim3(unsigned(g)), dim3(256), 0, st, static_cast<const u32x4*>(src_dev),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

hipError_t upload_append(const void* src_dev, void* dst, size_t bytes, const int32_t* slots_dev, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache, int T, int Hkv, int d, int num_pages,
                         hipStream_t st) {
  const int64_t n16 = int64_t(bytes / 16);
  const int64_t copy_wgs = std::max<int64_t>(1, std::min<int64_t>((n16 + 255) / 256, 1024));
  const int64_t append_wgs = (int64_t(T) + kAppendTokens - 1) / kAppendTokens * Hkv;
  const int64_t grid = copy_wgs + append_wgs;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int64_t num_slots = int64_t(num_pages) * kPageSize;
  const u32x4* s = static_cast<const u32x4*>(src_dev);
  u32x4* o = static_cast<u32x4*>(dst);
  const uint16_t* kn = static_cast<const uint16_t*>(k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(v_new);
  uint16_t* kc = static_cast<uint16_t*>(k_cache);
  uint16_t* vc = static_cast<uint16_t*>(v_cache);
  if (d == 64)
    hipLaunchKernelGGL(upload_append_kernel<64>, dim3(unsigned(grid)), dim3(256), 0, st, s, o, n16, int(copy_wgs), kn, vn,
                       kc, vc, slots_dev, T, Hkv, num_slots);
  else
    hipLaunchKernelGGL(upload_append_kernel<128>, dim3(unsigned(grid)), dim3(256), 0, st, s, o, n16, int(copy_wgs), kn,
                       vn, kc, vc, slots_dev, T, Hkv, num_slots);
  return hipGetLastError();
}
}  // namespace sa

extern "C" {

sa_status sa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int32_t* slot_mapping,
                       int32_t T, int32_t Hkv, int32_t d, int32_t num_pages, void* stream) {
  if (T < 0 || Hkv < 1 || num_pages < 1) return sa::fail(SA_ERR_INVALID_ARG, "sa_kv_append: T %d, Hkv %d, pages %d", T, Hkv, num_pages);
  if (d != 64 && d != 128) return sa::fail(SA_ERR_UNSUPPORTED, "sa_kv_append: head_dim %d (64 or 128 supported)", d);
  if (T == 0) return SA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_kv_append: null pointer");
  for (const void* p : {k_new, v_new, (const void*)k_cache, (const void*)v_cache})
    if (reinterpret_cast<uintptr_t>(p) & 15) return sa::fail(SA_ERR_INVALID_ARG, "sa_kv_append: tensors must be 16-byte aligned");
  if (Hkv > 65535) return sa::fail(SA_ERR_UNSUPPORTED, "sa_kv_append: %d kv heads", Hkv);
  const dim3 grid(unsigned((int64_t(T) + kAppendTokens - 1) / kAppendTokens), unsigned(Hkv)), block(256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t num_slots = int64_t(num_pages) * sa::kPageSize;
  if (d == 64)
    hipLaunchKernelGGL(kv_append_kernel<64>, grid, block, 0, st, static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), slot_mapping, T, Hkv, num_slots);
  else
    hipLaunchKernelGGL(kv_append_kernel<128>, grid, block, 0, st, static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), slot_mapping, T, Hkv, num_slots);
  return launch_status("sa_kv_append");
}

sa_status sa_hybrid_attn_workspace_size(const sa_batch_dev* b, size_t* bytes) {
  if (!b || !bytes) return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn_workspace_size: null pointer");
  *bytes = sa::workspace_bytes(b->num_partials, b->head_dim);
  return SA_OK;
}

sa_status sa_hybrid_attn(const void* q, const void* k_cache, const void* v_cache, const sa_batch_dev* b,
                         float softmax_scale, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!b) return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: null batch");
  const int d = b->head_dim;
  if (d != 64 && d != 128) return sa::fail(SA_ERR_UNSUPPORTED, "sa_hybrid_attn: head_dim %d", d);
  if (b->num_q_heads < 1 || b->num_kv_heads < 1 || b->num_q_heads % b->num_kv_heads)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: heads %d / %d", b->num_q_heads, b->num_kv_heads);
  if (b->num_work_items == 0) return SA_OK;
  if (!q || !k_cache || !v_cache || !out || !b->work || !b->cu_seqlens_q || !b->block_table_offsets)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: null pointer");
  for (const void* p : {q, k_cache, v_cache, (const void*)out})
    if (reinterpret_cast<uintptr_t>(p) & 15) return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: tensors must be 16-byte aligned");
  const size_t need = sa::workspace_bytes(b->num_partials, d);
  if (workspace_bytes < need || (need && !workspace))
    return sa::fail(SA_ERR_CAPACITY, "sa_hybrid_attn: workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (b->sliding_window < 0) return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: sliding window %d", b->sliding_window);
  if (!(softmax_scale > 0.f) || !(softmax_scale < INFINITY))
    return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: softmax_scale must be positive and finite");

  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.cu_q = b->cu_seqlens_q;
  a.ctx_lens = b->context_lens;
  a.bt = b->block_tables;
  a.bt_off = b->block_table_offsets;
  a.items = b->work;
  a.groups = b->combine;
  a.out = static_cast<uint16_t*>(out);
  a.part_ml = static_cast<float*>(workspace);
  a.part_o = a.part_ml + int64_t(b->num_partials) * sa::kCols * 2;
  a.Hq = b->num_q_heads;
  a.Hkv = b->num_kv_heads;
  a.group = b->num_q_heads / b->num_kv_heads;
  a.window = b->sliding_window;
  a.scale_log2 = softmax_scale * kLog2e;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool wide = b->num_q_heads / b->num_kv_heads > 16;   // must match the plan's decode block width
  const bool win = b->sliding_window > 0;
  const bool nt = (b->plan_flags & SA_PLAN_STREAM_KV) != 0;
  const int n = b->num_work_items;
  if (d == 64)
    win ? launch_attn<64, true>(a, n, wide, nt, st) : launch_attn<64, false>(a, n, wide, nt, st);
  else
    win ? launch_attn<128, true>(a, n, wide, nt, st) : launch_attn<128, false>(a, n, wide, nt, st);
  sa_status r = launch_status("sa_hybrid_attn");
  if (r != SA_OK || b->num_combine_groups == 0) return r;
  if (d == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(unsigned(b->num_combine_groups)), dim3(256), 0, st, b->combine,
                       b->cu_seqlens_q, a.part_ml, a.part_o, a.out, a.Hq);
  else
    hipLaunchKernelGGL(merge_kernel<128>, dim3(unsigned(b->num_combine_groups)), dim3(256), 0, st, b->combine,
                       b->cu_seqlens_q, a.part_ml, a.part_o, a.out, a.Hq);
  return launch_status("sa_hybrid_attn (merge)");
}

sa_status sa_hybrid_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, const sa_batch_dev* b,
                                 float softmax_scale, void* out, void* stream) {
  if (!b) return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn_noalloc: null batch");
  if (b->num_partials < 0) return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn_noalloc: num_partials %d", b->num_partials);
  const size_t need = sa::workspace_bytes(b->num_partials, b->head_dim);
  if (need > kStaticWorkspaceBytes)
    return sa::fail(SA_ERR_CAPACITY, "sa_hybrid_attn_noalloc: the plan needs %zu bytes of workspace; the static "
                    "workspace holds %zu (use sa_hybrid_attn with a caller workspace)", need, kStaticWorkspaceBytes);
  if (b->num_work_items == 0) return SA_OK;
  void* ws = nullptr;
  const sa_status st = scratch_address(&ws);
  if (st != SA_OK) return st;
  return sa_hybrid_attn(q, k_cache, v_cache, b, softmax_scale, out, ws, kStaticWorkspaceBytes, stream);
}

}  // extern "C"
