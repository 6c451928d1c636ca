// gfx950 kernels of libsarathi_attn: paged KV append and hybrid-batch attention.
//
// Attention of a hybrid batch ("Sarathi-Serve：以 chunked-prefills 与 stall-free
// batching 驯服 LLM 推理的吞吐—延迟权衡", GPU / 系统数据路径 steps ③-⑤): single-token
// decodes and prefill chunks run in one step; a chunk row at absolute position
// p attends to keys 0..p of its own prompt (earlier chunks are re-read from the
// paged cache) and a decode attends to its whole history ("In-flight
// Batching", 技术原理).  All K/V reads go through 16-token pages.
//
// One wavefront runs one work item (see plan.cpp): up to 32 columns, each a
// (query row, q head) pair sharing one kv head, over a key range.  Per 32-key
// step it computes S^T = K * Q^T on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16: rows = keys, columns = the item's columns), an
// online softmax in fp32 (running max in log2 units, exp2), and O^T += V^T * P^T
// on the matrix cores.  Because S^T puts one column's scores in one lane
// (16 keys) and its twin lane (lane ^ 32), the softmax row reductions need a
// single cross-lane exchange.  The K rows fed to the first product are
// permuted so that each lane ends up holding 8 *consecutive* keys of its
// column, which is exactly the B operand layout of the second product, and V
// is stored dim-major inside a page so its A operand is one 16-byte load.
// The online softmax follows the published streaming-softmax method
// (Milakov & Gimelshein, 2018) as used by tiled attention kernels.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---------------------------------------------------------------- append ---
// One thread per (token, kv head, 8-dim group).  K goes token-major, V goes
// dim-major (transposed) inside the page.
template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new,
                                                        uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                                        const int32_t* __restrict__ slot_mapping, int T, int Hkv,
                                                        int64_t num_slots) {
  constexpr int G = D / 8;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= int64_t(T) * Hkv * G) return;
  const int grp = int(gid % G);
  const int64_t th = gid / G;          // token * Hkv + kv head
  const int kh = int(th % Hkv);
  const int t = int(th / Hkv);
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || int64_t(slot) >= num_slots) return;
  const int64_t page = slot >> 4;
  const int off = slot & 15;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + th * D + grp * 8);
  *reinterpret_cast<u32x4*>(k_cache + ((page * Hkv + kh) * 16 + off) * D + grp * 8) = kv;
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + th * D + grp * 8);
  uint16_t* vdst = v_cache + ((page * Hkv + kh) * D + grp * 8) * 16 + off;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vdst[(2 * i) * 16] = uint16_t(vv[i] & 0xffffu);
    vdst[(2 * i + 1) * 16] = uint16_t(vv[i] >> 16);
  }
}

// ------------------------------------------------------------- attention ---
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* cu_q;
  const int32_t* ctx_lens;
  const int32_t* bt;
  const int32_t* items;
  const int32_t* groups;
  uint16_t* out;
  int32_t* counters;
  float* part_ml;
  float* part_o;
  int n_items;
  int bt_stride;
  int Hq;
  int Hkv;
  float scale_log2;   // softmax_scale * log2(e)
};

// Key held by row r of the K operand.  With r = 8a + 4h + b, MFMA output
// register j of lane l (h = l / 32) is row 8(j/4) + 4h + j%4; the mapping
// below makes that row key 16(j/8) + 8h + j%8, i.e. lane l holds keys
// 8h..8h+7 in registers 0..7 and 16+8h..16+8h+7 in registers 8..15.
__device__ __forceinline__ int key_of_row(int r) {
  const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

// Merge of the split partials of one column block, run by the wavefront that
// finishes last: with M the largest running max, out = sum_i 2^(m_i - M) o_i
// / sum_i 2^(m_i - M) l_i.  Arrival is counted with an agent-scope atomic;
// the release fence before it publishes this wave's partial (also across the
// per-XCD L2 caches) and the acquire fence after it makes the other waves'
// partials visible.  The last wave resets the counter for the next call.
template <int D>
__device__ __forceinline__ void merge_if_last(const AttnArgs& A, int group, int s, int head0, int nrows, int nheads,
                                              int row0, int ncols, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // partial stores before the arrival count
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(A.counters + group, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  const int32_t* g = A.groups + int64_t(group) * sa::kGroupWords;
  const int p0 = uniform(g[0]), ns = uniform(g[1]);
  if (old != ns - 1) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (lane == 0) __hip_atomic_store(A.counters + group, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // per column c (lane c < 32): largest max and the merged sum
  float M = -INFINITY, den = 0.f;
  if (lane < ncols) {
    for (int i = 0; i < ns; ++i) M = fmaxf(M, A.part_ml[(int64_t(p0 + i) * sa::kCols + lane) * 2]);
    for (int i = 0; i < ns; ++i) {
      const int64_t pc = int64_t(p0 + i) * sa::kCols + lane;
      const float mi = A.part_ml[pc * 2];
      den += mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - M) * A.part_ml[pc * 2 + 1];
    }
  }
  constexpr int LPC = D / 4;          // lanes per column, 4 dims each
  constexpr int CPI = 64 / LPC;       // columns per pass
  const int cc = lane / LPC, e4 = (lane % LPC) * 4;
  const int64_t qbeg = A.cu_q[s];
  for (int c0 = 0; c0 < ncols; c0 += CPI) {
    const int c = c0 + cc;
    const float Mc = __shfl(M, c & 31);
    const float dc = __shfl(den, c & 31);
    if (c >= ncols) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < ns; ++i) {
      const int64_t pc = int64_t(p0 + i) * sa::kCols + c;
      const float mi = A.part_ml[pc * 2];
      const float f = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - Mc);
      const float4 v = *reinterpret_cast<const float4*>(A.part_o + pc * D + e4);
      acc.x += f * v.x; acc.y += f * v.y; acc.z += f * v.z; acc.w += f * v.w;
    }
    const float inv = 1.f / dc;
    f32x8 t{};
    t[0] = acc.x * inv; t[1] = acc.y * inv; t[2] = acc.z * inv; t[3] = acc.w * inv;
    const u32x4 u = __builtin_bit_cast(u32x4, __builtin_convertvector(t, bf16x8));
    const int ri = c / nheads, head = head0 + (c - ri * nheads);
    *reinterpret_cast<u32x2*>(A.out + ((qbeg + row0 + ri) * A.Hq + head) * D + e4) = u32x2{u[0], u[1]};
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_items_kernel(AttnArgs A) {
  constexpr int KB = D / 16;   // k-blocks of the S product (16 dims each)
  constexpr int DB = D / 32;   // 32-dim blocks of the output
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= A.n_items) return;   // whole wavefront leaves; no block barrier is used

  const int32_t* w = A.items + int64_t(item) * sa::kItemWords;
  const int s = uniform(w[0]);
  const int kh = uniform(w[1]);
  const int head0 = uniform(w[2]);
  const int packed = uniform(w[3]);
  const int nrows = packed & 0xffff, nheads = packed >> 16;
  const int row0 = uniform(w[4]);
  const int k0 = uniform(w[5]);
  const int k1 = uniform(w[6]);
  const int part = uniform(w[7]);
  const int group = uniform(w[8]);

  const int ctx = uniform(A.ctx_lens[s]);
  const int qbeg = uniform(A.cu_q[s]);
  const int kv_len = ctx + uniform(A.cu_q[s + 1]) - qbeg;   // keys that exist in the cache
  const int32_t* btrow = A.bt + int64_t(s) * A.bt_stride;

  const int col = lane & 31;
  const int hi = lane >> 5;
  const int ncols = nrows * nheads;
  const bool col_ok = col < ncols;
  const int ri = col_ok ? col / nheads : 0;
  const int head = head0 + (col_ok ? col - ri * nheads : 0);
  const int64_t qrow = qbeg + row0 + ri;
  const int pos = ctx + row0 + ri;                       // absolute position of this column's row
  const int kend_col = col_ok ? min(k1, pos + 1) : k0;   // visible keys of this column: [k0, kend_col)
  const int kend = min(k1, ctx + row0 + nrows);          // wave-wide loop end

  // Q^T as the B operand: lane holds dims 16kb + 8hi .. +7 of its column.
  bf16x8 qf[KB];
  const uint16_t* qp = A.q + (qrow * A.Hq + head) * D + 8 * hi;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) qf[kb] = col_ok ? load8(qp + 16 * kb) : zero8();

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY;   // running max (log2 units), shared by lanes l and l^32
  float l = 0.f;         // this lane's share of the running sum

  const int krow = key_of_row(col);   // key offset of this lane's K row within a tile
  const int64_t hstride = int64_t(A.Hkv);

  for (int kt = k0; kt < kend; kt += sa::kKeyTile) {
    // ---- S^T = K * Q^T ----
    const int key = kt + krow;
    bf16x8 kf[KB];
    if (key < kv_len) {
      const int64_t page = btrow[key >> 4];
      const uint16_t* kp = A.k_cache + ((page * hstride + kh) * 16 + (key & 15)) * D + 8 * hi;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kf[kb] = load8(kp + 16 * kb);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kf[kb] = zero8();
    }
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb], qf[kb], sacc, 0, 0, 0);

    // ---- V^T operands for this tile (issued early to overlap the softmax) ----
    bf16x8 vf[2][DB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kb0 = kt + 16 * ks;          // first key of this 16-key half (page aligned)
      const int kfirst = kb0 + 8 * hi;       // this lane's 8 keys: kfirst .. kfirst+7
      if (kb0 < kv_len) {
        const int64_t page = btrow[kb0 >> 4];
        const uint16_t* vp = A.v_cache + ((page * hstride + kh) * D + col) * 16 + 8 * hi;
#pragma unroll
        for (int db = 0; db < DB; ++db) vf[ks][db] = load8(vp + 32 * 16 * db);
        if (kfirst + 8 > kv_len) {           // keys past the sequence end may hold anything
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            u32x4 u = __builtin_bit_cast(u32x4, vf[ks][db]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (kfirst + e >= kv_len) {
                const uint32_t mask = (e & 1) ? 0x0000ffffu : 0xffff0000u;
                u[e >> 1] &= mask;
              }
            }
            vf[ks][db] = __builtin_bit_cast(bf16x8, u);
          }
        }
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) vf[ks][db] = zero8();
      }
    }

    // ---- online softmax over this tile ----
    float sv[16];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kt + 16 * (j >> 3) + 8 * hi + (j & 7);
      sv[j] = kj < kend_col ? sacc[j] * A.scale_log2 : -INFINITY;
      mt = fmaxf(mt, sv[j]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;   // nothing visible yet: keep exp2 finite
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    f32x8 p0, p1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p0[j] = __builtin_amdgcn_exp2f(sv[j] - m_use);
      p1[j] = __builtin_amdgcn_exp2f(sv[8 + j] - m_use);
    }
    const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
    const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
    // the sum uses the same bf16-rounded weights that multiply V
    const f32x8 r0 = __builtin_convertvector(pb0, f32x8);
    const f32x8 r1 = __builtin_convertvector(pb1, f32x8);
#pragma unroll
    for (int j = 0; j < 8; ++j) l += r0[j] + r1[j];

    // ---- O^T += V^T * P^T ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[0][db], pb0, o[db], 0, 0, 0);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[1][db], pb1, o[db], 0, 0, 0);
    }
  }

  l += __shfl_xor(l, 32);
  // lane holds dims 32db + 8(j/4) + 4hi + j%4 of its column
  if (part < 0) {
    if (!col_ok) return;
    const float inv = 1.f / l;
    uint16_t* op = A.out + (qrow * A.Hq + head) * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x8 t{};
        t[0] = o[db][4 * jj] * inv;
        t[1] = o[db][4 * jj + 1] * inv;
        t[2] = o[db][4 * jj + 2] * inv;
        t[3] = o[db][4 * jj + 3] * inv;
        const bf16x8 tb = __builtin_convertvector(t, bf16x8);
        const u32x4 u = __builtin_bit_cast(u32x4, tb);
        *reinterpret_cast<u32x2*>(op + 32 * db + 8 * jj) = u32x2{u[0], u[1]};
      }
    }
    return;
  }

  // ---- split item: publish the partial, the last split of the group merges ----
  if (col_ok) {
    float* po = A.part_o + (int64_t(part) * sa::kCols + col) * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float4 t = make_float4(o[db][4 * jj], o[db][4 * jj + 1], o[db][4 * jj + 2], o[db][4 * jj + 3]);
      *reinterpret_cast<float4*>(po + 32 * db + 8 * jj) = t;
      }
    if (hi == 0) {
      float* pm = A.part_ml + (int64_t(part) * sa::kCols + col) * 2;
      pm[0] = m;
      pm[1] = l;
    }
  }
  merge_if_last<D>(A, group, s, head0, nrows, nheads, row0, ncols, lane);
}

sa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sa::fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SA_OK;
}

}  // namespace

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
  const int64_t threads = int64_t(T) * Hkv * (d / 8);
  const dim3 grid(unsigned((threads + 255) / 256)), block(256);
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
  *bytes = sa::workspace_bytes(b->num_combine_groups, b->num_partials, b->head_dim);
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
  if (!q || !k_cache || !v_cache || !out || !b->work || !b->cu_seqlens_q)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: null pointer");
  for (const void* p : {q, k_cache, v_cache, (const void*)out})
    if (reinterpret_cast<uintptr_t>(p) & 15) return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: tensors must be 16-byte aligned");
  const size_t need = sa::workspace_bytes(b->num_combine_groups, b->num_partials, d);
  if (workspace_bytes < need || (need && !workspace))
    return sa::fail(SA_ERR_CAPACITY, "sa_hybrid_attn: workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (!(softmax_scale > 0.f) || !(softmax_scale < INFINITY))
    return sa::fail(SA_ERR_INVALID_ARG, "sa_hybrid_attn: softmax_scale must be positive and finite");

  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.cu_q = b->cu_seqlens_q;
  a.ctx_lens = b->context_lens;
  a.bt = b->block_tables;
  a.items = b->work;
  a.groups = b->combine;
  a.out = static_cast<uint16_t*>(out);
  a.counters = static_cast<int32_t*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + sa::counter_bytes(b->num_combine_groups));
  a.part_o = a.part_ml + int64_t(b->num_partials) * sa::kCols * 2;
  a.n_items = b->num_work_items;
  a.bt_stride = b->bt_stride;
  a.Hq = b->num_q_heads;
  a.Hkv = b->num_kv_heads;
  a.scale_log2 = softmax_scale * kLog2e;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned((b->num_work_items + 3) / 4)), block(256);
  if (d == 64)
    hipLaunchKernelGGL(attn_items_kernel<64>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(attn_items_kernel<128>, grid, block, 0, st, a);
  return launch_status("sa_hybrid_attn");
}

}  // extern "C"
