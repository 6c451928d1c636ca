// gfx950 kernel of libsarathi_attn: the token-batch linear layer y = x w^T.
//
// Every layer of a hybrid step runs the batch's token rows through linear
// layers on either side of attention ("Sarathi-Serve：以 chunked-prefills 与
// stall-free batching 驯服 LLM 推理的吞吐—延迟权衡", 端到端文字序列 step ④), and
// those GEMMs take most of the time of both phases (两阶段天然不对称).  Their
// row count is the token budget B, which meets the GPU's tile quantisation
// (3 · token 预算的三个约束).
//
// x: [M, K] token rows, w: [N, K] weight rows (one output feature per row),
// y: [M, N]; bf16 in, fp32 accumulation on the matrix cores, bf16 out.
//
// A workgroup (WN x WM wavefronts) owns a BN x BM tile of y^T = w x^T: BN
// weight rows by BM token rows.  Per BK-wide K step the tile's rows of w and
// x are staged in LDS by direct global->LDS loads through a ring of STAGES
// buffers (STAGES - 1 steps of loads in flight), and each wave runs
// v_mfma_f32_32x32x16_bf16 over its (BN/WN) x (BM/WM) sub-tile: the A operand
// is 8 consecutive K values of a weight row, the B operand 8 of a token row,
// so both are single 16-byte LDS reads.  A lane of the result holds 4
// consecutive output features of one token row, stored as one 8-byte write.
// Two shapes: 256 x 256 tiles for large products, where the per-CU load rate
// from L2 and the LDS read rate must stay well below the matrix cores'
// appetite -- one workgroup of 8 waves per CU (two per SIMD, so one wave's
// MFMAs cover the other's barrier and LDS waits), each wave 128 x 64; and
// 128 x 128 tiles of 4 waves (two workgroups per CU) with split K when the
// large tiles cannot fill the chip.  Both keep three K steps of loads in
// flight per workgroup: with few token rows the product streams the weights,
// and a shallower ring leaves it waiting on memory latency.
//
// Split K: when the tiles alone cannot fill the chip, the K steps of a tile
// are divided over `splits` workgroups, each writing an fp32 partial product
// to the workspace; a second kernel adds the partials in split order and
// rounds to bf16.  (Reducing inside the GEMM kernel, by the last workgroup of
// a tile to arrive, needs a device-scope release and acquire per workgroup:
// on this chip, whose L2 is private to each XCD, those write back and
// invalidate the whole L2, which costs far more than the second launch.)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 256;
constexpr int kKAlign = 64;      // K must be a multiple of this (both tile shapes' K step divides it)

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// 4 floats -> 4 bf16 (round to nearest even), packed in 8 bytes.
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  f32x8 t{};
  t[0] = a; t[1] = b; t[2] = c; t[3] = d;
  const u32x4 u = __builtin_bit_cast(u32x4, __builtin_convertvector(t, bf16x8));
  return u32x2{u[0], u[1]};
}

// Waits until at most N direct loads of this wave are outstanding.
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

struct LinArgs {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  float* part;         // fp32 partial products (split K only): per (tile, split), [group][thread] f32x4
  int M, N, K;
  int tiles_m, splits, ksteps;
};

// LDS stage: BN weight rows then BM token rows of BK bf16 each; the 16-byte
// chunk c of row r sits at chunk c ^ swz(r), so that the 16 lanes of a
// fragment read (16 consecutive rows, one chunk) hit distinct banks: with
// 128-byte rows two rows share a 256-byte bank window, with 64-byte rows four.
template <int BK>
__device__ __forceinline__ int swz(int r) { return BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3; }

// WN x WM waves; wave (wn, wm) owns weight rows wn*BN/WN .. and token rows
// wm*BM/WM .. of the tile.
template <int BN, int BM, int BK, int STAGES, int WN, int WM>
__device__ __forceinline__ void linear_tile(const LinArgs& a, uint16_t* lds) {
  constexpr int NW = WN * WM;                 // waves per workgroup
  constexpr int TN = BN / WN, TM = BM / WM;   // wave tile
  constexpr int NT = TN / 32, MT = TM / 32;   // 32 x 32 MFMA tiles per wave along n and m
  constexpr int ROWS = BN + BM;
  constexpr int STAGE = ROWS * BK;            // bf16 elements per stage
  constexpr int CPR = BK / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows per 1 KB direct load
  constexpr int PER_WAVE = ROWS / RPI / NW;   // direct loads per wave per step
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(TN % 32 == 0 && TM % 32 == 0 && (ROWS / RPI) % NW == 0, "tile shape");

  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wn = wave / WM, wm = wave % WM;

  // Logical tile of this workgroup.  Consecutive workgroups are dispatched
  // round-robin over the 8 XCDs; give each XCD a contiguous run of logical
  // ids so that the workgroups sharing weight rows (same n tile and split,
  // consecutive m tiles) share an L2.
  const int G = gridDim.x, g = blockIdx.x;
  const int q = G >> 3, rr = G & 7, xcd = g & 7, slot = g >> 3;
  const int L = (xcd < rr ? xcd * (q + 1) : rr * (q + 1) + (xcd - rr) * q) + slot;
  const int tm = L % a.tiles_m;
  const int rest = L / a.tiles_m;
  const int split_idx = rest % a.splits;
  const int tn = rest / a.splits;
  const int n0 = tn * BN, m0 = tm * BM;
  const int ks0 = int(int64_t(split_idx) * a.ksteps / a.splits);
  const int ks1 = int(int64_t(split_idx + 1) * a.ksteps / a.splits);
  const int nk = ks1 - ks0;

  // this wave's direct loads: instruction j = wave + NW i covers rows
  // RPI j .. RPI j + RPI-1 of the stage, lane l the chunk at slot l % CPR of
  // row RPI j + l / CPR; rows past M or N re-read the last row (their results
  // are never stored)
  const uint16_t* src[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int row = RPI * (wave + NW * i) + lane / CPR;
    const int c = (lane % CPR) ^ swz<BK>(row);
    if (row < BN) src[i] = a.w + int64_t(min(n0 + row, a.N - 1)) * a.K + ks0 * BK + 8 * c;
    else src[i] = a.x + int64_t(min(m0 + row - BN, a.M - 1)) * a.K + ks0 * BK + 8 * c;
  }
  auto issue = [&](int step, int st) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(src[i] + step * BK),
                                       (lds_void*)(lds + st * STAGE + (wave + NW * i) * 512), 16, 0, 0);
  };

  // fragment offsets: row base per tile, chunk per K sub-step (the swizzle
  // depends on the lane only, since tiles start at multiples of 32 rows)
  constexpr int KS = BK / 16;                 // MFMA K sub-steps per step
  const int r32 = lane & 31, hi = lane >> 5;
  int coff[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) coff[kk] = ((2 * kk + hi) ^ swz<BK>(r32)) * 8;
  const int arow = (wn * TN + r32) * BK;                    // + 32 * BK * t
  const int brow = (BN + wm * TM + r32) * BK;

  f32x16 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = f32x16{};

#pragma unroll
  for (int i = 0; i < STAGES - 1; ++i)
    if (i < nk) issue(i, i);
  for (int t = 0; t < nk; ++t) {
    if (t + STAGES - 2 < nk) wait_vmcnt<PER_WAVE * (STAGES - 2)>();
    else wait_vmcnt<0>();
    lds_barrier();                         // step t is in LDS; every wave is done with step t - 1
    const uint16_t* st = lds + (t % STAGES) * STAGE;
    // fragments double-buffered across the K sub-steps: the reads of sub-step
    // kk + 1 are in flight while the matrix cores run sub-step kk (the
    // scheduling barriers keep the compiler from regrouping them)
    bf16x8 af[2][NT], bf[2][MT];
    auto frag = [&](int kk, int b) {
#pragma unroll
      for (int u = 0; u < NT; ++u) af[b][u] = lds8(st + arow + u * 32 * BK + coff[kk]);
#pragma unroll
      for (int u = 0; u < MT; ++u) bf[b][u] = lds8(st + brow + u * 32 * BK + coff[kk]);
    };
    if (t + STAGES - 1 < nk) issue(t + STAGES - 1, (t + STAGES - 1) % STAGES);   // refill step t - 1's stage
    frag(0, 0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk + 1 < KS) frag(kk + 1, (kk + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int v = 0; v < MT; ++v)
          acc[u][v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][u], bf[kk & 1][v], acc[u][v], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // acc[u][v] register 4 jj + e: feature n0 + wn*TN + 32u + 8jj + 4hi + e, token m0 + wm*TM + 32v + r32
  if (a.splits > 1) {
    // the partial tile in accumulator order, group g = (u MT + v) 4 + jj of
    // every thread side by side, so each store instruction writes 1 KB
    // contiguous per wave (the reduction reads it back the same way)
    constexpr int G = NT * MT * 4;
    const int tile = tn * a.tiles_m + tm;
    f32x4* p = reinterpret_cast<f32x4*>(a.part) + (int64_t(tile) * a.splits + split_idx) * G * (64 * NW) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int v = 0; v < MT; ++v)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          p[((u * MT + v) * 4 + jj) * (64 * NW)] =
              f32x4{acc[u][v][4 * jj], acc[u][v][4 * jj + 1], acc[u][v][4 * jj + 2], acc[u][v][4 * jj + 3]};
    return;
  }
#pragma unroll
  for (int v = 0; v < MT; ++v) {
    const int m = m0 + wm * TM + 32 * v + r32;
    if (m >= a.M) continue;
    uint16_t* yrow = a.y + int64_t(m) * a.N;
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n = n0 + wn * TN + 32 * u + 8 * jj + 4 * hi;
        if (n < a.N)
          *reinterpret_cast<u32x2*>(yrow + n) =
              pack4(acc[u][v][4 * jj], acc[u][v][4 * jj + 1], acc[u][v][4 * jj + 2], acc[u][v][4 * jj + 3]);
      }
  }
}

// y = sum over splits of the partial tiles, in split order, rounded to bf16.
// Thread i of the grid takes the i-th f32x4 of the first split's partials
// (so consecutive threads read consecutive 16 bytes) and maps it back to its
// 4 outputs the way linear_tile laid the accumulators out.
template <int BN, int BM, int WN, int WM>
__global__ __launch_bounds__(kThreads) void linear_reduce_kernel(const f32x4* __restrict__ part,
                                                                  uint16_t* __restrict__ y, int M, int N,
                                                                  int tiles_m, int splits, int64_t total) {
  constexpr int TN = BN / WN, TM = BM / WM, NT = TN / 32, MT = TM / 32, G = NT * MT * 4, WT = 64 * WN * WM;
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int t = int(i % WT);
  const int64_t rest = i / WT;
  const int g = int(rest % G);
  const int64_t tile = rest / G;
  const int tn = int(tile / tiles_m), tm = int(tile % tiles_m);
  const int wave = t >> 6, lane = t & 63;
  const int jj = g & 3, v = (g >> 2) % MT, u = (g >> 2) / MT;
  const int m = tm * BM + (wave % WM) * TM + 32 * v + (lane & 31);
  const int n = tn * BN + (wave / WM) * TN + 32 * u + 8 * jj + 4 * (lane >> 5);
  if (m >= M || n >= N) return;
  const f32x4* p = part + (tile * splits * G + g) * WT + t;
  f32x4 acc = p[0];
  for (int s = 1; s < splits; ++s) acc += p[int64_t(s) * G * WT];
  *reinterpret_cast<u32x2*>(y + int64_t(m) * N + n) = pack4(acc[0], acc[1], acc[2], acc[3]);
}

template <int BN, int BM, int BK, int STAGES, int OCC, int WN, int WM>
__global__ __launch_bounds__(64 * WN * WM, OCC) void linear_kernel(LinArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[STAGES * (BN + BM) * BK];
  linear_tile<BN, BM, BK, STAGES, WN, WM>(a, lds);
}

// Launch shape of one call: tile, workgroups per CU, split count.
struct LinCfg {
  int bn, bm, bk, occ;
  int tiles_m, tiles_n, splits, ksteps;
  int64_t tiles() const { return int64_t(tiles_m) * tiles_n; }
};

size_t part_bytes(const LinCfg& c) {   // whole tiles, accumulator order: BN x BM fp32 per tile and split
  return c.splits > 1 ? size_t(c.tiles()) * c.splits * size_t(c.bn) * size_t(c.bm) * sizeof(float) : 0;
}

constexpr int kCUs = 256;

// Split K while one round of workgroups is not full, at most max_splits ways
// (the partials cost 4 bytes per output and split each way) and >= 4 steps
// per split.
LinCfg with_splits(LinCfg c, int M, int N, int K, int max_splits = 4) {
  c.tiles_m = (M + c.bm - 1) / c.bm;
  c.tiles_n = (N + c.bn - 1) / c.bn;
  c.ksteps = K / c.bk;
  const int64_t slots = int64_t(kCUs) * c.occ;
  int64_t s = c.tiles() >= slots ? 1 : slots / c.tiles();
  s = std::min<int64_t>({s, max_splits, std::max(1, c.ksteps / 4)});
  c.splits = int(std::max<int64_t>(1, s));
  return c;
}

// The launch shape comes from a cost estimate over the five tile shapes:
//   192 x 256  weight x token rows, K steps of 64, 8 waves, never split;
//   256 x 256  K steps of 32, 8 waves, never split;
//   128 x 256  K steps of 64, 4 waves (accumulators in AGPRs), K split up to 4;
//   128 x 288  K steps of 64, 4 waves of 32 weight rows x 9 MFMA row tiles,
//              K split up to 8 (token counts just past a multiple of 256);
//   128 x 128  K steps of 32, two workgroups per CU, K split up to 4.
// Each shape, with its split count from with_splits, is timed as
//   rounds x (MACs per workgroup x a + b) + split partial bytes x c,
// rounds = ceil(workgroups / CUs): two resident workgroups of a CU take about
// as long as the same two one after the other, so the 128 x 128 tiles count
// per CU too.  a and b per shape and the one c were fitted (least squares,
// non-negative, relative error) to the kernel times of every projection of
// four layers (QKV, O, MLP up/gate and down of Mistral-7B, Yi-34B, LLaMA2-70B
// and one TP4 share of Falcon-180B) at M = 256, 257, 384, 512, 513, 768, 1024,
// 1025, 1536, 2048, 2049 -- 176 shapes.  Over them the chosen shapes take
// 51.0 ms in all, the best shape of each case 50.9 ms (fitted on three of the
// layers and chosen for the fourth: the same 51.0), the earlier fixed rules
// 54.3 ms; no case is more than 6% slower than its best shape.  Token counts
// just past a multiple of 256 gain most (the 288-row tiles, or 192-row weight
// tiles that fill the chip in fewer rounds).
struct TileShape {
  int bn, bm, bk, occ, max_splits;
  double us_per_mac, us_fixed;   // per workgroup
};
constexpr TileShape kShapes[] = {
    {256, 256, 32, 1, 1, 3.71e-7, 7.26},
    {192, 256, 64, 1, 1, 3.98e-7, 6.83},
    {128, 256, 64, 1, 4, 4.98e-7, 1.56},
    {128, 288, 64, 1, 8, 5.39e-7, 0.0},
    {128, 128, 32, 2, 4, 5.86e-7, 0.0},
};
constexpr double kUsPerPartialByte = 5.53e-7;   // split-K partials: written, then read by the reduction

LinCfg choose(int M, int N, int K) {
  LinCfg best{};
  double best_us = 0;
  bool first = true;
  for (const TileShape& t : kShapes) {
    LinCfg c{};
    c.bn = t.bn; c.bm = t.bm; c.bk = t.bk; c.occ = t.occ;
    c = with_splits(c, M, N, K, t.max_splits);
    const double rounds = std::ceil(double(c.tiles()) * c.splits / double(kCUs));
    const double macs = double(c.bn) * c.bm * K / c.splits;
    const double us = rounds * (macs * t.us_per_mac + t.us_fixed) + double(part_bytes(c)) * kUsPerPartialByte;
    if (first || us < best_us) {
      best = c;
      best_us = us;
      first = false;
    }
  }
  return best;
}

sa_status check_linear(const void* x, const void* w, const void* y, int M, int N, int K) {
  if (M < 0 || N < 1 || K < 1) return sa::fail(SA_ERR_INVALID_ARG, "sa_linear: M %d, N %d, K %d", M, N, K);
  if (K % kKAlign) return sa::fail(SA_ERR_UNSUPPORTED, "sa_linear: K %d is not a multiple of %d", K, kKAlign);
  if (N % 8) return sa::fail(SA_ERR_UNSUPPORTED, "sa_linear: N %d is not a multiple of 8", N);
  if (M == 0) return SA_OK;
  if (!x || !w || !y) return sa::fail(SA_ERR_INVALID_ARG, "sa_linear: null pointer");
  for (const void* p : {x, w, y})
    if (reinterpret_cast<uintptr_t>(p) & 15) return sa::fail(SA_ERR_INVALID_ARG, "sa_linear: tensors must be 16-byte aligned");
  if (int64_t(M) * K > (int64_t(1) << 40) || int64_t(N) * K > (int64_t(1) << 40))
    return sa::fail(SA_ERR_INVALID_ARG, "sa_linear: operand too large");
  return SA_OK;
}

}  // namespace

extern "C" {

sa_status sa_linear_workspace_size(int32_t M, int32_t N, int32_t K, size_t* bytes) {
  if (!bytes) return sa::fail(SA_ERR_INVALID_ARG, "sa_linear_workspace_size: null bytes");
  if (M < 0 || N < 1 || K < kKAlign || K % kKAlign || N % 8)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_linear_workspace_size: M %d, N %d, K %d", M, N, K);
  if (M == 0) { *bytes = 0; return SA_OK; }
  *bytes = part_bytes(choose(M, N, K));
  return SA_OK;
}

sa_status sa_linear(const void* x, const void* w, void* y, int32_t M, int32_t N, int32_t K, void* workspace,
                    size_t workspace_bytes, void* stream) {
  sa_status st = check_linear(x, w, y, M, N, K);
  if (st != SA_OK || M == 0) return st;
  const LinCfg c = choose(M, N, K);
  const size_t need = part_bytes(c);
  if (need && (!workspace || workspace_bytes < need))
    return sa::fail(SA_ERR_CAPACITY, "sa_linear: workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (need && (reinterpret_cast<uintptr_t>(workspace) & 15))
    return sa::fail(SA_ERR_INVALID_ARG, "sa_linear: workspace must be 16-byte aligned");
  const int64_t blocks = c.tiles() * c.splits;
  if (blocks > 0x7fffffff) return sa::fail(SA_ERR_INVALID_ARG, "sa_linear: too many tiles");
  LinArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.part = static_cast<float*>(workspace);
  a.M = M; a.N = N; a.K = K;
  a.tiles_m = c.tiles_m; a.splits = c.splits; a.ksteps = c.ksteps;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (c.bn == 256)
    hipLaunchKernelGGL((linear_kernel<256, 256, 32, 4, 1, 2, 4>), dim3(unsigned(blocks)), dim3(512), 0, hs, a);
  else if (c.bm == 288)
    hipLaunchKernelGGL((linear_kernel<128, 288, 64, 2, 1, 4, 1>), dim3(unsigned(blocks)), dim3(kThreads), 0, hs, a);
  else if (c.bn == 192)
    hipLaunchKernelGGL((linear_kernel<192, 256, 64, 2, 1, 2, 4>), dim3(unsigned(blocks)), dim3(512), 0, hs, a);
  else if (c.bm == 256)
    hipLaunchKernelGGL((linear_kernel<128, 256, 64, 2, 1, 2, 2>), dim3(unsigned(blocks)), dim3(kThreads), 0, hs, a);
  else
    hipLaunchKernelGGL((linear_kernel<128, 128, 32, 4, 2, 2, 2>), dim3(unsigned(blocks)), dim3(kThreads), 0, hs, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sa::fail(SA_ERR_HIP, "sa_linear: %s", hipGetErrorString(e));
  if (c.splits > 1) {                        // only the 128-weight-row tiles split K
    const int64_t total = c.tiles() * c.bn * c.bm / 4;       // f32x4 groups of one split
    const int64_t groups = (total + kThreads - 1) / kThreads;
    if (c.bm == 288)
      hipLaunchKernelGGL((linear_reduce_kernel<128, 288, 4, 1>), dim3(unsigned(groups)), dim3(kThreads), 0, hs,
                         reinterpret_cast<const f32x4*>(a.part), a.y, M, N, c.tiles_m, c.splits, total);
    else if (c.bm == 256)
      hipLaunchKernelGGL((linear_reduce_kernel<128, 256, 2, 2>), dim3(unsigned(groups)), dim3(kThreads), 0, hs,
                         reinterpret_cast<const f32x4*>(a.part), a.y, M, N, c.tiles_m, c.splits, total);
    else
      hipLaunchKernelGGL((linear_reduce_kernel<128, 128, 2, 2>), dim3(unsigned(groups)), dim3(kThreads), 0, hs,
                         reinterpret_cast<const f32x4*>(a.part), a.y, M, N, c.tiles_m, c.splits, total);
    e = hipGetLastError();
    if (e != hipSuccess) return sa::fail(SA_ERR_HIP, "sa_linear (reduce): %s", hipGetErrorString(e));
  }
  return SA_OK;
}

}  // extern "C"
