// Key-norm anchors per precomputed chunk (QCFuse technical summary (zh), §2.A anchor-based
// lightweight query probing: offline, each chunk keeps the few tokens with the largest key norm
// as a compressed semantic summary).
//
// Two launches, both wide: (1) one wave per token row reduces the squares of its key (all KV heads
// and dims) in float64 -- squares of bf16/f32 values are exact there, so the ranking matches an
// exact computation up to the last float64 bit -- into the workspace; (2) one wave per chunk picks
// the k largest in the order (larger norm first, lower token offset on a tie).
#include <float.h>

#include "common.h"

namespace sra {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ double sumsq16(u32x4 v);
template <>
__device__ __forceinline__ double sumsq16<uint16_t>(u32x4 v) {
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double a = __uint_as_float(v[k] << 16), b = __uint_as_float(v[k] & 0xffff0000u);
    acc += a * a;
    acc += b * b;
  }
  return acc;
}
template <>
__device__ __forceinline__ double sumsq16<float>(u32x4 v) {
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double a = __uint_as_float(v[k]);
    acc += a * a;
  }
  return acc;
}

// Table use: entry e = one chunk; src/len its store rows; dst its output slot; delta its offset in
// the sum-of-squares workspace. blk0 counts blocks of 4 rows (one wave per row).
template <typename T>
__global__ __launch_bounds__(256) void k_row_sumsq(ChunkTab tab, int row_elems,
                                                   const T* __restrict__ ks,
                                                   double* __restrict__ ss,
                                                   float* __restrict__ norms) {
  const int e = find_entry(tab, blockIdx.x);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = (blockIdx.x - tab.blk0[e]) * 4 + wave;
  if (t >= tab.len[e]) return;
  const int64_t row = (int64_t)tab.src[e] + t;
  const u32x4* p = reinterpret_cast<const u32x4*>(ks + row * row_elems);
  const int n16 = row_elems * (int)sizeof(T) / 16;
  double acc = 0.0;
  for (int u = lane; u < n16; u += 64) acc += sumsq16<T>(p[u]);
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_down(acc, off, 64);  // fixed-order tree
  if (lane == 0) {
    ss[tab.delta[e] + t] = acc;
    if (norms) norms[row] = (float)sqrt(acc);
  }
}

// One wave per chunk. The ranking (larger sum first, lower offset on a tie) is a strict total
// order, so round r picks the best element ranked after the pick of round r-1: nothing is written
// back, every round reads the same sums. Sums of squares are non-negative, so their float64 bit
// patterns order like the values and every comparison is a branch-free 64-bit integer select.
__global__ __launch_bounds__(256) void k_anchor_topk(ChunkTab tab, int k, const double* __restrict__ ss,
                                                     int32_t* __restrict__ anchors) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= tab.n) return;
  const int lane = threadIdx.x & 63;
  const int len = tab.len[e];
  const unsigned long long* s = reinterpret_cast<const unsigned long long*>(ss + tab.delta[e]);
  // the first 64*kCache sums stay in registers (one batch of independent loads); longer chunks
  // read the rest from memory each round
  constexpr int kCache = 16;
  unsigned long long cv[kCache];
#pragma unroll
  for (int u = 0; u < kCache; ++u) {
    const int t = lane + 64 * u;
    cv[u] = s[min(t, len - 1)];
  }
  unsigned long long pv = ~0ull;   // previous pick (value, offset); starts above everything
  int pt = -1;
  auto consider = [&](unsigned long long v, int t, bool& have, unsigned long long& bv, int& bt) {
    const bool after = t < len && (v < pv || (v == pv && t > pt));
    const bool better = after && (!have || v > bv || (v == bv && t < bt));
    bv = better ? v : bv;
    bt = better ? t : bt;
    have = have || better;
  };
  for (int round = 0; round < k; ++round) {
    bool have = false;
    unsigned long long bv = 0;
    int bt = INT_MAX;
#pragma unroll
    for (int u = 0; u < kCache; ++u) consider(cv[u], lane + 64 * u, have, bv, bt);
    for (int t = lane + 64 * kCache; t < len; t += 64) consider(s[t], t, have, bv, bt);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const unsigned long long ov = __shfl_xor(bv, off, 64);
      const int ot = __shfl_xor(bt, off, 64);
      const bool oh = __shfl_xor((int)have, off, 64) != 0;
      const bool better = oh && (!have || ov > bv || (ov == bv && ot < bt));
      bv = better ? ov : bv;
      bt = better ? ot : bt;
      have = have || oh;
    }
    if (lane == 0) anchors[(int64_t)tab.dst[e] * k + round] = bt;
    pv = bv;
    pt = bt;
  }
}

}  // namespace

hipError_t launch_anchors(int dtype, int row_elems, const ChunkTab& tab, int k, const void* ks,
                          double* ss, int32_t* anchors, float* norms, hipStream_t st) {
  // tab.blk0 counts blocks of 4 rows per chunk
  if (tab.n == 0) return hipSuccess;
  const int nblk = tab.blk0[tab.n];
  if (dtype == 0)
    k_row_sumsq<uint16_t><<<dim3(nblk), dim3(256), 0, st>>>(tab, row_elems, (const uint16_t*)ks, ss, norms);
  else
    k_row_sumsq<float><<<dim3(nblk), dim3(256), 0, st>>>(tab, row_elems, (const float*)ks, ss, norms);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  k_anchor_topk<<<dim3((tab.n + 3) / 4), dim3(256), 0, st>>>(tab, k, ss, anchors);
  return hipGetLastError();
}

}  // namespace sra
