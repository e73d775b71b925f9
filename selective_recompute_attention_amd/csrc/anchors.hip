// Key-norm anchors per precomputed chunk (QCFuse technical summary (zh), §2.A anchor-based
// lightweight query probing: offline, each chunk keeps the few tokens with the largest key norm
// as a compressed semantic summary).
//
// Two launches, both wide: (1) the squares of every token's key (all KV heads and dims) summed in
// float64 -- squares of bf16/f32 values are exact there -- into the workspace; (2) one wave per chunk
// picks the k largest in the order (larger norm first, lower token offset on a tie).
#include <float.h>

#include "common.h"

namespace sra {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Table use: entry e = one chunk; src/len its store rows; dst its output slot; delta the offset of
// its sums of squares in the workspace. One thread per (row, KV head) sums that head's d squares in
// order (float64); the row's thread then adds the heads in order. The scoring pass forms the same
// per-head sums from its LDS tile, so fused and standalone anchors agree bit for bit.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_row_sumsq(ChunkTab tab, int Hkv,
                                                   const T* __restrict__ ks,
                                                   double* __restrict__ ss,
                                                   float* __restrict__ norms) {
  constexpr int NC = D * (int)sizeof(T) / 16;   // 16-byte pieces of one head
  __shared__ double part[256];
  const int e = find_entry(tab, blockIdx.x);
  const int rpb = anchor_rows_per_block(Hkv);
  const int rl = threadIdx.x / Hkv, h = threadIdx.x % Hkv;
  const int t0 = (blockIdx.x - tab.blk0[e]) * rpb;
  const int t = t0 + rl;
  const bool active = rl < rpb && t < tab.len[e];
  const u32x4* p = reinterpret_cast<const u32x4*>(
      ks + (((int64_t)tab.src[e] + (active ? t : 0)) * Hkv + (active ? h : 0)) * D);
  u32x4 w[NC];   // one batch of loads
#pragma unroll
  for (int c = 0; c < NC; ++c) w[c] = p[c];
  double acc = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t x[4] = {w[c][0], w[c][1], w[c][2], w[c][3]};
    acc = sumsq16<T>(acc, x);
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  if ((int)threadIdx.x < rpb && t0 + (int)threadIdx.x < tab.len[e]) {
    double tot = 0.0;
    for (int hh = 0; hh < Hkv; ++hh) tot += part[threadIdx.x * Hkv + hh];
    const int tt = t0 + threadIdx.x;
    ss[tab.delta[e] + tt] = tot;
    if (norms) norms[(int64_t)tab.src[e] + tt] = (float)sqrt(tot);
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

hipError_t launch_anchors(int dtype, int Hkv, int D, const ChunkTab& tab, int k, const void* ks,
                          double* ss, int32_t* anchors, float* norms, hipStream_t st) {
  if (tab.n == 0) return hipSuccess;
  const int nblk = tab.blk0[tab.n];
  const dim3 g(nblk), b(256);
  if (dtype == 0 && D == 128) k_row_sumsq<uint16_t, 128><<<g, b, 0, st>>>(tab, Hkv, (const uint16_t*)ks, ss, norms);
  else if (dtype == 0) k_row_sumsq<uint16_t, 64><<<g, b, 0, st>>>(tab, Hkv, (const uint16_t*)ks, ss, norms);
  else if (D == 128) k_row_sumsq<float, 128><<<g, b, 0, st>>>(tab, Hkv, (const float*)ks, ss, norms);
  else k_row_sumsq<float, 64><<<g, b, 0, st>>>(tab, Hkv, (const float*)ks, ss, norms);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  k_anchor_topk<<<dim3((tab.n + 3) / 4), dim3(256), 0, st>>>(tab, k, ss, anchors);
  return hipGetLastError();
}

}  // namespace sra
