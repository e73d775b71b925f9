// Key-norm anchors per precomputed chunk (QCFuse technical summary (zh), §2.A anchor-based
// lightweight query probing: offline, each chunk keeps the few tokens with the largest key norm
// as a compressed semantic summary).
//
// One block per chunk. Each wave reduces the squared entries of one token's key row (all KV
// heads and dims) in float64 -- squares of bf16/f32 values are exact there, so the ranking
// matches an exact computation up to the last float64 bit -- then k block-wide argmax rounds
// pick the anchors in the order (larger norm first, lower token offset on a tie).
#include <float.h>

#include "common.h"

namespace sra {
namespace {

constexpr int kAnchorTokens = 8192;

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

template <typename T>
__global__ __launch_bounds__(256) void k_anchors(ChunkTab tab, int row_elems, int k,
                                                 const T* __restrict__ ks,
                                                 int32_t* __restrict__ anchors,
                                                 float* __restrict__ norms) {
  __shared__ double ss[kAnchorTokens];
  __shared__ double red_v[4];
  __shared__ int red_t[4];
  const int e = blockIdx.x;
  const int src = tab.src[e], len = tab.len[e], out = tab.dst[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = row_elems * (int)sizeof(T) / 16;
  for (int t = wave; t < len; t += 4) {
    const u32x4* row = reinterpret_cast<const u32x4*>(ks + ((int64_t)src + t) * row_elems);
    double acc = 0.0;
    for (int u = lane; u < n16; u += 64) acc += sumsq16<T>(row[u]);
    // fixed-order tree: lane 0 ends with the same sum on every run
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_down(acc, off, 64);
    if (lane == 0) {
      ss[t] = acc;
      if (norms) norms[(int64_t)src + t] = (float)sqrt(acc);
    }
  }
  __syncthreads();
  for (int round = 0; round < k; ++round) {
    double bv = -DBL_MAX;
    int bt = INT_MAX;
    for (int t = threadIdx.x; t < len; t += blockDim.x) {
      const double v = ss[t];
      if (v > bv || (v == bv && t < bt)) { bv = v; bt = t; }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const double ov = __shfl_down(bv, off, 64);
      const int ot = __shfl_down(bt, off, 64);
      if (ov > bv || (ov == bv && ot < bt)) { bv = ov; bt = ot; }
    }
    if (lane == 0) { red_v[wave] = bv; red_t[wave] = bt; }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < 4; ++w)
        if (red_v[w] > bv || (red_v[w] == bv && red_t[w] < bt)) { bv = red_v[w]; bt = red_t[w]; }
      anchors[(int64_t)out * k + round] = bt;
      ss[bt] = -1.0;  // below every sum of squares: never picked again
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_anchors(int dtype, int row_elems, const ChunkTab& tab, int k, const void* ks,
                          int32_t* anchors, float* norms, hipStream_t st) {
  if (tab.n == 0) return hipSuccess;
  if (dtype == 0)
    k_anchors<uint16_t><<<dim3(tab.n), dim3(256), 0, st>>>(tab, row_elems, k, (const uint16_t*)ks,
                                                           anchors, norms);
  else
    k_anchors<float><<<dim3(tab.n), dim3(256), 0, st>>>(tab, row_elems, k, (const float*)ks,
                                                        anchors, norms);
  return hipGetLastError();
}

}  // namespace sra
