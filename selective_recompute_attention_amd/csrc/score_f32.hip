// Float32-storage scoring (exact float32 inputs): plain dot products, one block per query vector,
// then fixed-order column sums. Same definition as the bf16 path (see score.hip): softmax over the
// context keys of each (query row, head), summed over heads and query rows.
#include <float.h>

#include "common.h"

namespace sra {
namespace {

// grid (Hq*Lq, n_req): one block per query vector (i, h) of one request; writes its softmax row
// prob[req][i*Hq + h][0..Lctx).
template <int D>
__global__ __launch_bounds__(256) void k_score_f32(ChunkTab tab, int Lq, int Hq, int Hkv, int Lctx,
                                                   const float* __restrict__ qc,
                                                   const float* __restrict__ kc,
                                                   float* __restrict__ prob, float scale_log2,
                                                   Theta th) {
  constexpr int H = D / 2;
  __shared__ float qr[D];
  __shared__ float red[256];
  const int qv = blockIdx.x, req = blockIdx.y;
  const int i = qv / Hq, h = qv % Hq, kvh = h / (Hq / Hkv);
  const float* q = qc + (((int64_t)req * Lq + i) * Hq + h) * D;
  float* row = prob + ((int64_t)req * Lq * Hq + qv) * Lctx;
  for (int e = 0; e < tab.n; ++e) {
    if (tab.req[e] != req) continue;
    const double pos = (double)Lctx + (double)i - (double)tab.delta[e];
    if (threadIdx.x < H) {
      const float2 c = rope_cs(pos, th.v[threadIdx.x]);
      const float a = q[threadIdx.x], b = q[threadIdx.x + H];
      qr[threadIdx.x] = a * c.x - b * c.y;
      qr[threadIdx.x + H] = a * c.y + b * c.x;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < tab.len[e]; t += blockDim.x) {
      const float* k = kc + (((int64_t)tab.src[e] + t) * Hkv + kvh) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot += qr[d] * k[d];
      row[tab.dst[e] + t] = dot * scale_log2;
    }
    __syncthreads();
  }
  float m = -INFINITY;
  for (int j = threadIdx.x; j < Lctx; j += blockDim.x) m = fmaxf(m, row[j]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int j = threadIdx.x; j < Lctx; j += blockDim.x) sum += exp2f(row[j] - M);
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const float inv = 1.f / red[0];
  for (int j = threadIdx.x; j < Lctx; j += blockDim.x) row[j] = exp2f(row[j] - M) * inv;
}

__global__ void k_colsum_f32(int n_req, int rows, int Lctx, const float* __restrict__ prob,
                             float* __restrict__ parts) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_req * Lctx) return;
  const int j = (int)(idx % Lctx), req = (int)(idx / Lctx);
  const float* p = prob + (int64_t)req * rows * Lctx + j;
  float s = 0.f;
  for (int v = 0; v < rows; ++v) s += p[(int64_t)v * Lctx];
  parts[idx] = s;
}

}  // namespace

hipError_t launch_score_f32(int D, const ChunkTab& tab_req, int n_req, int Lq, int Hq, int Hkv,
                            int Lctx, const float* qc, const float* kc, float* prob,
                            float scale_log2, double base, hipStream_t st) {
  dim3 g(Hq * Lq, n_req), b(256);
  const Theta th = make_theta(D, base);
  if (D == 128)
    k_score_f32<128><<<g, b, 0, st>>>(tab_req, Lq, Hq, Hkv, Lctx, qc, kc, prob, scale_log2, th);
  else
    k_score_f32<64><<<g, b, 0, st>>>(tab_req, Lq, Hq, Hkv, Lctx, qc, kc, prob, scale_log2, th);
  return hipGetLastError();
}

hipError_t launch_colsum_f32(int n_req, int rows, int Lctx, const float* prob, float* parts,
                             hipStream_t st) {
  const int64_t n = (int64_t)n_req * Lctx;
  if (n == 0) return hipSuccess;
  k_colsum_f32<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(n_req, rows, Lctx, prob,
                                                                       parts);
  return hipGetLastError();
}

}  // namespace sra
