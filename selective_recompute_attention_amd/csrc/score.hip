// Query-centric scoring against one critical layer (QCFuse technical summary (zh), §2.A critical-
// layer attention profiling; (ja) §2 system workflow: only the critical middle layer's K is
// loaded, the attention of the query's Q against it ranks the context tokens).
//
//   s_j = sum_{h < Hq} sum_{i < Lq} softmax_j( R(L_ctx+i) q_{i,h} . R(delta_c) k_{j,h/g} / sqrt(d) )
//
// bf16 path (matrix cores). The rotation is moved entirely to the query side: since rotations of
// the same pair commute and are orthogonal, R(a)q . R(b)k = R(a-b)q . k, so every chunk c gets its
// own rotated query q'' = R(L_ctx + i - delta_c) q and the cached keys are used exactly as stored
// (exact bf16 operands). q'' is float32; it is split into hi = bf16(q'') and lo = bf16(q'' - hi),
// and both halves are multiplied against the same keys (two MFMAs), which keeps the logits within a
// few 1e-6 of the exact value -- tight enough that the top-N choice matches an exact computation.
//   prep   : q'' hi/lo per (request, chunk, KV head), laid out as 32x32x16 MFMA operands.
//   pass 1 : per 128-key block, per query vector, the block's (max, sum of exp) of the logits.
//   merge  : per query vector, the (max, 1/sum) over all key blocks, in block order.
//   pass 2 : per key, the sum over its KV head's query vectors of exp(logit - max) / sum, written
//            per KV head; the selection kernel adds the KV heads in order. No float atomics.
// f32 path (exact float32 storage): plain dot products, one block per query vector.
#include <float.h>

#include "common.h"

namespace sra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// grid (Lq, entries): one block per (query row i, chunk entry).
template <int D>
__global__ __launch_bounds__(256) void k_score_prep(ChunkTab tab, int Lq, int Hq, int Hkv, int Mpad,
                                                    int Lctx, const uint16_t* __restrict__ qc,
                                                    uint16_t* __restrict__ qrot, int64_t plane,
                                                    int entry_base, double base) {
  constexpr int H = D / 2;
  __shared__ float2 cs[H];
  const int i = blockIdx.x, e = blockIdx.y;
  const int req = tab.req[e];
  const double pos = (double)Lctx + (double)i - (double)tab.delta[e];
  for (int j = threadIdx.x; j < H; j += blockDim.x) cs[j] = rope_cs(pos, j, D, base);
  __syncthreads();
  const int g = Hq / Hkv;
  const int eg = entry_base + e;
  const uint16_t* q = qc + ((int64_t)req * Lq + i) * Hq * D;
  for (int u = threadIdx.x; u < Hq * H; u += blockDim.x) {
    const int h = u / H, j = u % H;
    const float a = bf2f(q[h * D + j]), b = bf2f(q[h * D + j + H]);
    const float c = cs[j].x, s = cs[j].y;
    const float r0 = a * c - b * s, r1 = a * s + b * c;
    const uint32_t h0 = f2bf(r0), h1 = f2bf(r1);
    const uint32_t l0 = f2bf(r0 - bf2f(h0)), l1 = f2bf(r1 - bf2f(h1));
    const int kvh = h / g, v = i * g + (h % g);
    const int64_t o = ((int64_t)(eg * Hkv + kvh) * Mpad + v) * D;
    qrot[o + j] = (uint16_t)h0;
    qrot[o + j + H] = (uint16_t)h1;
    qrot[plane + o + j] = (uint16_t)l0;
    qrot[plane + o + j + H] = (uint16_t)l1;
  }
  if (i == 0) {  // zero the padding query vectors [Lq*g, Mpad) of every KV head
    const int pad = Mpad - Lq * g;
    for (int u = threadIdx.x; u < Hkv * pad * D; u += blockDim.x) {
      const int kvh = u / (pad * D), rem = u % (pad * D);
      const int64_t o = ((int64_t)(eg * Hkv + kvh) * Mpad + Lq * g) * D + rem;
      qrot[o] = 0;
      qrot[plane + o] = 0;
    }
  }
}

// grid (key blocks, Hkv); 4 waves, each owning 32 keys of a 128-key block of one chunk.
// PASS 1 writes ml_part[blk][kvh][v] = (max, sum exp2(y - max)) over the block's keys;
// PASS 2 writes colsum[req][kvh][j] = sum_v exp2(y - M_v) * invS_v.
template <int D, int PASS>
__global__ __launch_bounds__(256) void k_score_pass(ChunkTab tab, int Hkv, int Mpad, int Mvalid,
                                                    int Lctx, const uint16_t* __restrict__ kc,
                                                    const uint16_t* __restrict__ qrot,
                                                    int64_t plane, int entry_base, int blk_base,
                                                    float2* __restrict__ ml_part,
                                                    const float2* __restrict__ ml_final,
                                                    float* __restrict__ colsum, float scale_log2) {
  constexpr int NKS = D / 16;
  extern __shared__ float2 smem[];
  const int blk = blockIdx.x, kvh = blockIdx.y;
  const int e = find_entry(tab, blk);
  const int kb = blk - tab.blk0[e];
  const int req = tab.req[e], len = tab.len[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int t_base = kb * 128 + wave * 32;
  const int tk = t_base + l32;
  const bool kvalid = tk < len;
  const int64_t trow = (int64_t)tab.src[e] + min(tk, len - 1);

  // this lane's key row (32x32x16 operand: key = l32, dims 16*ks + 8*hh .. +8)
  bf16x8 kreg[NKS];
  const uint16_t* kp = kc + (trow * Hkv + kvh) * D + 8 * hh;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) kreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + 16 * ks));

  const uint16_t* qb = qrot + (int64_t)((entry_base + e) * Hkv + kvh) * Mpad * D + 8 * hh;
  const int nqt = Mpad / 32;

  if constexpr (PASS == 1) {
    float2* wpart = smem;  // [4][Mpad]
    for (int qt = 0; qt < nqt; ++qt) {
      const uint16_t* qp = qb + (int64_t)(32 * qt + l32) * D;
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 qh = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * ks));
        const bf16x8 ql = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + plane + 16 * ks));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreg[ks], qh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreg[ks], ql, acc, 0, 0, 0);
      }
      // acc[r] = logit of key t_base + 8*(r/4) + 4*hh + r%4 for query vector 32*qt + l32
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t_base + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key < len) m = fmaxf(m, acc[r] * scale_log2);
      }
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t_base + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key < len) s += exp2f(acc[r] * scale_log2 - m);
        }
      }
      s += __shfl_xor(s, 32, 64);
      if (hh == 0) wpart[wave * Mpad + 32 * qt + l32] = make_float2(m, s);
    }
    __syncthreads();
    float2* dst = ml_part + ((int64_t)(blk_base + blk) * Hkv + kvh) * Mpad;
    for (int v = threadIdx.x; v < Mpad; v += blockDim.x) {
      float M = -INFINITY;
      for (int w = 0; w < 4; ++w) M = fmaxf(M, wpart[w * Mpad + v].x);
      float S = 0.f;
      if (M != -INFINITY)
        for (int w = 0; w < 4; ++w) {
          const float2 p = wpart[w * Mpad + v];
          if (p.x != -INFINITY) S += p.y * exp2f(p.x - M);
        }
      dst[v] = make_float2(M, S);
    }
  } else {
    float2* mlf = smem;  // [Mpad]
    const float2* src = ml_final + ((int64_t)req * Hkv + kvh) * Mpad;
    for (int v = threadIdx.x; v < Mpad; v += blockDim.x) mlf[v] = src[v];
    __syncthreads();
    float col = 0.f;
    for (int qt = 0; qt < nqt; ++qt) {
      const uint16_t* qp = qb + (int64_t)(32 * qt + l32) * D;
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 qh = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * ks));
        const bf16x8 ql = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + plane + 16 * ks));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh, kreg[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql, kreg[ks], acc, 0, 0, 0);
      }
      // acc[r] = logit of query vector 32*qt + 8*(r/4) + 4*hh + r%4 against key t_base + l32
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float2 ml = mlf[32 * qt + 8 * (r >> 2) + 4 * hh + (r & 3)];
        col += exp2f(acc[r] * scale_log2 - ml.x) * ml.y;
      }
    }
    col += __shfl_xor(col, 32, 64);
    if (hh == 0 && kvalid) colsum[((int64_t)req * Hkv + kvh) * Lctx + tab.dst[e] + tk] = col;
  }
}

struct ReqBlocks {
  int blk0[kMaxEntries + 1];
};

__global__ void k_score_merge(int n_req, int Hkv, int Mpad, int Mvalid, ReqBlocks rb,
                              const float2* __restrict__ ml_part, float2* __restrict__ ml_final) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_req * Hkv * Mpad) return;
  const int v = (int)(idx % Mpad);
  const int kvh = (int)((idx / Mpad) % Hkv);
  const int req = (int)(idx / ((int64_t)Mpad * Hkv));
  if (v >= Mvalid) {
    ml_final[idx] = make_float2(0.f, 0.f);
    return;
  }
  float M = -INFINITY;
  for (int b = rb.blk0[req]; b < rb.blk0[req + 1]; ++b)
    M = fmaxf(M, ml_part[((int64_t)b * Hkv + kvh) * Mpad + v].x);
  float S = 0.f;
  for (int b = rb.blk0[req]; b < rb.blk0[req + 1]; ++b) {
    const float2 p = ml_part[((int64_t)b * Hkv + kvh) * Mpad + v];
    if (p.x != -INFINITY) S += p.y * exp2f(p.x - M);
  }
  ml_final[idx] = make_float2(M, S > 0.f ? 1.f / S : 0.f);
}

// ---------------------------------------------------------------------------- float32 path
// grid (Hq*Lq, n_req): one block per query vector (i, h) of one request; writes its softmax row
// prob[req][i*Hq + h][0..Lctx).
template <int D>
__global__ __launch_bounds__(256) void k_score_f32(ChunkTab tab, int Lq, int Hq, int Hkv, int Lctx,
                                                   const float* __restrict__ qc,
                                                   const float* __restrict__ kc,
                                                   float* __restrict__ prob, float scale_log2,
                                                   double base) {
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
      const float2 c = rope_cs(pos, threadIdx.x, D, base);
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

hipError_t launch_score_prep(int D, const ChunkTab& tab, int Lq, int Hq, int Hkv, int Mpad,
                             int Lctx, const void* qc, uint16_t* qrot, int64_t plane,
                             int entry_base, double base, hipStream_t st) {
  if (tab.n == 0 || Lq == 0) return hipSuccess;
  dim3 g(Lq, tab.n), b(256);
  if (D == 128)
    k_score_prep<128><<<g, b, 0, st>>>(tab, Lq, Hq, Hkv, Mpad, Lctx, (const uint16_t*)qc, qrot,
                                        plane, entry_base, base);
  else
    k_score_prep<64><<<g, b, 0, st>>>(tab, Lq, Hq, Hkv, Mpad, Lctx, (const uint16_t*)qc, qrot,
                                       plane, entry_base, base);
  return hipGetLastError();
}

hipError_t launch_score_pass(int pass, int D, const ChunkTab& tab, int Hkv, int Mpad, int Mvalid,
                             int Lctx, const void* kc, const uint16_t* qrot, int64_t plane,
                             int entry_base, int blk_base, float2* ml_part, const float2* ml_final,
                             float* colsum, float scale_log2, hipStream_t st) {
  const int nblk = tab.blk0[tab.n];
  if (nblk == 0) return hipSuccess;
  dim3 g(nblk, Hkv), b(256);
  const size_t lds = (pass == 1 ? 4 : 1) * (size_t)Mpad * sizeof(float2);
  const uint16_t* k = (const uint16_t*)kc;
#define SRA_PASS(DD, PP)                                                                        \
  k_score_pass<DD, PP><<<g, b, lds, st>>>(tab, Hkv, Mpad, Mvalid, Lctx, k, qrot, plane,         \
                                          entry_base, blk_base, ml_part, ml_final, colsum,      \
                                          scale_log2)
  if (D == 128 && pass == 1) SRA_PASS(128, 1);
  else if (D == 128) SRA_PASS(128, 2);
  else if (pass == 1) SRA_PASS(64, 1);
  else SRA_PASS(64, 2);
#undef SRA_PASS
  return hipGetLastError();
}

hipError_t launch_score_merge(int n_req, int Hkv, int Mpad, int Mvalid, const int* req_blk0,
                              const float2* ml_part, float2* ml_final, hipStream_t st) {
  ReqBlocks rb;
  for (int r = 0; r <= n_req; ++r) rb.blk0[r] = req_blk0[r];
  const int64_t n = (int64_t)n_req * Hkv * Mpad;
  k_score_merge<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(n_req, Hkv, Mpad, Mvalid,
                                                                         rb, ml_part, ml_final);
  return hipGetLastError();
}

hipError_t launch_score_f32(int D, const ChunkTab& tab_req, int n_req, int Lq, int Hq, int Hkv,
                            int Lctx, const float* qc, const float* kc, float* prob,
                            float scale_log2, double base, hipStream_t st) {
  dim3 g(Hq * Lq, n_req), b(256);
  if (D == 128)
    k_score_f32<128><<<g, b, 0, st>>>(tab_req, Lq, Hq, Hkv, Lctx, qc, kc, prob, scale_log2, base);
  else
    k_score_f32<64><<<g, b, 0, st>>>(tab_req, Lq, Hq, Hkv, Lctx, qc, kc, prob, scale_log2, base);
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
