// Attention statistics of a full causal prefill for chunk-level recompute decisions (Cache-Craft:
// the inter-attention between chunks, KVCache reuse 01 §2.3.1, and the per-token table the token
// selection sums, Cache-Craft CSDN article §2.2.2).
//
// For context token t (query rotated at t) and chunk j:
//   inter[t][j] = sum over query heads h of  sum_{s in chunk j, s <= t} softmax_{s' <= t}(q_th . k_s' / sqrt(d))
// with the keys as the prefill's cache stores them.
//
// bf16, gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), exact to float32 rounding:
//   * A work group owns one tile of 128 query vectors (flattened (token, head in group) pairs, as
//     in the sparse attention) of one (request, KV head) and walks every key unit (64 keys) up to
//     its last token twice. Pass 1 forms each query's exact float32 maximum and sum (query operand
//     split into bf16 hi/lo, keys exact bf16); pass 2 recomputes the logits, normalises them and
//     adds the probabilities of each chunk's keys.
//   * Each query vector's chunk totals go to 64-bit fixed-point slots [token][chunk] (value x 2^40)
//     with system-scope atomics, so the sum over heads and work groups is exact and independent of
//     order. Tiles are dealt heaviest first (the last tokens see the most keys).
//   * A finishing kernel turns the slots into inter[t][j], the token scores sum_{j < c(t)} inter[t][j]
//     and per chunk CCI = sigmoid(sum inter / sum intra) from exact 64-bit totals.
#include "common.h"

namespace sra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr double kStatsFix = 1099511627776.0;   // 2^40

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// tab: one entry per (request, chunk) of this launch's requests, in request then chunk order:
// req, dst = first token, len = tokens.
struct StatsArgs {
  const uint16_t* qop;
  const uint16_t* kc;
  unsigned long long* fx;
  int qop_blocks, Hkv, g, Lk, Lctx, n_chunks, n_tiles, req0;
};

template <int D>
__global__ __launch_bounds__(256, 2) void k_chunk_stats(StatsArgs a, ChunkTab tab) {
  constexpr int NKS = D / 16;
  constexpr int KT = 64;
  constexpr int KST = D + 8;
  constexpr int NKL = KT * (D / 8) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KST];
  __shared__ int cst[kMaxEntries + 1];   // this request's chunk starts, then L_ctx

  const int tile = a.n_tiles - 1 - (int)blockIdx.x;   // heaviest tiles first
  const int gl = blockIdx.y;                          // (request within the launch, KV head)
  const int rq = gl / a.Hkv, kvh = gl % a.Hkv;
  const int req = a.req0 + rq;
  const int group = req * a.Hkv + kvh;
  const int g = a.g;
  const int Mv = a.Lctx * g;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int e0 = rq * a.n_chunks;                     // this request's first chunk entry
  for (int i = threadIdx.x; i <= a.n_chunks; i += 256) cst[i] = i < a.n_chunks ? tab.dst[e0 + i] : a.Lctx;
  auto cstart = [&](int c) { return cst[c]; };         // read after the first barrier below

  const int v = tile * 128 + wave * 32 + l32;
  const bool qvalid = v < Mv;
  const int t = min(v, Mv - 1) / g;                  // this lane's token
  const int tmax = min((tile * 128 + 127) / g, a.Lctx - 1);
  const int kend = tmax + 1;                          // keys 0 .. tmax

  bf16x8 qhi[NKS], qlo[NKS];
  {
    const char* qb = reinterpret_cast<const char*>(a.qop + qop_index(group, tile * 4 + wave, 0, 0, 0, 0, a.qop_blocks, NKS));
    const uint32_t lo = (uint32_t)(l32 * 16 + hh * 8) * 2u;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qhi[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qb + ((uint32_t)(ks * 2 + 0) * 1024u + lo)));
      qlo[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qb + ((uint32_t)(ks * 2 + 1) * 1024u + lo)));
    }
    if (!qvalid) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qhi[ks] = qlo[ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }
  const char* kbase = reinterpret_cast<const char*>(a.kc + ((int64_t)req * a.Lk * a.Hkv + kvh) * D);
  const uint32_t row_bytes = (uint32_t)(a.Hkv * D * 2);
  u32x4 kr[NKL];
  auto prefetch = [&](int kt0) {   // clamped rows: keys past kend are masked
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int u = threadIdx.x + 256 * i;
      const uint32_t j = (uint32_t)min(kt0 + u / (D / 8), kend - 1);
      kr[i] = *reinterpret_cast<const u32x4*>(kbase + (j * row_bytes + 16u * (uint32_t)(u % (D / 8))));
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int uu = threadIdx.x + 256 * i;
      *reinterpret_cast<u32x4*>(&Ks[buf][(uu / (D / 8)) * KST + 8 * (uu % (D / 8))]) = kr[i];
    }
  };
  // S^T[key][q] of a tile's two 32-key halves in the log2 domain (query pre-scaled), causal mask
  auto logits = [&](const uint16_t* Kc, int kt0, f32x16 (&sc)[2]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sc[st] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(Kc + (32 * st + l32) * KST + 16 * ks + 8 * hh));
        sc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qhi[ks], sc[st], 0, 0, 0);
        sc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qlo[ks], sc[st], 0, 0, 0);
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = kt0 + 32 * st + 8 * (rr >> 2) + 4 * hh + (rr & 3);
        if (key > t) sc[st][rr] = -INFINITY;
      }
    }
  };
  // walks the key units with double-buffered LDS tiles; body(Kc, kt0) per unit
  auto walk = [&](auto&& body) {
    prefetch(0);
    store_tile(0);
    if (KT < kend) prefetch(KT);
    __syncthreads();
    int cur = 0;
    for (int kt0 = 0; kt0 < kend; kt0 += KT) {
      body(Ks[cur], kt0);
      if (kt0 + KT < kend) {
        store_tile(cur ^ 1);
        if (kt0 + 2 * KT < kend) prefetch(kt0 + 2 * KT);
      }
      __syncthreads();
      cur ^= 1;
    }
  };

  // pass 1: exact maximum and sum per query vector
  float m = -INFINITY, l = 0.f;
  walk([&](const uint16_t* Kc, int kt0) {
    f32x16 sc[2];
    logits(Kc, kt0, sc);
    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, sc[st][rr]);
    mt = half_max(mt);
    const float mn = fmaxf(m, mt);
    float s = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s += fast_exp2(sc[st][rr] - mn);
    l = (m == -INFINITY ? 0.f : l * fast_exp2(m - mn)) + s;
    m = mn;
  });
  const float inv = 1.f / half_sum(l);   // key 0 <= t: the sum is at least 1

  // pass 2: probabilities per chunk, flushed to the token's slot when the chunk changes (the chunk
  // index is the same in every lane)
  int cc = 0;
  float acc = 0.f;
  auto flush = [&]() {
    const float vsum = half_sum(acc);
    if (hh == 0 && qvalid)
      __hip_atomic_fetch_add(a.fx + ((int64_t)req * a.Lctx + t) * a.n_chunks + cc,
                             (unsigned long long)__double2ll_rn((double)vsum * kStatsFix), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_SYSTEM);
    acc = 0.f;
  };
  walk([&](const uint16_t* Kc, int kt0) {
    f32x16 sc[2];
    logits(Kc, kt0, sc);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sc[st][rr] = fast_exp2(sc[st][rr] - m) * inv;
    const int kt1 = min(kt0 + KT, kend);
    for (;;) {   // chunks overlapping [kt0, kt1), in order (uniform over the wave)
      const int c0 = max(cstart(cc), kt0), c1 = min(cstart(cc + 1), kt1);
      float s = 0.f;
      if (c0 == kt0 && c1 == kt1) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) s += sc[st][rr];
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int key = kt0 + 32 * st + 8 * (rr >> 2) + 4 * hh + (rr & 3);
            s += (key >= c0 && key < c1) ? sc[st][rr] : 0.f;
          }
      }
      acc += s;
      if (cstart(cc + 1) >= kt1) break;
      flush();
      cc = __builtin_amdgcn_readfirstlane(cc + 1);
    }
  });
  flush();
}

// One block per (chunk, request): slots to floats, token scores, and the chunk's CCI.
__global__ __launch_bounds__(256) void k_stats_finish(ChunkTab tab, const unsigned long long* __restrict__ fx,
                                                      int Lctx, int n_chunks, int req0, float* __restrict__ inter,
                                                      float* __restrict__ score, float* __restrict__ cci) {
  __shared__ unsigned long long sa, sb;
  const int rq = blockIdx.y, c = blockIdx.x;
  const int e = rq * n_chunks + c;
  const int req = req0 + rq;
  const int t0 = tab.dst[e], T = tab.len[e];
  if (threadIdx.x == 0) { sa = 0ull; sb = 0ull; }
  __syncthreads();
  unsigned long long ea = 0ull, eb = 0ull;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    const int t = t0 + i;
    const unsigned long long* row = fx + ((int64_t)req * Lctx + t) * n_chunks;
    unsigned long long before = 0ull;
    for (int j = 0; j < n_chunks; ++j) {
      const unsigned long long x = row[j];
      if (inter) inter[((int64_t)req * Lctx + t) * n_chunks + j] = (float)((double)x / kStatsFix);
      if (j < c) before += x;
    }
    if (score) score[(int64_t)req * Lctx + t] = (float)((double)before / kStatsFix);
    ea += before;
    eb += row[c];
  }
  atomicAdd(&sa, ea);
  atomicAdd(&sb, eb);
  __syncthreads();
  if (threadIdx.x == 0 && cci) {
    const double r = sb > 0 ? (double)sa / (double)sb : 0.0;
    cci[(int64_t)req * n_chunks + c] = (float)(1.0 / (1.0 + exp(-r)));
  }
}

}  // namespace

hipError_t launch_chunk_stats(int D, int n_req_launch, int req0, int Hq, int Hkv, int Lctx, int Lk,
                              const uint16_t* qop, int qop_blocks, const uint16_t* kc, const ChunkTab& tab,
                              int n_chunks, unsigned long long* fx, float* inter, float* score, float* cci,
                              hipStream_t st) {
  if (n_req_launch == 0 || Lctx == 0) return hipSuccess;
  StatsArgs a;
  a.qop = qop; a.kc = kc; a.fx = fx;
  a.qop_blocks = qop_blocks; a.Hkv = Hkv; a.g = Hq / Hkv; a.Lk = Lk; a.Lctx = Lctx;
  a.n_chunks = n_chunks; a.n_tiles = (Lctx * a.g + 127) / 128; a.req0 = req0;
  if (qop_blocks < 4 * a.n_tiles) return hipErrorInvalidValue;
  const dim3 g((unsigned)a.n_tiles, (unsigned)(n_req_launch * Hkv));
  if (D == 128) k_chunk_stats<128><<<g, dim3(256), 0, st>>>(a, tab);
  else k_chunk_stats<64><<<g, dim3(256), 0, st>>>(a, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_stats_finish<<<dim3((unsigned)n_chunks, (unsigned)n_req_launch), dim3(256), 0, st>>>(tab, fx, Lctx, n_chunks, req0,
                                                                                       inter, score, cci);
  return hipGetLastError();
}

}  // namespace sra
