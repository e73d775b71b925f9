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
//   pass 1 : per 128-key block, per query vector, the block's (max, sum of exp2) of the logits.
//   merge  : per query vector, (max, 1/sum) over all blocks of its request in block order -- inside
//            pass 2 when a request's partials are small, else as its own wide kernel.
//   pass 2 : per key, the sum over its KV head's query vectors of exp2(logit - max) / sum, added
//            over KV heads as 64-bit fixed point (integer atomics: exact, order-free).
// Every float reduction has a fixed order and there are no float atomics: runs are bit-reproducible.
// Cross-block results only meet at kernel boundaries (no device-scope fences, which on this GPU
// write back the L2).
#include <float.h>

#include "common.h"
#include "rerotate.h"

#include <algorithm>

namespace sra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// grid (Lq, entries): one block per (query row i, chunk entry); a thread rotates 8 pairs of one
// head with 16-byte loads and stores. The first batch of loads goes out before the angles.
template <int D>
__global__ __launch_bounds__(256) void k_score_prep(ChunkTab tab, int Lq, int Hq, int Hkv, int Mpad,
                                                    int Lctx, const uint16_t* __restrict__ qc,
                                                    uint16_t* __restrict__ qrot, int64_t plane,
                                                    int entry_base, float scale_log2,
                                                    unsigned long long* __restrict__ fx, Theta th) {
  constexpr int H = D / 2;
  __shared__ float2 cs[H];
  const int i = blockIdx.x, e = blockIdx.y;
  const int req = tab.req[e];
  const int eg = entry_base + e;
  // every argument, fetched as one batch of scalar loads (the asm takes them all, and hands back
  // the head counts so the division waits for it)
  int hq = Hq, hkv = Hkv;
  {
    const int delta_e = tab.delta[e];
    asm volatile("" : "+s"(hq), "+s"(hkv) : "s"(req), "s"(delta_e), "s"(qc), "s"(qrot), "s"(plane), "s"(eg),
                 "s"(Lq), "s"(Mpad), "s"(Lctx), "s"(scale_log2), "s"(fx));
  }
  const int g = hq / hkv;
  const uint16_t* q = qc + ((int64_t)req * Lq + i) * Hq * D;
  const int nu = Hq * (H / 8);
  const int u0 = min((int)threadIdx.x, nu - 1);
  const u32x4 wa0 = *reinterpret_cast<const u32x4*>(q + (u0 / (H / 8)) * D + (u0 % (H / 8)) * 8);
  const u32x4 wb0 = *reinterpret_cast<const u32x4*>(q + (u0 / (H / 8)) * D + (u0 % (H / 8)) * 8 + H);
  const double pos = (double)Lctx + (double)i - (double)tab.delta[e];
  for (int j = threadIdx.x; j < H; j += blockDim.x) cs[j] = rope_cs(pos, th.v[j]);
  __syncthreads();
  auto rotate_store = [&](int u, u32x4 wa, u32x4 wb) {
    const int h = u / (H / 8), j0 = (u % (H / 8)) * 8;
    u32x4 hi0, hi1, lo0, lo1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t ha[2], hb[2], la[2], lb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float a = bf2f((wa[k] >> (16 * t)) & 0xffffu), b = bf2f((wb[k] >> (16 * t)) & 0xffffu);
        const float2 c = cs[j0 + 2 * k + t];
        // log2(e)/sqrt(d) is folded in: the products come out as exp2 exponents
        const float r0 = (a * c.x - b * c.y) * scale_log2, r1 = (a * c.y + b * c.x) * scale_log2;
        ha[t] = f2bf(r0);
        hb[t] = f2bf(r1);
        la[t] = f2bf(r0 - bf2f(ha[t]));
        lb[t] = f2bf(r1 - bf2f(hb[t]));
      }
      hi0[k] = ha[0] | (ha[1] << 16);
      hi1[k] = hb[0] | (hb[1] << 16);
      lo0[k] = la[0] | (la[1] << 16);
      lo1[k] = lb[0] | (lb[1] << 16);
    }
    const int kvh = h / g, v = i * g + (h % g);
    const int64_t o = ((int64_t)(eg * Hkv + kvh) * Mpad + v) * D + j0;
    *reinterpret_cast<u32x4*>(qrot + o) = hi0;
    *reinterpret_cast<u32x4*>(qrot + o + H) = hi1;
    *reinterpret_cast<u32x4*>(qrot + plane + o) = lo0;
    *reinterpret_cast<u32x4*>(qrot + plane + o + H) = lo1;
  };
  if ((int)threadIdx.x < nu) rotate_store(threadIdx.x, wa0, wb0);
  for (int u = threadIdx.x + blockDim.x; u < nu; u += blockDim.x) {
    const uint16_t* src = q + (u / (H / 8)) * D + (u % (H / 8)) * 8;
    rotate_store(u, *reinterpret_cast<const u32x4*>(src), *reinterpret_cast<const u32x4*>(src + H));
  }
  if (i == 0 && fx) {  // clear this chunk's score accumulators (pass 2 adds into them)
    unsigned long long* f = fx + (int64_t)req * Lctx + tab.dst[e];
    for (int t = threadIdx.x; t < tab.len[e]; t += blockDim.x) f[t] = 0ull;
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

// Online merge of one (max, sum of exp2(y - max)) pair into a running pair. Branch-free: an empty
// pair (-inf, 0) scales the running sum by exp2(0) = 1 and adds 0, so it leaves the pair's bits as
// they are; when both maxima are -inf the shift is 0 and the sum stays 0. The bare exp2 flushes
// results below 2^-126 to zero: one of the two terms has weight exp2(0) = 1 on a sum >= 1 (a
// non-empty pair counts its own maximum once), and a sum counts fewer than 2^31 keys, so a flushed
// term (below 2^31 * 2^-126) could not have changed the float32 result.
__device__ __forceinline__ void ml_merge(float& M, float& S, float2 p) {
  const float nm = fmaxf(M, p.x);
  const float sh = nm == -INFINITY ? 0.f : nm;
  S = S * fast_exp2(M - sh) + p.y * fast_exp2(p.x - sh);
  M = nm;
}

// (max, 1/sum) over blocks [b0, b1) of query vectors [v_lo, v_lo + v_cnt) of one (request, KV head),
// written to out[v]. T = 256 / v_cnt threads share a vector; thread j covers blocks b0+j, b0+j+T,
// ... in order (loads issued 8 at a time), then thread 0 of the vector merges j = 0..T-1 in order.
__device__ void merge_rows(int b0, int b1, int Hkv, int kvh, int Mpad, int v_lo, int v_cnt,
                           int Mvalid, const float2* __restrict__ ml_part, float2* out) {
  __shared__ float2 part[256];
  const int T = v_cnt >= 256 ? 1 : 256 / v_cnt;
  const int j = threadIdx.x % T;
  for (int vb = 0; vb < v_cnt; vb += 256 / T) {
    const int vl = vb + threadIdx.x / T;
    const int v = v_lo + vl;
    float M = -INFINITY, S = 0.f;
    if (vl < v_cnt && v < Mvalid) {
      for (int b = b0 + j; b < b1; b += 8 * T) {
        float2 p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          p[u] = ml_part[((int64_t)min(b + u * T, b1 - 1) * Hkv + kvh) * Mpad + v];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (b + u * T >= b1) p[u] = make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int u = 0; u < 8; ++u) ml_merge(M, S, p[u]);
      }
    }
    part[threadIdx.x] = make_float2(M, S);
    __syncthreads();
    if (j == 0 && vl < v_cnt) {
      float MM = -INFINITY, SS = 0.f;
      for (int i = 0; i < T; ++i) ml_merge(MM, SS, part[threadIdx.x + i]);
      out[v] = (v < Mvalid && SS > 0.f) ? make_float2(MM, 1.f / SS) : make_float2(0.f, 0.f);
    }
    __syncthreads();
  }
}

// Global block index ranges of each request: blocks [blk0[q], blk0[q+1]).
struct ReqBlocks {
  int blk0[kMaxEntries + 1];
};

// grid (n_req * Hkv, ceil(Mpad / 64)): the separate merge for large partial sets.
__global__ __launch_bounds__(256) void k_score_merge(ReqBlocks rb, int Hkv, int Mpad, int Mvalid,
                                                     const float2* __restrict__ ml_part,
                                                     float2* __restrict__ ml_final) {
  const int req = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
  const int v_lo = blockIdx.y * 64;
  merge_rows(rb.blk0[req], rb.blk0[req + 1], Hkv, kvh, Mpad, v_lo, min(64, Mpad - v_lo), Mvalid,
             ml_part, ml_final + ((int64_t)req * Hkv + kvh) * Mpad);
}

template <int NKS>
__device__ __forceinline__ void load_q(const uint16_t* qp, int64_t plane, bf16x8* h, bf16x8* l) {
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    h[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * ks));
    l[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + plane + 16 * ks));
  }
}

// Anchors of chunk entry e (one block): the key-norm totals (per-head sums added in head order) go
// to LDS, then wave 0 takes k rounds, each picking the best token ranked after the previous pick
// (larger sum first, lower offset on a tie; float64 sums of squares order like their bit patterns).
// Chunks of up to 512 tokens keep a lane's totals in registers across the rounds; a round's wave
// reduction carries (total, offset) only, "nothing found" being (0, INT_MAX), which any token beats
// (totals are sums of squares, so never below +0).
// (Scalar arguments only: a reference to the kernel-argument table would copy it to scratch.)
__device__ __forceinline__ void anchor_block(int len, int64_t base, int src, int64_t out_slot, int Hkv,
                                             const AnchorOut& anc, unsigned long long* tot) {
  // len <= kAnchorFusedMaxLen (checked by the host); base = the chunk's first context position.
  // Two tokens per thread per step, every head's load of both issued before any is added.
  for (int t0 = threadIdx.x; t0 < len; t0 += 2 * blockDim.x) {
    const int t1 = t0 + blockDim.x, t1c = min(t1, len - 1);
    double s0 = 0.0, s1 = 0.0;
    for (int h0 = 0; h0 < Hkv; h0 += 8) {
      double v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const double* row = anc.ssp + (int64_t)min(h0 + u, Hkv - 1) * anc.stride + base;
        v0[u] = row[t0];
        v1[u] = row[t1c];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (h0 + u < Hkv) {
          s0 += v0[u];
          s1 += v1[u];
        }
    }
    tot[t0] = __double_as_longlong(s0);
    if (anc.norms) anc.norms[(int64_t)src + t0] = (float)sqrt(s0);
    if (t1 < len) {
      tot[t1] = __double_as_longlong(s1);
      if (anc.norms) anc.norms[(int64_t)src + t1] = (float)sqrt(s1);
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  constexpr int RJ = 8;   // register-held totals per lane
  const bool in_reg = len <= 64 * RJ;
  unsigned long long rv[RJ];
  if (in_reg) {
#pragma unroll
    for (int j = 0; j < RJ; ++j) rv[j] = tot[min(lane + 64 * j, len - 1)];
  }
  unsigned long long pv = ~0ull;   // previous pick (value, offset); starts above everything
  int pt = -1;
  for (int round = 0; round < anc.k; ++round) {
    unsigned long long bv = 0;
    int bt = INT_MAX;
    // bitwise rather than short-circuit logic: the conditions become mask operations, not branches
    auto consider = [&](unsigned long long v, int t, bool valid) {
      const bool after = (v < pv) | ((v == pv) & (t > pt));
      const bool better = valid & after & ((v > bv) | ((v == bv) & (t < bt)));
      bv = better ? v : bv;
      bt = better ? t : bt;
    };
    if (in_reg) {
#pragma unroll
      for (int j = 0; j < RJ; ++j) consider(rv[j], lane + 64 * j, lane + 64 * j < len);
    } else {
      for (int t = lane; t < len; t += 64) consider(tot[t], t, true);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const unsigned long long ov = __shfl_xor(bv, off, 64);
      const int ot = __shfl_xor(bt, off, 64);
      const bool better = (ov > bv) | ((ov == bv) & (ot < bt));
      bv = better ? ov : bv;
      bt = better ? ot : bt;
    }
    if (lane == 0) anc.rows[out_slot * anc.k + round] = bt;
    pv = bv;
    pt = bt;
  }
}

// The global block range of each entry's request (the blocks whose partials pass 2 merges).
struct EntryReqBlocks {
  int lo[kMaxEntries];
  int hi[kMaxEntries];
};

// grid (bmax key blocks + extra blocks, Hkv, chunk entries). A block owns 128 keys of one chunk
// (staged once in LDS, rows padded for conflict-free 16-byte reads); wave w owns the 32-vector
// query tiles w, w+4, ... with their operands in registers. Every global load of a tile (K, Q and,
// in pass 2, the merge inputs) is issued before any of them is waited on, so each block pays about
// one memory latency after one round of kernel-argument reads.
// PASS 1 writes ml_part[blk][kvh][v] = (max, sum exp2(y - max)) over the block's keys (S^T = K Q^T:
// one query vector per lane column, its 128 keys across the registers of both half-waves).
// PASS 2 adds sum_v exp2(y - M_v) * invS_v of its KV head to the key's fixed-point score (S = Q K^T:
// one key per lane column), the four waves' sums added in wave order first.
// OWN: the pass forms its own inputs. Pass 1 rotates, scales and splits the raw query itself (and
// writes the operand for pass 2); otherwise it reads the operand that the preparation kernel wrote.
// Pass 2 merges the request's block partials itself; otherwise it reads the merged pairs.

template <int D, int PASS, bool OWN>
__global__ __launch_bounds__(256) void k_score_pass(ChunkTab tab, EntryReqBlocks erb, int bmax, int Hkv, int Mpad,
                                                    int Mvalid, int Lctx,
                                                    const uint16_t* __restrict__ kc,
                                                    uint16_t* __restrict__ qrot,
                                                    int64_t plane, int entry_base, int blk_base,
                                                    float2* __restrict__ ml_part,
                                                    const float2* __restrict__ ml_final,
                                                    unsigned long long* __restrict__ fx,
                                                    AnchorOut anc, RerotFused rf, QueryRot qr, Theta th) {
  constexpr int NKS = D / 16;
  constexpr int H = D / 2;
  constexpr int KB = 128;          // keys per block
  constexpr int KST = D + 8;       // LDS row stride (elements)
  constexpr int NKL = KB * (D / 8) / 256;
  constexpr int MB = 10;           // merge inputs per lane per batch
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KB * KST];
  __shared__ float colred[4][KB];
  __shared__ float2 mlw[4][32];
  __shared__ float2 qcs[PASS == 1 && OWN ? kInRotMaxLq * H : 1];   // cos/sin per (query row, i)
  // grid (bmax + extra, Hkv, entries): the entry comes from the grid, so every field of it is
  // one independent scalar load
  const int e = blockIdx.z, kvh = blockIdx.y, x = blockIdx.x;
  const int b0e = tab.blk0[e], nbe = tab.blk0[e + 1] - b0e;
  {   // every argument the block's first loads depend on, fetched as one batch of scalar loads
    const int len_e = tab.len[e], src_e = tab.src[e], req_e = tab.req[e], dst_e = tab.dst[e];
    const int lo_e = erb.lo[e], hi_e = erb.hi[e], delta_e = tab.delta[e];
    asm volatile("" ::"s"(b0e), "s"(nbe), "s"(bmax), "s"(len_e), "s"(src_e), "s"(req_e), "s"(dst_e),
                 "s"(lo_e), "s"(hi_e), "s"(kc), "s"(qrot), "s"(ml_part), "s"(ml_final), "s"(plane),
                 "s"(entry_base), "s"(blk_base), "s"(Mpad), "s"(Hkv), "s"(fx),
                 "s"(delta_e), "s"(qr.qc), "s"(qr.Lq), "s"(qr.Hq));
  }
  if (x >= bmax) {
    if constexpr (PASS == 1) {   // extra blocks: S1 for a contiguous share of kS1Fold key blocks' rows
      constexpr int SPAN = kS1Fold * KB;
      const int per = (SPAN + Hkv - 1) / Hkv;
      const int r0 = (x - bmax) * SPAN + kvh * per;
      const int nr = min(min(per, SPAN - kvh * per), tab.len[e] - r0);
      // one block per CU here: a thread's whole share of a 32-row span (bf16, d 128, 8 KV heads)
      // is one batch of loads
      if (nr > 0)
        rerot::rows<uint16_t, D, 16, 8>(tab, e, r0, nr, Hkv, rf.ks, rf.vs, rf.kf, rf.vf, rf.L, th,
                                        reinterpret_cast<float2*>(Ks), rf.sh);
    } else {   // one block per chunk entry picks its anchors
      if (kvh == 0)
        anchor_block(tab.len[e], (int64_t)tab.req[e] * Lctx + tab.dst[e], tab.src[e],
                     (int64_t)tab.req[e] * anc.n_chunks + tab.aux[e], Hkv, anc,
                     reinterpret_cast<unsigned long long*>(Ks));
    }
    return;
  }
  if (x >= nbe) return;   // a shorter entry's padding
  const int blk = b0e + x;
  const int t0 = x * KB;
  const int req = tab.req[e];
  const int nk = min(KB, tab.len[e] - t0);   // valid keys of this block (>= 1)
  const int rb0 = erb.lo[e], rb1 = erb.hi[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int nqt = Mpad / 32;
  const int v0 = min(32 * wave + l32, Mpad - 1);   // the wave's first query vector, clamped

  // Every global load of the block goes out before any of them is waited on: K rows (dims
  // fastest, 16 bytes per load; clamped rows, zeroed on their way to LDS), the wave's first query
  // tile and, in pass 2, that tile's first batch of merge inputs. Pass 1's query angles need one
  // frequency per thread (an indexed load): it goes first, as loads complete in order.
  double th_j = 0.0;
  if constexpr (PASS == 1 && OWN) {
    th_j = th.v[threadIdx.x % H];
    __builtin_amdgcn_sched_barrier(0);   // keep it ahead of the data loads
  }
  u32x4 kr[NKL];
  const uint16_t* kbase = kc + (((int64_t)tab.src[e] + t0) * Hkv + kvh) * D;
#pragma unroll
  for (int i = 0; i < NKL; ++i) {
    const int u = threadIdx.x + 256 * i;
    const int row = u / (D / 8);
    kr[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)min(row, nk - 1) * Hkv * D + 8 * (u % (D / 8)));
  }
  uint16_t* qb = qrot + (int64_t)((entry_base + e) * Hkv + kvh) * Mpad * D + 8 * hh;   // pass 1 may write it
  bf16x8 qh[NKS], ql[NKS];
  // pass 1 with OWN (one query tile per wave): the wave's raw query vectors instead, rotated
  // below; vector v = 32 wave + l32 is (row v / g, head kvh g + v % g), zero past Lq g
  u32x4 qraw[NKS];
  int qrow = 0;
  bool qok = false;
  if constexpr (PASS == 1 && OWN) {
    const int g = qr.Hq / Hkv, v = 32 * wave + l32, vc = min(v, qr.Lq * g - 1);
    qok = v < qr.Lq * g;
    qrow = vc / g;
    const uint16_t* src = qr.qc + (((int64_t)req * qr.Lq + qrow) * qr.Hq + kvh * g + vc % g) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qraw[ks] = *reinterpret_cast<const u32x4*>(src + 16 * ks);
  } else {   // unconditional (a wave past the last tile loads a valid vector it never uses), so no
             // value merges across a branch and forces a wait in the middle of the batch
    load_q<NKS>(qb + (int64_t)v0 * D, plane, qh, ql);
  }

  // pass 2: (max, 1/sum) of query vector 32 qt + l32 over the request's blocks; the two half-waves
  // take alternate blocks (batches of MB, clamped loads) and merge in a fixed order
  auto load_batch = [&](int v, int b, float2* pm) {
    const int b1 = rb1;
#pragma unroll
    for (int u = 0; u < MB; ++u)
      pm[u] = ml_part[((int64_t)min(b + 2 * u, b1 - 1) * Hkv + kvh) * Mpad + v];
  };
  auto merge_batch = [&](float& M, float& S, int b, const float2* pm) {
    const int b1 = rb1;
#pragma unroll
    for (int u = 0; u < MB; ++u) ml_merge(M, S, b + 2 * u < b1 ? pm[u] : make_float2(-INFINITY, 0.f));
  };
  auto finish_ml = [&](float M, float S, int v) -> float2 {
    float Mo = half_partner(M), So = half_partner(S);
    if (hh == 1) { const float tm = M, ts = S; M = Mo; S = So; Mo = tm; So = ts; }
    ml_merge(M, S, make_float2(Mo, So));   // half 0's blocks first, then half 1's
    return (v < Mvalid && S > 0.f) ? make_float2(M, 1.f / S) : make_float2(0.f, 0.f);
  };
  auto merged_ml = [&](int qt) -> float2 {   // later query tiles
    const int v = 32 * qt + l32;
    if (!OWN) return ml_final[((int64_t)req * Hkv + kvh) * Mpad + v];
    float M = -INFINITY, S = 0.f;
    for (int b = rb0 + hh; b < rb1; b += 2 * MB) {
      float2 pm[MB];
      load_batch(v, b, pm);
      merge_batch(M, S, b, pm);
    }
    return finish_ml(M, S, v);
  };
  float2 pm0[MB];   // the first tile's first batch (or its merged pair)
  if constexpr (PASS == 2) {   // unconditional too, from the clamped vector
    if constexpr (OWN) load_batch(v0, rb0 + hh, pm0);
    else pm0[0] = ml_final[((int64_t)req * Hkv + kvh) * Mpad + v0];
  }

  if constexpr (PASS == 1 && OWN) {
    // the query rows' angles (L_ctx + i - delta) theta_j: thread t takes frequency j = t % H and
    // rows t / H, t / H + 256 / H, ...: one float64 sin/cos for its first row and one for the row
    // step, then the rows by complex multiplication in float64, rounded to float32. The first row
    // is stored by every thread (row t / H < 256 / H is inside the table; one past L_q is never
    // read), so the frequency load, issued first, is used in straight-line code and the sin/cos
    // overlaps the data loads' latency.
    const int j = threadIdx.x % H;
    constexpr int RS = 256 / H;
    static_assert(RS <= kInRotMaxLq, "first rows inside the angle table");
    const double p0 = (double)Lctx + (double)(threadIdx.x / H) - (double)tab.delta[e];
    double c, sn, cs, ss;
    sincos(p0 * th_j, &sn, &c);
    sincos((double)RS * th_j, &ss, &cs);
    qcs[threadIdx.x] = make_float2((float)c, (float)sn);
    for (int i = threadIdx.x / H + RS; i < qr.Lq; i += RS) {
      const double cn = c * cs - sn * ss;
      sn = sn * cs + c * ss;
      c = cn;
      qcs[i * H + j] = make_float2((float)c, (float)sn);
    }
    // this block clears its keys' score accumulators (pass 2 adds into them)
    if (kvh == 0 && (int)threadIdx.x < nk) fx[(int64_t)req * Lctx + tab.dst[e] + t0 + threadIdx.x] = 0ull;
  }
#pragma unroll
  for (int i = 0; i < NKL; ++i) {
    const int u = threadIdx.x + 256 * i;
    // masked rather than selected: a select lets the compiler move the row's load behind a branch
    const uint32_t m = u / (D / 8) < nk ? ~0u : 0u;
    *reinterpret_cast<u32x4*>(Ks + (u / (D / 8)) * KST + 8 * (u % (D / 8))) = kr[i] & m;
  }
  float2 mlv = make_float2(0.f, 0.f);
  if constexpr (PASS == 2) {
    // the first tile, from the batch loaded above: every wave merges it in straight-line code
    // beside the loads (a use behind a branch lets the compiler sink the loads after the waits)
    if constexpr (OWN) {
      float M = -INFINITY, S = 0.f;
      int b = rb0 + hh;
      merge_batch(M, S, b, pm0);
      for (b += 2 * MB; b < rb1; b += 2 * MB) {
        float2 pm[MB];
        load_batch(v0, b, pm);
        merge_batch(M, S, b, pm);
      }
      mlv = finish_ml(M, S, 32 * wave + l32);
    } else {
      mlv = pm0[0];
    }
    if (wave < nqt) mlw[wave][l32] = mlv;   // before the barrier: the merge is done before the MFMAs
  }
  __syncthreads();
  if constexpr (PASS == 1 && OWN) {
    // rotate (pairs d, d + H sit in K-steps ks and ks + NKS/2 of the same lane), fold in
    // log2(e)/sqrt(d) and split into bf16 hi/lo, as the query preparation kernel does; the first
    // key block of each (entry, KV head) also writes the operand for pass 2
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks) {
      u32x4 ha, hb, la, lb;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float r[2][2];   // [a or b output][element of the pair]
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float a = bf2f((qraw[ks][k] >> (16 * t)) & 0xffffu);
          const float b = bf2f((qraw[ks + NKS / 2][k] >> (16 * t)) & 0xffffu);
          const float2 cw = qcs[qrow * H + 16 * ks + 8 * hh + 2 * k + t];
          r[0][t] = (a * cw.x - b * cw.y) * qr.scale_log2;
          r[1][t] = (a * cw.y + b * cw.x) * qr.scale_log2;
        }
        // hi = bf16(r), lo = bf16(r - hi), both rounded to nearest even, one pair per conversion
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          hw[o] = pack_bf2(r[o][0], r[o][1]);
          lw[o] = pack_bf2(r[o][0] - bf2f(hw[o] & 0xffffu), r[o][1] - __uint_as_float(hw[o] & 0xffff0000u));
        }
        ha[k] = qok ? hw[0] : 0u;
        hb[k] = qok ? hw[1] : 0u;
        la[k] = qok ? lw[0] : 0u;
        lb[k] = qok ? lw[1] : 0u;
      }
      qh[ks] = as_bf16x8(ha);
      qh[ks + NKS / 2] = as_bf16x8(hb);
      ql[ks] = as_bf16x8(la);
      ql[ks + NKS / 2] = as_bf16x8(lb);
    }
    if (x == 0 && wave < nqt) {
      uint16_t* qo = qb + (int64_t)(32 * wave + l32) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        *reinterpret_cast<u32x4*>(qo + 16 * ks) = __builtin_bit_cast(u32x4, qh[ks]);
        *reinterpret_cast<u32x4*>(qo + plane + 16 * ks) = __builtin_bit_cast(u32x4, ql[ks]);
      }
    }
  }
  if constexpr (PASS == 1) {
    if (anc.k > 0 && (int)threadIdx.x < nk) {   // this KV head's share of the key norms
      const uint32_t* row = reinterpret_cast<const uint32_t*>(Ks + threadIdx.x * KST);
      double acc = 0.0;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) acc = sumsq16<uint16_t>(acc, row + 4 * c);
      anc.ssp[kvh * anc.stride + (int64_t)req * Lctx + tab.dst[e] + t0 + threadIdx.x] = acc;
    }
  }

  float col[4] = {0.f, 0.f, 0.f, 0.f};   // pass 2: keys 32 st + l32
  for (int qt = wave; qt < nqt; qt += 4) {
    if (qt != wave) {
      load_q<NKS>(qb + (int64_t)(32 * qt + l32) * D, plane, qh, ql);
      if constexpr (PASS == 2) mlv = merged_ml(qt);
    }
    f32x16 acc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) acc[st] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 kb =
            as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + (32 * st + l32) * KST + 16 * ks + 8 * hh));
        if constexpr (PASS == 1) {
          acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qh[ks], acc[st], 0, 0, 0);
          acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, ql[ks], acc[st], 0, 0, 0);
        } else {
          acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[ks], kb, acc[st], 0, 0, 0);
          acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql[ks], kb, acc[st], 0, 0, 0);
        }
      }
    }
    if constexpr (PASS == 1) {
      // acc[st][r] = exp2 exponent of key 32 st + 8 (r/4) + 4 hh + r%4 for query vector 32 qt + l32
      if (nk < KB) {   // partial block: drop the keys past the chunk's end
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * st + 8 * (r >> 2) + 4 * hh + (r & 3) >= nk) acc[st][r] = -INFINITY;
      }
      float m = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[st][r]);
      m = half_max(m);
      const float m_use = (m == -INFINITY) ? 0.f : m;
      float sum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += fast_exp2(acc[st][r] - m_use);
      sum = half_sum(sum);
      if (hh == 0)
        ml_part[((int64_t)(blk_base + blk) * Hkv + kvh) * Mpad + 32 * qt + l32] = make_float2(m, sum);
    } else {
      // acc[st][r] = logit of query vector 32 qt + 8 (r/4) + 4 hh + r%4 against key 32 st + l32;
      // that vector's (max, 1/sum) sits in lane 8 (r/4) + 4 hh + r%4 of this wave
      // (a wave's LDS accesses complete in program order, so no barrier is needed here)
      mlw[wave][l32] = mlv;   // both halves hold the same value
      float2 mr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) mr[r] = mlw[wave][8 * (r >> 2) + 4 * hh + (r & 3)];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float c = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) c += fast_exp2(acc[st][r] - mr[r].x) * mr[r].y;
        col[st] += c;
      }
    }
  }
  if constexpr (PASS == 2) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float c = half_sum(col[st]);
      if (hh == 0) colred[wave][32 * st + l32] = c;
    }
    __syncthreads();
    if (threadIdx.x < nk) {
      const int j = threadIdx.x;
      const float c = ((colred[0][j] + colred[1][j]) + colred[2][j]) + colred[3][j];
      // this KV head's share of the score, added in fixed point (c >= 0). System scope: the add is
      // performed past the per-XCD L2s, where the blocks of every KV head meet.
      __hip_atomic_fetch_add(fx + (int64_t)req * Lctx + tab.dst[e] + t0 + j,
                             (unsigned long long)__double2ll_rn((double)c * kScoreFixScale),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

}  // namespace

hipError_t launch_score_prep(int D, const ChunkTab& tab, int Lq, int Hq, int Hkv, int Mpad,
                             int Lctx, const void* qc, uint16_t* qrot, int64_t plane,
                             int entry_base, float scale_log2, unsigned long long* fx, double base,
                             hipStream_t st) {
  if (tab.n == 0 || Lq == 0) return hipSuccess;
  dim3 g(Lq, tab.n), b(256);
  const Theta th = make_theta(D, base);
  if (D == 128)
    k_score_prep<128><<<g, b, 0, st>>>(tab, Lq, Hq, Hkv, Mpad, Lctx, (const uint16_t*)qc, qrot,
                                        plane, entry_base, scale_log2, fx, th);
  else
    k_score_prep<64><<<g, b, 0, st>>>(tab, Lq, Hq, Hkv, Mpad, Lctx, (const uint16_t*)qc, qrot,
                                       plane, entry_base, scale_log2, fx, th);
  return hipGetLastError();
}

hipError_t launch_score_pass(int pass, int D, const ChunkTab& tab, const int* req_blk0, int n_req,
                             int Hkv, int Mpad, int Mvalid, int Lctx, const void* kc,
                             uint16_t* qrot, int64_t plane, int entry_base, int blk_base,
                             float2* ml_part, const float2* ml_final, int fuse_merge,
                             unsigned long long* fx, const AnchorOut& anc, const RerotFused& rf,
                             const QueryRot& qr, double base, hipStream_t st) {
  if (tab.n == 0 || tab.blk0[tab.n] == 0) return hipSuccess;
  (void)n_req;
  EntryReqBlocks erb;
  int bmax = 0;
  for (int i = 0; i < tab.n; ++i) {
    erb.lo[i] = req_blk0[tab.req[i]];
    erb.hi[i] = req_blk0[tab.req[i] + 1];
    bmax = std::max(bmax, tab.blk0[i + 1] - tab.blk0[i]);
  }
  // pass 1 may carry S1 (per entry and KV head, one extra block per kS1Fold key blocks), pass 2
  // the anchors (one extra block per entry)
  const int extra = pass == 1 ? (rf.kf ? (bmax + kS1Fold - 1) / kS1Fold : 0) : (anc.k > 0 ? 1 : 0);
  dim3 g(bmax + extra, Hkv, tab.n), b(256);
  const uint16_t* k = (const uint16_t*)kc;
  const Theta th = make_theta(D, base);
#define SRA_PASS(DD, PP, FF)                                                                        \
  k_score_pass<DD, PP, FF><<<g, b, 0, st>>>(tab, erb, bmax, Hkv, Mpad, Mvalid, Lctx, k, qrot, plane, \
                                              entry_base, blk_base, ml_part, ml_final, fx, anc, rf,  \
                                              pass == 1 ? qr : QueryRot{}, th)
  // pass 1 forms its own operand when qr.on, pass 2 merges its own partials when fuse_merge
  const bool own = pass == 1 ? qr.on != 0 : fuse_merge != 0;
  if (D == 128 && pass == 1 && own) SRA_PASS(128, 1, true);
  else if (D == 128 && pass == 1) SRA_PASS(128, 1, false);
  else if (D == 128 && own) SRA_PASS(128, 2, true);
  else if (D == 128) SRA_PASS(128, 2, false);
  else if (pass == 1 && own) SRA_PASS(64, 1, true);
  else if (pass == 1) SRA_PASS(64, 1, false);
  else if (own) SRA_PASS(64, 2, true);
  else SRA_PASS(64, 2, false);
#undef SRA_PASS
  return hipGetLastError();
}

hipError_t launch_score_merge(const int* req_blk0, int n_req, int Hkv, int Mpad, int Mvalid,
                              const float2* ml_part, float2* ml_final, hipStream_t st) {
  ReqBlocks rb;
  for (int r = 0; r <= n_req; ++r) rb.blk0[r] = req_blk0[r];
  dim3 g(n_req * Hkv, (Mpad + 63) / 64), b(256);
  k_score_merge<<<g, b, 0, st>>>(rb, Hkv, Mpad, Mvalid, ml_part, ml_final);
  return hipGetLastError();
}

}  // namespace sra
