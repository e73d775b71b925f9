// Streaming rotary kernels: S1 re-rotation of cached chunk keys into the fused cache (its body is
// shared with the scoring pass that can carry it), S3 scatter of fresh K/V rows together with the
// sparse attention's per-row inputs (angle table or prepared query operand), and the row check.
//
// S3 follows the per-layer selective recompute flow (KVCache reuse 01, §1.3.4): fresh K/V of the
// selected tokens replace the reused rows, K rotated at the token's absolute position.
//
// Both are pure HBM streams: every thread moves 16-byte vectors, rows are contiguous, angles are
// formed once per block in float64 and kept in LDS as float32 cos/sin.
#include <algorithm>

#include "common.h"
#include "rerotate.h"

namespace sra {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

using rerot::Vec;

// One block per (chunk entry, block of rows_per_blk rows of that chunk), all KV heads.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_rerotate(ChunkTab tab, int Hkv, int rows_per_blk,
                                                  const T* __restrict__ ks,
                                                  const T* __restrict__ vs, T* __restrict__ kf,
                                                  T* __restrict__ vf, int64_t L, Theta th, F16Shadow sh) {
  __shared__ float2 cs[D / 2];
  const int e = find_entry(tab, blockIdx.x);
  const int t0 = (blockIdx.x - tab.blk0[e]) * rows_per_blk;
  rerot::rows<T, D>(tab, e, t0, min(rows_per_blk, tab.len[e] - t0), Hkv, ks, vs, kf, vf, L, th, cs, sh);
}

// fp16 copy of fused bf16 keys for the attention (the standalone attention entry, whose keys come from
// the caller): n16 16-byte vectors of [n_req][L][Hkv][D], grid-stride; a key beyond fp16's range flags
// its (request, KV head).
template <int D>
__global__ __launch_bounds__(256) void k_to_f16(int64_t n16, int Hkv, int64_t L, const uint16_t* __restrict__ kf,
                                                F16Shadow sh) {
  constexpr int VPH = D / 8;   // 16-byte vectors per head row
  const u32x4* src = reinterpret_cast<const u32x4*>(kf);
  u32x4* dst = reinterpret_cast<u32x4*>(sh.kh);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const u32x4 w = src[i];
    float amax = 0.f;
    u32x4 h;
#pragma unroll
    for (int k = 0; k < 4; ++k) h[k] = bf2_to_h2(w[k], amax);
    dst[i] = h;
    if (amax > kF16Max) {
      const int64_t head_row = i / VPH;   // (req, position, KV head)
      sh.flags[(head_row / (L * Hkv)) * Hkv + head_row % Hkv] = sh.call_id;
    }
  }
}

// One block per (recomputed row r, request) at position p = row_pos[r]: forms the row's angles
// once, then (each part optional) writes them out, scatters the fresh K/V row to fused row p with
// K rotated at p (and, with sh.kh, the stored key's fp16 copy for the attention, flagging a key
// beyond fp16's range), and writes the attention's query operand: every query head rotated at p, scaled
// by log2(e)/sqrt(d) and either split into bf16 hi/lo planes (Q16 false: the statistics' exact
// products) or rounded once to fp16 in plane 0 (Q16 true: the attention's operand), in the
// matrix-operand order of qop_index (a scaled query beyond fp16's range flags its group).
// Fresh rows are compact (row r) or position-indexed (row p). Rows outside [0, L) write nothing
// but zero query operands. The first batch of every part is loaded before the angles are formed.
// FULL: kn and qop are both set (bf16), so every first-batch load is unconditional and the
// angles wait on the frequency load alone.
template <typename T, int D, bool FULL, bool Q16>
__global__ __launch_bounds__(128) void k_scatter(int Hq, int Hkv, int R, int L,
                                                 const T* __restrict__ qn, const T* __restrict__ kn,
                                                 const T* __restrict__ vn, int fresh_rows,
                                                 int indexed, const int* __restrict__ row_pos,
                                                 T* __restrict__ kf, T* __restrict__ vf,
                                                 float2* __restrict__ cs_out, uint16_t* __restrict__ qop,
                                                 int qop_blocks, float scale_log2, Theta th, F16Shadow sh) {
  constexpr int H = D / 2;
  constexpr int NKS = D / 16;
  constexpr int VW = Vec<T>::N;
  constexpr int UPH = H / VW;
  constexpr int NT = 128;
  // the attention that follows takes work from per-group queues: they start empty (system-scope
  // stores: the queues are taken with system-scope atomics, past the XCDs' caches)
  if (sh.queue && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < sh.n_queue; i += NT) __hip_atomic_store(sh.queue + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __shared__ float2 cs[H];
  const int r = blockIdx.x, q = blockIdx.y;
  const int p = row_pos ? row_pos[(int64_t)q * R + r] : r;   // no table: row r sits at position r
  const bool valid = p >= 0 && p < L;  // rows outside the cache are never written
  const int srow = valid ? (indexed ? p : r) : 0;
  const int64_t row_elems = (int64_t)Hkv * D;
  const int64_t src0 = ((int64_t)q * fresh_rows + srow) * row_elems;
  const int64_t dst0 = ((int64_t)q * L + (valid ? p : 0)) * row_elems;
  const int nV = (int)(row_elems * (int64_t)sizeof(T) / 16), nK = Hkv * UPH;
  const bool do_kv = valid && (FULL || kn);
  // the thread's frequency (an indexed load) goes out before the row's data: loads complete in
  // order, so one issued after them would hold the angles back until all the data has arrived
  static_assert(H <= NT, "one frequency per thread");
  const double th_i = th.v[min((int)threadIdx.x, H - 1)];
  __builtin_amdgcn_sched_barrier(0);
  // first batch: V chunks tid, tid+128; K pair tid; query units tid, tid+128
  u32x4 v0 = {}, v1 = {}, ka = {}, kb = {};
  if (FULL || kn) {
    const u32x4* vsrc = reinterpret_cast<const u32x4*>(vn + src0);
    v0 = vsrc[min((int)threadIdx.x, nV - 1)];
    v1 = vsrc[min((int)threadIdx.x + NT, nV - 1)];
    const int u = min((int)threadIdx.x, nK - 1);
    const T* ap = kn + src0 + (u / UPH) * D + (u % UPH) * VW;
    ka = *reinterpret_cast<const u32x4*>(ap);
    kb = *reinterpret_cast<const u32x4*>(ap + H);
  }
  const int g = Hq / Hkv;
  const int nQ = Hq * NKS;   // unit = (head, 16-dim step ks < NKS/2, half hh)
  auto qsrc = [&](int u) { return qn + (((int64_t)q * fresh_rows + srow) * Hq + u / NKS) * D + 16 * ((u % NKS) >> 1) + 8 * (u & 1); };
  u32x4 qx[2] = {}, qy[2] = {};
  if constexpr (sizeof(T) == 2) {
    if (FULL || qop) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const T* src = qsrc(min((int)threadIdx.x + NT * k, nQ - 1));
        qx[k] = *reinterpret_cast<const u32x4*>(src);
        qy[k] = *reinterpret_cast<const u32x4*>(src + H);
      }
    }
  }
  {   // every thread forms an angle and stores it (threads past d/2 repeat the last frequency with
      // the same value; an invalid row's angles are never used), so the frequency load stays in
      // straight-line code and the float64 sin/cos overlaps the data loads
    const float2 c = rope_cs((double)(valid ? p : 0), th_i);
    cs[min((int)threadIdx.x, H - 1)] = c;
    if (valid && cs_out && (int)threadIdx.x < H) cs_out[((int64_t)q * R + r) * H + threadIdx.x] = c;
  }
  __syncthreads();

  auto rot_store = [&](int u, u32x4 a, u32x4 b) {   // K pair unit u of the row
    const int i0 = (u % UPH) * VW;
    T* o = kf + dst0 + (u / UPH) * D + i0;
    float fa[VW], fb[VW], ra[VW], rb[VW];
    Vec<T>::unpack(a, fa);
    Vec<T>::unpack(b, fb);
#pragma unroll
    for (int k = 0; k < VW; ++k) {
      const float c = cs[i0 + k].x, sn = cs[i0 + k].y;
      ra[k] = fa[k] * c - fb[k] * sn;
      rb[k] = fa[k] * sn + fb[k] * c;
    }
    const u32x4 wa = Vec<T>::pack(ra), wb = Vec<T>::pack(rb);
    *reinterpret_cast<u32x4*>(o) = wa;
    *reinterpret_cast<u32x4*>(o + H) = wb;
    if constexpr (sizeof(T) == 2) {
      if (sh.kh) {   // the attention's fp16 copy of the stored key
        float amax = 0.f;
        u32x4 ha, hb;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ha[k] = bf2_to_h2(wa[k], amax);
          hb[k] = bf2_to_h2(wb[k], amax);
        }
        uint16_t* oh = sh.kh + (o - kf);
        *reinterpret_cast<u32x4*>(oh) = ha;
        *reinterpret_cast<u32x4*>(oh + H) = hb;
        if (amax > kF16Max) sh.flags[(int64_t)q * Hkv + u / UPH] = sh.call_id;
      }
    }
  };
  if (do_kv) {
    u32x4* vdst = reinterpret_cast<u32x4*>(vf + dst0);
    const u32x4* vsrc = reinterpret_cast<const u32x4*>(vn + src0);
    if ((int)threadIdx.x < nV) vdst[threadIdx.x] = v0;
    if ((int)threadIdx.x + NT < nV) vdst[threadIdx.x + NT] = v1;
    for (int u = threadIdx.x + 2 * NT; u < nV; u += NT) vdst[u] = vsrc[u];
    if ((int)threadIdx.x < nK) rot_store(threadIdx.x, ka, kb);
    for (int u = threadIdx.x + NT; u < nK; u += NT) {
      const T* ap = kn + src0 + (u / UPH) * D + (u % UPH) * VW;
      rot_store(u, *reinterpret_cast<const u32x4*>(ap), *reinterpret_cast<const u32x4*>(ap + H));
    }
  }
  if constexpr (sizeof(T) == 2) {
    if (FULL || qop) {
      auto q_store = [&](int u, u32x4 wx, u32x4 wy) {
        const int h = u / NKS, ks = (u % NKS) >> 1, hh = u & 1;
        const int d0 = 16 * ks + 8 * hh;
        float x[8], y[8];
        if (valid) {
          Vec<T>::unpack(wx, x);
          Vec<T>::unpack(wy, y);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float2 c = cs[d0 + k];
            const float a = x[k] * c.x - y[k] * c.y, b = x[k] * c.y + y[k] * c.x;
            x[k] = a * scale_log2;
            y[k] = b * scale_log2;
          }
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = y[k] = 0.f;
        }
        const int v = r * g + h % g;
        const int64_t grp = (int64_t)q * Hkv + h / g;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const float* f = half ? y : x;
          const int kss = ks + half * (NKS / 2);
          if constexpr (Q16) {
            u32x4 wq;
            float amax = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              amax = fmaxf(amax, fmaxf(fabsf(f[2 * k]), fabsf(f[2 * k + 1])));
              wq[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[2 * k]) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[2 * k + 1]) << 16);
            }
            *reinterpret_cast<u32x4*>(qop + qop_index(grp, v >> 5, kss, 0, v & 31, hh, qop_blocks, NKS)) = wq;
            // a scaled query at or beyond 65520 has no fp16 value (65504 < x < 65520 rounds to 65504)
            if (sh.flags && amax >= 65520.f) sh.flags[grp] = sh.call_id;
          } else {
            u32x4 wh, wl;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              wh[k] = pack_bf2(f[2 * k], f[2 * k + 1]);
              wl[k] = pack_bf2(f[2 * k] - bf2f(wh[k] & 0xffffu), f[2 * k + 1] - bf2f(wh[k] >> 16));
            }
            *reinterpret_cast<u32x4*>(qop + qop_index(grp, v >> 5, kss, 0, v & 31, hh, qop_blocks, NKS)) = wh;
            *reinterpret_cast<u32x4*>(qop + qop_index(grp, v >> 5, kss, 1, v & 31, hh, qop_blocks, NKS)) = wl;
          }
        }
      };
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if ((int)threadIdx.x + NT * k < nQ) q_store(threadIdx.x + NT * k, qx[k], qy[k]);
      for (int u = threadIdx.x + 2 * NT; u < nQ; u += NT) {
        const T* src = qsrc(u);
        q_store(u, *reinterpret_cast<const u32x4*>(src), *reinterpret_cast<const u32x4*>(src + H));
      }
    }
  }
}

// Anchor probe prefix (QCFuse summary (zh) §2.A: the chunks' anchors enter the query's forward
// pass as a lightweight prefix). One block per prefix row a = c * k + j of a request: the j-th
// smallest of chunk c's k anchor offsets t (offsets ranked in LDS, ties by index) is cached at
// position orig_c + t and moves to row a, so its key turns by a - orig_c - t (bits kept when that
// is 0); V is copied. Offsets are clamped into the chunk (distinct in-range offsets are the
// caller's contract). tab entries: (req, src, len, dst = first prefix row, delta = orig, aux = c).
template <typename T, int D>
__global__ __launch_bounds__(128) void k_anchor_prefix(ChunkTab tab, int k, int n_chunks, const int* __restrict__ anchors,
                                                       int Hkv, const T* __restrict__ ks, const T* __restrict__ vs,
                                                       T* __restrict__ kp, T* __restrict__ vp, int Lp, Theta th) {
  constexpr int H = D / 2;
  constexpr int VW = Vec<T>::N;
  constexpr int UPH = H / VW;
  constexpr int NT = 128;
  __shared__ float2 cs[H];
  __shared__ int sh_t;
  const int e = find_entry(tab, blockIdx.x);
  const int j = blockIdx.x - tab.blk0[e];
  const int q = tab.req[e], len = tab.len[e];
  const int* arow = anchors + ((int64_t)q * n_chunks + tab.aux[e]) * k;
  if ((int)threadIdx.x < k) {
    const int ti = min(max(arow[threadIdx.x], 0), len - 1);
    int rank = 0;
    for (int i = 0; i < k; ++i) {
      const int tv = min(max(arow[i], 0), len - 1);
      rank += (tv < ti || (tv == ti && i < (int)threadIdx.x)) ? 1 : 0;
    }
    if (rank == j) sh_t = ti;
  }
  __syncthreads();
  const int t = sh_t;
  const int a = tab.dst[e] + j;
  const int delta = a - tab.delta[e] - t;
  if (delta != 0)
    for (int i = threadIdx.x; i < H; i += NT) cs[i] = rope_cs((double)delta, th.v[i]);
  __syncthreads();
  const int64_t row_elems = (int64_t)Hkv * D;
  const int64_t src0 = ((int64_t)tab.src[e] + t) * row_elems;
  const int64_t dst0 = ((int64_t)q * Lp + a) * row_elems;
  const int nV = (int)(row_elems * (int64_t)sizeof(T) / 16), nK = Hkv * UPH;
  const u32x4* vsrc = reinterpret_cast<const u32x4*>(vs + src0);
  u32x4* vdst = reinterpret_cast<u32x4*>(vp + dst0);
  for (int u = threadIdx.x; u < nV; u += NT) vdst[u] = vsrc[u];
  for (int u = threadIdx.x; u < nK; u += NT) {
    const int i0 = (u % UPH) * VW;
    const int64_t o = (u / UPH) * D + i0;
    const u32x4 ka = *reinterpret_cast<const u32x4*>(ks + src0 + o);
    const u32x4 kb = *reinterpret_cast<const u32x4*>(ks + src0 + o + H);
    if (delta == 0) {
      *reinterpret_cast<u32x4*>(kp + dst0 + o) = ka;
      *reinterpret_cast<u32x4*>(kp + dst0 + o + H) = kb;
    } else {
      float fa[VW], fb[VW], ra[VW], rb[VW];
      Vec<T>::unpack(ka, fa);
      Vec<T>::unpack(kb, fb);
#pragma unroll
      for (int m = 0; m < VW; ++m) {
        const float c = cs[i0 + m].x, sn = cs[i0 + m].y;
        ra[m] = fa[m] * c - fb[m] * sn;
        rb[m] = fa[m] * sn + fb[m] * c;
      }
      *reinterpret_cast<u32x4*>(kp + dst0 + o) = Vec<T>::pack(ra);
      *reinterpret_cast<u32x4*>(kp + dst0 + o + H) = Vec<T>::pack(rb);
    }
  }
}

// KV deviation of recomputed rows (KVCache reuse 01, §1.3.2-§1.3.3: tokens are ranked by the
// difference between their reused and their recomputed KV). One block per (row r < n_dev,
// request), at p = row_pos[r]: the Euclidean norm over every KV head and dimension of the fresh K
// rotated at p and rounded as the scatter stores it, minus the reused K at p, together with the
// fresh V minus the reused V. Differences and squares are float64; the block total is rounded to
// float32 once. Fresh rows are compact (row r) or position-indexed (row p). Rows must lie in
// [0, L) (the row check's contract); others are measured at row 0.
template <typename T, int D>
__global__ __launch_bounds__(128) void k_kv_deviation(int Hkv, int R, int L, const T* __restrict__ kn,
                                                      const T* __restrict__ vn, int fresh_rows,
                                                      int indexed, const int* __restrict__ row_pos,
                                                      const T* __restrict__ kf, const T* __restrict__ vf,
                                                      float* __restrict__ dev, int n_dev, Theta th) {
  constexpr int H = D / 2;
  constexpr int VW = Vec<T>::N;
  constexpr int UPH = H / VW;
  constexpr int NT = 128;
  __shared__ float2 cs[H];
  __shared__ double wtot[NT / 64];
  const int r = blockIdx.x, q = blockIdx.y;
  const int p0 = row_pos[(int64_t)q * R + r];
  const int p = (p0 >= 0 && p0 < L) ? p0 : 0;
  const int64_t row_elems = (int64_t)Hkv * D;
  const int64_t src0 = ((int64_t)q * fresh_rows + (indexed ? p : r)) * row_elems;
  const int64_t old0 = ((int64_t)q * L + p) * row_elems;
  const int nV = (int)(row_elems * (int64_t)sizeof(T) / 16), nK = Hkv * UPH;
  // first batch (V chunk tid, K pair tid, fresh and reused) before the angles are formed
  const u32x4* vsrc = reinterpret_cast<const u32x4*>(vn + src0);
  const u32x4* vold = reinterpret_cast<const u32x4*>(vf + old0);
  const int u0 = min((int)threadIdx.x, nK - 1);
  const int64_t k0 = (u0 / UPH) * D + (u0 % UPH) * VW;
  u32x4 va = vsrc[min((int)threadIdx.x, nV - 1)], vb = vold[min((int)threadIdx.x, nV - 1)];
  u32x4 ka = *reinterpret_cast<const u32x4*>(kn + src0 + k0), kb = *reinterpret_cast<const u32x4*>(kn + src0 + k0 + H);
  u32x4 oa = *reinterpret_cast<const u32x4*>(kf + old0 + k0), ob = *reinterpret_cast<const u32x4*>(kf + old0 + k0 + H);
  for (int i = threadIdx.x; i < H; i += NT) cs[i] = rope_cs((double)p, th.v[i]);
  __syncthreads();

  double acc = 0.0;
  auto vdiff = [&](u32x4 a, u32x4 b) {
    float fa[VW], fb[VW];
    Vec<T>::unpack(a, fa);
    Vec<T>::unpack(b, fb);
#pragma unroll
    for (int k = 0; k < VW; ++k) {
      const double d = (double)fa[k] - (double)fb[k];
      acc += d * d;
    }
  };
  // the fresh pair rotated at p exactly as the scatter computes and rounds it
  auto kdiff = [&](int u, u32x4 a, u32x4 b, u32x4 oa_, u32x4 ob_) {
    const int i0 = (u % UPH) * VW;
    float fa[VW], fb[VW], ra[VW], rb[VW];
    Vec<T>::unpack(a, fa);
    Vec<T>::unpack(b, fb);
#pragma unroll
    for (int k = 0; k < VW; ++k) {
      const float c = cs[i0 + k].x, sn = cs[i0 + k].y;
      ra[k] = fa[k] * c - fb[k] * sn;
      rb[k] = fa[k] * sn + fb[k] * c;
    }
    vdiff(Vec<T>::pack(ra), oa_);
    vdiff(Vec<T>::pack(rb), ob_);
  };
  if ((int)threadIdx.x < nV) vdiff(va, vb);
  for (int u = threadIdx.x + NT; u < nV; u += NT) vdiff(vsrc[u], vold[u]);
  if ((int)threadIdx.x < nK) kdiff(threadIdx.x, ka, kb, oa, ob);
  for (int u = threadIdx.x + NT; u < nK; u += NT) {
    const int64_t o = (u / UPH) * D + (u % UPH) * VW;
    kdiff(u, *reinterpret_cast<const u32x4*>(kn + src0 + o), *reinterpret_cast<const u32x4*>(kn + src0 + o + H),
          *reinterpret_cast<const u32x4*>(kf + old0 + o), *reinterpret_cast<const u32x4*>(kf + old0 + o + H));
  }
  // block total in a fixed order: lane tree within each wave, then the waves in order
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if ((threadIdx.x & 63) == 0) wtot[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) t += wtot[w];
    dev[(int64_t)q * n_dev + r] = (float)sqrt(t);
  }
}

template <int D>
__global__ void k_rope_table(int R, const int* __restrict__ row_pos, float2* __restrict__ cs_out,
                             Theta th) {
  constexpr int H = D / 2;
  const int r = blockIdx.x, q = blockIdx.y;
  const int p = row_pos[(int64_t)q * R + r];
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    cs_out[((int64_t)q * R + r) * H + i] = rope_cs((double)p, th.v[i]);
}

__global__ void k_check_rows(const int* __restrict__ row_pos, int n_req, int R, int L,
                             int* __restrict__ bad) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_req * R) return;
  const int r = (int)(idx % R);
  const int v = row_pos[idx];
  bool ok = v >= 0 && v < L;
  if (r > 0) ok = ok && row_pos[idx - 1] < v;
  if (!ok) atomicMin(bad, (int)idx);
}

}  // namespace

hipError_t launch_rerotate(int dtype, int D, int Hkv, const ChunkTab& tab, int rows_per_blk,
                           const void* ks, const void* vs, void* kf, void* vf, int64_t L,
                           double base, hipStream_t st, const F16Shadow& sh) {
  const int nblk = tab.blk0[tab.n];
  if (nblk == 0) return hipSuccess;
  dim3 g(nblk), b(256);
  const Theta th = make_theta(D, base);
  if (dtype == 0 && D == 128)
    k_rerotate<uint16_t, 128><<<g, b, 0, st>>>(tab, Hkv, rows_per_blk, (const uint16_t*)ks,
                                                (const uint16_t*)vs, (uint16_t*)kf, (uint16_t*)vf, L, th, sh);
  else if (dtype == 0 && D == 64)
    k_rerotate<uint16_t, 64><<<g, b, 0, st>>>(tab, Hkv, rows_per_blk, (const uint16_t*)ks,
                                               (const uint16_t*)vs, (uint16_t*)kf, (uint16_t*)vf, L, th, sh);
  else if (dtype == 1 && D == 128)
    k_rerotate<float, 128><<<g, b, 0, st>>>(tab, Hkv, rows_per_blk, (const float*)ks,
                                             (const float*)vs, (float*)kf, (float*)vf, L, th, F16Shadow());
  else
    k_rerotate<float, 64><<<g, b, 0, st>>>(tab, Hkv, rows_per_blk, (const float*)ks,
                                            (const float*)vs, (float*)kf, (float*)vf, L, th, F16Shadow());
  return hipGetLastError();
}

hipError_t launch_k_to_f16(int D, int Hkv, int n_req, int L, const uint16_t* kf, const F16Shadow& sh,
                           hipStream_t st) {
  const int64_t n16 = (int64_t)n_req * L * Hkv * D / 8;
  if (n16 == 0) return hipSuccess;
  const unsigned nblk = (unsigned)std::min<int64_t>((n16 + 255) / 256, 4096);
  if (D == 128) k_to_f16<128><<<dim3(nblk), dim3(256), 0, st>>>(n16, Hkv, L, kf, sh);
  else k_to_f16<64><<<dim3(nblk), dim3(256), 0, st>>>(n16, Hkv, L, kf, sh);
  return hipGetLastError();
}

hipError_t launch_scatter(int dtype, int D, int Hq, int Hkv, int n_req, int R, int L,
                          const void* qn, const void* kn, const void* vn, int fresh_rows,
                          int indexed, const int* row_pos, void* kf, void* vf, float2* cs_out,
                          uint16_t* qop, int qop_blocks, bool q16, float scale_log2, double base,
                          hipStream_t st, const F16Shadow& sh) {
  if (R == 0 || n_req == 0) return hipSuccess;
  dim3 g(R, n_req), b(128);
  const Theta th = make_theta(D, base);
#define SRA_SCATTER(TT, DD, FF, QQ)                                                                     \
  k_scatter<TT, DD, FF, QQ><<<g, b, 0, st>>>(Hq, Hkv, R, L, (const TT*)qn, (const TT*)kn, (const TT*)vn,       \
                                         fresh_rows, indexed, row_pos, (TT*)kf, (TT*)vf, cs_out,         \
                                         dtype == 0 ? qop : nullptr, qop_blocks, scale_log2, th,       \
                                         dtype == 0 ? sh : F16Shadow())
  const bool full = dtype == 0 && kn && qop;
  if (dtype == 0 && D == 128 && full && q16) SRA_SCATTER(uint16_t, 128, true, true);   // fused layer
  else if (dtype == 0 && D == 128 && full) SRA_SCATTER(uint16_t, 128, true, false);
  else if (dtype == 0 && D == 128 && q16) SRA_SCATTER(uint16_t, 128, false, true);
  else if (dtype == 0 && D == 128) SRA_SCATTER(uint16_t, 128, false, false);
  else if (dtype == 0 && D == 64 && full && q16) SRA_SCATTER(uint16_t, 64, true, true);
  else if (dtype == 0 && D == 64 && full) SRA_SCATTER(uint16_t, 64, true, false);
  else if (dtype == 0 && D == 64 && q16) SRA_SCATTER(uint16_t, 64, false, true);
  else if (dtype == 0 && D == 64) SRA_SCATTER(uint16_t, 64, false, false);
  else if (dtype == 1 && D == 128) SRA_SCATTER(float, 128, false, false);
  else SRA_SCATTER(float, 64, false, false);
#undef SRA_SCATTER
  return hipGetLastError();
}

hipError_t launch_anchor_prefix(int dtype, int D, int Hkv, const ChunkTab& tab, int k, int n_chunks,
                                const int* anchors, const void* ks, const void* vs, void* kp, void* vp, int Lp,
                                double base, hipStream_t st) {
  if (tab.n == 0 || tab.blk0[tab.n] == 0) return hipSuccess;
  const dim3 g((unsigned)tab.blk0[tab.n]), b(128);
  const Theta th = make_theta(D, base);
  if (dtype == 0) {
    auto k_ = (const uint16_t*)ks;
    auto v_ = (const uint16_t*)vs;
    if (D == 128)
      k_anchor_prefix<uint16_t, 128><<<g, b, 0, st>>>(tab, k, n_chunks, anchors, Hkv, k_, v_, (uint16_t*)kp,
                                                      (uint16_t*)vp, Lp, th);
    else
      k_anchor_prefix<uint16_t, 64><<<g, b, 0, st>>>(tab, k, n_chunks, anchors, Hkv, k_, v_, (uint16_t*)kp,
                                                     (uint16_t*)vp, Lp, th);
  } else {
    auto k_ = (const float*)ks;
    auto v_ = (const float*)vs;
    if (D == 128)
      k_anchor_prefix<float, 128><<<g, b, 0, st>>>(tab, k, n_chunks, anchors, Hkv, k_, v_, (float*)kp,
                                                   (float*)vp, Lp, th);
    else
      k_anchor_prefix<float, 64><<<g, b, 0, st>>>(tab, k, n_chunks, anchors, Hkv, k_, v_, (float*)kp,
                                                  (float*)vp, Lp, th);
  }
  return hipGetLastError();
}

hipError_t launch_kv_deviation(int dtype, int D, int Hkv, int n_req, int R, int L, const void* kn,
                               const void* vn, int fresh_rows, int indexed, const int* row_pos,
                               const void* kf, const void* vf, float* dev, int n_dev, double base,
                               hipStream_t st) {
  if (n_dev == 0 || n_req == 0) return hipSuccess;
  const dim3 g((unsigned)n_dev, (unsigned)n_req), b(128);
  const Theta th = make_theta(D, base);
  if (dtype == 0) {
    auto k = (const uint16_t*)kn;
    auto v = (const uint16_t*)vn;
    if (D == 128)
      k_kv_deviation<uint16_t, 128><<<g, b, 0, st>>>(Hkv, R, L, k, v, fresh_rows, indexed, row_pos,
                                                     (const uint16_t*)kf, (const uint16_t*)vf, dev, n_dev, th);
    else
      k_kv_deviation<uint16_t, 64><<<g, b, 0, st>>>(Hkv, R, L, k, v, fresh_rows, indexed, row_pos,
                                                    (const uint16_t*)kf, (const uint16_t*)vf, dev, n_dev, th);
  } else {
    auto k = (const float*)kn;
    auto v = (const float*)vn;
    if (D == 128)
      k_kv_deviation<float, 128><<<g, b, 0, st>>>(Hkv, R, L, k, v, fresh_rows, indexed, row_pos,
                                                  (const float*)kf, (const float*)vf, dev, n_dev, th);
    else
      k_kv_deviation<float, 64><<<g, b, 0, st>>>(Hkv, R, L, k, v, fresh_rows, indexed, row_pos,
                                                 (const float*)kf, (const float*)vf, dev, n_dev, th);
  }
  return hipGetLastError();
}

hipError_t launch_rope_table(int D, int n_req, int R, const int* row_pos, float2* cs_out,
                             double base, hipStream_t st) {
  if (R == 0 || n_req == 0) return hipSuccess;
  dim3 g(R, n_req), b(64);
  const Theta th = make_theta(D, base);
  if (D == 128)
    k_rope_table<128><<<g, b, 0, st>>>(R, row_pos, cs_out, th);
  else
    k_rope_table<64><<<g, b, 0, st>>>(R, row_pos, cs_out, th);
  return hipGetLastError();
}

hipError_t launch_check_rows(const int* row_pos, int n_req, int R, int L, int* bad,
                             hipStream_t st) {
  const int64_t n = (int64_t)n_req * R;
  if (n == 0) return hipSuccess;
  k_check_rows<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(row_pos, n_req, R, L, bad);
  return hipGetLastError();
}

}  // namespace sra
