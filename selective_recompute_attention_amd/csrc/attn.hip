// Location-aware sparse causal attention (QCFuse technical summary (zh), §2.A: the recomputed
// tokens come as a discrete index table and attend under a strict causal constraint; KVCache
// reuse 01, §1.3.4: attention of the selected tokens against all tokens).
//
// For recomputed row r at absolute position p = row_pos[r] and query head h (KV head h/g):
//   q = R(p) q_new[r][h];  out = sum_{j <= p} softmax_j(q . k_j / sqrt(d)) v_j
//
// bf16 path, gfx950 matrix cores (v_mfma_f32_32x32x16_bf16):
//   * A work group owns 128 query vectors of one (request, KV head): the flattened (row, head in
//     group) pairs v = r*g + hh, so any group size g packs without padding. Rows are ascending, so
//     the tile's key range ends at the position of its last row; every vector masks its own tail.
//   * Four waves, 32 query vectors each. S^T = K Q^T puts one query vector per lane column, so the
//     online-softmax row reductions stay in-lane plus one cross-half shuffle, and the probabilities
//     feed O^T = V^T P^T directly from registers (keys permuted consistently on both operands).
//   * 64-key tiles of K (row-major, padded) and V (transposed on the way into LDS) are shared by
//     the four waves; float32 accumulation, exp2 with log2(e)/sqrt(d) folded into the logits.
//   * Small problems split the key range (flash-decoding style, at most kMaxSplits pieces); a wide
//     second kernel merges the splits of every query vector in split order. Blocks are ordered with the (request, KV head) index fastest, so every block
//     of one KV head lands on the same XCD (blocks are dealt round-robin over the 8 XCDs) and its
//     K/V stay in that XCD's L2; longest tiles are dispatched first.
// f32 path: plain float32 arithmetic, one block per (row, KV head), exact online softmax.
#include <float.h>

#include "common.h"

namespace sra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr int kMaxSplits = 16;   // key splits per tile (the host's split plan never exceeds it)

struct AttnArgs {
  const uint16_t* q;
  const int* row_pos;
  const float2* cs;
  const uint16_t* kf;
  const uint16_t* vf;
  uint16_t* out;
  float* lse;
  float* part_o;
  float2* part_ml;
  int n_req, Hq, Hkv, g, R, L, q_rows, indexed;
  int n_groups, n_tiles, n_splits, key_split;
  float scale_log2;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D, bool SPLIT>
__global__ __launch_bounds__(256, 2) void k_attn_mfma(AttnArgs a) {
  constexpr int NKS = D / 16;   // K-steps of S^T = K Q^T
  constexpr int NDT = D / 32;   // 32-row d tiles of O^T
  constexpr int H = D / 2;
  constexpr int KT = 64;        // keys per LDS tile
  constexpr int KST = D + 8;    // K row stride in LDS (elements): conflict-free 16-byte reads
  constexpr int VST = KT + 4;   // V^T row stride in LDS (elements): conflict-free 8-byte reads
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VST];

  const int wg = blockIdx.x;
  const int group = wg % a.n_groups;
  const int rest = wg / a.n_groups;
  const int split = rest % a.n_splits;
  const int tile = a.n_tiles - 1 - rest / a.n_splits;
  const int req = group / a.Hkv, kvh = group % a.Hkv;
  const int g = a.g;
  const int Mv = a.R * g;
  const int v0 = tile * 128;
  const int* rp = a.row_pos + (int64_t)req * a.R;
  const int maxkey = min(rp[min(v0 + 127, Mv - 1) / g], a.L - 1);  // keys never read past the cache
  const int kbeg = split * a.key_split;
  if (kbeg > maxkey) return;
  const int kend = min(kbeg + a.key_split, maxkey + 1);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int v = v0 + wave * 32 + l32;
  const bool qvalid = v < Mv && rp[min(v, Mv - 1) / g] >= 0;  // negative positions are skipped
  const int r = qvalid ? v / g : 0;
  const int hq = kvh * g + (qvalid ? v % g : 0);
  const int pq = qvalid ? min(rp[r], a.L - 1) : -1;

  // Q as the B operand of S^T: this lane holds dims 16*ks + 8*hh + s, rotated at position pq. The
  // rotated float32 query is split into hi = bf16(q) and lo = bf16(q - hi): rounding it to a single
  // bf16 would move the logits by ~1e-3 relative, the dominant error of the output.
  bf16x8 qhi[NKS], qlo[NKS];
  {
    float qf[NKS][8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[ks][s] = 0.f;
    if (qvalid) {
      const int srow = a.indexed ? pq : r;
      const uint16_t* qp = a.q + (((int64_t)req * a.q_rows + srow) * a.Hq + hq) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          qf[ks][2 * k] = __uint_as_float(w[k] << 16);
          qf[ks][2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
      }
      const float2* csr = a.cs + ((int64_t)req * a.R + r) * H + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float2 c = csr[16 * ks + s];
          const float x = qf[ks][s], y = qf[ks + NKS / 2][s];
          qf[ks][s] = x * c.x - y * c.y;
          qf[ks + NKS / 2][s] = x * c.y + y * c.x;
        }
    }
    // log2(e)/sqrt(d) is folded into the query, so the products come out as exp2 exponents
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 wh, wl;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = qf[ks][2 * k] * a.scale_log2, x1 = qf[ks][2 * k + 1] * a.scale_log2;
        wh[k] = pack_bf2(x0, x1);
        wl[k] = pack_bf2(x0 - bf2f(wh[k] & 0xffffu), x1 - bf2f(wh[k] >> 16));
      }
      qhi[ks] = as_bf16x8(wh);
      qlo[ks] = as_bf16x8(wl);
    }
  }
  // smallest position among this wave's query vectors: tiles entirely at or below it need no mask
  int pmin = qvalid ? pq : INT_MAX;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) pmin = min(pmin, __shfl_xor(pmin, off, 64));

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int64_t kv_base = ((int64_t)req * a.L * a.Hkv + kvh) * D;
  const int64_t kv_row = (int64_t)a.Hkv * D;

  // Tile loads. K: 16-byte chunks, dims fastest (coalesced rows). V: each task holds 4 keys x 8
  // dims and writes them transposed; key quads vary fastest across lanes, so the 16 lanes an LDS
  // write serves together hit 16 distinct bank pairs. The next tile's loads are issued into
  // registers before the current tile is computed, hiding the global-memory latency.
  constexpr int NKL = KT * (D / 8) / 256;           // K chunks per thread
  const bool vtask = threadIdx.x < (KT / 4) * (D / 8);
  const int vkq = threadIdx.x % (KT / 4), vc = threadIdx.x / (KT / 4);
  u32x4 kr[NKL], vr[4];
  auto prefetch = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int u = threadIdx.x + 256 * i;
      const int j = kt0 + u / (D / 8);
      kr[i] = u32x4{0u, 0u, 0u, 0u};
      if (j < kend) kr[i] = *reinterpret_cast<const u32x4*>(a.kf + kv_base + j * kv_row + 8 * (u % (D / 8)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = kt0 + 4 * vkq + i;
      vr[i] = u32x4{0u, 0u, 0u, 0u};
      if (vtask && j < kend) vr[i] = *reinterpret_cast<const u32x4*>(a.vf + kv_base + j * kv_row + 8 * vc);
    }
  };
  prefetch(kbeg);

  for (int kt0 = kbeg; kt0 < kend; kt0 += KT) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int u = threadIdx.x + 256 * i;
      *reinterpret_cast<u32x4*>(Ks + (u / (D / 8)) * KST + 8 * (u % (D / 8))) = kr[i];
    }
    if (vtask) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {  // word p: dims 8c+2p (low half) and 8c+2p+1 (high half)
        u32x2 lo, hi;
        lo[0] = (vr[0][p] & 0xffffu) | (vr[1][p] << 16);
        lo[1] = (vr[2][p] & 0xffffu) | (vr[3][p] << 16);
        hi[0] = (vr[0][p] >> 16) | (vr[1][p] & 0xffff0000u);
        hi[1] = (vr[2][p] >> 16) | (vr[3][p] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(Vt + (8 * vc + 2 * p) * VST + 4 * vkq) = lo;
        *reinterpret_cast<u32x2*>(Vt + (8 * vc + 2 * p + 1) * VST + 4 * vkq) = hi;
      }
    }
    __syncthreads();
    if (kt0 + KT < kend) prefetch(kt0 + KT);

    // S^T[key][q] for two 32-key sub-tiles
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 ka =
            as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + (32 * st + l32) * KST + 16 * ks + 8 * hh));
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qhi[ks], s[st], 0, 0, 0);
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qlo[ks], s[st], 0, 0, 0);
      }
    }
    // causal mask by absolute position (only on tiles that reach past the wave's smallest
    // position or the split's end), online softmax in the log2 domain
    float mt = -INFINITY;
    if (kt0 + KT <= kend && kt0 + KT - 1 <= pmin) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, s[st][rr]);
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = kt0 + 32 * st + 8 * (rr >> 2) + 4 * hh + (rr & 3);
          if (!(key < kend && key <= pq)) s[st][rr] = -INFINITY;
          mt = fmaxf(mt, s[st][rr]);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // all masked so far: every p is 0
    const float alpha = fast_exp2(m_run - m_use);
    float lsum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float p = fast_exp2(s[st][rr] - m_use);
        s[st][rr] = p;
        lsum += p;
      }
    l_run = l_run * alpha + lsum;
    // rescale the accumulator only when some lane's running max grew (alpha is 1 elsewhere)
    if (__any(m_new > m_run)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    m_run = m_new;

    // O^T[d][q] += V^T[d][key] P^T[key][q]; hardware k = 8*hh + s <-> key 32st + 16mp + 8(s/4) + 4hh + s%4
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {
        u32x4 pw;
#pragma unroll
        for (int k = 0; k < 4; ++k) pw[k] = pack_bf2(s[st][8 * mp + 2 * k], s[st][8 * mp + 2 * k + 1]);
        const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint16_t* vrow = Vt + (32 * dt + l32) * VST + 32 * st + 16 * mp + 4 * hh;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          const u32x4 vw = {lo[0], lo[1], hi[0], hi[1]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), pb, o[dt], 0, 0, 0);
        }
      }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  // o[dt][rr] holds dim 32*dt + 8*(rr/4) + 4*hh + rr%4 of query vector v
  if constexpr (!SPLIT) {
    if (qvalid) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* op = a.out + (((int64_t)req * a.R + r) * a.Hq + hq) * D + 4 * hh;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          u32x2 w;
          w[0] = pack_bf2(o[dt][4 * b4] * inv, o[dt][4 * b4 + 1] * inv);
          w[1] = pack_bf2(o[dt][4 * b4 + 2] * inv, o[dt][4 * b4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * b4) = w;
        }
      if (hh == 0 && a.lse)
        a.lse[((int64_t)req * a.R + r) * a.Hq + hq] =
            l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  } else {
    const int64_t pi =
        ((int64_t)(group * a.n_tiles + tile) * a.n_splits + split) * 128 + wave * 32 + l32;
    float* po = a.part_o + pi * D + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const f32x4 w = {o[dt][4 * b4], o[dt][4 * b4 + 1], o[dt][4 * b4 + 2], o[dt][4 * b4 + 3]};
        *reinterpret_cast<f32x4*>(po + 32 * dt + 8 * b4) = w;
      }
    if (hh == 0) a.part_ml[pi] = make_float2(m_run, l_tot);
  }
}

// Merge the key splits in split order. One thread per (query vector, 4 dims): every load of a
// thread is independent of the others (fixed-size unrolled split loop), so the kernel runs at
// memory speed instead of a chain of load latencies.
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  constexpr int TPV = D / 4;                 // threads per query vector
  constexpr int VPB = 256 / TPV;             // query vectors per block
  const int slab = blockIdx.x % (128 / VPB);
  const int gt = blockIdx.x / (128 / VPB);   // group-major (group, tile) index
  const int group = gt % a.n_groups, tile = gt / a.n_groups;
  const int req = group / a.Hkv, kvh = group % a.Hkv;
  const int g = a.g, Mv = a.R * g, v0 = tile * 128;
  const int ql = slab * VPB + threadIdx.x / TPV, dc = threadIdx.x % TPV;
  const int v = v0 + ql;
  if (v >= Mv) return;
  const int* rp = a.row_pos + (int64_t)req * a.R;
  const int maxkey = min(rp[min(v0 + 127, Mv - 1) / g], a.L - 1);
  if (maxkey < 0) return;
  const int nvalid = min(a.n_splits, maxkey / a.key_split + 1);
  const int64_t base = (int64_t)(group * a.n_tiles + tile) * a.n_splits * 128 + ql;
  float2 ml[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    ml[s] = s < nvalid ? a.part_ml[base + s * 128] : make_float2(-INFINITY, 0.f);
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) M = fmaxf(M, ml[s].x);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float Ls = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < nvalid && ml[s].x != -INFINITY) {
      const float w = exp2f(ml[s].x - M);
      Ls += ml[s].y * w;
      acc += w * *reinterpret_cast<const f32x4*>(a.part_o + (base + s * 128) * D + 4 * dc);
    }
  }
  const int r = v / g, hq = kvh * g + v % g;
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  u32x2 w;
  w[0] = pack_bf2(acc[0] * inv, acc[1] * inv);
  w[1] = pack_bf2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(a.out + (((int64_t)req * a.R + r) * a.Hq + hq) * D + 4 * dc) = w;
  if (dc == 0 && a.lse)
    a.lse[((int64_t)req * a.R + r) * a.Hq + hq] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------- float32 path
constexpr int kF32MaxGroup = 16;

template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(int Hq, int Hkv, int R, int L, const float* __restrict__ q,
                                                  int q_rows, int indexed, const int* __restrict__ row_pos,
                                                  const float2* __restrict__ cs,
                                                  const float* __restrict__ kf,
                                                  const float* __restrict__ vf,
                                                  float* __restrict__ out, float* __restrict__ lse,
                                                  float scale_log2) {
  constexpr int H = D / 2;
  constexpr int KC = 256;
  __shared__ float qs[kF32MaxGroup][D];
  __shared__ float ys[kF32MaxGroup][KC];
  __shared__ float m_s[kF32MaxGroup], l_s[kF32MaxGroup], alpha_s[kF32MaxGroup];
  const int r = blockIdx.x, kvh = blockIdx.y, req = blockIdx.z;
  const int g = Hq / Hkv;
  const int p = min(row_pos[(int64_t)req * R + r], L - 1);  // keys never read past the cache
  if (p < 0) return;
  const int srow = indexed ? p : r;
  const float2* csr = cs + ((int64_t)req * R + r) * H;
  for (int idx = threadIdx.x; idx < g * H; idx += blockDim.x) {
    const int hh = idx / H, i = idx % H;
    const float* qp = q + (((int64_t)req * q_rows + srow) * Hq + kvh * g + hh) * D;
    const float x = qp[i], y = qp[i + H];
    const float2 c = csr[i];
    qs[hh][i] = x * c.x - y * c.y;
    qs[hh][i + H] = x * c.y + y * c.x;
  }
  if (threadIdx.x < g) {
    m_s[threadIdx.x] = -INFINITY;
    l_s[threadIdx.x] = 0.f;
  }
  constexpr int kMaxPer = kF32MaxGroup * D / 256;
  float oacc[kMaxPer];
  for (int k = 0; k < kMaxPer; ++k) oacc[k] = 0.f;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t kv0 = (int64_t)req * L * Hkv + kvh;
  for (int kc = 0; kc <= p; kc += KC) {
    const int j = kc + threadIdx.x;
    for (int hh = 0; hh < g; ++hh) {
      float y = -INFINITY;
      if (j <= p) {
        const float* kp = kf + (kv0 + (int64_t)j * Hkv) * D;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot += qs[hh][d] * kp[d];
        y = dot * scale_log2;
      }
      ys[hh][threadIdx.x] = y;
    }
    __syncthreads();
    for (int hh = wave; hh < g; hh += 4) {
      float mx = -INFINITY;
      for (int k = 0; k < KC / 64; ++k) mx = fmaxf(mx, ys[hh][lane + 64 * k]);
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_down(mx, off, 64));
      mx = __shfl(mx, 0, 64);
      const float m_new = fmaxf(m_s[hh], mx);
      float sum = 0.f;
      for (int k = 0; k < KC / 64; ++k) {
        const float y = ys[hh][lane + 64 * k];
        const float e = (y == -INFINITY) ? 0.f : exp2f(y - m_new);
        ys[hh][lane + 64 * k] = e;
        sum += e;
      }
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_down(sum, off, 64);
      if (lane == 0) {
        const float alpha = (m_s[hh] == -INFINITY) ? 0.f : exp2f(m_s[hh] - m_new);
        alpha_s[hh] = alpha;
        l_s[hh] = l_s[hh] * alpha + sum;
        m_s[hh] = m_new;
      }
    }
    __syncthreads();
    const int nk = min(KC, p + 1 - kc);
    for (int k = 0; k < kMaxPer; ++k) {
      const int idx = threadIdx.x + 256 * k;
      if (idx >= g * D) break;
      const int hh = idx / D, d = idx % D;
      float o = oacc[k] * alpha_s[hh];
      for (int jj = 0; jj < nk; ++jj) o += ys[hh][jj] * vf[(kv0 + (int64_t)(kc + jj) * Hkv) * D + d];
      oacc[k] = o;
    }
    __syncthreads();
  }
  for (int k = 0; k < kMaxPer; ++k) {
    const int idx = threadIdx.x + 256 * k;
    if (idx >= g * D) break;
    const int hh = idx / D, d = idx % D;
    const int hq = kvh * g + hh;
    out[(((int64_t)req * R + r) * Hq + hq) * D + d] = oacc[k] / l_s[hh];
    if (d == 0 && lse) lse[((int64_t)req * R + r) * Hq + hq] = (m_s[hh] + log2f(l_s[hh])) * kLn2;
  }
}

}  // namespace

hipError_t launch_attn_bf16(int D, int n_req, int Hq, int Hkv, int R, int L, const uint16_t* q,
                            int q_rows, int indexed, const int* row_pos, const float2* cs,
                            const uint16_t* kf, const uint16_t* vf, uint16_t* out, float* lse,
                            int n_splits, int key_split, float* part_o, float2* part_ml,
                            hipStream_t st) {
  if (R == 0 || n_req == 0) return hipSuccess;
  AttnArgs a;
  a.q = q; a.row_pos = row_pos; a.cs = cs; a.kf = kf; a.vf = vf; a.out = out; a.lse = lse;
  a.part_o = part_o; a.part_ml = part_ml;
  a.n_req = n_req; a.Hq = Hq; a.Hkv = Hkv; a.g = Hq / Hkv; a.R = R; a.L = L; a.q_rows = q_rows;
  a.indexed = indexed;
  a.n_groups = n_req * Hkv;
  a.n_tiles = (R * a.g + 127) / 128;
  a.n_splits = n_splits;
  a.key_split = key_split;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const unsigned nblk = (unsigned)(a.n_groups * a.n_tiles * n_splits);
  if (n_splits == 1) {
    if (D == 128) k_attn_mfma<128, false><<<dim3(nblk), dim3(256), 0, st>>>(a);
    else k_attn_mfma<64, false><<<dim3(nblk), dim3(256), 0, st>>>(a);
  } else {
    if (D == 128) k_attn_mfma<128, true><<<dim3(nblk), dim3(256), 0, st>>>(a);
    else k_attn_mfma<64, true><<<dim3(nblk), dim3(256), 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const unsigned ncomb = (unsigned)(a.n_groups * a.n_tiles * (D == 128 ? 16 : 8));
    if (D == 128) k_attn_combine<128><<<dim3(ncomb), dim3(256), 0, st>>>(a);
    else k_attn_combine<64><<<dim3(ncomb), dim3(256), 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(int D, int n_req, int Hq, int Hkv, int R, int L, const float* q,
                           int q_rows, int indexed, const int* row_pos, const float2* cs,
                           const float* kf, const float* vf, float* out, float* lse,
                           hipStream_t st) {
  if (R == 0 || n_req == 0) return hipSuccess;
  dim3 g(R, Hkv, n_req), b(256);
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  if (D == 128)
    k_attn_f32<128><<<g, b, 0, st>>>(Hq, Hkv, R, L, q, q_rows, indexed, row_pos, cs, kf, vf, out, lse, sl2);
  else
    k_attn_f32<64><<<g, b, 0, st>>>(Hq, Hkv, R, L, q, q_rows, indexed, row_pos, cs, kf, vf, out, lse, sl2);
  return hipGetLastError();
}

}  // namespace sra
