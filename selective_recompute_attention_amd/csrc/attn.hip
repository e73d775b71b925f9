// Location-aware sparse causal attention (QCFuse technical summary (zh), §2.A: the recomputed
// tokens come as a discrete index table and attend under a strict causal constraint; KVCache
// reuse 01, §1.3.4: attention of the selected tokens against all tokens).
//
// For recomputed row r at absolute position p = row_pos[r] and query head h (KV head h/g):
//   q = R(p) q_new[r][h];  out = sum_{j <= p} softmax_j(q . k_j / sqrt(d)) v_j
//
// bf16 path, gfx950 matrix cores (v_mfma_f32_32x32x16_f16 for S, v_mfma_f32_32x32x16_bf16 for O):
//   * A tile is 128 query vectors of one (request, KV head) group: the flattened (row, head in
//     group) pairs v = r*g + hh, so any group size g packs without padding. Rows are ascending, so
//     a tile's key range ends at the position of its last row and takes ceil((p_last+1)/64) units
//     of 64 keys.
//   * Persistent split: a fixed grid of work groups per group (two per compute unit in total).
//     Each work group computes the tiles' unit counts from row_pos, takes the contiguous unit range
//     [U i / P, U (i+1) / P) and walks it tile by tile. A tile it covers whole is written directly;
//     a cut tile leaves a partial (O as fp16 scaled by the vector's largest |O|, max, sum) in one of
//     two slots (first / last tile of the range) and the merge kernel combines the pieces of such
//     tiles in key order. Every work group therefore gets the same number of key units, whatever
//     the position mix.
//   * Four waves, 32 query vectors each. S^T = K Q^T puts one query vector per lane column, so the
//     online-softmax row reductions stay in-lane plus one cross-half shuffle, and the probabilities
//     feed O^T = V^T P^T directly from registers (keys permuted consistently on both operands).
//   * Operands of S are fp16: the query comes pre-rotated, pre-scaled by log2(e)/sqrt(d) and rounded
//     once to fp16 (an 11-bit significand: the logits move by ~1e-4 relative, where one bf16
//     rounding would move them by ~1e-3 and dominate the output error), the keys come from the fp16
//     copy that the kernels writing the fused keys keep beside them (every bf16 key of magnitude
//     2^-14 .. 65504 is exact in fp16). Keys or scaled queries beyond fp16's range flag their group,
//     and the merge kernel recomputes that group exactly in float32 from the bf16 inputs.
//   * The S accumulator starts at minus the softmax reference, so the products come out already
//     relative to it. The reference is the maximum of a segment's first 32 keys; later keys are
//     exponentiated against it directly, and only when a 32-key block's probability sum exceeds
//     2^kLazyMax (some logit more than kLazyMax above the reference) does the reference move, with
//     the accumulator rescaled: no per-block maximum or subtraction in the common case.
//   * 64-key tiles: K row-major (fp16, padded rows) and V transposed on its way into LDS with the key
//     order of the probabilities (bits 2 and 3 of the key index swapped), so each P V operand is one
//     16-byte LDS read; both double-buffered, one barrier per tile, the next tile's rows loaded into
//     registers a tile ahead. Work groups are numbered with the group index fastest, so all work of
//     one KV head lands on one XCD (work groups are dealt round-robin over the 8 XCDs) and its K/V
//     stay in that XCD's L2.
// f32 path: plain float32 arithmetic, one block per (row, KV head), exact online softmax.
#include <float.h>

#include "common.h"

namespace sra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLazyMax = 16.f;       // log2 headroom of the attention softmax reference
constexpr float kSumCap = 65536.f;     // 2^kLazyMax: a 32-key block sum above it moves the reference

struct AttnArgs {
  const uint16_t* qop;
  const int* row_pos;
  const uint16_t* kh;     // fp16 copy of the fused keys
  const uint16_t* kf;     // bf16 fused keys (exact recomputation of flagged groups)
  const uint16_t* vf;
  uint16_t* out;
  float* lse;
  int* tilecum;
  uint16_t* part_o;   // fp16, scaled per vector
  float4* part_ml;    // (max, sum, scale, 0) per vector
  const uint16_t* qx;       // fresh queries before rotation (exact recomputation)
  const unsigned* flags;    // [n_groups]: call_id where an fp16 operand overflowed
  int* fallback;            // optional [n_groups] report
  unsigned call_id;
  int q_rows, q_indexed;
  int n_req, Hq, Hkv, g, R, L;
  int n_groups, n_tiles, qop_blocks, pieces;
  Theta th;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// float pair -> two fp16 (round to nearest even) in one word, and back
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ __forceinline__ float h2f(uint32_t h16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h16); }

__device__ __forceinline__ int64_t part_index(const AttnArgs& a, int group, int piece, int slot) {
  return ((int64_t)(group * a.pieces + piece) * 2 + slot) * 128;
}

// Position of tile-local key k in the transposed V tile: bits 2 and 3 swapped, which lists each
// lane's eight probabilities of a 16-key step (keys 8s' + 4hh + e, s' and e free) contiguously.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Probabilities of one 32-key half against the current reference (x already relative to it): bf16
// operands of the P V products and their sum (the same rounded values, one v_dot2c_f32_bf16 per
// pair, so the output weights stay a convex combination).
__device__ __forceinline__ void probs(const f32x16& x, u32x4* pw, float& lsum) {
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int mp = 0; mp < 2; ++mp)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // (the pair is taken from a scalar word: a bit cast of a vector element picked the wrong
      // element here)
      const uint32_t pk = pack_bf2(fast_exp2(x[8 * mp + 2 * k]), fast_exp2(x[8 * mp + 2 * k + 1]));
      pw[mp][k] = pk;
      if (k & 1) s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, s1, false);
      else s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, s0, false);
    }
  lsum = s0 + s1;
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_mfma(AttnArgs a) {
  constexpr int NKS = D / 16;   // K-steps of S^T = K Q^T
  constexpr int NDT = D / 32;   // 32-row d tiles of O^T
  constexpr int KT = 64;        // keys per LDS tile (one unit)
  constexpr int KST = D + 8;    // K row stride in LDS (elements): conflict-free 16-byte reads
  constexpr int VST = KT + 8;   // V^T row stride in LDS (elements): conflict-free 16-byte reads
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KST];   // double-buffered tiles
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VST];
  __shared__ int cum[kAttnMaxTiles + 1];
  __shared__ int wsum[4];

  const int group = blockIdx.x % a.n_groups;
  const int piece = blockIdx.x / a.n_groups;
  const int req = group / a.Hkv, kvh = group % a.Hkv;
  const int g = a.g;
  const int Mv = a.R * g;
  const int nt = a.n_tiles;
  const int* rp = a.row_pos + (int64_t)req * a.R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;

  // Units per tile and their prefix sums (cum[t] = units before tile t). Keys never reach past
  // the cache; a tile whose last position is negative has no keys.
  {
    const int per = (nt + 255) / 256;
    const int t_lo = min((int)threadIdx.x * per, nt), t_hi = min(t_lo + per, nt);
    int local = 0;
    for (int t = t_lo; t < t_hi; ++t) {
      const int mk = min(rp[min(t * 128 + 127, Mv - 1) / g], a.L - 1);
      const int n = mk >= 0 ? mk / KT + 1 : 0;
      cum[t + 1] = n;
      local += n;
    }
    const int incl = (int)wave_incl_sum((uint32_t)local);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int t = t_lo; t < t_hi; ++t) {
      run += cum[t + 1];
      cum[t + 1] = run;
    }
    if (threadIdx.x == 0) cum[0] = 0;
    __syncthreads();
  }
  const int U = cum[nt];
  const int P = attn_pieces_used(U, a.pieces);
  if (kvh == 0 && piece == 0)
    for (int t = threadIdx.x; t <= nt; t += 256) a.tilecum[(int64_t)req * (nt + 1) + t] = cum[t];
  if (piece >= P) return;
  const int u0 = attn_piece_start(U, P, piece), u1 = attn_piece_start(U, P, piece + 1);
  int t = 0;  // last tile with cum[t] <= u0
  {
    int hi = nt - 1;
    while (t < hi) {
      const int mid = (t + hi + 1) >> 1;
      if (cum[mid] <= u0) t = mid;
      else hi = mid - 1;
    }
  }

  // uniform base of this (request, KV head); per-thread byte offsets fit 32 bits (checked by the host)
  const char* kbase = reinterpret_cast<const char*>(a.kh + ((int64_t)req * a.L * a.Hkv + kvh) * D);
  const char* vbase = reinterpret_cast<const char*>(a.vf + ((int64_t)req * a.L * a.Hkv + kvh) * D);
  const uint32_t row_bytes = (uint32_t)(a.Hkv * D * 2);
  // Tile loads. K: 16-byte chunks, dims fastest (coalesced rows). V: each task holds 4 keys x 8
  // dims and writes them transposed; key quads vary fastest across lanes, so the 16 lanes an LDS
  // write serves together hit 16 distinct bank pairs. The next tile's loads are issued into
  // registers before the current tile is computed, hiding the global-memory latency.
  constexpr int NKL = KT * (D / 8) / 256;           // K chunks per thread
  const bool vtask = threadIdx.x < (KT / 4) * (D / 8);
  const int vkq = threadIdx.x % (KT / 4), vc = threadIdx.x / (KT / 4);
  u32x4 kr[NKL], vr[4];
  auto prefetch = [&](int kt0, int kend) {
    // unconditional loads of clamped rows (kt0 < kend): rows past the range repeat row kend - 1,
    // whose keys the mask removes (probability 0 on finite values). Nothing reads the registers
    // until the tile is stored, so no load waits for another.
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int u = threadIdx.x + 256 * i;
      const uint32_t j = (uint32_t)min(kt0 + u / (D / 8), kend - 1);
      kr[i] = *reinterpret_cast<const u32x4*>(kbase + (j * row_bytes + 16u * (uint32_t)(u % (D / 8))));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t j = (uint32_t)min(kt0 + 4 * vkq + i, kend - 1);
      vr[i] = *reinterpret_cast<const u32x4*>(vbase + (j * row_bytes + 16u * (uint32_t)(vtask ? vc : 0)));
    }
  };

  int slot = 0;
  for (int u = u0; u < u1; ++t) {
    const int c0 = cum[t], c1 = cum[t + 1];
    const int se = min(u1, c1);
    if (se <= u) continue;  // tile without keys
    const bool direct = (u == c0 && se == c1);
    // keys stop at the tile's last position: rows past it are never read
    const int maxkey = min(rp[min(t * 128 + 127, Mv - 1) / g], a.L - 1);
    const int kbeg = KT * (u - c0), kend = min(KT * (se - c0), maxkey + 1);

    // query operand, K/V prefetch and the row position all go out before the first wait
    const int v = t * 128 + wave * 32 + l32;
    f16x8 q16[NKS];
    {
      // the wave's 32-vector block, fp16 plane 0: a uniform base and 32-bit lane offsets (layout of
      // qop_index)
      const char* qb = reinterpret_cast<const char*>(a.qop + qop_index(group, t * 4 + wave, 0, 0, 0, 0, a.qop_blocks, NKS));
      const uint32_t lo = (uint32_t)(l32 * 16 + hh * 8) * 2u;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        q16[ks] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(qb + ((uint32_t)(ks * 2) * 1024u + lo)));
    }
    prefetch(kbeg, kend);
    const int r = min(v, Mv - 1) / g;
    const int hq = kvh * g + v % g;
    const int p_r = rp[r];
    const bool qvalid = v < Mv && p_r >= 0;  // negative positions are skipped
    const int pq = qvalid ? min(p_r, a.L - 1) : -1;
    if (!qvalid) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) q16[ks] = __builtin_bit_cast(f16x8, u32x4{0u, 0u, 0u, 0u});
    }
    // smallest position among this wave's query vectors: tiles entirely at or below it need no mask
    const int pmin = (int)wave_reduce(qvalid ? (uint32_t)pq : (uint32_t)INT_MAX,
                                      [](uint32_t x, uint32_t y) { return x < y ? x : y; });

    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
    float m_ref = 0.f, l_run = 0.f;   // softmax reference (log2 domain) and running sum
    f32x16 negm = {};                 // -m_ref in every element: the S accumulator's start value
    bool first = true;                // wave-uniform: the segment's first half sets the reference

    // K row-major; V transposed on the way in (word pp of a task: dims 8c+2pp in the low half
    // and 8c+2pp+1 in the high half, four keys each, at the keys' permuted position)
    const int vpos = vt_pos(4 * vkq);
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int i = 0; i < NKL; ++i) {
        const int uu = threadIdx.x + 256 * i;
        *reinterpret_cast<u32x4*>(&Ks[buf][(uu / (D / 8)) * KST + 8 * (uu % (D / 8))]) = kr[i];
      }
      if (vtask) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          u32x2 lo, hi;
          lo[0] = __builtin_amdgcn_perm(vr[1][pp], vr[0][pp], 0x05040100u);
          lo[1] = __builtin_amdgcn_perm(vr[3][pp], vr[2][pp], 0x05040100u);
          hi[0] = __builtin_amdgcn_perm(vr[1][pp], vr[0][pp], 0x07060302u);
          hi[1] = __builtin_amdgcn_perm(vr[3][pp], vr[2][pp], 0x07060302u);
          *reinterpret_cast<u32x2*>(&Vt[buf][(8 * vc + 2 * pp) * VST + vpos]) = lo;
          *reinterpret_cast<u32x2*>(&Vt[buf][(8 * vc + 2 * pp + 1) * VST + vpos]) = hi;
        }
      }
    };
    // Both buffers are free here: the previous segment's loop ended with a barrier. Tile t is
    // computed from buffer t%2 while tile t+1 is written to the other one, so one barrier per tile
    // both publishes the next tile and retires the current one.
    store_tile(0);
    if (kbeg + KT < kend) prefetch(kbeg + KT, kend);
    __syncthreads();
    int cur = 0;
    for (int kt0 = kbeg; kt0 < kend; kt0 += KT) {
      const uint16_t* Kc = Ks[cur];
      const uint16_t* Vc = Vt[cur];

      // S^T[key][q] - m_ref for the two 32-key halves. The halves then go through softmax and P V
      // one after the other, so the second half's products are still running while the first
      // half's probabilities are formed.
      f32x16 sc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const f16x8 ka = __builtin_bit_cast(
              f16x8, *reinterpret_cast<const u32x4*>(Kc + (32 * st + l32) * KST + 16 * ks + 8 * hh));
          sc[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, q16[ks], ks == 0 ? negm : sc[st], 0, 0, 0);
        }
      }
      // both halves' products started from the reference of the tile's start; when the first half
      // moves it (the segment's first half, or a rescale), the second half follows by the difference
      const float m_tile = m_ref;
      bool moved = false;   // wave-uniform
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x16 x = sc[st];
        if (moved) {
          const float dm = m_tile - m_ref;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) x[rr] += dm;
        }
        // causal mask by absolute position where the half reaches past the wave's smallest position
        // or the range's end: element rr holds key kt0 + 32 st + 4 hh + (8 (rr / 4) + rr % 4)
        const int klast = kt0 + 32 * st + 31;
        if (!(klast < kend && klast <= pmin)) {
          const int lim = min(kend - 1, pq) - (kt0 + 32 * st + 4 * hh);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (8 * (rr >> 2) + (rr & 3) > lim) x[rr] = -INFINITY;
        }
        if (first) {   // the segment's first half: its maximum becomes the reference (x was the logit)
          float mt = -INFINITY;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, x[rr]);
          mt = half_max(mt);
          const float r0 = mt == -INFINITY ? 0.f : mt;   // no visible key in the segment: stays 0
          m_ref = r0;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            x[rr] -= r0;
            negm[rr] = -r0;
          }
          first = false;
          moved = true;
        }
        u32x4 pw[2];
        float lsum;
        probs(x, pw, lsum);
        if (__any(lsum > kSumCap)) {   // a logit more than kLazyMax above the reference: move it
          float mt = -INFINITY;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, x[rr]);
          mt = half_max(mt);
          const float sh = mt > 0.f ? mt : 0.f;
          const float alpha = fast_exp2(-sh);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
          l_run *= alpha;
          m_ref += sh;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            x[rr] -= sh;
            negm[rr] = -m_ref;
          }
          moved = true;
          probs(x, pw, lsum);
        }
        l_run += lsum;

        // O^T[d][q] += V^T[d][key] P^T[key][q]; hardware k = 8*hh + s <-> key 32st + 16mp + 8(s/4) + 4hh + s%4,
        // stored at V^T position 32st + 16mp + 8hh + s
#pragma unroll
        for (int mp = 0; mp < 2; ++mp) {
          const bf16x8 pb = as_bf16x8(pw[mp]);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const u32x4 vw = *reinterpret_cast<const u32x4*>(Vc + (32 * dt + l32) * VST + 32 * st + 16 * mp + 8 * hh);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), pb, o[dt], 0, 0, 0);
          }
        }
      }

      if (kt0 + KT < kend) {
        store_tile(cur ^ 1);   // its previous tile was retired by the last barrier
        if (kt0 + 2 * KT < kend) prefetch(kt0 + 2 * KT, kend);
      }
      __syncthreads();
      cur ^= 1;
    }

    const float l_tot = half_sum(l_run);
    // the lane's store offsets are formed here from an opaque copy of the lane index, so that the
    // compiler does not hold 64-bit lane addresses across the key loop (they would spill)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int e32 = ln & 31, ehh = ln >> 5;
    // o[dt][rr] holds dim 32*dt + 8*(rr/4) + 4*hh + rr%4 of query vector v
    if (direct) {
      if (qvalid) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        // uniform request base and a 32-bit lane offset (the host bounds R*Hq*D)
        uint16_t* ob = a.out + (int64_t)req * a.R * a.Hq * D;
        const uint32_t lo = (uint32_t)((r * a.Hq + hq) * D + 4 * ehh);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            u32x2 w;
            w[0] = pack_bf2(o[dt][4 * b4] * inv, o[dt][4 * b4 + 1] * inv);
            w[1] = pack_bf2(o[dt][4 * b4 + 2] * inv, o[dt][4 * b4 + 3] * inv);
            *reinterpret_cast<u32x2*>(ob + (lo + (uint32_t)(32 * dt + 8 * b4))) = w;
          }
        if (hh == 0 && a.lse)
          a.lse[((int64_t)req * a.R + r) * a.Hq + hq] =
              l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
      }
    } else {
      // the wave's 32 vectors of the slot (a uniform base and 32-bit lane offsets), O as fp16 scaled by
      // the vector's largest |O|: half the bytes of float32, 11-bit significands at any magnitude
      float mx = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, fabsf(o[dt][rr]));
      mx = half_max(mx);
      const float osc = mx > 0.f ? mx : 1.f, oinv = 1.f / osc;
      const int64_t pw = part_index(a, group, piece, slot) + __builtin_amdgcn_readfirstlane(wave) * 32;
      uint16_t* pob = a.part_o + pw * D;
      const uint32_t lo = (uint32_t)(e32 * D + 4 * ehh);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          u32x2 w;
          w[0] = pack_h2(o[dt][4 * b4] * oinv, o[dt][4 * b4 + 1] * oinv);
          w[1] = pack_h2(o[dt][4 * b4 + 2] * oinv, o[dt][4 * b4 + 3] * oinv);
          *reinterpret_cast<u32x2*>(pob + (lo + (uint32_t)(32 * dt + 8 * b4))) = w;
        }
      if (ehh == 0) a.part_ml[pw + e32] = make_float4(l_tot > 0.f ? m_ref : -INFINITY, l_tot, osc, 0.f);
    }
    slot = 1;
    u = se;
  }
}

// Exact float32 attention of one query vector per 32 threads (4 dims each), for a group whose fp16
// operands overflowed: the fresh query rotated at p with float64 angles, logits over the bf16 keys
// j <= p summed across the vector's threads, an online softmax with the exact running maximum, and
// the bf16 values; out and lse as the fast path writes them.
template <int D>
__device__ void exact_vector(const AttnArgs& a, int req, int kvh, int v) {
  constexpr int TPV = D / 4;
  const int dc = threadIdx.x % TPV;
  const int r = v / a.g, hq = kvh * a.g + v % a.g;
  const int p0 = a.row_pos[(int64_t)req * a.R + r];
  if (p0 < 0) return;   // rows outside the cache are skipped, as by the fast path
  const int p = min(p0, a.L - 1);
  const int srow = a.q_indexed ? p : r;
  const uint16_t* qrow = a.qx + (((int64_t)req * a.q_rows + srow) * a.Hq + hq) * D;
  const float scale = 1.f / sqrtf((float)D);
  float qv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * dc + k, i0 = i % (D / 2);
    const float x = bf2f(qrow[i0]), y = bf2f(qrow[i0 + D / 2]);
    const float2 c = rope_cs((double)p, a.th.v[i0]);
    qv[k] = (i < D / 2 ? x * c.x - y * c.y : x * c.y + y * c.x) * scale;
  }
  float m = -INFINITY, l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* kcol = a.kf + ((int64_t)req * a.L * a.Hkv + kvh) * D + 4 * dc;
  const uint16_t* vcol = a.vf + ((int64_t)req * a.L * a.Hkv + kvh) * D + 4 * dc;
  const int64_t stride = (int64_t)a.Hkv * D;
  for (int j = 0; j <= p; ++j) {
    const u32x2 kw = *reinterpret_cast<const u32x2*>(kcol + j * stride);
    float x = qv[0] * bf2f(kw[0] & 0xffffu) + qv[1] * bf2f(kw[0] >> 16) + qv[2] * bf2f(kw[1] & 0xffffu) +
              qv[3] * bf2f(kw[1] >> 16);
#pragma unroll
    for (int msk = TPV / 2; msk >= 1; msk >>= 1) x += __shfl_xor(x, msk, TPV);
    const float mn = fmaxf(m, x);
    const float c = m == -INFINITY ? 0.f : expf(m - mn), e = expf(x - mn);
    const u32x2 vw = *reinterpret_cast<const u32x2*>(vcol + j * stride);
    l = l * c + e;
    o[0] = o[0] * c + e * bf2f(vw[0] & 0xffffu);
    o[1] = o[1] * c + e * bf2f(vw[0] >> 16);
    o[2] = o[2] * c + e * bf2f(vw[1] & 0xffffu);
    o[3] = o[3] * c + e * bf2f(vw[1] >> 16);
    m = mn;
  }
  const float inv = 1.f / l;
  u32x2 w;
  w[0] = pack_bf2(o[0] * inv, o[1] * inv);
  w[1] = pack_bf2(o[2] * inv, o[3] * inv);
  *reinterpret_cast<u32x2*>(a.out + (((int64_t)req * a.R + r) * a.Hq + hq) * D + 4 * dc) = w;
  if (dc == 0 && a.lse) a.lse[((int64_t)req * a.R + r) * a.Hq + hq] = m + logf(l);
}

// Merge the pieces of every cut tile in key order. One thread per (query vector, 4 dims); the
// pieces' loads go out in independent batches of eight. A group whose fp16 operands overflowed is
// recomputed exactly here instead (every tile of it, cut or not).
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  constexpr int TPV = D / 4;                 // threads per query vector
  constexpr int VPB = 256 / TPV;             // query vectors per block
  constexpr int B = 8;
  const int slab = blockIdx.x % (128 / VPB);
  const int gt = blockIdx.x / (128 / VPB);   // group-fastest (group, tile) index
  const int group = gt % a.n_groups, tile = gt / a.n_groups;
  const int req = group / a.Hkv, kvh = group % a.Hkv;
  const int nt = a.n_tiles;
  const int* cum = a.tilecum + (int64_t)req * (nt + 1);
  // the tile's unit range, the request's total and the group's flag as one batch of loads
  int c0 = cum[tile], c1 = cum[tile + 1], U = cum[nt], pieces = a.pieces;
  unsigned fl = a.flags[group];
  asm volatile("" : "+s"(c0), "+s"(c1), "+s"(U), "+s"(pieces), "+s"(fl) : "s"(a.row_pos), "s"(a.part_ml), "s"(a.part_o));
  const bool exact = fl == a.call_id;
  if (tile == 0 && slab == 0 && threadIdx.x == 0 && a.fallback) a.fallback[group] = exact ? 1 : 0;
  const int g = a.g, Mv = a.R * g;
  if (exact) {
    const int v = tile * 128 + slab * VPB + (int)threadIdx.x / TPV;
    if (v < Mv) exact_vector<D>(a, req, kvh, v);
    return;
  }
  if (c1 <= c0) return;
  const int P = attn_pieces_used(U, pieces);
  const int i0 = attn_piece_of(U, P, c0), i1 = attn_piece_of(U, P, c1 - 1);
  if (i0 == i1) return;  // written directly by its only piece
  const int ql = slab * VPB + threadIdx.x / TPV, dc = threadIdx.x % TPV;
  const int v = tile * 128 + ql;
  if (v >= Mv) return;
  const int r = v / g, hq = kvh * g + v % g;
  // the row's position is loaded with the first batch of pieces and checked at the end
  const int pos_r = a.row_pos[(int64_t)req * a.R + r];
  // piece i0 ends in this tile: its slot is 1 unless the tile is also where it starts
  const int slot0 = attn_piece_start(U, P, i0) < c0 ? 1 : 0;
  const int n = i1 - i0 + 1;
  auto pidx = [&](int k) { return part_index(a, group, i0 + k, k == 0 ? slot0 : 0) + ql; };
  // online merge over batches of eight pieces; every load of a batch is independent
  float M = -INFINITY, Ls = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += B) {
    float4 ml[B];
    u32x2 hv[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {   // clamped, unconditional loads: all in flight at once
      const int64_t pi = pidx(min(k0 + k, n - 1));
      ml[k] = a.part_ml[pi];
      hv[k] = *reinterpret_cast<const u32x2*>(a.part_o + pi * D + 4 * dc);
    }
    // both halves of the batch are in flight before either is used (a piece skipped below would
    // otherwise have its values loaded only after that test)
    asm volatile("" ::"v"(hv[0][0]), "v"(hv[0][1]), "v"(hv[1][0]), "v"(hv[1][1]), "v"(hv[2][0]), "v"(hv[2][1]),
                 "v"(hv[3][0]), "v"(hv[3][1]), "v"(hv[4][0]), "v"(hv[4][1]), "v"(hv[5][0]), "v"(hv[5][1]),
                 "v"(hv[6][0]), "v"(hv[6][1]), "v"(hv[7][0]), "v"(hv[7][1]));
    f32x4 ov[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (k0 + k >= n) ml[k] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
      ov[k] = f32x4{h2f(hv[k][0] & 0xffffu), h2f(hv[k][0] >> 16), h2f(hv[k][1] & 0xffffu), h2f(hv[k][1] >> 16)} * ml[k].z;
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < B; ++k) mb = fmaxf(mb, ml[k].x);
    if (mb == -INFINITY) continue;
    const float sc = exp2f(M - mb);  // 0 while nothing has been merged (M = -inf)
    Ls *= sc;
    acc *= sc;
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (ml[k].x != -INFINITY) {
        const float w = exp2f(ml[k].x - mb);
        Ls += ml[k].y * w;
        acc += w * ov[k];
      }
    }
    M = mb;
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  u32x2 w;
  w[0] = pack_bf2(acc[0] * inv, acc[1] * inv);
  w[1] = pack_bf2(acc[2] * inv, acc[3] * inv);
  // the merge is finished for every row (the asm keeps it out of the branch), and only then a row
  // outside the cache is dropped: nothing is written for it
  asm volatile("" ::"v"(w[0]), "v"(w[1]), "v"(M), "v"(Ls));
  if (pos_r < 0) return;
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

hipError_t launch_attn_bf16(int D, int n_req, int Hq, int Hkv, int R, int L, const uint16_t* qop,
                            int qop_blocks, const int* row_pos, const uint16_t* kh, const uint16_t* kf,
                            const uint16_t* vf, uint16_t* out, float* lse, int pieces,
                            int* tilecum, uint16_t* part_o, float4* part_ml, const AttnExact& ex,
                            hipStream_t st) {
  if (R == 0 || n_req == 0) return hipSuccess;
  if (!ex.flags || !ex.q) return hipErrorInvalidValue;
  AttnArgs a;
  a.qop = qop; a.row_pos = row_pos; a.kh = kh; a.kf = kf; a.vf = vf; a.out = out; a.lse = lse;
  a.tilecum = tilecum; a.part_o = part_o; a.part_ml = part_ml;
  a.qx = ex.q; a.flags = ex.flags; a.fallback = ex.fallback; a.call_id = ex.call_id;
  a.q_rows = ex.q_rows; a.q_indexed = ex.indexed;
  a.th = make_theta(D, ex.base);
  a.n_req = n_req; a.Hq = Hq; a.Hkv = Hkv; a.g = Hq / Hkv; a.R = R; a.L = L;
  a.n_groups = n_req * Hkv;
  a.n_tiles = (R * a.g + 127) / 128;
  a.qop_blocks = qop_blocks;
  a.pieces = pieces;
  if (a.n_tiles > kAttnMaxTiles || qop_blocks < 4 * a.n_tiles || pieces < 1) return hipErrorInvalidValue;
  const unsigned nblk = (unsigned)(a.n_groups * pieces);
  if (D == 128) k_attn_mfma<128><<<dim3(nblk), dim3(256), 0, st>>>(a);
  else k_attn_mfma<64><<<dim3(nblk), dim3(256), 0, st>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned ncomb = (unsigned)(a.n_groups * a.n_tiles * (D == 128 ? 16 : 8));
  if (D == 128) k_attn_combine<128><<<dim3(ncomb), dim3(256), 0, st>>>(a);
  else k_attn_combine<64><<<dim3(ncomb), dim3(256), 0, st>>>(a);
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
