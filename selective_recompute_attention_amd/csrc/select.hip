// Top-N selection of context tokens by score (QCFuse technical summary (zh), §2.A: the Top-N
// context token indices from the critical-layer attention distribution; ties follow a stable
// sort by descending score, Cache-Craft CSDN article §2.2.2, so the lower index wins).
//
// One block of 1024 threads per selection unit (a whole request, or one chunk of a request when
// per-chunk quotas are given, or one (level, request) of a nested selection among earlier rows).
// The block first forms the scores (fixed-point totals over KV heads, or per-head float partials
// added in a fixed order), then finds the score of the N-th best token
// exactly with an 8-bit radix select over order-preserving 32-bit keys (leading bytes shared by
// every key are skipped), and finally writes, in ascending position order, every token above that
// score plus the lowest-index tokens equal to it. All decisions are integer comparisons of the
// same float32 bits, so the result is deterministic.
//
// The kernel is a chain of dependent steps on one CU, so it is written for latency: the score
// loads go out before the histograms are cleared, each radix pass costs two barriers (count, then
// one wave scans the 256 bins with 16-byte LDS reads), and one two-value block scan places the
// output.
#include "common.h"

namespace sra {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelLdsKeys = 32768;   // keys of one selection unit kept in LDS (128 KB of the 160 KB)
constexpr int kSelSub = 4;           // copies of each histogram bin, chosen by lane (a multiple of 4)
static_assert(kSelSub % 4 == 0 && 4 * 256 * kSelSub % (4 * kSelThreads) == 0, "histogram layout");

// Score sources: fixed-point totals, per-head partials (both written back as the float scores), the
// scores themselves, or the scores of the rows an index map lists (unit index j -> map[j]).
enum SelSrc { kFromFixed = 0, kFromParts = 1, kFromScores = 2, kFromGather = 3 };

// Order-preserving key of a score; -0 and +0 are equal scores (their ties go by position) and get
// the key of +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int SRC>
__global__ __launch_bounds__(kSelThreads) void k_select(SelTab tab, const unsigned long long* __restrict__ fx,
                                                        int nparts, int Lctx, int Lq, int sstride,
                                                        const float* __restrict__ parts,
                                                        float* __restrict__ scores,
                                                        const int* __restrict__ map, int map_stride) {
  constexpr bool kWritesScores = SRC == kFromFixed || SRC == kFromParts;
  constexpr int NW = kSelThreads / 64;
  constexpr int KREG = 4;    // keys per thread held in registers (units up to 4096 keys)
  // one histogram per key byte, kSelSub copies of each bin (lanes of a wave that hit the same bin,
  // common while the leading bytes take few values, spread over the copies)
  __shared__ __attribute__((aligned(16))) uint32_t hist[4][256 * kSelSub];
  __shared__ uint32_t kl[kSelLdsKeys];   // the unit's keys when they fit
  __shared__ uint32_t sh_and[NW], sh_or[NW], sh_sel[2];
  __shared__ uint32_t wsum[2][NW];
  const int e = blockIdx.x;
  const int req = tab.req[e], begin = tab.begin[e], len = tab.len[e];
  const int quota = tab.quota[e], off = tab.out_off[e], wq = tab.writes_query[e], R = tab.rows[e];
  int* out = tab.out[e];
  // every argument, fetched as one batch of scalar loads before the first global load
  asm volatile("" ::"s"(req), "s"(begin), "s"(len), "s"(quota), "s"(off), "s"(wq), "s"(fx), "s"(parts),
               "s"(scores), "s"(out), "s"(map), "s"(map_stride), "s"(nparts), "s"(Lctx), "s"(Lq), "s"(R),
               "s"(sstride));
  float* srow = scores + (int64_t)req * sstride + begin;
  const int* mrow = map ? map + (int64_t)req * map_stride : nullptr;   // index -> written value
  // score of unit index j where it is stored (written back above for the computed sources); a
  // gathered row outside the score row is clamped into it, so no read leaves the scores
  auto stored = [&](int j) -> float {
    if constexpr (SRC == kFromGather) return srow[min((uint32_t)mrow[begin + j], (uint32_t)(sstride - 1))];
    else return srow[j];
  };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // thread t owns the contiguous positions [jlo, jhi): block prefix sums of per-thread counts then
  // give ascending output slots
  const int per = (len + kSelThreads - 1) / kSelThreads;
  const int jlo = min((int)threadIdx.x * per, len), jhi = min(jlo + per, len), cnt = jhi - jlo;
  const bool in_regs = len > 0 && per <= KREG;
  const bool in_lds = len <= kSelLdsKeys;
  auto clear_hist = [&]() {
    uint4* h = reinterpret_cast<uint4*>(&hist[0][0]);
#pragma unroll
    for (int i = 0; i < 4 * 256 * kSelSub / 4 / kSelThreads; ++i) h[threadIdx.x + kSelThreads * i] = uint4{0u, 0u, 0u, 0u};
  };
  auto score_at = [&](int j) -> float {   // one score, loads in order (large units)
    if constexpr (SRC == kFromFixed) {
      return (float)((double)fx[(int64_t)req * Lctx + begin + j] * (1.0 / kScoreFixScale));
    } else if constexpr (SRC == kFromParts) {
      const float* prow = parts + (int64_t)req * nparts * Lctx + begin;
      float sv = 0.f;
      for (int p0 = 0; p0 < nparts; p0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = prow[(int64_t)min(p0 + u, nparts - 1) * Lctx + j];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (p0 + u < nparts) sv += v[u];
      }
      return sv;
    } else {
      return stored(j);
    }
  };

  // scores -> order-preserving keys; coalesced loads (position j = tid + 256 i), all issued before
  // the histograms are cleared; small units then pass their keys through LDS into this thread's
  // contiguous range of registers
  uint32_t kreg[KREG];
  uint32_t kand = ~0u, kor = 0u;
  if (in_regs) {
    float sv[KREG];
    if constexpr (SRC == kFromFixed) {
      const unsigned long long* frow = fx + (int64_t)req * Lctx + begin;
      unsigned long long fv[KREG];
#pragma unroll
      for (int i = 0; i < KREG; ++i) fv[i] = frow[min((int)threadIdx.x + kSelThreads * i, len - 1)];
      clear_hist();
#pragma unroll
      for (int i = 0; i < KREG; ++i) sv[i] = (float)((double)fv[i] * (1.0 / kScoreFixScale));
    } else if constexpr (SRC == kFromParts) {
      const float* prow = parts + (int64_t)req * nparts * Lctx + begin;
#pragma unroll
      for (int i = 0; i < KREG; ++i) sv[i] = 0.f;
      for (int p0 = 0; p0 < nparts; p0 += 8) {
        float v[KREG][8];   // clamped, unconditional loads: the whole batch is in flight at once
#pragma unroll
        for (int i = 0; i < KREG; ++i)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[i][u] = prow[(int64_t)min(p0 + u, nparts - 1) * Lctx + min((int)threadIdx.x + kSelThreads * i, len - 1)];
        if (p0 == 0) clear_hist();
#pragma unroll
        for (int i = 0; i < KREG; ++i)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (p0 + u < nparts) sv[i] += v[i][u];
      }
      if (nparts <= 0) clear_hist();
    } else {
#pragma unroll
      for (int i = 0; i < KREG; ++i) sv[i] = stored(min((int)threadIdx.x + kSelThreads * i, len - 1));
      clear_hist();
    }
#pragma unroll
    for (int i = 0; i < KREG; ++i) {
      const int j = threadIdx.x + kSelThreads * i;
      if (j < len) {
        const uint32_t u = order_key(sv[i]);
        if constexpr (kWritesScores) srow[j] = sv[i];
        kl[j] = u;
        kand &= u;
        kor |= u;
      }
    }
  } else {
    clear_hist();
    // batches of eight positions per thread, every load of a batch in flight before any is used
    constexpr int BT = 8;
    for (int j0 = threadIdx.x; j0 < len; j0 += kSelThreads * BT) {
      float sv[BT];
#pragma unroll
      for (int u = 0; u < BT; ++u) sv[u] = score_at(min(j0 + kSelThreads * u, len - 1));
#pragma unroll
      for (int u = 0; u < BT; ++u) {
        const int j = j0 + kSelThreads * u;
        if (j < len) {
          if constexpr (kWritesScores) srow[j] = sv[u];
          const uint32_t key = order_key(sv[u]);
          if (in_lds) kl[j] = key;
          kand &= key;
          kor |= key;
        }
      }
    }
  }
  // bits shared by every key of the unit (the same barrier publishes the keys in LDS)
  kand = wave_reduce(kand, [](uint32_t a, uint32_t b) { return a & b; });
  kor = wave_reduce(kor, [](uint32_t a, uint32_t b) { return a | b; });
  if (lane == 0) { sh_and[wave] = kand; sh_or[wave] = kor; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) { kand &= sh_and[w]; kor |= sh_or[w]; }
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < KREG; ++i) kreg[i] = kl[min(jlo + i, len - 1)];
  }
  // keys of large units are read back from LDS, or re-derived from the scores written above
  auto key_at = [&](int j) -> uint32_t { return in_lds ? kl[j] : order_key(stored(j)); };

  if (quota > 0 && len > 0) {
    uint32_t thr = 0, need_eq = 0;
    if (quota < len) {
      uint32_t prefix = 0, mask = 0, remaining = (uint32_t)quota;
      int shift = 24;
      // a byte equal in every key is the N-th key's byte too
      for (; shift >= 0 && (((kand ^ kor) >> shift) & 255u) == 0; shift -= 8) {
        prefix |= kand & (255u << shift);
        mask |= 255u << shift;
      }
      for (; shift >= 0; shift -= 8) {
        uint32_t* h = hist[shift >> 3];
        const uint32_t sub = lane & (kSelSub - 1);
        if (in_regs) {
#pragma unroll
          for (int i = 0; i < KREG; ++i)
            if (i < cnt && (kreg[i] & mask) == prefix) atomicAdd(&h[((kreg[i] >> shift) & 255u) * kSelSub + sub], 1u);
        } else {
          for (int j = jlo; j < jhi; ++j) {
            const uint32_t u = key_at(j);
            if ((u & mask) == prefix) atomicAdd(&h[((u >> shift) & 255u) * kSelSub + sub], 1u);
          }
        }
        __syncthreads();
        if (wave == 0) {
          // lane l holds bins 255-4l .. 252-4l (descending): the 4 kSelSub copies of bins 252-4l ..
          // 255-4l are contiguous, kSelSub 16-byte reads
          constexpr int QB = kSelSub / 4;   // 16-byte reads per bin
          const uint4* hp = reinterpret_cast<const uint4*>(h + (252 - 4 * lane) * kSelSub);
          uint32_t c[4], tot = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {   // bin 255 - 4 lane - k
            c[k] = 0;
#pragma unroll
            for (int q = 0; q < QB; ++q) {
              const uint4 a = hp[QB * (3 - k) + q];
              c[k] += (a.x + a.y) + (a.z + a.w);
            }
            tot += c[k];
          }
          const uint32_t incl = wave_incl_sum(tot);
          uint32_t cum = incl - tot, before = 0;
          int found = -1;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (found < 0 && cum + c[k] >= remaining) {
              found = 255 - 4 * lane - k;
              before = cum;
            }
            cum += c[k];
          }
          // the lowest lane with a hit holds the highest qualifying bin
          const int first = __ffsll((unsigned long long)__ballot(found >= 0)) - 1;
          const int bsel = __builtin_amdgcn_readlane(found, first);
          const uint32_t bef = __builtin_amdgcn_readlane(before, first);
          if (lane == 0) {
            sh_sel[0] = prefix | ((uint32_t)bsel << shift);
            sh_sel[1] = remaining - bef;
          }
        }
        __syncthreads();
        prefix = sh_sel[0];
        remaining = sh_sel[1];
        mask |= 255u << shift;
      }
      thr = prefix;
      need_eq = remaining;
    }
    // quota >= len: take every token
    const bool all = quota >= len;
    uint32_t n_gt = 0, n_eq = 0;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < KREG; ++i)
        if (i < cnt) {
          n_gt += (all || kreg[i] > thr) ? 1u : 0u;
          n_eq += (!all && kreg[i] == thr) ? 1u : 0u;
        }
    } else {
      for (int j = jlo; j < jhi; ++j) {
        const uint32_t u = key_at(j);
        n_gt += (all || u > thr) ? 1u : 0u;
        n_eq += (!all && u == thr) ? 1u : 0u;
      }
    }
    // exclusive block sums of both counts (threads in order); the ties taken before this thread
    // are the first need_eq of them, so its first slot is gt_before + min(need_eq, eq_before)
    const uint32_t gi = wave_incl_sum(n_gt), ei = wave_incl_sum(n_eq);
    if (lane == 63) { wsum[0][wave] = gi; wsum[1][wave] = ei; }
    __syncthreads();
    uint32_t gt_before = gi - n_gt, eq_before = ei - n_eq;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) { gt_before += wsum[0][w]; eq_before += wsum[1][w]; }
    uint32_t eq_rank = eq_before;
    uint32_t pos = gt_before + min(need_eq, eq_before);
    auto emit = [&](uint32_t u, int j) {
      bool take = all || u > thr;
      if (!all && u == thr) {
        take = eq_rank < need_eq;
        ++eq_rank;
      }
      if (take) {
        if (pos < (uint32_t)quota) out[off + pos] = mrow ? mrow[begin + j] : begin + j;
        ++pos;
      }
    };
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < KREG; ++i)
        if (i < cnt) emit(kreg[i], jlo + i);
    } else {
      for (int j = jlo; j < jhi; ++j) emit(key_at(j), j);
    }
  }
  if (wq) {
    for (int i = threadIdx.x; i < Lq; i += blockDim.x) out[R - Lq + i] = mrow ? mrow[Lctx + i] : Lctx + i;
  }
}

}  // namespace

hipError_t launch_select(const SelTab& tab, const unsigned long long* fx, int nparts, int Lctx, int Lq,
                         int sstride, const float* parts, float* scores, hipStream_t st, const int* map,
                         int map_stride, bool gather) {
  if (tab.n == 0) return hipSuccess;
  if (gather && !map) return hipErrorInvalidValue;
  const dim3 g(tab.n), b(kSelThreads);
  if (fx)
    k_select<kFromFixed><<<g, b, 0, st>>>(tab, fx, 0, Lctx, Lq, sstride, parts, scores, map, map_stride);
  else if (nparts > 0)
    k_select<kFromParts><<<g, b, 0, st>>>(tab, nullptr, nparts, Lctx, Lq, sstride, parts, scores, map, map_stride);
  else if (gather)
    k_select<kFromGather><<<g, b, 0, st>>>(tab, nullptr, 0, Lctx, Lq, sstride, parts, scores, map, map_stride);
  else
    k_select<kFromScores><<<g, b, 0, st>>>(tab, nullptr, 0, Lctx, Lq, sstride, parts, scores, map, map_stride);
  return hipGetLastError();
}

}  // namespace sra
