// Top-N selection of context tokens by score (QCFuse technical summary (zh), §2.A: the Top-N
// context token indices from the critical-layer attention distribution; ties follow a stable
// sort by descending score, Cache-Craft CSDN article §2.2.2, so the lower index wins).
//
// One block of 256 threads per selection unit (a whole request, or one chunk of a request when
// per-chunk quotas are given). The block first forms the scores (fixed-point totals over KV heads,
// or per-head float partials added in a fixed order), then finds the score of the N-th best token exactly with an 8-bit radix
// select over order-preserving 32-bit keys (leading bytes shared by every key are skipped), and
// finally writes, in ascending position order, every token above that score plus the lowest-index
// tokens equal to it. All decisions are integer comparisons of the same float32 bits, so the result
// is deterministic.
#include "common.h"

namespace sra {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelLdsKeys = 12288;   // keys of one selection unit kept in LDS (48 KB)

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of x over the block (4 waves, in thread order); also the total.
__device__ __forceinline__ int block_excl_sum(int x, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = (int)wave_incl_sum((uint32_t)x);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int c = wsum[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + incl - x;
}

__global__ __launch_bounds__(kSelThreads) void k_select(SelTab tab, const unsigned long long* __restrict__ fx,
                                                        int nparts, int Lctx, int Lq, int R,
                                                        const float* __restrict__ parts,
                                                        float* __restrict__ scores,
                                                        int* __restrict__ row_pos,
                                                        const int* __restrict__ map, int map_stride) {
  constexpr int NW = kSelThreads / 64;
  constexpr int KREG = 16;   // keys per thread held in registers (units up to 4096 keys)
  constexpr int kSub = 4;
  __shared__ unsigned hist[4][NW][256 * kSub];   // per radix pass and wave: kSub copies of each bin
  __shared__ uint32_t sh_prefix, sh_remaining;
  __shared__ uint32_t sh_and[NW], sh_or[NW];
  __shared__ int wsum[NW];
  __shared__ uint32_t kl[kSelLdsKeys];   // larger units' keys when they fit
  const int e = blockIdx.x;
  const int req = tab.req[e], begin = tab.begin[e], len = tab.len[e];
  const int quota = tab.quota[e], off = tab.out_off[e];
  float* srow = scores + (int64_t)req * Lctx + begin;
  int* out = row_pos + (int64_t)req * R;
  const int* mrow = map ? map + (int64_t)req * map_stride : nullptr;   // index -> written value
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // thread t owns the contiguous positions [jlo, jhi): block prefix sums of per-thread counts then
  // give ascending output slots
  const int per = (len + kSelThreads - 1) / kSelThreads;
  const int jlo = min((int)threadIdx.x * per, len), jhi = min(jlo + per, len), cnt = jhi - jlo;
  const bool in_regs = len > 0 && per <= KREG;
  const bool in_lds = len <= kSelLdsKeys;
  for (int i = threadIdx.x; i < 4 * NW * 256 * kSub; i += kSelThreads) (&hist[0][0][0])[i] = 0;

  // scores: per-KV-head partial column sums added in head order, then order-preserving keys. The
  // loads are coalesced (position j = tid + 256 i); small units then pass their keys through LDS
  // into this thread's contiguous range of registers.
  const float* prow = parts + (int64_t)req * nparts * Lctx + begin;
  uint32_t kreg[KREG];
  uint32_t kand = ~0u, kor = 0u;
  if (in_regs) {
    float sv[KREG];
    if (fx) {
      const unsigned long long* frow = fx + (int64_t)req * Lctx + begin;
      unsigned long long fv[KREG];   // one batch of independent loads
#pragma unroll
      for (int i = 0; i < KREG; ++i) fv[i] = frow[min((int)threadIdx.x + kSelThreads * i, len - 1)];
#pragma unroll
      for (int i = 0; i < KREG; ++i) sv[i] = (float)((double)fv[i] * (1.0 / kScoreFixScale));
    } else if (nparts > 0) {
#pragma unroll
      for (int i = 0; i < KREG; ++i) sv[i] = 0.f;
      for (int p0 = 0; p0 < nparts; p0 += 8) {
        float v[KREG][8];   // clamped, unconditional loads: the whole batch is in flight at once
#pragma unroll
        for (int i = 0; i < KREG; ++i)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[i][u] = (i < per) ? prow[(int64_t)min(p0 + u, nparts - 1) * Lctx +
                                       min((int)threadIdx.x + kSelThreads * i, len - 1)] : 0.f;
#pragma unroll
        for (int i = 0; i < KREG; ++i)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (p0 + u < nparts) sv[i] += v[i][u];
      }
    } else {
#pragma unroll
      for (int i = 0; i < KREG; ++i)
        sv[i] = (i < per) ? srow[min((int)threadIdx.x + kSelThreads * i, len - 1)] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < KREG; ++i) {
      const int j = threadIdx.x + kSelThreads * i;
      if (i < per && j < len) {
        if (fx || nparts > 0) srow[j] = sv[i];
        kl[j] = order_key(sv[i]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KREG; ++i) {
      kreg[i] = kl[min(jlo + i, len - 1)];
      if (i < cnt) {
        kand &= kreg[i];
        kor |= kreg[i];
      }
    }
  } else {
    for (int i = 0; i < per; ++i) {
      const int j = threadIdx.x + kSelThreads * i;
      if (j >= len) break;
      float sv = 0.f;
      if (fx) {
        sv = (float)((double)fx[(int64_t)req * Lctx + begin + j] * (1.0 / kScoreFixScale));
        srow[j] = sv;
      } else if (nparts > 0) {
        for (int p0 = 0; p0 < nparts; p0 += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = prow[(int64_t)min(p0 + u, nparts - 1) * Lctx + j];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (p0 + u < nparts) sv += v[u];
        }
        srow[j] = sv;
      } else {
        sv = srow[j];
      }
      const uint32_t u = order_key(sv);
      if (in_lds) kl[j] = u;
      kand &= u;
      kor |= u;
    }
  }
  // bits shared by every key of the unit
  kand = wave_reduce(kand, [](uint32_t a, uint32_t b) { return a & b; });
  kor = wave_reduce(kor, [](uint32_t a, uint32_t b) { return a | b; });
  if (lane == 0) { sh_and[wave] = kand; sh_or[wave] = kor; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) { kand &= sh_and[w]; kor |= sh_or[w]; }
  // keys are read back after the barrier below (LDS, or global writes of this block)
  auto key_at = [&](int j) -> uint32_t { return in_lds ? kl[j] : order_key(srow[j]); };

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
        unsigned* h = &hist[shift >> 3][wave][0];
        // each bin has kSub copies, chosen by lane: lanes of one wave that hit the same bin (the
        // leading bytes of the scores take few values) spread over kSub addresses
        auto count = [&](uint32_t u, bool valid) {
          if (valid && (u & mask) == prefix) atomicAdd(&h[((u >> shift) & 255u) * kSub + (lane & (kSub - 1))], 1u);
        };
        if (in_regs) {
#pragma unroll
          for (int i = 0; i < KREG; ++i)
            if (i < per) count(kreg[i], i < cnt);
        } else {
          for (int i = 0; i < per; ++i) count(key_at(min(jlo + i, len - 1)), i < cnt);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
          // one wave scans the 256 bins from the top: lane l holds bins 255-4l .. 252-4l
          uint32_t c[4], tot = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int bin = 255 - 4 * lane - i;
            uint32_t cc = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
              for (int sb = 0; sb < kSub; ++sb) cc += hist[shift >> 3][w][bin * kSub + sb];
            c[i] = cc;
            tot += cc;
          }
          const uint32_t incl = wave_incl_sum(tot);
          uint32_t cum = incl - tot, before = 0;
          int found = -1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (found < 0 && cum + c[i] >= remaining) {
              found = 255 - 4 * lane - i;
              before = cum;
            }
            cum += c[i];
          }
          // the lowest lane with a hit holds the highest qualifying bin
          const int first = __ffsll((unsigned long long)__ballot(found >= 0)) - 1;
          const int bsel = __builtin_amdgcn_readlane(found, first);
          const uint32_t bef = __builtin_amdgcn_readlane(before, first);
          if (lane == 0) {
            sh_prefix = prefix | ((uint32_t)bsel << shift);
            sh_remaining = remaining - bef;
          }
        }
        __syncthreads();
        prefix = sh_prefix;
        remaining = sh_remaining;
        mask |= 255u << shift;
      }
      thr = prefix;
      need_eq = remaining;
    }
    // quota >= len: take every token
    const bool all = quota >= len;
    int n_gt = 0, n_eq = 0;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < KREG; ++i)
        if (i < cnt) {
          n_gt += (all || kreg[i] > thr) ? 1 : 0;
          n_eq += (!all && kreg[i] == thr) ? 1 : 0;
        }
    } else {
      for (int j = jlo; j < jhi; ++j) {
        const uint32_t u = key_at(j);
        n_gt += (all || u > thr) ? 1 : 0;
        n_eq += (!all && u == thr) ? 1 : 0;
      }
    }
    int tot;
    int eq_rank = block_excl_sum(n_eq, wsum, tot);
    const int eq_take = max(0, min(n_eq, (int)need_eq - eq_rank));   // the lowest-index ties win
    int pos = block_excl_sum(n_gt + eq_take, wsum, tot);
    auto emit = [&](uint32_t u, int j) {
      bool take = all || u > thr;
      if (!all && u == thr) {
        take = (uint32_t)eq_rank < need_eq;
        ++eq_rank;
      }
      if (take) {
        if (pos < quota) out[off + pos] = mrow ? mrow[begin + j] : begin + j;
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
  if (tab.writes_query[e]) {
    for (int i = threadIdx.x; i < Lq; i += blockDim.x) out[R - Lq + i] = mrow ? mrow[Lctx + i] : Lctx + i;
  }
}

}  // namespace

hipError_t launch_select(const SelTab& tab, const unsigned long long* fx, int nparts, int Lctx, int Lq,
                         int R, const float* parts, float* scores, int* row_pos, hipStream_t st,
                         const int* map, int map_stride) {
  if (tab.n == 0) return hipSuccess;
  k_select<<<dim3(tab.n), dim3(kSelThreads), 0, st>>>(tab, fx, nparts, Lctx, Lq, R, parts, scores, row_pos,
                                                      map, map_stride);
  return hipGetLastError();
}

}  // namespace sra
