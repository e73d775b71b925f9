// Top-N selection of context tokens by score (QCFuse technical summary (zh), §2.A: the Top-N
// context token indices from the critical-layer attention distribution; ties follow a stable
// sort by descending score, Cache-Craft CSDN article §2.2.2, so the lower index wins).
//
// One block of 1024 threads per selection unit (a whole request, or one chunk of a request when
// per-chunk quotas are given). The block first sums the per-KV-head partial column sums in a fixed
// order (the scores), then finds the score of the N-th best token exactly with a 4-pass 8-bit radix
// select over order-preserving 32-bit keys, and finally writes, in ascending position order,
// every token above that score plus the lowest-index tokens equal to it. All decisions are integer
// comparisons of the same float32 bits, so the result is deterministic.
#include "common.h"

namespace sra {
namespace {

constexpr int kSelLdsKeys = 12288;   // keys of one selection unit kept in LDS (48 KB)

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix count of `flag` over the block (1024 threads = 16 waves); also the total.
__device__ __forceinline__ int block_excl_count(bool flag, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int before = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) {
    const int c = wsum[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return off + before;
}

__global__ __launch_bounds__(1024) void k_select(SelTab tab, int nparts, int Lctx, int Lq, int R,
                                                 const float* __restrict__ parts,
                                                 float* __restrict__ scores,
                                                 int* __restrict__ row_pos) {
  __shared__ unsigned hist[256];
  __shared__ unsigned sh_prefix, sh_remaining;
  __shared__ int wsum[16];
  __shared__ uint32_t kl[kSelLdsKeys];   // the unit's keys when they fit
  const int e = blockIdx.x;
  const int req = tab.req[e], begin = tab.begin[e], len = tab.len[e];
  const int quota = tab.quota[e], off = tab.out_off[e];
  float* srow = scores + (int64_t)req * Lctx + begin;
  int* out = row_pos + (int64_t)req * R;
  const bool in_lds = len <= kSelLdsKeys;

  // scores: per-KV-head partial column sums added in head order (loads issued 8 at a time)
  const float* prow = parts + (int64_t)req * nparts * Lctx + begin;
  for (int j = threadIdx.x; j < len; j += blockDim.x) {
    float s = 0.f;
    if (nparts > 0) {
      int p = 0;
      for (; p + 8 <= nparts; p += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = prow[(int64_t)(p + u) * Lctx + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      for (; p < nparts; ++p) s += prow[(int64_t)p * Lctx + j];
      srow[j] = s;
    } else {
      s = srow[j];
    }
    if (in_lds) kl[j] = order_key(s);
  }
  __syncthreads();
  // every thread reads back only keys it wrote itself or keys in LDS after the barrier
  auto key_at = [&](int j) -> uint32_t { return in_lds ? kl[j] : order_key(srow[j]); };

  if (quota > 0) {
    uint32_t thr = 0, need_eq = 0;
    if (quota < len) {
      uint32_t prefix = 0, mask = 0, remaining = (uint32_t)quota;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (threadIdx.x < 256) hist[threadIdx.x] = 0;
        __syncthreads();
        for (int j = threadIdx.x; j < len; j += blockDim.x) {
          const uint32_t u = key_at(j);
          if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
          // one wave scans the 256 bins from the top: lane l holds bins 255-4l .. 252-4l
          const int lane = threadIdx.x;
          uint32_t c[4], tot = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            c[i] = hist[255 - 4 * lane - i];
            tot += c[i];
          }
          uint32_t incl = tot;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const uint32_t o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
          }
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
          const int b = __shfl(found, first, 64);
          const uint32_t bef = __shfl(before, first, 64);
          if (lane == 0) {
            sh_prefix = prefix | ((uint32_t)b << shift);
            sh_remaining = remaining - bef;
          }
        }
        __syncthreads();
        prefix = sh_prefix;
        remaining = sh_remaining;
        mask |= 255u << shift;
        __syncthreads();
      }
      thr = prefix;
      need_eq = remaining;
    }
    // quota >= len: thr = 0 and need_eq = 0 take every token (all keys of real scores exceed 0)
    int run_eq = 0, run_sel = 0;
    for (int base = 0; base < len; base += blockDim.x) {
      const int j = base + threadIdx.x;
      const bool valid = j < len;
      const uint32_t u = valid ? key_at(j) : 0u;
      const bool gt = valid && (quota >= len || u > thr);
      const bool eq = valid && quota < len && u == thr;
      int tot_eq, tot_sel;
      const int eq_rank = run_eq + block_excl_count(eq, wsum, tot_eq);
      const bool take = gt || (eq && (uint32_t)eq_rank < need_eq);
      const int pos = run_sel + block_excl_count(take, wsum, tot_sel);
      if (take && pos < quota) out[off + pos] = begin + j;
      run_eq += tot_eq;
      run_sel += tot_sel;
    }
  }
  if (tab.writes_query[e]) {
    for (int i = threadIdx.x; i < Lq; i += blockDim.x) out[R - Lq + i] = Lctx + i;
  }
}

}  // namespace

hipError_t launch_select(const SelTab& tab, int nparts, int Lctx, int Lq, int R, const float* parts,
                         float* scores, int* row_pos, hipStream_t st) {
  if (tab.n == 0) return hipSuccess;
  k_select<<<dim3(tab.n), dim3(1024), 0, st>>>(tab, nparts, Lctx, Lq, R, parts, scores, row_pos);
  return hipGetLastError();
}

}  // namespace sra
