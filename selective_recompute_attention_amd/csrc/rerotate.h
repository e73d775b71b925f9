// S1 re-rotation of a run of cached chunk rows into the fused cache, shared by the standalone
// re-rotation kernel and by the critical-layer scoring pass, whose spare blocks carry it.
//
// S1 follows "full KV reuse after adjusting the position encoding" (CacheBlend problem definition
// page, §2.4): a chunk cached at original positions orig + t moves to fused rows n_c + t, so each
// key pair (x_i, x_{i+d/2}) turns by delta_c * theta_i with delta_c = n_c - orig.
#pragma once
#include <type_traits>

#include "common.h"

namespace sra {
namespace rerot {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec;  // 16-byte vector of T, unpacked to float
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(v4u v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(v[k] << 16);
      f[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
    }
  }
  __device__ static v4u pack(const float* f) {
    v4u v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = pack_bf2(f[2 * k], f[2 * k + 1]);
    return v;
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void unpack(v4u v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(v[k]);
  }
  __device__ static v4u pack(const float* f) {
    v4u v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __float_as_uint(f[k]);
    return v;
  }
};

// Rows [t0, t0 + nr) of chunk entry e (nr >= 1), all KV heads, by one block of 256 threads (every
// thread must call it). Each batch loads its V chunks and K pairs (16 bytes per half) before the
// angles are formed, so the memory latency overlaps the float64 sin/cos; V is stored as is and K
// rotated, its bits kept when delta = 0. cs is LDS scratch of d/2 float2. UV and UK are a thread's
// V chunks and K pair units per batch: small where many blocks share a CU, large where one block
// has a CU (more bytes in flight per round trip). With sh.kh set (bf16 storage), every stored K vector
// is also written as fp16 to the same place of sh.kh, and a key beyond fp16's range flags its
// (request, KV head).
template <typename T, int D, int UV = 4, int UK = 2>
__device__ __forceinline__ void rows(const ChunkTab& tab, int e, int t0, int nr, int Hkv,
                                     const T* __restrict__ ks, const T* __restrict__ vs,
                                     T* __restrict__ kf, T* __restrict__ vf, int64_t L,
                                     const Theta& th, float2* cs, const F16Shadow& sh = F16Shadow()) {
  constexpr int H = D / 2;
  constexpr int VW = Vec<T>::N;
  constexpr int UPH = H / VW;   // K pair units per head
  static_assert(H <= 256, "one frequency per thread");
  const int delta = tab.delta[e];
  const int64_t row_elems = (int64_t)Hkv * D;
  const int64_t src0 = ((int64_t)tab.src[e] + t0) * row_elems;
  const int64_t dst0 = ((int64_t)tab.req[e] * L + tab.dst[e] + t0) * row_elems;
  const int64_t nV = (int64_t)nr * row_elems * (int64_t)sizeof(T) / 16;   // V 16-byte chunks
  const int64_t nK = (int64_t)nr * Hkv * UPH;                             // K pair units
  const v4u* vsrc = reinterpret_cast<const v4u*>(vs + src0);
  v4u* vdst = reinterpret_cast<v4u*>(vf + dst0);
  // the thread's frequency (indexed, so a memory load) goes out before the data: loads complete in
  // order, so one issued after them would hold the angles back until all the data has arrived
  const double th_i = th.v[min((int)threadIdx.x, H - 1)];
  __builtin_amdgcn_sched_barrier(0);   // keep it ahead of the data loads
  // one batch: its loads, then (first batch only) the angles while they are in flight, then the
  // stores
  auto batch = [&](int64_t bv, int64_t bk, auto first_tag) {
    v4u v[UV], ka[UK], kb[UK];
#pragma unroll
    for (int i = 0; i < UV; ++i) v[i] = vsrc[min(bv + threadIdx.x + 256 * i, nV - 1)];
#pragma unroll
    for (int i = 0; i < UK; ++i) {
      const int64_t u = min(bk + threadIdx.x + 256 * i, nK - 1);
      const T* a = ks + src0 + (u / UPH) * D + (u % UPH) * VW;
      ka[i] = *reinterpret_cast<const v4u*>(a);
      kb[i] = *reinterpret_cast<const v4u*>(a + H);
    }
    if constexpr (decltype(first_tag)::value) {
      // every thread forms an angle and stores it (threads past d/2 repeat the last frequency
      // with the same value), so nothing here sits behind a branch that the compiler could move
      // the frequency load into
      cs[min((int)threadIdx.x, H - 1)] = rope_cs((double)delta, th_i);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < UV; ++i)
      if (bv + threadIdx.x + 256 * i < nV) vdst[bv + threadIdx.x + 256 * i] = v[i];
#pragma unroll
    for (int i = 0; i < UK; ++i) {
      const int64_t u = bk + threadIdx.x + 256 * i;
      if (u >= nK) continue;
      const int i0 = (int)(u % UPH) * VW;
      const int64_t off = dst0 + (u / UPH) * D + i0;
      T* o = kf + off;
      v4u wa = ka[i], wb = kb[i];
      if (delta != 0) {   // rotation by zero is the identity: keep the cached bits
        float fa[VW], fb[VW], ra[VW], rb[VW];
        Vec<T>::unpack(ka[i], fa);
        Vec<T>::unpack(kb[i], fb);
#pragma unroll
        for (int k = 0; k < VW; ++k) {
          const float c = cs[i0 + k].x, sn = cs[i0 + k].y;
          ra[k] = fa[k] * c - fb[k] * sn;
          rb[k] = fa[k] * sn + fb[k] * c;
        }
        wa = Vec<T>::pack(ra);
        wb = Vec<T>::pack(rb);
      }
      *reinterpret_cast<v4u*>(o) = wa;
      *reinterpret_cast<v4u*>(o + H) = wb;
      if constexpr (sizeof(T) == 2) {
        if (sh.kh) {
          float amax = 0.f;
          v4u ha, hb;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            ha[k] = bf2_to_h2(wa[k], amax);
            hb[k] = bf2_to_h2(wb[k], amax);
          }
          *reinterpret_cast<v4u*>(sh.kh + off) = ha;
          *reinterpret_cast<v4u*>(sh.kh + off + H) = hb;
          if (amax > kF16Max) sh.flags[(int64_t)tab.req[e] * Hkv + (int)(u / UPH) % Hkv] = sh.call_id;
        }
      }
    }
  };
  batch(0, 0, std::true_type{});   // nr >= 1: the first batch has work
  for (int64_t bv = 256 * UV, bk = 256 * UK; bv < nV || bk < nK; bv += 256 * UV, bk += 256 * UK)
    batch(bv, bk, std::false_type{});
}

}  // namespace rerot
}  // namespace sra
