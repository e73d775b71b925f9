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
//   * Persistent work groups: a fixed grid of work groups per group (two per compute unit in total).
//     Where a group has several tiles per work group, its work groups take whole tiles from the
//     group's queue, largest first, and write each one directly. Otherwise each work group computes
//     the tiles' unit counts from row_pos, takes a contiguous unit range (shares weighted by dispatch
//     order) and walks it tile by tile: a tile it covers whole is written directly, a cut tile leaves
//     a partial (O as fp16 scaled by the vector's largest |O|, max, sum) in one of two slots (first /
//     last tile of the range) and the merge kernel combines the pieces of such tiles in key order.
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
//     kSumCap = 2^16 (some logit more than 16 above the reference, log2 domain) does the reference move, with
//     the accumulator rescaled: no per-block maximum or subtraction in the common case.
//   * Software pipeline in steps of 32 keys, the same in every wave: step j issues the products of
//     S_{j+1} on the matrix cores interleaved with the exponentials of S_j on the vector units, then
//     O += V_j^T P_j. Register use allows two waves per SIMD, which fill each other's stalls.
//   * K and V tiles go straight from global memory into four-slot LDS rings (direct loads, no
//     registers), issued three steps ahead; an explicit count of outstanding loads and one LDS-only
//     barrier per step publish a tile, so later loads stay in flight across the barrier. K slots are
//     [16-row block][chunk][row % 16] (each S operand read is a lane base plus a constant and hits 16
//     consecutive slots); V slots are row-major with chunks swizzled by key, and each P V operand is
//     two transposing LDS reads (ds_read_b64_tr_b16) whose key order matches the probabilities'.
//   * Work groups are numbered with the group index fastest, so all work of one KV head lands on one
//     XCD (work groups are dealt round-robin over the 8 XCDs) and its K/V stay in that XCD's L2.
// f32 path: plain float32 arithmetic, one block per (row, KV head), exact online softmax.
#include <float.h>

#include <type_traits>

#include "common.h"

namespace sra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kSumCap = 65536.f;     // 2^16: a 32-key block sum above it moves the softmax reference

struct AttnArgs {
  const uint16_t* qop;
  const int* row_pos;
  const uint16_t* kh;     // fp16 copy of the fused keys
  const uint16_t* kf;     // bf16 fused keys (exact recomputation of flagged groups)
  const uint16_t* vf;
  uint16_t* out;
  float* lse;
  int* tilecum;
  int4* merge;      // [n_groups][pieces]: the cut tile a piece merges (its first, when it is the last piece
                    // over it) as (tile, first piece over it, number of pieces, slot of the first piece's
                    // partial), or tile -1
  uint16_t* part_o;   // fp16, scaled per vector
  float4* part_ml;    // (max, sum, scale, 0) per vector
  const uint16_t* qx;       // fresh queries before rotation (exact recomputation)
  const unsigned* flags;    // [n_groups]: call_id where an fp16 operand overflowed
  int* fallback;            // optional [n_groups] report
  unsigned call_id;
  int q_rows, q_indexed;
  int n_req, Hq, Hkv, g, R, L;
  int n_groups, n_tiles, qop_blocks, pieces;
  int dynamic;      // whole tiles from each group's queue (largest first) instead of the static split
  int* queue;       // [n_groups] next item of each group's queue (dynamic), zeroed before the launch
  int comb_idx;     // index range of the merge kernel's grid (its exact path strides by it)
  Theta th;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Wait until at most N vector memory operations of this wave are outstanding (s_waitcnt with the
// export and LDS counters left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Work-group barrier that waits for this wave's LDS operations only. Tiles that direct loads write into
// LDS are published by an explicit vmcnt wait before it, so loads of later tiles stay in flight across
// the barrier (a __syncthreads() fence would wait for all of them). The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// float pair -> two fp16 (round to nearest even) in one word, and back
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ __forceinline__ float h2f(uint32_t h16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h16); }

__device__ __forceinline__ int64_t part_index(const AttnArgs& a, int group, int piece, int slot) {
  return ((int64_t)(group * a.pieces + piece) * 2 + slot) * 128;
}

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

// Tile-local row and 16-byte chunk (as a byte offset) that lane `lane` of direct load instruction n
// brings into an LDS ring slot (instruction n fills the slot's n-th kilobyte, lane l at byte 16 l).
// K slots are [16-row block][chunk][row % 16]; V slots are row-major with chunk c of row k at slot
// c ^ ((k % (D / 32)) << 2).
template <int D>
__device__ __forceinline__ int ring_k_row(int n, int lane) { return 16 * (n / (D / 32)) + (lane & 15); }
template <int D>
__device__ __forceinline__ uint32_t ring_k_chunk(int n, int lane) {
  return 16u * (uint32_t)(4 * (n % (D / 32)) + (lane >> 4));
}
template <int D>
__device__ __forceinline__ int ring_v_row(int n, int lane) { return (512 / D) * n + lane / (D / 8); }
template <int D>
__device__ __forceinline__ uint32_t ring_v_chunk(int n, int lane) {
  return 16u * ((uint32_t)(lane % (D / 8)) ^ ((uint32_t)(ring_v_row<D>(n, lane) % (D / 32)) << 2));
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_mfma(AttnArgs a) {
  constexpr int NKS = D / 16;   // K-steps of S^T = K Q^T
  constexpr int NDT = D / 32;   // 32-row d tiles of O^T
  constexpr int KT = 64;              // keys per work unit (the granularity of the split)
  constexpr int ST = 32;              // keys per pipeline step
  constexpr int CPR = D / 8;          // 16-byte chunks per key row
  constexpr int RB = D * 2;           // bytes per key row in LDS (rows unpadded, chunks swizzled)
  constexpr int TB = ST * RB;         // bytes per step tile
  constexpr int RPI = 64 / CPR;       // rows per direct load instruction (64 lanes x 16 bytes)
  constexpr int NIW = ST / RPI / 4;   // direct load instructions per wave per tile
  static_assert(NIW >= 1 && NIW * 4 * RPI == ST, "a step tile splits evenly over the four waves");
  // four-deep rings of step tiles, filled straight from global memory (one array per slot)
  __shared__ __attribute__((aligned(1024))) unsigned char K0s[TB], K1s[TB], K2s[TB], K3s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char V0s[TB], V1s[TB], V2s[TB], V3s[TB];
  unsigned char* const Kring[4] = {K0s, K1s, K2s, K3s};
  unsigned char* const Vring[4] = {V0s, V1s, V2s, V3s};
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
  if (kvh == 0 && piece == 0)
    for (int t = threadIdx.x; t <= nt; t += 256) a.tilecum[(int64_t)req * (nt + 1) + t] = cum[t];
  // Static split: this piece's unit range [u0, u1) and the tile holding u0. Dynamic: every work
  // group of the group takes whole tiles, largest first (item k is tile nt - 1 - k, tiles grow with
  // their last position): item `piece` first, then items pieces, pieces + 1, ... from the group's
  // queue until it is empty; a work group that finishes a tile early takes the next one, so uneven
  // speeds of the work groups even out.
  const bool dyn = a.dynamic != 0;
  __shared__ int s_item;
  int u0 = 0, u1 = 0, t = 0, item = 0, item_next = 0;
  int* queue = a.queue + group;
  if (dyn) {
    item = piece;
  } else {
    const AttnSplit sp = attn_split(U, a.pieces, group, a.n_groups);
    int4* merge = a.merge + (int64_t)group * a.pieces + piece;
    if (piece >= sp.P) {
      if (threadIdx.x == 0) *merge = make_int4(-1, 0, 0, 0);
      return;
    }
    u0 = attn_piece_start(sp, piece);
    u1 = attn_piece_start(sp, piece + 1);
    {   // last tile with cum[t] <= u0: the tile holding unit u0
      int hi = nt - 1;
      while (t < hi) {
        const int mid = (t + hi + 1) >> 1;
        if (cum[mid] <= u0) t = mid;
        else hi = mid - 1;
      }
    }
    // a piece that starts inside its first tile and reaches that tile's end is the last of the
    // pieces over it: it is the one whose merge work group combines the tile's partials. The pieces
    // over the tile run from the one holding its first unit to this one; the first piece's partial
    // of the tile is in slot 1 unless the tile is also where that piece starts.
    if (threadIdx.x == 0) {
      int4 rec = make_int4(-1, 0, 0, 0);
      if (u0 > cum[t] && u1 >= cum[t + 1]) {
        const int i0 = attn_piece_of(sp, cum[t]);
        rec = make_int4(t, i0, piece - i0 + 1, attn_piece_start(sp, i0) < cum[t] ? 1 : 0);
      }
      *merge = rec;
    }
  }

  // uniform base of this (request, KV head); per-thread byte offsets fit 32 bits (checked by the host)
  const char* kbase = reinterpret_cast<const char*>(a.kh + ((int64_t)req * a.L * a.Hkv + kvh) * D);
  const char* vbase = reinterpret_cast<const char*>(a.vf + ((int64_t)req * a.L * a.Hkv + kvh) * D);
  const uint32_t row_bytes = (uint32_t)(a.Hkv * D * 2);
  // Tiles move straight from global memory into the LDS rings (16 bytes per lane, no registers), a
  // four-tile ring each for K and V; direct load instruction n of a tile fills its n-th kilobyte (lane l
  // at byte 16 l).
  //  * K: [16-row block][chunk][row % 16], 16 bytes each. Instruction n holds row block n / (CPR / 4) and
  //    chunks 4 (n % (CPR / 4)) .. + 3 (lane l: row 16 block + l % 16, chunk 4 (n % (CPR / 4)) + l / 16).
  //    The S operand read of lane (l32, hh), row l32 and chunk 2 ks + hh, is a lane base plus 512 ks,
  //    and any 16 lanes read 16 consecutive slots.
  //  * V: row-major (instruction n: rows RPI n .., lane l: row RPI n + l / CPR), 16-byte chunk c of row k
  //    at slot c ^ ((k % NDT) << 2): the transposing P V operand reads of any 32 lanes hit distinct
  //    8-byte bank pairs, and the key block stays a compile-time offset.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t kvo[NIW], vvo[NIW];     // byte offsets of the lane's loads from the tile's first row
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    kvo[i] = (uint32_t)ring_k_row<D>(NIW * wv + i, lane) * row_bytes + ring_k_chunk<D>(NIW * wv + i, lane);
    vvo[i] = (uint32_t)ring_v_row<D>(NIW * wv + i, lane) * row_bytes + ring_v_chunk<D>(NIW * wv + i, lane);
  }
  // operand read offsets: S (row l32, chunk 2 ks + hh: + 512 ks) and the transposing V reads (lane as
  // address source: key 4 hh + (l32 % 16) / 4 of an 8-key block, dims 32 dt + 16 (l32 / 16) + 4 (l32 % 4))
  const uint32_t kofs = (uint32_t)((l32 >> 4) * (CPR * 256) + hh * 256 + (l32 & 15) * 16);
  uint32_t vofs[NDT];
  {
    const uint32_t kl = 4 * hh + ((l32 & 15) >> 2), c01 = 2 * (l32 >> 4) + ((l32 & 3) >> 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      vofs[dt] = kl * RB + 16u * (4u * ((uint32_t)dt ^ ((uint32_t)(l32 >> 2) & (NDT - 1))) + c01) + 8u * (l32 & 1);
  }
  // buffer resources over this (request, KV head)'s rows: row r at byte r * row_bytes
  const int nrec = (int)((uint32_t)(a.L - 1) * row_bytes + RB);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase), (short)0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase), (short)0, nrec, 0x00020000);

  int slot = 0;
  for (;;) {   // items of the queue (dynamic), or the one static range
  if (dyn) {
    if (item >= nt) break;
    t = nt - 1 - item;
    u0 = cum[t];
    u1 = cum[t + 1];
    // the next item is claimed now (one vector memory operation ahead of this tile's loads: the
    // tile waits count it among the older ones, so they only get stricter)
    if (threadIdx.x == 0)
      item_next = a.pieces + __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  for (int u = u0; u < u1; ++t) {
    const int c0 = cum[t], c1 = cum[t + 1];
    const int se = min(u1, c1);
    if (se <= u) continue;  // tile without keys
    const bool direct = (u == c0 && se == c1);
    // keys stop at the tile's last position: rows past it are never read
    const int maxkey = min(rp[min(t * 128 + 127, Mv - 1) / g], a.L - 1);
    const int kbeg = KT * (u - c0), kend = min(KT * (se - c0), maxkey + 1);   // kbeg < kend
    const int nst = (kend - kbeg + ST - 1) / ST;   // pipeline steps

    // Step tile x of the segment into ring slot b. In a tile that reaches past the range, rows repeat
    // row kend - 1, whose keys the mask removes (probability 0 on finite values).
    auto issue = [&](__amdgpu_buffer_rsrc_t rs, unsigned char* ring, const uint32_t* vo, bool is_v, int x) {
      int rl[NIW];   // tile-local rows of the lane's loads
#pragma unroll
      for (int i = 0; i < NIW; ++i) rl[i] = is_v ? ring_v_row<D>(NIW * wv + i, lane) : ring_k_row<D>(NIW * wv + i, lane);
      const int kt = kbeg + ST * x;
      typedef __attribute__((address_space(3))) void lds_t;
      // the destination is laundered through an empty asm: the compiler then does not tie the load to
      // the slot's array and adds no wait of its own before reads of it (the waits here are explicit)
      __attribute__((address_space(3))) unsigned char* dst = (__attribute__((address_space(3))) unsigned char*)ring;
      asm volatile("" : "+s"(dst));
      if (kt + ST <= kend) {
#pragma unroll
        for (int i = 0; i < NIW; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (lds_t*)(dst + 1024 * (NIW * wv + i)), 16, vo[i],
              kt * (int)row_bytes, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < NIW; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (lds_t*)(dst + 1024 * (NIW * wv + i)), 16,
              vo[i] + (uint32_t)(min(kt + rl[i], kend - 1) - rl[i]) * row_bytes, 0, 0, 0);
      }
    };
    auto issue_k = [&](int x, int b) { issue(rk, Kring[b], kvo, false, x); };
    auto issue_v = [&](int x, int b) { issue(rv, Vring[b], vvo, true, x); };

    // query operand and the first tiles' loads go out before the first wait
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
    const int r = min(v, Mv - 1) / g;
    const int hq = kvh * g + v % g;
    const int p_r = rp[r];
    // K_0, K_1, V_0 first; then what the steps -2 and -1 would have issued (K_2, V_1 and K_3, V_2). All
    // ring slots are free: the previous segment ended with a barrier. (The loads above are issued first:
    // a wait for them then does not wait for the tiles.)
    issue_k(0, 0);
    issue_k(1, 1);
    issue_v(0, 0);
    issue_k(2, 2);
    issue_v(1, 1);
    issue_k(3, 3);
    issue_v(2, 2);
    const bool qvalid = v < Mv && p_r >= 0;  // negative positions are skipped
    const int pq = qvalid ? min(p_r, a.L - 1) : -1;
    if (!qvalid) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) q16[ks] = __builtin_bit_cast(f16x8, u32x4{0u, 0u, 0u, 0u});
    }
    // smallest position among this wave's query vectors: steps entirely at or below it need no mask
    const int pmin = (int)wave_reduce(qvalid ? (uint32_t)pq : (uint32_t)INT_MAX,
                                      [](uint32_t x, uint32_t y) { return x < y ? x : y; });

    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
    float m_ref = 0.f, l_run = 0.f;   // softmax reference (log2 domain) and running sum
    f32x16 negm;                      // -m_ref in every element: the S accumulator's start value

    // causal mask by absolute position where step j reaches past the wave's smallest position or the
    // range's end: element rr holds key kbeg + 32 j + 4 hh + 8 (rr / 4) + rr % 4
    auto mask = [&](int j, f32x16& x) {
      const int kt = kbeg + ST * j;
      if (!(kt + ST - 1 < kend && kt + ST - 1 <= pmin)) {
        const int lim = min(kend - 1, pq) - (kt + 4 * hh);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (8 * (rr >> 2) + (rr & 3) > lim) x[rr] = -INFINITY;
      }
    };
    auto s_prod = [&](const unsigned char* Kc, f32x16& acc, bool from_ref) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const f16x8 ka = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(Kc + kofs + 512 * ks));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, q16[ks], ks == 0 ? (from_ref ? negm : f32x16{}) : acc, 0, 0, 0);
      }
    };

    // K_0, K_1 and V_0 have landed (their loads are followed by eight per wave at most); S_0 gives the
    // reference
    wait_vmcnt<4 * NIW>();
    lds_barrier();
    f32x16 sA, sB;
    s_prod(Kring[0], sA, false);
    mask(0, sA);
    {
      float mt = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, sA[rr]);
      mt = half_max(mt);
      m_ref = mt == -INFINITY ? 0.f : mt;   // no visible key in the segment: stays 0
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        sA[rr] -= m_ref;
        negm[rr] = -m_ref;
      }
    }
    lds_barrier();   // K_0's slot takes K_4 in the first step

    // Step j (ring slot B = j % 4), with S_j complete in sa (relative to the reference): K_{j+4} and
    // V_{j+3} go out into the slots of K_j and V_{j-1} (both retired by the previous step's barrier);
    // the matrix cores form S_{j+1} from K_{j+1} into sb while the vector units turn S_j into
    // probabilities; O += V_j^T P_j; then K_{j+2} and V_{j+1} (issued two steps back) are waited for
    // and one barrier publishes them.
    auto step = [&](auto b_tag, const int j, f32x16& sa, f32x16& sb, auto more_tag) {
      constexpr int B = decltype(b_tag)::value;
      constexpr bool MORE = decltype(more_tag)::value;   // S_{j+1} exists
      if constexpr (MORE) {
        issue_k(j + 4, B);
        issue_v(j + 3, (B + 3) & 3);
      }
      mask(j, sa);
      u32x4 pw[2];
      float lsum;
      if constexpr (MORE) s_prod(Kring[(B + 1) & 3], sb, true);
      probs(sa, pw, lsum);
      if (__any(lsum > kSumCap)) {   // a logit more than 16 above the reference: move it
        float mt = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, sa[rr]);
        mt = half_max(mt);
        const float sh = mt > 0.f ? mt : 0.f;
        const float alpha = fast_exp2(-sh);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        l_run *= alpha;
        m_ref += sh;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          sa[rr] -= sh;
          negm[rr] = -m_ref;
        }
        if constexpr (MORE) {   // S_{j+1} started from the old reference
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) sb[rr] -= sh;
        }
        probs(sa, pw, lsum);
      }
      l_run += lsum;
      // O^T[d][q] += V^T[d][key] P^T[key][q]; hardware k = 8*hh + s <-> key 16mp + 8(s/4) + 4hh + s%4.
      // Each operand is two transposing reads of four keys.
      typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
      const __attribute__((address_space(3))) unsigned char* Vc = (const __attribute__((address_space(3))) unsigned char*)Vring[B];
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {
        const bf16x8 pb = as_bf16x8(pw[mp]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Vc + vofs[dt] + (16 * mp) * RB));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Vc + vofs[dt] + (16 * mp + 8) * RB));
          const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dt], 0, 0, 0);
        }
      }
      if constexpr (MORE) wait_vmcnt<4 * NIW>();
      lds_barrier();
    };
    typedef std::integral_constant<int, 0> B0;
    typedef std::integral_constant<int, 1> B1;
    typedef std::integral_constant<int, 2> B2;
    typedef std::integral_constant<int, 3> B3;
    int j = 0;
    for (; j + 4 < nst; j += 4) {   // four steps with a successor each
      step(B0{}, j, sA, sB, std::true_type{});
      step(B1{}, j + 1, sB, sA, std::true_type{});
      step(B2{}, j + 2, sA, sB, std::true_type{});
      step(B3{}, j + 3, sB, sA, std::true_type{});
    }
    // the last one to four steps (j % 4 == 0)
    if (j + 1 < nst) {
      step(B0{}, j, sA, sB, std::true_type{});
      if (j + 2 < nst) {
        step(B1{}, j + 1, sB, sA, std::true_type{});
        if (j + 3 < nst) {
          step(B2{}, j + 2, sA, sB, std::true_type{});
          step(B3{}, j + 3, sB, sA, std::false_type{});
        } else {
          step(B2{}, j + 2, sA, sB, std::false_type{});
        }
      } else {
        step(B1{}, j + 1, sB, sA, std::false_type{});
      }
    } else {
      step(B0{}, j, sA, sB, std::false_type{});
    }
    // loads of tiles past the segment may still be landing in the rings: none outlives the segment
    wait_vmcnt<0>();

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
  if (!dyn) break;
  if (threadIdx.x == 0) s_item = item_next;
  __syncthreads();
  item = s_item;
  }
}

// Empties the groups' queues before a dynamic launch (system-scope stores: the queue is taken with
// system-scope atomics, which work past the XCDs' caches)
__global__ __launch_bounds__(64) void k_attn_queue_reset(int* q, int n) {
  for (int i = threadIdx.x; i < n; i += 64) __hip_atomic_store(q + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
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

// Merge the pieces of every cut tile in key order. One work group per (group, index, slab of query
// vectors), the index running over the group's tiles when a group has fewer tiles than pieces, else
// over its pieces: piece i then merges the cut tile of the record the attention kernel wrote for it
// (the tile it is the last piece over, with the range of pieces over it), and the work groups of
// pieces without one exit after a single load. One thread per (query vector, 8 dims); the pieces'
// loads go out in independent batches of four. A group whose fp16 operands overflowed is recomputed
// exactly here instead: work group (index, slab) takes that slab of the group's tiles index,
// index + stride, ... (stride: the index range).
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  constexpr int TPV = D / 8;                 // threads per query vector
  constexpr int VPB = 256 / TPV;             // query vectors per work group
  constexpr int NSLAB = 128 / VPB;           // slabs per tile
  constexpr int B = 4;                       // pieces per batch of loads
  static_assert(B == 4, "the batch's keep-alive below lists four pieces");
  const int slab = blockIdx.x % NSLAB;
  const int gi = blockIdx.x / NSLAB;         // group-fastest (group, index) index
  const int group = gi % a.n_groups, idx = gi / a.n_groups;
  const int req = group / a.Hkv, kvh = group % a.Hkv;
  const int nt = a.n_tiles;
  const bool by_tile = nt <= a.pieces;
  // the merge record (by piece) and the group's flag as one batch of loads
  int4 rec = by_tile ? make_int4(idx, 0, 0, 0) : a.merge[(int64_t)group * a.pieces + idx];
  unsigned fl = a.flags[group];
  asm volatile("" : "+s"(rec.x), "+s"(rec.y), "+s"(rec.z), "+s"(rec.w), "+s"(fl)
               : "s"(a.row_pos), "s"(a.part_ml), "s"(a.part_o));
  const bool exact = fl == a.call_id;
  if (idx == 0 && slab == 0 && threadIdx.x == 0 && a.fallback) a.fallback[group] = exact ? 1 : 0;
  const int g = a.g, Mv = a.R * g;
  if (exact) {
    constexpr int VPE = 256 / (D / 4);   // vectors per pass of exact_vector (4 dims per thread)
    const int stride = a.comb_idx;
    for (int t = idx; t < nt; t += stride)
      for (int sub = 0; sub < VPB / VPE; ++sub) {
        const int v = t * 128 + slab * VPB + sub * VPE + (int)threadIdx.x / (D / 4);
        if (v < Mv) exact_vector<D>(a, req, kvh, v);
      }
    return;
  }
  if (a.dynamic) return;   // every tile was written whole by one work group
  int tile = rec.x, i0 = rec.y, n = rec.z, slot0 = rec.w;
  if (by_tile) {   // the tile's unit range and the request's total give its pieces
    const int* cum = a.tilecum + (int64_t)req * (nt + 1);
    const int c0 = cum[tile], c1 = cum[tile + 1], U = cum[nt];
    if (c1 <= c0) return;
    const AttnSplit sp = attn_split(U, a.pieces, group, a.n_groups);
    i0 = attn_piece_of(sp, c0);
    n = attn_piece_of(sp, c1 - 1) - i0 + 1;
    slot0 = attn_piece_start(sp, i0) < c0 ? 1 : 0;
  }
  if (tile < 0 || n < 2) return;  // no cut tile, or one written directly by its only piece
  const int ql = slab * VPB + threadIdx.x / TPV, dc = threadIdx.x % TPV;
  const int v = tile * 128 + ql;
  if (v >= Mv) return;
  const int r = v / g, hq = kvh * g + v % g;
  // the row's position is loaded with the first batch of pieces and checked at the end
  const int pos_r = a.row_pos[(int64_t)req * a.R + r];
  auto pidx = [&](int k) { return part_index(a, group, i0 + k, k == 0 ? slot0 : 0) + ql; };
  // online merge over batches of four pieces; every load of a batch is independent
  float M = -INFINITY, Ls = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += B) {
    float4 ml[B];
    u32x4 hv[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {   // clamped, unconditional loads: all in flight at once
      const int64_t pi = pidx(min(k0 + k, n - 1));
      ml[k] = a.part_ml[pi];
      hv[k] = *reinterpret_cast<const u32x4*>(a.part_o + pi * D + 8 * dc);
    }
    // the whole batch is in flight before any of it is used (a piece skipped below would otherwise
    // have its values loaded only after that test)
    asm volatile("" ::"v"(hv[0][0]), "v"(hv[0][1]), "v"(hv[0][2]), "v"(hv[0][3]), "v"(hv[1][0]), "v"(hv[1][1]),
                 "v"(hv[1][2]), "v"(hv[1][3]), "v"(hv[2][0]), "v"(hv[2][1]), "v"(hv[2][2]), "v"(hv[2][3]),
                 "v"(hv[3][0]), "v"(hv[3][1]), "v"(hv[3][2]), "v"(hv[3][3]));
    float mb = M;
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (k0 + k >= n) ml[k] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
      mb = fmaxf(mb, ml[k].x);
    }
    if (mb == -INFINITY) continue;
    const float sc = exp2f(M - mb);  // 0 while nothing has been merged (M = -inf)
    Ls *= sc;
    acc0 *= sc;
    acc1 *= sc;
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (ml[k].x != -INFINITY) {
        const float w = exp2f(ml[k].x - mb);
        const f32x4 o0 = f32x4{h2f(hv[k][0] & 0xffffu), h2f(hv[k][0] >> 16), h2f(hv[k][1] & 0xffffu), h2f(hv[k][1] >> 16)} * ml[k].z;
        const f32x4 o1 = f32x4{h2f(hv[k][2] & 0xffffu), h2f(hv[k][2] >> 16), h2f(hv[k][3] & 0xffffu), h2f(hv[k][3] >> 16)} * ml[k].z;
        Ls += ml[k].y * w;
        acc0 += w * o0;
        acc1 += w * o1;
      }
    }
    M = mb;
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  u32x4 w;
  w[0] = pack_bf2(acc0[0] * inv, acc0[1] * inv);
  w[1] = pack_bf2(acc0[2] * inv, acc0[3] * inv);
  w[2] = pack_bf2(acc1[0] * inv, acc1[1] * inv);
  w[3] = pack_bf2(acc1[2] * inv, acc1[3] * inv);
  // the merge is finished for every row (the asm keeps it out of the branch), and only then a row
  // outside the cache is dropped: nothing is written for it
  asm volatile("" ::"v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(M), "v"(Ls));
  if (pos_r < 0) return;
  *reinterpret_cast<u32x4*>(a.out + (((int64_t)req * a.R + r) * a.Hq + hq) * D + 8 * dc) = w;
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
  // the pieces' merge records follow the tiles' unit prefix sums in the same buffer (16-byte aligned),
  // then the groups' queues
  a.merge = reinterpret_cast<int4*>(tilecum + attn_merge_offset(n_req, a.n_tiles));
  a.queue = tilecum + attn_queue_offset(n_req, a.n_tiles, a.n_groups, pieces);
  // whole tiles from queues where every work group gets several of them
  a.dynamic = attn_dynamic(a.n_tiles, pieces) ? 1 : 0;
  a.comb_idx = a.dynamic ? min(16, pieces) : min(a.n_tiles, pieces);
  hipError_t err;
  if (a.dynamic && !ex.queue_ready) {
    k_attn_queue_reset<<<dim3(1), dim3(64), 0, st>>>(a.queue, a.n_groups);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const unsigned nblk = (unsigned)(a.n_groups * pieces);
  if (D == 128) k_attn_mfma<128><<<dim3(nblk), dim3(256), 0, st>>>(a);
  else k_attn_mfma<64><<<dim3(nblk), dim3(256), 0, st>>>(a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned ncomb = (unsigned)(a.n_groups * a.comb_idx * (D == 128 ? 8 : 4));
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
