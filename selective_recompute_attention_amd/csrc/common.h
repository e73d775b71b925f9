// Shared definitions of the HIP kernels of the KV-cache fusion step (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace sra {

// Chunk/segment table passed by value as a kernel argument (no host-to-device copy).
// Entry e covers rows [0, len[e]) of one chunk of request req[e]: store rows src[e] + t,
// fused rows dst[e] + t, re-rotation delta[e]. blk0 is the exclusive prefix of the number
// of thread blocks each entry gets; a launch handles blocks [0, blk0[n]). Longer tables are
// split across several launches.
constexpr int kMaxEntries = 80;
struct ChunkTab {
  int n;
  int req[kMaxEntries];
  int src[kMaxEntries];
  int len[kMaxEntries];
  int dst[kMaxEntries];
  int delta[kMaxEntries];
  int aux[kMaxEntries];      // the entry's chunk index within its request
  int blk0[kMaxEntries + 1];
};

// Selection units: top-`quota` of fused context positions [begin, begin + len) of request
// req, written at row_pos[req][out_off ...]; the unit with writes_query set also appends
// the query positions.
struct SelTab {
  int n;
  int req[kMaxEntries];
  int begin[kMaxEntries];
  int len[kMaxEntries];
  int quota[kMaxEntries];
  int out_off[kMaxEntries];
  int writes_query[kMaxEntries];
  int* out[kMaxEntries];    // the entry's output row: out_off + i for its selected rows, rows - Lq + i
  int rows[kMaxEntries];    // for the query rows
};

// The entry owning block blk: the number of entries i >= 1 with blk0[i] <= blk (blk0 ascends),
// counted over batches of 16 independent scalar loads at fixed offsets rather than a chain of
// dependent ones (constant indices keep the table in the kernel arguments).
__device__ __forceinline__ int find_entry(const ChunkTab& t, int blk) {
  int e = 0;
#pragma unroll
  for (int b = 1; b <= kMaxEntries; b += 16) {
    if (b >= t.n) break;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (b + k <= kMaxEntries) e += (b + k < t.n && t.blk0[b + k] <= blk) ? 1 : 0;
  }
  return e;
}

// bfloat16 <-> float32. The narrowing conversion is the hardware's round-to-nearest-even
// (v_cvt_pk_bf16_f32 on gfx950: two values per instruction).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ uint32_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the bare hardware instruction (v_exp_f32: about 1 ulp; results below 2^-126 flush to
// zero, which softmax weights can afford; -inf gives exactly 0). exp2f adds a denormal-range fixup
// of four more instructions per call.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the two 32-lane halves of a wave with v_permlane32_swap (a VALU lane swap)
// instead of an LDS permute. With both operands x, the swap returns (x[l], x[l+32]) in lanes 0-31
// and (x[l-32], x[l]) in lanes 32-63, so each lane sees the pair in the same order.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The value of lane l ^ 32.
__device__ __forceinline__ float half_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Sum of squares of the 16 bytes of one key in float64, element by element in order. A square of a
// bf16 or float32 value is exact in float64, so this sequence gives the same bits wherever it runs.
template <typename T>
__device__ __forceinline__ double sumsq16(double acc, const uint32_t* w);
template <>
__device__ __forceinline__ double sumsq16<uint16_t>(double acc, const uint32_t* w) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double a = __uint_as_float(w[k] << 16), b = __uint_as_float(w[k] & 0xffff0000u);
    acc += a * a;
    acc += b * b;
  }
  return acc;
}
template <>
__device__ __forceinline__ double sumsq16<float>(double acc, const uint32_t* w) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double a = __uint_as_float(w[k]);
    acc += a * a;
  }
  return acc;
}
// Key-norm sums: one float64 sum per (token, KV head) over its d values in order, then the heads in
// order. Rows of one block of the row-sum kernel: one thread per (row, head).
__host__ __device__ __forceinline__ int anchor_rows_per_block(int Hkv) { return Hkv >= 256 ? 1 : 256 / Hkv; }
// Longest chunk whose anchors the scoring pass picks itself (its sums fit the pass's LDS tile).
constexpr int kAnchorFusedMaxLen = 4352;

// Whole-wave scans and reductions on DPP lane moves (row shifts inside 16-lane rows, then the
// row broadcasts of lanes 15 and 31), all plain VALU instructions.
template <int CTRL, int ROW_MASK, bool BC>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, BC);
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += dpp_mov<0x111, 0xf, true>(0u, v);    // row_shr:1
  v += dpp_mov<0x112, 0xf, true>(0u, v);    // row_shr:2
  v += dpp_mov<0x114, 0xf, true>(0u, v);    // row_shr:4
  v += dpp_mov<0x118, 0xf, true>(0u, v);    // row_shr:8
  v += dpp_mov<0x142, 0xa, false>(0u, v);   // row_bcast:15 -> rows 1 and 3
  v += dpp_mov<0x143, 0xc, false>(0u, v);   // row_bcast:31 -> rows 2 and 3
  return v;
}
// Reduction with an idempotent operation (lanes without a source keep their own value); the
// result of the whole wave, returned in every lane.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  v = op(v, dpp_mov<0x111, 0xf, false>(v, v));
  v = op(v, dpp_mov<0x112, 0xf, false>(v, v));
  v = op(v, dpp_mov<0x114, 0xf, false>(v, v));
  v = op(v, dpp_mov<0x118, 0xf, false>(v, v));
  v = op(v, dpp_mov<0x142, 0xa, false>(v, v));
  v = op(v, dpp_mov<0x143, 0xc, false>(v, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Rotary frequencies theta_i = base^(-2i/d), i < d/2, formed once on the host in float64 and passed
// by value; a kernel forms the angle pos * theta_i and its cos/sin in float64, rounded to float32.
struct Theta {
  double v[64];
};
inline Theta make_theta(int d, double base) {
  Theta t;
  for (int i = 0; i < 64; ++i) t.v[i] = i < d / 2 ? std::pow(base, -2.0 * (double)i / (double)d) : 0.0;
  return t;
}
__device__ __forceinline__ float2 rope_cs(double pos, double theta) {
  double s, c;
  sincos(pos * theta, &s, &c);
  return make_float2((float)c, (float)s);
}

// fp16 copy of the fused keys for the attention's query-key products (bf16 storage only). Kernels that
// write fused K rows (re-rotation, scatter, the attention entry's conversion) also write each row's
// fp16 value to kh (same [n_req][L][Hkv][d] layout); a bf16 key of magnitude above 65504 has no fp16
// value, so its writer sets flags[req * Hkv + kv_head] = call_id, and so does the scatter for a scaled
// query beyond fp16. The attention recomputes a flagged (request, KV head) group exactly in float32.
// call_id differs between calls, so stale flags of another call never match (a graph replay reuses its
// call's id: a flag it left makes a later replay recompute that group too, which is still exact).
struct F16Shadow {
  uint16_t* kh = nullptr;
  unsigned* flags = nullptr;
  unsigned call_id = 0;
  int* queue = nullptr;   // the attention's group queues, emptied by the scatter that precedes it
  int n_queue = 0;
};
// fp16 of the two bf16 values of word w (exact for magnitudes 2^-14 .. 65504; beyond 65504 infinity),
// with the larger magnitude of the two folded into amax.
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t w, float& amax) {
  const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
  amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// Largest finite fp16 magnitude; values at or above 65520 round to infinity.
constexpr float kF16Max = 65504.f;

// Prepared query operand of the bf16 attention (written by the row kernel, read by the attention).
// Query vectors of one (request, KV head) group are numbered v = r * g + (h % g) and cut into
// blocks of 32. For block b, 16-dimension step ks and plane (0: hi = bf16(x), 1: lo = bf16(x - hi))
// the 32 vectors' dimensions 16 ks + 8 hh + s (hh = 0, 1; s = 0..7) are contiguous, lane-major: one
// wave reads the B operand of one matrix instruction as 1 KB of consecutive bytes.
__host__ __device__ __forceinline__ int64_t qop_index(int64_t group, int b, int ks, int plane, int l,
                                                      int hh, int n_blk, int nks) {
  return ((((group * n_blk + b) * nks + ks) * 2 + plane) * 32 + l) * 16 + hh * 8;
}

// Work split of the bf16 attention. A group's 128-vector tiles need ceil((p_last + 1) / 64) units
// of 64 keys each; the U units of a group are dealt to `pieces_used` work groups as contiguous
// ranges. kAttnSlots is the number of resident attention work groups on 256 compute units (two per
// unit): work groups b and b + kAttnSlots / 2 share a unit, and the first of the two runs faster
// while both are resident (the older waves win the issue arbitration), so a piece whose work group
// is the first on its unit takes kAttnFirstW parts of the units to the second's kAttnSecondW.
#ifndef SRA_ATTN_FIRST_W
#define SRA_ATTN_FIRST_W 11
#endif
constexpr int kAttnSlots = 512;
constexpr int kAttnMinUnits = 3;
constexpr int kAttnMaxTiles = 2048;
constexpr int kAttnFirstW = SRA_ATTN_FIRST_W, kAttnSecondW = 10;
__host__ __device__ __forceinline__ int attn_pieces_used(int U, int pieces) {
  const int p = (U + kAttnMinUnits - 1) / kAttnMinUnits;
  return p < 1 ? 1 : (p < pieces ? p : pieces);
}
// The split of one (request, KV head) group: U units over P pieces, the first P1 of them (work
// groups group + n_groups i below kAttnSlots / 2) weighted kAttnFirstW, the rest kAttnSecondW.
struct AttnSplit {
  int U, P, P1;
};
__host__ __device__ __forceinline__ AttnSplit attn_split(int U, int pieces, int group, int n_groups) {
  AttnSplit s;
  s.U = U;
  s.P = attn_pieces_used(U, pieces);
  const int h = kAttnSlots / 2 - group;
  const int p1 = h > 0 ? (h + n_groups - 1) / n_groups : 0;
  s.P1 = p1 < s.P ? p1 : s.P;
  return s;
}
__host__ __device__ __forceinline__ int64_t attn_weight_before(const AttnSplit& s, int i) {
  const int a = i < s.P1 ? i : s.P1, b = i > s.P1 ? i - s.P1 : 0;
  return (int64_t)kAttnFirstW * a + (int64_t)kAttnSecondW * b;
}
// first unit of piece i (i = P gives U)
__host__ __device__ __forceinline__ int attn_piece_start(const AttnSplit& s, int i) {
  return (int)((int64_t)s.U * attn_weight_before(s, i) / attn_weight_before(s, s.P));
}
// the piece whose range holds unit u (0 <= u < U): the last piece starting at or before it
__host__ __device__ __forceinline__ int attn_piece_of(const AttnSplit& s, int u) {
  int lo = 0, hi = s.P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (attn_piece_start(s, mid) <= u) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
// ints before the pieces' 16-byte merge records in the attention's tilecum buffer
__host__ __device__ __forceinline__ int64_t attn_merge_offset(int n_req, int n_tiles) {
  return ((int64_t)n_req * (n_tiles + 1) + 3) & ~(int64_t)3;
}
// ints before the groups' work queues (after the merge records); the buffer holds
// attn_queue_offset + n_groups ints
__host__ __device__ __forceinline__ int64_t attn_queue_offset(int n_req, int n_tiles, int n_groups, int pieces) {
  return attn_merge_offset(n_req, n_tiles) + (int64_t)n_groups * pieces * 4;
}
// the attention takes whole tiles from per-group queues when a group has at least 2.25 tiles per work
// group (fewer, and the largest tiles outweigh a work group's share: the static split is then better)
__host__ __device__ __forceinline__ bool attn_dynamic(int n_tiles, int pieces) { return 4 * n_tiles >= 9 * pieces; }

}  // namespace sra

// ---------------------------------------------------------------------------- launchers
// Each returns the hipError_t of its launch(es). dtype: 0 bf16, 1 f32.
namespace sra {
hipError_t launch_rerotate(int dtype, int D, int Hkv, const ChunkTab& tab, int rows_per_blk,
                           const void* ks, const void* vs, void* kf, void* vf, int64_t L,
                           double base, hipStream_t st, const F16Shadow& sh = F16Shadow());
// fp16 copy of n_rows fused K rows of every request ([n_req][L][Hkv][D] bf16 -> sh.kh), with the
// overflow flags of sh.
hipError_t launch_k_to_f16(int D, int Hkv, int n_req, int L, const uint16_t* kf, const F16Shadow& sh,
                           hipStream_t st);
// Per recomputed row (row_pos[r] = p in [0, L); row_pos NULL: p = r): the row's cos/sin table (cs_out, optional), the
// fresh K/V scatter (kn/vn optional) and, for bf16, the attention's prepared query operand (qn/qop
// optional; rows outside [0, L) get zeros). Fresh rows are compact (row r) or, when indexed,
// position-indexed (row p); fresh_rows is their count per request.
hipError_t launch_scatter(int dtype, int D, int Hq, int Hkv, int n_req, int R, int L,
                          const void* qn, const void* kn, const void* vn, int fresh_rows,
                          int indexed, const int* row_pos, void* kf, void* vf, float2* cs_out,
                          uint16_t* qop, int qop_blocks, bool q16, float scale_log2, double base,
                          hipStream_t st, const F16Shadow& sh = F16Shadow());
hipError_t launch_rope_table(int D, int n_req, int R, const int* row_pos, float2* cs_out,
                             double base, hipStream_t st);
// Anchor probe prefix rows [0, n_chunks * k) of [n_req][Lp][Hkv][D] probe caches; tab entries
// (req, src, len, dst = first prefix row, delta = orig_pos, aux = chunk index), k blocks each.
hipError_t launch_anchor_prefix(int dtype, int D, int Hkv, const ChunkTab& tab, int k, int n_chunks,
                                const int* anchors, const void* ks, const void* vs, void* kp, void* vp, int Lp,
                                double base, hipStream_t st);
// Chunk attention statistics of requests [req0, req0 + n_req_launch): tab holds their
// (request, chunk) entries (dst = first token, len); fx: zeroed [n_req][Lctx][n_chunks] slots.
hipError_t launch_chunk_stats(int D, int n_req_launch, int req0, int Hq, int Hkv, int Lctx, int Lk,
                              const uint16_t* qop, int qop_blocks, const uint16_t* kc, const ChunkTab& tab,
                              int n_chunks, unsigned long long* fx, float* inter, float* score, float* cci,
                              hipStream_t st);
// KV deviation of the first n_dev recomputed rows (dev: [n_req][n_dev] float32). Fresh rows are
// compact or position-indexed as in launch_scatter; kf/vf hold the reused rows (not yet scattered).
hipError_t launch_kv_deviation(int dtype, int D, int Hkv, int n_req, int R, int L, const void* kn,
                               const void* vn, int fresh_rows, int indexed, const int* row_pos,
                               const void* kf, const void* vf, float* dev, int n_dev, double base,
                               hipStream_t st);
// tab: entries = chunks (src, len), dst = output slot, delta = offset of the chunk's sums in ss,
// blk0 in blocks of anchor_rows_per_block(Hkv) rows.
hipError_t launch_anchors(int dtype, int Hkv, int D, const ChunkTab& tab, int k, const void* ks,
                          double* ss, int32_t* anchors, float* norms, hipStream_t st);
// Anchors taken inside the scoring passes: pass 1 writes per-head sums of squares (ssp
// [Hkv][stride], stride = n_req * L_ctx, at the token's context position), pass 2 adds one block per
// chunk entry that picks the k largest totals (k == 0: none).
struct AnchorOut {
  int k = 0;
  double* ssp = nullptr;
  int64_t stride = 0;
  int32_t* rows = nullptr;   // [n_req][n_chunks][k]
  float* norms = nullptr;    // [store rows] or NULL
  int n_chunks = 0;
};
// Critical-layer scores are accumulated over KV heads as 64-bit fixed point (kScoreFixScale units):
// integer additions are exact and associative, so the total does not depend on their order.
constexpr double kScoreFixScale = 1099511627776.0;   // 2^40
hipError_t launch_score_prep(int D, const ChunkTab& tab, int Lq, int Hq, int Hkv, int Mpad,
                             int Lctx, const void* qc, uint16_t* qrot, int64_t plane,
                             int entry_base, float scale_log2, unsigned long long* fx, double base,
                             hipStream_t st);
// S1 carried by pass 1 (bfloat16 storage): the pass adds, per chunk entry and KV head y, one block
// per kS1Fold key blocks that re-rotates every head of rows [y * ceil(span / Hkv), ...) of that
// span of the stored chunk (the same rows and chunk entries as a standalone re-rotation). Pass 1
// holds one work group per CU, so the extra blocks are few and move their share in one batch,
// beside the scoring blocks in the same round. kf == NULL: none.
constexpr int kS1Fold = 2;
// Pass 1 may prepare the query operand itself (instead of the preparation kernel) when every wave
// has one query tile (Lq * g <= 128) and Lq <= kInRotMaxLq: it rotates the raw critical-layer
// queries [n_req][Lq][Hq][d] with an LDS angle table and writes the operand for pass 2. on == 0:
// the operand comes from the preparation kernel.
constexpr int kInRotMaxLq = 64;
struct QueryRot {
  const uint16_t* qc = nullptr;
  int Lq = 0;
  int Hq = 0;
  float scale_log2 = 0.f;
  int on = 0;
};
struct RerotFused {
  const uint16_t* ks = nullptr;
  const uint16_t* vs = nullptr;
  uint16_t* kf = nullptr;
  uint16_t* vf = nullptr;
  int64_t L = 0;
  double base = 0.0;
  F16Shadow sh;   // optional fp16 copy of the re-rotated keys
};
hipError_t launch_score_pass(int pass, int D, const ChunkTab& tab, const int* req_blk0, int n_req,
                             int Hkv, int Mpad, int Mvalid, int Lctx, const void* kc,
                             uint16_t* qrot, int64_t plane, int entry_base, int blk_base,
                             float2* ml_part, const float2* ml_final, int fuse_merge,
                             unsigned long long* fx, const AnchorOut& anc, const RerotFused& rf,
                             const QueryRot& qr, double base, hipStream_t st);
hipError_t launch_score_merge(const int* req_blk0, int n_req, int Hkv, int Mpad, int Mvalid,
                              const float2* ml_part, float2* ml_final, hipStream_t st);
hipError_t launch_score_f32(int D, const ChunkTab& tab_req, int n_req, int Lq, int Hq, int Hkv,
                            int Lctx, const float* qc, const float* kc, float* prob,
                            float scale_log2, double base, hipStream_t st);
hipError_t launch_colsum_f32(int n_req, int rows, int Lctx, const float* prob, float* parts,
                             hipStream_t st);
// Scores come from fixed-point totals (fx), from nparts float partials added in order, or (both
// absent) from `scores` itself, row req at scores + req * sstride. With map, every written index i
// becomes map[req * map_stride + i] (the query rows are indices Lctx .. Lctx + Lq - 1); with gather
// (map required) the score of unit index j is the stored score of row map[j] instead of that of j.
// Entry e writes into tab.out[e] (tab.rows[e] entries, the query rows last).
hipError_t launch_select(const SelTab& tab, const unsigned long long* fx, int nparts, int Lctx, int Lq,
                         int sstride, const float* parts, float* scores, hipStream_t st,
                         const int* map = nullptr, int map_stride = 0, bool gather = false);
// qop: prepared query operand (qop_blocks blocks of 32 vectors per group); kh: fp16 copy of the fused
// keys; tilecum: [n_req][tiles+1] ints, then (from int attn_merge_offset) [n_groups][pieces] int4 (each
// piece's merge record); part_o
// ([..][D] fp16, scaled) / part_ml ((max, sum, scale, 0)):
// [n_groups][pieces][2][128] partial results. Groups whose flag equals call_id are recomputed exactly
// from the fresh queries q ([n_req][q_rows][Hq][D] before rotation, row p when indexed, else row r)
// and the bf16 K/V; fallback (optional, [n_req][Hkv]) receives 1 for those groups and 0 for the rest.
struct AttnExact {
  int queue_ready = 0;   // the group queues were emptied by an earlier launch (the row scatter)
  const uint16_t* q = nullptr;
  int q_rows = 0;
  int indexed = 0;
  const unsigned* flags = nullptr;
  unsigned call_id = 0;
  int* fallback = nullptr;
  double base = 10000.0;
};
hipError_t launch_attn_bf16(int D, int n_req, int Hq, int Hkv, int R, int L, const uint16_t* qop,
                            int qop_blocks, const int* row_pos, const uint16_t* kh, const uint16_t* kf,
                            const uint16_t* vf, uint16_t* out, float* lse, int pieces,
                            int* tilecum, uint16_t* part_o, float4* part_ml, const AttnExact& ex,
                            hipStream_t st);
hipError_t launch_attn_f32(int D, int n_req, int Hq, int Hkv, int R, int L, const float* q,
                           int q_rows, int indexed, const int* row_pos, const float2* cs,
                           const float* kf, const float* vf, float* out, float* lse,
                           hipStream_t st);
hipError_t launch_check_rows(const int* row_pos, int n_req, int R, int L, int* bad,
                             hipStream_t st);
}  // namespace sra
