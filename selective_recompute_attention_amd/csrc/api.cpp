// Host side of the C ABI declared in include/sra.h: argument validation, workspace planning,
// kernel-argument chunk tables and launch sequencing on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <mutex>
#include <string>
#include <vector>

#include "sra.h"
#include "common.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SRA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SRA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t elem_size(const sra_shape* s) { return s->dtype == SRA_DTYPE_BF16 ? 2 : 4; }

int check_shape(const sra_shape* s) {
  if (!s) return fail(SRA_E_NULL, "shape is NULL");
  if (s->dtype != SRA_DTYPE_BF16 && s->dtype != SRA_DTYPE_F32)
    return fail(SRA_E_DTYPE, "dtype %d is neither SRA_DTYPE_BF16 nor SRA_DTYPE_F32", s->dtype);
  if (s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->n_q_heads % s->n_kv_heads != 0)
    return fail(SRA_E_SHAPE, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SRA_E_SHAPE, "head_dim %d is not 64 or 128", s->head_dim);
  if (!(s->rope_base > 1.0) || !std::isfinite(s->rope_base))
    return fail(SRA_E_SHAPE, "rope_base must be finite and > 1");
  return SRA_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(SRA_E_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(SRA_E_SHAPE, "%s is not 16-byte aligned", name);
  return SRA_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Validate a [n_req][n_chunks] table: chunks tile [0, L_ctx) in request order, store rows in
// range, equal L_ctx for every request. Returns L_ctx through *lctx.
int check_chunks(const sra_chunk* ch, int n_req, int n_chunks, int64_t store_rows, int* lctx) {
  if (!ch) return fail(SRA_E_NULL, "chunks is NULL");
  if (n_chunks <= 0) return fail(SRA_E_SHAPE, "n_chunks must be positive");
  int first = -1;
  for (int q = 0; q < n_req; ++q) {
    int64_t n = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const sra_chunk& k = ch[(int64_t)q * n_chunks + c];
      if (k.n_tokens < 0) return fail(SRA_E_CHUNKS, "request %d chunk %d: negative n_tokens", q, c);
      if (k.dst_row != n)
        return fail(SRA_E_CHUNKS, "request %d chunk %d: dst_row %d, expected %lld (chunks must tile the context in order)",
                    q, c, k.dst_row, (long long)n);
      if (k.src_row < 0 || (int64_t)k.src_row + k.n_tokens > store_rows)
        return fail(SRA_E_CHUNKS, "request %d chunk %d: store rows [%d, %lld) outside [0, %lld)", q, c,
                    k.src_row, (long long)k.src_row + k.n_tokens, (long long)store_rows);
      n += k.n_tokens;
      if (n > std::numeric_limits<int32_t>::max() / 2)
        return fail(SRA_E_SHAPE, "context too long");
    }
    if (first < 0) first = (int)n;
    else if (n != first)
      return fail(SRA_E_SHAPE, "request %d has context length %lld, request 0 has %d", q, (long long)n, first);
  }
  *lctx = first;
  return SRA_OK;
}

// ------------------------------------------------------------------------------ workspace plan
// Attention work groups per (request, KV head) group: the resident capacity shared out.
int attn_pieces(int n_req, int Hkv) {
  const int64_t groups = (int64_t)n_req * Hkv;
  return (int)std::max<int64_t>(1, sra::kAttnSlots / std::max<int64_t>(groups, 1));
}

struct Plan {
  // offsets in bytes from the workspace base
  size_t cs = 0;          // rotary table [n_req][R][d/2] float2
  size_t k16 = 0;         // fp16 copy of the fused keys [n_req][L][Hkv][d] (bf16 attention)
  size_t flags = 0;       // fp16 overflow flags [n_req][Hkv]
  size_t region = 0;      // start of the union of the score and attention regions
  // score (bf16)
  int Mpad = 0;
  int64_t max_blocks = 0;
  size_t qrot = 0, ml_part = 0, ml_final = 0, colsum = 0, scores_tmp = 0, ssp = 0;
  int64_t qrot_plane = 0;  // elements per hi/lo plane
  // score (f32)
  size_t prob = 0, parts = 0;
  // attention (bf16): prepared query operand, tile prefix sums, partial results
  int n_tiles = 0, qop_blocks = 0, pieces = 1, n_groups = 0;
  size_t qop = 0, tilecum = 0, queue = 0, part_o = 0, part_ml = 0;
  size_t score_end = 0, attn_end = 0, total = 0;
};

Plan make_plan(const sra_shape* s, int n_req, int n_chunks, int L, int R, int Lq) {
  Plan p;
  const int D = s->head_dim, Hq = s->n_q_heads, Hkv = s->n_kv_heads, g = Hq / Hkv;
  const int Lctx = std::max(L - Lq, 0);
  size_t off = 0;
  p.cs = off;  // the float32 attention's angle table
  if (s->dtype == SRA_DTYPE_F32) off = align256(off + (size_t)n_req * R * (D / 2) * sizeof(float2));
  // the bf16 attention's fp16 keys and overflow flags, outside the union below: the re-rotation
  // writes them while the scoring still uses its region
  p.k16 = off;
  p.flags = off;
  if (s->dtype == SRA_DTYPE_BF16) {
    off = align256(off + (size_t)n_req * L * Hkv * D * sizeof(uint16_t));
    p.flags = off;
    off = align256(off + (size_t)n_req * Hkv * sizeof(unsigned));
  }
  p.region = off;
  // score region
  size_t so = off;
  if (s->dtype == SRA_DTYPE_BF16) {
    p.Mpad = (int)ceil_div((int64_t)Lq * g, 32) * 32;
    p.max_blocks = (int64_t)n_req * (ceil_div(Lctx, 128) + n_chunks);
    p.qrot_plane = (int64_t)n_req * n_chunks * Hkv * p.Mpad * D;
    p.qrot = so; so = align256(so + (size_t)p.qrot_plane * 2 * sizeof(uint16_t));
    p.ml_part = so; so = align256(so + (size_t)p.max_blocks * Hkv * p.Mpad * sizeof(float2));
    p.ml_final = so; so = align256(so + (size_t)n_req * Hkv * p.Mpad * sizeof(float2));
    p.colsum = so; so = align256(so + (size_t)n_req * Lctx * sizeof(unsigned long long));  // fixed-point scores
  } else {
    p.prob = so; so = align256(so + (size_t)n_req * Hq * Lq * Lctx * sizeof(float));
    p.parts = so; so = align256(so + (size_t)n_req * Lctx * sizeof(float));
  }
  p.scores_tmp = so; so = align256(so + (size_t)n_req * Lctx * sizeof(float));
  // anchors: per-head float64 sums of squares of the critical layer's keys
  p.ssp = so; so = align256(so + (size_t)Hkv * n_req * Lctx * sizeof(double));
  p.score_end = so;
  // attention region (same start: scoring is finished before the scatter writes it)
  size_t ao = off;
  if (s->dtype == SRA_DTYPE_BF16) {
    const int64_t groups = (int64_t)n_req * Hkv;
    p.n_tiles = (int)ceil_div((int64_t)R * g, 128);
    p.qop_blocks = 4 * p.n_tiles;
    p.pieces = attn_pieces(n_req, Hkv);
    p.qop = ao; ao = align256(ao + (size_t)groups * p.qop_blocks * 32 * 2 * D * sizeof(uint16_t));
    // the tiles' unit prefix sums, then each piece's merge record (four ints), then the groups' queues
    p.tilecum = ao;
    p.n_groups = (int)groups;
    p.queue = ao + (size_t)sra::attn_queue_offset(n_req, p.n_tiles, (int)groups, p.pieces) * sizeof(int);
    ao = align256(p.queue + (size_t)groups * sizeof(int));
    const int64_t slots = groups * p.pieces * 2 * 128;
    p.part_o = ao; ao = align256(ao + (size_t)slots * D * sizeof(uint16_t));
    p.part_ml = ao; ao = align256(ao + (size_t)slots * sizeof(float4));
  }
  p.attn_end = ao;
  p.total = std::max(p.score_end, p.attn_end);
  return p;
}

char* wsp(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// A distinct id per attention call, never 0: fp16 overflow flags of another call never match it.
std::atomic<unsigned> g_call_id{0};
unsigned next_call_id() {
  unsigned v = ++g_call_id;
  while (v == 0) v = ++g_call_id;
  return v;
}
sra::F16Shadow shadow_of(const sra_shape* s, void* ws, const Plan& p, unsigned call_id) {
  sra::F16Shadow sh;
  if (s->dtype != SRA_DTYPE_BF16) return sh;
  sh.kh = reinterpret_cast<uint16_t*>(wsp(ws, p.k16));
  sh.flags = reinterpret_cast<unsigned*>(wsp(ws, p.flags));
  sh.call_id = call_id;
  if (p.n_groups > 0) {   // the attention's queues (the scatter before each attention empties them)
    sh.queue = reinterpret_cast<int*>(wsp(ws, p.queue));
    sh.n_queue = p.n_groups;
  }
  return sh;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SRA_OK;
  if (!ws) return fail(SRA_E_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(SRA_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(SRA_E_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
  return SRA_OK;
}

// ------------------------------------------------------------------------------ table packing
struct Entry {
  int req, src, len, dst, delta, blocks;
  int c = 0;   // chunk index within the request
};

// Pack entries into launch-sized tables; calls fn(tab, first_entry_index, first_block_index).
template <typename Fn>
hipError_t for_each_tab(const std::vector<Entry>& ents, Fn fn) {
  size_t i = 0;
  int64_t blk_base = 0;
  while (i < ents.size()) {
    sra::ChunkTab tab;
    std::memset(&tab, 0, sizeof(tab));
    const size_t first = i;
    int blk = 0;
    while (i < ents.size() && tab.n < sra::kMaxEntries) {
      const Entry& e = ents[i];
      tab.req[tab.n] = e.req;
      tab.src[tab.n] = e.src;
      tab.len[tab.n] = e.len;
      tab.dst[tab.n] = e.dst;
      tab.delta[tab.n] = e.delta;
      tab.aux[tab.n] = e.c;
      tab.blk0[tab.n] = blk;
      blk += e.blocks;
      ++tab.n;
      ++i;
    }
    tab.blk0[tab.n] = blk;
    hipError_t err = fn(tab, (int)first, (int)blk_base);
    if (err != hipSuccess) return err;
    blk_base += blk;
  }
  return hipSuccess;
}

std::vector<Entry> chunk_entries(const sra_chunk* ch, int n_req, int n_chunks, int rows_per_blk) {
  std::vector<Entry> v;
  for (int q = 0; q < n_req; ++q)
    for (int c = 0; c < n_chunks; ++c) {
      const sra_chunk& k = ch[(int64_t)q * n_chunks + c];
      if (k.n_tokens == 0) continue;
      v.push_back({q, k.src_row, k.n_tokens, k.dst_row, k.dst_row - k.orig_pos,
                   (int)ceil_div(k.n_tokens, rows_per_blk), c});
    }
  return v;
}

// ------------------------------------------------------------------------------ stage bodies
int do_rerotate(const sra_shape* s, int n_req, const void* ks, const void* vs,
                const sra_chunk* ch, int n_chunks, void* kf, void* vf, int L, hipStream_t st,
                const sra::F16Shadow& sh = sra::F16Shadow()) {
  const int D = s->head_dim, Hkv = s->n_kv_heads;
  const int64_t row_bytes = (int64_t)Hkv * D * elem_size(s);
  const int rpb = (int)std::max<int64_t>(1, 32768 / (2 * row_bytes));
  auto ents = chunk_entries(ch, n_req, n_chunks, rpb);
  hipError_t e = for_each_tab(ents, [&](const sra::ChunkTab& tab, int, int) {
    return sra::launch_rerotate(s->dtype, D, Hkv, tab, rpb, ks, vs, kf, vf, L, s->rope_base, st, sh);
  });
  if (e != hipSuccess) return hip_fail(e, "re-rotation launch");
  return SRA_OK;
}

// Selection units and launch.
int do_select(int n_req, int Lctx, int Lq, int R, int N, const int32_t* quota, const sra_chunk* ch,
              int n_chunks, const unsigned long long* fx, int nparts, const float* parts, float* scores,
              int32_t* row_pos, hipStream_t st) {
  struct U { int req, begin, len, quota, off, wq; };
  std::vector<U> units;
  for (int q = 0; q < n_req; ++q) {
    if (!quota) {
      units.push_back({q, 0, Lctx, N, 0, 1});
    } else {
      int off = 0;
      for (int c = 0; c < n_chunks; ++c) {
        const sra_chunk& k = ch[(int64_t)q * n_chunks + c];
        const int qc = quota[(int64_t)q * n_chunks + c];
        units.push_back({q, k.dst_row, k.n_tokens, qc, off, c == 0 ? 1 : 0});
        off += qc;
      }
    }
  }
  size_t i = 0;
  while (i < units.size()) {
    sra::SelTab tab;
    std::memset(&tab, 0, sizeof(tab));
    while (i < units.size() && tab.n < sra::kMaxEntries) {
      const U& u = units[i++];
      tab.req[tab.n] = u.req;
      tab.begin[tab.n] = u.begin;
      tab.len[tab.n] = u.len;
      tab.quota[tab.n] = u.quota;
      tab.out_off[tab.n] = u.off;
      tab.writes_query[tab.n] = u.wq;
      tab.out[tab.n] = row_pos + (int64_t)u.req * R;
      tab.rows[tab.n] = R;
      ++tab.n;
    }
    hipError_t e = sra::launch_select(tab, fx, nparts, Lctx, Lq, Lctx, parts, scores, st);
    if (e != hipSuccess) return hip_fail(e, "selection launch");
  }
  return SRA_OK;
}

// Gradual filtering: deviation of the previous layer's n_prev context rows, then per request the
// n_keep rows of highest deviation (ascending), mapped back to their positions, then the query rows.
int do_hkvd(const sra_shape* s, int n_req, const void* kn, const void* vn, int fresh_rows, int indexed,
            const int32_t* prev, int R_prev, int n_prev, const void* kf, const void* vf, int L, int n_keep,
            float* dev, int32_t* rows_out, hipStream_t st) {
  hipError_t e = sra::launch_kv_deviation(s->dtype, s->head_dim, s->n_kv_heads, n_req, R_prev, L, kn, vn,
                                          fresh_rows, indexed, prev, kf, vf, dev, n_prev, s->rope_base, st);
  if (e != hipSuccess) return hip_fail(e, "deviation launch");
  const int Lq = R_prev - n_prev;
  for (int q0 = 0; q0 < n_req; q0 += sra::kMaxEntries) {
    sra::SelTab tab;
    std::memset(&tab, 0, sizeof(tab));
    for (int q = q0; q < n_req && tab.n < sra::kMaxEntries; ++q) {
      tab.req[tab.n] = q;
      tab.begin[tab.n] = 0;
      tab.len[tab.n] = n_prev;
      tab.quota[tab.n] = n_keep;
      tab.out_off[tab.n] = 0;
      tab.writes_query[tab.n] = 1;
      tab.out[tab.n] = rows_out + (int64_t)q * (n_keep + Lq);
      tab.rows[tab.n] = n_keep + Lq;
      ++tab.n;
    }
    e = sra::launch_select(tab, nullptr, 0, n_prev, Lq, n_prev, nullptr, dev, st, prev, R_prev);
    if (e != hipSuccess) return hip_fail(e, "selection launch");
  }
  return SRA_OK;
}

// Validates quota/n_select and returns N (selected context tokens per request).
int resolve_count(int n_req, int n_chunks, const sra_chunk* ch, int Lctx, int n_select,
                  const int32_t* quota, int* N) {
  if (!quota) {
    if (n_select < 0 || n_select > Lctx)
      return fail(SRA_E_SHAPE, "n_select %d outside [0, %d]", n_select, Lctx);
    *N = n_select;
    return SRA_OK;
  }
  int first = -1;
  for (int q = 0; q < n_req; ++q) {
    int64_t tot = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const int qc = quota[(int64_t)q * n_chunks + c];
      const int len = ch[(int64_t)q * n_chunks + c].n_tokens;
      if (qc < 0 || qc > len)
        return fail(SRA_E_SHAPE, "request %d chunk %d: quota %d outside [0, %d]", q, c, qc, len);
      tot += qc;
    }
    if (first < 0) first = (int)tot;
    else if (tot != first)
      return fail(SRA_E_SHAPE, "request %d selects %lld tokens, request 0 selects %d", q, (long long)tot, first);
  }
  *N = first;
  return SRA_OK;
}

int do_score_select(const sra_shape* s, int n_req, const void* qc, int Lq, const void* kc,
                    const sra_chunk* ch, int n_chunks, int Lctx, int N, const int32_t* quota,
                    float* scores, int32_t* row_pos, void* ws, const Plan& p, hipStream_t st,
                    const sra::AnchorOut& anc = sra::AnchorOut(),
                    const sra::RerotFused& rf = sra::RerotFused()) {
  const int D = s->head_dim, Hq = s->n_q_heads, Hkv = s->n_kv_heads, g = Hq / Hkv;
  const int R = N + Lq;
  float* sc = scores ? scores : reinterpret_cast<float*>(wsp(ws, p.scores_tmp));
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  hipError_t e;
  if (s->dtype == SRA_DTYPE_BF16) {
    uint16_t* qrot = reinterpret_cast<uint16_t*>(wsp(ws, p.qrot));
    float2* ml_part = reinterpret_cast<float2*>(wsp(ws, p.ml_part));
    float2* ml_final = reinterpret_cast<float2*>(wsp(ws, p.ml_final));
    unsigned long long* fx = reinterpret_cast<unsigned long long*>(wsp(ws, p.colsum));
    auto ents = chunk_entries(ch, n_req, n_chunks, 128);
    // per-request block ranges in the global block numbering (entries are ordered by request)
    std::vector<int> req_blk0(n_req + 1, 0);
    for (const Entry& en : ents) req_blk0[en.req + 1] += en.blocks;
    for (int q = 0; q < n_req; ++q) req_blk0[q + 1] += req_blk0[q];
    // pass 1 prepares the query operand itself when each wave has one query tile and the angle
    // table fits; otherwise the preparation kernel does
    sra::QueryRot qr;
    if (p.Mpad <= 128 && Lq <= sra::kInRotMaxLq) {
      qr.qc = static_cast<const uint16_t*>(qc);
      qr.Lq = Lq;
      qr.Hq = Hq;
      qr.scale_log2 = scale_log2;
      qr.on = 1;
    } else {
      e = for_each_tab(ents, [&](const sra::ChunkTab& tab, int first, int) {
        return sra::launch_score_prep(D, tab, Lq, Hq, Hkv, p.Mpad, Lctx, qc, qrot, p.qrot_plane,
                                      first, scale_log2, fx, s->rope_base, st);
      });
      if (e != hipSuccess) return hip_fail(e, "score prep launch");
    }
    // Pass 2 merges a request's (max, sum) partials itself when they are few; otherwise a wide
    // merge kernel runs between the passes.
    int max_blocks = 0;
    for (int q = 0; q < n_req; ++q) max_blocks = std::max(max_blocks, req_blk0[q + 1] - req_blk0[q]);
    // pass 2 merges in place while each wave's share (blocks x its query tiles) stays small
    const int fuse_merge = (int64_t)max_blocks * ceil_div(p.Mpad / 32, 4) <= 128 ? 1 : 0;
    for (int pass = 1; pass <= 2; ++pass) {
      if (pass == 2 && !fuse_merge) {
        e = sra::launch_score_merge(req_blk0.data(), n_req, Hkv, p.Mpad, Lq * g, ml_part, ml_final, st);
        if (e != hipSuccess) return hip_fail(e, "score merge launch");
      }
      e = for_each_tab(ents, [&](const sra::ChunkTab& tab, int first, int blk_base) {
        return sra::launch_score_pass(pass, D, tab, req_blk0.data(), n_req, Hkv, p.Mpad, Lq * g, Lctx, kc,
                                      qrot, p.qrot_plane, first, blk_base, ml_part, ml_final, fuse_merge,
                                      fx, anc, rf, qr, s->rope_base, st);
      });
      if (e != hipSuccess) return hip_fail(e, pass == 1 ? "score pass 1 launch" : "score pass 2 launch");
    }
    return do_select(n_req, Lctx, Lq, R, N, quota, ch, n_chunks, fx, 0, nullptr, sc, row_pos, st);
  }
  // float32 storage: one softmax row per query vector, then fixed-order column sums
  auto ents = chunk_entries(ch, n_req, n_chunks, 1);
  sra::ChunkTab tab;
  std::memset(&tab, 0, sizeof(tab));
  for (const Entry& en : ents) {
    tab.req[tab.n] = en.req;
    tab.src[tab.n] = en.src;
    tab.len[tab.n] = en.len;
    tab.dst[tab.n] = en.dst;
    tab.delta[tab.n] = en.delta;
    ++tab.n;
  }
  float* prob = reinterpret_cast<float*>(wsp(ws, p.prob));
  float* parts = reinterpret_cast<float*>(wsp(ws, p.parts));
  e = sra::launch_score_f32(D, tab, n_req, Lq, Hq, Hkv, Lctx, (const float*)qc, (const float*)kc,
                            prob, scale_log2, s->rope_base, st);
  if (e != hipSuccess) return hip_fail(e, "f32 score launch");
  e = sra::launch_colsum_f32(n_req, Hq * Lq, Lctx, prob, parts, st);
  if (e != hipSuccess) return hip_fail(e, "f32 column-sum launch");
  return do_select(n_req, Lctx, Lq, R, N, quota, ch, n_chunks, nullptr, 1, parts, sc, row_pos, st);
}

// S4 on rows whose per-row inputs are ready: the prepared query operand (bf16) or the angle
// table (f32) in the workspace.
int do_attn(const sra_shape* s, int n_req, const void* q, int q_rows, int indexed,
            const int32_t* row_pos, int R, const void* kf, const void* vf, int L, void* out,
            float* lse, void* ws, const Plan& p, hipStream_t st, unsigned call_id = 0,
            int32_t* fallback = nullptr) {
  const int D = s->head_dim, Hq = s->n_q_heads, Hkv = s->n_kv_heads;
  hipError_t e;
  if (s->dtype == SRA_DTYPE_BF16) {
    sra::AttnExact ex;
    ex.q = static_cast<const uint16_t*>(q);
    ex.q_rows = q_rows;
    ex.indexed = indexed;
    ex.flags = reinterpret_cast<const unsigned*>(wsp(ws, p.flags));
    ex.call_id = call_id;
    ex.fallback = fallback;
    ex.base = s->rope_base;
    ex.queue_ready = 1;   // both callers ran the row scatter with the plan's shadow just before
    e = sra::launch_attn_bf16(D, n_req, Hq, Hkv, R, L, reinterpret_cast<const uint16_t*>(wsp(ws, p.qop)),
                              p.qop_blocks, row_pos, reinterpret_cast<const uint16_t*>(wsp(ws, p.k16)),
                              (const uint16_t*)kf, (const uint16_t*)vf,
                              (uint16_t*)out, lse, p.pieces, reinterpret_cast<int*>(wsp(ws, p.tilecum)),
                              reinterpret_cast<uint16_t*>(wsp(ws, p.part_o)),
                              reinterpret_cast<float4*>(wsp(ws, p.part_ml)), ex, st);
  } else {
    e = sra::launch_attn_f32(D, n_req, Hq, Hkv, R, L, (const float*)q, q_rows, indexed, row_pos,
                             reinterpret_cast<const float2*>(wsp(ws, p.cs)), (const float*)kf,
                             (const float*)vf, (float*)out, lse, st);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return SRA_OK;
}

float attn_scale_log2(int D) { return 1.4426950408889634f / std::sqrt((float)D); }

int check_attn_limits(const sra_shape* s, int R, int L) {
  if (s->dtype == SRA_DTYPE_F32 && s->n_q_heads / s->n_kv_heads > 16)
    return fail(SRA_E_LIMIT, "float32 attention supports at most 16 query heads per KV head");
  if (s->dtype == SRA_DTYPE_BF16 &&
      ceil_div((int64_t)R * (s->n_q_heads / s->n_kv_heads), 128) > sra::kAttnMaxTiles)
    return fail(SRA_E_LIMIT, "bf16 attention supports at most %d query vectors per KV head and request",
                sra::kAttnMaxTiles * 128);
  // the bf16 kernel addresses one request's K/V rows and output rows with 32-bit offsets
  if (s->dtype == SRA_DTYPE_BF16 && (int64_t)L * s->n_kv_heads * s->head_dim * 2 > (int64_t)UINT32_MAX)
    return fail(SRA_E_LIMIT, "bf16 attention: one request's fused K or V exceeds 4 GiB");
  if (s->dtype == SRA_DTYPE_BF16 && (int64_t)R * s->n_q_heads * s->head_dim > (int64_t)INT32_MAX)
    return fail(SRA_E_LIMIT, "bf16 attention: one request's output exceeds 2^31 elements");
  return SRA_OK;
}

int check_score_limits(const sra_shape* s, int n_req, int n_chunks, int Lq) {
  const int g = s->n_q_heads / s->n_kv_heads;
  if (n_req > sra::kMaxEntries) return fail(SRA_E_LIMIT, "at most %d requests per scoring call", sra::kMaxEntries);
  if (s->dtype == SRA_DTYPE_BF16 && (int64_t)Lq * g > 2048)
    return fail(SRA_E_LIMIT, "query rows x group size (%lld) exceeds 2048", (long long)Lq * g);
  if (s->dtype == SRA_DTYPE_F32 && (int64_t)n_req * n_chunks > sra::kMaxEntries)
    return fail(SRA_E_LIMIT, "float32 scoring supports at most %d chunks per call", sra::kMaxEntries);
  return SRA_OK;
}

}  // namespace

// ==================================================================================== C ABI
extern "C" {

const char* sra_error_string(int status) {
  switch (status) {
    case SRA_OK: return "success";
    case SRA_E_NULL: return "a required pointer is NULL";
    case SRA_E_SHAPE: return "invalid sizes or shape";
    case SRA_E_CHUNKS: return "invalid chunk table";
    case SRA_E_ALIAS: return "an input overlaps an output";
    case SRA_E_WORKSPACE: return "workspace missing or too small";
    case SRA_E_DTYPE: return "unknown dtype";
    case SRA_E_ROWS: return "row positions unsorted, duplicated or out of range";
    case SRA_E_HIP: return "HIP runtime error";
    case SRA_E_LIMIT: return "size exceeds an implementation limit";
    default: return "unknown status";
  }
}

const char* sra_last_error(void) { return g_last_error.c_str(); }

int sra_select_count(int64_t num, int64_t den, int32_t ctx_len, int32_t* n_out) {
  if (!n_out) return fail(SRA_E_NULL, "n_out is NULL");
  if (num < 0 || den <= 0 || ctx_len < 0) return fail(SRA_E_SHAPE, "need num >= 0, den > 0, ctx_len >= 0");
  if (num > (int64_t)1 << 31) return fail(SRA_E_SHAPE, "num too large");
  const int64_t prod = num * (int64_t)ctx_len;
  const int64_t n = (prod + den - 1) / den;
  if (n > ctx_len) return fail(SRA_E_SHAPE, "ratio %lld/%lld exceeds 1", (long long)num, (long long)den);
  *n_out = (int32_t)n;
  return ok();
}

size_t sra_workspace_size(const sra_shape* shape, int32_t n_req, int32_t n_chunks, int32_t L,
                          int32_t R, int32_t Lq) {
  if (!shape || shape->n_kv_heads <= 0 || shape->n_q_heads <= 0 ||
      shape->n_q_heads % shape->n_kv_heads != 0 || (shape->head_dim != 64 && shape->head_dim != 128) ||
      (shape->dtype != SRA_DTYPE_BF16 && shape->dtype != SRA_DTYPE_F32) || n_req <= 0 ||
      n_chunks <= 0 || L <= 0 || R < 0 || Lq < 0 || Lq > L)
    return 0;
  return make_plan(shape, n_req, n_chunks, L, R, Lq).total;
}

int sra_fuse_rerotate(const sra_shape* shape, int32_t n_req, const void* k_store, const void* v_store,
                      int64_t store_rows, const sra_chunk* chunks, int32_t n_chunks, void* k_fused,
                      void* v_fused, int32_t L, hipStream_t stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if (n_req <= 0) return fail(SRA_E_SHAPE, "n_req must be positive");
  if ((rc = check_ptr(k_store, "k_store")) || (rc = check_ptr(v_store, "v_store")) ||
      (rc = check_ptr(k_fused, "k_fused")) || (rc = check_ptr(v_fused, "v_fused")))
    return rc;
  int Lctx = 0;
  if ((rc = check_chunks(chunks, n_req, n_chunks, store_rows, &Lctx))) return rc;
  if (Lctx > L) return fail(SRA_E_SHAPE, "context length %d exceeds L = %d", Lctx, L);
  const size_t es = elem_size(shape), row = (size_t)shape->n_kv_heads * shape->head_dim * es;
  const size_t sb = (size_t)store_rows * row, fb = (size_t)n_req * L * row;
  if (overlap(k_store, sb, k_fused, fb) || overlap(k_store, sb, v_fused, fb) ||
      overlap(v_store, sb, k_fused, fb) || overlap(v_store, sb, v_fused, fb) ||
      overlap(k_fused, fb, v_fused, fb))
    return fail(SRA_E_ALIAS, "chunk store and fused cache buffers overlap");
  if ((rc = do_rerotate(shape, n_req, k_store, v_store, chunks, n_chunks, k_fused, v_fused, L, stream)))
    return rc;
  return ok();
}

int sra_extract_anchors(const sra_shape* shape, const void* k_store, int64_t store_rows,
                        const sra_chunk* chunks, int32_t n_chunks, int32_t k, int32_t* anchor_rows,
                        float* norms, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if ((rc = check_ptr(k_store, "k_store"))) return rc;
  if (!anchor_rows) return fail(SRA_E_NULL, "anchor_rows is NULL");
  if (!chunks) return fail(SRA_E_NULL, "chunks is NULL");
  if (n_chunks <= 0) return fail(SRA_E_SHAPE, "n_chunks must be positive");
  if (k < 1) return fail(SRA_E_SHAPE, "k must be >= 1");
  if (k > SRA_MAX_ANCHOR_K) return fail(SRA_E_LIMIT, "k = %d exceeds %d", k, SRA_MAX_ANCHOR_K);
  if (shape->n_kv_heads > 256) return fail(SRA_E_LIMIT, "anchors support at most 256 KV heads");
  const int rpb = sra::anchor_rows_per_block(shape->n_kv_heads);
  std::vector<Entry> ents;
  int64_t total = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const sra_chunk& ch = chunks[c];
    if (ch.src_row < 0 || ch.n_tokens < 0 || (int64_t)ch.src_row + ch.n_tokens > store_rows)
      return fail(SRA_E_CHUNKS, "chunk %d reads outside the store", c);
    if (ch.n_tokens < k) return fail(SRA_E_SHAPE, "chunk %d has %d tokens < k = %d", c, ch.n_tokens, k);
    // dst: output slot; delta: offset of the chunk's sums of squares in the workspace
    ents.push_back({0, ch.src_row, ch.n_tokens, c, (int)total, (int)ceil_div(ch.n_tokens, rpb), c});
    total += ch.n_tokens;
  }
  if (total > std::numeric_limits<int32_t>::max()) return fail(SRA_E_LIMIT, "too many chunk tokens");
  if ((rc = check_ws(ws, ws_bytes, (size_t)total * sizeof(double)))) return rc;
  double* ss = static_cast<double*>(ws);
  hipError_t e = for_each_tab(ents, [&](const sra::ChunkTab& tab, int, int) {
    return sra::launch_anchors(shape->dtype, shape->n_kv_heads, shape->head_dim, tab, k, k_store, ss,
                               anchor_rows, norms, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "anchor launch");
  return ok();
}

int sra_anchor_prefix(const sra_shape* shape, int32_t n_req, const void* k_store, const void* v_store,
                      int64_t store_rows, const sra_chunk* chunks, int32_t n_chunks, const int32_t* anchor_rows,
                      int32_t k, void* k_probe, void* v_probe, int32_t L_probe, hipStream_t stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if (n_req <= 0 || n_chunks <= 0) return fail(SRA_E_SHAPE, "need n_req > 0 and n_chunks > 0");
  if ((rc = check_ptr(k_store, "k_store")) || (rc = check_ptr(v_store, "v_store")) ||
      (rc = check_ptr(k_probe, "k_probe")) || (rc = check_ptr(v_probe, "v_probe")))
    return rc;
  if (!anchor_rows || !chunks) return fail(SRA_E_NULL, "anchor_rows or chunks is NULL");
  if (k < 1) return fail(SRA_E_SHAPE, "k must be >= 1");
  if (k > SRA_MAX_ANCHOR_K) return fail(SRA_E_LIMIT, "k = %d exceeds %d", k, SRA_MAX_ANCHOR_K);
  if ((int64_t)n_chunks * k > L_probe) return fail(SRA_E_SHAPE, "prefix of %lld rows exceeds L_probe = %d",
                                                   (long long)n_chunks * k, L_probe);
  std::vector<Entry> ents;
  for (int q = 0; q < n_req; ++q)
    for (int c = 0; c < n_chunks; ++c) {
      const sra_chunk& ch = chunks[(int64_t)q * n_chunks + c];
      if (ch.src_row < 0 || ch.n_tokens < 0 || (int64_t)ch.src_row + ch.n_tokens > store_rows)
        return fail(SRA_E_CHUNKS, "chunk %d of request %d reads outside the store", c, q);
      if (ch.n_tokens < k) return fail(SRA_E_SHAPE, "chunk %d has %d tokens < k = %d", c, ch.n_tokens, k);
      ents.push_back({q, ch.src_row, ch.n_tokens, c * k, ch.orig_pos, k, c});
    }
  const size_t row = (size_t)shape->n_kv_heads * shape->head_dim * elem_size(shape);
  const size_t sb = (size_t)store_rows * row, pb = (size_t)n_req * L_probe * row;
  if (overlap(k_store, sb, k_probe, pb) || overlap(k_store, sb, v_probe, pb) || overlap(v_store, sb, k_probe, pb) ||
      overlap(v_store, sb, v_probe, pb) || overlap(k_probe, pb, v_probe, pb))
    return fail(SRA_E_ALIAS, "the store and the probe caches overlap");
  hipError_t e = for_each_tab(ents, [&](const sra::ChunkTab& tab, int, int) {
    return sra::launch_anchor_prefix(shape->dtype, shape->head_dim, shape->n_kv_heads, tab, k, n_chunks,
                                     anchor_rows, k_store, v_store, k_probe, v_probe, L_probe, shape->rope_base,
                                     stream);
  });
  if (e != hipSuccess) return hip_fail(e, "anchor prefix launch");
  return ok();
}

}  // extern "C"

namespace {
struct StatsPlan {
  int n_tiles = 0, qop_blocks = 0;
  size_t qop = 0, fx = 0, total = 0;
};
StatsPlan stats_plan(const sra_shape* s, int n_req, int Lctx, int n_chunks) {
  StatsPlan p;
  const int g = s->n_q_heads / s->n_kv_heads;
  p.n_tiles = (int)ceil_div((int64_t)Lctx * g, 128);
  p.qop_blocks = 4 * p.n_tiles;
  size_t o = 0;
  p.qop = o; o = align256(o + (size_t)n_req * s->n_kv_heads * p.qop_blocks * 32 * 2 * s->head_dim * sizeof(uint16_t));
  p.fx = o; o = align256(o + (size_t)n_req * Lctx * n_chunks * sizeof(unsigned long long));
  p.total = o;
  return p;
}
}  // namespace

extern "C" {

size_t sra_stats_workspace_size(const sra_shape* shape, int32_t n_req, int32_t ctx_len, int32_t n_chunks) {
  if (!shape || check_shape(shape) != SRA_OK || n_req <= 0 || ctx_len <= 0 || n_chunks <= 0) return 0;
  return stats_plan(shape, n_req, ctx_len, n_chunks).total;
}

int sra_chunk_attention_stats(const sra_shape* shape, int32_t n_req, const void* q_fresh, int32_t q_rows,
                              const void* k_cache, int32_t k_rows, const sra_chunk* chunks, int32_t n_chunks,
                              float* inter, float* token_scores, float* cci, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if (shape->dtype != SRA_DTYPE_BF16) return fail(SRA_E_DTYPE, "chunk attention statistics are bf16 only");
  if (n_req <= 0) return fail(SRA_E_SHAPE, "n_req must be positive");
  if ((rc = check_ptr(q_fresh, "q_fresh")) || (rc = check_ptr(k_cache, "k_cache"))) return rc;
  int Lctx = 0;
  if ((rc = check_chunks(chunks, n_req, n_chunks, std::numeric_limits<int32_t>::max(), &Lctx))) return rc;
  if (q_rows < Lctx || k_rows < Lctx) return fail(SRA_E_SHAPE, "q_rows %d and k_rows %d must cover the context %d",
                                                  q_rows, k_rows, Lctx);
  if (n_chunks > sra::kMaxEntries) return fail(SRA_E_LIMIT, "at most %d chunks per request", sra::kMaxEntries);
  if ((int64_t)Lctx * (shape->n_q_heads / shape->n_kv_heads) > (int64_t)sra::kAttnMaxTiles * 128)
    return fail(SRA_E_LIMIT, "context too long for the statistics kernel");
  const StatsPlan p = stats_plan(shape, n_req, Lctx, n_chunks);
  if ((rc = check_ws(ws, ws_bytes, p.total))) return rc;
  const size_t kb = (size_t)n_req * k_rows * shape->n_kv_heads * shape->head_dim * 2;
  const size_t fb = (size_t)n_req * Lctx * n_chunks * sizeof(float);
  if ((inter && (overlap(inter, fb, k_cache, kb) || overlap(inter, fb, ws, p.total))) ||
      (cci && overlap(cci, (size_t)n_req * n_chunks * sizeof(float), ws, p.total)) ||
      (token_scores && overlap(token_scores, (size_t)n_req * Lctx * sizeof(float), ws, p.total)) ||
      overlap(k_cache, kb, ws, p.total))
    return fail(SRA_E_ALIAS, "outputs overlap the inputs or the workspace");
  uint16_t* qop = reinterpret_cast<uint16_t*>(wsp(ws, p.qop));
  unsigned long long* fx = reinterpret_cast<unsigned long long*>(wsp(ws, p.fx));
  hipError_t e = hipMemsetAsync(fx, 0, (size_t)n_req * Lctx * n_chunks * sizeof(unsigned long long), stream);
  if (e != hipSuccess) return hip_fail(e, "statistics slots clear");
  // the query of every context token, rotated at its position and split hi/lo (identity rows)
  e = sra::launch_scatter(shape->dtype, shape->head_dim, shape->n_q_heads, shape->n_kv_heads, n_req, Lctx, Lctx,
                          q_fresh, nullptr, nullptr, q_rows, 1, nullptr, nullptr, nullptr, nullptr, qop,
                          p.qop_blocks, false, attn_scale_log2(shape->head_dim), shape->rope_base, stream);
  if (e != hipSuccess) return hip_fail(e, "query operand launch");
  const int per = std::max(1, sra::kMaxEntries / n_chunks);   // requests per launch
  for (int q0 = 0; q0 < n_req; q0 += per) {
    const int nq = std::min(per, n_req - q0);
    sra::ChunkTab tab;
    std::memset(&tab, 0, sizeof(tab));
    for (int q = q0; q < q0 + nq; ++q)
      for (int c = 0; c < n_chunks; ++c) {
        const sra_chunk& ch = chunks[(int64_t)q * n_chunks + c];
        tab.req[tab.n] = q;
        tab.dst[tab.n] = ch.dst_row;
        tab.len[tab.n] = ch.n_tokens;
        ++tab.n;
      }
    e = sra::launch_chunk_stats(shape->head_dim, nq, q0, shape->n_q_heads, shape->n_kv_heads, Lctx, k_rows, qop,
                                p.qop_blocks, reinterpret_cast<const uint16_t*>(k_cache), tab, n_chunks, fx, inter,
                                token_scores, cci, stream);
    if (e != hipSuccess) return hip_fail(e, "statistics launch");
  }
  return ok();
}

int sra_prefix_overlap(const double* inter_to_old, const int32_t* old_ids, int32_t n_old, const int32_t* new_ids,
                       int32_t n_new, double* beta_out) {
  if (!beta_out || (n_old > 0 && (!inter_to_old || !old_ids)) || (n_new > 0 && !new_ids))
    return fail(SRA_E_NULL, "a required array is NULL");
  if (n_old < 0 || n_new < 0) return fail(SRA_E_SHAPE, "negative prefix length");
  double den = 0.0, num = 0.0;
  std::vector<int> pos_new;   // position in the new prefix of each shared old chunk, in old order
  for (int i = 0; i < n_old; ++i) {
    den += inter_to_old[i];
    for (int j = 0; j < n_new; ++j)
      if (new_ids[j] == old_ids[i]) {
        num += inter_to_old[i];
        pos_new.push_back(j);
        break;
      }
  }
  if (den <= 0.0) {
    *beta_out = 0.0;
    return ok();
  }
  const int n = (int)pos_new.size();
  double gamma = 0.0;
  if (n >= 2) {
    int64_t disc = 0;
    for (int i = 0; i < n; ++i)
      for (int j = i + 1; j < n; ++j) disc += pos_new[i] > pos_new[j] ? 1 : 0;
    gamma = (double)disc / ((double)n * (n - 1) / 2.0);
  }
  *beta_out = num * (1.0 - gamma) / den;
  return ok();
}

int sra_cachecraft_count(double alpha, double cci, double beta, int32_t n_tokens, int32_t* n_out) {
  if (!n_out) return fail(SRA_E_NULL, "n_out is NULL");
  if (n_tokens < 0) return fail(SRA_E_SHAPE, "n_tokens must be >= 0");
  const double x = alpha * cci * (1.0 - beta) * (double)n_tokens;
  double n = std::ceil(x);
  n = std::min(std::max(n, 0.0), (double)n_tokens);
  *n_out = (int32_t)n;
  return ok();
}

int sra_score_select(const sra_shape* shape, int32_t n_req, const void* q_crit, int32_t Lq,
                     const void* k_crit_store, int64_t store_rows, const sra_chunk* chunks,
                     int32_t n_chunks, int32_t n_select, const int32_t* chunk_quota, float* scores,
                     int32_t* row_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if (n_req <= 0) return fail(SRA_E_SHAPE, "n_req must be positive");
  if (Lq < 1) return fail(SRA_E_SHAPE, "scoring needs at least one query row");
  if ((rc = check_ptr(q_crit, "q_crit")) || (rc = check_ptr(k_crit_store, "k_crit_store"))) return rc;
  if (!row_pos) return fail(SRA_E_NULL, "row_pos is NULL");
  int Lctx = 0, N = 0;
  if ((rc = check_chunks(chunks, n_req, n_chunks, store_rows, &Lctx))) return rc;
  if (Lctx < 1) return fail(SRA_E_SHAPE, "empty context");
  if ((rc = check_score_limits(shape, n_req, n_chunks, Lq))) return rc;
  if ((rc = resolve_count(n_req, n_chunks, chunks, Lctx, n_select, chunk_quota, &N))) return rc;
  const Plan p = make_plan(shape, n_req, n_chunks, Lctx + Lq, N + Lq, Lq);
  if ((rc = check_ws(ws, ws_bytes, p.score_end))) return rc;
  if ((rc = do_score_select(shape, n_req, q_crit, Lq, k_crit_store, chunks, n_chunks, Lctx, N,
                            chunk_quota, scores, row_pos, ws, p, stream)))
    return rc;
  return ok();
}

int sra_select_topn(const float* scores, int32_t n_req, int32_t ctx_len, int32_t n_select,
                    const int32_t* chunk_quota, const sra_chunk* chunks, int32_t n_chunks,
                    int32_t Lq, int32_t* row_pos, hipStream_t stream) {
  if (!scores) return fail(SRA_E_NULL, "scores is NULL");
  if (!row_pos) return fail(SRA_E_NULL, "row_pos is NULL");
  if (n_req <= 0 || ctx_len < 1 || Lq < 0) return fail(SRA_E_SHAPE, "need n_req > 0, ctx_len > 0, Lq >= 0");
  int N = 0, rc;
  if (chunk_quota) {
    int Lctx = 0;
    if ((rc = check_chunks(chunks, n_req, n_chunks, std::numeric_limits<int32_t>::max(), &Lctx))) return rc;
    if (Lctx != ctx_len) return fail(SRA_E_CHUNKS, "chunks cover %d positions, ctx_len is %d", Lctx, ctx_len);
  }
  if ((rc = resolve_count(n_req, n_chunks, chunks, ctx_len, n_select, chunk_quota, &N))) return rc;
  if ((rc = do_select(n_req, ctx_len, Lq, N + Lq, N, chunk_quota, chunks, n_chunks, nullptr, 0, nullptr,
                      const_cast<float*>(scores), row_pos, stream)))
    return rc;
  return ok();
}

int sra_select_topn_nested(const float* scores, int32_t n_req, int32_t ctx_len, const int32_t* prev_rows,
                           int32_t prev_stride, int32_t n_prev, int32_t Lq, int32_t n_levels,
                           const int32_t* n_select, int32_t* const* row_pos, hipStream_t stream) {
  if (!scores) return fail(SRA_E_NULL, "scores is NULL");
  if (!prev_rows) return fail(SRA_E_NULL, "prev_rows is NULL");
  if (!n_select || !row_pos) return fail(SRA_E_NULL, "n_select or row_pos is NULL");
  if (n_req <= 0 || ctx_len < 1 || Lq < 0 || n_levels < 1 || n_prev < 0 || n_prev > ctx_len)
    return fail(SRA_E_SHAPE, "need n_req > 0, ctx_len > 0, Lq >= 0, n_levels > 0, 0 <= n_prev <= ctx_len");
  if ((int64_t)prev_stride < (int64_t)n_prev + Lq)
    return fail(SRA_E_SHAPE, "prev_stride %d is below n_prev + Lq = %lld", prev_stride, (long long)n_prev + Lq);
  const size_t pb = ((size_t)(n_req - 1) * prev_stride + n_prev + Lq) * sizeof(int32_t);
  for (int l = 0; l < n_levels; ++l) {
    if (n_select[l] < 0 || n_select[l] > n_prev)
      return fail(SRA_E_SHAPE, "level %d selects %d of %d rows", l, n_select[l], n_prev);
    if (!row_pos[l]) return fail(SRA_E_NULL, "row_pos[%d] is NULL", l);
    if (overlap(row_pos[l], (size_t)n_req * (n_select[l] + Lq) * sizeof(int32_t), prev_rows, pb))
      return fail(SRA_E_ALIAS, "row_pos[%d] overlaps prev_rows", l);
  }
  // one selection unit per (level, request): the unit's indices are prev_rows' entries
  sra::SelTab tab;
  std::memset(&tab, 0, sizeof(tab));
  auto flush = [&]() -> int {
    hipError_t e = sra::launch_select(tab, nullptr, 0, n_prev, Lq, ctx_len, nullptr, const_cast<float*>(scores),
                                      stream, prev_rows, prev_stride, true);
    if (e != hipSuccess) return hip_fail(e, "selection launch");
    std::memset(&tab, 0, sizeof(tab));
    return SRA_OK;
  };
  int rc;
  for (int l = 0; l < n_levels; ++l)
    for (int q = 0; q < n_req; ++q) {
      tab.req[tab.n] = q;
      tab.begin[tab.n] = 0;
      tab.len[tab.n] = n_prev;
      tab.quota[tab.n] = n_select[l];
      tab.out_off[tab.n] = 0;
      tab.writes_query[tab.n] = 1;
      tab.out[tab.n] = row_pos[l] + (int64_t)q * (n_select[l] + Lq);
      tab.rows[tab.n] = n_select[l] + Lq;
      if (++tab.n == sra::kMaxEntries && (rc = flush())) return rc;
    }
  if (tab.n > 0 && (rc = flush())) return rc;
  return ok();
}

int sra_scatter_kv(const sra_shape* shape, int32_t n_req, const void* k_new, const void* v_new,
                   const int32_t* row_pos, int32_t R, void* k_fused, void* v_fused, int32_t L,
                   hipStream_t stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if (n_req <= 0 || R < 0 || L <= 0 || R > L) return fail(SRA_E_SHAPE, "need n_req > 0, 0 <= R <= L");
  if ((rc = check_ptr(k_new, "k_new")) || (rc = check_ptr(v_new, "v_new")) ||
      (rc = check_ptr(k_fused, "k_fused")) || (rc = check_ptr(v_fused, "v_fused")))
    return rc;
  if (!row_pos) return fail(SRA_E_NULL, "row_pos is NULL");
  const size_t row = (size_t)shape->n_kv_heads * shape->head_dim * elem_size(shape);
  const size_t nb = (size_t)n_req * R * row, fb = (size_t)n_req * L * row;
  if (overlap(k_new, nb, k_fused, fb) || overlap(k_new, nb, v_fused, fb) || overlap(v_new, nb, k_fused, fb) ||
      overlap(v_new, nb, v_fused, fb) || overlap(k_fused, fb, v_fused, fb))
    return fail(SRA_E_ALIAS, "fresh rows and fused cache overlap");
  hipError_t e = sra::launch_scatter(shape->dtype, shape->head_dim, shape->n_q_heads, shape->n_kv_heads,
                                     n_req, R, L, nullptr, k_new, v_new, R, 0, row_pos, k_fused, v_fused,
                                     nullptr, nullptr, 0, false, 0.f, shape->rope_base, stream);
  if (e != hipSuccess) return hip_fail(e, "scatter launch");
  return ok();
}

int sra_hkvd_select(const sra_shape* shape, int32_t n_req, const void* k_fused, const void* v_fused,
                    int32_t L, const void* k_new, const void* v_new, const int32_t* row_pos_prev,
                    int32_t R_prev, int32_t n_prev, int32_t n_keep, float* dev, int32_t* row_pos_next,
                    hipStream_t stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if (n_req <= 0 || L <= 0 || n_prev < 0 || R_prev < n_prev || R_prev > L || n_keep < 0 || n_keep > n_prev)
    return fail(SRA_E_SHAPE, "need n_req > 0, 0 <= n_keep <= n_prev <= R_prev <= L");
  if ((rc = check_ptr(k_fused, "k_fused")) || (rc = check_ptr(v_fused, "v_fused")) ||
      (rc = check_ptr(k_new, "k_new")) || (rc = check_ptr(v_new, "v_new")))
    return rc;
  if (!row_pos_prev || !row_pos_next || !dev) return fail(SRA_E_NULL, "row_pos_prev, row_pos_next or dev is NULL");
  const size_t ib = (size_t)n_req * R_prev * sizeof(int32_t);
  const size_t ob = (size_t)n_req * (n_keep + (R_prev - n_prev)) * sizeof(int32_t);
  const size_t db = (size_t)n_req * n_prev * sizeof(float);
  if (overlap(row_pos_prev, ib, row_pos_next, ob) || overlap(dev, db, row_pos_next, ob) ||
      overlap(dev, db, row_pos_prev, ib))
    return fail(SRA_E_ALIAS, "row_pos_prev, row_pos_next and dev must not overlap");
  if ((rc = do_hkvd(shape, n_req, k_new, v_new, R_prev, 0, row_pos_prev, R_prev, n_prev, k_fused, v_fused, L,
                    n_keep, dev, row_pos_next, stream)))
    return rc;
  return ok();
}

int sra_sparse_causal_attn(const sra_shape* shape, int32_t n_req, const void* q_new,
                           const int32_t* row_pos, int32_t R, const void* k_fused,
                           const void* v_fused, int32_t L, void* out, float* lse, int32_t* fallback,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if (n_req <= 0 || R < 0 || L <= 0 || R > L) return fail(SRA_E_SHAPE, "need n_req > 0, 0 <= R <= L");
  if ((rc = check_ptr(q_new, "q_new")) || (rc = check_ptr(k_fused, "k_fused")) ||
      (rc = check_ptr(v_fused, "v_fused")) || (rc = check_ptr(out, "out")))
    return rc;
  if (!row_pos) return fail(SRA_E_NULL, "row_pos is NULL");
  if ((rc = check_attn_limits(shape, R, L))) return rc;
  const size_t es = elem_size(shape);
  const size_t ob = (size_t)n_req * R * shape->n_q_heads * shape->head_dim * es;
  const size_t fb = (size_t)n_req * L * shape->n_kv_heads * shape->head_dim * es;
  if (overlap(out, ob, k_fused, fb) || overlap(out, ob, v_fused, fb) || overlap(out, ob, q_new, ob))
    return fail(SRA_E_ALIAS, "out overlaps an input");
  const Plan p = make_plan(shape, n_req, 1, L, R, 1);
  if ((rc = check_ws(ws, ws_bytes, p.attn_end))) return rc;
  if (fallback && overlap(fallback, (size_t)n_req * shape->n_kv_heads * sizeof(int32_t), out, ob))
    return fail(SRA_E_ALIAS, "fallback overlaps out");
  const unsigned call_id = next_call_id();
  const sra::F16Shadow sh = shadow_of(shape, ws, p, call_id);
  hipError_t e;
  if (shape->dtype == SRA_DTYPE_BF16) {
    // the caller's keys: their fp16 copy first (flagging keys beyond fp16), then the query operand
    e = sra::launch_k_to_f16(shape->head_dim, shape->n_kv_heads, n_req, L, (const uint16_t*)k_fused, sh, stream);
    if (e == hipSuccess)
      e = sra::launch_scatter(shape->dtype, shape->head_dim, shape->n_q_heads, shape->n_kv_heads, n_req, R, L,
                              q_new, nullptr, nullptr, R, 0, row_pos, nullptr, nullptr, nullptr,
                              reinterpret_cast<uint16_t*>(wsp(ws, p.qop)), p.qop_blocks, true,
                              attn_scale_log2(shape->head_dim), shape->rope_base, stream, sh);
  } else {
    e = sra::launch_rope_table(shape->head_dim, n_req, R, row_pos, reinterpret_cast<float2*>(wsp(ws, p.cs)),
                               shape->rope_base, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "attention row-input launch");
  if ((rc = do_attn(shape, n_req, q_new, R, 0, row_pos, R, k_fused, v_fused, L, out, lse, ws, p, stream, call_id,
                    fallback)))
    return rc;
  return ok();
}

}  // extern "C"

namespace {

// Validates one layer's arguments and, unless dry, enqueues its stages on `stream`.
int fused_layer_impl(const sra_layer_args* a, void* ws, size_t ws_bytes, hipStream_t stream, bool dry) {
  int rc;
  if (!a) return fail(SRA_E_NULL, "args is NULL");
  const sra_shape* s = &a->shape;
  if ((rc = check_shape(s))) return rc;
  const int n_req = a->n_req, L = a->total_len, Lq = a->query_len, R = a->n_rows;
  if (n_req <= 0 || Lq < 0 || L <= 0) return fail(SRA_E_SHAPE, "need n_req > 0, query_len >= 0, total_len > 0");
  if ((rc = check_ptr(a->k_store, "k_store")) || (rc = check_ptr(a->v_store, "v_store")) ||
      (rc = check_ptr(a->q_fresh, "q_fresh")) || (rc = check_ptr(a->k_fresh, "k_fresh")) ||
      (rc = check_ptr(a->v_fresh, "v_fresh")) || (rc = check_ptr(a->k_fused, "k_fused")) ||
      (rc = check_ptr(a->v_fused, "v_fused")) || (rc = check_ptr(a->out, "out")))
    return rc;
  if (!a->row_pos) return fail(SRA_E_NULL, "row_pos is NULL");
  int Lctx = 0;
  if ((rc = check_chunks(a->chunks, n_req, a->n_chunks, a->store_rows, &Lctx))) return rc;
  if (Lctx + Lq != L) return fail(SRA_E_SHAPE, "total_len %d != context %d + query %d", L, Lctx, Lq);
  if (R < Lq || R > L) return fail(SRA_E_SHAPE, "n_rows %d outside [query_len, total_len]", R);
  if ((rc = check_attn_limits(s, R, L))) return rc;
  const size_t es = elem_size(s);
  const size_t kvrow = (size_t)s->n_kv_heads * s->head_dim * es;
  const size_t sb = (size_t)a->store_rows * kvrow, fb = (size_t)n_req * L * kvrow;
  const size_t ob = (size_t)n_req * R * s->n_q_heads * s->head_dim * es;
  if (overlap(a->k_store, sb, a->k_fused, fb) || overlap(a->k_store, sb, a->v_fused, fb) ||
      overlap(a->v_store, sb, a->k_fused, fb) || overlap(a->v_store, sb, a->v_fused, fb) ||
      overlap(a->k_fused, fb, a->v_fused, fb) || overlap(a->out, ob, a->k_fused, fb) ||
      overlap(a->out, ob, a->v_fused, fb) || overlap(a->k_fresh, fb, a->k_fused, fb) ||
      overlap(a->v_fresh, fb, a->v_fused, fb) || overlap(a->k_fresh, fb, a->v_fused, fb) ||
      overlap(a->v_fresh, fb, a->k_fused, fb))
    return fail(SRA_E_ALIAS, "an input buffer overlaps an output buffer");
  int N = R - Lq;
  const bool hkvd = a->hkvd_prev != nullptr;
  if (hkvd) {
    if (a->q_crit) return fail(SRA_E_SHAPE, "gradual filtering and scoring are exclusive: q_crit must be NULL");
    if (!a->hkvd_dev) return fail(SRA_E_NULL, "hkvd_dev is NULL");
    const int npv = a->hkvd_prev_ctx;
    if (npv < 0 || a->hkvd_prev_rows != npv + Lq || npv > Lctx)
      return fail(SRA_E_SHAPE, "hkvd_prev_rows %d != hkvd_prev_ctx %d + query %d", a->hkvd_prev_rows, npv, Lq);
    if (a->n_select < 0 || a->n_select > npv)
      return fail(SRA_E_SHAPE, "n_select %d outside [0, hkvd_prev_ctx = %d]", a->n_select, npv);
    N = a->n_select;
    if (N + Lq != R) return fail(SRA_E_SHAPE, "n_rows %d != kept %d + query %d", R, N, Lq);
    const size_t ib = (size_t)n_req * a->hkvd_prev_rows * sizeof(int32_t), rb = (size_t)n_req * R * sizeof(int32_t);
    if (overlap(a->hkvd_prev, ib, a->row_pos, rb)) return fail(SRA_E_ALIAS, "hkvd_prev overlaps row_pos");
  }
  if (a->q_crit) {
    if (Lq < 1) return fail(SRA_E_SHAPE, "scoring needs at least one query row");
    if ((rc = check_ptr(a->k_crit_store, "k_crit_store"))) return rc;
    int Lc2 = 0;
    if ((rc = check_chunks(a->chunks, n_req, a->n_chunks, a->crit_store_rows, &Lc2))) return rc;
    if ((rc = check_score_limits(s, n_req, a->n_chunks, Lq))) return rc;
    if ((rc = resolve_count(n_req, a->n_chunks, a->chunks, Lctx, a->n_select, a->chunk_quota, &N))) return rc;
    if (N + Lq != R) return fail(SRA_E_SHAPE, "n_rows %d != selected %d + query %d", R, N, Lq);
  }
  const int ak = a->anchors_k;
  bool anchors_fused = false;
  if (ak != 0) {
    if (!a->q_crit) return fail(SRA_E_SHAPE, "anchors are taken with the scoring: q_crit is NULL");
    if (ak < 1) return fail(SRA_E_SHAPE, "anchors_k must be >= 0");
    if (ak > SRA_MAX_ANCHOR_K) return fail(SRA_E_LIMIT, "anchors_k = %d exceeds %d", ak, SRA_MAX_ANCHOR_K);
    if (!a->anchor_rows) return fail(SRA_E_NULL, "anchor_rows is NULL");
    if (s->n_kv_heads > 256) return fail(SRA_E_LIMIT, "anchors support at most 256 KV heads");
    anchors_fused = s->dtype == SRA_DTYPE_BF16;
    for (int64_t i = 0; i < (int64_t)n_req * a->n_chunks; ++i) {
      const int nt = a->chunks[i].n_tokens;
      if (nt < ak) return fail(SRA_E_SHAPE, "chunk %lld has %d tokens < anchors_k = %d", (long long)i, nt, ak);
      if (nt > sra::kAnchorFusedMaxLen) anchors_fused = false;
    }
  }
  const Plan p = make_plan(s, n_req, a->n_chunks, L, R, Lq);
  const size_t need = a->q_crit ? p.total : p.attn_end;
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  if (dry) return SRA_OK;

  const unsigned call_id = next_call_id();
  const sra::F16Shadow sh = shadow_of(s, ws, p, call_id);
  hipEvent_t* ev = a->stage_events;
  auto mark = [&](int i) -> int {
    if (!ev) return SRA_OK;
    hipError_t er = hipEventRecord(ev[i], stream);
    return er == hipSuccess ? SRA_OK : hip_fail(er, "stage event record");
  };
  // One stream: a second stream's fork/join costs more host and GPU time than S1 || S2 saves.
  // With bfloat16 scoring, S1 runs as extra blocks of scoring pass 1 instead (pass 1 fills a
  // fraction of the chip), so S1's stage events then mark an empty interval.
  const bool s1_in_score = a->q_crit && s->dtype == SRA_DTYPE_BF16;
  sra::RerotFused rf;
  if (s1_in_score) {
    rf.ks = static_cast<const uint16_t*>(a->k_store);
    rf.vs = static_cast<const uint16_t*>(a->v_store);
    rf.kf = static_cast<uint16_t*>(a->k_fused);
    rf.vf = static_cast<uint16_t*>(a->v_fused);
    rf.L = L;
    rf.base = s->rope_base;
    rf.sh = sh;
  }
  if ((rc = mark(0))) return rc;
  if (!s1_in_score && (rc = do_rerotate(s, n_req, a->k_store, a->v_store, a->chunks, a->n_chunks, a->k_fused,
                                        a->v_fused, L, stream, sh)))
    return rc;
  if ((rc = mark(1)) || (rc = mark(2))) return rc;
  if (hkvd) {   // deviation against the re-rotated reused rows, before the scatter replaces them
    if ((rc = do_hkvd(s, n_req, a->k_fresh, a->v_fresh, L, 1, a->hkvd_prev, a->hkvd_prev_rows, a->hkvd_prev_ctx,
                      a->k_fused, a->v_fused, L, N, a->hkvd_dev, a->row_pos, stream)))
      return rc;
  }
  if (a->q_crit) {
    sra::AnchorOut anc;
    if (anchors_fused) {   // the scoring passes take the anchors from their own K loads
      anc.k = ak;
      anc.ssp = reinterpret_cast<double*>(wsp(ws, p.ssp));
      anc.stride = (int64_t)n_req * Lctx;
      anc.rows = a->anchor_rows;
      anc.norms = a->anchor_norms;
      anc.n_chunks = a->n_chunks;
    }
    if ((rc = do_score_select(s, n_req, a->q_crit, Lq, a->k_crit_store, a->chunks, a->n_chunks, Lctx,
                              N, a->chunk_quota, a->scores, a->row_pos, ws, p, stream, anc, rf)))
      return rc;
    if (ak > 0 && !anchors_fused) {   // the standalone kernels, over every (request, chunk)
      std::vector<Entry> ents;
      const int rpb = sra::anchor_rows_per_block(s->n_kv_heads);
      for (int q = 0; q < n_req; ++q)
        for (int c = 0; c < a->n_chunks; ++c) {
          const sra_chunk& k = a->chunks[(int64_t)q * a->n_chunks + c];
          ents.push_back({0, k.src_row, k.n_tokens, q * a->n_chunks + c, q * Lctx + k.dst_row,
                          (int)ceil_div(k.n_tokens, rpb), c});
        }
      double* ss = reinterpret_cast<double*>(wsp(ws, p.ssp));
      hipError_t e = for_each_tab(ents, [&](const sra::ChunkTab& tab, int, int) {
        return sra::launch_anchors(s->dtype, s->n_kv_heads, s->head_dim, tab, ak, a->k_crit_store, ss,
                                   a->anchor_rows, a->anchor_norms, stream);
      });
      if (e != hipSuccess) return hip_fail(e, "anchor launch");
    }
  }
  if ((rc = mark(3)) || (rc = mark(4))) return rc;
  // the scatter kernel also writes the attention's per-row inputs (query operand or angle table)
  const bool bf = s->dtype == SRA_DTYPE_BF16;
  hipError_t e = sra::launch_scatter(
      s->dtype, s->head_dim, s->n_q_heads, s->n_kv_heads, n_req, R, L, a->q_fresh, a->k_fresh, a->v_fresh,
      L, 1, a->row_pos, a->k_fused, a->v_fused, bf ? nullptr : reinterpret_cast<float2*>(wsp(ws, p.cs)),
      bf ? reinterpret_cast<uint16_t*>(wsp(ws, p.qop)) : nullptr, p.qop_blocks, true, attn_scale_log2(s->head_dim),
      s->rope_base, stream, sh);
  if (e != hipSuccess) return hip_fail(e, "scatter launch");
  if ((rc = mark(5)) || (rc = mark(6))) return rc;
  if ((rc = do_attn(s, n_req, a->q_fresh, L, 1, a->row_pos, R, a->k_fused, a->v_fused, L, a->out,
                    a->lse, ws, p, stream, call_id, a->attn_fallback)))
    return rc;

  if ((rc = mark(7))) return rc;
  return ok();
}

}  // namespace

extern "C" {

int sra_fused_layer(const sra_layer_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fused_layer_impl(a, ws, ws_bytes, stream, false);
}

}  // extern "C"

namespace {

// Scratch of sra_fused_layer_static: a file-scope device array, one copy per GPU held until the
// process ends. Host code never uses its name as an address: each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SRA_E_LIMIT, "device %d: the static scratch serves devices 0..%d", dev,
                                                 kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SRA_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SRA_OK;
}

}  // namespace

extern "C" {

int sra_fused_layer_static(const sra_layer_args* a, hipStream_t stream) {
  int rc;
  void* ws = nullptr;
  if ((rc = static_scratch(&ws))) return rc;
  // every argument check first (the scratch stands in for a workspace of unbounded size), then the
  // workspace this layer needs against the scratch
  if ((rc = fused_layer_impl(a, ws, std::numeric_limits<size_t>::max(), stream, true))) return rc;
  const Plan p = make_plan(&a->shape, a->n_req, a->n_chunks, a->total_len, a->n_rows, a->query_len);
  const size_t need = a->q_crit ? p.total : p.attn_end;
  if (need > kStaticScratchBytes)
    return fail(SRA_E_LIMIT, "this layer needs %zu bytes of scratch; the static scratch holds %zu (use sra_fused_layer "
                "with a workspace)", need, kStaticScratchBytes);
  return fused_layer_impl(a, ws, kStaticScratchBytes, stream, false);
}

int sra_pipelined_layers(const sra_layer_args* layers, int32_t n_layers, const void* const* host_k,
                         const void* const* host_v, size_t store_bytes, void* const* k_buf, void* const* v_buf,
                         int32_t n_buf, hipEvent_t* events, void* ws, size_t ws_bytes, hipStream_t stream,
                         hipStream_t copy_stream) {
  int rc;
  if (!layers || !host_k || !host_v || !k_buf || !v_buf || !events)
    return fail(SRA_E_NULL, "layers, host stores, buffers or events is NULL");
  if (n_layers < 1) return fail(SRA_E_SHAPE, "n_layers must be >= 1");
  if (n_buf < 2 || n_buf > 64) return fail(SRA_E_SHAPE, "n_buf must be in [2, 64]");
  std::vector<void*> bufs;
  for (int b = 0; b < n_buf; ++b) {
    if (!k_buf[b] || !v_buf[b]) return fail(SRA_E_NULL, "device store buffer %d is NULL", b);
    bufs.push_back(k_buf[b]);
    bufs.push_back(v_buf[b]);
  }
  for (int i = 0; i < 2 * n_buf; ++i)
    if (!events[i]) return fail(SRA_E_NULL, "event %d is NULL", i);
  for (size_t i = 0; i < bufs.size(); ++i)
    for (size_t j = i + 1; j < bufs.size(); ++j)
      if (overlap(bufs[i], store_bytes, bufs[j], store_bytes))
        return fail(SRA_E_ALIAS, "the device store buffers must be disjoint");
  std::vector<sra_layer_args> la(layers, layers + n_layers);
  std::vector<size_t> bytes(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    if (!host_k[l] || !host_v[l]) return fail(SRA_E_NULL, "host store of layer %d is NULL", l);
    la[l].k_store = k_buf[l % n_buf];
    la[l].v_store = v_buf[l % n_buf];
    if ((rc = check_shape(&la[l].shape))) return rc;
    bytes[l] = (size_t)la[l].store_rows * la[l].shape.n_kv_heads * la[l].shape.head_dim * elem_size(&la[l].shape);
    if (la[l].store_rows < 0 || bytes[l] > store_bytes)
      return fail(SRA_E_SHAPE, "layer %d's store (%zu bytes) exceeds the buffers (%zu)", l, bytes[l], store_bytes);
    const size_t es = elem_size(&la[l].shape);
    const size_t fb = (size_t)la[l].n_req * la[l].total_len * la[l].shape.n_kv_heads * la[l].shape.head_dim * es;
    const size_t ob = (size_t)la[l].n_req * la[l].n_rows * la[l].shape.n_q_heads * la[l].shape.head_dim * es;
    for (void* buf : bufs)
      if (overlap(buf, store_bytes, la[l].k_fused, fb) || overlap(buf, store_bytes, la[l].v_fused, fb) ||
          overlap(buf, store_bytes, la[l].out, ob))
        return fail(SRA_E_ALIAS, "layer %d writes into a store buffer", l);
    if ((rc = fused_layer_impl(&la[l], ws, ws_bytes, stream, true))) return rc;
  }
  hipEvent_t* copied = events;            // copied[b]: buffer b holds its newest layer's store
  hipEvent_t* stepped = events + n_buf;    // stepped[b]: the newest layer reading buffer b is done
  auto copy = [&](int l) -> int {
    const int b = l % n_buf;
    hipError_t e = hipSuccess;
    if (l >= n_buf) e = hipStreamWaitEvent(copy_stream, stepped[b], 0);   // layer l - n_buf is done with b
    if (e == hipSuccess) e = hipMemcpyAsync(k_buf[b], host_k[l], bytes[l], hipMemcpyHostToDevice, copy_stream);
    if (e == hipSuccess) e = hipMemcpyAsync(v_buf[b], host_v[l], bytes[l], hipMemcpyHostToDevice, copy_stream);
    if (e == hipSuccess) e = hipEventRecord(copied[b], copy_stream);
    return e == hipSuccess ? SRA_OK : hip_fail(e, "store prefetch");
  };
  // the buffers may still be read by work queued earlier on `stream` (a previous call): the
  // copies start after it
  hipError_t e0 = hipEventRecord(stepped[0], stream);
  if (e0 == hipSuccess) e0 = hipStreamWaitEvent(copy_stream, stepped[0], 0);
  if (e0 != hipSuccess) return hip_fail(e0, "join before the first copy");
  if ((rc = copy(0))) return rc;
  for (int l = 0; l < n_layers; ++l) {
    if (l + 1 < n_layers && (rc = copy(l + 1))) return rc;   // overlaps layer l's step
    hipError_t e = hipStreamWaitEvent(stream, copied[l % n_buf], 0);
    if (e != hipSuccess) return hip_fail(e, "wait for a layer's store");
    if ((rc = fused_layer_impl(&la[l], ws, ws_bytes, stream, false))) return rc;
    if (l + n_buf >= n_layers) continue;   // no later copy reuses this buffer
    e = hipEventRecord(stepped[l % n_buf], stream);
    if (e != hipSuccess) return hip_fail(e, "layer step event");
  }
  return ok();
}

int sra_check_rows(const int32_t* row_pos, int32_t n_req, int32_t R, int32_t L, int32_t* first_bad,
                   hipStream_t stream) {
  if (!row_pos) return fail(SRA_E_NULL, "row_pos is NULL");
  if (n_req <= 0 || R < 0 || L <= 0) return fail(SRA_E_SHAPE, "need n_req > 0, R >= 0, L > 0");
  int* d_bad = nullptr;
  hipError_t e = hipMalloc(&d_bad, sizeof(int));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc");
  int h_bad = std::numeric_limits<int>::max();
  e = hipMemcpyAsync(d_bad, &h_bad, sizeof(int), hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = sra::launch_check_rows(row_pos, n_req, R, L, d_bad, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(&h_bad, d_bad, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  const hipError_t ef = hipFree(d_bad);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return hip_fail(e, "row check");
  if (h_bad != std::numeric_limits<int>::max()) {
    if (first_bad) *first_bad = h_bad;
    return fail(SRA_E_ROWS, "row_pos[%d] breaks strictly increasing order or range [0, %d)", h_bad, L);
  }
  if (first_bad) *first_bad = -1;
  return ok();
}

}  // extern "C"
