// libmla C ABI: argument validation (before any HIP call), split planning,
// workspace carving and the kernel sequence of each entry point.
//
// Kernel sequences (equations of section 2.1 of the DeepSeek-V3
// paper-reading notes):
//   prefill: [c_Q | c_KV | k_R] = h [W_DQ; W_DKV; W_KR]^T  (RoPE on k_R, cache write)
//            q = c_Q [W_UQ; W_QR]^T                       (RoPE on q_R, head layout)
//            K_C = c_KV W_UK^T;  V^T = (c_KV W_UV^T)^T
//            o = causal flash attention;  u = o W_O^T
//   decode:  the same first two projections (cache append at len-n_q+i),
//            q_lat,i = W_UK,i^T q_C,i (absorption), split-KV attention over the
//            latent cache, combine, o_i = W_UV,i o_lat,i, u = o W_O^T.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace mla {
int gemm_bk(int dtype, int tile);
int gemm_bm(int dtype, int tile);
int skinny_nst_supported(int nst);
}

using namespace mla;

namespace {

const int kCUs = 256;  // MI355X compute units; the split plan targets one wave of workgroups

size_t esize(const mla_config *c) { return c->dtype == MLA_BF16 ? 2 : 4; }

// YaRN is on for any factor other than 0 and 1 (a zero-initialised config
// keeps plain RoPE)
bool yarn_on(const mla_config *c) { return c->yarn_factor != 0.0 && c->yarn_factor != 1.0; }

mla_status check_config(const mla_config *c) {
  if (!c) return MLA_ERR_NULL;
  if (c->dtype != MLA_FP32 && c->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (c->d_model <= 0 || c->n_heads <= 0 || c->d_nope <= 0 || c->d_rope <= 0 || c->d_v <= 0 ||
      c->d_c <= 0 || c->d_cq <= 0)
    return MLA_ERR_SHAPE;
  if (c->d_rope % 2 != 0) return MLA_ERR_SHAPE;
  if (!(c->rope_base > 0.0) || !isfinite(c->rope_base)) return MLA_ERR_SHAPE;
  if (yarn_on(c)) {
    if (!(c->yarn_factor > 1.0) || !isfinite(c->yarn_factor) || c->yarn_orig_len <= 0) return MLA_ERR_SHAPE;
    if (!(c->yarn_beta_slow > 0.0) || !(c->yarn_beta_fast > c->yarn_beta_slow) || !isfinite(c->yarn_beta_fast))
      return MLA_ERR_SHAPE;
  }
  if (c->d_rope / 2 > MLA_MAX_ROPE_PAIRS) return MLA_ERR_UNSUPPORTED;
  if ((long)c->n_heads * (c->d_nope + c->d_rope) > (1L << 24) || c->d_model > (1 << 20))
    return MLA_ERR_UNSUPPORTED;
  const int big = c->dtype == MLA_BF16 ? 64 : 32, small = c->dtype == MLA_BF16 ? 32 : 16;
  if (c->d_model % big || c->d_cq % big || c->d_c % big || c->d_nope % big ||
      ((long)c->n_heads * c->d_v) % big || c->d_rope % small || c->d_v % small)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

bool attention_supported(const mla_config *c, int op) {
  if (c->dtype == MLA_BF16) {
    if (op == MLA_OP_PREFILL) return c->d_nope == 128 && c->d_rope == 64 && c->d_v == 128;
    return c->d_c == 512 && c->d_rope == 64;
  }
  if (op == MLA_OP_PREFILL) return c->d_nope == 32 && c->d_rope == 16 && c->d_v == 32;
  return c->d_c == 64 && c->d_rope == 16;
}

mla_status check_weights(const mla_weights *w) {
  if (!w) return MLA_ERR_NULL;
  if (!w->w_dq || !w->w_uq || !w->w_qr || !w->w_dkv || !w->w_kr || !w->w_uk || !w->w_uv || !w->w_o)
    return MLA_ERR_NULL;
  return MLA_OK;
}

// The cache must hold positions [0, need_len) of sequences [0, batch).
mla_status check_cache(const mla_cache *k, int32_t batch, int64_t need_len) {
  if (!k) return MLA_ERR_NULL;
  if (!k->pool) return MLA_ERR_NULL;
  if (k->block_table) {
    if (k->block_size <= 0 || k->n_blocks <= 0 || k->max_blocks_per_seq <= 0) return MLA_ERR_CACHE;
    if ((int64_t)k->max_blocks_per_seq * k->block_size < need_len) return MLA_ERR_CACHE;
    if ((int64_t)k->n_blocks * k->block_size > (int64_t)INT32_MAX * 4) return MLA_ERR_CACHE;
  } else {
    if (k->max_len <= 0 || k->max_len < need_len) return MLA_ERR_CACHE;
  }
  (void)batch;
  return MLA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// Workspace plans
// ---------------------------------------------------------------------------
struct PrefillPlan {
  size_t c_q, ckv, kr, q, k, vt, o, flags, total;
};
PrefillPlan plan_prefill(const mla_config *c, int64_t T) {
  const size_t e = esize(c);
  PrefillPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  p.c_q = take((size_t)T * c->d_cq * e);
  p.ckv = take((size_t)T * c->d_c * e);
  p.kr = take((size_t)T * c->d_rope * e);
  p.q = take((size_t)T * c->n_heads * (c->d_nope + c->d_rope) * e);
  p.k = take((size_t)T * c->n_heads * c->d_nope * e);
  p.vt = take((size_t)T * c->n_heads * c->d_v * e);
  p.o = take((size_t)T * c->n_heads * c->d_v * e);
  p.flags = take((size_t)T * c->n_heads);
  p.total = off;
  return p;
}

struct SplitK { int splits, k_chunk; };

// 256x256 tiles (bf16) unless they would leave all but a few CUs idle: a
// few hundred tokens against a narrow weight (a 512-token chunk: 18 tiles for
// the down projection) go to the 32x64-tile kernel, which spreads over every
// CU (180 -> 90 us there); from 32 tiles on the big tiles win (W_O at 512
// tokens, 56 tiles: 362 against 393 us).
int gemm_tile_for(int dtype, int64_t M, int64_t N, int64_t batch) {
  if (dtype != MLA_BF16 || M < 256) return TILE_SKINNY;
  return ((M + 255) / 256) * ((N + 255) / 256) * batch >= kCUs / 8 ? TILE_BIG : TILE_SKINNY;
}

// Split K only as far as needed for about two workgroups per CU: the
// weight-streaming kernel (bf16, up to 128 tokens) works on 64-feature tiles
// and 256-wide k stages (128 above 64 tokens); other shapes use 32x64 tiles.
SplitK choose_splitk(int dtype, int64_t M, int64_t N, int64_t K, int batch) {
  SplitK r;
  r.splits = 1;
  r.k_chunk = (int)K;
  const int tile = gemm_tile_for(dtype, M, N, batch);
  if (tile != TILE_SKINNY) return r;
  int bk, bn;
  if (dtype == MLA_BF16 && M <= 128) {
    bk = M <= 64 ? 256 : 128;
    bn = 64;
    if (K % bk) { bk = gemm_bk(dtype, tile); bn = 64; }
  } else {
    bk = gemm_bk(dtype, tile);
    bn = dtype == MLA_BF16 ? 64 : 32;
  }
  const int bm = dtype == MLA_BF16 && M <= 128 ? (int)M : gemm_bm(dtype, tile);
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * batch;
  const int64_t nkt = K / bk;
  const int64_t want = std::max<int64_t>(1, (2 * kCUs) / tiles);
  const bool stream = dtype == MLA_BF16 && M <= 128 && K % bk == 0;
  for (int64_t s = 1; s <= nkt && s <= 32; ++s)
    if (nkt % s == 0 && s <= want && (!stream || skinny_nst_supported((int)(nkt / s)))) r.splits = (int)s;
  r.k_chunk = (int)(K / r.splits);
  return r;
}

struct DecodePlan {
  int splits, chunk, row_groups, rows;
  SplitK sk1, sk2, sk5;
  size_t c_q, q_nope, q_abs, o_part, lse, o_lat, o, partial, total;
};
DecodePlan plan_decode(const mla_config *c, int32_t B, int32_t n_q, int32_t max_len) {
  DecodePlan p;
  const int dt = c->dtype;
  const int64_t T = (int64_t)B * n_q;
  const int64_t R = (int64_t)n_q * c->n_heads;
  const int rows = decode_rows_per_group(dt == MLA_BF16 ? 1 : 0, B, R, kCUs);
  const int kvt = decode_kv_tile(dt);
  p.rows = rows;
  p.row_groups = (int)((R + rows - 1) / rows);
  const int64_t per_seq_units = (int64_t)B * p.row_groups;
  int64_t s = (kCUs + per_seq_units - 1) / per_seq_units;
  const int64_t max_tiles = (max_len + kvt - 1) / kvt;
  if (s > max_tiles) s = max_tiles;
  if (s < 1) s = 1;
  int64_t chunk = (max_len + s - 1) / s;
  chunk = ((chunk + kvt - 1) / kvt) * kvt;
  p.chunk = (int)chunk;
  p.splits = (int)((max_len + chunk - 1) / chunk);
  const int64_t N1 = c->d_cq + c->d_c + c->d_rope;
  p.sk1 = choose_splitk(dt, T, N1, c->d_model, 1);
  p.sk2 = choose_splitk(dt, T, (int64_t)c->n_heads * (c->d_nope + c->d_rope), c->d_cq, 1);
  p.sk5 = choose_splitk(dt, T, c->d_model, (int64_t)c->n_heads * c->d_v, 1);
  const size_t e = esize(c);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  const int64_t D = c->d_c + c->d_rope;
  p.c_q = take((size_t)T * c->d_cq * e);
  p.q_nope = take((size_t)T * c->n_heads * c->d_nope * e);
  p.q_abs = take((size_t)T * c->n_heads * D * e);
  p.o_part = take((size_t)B * p.splits * R * c->d_c * e);
  p.lse = take((size_t)B * p.splits * R * 4);
  p.o_lat = take((size_t)T * c->n_heads * c->d_c * e);
  p.o = take((size_t)T * c->n_heads * c->d_v * e);
  size_t part = 0;
  auto need = [&](SplitK sk, int64_t N) {
    if (sk.splits > 1) part = std::max(part, (size_t)sk.splits * T * N * 4);
  };
  need(p.sk1, N1);
  need(p.sk2, (int64_t)c->n_heads * (c->d_nope + c->d_rope));
  need(p.sk5, c->d_model);
  if (dt == MLA_BF16 && T <= 64) part = std::max(part, gemm_stream_partial_bytes((int)T));
  p.partial = take(part);
  p.total = off;
  return p;
}

// RoPE frequency of pair k (fp64, host).  With YaRN the pair's rotation
// count over the original context, r = L * theta / (2 pi), blends the
// interpolated frequency theta / s (r <= beta_slow) into the original one
// (r >= beta_fast), linearly in r.
void fill_inv_freq(const mla_config *c, Epi &e) {
  const double two_pi = 6.283185307179586476925287;
  for (int k = 0; k < MLA_MAX_ROPE_PAIRS; ++k) {
    if (2 * k >= c->d_rope) { e.inv_freq[k] = 0.0; continue; }
    const double theta = pow(c->rope_base, -2.0 * k / c->d_rope);
    if (!yarn_on(c)) { e.inv_freq[k] = theta; continue; }
    const double r = (double)c->yarn_orig_len * theta / two_pi;
    double g = (r - c->yarn_beta_slow) / (c->yarn_beta_fast - c->yarn_beta_slow);
    g = g < 0.0 ? 0.0 : g > 1.0 ? 1.0 : g;
    e.inv_freq[k] = (1.0 - g) * (theta / c->yarn_factor) + g * theta;
  }
}

// Softmax scale in log2 units: log2(e) / sqrt(d_nope + d_rope), times the
// YaRN temperature factor (0.1 ln s + 1)^2 when enabled.
float softmax_scale_log2(const mla_config *c) {
  double s = 1.4426950408889634 / sqrt((double)(c->d_nope + c->d_rope));
  if (yarn_on(c)) {
    const double m = 0.1 * log(c->yarn_factor) + 1.0;
    s *= m * m;
  }
  return (float)s;
}

CacheRef cache_ref(const mla_config *c, const mla_cache *k, int32_t batch) {
  CacheRef r;
  r.batch = batch;
  r.cap = k->block_table ? (long)k->max_blocks_per_seq * k->block_size : (long)k->max_len;
  r.pool = k->pool;
  r.table = k->block_table;
  r.block_size = k->block_table ? k->block_size : 1;
  r.max_blocks = k->max_blocks_per_seq;
  r.max_len = k->max_len;
  r.d_row = c->d_c + c->d_rope;
  r.bs_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == r.block_size) r.bs_shift = sh;
  return r;
}

Seg seg_plain(int n_end, void *dst, long ld) {
  Seg s;
  memset(&s, 0, sizeof(s));
  s.n_end = n_end;
  s.kind = SEG_PLAIN;
  s.head_w = 1;
  s.scale = 1.0f;
  s.dst = dst;
  s.ld = ld;
  return s;
}

GemmArgs gemm_args(const void *x, long ldx, int M, int N, int K) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.ldx = ldx;
  a.M = M;
  a.N = N;
  a.K = K;
  a.splits = 1;
  a.k_chunk = K;
  a.batch = 1;
  a.nw = 1;
  return a;
}

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// [c_Q | c_KV | k_R] = h [W_DQ; W_DKV; W_KR]^T with RoPE on k_R and the cache write.
// with_q = false drops the W_DQ segment (plain cache compression).
hipError_t run_compress(const mla_config *c, const mla_weights *w, const void *h, int M, RowMap rows,
                        const mla_cache *cache, int32_t batch, bool with_q, void *c_q, void *ckv_mirror, void *kr_mirror,
                        SplitK sk, float *partial, hipStream_t st) {
  const int dt = c->dtype;
  const int N = (with_q ? c->d_cq : 0) + c->d_c + c->d_rope;
  GemmArgs a = gemm_args(h, c->d_model, M, N, c->d_model);
  int ns = 0, nw = 0;
  if (with_q) {
    a.w[nw] = w->w_dq;
    a.w_end[nw++] = c->d_cq;
    a.epi.seg[ns++] = seg_plain(c->d_cq, c_q, c->d_cq);
  }
  const int off = with_q ? c->d_cq : 0;
  a.w[nw] = w->w_dkv;
  a.w_end[nw++] = off + c->d_c;
  a.w[nw] = w->w_kr;
  a.w_end[nw++] = N;
  a.nw = nw;
  a.ldw = c->d_model;
  Seg s1 = seg_plain(off + c->d_c, nullptr, 0);
  s1.kind = SEG_CACHE;
  s1.col_off = 0;
  s1.dst2 = ckv_mirror;
  s1.ld2 = c->d_c;
  Seg s2 = seg_plain(N, nullptr, 0);
  s2.kind = SEG_CACHE;
  s2.rope = 1;
  s2.head_w = c->d_rope;
  s2.col_off = c->d_c;
  s2.dst2 = kr_mirror;
  s2.ld2 = c->d_rope;
  a.epi.seg[ns++] = s1;
  a.epi.seg[ns++] = s2;
  a.epi.nseg = ns;
  a.epi.rows = rows;
  a.epi.cache = cache_ref(c, cache, batch);
  fill_inv_freq(c, a.epi);
  a.splits = sk.splits;
  a.k_chunk = sk.k_chunk;
  a.partial = partial;
  a.name = with_q ? "q_kv_down" : "kv_compress";
  a.reduce_name = "q_kv_down.reduce";
  return launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch), 1, 0, a, st);
}

// q = c_Q [W_UQ; W_QR]^T with RoPE on the q_R part.  The content part goes to
// (qc, qc_ld, qc_head_ld, 0) and the rope part to (qr, qr_ld, qr_head_ld, qr_off).
GemmArgs query_args(const mla_config *c, const mla_weights *w, const void *c_q, int M, RowMap rows,
                    void *qc, long qc_ld, long qc_head_ld, void *qr, long qr_ld, long qr_head_ld, int qr_off,
                    SplitK sk, float *partial) {
  const int dt = c->dtype;
  const int Nc = c->n_heads * c->d_nope, N = Nc + c->n_heads * c->d_rope;
  GemmArgs a = gemm_args(c_q, c->d_cq, M, N, c->d_cq);
  a.w[0] = w->w_uq;
  a.w_end[0] = Nc;
  a.w[1] = w->w_qr;
  a.w_end[1] = N;
  a.nw = 2;
  a.ldw = c->d_cq;
  Seg s0 = seg_plain(Nc, qc, qc_ld);
  s0.kind = SEG_HEADS;
  s0.head_w = c->d_nope;
  s0.head_ld = qc_head_ld;
  Seg s1 = seg_plain(N, qr, qr_ld);
  s1.kind = SEG_HEADS;
  s1.rope = 1;
  s1.head_w = c->d_rope;
  s1.head_ld = qr_head_ld;
  s1.col_off = qr_off;
  a.epi.seg[0] = s0;
  a.epi.seg[1] = s1;
  a.epi.nseg = 2;
  a.epi.rows = rows;
  fill_inv_freq(c, a.epi);
  a.splits = sk.splits;
  a.k_chunk = sk.k_chunk;
  a.partial = partial;
  a.name = "q_up";
  a.reduce_name = "q_up.reduce";
  return a;
}

hipError_t run_query(const mla_config *c, const mla_weights *w, const void *c_q, int M, RowMap rows,
                     void *qc, long qc_ld, long qc_head_ld, void *qr, long qr_ld, long qr_head_ld, int qr_off,
                     SplitK sk, float *partial, hipStream_t st) {
  GemmArgs a = query_args(c, w, c_q, M, rows, qc, qc_ld, qc_head_ld, qr, qr_ld, qr_head_ld, qr_off, sk, partial);
  return launch_gemm(c->dtype == MLA_BF16, gemm_tile_for(c->dtype, M, a.N, a.batch), 1, 0, a, st);
}

// u = o W_O^T
hipError_t run_output(const mla_config *c, const mla_weights *w, const void *o, int M, void *u, SplitK sk,
                      float *partial, hipStream_t st) {
  const int K = c->n_heads * c->d_v;
  GemmArgs a = gemm_args(o, K, M, c->d_model, K);
  a.w[0] = w->w_o;
  a.w_end[0] = c->d_model;
  a.ldw = K;
  a.epi.seg[0] = seg_plain(c->d_model, u, c->d_model);
  a.epi.nseg = 1;
  a.splits = sk.splits;
  a.k_chunk = sk.k_chunk;
  a.partial = partial;
  a.name = "o_proj";
  a.reduce_name = "o_proj.reduce";
  return launch_gemm(c->dtype == MLA_BF16, gemm_tile_for(c->dtype, M, a.N, a.batch), 1, 0, a, st);
}

// ---------------------------------------------------------------------------
// Kernel timing
// ---------------------------------------------------------------------------
struct TimedLaunch { const char *name; hipEvent_t start, stop; };
bool g_timing = false;
std::vector<TimedLaunch> g_events;
size_t g_used = 0;

}  // namespace

namespace mla {
void timing_before(const char *name, hipStream_t st) {
  if (!g_timing) return;
  if (g_used == g_events.size()) {
    TimedLaunch t;
    t.name = name;
    if (hipEventCreate(&t.start) != hipSuccess || hipEventCreate(&t.stop) != hipSuccess) return;
    g_events.push_back(t);
  }
  g_events[g_used].name = name;
  (void)hipEventRecord(g_events[g_used].start, st);
}
void timing_after(const char *name, hipStream_t st) {
  if (!g_timing || g_used >= g_events.size() || g_events[g_used].name != name) return;
  (void)hipEventRecord(g_events[g_used].stop, st);
  ++g_used;
}
}  // namespace mla

extern "C" {

size_t mla_cache_bytes_per_token(const mla_config *cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return (size_t)(cfg->d_c + cfg->d_rope) * esize(cfg);
}

size_t mla_mha_cache_elements_per_token(const mla_config *cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return (size_t)2 * cfg->n_heads * cfg->d_nope;
}

mla_status mla_workspace_size(const mla_config *cfg, int32_t op, int32_t batch, int32_t len_or_nq,
                              int32_t max_cache_len, size_t *bytes) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (!bytes) return MLA_ERR_NULL;
  if (batch <= 0 || len_or_nq <= 0) return MLA_ERR_SHAPE;
  if (op == MLA_OP_PREFILL) {
    *bytes = plan_prefill(cfg, (int64_t)batch * len_or_nq).total;
    return MLA_OK;
  }
  if (op == MLA_OP_DECODE) {
    if (max_cache_len < len_or_nq) return MLA_ERR_SHAPE;
    *bytes = plan_decode(cfg, batch, len_or_nq, max_cache_len).total;
    return MLA_OK;
  }
  return MLA_ERR_SHAPE;
}

mla_status mla_compress_kv(const mla_config *cfg, const mla_weights *w, const void *h, int32_t n,
                           const int32_t *seq_idx, const int32_t *pos, int32_t batch, const mla_cache *cache,
                           void *stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (!w || !w->w_dkv || !w->w_kr) return MLA_ERR_NULL;
  if (!h || !seq_idx || !pos) return MLA_ERR_NULL;
  if (n <= 0 || batch <= 0) return MLA_ERR_SHAPE;
  if ((s = check_cache(cache, batch, 1)) != MLA_OK) return s;
  RowMap rows = {ROWS_EXPLICIT, 1, nullptr, seq_idx, pos};
  SplitK sk = {1, cfg->d_model};
  return hip_status(run_compress(cfg, w, h, n, rows, cache, batch, false, nullptr, nullptr, nullptr, sk, nullptr,
                                 (hipStream_t)stream));
}

mla_status mla_prefill(const mla_config *cfg, const mla_weights *w, const void *h, int32_t batch, int32_t len,
                       const mla_cache *cache, void *u, void *o_heads, void *workspace, size_t workspace_bytes,
                       void *stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_weights(w)) != MLA_OK) return s;
  if (!h || !u) return MLA_ERR_NULL;
  if (batch <= 0 || len <= 0) return MLA_ERR_SHAPE;
  const int64_t T = (int64_t)batch * len;
  if (T > (1L << 24)) return MLA_ERR_UNSUPPORTED;
  if (!attention_supported(cfg, MLA_OP_PREFILL)) return MLA_ERR_UNSUPPORTED;
  if ((s = check_cache(cache, batch, len)) != MLA_OK) return s;
  const PrefillPlan p = plan_prefill(cfg, T);
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < p.total) return MLA_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  const int dt = cfg->dtype;
  const int M = (int)T;
  const int NH = cfg->n_heads, DQK = cfg->d_nope + cfg->d_rope;
  RowMap rows = {ROWS_DENSE, len, nullptr, nullptr, nullptr};
  SplitK one = {1, 0};
  void *o = o_heads ? o_heads : (void *)(ws + p.o);
  hipError_t e;

  one.k_chunk = cfg->d_model;
  e = run_compress(cfg, w, h, M, rows, cache, batch, true, ws + p.c_q, ws + p.ckv, ws + p.kr, one, nullptr, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  one.k_chunk = cfg->d_cq;
  e = run_query(cfg, w, ws + p.c_q, M, rows, ws + p.q, (long)NH * DQK, DQK, ws + p.q, (long)NH * DQK, DQK,
                cfg->d_nope, one, nullptr, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  {  // K_C = c_KV W_UK^T  -> [T][n_h][d_nope]
    GemmArgs a = gemm_args(ws + p.ckv, cfg->d_c, M, NH * cfg->d_nope, cfg->d_c);
    a.w[0] = w->w_uk;
    a.w_end[0] = NH * cfg->d_nope;
    a.ldw = cfg->d_c;
    a.epi.seg[0] = seg_plain(NH * cfg->d_nope, ws + p.k, (long)NH * cfg->d_nope);
    a.epi.nseg = 1;
    a.name = "k_up";
    e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch), 1, 0, a, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  {  // V^T = (c_KV W_UV^T)^T -> [n_h*d_v][T]
    GemmArgs a = gemm_args(ws + p.ckv, cfg->d_c, M, NH * cfg->d_v, cfg->d_c);
    a.w[0] = w->w_uv;
    a.w_end[0] = NH * cfg->d_v;
    a.ldw = cfg->d_c;
    a.epi.seg[0] = seg_plain(NH * cfg->d_v, ws + p.vt, (long)T);
    a.epi.nseg = 1;
    a.name = "v_up";
    e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch), 0, 0, a, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  {
    FlashArgs f;
    f.q = ws + p.q;
    f.k = ws + p.k;
    f.kr = ws + p.kr;
    f.vt = ws + p.vt;
    f.o = o;
    f.flags = (unsigned char *)(ws + p.flags);
    f.B = batch;
    f.L = len;
    f.n_h = NH;
    f.d_nope = cfg->d_nope;
    f.d_rope = cfg->d_rope;
    f.d_v = cfg->d_v;
    f.scale_log2 = softmax_scale_log2(cfg);
    e = launch_flash_prefill(dt == MLA_BF16, f, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  one.k_chunk = NH * cfg->d_v;
  e = run_output(cfg, w, o, M, u, one, nullptr, st);
  return hip_status(e);
}

mla_status mla_decode(const mla_config *cfg, const mla_weights *w, const void *h, int32_t batch, int32_t n_q,
                      const int32_t *cache_lens, int32_t max_cache_len, const mla_cache *cache, void *u,
                      void *o_heads, void *workspace, size_t workspace_bytes, void *stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_weights(w)) != MLA_OK) return s;
  if (!h || !u || !cache_lens) return MLA_ERR_NULL;
  if (batch <= 0 || n_q <= 0 || max_cache_len < n_q) return MLA_ERR_SHAPE;
  if ((int64_t)batch * n_q > (1L << 20) || (int64_t)n_q * cfg->n_heads > (1L << 20)) return MLA_ERR_UNSUPPORTED;
  if (!attention_supported(cfg, MLA_OP_DECODE)) return MLA_ERR_UNSUPPORTED;
  if ((s = check_cache(cache, batch, max_cache_len)) != MLA_OK) return s;
  const DecodePlan p = plan_decode(cfg, batch, n_q, max_cache_len);
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < p.total) return MLA_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  const int dt = cfg->dtype;
  const int M = batch * n_q;
  const int NH = cfg->n_heads, D = cfg->d_c + cfg->d_rope;
  float *partial = (float *)(ws + p.partial);
  RowMap rows = {ROWS_DECODE, n_q, cache_lens, nullptr, nullptr};
  void *o = o_heads ? o_heads : (void *)(ws + p.o);
  hipError_t e;

  e = run_compress(cfg, w, h, M, rows, cache, batch, true, ws + p.c_q, nullptr, nullptr, p.sk1, partial, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (dt == MLA_BF16 && decode_q_supported(cfg->d_cq, cfg->d_nope, cfg->d_rope, cfg->d_c, M)) {
    // up-projection, RoPE and absorption in one launch
    const GemmArgs qa = query_args(cfg, w, ws + p.c_q, M, rows, ws + p.q_nope, (long)NH * cfg->d_nope, cfg->d_nope,
                                   ws + p.q_abs, (long)NH * D, D, cfg->d_c, p.sk2, partial);
    DecodeQArgs q;
    q.cq = (const bf16 *)(ws + p.c_q);
    q.w_uq = (const bf16 *)w->w_uq;
    q.w_qr = (const bf16 *)w->w_qr;
    q.w_uk = (const bf16 *)w->w_uk;
    q.q_abs = (bf16 *)(ws + p.q_abs);
    q.T = M;
    q.n_h = NH;
    q.epi = qa.epi;
    e = launch_decode_q(q, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  } else {
    e = run_query(cfg, w, ws + p.c_q, M, rows, ws + p.q_nope, (long)NH * cfg->d_nope, cfg->d_nope, ws + p.q_abs,
                  (long)NH * D, D, cfg->d_c, p.sk2, partial, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    {  // absorption: q_abs[t][i][0:d_c] = W_UK,i^T q_C[t][i]   (W_UK,i is [d_nope][d_c])
      GemmArgs a = gemm_args(ws + p.q_nope, (long)NH * cfg->d_nope, M, cfg->d_c, cfg->d_nope);
      a.x_bs = cfg->d_nope;
      a.w[0] = w->w_uk;
      a.w_end[0] = cfg->d_c;
      a.ldw = cfg->d_c;
      a.w_bs = (long)cfg->d_nope * cfg->d_c;
      a.batch = NH;
      Seg sg = seg_plain(cfg->d_c, ws + p.q_abs, (long)NH * D);
      sg.batch_stride = D;
      a.epi.seg[0] = sg;
      a.epi.nseg = 1;
      a.partial = partial;
      a.name = "absorb";
      e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch), 1, 1, a, st);
      if (e != hipSuccess) return MLA_ERR_HIP;
    }
  }
  DecodeArgs d;
  memset(&d, 0, sizeof(d));
  d.q = ws + p.q_abs;
  d.cache = cache_ref(cfg, cache, batch);
  d.lens = cache_lens;
  d.B = batch;
  d.n_q = n_q;
  d.n_h = NH;
  d.d_c = cfg->d_c;
  d.d_rope = cfg->d_rope;
  d.scale_log2 = softmax_scale_log2(cfg);
  d.chunk = p.chunk;
  d.n_splits = p.splits;
  d.row_groups = p.row_groups;
  d.rows = p.rows;
  d.o_part = ws + p.o_part;
  d.lse_part = (float *)(ws + p.lse);
  d.o_lat = ws + p.o_lat;
  e = launch_decode_attn(dt == MLA_BF16, d, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  e = dt == MLA_BF16 ? launch_decode_combine_uv(d, cfg->d_v, w->w_uv, o, st) : hipErrorNotSupported;
  if (e != hipSuccess && e != hipErrorNotSupported) return MLA_ERR_HIP;
  if (e == hipErrorNotSupported) {   // nothing was launched
    e = launch_decode_combine(dt == MLA_BF16, d, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    // un-absorb: o[t][i] = W_UV,i o_lat[t][i]   (W_UV,i is [d_v][d_c])
    GemmArgs a = gemm_args(ws + p.o_lat, (long)NH * cfg->d_c, M, cfg->d_v, cfg->d_c);
    a.x_bs = cfg->d_c;
    a.w[0] = w->w_uv;
    a.w_end[0] = cfg->d_v;
    a.ldw = cfg->d_c;
    a.w_bs = (long)cfg->d_v * cfg->d_c;
    a.batch = NH;
    Seg sg = seg_plain(cfg->d_v, o, (long)NH * cfg->d_v);
    sg.batch_stride = cfg->d_v;
    a.epi.seg[0] = sg;
    a.epi.nseg = 1;
    a.partial = partial;
    a.name = "unabsorb";
    e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch), 1, 0, a, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  e = run_output(cfg, w, o, M, u, p.sk5, partial, st);
  return hip_status(e);
}

const char *mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "required pointer is NULL";
    case MLA_ERR_SHAPE: return "size or dimension out of range";
    case MLA_ERR_DTYPE: return "unknown dtype";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_CACHE: return "cache descriptor invalid or too small";
    case MLA_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case MLA_ERR_UNSUPPORTED: return "shape outside the supported envelope";
  }
  return "unknown status";
}

const char *mla_version(void) { return "libmla 0.2 (gfx950)"; }

mla_status mla_timing_enable(int32_t on) {
  g_timing = on != 0;
  g_used = 0;
  return MLA_OK;
}

int32_t mla_timing_read(const char **names, double *total_ms, int64_t *launches, int32_t cap) {
  std::vector<std::string> keys;
  std::vector<double> ms;
  std::vector<int64_t> cnt;
  for (size_t i = 0; i < g_used; ++i) {
    float t = 0.f;
    if (hipEventSynchronize(g_events[i].stop) != hipSuccess) return MLA_ERR_HIP;
    if (hipEventElapsedTime(&t, g_events[i].start, g_events[i].stop) != hipSuccess) return MLA_ERR_HIP;
    size_t k = 0;
    while (k < keys.size() && keys[k] != g_events[i].name) ++k;
    if (k == keys.size()) {
      keys.push_back(g_events[i].name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[k] += t;
    cnt[k] += 1;
  }
  for (size_t k = 0; k < keys.size() && (int32_t)k < cap; ++k) {
    // names point at the static strings the launchers pass
    for (size_t i = 0; i < g_used; ++i)
      if (keys[k] == g_events[i].name) { if (names) names[k] = g_events[i].name; break; }
    if (total_ms) total_ms[k] = ms[k];
    if (launches) launches[k] = cnt[k];
  }
  g_used = 0;
  return (int32_t)keys.size();
}

}  // extern "C"
