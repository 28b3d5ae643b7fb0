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
#include <mutex>
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

bool cache_fp8(const mla_config *c) { return c->cache_dtype == MLA_CACHE_FP8_E4M3; }

// block-scaled FP8 projections (W_DQ, W_DKV, W_KR, W_O)
bool weights_fp8(const mla_config *c) { return c->weight_dtype == MLA_WEIGHTS_FP8_BLOCK; }

// widest input of an FP8 projection (h, or the attention output o)
int64_t fp8_act_width(const mla_config *c) { return std::max<int64_t>(c->d_model, (int64_t)c->n_heads * c->d_v); }
// tokens per row of the activation scale exponents (whole 256-token tiles)
int64_t fp8_scale_ld(int64_t T) { return (T + 255) / 256 * 256; }

// bytes of one cached row: (d_c + d_R) elements, or the FP8 row (codes,
// bf16 k_R, a float32 scale per 128 columns)
size_t row_bytes(const mla_config *c) {
  if (cache_fp8(c)) return (size_t)c->d_c + 2 * (size_t)c->d_rope + 4 * (size_t)(c->d_c / 128);
  return (size_t)(c->d_c + c->d_rope) * esize(c);
}

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
  // every width within 2^20 (n_heads 2^16), so sums and products of widths
  // below stay far inside int32 / int64
  if (c->d_model > (1 << 20) || c->d_cq > (1 << 20) || c->d_c > (1 << 20) || c->d_nope > (1 << 20) ||
      c->d_rope > (1 << 20) || c->d_v > (1 << 20) || c->n_heads > (1 << 16))
    return MLA_ERR_UNSUPPORTED;
  if (!(c->rope_base > 0.0) || !isfinite(c->rope_base)) return MLA_ERR_SHAPE;
  if (yarn_on(c)) {
    if (!(c->yarn_factor > 1.0) || !isfinite(c->yarn_factor) || c->yarn_orig_len <= 0) return MLA_ERR_SHAPE;
    if (!(c->yarn_beta_slow > 0.0) || !(c->yarn_beta_fast > c->yarn_beta_slow) || !isfinite(c->yarn_beta_fast))
      return MLA_ERR_SHAPE;
  }
  if (c->cache_dtype != MLA_CACHE_LAYER && c->cache_dtype != MLA_CACHE_FP8_E4M3) return MLA_ERR_DTYPE;
  if (c->cache_dtype == MLA_CACHE_FP8_E4M3 && (c->dtype != MLA_BF16 || c->d_c % 128 || c->d_rope % 8))
    return MLA_ERR_UNSUPPORTED;
  if (c->weight_dtype != MLA_WEIGHTS_LAYER && c->weight_dtype != MLA_WEIGHTS_FP8_BLOCK) return MLA_ERR_DTYPE;
  if (c->weight_dtype == MLA_WEIGHTS_FP8_BLOCK &&
      (c->dtype != MLA_BF16 || c->d_model % 512 || ((long)c->n_heads * c->d_v) % 512 ||
       c->d_model > 16384 || (long)c->n_heads * c->d_v > 16384))
    return MLA_ERR_UNSUPPORTED;
  if (c->d_rope / 2 > MLA_MAX_ROPE_PAIRS) return MLA_ERR_UNSUPPORTED;
  if ((long)c->n_heads * ((long)c->d_nope + c->d_rope) > (1L << 24)) return MLA_ERR_UNSUPPORTED;
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

mla_status check_weights(const mla_config *c, const mla_weights *w) {
  if (!w) return MLA_ERR_NULL;
  if (!w->w_dq || !w->w_uq || !w->w_qr || !w->w_dkv || !w->w_kr || !w->w_uk || !w->w_uv || !w->w_o)
    return MLA_ERR_NULL;
  if (weights_fp8(c) && (!w->s_dq || !w->s_dkv || !w->s_kr || !w->s_o)) return MLA_ERR_NULL;
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
struct SplitK { int splits, k_chunk; };
struct PrefillPlan {
  size_t c_q, ckv, kr, q, k, vt, o, x8, xs, partial, total;
  SplitK sko;   // W_O's split over k
};
SplitK choose_splitk(int dtype, int64_t M, int64_t N, int64_t K, int batch);
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
  // FP8 projections: the quantised h / o (codes and scale exponents), and
  // up to 128 tokens the streaming kernel's partial sums
  const bool f8 = weights_fp8(c);
  p.x8 = take(f8 ? (size_t)T * fp8_act_width(c) : 0);
  p.xs = take(f8 ? (size_t)(fp8_act_width(c) / 128) * fp8_scale_ld(T) : 0);
  // W_O split over k (few 256x256 tiles): fp32 partials [splits][T][d_model]
  p.sko = choose_splitk(c->dtype, T, c->d_model, (int64_t)c->n_heads * c->d_v, 1);
  size_t part = p.sko.splits > 1 ? (size_t)p.sko.splits * T * c->d_model * 4 : 0;
  // a partial buffer lets products of up to 128 tokens stream (they need
  // the streaming kernel's layout); FP8 products of that size always do
  if ((part || f8) && T <= 128 && c->dtype == MLA_BF16) part = std::max(part, gemm_stream_partial_bytes((int)T));
  p.partial = take(part);
  p.total = off;
  return p;
}

// Standalone cache compression of n tokens: with an FP8 cache the rows'
// c_KV and k_R before quantisation; with FP8 projections the quantised h and,
// up to 128 tokens, the streaming kernel's partial sums.  Nothing otherwise.
struct CompressPlan {
  size_t ckv, kr, x8, xs, partial, total;
};
CompressPlan plan_compress(const mla_config *c, int64_t n) {
  CompressPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  const bool f8 = weights_fp8(c), c8 = cache_fp8(c);
  p.ckv = take(c8 ? (size_t)n * c->d_c * esize(c) : 0);
  p.kr = take(c8 ? (size_t)n * c->d_rope * esize(c) : 0);
  p.x8 = take(f8 ? (size_t)n * c->d_model : 0);
  p.xs = take(f8 ? (size_t)(c->d_model / 128) * fp8_scale_ld(n) : 0);
  p.partial = take(f8 && n <= 128 ? gemm_stream_partial_bytes((int)n) : 0);
  p.total = off;
  return p;
}

// Split over k of the 256x256 kernel's tiles when they fill at most half the
// CUs (a few hundred tokens against a wide weight): about one wave of
// workgroups, at least 1024 k per split, then the ordered reduce.
int big_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles <= kCUs / 2)
    for (int s = 8; s >= 2; --s)
      if (s * tiles <= kCUs && K % (128 * s) == 0 && K / s >= 1024) return s;
  return 1;
}

// 256x256 tiles (bf16) unless they would leave all but a few CUs idle: a
// few hundred tokens against a narrow weight (a 512-token chunk: 18 tiles for
// the down projection) go to the 32x64-tile kernel, which spreads over every
// CU (180 -> 90 us there); from 32 tiles on the big tiles win (W_O at 512
// tokens, 56 tiles: 362 against 393 us).  From 96 to 255 tokens the
// weight-streaming kernels re-read the activation slice with every 64-column
// unit (at 128 tokens twice the weight bytes); the 256x256 kernel (rows past
// M clamped) takes such a product when its tiles, split over k, fill three
// quarters of the CUs (W_O at 128 tokens: 118 -> 73 us; the query
// up-projection's 96 unsplit tiles were slower than streaming).
int gemm_tile_for(int dtype, int64_t M, int64_t N, int64_t batch, int64_t K) {
  if (dtype == MLA_BF16 && batch == 1 && M >= 96 && M < 256)
    return ((N + 255) / 256) * big_splits(M, N, K) >= kCUs * 3 / 4 ? TILE_BIG : TILE_SKINNY;
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
  const int tile = gemm_tile_for(dtype, M, N, batch, K);
  if (tile != TILE_SKINNY) {
    if (dtype == MLA_BF16 && batch == 1) {
      r.splits = big_splits(M, N, K);
      r.k_chunk = (int)(K / r.splits);
    }
    return r;
  }
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

// decode size envelope: at most 2^20 new tokens and 2^20 query rows per
// sequence, so every product in the plan stays far inside int64 / size_t
bool decode_sizes_ok(const mla_config *c, int32_t batch, int32_t n_q) {
  return (int64_t)batch * n_q <= (1L << 20) && (int64_t)n_q * c->n_heads <= (1L << 20);
}

struct DecodePlan {
  int W, slots, row_groups, rows;
  SplitK sk1, sk2, sk5;
  size_t c_q, q_nope, q_abs, o_part, lse, o_lat, o, ckv, kr, x8, xs, partial, total;
  // many new tokens per sequence (a chunk after a cached prefix): the
  // up-projected form, the prefix gathered into Lpad dense rows per sequence
  bool flash;
  int Lpad;
  size_t qf, ckvd, krd, kf, vtf;
};

// New tokens per sequence from which decode takes the up-projected (flash)
// form: its flops per cached row, 2*n_h*d_c*(d_nope + d_v) for the
// up-projections plus 2*n_q*n_h*(d_nope + d_rope + d_v) for the attention,
// fall below the absorbed form's 2*n_q*n_h*(2 d_c + d_rope) from about 170
// tokens on (DeepSeek-V3 widths), and its kernels run faster.
const int kFlashMinNq = 256;
// ... while its dense keys and values stay within 4 GiB
const int64_t kFlashMaxKvBytes = 1LL << 32;
// The attention's split plan: W workgroups per row group (one wave of
// workgroups over the CUs), each taking an equal share of the batch's cached
// tiles (computed on the device from the lengths), and at most W + B partial
// slots; neither depends on the lengths, so the workspace size does not.
DecodePlan plan_decode(const mla_config *c, int32_t B, int32_t n_q, int32_t max_len, bool allow_flash = true) {
  DecodePlan p;
  const int dt = c->dtype;
  const int64_t T = (int64_t)B * n_q;
  const int64_t Lpad = ((int64_t)max_len + 63) / 64 * 64;
  // bytes of K_C and V^T per dense row (each factor within 2^21, so no overflow)
  const int64_t kv_row = (int64_t)c->n_heads * (c->d_nope + c->d_v) * 2;
  p.flash = allow_flash && dt == MLA_BF16 && !cache_fp8(c) && n_q >= kFlashMinNq &&
            flash_prefix_supported(1, c->d_nope, c->d_rope, c->d_v) && (int64_t)B * Lpad <= kFlashMaxKvBytes / kv_row;
  p.Lpad = (int)Lpad;
  const int64_t R = (int64_t)n_q * c->n_heads;
  const int rows = decode_rows_per_group(dt == MLA_BF16 ? 1 : 0, B, R, kCUs);
  p.rows = rows;
  p.row_groups = (int)((R + rows - 1) / rows);
  p.W = std::max(1, kCUs / p.row_groups);
  p.slots = p.W + B;
  (void)max_len;
  const int64_t N1 = c->d_cq + c->d_c + c->d_rope;
  p.sk1 = choose_splitk(dt, T, N1, c->d_model, 1);
  p.sk2 = choose_splitk(dt, T, (int64_t)c->n_heads * (c->d_nope + c->d_rope), c->d_cq, 1);
  p.sk5 = choose_splitk(dt, T, c->d_model, (int64_t)c->n_heads * c->d_v, 1);
  const size_t e = esize(c);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  const int64_t D = c->d_c + c->d_rope;
  const bool ab = !p.flash;   // the absorbed form's buffers
  p.c_q = take((size_t)T * c->d_cq * e);
  p.q_nope = take(ab ? (size_t)T * c->n_heads * c->d_nope * e : 0);
  p.q_abs = take(ab ? (size_t)T * c->n_heads * D * e : 0);
  p.o_part = take(ab ? (size_t)p.slots * R * c->d_c * e : 0);
  p.lse = take(ab ? (size_t)p.slots * R * 4 : 0);
  p.o_lat = take(ab ? (size_t)T * c->n_heads * c->d_c * e : 0);
  p.o = take((size_t)T * c->n_heads * c->d_v * e);
  // the up-projected form: q [T][n_h][d_nope + d_rope], the prefix's dense
  // c_KV and k_R, K_C [B*Lpad][n_h][d_nope] and V^T [n_h*d_v][B*Lpad]
  p.qf = take(p.flash ? (size_t)T * c->n_heads * (c->d_nope + c->d_rope) * e : 0);
  p.ckvd = take(p.flash ? (size_t)B * Lpad * c->d_c * e : 0);
  p.krd = take(p.flash ? (size_t)B * Lpad * c->d_rope * e : 0);
  p.kf = take(p.flash ? (size_t)B * Lpad * c->n_heads * c->d_nope * e : 0);
  p.vtf = take(p.flash ? (size_t)B * Lpad * c->n_heads * c->d_v * e : 0);
  // FP8 cache: the new tokens' c_KV and k_R before quantisation
  p.ckv = take(cache_fp8(c) ? (size_t)T * c->d_c * e : 0);
  p.kr = take(cache_fp8(c) ? (size_t)T * c->d_rope * e : 0);
  // FP8 projections: the quantised h / o
  p.x8 = take(weights_fp8(c) ? (size_t)T * fp8_act_width(c) : 0);
  p.xs = take(weights_fp8(c) ? (size_t)(fp8_act_width(c) / 128) * fp8_scale_ld(T) : 0);
  size_t part = 0;
  auto need = [&](SplitK sk, int64_t N) {
    if (sk.splits > 1) part = std::max(part, (size_t)sk.splits * T * N * 4);
  };
  need(p.sk1, N1);
  need(p.sk2, (int64_t)c->n_heads * (c->d_nope + c->d_rope));
  need(p.sk5, c->d_model);
  if (dt == MLA_BF16 && T <= 128) part = std::max(part, gemm_stream_partial_bytes((int)T));
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

#ifdef MLA_DEBUG_CHECKS
// Debug builds: one error word per device (its device address fetched once
// per device, like the allocation-free decode's array), cleared before a
// call's kernels and read after them.
static __device__ unsigned dbg_word;
std::mutex g_dbg_mu;
unsigned *g_dbg_ptr[256];

unsigned *debug_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return nullptr;
  std::lock_guard<std::mutex> lock(g_dbg_mu);
  if (!g_dbg_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(dbg_word)) != hipSuccess || !ptr) return nullptr;
    g_dbg_ptr[dev] = (unsigned *)ptr;
  }
  return g_dbg_ptr[dev];
}

mla_status debug_begin(hipStream_t st) {
  unsigned *d = debug_word();
  if (!d) return MLA_ERR_HIP;
  return hipMemsetAsync(d, 0, sizeof(unsigned), st) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// after the call's kernels: wait for them and report what they recorded
mla_status debug_end(hipStream_t st, mla_status s) {
  if (s != MLA_OK) return s;
  unsigned hv = 0;
  if (hipMemcpyAsync(&hv, debug_word(), sizeof hv, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return MLA_ERR_HIP;
  return hv ? MLA_ERR_CACHE : MLA_OK;
}
#else
unsigned *debug_word() { return nullptr; }
mla_status debug_begin(hipStream_t) { return MLA_OK; }
mla_status debug_end(hipStream_t, mla_status s) { return s; }
#endif

CacheRef cache_ref(const mla_config *c, const mla_cache *k, int32_t batch) {
  CacheRef r;
  r.n_blocks = k->block_table ? k->n_blocks : 0;
  r.dbg = debug_word();
  r.batch = batch;
  r.cap = k->block_table ? (long)k->max_blocks_per_seq * k->block_size : (long)k->max_len;
  r.pool = k->pool;
  r.table = k->block_table;
  r.block_size = k->block_table ? k->block_size : 1;
  r.max_blocks = k->max_blocks_per_seq;
  r.max_len = k->max_len;
  r.d_row = c->d_c + c->d_rope;
  r.row_bytes = (int)row_bytes(c);
  r.fp8 = cache_fp8(c) ? 1 : 0;
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

// A partial-sum buffer of the workspace and its size in bytes.
struct Part {
  float *p;
  size_t bytes;
};

// Quantise x [M][K] (bf16, row stride K) into f, unless its producer already
// wrote it there, and point the product's activation operand at it; the
// weights are E4M3 with the scales wsc.
hipError_t fp8_operands(const Fp8Out &f, const void *x, int M, int K, GemmArgs &a, bool quantised, hipStream_t st) {
  if (!quantised) {
    hipError_t e = launch_quant_act_fp8((const bf16 *)x, K, M, K, f.codes, f.scales, f.ld_s, st);
    if (e != hipSuccess) return e;
  }
  a.x = f.codes;
  a.ldx = K;
  a.fp8 = 1;
  a.xs = f.scales;
  a.xs_ld = f.ld_s;
  a.wsc_ld = K / 128;
  return hipSuccess;
}

// [c_Q | c_KV | k_R] = h [W_DQ; W_DKV; W_KR]^T with RoPE on k_R and the cache write.
// with_q = false drops the W_DQ segment (plain cache compression).
hipError_t run_compress(const mla_config *c, const mla_weights *w, const void *h, int M, RowMap rows,
                        const mla_cache *cache, int32_t batch, bool with_q, void *c_q, void *ckv_mirror, void *kr_mirror,
                        SplitK sk, Part partial, const Fp8Out *f8, hipStream_t st) {
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
  const bool fp8 = cache_fp8(c);
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
  if (fp8) {
    // the FP8 row needs its group maxima first: c_KV and k_R go to the
    // mirrors, and the append kernel quantises and writes the rows
    s1 = seg_plain(off + c->d_c, ckv_mirror, c->d_c);
    s2 = seg_plain(N, kr_mirror, c->d_rope);
    s2.rope = 1;
    s2.head_w = c->d_rope;
  }
  a.epi.seg[ns++] = s1;
  a.epi.seg[ns++] = s2;
  a.epi.nseg = ns;
  a.epi.rows = rows;
  a.epi.cache = cache_ref(c, cache, batch);
  fill_inv_freq(c, a.epi);
  a.splits = sk.splits;
  a.k_chunk = sk.k_chunk;
  a.partial = partial.p;
  a.partial_bytes = partial.bytes;
  a.name = with_q ? "q_kv_down" : "kv_compress";
  a.reduce_name = "q_kv_down.reduce";
  if (f8) {
    int i = 0;
    if (with_q) a.wsc[i++] = w->s_dq;
    a.wsc[i++] = w->s_dkv;
    a.wsc[i++] = w->s_kr;
    hipError_t e = fp8_operands(*f8, h, M, c->d_model, a, false, st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch, a.K), 1, 0, a, st);
  if (e != hipSuccess || !fp8) return e;
  CacheAppendArgs ap;
  ap.ckv = (const bf16 *)ckv_mirror;
  ap.kr = (const bf16 *)kr_mirror;
  ap.T = M;
  ap.d_c = c->d_c;
  ap.d_rope = c->d_rope;
  ap.rows = rows;
  ap.cache = a.epi.cache;
  return launch_cache_append_fp8(ap, st);
}

// q = c_Q [W_UQ; W_QR]^T with RoPE on the q_R part.  The content part goes to
// (qc, qc_ld, qc_head_ld, 0) and the rope part to (qr, qr_ld, qr_head_ld, qr_off).
GemmArgs query_args(const mla_config *c, const mla_weights *w, const void *c_q, int M, RowMap rows,
                    void *qc, long qc_ld, long qc_head_ld, void *qr, long qr_ld, long qr_head_ld, int qr_off,
                    SplitK sk, Part partial) {
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
  a.partial = partial.p;
  a.partial_bytes = partial.bytes;
  a.name = "q_up";
  a.reduce_name = "q_up.reduce";
  return a;
}

hipError_t run_query(const mla_config *c, const mla_weights *w, const void *c_q, int M, RowMap rows,
                     void *qc, long qc_ld, long qc_head_ld, void *qr, long qr_ld, long qr_head_ld, int qr_off,
                     SplitK sk, Part partial, hipStream_t st) {
  GemmArgs a = query_args(c, w, c_q, M, rows, qc, qc_ld, qc_head_ld, qr, qr_ld, qr_head_ld, qr_off, sk, partial);
  return launch_gemm(c->dtype == MLA_BF16, gemm_tile_for(c->dtype, M, a.N, a.batch, a.K), 1, 0, a, st);
}

// u = o W_O^T
// f8_ready: the attention already wrote o's quantised form into *f8
hipError_t run_output(const mla_config *c, const mla_weights *w, const void *o, int M, void *u, SplitK sk,
                      Part partial, const Fp8Out *f8, bool f8_ready, hipStream_t st) {
  const int K = c->n_heads * c->d_v;
  GemmArgs a = gemm_args(o, K, M, c->d_model, K);
  a.w[0] = w->w_o;
  a.w_end[0] = c->d_model;
  a.ldw = K;
  a.epi.seg[0] = seg_plain(c->d_model, u, c->d_model);
  a.epi.nseg = 1;
  a.splits = sk.splits;
  a.k_chunk = sk.k_chunk;
  a.partial = partial.p;
  a.partial_bytes = partial.bytes;
  a.name = "o_proj";
  a.reduce_name = "o_proj.reduce";
  if (f8) {
    a.wsc[0] = w->s_o;
    hipError_t e = fp8_operands(*f8, o, M, K, a, f8_ready, st);
    if (e != hipSuccess) return e;
  }
  return launch_gemm(c->dtype == MLA_BF16, gemm_tile_for(c->dtype, M, a.N, a.batch, a.K), 1, 0, a, st);
}

// ---------------------------------------------------------------------------
// Kernel timing
// ---------------------------------------------------------------------------
// One slot per timed launch.  The slots, the count and the session number are
// guarded by g_timing_mu; a bracket opened by timing_before is closed by the
// same host thread's timing_after (t_open), so launches from several threads
// get their own slots.  A slot counts once its stop event is recorded in the
// session that opened it.
struct TimedLaunch { const char *name; hipEvent_t start, stop; bool done; };
std::mutex g_timing_mu;
bool g_timing = false;
std::vector<TimedLaunch> g_events;
size_t g_used = 0;
unsigned long g_session = 0;
struct OpenBracket { long slot = -1; unsigned long session = 0; };
thread_local OpenBracket t_open;

}  // namespace

namespace mla {
void timing_before(const char *name, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  t_open.slot = -1;
  if (!g_timing) return;
  if (g_used == g_events.size()) {
    TimedLaunch t{name, nullptr, nullptr, false};
    if (hipEventCreate(&t.start) != hipSuccess) return;
    if (hipEventCreate(&t.stop) != hipSuccess) {
      (void)hipEventDestroy(t.start);
      return;
    }
    g_events.push_back(t);
  }
  TimedLaunch &t = g_events[g_used];
  t.name = name;
  t.done = false;
  if (hipEventRecord(t.start, st) != hipSuccess) return;
  t_open.slot = (long)g_used++;
  t_open.session = g_session;
}
void timing_after(const char *name, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  const OpenBracket o = t_open;
  t_open.slot = -1;
  if (!g_timing || o.slot < 0 || o.session != g_session || (size_t)o.slot >= g_used) return;
  TimedLaunch &t = g_events[o.slot];
  if (strcmp(t.name, name) != 0) return;
  t.done = hipEventRecord(t.stop, st) == hipSuccess;
}
}  // namespace mla

extern "C" {

size_t mla_cache_bytes_per_token(const mla_config *cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return row_bytes(cfg);
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
  // the same size envelopes as the entry points (they bound every product
  // in the plans)
  if (op == MLA_OP_PREFILL) {
    if ((int64_t)batch * len_or_nq > (1L << 24)) return MLA_ERR_UNSUPPORTED;
    *bytes = plan_prefill(cfg, (int64_t)batch * len_or_nq).total;
    return MLA_OK;
  }
  if (op == MLA_OP_DECODE) {
    if (max_cache_len < len_or_nq) return MLA_ERR_SHAPE;
    if (!decode_sizes_ok(cfg, batch, len_or_nq)) return MLA_ERR_UNSUPPORTED;
    *bytes = plan_decode(cfg, batch, len_or_nq, max_cache_len).total;
    return MLA_OK;
  }
  if (op == MLA_OP_COMPRESS) {
    if (len_or_nq > (1 << 24)) return MLA_ERR_UNSUPPORTED;
    *bytes = plan_compress(cfg, len_or_nq).total;
    return MLA_OK;
  }
  return MLA_ERR_SHAPE;
}

mla_status mla_compress_kv(const mla_config *cfg, const mla_weights *w, const void *h, int32_t n,
                           const int32_t *seq_idx, const int32_t *pos, int32_t batch, const mla_cache *cache,
                           void *workspace, size_t workspace_bytes, void *stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (!w || !w->w_dkv || !w->w_kr) return MLA_ERR_NULL;
  if (weights_fp8(cfg) && (!w->s_dkv || !w->s_kr)) return MLA_ERR_NULL;
  if (!h || !seq_idx || !pos) return MLA_ERR_NULL;
  if (n <= 0 || batch <= 0) return MLA_ERR_SHAPE;
  if (n > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  if ((s = check_cache(cache, batch, 1)) != MLA_OK) return s;
  if (cache_fp8(cfg) && cache->block_table && cache->block_size % 32) return MLA_ERR_UNSUPPORTED;
  const CompressPlan p = plan_compress(cfg, n);
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return MLA_ERR_WORKSPACE;
  RowMap rows = {ROWS_EXPLICIT, 1, nullptr, seq_idx, pos};
  SplitK sk = {1, cfg->d_model};
  char *ws = (char *)workspace;
  const Fp8Out f8 = {p.x8 < p.total ? (unsigned char *)(ws + p.x8) : nullptr,
                     p.xs < p.total ? (unsigned char *)(ws + p.xs) : nullptr, (long)fp8_scale_ld(n)};
  const bool c8 = cache_fp8(cfg), w8 = weights_fp8(cfg);
  const Part part = {w8 && n <= 128 ? (float *)(ws + p.partial) : nullptr, w8 && n <= 128 ? p.total - p.partial : 0};
  const hipStream_t st = (hipStream_t)stream;
  if ((s = debug_begin(st)) != MLA_OK) return s;
  return debug_end(st, hip_status(run_compress(cfg, w, h, n, rows, cache, batch, false, nullptr,
                                               c8 ? ws + p.ckv : nullptr, c8 ? ws + p.kr : nullptr, sk, part,
                                               w8 ? &f8 : nullptr, st)));
}

mla_status mla_prefill(const mla_config *cfg, const mla_weights *w, const void *h, int32_t batch, int32_t len,
                       const mla_cache *cache, void *u, void *o_heads, void *workspace, size_t workspace_bytes,
                       void *stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_weights(cfg, w)) != MLA_OK) return s;
  if (!h || !u) return MLA_ERR_NULL;
  if (batch <= 0 || len <= 0) return MLA_ERR_SHAPE;
  const int64_t T = (int64_t)batch * len;
  if (T > (1L << 24)) return MLA_ERR_UNSUPPORTED;
  if (!attention_supported(cfg, MLA_OP_PREFILL)) return MLA_ERR_UNSUPPORTED;
  if ((s = check_cache(cache, batch, len)) != MLA_OK) return s;
  if (cache_fp8(cfg) && cache->block_table && cache->block_size % 32) return MLA_ERR_UNSUPPORTED;
  const PrefillPlan p = plan_prefill(cfg, T);
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < p.total) return MLA_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  if ((s = debug_begin(st)) != MLA_OK) return s;
  char *ws = (char *)workspace;
  const int dt = cfg->dtype;
  const int M = (int)T;
  const int NH = cfg->n_heads, DQK = cfg->d_nope + cfg->d_rope;
  RowMap rows = {ROWS_DENSE, len, nullptr, nullptr, nullptr};
  SplitK one = {1, 0};
  void *o = o_heads ? o_heads : (void *)(ws + p.o);
  hipError_t e;

  const Fp8Out f8 = {(unsigned char *)(ws + p.x8), (unsigned char *)(ws + p.xs), (long)fp8_scale_ld(T)};
  const Fp8Out *f8p = weights_fp8(cfg) ? &f8 : nullptr;
  // partial sums: the FP8 streaming kernel (up to 128 tokens) or W_O's split
  const bool has_part = p.total > p.partial;
  const Part partial = {has_part ? (float *)(ws + p.partial) : nullptr, p.total - p.partial};
  one.k_chunk = cfg->d_model;
  e = run_compress(cfg, w, h, M, rows, cache, batch, true, ws + p.c_q, ws + p.ckv, ws + p.kr, one, partial, f8p, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  one.k_chunk = cfg->d_cq;
  e = run_query(cfg, w, ws + p.c_q, M, rows, ws + p.q, (long)NH * DQK, DQK, ws + p.q, (long)NH * DQK, DQK,
                cfg->d_nope, one, Part{nullptr, 0}, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  {  // K_C = c_KV W_UK^T  -> [T][n_h][d_nope]
    GemmArgs a = gemm_args(ws + p.ckv, cfg->d_c, M, NH * cfg->d_nope, cfg->d_c);
    a.w[0] = w->w_uk;
    a.w_end[0] = NH * cfg->d_nope;
    a.ldw = cfg->d_c;
    a.epi.seg[0] = seg_plain(NH * cfg->d_nope, ws + p.k, (long)NH * cfg->d_nope);
    a.epi.nseg = 1;
    a.name = "k_up";
    e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch, a.K), 1, 0, a, st);
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
    e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch, a.K), 0, 0, a, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  {
    FlashArgs f;
    memset(&f, 0, sizeof(f));   // lens = nullptr: queries are positions 0..len-1
    f.q = ws + p.q;
    f.k = ws + p.k;
    f.kr = ws + p.kr;
    f.vt = ws + p.vt;
    f.o = o;
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
  e = run_output(cfg, w, o, M, u, p.sko, partial, f8p, false, st);
  return debug_end(st, hip_status(e));
}

}  // extern "C"

namespace {

// Validation shared by the decode entry points (no HIP call).
mla_status check_decode(const mla_config *cfg, const mla_weights *w, const void *h, int32_t batch, int32_t n_q,
                        const int32_t *cache_lens, const int32_t *cache_lens_host, int32_t max_cache_len,
                        const mla_cache *cache, const void *u, DecodePlan *plan, bool noalloc) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_weights(cfg, w)) != MLA_OK) return s;
  if (!h || !u || !cache_lens) return MLA_ERR_NULL;
  if (batch <= 0 || n_q <= 0 || max_cache_len < n_q) return MLA_ERR_SHAPE;
  if (cache_lens_host)
    for (int32_t b = 0; b < batch; ++b)
      if (cache_lens_host[b] < n_q || cache_lens_host[b] > max_cache_len) return MLA_ERR_SHAPE;
  if (!decode_sizes_ok(cfg, batch, n_q)) return MLA_ERR_UNSUPPORTED;
  if (!attention_supported(cfg, MLA_OP_DECODE)) return MLA_ERR_UNSUPPORTED;
  if ((s = check_cache(cache, batch, max_cache_len)) != MLA_OK) return s;
  if (cache_fp8(cfg) && cache->block_table && cache->block_size % 32) return MLA_ERR_UNSUPPORTED;
  *plan = plan_decode(cfg, batch, n_q, max_cache_len);
  // the allocation-free decode keeps to its array: the absorbed form when
  // the up-projected one would not fit
  if (noalloc && plan->total > (size_t)MLA_NOALLOC_WORKSPACE_BYTES)
    *plan = plan_decode(cfg, batch, n_q, max_cache_len, false);
  return MLA_OK;
}

// The decode kernel sequence on a validated call, with its workspace at ws.
mla_status decode_steps(const mla_config *cfg, const mla_weights *w, const void *h, int32_t batch, int32_t n_q,
                        const int32_t *cache_lens, const mla_cache *cache, void *u, void *o_heads, char *ws,
                        const DecodePlan &p, void *stream) {
  hipStream_t st = (hipStream_t)stream;
  const int dt = cfg->dtype;
  const int M = batch * n_q;
  const int NH = cfg->n_heads, D = cfg->d_c + cfg->d_rope;
  const Part partial = {(float *)(ws + p.partial), p.total - p.partial};
  RowMap rows = {ROWS_DECODE, n_q, cache_lens, nullptr, nullptr};
  void *o = o_heads ? o_heads : (void *)(ws + p.o);
  hipError_t e;

  const bool fp8 = cache_fp8(cfg);
  const Fp8Out f8 = {(unsigned char *)(ws + p.x8), (unsigned char *)(ws + p.xs), (long)fp8_scale_ld(M)};
  const Fp8Out *f8p = weights_fp8(cfg) ? &f8 : nullptr;
  e = run_compress(cfg, w, h, M, rows, cache, batch, true, ws + p.c_q, fp8 ? ws + p.ckv : nullptr,
                   fp8 ? ws + p.kr : nullptr, p.sk1, partial, f8p, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (p.flash) {
    // Many new tokens per sequence (a chunk after its cached prefix): the
    // up-projected form of p5 section 2.1, as in prefill.  Queries with RoPE
    // at their positions; every cached row (the chunk's own just appended)
    // gathered densely and up-projected to K_C and V^T; the flash kernel
    // with each sequence's queries after its prefix; then W_O.
    const int DQK = cfg->d_nope + cfg->d_rope;
    e = run_query(cfg, w, ws + p.c_q, M, rows, ws + p.qf, (long)NH * DQK, DQK, ws + p.qf, (long)NH * DQK, DQK,
                  cfg->d_nope, p.sk2, partial, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    e = launch_prefix_gather(cache_ref(cfg, cache, batch), cache_lens, batch, p.Lpad, cfg->d_c, cfg->d_rope,
                             ws + p.ckvd, ws + p.krd, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    const int MK = batch * p.Lpad;
    {  // K_C = c_KV W_UK^T -> [B*Lpad][n_h][d_nope]
      GemmArgs a = gemm_args(ws + p.ckvd, cfg->d_c, MK, NH * cfg->d_nope, cfg->d_c);
      a.w[0] = w->w_uk;
      a.w_end[0] = NH * cfg->d_nope;
      a.ldw = cfg->d_c;
      a.epi.seg[0] = seg_plain(NH * cfg->d_nope, ws + p.kf, (long)NH * cfg->d_nope);
      a.epi.nseg = 1;
      a.name = "k_up";
      e = launch_gemm(1, gemm_tile_for(dt, MK, a.N, 1, a.K), 1, 0, a, st);
      if (e != hipSuccess) return MLA_ERR_HIP;
    }
    {  // V^T = (c_KV W_UV^T)^T -> [n_h*d_v][B*Lpad]
      GemmArgs a = gemm_args(ws + p.ckvd, cfg->d_c, MK, NH * cfg->d_v, cfg->d_c);
      a.w[0] = w->w_uv;
      a.w_end[0] = NH * cfg->d_v;
      a.ldw = cfg->d_c;
      a.epi.seg[0] = seg_plain(NH * cfg->d_v, ws + p.vtf, (long)MK);
      a.epi.nseg = 1;
      a.name = "v_up";
      e = launch_gemm(1, gemm_tile_for(dt, MK, a.N, 1, a.K), 0, 0, a, st);
      if (e != hipSuccess) return MLA_ERR_HIP;
    }
    FlashArgs f;
    memset(&f, 0, sizeof(f));
    f.q = ws + p.qf;
    f.k = ws + p.kf;
    f.kr = ws + p.krd;
    f.vt = ws + p.vtf;
    f.o = o;
    f.B = batch;
    f.L = p.Lpad;
    f.n_h = NH;
    f.d_nope = cfg->d_nope;
    f.d_rope = cfg->d_rope;
    f.d_v = cfg->d_v;
    f.scale_log2 = softmax_scale_log2(cfg);
    f.lens = cache_lens;
    f.Lq = n_q;
    e = launch_flash_prefill(1, f, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    return hip_status(run_output(cfg, w, o, M, u, p.sk5, partial, f8p, false, st));
  }
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
      a.partial = partial.p;
      a.partial_bytes = partial.bytes;
      a.name = "absorb";
      e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch, a.K), 1, 1, a, st);
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
  d.W = p.W;
  d.slots = p.slots;
  d.row_groups = p.row_groups;
  d.rows = p.rows;
  d.o_part = ws + p.o_part;
  d.lse_part = (float *)(ws + p.lse);
  d.o_lat = ws + p.o_lat;
  e = launch_decode_attn(dt == MLA_BF16, d, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  // with FP8 projections the combine also writes o's quantised form (when
  // its group of 128 columns is one head: d_v = 128)
  const bool o8 = f8p && cfg->d_v == 128;
  e = dt == MLA_BF16 ? launch_decode_combine_uv(d, cfg->d_v, w->w_uv, o, o8 ? f8 : Fp8Out{nullptr, nullptr, 0}, st)
                     : hipErrorNotSupported;
  if (e != hipSuccess && e != hipErrorNotSupported) return MLA_ERR_HIP;
  const bool o_ready = o8 && e == hipSuccess;
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
    a.partial = partial.p;
    a.partial_bytes = partial.bytes;
    a.name = "unabsorb";
    e = launch_gemm(dt == MLA_BF16, gemm_tile_for(dt, M, a.N, a.batch, a.K), 1, 0, a, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  e = run_output(cfg, w, o, M, u, p.sk5, partial, f8p, o_ready, st);
  return hip_status(e);
}

// The allocation-free decode's workspace: one array per device, its device
// address looked up once per device (the array's host-side name is only a
// stand-in and never reaches a kernel).
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_WORKSPACE_BYTES];
std::mutex g_scratch_mu;
void *g_scratch_ptr[256];

hipError_t scratch_for_current_device(char **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char *)g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

mla_status mla_decode(const mla_config *cfg, const mla_weights *w, const void *h, int32_t batch, int32_t n_q,
                      const int32_t *cache_lens, const int32_t *cache_lens_host, int32_t max_cache_len,
                      const mla_cache *cache, void *u, void *o_heads, void *workspace, size_t workspace_bytes,
                      void *stream) {
  DecodePlan p;
  mla_status s = check_decode(cfg, w, h, batch, n_q, cache_lens, cache_lens_host, max_cache_len, cache, u, &p, false);
  if (s != MLA_OK) return s;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < p.total) return MLA_ERR_WORKSPACE;
  if ((s = debug_begin((hipStream_t)stream)) != MLA_OK) return s;
  return debug_end((hipStream_t)stream,
                   decode_steps(cfg, w, h, batch, n_q, cache_lens, cache, u, o_heads, (char *)workspace, p, stream));
}

mla_status mla_decode_noalloc(const mla_config *cfg, const mla_weights *w, const void *h, int32_t batch, int32_t n_q,
                              const int32_t *cache_lens, const int32_t *cache_lens_host, int32_t max_cache_len,
                              const mla_cache *cache, void *u, void *o_heads, void *stream) {
  DecodePlan p;
  mla_status s = check_decode(cfg, w, h, batch, n_q, cache_lens, cache_lens_host, max_cache_len, cache, u, &p, true);
  if (s != MLA_OK) return s;
  if (p.total > (size_t)MLA_NOALLOC_WORKSPACE_BYTES) return MLA_ERR_WORKSPACE;
  char *ws = nullptr;
  if (scratch_for_current_device(&ws) != hipSuccess) return MLA_ERR_HIP;
  if ((s = debug_begin((hipStream_t)stream)) != MLA_OK) return s;
  return debug_end((hipStream_t)stream, decode_steps(cfg, w, h, batch, n_q, cache_lens, cache, u, o_heads, ws, p, stream));
}

const char *mla_status_string(mla_status s) {
  // callers may pass any int: its bytes are read as an int (loading an enum
  // value outside the enumerators' range is undefined in C++)
  int code;
  memcpy(&code, &s, sizeof code);
  switch (code) {
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
  std::lock_guard<std::mutex> lock(g_timing_mu);
  g_timing = on != 0;
  g_used = 0;
  ++g_session;
  return MLA_OK;
}

int32_t mla_timing_read(const char **names, double *total_ms, int64_t *launches, int32_t cap) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  std::vector<const char *> keys;   // the static strings the launchers pass
  std::vector<double> ms;
  std::vector<int64_t> cnt;
  for (size_t i = 0; i < g_used; ++i) {
    const TimedLaunch &t = g_events[i];
    if (!t.done) continue;
    float el = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess) return MLA_ERR_HIP;
    if (hipEventElapsedTime(&el, t.start, t.stop) != hipSuccess) return MLA_ERR_HIP;
    size_t k = 0;
    while (k < keys.size() && strcmp(keys[k], t.name) != 0) ++k;
    if (k == keys.size()) {
      keys.push_back(t.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[k] += el;
    cnt[k] += 1;
  }
  for (size_t k = 0; k < keys.size() && (int32_t)k < cap; ++k) {
    if (names) names[k] = keys[k];
    if (total_ms) total_ms[k] = ms[k];
    if (launches) launches[k] = cnt[k];
  }
  g_used = 0;
  ++g_session;
  return (int32_t)keys.size();
}

}  // extern "C"
