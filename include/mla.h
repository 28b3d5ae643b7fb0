/*
 * libmla — DeepSeek-V3 Multi-head Latent Attention (MLA) on AMD MI355X (gfx950).
 *
 * The operation.  For a token with hidden state h (width d_model) at position
 * t of its sequence, MLA as written in the DeepSeek-V3 paper-reading notes
 * (hk.pswp.cn), section 2.1 "Multi-Head Latent Attention":
 *
 *   c_KV = W_DKV h                       joint key/value latent (width d_c)
 *   k_R  = RoPE(W_KR h, t)               decoupled RoPE key, one per token,
 *                                        shared by every head   (width d_R)
 *   c_Q  = W_DQ h                        query latent           (width d_cq)
 *   q_C,i = (W_UQ c_Q)_i,  q_R,i = RoPE((W_QR c_Q)_i, t)   per head i
 *   k_C,j,i = (W_UK c_KV,j)_i,  v_j,i = (W_UV c_KV,j)_i   per head i
 *   o_t,i = sum_{j<=t} softmax_j([q_C,i; q_R,i] . [k_C,j,i; k_R,j] / sqrt(d_h+d_R)) v_j,i
 *   u_t  = W_O [o_t,1; ...; o_t,n_h]
 *
 * Only [c_KV || k_R] is cached per token ("advantages of MLA" in the same
 * section): (d_c + d_R) elements per token and layer.
 *
 * Conventions (readings of the pages, which lost their sub/superscripts):
 *   - every weight is row-major [out][in] (the pages write W*h);
 *   - head i owns rows i*d_h..(i+1)*d_h-1 of W_UQ/W_UK (d_R for W_QR, d_v for
 *     W_UV) and columns i*d_v..(i+1)*d_v-1 of W_O;
 *   - RoPE rotates interleaved pairs (x[2k], x[2k+1]) by t * base^(-2k/d_R),
 *     t the 0-based position in the sequence;
 *   - attention is causal; the scale is 1/sqrt(d_nope + d_rope);
 *   - a cached row is [c_KV (d_c) || k_R (d_rope)] in the config dtype.
 *
 * Ownership: the caller owns every buffer (weights, cache pool, block table,
 * inputs, outputs, workspace).  The library never allocates device memory and
 * keeps no state between calls apart from optional kernel timing (below).
 * Unless a name ends in _host, pointers are device pointers.
 *
 * Errors: every argument is checked before any HIP call, so invalid calls
 * return an error code on any host, with or without a GPU.  A failed kernel
 * launch returns MLA_ERR_HIP.  Faults inside kernels surface at the caller's
 * next synchronisation of `stream`.  Calls are asynchronous on `stream`
 * (a hipStream_t passed as void*; NULL is the null stream).  Calls on distinct
 * streams with distinct buffers may run concurrently.
 */
#ifndef LIBMLA_MLA_H
#define LIBMLA_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = -2,       /* a size or dimension is out of range or inconsistent */
  MLA_ERR_DTYPE = -3,       /* unknown dtype */
  MLA_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than mla_workspace_size */
  MLA_ERR_CACHE = -5,       /* cache descriptor invalid or too small for the request */
  MLA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
  MLA_ERR_UNSUPPORTED = -7  /* valid MLA shape outside this build's envelope */
} mla_status;

typedef enum mla_dtype {
  MLA_FP32 = 0,  /* float32 storage and arithmetic throughout */
  MLA_BF16 = 1   /* bfloat16 storage, float32 accumulation */
} mla_dtype;

/* Layer dimensions.  Supported envelope (checked, MLA_ERR_UNSUPPORTED
 * otherwise): d_rope even; for BF16 d_model, d_cq, d_c multiples of 64,
 * d_nope, d_rope, d_v multiples of 32, n_heads*d_v a multiple of 64; for FP32
 * the same with 32 and 16.  DeepSeek-V3: 7168, 128, 128, 64, 128, 512, 1536. */
typedef struct mla_config {
  int32_t d_model;   /* hidden width of h and u */
  int32_t n_heads;   /* n_h */
  int32_t d_nope;    /* d_h: per-head content query/key width */
  int32_t d_rope;    /* d_R: decoupled RoPE query/key width */
  int32_t d_v;       /* per-head value width */
  int32_t d_c;       /* KV latent width */
  int32_t d_cq;      /* query latent width */
  int32_t dtype;     /* mla_dtype */
  double rope_base;  /* RoPE base (10000 for DeepSeek-V3) */
  /* YaRN context extension (the V3 highlights page, highlight 13, extends
   * the context from 4K to 128K with YaRN and the constants 40, 1, 32).
   * yarn_factor 0 or 1 leaves plain RoPE (the other three fields are then
   * ignored).  Otherwise pair k, of frequency theta_k = base^(-2k/d_rope),
   * turns r_k = yarn_orig_len * theta_k / (2 pi) times over the original
   * context and rotates at (1 - g) theta_k / yarn_factor + g theta_k with
   * g = clamp((r_k - beta_slow) / (beta_fast - beta_slow), 0, 1), and the
   * softmax scale is multiplied by (0.1 ln yarn_factor + 1)^2.
   * DeepSeek-V3 at 128K: 40, 4096, 1, 32.  MLA_ERR_SHAPE unless
   * yarn_factor > 1, yarn_orig_len > 0 and 0 < beta_slow < beta_fast (all
   * finite) when enabled. */
  double yarn_factor;
  double yarn_beta_slow;
  double yarn_beta_fast;
  int32_t yarn_orig_len;
} mla_config;

/* The eight projections, each row-major [out][in] in the config dtype:
 *   w_dq [d_cq][d_model]            w_uq [n_heads*d_nope][d_cq]
 *   w_qr [n_heads*d_rope][d_cq]     w_dkv [d_c][d_model]
 *   w_kr [d_rope][d_model]          w_uk [n_heads*d_nope][d_c]
 *   w_uv [n_heads*d_v][d_c]         w_o  [d_model][n_heads*d_v]            */
typedef struct mla_weights {
  const void *w_dq, *w_uq, *w_qr, *w_dkv, *w_kr, *w_uk, *w_uv, *w_o;
} mla_weights;

/* Latent cache.  pool holds n_blocks*block_size rows of (d_c + d_rope)
 * elements in the config dtype.
 *   Contiguous (block_table == NULL): position t of sequence b is row
 *     b*max_len + t; the pool must hold batch*max_len rows.
 *   Paged (block_table != NULL): block_table is int32 [batch][max_blocks_per_seq]
 *     on the device; position t of sequence b is row
 *     block_table[b*max_blocks_per_seq + t/block_size]*block_size + t%block_size.
 *     The caller allocates the blocks a call writes or reads; entries are
 *     not range-checked on the device. */
typedef struct mla_cache {
  void *pool;
  int32_t block_size;          /* rows per block (paged); any value >= 1 */
  int32_t n_blocks;            /* blocks in pool (paged) */
  const int32_t *block_table;  /* NULL = contiguous */
  int32_t max_blocks_per_seq;  /* paged: table row length */
  int32_t max_len;             /* contiguous: rows per sequence; paged: ignored */
} mla_cache;

/* Elements cached per token and layer, times the dtype size:
 * (d_c + d_rope) * sizeof(dtype).  1152 bytes for DeepSeek-V3 in BF16.
 * Returns 0 for an invalid config. */
size_t mla_cache_bytes_per_token(const mla_config *cfg);

/* Elements a standard multi-head attention would cache per token:
 * 2 * n_heads * d_nope (a key and a value per head).  0 if invalid. */
size_t mla_mha_cache_elements_per_token(const mla_config *cfg);

/* Operation codes for mla_workspace_size. */
#define MLA_OP_PREFILL 0
#define MLA_OP_DECODE 1

/* Bytes of device workspace a call needs.
 *   MLA_OP_PREFILL: batch sequences of len_or_nq tokens; max_cache_len unused.
 *   MLA_OP_DECODE : batch sequences of len_or_nq new tokens each, whose
 *     cache lengths (after appending) are at most max_cache_len; the split
 *     plan, and with it the size, depends only on these numbers.
 * The decode call must be given the same max_cache_len. */
mla_status mla_workspace_size(const mla_config *cfg, int32_t op, int32_t batch,
                              int32_t len_or_nq, int32_t max_cache_len, size_t *bytes);

/* Latent projection + RoPE key + cache append (section 2.1, "Key and Value
 * compression"; the cache holds only c_KV and k_R).
 *   h       [n][d_model] tokens to compress;
 *   seq_idx [n] int32 device: sequence of each token (0 <= seq_idx < batch);
 *   pos     [n] int32 device: position of each token within its sequence;
 *   batch   number of sequences the cache describes.
 * Writes row [c_KV || RoPE(W_KR h, pos)] for every token. */
mla_status mla_compress_kv(const mla_config *cfg, const mla_weights *w, const void *h,
                           int32_t n, const int32_t *seq_idx, const int32_t *pos,
                           int32_t batch, const mla_cache *cache, void *stream);

/* Causal prefill of `batch` sequences of `len` tokens (section 2.1 in full).
 *   h [batch][len][d_model] -> u [batch][len][d_model];
 *   writes cache positions 0..len-1 of every sequence;
 *   o_heads: optional [batch*len][n_heads][d_v] per-head attention outputs
 *   (before W_O), or NULL;
 *   workspace of at least mla_workspace_size(cfg, MLA_OP_PREFILL, batch, len, 0). */
mla_status mla_prefill(const mla_config *cfg, const mla_weights *w, const void *h,
                       int32_t batch, int32_t len, const mla_cache *cache, void *u,
                       void *o_heads, void *workspace, size_t workspace_bytes, void *stream);

/* Decode `n_q` new tokens per sequence against the latent cache.
 *   h [batch][n_q][d_model] -> u [batch][n_q][d_model];
 *   cache_lens [batch] int32 device: sequence lengths AFTER appending the new
 *     tokens (1 <= n_q <= cache_lens[b] <= max_cache_len).  The new tokens
 *     take positions cache_lens[b]-n_q .. cache_lens[b]-1 and query i sees
 *     keys 0..cache_lens[b]-n_q+i (causal among the new tokens);
 *   max_cache_len: host-side bound on cache_lens, also used for the split plan;
 *   o_heads: optional [batch*n_q][n_heads][d_v], or NULL.
 * Queries are absorbed into the latent space (W_UK folded into q, W_UV applied
 * after the softmax-weighted latent sum), so attention reads each cached row
 * once for all heads.  Workspace: mla_workspace_size(cfg, MLA_OP_DECODE,
 * batch, n_q, max_cache_len). */
mla_status mla_decode(const mla_config *cfg, const mla_weights *w, const void *h,
                      int32_t batch, int32_t n_q, const int32_t *cache_lens,
                      int32_t max_cache_len, const mla_cache *cache, void *u, void *o_heads,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static string). */
const char *mla_status_string(mla_status s);

/* Library version string (static). */
const char *mla_version(void);

/* Kernel timing, for profiling.  While enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on the stream it is
 * launched on; mla_timing_read synchronises those events and accumulates the
 * elapsed milliseconds per kernel name.  Not thread-safe; off by default.
 *   mla_timing_enable(1) starts (and clears) a session, 0 stops it.
 *   mla_timing_read fills up to `cap` entries (names are static strings) and
 *   returns the number of distinct kernel names, or a negative mla_status. */
mla_status mla_timing_enable(int32_t on);
int32_t mla_timing_read(const char **names, double *total_ms, int64_t *launches, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* LIBMLA_MLA_H */
