// Internal definitions shared by the libmla HIP sources (not part of the ABI).
//
// Matrix-core conventions used by every kernel (CDNA3/CDNA4 16x16 MFMA):
//   A operand (16 x K): lane l holds row (l & 15), k-slots [(l>>4)*KPL, +KPL)
//   B operand (K x 16): lane l holds col (l & 15), k-slots [(l>>4)*KPL, +KPL)
//   C/D (16 x 16 fp32): lane l holds col (l & 15), rows 4*(l>>4) + [0, 4)
// KPL = 8 for v_mfma_f32_16x16x32_bf16 and 1 for v_mfma_f32_16x16x4_f32.
//
// A contraction of length D is always fed as four contiguous runs: lane group
// g = l>>4 owns k in [g*D/4, (g+1)*D/4) and instruction s uses the slots
// [g*D/4 + s*KPL, +KPL).  A and B use the same assignment, so the sum is the
// full dot product (in a different order), and each lane reads one contiguous
// run per operand row: 16-byte LDS and global reads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// elements per 16-byte chunk
template <typename T> struct Vec { static constexpr int N = 16 / sizeof(T); };

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------
// Row -> (sequence, position) maps used by the GEMM epilogues
// ---------------------------------------------------------------------------
enum RowMode { ROWS_DENSE = 0, ROWS_DECODE = 1, ROWS_EXPLICIT = 2 };
struct RowMap {
  int mode;
  int per_seq;          // DENSE: tokens per sequence; DECODE: n_q
  const int *lens;      // DECODE: [batch] lengths after append
  const int *seq_idx;   // EXPLICIT
  const int *pos;       // EXPLICIT
};

__device__ inline void row_seq_pos(const RowMap &r, int m, int &seq, int &pos) {
  if (r.mode == ROWS_DENSE) {
    seq = m / r.per_seq;
    pos = m - seq * r.per_seq;
  } else if (r.mode == ROWS_DECODE) {
    seq = m / r.per_seq;
    pos = r.lens[seq] - r.per_seq + (m - seq * r.per_seq);
  } else {
    seq = r.seq_idx[m];
    pos = r.pos[m];
  }
}

struct CacheRef {
  void *pool;
  const int *table;   // NULL = contiguous
  int block_size;
  int max_blocks;
  int max_len;
  int d_row;          // elements per cached row (layer-dtype rows)
  int batch;          // sequences the descriptor covers
  long cap;           // positions per sequence: max_len, or max_blocks * block_size
  int bs_shift;       // log2(block_size) when it is a power of two, else -1
  int row_bytes;      // bytes per cached row
  int fp8;            // rows in the FP8 layout: d_c E4M3 codes | d_R bf16 | d_c/128 fp32 scales
  int n_blocks;       // blocks in the pool (paged)
  unsigned *dbg;      // debug builds: error word (bits MLA_DBG_*), else unused
};

// Debug builds (MLA_DEBUG_CHECKS) check on the device every block-table
// entry a kernel uses and every cache length it is given, and record what
// they find in the error word; the host reads it after the call.
#define MLA_DBG_BLOCK 1u    // a block-table entry outside [0, n_blocks)
#define MLA_DBG_LENGTH 2u   // a cache length or position outside the cache

__device__ inline void dbg_flag(const CacheRef &c, unsigned bit) {
#ifdef MLA_DEBUG_CHECKS
  atomicOr(c.dbg, bit);
#else
  (void)c;
  (void)bit;
#endif
}

// A block-table entry as used: in debug builds one outside the pool is
// reported and replaced by block 0 (in bounds), so a read stays inside the
// pool; writers ask cache_row_ok first and skip such a row.
__device__ inline int checked_block(const CacheRef &c, int blk) {
#ifdef MLA_DEBUG_CHECKS
  if (blk < 0 || blk >= c.n_blocks) {
    dbg_flag(c, MLA_DBG_BLOCK);
    return 0;
  }
#endif
  return blk;
}

__device__ inline int block_of(const CacheRef &c, int pos) {
  return c.bs_shift >= 0 ? (pos >> c.bs_shift) : pos / c.block_size;
}

__device__ inline long cache_row(const CacheRef &c, int seq, int pos) {
  if (c.table) {
    const int q = block_of(c, pos);
    const int blk = checked_block(c, c.table[(long)seq * c.max_blocks + q]);
    return (long)blk * c.block_size + (pos - q * c.block_size);
  }
  return (long)seq * c.max_len + pos;
}

// May a writer store position pos of sequence seq?  Rows outside the
// described cache are never written (silently in release builds; debug
// builds report them, and a block-table entry outside the pool).
__device__ inline bool cache_row_ok(const CacheRef &c, int seq, int pos) {
  if (seq < 0 || seq >= c.batch || pos < 0 || pos >= c.cap) {
    dbg_flag(c, MLA_DBG_LENGTH);
    return false;
  }
#ifdef MLA_DEBUG_CHECKS
  if (c.table) {
    const int blk = c.table[(long)seq * c.max_blocks + block_of(c, pos)];
    if (blk < 0 || blk >= c.n_blocks) {
      dbg_flag(c, MLA_DBG_BLOCK);
      return false;
    }
  }
#endif
  return true;
}

// ---------------------------------------------------------------------------
// GEMM epilogue: the output columns [0, N) are cut into up to four segments,
// each with its own destination.  A lane always holds four consecutive
// columns of one row; segment and RoPE-group widths are multiples of 4.
// ---------------------------------------------------------------------------
enum SegKind { SEG_PLAIN = 0, SEG_HEADS = 1, SEG_CACHE = 2 };
struct Seg {
  int n_end;      // exclusive end column
  int kind;
  int rope;       // rotate pairs (2k, 2k+1) inside each group of head_w columns
  int head_w;     // HEADS: columns per head; rope: group width
  float scale;    // applied after RoPE
  int out_f32;    // 1: store fp32 instead of the element type
  void *dst;      // PLAIN: dst[m*ld + col_off + c]; HEADS: dst[m*ld + h*head_ld + col_off + d]
  long ld;
  long head_ld;
  int col_off;    // also CACHE: column offset inside the cached row
  void *dst2;     // optional PLAIN mirror: dst2[m*ld2 + c] (element type)
  long ld2;
  long batch_stride;  // added to dst per batch index (batched GEMMs)
};
#define MLA_MAX_ROPE_PAIRS 64
struct Epi {
  Seg seg[4];
  int nseg;
  RowMap rows;
  CacheRef cache;
  double inv_freq[MLA_MAX_ROPE_PAIRS];  // base^(-2k/d_R), computed on the host in fp64
};

// angle = pos * inv_freq[k]: formed and reduced modulo 2*pi in fp64 so that
// positions up to 2^20 keep full fp32 accuracy, then sin/cos in fp32.
__device__ inline void rope_sincos(int pos, double inv_freq, float &s, float &c) {
  // turns = angle / 2pi in fp64, reduced to [-1/2, 1/2]; the hardware sin/cos
  // take turns (max abs error ~2e-7 over positions < 2^16, as sincosf)
  const double turns = (double)pos * inv_freq * 0.15915494309189533576888;
  const float f = (float)(turns - rint(turns));
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

template <typename T>
__device__ inline void store4(void *base, long off, const float v[4], int as_f32) {
  if (as_f32) {
    float *p = (float *)base + off;
    *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
  } else if (sizeof(T) == 2) {
    bf16x4 w = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *(bf16x4 *)((bf16 *)base + off) = w;
  } else {
    float *p = (float *)base + off;
    *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
  }
}

// Apply the epilogue to columns n..n+3 of row m (batch index z).
template <typename T>
__device__ inline void epi_store4(const Epi &e, int z, int m, int n, float v[4]) {
  int s = 0, nb = 0;
  while (s < e.nseg - 1 && n >= e.seg[s].n_end) { nb = e.seg[s].n_end; ++s; }
  const Seg &g = e.seg[s];
  const int c = n - nb;
  int seq = 0, pos = 0;
  if (g.rope || g.kind == SEG_CACHE) row_seq_pos(e.rows, m, seq, pos);
  if (g.rope) {
    const int k0 = (c % g.head_w) >> 1;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float sn, cs;
      rope_sincos(pos, e.inv_freq[k0 + p], sn, cs);
      float x0 = v[2 * p], x1 = v[2 * p + 1];
      v[2 * p] = x0 * cs - x1 * sn;
      v[2 * p + 1] = x0 * sn + x1 * cs;
    }
  }
  if (g.scale != 1.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= g.scale;
  }
  long off;
  void *base = g.dst;
  if (g.kind == SEG_PLAIN) {
    off = (long)z * g.batch_stride + (long)m * g.ld + g.col_off + c;
  } else if (g.kind == SEG_HEADS) {
    const int hh = c / g.head_w, d = c - hh * g.head_w;
    off = (long)z * g.batch_stride + (long)m * g.ld + (long)hh * g.head_ld + g.col_off + d;
  } else {
    // rows outside the described cache are never written
    if (!cache_row_ok(e.cache, seq, pos)) return;
    base = e.cache.pool;
    off = cache_row(e.cache, seq, pos) * e.cache.d_row + g.col_off + c;
  }
  store4<T>(base, off, v, g.out_f32);
  if (g.dst2) store4<T>(g.dst2, (long)m * g.ld2 + c, v, 0);
}

// The same epilogue for a thread whose columns n..n+3 are fixed (a tile that
// lies inside one segment): everything that depends on the columns, including
// the kernel-argument reads, is prepared once, so the per-row store issues no
// memory reads (on gfx9 a read after stores waits for those stores).
struct ColPlan {
  int kind, rope, out_f32, c;
  float scale;
  void *dst;
  long ld, col;        // element offset of the columns inside a row (PLAIN/HEADS) or cached row (CACHE)
  long batch_stride;
  void *dst2;
  long ld2;
  double inv0, inv1;   // RoPE frequencies of the two column pairs
};

__device__ inline int epi_segment(const Epi &e, int n, int &nb) {
  int s = 0;
  nb = 0;
  while (s < e.nseg - 1 && n >= e.seg[s].n_end) { nb = e.seg[s].n_end; ++s; }
  return s;
}

// Plan for columns n..n+3 inside segment sg (starting at column nb).  With a
// wave-uniform segment the kernel-argument reads are scalar loads; a per-lane
// segment search reads them with dependent vector loads.
__device__ inline ColPlan col_plan_in(const Epi &e, int sg, int nb, int n) {
  const Seg &g = e.seg[sg];
  ColPlan p;
  p.c = n - nb;
  p.kind = g.kind;
  p.rope = g.rope;
  p.out_f32 = g.out_f32;
  p.scale = g.scale;
  p.dst = g.dst;
  p.ld = g.ld;
  p.batch_stride = g.batch_stride;
  p.dst2 = g.dst2;
  p.ld2 = g.ld2;
  if (g.kind == SEG_HEADS) {
    const int hh = p.c / g.head_w, d = p.c - hh * g.head_w;
    p.col = (long)hh * g.head_ld + g.col_off + d;
  } else {
    p.col = g.col_off + p.c;
  }
  p.inv0 = p.inv1 = 0.0;
  if (g.rope) {
    const int k0 = (p.c % g.head_w) >> 1;
    p.inv0 = e.inv_freq[k0];
    p.inv1 = e.inv_freq[k0 + 1];
  }
  return p;
}

__device__ inline ColPlan col_plan(const Epi &e, int n) {
  int nb;
  const int sg = epi_segment(e, n, nb);
  return col_plan_in(e, sg, nb, n);
}

// Plan for a lane whose columns lie in the same segment as column n0, a
// value the whole wave shares (the first column of a tile that never
// straddles two segments).
__device__ inline ColPlan col_plan_tile(const Epi &e, int n0, int n) {
  int nb;
  const int sg = epi_segment(e, __builtin_amdgcn_readfirstlane(n0), nb);
  return col_plan_in(e, __builtin_amdgcn_readfirstlane(sg), __builtin_amdgcn_readfirstlane(nb), n);
}

template <typename T>
__device__ inline void col_store(const ColPlan &p, const Epi &e, int z, int m, float v[4]) {
  int seq = 0, pos = 0;
  if (p.rope || p.kind == SEG_CACHE) row_seq_pos(e.rows, m, seq, pos);
  if (p.rope) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float sn, cs;
      rope_sincos(pos, q ? p.inv1 : p.inv0, sn, cs);
      const float x0 = v[2 * q], x1 = v[2 * q + 1];
      v[2 * q] = x0 * cs - x1 * sn;
      v[2 * q + 1] = x0 * sn + x1 * cs;
    }
  }
  if (p.scale != 1.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= p.scale;
  }
  long off;
  void *base = p.dst;
  if (p.kind != SEG_CACHE) {
    off = (long)z * p.batch_stride + (long)m * p.ld + p.col;
  } else {
    if (!cache_row_ok(e.cache, seq, pos)) return;
    base = e.cache.pool;
    off = cache_row(e.cache, seq, pos) * e.cache.d_row + p.col;
  }
  store4<T>(base, off, v, p.out_f32);
  if (p.dst2) store4<T>(p.dst2, (long)m * p.ld2 + p.c, v, 0);
}

// ---------------------------------------------------------------------------
// Host-side launch descriptions
// ---------------------------------------------------------------------------
enum GemmTile { TILE_BIG = 0, TILE_SKINNY = 1 };

struct GemmArgs {
  const void *x; long ldx; long x_bs;           // X [M][K], row stride ldx, batch stride x_bs
  const void *w[4]; int w_end[4]; int nw;       // row segments of W ([N][K]) or one [K][N] matrix
  long ldw; long w_bs;
  int M, N, K;
  int splits, k_chunk;                          // split-K: K = splits * k_chunk
  int batch;
  float *partial;                               // splits > 1: [batch][splits][M][N]
  size_t partial_bytes;                         // its size: launchers refuse a layout that does not fit
  int tiles_m, tiles_n;
  int grouped;               // 8x8 tile groups per XCD (set by the launcher)
  const char *name;          // timing labels (static strings)
  const char *reduce_name;
  Epi epi;
  // Block-scaled FP8 operands (bf16 layers with FP8 projections): x holds
  // E4M3 codes [M][K] (ldx counts bytes), xs the activation scales as
  // biased 8-bit exponents [K/128][xs_ld] (xs_ld >= M rounded up to 256),
  // w[] E4M3 codes with power-of-two float32 scales wsc[] per block of 128
  // rows by 128 columns ([rows/128][wsc_ld], wsc_ld = K/128)
  int fp8;
  const unsigned char *xs;
  long xs_ld;
  const float *wsc[4];
  int wsc_ld;
};

// dtype: 0 fp32, 1 bf16.  swap: 1 -> output rows are tokens (segment
// epilogue); 0 -> transposed plain store dst[n*ld + m].  wkn: W stored [K][N].
hipError_t launch_gemm(int dtype, int tile, int swap, int wkn, GemmArgs &a, hipStream_t st);

// weight-streaming GEMM for up to 64 activation rows (bf16): usable when K is
// a multiple of 128, weight segments start on 64-row boundaries and a
// partial buffer of gemm_stream_partial_bytes(M) is given
bool gemm_stream_ok(const GemmArgs &a, int wkn);
// 256x128-tile GEMM for many tokens (bf16, W stored [N][K], batch 1)
bool gemm_big_ok(const GemmArgs &a);
hipError_t launch_gemm_big(GemmArgs &a, int swap, hipStream_t st);
size_t gemm_stream_partial_bytes(int M);
hipError_t launch_gemm_stream(GemmArgs &a, int wkn, hipStream_t st);

// Decode query path in one launch (decode_q.hip): q_up with RoPE and the
// absorption of W_UK, bf16 with d_cq 1536, d_nope 128, d_R 64, d_c 512 and
// up to 32 tokens.
struct DecodeQArgs {
  const bf16 *cq;                     // c_Q [T][d_cq]
  const bf16 *w_uq, *w_qr, *w_uk;     // [n_h*d_nope][d_cq], [n_h*d_R][d_cq], [n_h*d_nope][d_c]
  bf16 *q_abs;                        // [T][n_h][d_c + d_R]: q_lat, then the roped q_R
  int T, n_h;
  Epi epi;                            // the up-projection's epilogue (its RoPE segment stores q_R)
};
bool decode_q_supported(int d_cq, int d_nope, int d_rope, int d_c, int T);
hipError_t launch_decode_q(const DecodeQArgs &a, hipStream_t st);

// The quantised copy of an activation that feeds an FP8 projection: E4M3
// codes [T][K] and the scales' biased exponents [K/128][ld_s]; codes ==
// nullptr: none.
struct Fp8Out {
  unsigned char *codes, *scales;
  long ld_s;
};

struct FlashArgs {
  const void *q;    // [B*Lq][n_h][d_nope + d_rope] (q_C, then roped q_R)
  const void *k;    // [B*L][n_h][d_nope]
  const void *kr;   // [B*L][d_rope]
  const void *vt;   // [n_h*d_v][B*L]
  void *o;          // [B*Lq][n_h][d_v]
  int B, L, n_h, d_nope, d_rope, d_v;
  float scale_log2;  // softmax scale * log2(e)
  // Queries after a cached prefix (lens != nullptr): sequence b holds
  // lens[b] keys (rows b*L ..), and its Lq queries are its last Lq
  // positions, lens[b]-Lq .. lens[b]-1.  lens == nullptr: Lq = L and the
  // queries are positions 0..L-1 (plain prefill).
  const int *lens;
  int Lq;
};
hipError_t launch_flash_prefill(int dtype, const FlashArgs &a, hipStream_t st);
// the widths the queries-after-a-prefix form runs at (bf16 128/64/128)
bool flash_prefix_supported(int dtype, int d_nope, int d_rope, int d_v);
// rows 0..Lpad-1 of every sequence's cache (bf16 layout) as dense c_KV
// [B*Lpad][d_c] and k_R [B*Lpad][d_rope], zero past each length
hipError_t launch_prefix_gather(const CacheRef &c, const int *lens, int B, int Lpad, int d_c, int d_rope, void *ckv,
                                void *kr, hipStream_t st);

struct DecodeArgs {
  const void *q;      // absorbed queries [B*n_q][n_h][d_c + d_rope]
  CacheRef cache;
  const int *lens;    // [B]
  int B, n_q, n_h, d_c, d_rope;
  float scale_log2;   // softmax scale * log2(e)
  // Split plan.  The cached rows of all sequences, in KV tiles, are laid end
  // to end in sequence order; each row group's W workgroups take equal
  // contiguous ranges of ceil(total tiles / W) tiles, so a workgroup may hold
  // the end of one sequence and the start of the next.  The part of sequence
  // b that workgroup w holds writes partial slot w + b (unique, and a
  // sequence's slots are consecutive); slots = W + B bounds them.
  int W;              // workgroups per row group
  int slots;          // partial slots: W + B
  int row_groups;     // groups of query rows (n_q*n_h rows per sequence)
  int rows;           // query rows per group (the workgroup's share)
  void *o_part;       // [slots][n_q*n_h][d_c], normalised, in the layer's dtype
  float *lse_part;    // [slots][n_q*n_h]  (log2 units)
  void *o_lat;        // combine output [B*n_q][n_h][d_c]
};
int decode_rows_per_group(int dtype, long B, long R, int cus);
int decode_kv_tile(int dtype);
hipError_t launch_decode_attn(int dtype, const DecodeArgs &a, hipStream_t st);
hipError_t launch_decode_combine(int dtype, const DecodeArgs &a, hipStream_t st);
// bf16 split combine fused with o = W_UV o_lat (hipErrorNotSupported outside
// d_c = 512, d_R = 64, d_v = 128: then combine and un-absorb run separately)
// q8: also write o in that form (the W_O input of the FP8 projections)
hipError_t launch_decode_combine_uv(const DecodeArgs &a, int d_v, const void *w_uv, void *o, Fp8Out q8,
                                    hipStream_t st);

// FP8 cache append: token m's c_KV (ckv[m][0:d_c], bf16) and RoPE key
// (kr[m][0:d_rope], bf16) are quantised (a scale per 128 columns) and written
// to row (seq, pos) of the cache as the RowMap gives it.
struct CacheAppendArgs {
  const bf16 *ckv;
  const bf16 *kr;
  int T, d_c, d_rope;
  RowMap rows;
  CacheRef cache;
};
hipError_t launch_cache_append_fp8(const CacheAppendArgs &a, hipStream_t st);

// Activations of the FP8 projections (quant_fp8.hip): x [T][K] bf16 (row
// stride ldx) -> E4M3 codes [T][K] and per token and 128 columns the scale's
// biased exponent, stored [K/128][ld_s].  K a multiple of 512.
hipError_t launch_quant_act_fp8(const bf16 *x, long ldx, int T, int K, unsigned char *codes, unsigned char *scales,
                                long ld_s, hipStream_t st);

// kernel timing hooks (implemented with the C ABI)
void timing_before(const char *name, hipStream_t st);
void timing_after(const char *name, hipStream_t st);

}  // namespace mla
