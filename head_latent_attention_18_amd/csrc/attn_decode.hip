// Absorbed MLA decode attention over the latent cache, split along the cache
// positions, and the log-sum-exp combine of the splits.
//
// With W_UK folded into the query (q_lat,i = W_UK,i^T q_C,i) the score of head
// i against cached row j is [q_lat,i ; q_R,i] . [c_KV,j ; k_R,j], and with W_UV
// applied after the softmax the latent output is o_lat,i = sum_j p_j c_KV,j
// (associativity of the products in section 2.1 of the DeepSeek-V3
// paper-reading notes: "Key and Value compression", "attention
// computation").  Every cached row is therefore read once for all heads.
//
// One workgroup = (sequence b, split s, group of 16*NW*HB query rows); a query
// row is a (new token, head) pair; each wave owns 16*HB rows.  Per 32-row cache tile:
//   * the tile is staged in LDS twice: as rows ([kv][d_c+d_R], for the
//     scores) and transposed ([d][kv], latent part only, for P.V), so both
//     MFMA contractions read 16-byte runs;
//   * S^T = C . Q^T on the matrix cores: each lane ends with the scores of
//     one query row for eight cache rows, so the running max and sum are
//     lane-local plus two cross-lane-group shuffles;
//   * the cache rows feeding the A operand are permuted so that those eight
//     rows are consecutive, and the probabilities become the B operand of
//     O^T += C_lat^T . P^T straight from registers.
// Split results are stored normalised with their log2-sum-exp; the combine
// weights them by exp2(lse_s - max lse).
#include <type_traits>

#include "mla_internal.h"

namespace mla {

// Block -> work item (unit = (sequence, split), row group).  Items in unit
// order, a contiguous eighth of them per XCD (blocks x, x+8, x+16, .. run on
// XCD x): with eight units or more the row groups of a unit and the splits of
// a sequence share an XCD, whose L2 serves their common reads (queries, cache
// tiles); with fewer units (one long sequence, many query rows) the row
// groups still spread over all eight XCDs.
__device__ inline bool decode_item(const DecodeArgs &a, int &unit, int &rg) {
  const int W = a.B * a.n_splits * a.row_groups, per = (W + 7) / 8;
  const int slot = blockIdx.x >> 3, item = (blockIdx.x & 7) * per + slot;
  if (slot >= per || item >= W) return false;
  unit = item / a.row_groups;
  rg = item - unit * a.row_groups;
  return true;
}
inline int decode_grid(const DecodeArgs &a) { return 8 * ((a.B * a.n_splits * a.row_groups + 7) / 8); }

constexpr int KVT = 32;  // cache rows per tile (two 16-row MFMA blocks)

template <typename T, int NW, int HB, int DC, int DR>
__global__ __launch_bounds__(64 * NW, 1) void decode_attn_kernel(DecodeArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int D = DC + DR;
  constexpr int KPL = Mma<T>::KPL;
  constexpr int VE = Vec<T>::N;
  constexpr int RUN = D / 4;
  constexpr int QS = RUN / KPL;
  constexpr int PRUN = KVT / 4;
  constexpr int PS = PRUN / KPL;
  constexpr int DB = DC / 16;
  constexpr int LDC = D + VE;
  constexpr int LDT = KVT + VE;
  constexpr int ROWS = 16 * NW * HB;
  static_assert(RUN % KPL == 0 && PRUN % KPL == 0, "");
  static_assert(DC % VE == 0 && DR % VE == 0, "");
  constexpr int LAT_ITEMS = (KVT / 4) * (DC / VE);   // 4 rows x one chunk each
  constexpr int ROPE_ITEMS = KVT * (DR / VE);
  constexpr int LPT = (LAT_ITEMS + NT - 1) / NT;
  constexpr int RPT = (ROPE_ITEMS + NT - 1) / NT;
  typedef typename Mma<T>::frag frag;

  __shared__ __attribute__((aligned(16))) T cn[2][KVT * LDC];
  __shared__ __attribute__((aligned(16))) T ct[2][DC * LDT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;

  // block -> (unit = (b, s), row group)
  int unit, rg;
  if (!decode_item(a, unit, rg)) return;
  const int b = unit / a.n_splits, s = unit % a.n_splits;
  // lengths beyond the plan or the cache are clamped, so no read leaves the cache
  const int len = (int)min((long)a.lens[b], min((long)a.n_splits * a.chunk, a.cache.cap));
  const int kv_beg = s * a.chunk;
  if (kv_beg >= len) return;
  const int kv_end = min(len, kv_beg + a.chunk);
  const int R = a.n_q * a.n_h;
  const int row0 = rg * ROWS + wave * 16 * HB;
  const float sl2 = a.scale_log2;

  // query fragments (B operand), kept in registers for the whole split
  frag qf[HB][QS];
  int limit[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int r = min(row0 + hb * 16 + lrow, R - 1);
    const T *qrow = (const T *)a.q + ((long)b * R + r) * D + lgrp * RUN;
#pragma unroll
    for (int q = 0; q < QS; ++q) qf[hb][q] = *(const frag *)(qrow + q * KPL);
    limit[hb] = min(len - a.n_q + r / a.n_h, kv_end - 1);
  }

  f32x4 oacc[DB][HB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < HB; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun[HB], lrun[HB];
#pragma unroll
  for (int j = 0; j < HB; ++j) { mrun[j] = -1e30f; lrun[j] = 0.f; }

  const T *pool = (const T *)a.cache.pool;
  u32x4 lr[LPT][4], rr[RPT];
  auto row_ptr = [&](int kv) -> const T * {
    kv = min(kv, kv_end - 1);
    return pool + cache_row(a.cache, b, kv) * (long)D;
  };
  auto gload = [&](int kvb) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int it = tid + i * NT;
      if (it < LAT_ITEMS) {
        const int quad = it % (KVT / 4), cc = it / (KVT / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) lr[i][r] = *(const u32x4 *)(row_ptr(kvb + quad * 4 + r) + cc * VE);
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int it = tid + i * NT;
      if (it < ROPE_ITEMS) {
        const int kv = it % KVT, cc = it / KVT;
        rr[i] = *(const u32x4 *)(row_ptr(kvb + kv) + DC + cc * VE);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int it = tid + i * NT;
      if (it < LAT_ITEMS) {
        const int quad = it % (KVT / 4), cc = it / (KVT / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) *(u32x4 *)&cn[buf][(quad * 4 + r) * LDC + cc * VE] = lr[i][r];
        const T *e0 = (const T *)&lr[i][0], *e1 = (const T *)&lr[i][1];
        const T *e2 = (const T *)&lr[i][2], *e3 = (const T *)&lr[i][3];
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          T *dst = &ct[buf][(cc * VE + j) * LDT + quad * 4];
          if constexpr (sizeof(T) == 2) {
            *(bf16x4 *)dst = bf16x4{e0[j], e1[j], e2[j], e3[j]};
          } else {
            *(f32x4 *)dst = f32x4{e0[j], e1[j], e2[j], e3[j]};
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int it = tid + i * NT;
      if (it < ROPE_ITEMS) {
        const int kv = it % KVT, cc = it / KVT;
        *(u32x4 *)&cn[buf][kv * LDC + DC + cc * VE] = rr[i];
      }
    }
  };

  const int ntiles = (kv_end - kv_beg + KVT - 1) / KVT;
  gload(kv_beg);
  lstore(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kvb = kv_beg + t * KVT;
    if (t + 1 < ntiles) gload(kvb + KVT);

    // scores: S^T[kv][row] for two 16-row kv blocks
    f32x4 sacc[2][HB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) sacc[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kvl0 = 8 * (lrow >> 2) + (lrow & 3);  // permuted cache row of this A slot
#pragma unroll
    for (int q = 0; q < QS; ++q) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const frag ca = *(const frag *)&cn[buf][(kvl0 + 4 * kb) * LDC + lgrp * RUN + q * KPL];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) sacc[kb][hb] = Mma<T>::mma(ca, qf[hb][q], sacc[kb][hb]);
      }
    }

    // online softmax (base 2); lane holds rows kv = kvb + 8*lgrp + 4*kb + i
    typename Mma<T>::frag pf[HB][PS];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float sv[2][4];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kv = kvb + 8 * lgrp + 4 * kb + i;
          const float x = sacc[kb][hb][i] * sl2;
          sv[kb][i] = (kv <= limit[hb]) ? x : -INFINITY;
          mt = fmaxf(mt, sv[kb][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mnew = fmaxf(mrun[hb], mt);
      const float alpha = exp2f(mrun[hb] - mnew);
      mrun[hb] = mnew;
      float psum = 0.f;
      float p[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = exp2f(sv[kb][i] - mnew);
          psum += p[kb][i];
        }
      lrun[hb] = lrun[hb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db][hb] *= alpha;
      if constexpr (KPL == 8) {
        bf16x8 f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (bf16)p[j >> 2][j & 3];
        pf[hb][0] = f;
      } else {
#pragma unroll
        for (int j = 0; j < PS; ++j) pf[hb][j] = p[j >> 2][j & 3];
      }
    }

    // O^T[d][row] += C_lat^T[d][kv] . P^T[kv][row]
#pragma unroll
    for (int ps = 0; ps < PS; ++ps)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const frag va = *(const frag *)&ct[buf][(db * 16 + lrow) * LDT + lgrp * PRUN + ps * KPL];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) oacc[db][hb] = Mma<T>::mma(va, pf[hb][ps], oacc[db][hb]);
      }

    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // normalise and store this split's partial result
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float l = lrun[hb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = row0 + hb * 16 + lrow;
    if (r < R) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const long pbase = ((long)b * a.n_splits + s) * R + r;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 o4 = oacc[db][hb] * inv;
        const float v[4] = {o4[0], o4[1], o4[2], o4[3]};
        store4<T>(a.o_part, pbase * DC + db * 16 + 4 * lgrp, v, 0);
      }
      if (lgrp == 0) a.lse_part[pbase] = l > 0.f ? mrun[hb] + log2f(l) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel for gfx950 (d_c = 512, d_R = 64), ROWS = 128 or 64 query rows
// per workgroup.  The cache tile goes HBM -> LDS with global_load_lds_dwordx4
// (lane i's 16 bytes land at base + 16*i; no staging registers) into a ring
// of four stages, two tiles ahead.  Per tile, two phases separated by a
// barrier:
//   A (scores): wave w owns query rows (ROWS/4)w.. and computes their scores
//     against the 32 cached rows, S^T = C . Q^T, from 16-byte row reads of the
//     stage; the softmax is lane-local (each lane holds eight scores of one
//     query row) plus two shuffles.  The bf16 probabilities go to LDS.
//   B (P.V): wave w owns latent columns 128w..128w+127 for all ROWS query rows:
//     O^T[d][row] += C_lat^T[d][kv] . P^T[kv][row], with C_lat^T read by
//     ds_read_b64_tr_b16 (lane i of a 16-lane group receives column i of the
//     4x16 block of 16-bit elements the group addresses) and P^T from LDS.
// So each wave reads the tile once as rows and only its own quarter of the
// latent part transposed.  One wave per SIMD: at ROWS = 128, 512 registers
// hold the queries of 32 rows and the 128x128 O^T block (in AGPRs).  The
// softmax reference of a row is the max of its first tile and never moves (no
// O rescale: numerator and denominator share the reference, so the result is
// the same softmax); a row whose scores later rise more than 2^32 above it is
// flagged and recomputed exactly by the combine.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
#ifndef DECODE_PF
#define DECODE_PF 2               // score steps of cache fragments read ahead
#endif
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4)); }

// HBM -> LDS copy of 16 bytes per lane: lane i's bytes from gbase + off land
// at LDS address lds + 16*i (lds wave-uniform).  Issued as an asm statement,
// so the compiler does not see an LDS write that it would order every later
// LDS read after (with a wait for all loads in flight): the kernels using it
// wait for their copies themselves (vmcnt, then a barrier) before reading.
__device__ inline void dma16(const void *gbase, unsigned off, unsigned lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(gbase)
      : "memory", "m0");
}

// Max over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the
// gfx950 cross-row swaps (VALU, no LDS round trip).
__device__ inline float row_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Workgroup barrier without the release/acquire fences of __syncthreads (those
// would also wait for the cache copies still in flight).  The empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ inline void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DC, int DR, bool PAGED, int ROWS>
__global__ __launch_bounds__(256, 1) void decode_attn_dma_kernel(DecodeArgs a) {
  constexpr int NW = 4, NT = 64 * NW;
  constexpr int D = DC + DR;
  constexpr int CH = D / 8;                          // 16-byte chunks per cached row
  constexpr int LOADS = KVT * CH / NT;               // copy instructions per wave per tile
  constexpr int STAGE = KVT * D;                     // elements per stage
  constexpr int NS = 4;                              // ring stages (two tiles ahead)
  constexpr int QS = D / 32;                         // 32-wide k steps of the scores
  constexpr int HA = ROWS / (16 * NW);               // 16-row blocks per wave in the scores
  constexpr int DW = DC / NW, DBW = DW / 16;         // latent columns per wave in P.V
  constexpr int HBS = ROWS / 16;                     // 16-row blocks in P.V
  constexpr int PF = DECODE_PF;                      // score steps read ahead
  constexpr int PVS = HBS - HA;                      // P.V row blocks interleaved with the scores
  // P = exp2(score - reference) stays below 2^TAU, so P (bf16), l and O (fp32)
  // keep their range without ever rescaling O
  constexpr float TAU = 32.0f, MREF0 = -1e30f;
  static_assert(KVT * CH % NT == 0 && CH % 8 == 0 && DC % (16 * NW) == 0 && DBW == 8, "");
  static_assert(ROWS % (16 * NW) == 0 && HA >= 1 && HA <= 2, "");
  static_assert(QS > PF && QS >= 2 * PVS && QS >= 2 * LOADS, "");

  // 4 x 36 KB stages + 2 x 8 KB of P = 160 KB.  Rows have no padding: the
  // 16-byte chunk index is XORed with (row & 7), which keeps both the 16-byte
  // score reads and the transposed reads free of bank conflicts.
  __shared__ __attribute__((aligned(16))) bf16 stages[NS * STAGE];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2 * 4 * ROWS];   // P[buf][g][row]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  int unit, rg;
  if (!decode_item(a, unit, rg)) return;
  const int b = unit / a.n_splits, s = unit % a.n_splits;
  const int len = (int)min((long)a.lens[b], min((long)a.n_splits * a.chunk, a.cache.cap));
  const int kv_beg = s * a.chunk;
  if (kv_beg >= len) return;
  const int kv_end = min(len, kv_beg + a.chunk);
  const int R = a.n_q * a.n_h;
  const int rbase = rg * ROWS;
  const float sl2 = a.scale_log2;
  const bf16 *pool = (const bf16 *)a.cache.pool;
  const long seq_row0 = (long)b * a.cache.max_len;
  const unsigned lds_stages = (unsigned)(size_t)(lds_void *)stages;
  const int ntiles = (kv_end - kv_beg + KVT - 1) / KVT;

  // Copies.  Stage slot (row, c) holds cache chunk (row, c ^ (row & 7)); a
  // tile lies inside one cache block (block_size is a multiple of the tile),
  // so its rows are contiguous: a uniform base plus 32-bit lane offsets.  The
  // lane's slot of instruction i is i*NT + tid; its (row, chunk) advances by
  // NT = 3*CH + 40 per instruction.  Rows past the end of a partial last tile
  // repeat its last row (finite values; their probabilities are 0).
  static_assert(NT / CH == 3 && NT % CH == 40, "");
  const int r0 = tid / CH, c0 = tid - (tid / CH) * CH;
  auto tile_src = [&](int t) {
    const int kvb = kv_beg + t * KVT;
    long trow;
    if constexpr (PAGED) {
      const int q = block_of(a.cache, kvb);
      const int blk = __builtin_amdgcn_readfirstlane(a.cache.table[(long)b * a.cache.max_blocks + q]);
      trow = (long)blk * a.cache.block_size + (kvb - q * a.cache.block_size);
    } else {
      trow = seq_row0 + kvb;
    }
    return (const char *)(pool + trow * D);
  };
  struct Cursor { int r, c; };
  auto copy_next = [&](const char *src, int t, int i, Cursor &cu) {
    const int last = min(KVT, kv_end - (kv_beg + t * KVT)) - 1;
    const int r = min(cu.r, last);
    const unsigned dst = lds_stages + (unsigned)((t % NS) * STAGE * 2) + i * NT * 16 + wave * 1024;
    dma16(src, (unsigned)(r * D + ((cu.c ^ (r & 7)) << 3)) * 2u, dst);
    cu.c += NT % CH;
    const bool wrap = cu.c >= CH;
    cu.c -= wrap ? CH : 0;
    cu.r += NT / CH + (wrap ? 1 : 0);
  };

  // score state: this wave's HA blocks of 16 query rows
  bf16x8 qf[HA][QS];
  int limit[HA];
  float mref[HA], lrun[HA];
#pragma unroll
  for (int ha = 0; ha < HA; ++ha) {
    const int r = min(rbase + (wave * HA + ha) * 16 + lrow, R - 1);
    const bf16 *qrow = (const bf16 *)a.q + ((long)b * R + r) * D + lgrp * 8;
#pragma unroll
    for (int q = 0; q < QS; ++q) qf[ha][q] = *(const bf16x8 *)(qrow + q * 32);
    limit[ha] = min(len - a.n_q + r / a.n_h, kv_end - 1);
    mref[ha] = MREF0;
    lrun[ha] = 0.f;
  }
  bool ovf = false;

  // P.V state: O^T for latent columns wave*DW.. and all ROWS rows
  f32x4 oacc[DBW][HBS];
#pragma unroll
  for (int i = 0; i < DBW; ++i)
#pragma unroll
    for (int j = 0; j < HBS; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the queries are in registers before the first copy is issued, so no wait
  // for them is left inside the loop (where it would also wait for copies)
  wait_vmcnt<0>();
  for (int t = 0; t < 2 && t < ntiles; ++t) {
    const char *src = tile_src(t);
    Cursor cu = {r0, c0};
#pragma unroll
    for (int i = 0; i < LOADS; ++i) copy_next(src, t, i, cu);
  }

  // Score reads: rows lrow and 16+lrow, logical chunk 4q+lgrp (natural k
  // order), physical chunk (4q+lgrp) ^ (lrow & 7) = 4(q ^ fq) + (lgrp ^ (lrow & 3))
  // with fq = (lrow >> 2) & 1: even and odd steps use two base offsets.
  // Lane group g then holds the scores of rows 4g..4g+3 and 16+4g..16+4g+3,
  // and the transposed reads of P.V fetch exactly those rows (any four rows
  // can form the 4x16 block), so P keeps that key order in LDS.
  const int fq = (lrow >> 2) & 1, gq = lgrp ^ (lrow & 3);
  const int a_even = lrow * D + (4 * fq + gq) * 8, a_odd = lrow * D + (gq - 4 * fq) * 8;
  // Transposed reads: row r = 4*lgrp + (lrow >> 2) (and r + 16), elements
  // 4*(lrow & 3).. of the wave's 16-column block db: physical chunk
  // wave*16 + 2*(db ^ fh) + cl, fh = (r & 7) >> 1, cl = ((lrow & 3) >> 1) ^ (r & 1).
  int t_base, t_fh;
  {
    const int r = 4 * lgrp + (lrow >> 2), fr = r & 7;
    const int cl = ((lrow & 3) >> 1) ^ (fr & 1), half = (lrow & 1) * 4;
    t_base = r * D + (wave * 16 + cl) * 8 + half;
    t_fh = fr >> 1;
  }
  constexpr int TRH = 16 * D;   // sixteen rows further
  const lds_bf16 *st_base = (const lds_bf16 *)stages;
  lds_bf16x8 *pl = (lds_bf16x8 *)pbuf;

  // P.V of tile u (stage u % NS, P buffer u & 1); the V^T fragments of the
  // wave's columns are read once per tile
  bf16x8 va[DBW];
  auto load_v = [&](int u) {
    const lds_bf16 *st = st_base + (u % NS) * STAGE;
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      const int o = t_base + 16 * ((db & 3) ^ t_fh) + 64 * (db >> 2);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + o));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + o + TRH));
      va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto pv_block = [&](int u, int hb) {
    const bf16x8 pb = pl[((u & 1) * 4 + lgrp) * ROWS + hb * 16 + lrow];
#pragma unroll
    for (int db = 0; db < DBW; ++db) oacc[db][hb] = Mma<bf16>::mma(va[db], pb, oacc[db][hb]);
  };

  // Scores and softmax of tile t (stage t % NS) into P buffer t & 1.  When
  // WITH_PV, the P.V of tile t-1 is interleaved: row blocks 0..PVS-1 between
  // the score steps, the last two with the softmax.  The copy of tile t+2 is
  // spread over the odd score steps (one instruction each).
  auto scores = [&](int t, auto with_pv_c) {
    constexpr bool WITH_PV = decltype(with_pv_c)::value;
    const lds_bf16 *ca_p = st_base + (t % NS) * STAGE;
    const int kvb = kv_beg + t * KVT;
    if (t + 2 < ntiles) {
      const char *src = tile_src(t + 2);
      Cursor cu = {r0, c0};
#pragma unroll
      for (int i = 0; i < LOADS; ++i) copy_next(src, t + 2, i, cu);
    }
    f32x4 sacc[2][HA];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ha = 0; ha < HA; ++ha) sacc[kb][ha] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto rd = [&](int q, int kb) {
      return *(const lds_bf16x8 *)(ca_p + ((q & 1) ? a_odd : a_even) + q * 32 + kb * 16 * D);
    };
    bf16x8 ca[PF + 1][2];
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      ca[q][0] = rd(q, 0);
      ca[q][1] = rd(q, 1);
    }
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      if (q + PF < QS) {
        ca[(q + PF) % (PF + 1)][0] = rd(q + PF, 0);
        ca[(q + PF) % (PF + 1)][1] = rd(q + PF, 1);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ha = 0; ha < HA; ++ha) sacc[kb][ha] = Mma<bf16>::mma(ca[q % (PF + 1)][kb], qf[ha][q], sacc[kb][ha]);
      if constexpr (WITH_PV) {
        if (q % 2 == 1 && q / 2 < PVS) pv_block(t - 1, q / 2);
      }

      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ha = 0; ha < HA; ++ha) {
      float sv[2][4];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kv = kvb + 16 * kb + 4 * lgrp + i;
          const float x = sacc[kb][ha][i] * sl2;
          sv[kb][i] = (kv <= limit[ha]) ? x : -INFINITY;
          mt = fmaxf(mt, sv[kb][i]);
        }
      // The first tile fixes the reference of each row (max over the four
      // lane groups that share it).  Later tiles only check, per lane, that
      // their scores stay within TAU of it; the flags are merged at the end.
      if (t == 0) mref[ha] = fmaxf(row_max(mt), MREF0);
      else ovf |= mt > mref[ha] + TAU;
      bf16x8 pf;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(sv[j >> 2][j & 3] - mref[ha]);
        psum += p;
        pf[j] = (bf16)p;
      }
      lrun[ha] += psum;
      pl[((t & 1) * 4 + lgrp) * ROWS + (wave * HA + ha) * 16 + lrow] = pf;
      if constexpr (WITH_PV) pv_block(t - 1, PVS + ha);
    }
  };

  // Iteration i: tile i has landed (tile i+1 may still be in flight); the
  // scores of tile i run with the P.V of tile i-1 (whose P every wave wrote in
  // iteration i-1) and the copy of tile i+2 into stage (i+2) % 4, last read by
  // the P.V of tile i-2 in the previous iteration.  One barrier per iteration.
  auto sync = [&](int i) {
    if (i + 1 < ntiles) wait_vmcnt<LOADS>();   // this wave's copies of tile i
    else wait_vmcnt<0>();
    wait_lgkm0();                              // this wave's P of tile i-1
    bar();
  };
  sync(0);
  scores(0, std::false_type());
  for (int i = 1; i < ntiles; ++i) {
    sync(i);
    load_v(i - 1);
    scores(i, std::true_type());
  }
  sync(ntiles);
  load_v(ntiles - 1);
#pragma unroll
  for (int hb = 0; hb < HBS; ++hb) pv_block(ntiles - 1, hb);

  // normalise and store this split's partial result: the score lanes hold l
  // and the reference of their rows, the P.V lanes the O columns.  A row
  // marked in overflow gets lse = NaN; the combine recomputes it exactly.
  ovf = row_max(ovf ? 1.f : 0.f) > 0.f;
  __syncthreads();   // P no longer read: its space holds 1/l per row
  float *fac = (float *)pbuf;
#pragma unroll
  for (int ha = 0; ha < HA; ++ha) {
    float l = lrun[ha];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int rl = (wave * HA + ha) * 16 + lrow;
    if (lgrp == 0) {
      fac[rl] = l > 0.f ? 1.f / l : 0.f;
      if (rbase + rl < R)
        a.lse_part[((long)b * a.n_splits + s) * R + rbase + rl] =
            ovf ? __builtin_nanf("") : l > 0.f ? mref[ha] + log2f(l) : -INFINITY;
    }
  }
  __syncthreads();
  // The normalised rows go through the (now idle) stages as bf16 [ROWS][DC],
  // 16-byte chunk c of row r at chunk c ^ (r & 15), and leave one whole row
  // per wave instruction: a lane's own four columns per 16-row block would
  // make every store touch sixteen rows.
  static_assert(ROWS * DC <= NS * STAGE && DC / 8 == 64, "");
  lds_bf16 *ot = (lds_bf16 *)stages;
#pragma unroll
  for (int hb = 0; hb < HBS; ++hb) {
    const int rl = hb * 16 + lrow;
    const float inv = fac[rl];
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      const f32x4 o4 = oacc[db][hb] * inv;
      const int c = (wave * 16 + db * 2 + (lgrp >> 1)) ^ lrow;
      *(lds_bf16x4 *)(ot + rl * DC + c * 8 + (lgrp & 1) * 4) =
          bf16x4{(bf16)o4[0], (bf16)o4[1], (bf16)o4[2], (bf16)o4[3]};
    }
  }
  __syncthreads();
  bf16 *op = (bf16 *)a.o_part + (((long)b * a.n_splits + s) * R + rbase) * DC + lane * 8;
  for (int rl = wave; rl < ROWS && rbase + rl < R; rl += NW)
    *(bf16x8 *)(op + (long)rl * DC) = *(const lds_bf16x8 *)(ot + rl * DC + (lane ^ (rl & 15)) * 8);
}

// Two waves per SIMD: 64 query rows, 8 waves.  With one wave per SIMD the
// waits of that wave (copies, LDS reads, the softmax's VALU chain) leave its
// matrix core idle; here a second wave can issue meanwhile, and the registers
// of each (queries of 16 rows, O^T of 64 columns x 64 rows) fit in 256.
//   A (scores): waves w and w+4 hold the queries of rows 16(w&3)..+15; wave
//     w scores them against cache rows 0..15 of the tile, wave w+4 against
//     rows 16..31.  The reference of a row is the max over both halves of its
//     first tile (exchanged once through LDS).  Each lane writes its four
//     probabilities into its half's part of the P entry, so P has the layout
//     of the kernel above.
//   B (P.V): wave w owns latent columns 64w..64w+63 for all 64 rows.
// Waves 0..3 issue the cache copies (the pattern of the kernel above) and,
// first, the copies of the 64 query rows, which reach registers through
// stages 2 and 3 (whole rows per copy instead of sixteen-row register loads).
template <int DC, int DR, bool PAGED>
__global__ __launch_bounds__(512, 1) void decode_attn_dma8_kernel(DecodeArgs a) {
  constexpr int NW = 8, NC = 256;                    // waves; threads issuing copies
  constexpr int D = DC + DR;
  constexpr int CH = D / 8;                          // 16-byte chunks per cached row
  constexpr int LOADS = KVT * CH / NC;               // copy instructions per copying wave per tile
  constexpr int STAGE = KVT * D;
  constexpr int NS = 4;                              // ring stages (two tiles ahead)
  constexpr int QS = D / 32;
  constexpr int ROWS = 64;
  constexpr int DW = DC / NW, DBW = DW / 16;         // latent columns per wave in P.V
  constexpr int HBS = ROWS / 16;
  constexpr int PF = DECODE_PF;
  constexpr int PVS = HBS - 1;                       // P.V row blocks interleaved with the scores
  constexpr float TAU = 32.0f, MREF0 = -1e30f;
  static_assert(KVT * CH % NC == 0 && DBW == 4 && QS > PF && QS >= 2 * PVS && QS >= 2 * LOADS, "");

  __shared__ __attribute__((aligned(16))) bf16 stages[NS * STAGE];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2 * 4 * ROWS];   // P[buf][g][row]
  __shared__ float xch[2][ROWS];                                       // per key half: row max, then row sum
  __shared__ int xov[2][ROWS];                                         // per key half: row overflowed

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int rw = wave & 3, kh = wave >> 2;          // score roles: row block, key half
  int unit, rg;
  if (!decode_item(a, unit, rg)) return;
  const int b = unit / a.n_splits, s = unit % a.n_splits;
  const int len = (int)min((long)a.lens[b], min((long)a.n_splits * a.chunk, a.cache.cap));
  const int kv_beg = s * a.chunk;
  if (kv_beg >= len) return;
  const int kv_end = min(len, kv_beg + a.chunk);
  const int R = a.n_q * a.n_h;
  const int rbase = rg * ROWS;
  const float sl2 = a.scale_log2;
  const bf16 *pool = (const bf16 *)a.cache.pool;
  const long seq_row0 = (long)b * a.cache.max_len;
  const unsigned lds_stages = (unsigned)(size_t)(lds_void *)stages;
  const int ntiles = (kv_end - kv_beg + KVT - 1) / KVT;

  static_assert(NC / CH == 3 && NC % CH == 40, "");
  const int r0 = tid / CH, c0 = tid - (tid / CH) * CH;
  auto tile_src = [&](int t) {
    const int kvb = kv_beg + t * KVT;
    long trow;
    if constexpr (PAGED) {
      const int q = block_of(a.cache, kvb);
      const int blk = __builtin_amdgcn_readfirstlane(a.cache.table[(long)b * a.cache.max_blocks + q]);
      trow = (long)blk * a.cache.block_size + (kvb - q * a.cache.block_size);
    } else {
      trow = seq_row0 + kvb;
    }
    return (const char *)(pool + trow * D);
  };
  // copies of rows r_off..r_off+31 of src (rows past `last` repeat it) into
  // stage st (waves 0..3 only: a wave-uniform branch)
  auto copy_rows = [&](const char *src, int r_off, int last, int st) {
    if (wave >= NC / 64) return;
    int cr = r0, cc = c0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = min(r_off + cr, last);
      const unsigned dst = lds_stages + (unsigned)(st * STAGE * 2) + i * NC * 16 + wave * 1024;
      dma16(src, (unsigned)(r * D + ((cc ^ (r & 7)) << 3)) * 2u, dst);
      cc += NC % CH;
      const bool wrap = cc >= CH;
      cc -= wrap ? CH : 0;
      cr += NC / CH + (wrap ? 1 : 0);
    }
  };
  auto copy_tile = [&](int t) { copy_rows(tile_src(t), 0, min(KVT, kv_end - (kv_beg + t * KVT)) - 1, t % NS); };

  // the workgroup's 64 query rows reach LDS through stages 2 and 3 (whole
  // rows per copy instruction; rows past the last query row repeat it) while
  // tiles 0 and 1 are copied into stages 0 and 1
  {
    const char *qsrc = (const char *)((const bf16 *)a.q + ((long)b * R + rbase) * D);
    copy_rows(qsrc, 0, R - 1 - rbase, 2);
    copy_rows(qsrc, KVT, R - 1 - rbase, 3);
  }
  for (int t = 0; t < 2 && t < ntiles; ++t) copy_tile(t);
  // this wave's query copies (the tiles may still be in flight)
  if (ntiles >= 2) wait_vmcnt<2 * LOADS>();
  else wait_vmcnt<LOADS>();
  bar();
  // score state: the queries of rows rbase + 16*rw.. (B operand), read with
  // the tiles' chunk swizzle; stage 2 is next written by the copy of tile 2,
  // after the barrier of sync(0), which follows these reads (lgkm wait)
  bf16x8 qf[QS];
  const int qr = min(rbase + rw * 16 + lrow, R - 1);
  {
    const int rr = (rw * 16 + lrow) & (KVT - 1);
    const lds_bf16 *qs = (const lds_bf16 *)stages + (2 + (rw >> 1)) * STAGE + rr * D;
#pragma unroll
    for (int q = 0; q < QS; ++q) qf[q] = *(const lds_bf16x8 *)(qs + (((4 * q + lgrp) ^ (rr & 7)) << 3));
  }
  const int limit = min(len - a.n_q + qr / a.n_h, kv_end - 1);
  float mref = MREF0, lrun = 0.f;
  bool ovf = false;

  // P.V state: O^T for latent columns wave*DW.. and all ROWS rows
  f32x4 oacc[DBW][HBS];
#pragma unroll
  for (int i = 0; i < DBW; ++i)
#pragma unroll
    for (int j = 0; j < HBS; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};


  // score reads: the kernel above's addressing, in this wave's half of the tile
  const int fq = (lrow >> 2) & 1, gq = lgrp ^ (lrow & 3);
  const int a_even = (kh * 16 + lrow) * D + (4 * fq + gq) * 8;
  const int a_odd = (kh * 16 + lrow) * D + (gq - 4 * fq) * 8;
  // transposed reads of the wave's 64 columns (8 chunks): row r = 4*lgrp +
  // (lrow >> 2) (and r + 16), physical chunk wave*8 + 2*(db ^ fh) + cl
  int t_base, t_fh;
  {
    const int r = 4 * lgrp + (lrow >> 2), fr = r & 7;
    const int cl = ((lrow & 3) >> 1) ^ (fr & 1), half = (lrow & 1) * 4;
    t_base = r * D + (wave * 8 + cl) * 8 + half;
    t_fh = fr >> 1;
  }
  constexpr int TRH = 16 * D;
  const lds_bf16 *st_base = (const lds_bf16 *)stages;
  lds_bf16x8 *pl = (lds_bf16x8 *)pbuf;

  bf16x8 va[DBW];
  auto load_v = [&](int u) {
    const lds_bf16 *st = st_base + (u % NS) * STAGE;
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      const int o = t_base + 16 * (db ^ t_fh);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + o));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + o + TRH));
      va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto pv_block = [&](int u, int hb) {
    const bf16x8 pb = pl[((u & 1) * 4 + lgrp) * ROWS + hb * 16 + lrow];
#pragma unroll
    for (int db = 0; db < DBW; ++db) oacc[db][hb] = Mma<bf16>::mma(va[db], pb, oacc[db][hb]);
  };

  // Scores and softmax of tile t (stage t % NS) into P buffer t & 1, with the
  // P.V of tile t-1 interleaved when WITH_PV; two accumulators (even and odd
  // k steps) halve the dependent MFMA chain.
  auto scores = [&](int t, auto with_pv_c) {
    constexpr bool WITH_PV = decltype(with_pv_c)::value;
    const lds_bf16 *ca_p = st_base + (t % NS) * STAGE;
    const int kvb = kv_beg + t * KVT;
    if (t + 2 < ntiles) copy_tile(t + 2);
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    auto rd = [&](int q) { return *(const lds_bf16x8 *)(ca_p + ((q & 1) ? a_odd : a_even) + q * 32); };
    bf16x8 ca[PF + 1];
#pragma unroll
    for (int q = 0; q < PF; ++q) ca[q] = rd(q);
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      if (q + PF < QS) ca[(q + PF) % (PF + 1)] = rd(q + PF);
      sacc[q & 1] = Mma<bf16>::mma(ca[q % (PF + 1)], qf[q], sacc[q & 1]);
      if constexpr (WITH_PV) {
        if (q % 2 == 1 && q / 2 < PVS) pv_block(t - 1, q / 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kv = kvb + 16 * kh + 4 * lgrp + i;
      const float x = (sacc[0][i] + sacc[1][i]) * sl2;
      sv[i] = (kv <= limit) ? x : -INFINITY;
      mt = fmaxf(mt, sv[i]);
    }
    // the first tile fixes the reference of each row: the max over both key
    // halves; later tiles only check, per lane, that they stay within TAU
    if (t == 0) {
      const float m16 = row_max(mt);
      if (lgrp == 0) xch[kh][rw * 16 + lrow] = m16;
      wait_lgkm0();
      bar();
      mref = fmaxf(fmaxf(xch[0][rw * 16 + lrow], xch[1][rw * 16 + lrow]), MREF0);
    } else {
      ovf |= mt > mref + TAU;
    }
    bf16x4 pf;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = __builtin_amdgcn_exp2f(sv[j] - mref);
      psum += p;
      pf[j] = (bf16)p;
    }
    lrun += psum;
    *(lds_bf16x4 *)((lds_bf16 *)(pl + ((t & 1) * 4 + lgrp) * ROWS + rw * 16 + lrow) + kh * 4) = pf;
    if constexpr (WITH_PV) pv_block(t - 1, PVS);
  };

  auto sync = [&](int i) {
    if (i + 1 < ntiles) wait_vmcnt<LOADS>();   // this wave's copies of tile i (none for waves 4..7)
    else wait_vmcnt<0>();
    wait_lgkm0();
    bar();
  };
  sync(0);
  scores(0, std::false_type());
  for (int i = 1; i < ntiles; ++i) {
    sync(i);
    load_v(i - 1);
    scores(i, std::true_type());
  }
  sync(ntiles);
  load_v(ntiles - 1);
#pragma unroll
  for (int hb = 0; hb < HBS; ++hb) pv_block(ntiles - 1, hb);

  // row sums and overflow marks of the two key halves meet in LDS
  {
    float l = lrun;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const bool rov = row_max(ovf ? 1.f : 0.f) > 0.f;   // any lane of the row
    if (lgrp == 0) {
      xch[kh][rw * 16 + lrow] = l;
      xov[kh][rw * 16 + lrow] = rov ? 1 : 0;
    }
  }
  __syncthreads();   // P no longer read: its space holds 1/l per row
  float *fac = (float *)pbuf;
  if (kh == 0 && lgrp == 0) {
    const int rl = rw * 16 + lrow;
    const float l = xch[0][rl] + xch[1][rl];
    const bool ov = (xov[0][rl] | xov[1][rl]) != 0;
    fac[rl] = l > 0.f ? 1.f / l : 0.f;
    if (rbase + rl < R)
      a.lse_part[((long)b * a.n_splits + s) * R + rbase + rl] =
          ov ? __builtin_nanf("") : l > 0.f ? mref + log2f(l) : -INFINITY;
  }
  __syncthreads();
  // normalised rows through the idle stages, then one whole row per store
  static_assert(ROWS * DC <= NS * STAGE && DC / 8 == 64, "");
  lds_bf16 *ot = (lds_bf16 *)stages;
#pragma unroll
  for (int hb = 0; hb < HBS; ++hb) {
    const int rl = hb * 16 + lrow;
    const float inv = fac[rl];
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      const f32x4 o4 = oacc[db][hb] * inv;
      const int c = (wave * 8 + db * 2 + (lgrp >> 1)) ^ lrow;
      *(lds_bf16x4 *)(ot + rl * DC + c * 8 + (lgrp & 1) * 4) =
          bf16x4{(bf16)o4[0], (bf16)o4[1], (bf16)o4[2], (bf16)o4[3]};
    }
  }
  __syncthreads();
  bf16 *op = (bf16 *)a.o_part + (((long)b * a.n_splits + s) * R + rbase) * DC + lane * 8;
  // streaming stores: the partials are read once, by the combine, from
  // other XCDs (47.1 -> 45.2 us against write-allocating stores)
  for (int rl = wave; rl < ROWS && rbase + rl < R; rl += NW)
    __builtin_nontemporal_store(*(const lds_bf16x8 *)(ot + rl * DC + (lane ^ (rl & 15)) * 8),
                                (bf16x8 *)(op + (long)rl * DC));
}

// Exact attention of one query row over its whole sequence, straight from the
// cache, for rows an attention kernel flagged (lse = NaN): two passes, the
// first for the max, the second for the sum and the weighted latent rows.
// res[i] receives latent column col(i): lane + 64*i, or lane*PER + i when
// CHUNKED (the lane's PER consecutive columns).
template <typename T, int DC, int DR, bool CHUNKED>
__device__ void decode_row_exact(const DecodeArgs &a, int b, int r, int len, float (&res)[(DC + 63) / 64]) {
  constexpr int D = DC + DR, PER = (DC + 63) / 64, QP = (D + 63) / 64;
  static_assert(!CHUNKED || DC == 64 * PER, "");
  const int lane = threadIdx.x & 63;
  const int R = a.n_q * a.n_h;
  const T *qrow = (const T *)a.q + ((long)b * R + r) * D;
  float qv[QP];
#pragma unroll
  for (int i = 0; i < QP; ++i) qv[i] = (lane + 64 * i < D) ? to_f32(qrow[lane + 64 * i]) : 0.f;
  const int limit = min(len - a.n_q + r / a.n_h, len - 1);
  auto score = [&](const T *crow) {
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < QP; ++i)
      if (lane + 64 * i < D) dot += qv[i] * to_f32(crow[lane + 64 * i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
    return dot * a.scale_log2;
  };
  float m = -INFINITY;
  for (int kv = 0; kv <= limit; ++kv) m = fmaxf(m, score((const T *)a.cache.pool + cache_row(a.cache, b, kv) * D));
  float l = 0.f, acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int kv = 0; kv <= limit; ++kv) {
    const T *crow = (const T *)a.cache.pool + cache_row(a.cache, b, kv) * D;
    const float p = exp2f(score(crow) - m);
    l += p;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = CHUNKED ? lane * PER + i : lane + 64 * i;
      if (c < DC) acc[i] += p * to_f32(crow[c]);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) res[i] = acc[i] * inv;
}

template <typename T, int N>
struct alignas(N * sizeof(T)) Pack { T x[N]; };

// One wave per query row: merge the splits of its sequence.
template <typename T, int DC, int DR>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  static_assert(DC % 64 == 0, "");
  constexpr int PER = DC / 64;
  const int lane = threadIdx.x & 63;
  const int R = a.n_q * a.n_h;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)a.B * R) return;
  const int b = (int)(row / R), r = (int)(row % R);
  const int len = (int)min((long)a.lens[b], min((long)a.n_splits * a.chunk, a.cache.cap));
  const int nsp = len > 0 ? min(a.n_splits, (len + a.chunk - 1) / a.chunk) : 0;
  const long base = (long)b * a.n_splits * R + r;
  T *out = (T *)a.o_lat + row * DC;
  // split weights: lane s holds split s (for up to 64 splits; more are
  // read in rounds)
  float lmax = -INFINITY;
  bool flagged = false;
  for (int s0 = 0; s0 < nsp; s0 += 64) {
    const float ls = s0 + lane < nsp ? a.lse_part[base + (long)(s0 + lane) * R] : -INFINITY;
    flagged |= ls != ls;
    lmax = fmaxf(lmax, ls);
  }
  if (__any(flagged)) {
    float res[PER];
    decode_row_exact<T, DC, DR, false>(a, b, r, len, res);
#pragma unroll
    for (int i = 0; i < PER; ++i) out[lane + 64 * i] = from_f32<T>(res[i]);
    return;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
  // lane owns PER consecutive latent columns (one 16-byte load per split for
  // bf16 and d_c = 512); loads of 8 splits are issued together
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  constexpr int SB = 8;
  for (int s0 = 0; s0 < nsp; s0 += SB) {
    Pack<T, PER> v[SB];
    float w[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const int s = min(s0 + j, nsp - 1);
      v[j] = *(const Pack<T, PER> *)((const T *)a.o_part + (base + (long)s * R) * DC + lane * PER);
      const float ls = a.lse_part[base + (long)s * R];
      w[j] = (s0 + j >= nsp || ls == -INFINITY) ? 0.f : exp2f(ls - lmax);
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      wsum += w[j];
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += w[j] * to_f32(v[j].x[i]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  Pack<T, PER> o;
#pragma unroll
  for (int i = 0; i < PER; ++i) o.x[i] = from_f32<T>(acc[i] * inv);
  *(Pack<T, PER> *)(out + lane * PER) = o;
}

// Split combine fused with the value un-absorption o_t,i = W_UV,i o_lat,t,i
// (W_UV applied after the attention, by the associativity of the products in
// section 2.1 of the DeepSeek-V3 paper-reading notes), bf16, d_c = 512.  One
// workgroup = (head i, 16 tokens): its four waves merge the splits of the 16
// latent rows (a wave per four tokens, a lane per eight columns) into LDS,
// rounded to bf16 as a stored o_lat would be, while W_UV,i (128 KB) streams
// into registers; then O^T[v][t] = W_UV,i[v][:] . o_lat[t][:] on the matrix
// cores, wave w taking features (DV/4)w...  The token groups of a head share
// an XCD, whose L2 serves their common reads of W_UV,i.  Rows marked for
// exact recomputation take the two-pass path of the combine kernel.
template <int DC, int DR, int DV>
__global__ __launch_bounds__(256, 1) void decode_combine_uv_kernel(DecodeArgs a, const bf16 *w_uv, bf16 *o) {
  constexpr int TT = 16, NW = 4;         // tokens per workgroup, waves
  constexpr int KS = DC / 32;            // k steps
  constexpr int VB = DV / (16 * NW);     // 16-feature blocks per wave
  constexpr int PER = DC / 64;           // latent columns per lane in the merge
  constexpr int SB = 4;                  // splits per token requested up front
  static_assert(DC == 512 && PER == 8 && VB >= 1 && DV % (16 * NW) == 0, "");
  // token row tl of the group: 16-byte chunk c at chunk c ^ (tl & 15)
  __shared__ __attribute__((aligned(16))) bf16 olat[TT * DC];
  // W_UV,i [DV][DC]: chunk c of row v at chunk c ^ (v & 15)
  __shared__ __attribute__((aligned(16))) bf16 wuv[DV * DC];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int T = a.B * a.n_q, R = a.n_q * a.n_h;
  const int ntg = (T + TT - 1) / TT;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int h = (slot / ntg) * 8 + xcd, tg = slot % ntg;
  if (h >= a.n_h) return;

  // W_UV,i -> LDS, whole rows per copy instruction (the merge's loads below
  // return after these: the counter is in order)
  {
    constexpr int WLOADS = DV * DC / 8 / 256;
    const unsigned lw = (unsigned)(size_t)(lds_void *)wuv;
    const bf16 *wh = w_uv + (long)h * DV * DC;
#pragma unroll
    for (int j = 0; j < WLOADS; ++j) {
      const int sl = j * 256 + threadIdx.x, v = sl / (DC / 8), pc = sl % (DC / 8);
      const int c = pc ^ (v & 15);
      dma16(wh, (unsigned)((v * DC + c * 8) * 2), lw + (unsigned)(j * 256 + wave * 64) * 16);
    }
  }

  // merge: wave w takes tokens 4w..4w+3 of the group.  The log-sum-exps
  // (lane s: split s) and the first SB partial rows of all four tokens are
  // requested before any of them is used, so the merge costs one round trip
  // (more splits than SB, or than 64, take extra rounds).
  constexpr int TW = TT / NW;
  int bq[TW], rq[TW], lq[TW], nsp[TW];
  long base[TW];
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int t = tg * TT + wave * TW + j;
    bq[j] = 0; rq[j] = 0; lq[j] = 0; nsp[j] = 0; base[j] = 0;
    if (t < T) {
      bq[j] = t / a.n_q;
      rq[j] = (t % a.n_q) * a.n_h + h;
      lq[j] = (int)min((long)a.lens[bq[j]], min((long)a.n_splits * a.chunk, a.cache.cap));
      nsp[j] = lq[j] > 0 ? min(a.n_splits, (lq[j] + a.chunk - 1) / a.chunk) : 0;
      base[j] = (long)bq[j] * a.n_splits * R + rq[j];
    }
  }
  // addresses from the plan only (not from the lengths), so these loads do
  // not wait for the length loads; splits past a sequence's end are masked
  float ls[TW];
  bf16x8 v[TW][SB];
  const int lsp = min(lane, a.n_splits - 1);
#pragma unroll
  for (int j = 0; j < TW; ++j) ls[j] = a.lse_part[base[j] + (long)lsp * R];
#pragma unroll
  for (int j = 0; j < TW; ++j)
#pragma unroll
    for (int jj = 0; jj < SB; ++jj) {
      const int sp = min(jj, a.n_splits - 1);
      v[j][jj] = *(const bf16x8 *)((const bf16 *)a.o_part + (base[j] + (long)sp * R) * DC + lane * PER);
    }
#pragma unroll
  for (int j = 0; j < TW; ++j) ls[j] = lane < nsp[j] ? ls[j] : -INFINITY;
  lds_bf16 *ol = (lds_bf16 *)olat;
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int tl = wave * TW + j;
    float res[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) res[i] = 0.f;
    if (nsp[j] > 0) {
      float lmax = ls[j];
      bool flagged = ls[j] != ls[j];
      for (int s0 = 64; s0 < nsp[j]; s0 += 64) {
        const float x = s0 + lane < nsp[j] ? a.lse_part[base[j] + (long)(s0 + lane) * R] : -INFINITY;
        flagged |= x != x;
        lmax = fmaxf(lmax, x);
      }
      if (__any(flagged)) {
        decode_row_exact<bf16, DC, DR, true>(a, bq[j], rq[j], lq[j], res);
      } else {
#pragma unroll
        for (int o2 = 32; o2 > 0; o2 >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o2));
        float wsum = 0.f;
#pragma unroll
        for (int jj = 0; jj < SB; ++jj) {
          const float lsj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[j]), jj));
          const float w = (jj < nsp[j] && lsj != -INFINITY) ? exp2f(lsj - lmax) : 0.f;
          wsum += w;
#pragma unroll
          for (int i = 0; i < PER; ++i) res[i] += w * (float)v[j][jj][i];
        }
        for (int sp = SB; sp < nsp[j]; ++sp) {
          const float lsj = a.lse_part[base[j] + (long)sp * R];
          const bf16x8 vv = *(const bf16x8 *)((const bf16 *)a.o_part + (base[j] + (long)sp * R) * DC + lane * PER);
          const float w = lsj != -INFINITY ? exp2f(lsj - lmax) : 0.f;
          wsum += w;
#pragma unroll
          for (int i = 0; i < PER; ++i) res[i] += w * (float)vv[i];
        }
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) res[i] *= inv;
      }
    }
    bf16x8 pk;
#pragma unroll
    for (int i = 0; i < PER; ++i) pk[i] = (bf16)res[i];
    *(lds_bf16x8 *)(ol + tl * DC + (lane ^ (tl & 15)) * 8) = pk;
  }
  wait_vmcnt<0>();   // this wave's W_UV copies
  __syncthreads();

  // A operand: W_UV,i row (wave*VB + vb)*16 + lrow, k = 32*ks + 8*lgrp..
  const lds_bf16 *wl = (const lds_bf16 *)wuv;
  f32x4 acc[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) acc[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 xb = *(const lds_bf16x8 *)(ol + lrow * DC + (((4 * ks + lgrp) ^ lrow) * 8));
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const bf16x8 wf = *(const lds_bf16x8 *)(wl + ((wave * VB + vb) * 16 + lrow) * DC + (((4 * ks + lgrp) ^ lrow) * 8));
      acc[vb] = Mma<bf16>::mma(wf, xb, acc[vb]);
    }
  }
  // lane: features (wave*VB + vb)*16 + 4*lgrp + 0..3 of token lrow
  const int t = tg * TT + lrow;
  if (t < T) {
    bf16 *orow = o + ((long)t * a.n_h + h) * DV + wave * VB * 16 + 4 * lgrp;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
      *(bf16x4 *)(orow + vb * 16) = bf16x4{(bf16)acc[vb][0], (bf16)acc[vb][1], (bf16)acc[vb][2], (bf16)acc[vb][3]};
  }
}

hipError_t launch_decode_combine_uv(const DecodeArgs &a, int d_v, const void *w_uv, void *o, hipStream_t st) {
  if (a.d_c != 512 || a.d_rope != 64 || d_v != 128) return hipErrorNotSupported;
  const int T = a.B * a.n_q;
  const int grid = ((a.n_h + 7) / 8) * 8 * ((T + 15) / 16);
  timing_before("decode_combine_uv", st);
  hipLaunchKernelGGL((decode_combine_uv_kernel<512, 64, 128>), dim3(grid), dim3(256), 0, st, a,
                     (const bf16 *)w_uv, (bf16 *)o);
  timing_after("decode_combine_uv", st);
  return hipGetLastError();
}

int decode_kv_tile(int) { return KVT; }
// Query rows per workgroup.  bf16 takes 128 (a quarter per wave), or 64 when
// every sequence still gets at least four splits from one wave of workgroups
// over the CUs: halving the partial results written per split, and the
// combine's reads of them, then outweighs the second read of each cache tile
// (an L2 hit) by the other row group.
int decode_rows_per_group(int dtype, long B, long R, int cus) {
  if (dtype != 1) return 64;
  return (R <= 64 || (R <= 128 && B * 2 * 4 <= cus)) ? 64 : 128;
}

template <typename T, int NW, int HB, int DC, int DR>
static hipError_t launch_attn(const DecodeArgs &a, hipStream_t st) {
  const int grid = decode_grid(a);
  timing_before("decode_attn", st);
  hipLaunchKernelGGL((decode_attn_kernel<T, NW, HB, DC, DR>), dim3(grid), dim3(64 * NW), 0, st, a);
  timing_after("decode_attn", st);
  return hipGetLastError();
}

hipError_t launch_decode_attn(int dtype, const DecodeArgs &a, hipStream_t st) {
  const bool tile_in_block = !a.cache.table || (a.cache.block_size % KVT == 0);
  if (dtype == 1 && a.d_c == 512 && a.d_rope == 64 && tile_in_block) {
    const int grid = decode_grid(a);
    timing_before("decode_attn", st);
    if (a.rows == 64) {
      if (a.cache.table)
        hipLaunchKernelGGL((decode_attn_dma8_kernel<512, 64, true>), dim3(grid), dim3(512), 0, st, a);
      else
        hipLaunchKernelGGL((decode_attn_dma8_kernel<512, 64, false>), dim3(grid), dim3(512), 0, st, a);
    } else {
      if (a.cache.table)
        hipLaunchKernelGGL((decode_attn_dma_kernel<512, 64, true, 128>), dim3(grid), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((decode_attn_dma_kernel<512, 64, false, 128>), dim3(grid), dim3(256), 0, st, a);
    }
    timing_after("decode_attn", st);
    return hipGetLastError();
  }
  if (dtype == 1 && a.d_c == 512 && a.d_rope == 64)
    return a.rows == 64 ? launch_attn<bf16, 4, 1, 512, 64>(a, st) : launch_attn<bf16, 8, 1, 512, 64>(a, st);
  if (dtype == 0 && a.d_c == 64 && a.d_rope == 16) return launch_attn<float, 4, 1, 64, 16>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(int dtype, const DecodeArgs &a, hipStream_t st) {
  const long rows = (long)a.B * a.n_q * a.n_h;
  dim3 grid((unsigned)((rows + 3) / 4));
  timing_before("decode_combine", st);
  if (dtype == 1 && a.d_c == 512 && a.d_rope == 64)
    hipLaunchKernelGGL((decode_combine_kernel<bf16, 512, 64>), grid, dim3(256), 0, st, a);
  else if (dtype == 0 && a.d_c == 64 && a.d_rope == 16)
    hipLaunchKernelGGL((decode_combine_kernel<float, 64, 16>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  timing_after("decode_combine", st);
  return hipGetLastError();
}

}  // namespace mla
