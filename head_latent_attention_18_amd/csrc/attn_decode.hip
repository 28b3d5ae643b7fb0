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

  // block -> (unit = (b, s), row group); the row groups of one unit share an XCD
  const int units = a.B * a.n_splits;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int rg = slot % a.row_groups;
  const int unit = (slot / a.row_groups) * 8 + xcd;
  if (unit >= units) return;
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
      float *op = a.o_part + pbase * DC;
#pragma unroll
      for (int db = 0; db < DB; ++db) *(f32x4 *)(op + db * 16 + 4 * lgrp) = oacc[db][hb] * inv;
      if (lgrp == 0) a.lse_part[pbase] = l > 0.f ? mrun[hb] + log2f(l) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel for gfx950.  The cache tile goes HBM -> LDS with
// global_load_lds_dwordx4 (lane i's 16 bytes land at base + 16*i; no staging
// registers) into a ring of stages, one barrier per tile.  Both contractions
// read the one row-major copy: the scores with 16-byte row reads, P.V with
// ds_read_b64_tr_b16, which hands lane i column i of the 4x16 block of 16-bit
// elements that its 16-lane group addresses (row j>>2, columns 4*(j&3)..+3
// from lane j).  The running max is only moved when a tile's max exceeds it
// by more than 8 (log2 units), so the O rescale is rare; the result is the
// same softmax since numerator and denominator share the reference.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
constexpr int DECODE_TBL = 256;   // block-table entries a split may span (staged in LDS)
#ifndef DECODE_NW
#define DECODE_NW 8               // waves per workgroup; each owns 128/NW query rows
#endif
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

template <int DC, int DR, bool PAGED, int NW, int HB>
__global__ __launch_bounds__(64 * NW, 1) void decode_attn_dma_kernel(DecodeArgs a) {
  constexpr int D = DC + DR, NT = 64 * NW;
  constexpr int CH = D / 8;                          // 16-byte chunks per cached row
  constexpr int PITCH = CH + 1;                      // LDS row pitch in chunks (one pad chunk)
  constexpr int LDC = PITCH * 8;                     // ... in elements
  constexpr int LOADS = (KVT * PITCH + NT - 1) / NT; // DMA instructions per wave per tile
  constexpr int STAGE = LOADS * NT * 8;              // elements per stage, including the tail slots
  constexpr int RUN = D / 4, QS = RUN / 8, DB = DC / 16;
  constexpr int ROWS = 16 * NW * HB;
  constexpr float TAU = 8.0f;
  static_assert(D % 32 == 0 && DC % 16 == 0, "");

  // Three stages in three separate LDS objects: reads of one stage are then
  // provably disjoint from the copies in flight into the others, so the
  // compiler adds no wait for those copies before the reads.
  __shared__ __attribute__((aligned(16))) bf16 stage0[STAGE];
  __shared__ __attribute__((aligned(16))) bf16 stage1[STAGE];
  __shared__ __attribute__((aligned(16))) bf16 stage2[STAGE];
  __shared__ int tbl[PAGED ? DECODE_TBL : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int units = a.B * a.n_splits;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int rg = slot % a.row_groups;
  const int unit = (slot / a.row_groups) * 8 + xcd;
  if (unit >= units) return;
  const int b = unit / a.n_splits, s = unit % a.n_splits;
  const int len = (int)min((long)a.lens[b], min((long)a.n_splits * a.chunk, a.cache.cap));
  const int kv_beg = s * a.chunk;
  if (kv_beg >= len) return;
  const int kv_end = min(len, kv_beg + a.chunk);
  const int R = a.n_q * a.n_h;
  const int row0 = rg * ROWS + wave * 16 * HB;
  const float sl2 = a.scale_log2;
  const bf16 *pool = (const bf16 *)a.cache.pool;

  // block-table slice of this split (the host keeps it within DECODE_TBL entries)
  int blk0 = 0;
  bool tbl_ok = false;
  if constexpr (PAGED) {
    blk0 = block_of(a.cache, kv_beg);
    const int nblk = block_of(a.cache, kv_end - 1) - blk0 + 1;
    tbl_ok = nblk <= DECODE_TBL;
    if (tbl_ok)
      for (int i = tid; i < nblk; i += NT) tbl[i] = a.cache.table[(long)b * a.cache.max_blocks + blk0 + i];
    __syncthreads();
  }
  const long seq_row0 = (long)b * a.cache.max_len;

  // DMA of tile t into stage st: every wave issues exactly LOADS instructions;
  // the tail and pad slots fetch a valid chunk into slots nobody reads.  A
  // tile lies inside one cache block (block_size is a multiple of the tile),
  // so its rows are contiguous: a uniform base plus 32-bit lane offsets.
  auto issue = [&](int t, auto st) {
    const int kvb = kv_beg + t * KVT;
    const int last = min(KVT, kv_end - kvb) - 1;
    long trow;
    if constexpr (PAGED) {
      const int q = block_of(a.cache, kvb);
      const int blk = __builtin_amdgcn_readfirstlane(tbl_ok ? tbl[q - blk0]
                                                            : a.cache.table[(long)b * a.cache.max_blocks + q]);
      trow = (long)blk * a.cache.block_size + (kvb - q * a.cache.block_size);
    } else {
      trow = seq_row0 + kvb;
    }
    const char *tbase = (const char *)(pool + trow * D);
    bf16 *sbase = (st.value == 0 ? stage0 : st.value == 1 ? stage1 : stage2) + wave * 64 * 8;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int sl = i * NT + tid;
      const int r = sl / PITCH;
      const int row = min(r, last), ch = min(sl - r * PITCH, CH - 1);
      const unsigned off = (unsigned)(row * D + ch * 8) * 2u;
      __builtin_amdgcn_global_load_lds((const void *)(tbase + off), (lds_void *)(sbase + i * NT * 8), 16, 0, 0);
    }
  };

  bf16x8 qf[HB][QS];
  int limit[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int r = min(row0 + hb * 16 + lrow, R - 1);
    const bf16 *qrow = (const bf16 *)a.q + ((long)b * R + r) * D + lgrp * RUN;
#pragma unroll
    for (int q = 0; q < QS; ++q) qf[hb][q] = *(const bf16x8 *)(qrow + q * 8);
    limit[hb] = min(len - a.n_q + r / a.n_h, kv_end - 1);
  }
  f32x4 oacc[DB][HB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < HB; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref[HB], lrun[HB];
#pragma unroll
  for (int j = 0; j < HB; ++j) { mref[j] = -1e30f; lrun[j] = 0.f; }

  const int ntiles = (kv_end - kv_beg + KVT - 1) / KVT;
  issue(0, std::integral_constant<int, 0>());
  if (ntiles > 1) issue(1, std::integral_constant<int, 1>());
  // Scores use the tile rows in natural order (A slot = row, conflict-free
  // 16-byte reads): lane group g then holds rows 4g..4g+3 and 16+4g..16+4g+3.
  // The transposed reads of P.V fetch exactly those rows (any four rows can
  // form the 4x16 block), so the probabilities stay in registers.
  const int a_off = lrow * LDC + lgrp * RUN;
  const int t_off = (4 * lgrp + (lrow >> 2)) * LDC + 4 * (lrow & 3);

  // one tile; CUR is the stage holding it (compile-time, see above)
  auto step = [&](int t, auto cur_c) {
    constexpr int CUR = decltype(cur_c)::value;
    if (t + 1 < ntiles) wait_vmcnt<LOADS>();   // tile t+1 may stay in flight
    else wait_vmcnt<0>();
    // Workgroup barrier without the release/acquire fences of __syncthreads:
    // this wave's copies of tile t are complete (wait above), and its reads of
    // the stage about to be refilled were consumed by MFMAs before this point.
    // The empty asm statements keep the compiler from moving LDS accesses
    // across the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 2 < ntiles) issue(t + 2, std::integral_constant<int, (CUR + 2) % 3>());
    const lds_bf16 *cur = (const lds_bf16 *)(CUR == 0 ? stage0 : CUR == 1 ? stage1 : stage2);
    const lds_bf16 *ca_p = cur + a_off;
    lds_v4i16 *tr_p = (lds_v4i16 *)(cur + t_off);
    const int kvb = kv_beg + t * KVT;

    // S^T = C . Q^T; the A fragments of step q+1 are read while step q multiplies
    f32x4 sacc[2][HB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) sacc[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 ca[2][2];
    ca[0][0] = *(const lds_bf16x8 *)(ca_p);
    ca[0][1] = *(const lds_bf16x8 *)(ca_p + 16 * LDC);
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      if (q + 1 < QS) {
        ca[(q + 1) & 1][0] = *(const lds_bf16x8 *)(ca_p + (q + 1) * 8);
        ca[(q + 1) & 1][1] = *(const lds_bf16x8 *)(ca_p + 16 * LDC + (q + 1) * 8);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) sacc[kb][hb] = Mma<bf16>::mma(ca[q & 1][kb], qf[hb][q], sacc[kb][hb]);
      __builtin_amdgcn_sched_barrier(0);
    }

    bf16x8 pf[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float sv[2][4];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kv = kvb + 16 * kb + 4 * lgrp + i;
          const float x = sacc[kb][hb][i] * sl2;
          sv[kb][i] = (kv <= limit[hb]) ? x : -INFINITY;
          mt = fmaxf(mt, sv[kb][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (__any(mt > mref[hb] + TAU)) {
        const float mnew = fmaxf(mref[hb], mt);
        const float alpha = exp2f(mref[hb] - mnew);
        mref[hb] = mnew;
        lrun[hb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][hb] *= alpha;
      }
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = exp2f(sv[j >> 2][j & 3] - mref[hb]);
        psum += p;
        pf[hb][j] = (bf16)p;
      }
      lrun[hb] += psum;
    }

    // O^T[d][row] += C_lat^T[d][kv] . P^T[kv][row]; C_lat^T is read transposed
    // out of the row tile, one 16-dim block ahead of its MFMAs
    constexpr int TRH = 4 * LDC;   // sixteen rows further, in 4-element units
    v4i16 vt[2][2];
    vt[0][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(tr_p);
    vt[0][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(tr_p + TRH);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db + 1 < DB) {
        vt[(db + 1) & 1][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(tr_p + (db + 1) * 4);
        vt[(db + 1) & 1][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(tr_p + TRH + (db + 1) * 4);
      }
      const bf16x8 va =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(vt[db & 1][0], vt[db & 1][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) oacc[db][hb] = Mma<bf16>::mma(va, pf[hb], oacc[db][hb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int t = 0; t < ntiles; t += 3) {
    step(t, std::integral_constant<int, 0>());
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>());
    if (t + 2 < ntiles) step(t + 2, std::integral_constant<int, 2>());
  }

#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float l = lrun[hb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = row0 + hb * 16 + lrow;
    if (r < R) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const long pbase = ((long)b * a.n_splits + s) * R + r;
      float *op = a.o_part + pbase * DC;
#pragma unroll
      for (int db = 0; db < DB; ++db) *(f32x4 *)(op + db * 16 + 4 * lgrp) = oacc[db][hb] * inv;
      if (lgrp == 0) a.lse_part[pbase] = l > 0.f ? mref[hb] + log2f(l) : -INFINITY;
    }
  }
}

// One wave per query row: merge the splits of its sequence.
template <typename T, int DC>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int PER = (DC + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int R = a.n_q * a.n_h;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)a.B * R) return;
  const int b = (int)(row / R), r = (int)(row % R);
  const int len = (int)min((long)a.lens[b], min((long)a.n_splits * a.chunk, a.cache.cap));
  const int nsp = len > 0 ? min(a.n_splits, (len + a.chunk - 1) / a.chunk) : 0;
  const long base = (long)b * a.n_splits * R + r;
  float lmax = -INFINITY;
  for (int s = 0; s < nsp; ++s) lmax = fmaxf(lmax, a.lse_part[base + (long)s * R]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  for (int s = 0; s < nsp; ++s) {
    const float ls = a.lse_part[base + (long)s * R];
    const float w = (ls == -INFINITY) ? 0.f : exp2f(ls - lmax);
    wsum += w;
    const float *op = a.o_part + (base + (long)s * R) * DC;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + 64 * i;
      if (d < DC) acc[i] += w * op[d];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  T *out = (T *)a.o_lat + row * DC;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = lane + 64 * i;
    if (d < DC) out[d] = from_f32<T>(acc[i] * inv);
  }
}

int decode_kv_tile(int) { return KVT; }
int decode_rows_per_group(int dtype) { return dtype == 1 ? 128 : 64; }

template <typename T, int NW, int HB, int DC, int DR>
static hipError_t launch_attn(const DecodeArgs &a, hipStream_t st) {
  const int units = a.B * a.n_splits;
  const int grid = ((units + 7) / 8) * 8 * a.row_groups;
  timing_before("decode_attn", st);
  hipLaunchKernelGGL((decode_attn_kernel<T, NW, HB, DC, DR>), dim3(grid), dim3(64 * NW), 0, st, a);
  timing_after("decode_attn", st);
  return hipGetLastError();
}

hipError_t launch_decode_attn(int dtype, const DecodeArgs &a, hipStream_t st) {
  const bool tile_in_block = !a.cache.table || (a.cache.block_size % KVT == 0);
  if (dtype == 1 && a.d_c == 512 && a.d_rope == 64 && tile_in_block) {
    const int units = a.B * a.n_splits;
    const int grid = ((units + 7) / 8) * 8 * a.row_groups;
    timing_before("decode_attn", st);
    constexpr int NW = DECODE_NW, HB = 8 / DECODE_NW;
    if (a.cache.table)
      hipLaunchKernelGGL((decode_attn_dma_kernel<512, 64, true, NW, HB>), dim3(grid), dim3(64 * NW), 0, st, a);
    else
      hipLaunchKernelGGL((decode_attn_dma_kernel<512, 64, false, NW, HB>), dim3(grid), dim3(64 * NW), 0, st, a);
    timing_after("decode_attn", st);
    return hipGetLastError();
  }
  if (dtype == 1 && a.d_c == 512 && a.d_rope == 64) return launch_attn<bf16, 8, 1, 512, 64>(a, st);
  if (dtype == 0 && a.d_c == 64 && a.d_rope == 16) return launch_attn<float, 4, 1, 64, 16>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(int dtype, const DecodeArgs &a, hipStream_t st) {
  const long rows = (long)a.B * a.n_q * a.n_h;
  dim3 grid((unsigned)((rows + 3) / 4));
  timing_before("decode_combine", st);
  if (dtype == 1 && a.d_c == 512) hipLaunchKernelGGL((decode_combine_kernel<bf16, 512>), grid, dim3(256), 0, st, a);
  else if (dtype == 0 && a.d_c == 64) hipLaunchKernelGGL((decode_combine_kernel<float, 64>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  timing_after("decode_combine", st);
  return hipGetLastError();
}

}  // namespace mla
