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
// One workgroup = (its share of the batch's cached tiles, group of query
// rows); a query row is a (new token, head) pair.  The bf16 kernel for the
// DeepSeek-V3 widths (decode_attn_ws_kernel) stages tiles in LDS by DMA and
// runs both contractions on the matrix cores; decode_attn_kernel is the
// register-staged form for the other shapes (fp32, block sizes that do not
// hold whole 32-row tiles).  Split results are stored normalised with their
// log2-sum-exp; the combine weights them by exp2(lse_s - max lse).
#include <type_traits>

#include "mla_internal.h"

namespace mla {

constexpr int KVT = 32;  // cache rows per tile (two 16-row MFMA blocks)

// Block -> work item (w, row group), w-major, a contiguous eighth of the
// items per XCD (blocks x, x+8, x+16, .. run on XCD x): the row groups of a
// range of tiles, and the neighbouring ranges (the rest of the same
// sequence), share an XCD, whose L2 serves their common reads (cache tiles,
// queries).
__device__ inline bool decode_item(const DecodeArgs &a, int &w, int &rg) {
  const int n = a.W * a.row_groups, per = (n + 7) / 8;
  const int slot = blockIdx.x >> 3, item = (blockIdx.x & 7) * per + slot;
  if (slot >= per || item >= n) return false;
  w = item / a.row_groups;
  rg = item - w * a.row_groups;
  return true;
}
inline int decode_grid(const DecodeArgs &a) { return 8 * ((a.W * a.row_groups + 7) / 8); }

// ---------------------------------------------------------------------------
// Split plan (DecodeArgs): the cached rows of every sequence, in KVT-row
// tiles, end to end in sequence order; workgroup w of a row group takes
// tiles [w*P, (w+1)*P) with P = ceil(total / W), i.e. the rows are divided
// over the compute units in proportion to each sequence's length.  Every
// wave computes the plan from the lengths with wave-wide scans, so the
// results are wave-uniform and identical in every kernel that needs them.
// ---------------------------------------------------------------------------
// cache rows of sequence b the plan covers: its length, clamped to the cache
__device__ inline int plan_len(const DecodeArgs &a, int b) {
  const int len = a.lens[b];
  // a length outside [n_q, cache capacity] is clamped (and reported in
  // debug builds)
  if (len < a.n_q || len > a.cache.cap) dbg_flag(a.cache, MLA_DBG_LENGTH);
  return (int)max(0L, min((long)len, a.cache.cap));
}
__device__ inline int plan_tiles(int len) { return (len + KVT - 1) / KVT; }

__device__ inline int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ inline int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// total tiles over all sequences, and tiles per workgroup
__device__ inline void plan_totals(const DecodeArgs &a, int &total, int &P) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64)
    sum += b0 + lane < a.B ? plan_tiles(plan_len(a, b0 + lane)) : 0;
  total = __builtin_amdgcn_readfirstlane(wave_sum_i(sum));
  P = (total + a.W - 1) / a.W;
}

struct SeqSpan { int b, t0, tiles, len; };   // sequence, its first tile, its tiles, its rows

// The sequence holding global tile g (g < total), or {B, total, 0, 0}.
__device__ inline SeqSpan plan_locate(const DecodeArgs &a, int g) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const bool in = b0 + lane < a.B;
    const int len = in ? plan_len(a, b0 + lane) : 0, t = plan_tiles(len);
    const int incl = wave_incl_scan(t) + carry;
    const unsigned long long m = __ballot(in && incl > g);
    if (m) {
      const int l = __builtin_ctzll(m);
      const int tl = __shfl(t, l);
      return SeqSpan{b0 + l, __shfl(incl, l) - tl, tl, __shfl(len, l)};
    }
    carry = __shfl(incl, 63);
  }
  return SeqSpan{a.B, carry, 0, 0};
}

// The span of sequence b (0 <= b < B).
__device__ inline SeqSpan plan_seq(const DecodeArgs &a, int b) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int b0 = 0;; b0 += 64) {
    const bool in = b0 + lane < a.B;
    const int len = in ? plan_len(a, b0 + lane) : 0, t = plan_tiles(len);
    const int incl = wave_incl_scan(t) + carry;
    if (b < b0 + 64) {
      const int l = b - b0, tl = __shfl(t, l);
      return SeqSpan{b, __shfl(incl, l) - tl, tl, __shfl(len, l)};
    }
    carry = __shfl(incl, 63);
  }
}

// Partial slots of sequence sp: the first, and how many (workgroups
// sp.t0/P .. (sp.t0 + tiles - 1)/P hold its tiles).
__device__ inline void plan_slots(const SeqSpan &sp, int P, int &slot0, int &n) {
  if (sp.tiles <= 0 || P <= 0) { slot0 = sp.b; n = 0; return; }
  const int w0 = sp.t0 / P, w1 = (sp.t0 + sp.tiles - 1) / P;
  slot0 = w0 + sp.b;
  n = w1 - w0 + 1;
}

// The spans of N sequences bs[] (0 <= bs[j] < B) and the total tiles, in
// one pass over the lengths.
template <int N>
__device__ inline void plan_spans(const DecodeArgs &a, const int (&bs)[N], SeqSpan (&sp)[N], int &total) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < N; ++j) sp[j] = SeqSpan{bs[j], 0, 0, 0};
  int carry = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const bool in = b0 + lane < a.B;
    const int len = in ? plan_len(a, b0 + lane) : 0, t = plan_tiles(len);
    const int incl = wave_incl_scan(t) + carry;
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (bs[j] >= b0 && bs[j] < b0 + 64) {
        const int l = bs[j] - b0, tl = __shfl(t, l);
        sp[j] = SeqSpan{bs[j], __shfl(incl, l) - tl, tl, __shfl(len, l)};
      }
    carry = __shfl(incl, 63);
  }
  total = carry;
}

// Run seg(b, len, kv_beg, kv_end, slot) for each part of a sequence that
// workgroup w holds, in order (kv_beg < kv_end <= len).
template <typename F>
__device__ inline void for_each_segment(const DecodeArgs &a, int w, F &&seg) {
  int total, P;
  plan_totals(a, total, P);
  int g = w * P;
  const int g_end = min(g + P, total);
  while (g < g_end) {
    const SeqSpan sp = plan_locate(a, g);
    if (sp.b >= a.B) break;
    const int end = __builtin_amdgcn_readfirstlane(min(g_end, sp.t0 + sp.tiles));
    const int kv_beg = (g - sp.t0) * KVT, kv_end = min(sp.len, (end - sp.t0) * KVT);
    // wave-uniform values the compiler cannot prove uniform (they come out
    // of cross-lane operations): put them in scalar registers
    if (kv_beg < kv_end)
      seg(__builtin_amdgcn_readfirstlane(sp.b), __builtin_amdgcn_readfirstlane(sp.len),
          __builtin_amdgcn_readfirstlane(kv_beg), __builtin_amdgcn_readfirstlane(kv_end),
          __builtin_amdgcn_readfirstlane(w + sp.b));
    g = end;
  }
}

// Lane and wave indices, formed afresh for each part a workgroup processes:
// the opaque copy of threadIdx.x keeps the compiler from hoisting every
// lane-dependent address out of the loop over parts, which would hold them
// in registers across the whole kernel (and spill).
#define LANE_IDS_PER_PART                                                      \
  int tid = threadIdx.x;                                                       \
  asm volatile("" : "+v"(tid));                                                \
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  \
  const int lrow = lane & 15, lgrp = lane >> 4

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

  int w_item, rg;
  if (!decode_item(a, w_item, rg)) return;
  bool first_seg = true;
  for_each_segment(a, w_item, [&](const int b, const int len, const int kv_beg, const int kv_end, const int slot) {
  if (!first_seg) __syncthreads();   // the previous part's LDS reads are done
  first_seg = false;
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
      const long pbase = (long)slot * R + r;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 o4 = oacc[db][hb] * inv;
        const float v[4] = {o4[0], o4[1], o4[2], o4[3]};
        store4<T>(a.o_part, pbase * DC + db * 16 + 4 * lgrp, v, 0);
      }
      if (lgrp == 0) a.lse_part[pbase] = l > 0.f ? mrun[hb] + log2f(l) : -INFINITY;
    }
  }
  });
}

// ---------------------------------------------------------------------------
// bf16 kernel for gfx950 (d_c = 512, d_R = 64), 64 query rows per
// workgroup.  The cache tile goes HBM -> LDS with global_load_lds_dwordx4
// (lane i's 16 bytes land at base + 16*i; no staging registers) into a ring
// of four stages, three tiles ahead (two with an FP8 cache).  Per tile, two
// phases:
//   A (scores): S^T = C . Q^T against the 32 cached rows of the tile, from
//     16-byte row reads of the stage; the softmax is lane-local (each lane
//     holds the scores of one query row for four cached rows) plus cross-lane
//     swaps.  The bf16 probabilities go to LDS.
//   B (P.V): O^T[d][row] += C_lat^T[d][kv] . P^T[kv][row], with C_lat^T read
//     by ds_read_b64_tr_b16 (lane i of a 16-lane group receives column i of
//     the 4x16 block of 16-bit elements the group addresses) and P^T from LDS.
// The softmax reference of a row is the max of its first tile and never
// moves (no O rescale: numerator and denominator share the reference, so the
// result is the same softmax).  Scores that later rise more than 2^32 above
// it would overflow the probabilities: the workgroup then runs its segment a
// second time, with each row's reference set to the row's maximum over the
// segment, which the first pass tracked (the same MFMA path, at most twice
// the work, and no probability above 1).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
#ifndef DECODE_WS_PF
#define DECODE_WS_PF 6            // score steps of cache fragments read ahead
#endif
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

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

// 64 query rows, 8 waves, and on each SIMD one score wave and one P.V wave
// (waves w and w+4 share SIMD w).  Earlier forms in which every wave did
// both phases (one or two waves per SIMD, each reading every cache fragment
// for one 16-row query block) spent longer per tile: the score reads of each
// tile were four full passes over it.
//   score waves s = 0..3: query rows 32(s>>1)..+31 (two 16-row blocks in
//     registers), cache rows 16(s&1)..+15 of each tile.  Every 16-byte cache
//     fragment read from LDS feeds two MFMAs (one per query block): the
//     scores read each tile from LDS twice in all, not four times.
//   P.V waves p = 0..3 (waves 4..7): latent columns 128p..128p+127 for all
//     64 rows (O^T in 128 registers); they also issue the tile copies.
// In iteration i the score waves process tile i while the P.V waves process
// tile i-1 (its P written in iteration i-1); one barrier per iteration.
// FP8: the cache holds FP8 rows (d_c E4M3 codes | d_R bf16 | d_c/128 fp32
// scales); the P.V waves load each tile into registers and write it to the
// stage already converted to bf16 (codes times their group's scale, a power
// of two, by the hardware's scaled conversion: two codes per instruction,
// exact), so the stage layout, and every read of it, is that of a bf16
// cache.  HBM then carries 656 bytes per cached row
// instead of 1152.
template <int DC, int DR, bool PAGED, bool FP8>
__global__ __launch_bounds__(512, 1) void decode_attn_ws_kernel(DecodeArgs a) {
  constexpr int NC = 256;                            // threads issuing copies (the P.V waves)
  constexpr int D = DC + DR;
  constexpr int CH = D / 8;                          // 16-byte chunks per cached row
  constexpr int LOADS = KVT * CH / NC;               // copy instructions per copying wave per tile
  constexpr int STAGE = KVT * D;
  constexpr int NS = 4;                              // ring stages
  constexpr int QS = D / 32;                         // 32-wide k steps of the scores
  constexpr int ROWS = 64;
  constexpr int DBW = DC / 4 / 16;                   // 16-column blocks per P.V wave
  constexpr int HBS = ROWS / 16;                     // 16-row blocks in P.V
  constexpr int PF = DECODE_WS_PF;                   // score steps read ahead
  constexpr float TAU = 32.0f, MREF0 = -1e30f;
  static_assert(KVT * CH % NC == 0 && DBW == 8 && QS > PF && DC / 8 == 64, "");

  __shared__ __attribute__((aligned(16))) bf16 stages[NS * STAGE];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2 * 4 * ROWS];   // P[buf][g][row]
  __shared__ float xch[2][ROWS];                                       // per key half: row max, then row sum
  __shared__ int xov[2][ROWS];                                         // per key half: row overflowed
  __shared__ float xmx[2][ROWS];                                       // per key half: row max over the segment
  __shared__ int xredo;                                                // a row overflowed: second pass
  constexpr int BTAB = PAGED ? 1024 : 1;
  __shared__ int btab[BTAB];

  int w_item, rg;
  if (!decode_item(a, w_item, rg)) return;
  bool first_seg = true;
  for_each_segment(a, w_item, [&](const int b, const int len, const int kv_beg, const int kv_end, const int slot) {
  LANE_IDS_PER_PART;
  const bool pv_wave = wave >= 4;                    // wave-uniform role
  const int sw = wave & 3;                           // score wave index / P.V wave index
  const int qb = sw >> 1, kh = sw & 1;               // score roles: 32-row query block, key half
  if (!first_seg) {
    wait_vmcnt<0>();
    __syncthreads();
  }
  first_seg = false;
  const int R = a.n_q * a.n_h;
  const int rbase = rg * ROWS;
  const float sl2 = a.scale_log2;
  const long seq_row0 = (long)b * a.cache.max_len;
  const unsigned lds_stages = (unsigned)(size_t)(lds_void *)stages;
  const int ntiles = (kv_end - kv_beg + KVT - 1) / KVT;
  int q0 = 0;
  bool tab_lds = false;
  if constexpr (PAGED) {
    q0 = block_of(a.cache, kv_beg);
    const int nbq = block_of(a.cache, kv_end - 1) - q0 + 1;
    tab_lds = nbq <= BTAB;
    if (tab_lds) {
      const int *trow = a.cache.table + (long)b * a.cache.max_blocks + q0;
      for (int i = tid; i < nbq; i += 512) btab[i] = trow[i];
      __syncthreads();
    }
  }

  // Copies (P.V waves; copying thread index ct = tid - 256).  Stage slot
  // (row, c) holds cache chunk (row, c ^ (row & 7)) (no padding; the XOR
  // keeps the 16-byte score reads and the transposed reads free of bank
  // conflicts).  A tile lies inside one cache block (block_size is a multiple
  // of the tile), so its rows are contiguous: a uniform base plus 32-bit lane
  // offsets.  The lane's slot of instruction i is i*NC + ct; its (row, chunk)
  // advances by NC = 3*CH + 40 per instruction.  Rows past the end of a
  // partial last tile repeat its last row (finite values; their
  // probabilities are 0).
  static_assert(NC / CH == 3 && NC % CH == 40, "");
  const int ct = tid - NC;
  const int r0 = ct / CH, c0 = ct - (ct / CH) * CH;
  constexpr int RBYTES = FP8 ? DC + 2 * DR + 4 * (DC / 128) : 2 * D;   // bytes per cached row
  auto tile_src = [&](int t) {
    const int kvb = kv_beg + t * KVT;
    long trow;
    if constexpr (PAGED) {
      const int q = block_of(a.cache, kvb);
      const int blk = checked_block(a.cache, __builtin_amdgcn_readfirstlane(
                                                 tab_lds ? btab[q - q0] : a.cache.table[(long)b * a.cache.max_blocks + q]));
      trow = (long)blk * a.cache.block_size + (kvb - q * a.cache.block_size);
    } else {
      trow = seq_row0 + kvb;
    }
    return (const char *)a.cache.pool + trow * RBYTES;
  };
  auto copy_rows = [&](const char *src, int r_off, int last, int st) {
    int cr = r0, cc = c0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = min(r_off + cr, last);
      const unsigned dst = lds_stages + (unsigned)(st * STAGE * 2) + i * NC * 16 + (wave - 4) * 1024;
      dma16(src, (unsigned)(r * D + ((cc ^ (r & 7)) << 3)) * 2u, dst);
      cc += NC % CH;
      const bool wrap = cc >= CH;
      cc -= wrap ? CH : 0;
      cr += NC / CH + (wrap ? 1 : 0);
    }
  };
  // A full tile's per-lane source offsets are the same for every tile (only
  // the tile's base, a scalar, changes): formed once, they leave the copy of
  // a full tile with no vector arithmetic; a partial last tile clamps.
  unsigned full_off[LOADS];
  {
    int cr = r0, cc = c0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      full_off[i] = (unsigned)(cr * D + ((cc ^ (cr & 7)) << 3)) * 2u;
      cc += NC % CH;
      const bool wrap = cc >= CH;
      cc -= wrap ? CH : 0;
      cr += NC / CH + (wrap ? 1 : 0);
    }
  }
  auto copy_tile = [&](int t) {
    const int last = min(KVT, kv_end - (kv_beg + t * KVT)) - 1;
    if (last == KVT - 1) {
      const char *src = tile_src(t);
      const unsigned dst0 = lds_stages + (unsigned)((t % NS) * STAGE * 2) + (wave - 4) * 1024;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) dma16(src, full_off[i], dst0 + i * NC * 16);
    } else {
      copy_rows(tile_src(t), 0, last, t % NS);
    }
  };

  // FP8 tiles: copying thread ct converts row ct >> 3 of a tile, part
  // j = ct & 7: the 16-code pieces j + 8i (i = 0..3; codes 16(j + 8i) ..
  // +15, logical chunks 2(j + 8i) and 2(j + 8i) + 1 of the bf16 row), k_R
  // values 8j..8j+7 (chunk 64 + j) and the four group scales (piece j + 8i
  // lies in group i).  Interleaving the pieces over the lanes keeps each
  // row's loads 128 contiguous bytes and the 16-byte LDS writes free of bank
  // conflicts (a row's eight lanes hit eight distinct 4-bank groups of one
  // parity, the next row's swizzle the other parity).  The loads of tile t
  // are issued one iteration before the conversion writes it.
  static_assert(!FP8 || (DC == 512 && DR == 64 && NC == 8 * KVT), "");
  u32x4 f8c[4], f8r, f8s;
  auto fp8_load = [&](int t) {
    const int r = min(ct >> 3, min(KVT, kv_end - (kv_beg + t * KVT)) - 1), j = ct & 7;
    const char *row = tile_src(t) + (long)r * RBYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) f8c[i] = *(const u32x4 *)(row + 16 * (j + 8 * i));
    f8r = *(const u32x4 *)(row + DC + 16 * j);
    f8s = *(const u32x4 *)(row + DC + 2 * DR);   // the four group scales
  };
  auto fp8_store = [&](int t) {
    const int r = ct >> 3, j = ct & 7;
    lds_bf16 *st = (lds_bf16 *)stages + (t % NS) * STAGE + r * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // 16 codes -> two 8-element chunks (logical 2(j + 8i), 2(j + 8i) + 1)
      // columns 16(j + 8i).. lie in group i (the element is copied out first:
      // a bit cast of the vector element itself reads element 0)
      const unsigned sbits = f8s[i];
      const float scale = __builtin_bit_cast(float, sbits);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 v;
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          // the scaled conversion applies the power of two of its scale
          // operand (an MX-style scale), which is the whole of the scale
          const unsigned word = f8c[i][2 * h2 + w2];
          const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, scale, false);
          const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, scale, true);
          v[4 * w2] = lo[0];
          v[4 * w2 + 1] = lo[1];
          v[4 * w2 + 2] = hi[0];
          v[4 * w2 + 3] = hi[1];
        }
        const int c = 2 * (j + 8 * i) + h2;
        *(lds_bf16x8 *)(st + ((c ^ (r & 7)) << 3)) = v;
      }
    }
    *(lds_u32x4 *)(st + (((64 + j) ^ (r & 7)) << 3)) = f8r;
  };

  // pass 1 (only after a row overflowed in pass 0): each row's reference
  // is its maximum over the segment (score waves)
  float mfix[2] = {MREF0, MREF0};
  // returns true when pass 0 found an overflow (pass 1 must follow)
  auto run_pass = [&](const int pass) -> bool {
  // the 64 query rows reach LDS through stages 2 and 3 while tiles 0 and 1
  // are copied into stages 0 and 1 (FP8: tile 0 converted, tile 1 loaded)
  if (pv_wave) {
    const char *qsrc = (const char *)((const bf16 *)a.q + ((long)b * R + rbase) * D);
    copy_rows(qsrc, 0, R - 1 - rbase, 2);
    copy_rows(qsrc, KVT, R - 1 - rbase, 3);
    if constexpr (FP8) {
      fp8_load(0);
      wait_vmcnt<0>();
      fp8_store(0);
      if (ntiles >= 2) fp8_load(1);
    } else {
      for (int t = 0; t < 2 && t < ntiles; ++t) copy_tile(t);
      if (ntiles >= 2) wait_vmcnt<2 * LOADS>();   // the query copies
      else wait_vmcnt<LOADS>();
    }
  }
  bar();

  constexpr int TRH = 16 * D;
  const lds_bf16 *st_base = (const lds_bf16 *)stages;
  lds_bf16x8 *pl = (lds_bf16x8 *)pbuf;
  float *fac = (float *)pbuf;                // after the loop: 1/l per row
  lds_bf16 *ot = (lds_bf16 *)stages;         // after the loop: normalised rows
  static_assert(ROWS * DC <= NS * STAGE, "");

  // The two roles run separate code (their register state differs); both
  // pass the same barriers in the same order:
  //   B0 (tile 0 visible, query reads done), per iteration i: [i == 0: the
  //   reference exchange] + end of iteration, then E1, E2, E3 around the
  //   epilogue.
  if (!pv_wave) {
    // ------------------------------------------------------------ score waves
    bf16x8 qf[2][QS];
    int limit[2];
    float mref[2] = {MREF0, MREF0}, lrun[2] = {0.f, 0.f};
    float mx[2] = {-INFINITY, -INFINITY};              // the lane's maximum so far (pass 0)
    bool ovf[2] = {false, false};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rl = qb * 32 + j * 16 + lrow;          // row within the group
      const int rr = rl & (KVT - 1);
      const lds_bf16 *qs = (const lds_bf16 *)stages + (2 + (rl >> 5)) * STAGE + rr * D;
#pragma unroll
      for (int q = 0; q < QS; ++q) qf[j][q] = *(const lds_bf16x8 *)(qs + (((4 * q + lgrp) ^ (rr & 7)) << 3));
      const int qr = min(rbase + rl, R - 1);
      limit[j] = min(len - a.n_q + qr / a.n_h, kv_end - 1);
    }
    // the wave's smallest limit: tiles ending at or below it need no mask
    int lim_all = min(limit[0], limit[1]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lim_all = min(lim_all, __shfl_xor(lim_all, o));
    lim_all = __builtin_amdgcn_readfirstlane(lim_all);
    // Score reads: row kh*16 + lrow of the tile, logical chunk 4q+lgrp
    // (natural k order), physical chunk (4q+lgrp) ^ (lrow & 7) =
    // 4(q ^ fq) + (lgrp ^ (lrow & 3)) with fq = (lrow >> 2) & 1: even and odd
    // steps use two base offsets.  Lane group g then holds the scores of
    // rows 4g..4g+3 of the half, and the transposed reads of P.V fetch exactly
    // those rows (any four rows can form the 4x16 block), so P keeps that key
    // order in LDS: entry (g, row) holds keys 4g..4g+3 of the first half and
    // 16+4g..16+4g+3 of the second.
    const int fq = (lrow >> 2) & 1, gq = lgrp ^ (lrow & 3);
    const int a_even = (kh * 16 + lrow) * D + (4 * fq + gq) * 8;
    const int a_odd = (kh * 16 + lrow) * D + (gq - 4 * fq) * 8;
    wait_lgkm0();
    bar();                                             // B0
    if (tid == 0) xredo = 0;   // every read of the last pass's flag is behind B0

    for (int t = 0; t <= ntiles; ++t) {
      if (t < ntiles) {
        // scores and softmax of tile t into P buffer t & 1
        const lds_bf16 *ca_p = st_base + (t % NS) * STAGE;
        const int kvb = kv_beg + t * KVT;
        f32x4 sacc[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) sacc[j][0] = sacc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto rd = [&](int q) { return *(const lds_bf16x8 *)(ca_p + ((q & 1) ? a_odd : a_even) + q * 32); };
        bf16x8 ca[PF + 1];
#pragma unroll
        for (int q = 0; q < PF; ++q) ca[q] = rd(q);
#pragma unroll
        for (int q = 0; q < QS; ++q) {
          if (q + PF < QS) ca[(q + PF) % (PF + 1)] = rd(q + PF);
#pragma unroll
          for (int j = 0; j < 2; ++j) sacc[j][q & 1] = Mma<bf16>::mma(ca[q % (PF + 1)], qf[j][q], sacc[j][q & 1]);
          __builtin_amdgcn_sched_barrier(0);   // keep the read-ahead distance as written
        }
        float sv[2][4], mt[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[j][i] = (sacc[j][0][i] + sacc[j][1][i]) * sl2;
        if (kvb + KVT - 1 > lim_all) {                 // wave-uniform: a key past some row's limit
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (kvb + 16 * kh + 4 * lgrp + i > limit[j]) sv[j][i] = -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          mt[j] = fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3]));
          mx[j] = fmaxf(mx[j], mt[j]);
        }
        // the first tile fixes the reference of each row (max over both key
        // halves, exchanged through LDS); later tiles only check that they
        // stay within TAU of it
        if (t == 0) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float m16 = row_max(mt[j]);
            if (lgrp == 0) xch[kh][qb * 32 + j * 16 + lrow] = m16;
          }
          wait_lgkm0();
          bar();                                       // reference exchange
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int rl = qb * 32 + j * 16 + lrow;
            mref[j] = pass ? mfix[j] : fmaxf(fmaxf(xch[0][rl], xch[1][rl]), MREF0);
          }
        } else if (pass == 0) {
#pragma unroll
          for (int j = 0; j < 2; ++j) ovf[j] |= mt[j] > mref[j] + TAU;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x4 pf;
          float psum = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(sv[j][i] - mref[j]);
            psum += p;
            pf[i] = (bf16)p;
          }
          lrun[j] += psum;
          *(lds_bf16x4 *)((lds_bf16 *)(pl + ((t & 1) * 4 + lgrp) * ROWS + qb * 32 + j * 16 + lrow) + kh * 4) = pf;
        }
      }
      wait_lgkm0();
      bar();                                           // end of iteration t
    }

    // row sums, overflow marks and row maxima of the two key halves meet in
    // LDS
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool rov = row_max(ovf[j] ? 1.f : 0.f) > 0.f;
      const float rmx = row_max(mx[j]);
      float l = lrun[j];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      if (lgrp == 0) {
        xch[kh][qb * 32 + j * 16 + lrow] = l;
        xov[kh][qb * 32 + j * 16 + lrow] = rov ? 1 : 0;
        xmx[kh][qb * 32 + j * 16 + lrow] = rmx;
      }
    }
    __syncthreads();                                   // E1 (P no longer read)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rl = qb * 32 + j * 16 + lrow;
      mfix[j] = fmaxf(fmaxf(xmx[0][rl], xmx[1][rl]), MREF0);
    }
    if (kh == 0 && lgrp == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rl = qb * 32 + j * 16 + lrow;
        const float l = xch[0][rl] + xch[1][rl];
        // overflow in pass 0 sends the whole workgroup through pass 1 (rows
        // of the group past R repeat the scores of row R - 1); the sums of
        // pass 0 are then overwritten
        if (pass == 0 && (xov[0][rl] | xov[1][rl]) != 0) xredo = 1;
        fac[rl] = l > 0.f ? 1.f / l : 0.f;
        if (rbase + rl < R)
          a.lse_part[(long)slot * R + rbase + rl] = l > 0.f ? mref[j] + log2f(l) : -INFINITY;
      }
    }
    __syncthreads();                                   // E2
    __syncthreads();                                   // E3
  } else {
    // ------------------------------------------------------------ P.V waves
    // tile 0 has landed (tile 1 may still be in flight)
    if constexpr (!FP8) {
      if (ntiles >= 2) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
    }
    f32x4 oacc[DBW][HBS];
#pragma unroll
    for (int i = 0; i < DBW; ++i)
#pragma unroll
      for (int j = 0; j < HBS; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // transposed reads of the wave's 128 columns (16 chunks): row r = 4*lgrp
    // + (lrow >> 2) (and r + 16), logical chunk 16p + 2db + ((lrow & 3) >> 1),
    // physical chunk 16p + 8(db >> 2) + 2((db & 3) ^ fh) + cl
    const int r = 4 * lgrp + (lrow >> 2), fr = r & 7;
    const int cl = ((lrow & 3) >> 1) ^ (fr & 1), half = (lrow & 1) * 4;
    const int t_base = r * D + (sw * 16 + cl) * 8 + half;
    const int t_fh = fr >> 1;
    wait_lgkm0();                                      // FP8: this wave's writes of tile 0
    bar();                                             // B0

    // bf16: the V^T fragments of tile i are read in iteration i, beside its
    // scores, and multiplied in iteration i+1 (with P of tile i), so a stage
    // is free one iteration after its tile arrives and the copies run three
    // tiles ahead
    bf16x8 va[DBW];
    for (int i = 0; i <= ntiles; ++i) {
      // FP8: tile i+1, loaded in iteration i-1, is converted into the stage
      // of tile i-3, and the loads of tile i+2 go out.  bf16: tile i+3 goes
      // into the stage of tile i-1, which every wave finished reading in
      // iteration i-1 (iteration 0 also issues tile 2: stages 2 and 3 held
      // the query rows until B0)
      if constexpr (FP8) {
        if (i + 1 < ntiles) {
          wait_vmcnt<0>();
          fp8_store(i + 1);
          if (i + 2 < ntiles) fp8_load(i + 2);
        }
      } else {
        if (i == 0 && 2 < ntiles) copy_tile(2);
        if (i + 3 < ntiles) copy_tile(i + 3);
      }
      if (i == 0) bar();                               // the score waves' reference exchange
      if constexpr (!FP8) {
        if (i >= 1) {
          const int u = i - 1;
          bf16x8 pb[HBS];
#pragma unroll
          for (int hb = 0; hb < HBS; ++hb) pb[hb] = pl[((u & 1) * 4 + lgrp) * ROWS + hb * 16 + lrow];
#pragma unroll
          for (int db = 0; db < DBW; ++db)
#pragma unroll
            for (int hb = 0; hb < HBS; ++hb) oacc[db][hb] = Mma<bf16>::mma(va[db], pb[hb], oacc[db][hb]);
        }
        // then this tile's fragments replace them
        if (i < ntiles) {
          const lds_bf16 *st = st_base + (i % NS) * STAGE;
#pragma unroll
          for (int db = 0; db < DBW; ++db) {
            const int o = t_base + 16 * ((db & 3) ^ t_fh) + 64 * (db >> 2);
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + o));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + o + TRH));
            va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
        // tile i+1 has landed (tiles i+2 and i+3 may stay in flight)
        if (i + 3 < ntiles) wait_vmcnt<2 * LOADS>();
        else if (i + 2 < ntiles) wait_vmcnt<LOADS>();
        else wait_vmcnt<0>();
      } else if (i >= 1) {
        const int u = i - 1;
        const lds_bf16 *st = st_base + (u % NS) * STAGE;
        bf16x8 vb[DBW], pb[HBS];
#pragma unroll
        for (int hb = 0; hb < HBS; ++hb) pb[hb] = pl[((u & 1) * 4 + lgrp) * ROWS + hb * 16 + lrow];
#pragma unroll
        for (int db = 0; db < DBW; ++db) {
          const int o = t_base + 16 * ((db & 3) ^ t_fh) + 64 * (db >> 2);
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + o));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + o + TRH));
          vb[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int db = 0; db < DBW; ++db)
#pragma unroll
          for (int hb = 0; hb < HBS; ++hb) oacc[db][hb] = Mma<bf16>::mma(vb[db], pb[hb], oacc[db][hb]);
      }
      wait_lgkm0();
      bar();                                           // end of iteration i
    }
    __syncthreads();                                   // E1
    __syncthreads();                                   // E2 (1/l per row is in LDS)
    // normalised rows through the idle stages: chunk c of row r at c ^ (r & 15)
#pragma unroll
    for (int hb = 0; hb < HBS; ++hb) {
      const int rl = hb * 16 + lrow;
      const float inv = fac[rl];
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        const f32x4 o4 = oacc[db][hb] * inv;
        const int c = (sw * 16 + db * 2 + (lgrp >> 1)) ^ lrow;
        *(lds_bf16x4 *)(ot + rl * DC + c * 8 + (lgrp & 1) * 4) =
            bf16x4{(bf16)o4[0], (bf16)o4[1], (bf16)o4[2], (bf16)o4[3]};
      }
    }
    __syncthreads();                                   // E3
  }
  // the flag was written before E2 and is reset after the next B0
  if (pass == 0 && xredo != 0) return true;
  // one whole row per store instruction
  bf16 *op = (bf16 *)a.o_part + ((long)slot * R + rbase) * DC + lane * 8;
  for (int rl = wave; rl < ROWS && rbase + rl < R; rl += 8)
    __builtin_nontemporal_store(*(const lds_bf16x8 *)(ot + rl * DC + (lane ^ (rl & 15)) * 8),
                                (bf16x8 *)(op + (long)rl * DC));
  return false;
  };
  if (run_pass(0)) {
    wait_vmcnt<0>();
    __syncthreads();
    run_pass(1);
  }
  });
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
  int total, P, slot0, nsp;
  plan_totals(a, total, P);
  const SeqSpan sp = plan_seq(a, b);
  plan_slots(sp, P, slot0, nsp);
  const long base = (long)slot0 * R + r;
  T *out = (T *)a.o_lat + row * DC;
  // split weights: lane s holds split s (for up to 64 splits; more are
  // read in rounds)
  float lmax = -INFINITY;
  for (int s0 = 0; s0 < nsp; s0 += 64) {
    const float ls = s0 + lane < nsp ? a.lse_part[base + (long)(s0 + lane) * R] : -INFINITY;
    lmax = fmaxf(lmax, ls);
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
// workgroup = (head i, 16 tokens), eight waves in two roles whose memory
// counters are separate, so neither waits for the other's loads:
//   waves 0..3 merge the splits of four tokens each (wave w: tokens w, w+4,
//     w+8, w+12; a lane per eight latent columns) into LDS, rounded to bf16
//     as a stored o_lat would be; only
//     the splits a token has are loaded, all of them before any is used;
//   waves 4..7 copy W_UV,i (128 KB) into LDS.
// Then O^T[v][t] = W_UV,i[v][:] . o_lat[t][:] on the matrix cores, wave w
// taking features 16w..16w+15.  The token groups of a head share an XCD,
// whose L2 serves their common reads of W_UV,i.
template <int DC, int DR, int DV>
__global__ __launch_bounds__(512, 1) void decode_combine_uv_kernel(DecodeArgs a, const bf16 *w_uv, bf16 *o,
                                                                    Fp8Out q8) {
  constexpr int TT = 16, NM = 4;         // tokens per workgroup, merging waves
  constexpr int NW = 8;                  // waves
  constexpr int KS = DC / 32;            // k steps
  constexpr int PER = DC / 64;           // latent columns per lane in the merge
  constexpr int SB = 8;                  // splits per token requested up front
  static_assert(DC == 512 && PER == 8 && DV == 16 * NW, "");
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

  if (wave >= NM) {
    // W_UV,i -> LDS, whole rows per copy instruction
    constexpr int NC = 64 * (NW - NM);
    constexpr int WLOADS = DV * DC / 8 / NC;
    const int ct = threadIdx.x - 64 * NM;
    const unsigned lw = (unsigned)(size_t)(lds_void *)wuv;
    const bf16 *wh = w_uv + (long)h * DV * DC;
#pragma unroll
    for (int j = 0; j < WLOADS; ++j) {
      const int sl = j * NC + ct, v = sl / (DC / 8), pc = sl % (DC / 8);
      const int c = pc ^ (v & 15);
      dma16(wh, (unsigned)((v * DC + c * 8) * 2), lw + (unsigned)(j * NC + (wave - NM) * 64) * 16);
    }
    wait_vmcnt<0>();
  } else {
    // merge: wave w takes tokens w, w+4, w+8, w+12 of the group (interleaved,
    // so that a group of fewer tokens still spreads over the four waves)
    constexpr int TW = TT / NM;
    int bq[TW], rq[TW], nsp[TW];
    long base[TW];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int t = min(tg * TT + j * NM + wave, T - 1);
      bq[j] = t / a.n_q;
      rq[j] = (t % a.n_q) * a.n_h + h;
    }
    {
      SeqSpan sp[TW];
      int total;
      plan_spans<TW>(a, bq, sp, total);
      const int P = (total + a.W - 1) / a.W;
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        int slot0;
        plan_slots(sp[j], P, slot0, nsp[j]);
        if (tg * TT + j * NM + wave >= T) nsp[j] = 0;
        nsp[j] = __builtin_amdgcn_readfirstlane(nsp[j]);
        base[j] = (long)slot0 * R + rq[j];
      }
    }
    // the log-sum-exps (lane s: split s) and the first SB partial rows of
    // each token are requested before any is used; splits at or past a
    // sequence's own count are neither loaded nor used (this call did not
    // write them: they hold whatever the workspace held, possibly NaN bits)
    float ls[TW];
    bf16x8 v[TW][SB];
#pragma unroll
    for (int j = 0; j < TW; ++j) ls[j] = a.lse_part[base[j] + (long)min(lane, max(nsp[j] - 1, 0)) * R];
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int jj = 0; jj < SB; ++jj)
        if (jj < nsp[j]) v[j][jj] = *(const bf16x8 *)((const bf16 *)a.o_part + (base[j] + (long)jj * R) * DC + lane * PER);
#pragma unroll
    for (int j = 0; j < TW; ++j) ls[j] = lane < nsp[j] ? ls[j] : -INFINITY;
    lds_bf16 *ol = (lds_bf16 *)olat;
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int tl = j * NM + wave;
      float res[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) res[i] = 0.f;
      if (nsp[j] > 0) {
        float lmax = ls[j];
        for (int s0 = 64; s0 < nsp[j]; s0 += 64) {
          const float x = s0 + lane < nsp[j] ? a.lse_part[base[j] + (long)(s0 + lane) * R] : -INFINITY;
          lmax = fmaxf(lmax, x);
        }
        {
#pragma unroll
          for (int o2 = 32; o2 > 0; o2 >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o2));
          float wsum = 0.f;
#pragma unroll
          for (int jj = 0; jj < SB; ++jj) {
            // the condition is wave-uniform
            const float lsj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[j]), jj));
            if (jj < nsp[j] && lsj != -INFINITY) {
              const float w = exp2f(lsj - lmax);
              wsum += w;
#pragma unroll
              for (int i = 0; i < PER; ++i) res[i] += w * (float)v[j][jj][i];
            }
          }
          // the remaining splits in batches of eight, every load of a batch
          // issued before any is used (one round trip per batch)
          for (int s0 = SB; s0 < nsp[j]; s0 += 8) {
            bf16x8 vv[8];
            float lsv[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const int sp = min(s0 + jj, nsp[j] - 1);
              vv[jj] = *(const bf16x8 *)((const bf16 *)a.o_part + (base[j] + (long)sp * R) * DC + lane * PER);
              lsv[jj] = sp < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[j]), sp))
                                : a.lse_part[base[j] + (long)sp * R];
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
              if (s0 + jj < nsp[j] && lsv[jj] != -INFINITY) {
                const float w = exp2f(lsv[jj] - lmax);
                wsum += w;
#pragma unroll
                for (int i = 0; i < PER; ++i) res[i] += w * (float)vv[jj][i];
              }
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
  }
  __syncthreads();

  // A operand: W_UV,i row 16*wave + lrow, k = 32*ks + 8*lgrp..
  const lds_bf16 *wl = (const lds_bf16 *)wuv;
  const lds_bf16 *ol = (const lds_bf16 *)olat;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 xb = *(const lds_bf16x8 *)(ol + lrow * DC + (((4 * ks + lgrp) ^ lrow) * 8));
    const bf16x8 wf = *(const lds_bf16x8 *)(wl + (wave * 16 + lrow) * DC + (((4 * ks + lgrp) ^ lrow) * 8));
    acc = Mma<bf16>::mma(wf, xb, acc);
  }
  // lane: features 16*wave + 4*lgrp + 0..3 of token lrow
  const int t = tg * TT + lrow;
  const bf16x4 ob = bf16x4{(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
  if (t < T) *(bf16x4 *)(o + ((long)t * a.n_h + h) * DV + wave * 16 + 4 * lgrp) = ob;
  if (q8.codes) {
    // FP8 projections: the head's 128 outputs of a token (its bf16 values)
    // are one quantisation group; their maximum magnitude is gathered from
    // the lane's four, the token's four lane groups and the eight waves
    __shared__ float gmax[NW][TT];
    float v[4], m = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = (float)ob[e];
      m = fmaxf(m, fabsf(v[e]));
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lgrp == 0) gmax[wave][lrow] = m;
    __syncthreads();
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) amax = fmaxf(amax, gmax[w][lrow]);
    // smallest power of two 2^k with 448 * 2^k >= amax (as the activation quantiser)
    int k = 0;
    if (amax > 0.f) {
      int e;
      const float f = frexpf(amax, &e);
      k = max(e - 9 + (f > 0.875f ? 1 : 0), -126);
    }
    const float inv = ldexpf(1.f, -k);
    const unsigned lo = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(v[0] * inv, v[1] * inv, 0, false) & 0xFFFFu;
    const unsigned hi = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(v[2] * inv, v[3] * inv, 0, false) & 0xFFFFu;
    if (t < T) {
      *(unsigned *)(q8.codes + ((long)t * a.n_h + h) * DV + wave * 16 + 4 * lgrp) = lo | (hi << 16);
      if (wave == 0 && lgrp == 0) q8.scales[(long)h * q8.ld_s + t] = (unsigned char)(k + 127);
    }
  }
}

hipError_t launch_decode_combine_uv(const DecodeArgs &a, int d_v, const void *w_uv, void *o, Fp8Out q8,
                                    hipStream_t st) {
  if (a.d_c != 512 || a.d_rope != 64 || d_v != 128) return hipErrorNotSupported;
  const int T = a.B * a.n_q;
  const int grid = ((a.n_h + 7) / 8) * 8 * ((T + 15) / 16);
  timing_before("decode_combine_uv", st);
  hipLaunchKernelGGL((decode_combine_uv_kernel<512, 64, 128>), dim3(grid), dim3(512), 0, st, a,
                     (const bf16 *)w_uv, (bf16 *)o, q8);
  timing_after("decode_combine_uv", st);
  return hipGetLastError();
}

int decode_kv_tile(int) { return KVT; }
// Query rows per workgroup: 64 (the two-waves-per-SIMD kernel for bf16).
int decode_rows_per_group(int dtype, long B, long R, int cus) {
  (void)dtype; (void)B; (void)R; (void)cus;
  return 64;
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
  if (dtype == 1 && a.d_c == 512 && a.d_rope == 64 && tile_in_block && a.rows == 64) {
    const int grid = decode_grid(a);
    timing_before("decode_attn", st);
    if (a.cache.fp8) {
      if (a.cache.table)
        hipLaunchKernelGGL((decode_attn_ws_kernel<512, 64, true, true>), dim3(grid), dim3(512), 0, st, a);
      else
        hipLaunchKernelGGL((decode_attn_ws_kernel<512, 64, false, true>), dim3(grid), dim3(512), 0, st, a);
    } else {
      if (a.cache.table)
        hipLaunchKernelGGL((decode_attn_ws_kernel<512, 64, true, false>), dim3(grid), dim3(512), 0, st, a);
      else
        hipLaunchKernelGGL((decode_attn_ws_kernel<512, 64, false, false>), dim3(grid), dim3(512), 0, st, a);
    }
    timing_after("decode_attn", st);
    return hipGetLastError();
  }
  if (a.cache.fp8) return hipErrorInvalidValue;   // FP8 rows: the DeepSeek-V3 kernel only
  if (dtype == 1 && a.d_c == 512 && a.d_rope == 64)
    return launch_attn<bf16, 4, 1, 512, 64>(a, st);
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
