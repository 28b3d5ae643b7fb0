// Causal MLA prefill attention, flash-style (tiled, exact softmax), in the
// up-projected form of section 2.1 of the DeepSeek-V3 paper-reading notes:
// for head i, q = [q_C,i ; q_R,i] against k = [k_C,j,i ; k_R,j] (k_R shared
// by all heads), values v_j,i, scale 1/sqrt(d_h + d_R).
//
// Common to the kernels here: one workgroup = (sequence, head, block of
// queries), its waves walk the 64-key tiles up to the diagonal, query blocks
// start from the longest (causal work imbalance).  Scores are formed
// transposed (S^T = K . Q^T) so that each lane owns one query column: the
// softmax max/sum are lane-local plus a shuffle, and after permuting the key
// rows of the A operand the probabilities are already the B operand of
// O^T += V^T . P^T.  V arrives transposed ([n_h*d_v][tokens], written that
// way by the V up-projection), so both contractions read 16-byte runs.
//
//   flash_prefill_m32_kernel  bf16, lengths a multiple of 8: 32x32x16 MFMAs,
//                             copy-fed LDS ring, softmax reference fixed on
//                             the first tile (a workgroup with a row that
//                             outgrows it runs a second pass with each row's
//                             maximum as the reference);
//   flash_prefill_kernel      fp32, and bf16 at other lengths: tiles staged
//                             through registers, 16x16 MFMAs, reference
//                             moved lazily.
#include "mla_internal.h"

namespace mla {

#ifndef FLASH_QB
#define FLASH_QB 2   // 16-query blocks per wave (flash_prefill_kernel, bf16)
#define FLASH_NW 8   // waves per workgroup (flash_prefill_kernel, bf16)
#endif

template <typename T, int QB, int NW, int DN, int DR, int DV>
__global__ __launch_bounds__(64 * NW, 1) void flash_prefill_kernel(FlashArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int KVB = 4, KVT = 64;
  constexpr int DQK = DN + DR;
  constexpr int KPL = Mma<T>::KPL;
  constexpr int VE = Vec<T>::N;
  constexpr int RUNQ = DQK / 4;
  constexpr int QS = RUNQ / KPL;
  constexpr int PRUN = KVT / 4;
  constexpr int PS = PRUN / KPL;
  constexpr int DVB = DV / 16;
  constexpr int LDK = DQK + VE;
  constexpr int LDV = KVT + VE;
  constexpr int BQ = 16 * QB * NW;
  static_assert(RUNQ % KPL == 0 && PRUN % KPL == 0, "");
  static_assert(DN % VE == 0 && DR % VE == 0 && KVT % VE == 0, "");
  constexpr int KCH = KVT * (DQK / VE);
  constexpr int VCH = DV * (KVT / VE);
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VPT = (VCH + NT - 1) / NT;
  typedef typename Mma<T>::frag frag;
  typedef __attribute__((address_space(3))) T lds_T;
  typedef __attribute__((address_space(3))) frag lds_frag;

  __shared__ __attribute__((aligned(16))) T ks[2][KVT * LDK];
  __shared__ __attribute__((aligned(16))) T vs[2][DV * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int L = a.L, NH = a.n_h;
  const int qtiles = (L + BQ - 1) / BQ;

  // block -> (query tile, longest first; sequence; head).  Heads that share
  // bid % 8 land on one XCD, so the query tiles of a head running together
  // share its K/V tiles in that XCD's L2; longest-first keeps the causal tail
  // short.
  int bid = blockIdx.x, h, b, qt_rev;
  if ((NH & 7) == 0) {
    const int hx = bid & 7;
    int rest = bid >> 3;
    const int hh = rest % (NH >> 3);
    rest /= (NH >> 3);
    b = rest % a.B;
    qt_rev = rest / a.B;
    h = hh * 8 + hx;
  } else {
    h = bid % NH;
    int rest = bid / NH;
    b = rest % a.B;
    qt_rev = rest / a.B;
  }
  const int qt = qtiles - 1 - qt_rev;
  const long tok0 = (long)b * L;              // first token of the sequence
  const long ntok = (long)a.B * L;            // V^T row length
  const int q0 = qt * BQ + wave * 16 * QB;    // first query of this wave
  const int wave_qmax = min(q0 + 16 * QB - 1, L - 1);
  const int blk_qmax = min(qt * BQ + BQ - 1, L - 1);
  const float sl2 = a.scale_log2;

  frag qf[QB][QS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = min(q0 + qb * 16 + lrow, L - 1);
    const T *qrow = (const T *)a.q + ((tok0 + t) * NH + h) * DQK + lgrp * RUNQ;
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[qb][s] = *(const frag *)(qrow + s * KPL);
  }

  f32x4 oacc[DVB][QB];
#pragma unroll
  for (int i = 0; i < DVB; ++i)
#pragma unroll
    for (int j = 0; j < QB; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref[QB], lrun[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) { mref[j] = -1e30f; lrun[j] = 0.f; }

  const T *Kn = (const T *)a.k;
  const T *Kr = (const T *)a.kr;
  const T *Vt = (const T *)a.vt;
  u32x4 kr_[KPT], vr_[VPT];
  auto gload = [&](int kvb) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (c < KCH) {
        const int r = c / (DQK / VE), cc = (c % (DQK / VE)) * VE;
        const long tok = tok0 + min(kvb + r, L - 1);
        const T *src = cc < DN ? Kn + (tok * NH + h) * DN + cc : Kr + tok * DR + (cc - DN);
        kr_[i] = *(const u32x4 *)src;
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      if (c < VCH) {
        const int d = c / (KVT / VE), kc = (c % (KVT / VE)) * VE;
        const int kv = kvb + kc;
        const T *src = Vt + (long)(h * DV + d) * ntok + tok0 + kv;
        if (kv + VE <= L) {
          vr_[i] = *(const u32x4 *)src;
        } else {
          T tmp[VE];
#pragma unroll
          for (int j = 0; j < VE; ++j) tmp[j] = (kv + j < L) ? src[j] : from_f32<T>(0.f);
          vr_[i] = *(const u32x4 *)tmp;
        }
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (c < KCH) {
        const int r = c / (DQK / VE), cc = (c % (DQK / VE)) * VE;
        *(u32x4 *)&ks[buf][r * LDK + cc] = kr_[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      if (c < VCH) {
        const int d = c / (KVT / VE), kc = (c % (KVT / VE)) * VE;
        *(u32x4 *)&vs[buf][d * LDV + kc] = vr_[i];
      }
    }
  };

  const int ntiles = blk_qmax / KVT + 1;
  // Scores use the key rows in natural order (A slot = row); lane group g
  // then holds keys 4g+i of each 16-key block, and V^T is read with the same
  // key order for P.V.
  const int a_off = lrow * LDK + lgrp * RUNQ;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int kvb = t * KVT;
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(kvb + KVT);
    if (kvb <= wave_qmax) {   // otherwise every key of this tile is after every query of this wave
      const lds_T *kb_p = (const lds_T *)ks[buf] + a_off;
      const lds_T *vb_p = (const lds_T *)vs[buf];
      f32x4 sacc[KVB][QB];
#pragma unroll
      for (int kb = 0; kb < KVB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < QS; ++s) {
#pragma unroll
        for (int kb = 0; kb < KVB; ++kb) {
          const frag ka = *(const lds_frag *)(kb_p + kb * 16 * LDK + s * KPL);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = Mma<T>::mma(ka, qf[qb][s], sacc[kb][qb]);
        }
      }

      const bool diag = kvb + KVT - 1 > q0;
      frag pf[QB][PS];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qpos = q0 + qb * 16 + lrow;
        float sv[KVB][4];
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KVB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kv = kvb + 16 * kb + 4 * lgrp + i;
            float x = sacc[kb][qb][i] * sl2;
            if (diag && kv > qpos) x = -INFINITY;
            sv[kb][i] = x;
            mt = fmaxf(mt, x);
          }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // the running reference max only moves when a tile exceeds it by 2^8
        if (__any(mt > mref[qb] + 8.0f)) {
          const float mnew = fmaxf(mref[qb], mt);
          const float alpha = exp2f(mref[qb] - mnew);
          mref[qb] = mnew;
          lrun[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DVB; ++db) oacc[db][qb] *= alpha;
        }
        float psum = 0.f;
        float p[KVB][4];
#pragma unroll
        for (int kb = 0; kb < KVB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kb][i] = exp2f(sv[kb][i] - mref[qb]);
            psum += p[kb][i];
          }
        lrun[qb] += psum;
        // P.V step ps covers key blocks 2ps/KPL... : slot j of lane group g is
        // key 16*(j/4) + 4g + (j%4) of the tile
        if constexpr (KPL == 8) {
#pragma unroll
          for (int ps = 0; ps < PS; ++ps) {
            bf16x8 f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int jj = ps * 8 + j;
              f[j] = (bf16)p[jj >> 2][jj & 3];
            }
            pf[qb][ps] = f;
          }
        } else {
#pragma unroll
          for (int ps = 0; ps < PS; ++ps) pf[qb][ps] = p[ps >> 2][ps & 3];
        }
      }

      // V^T rows d, key slots in the same order as the probabilities: slot j
      // of lane group g is key 16*(j/4) + 4g + (j%4), i.e. two 4-key runs
#pragma unroll
      for (int ps = 0; ps < PS; ++ps)
#pragma unroll
        for (int db = 0; db < DVB; ++db) {
          frag va;
          if constexpr (KPL == 8) {
            typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
            const lds_T *row = vb_p + (db * 16 + lrow) * LDV + 4 * lgrp;
            const bf16x4 lo = *(const lds_bf16x4 *)(row + 32 * ps);
            const bf16x4 hi = *(const lds_bf16x4 *)(row + 32 * ps + 16);
            va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          } else {
            va = *(const lds_frag *)(vb_p + (db * 16 + lrow) * LDV + 16 * (ps >> 2) + 4 * lgrp + (ps & 3));
          }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = Mma<T>::mma(va, pf[qb][ps], oacc[db][qb]);
        }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = lrun[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int t = q0 + qb * 16 + lrow;
    if (t < L) {
      const float inv = 1.f / l;
      T *orow = (T *)a.o + ((tok0 + t) * NH + h) * DV;
#pragma unroll
      for (int db = 0; db < DVB; ++db) {
        float v[4] = {oacc[db][qb][0] * inv, oacc[db][qb][1] * inv, oacc[db][qb][2] * inv, oacc[db][qb][3] * inv};
        store4<T>(orow, db * 16 + 4 * lgrp, v, 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel for gfx950 (d_nope 128, d_R 64, d_v 128, L a multiple of 8):
// causal flash attention over one (sequence, head, 256-query) block, 8 waves
// of 32 queries on 32x32x16 MFMAs.  The K_C, k_R and V^T tiles of 64 keys go
// HBM -> LDS with global_load_lds_dwordx4 into a four-stage ring (copies
// three tiles ahead, one barrier per tile, no staging registers); each row's
// 16-byte chunks are XORed with the row index so that the 32-row fragment
// reads of a quarter wave hit distinct banks.  Keys past the end of the
// sequence repeat valid data (their probabilities are 0).  The softmax
// reference of a row is fixed on the first tile (see the kernel body).
//
// S^T = K.Q^T for a 32-key block leaves lane (query l%32, half h = l/32)
// holding rows 8j + 4h + i.  Loading key swap23(R) into K row R of the tile
// (bits 2 and 3 of the row index exchanged) makes the 8 values a lane feeds
// as P^T to P.V step m the contiguous keys 16m + 8h .. 16m + 8h + 7, so that
// V^T is read in whole 16-byte chunks.
// ---------------------------------------------------------------------------
namespace {
typedef __attribute__((address_space(3))) void lds_void_t;
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int N>
__device__ inline void fp_wait_vm() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}
template <int N>
__device__ inline void fp_wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4));
}
__device__ inline void fp_dma16(const void *gbase, unsigned off, unsigned lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(gbase)
      : "memory", "m0");
}
__device__ inline void fp_bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace

__device__ inline int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void flash_prefill_m32_kernel(FlashArgs a) {
  constexpr int DN = 128, DR = 64, DV = 128, KVT = 64, NT = 64 * NW;
  constexpr int QS = (DN + DR) / 16, DVB = DV / 32;
  constexpr int KN_E = KVT * DN, KR_E = KVT * DR, V_E = DV * KVT;
  constexpr int STAGE = KN_E + KR_E + V_E;       // elements (40 KB)
#ifndef FLASH_NS
#define FLASH_NS 4
#endif
  constexpr int NS = FLASH_NS;   // stages (at most four fit)
  static_assert(NS >= 2 && NS <= 4, "");
  constexpr int LKN = KN_E / 8 / NT, LKR = KR_E / 8 / NT, LV = V_E / 8 / NT;
  constexpr int LOADS = LKN + LKR + LV;
  constexpr int BQ = 32 * NW;
  static_assert(KN_E % (8 * NT) == 0 && KR_E % (8 * NT) == 0 && V_E % (8 * NT) == 0, "");
  typedef __attribute__((address_space(3))) bf16x8 lds_frag;
  typedef __attribute__((address_space(3))) char lds_char;

  __shared__ __attribute__((aligned(1024))) bf16 stages[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lc = lane & 31, hh = lane >> 5;
  const int L = a.L, NH = a.n_h;
  const int Lq = a.lens ? a.Lq : L;   // queries per sequence
  const int qtiles = (Lq + BQ - 1) / BQ;

  int bid = blockIdx.x, h, b, qt_rev;
  if ((NH & 7) == 0) {
    const int hx = bid & 7;
    int rest = bid >> 3;
    const int hq = rest % (NH >> 3);
    rest /= (NH >> 3);
    b = rest % a.B;
    qt_rev = rest / a.B;
    h = hq * 8 + hx;
  } else {
    h = bid % NH;
    int rest = bid / NH;
    b = rest % a.B;
    qt_rev = rest / a.B;
  }
  const int qt = qtiles - 1 - qt_rev;
  const long tok0 = (long)b * L;      // first key row of the sequence
  const long tok0q = (long)b * Lq;    // first query row
  const long ntok = (long)a.B * L;
  // position of query 0: after a prefix of lens[b] - Lq keys (lens clamped
  // into [Lq, L], so that no access leaves the sequence's rows)
  const int pos0 = a.lens ? min(max(a.lens[b], Lq), L) - Lq : 0;
  const int q0 = qt * BQ + wave * 32;                         // query index
  const int qpos = pos0 + q0 + lc;                            // its position
  const int wave_qmax = pos0 + min(q0 + 31, Lq - 1);
  const int blk_qmax = pos0 + min(qt * BQ + BQ - 1, Lq - 1);
  const float sl2 = a.scale_log2;

  // Q^T fragments with the softmax scale (in log2 units) folded in
  bf16x8 qf[QS];
  {
    const bf16 *qrow = (const bf16 *)a.q + ((tok0q + min(q0 + lc, Lq - 1)) * NH + h) * (DN + DR) + hh * 8;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      const bf16x8 x = *(const bf16x8 *)(qrow + s * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = (bf16)((float)x[e] * sl2);
    }
  }
  // One more (short) k-step subtracts the reference: K side all ones in k
  // slot 0, Q side -mref (a bf16 value, so the subtraction is exact).
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  s16x4 kone = {0, 0, 0, 0}, qref = {0, 0, 0, 0};
  if (hh == 0) kone[0] = (short)0x3f80;
  f32x16 oacc[DVB];
  float lrun = 0.f;
  bool bad = false;
  // pass 0: the lane's largest score relative to the reference (the row's
  // maximum minus the reference, once the lane pair is combined)
  float smax = -INFINITY, mref0 = 0.f;

  // Copies.  Stage layout (bytes): K_C rows of 256 at 0, k_R rows of 128 at
  // 16384, V^T rows of 128 at 24576; chunk c of row r sits at position
  // c ^ (r & 15) (K_C) or c ^ ((r >> 1) & 7) (k_R, V^T).
  const unsigned lds0 = (unsigned)(size_t)(lds_void_t *)stages;
  auto issue = [&](int t) {
    const int kvb = t * KVT;
    const unsigned dst = lds0 + (unsigned)((t % NS) * STAGE * 2) + wave * 1024;
    const char *kn = (const char *)((const bf16 *)a.k + ((tok0 + kvb) * NH + h) * DN);
    const char *kr = (const char *)((const bf16 *)a.kr + (tok0 + kvb) * DR);
    const char *vt = (const char *)((const bf16 *)a.vt + (long)h * DV * ntok + tok0 + kvb);
    // rows past the end repeat the last key, V^T chunks past the end repeat
    // the last 8 keys (their probabilities are 0)
    const int last = min(KVT, L - kvb) - 1;
    const int vlast = min(KVT, L - kvb) - 8;
#pragma unroll
    for (int i = 0; i < LKN; ++i) {
      const int sl = i * NT + tid, r = sl >> 4, c = (sl & 15) ^ (r & 15);
      fp_dma16(kn, (unsigned)(min(swap23(r), last) * NH * DN + c * 8) * 2u, dst + i * NT * 16);
    }
#pragma unroll
    for (int i = 0; i < LKR; ++i) {
      const int sl = i * NT + tid, r = sl >> 3, c = (sl & 7) ^ ((r >> 1) & 7);
      fp_dma16(kr, (unsigned)(min(swap23(r), last) * DR + c * 8) * 2u, dst + KN_E * 2 + i * NT * 16);
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int sl = i * NT + tid, d = sl >> 3, c = (sl & 7) ^ ((d >> 1) & 7);
      fp_dma16(vt, (unsigned)((long)d * ntok + min(c * 8, vlast)) * 2u, dst + (KN_E + KR_E) * 2 + i * NT * 16);
    }
  };

  // Fragment reads.  With the stage offset so, the K_C fragment of k-step s
  // (chunk 2s + h) for key row kb*32 + lc is at ((so + lk) ^ 32s) + 8192kb,
  // the k_R one of step 8 + s at ((so + lr) ^ 32s) + 4096kb, and the V^T
  // fragment of P.V step (kb, m) for rows db*32 + lc at ((so + lv) ^ (64kb +
  // 32m)) + 4096db: the XOR only touches the chunk bits of the row.
  const lds_char *lbase = (const lds_char *)stages;
  const unsigned lk = lc * 256 + ((unsigned)(hh ^ (lc & 15)) << 4);
  const unsigned lr = 16384 + lc * 128 + ((unsigned)(hh ^ ((lc >> 1) & 7)) << 4);
  const unsigned lv = 24576 + lc * 128 + ((unsigned)(hh ^ ((lc >> 1) & 7)) << 4);
  auto kfrag = [&](unsigned so, int s, int kb) {
    if (s < DN / 16) return *(const lds_frag *)(lbase + (((so + lk) ^ (32u * s)) + 8192u * kb));
    return *(const lds_frag *)(lbase + (((so + lr) ^ (32u * (s - DN / 16))) + 4096u * kb));
  };
  auto vfrag = [&](unsigned so, int i) {
    const int kb = i / (2 * DVB), m = (i / DVB) & 1, db = i % DVB;
    return *(const lds_frag *)(lbase + (((so + lv) ^ (64u * kb + 32u * m)) + 4096u * db));
  };

  // S^T of tile t minus the reference, in log2 units: two accumulators (the
  // two 32-key halves), K fragments read two k-steps ahead.
  f32x16 sacc[2];
  auto scores = [&](int t) {
    const unsigned so = (unsigned)((t % NS) * STAGE * 2);
    bf16x8 kf[3][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[i][kb] = kfrag(so, i, kb);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(kone, qref, sacc[kb], 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      if (s + 2 < QS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kf[(s + 2) % 3][kb] = kfrag(so, s + 2, kb);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % 3][kb], qf[s], sacc[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // softmax of tile t (scores in sacc) and O^T += V^T . P^T
  auto softmax_pv = [&](int t, int pass) {
    const int kvb = t * KVT;
    const unsigned so = (unsigned)((t % NS) * STAGE * 2);
    // V^T fragments of the P.V steps, in order (kb, m, db); the first ones
    // are read before the softmax
    constexpr int PVN = 2 * 2 * DVB, VPF = 4;
    bf16x8 vf[VPF + 1];
#pragma unroll
    for (int i = 0; i < VPF; ++i) vf[i] = vfrag(so, i);
    __builtin_amdgcn_sched_barrier(0);

    // sacc[kb][4j + i] is key kvb + 32kb + 16(j/2) + 8h + 4(j%2) + i
    if (kvb + KVT - 1 > pos0 + q0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = e >> 2, i = e & 3;
          const int kv = kvb + 32 * kb + 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + i;
          if (kv > qpos) sacc[kb][e] = -INFINITY;
        }
    }
    // The reference is fixed on the first tile: its row maximum, rounded up
    // to a bf16 value.  Later probabilities may exceed 1; a row whose lane
    // sums pass 2^40 (or overflow) sends the workgroup through pass 1, whose
    // reference is the row's maximum (set before the first tile).
    if (t == 0 && pass == 0) {
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      unsigned uu = __float_as_uint(mx);
      uu = (uu & 0x80000000u) ? (uu & 0xffff0000u) : ((uu + 0xffffu) & 0xffff0000u);
      const float mref = __uint_as_float(uu);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] -= mref;
      if (hh == 0) qref[0] = (short)(__float_as_uint(-mref) >> 16);
      mref0 = mref;
    }
    if (pass == 0) {
      float tm = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) tm = fmaxf(tm, sacc[kb][e]);
      smax = fmaxf(smax, tm);
    }
    bf16x8 pf[2][2];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)__builtin_amdgcn_exp2f(sacc[kb][8 * m + e]);
        pf[kb][m] = f;
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          ps[e / 2] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[e], f[e + 1]}, bf16x2{(bf16)1.f, (bf16)1.f}, ps[e / 2], false);
      }
    const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    bad |= !(psum <= 0x1p40f);
    lrun += psum;

    // keys 32kb + 16m + 8h .. +7
#pragma unroll
    for (int i = 0; i < PVN; ++i) {
      if (i + VPF < PVN) vf[(i + VPF) % (VPF + 1)] = vfrag(so, i + VPF);
      const int kb = i / (2 * DVB), m = (i / DVB) & 1, db = i % DVB;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % (VPF + 1)], pf[kb][m], oacc[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Copies run NS-1 tiles ahead of the tile read.
  const int ntiles = blk_qmax / KVT + 1;
  const int wtiles = wave_qmax / KVT + 1;   // tiles with a key at or before one of this wave's queries
  // returns true when pass 0 found a row that outgrew its reference (the
  // workgroup then runs pass 1; nothing of pass 0 is stored)
  auto run = [&](const int pass) -> bool {
#pragma unroll
  for (int i = 0; i < DVB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  lrun = 0.f;
  bad = false;
  fp_wait_vm<0>();   // queries in registers before the copies start
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < ntiles) issue(i);
  for (int t = 0; t < ntiles; ++t) {
    // tile t landed for every wave (the next NS-2 may stay in flight);
    // every LDS read of iteration t-1 done
    const int ahead = min(ntiles - 1 - t, NS - 2);
    if (ahead >= 2) fp_wait_vm_lgkm<2 * LOADS>();
    else if (ahead == 1) fp_wait_vm_lgkm<LOADS>();
    else fp_wait_vm_lgkm<0>();
    fp_bar();
    if (t + NS - 1 < ntiles) issue(t + NS - 1);
    if (t < wtiles) {
      scores(t);
      softmax_pv(t, pass);
    }
  }
  if (pass == 0) {
    // one bit per wave in the last stage (every copy has landed and, past
    // this barrier, every read of the stages is done; the next pass writes
    // that stage only after its first barrier)
    fp_bar();
    volatile int *wbad = (volatile int *)(stages + (NS - 1) * STAGE);
    const bool any_bad = __any(bad);
    if (lane == 0) wbad[wave] = any_bad ? 1 : 0;
    fp_wait_vm_lgkm<0>();
    fp_bar();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) redo |= wbad[w];
    if (redo) {
      // pass 1's reference: the row's maximum, rounded up to a bf16 value
      const float m = mref0 + fmaxf(smax, __shfl_xor(smax, 32));
      unsigned uu = __float_as_uint(m);
      uu = (uu & 0x80000000u) ? (uu & 0xffff0000u) : ((uu + 0xffffu) & 0xffff0000u);
      if (hh == 0) qref[0] = (short)(__float_as_uint(-__uint_as_float(uu)) >> 16);
      return true;
    }
  }

  const float l = lrun + __shfl_xor(lrun, 32);
  if (q0 + lc < Lq) {
    const float inv = 1.f / l;
    bf16 *orow = (bf16 *)a.o + ((tok0q + q0 + lc) * NH + h) * DV;
#pragma unroll
    for (int db = 0; db < DVB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v[4] = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv, oacc[db][4 * j + 2] * inv,
                      oacc[db][4 * j + 3] * inv};
        store4<bf16>(orow, db * 32 + 8 * j + 4 * hh, v, 0);
      }
  }
  return false;
  };
  if (run(0)) run(1);
}

template <typename T, int QB, int NW, int DN, int DR, int DV>
static hipError_t launch_fp(const FlashArgs &a, hipStream_t st) {
  const int qtiles = (a.L + 16 * QB * NW - 1) / (16 * QB * NW);
  const long grid = (long)qtiles * a.B * a.n_h;
  timing_before("flash_prefill", st);
  hipLaunchKernelGGL((flash_prefill_kernel<T, QB, NW, DN, DR, DV>), dim3((unsigned)grid), dim3(64 * NW), 0, st, a);
  timing_after("flash_prefill", st);
  return hipGetLastError();
}

// A cached prefix as dense rows for the up-projections and the flash kernel:
// rows 0..Lpad-1 of every sequence, c_KV into ckv [B*Lpad][d_c] and k_R into
// kr [B*Lpad][d_rope] (bf16).  Rows at or past the sequence's length
// (clamped to the cache's capacity) are zero, so that the keys the flash
// kernel masks out still hold finite values.  One wave per row.
__global__ __launch_bounds__(256) void prefix_gather_kernel(CacheRef c, const int *lens, int B, int Lpad, int d_c,
                                                            int d_rope, bf16 *ckv, bf16 *kr) {
  const int lane = threadIdx.x & 63;
  const long g = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nr = Lpad;
  if (g >= (long)B * nr) return;
  const int b = (int)(g / nr), r = (int)(g - (long)b * nr);
  const int len = (int)min((long)max(lens[b], 0), min((long)Lpad, c.cap));
  const int nch = d_c / 8, rch = d_rope / 8;   // 16-byte chunks
  bf16 *dc = ckv + g * d_c, *dr = kr + g * d_rope;
  if (r < len) {
    const bf16 *row = (const bf16 *)c.pool + cache_row(c, b, r) * c.d_row;
    for (int i = lane; i < nch + rch; i += 64) {
      const bf16x8 v = *(const bf16x8 *)(row + 8 * i);
      if (i < nch) *(bf16x8 *)(dc + 8 * i) = v;
      else *(bf16x8 *)(dr + 8 * (i - nch)) = v;
    }
  } else {
    const bf16x8 z = {};
    for (int i = lane; i < nch + rch; i += 64) {
      if (i < nch) *(bf16x8 *)(dc + 8 * i) = z;
      else *(bf16x8 *)(dr + 8 * (i - nch)) = z;
    }
  }
}

hipError_t launch_prefix_gather(const CacheRef &c, const int *lens, int B, int Lpad, int d_c, int d_rope, void *ckv,
                                void *kr, hipStream_t st) {
  if (c.fp8 || d_c % 8 || d_rope % 8) return hipErrorNotSupported;
  const long rows = (long)B * Lpad;
  if ((rows + 3) / 4 > 0x7fffffffL) return hipErrorInvalidValue;
  timing_before("prefix_gather", st);
  hipLaunchKernelGGL(prefix_gather_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, c, lens, B, Lpad, d_c,
                     d_rope, (bf16 *)ckv, (bf16 *)kr);
  timing_after("prefix_gather", st);
  return hipGetLastError();
}

bool flash_prefix_supported(int dtype, int d_nope, int d_rope, int d_v) {
  return dtype == 1 && d_nope == 128 && d_rope == 64 && d_v == 128;
}

hipError_t launch_flash_prefill(int dtype, const FlashArgs &a, hipStream_t st) {
  const bool m32 = dtype == 1 && a.d_nope == 128 && a.d_rope == 64 && a.d_v == 128 && a.L % 8 == 0 && a.L >= 8 &&
                   (long)a.B * a.L * 2 * 128 < (1L << 31) && (long)a.n_h * 128 * 64 * 2 < (1L << 31);
  // queries after a prefix: the 32x32 kernel only
  if (a.lens && (!m32 || a.Lq < 1 || a.Lq > a.L)) return hipErrorNotSupported;
  if (m32) {
    constexpr int NW = 8;
    const int qtiles = ((a.lens ? a.Lq : a.L) + 32 * NW - 1) / (32 * NW);
    const long grid = (long)qtiles * a.B * a.n_h;
    timing_before("flash_prefill", st);
    hipLaunchKernelGGL((flash_prefill_m32_kernel<NW>), dim3((unsigned)grid), dim3(64 * NW), 0, st, a);
    timing_after("flash_prefill", st);
    return hipGetLastError();
  }
  if (dtype == 1 && a.d_nope == 128 && a.d_rope == 64 && a.d_v == 128) return launch_fp<bf16, FLASH_QB, FLASH_NW, 128, 64, 128>(a, st);
  if (dtype == 0 && a.d_nope == 32 && a.d_rope == 16 && a.d_v == 32) return launch_fp<float, 1, 4, 32, 16, 32>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace mla
