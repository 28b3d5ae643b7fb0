// Causal MLA prefill attention, flash-style (tiled, exact online softmax),
// in the up-projected form of section 2.1 of the DeepSeek-V3 paper-reading
// notes: for head i, q = [q_C,i ; q_R,i] against k = [k_C,j,i ; k_R,j] (k_R
// shared by all heads), values v_j,i, scale 1/sqrt(d_h + d_R).
//
// One workgroup = (sequence, head, 64*QB queries); four waves of 16*QB
// queries each walk the 64-key tiles up to the diagonal.  Scores are formed
// transposed (S^T = K . Q^T) so that each lane owns one query column: the
// softmax max/sum are lane-local plus two shuffles, and after permuting the
// key rows of the A operand the probabilities are already the B operand of
// O^T += V^T . P^T.  V arrives transposed ([n_h*d_v][tokens], written that
// way by the V up-projection), so both contractions read 16-byte runs from
// LDS.  Tiles start from the longest query blocks (causal work imbalance).
#include "mla_internal.h"

namespace mla {

template <typename T, int QB, int DN, int DR, int DV>
__global__ __launch_bounds__(256, 1) void flash_prefill_kernel(FlashArgs a) {
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
  constexpr int BQ = 64 * QB;
  static_assert(RUNQ % KPL == 0 && PRUN % KPL == 0, "");
  static_assert(DN % VE == 0 && DR % VE == 0 && KVT % VE == 0, "");
  constexpr int KCH = KVT * (DQK / VE);
  constexpr int VCH = DV * (KVT / VE);
  constexpr int KPT = (KCH + 255) / 256;
  constexpr int VPT = (VCH + 255) / 256;
  typedef typename Mma<T>::frag frag;

  __shared__ __attribute__((aligned(16))) T ks[KVT * LDK];
  __shared__ __attribute__((aligned(16))) T vs[DV * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int L = a.L, NH = a.n_h;
  const int qtiles = (L + BQ - 1) / BQ;

  // block -> (query tile, longest first; sequence; head).  Heads that share
  // bid % 8 land on one XCD, so a head's K/V tiles stay in one L2.
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
  float mrun[QB], lrun[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) { mrun[j] = -1e30f; lrun[j] = 0.f; }

  const T *Kn = (const T *)a.k;
  const T *Kr = (const T *)a.kr;
  const T *Vt = (const T *)a.vt;
  u32x4 kr_[KPT], vr_[VPT];
  auto gload = [&](int kvb) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * 256;
      if (c < KCH) {
        const int r = c / (DQK / VE), cc = (c % (DQK / VE)) * VE;
        const long tok = tok0 + min(kvb + r, L - 1);
        const T *src = cc < DN ? Kn + (tok * NH + h) * DN + cc : Kr + tok * DR + (cc - DN);
        kr_[i] = *(const u32x4 *)src;
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * 256;
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
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * 256;
      if (c < KCH) {
        const int r = c / (DQK / VE), cc = (c % (DQK / VE)) * VE;
        *(u32x4 *)&ks[r * LDK + cc] = kr_[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * 256;
      if (c < VCH) {
        const int d = c / (KVT / VE), kc = (c % (KVT / VE)) * VE;
        *(u32x4 *)&vs[d * LDV + kc] = vr_[i];
      }
    }
  };

  const int ntiles = blk_qmax / KVT + 1;
  const int kvl0 = 4 * KVB * (lrow >> 2) + (lrow & 3);   // permuted key row of this A slot
  gload(0);
  for (int t = 0; t < ntiles; ++t) {
    const int kvb = t * KVT;
    __syncthreads();
    lstore();
    __syncthreads();
    if (t + 1 < ntiles) gload(kvb + KVT);
    if (kvb > wave_qmax) continue;   // every key of this tile is after every query of this wave

    f32x4 sacc[KVB][QB];
#pragma unroll
    for (int kb = 0; kb < KVB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < QS; ++s) {
#pragma unroll
      for (int kb = 0; kb < KVB; ++kb) {
        const frag ka = *(const frag *)&ks[(kvl0 + 4 * kb) * LDK + lgrp * RUNQ + s * KPL];
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
          const int kv = kvb + 4 * KVB * lgrp + 4 * kb + i;
          float x = sacc[kb][qb][i] * sl2;
          if (diag && kv > qpos) x = -INFINITY;
          sv[kb][i] = x;
          mt = fmaxf(mt, x);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mnew = fmaxf(mrun[qb], mt);
      const float alpha = exp2f(mrun[qb] - mnew);
      mrun[qb] = mnew;
      float psum = 0.f;
      float p[KVB][4];
#pragma unroll
      for (int kb = 0; kb < KVB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = exp2f(sv[kb][i] - mnew);
          psum += p[kb][i];
        }
      lrun[qb] = lrun[qb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DVB; ++db) oacc[db][qb] *= alpha;
      // lane-group run of 16 keys: slot j <-> key block j/4, row j%4
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

#pragma unroll
    for (int ps = 0; ps < PS; ++ps)
#pragma unroll
      for (int db = 0; db < DVB; ++db) {
        const frag va = *(const frag *)&vs[(db * 16 + lrow) * LDV + lgrp * PRUN + ps * KPL];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = Mma<T>::mma(va, pf[qb][ps], oacc[db][qb]);
      }
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

template <typename T, int QB, int DN, int DR, int DV>
static hipError_t launch_fp(const FlashArgs &a, hipStream_t st) {
  const int qtiles = (a.L + 64 * QB - 1) / (64 * QB);
  const long grid = (long)qtiles * a.B * a.n_h;
  timing_before("flash_prefill", st);
  hipLaunchKernelGGL((flash_prefill_kernel<T, QB, DN, DR, DV>), dim3((unsigned)grid), dim3(256), 0, st, a);
  timing_after("flash_prefill", st);
  return hipGetLastError();
}

hipError_t launch_flash_prefill(int dtype, const FlashArgs &a, hipStream_t st) {
  if (dtype == 1 && a.d_nope == 128 && a.d_rope == 64 && a.d_v == 128) return launch_fp<bf16, 4, 128, 64, 128>(a, st);
  if (dtype == 0 && a.d_nope == 32 && a.d_rope == 16 && a.d_v == 32) return launch_fp<float, 1, 32, 16, 32>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace mla
