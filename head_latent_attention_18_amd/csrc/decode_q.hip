// Decode query path in one launch: the query up-projection with RoPE and the
// absorption of W_UK into the query (bf16; d_cq = 1536, d_nope = 128,
// d_R = 64, d_c = 512; up to 32 tokens).
//
//   q_C,i = W_UQ,i c_Q          (128 features of head i)
//   q_R,i = RoPE(W_QR,i c_Q)    (64 features, pairs (2k, 2k+1))
//   q_lat,i = W_UK,i^T q_C,i    (512 latent columns)
//
// (DeepSeek-V3 paper-reading notes, section 2.1: "Query compression" and the
// absorption of W_UK into the query for attention over the latent cache.)
// Split in two launches, q_C would go to HBM and back and the absorption
// would pay its own ramp; here workgroup (head i, half hf) keeps everything
// on chip:
//   1. c_Q (32 x 1536, 96 KB) is copied HBM -> LDS once.  The 160 weight
//      rows the workgroup needs (W_UQ,i and half of W_QR,i) go HBM -> LDS as
//      stages of 16 rows x 512 k, one 1 KB run per row per copy instruction,
//      through a four-slot ring; the four waves split the k steps of every
//      stage and add their partial sums through LDS at the end.  Both halves
//      compute all of q_C,i (the absorption contracts over it); the second
//      read of W_UQ,i hits L2 (the two halves of a head share an XCD).  The
//      RoPE features 32hf.. are rotated with the same fp64-reduced angles as
//      the GEMM epilogue (positions and frequencies fetched at the start).
//   2. q_C,i, rounded to bf16 as a stored q_C would be, replaces the partial
//      sums in LDS; W_UK,i[:, 256hf..+256] (64 KB, copied into the freed ring
//      slots) is read transposed (ds_read_b64_tr_b16) as the A operand of
//      q_lat^T[d][t] = W_UK^T[d][f] q_C^T[f][t].
#include "mla_internal.h"

namespace mla {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes per lane HBM -> LDS (lane i lands at lds + 16*i); the kernel waits
// for its copies itself (vmcnt, then a barrier)
__device__ inline void dma16(const void *gbase, unsigned off, unsigned lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(gbase)
      : "memory", "m0");
}

__device__ inline void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4)); }

constexpr int DQ = 1536, DN = 128, DRP = 64, DCL = 512;
constexpr int TQ = 32;                   // tokens (two 16-row MFMA blocks)
constexpr int ROWS = DN + 32;            // weight rows per workgroup: q_C (128) and half of q_R (32)
constexpr int RB = ROWS / 16;            // 16-row blocks (10)
constexpr int SKW = 512;                 // k per stage: a 1 KB run of every weight row
constexpr int KC = DQ / SKW;             // k chunks (3)
constexpr int NSTG = RB * KC;            // stages (30)
constexpr int SCH = SKW / 8;             // 16-byte chunks per stage row (64)
constexpr int SLOADS = 16 * SCH / 256;   // copy instructions per wave per stage (4)
constexpr int RING = 4;                  // ring stages (three ahead)
constexpr int XCH = DQ / 8;              // chunks per c_Q row (192)
constexpr int XLOADS = TQ * XCH / 256;   // copy instructions per wave for c_Q (24)
constexpr int KCH = 256 / 8;             // chunks per row of the W_UK half (32)

}  // namespace

__global__ __launch_bounds__(256, 1) void decode_q_kernel(DecodeQArgs a) {
  static_assert(16 * SCH % 256 == 0 && TQ * XCH % 256 == 0 && 32 * KCH / 256 == SLOADS, "");
  static_assert(XLOADS + 3 * SLOADS < 64 && RING * 16 * SKW == DN * 256, "");
  static_assert(4 * RB * 2 * 64 * 16 + TQ * DN * 2 <= TQ * DQ * 2, "");
  // region A: c_Q [32][1536] (chunk c of token t at c ^ (t & 15)); after the
  // up-projection, the waves' partial sums and then q_C [32][128] (bf16)
  __shared__ __attribute__((aligned(16))) bf16 xs[TQ * DQ];
  // region B: the ring of weight stages ([16][512], chunk c of row r at
  // c ^ r); afterwards W_UK,i[f][256hf + 8c..] at chunk c ^ (f & 15) of row f
  __shared__ __attribute__((aligned(16))) bf16 ring[RING * 16 * SKW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int h = (slot >> 1) * 8 + xcd, hf = slot & 1;
  if (h >= a.n_h) return;
  const int T = a.T;
  const unsigned lxs = (unsigned)(size_t)(lds_void *)xs, lring = (unsigned)(size_t)(lds_void *)ring;

  // c_Q -> region A; rows past the last token repeat it
#pragma unroll
  for (int j = 0; j < XLOADS; ++j) {
    const int sl = j * 256 + tid, r = sl / XCH, p = sl - r * XCH;
    const int c = p ^ (r & 15);
    dma16(a.cq, (unsigned)((min(r, T - 1) * DQ + c * 8) * 2), lxs + (unsigned)sl * 16);
  }
  // stage s = (row block s / KC, k chunk s % KC) -> ring slot s % RING: each
  // wave instruction copies one whole 1 KB run of one row
  auto issue_stage = [&](int st) {
    const int rb = st / KC, j = st % KC;
    const bf16 *base = rb < DN / 16 ? a.w_uq + ((long)h * DN + rb * 16) * DQ
                                    : a.w_qr + ((long)h * DRP + hf * 32 + (rb - DN / 16) * 16) * DQ;
    base += j * SKW;
#pragma unroll
    for (int i = 0; i < SLOADS; ++i) {
      const int sl = i * 256 + tid, r = sl / SCH, p = sl - r * SCH;
      dma16(base, (unsigned)((r * DQ + ((p ^ r) << 3)) * 2),
            lring + (unsigned)((st % RING) * 16 * SKW * 2 + sl * 16));
    }
  };
  // quarter q of the W_UK half (rows 32q..32q+31) -> ring slot q
  auto issue_wuk = [&](int q) {
    const bf16 *base = a.w_uk + ((long)h * DN + 32 * q) * DCL + hf * 256;
#pragma unroll
    for (int i = 0; i < SLOADS; ++i) {
      const int sl = i * 256 + tid, fl = sl / KCH, p = sl - fl * KCH;
      const int f = 32 * q + fl;
      dma16(base, (unsigned)((fl * DCL + ((p ^ (f & 15)) << 3)) * 2), lring + (unsigned)((q * 1024 + sl) * 16));
    }
  };
#pragma unroll
  for (int st = 0; st < RING - 1; ++st) issue_stage(st);

  // RoPE inputs of the lane's rows, fetched now so that the epilogue waits
  // for no load chain: positions of tokens lrow and 16 + lrow (decode rows:
  // the last n_q positions of each sequence) and the frequencies of its
  // pairs in RoPE blocks 0 and 1 (features 32hf + 16blk + 4lgrp..)
  int rpos[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = min(tb * 16 + lrow, T - 1), nq = a.epi.rows.per_seq, sq = t / nq;
    rpos[tb] = a.epi.rows.lens[sq] - nq + (t - sq * nq);
  }
  double rfreq[2][2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) rfreq[blk][pp] = a.epi.inv_freq[hf * 16 + blk * 8 + 2 * lgrp + pp];

  // the wave's partial sums over its k quarter of every stage
  f32x4 acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const lds_bf16 *xl = (const lds_bf16 *)xs;
  const lds_bf16 *rl = (const lds_bf16 *)ring;
#pragma unroll
  for (int st = 0; st < NSTG; ++st) {
    // stage st landed (and, at st = 0, c_Q); the two after it may not have
    wait_vm<2 * SLOADS>();
    bar();   // every wave is done with the slot of stage st-1
    // next copy into that slot: stage st+3, or a quarter of W_UK once the
    // weight stages are all issued (quarters 2, 3, 0 here, 1 after the loop)
    if (st + RING - 1 < NSTG) issue_stage(st + RING - 1);
    else issue_wuk((st + RING - 1) % RING);
    const int rb = st / KC, j = st % KC;
    const lds_bf16 *ws = rl + (st % RING) * 16 * SKW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cw = 16 * wave + 4 * i + lgrp;           // chunk in the stage row
      const int cx = j * SCH + cw;                       // chunk in the c_Q row
      const bf16x8 wf = *(const lds_bf16x8 *)(ws + lrow * SKW + ((cw ^ lrow) << 3));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 xb = *(const lds_bf16x8 *)(xl + (tb * 16 + lrow) * DQ + ((cx ^ lrow) << 3));
        acc[rb][tb] = Mma<bf16>::mma(wf, xb, acc[rb][tb]);
      }
    }
  }
  bar();             // stage 29 (slot 1) and c_Q no longer read
  issue_wuk(1);

  // sum the four waves' partials through region A
  lds_f32x4 *pt = (lds_f32x4 *)xs;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) pt[((wave * RB + rb) * 2 + tb) * 64 + lane] = acc[rb][tb];
  wait_lgkm0();
  bar();
  lds_bf16 *ql = (lds_bf16 *)xs + 4 * RB * 2 * 64 * 8;   // q_C [32][128] after the partials
  for (int q = 0; q < RB * 2 / 4; ++q) {
    const int pr = wave * (RB * 2 / 4) + q, rb = pr >> 1, tb = pr & 1;
    f32x4 v = pt[(rb * 2 + tb) * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += pt[((w * RB + rb) * 2 + tb) * 64 + lane];
    // rows 16rb + 4lgrp + 0..3 of token 16tb + lrow
    const int t = tb * 16 + lrow;
    if (rb < DN / 16) {
      const int c = 2 * rb + (lgrp >> 1);
      *(lds_bf16x4 *)(ql + t * DN + ((c ^ lrow) << 3) + (lgrp & 1) * 4) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    } else if (t < T) {
      // RoPE features 32hf + 16(rb - 8) + 4lgrp.. : pairs (2k, 2k+1) rotated
      // by pos * inv_freq[k], stored after q_lat in the q_abs row
      const int blk = rb - DN / 16;
      float vv[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        float sn, cs;
        rope_sincos(rpos[tb], blk ? rfreq[1][pp] : rfreq[0][pp], sn, cs);
        const float x0 = vv[2 * pp], x1 = vv[2 * pp + 1];
        vv[2 * pp] = x0 * cs - x1 * sn;
        vv[2 * pp + 1] = x0 * sn + x1 * cs;
      }
      *(bf16x4 *)(a.q_abs + ((long)t * a.n_h + h) * (DCL + DRP) + DCL + hf * 32 + blk * 16 + 4 * lgrp) =
          bf16x4{(bf16)vv[0], (bf16)vv[1], (bf16)vv[2], (bf16)vv[3]};
    }
  }
  wait_vm<0>();      // this wave's W_UK copies
  wait_lgkm0();
  bar();

  // q_lat[t][256hf + d] for the wave's 64 latent columns: 4 blocks of 16
  const lds_bf16 *kl = (const lds_bf16 *)ring;
  f32x4 lat[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) lat[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DN / 32; ++ks) {
    bf16x8 qb[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) qb[tb] = *(const lds_bf16x8 *)(ql + (tb * 16 + lrow) * DN + ((4 * ks + lgrp) ^ lrow) * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // W_UK^T fragment: column d = (wave*4 + j)*16 + lrow, f = 32ks + 8lgrp + 0..7,
      // two transposed 4x16 reads
      const int f = 32 * ks + 8 * lgrp + (lrow >> 2);
      const int col = (wave * 4 + j) * 16 + 4 * (lrow & 3);
      const int c = col >> 3, half = col & 7;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(kl + f * 256 + (c ^ (f & 15)) * 8 + half));
      const int f2 = f + 4;
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(kl + f2 * 256 + (c ^ (f2 & 15)) * 8 + half));
      const bf16x8 wf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) lat[j][tb] = Mma<bf16>::mma(wf, qb[tb], lat[j][tb]);
    }
  }
  const long D = DCL + DRP;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = tb * 16 + lrow;
    if (t < T) {
      bf16 *dst = a.q_abs + ((long)t * a.n_h + h) * D + hf * 256 + wave * 64 + 4 * lgrp;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(bf16x4 *)(dst + j * 16) = bf16x4{(bf16)lat[j][tb][0], (bf16)lat[j][tb][1], (bf16)lat[j][tb][2], (bf16)lat[j][tb][3]};
    }
  }
}

bool decode_q_supported(int d_cq, int d_nope, int d_rope, int d_c, int T) {
  return d_cq == DQ && d_nope == DN && d_rope == DRP && d_c == DCL && T >= 1 && T <= TQ;
}

hipError_t launch_decode_q(const DecodeQArgs &a, hipStream_t st) {
  const int grid = ((a.n_h + 7) / 8) * 16;
  timing_before("q_up_absorb", st);
  hipLaunchKernelGGL(decode_q_kernel, dim3(grid), dim3(256), 0, st, a);
  timing_after("q_up_absorb", st);
  return hipGetLastError();
}

}  // namespace mla
