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
//   1. c_Q (32 x 1536, 96 KB) is copied HBM -> LDS once; W_UQ,i and half of
//      W_QR,i stream from HBM straight into MFMA A-operand registers (six
//      256-wide k stages, three in flight).  Waves 0..3 compute 32 features
//      of q_C,i each; wave 4 the 32 RoPE features 32hf.. (RoPE and the store
//      go through the shared GEMM epilogue, so the values are those of the
//      separate up-projection).  Both halves compute all of q_C,i: the
//      absorption contracts over it; the second read of W_UQ,i hits L2 (the
//      two halves of a head share an XCD).
//   2. q_C,i, rounded to bf16 as a stored q_C would be, replaces c_Q in LDS;
//      W_UK,i[:, 256hf..+256] (64 KB, copied to LDS during step 1) is read
//      transposed (ds_read_b64_tr_b16) as the A operand of
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

constexpr int DQ = 1536, DN = 128, DRP = 64, DCL = 512;
constexpr int TQ = 32;                 // tokens (two 16-row MFMA blocks)
constexpr int BK = 256, NST = DQ / BK; // k stages of the up-projection
constexpr int AH = 2;                  // stages in flight beyond the current one
constexpr int STEPS = BK / 32;
constexpr int XCH = DQ / 8;            // 16-byte chunks per c_Q row (192)
constexpr int KCH = 256 / 8;           // chunks per row of the W_UK half (32)
constexpr int XLOADS = TQ * XCH / 256; // copy instructions per copying wave
constexpr int KLOADS = DN * KCH / 256;

}  // namespace

__global__ __launch_bounds__(320, 1) void decode_q_kernel(DecodeQArgs a) {
  static_assert(TQ * XCH % 256 == 0 && DN * KCH % 256 == 0 && XLOADS + 2 * 2 * STEPS < 64, "");
  // c_Q [32][1536] (chunk c of row t at c ^ (t & 15)), later q_C [32][128]
  __shared__ __attribute__((aligned(16))) bf16 xs[TQ * DQ];
  // W_UK,i[f][256hf + 8c..] at chunk c ^ (f & 15) of row f
  __shared__ __attribute__((aligned(16))) bf16 wk[DN * 256];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int h = (slot >> 1) * 8 + xcd, hf = slot & 1;
  if (h >= a.n_h) return;
  const int T = a.T;
  const unsigned lxs = (unsigned)(size_t)(lds_void *)xs, lwk = (unsigned)(size_t)(lds_void *)wk;

  // c_Q -> LDS (waves 0..3); rows past the last token repeat it
  if (wave < 4) {
#pragma unroll
    for (int j = 0; j < XLOADS; ++j) {
      const int s = j * 256 + tid, r = s / XCH, p = s - r * XCH;
      const int c = p ^ (r & 15);
      dma16(a.cq, (unsigned)((min(r, T - 1) * DQ + c * 8) * 2), lxs + (unsigned)(j * 256 + wave * 64) * 16);
    }
  }

  // weight rows of this lane: two 16-row blocks
  const bf16 *wrow[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
    wrow[blk] = wave < 4 ? a.w_uq + ((long)h * DN + wave * 32 + blk * 16 + lrow) * DQ + lgrp * 8
                         : a.w_qr + ((long)h * DRP + hf * 32 + blk * 16 + lrow) * DQ + lgrp * 8;
  bf16x8 wr[AH + 1][2][STEPS];
  auto wload = [&](int st) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s = 0; s < STEPS; ++s) wr[st % (AH + 1)][blk][s] = *(const bf16x8 *)(wrow[blk] + st * BK + s * 32);
  };
#pragma unroll
  for (int st = 0; st < AH; ++st) wload(st);

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  wait_vm<2 * 2 * STEPS>();   // c_Q copies landed (the weight stages may not have)
  bar();

  const lds_bf16 *xl = (const lds_bf16 *)xs;
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    // the scheduler must not sink the next stage's loads below this stage's
    // MFMAs (it does, to save registers, and the pipe then drains)
    if (st + AH < NST) wload(st + AH);
    __builtin_amdgcn_sched_barrier(0);
    if (st == 3 && wave < 4) {
      // W_UK,i half -> LDS, now that every weight load has been issued
      const char *src = (const char *)(a.w_uk + (long)h * DN * DCL + hf * 256);
#pragma unroll
      for (int j = 0; j < KLOADS; ++j) {
        const int s = j * 256 + tid, f = s / KCH, p = s - f * KCH;
        const int c = p ^ (f & 15);
        dma16(src, (unsigned)((f * DCL + c * 8) * 2), lwk + (unsigned)(j * 256 + wave * 64) * 16);
      }
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int c = st * (BK / 8) + 4 * s + lgrp;
      bf16x8 xb[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) xb[tb] = *(const lds_bf16x8 *)(xl + (tb * 16 + lrow) * DQ + (c ^ lrow) * 8);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[blk][tb] = Mma<bf16>::mma(wr[st % (AH + 1)][blk][s], xb[tb], acc[blk][tb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  __syncthreads();   // c_Q no longer read
  lds_bf16 *ql = (lds_bf16 *)xs;
  if (wave < 4) {
    // q_C features wave*32 + blk*16 + 4*lgrp + i of token tb*16 + lrow, as bf16
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int t = tb * 16 + lrow;
        const int c = wave * 4 + blk * 2 + (lgrp >> 1);
        *(lds_bf16x4 *)(ql + t * DN + (c ^ lrow) * 8 + (lgrp & 1) * 4) =
            bf16x4{(bf16)acc[blk][tb][0], (bf16)acc[blk][tb][1], (bf16)acc[blk][tb][2], (bf16)acc[blk][tb][3]};
      }
  } else {
    // RoPE features: columns of the up-projection's output space
    const int n0 = a.n_h * DN + h * DRP + hf * 32 + 4 * lgrp;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int t = tb * 16 + lrow;
        if (t < T) {
          float v[4] = {acc[blk][tb][0], acc[blk][tb][1], acc[blk][tb][2], acc[blk][tb][3]};
          epi_store4<bf16>(a.epi, 0, t, n0 + blk * 16, v);
        }
      }
  }
  wait_vm<0>();      // this wave's W_UK copies
  __syncthreads();
  if (wave >= 4) return;

  // q_lat[t][256hf + d] for the wave's 64 latent columns: 4 blocks of 16
  const lds_bf16 *kl = (const lds_bf16 *)wk;
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
  hipLaunchKernelGGL(decode_q_kernel, dim3(grid), dim3(320), 0, st, a);
  timing_after("q_up_absorb", st);
  return hipGetLastError();
}

}  // namespace mla
