// Large-M GEMM (bf16, prefill): Y[m][n] = sum_k X[m][k] W[n][k] with the
// segment epilogues of the projections (W stored [N][K]).
//
//   * tile 256 tokens x 256 features, k slabs of 64; 8 waves (two per SIMD),
//     each computing a 128-token x 64-feature block of Y^T with 32x32x16
//     MFMAs;
//   * X and W slabs go HBM/L2 -> LDS with global_load_lds_dwordx4 into a
//     two-stage ring (no staging registers), one slab ahead: 64 KB per slab
//     for 8.4 MFLOP, so at the full MFMA rate a CU needs about 66 GB/s from
//     L2, close to what the L2 delivers with this access pattern (about
//     75 GB/s per CU with every CU copying);
//   * bf16 main loop, ping-pong: the two waves of each SIMD alternate a
//     slab's MFMA burst (all fragments in registers) and the LDS reads of
//     their next fragments, turns separated by workgroup barriers; FP8 main
//     loop: every wave reads fragments ahead of its MFMAs;
//   * LDS rows are 8 chunks of 16 bytes with the chunk index XORed by
//     (row >> 1) & 7, so the 16-row fragment reads hit 16 distinct bank groups;
//   * tiles are handed out in GxG groups per XCD (G = 8, 4, 2 or 1, the
//     largest that keeps the XCDs evenly loaded), so the X and W slabs of a
//     group are read from HBM once and reused from that XCD's L2;
//   * the epilogue goes through LDS (fp32, half a tile at a time) and runs as
//     a loop over (token, 4 features) items, so the segment/RoPE/cache
//     epilogue is compiled once instead of once per accumulator; the plain
//     outputs leave by streaming (non-temporal) stores of whole rows, since
//     the next kernel reads them from other XCDs (measured 5-10 us faster
//     per prefill than write-allocating stores);
//   * few tiles (a few hundred tokens against a wide weight): split-K over
//     blockIdx.y, each split writing its fp32 sums for the ordered reduce;
//   * block-scaled FP8 (F8): E4M3 operands, a slab row is the same 128 bytes
//     (128 k instead of 64), each 64-wide k step a scaled 32x32x64 MFMA
//     taking the weight block's power-of-two scale (uniform over a wave's
//     64 features) and each token's as 8-bit exponents; a slab is one 128-k
//     scale block, and its token exponents are loaded with the next slab's
//     copies.
#include <type_traits>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef int i32x8 __attribute__((ext_vector_type(8)));

#ifndef MLA_GEMM_PINGPONG
#define MLA_GEMM_PINGPONG 1
#endif
constexpr bool GEMM_PINGPONG = MLA_GEMM_PINGPONG != 0;
constexpr int GBM = 256, GBN = 256, GBK = 64;   // GBK: bf16 k per slab (FP8: 2 * GBK)
constexpr int GNT = 512;                        // threads (8 waves)
constexpr int GNS = 2;                          // ring stages
constexpr int RCH = GBK / 8;                    // 16-byte chunks per row of a slab (8)
constexpr int XCHK = GBM * RCH;                 // activation chunks per slab (2048)
constexpr int WCHK = GBN * RCH;                 // weight chunks per slab (2048)
constexpr int GLOADS = (XCHK + WCHK) / GNT;     // copy instructions per wave per slab (8)
constexpr int GSTAGE = (XCHK + WCHK) * 8;       // elements per stage (32768 = 64 KB)
constexpr int NSTEP = GBK / 16;                 // MFMA k steps per slab (4)
constexpr int EPI_LD = GBN + 4;                 // fp32 row pitch of the epilogue staging
// feature-major staging of the transposed store: 128 tokens per feature row,
// pitch 136 floats (4 rows apart = 32 banks apart, so the two lane halves of
// a 32x32 accumulator write disjoint banks)
constexpr int EPI_LDT = GBM / 2 + 8;
static_assert(GNT % (GBN / 4) == 0, "");
// LDS: the ring, reused for half a tile of fp32 results in the epilogue
constexpr int cmax(int x, int y) { return x > y ? x : y; }
constexpr int RING_ELEMS = cmax(GNS * GSTAGE, cmax(GBM / 2 * EPI_LD * 2, GBN * EPI_LDT * 2));

template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4)); }

// 16 bytes per lane HBM -> LDS (lane i lands at lds + 16*i).  An asm
// statement: the compiler sees no LDS write to order later reads after; the
// kernel waits for its copies itself (vmcnt, then a barrier).
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

// rows of 8 chunks: XOR by (row >> 1) & 7 spreads 16 consecutive rows over
// 16 distinct 16-byte bank groups
__device__ inline int swz(int row) { return (row >> 1) & 7; }

}  // namespace

template <bool SWAP, bool F8, bool SPLIT_COPY = false>
__global__ __launch_bounds__(GNT, 1) void gemm_big_kernel(GemmArgs a) {
  constexpr int ESZ = F8 ? 1 : 2;               // bytes per operand element
  constexpr int SK = GBK * 2 / ESZ;             // k per slab (128 bytes of each row)
  __shared__ __attribute__((aligned(16))) bf16 ring[RING_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;      // 128-token x 64-feature block of the wave

  // tile of this workgroup: GxG groups of tiles, one group per XCD at a time
  const int G = a.grouped;                      // group side (host-chosen)
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int gi = local / (G * G), ti = local % (G * G);
  const int groups_m = (a.tiles_m + G - 1) / G;
  const int group = gi * 8 + xcd;
  const int tm = (group % groups_m) * G + ti % G;
  const int tn = (group / groups_m) * G + ti / G;
  if (tm >= a.tiles_m || tn >= a.tiles_n) return;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int split = blockIdx.y, kofs = split * a.k_chunk;   // this split's k range

  int seg = 0, beg = 0;
  while (seg < a.nw - 1 && n0 >= a.w_end[seg]) { beg = a.w_end[seg]; ++seg; }
  const char *wsrc = (const char *)a.w[seg] + ((long)(n0 - beg) * a.ldw + kofs) * ESZ;
  const int wrows = min(GBN, a.w_end[seg] - n0);
  const char *xsrc = (const char *)a.x + ((long)m0 * a.ldx + kofs) * ESZ;
  const int xrows = min(GBM, a.M - m0);
  const unsigned lring = (unsigned)(size_t)(lds_void *)ring;

  // per-lane byte offsets of the slab copies (k-independent part); slots
  // 0..XCHK-1 are activation rows, then weight rows, RCH chunks per row
  constexpr int XL = XCHK / GNT;                 // the first XL instructions copy activations
  unsigned coff[GLOADS];
#pragma unroll
  for (int i = 0; i < GLOADS; ++i) {
    const int s = (i < XL ? i : i - XL) * GNT + tid, r = s / RCH, c = (s % RCH) ^ swz(r);
    coff[i] = i < XL ? (unsigned)(min(r, xrows - 1) * a.ldx * ESZ + c * 16)
                     : (unsigned)(min(r, wrows - 1) * a.ldw * ESZ + c * 16);
  }
  auto issue = [&](int kt, int st) {
    const unsigned dst = lring + (unsigned)(st * GSTAGE * 2) + wave * 1024;
    const char *xb = xsrc + kt * SK * ESZ, *wb = wsrc + kt * SK * ESZ;
#pragma unroll
    for (int i = 0; i < GLOADS; ++i) dma16(i < XL ? xb : wb, coff[i], dst + i * GNT * 16);
  };

  f32x16 acc[2][4];   // [feature block][token block]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const lds_bf16 *rl = (const lds_bf16 *)ring;
  // fragment rows of this lane: 32x32x16 operands hold row (lane & 31) and
  // k chunk 2s + (lane >> 5) of the 16-wide step s
  const int fr = lane & 31, fh = lane >> 5;
  bf16x8 wf[3][2], xf[3][4];   // three steps of fragments in flight
  auto rd = [&](int st, int s, int buf) {
    const lds_bf16 *xs = rl + st * GSTAGE;
    const lds_bf16 *ws = xs + XCHK * 8;
    const int c = 2 * s + fh;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int wr = wn * 64 + b * 32 + fr;
      wf[buf][b] = *(const lds_bf16x8 *)(ws + (wr * RCH + (c ^ swz(wr))) * 8);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int xr = wm * 128 + b * 32 + fr;
      xf[buf][b] = *(const lds_bf16x8 *)(xs + (xr * RCH + (c ^ swz(xr))) * 8);
    }
  };
  auto mm = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][i], xf[buf][j], acc[i][j], 0, 0, 0);
  };

  const int nkt = a.k_chunk / SK;
  if constexpr (F8) {
    // fragments of the two 64-wide k steps of a slab: lane group fh holds
    // logical chunks 4s + 2fh and 4s + 2fh + 1 of its row (both operands
    // alike, so the instruction's k order does not matter)
    i32x8 wq[2][2], xq[2][4];
    auto rd8 = [&](int st, int s) {
      const lds_bf16 *xs = rl + st * GSTAGE;
      const lds_bf16 *ws = xs + XCHK * 8;
      const int c = 4 * s + 2 * fh;
      auto frag = [&](const lds_bf16 *base, int r) {
        const lds_u32x4 *row = (const lds_u32x4 *)(base + r * RCH * 8);
        const u32x4 p0 = row[c ^ swz(r)], p1 = row[(c + 1) ^ swz(r)];
        return i32x8{(int)p0[0], (int)p0[1], (int)p0[2], (int)p0[3], (int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3]};
      };
#pragma unroll
      for (int b = 0; b < 2; ++b) wq[s][b] = frag(ws, wn * 64 + b * 32 + fr);
#pragma unroll
      for (int b = 0; b < 4; ++b) xq[s][b] = frag(xs, wm * 128 + b * 32 + fr);
    };
    // the weight block's exponent (uniform over the wave's 64 features) and
    // each of the lane's four tokens' exponent, per 128-k slab
    // (a wave past the segment's last row reads the last block's scales;
    // its rows are never stored)
    const int wblk = min((n0 - beg + wn * 64) >> 7, (a.w_end[seg] - beg - 1) >> 7);
    const float *wsp = a.wsc[seg] + (long)wblk * a.wsc_ld + kofs / 128;
    const unsigned char *xsp = a.xs + (long)(kofs / 128) * a.xs_ld + m0 + wm * 128 + fr;
    int sx[4], sxn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sxn[j] = xsp[j * 32];
    float wsn = wsp[0];   // the next slab's weight scale, loaded a slab ahead
    issue(0, 0);
    for (int kt = 0; kt < nkt; ++kt) {
      wait_vm<0>();     // this wave's copies of slab kt (and its token exponents)
      wait_lgkm0();     // its reads of slab kt-1 are in registers
      bar();            // slab kt landed for every wave; stage (kt+1) % 2 is free
#pragma unroll
      for (int j = 0; j < 4; ++j) sx[j] = sxn[j];
      const int sw = (int)((__builtin_bit_cast(unsigned, wsn) >> 23) & 0xFFu);
      if (kt + 1 < nkt) {
        issue(kt + 1, (kt + 1) % GNS);
#pragma unroll
        for (int j = 0; j < 4; ++j) sxn[j] = xsp[(long)(kt + 1) * a.xs_ld + j * 32];
        wsn = wsp[kt + 1];
      }
      const int st = kt % GNS;
      rd8(st, 0);
      rd8(st, 1);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wq[s][i], xq[s][j], acc[i][j], 0, 0, 0, sw,
                                                                        0, sx[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if constexpr (GEMM_PINGPONG) {
    // Two wave groups take turns on each SIMD (waves w and w+4 share SIMD
    // w): while one group runs a slab's 32 MFMAs from registers, the other
    // reads all of its fragments of that slab from LDS, so every matrix core
    // always has one wave's burst to run.  Group 0 also issues the copies,
    // one slab ahead, into the stage that both groups have finished reading.
    //   interval 2k:   group 0 copies slab k+1 and reads slab k
    //   interval 2k+1: group 0 multiplies slab k and waits for its copies;
    //                  group 1 reads slab k
    //   interval 2k+2: group 1 multiplies slab k
    // Each interval ends at a workgroup barrier; group 1 passes one more
    // barrier before its loop and group 0 one after its loop, so both pass
    // 2 nkt + 2 barriers.
    // SPLIT_COPY (chosen by the launcher when the grid leaves most CUs of
    // each XCD idle): group 1 issues the weight half of slab k+1 at the
    // start of interval 2k+1 instead (into the same free stage) and waits
    // for it before that interval's barrier; measured faster there (fewer
    // CUs share the L2, so a copy lands within the interval), slower when
    // three quarters of the CUs or more are busy.
    const int grp = wave >> 2;
    const int ct = tid & 255;                                 // the lane's slot within its group
    const int tr = ct >> 3;                                   // row of the lane's chunks
    const unsigned cb = (unsigned)(((ct & 7) ^ ((ct >> 4) & 7)) * 16);     // its (swizzled) chunk
    // half h (0: activation rows, 1: weight rows) of slab kt into stage st,
    // by the 256 threads of one group
    auto issue_half = [&](int kt, int st, int h) {
      const unsigned dst = lring + (unsigned)(st * GSTAGE * 2) + (wave & 3) * 1024 + h * XCHK * 16;
      const char *b = (h ? wsrc : xsrc) + kt * SK * ESZ;
      // row pitch in bytes: 256 rows of it stay below 2^31 (checked by the launcher)
      const unsigned ldb = (unsigned)((h ? a.ldw : a.ldx) * ESZ);
      const int rows = h ? wrows : xrows;
#pragma unroll
      for (int i = 0; i < XCHK / 256; ++i)
        dma16(b, (unsigned)min(i * 32 + tr, rows - 1) * ldb + cb, dst + i * 256 * 16);
    };
    static_assert(XCHK == WCHK && XCHK % 256 == 0, "");
    // both halves by group 0
    auto issue_pp = [&](int kt, int st) {
      const unsigned dst = lring + (unsigned)(st * GSTAGE * 2) + wave * 1024;
      const char *xb = xsrc + kt * SK * ESZ, *wb = wsrc + kt * SK * ESZ;
#pragma unroll
      for (int i = 0; i < XCHK / 256; ++i)
        dma16(xb, (unsigned)(min(i * 32 + tr, xrows - 1) * a.ldx * ESZ) + cb, dst + i * 256 * 16);
#pragma unroll
      for (int i = 0; i < WCHK / 256; ++i)
        dma16(wb, (unsigned)(min(i * 32 + tr, wrows - 1) * a.ldw * ESZ) + cb, dst + (XCHK / 256 + i) * 256 * 16);
    };
    bf16x8 pw[NSTEP][2], px[NSTEP][4];
    auto rd_all = [&](int st) {
      const lds_bf16 *xs = rl + st * GSTAGE;
      const lds_bf16 *ws = xs + XCHK * 8;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const int c = 2 * s + fh;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int wr = wn * 64 + b * 32 + fr;
          pw[s][b] = *(const lds_bf16x8 *)(ws + (wr * RCH + (c ^ swz(wr))) * 8);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int xr = wm * 128 + b * 32 + fr;
          px[s][b] = *(const lds_bf16x8 *)(xs + (xr * RCH + (c ^ swz(xr))) * 8);
        }
      }
    };
    auto mm_all = [&]() {
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pw[s][i], px[s][j], acc[i][j], 0, 0, 0);
    };
    if (grp == 0) {
      issue_pp(0, 0);
      wait_vm<0>();
      bar();                                   // slab 0 landed
      for (int kt = 0; kt < nkt; ++kt) {
        if (kt + 1 < nkt) {
          if constexpr (SPLIT_COPY) issue_half(kt + 1, (kt + 1) % GNS, 0);
          else issue_pp(kt + 1, (kt + 1) % GNS);
        }
        rd_all(kt % GNS);
        wait_lgkm0();
        __builtin_amdgcn_sched_barrier(0);
        bar();                                 // end of interval 2kt
        __builtin_amdgcn_sched_barrier(0);
        mm_all();
        __builtin_amdgcn_sched_barrier(0);     // the wait stays behind the burst
        wait_vm<0>();                          // slab kt+1 (this wave's copies)
        __builtin_amdgcn_sched_barrier(0);
        bar();                                 // end of interval 2kt+1
        __builtin_amdgcn_sched_barrier(0);
      }
      bar();                                   // end of interval 2nkt
    } else {
      bar();                                   // slab 0 landed
      bar();                                   // end of interval 0
      for (int kt = 0; kt < nkt; ++kt) {
        if constexpr (SPLIT_COPY) {
          if (kt + 1 < nkt) issue_half(kt + 1, (kt + 1) % GNS, 1);
        }
        rd_all(kt % GNS);
        wait_lgkm0();
        if constexpr (SPLIT_COPY) wait_vm<0>();   // the weight half of slab kt+1
        __builtin_amdgcn_sched_barrier(0);
        bar();                                 // end of interval 2kt+1
        __builtin_amdgcn_sched_barrier(0);
        mm_all();
        __builtin_amdgcn_sched_barrier(0);
        bar();                                 // end of interval 2kt+2
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
  issue(0, 0);
  // slab kt: wait for it, free the other stage for slab kt+1, multiply with
  // the fragments read two steps ahead (ring of three fragment buffers)
  for (int kt = 0; kt < nkt; ++kt) {
    wait_vm<0>();     // this wave's copies of slab kt
    wait_lgkm0();     // its reads of slab kt-1 are in registers
    bar();            // slab kt landed for every wave; stage (kt+1) % 2 is free
    if (kt + 1 < nkt) issue(kt + 1, (kt + 1) % GNS);
    const int st = kt % GNS;
    rd(st, 0, 0);
    rd(st, 1, 1);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if (s + 2 < NSTEP) rd(st, s + 2, (s + 2) % 3);
      mm(s % 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  }

  // Epilogue through LDS, half a tile (128 tokens) at a time: the waves of
  // that half store their accumulators as rows [token][feature] (fp32), then
  // all threads run the epilogue over (token, 4 features) items.
  lds_float *ep = (lds_float *)((lds_void *)ring);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    wait_lgkm0();
    __syncthreads();
    if (wm == half) {
      // acc[i][j]: features wn*64 + 32i + 8q + 4fh + 0..3, token 32j + fr;
      // rows [token][feature] for the row-major store, [feature][token] for
      // the transposed one
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = wn * 64 + i * 32 + 8 * q + 4 * fh, t = j * 32 + fr;
            if constexpr (SWAP) {
              *(lds_f32x4 *)(ep + t * EPI_LD + f) =
                  f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) ep[(f + e) * EPI_LDT + t] = acc[i][j][4 * q + e];
            }
          }
    }
    __syncthreads();
    const int mh = m0 + half * 128;
    if constexpr (SWAP) {
      // a thread always handles the same 4 features (GNT is a multiple of
      // GBN / 4): their column plan is prepared once, outside the row loop
      const int f = (tid % (GBN / 4)) * 4, n = n0 + f;
      constexpr int TS = GNT / (GBN / 4), IT = 128 / TS;   // rows between a thread's items, items
      const int t0 = tid / (GBN / 4);
      if (a.splits > 1) {
        // this split's fp32 sums, [split][M][N] (the reduce adds the splits
        // in order and runs the epilogue)
        if (n < a.N)
          for (int t = t0; t < 128; t += TS)
            if (mh + t < a.M)
              *(f32x4 *)(a.partial + ((long)split * a.M + mh + t) * a.N + n) = *(const lds_f32x4 *)(ep + t * EPI_LD + f);
      } else if (n < a.N) {
        const ColPlan cp = col_plan(a.epi, n);
        if (cp.kind != SEG_CACHE && !cp.dst2 && !cp.out_f32 && (!cp.rope || a.epi.rows.mode == ROWS_DENSE)) {
          // Plain and head-layout columns: all items are formed first and
          // stored afterwards, each store with registers of its own (a store
          // whose source registers are rewritten has to complete first, which
          // would serialise the stores).  Rows advance by TS per item; the
          // RoPE angles turn by TS positions per item (exact at the first row
          // and wherever a new sequence starts).
          bf16 *base = (bf16 *)cp.dst + cp.col;
          int m = mh + t0, seq = 0, pos = 0;
          float sn[2] = {0.f, 0.f}, cs[2] = {1.f, 1.f}, st[2] = {0.f, 0.f}, ct[2] = {1.f, 1.f};
          const int per = a.epi.rows.per_seq;
          if (cp.rope) {
            seq = m / per;
            pos = m - seq * per;
            rope_sincos(pos, cp.inv0, sn[0], cs[0]);
            rope_sincos(pos, cp.inv1, sn[1], cs[1]);
            rope_sincos(TS, cp.inv0, st[0], ct[0]);
            rope_sincos(TS, cp.inv1, st[1], ct[1]);
          }
          bf16x4 ov[IT];
#pragma unroll
          for (int i = 0; i < IT; ++i) {
            const f32x4 v4 = *(const lds_f32x4 *)(ep + (t0 + i * TS) * EPI_LD + f);
            float v[4] = {v4[0], v4[1], v4[2], v4[3]};
            if (cp.rope) {
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                const float x0 = v[2 * q], x1 = v[2 * q + 1];
                v[2 * q] = x0 * cs[q] - x1 * sn[q];
                v[2 * q + 1] = x0 * sn[q] + x1 * cs[q];
              }
              pos += TS;
              if (pos >= per) {
                seq += pos / per;
                pos %= per;
                rope_sincos(pos, cp.inv0, sn[0], cs[0]);
                rope_sincos(pos, cp.inv1, sn[1], cs[1]);
              } else {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                  const float c = cs[q] * ct[q] - sn[q] * st[q];
                  sn[q] = sn[q] * ct[q] + cs[q] * st[q];
                  cs[q] = c;
                }
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[i][e] = (bf16)(v[e] * cp.scale);
          }
#pragma unroll
          for (int i = 0; i < IT; ++i)
            if (m + i * TS < a.M) __builtin_nontemporal_store(ov[i], (bf16x4 *)(base + (long)(m + i * TS) * cp.ld));
        } else {
          for (int t = t0; t < 128; t += TS) {
            const int m = mh + t;
            if (m < a.M) {
              const f32x4 v4 = *(const lds_f32x4 *)(ep + t * EPI_LD + f);
              float v[4] = {v4[0], v4[1], v4[2], v4[3]};
              col_store<bf16>(cp, a.epi, 0, m, v);
            }
          }
        }
      }
    } else {
      // transposed plain store dst[n * ld + m]: items of 8 consecutive
      // tokens of one feature (two 16-byte LDS reads, one 16-byte store;
      // 16 lanes cover a feature's 128 tokens)
      const Seg &g = a.epi.seg[0];
      const bool vec = (g.ld & 7) == 0 && (((size_t)g.dst) & 15) == 0;
      for (int it = tid; it < GBN * (128 / 8); it += GNT) {
        const int f = it / 16, t = (it % 16) * 8;
        const int n = n0 + f, m = mh + t;
        if (n < a.N && m < a.M) {
          bf16 *dst = (bf16 *)g.dst + (long)n * g.ld + m;
          const f32x4 lo = *(const lds_f32x4 *)(ep + f * EPI_LDT + t);
          const f32x4 hi = *(const lds_f32x4 *)(ep + f * EPI_LDT + t + 4);
          if (m + 7 < a.M && vec) {
            __builtin_nontemporal_store(bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
                                               (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]},
                                        (bf16x8 *)dst);
          } else {
            const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (m + e < a.M) dst[e] = (bf16)v[e];
          }
        }
      }
    }
  }
}

hipError_t launch_splitk_reduce_bf16(GemmArgs &a, hipStream_t st);

bool gemm_big_ok(const GemmArgs &a) {
  // any number of tokens (the host sends bf16 products of 96 tokens or
  // more, FP8 ones of more than 128): a tile's surplus rows are clamped
  // copies of its last row and are not stored
  if (a.fp8 ? (a.batch != 1 || a.K % (2 * GBK) != 0 || !a.xs) : (a.batch != 1 || a.K % GBK != 0))
    return false;
  for (int s = 0; s < a.nw - 1; ++s)
    if (a.w_end[s] % GBN != 0) return false;   // a tile never straddles two weight segments
  // 32-bit lane offsets
  const int esz = a.fp8 ? 1 : 2;
  // split-K: whole slabs per split, fp32 partials, row-major outputs only
  if (a.splits > 1 && (a.k_chunk % (2 * GBK) != 0 || (long)a.splits * a.k_chunk != a.K || !a.partial || a.N % 4 ||
                       a.partial_bytes < (size_t)a.splits * a.M * a.N * sizeof(float)))
    return false;
  if ((long)GBM * a.ldx * esz >= (1L << 31) || (long)GBN * a.ldw * esz >= (1L << 31)) return false;
  return true;
}

hipError_t launch_gemm_big(GemmArgs &a, int swap, hipStream_t st) {
  a.tiles_m = (a.M + GBM - 1) / GBM;
  a.tiles_n = (a.N + GBN - 1) / GBN;
  int G = 1, groups = a.tiles_m * a.tiles_n;
  for (int g : {8, 4, 2}) {
    const int n = ((a.tiles_m + g - 1) / g) * ((a.tiles_n + g - 1) / g);
    if (n >= 8 && ((n + 7) / 8) * 8 <= n + n / 20) { G = g; groups = n; break; }
  }
  a.grouped = G;
  const int grid = ((groups + 7) / 8) * 8 * G * G;
  const char *name = a.name ? a.name : "gemm_big";
  if (a.splits > 1 && !swap) return hipErrorNotSupported;
  const dim3 g3(grid, a.splits);
  timing_before(name, st);
  if (a.fp8) {
    if (!swap) return hipErrorNotSupported;
    hipLaunchKernelGGL((gemm_big_kernel<true, true>), g3, dim3(GNT), 0, st, a);
  } else if (swap && GEMM_PINGPONG && (long)a.tiles_m * a.tiles_n * a.splits <= 160) {
    // at most 5/8 of the CUs busy: both wave groups issue copies (measured:
    // 144 workgroups faster, 192 and 224 slower)
    hipLaunchKernelGGL((gemm_big_kernel<true, false, true>), g3, dim3(GNT), 0, st, a);
  } else if (swap) {
    hipLaunchKernelGGL((gemm_big_kernel<true, false>), g3, dim3(GNT), 0, st, a);
  } else {
    hipLaunchKernelGGL((gemm_big_kernel<false, false>), g3, dim3(GNT), 0, st, a);
  }
  timing_after(name, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  return launch_splitk_reduce_bf16(a, st);
}

}  // namespace mla
