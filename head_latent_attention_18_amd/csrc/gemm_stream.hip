// Weight-streaming GEMM for few tokens (bf16, up to 128 rows of activations):
// Y[z][m][n] = sum_k X[z][m][k] W[z][n][k]   (W stored [N][K]: the down/up
// projections, W_UV and W_O), or W stored [K][N] (W_UK in the absorption).
//
// With 32 tokens every weight element feeds two MFMAs, so these products are
// bound by streaming the weights from HBM.  The kernel is built for that:
//   * the work is a flat list of units (matrix z, 64-row weight tile t,
//     k step j, 256 wide up to 32 tokens, else 128) of 32 or 16 KB of
//     weights; a persistent grid of workgroups takes equal contiguous ranges
//     of it (no tail wave);
//   * weights and the matching activation slice go HBM -> LDS with
//     global_load_lds_dwordx4 into a ring of stages, each row's slice of a
//     unit one contiguous run, several units ahead;
//   * LDS rows are k/8 chunks of 16 bytes with the chunk index XORed by the
//     row (no padding, no bank conflicts for the 16-row MFMA reads);
//   * a tile finished inside one workgroup goes straight through the
//     epilogue; a tile shared by several leaves fp32 partials that the reduce
//     kernel adds up in workgroup order (deterministic);
//   * block-scaled FP8 (F8): weights and activations are E4M3 codes, a unit
//     holds twice the k in the same bytes, and each 128-wide k step is one
//     scaled 16x16x128 MFMA taking the weight block's and the token's
//     power-of-two scales as 8-bit exponents (the activation exponents of
//     every k block sit in LDS from the start).
#include "mla_internal.h"

namespace mla {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int SBN = 64;          // weight rows (output features) per tile
constexpr int SNT = 256;         // threads per workgroup
constexpr int MAX_PARTS = 16;    // workgroups that may share one tile
constexpr int F8_MAX_KB = 128;   // FP8: k blocks of 128 whose activation exponents LDS holds

// k per unit.  Each weight row contributes one contiguous run of 2*BK bytes
// per unit: HBM serves 512-byte runs markedly faster than 256-byte ones
// (W_O at 32 tokens: 48.5 -> 44.6 us), so up to 32 tokens take 256-wide
// units; 64 tokens keep 128 (their activation slice would not fit beside).
template <int MB> constexpr int stream_bk() { return MB <= 2 ? 256 : 128; }
inline int stream_bk_for(int M) { return M <= 32 ? 256 : 128; }
// ring stages: as many units in flight as LDS holds (48 KB per unit at 32
// tokens, 32 KB at 64, 48 KB at 128)
template <int MB> constexpr int stream_stages() { return MB <= 2 ? 3 : MB <= 4 ? 4 : 3; }

template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

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

// first unit of workgroup b out of G over U units (U * G < 2^31, checked on the host)
__device__ __host__ inline int unit_start(int b, int U, int G) { return b * U / G; }
// workgroup holding unit u
__device__ __host__ inline int unit_owner(int u, int U, int G) { return ((u + 1) * G - 1) / U; }

}  // namespace

// MB: 16-row blocks of activations (M <= 16*MB).  WKN: W stored [K][N].
// F8: block-scaled E4M3 operands (GemmArgs fp8 fields).
template <int MB, bool WKN, bool F8>
__global__ __launch_bounds__(SNT, 1) void gemm_stream_kernel(GemmArgs a) {
  static_assert(!(F8 && WKN), "");
  constexpr int ESZ = F8 ? 1 : 2;                   // bytes per element
  constexpr int SBK = stream_bk<MB>() * 2 / ESZ;    // k per unit (the same bytes either way)
  constexpr int CPR = SBK * ESZ / 16;               // 16-byte chunks per row of a unit
  constexpr int SNS = stream_stages<MB>();
  constexpr int WCH = SBN * CPR;                    // weight chunks per unit
  constexpr int XCH = 16 * MB * CPR;                // activation chunks per unit
  constexpr int WLD = WCH / SNT, XLD = XCH / SNT;   // copy instructions per unit
  constexpr int LOADS = WLD + XLD;
  constexpr int STAGE = (WCH + XCH) * 8;            // bf16 elements per stage
  static_assert(WCH % SNT == 0 && XCH % SNT == 0 && LOADS * (SNS - 2) < 64, "");
  __shared__ __attribute__((aligned(16))) bf16 ring[SNS * STAGE];
  // FP8: activation scale exponents [k block][token]
  __shared__ unsigned char xsc[F8 ? F8_MAX_KB * 16 * MB : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int KS = a.K / SBK;                         // units per tile
  const int U = a.batch * a.tiles_n * KS;
  const int G = gridDim.x;
  const int u0 = unit_start(blockIdx.x, U, G), u1 = unit_start(blockIdx.x + 1, U, G);
  const int nu = u1 - u0;
  if (nu <= 0) return;
  const unsigned lring = (unsigned)(size_t)(lds_void *)ring;

  // copy of unit u into stage st
  auto issue = [&](int u, int st) {
    const int tt = u / KS;
    const int j = u - tt * KS;
    const int z = tt / a.tiles_n, t = tt - z * a.tiles_n;
    const int n0 = t * SBN, k0 = j * SBK;
    const unsigned lst = lring + (unsigned)(st * STAGE * 2) + wave * 1024;
    // weights
    if constexpr (!WKN) {
      int seg = 0, beg = 0;
      while (seg < a.nw - 1 && n0 >= a.w_end[seg]) { beg = a.w_end[seg]; ++seg; }
      const char *wb = (const char *)a.w[seg] + ((long)z * a.w_bs + (long)(n0 - beg) * a.ldw + k0) * ESZ;
      const int rows = min(SBN, a.w_end[seg] - n0);
#pragma unroll
      for (int i = 0; i < WLD; ++i) {
        const int s = i * SNT + tid, r = s / CPR, pc = s % CPR;
        const unsigned off = (unsigned)(min(r, rows - 1) * a.ldw * ESZ + ((pc ^ (r & 15)) << 4));
        dma16(wb, off, lst + i * SNT * 16);
      }
    } else {
      const char *wb = (const char *)((const bf16 *)a.w[0] + (long)z * a.w_bs + (long)k0 * a.ldw + n0);
#pragma unroll
      for (int i = 0; i < WLD; ++i) {
        const int s = i * SNT + tid, kr = s >> 3, pc = s & 7;
        const unsigned off = (unsigned)(kr * a.ldw + ((pc ^ (kr & 7)) << 3)) * 2u;
        dma16(wb, off, lst + i * SNT * 16);
      }
    }
    // activations
    const char *xb = (const char *)a.x + ((long)z * a.x_bs + k0) * ESZ;
#pragma unroll
    for (int i = 0; i < XLD; ++i) {
      const int s = i * SNT + tid, r = s / CPR, pc = s % CPR;
      const unsigned off = (unsigned)(min(r, a.M - 1) * a.ldx * ESZ + ((pc ^ (r & 15)) << 4));
      dma16(xb, off, lst + (WLD + i) * SNT * 16);
    }
  };

  f32x4 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const lds_bf16 *rl = (const lds_bf16 *)ring;
  const int first_tile = u0 / KS;

  // store (or leave as a partial) the tile of unit u, which ends here
  auto flush = [&](int u) {
    const int tt = u / KS;
    const int z = tt / a.tiles_n, t = tt - z * a.tiles_n;
    const bool whole = tt * KS >= u0 && (tt + 1) * KS <= u1;
    const int nn = t * SBN + wave * 16 + 4 * lgrp;
    // the lane's columns are fixed for all its rows: plan them once
    const ColPlan cp = (whole && nn < a.N) ? col_plan(a.epi, nn) : ColPlan{};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + lrow;
      if (m < a.M && nn < a.N) {
        float v[4] = {acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]};
        if (whole) {
          col_store<bf16>(cp, a.epi, z, m, v);
        } else {
          const int slot = tt == first_tile ? 0 : 1;
          float *p = a.partial + (((long)blockIdx.x * 2 + slot) * 16 * MB + m) * SBN + wave * 16 + 4 * lgrp;
          *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
      acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  for (int i = 0; i < SNS - 1 && i < nu; ++i) issue(u0 + i, i);
  if constexpr (F8) {
    // every k block's activation exponents, [k block][token] (visible after
    // the loop's first barrier)
    const int nkb = a.K / 128;
    for (int i = tid; i < nkb * 16 * MB; i += SNT) {
      const int kb = i / (16 * MB), m = i - kb * 16 * MB;
      xsc[i] = a.xs[(long)kb * a.xs_ld + min(m, a.M - 1)];
    }
  }
  for (int k = 0; k < nu; ++k) {
    if (k + SNS - 2 < nu) wait_vm<LOADS * (SNS - 2)>();
    else wait_vm<0>();
    bar();   // unit k landed for every wave; stage (k-1) % SNS is free
    if (k + SNS - 1 < nu) issue(u0 + k + SNS - 1, (k + SNS - 1) % SNS);
    const lds_bf16 *ws = rl + (k % SNS) * STAGE;
    const lds_bf16 *xs = ws + WCH * 8;
    if constexpr (F8) {
      // 128-wide k steps: lane group g holds logical chunks 8s + 2g and
      // 8s + 2g + 1 of its row (both operands alike); the weight block's
      // exponent is uniform over the unit's 64 rows, the token's comes from LDS
      const int u = u0 + k;
      const int tt = u / KS;
      const int j = u - tt * KS;
      const int z = tt / a.tiles_n, t = tt - z * a.tiles_n;
      const int n0 = t * SBN;
      int seg = 0, beg = 0;
      while (seg < a.nw - 1 && n0 >= a.w_end[seg]) { beg = a.w_end[seg]; ++seg; }
      const float *wsp = a.wsc[seg] + (long)((n0 - beg) >> 7) * a.wsc_ld + j * (SBK / 128);
      const lds_u8 *xsl = (const lds_u8 *)xsc;
#pragma unroll
      for (int s = 0; s < SBK / 128; ++s) {
        const int sw = (int)((__builtin_bit_cast(unsigned, wsp[s]) >> 23) & 0xFFu);
        const int c0 = 8 * s + 2 * lgrp;
        const int r = wave * 16 + lrow;
        const lds_u32x4 *wrow = (const lds_u32x4 *)((const lds_u8 *)ws + r * CPR * 16);
        const u32x4 w0 = wrow[c0 ^ (r & 15)], w1 = wrow[(c0 + 1) ^ (r & 15)];
        const i32x8 wf = {(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int rx = mb * 16 + lrow;
          const lds_u32x4 *xrow = (const lds_u32x4 *)((const lds_u8 *)xs + rx * CPR * 16);
          const u32x4 x0 = xrow[c0 ^ (rx & 15)], x1 = xrow[(c0 + 1) ^ (rx & 15)];
          const i32x8 xf = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
          const int sx = xsl[(j * (SBK / 128) + s) * 16 * MB + rx];
          acc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf, acc[mb], 0, 0, 0, sw, 0, sx);
        }
      }
    } else {
#pragma unroll
    for (int s = 0; s < SBK / 32; ++s) {
      const int c = 4 * s + lgrp;                  // logical 16-byte chunk of the k step
      bf16x8 wf;
      if constexpr (!WKN) {
        const int r = wave * 16 + lrow;
        wf = *(const lds_bf16x8 *)(ws + (r * CPR + (c ^ (r & 15))) * 8);
      } else {
        // W^T fragment: k = 32s + 8*lgrp + 0..7 for feature wave*16 + lrow,
        // two transposed 4x16 reads of the [k][n] tile
        const int kr = 32 * s + 8 * lgrp + (lrow >> 2);
        const int col = wave * 16 + 4 * (lrow & 3);        // element column
        const int ch = col >> 3, half = col & 7;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16 *)(ws + (kr * 8 + (ch ^ (kr & 7))) * 8 + half));
        const int kr2 = kr + 4;
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16 *)(ws + (kr2 * 8 + (ch ^ (kr2 & 7))) * 8 + half));
        wf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = mb * 16 + lrow;
        const bf16x8 xf = *(const lds_bf16x8 *)(xs + (r * CPR + (c ^ (r & 15))) * 8);
        acc[mb] = Mma<bf16>::mma(wf, xf, acc[mb]);
      }
    }
    }
    const int u = u0 + k;
    if ((u + 1) % KS == 0 || k == nu - 1) flush(u);
  }
}

// Sum the partials of tiles shared by several workgroups, in workgroup order,
// then the epilogue.  One thread per (tile, row, 4 columns); all partial loads
// are issued before the sum.
template <int MB>
__global__ __launch_bounds__(256) void gemm_stream_reduce_kernel(GemmArgs a, int G, int KS) {
  const int U = a.batch * a.tiles_n * KS;
  // workgroups of one tile: its segment and owners are uniform
  const int per_tile = a.M * (SBN / 4);
  const int wpt = (per_tile + 255) / 256;
  const int tt = blockIdx.x / wpt;
  const int rem = (blockIdx.x - tt * wpt) * 256 + threadIdx.x;
  if (tt >= a.batch * a.tiles_n || rem >= per_tile) return;
  const int m = rem / (SBN / 4), c4 = (rem % (SBN / 4)) * 4;
  const int bf = unit_owner(tt * KS, U, G), bl = unit_owner((tt + 1) * KS - 1, U, G);
  if (bf == bl) return;   // stored by its only workgroup
  const int z = tt / a.tiles_n, t = tt - z * a.tiles_n;
  const int n = t * SBN + c4;
  if (n >= a.N) return;
  const ColPlan cp = col_plan_tile(a.epi, t * SBN, n);
  // the first contributor holds the tile as its last one (slot 1) unless the
  // tile is also its first; every later contributor starts with it (slot 0)
  const int slot0 = unit_start(bf, U, G) / KS == tt ? 0 : 1;
  f32x4 v[MAX_PARTS];
#pragma unroll
  for (int i = 0; i < MAX_PARTS; ++i)
    if (bf + i <= bl) {
      const int b = bf + i, slot = i == 0 ? slot0 : 0;
      v[i] = *(const f32x4 *)(a.partial + ((b * 2 + slot) * 16 * MB + m) * SBN + c4);
    }
  f32x4 s = v[0];
#pragma unroll
  for (int i = 1; i < MAX_PARTS; ++i)
    if (bf + i <= bl) s += v[i];
  float o[4] = {s[0], s[1], s[2], s[3]};
  col_store<bf16>(cp, a.epi, z, m, o);
}

int gemm_stream_grid() { return 256; }

// Workgroups: whole tiles per workgroup when that keeps at least 3/4 of the
// CUs busy (no partials, no reduce); otherwise an even split of the units
// over at most one workgroup per CU, and fewer when a product has few tiles
// of many units (the cache compression alone: 9 tiles of 28), so that no
// tile is shared by more than MAX_PARTS workgroups (a workgroup holds
// floor(U/G) or one more units, so a tile of KS units meets at most
// KS / floor(U/G) + 2 of them).
static int stream_grid_for(int U, int KS, int tiles) {
  const int full = gemm_stream_grid();
  if (U > full)
    for (int g = full; g * 4 >= full * 3; --g)
      if (tiles % g == 0) return g;
  int g = std::min(U, full);
  while (g > 1 && KS / std::max(1, U / g) + 2 > MAX_PARTS) --g;
  return g;
}

size_t gemm_stream_partial_bytes(int M) {
  const int mb = M <= 32 ? 2 : M <= 64 ? 4 : 8;
  return (size_t)gemm_stream_grid() * 2 * 16 * mb * SBN * sizeof(float);
}

bool gemm_stream_ok(const GemmArgs &a, int wkn) {
  // Up to 32 tokens, long products only: the ring's fill and drain cost a
  // few microseconds, which shorter weight streams (q_up, W_UK, W_UV) do not
  // amortise; those keep the register-streaming kernels.  From 33 tokens on
  // every product whose k is a whole number of units streams here.  FP8
  // products always stream here (the only FP8 kernel for up to 128 tokens).
  if (a.fp8 && (wkn || a.K / 128 > F8_MAX_KB || !a.xs)) return false;
  if (wkn || (!a.fp8 && a.M <= 32 && a.K < 4096)) return false;
  const int bk = stream_bk_for(a.M) * (a.fp8 ? 2 : 1);
  if (a.M > 128 || a.K % bk != 0 || !a.partial) return false;
  if (a.partial_bytes < gemm_stream_partial_bytes(a.M)) return false;   // the partials' layout must fit
  const long units = (long)a.batch * ((a.N + SBN - 1) / SBN) * (a.K / bk);
  if (units * gemm_stream_grid() >= (1L << 31)) return false;
  // (the grid keeps the workgroups sharing a tile within MAX_PARTS)
  if (wkn) return a.N % SBN == 0 && a.nw == 1;
  for (int s = 0; s < a.nw - 1; ++s)
    if (a.w_end[s] % SBN != 0) return false;   // a tile never straddles two weight segments
  return true;
}


template <int MB, bool WKN, bool F8>
static hipError_t launch_stream_t(GemmArgs &a, hipStream_t st) {
  a.tiles_m = 1;
  a.tiles_n = (a.N + SBN - 1) / SBN;
  const int KS = a.K / (stream_bk<MB>() * (F8 ? 2 : 1));
  const int tiles = a.batch * a.tiles_n;
  const int U = tiles * KS;
  const int G = stream_grid_for(U, KS, tiles);
  timing_before(a.name ? a.name : "gemm_stream", st);
  hipLaunchKernelGGL((gemm_stream_kernel<MB, WKN, F8>), dim3(G), dim3(SNT), 0, st, a);
  timing_after(a.name ? a.name : "gemm_stream", st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bool split = false;   // does a workgroup boundary fall inside a tile?
  for (int b = 1; b < G && !split; ++b) split = unit_start(b, U, G) % KS != 0;
  if (!split) return hipSuccess;
  const long wgs = (long)tiles * ((a.M * (SBN / 4) + 255) / 256);
  const char *rn = a.reduce_name ? a.reduce_name : "gemm_stream.reduce";
  timing_before(rn, st);
  hipLaunchKernelGGL((gemm_stream_reduce_kernel<MB>), dim3((unsigned)wgs), dim3(256), 0, st, a, G, KS);
  timing_after(rn, st);
  return hipGetLastError();
}

hipError_t launch_gemm_stream(GemmArgs &a, int wkn, hipStream_t st) {
  if (a.fp8) {
    if (wkn) return hipErrorNotSupported;
    if (a.M <= 32) return launch_stream_t<2, false, true>(a, st);
    if (a.M <= 64) return launch_stream_t<4, false, true>(a, st);
    return launch_stream_t<8, false, true>(a, st);
  }
  // up to 32 tokens in 32 rows: the 16-row form streamed W_O at 8 tokens in
  // 55 us against 43 us for this one (the rows past M are computed and not
  // stored)
  if (a.M <= 32) return wkn ? launch_stream_t<2, true, false>(a, st) : launch_stream_t<2, false, false>(a, st);
  if (a.M <= 64) return wkn ? launch_stream_t<4, true, false>(a, st) : launch_stream_t<4, false, false>(a, st);
  return wkn ? launch_stream_t<8, true, false>(a, st) : launch_stream_t<8, false, false>(a, st);
}

}  // namespace mla
