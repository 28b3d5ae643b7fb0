// Projection GEMMs of the MLA layer: Y[M][N] = X[M][K] * W^T, with W stored
// [N][K] (the pages' W*h orientation, every projection of section 2.1 of the
// DeepSeek-V3 paper-reading notes) or, for the absorbed query, [K][N].
//
// One templated kernel serves the large-token tiles (prefill) and the
// skinny tiles (decode, weight streaming with split-K).  X and W tiles are
// staged through LDS in two buffers; the MFMA operands are read as 16-byte
// runs (see mla_internal.h).  With SWAP the weight tile is the MFMA A operand,
// so each lane ends with four consecutive output features of one token: the
// epilogue can apply RoPE to (2k, 2k+1) pairs and write cache rows without
// any cross-lane exchange.  Without SWAP the lane holds four consecutive
// tokens of one feature, which is what a transposed store (V^T) needs.
#include <type_traits>

#include "mla_internal.h"

namespace mla {

template <typename T, int BM, int BN, int BK, int WM, int WN, bool SWAP, bool WKN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs a) {
  constexpr int NT = 64 * WM * WN;
  constexpr int KPL = Mma<T>::KPL;
  constexpr int VE = Vec<T>::N;
  constexpr int LDK = BK + VE;          // LDS row stride: 16 bytes of padding
  constexpr int RUN = BK / 4;
  constexpr int STEPS = RUN / KPL;
  static_assert(RUN % KPL == 0, "k run must hold whole MFMA operands");
  static_assert(RUN % VE == 0 || !WKN, "transposed W tile needs whole chunks");
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 16x16 block");
  constexpr int XCH = BM * BK / VE;
  constexpr int WCH = BN * BK / VE;
  constexpr int XPT = (XCH + NT - 1) / NT;
  constexpr int WPT = (WCH + NT - 1) / NT;
  typedef typename Mma<T>::frag frag;

  __shared__ __attribute__((aligned(16))) T xs[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) T ws[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int lrow = lane & 15, lgrp = lane >> 4;

  // Tile order.  The dispatcher deals blocks round-robin over the 8 XCDs
  // (block b runs on XCD b % 8).  The tiles are cut into 8x8 groups; each XCD
  // takes whole groups, so the blocks running together on one XCD share eight
  // X row-tiles and eight W row-tiles: every k-slab they load is reused eight
  // times from that XCD's L2.  The grid covers the tile counts rounded up to
  // whole groups; blocks past the edge exit.
  int tm, tn;
  if (!a.grouped) {
    tm = blockIdx.x % a.tiles_m;
    tn = blockIdx.x / a.tiles_m;
  } else {
    const int bid = blockIdx.x, xcd = bid & 7, local = bid >> 3;
    const int gm_n = (a.tiles_m + 7) >> 3;                // groups along M
    const int g = (local >> 6) * 8 + xcd, w = local & 63;
    tm = (g % gm_n) * 8 + (w & 7);
    tn = (g / gm_n) * 8 + (w >> 3);
    if (tm >= a.tiles_m || tn >= a.tiles_n) return;
  }
  const int bz = blockIdx.y / a.splits, sp = blockIdx.y % a.splits;
  const int M = a.M, N = a.N;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = sp * a.k_chunk;
  const int nk = a.k_chunk / BK;

  const T *X = (const T *)a.x + (long)bz * a.x_bs;

  // per-thread source pointers (rows fixed across the k loop)
  const T *xsrc[XPT];
  int xdst[XPT];
  bool xok[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = tid + i * NT;
    xok[i] = c < XCH;
    const int r = c / (BK / VE), kc = c % (BK / VE);
    const int gm = min(m0 + r, M - 1);
    xsrc[i] = X + (long)gm * a.ldx + kbeg + kc * VE;
    xdst[i] = r * LDK + kc * VE;
  }
  const T *wsrc[WPT];
  int wdst[WPT];
  bool wok[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int c = tid + i * NT;
    wok[i] = c < WCH;
    if (!WKN) {
      const int r = c / (BK / VE), kc = c % (BK / VE);
      const int n = min(n0 + r, N - 1);
      int s = 0, beg = 0;
      while (s < a.nw - 1 && n >= a.w_end[s]) { beg = a.w_end[s]; ++s; }
      wsrc[i] = (const T *)a.w[s] + (long)bz * a.w_bs + (long)(n - beg) * a.ldw + kbeg + kc * VE;
      wdst[i] = r * LDK + kc * VE;
    } else {
      const int kr = c / (BN / VE), nc = c % (BN / VE);
      const int n = min(n0 + nc * VE, N - VE);
      wsrc[i] = (const T *)a.w[0] + (long)bz * a.w_bs + (long)(kbeg + kr) * a.ldw + n;
      wdst[i] = (nc * VE) * LDK + kr;
    }
  }

  u32x4 xr[XPT], wr[WPT];
  auto gload = [&](int kt) {
    const long koff = (long)kt * BK;
#pragma unroll
    for (int i = 0; i < XPT; ++i)
      if (xok[i]) xr[i] = *(const u32x4 *)(xsrc[i] + koff);
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      if (wok[i]) {
        if (!WKN) wr[i] = *(const u32x4 *)(wsrc[i] + koff);
        else wr[i] = *(const u32x4 *)(wsrc[i] + koff * a.ldw);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i)
      if (xok[i]) *(u32x4 *)&xs[buf][xdst[i]] = xr[i];
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      if (wok[i]) {
        if (!WKN) {
          *(u32x4 *)&ws[buf][wdst[i]] = wr[i];
        } else {
          const T *e = (const T *)&wr[i];
#pragma unroll
          for (int j = 0; j < VE; ++j) ws[buf][wdst[i] + j * LDK] = e[j];
        }
      }
    }
  };

  f32x4 acc[SWAP ? FN : FM][SWAP ? FM : FN];
#pragma unroll
  for (int i = 0; i < (SWAP ? FN : FM); ++i)
#pragma unroll
    for (int j = 0; j < (SWAP ? FM : FN); ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      frag xa[FM], wb[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f)
        xa[f] = *(const frag *)&xs[buf][(wm * TM + f * 16 + lrow) * LDK + lgrp * RUN + s * KPL];
#pragma unroll
      for (int f = 0; f < FN; ++f)
        wb[f] = *(const frag *)&ws[buf][(wn * TN + f * 16 + lrow) * LDK + lgrp * RUN + s * KPL];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (SWAP) acc[j][i] = Mma<T>::mma(wb[j], xa[i], acc[j][i]);
          else acc[i][j] = Mma<T>::mma(xa[i], wb[j], acc[i][j]);
        }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  if (SWAP) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + j * 16 + 4 * lgrp;
      if (n >= N) continue;
      // the lane's columns are fixed for all its rows: plan them once
      const ColPlan cp = a.splits > 1 ? ColPlan{} : col_plan(a.epi, n);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + i * 16 + lrow;
        if (m < M) {
          float v[4] = {acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]};
          if (a.splits > 1) {
            float *p = a.partial + (((long)bz * a.splits + sp) * M + m) * N + n;
            *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
          } else {
            col_store<T>(cp, a.epi, bz, m, v);
          }
        }
      }
    }
  } else {
    const Seg &g = a.epi.seg[0];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * TN + j * 16 + lrow;
        const int mb = m0 + wm * TM + i * 16 + 4 * lgrp;
        if (n < N) {
          T *dst = (T *)g.dst + (long)bz * g.batch_stride + (long)n * g.ld;
          if (mb + 3 < M && (g.ld & 3) == 0) {
            float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            store4<T>(dst, mb, v, 0);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (mb + r < M) dst[mb + r] = from_f32<T>(acc[i][j][r]);
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Weight-streaming GEMM for few tokens (decode): bf16, W stored [N][K].
// Each wave owns 16 output features and streams its weight rows straight from
// HBM into MFMA A-operand registers (a ring of three 256-wide k stages, so two
// stages are in flight while one is multiplied); the tokens' activations are
// staged in LDS once per workgroup and read as the B operand.  Within a stage,
// MFMA step s of lane group g uses the 16-byte chunk 4*s+g of its row, so one
// load instruction covers 64 contiguous bytes of each of 16 rows.
// ---------------------------------------------------------------------------
// The stage count NST is a template parameter and the pipeline is fully
// unrolled: with a loop, the compiler's wait-count tracking loses which load
// fills which ring slot at the back edge and waits for every load in flight.
#ifndef SKINNY_AHEAD
#define SKINNY_AHEAD 2
#endif
template <int MB, int BK, int NST>
__global__ __launch_bounds__(256, 2) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int NW = 4, BN = 16 * NW, VE = 8;
  constexpr int STEPS = BK / 32;              // MFMA k-steps per stage
  constexpr int CHS = BK / VE;                // 16-byte chunks per row per stage
  constexpr int XLD = BK + VE;                // LDS row pitch of the activation stage
  constexpr int XCH = 16 * MB * CHS;          // activation chunks per stage
  constexpr int XPT = (XCH + 255) / 256;
  constexpr int AHEAD = SKINNY_AHEAD;         // weight stages in flight beyond the current one
  static_assert(STEPS * 4 == CHS, "");
  __shared__ __attribute__((aligned(16))) bf16 xs[2][16 * MB * XLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int tn = bid;                                   // one N tile per block column (tiles_m == 1)
  const int bz = blockIdx.y / a.splits, sp = blockIdx.y % a.splits;
  const int M = a.M, N = a.N;
  const int n0 = tn * BN;
  const int kbeg = sp * a.k_chunk;

  // weight row of this lane (segments of W rows are separate matrices)
  const int n = min(n0 + wave * 16 + lrow, N - 1);
  int seg = 0, beg = 0;
  while (seg < a.nw - 1 && n >= a.w_end[seg]) { beg = a.w_end[seg]; ++seg; }
  const bf16 *wrow = (const bf16 *)a.w[seg] + (long)bz * a.w_bs + (long)(n - beg) * a.ldw + kbeg + lgrp * VE;
  const bf16 *X = (const bf16 *)a.x + (long)bz * a.x_bs;

  bf16x8 wr[NST][STEPS];
  auto wload = [&](int st) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) wr[st][s] = *(const bf16x8 *)(wrow + (long)st * BK + s * 4 * VE);
  };
  u32x4 xr[NST][XPT];   // activations travel AHEAD stages early, with their weights
  auto xload = [&](int st) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * 256;
      if (c < XCH) {
        const int r = c / CHS, kc = c % CHS;
        xr[st][i] = *(const u32x4 *)(X + (long)min(r, M - 1) * a.ldx + kbeg + (long)st * BK + kc * VE);
      }
    }
  };
  auto xstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * 256;
      if (c < XCH) {
        const int r = c / CHS, kc = c % CHS;
        *(u32x4 *)&xs[st & 1][r * XLD + kc * VE] = xr[st][i];
      }
    }
  };

  f32x4 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i <= AHEAD && i < NST; ++i) {
    xload(i);
    wload(i);
  }
  xstore(0);
  __syncthreads();
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const int buf = st & 1;
    if (st + AHEAD + 1 < NST) {                  // stage st+AHEAD+1 enters the pipe
      xload(st + AHEAD + 1);
      wload(st + AHEAD + 1);
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 xb = *(const bf16x8 *)&xs[buf][(mb * 16 + lrow) * XLD + (4 * s + lgrp) * VE];
        acc[mb] = Mma<bf16>::mma(wr[st][s], xb, acc[mb]);
      }
    }
    if (st + 1 < NST) {
      xstore(st + 1);
      __syncthreads();
    }
  }

  const int nn = n0 + wave * 16 + 4 * lgrp;
  if (nn < N) {
    // the lane's columns are fixed for all its rows: plan them once
    const ColPlan cp = a.splits > 1 ? ColPlan{} : col_plan(a.epi, nn);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + lrow;
      if (m < M) {
        float v[4] = {acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]};
        if (a.splits > 1) {
          float *p = a.partial + (((long)bz * a.splits + sp) * M + m) * N + nn;
          *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          col_store<bf16>(cp, a.epi, bz, m, v);
        }
      }
    }
  }
}

// Sum the split-K partials in split order (deterministic) and apply the epilogue.
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a) {
  const int n4 = a.N >> 2;
  const long total = (long)a.batch * a.M * n4;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int bz = (int)(idx / ((long)a.M * n4));
  const long rem = idx - (long)bz * a.M * n4;
  const int m = (int)(rem / n4), n = (int)(rem % n4) * 4;
  // issue the loads of eight splits before summing them (in split order)
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  const float *src = a.partial + ((long)bz * a.splits * a.M + m) * a.N + n;
  const long step = (long)a.M * a.N;
  int p = 0;
  for (; p + 8 <= a.splits; p += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *(const f32x4 *)(src + (p + j) * step);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  for (; p < a.splits; ++p) s += *(const f32x4 *)(src + p * step);
  float v[4] = {s[0], s[1], s[2], s[3]};
  epi_store4<T>(a.epi, bz, m, n, v);
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool SWAP, bool WKN>
static hipError_t launch_t(GemmArgs &a, hipStream_t st, const char *name) {
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.grouped = a.tiles_m >= 8 && a.tiles_n >= 8;
  // grouped: 8x8-tile groups dealt to the XCDs in rows of eight groups
  // (block -> group (block >> 9) * 8 + (block & 7)), so the grid covers whole
  // rows of groups even when the group count is not a multiple of eight
  const int groups = ((a.tiles_m + 7) / 8) * ((a.tiles_n + 7) / 8);
  dim3 grid(a.grouped ? ((groups + 7) / 8) * 8 * 64 : a.tiles_m * a.tiles_n, a.batch * a.splits);
  if (a.name) name = a.name;
  timing_before(name, st);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, SWAP, WKN>), grid, dim3(64 * WM * WN), 0, st, a);
  timing_after(name, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.splits > 1) {
    const long total = (long)a.batch * a.M * (a.N / 4);
    const char *rname = a.reduce_name ? a.reduce_name : "splitk_reduce";
    timing_before(rname, st);
    hipLaunchKernelGGL(splitk_reduce_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
    timing_after(rname, st);
    e = hipGetLastError();
  }
  return e;
}

// the ordered split-K reduce for the 256x256 kernel's splits (bf16 outputs)
hipError_t launch_splitk_reduce_bf16(GemmArgs &a, hipStream_t st) {
  const long total = (long)a.batch * a.M * (a.N / 4);
  const char *rname = a.reduce_name ? a.reduce_name : "splitk_reduce";
  timing_before(rname, st);
  hipLaunchKernelGGL(splitk_reduce_kernel<bf16>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  timing_after(rname, st);
  return hipGetLastError();
}

template <int MB, int BK, int NST>
static void launch_skinny_nst(GemmArgs &a, hipStream_t st, dim3 grid) {
  hipLaunchKernelGGL((gemm_skinny_kernel<MB, BK, NST>), grid, dim3(256), 0, st, a);
}
// stage counts with an instantiation (the host planner picks k_chunk among these)
int skinny_nst_supported(int nst) { return nst == 1 || nst == 2 || nst == 3 || nst == 4 || nst == 6 || nst == 8 || nst == 16; }
template <int MB, int BK>
static hipError_t launch_skinny(GemmArgs &a, hipStream_t st, const char *name) {
  a.tiles_m = 1;
  a.tiles_n = (a.N + 63) / 64;
  dim3 grid(a.tiles_n, a.batch * a.splits);
  if (a.name) name = a.name;
  const int nst = a.k_chunk / BK;
  timing_before(name, st);
  switch (nst) {
    case 1: launch_skinny_nst<MB, BK, 1>(a, st, grid); break;
    case 2: launch_skinny_nst<MB, BK, 2>(a, st, grid); break;
    case 3: launch_skinny_nst<MB, BK, 3>(a, st, grid); break;
    case 4: launch_skinny_nst<MB, BK, 4>(a, st, grid); break;
    case 6: launch_skinny_nst<MB, BK, 6>(a, st, grid); break;
    case 8: launch_skinny_nst<MB, BK, 8>(a, st, grid); break;
    case 16: launch_skinny_nst<MB, BK, 16>(a, st, grid); break;
    default: return hipErrorInvalidValue;
  }
  timing_after(name, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.splits > 1) {
    const long total = (long)a.batch * a.M * (a.N / 4);
    const char *rname = a.reduce_name ? a.reduce_name : "splitk_reduce";
    timing_before(rname, st);
    hipLaunchKernelGGL(splitk_reduce_kernel<bf16>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
    timing_after(rname, st);
    e = hipGetLastError();
  }
  return e;
}

// K granularity each tile needs (host checks K % gemm_bk == 0 per split).
int gemm_bk(int dtype, int tile) {
  if (dtype == 0) return 32;
  return 64;
}
int gemm_bm(int dtype, int tile) {
  if (dtype == 0) return 32;
  return tile == TILE_BIG ? 128 : 32;
}

#ifndef BIG_BM
#define BIG_BM 128
#define BIG_BN 128
#endif
#ifndef BIG_BK
#define BIG_BK 64
#define BIG_WM 2   // 8 waves: 64x32 per wave
#define BIG_WN 4
#endif
hipError_t launch_gemm(int dtype, int tile, int swap, int wkn, GemmArgs &a, hipStream_t st) {
  // split-K partials [batch][splits][M][N] must fit the buffer given
  if (a.splits > 1 && (!a.partial || a.partial_bytes < (size_t)a.batch * a.splits * a.M * a.N * sizeof(float)))
    return hipErrorInvalidValue;
  if (a.fp8) {
    // block-scaled FP8: up to 128 tokens stream the weights, more take the
    // 256x256 tiles
    if (dtype != 1 || wkn || !swap) return hipErrorNotSupported;
    if (a.M <= 128 && gemm_stream_ok(a, 0)) return launch_gemm_stream(a, 0, st);
    if (a.M > 128 && gemm_big_ok(a)) return launch_gemm_big(a, 1, st);
    return hipErrorNotSupported;
  }
  if (dtype == 1) {
    if (tile == TILE_BIG) {
      if (!wkn && gemm_big_ok(a)) return launch_gemm_big(a, swap, st);
      if (swap && !wkn) return launch_t<bf16, BIG_BM, BIG_BN, BIG_BK, BIG_WM, BIG_WN, true, false>(a, st, "gemm_bf16_big");
      if (!swap && !wkn) return launch_t<bf16, BIG_BM, BIG_BN, BIG_BK, BIG_WM, BIG_WN, false, false>(a, st, "gemm_bf16_big_t");
      if (swap && wkn) return launch_t<bf16, 128, 128, 64, 2, 2, true, true>(a, st, "gemm_bf16_128x128_kn");
    } else {
      // 96..128 tokens against a wide weight with short k (the query
      // up-projection of a 128-sequence decode step): 128x128 tiles read the
      // activations once per 128 weight rows, where the weight-streaming
      // kernel reads them once per 64 (q_up at 128 tokens: 46 against 69 us)
      if (swap && !wkn && a.batch == 1 && a.M >= 96 && a.M <= 128 && a.K <= 2048 && a.N >= 8192)
        return launch_t<bf16, BIG_BM, BIG_BN, BIG_BK, BIG_WM, BIG_WN, true, false>(a, st, "gemm_bf16_big");
      if (swap && gemm_stream_ok(a, wkn)) return launch_gemm_stream(a, wkn, st);
      if (swap && !wkn) {
        if (a.M <= 32 && a.k_chunk % 256 == 0 && skinny_nst_supported(a.k_chunk / 256))
          return launch_skinny<2, 256>(a, st, "gemm_bf16_stream_m32");
        if (a.M <= 64 && a.k_chunk % 256 == 0 && skinny_nst_supported(a.k_chunk / 256))
          return launch_skinny<4, 256>(a, st, "gemm_bf16_stream_m64");
        if (a.M <= 128 && a.k_chunk % 128 == 0 && skinny_nst_supported(a.k_chunk / 128))
          return launch_skinny<8, 128>(a, st, "gemm_bf16_stream_m128");
        return launch_t<bf16, 32, 64, 64, 1, 4, true, false>(a, st, "gemm_bf16_32x64");
      }
      if (!swap && !wkn) return launch_t<bf16, 32, 64, 64, 1, 4, false, false>(a, st, "gemm_bf16_32x64_t");
      if (swap && wkn) return launch_t<bf16, 32, 64, 64, 1, 4, true, true>(a, st, "gemm_bf16_32x64_kn");
    }
  } else {
    if (swap && !wkn) return launch_t<float, 32, 32, 32, 2, 2, true, false>(a, st, "gemm_f32_32x32");
    if (!swap && !wkn) return launch_t<float, 32, 32, 32, 2, 2, false, false>(a, st, "gemm_f32_32x32_t");
    if (swap && wkn) return launch_t<float, 32, 32, 32, 2, 2, true, true>(a, st, "gemm_f32_32x32_kn");
  }
  return hipErrorInvalidValue;
}

}  // namespace mla
