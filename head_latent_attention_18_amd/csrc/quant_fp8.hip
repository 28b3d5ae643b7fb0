// Activation quantiser of the block-scaled FP8 projections: each token's row
// is cut into groups of 128 columns, and a group is stored as E4M3 codes with
// one power-of-two scale (the FP8 framework of the V3 technical-report
// summary, "FP8 training framework" paragraph and figures 6 and 7:
// activations scaled in blocks, 128 elements per accumulation interval).
//
// Per group the scale is the smallest power of two s with 448 s >= max|x|
// (1 for an all-zero group; exponents below -126 are raised to -126), so
// x / s is exact and lies in [-448, 448]; each value takes the E4M3 code
// nearest to x / s, ties to even (the hardware conversion rounds so).  The
// scale leaves as its biased 8-bit exponent, the operand format of the
// scaled FP8 MFMAs, stored [group][token] so that the product kernels read
// a run of consecutive tokens per k block.
#include "mla_internal.h"

namespace mla {

namespace {
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
}

// blockIdx.y: a run of SPW 512-column slabs; four waves per block, one token
// each; lane l covers columns 8l..8l+7 of each slab (a group is sixteen
// lanes).  The run's loads are all issued before any is used.
constexpr int SPW = 4;

__global__ __launch_bounds__(256) void quant_act_fp8_kernel(const bf16 *x, long ldx, int T, int K,
                                                            unsigned char *codes, long ldc, unsigned char *scales,
                                                            long ld_s) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= T) return;
  const int s0 = blockIdx.y * SPW, ns = min(SPW, K / 512 - s0);
  bf16x8 in[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i)
    if (i < ns) in[i] = *(const bf16x8 *)(x + (long)m * ldx + (long)(s0 + i) * 512 + 8 * lane);
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    if (i >= ns) break;
    const long c = (long)(s0 + i) * 512 + 8 * lane;
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = (float)in[i][e];
      amax = fmaxf(amax, fabsf(v[e]));
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    // amax = f * 2^e with 0.5 <= f < 1: 448 * 2^(e-9) = 0.875 * 2^e, and
    // 448 * 2^(e-10) < 0.5 * 2^e <= amax, so k = e - 9, or e - 8 when f > 0.875
    int k = 0;
    if (amax > 0.f) {
      int e;
      const float f = frexpf(amax, &e);
      k = max(e - 9 + (f > 0.875f ? 1 : 0), -126);
    }
    const float inv = ldexpf(1.f, -k);
    unsigned w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const unsigned p = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(v[e] * inv, v[e + 1] * inv, 0, false) & 0xFFFFu;
      w[e >> 2] |= p << (16 * ((e >> 1) & 1));
    }
    *(u32x2v *)(codes + (long)m * ldc + c) = u32x2v{w[0], w[1]};
    if ((lane & 15) == 0) scales[(c >> 7) * ld_s + m] = (unsigned char)(k + 127);
  }
}

hipError_t launch_quant_act_fp8(const bf16 *x, long ldx, int T, int K, unsigned char *codes, unsigned char *scales,
                                long ld_s, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int runs = (K / 512 + SPW - 1) / SPW;
  if (K % 512 != 0 || runs > 65535) return hipErrorInvalidValue;
  timing_before("quant_fp8", st);
  hipLaunchKernelGGL(quant_act_fp8_kernel, dim3((unsigned)((T + 3) / 4), (unsigned)runs), dim3(256), 0, st, x, ldx,
                     T, K, codes, (long)K, scales, ld_s);
  timing_after("quant_fp8", st);
  return hipGetLastError();
}

}  // namespace mla
