// Cache append for the FP8 latent cache: quantise c_KV with one scale per 128
// columns and write the row [E4M3 codes | k_R bf16 | fp32 scales].
//
// The format follows the fine-grained FP8 scaling of the V3 technical-report
// summary ("FP8 training framework" paragraph and figure 7: values in FP8
// with a scale per small group of elements).  Per group the scale is the
// smallest power of two s with 448 s >= max|x| (1 for an all-zero group;
// exponents below -126 are raised to -126), so x / s is exact, lies in
// [-448, 448], and the dequantised value code * s is exact in bf16 (when it
// is a bf16 normal number); each value takes the E4M3 code nearest to x / s,
// ties to even (the hardware conversion rounds so).
#include "mla_internal.h"

namespace mla {

namespace {
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
}

// One wave per token; lane l covers columns 8l..8l+7 of each 512-column slab
// of c_KV (a 128-column group is sixteen lanes).
__global__ __launch_bounds__(256) void cache_append_fp8_kernel(CacheAppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= a.T) return;
  int seq = 0, pos = 0;
  row_seq_pos(a.rows, m, seq, pos);
  // rows outside the described cache are never written
  if (!cache_row_ok(a.cache, seq, pos)) return;
  unsigned char *row = (unsigned char *)a.cache.pool + cache_row(a.cache, seq, pos) * (long)a.cache.row_bytes;
  float *scales = (float *)(row + a.d_c + 2 * a.d_rope);
  const bf16 *x = a.ckv + (long)m * a.d_c;
  for (int c0 = 0; c0 < a.d_c; c0 += 512) {
    const int c = c0 + 8 * lane;
    float v[8];
    float amax = 0.f;
    if (c < a.d_c) {
      const bf16x8 in = *(const bf16x8 *)(x + c);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = (float)in[i];
        amax = fmaxf(amax, fabsf(v[i]));
      }
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
    const float scale = ldexpf(1.f, k), inv = ldexpf(1.f, -k);
    if (c < a.d_c) {
      unsigned w[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float q0 = v[i] * inv, q1 = v[i + 1] * inv;
        const unsigned p = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false) & 0xFFFFu;
        w[i >> 2] |= p << (16 * ((i >> 1) & 1));
      }
      *(u32x2v *)(row + c) = u32x2v{w[0], w[1]};
      if ((lane & 15) == 0) scales[c / 128] = scale;
    }
  }
  const bf16 *kr = a.kr + (long)m * a.d_rope;
  for (int j = lane; j < a.d_rope / 8; j += 64)
    *(bf16x8 *)(row + a.d_c + 16 * j) = *(const bf16x8 *)(kr + 8 * j);
}

hipError_t launch_cache_append_fp8(const CacheAppendArgs &a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  timing_before("cache_append_fp8", st);
  hipLaunchKernelGGL(cache_append_fp8_kernel, dim3((a.T + 3) / 4), dim3(256), 0, st, a);
  timing_after("cache_append_fp8", st);
  return hipGetLastError();
}

}  // namespace mla
