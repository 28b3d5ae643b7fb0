// Host-side check of the C ABI's argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code of the
// validation layer (mla_api.hip) and of this driver.  No call here reaches a
// kernel launch: each one fails a check first (a NULL, an out-of-range size,
// a cache descriptor, or a workspace far too small for the sizes given), so
// the fake device pointers are never dereferenced.  The sweeps drive the
// size arithmetic with extreme values, where an overflow or an out-of-bounds
// read would be undefined behaviour and the sanitizers abort.
//
// Exit status 0 when every returned code is the expected one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "mla.h"

namespace {

int failures = 0;
#define EXPECT_EQ(expr, want)                                                             \
  do {                                                                                    \
    const long got_ = (long)(expr);                                                       \
    if (got_ != (long)(want)) {                                                           \
      std::printf("FAIL %s:%d: %s = %ld, want %ld\n", __FILE__, __LINE__, #expr, got_, (long)(want)); \
      ++failures;                                                                         \
    }                                                                                     \
  } while (0)
#define EXPECT_TRUE(expr)                                                                 \
  do {                                                                                    \
    if (!(expr)) {                                                                        \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #expr);                         \
      ++failures;                                                                         \
    }                                                                                     \
  } while (0)

void *const FAKE = (void *)0x10000;

mla_config dsv3() {
  mla_config c;
  std::memset(&c, 0, sizeof c);
  c.d_model = 7168;
  c.n_heads = 128;
  c.d_nope = 128;
  c.d_rope = 64;
  c.d_v = 128;
  c.d_c = 512;
  c.d_cq = 1536;
  c.dtype = MLA_BF16;
  c.rope_base = 10000.0;
  return c;
}

mla_weights fake_weights() {
  mla_weights w;
  std::memset(&w, 0, sizeof w);
  w.w_dq = w.w_uq = w.w_qr = w.w_dkv = w.w_kr = w.w_uk = w.w_uv = w.w_o = FAKE;
  w.s_dq = w.s_dkv = w.s_kr = w.s_o = (const float *)FAKE;
  return w;
}

mla_cache contiguous(int32_t max_len) {
  mla_cache k;
  std::memset(&k, 0, sizeof k);
  k.pool = FAKE;
  k.max_len = max_len;
  return k;
}

mla_cache paged(int32_t bs, int32_t nb, int32_t mb) {
  mla_cache k;
  std::memset(&k, 0, sizeof k);
  k.pool = FAKE;
  k.block_size = bs;
  k.n_blocks = nb;
  k.block_table = (const int32_t *)FAKE;
  k.max_blocks_per_seq = mb;
  return k;
}

// deterministic generator (SplitMix64)
uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int32_t pick_i32() {
  static const int32_t special[] = {0, 1, -1, 2, 7, 8, 16, 31, 32, 63, 64, 96, 128, 512, 576, 1024, 1536, 4096,
                                    7168, 65535, 65536, 1 << 20, 1 << 24, 1 << 30,
                                    std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::min()};
  const uint64_t r = next_u64();
  if (r & 1) return special[(r >> 1) % (sizeof special / sizeof special[0])];
  return (int32_t)(r >> 32);
}
double pick_f64() {
  static const double special[] = {0.0, 1.0, -1.0, 0.5, 40.0, 10000.0, 1e300, -1e300,
                                   std::numeric_limits<double>::infinity(), std::nan("")};
  const uint64_t r = next_u64();
  return special[r % (sizeof special / sizeof special[0])];
}

void fixed_cases() {
  // status strings
  for (int s = -7; s <= 0; ++s) EXPECT_TRUE(std::strlen(mla_status_string((mla_status)s)) > 0);
  EXPECT_TRUE(std::strcmp(mla_status_string((mla_status)-99), "unknown status") == 0);
  EXPECT_TRUE(std::strstr(mla_version(), "libmla") != nullptr);

  mla_config c = dsv3();
  EXPECT_EQ(mla_cache_bytes_per_token(&c), 1152);
  c.cache_dtype = MLA_CACHE_FP8_E4M3;
  EXPECT_EQ(mla_cache_bytes_per_token(&c), 656);
  EXPECT_EQ(mla_cache_bytes_per_token(nullptr), 0);
  c = dsv3();
  c.d_rope = 63;
  EXPECT_EQ(mla_cache_bytes_per_token(&c), 0);

  size_t bytes = 0;
  c = dsv3();
  EXPECT_EQ(mla_workspace_size(&c, 1, 32, 1, 4096, &bytes), MLA_OK);
  EXPECT_TRUE(bytes > 0);
  EXPECT_EQ(mla_workspace_size(&c, 7, 1, 1, 1, &bytes), MLA_ERR_SHAPE);
  EXPECT_EQ(mla_workspace_size(&c, 1, 0, 1, 10, &bytes), MLA_ERR_SHAPE);
  EXPECT_EQ(mla_workspace_size(&c, 0, 1, 1, 0, nullptr), MLA_ERR_NULL);
  EXPECT_EQ(mla_workspace_size(nullptr, 0, 1, 1, 0, &bytes), MLA_ERR_NULL);

  const mla_weights w = fake_weights();
  mla_weights wnull = w;
  wnull.w_uk = nullptr;
  mla_cache k16 = contiguous(16), k64 = contiguous(64);
  // prefill
  EXPECT_EQ(mla_prefill(&c, &wnull, FAKE, 1, 16, &k16, FAKE, nullptr, FAKE, 1ull << 40, nullptr), MLA_ERR_NULL);
  EXPECT_EQ(mla_prefill(&c, &w, nullptr, 1, 16, &k16, FAKE, nullptr, FAKE, 1ull << 40, nullptr), MLA_ERR_NULL);
  EXPECT_EQ(mla_prefill(&c, &w, FAKE, 0, 16, &k16, FAKE, nullptr, FAKE, 1ull << 40, nullptr), MLA_ERR_SHAPE);
  mla_cache k8 = contiguous(8);
  EXPECT_EQ(mla_prefill(&c, &w, FAKE, 1, 16, &k8, FAKE, nullptr, FAKE, 1ull << 40, nullptr), MLA_ERR_CACHE);
  mla_cache pbad = paged(4, 4, 3);
  EXPECT_EQ(mla_prefill(&c, &w, FAKE, 1, 16, &pbad, FAKE, nullptr, FAKE, 1ull << 40, nullptr), MLA_ERR_CACHE);
  EXPECT_EQ(mla_prefill(&c, &w, FAKE, 1, 16, &k16, FAKE, nullptr, FAKE, 1024, nullptr), MLA_ERR_WORKSPACE);
  // decode
  const int32_t lens_ok[2] = {5, 64}, lens_long[2] = {5, 65}, lens_zero[2] = {0, 3};
  EXPECT_EQ(mla_decode(&c, &w, FAKE, 2, 1, nullptr, nullptr, 64, &k64, FAKE, nullptr, FAKE, 1ull << 40, nullptr),
            MLA_ERR_NULL);
  EXPECT_EQ(mla_decode(&c, &w, FAKE, 2, 65, (const int32_t *)FAKE, nullptr, 64, &k64, FAKE, nullptr, FAKE,
                       1ull << 40, nullptr), MLA_ERR_SHAPE);
  EXPECT_EQ(mla_decode(&c, &w, FAKE, 2, 1, (const int32_t *)FAKE, nullptr, 128, &k64, FAKE, nullptr, FAKE,
                       1ull << 40, nullptr), MLA_ERR_CACHE);
  EXPECT_EQ(mla_decode(&c, &w, FAKE, 2, 1, (const int32_t *)FAKE, lens_long, 64, &k64, FAKE, nullptr, FAKE,
                       1ull << 40, nullptr), MLA_ERR_SHAPE);
  EXPECT_EQ(mla_decode(&c, &w, FAKE, 2, 1, (const int32_t *)FAKE, lens_zero, 64, &k64, FAKE, nullptr, FAKE,
                       1ull << 40, nullptr), MLA_ERR_SHAPE);
  EXPECT_EQ(mla_decode(&c, &w, FAKE, 2, 1, (const int32_t *)FAKE, lens_ok, 64, &k64, FAKE, nullptr, nullptr,
                       1ull << 40, nullptr), MLA_ERR_WORKSPACE);
  EXPECT_EQ(mla_decode(&c, &w, FAKE, 2, 1, (const int32_t *)FAKE, lens_ok, 64, &k64, FAKE, nullptr, FAKE, 100,
                       nullptr), MLA_ERR_WORKSPACE);
  // the allocation-free decode: a workspace above its array is refused
  EXPECT_EQ(mla_decode_noalloc(&c, &w, FAKE, 2, 300, (const int32_t *)FAKE, nullptr, 633, &k64, FAKE, nullptr,
                               nullptr), MLA_ERR_CACHE);
  mla_cache k633 = contiguous(633);
  EXPECT_EQ(mla_decode_noalloc(&c, &w, FAKE, 2, 300, (const int32_t *)FAKE, nullptr, 633, &k633, FAKE, nullptr,
                               nullptr), MLA_ERR_WORKSPACE);
  // compression
  EXPECT_EQ(mla_compress_kv(&c, &w, FAKE, 0, (const int32_t *)FAKE, (const int32_t *)FAKE, 1, &k16, nullptr, 0,
                            nullptr),
            MLA_ERR_SHAPE);
  mla_cache k0 = contiguous(0);
  EXPECT_EQ(mla_compress_kv(&c, &w, FAKE, 4, (const int32_t *)FAKE, (const int32_t *)FAKE, 1, &k0, nullptr, 0,
                            nullptr),
            MLA_ERR_CACHE);
  c.cache_dtype = MLA_CACHE_FP8_E4M3;
  // the FP8 cache's rows are staged in the workspace: none, or too small
  EXPECT_EQ(mla_workspace_size(&c, MLA_OP_COMPRESS, 1, 4, 0, &bytes), MLA_OK);
  EXPECT_TRUE(bytes > 0);
  EXPECT_EQ(mla_compress_kv(&c, &w, FAKE, 4, (const int32_t *)FAKE, (const int32_t *)FAKE, 1, &k16, nullptr, 0,
                            nullptr),
            MLA_ERR_WORKSPACE);
  EXPECT_EQ(mla_compress_kv(&c, &w, FAKE, 4, (const int32_t *)FAKE, (const int32_t *)FAKE, 1, &k16, FAKE, bytes - 1,
                            nullptr),
            MLA_ERR_WORKSPACE);
  // block-scaled FP8 projections
  c = dsv3();
  c.weight_dtype = MLA_WEIGHTS_FP8_BLOCK;
  EXPECT_EQ(mla_workspace_size(&c, 1, 32, 1, 4096, &bytes), MLA_OK);
  mla_weights wns = w;
  wns.s_o = nullptr;
  EXPECT_EQ(mla_prefill(&c, &wns, FAKE, 1, 16, &k16, FAKE, nullptr, FAKE, 1ull << 40, nullptr), MLA_ERR_NULL);
  EXPECT_EQ(mla_compress_kv(&c, &w, FAKE, 4, (const int32_t *)FAKE, (const int32_t *)FAKE, 1, &k16, nullptr, 0,
                            nullptr),
            MLA_ERR_WORKSPACE);
  mla_weights wnk = w;
  wnk.s_kr = nullptr;   // the compression reads W_KR's scales
  EXPECT_EQ(mla_compress_kv(&c, &wnk, FAKE, 4, (const int32_t *)FAKE, (const int32_t *)FAKE, 1, &k16, FAKE,
                            1ull << 40, nullptr),
            MLA_ERR_NULL);
  c.weight_dtype = 5;
  EXPECT_EQ(mla_workspace_size(&c, 1, 32, 1, 4096, &bytes), MLA_ERR_DTYPE);
  c.weight_dtype = MLA_WEIGHTS_FP8_BLOCK;
  c.d_model = 7168 + 64;
  EXPECT_EQ(mla_workspace_size(&c, 1, 32, 1, 4096, &bytes), MLA_ERR_UNSUPPORTED);
}

// Random configurations and sizes: any status is acceptable, but no call may
// touch the GPU (each has a 1-byte workspace or a NULL), and the host code
// must stay free of undefined behaviour and out-of-bounds reads.
void sweeps(int n) {
  const mla_weights w = fake_weights();
  int32_t lens_host[64];
  for (int it = 0; it < n; ++it) {
    mla_config c = dsv3();
    switch (next_u64() % 4) {
      case 0: c.d_model = pick_i32(); break;
      case 1: c.n_heads = pick_i32(); c.d_v = pick_i32(); break;
      case 2: c.d_c = pick_i32(); c.d_rope = pick_i32(); c.d_cq = pick_i32(); break;
      default: c.d_nope = pick_i32(); break;
    }
    if (next_u64() % 3 == 0) c.dtype = pick_i32() & 3;
    if (next_u64() % 3 == 0) c.cache_dtype = pick_i32() & 3;
    if (next_u64() % 3 == 0) c.weight_dtype = pick_i32() & 3;
    if (next_u64() % 4 == 0) {
      c.yarn_factor = pick_f64();
      c.yarn_beta_slow = pick_f64();
      c.yarn_beta_fast = pick_f64();
      c.yarn_orig_len = pick_i32();
    }
    if (next_u64() % 8 == 0) c.rope_base = pick_f64();
    const int32_t b = pick_i32(), n = pick_i32(), ml = pick_i32();
    size_t bytes = 0;
    (void)mla_cache_bytes_per_token(&c);
    (void)mla_workspace_size(&c, (int32_t)(next_u64() % 3), b, n, ml, &bytes);
    mla_cache kc = contiguous(ml);
    mla_cache kp = paged(pick_i32(), pick_i32(), pick_i32());
    const mla_cache *kk = (next_u64() & 1) ? &kc : &kp;
    // a workspace of one byte: every call that passes the other checks stops here
    const mla_status sp = mla_prefill(&c, &w, FAKE, b, n, kk, FAKE, nullptr, FAKE, 1, nullptr);
    EXPECT_TRUE(sp != MLA_OK && sp != MLA_ERR_HIP);
    const int32_t nb = (b > 0 && b <= 64) ? b : 0;
    for (int i = 0; i < nb; ++i) lens_host[i] = pick_i32();
    const mla_status sd = mla_decode(&c, &w, FAKE, b, n, (const int32_t *)FAKE, nb ? lens_host : nullptr, ml, kk,
                                     FAKE, nullptr, FAKE, 1, nullptr);
    EXPECT_TRUE(sd != MLA_OK && sd != MLA_ERR_HIP);
    // the allocation-free decode: validation only (NULL output stops it)
    const mla_status sn = mla_decode_noalloc(&c, &w, FAKE, b, n, (const int32_t *)FAKE, nb ? lens_host : nullptr, ml,
                                             kk, nullptr, nullptr, nullptr);
    EXPECT_TRUE(sn != MLA_OK && sn != MLA_ERR_HIP);
    // compression with a NULL position array
    const mla_status sc = mla_compress_kv(&c, &w, FAKE, n, (const int32_t *)FAKE, nullptr, b, kk, nullptr, 0, nullptr);
    EXPECT_TRUE(sc != MLA_OK && sc != MLA_ERR_HIP);
  }
}

}  // namespace

int main() {
  fixed_cases();
  sweeps(20000);
  std::printf("abi sanitize driver: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
