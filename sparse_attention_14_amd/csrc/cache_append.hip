// Cache append: the new tokens' indexer keys and latent rows written into
// contiguous or paged caches, the step that puts a token in place before any
// query sees it ("GLM on an A100, in Vx", section "The model": a query scores
// every earlier token, its own included).  fp8 caches (keys, or latent rows)
// receive e4m3fn bytes with a float32 scale per token ("INT4, FP8 and BF16":
// FP8 is E4M3 with float32 scales): s = max(amax / 448, 2^-126) over the row,
// byte = nearest e4m3fn code of x / s (ties to even, saturating at 448), every
// decision in float32.
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int kAppendThreads = 64;   // one wavefront per new token

// Nearest e4m3fn code of a finite float32 (ties to the even code, magnitudes
// at or above 448 saturated, the sign bit kept).  Integer arithmetic on the
// bits only, so the result does not depend on the denormal mode.
__device__ __forceinline__ uint32_t e4m3fn_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t sign = (u >> 24) & 0x80u;
  uint32_t code;
  if (a >= 0x43E00000u) {
    code = 0x7Eu;                                    // |x| >= 448
  } else if (a >= 0x3C800000u) {
    // |x| >= 2^-6, a normal e4m3fn value: keep 3 of the 23 mantissa bits,
    // rounding the other 20 to nearest even; a carry moves into the exponent.
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);                  // exponent bias 127 -> 7
  } else {
    // Below 2^-6: a multiple of 2^-9 (subnormal e4m3fn, codes 0..8).  The
    // value is m * 2^(e - 150) with m the 24-bit significand, i.e. m >> sh
    // units of 2^-9, sh = 141 - e >= 21.
    const uint32_t e = a >> 23;
    const uint32_t m = e ? ((a & 0x7FFFFFu) | 0x800000u) : a;
    const uint32_t sh = min(141u - max(e, 1u), 31u);
    const uint32_t q = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1u);
    code = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  return sign | code;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint8_t *row_ptr(const CacheDev &c, int seq, int t, int64_t &block, int &slot) {
  block = cache_block(c, seq, t, slot);
  return const_cast<uint8_t *>(cache_row(c, block, slot));
}

struct AppendCache {
  CacheDev c;
  int dt;              // cache dtype; -1: this cache is not written
  const uint8_t *src;  // [n_new][width] new rows
  int src_dt;          // dtype of the new rows (kF32 or kBF16; the cache's own dtype for copies)
};

struct AppendArgs {
  AppendCache cache[2];   // keys, latent
  const int32_t *seq;
  const int32_t *pos;
};

constexpr int kMaxQuantWidth = 1024;   // elements of an fp8 row quantized by one wavefront

// Token i's row into cache slot (b, t): fp8 caches quantized with the row's
// own scale, other caches copied as 16-byte chunks.
__device__ __forceinline__ void write_row(const AppendCache &w, int i, int b, int t, int lane) {
  const int W = w.c.width;
  int64_t block;
  int slot;
  uint8_t *dst = row_ptr(w.c, b, t, block, slot);
  if (w.dt == kFP8) {
    // lane l holds elements l + 64 j
    float v[kMaxQuantWidth / 64];
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxQuantWidth / 64; ++j) {
      const int d = lane + 64 * j;
      float x = 0.0f;
      if (d < W) {
        const int64_t e = (int64_t)i * W + d;
        x = w.src_dt == kBF16 ? bf16_bits_to_float(reinterpret_cast<const uint16_t *>(w.src)[e])
                              : reinterpret_cast<const float *>(w.src)[e];
      }
      v[j] = x;
      am = fmaxf(am, fabsf(x));
    }
    const float s = fmaxf(wave_max(am) / 448.0f, 0x1p-126f);
#pragma unroll
    for (int j = 0; j < kMaxQuantWidth / 64; ++j) {
      const int d = lane + 64 * j;
      if (d < W) dst[d] = (uint8_t)e4m3fn_code(v[j] / s);
    }
    if (lane == 0) const_cast<float *>(w.c.scale)[block * w.c.scale_block_stride + slot] = s;
  } else {
    const int eb = w.dt == kF32 ? 4 : 2;
    const int chunks = W * eb / 16;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(w.src + (int64_t)i * W * eb);
    for (int c = lane; c < chunks; c += kAppendThreads) reinterpret_cast<u32x4 *>(dst)[c] = src[c];
  }
}

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  const int b = a.seq ? a.seq[i] : 0;
  const int t = a.pos[i];
  if (a.cache[0].dt >= 0) write_row(a.cache[0], i, b, t, lane);
  if (a.cache[1].dt >= 0) write_row(a.cache[1], i, b, t, lane);
}

}  // namespace

hipError_t launch_cache_append(const CacheDev *keys, int key_dt, const void *new_keys, int new_key_dt,
                               const CacheDev *latent, int latent_dt, const void *new_latent, int new_latent_dt,
                               const int32_t *seq, const int32_t *pos, int n_new, hipStream_t stream) {
  AppendArgs a{};
  a.cache[0].dt = keys ? key_dt : -1;
  if (keys) a.cache[0].c = *keys;
  a.cache[0].src = static_cast<const uint8_t *>(new_keys);
  a.cache[0].src_dt = new_key_dt;
  a.cache[1].dt = latent ? latent_dt : -1;
  if (latent) a.cache[1].c = *latent;
  a.cache[1].src = static_cast<const uint8_t *>(new_latent);
  a.cache[1].src_dt = new_latent_dt;
  a.seq = seq;
  a.pos = pos;
  hipLaunchKernelGGL(append_kernel, dim3(n_new), dim3(kAppendThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
