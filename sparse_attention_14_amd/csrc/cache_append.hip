// Cache append: the new tokens' indexer keys and latent rows written into
// contiguous or paged caches, the step that puts a token in place before any
// query sees it ("GLM on an A100, in Vx", section "The model": a query scores
// every earlier token, its own included).  fp8 key caches receive e4m3fn bytes
// with a float32 scale per token ("INT4, FP8 and BF16": FP8 is E4M3 with float32
// scales): s = max(amax / 448, 2^-126), byte = nearest e4m3fn code of k / s
// (ties to even, saturating at 448), every decision in float32.
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

struct AppendArgs {
  CacheDev keys;
  int key_dt;          // -1: no key cache
  const uint8_t *new_keys;
  int new_key_dt;      // kF32 or kBF16
  CacheDev latent;
  int has_latent;
  const uint8_t *new_latent;
  int latent_row_bytes;
  const int32_t *seq;
  const int32_t *pos;
};

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  const int b = a.seq ? a.seq[i] : 0;
  const int t = a.pos[i];
  if (a.key_dt >= 0) {
    const int D = a.keys.width;
    int64_t block;
    int slot;
    uint8_t *dst = row_ptr(a.keys, b, t, block, slot);
    if (a.key_dt == kFP8) {
      // Lane l holds elements l and l + 64 (widths up to 128).
      float v[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int d = lane + 64 * j;
        float x = 0.0f;
        if (d < D) {
          const int64_t e = (int64_t)i * D + d;
          x = a.new_key_dt == kBF16 ? bf16_bits_to_float(reinterpret_cast<const uint16_t *>(a.new_keys)[e])
                                    : reinterpret_cast<const float *>(a.new_keys)[e];
        }
        v[j] = x;
      }
      const float amax = wave_max(fmaxf(fabsf(v[0]), fabsf(v[1])));
      const float s = fmaxf(amax / 448.0f, 0x1p-126f);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int d = lane + 64 * j;
        if (d < D) dst[d] = (uint8_t)e4m3fn_code(v[j] / s);
      }
      if (lane == 0) const_cast<float *>(a.keys.scale)[block * a.keys.scale_block_stride + slot] = s;
    } else {
      const int eb = a.key_dt == kF32 ? 4 : 2;
      const int chunks = D * eb / 16;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(a.new_keys + (int64_t)i * D * eb);
      for (int c = lane; c < chunks; c += kAppendThreads) reinterpret_cast<u32x4 *>(dst)[c] = src[c];
    }
  }
  if (a.has_latent) {
    int64_t block;
    int slot;
    uint8_t *dst = row_ptr(a.latent, b, t, block, slot);
    const int chunks = a.latent_row_bytes / 16;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.new_latent + (int64_t)i * a.latent_row_bytes);
    for (int c = lane; c < chunks; c += kAppendThreads) reinterpret_cast<u32x4 *>(dst)[c] = src[c];
  }
}

}  // namespace

hipError_t launch_cache_append(const CacheDev *keys, int key_dt, const void *new_keys, int new_key_dt,
                               const CacheDev *latent, int latent_row_bytes, const void *new_latent,
                               const int32_t *seq, const int32_t *pos, int n_new, hipStream_t stream) {
  AppendArgs a{};
  a.key_dt = keys ? key_dt : -1;
  if (keys) a.keys = *keys;
  a.new_keys = static_cast<const uint8_t *>(new_keys);
  a.new_key_dt = new_key_dt;
  a.has_latent = latent != nullptr;
  if (latent) a.latent = *latent;
  a.new_latent = static_cast<const uint8_t *>(new_latent);
  a.latent_row_bytes = latent_row_bytes;
  a.seq = seq;
  a.pos = pos;
  hipLaunchKernelGGL(append_kernel, dim3(n_new), dim3(kAppendThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
