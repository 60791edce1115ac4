// Device-side building blocks shared by the libdsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kWave = 64;
constexpr int kHistBins = 4096;     // first radix level: top 12 bits of the ordered key
constexpr int kHistShift = 20;

// Cache descriptor as the kernels see it (mirrors dsa_cache; all byte strides).
struct CacheDev {
  const uint8_t *rows;
  const float *scale;
  int64_t row_stride;
  int64_t block_stride;
  int64_t scale_block_stride;
  const int32_t *table;
  int32_t block_size;
  int32_t max_blocks;
  int32_t width;
};

// Sequence of query qi: from q_seq, else qi itself (ident) or 0.
__device__ __forceinline__ int seq_of(const int32_t *q_seq, int qi, int ident) {
  return q_seq ? q_seq[qi] : (ident ? qi : 0);
}

// Physical block of token t of sequence seq and the token's slot inside it.
__device__ __forceinline__ int64_t cache_block(const CacheDev &c, int seq, int t, int &slot) {
  const int blk = t / c.block_size;
  slot = t - blk * c.block_size;
  return c.table ? (int64_t)c.table[(int64_t)seq * c.max_blocks + blk] : (int64_t)seq;
}

__device__ __forceinline__ const uint8_t *cache_row(const CacheDev &c, int64_t block, int slot) {
  return c.rows + block * c.block_stride + (int64_t)slot * c.row_stride;
}

// Order-preserving 32-bit image of a float score: a > b as numbers <=> key(a) > key(b);
// -0.0 and +0.0 share one key, every NaN maps to 0, below -inf (whose key is 0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Two e4m3fn bytes (bits [15:0] or [31:16] of w) -> two bf16, exact: every
// e4m3fn value, subnormals included, is representable in bf16.
template <bool HI>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// 8 e4m3fn bytes (two dwords) -> 8 bf16 MFMA operand elements in memory order.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  bf16x2 a = fp8x2_to_bf16x2<false>(w0), b = fp8x2_to_bf16x2<true>(w0);
  bf16x2 c = fp8x2_to_bf16x2<false>(w1), d = fp8x2_to_bf16x2<true>(w1);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte global load (the address must be 16-byte aligned).
__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x4 load16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Direct-to-LDS copies (global_load_lds): the bytes go from memory into LDS
// without passing through registers.  One instruction: lane l's 16 (or 4) bytes
// land at lds + 16 l (4 l).  Issued as assembly so that the compiler does not
// order later LDS reads behind them: it cannot tell which LDS bytes a copy
// writes and would otherwise make every LDS read wait for every copy in flight
// (the next step's included).  The caller waits for its copies itself
// (wait_copies, wait_vm) before their bytes are read.
__device__ __forceinline__ uint32_t lds_address(const void *lds) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t *)lds);
}
__device__ __forceinline__ void copy16_to_lds(const uint8_t *src, uint8_t *lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_address(lds)) : "memory");
}
// The same from a wavefront-uniform base plus a 32-bit lane offset.
__device__ __forceinline__ void copy16_to_lds(const uint8_t *base, uint32_t off, uint8_t *lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_address(lds))
               : "memory");
}
__device__ __forceinline__ void copy4_to_lds(const uint8_t *base, uint32_t off, uint8_t *lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_address(lds))
               : "memory");
}

// Waits for every vector-memory operation of the wavefront (its copies
// included), and keeps the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void wait_copies() {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// Waits until at most N vector-memory operations of the wavefront are in
// flight, also as a compiler memory barrier.  Loads and copies complete in the
// order they were issued, so the copies issued more than N such operations ago
// are then in LDS; stores may complete in any order and are not counted by
// callers (a store in flight only makes the wait longer).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// The same, and every LDS access of the wavefront done (so that a buffer it
// has read can be handed to new copies).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("" ::: "memory");
}

// Agent-scope release/acquire around the "last workgroup finishes" handshake.
__device__ __forceinline__ void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves (ALU
// only): row_shr 1, 2, 4, 8 scans each 16-lane row, then row_bcast 15 and
// row_bcast 31 carry the row totals forward.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  // dpp_ctrl: row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
  return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(x), 63);
}

// Minimum / maximum over the lanes of a wavefront (DPP; result in every lane).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x111, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x112, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x114, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x118, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x142, 0xA, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Largest key prefix T (the top `bits` bits; the rest zero) such that at least
// `need` of the keys x[0..N) held by the lanes of one wavefront are >= T: a lower
// bound on the need-th largest key.  Called by a whole wavefront.
template <int N>
__device__ __forceinline__ uint32_t wave_rank_bound(const uint32_t (&x)[N], uint32_t need, int bits) {
  // one bit per step from the top; the count of keys >= the trial prefix is a
  // sum of ballot population counts (scalar), not a cross-lane reduction
  uint32_t T = 0;
  for (int b = 31; b >= 32 - bits; --b) {
    const uint32_t c = T | (1u << b);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) m += (uint32_t)__popcll(__ballot(x[i] >= c));
    if (m >= need) T = c;
  }
  return T;
}

// Candidate bounds for the top-k.  A row is cut into groups; each of its G
// full groups reports a value with at least r distinct keys of the group at or
// above it (r = bound_rank(k, G, most)), the rest report 0.  The ceil(k / r)-th
// largest report then has at least k keys of the row at or above it.  r is half
// again the smallest rank that would make the minimum report a bound, which
// makes the chosen report a quantile of the groups instead of their minimum
// (fewer candidates).  0: no bound (a group offers at most `most` ranks).
__host__ __device__ inline int bound_rank(int k, int groups, int most) {
  if (groups <= 0 || k <= 0) return 0;
  const int base = (k + groups - 1) / groups;
  if (base > most) return 0;
  const int r = (3 * base + 1) / 2;
  return r > most ? most : r;
}

// Block-wide exclusive prefix sum of one uint32 per thread, in thread order.
// scratch: >= blockDim.x / 64 + 1 words of LDS.  Returns the exclusive prefix;
// *total receives the block sum.  All threads must call it.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch, uint32_t *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int i = 0; i < nwaves; ++i) {
    const uint32_t t = scratch[i];
    before += i < wave ? t : 0u;
    all += t;
  }
  *total = all;
  __syncthreads();
  return before + x - v;
}

}  // namespace dsa
