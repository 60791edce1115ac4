// Absorbed-MLA projections around the sparse attention ("Self-contained GLM-5
// serving stack", component list: absorbed MLA decode): per head h, a GEMM
//     C[i][h][n] = sum_k A[i][h][k] * B[h][k][n]
// with bf16 weights B.  Query absorption: A = q_nope (bf16), B = W_UK, C = the
// bf16 MLA query (its rope part copied behind the kv_lora columns).  Output
// projection: A = the fp32 attention output, split exactly enough into bf16
// hi + lo parts (two MFMAs), B = W_UV, C fp32.
//
// A workgroup (4 wavefronts) owns 64 rows x 64 columns of one head; K goes in
// steps of 32 through LDS: the A tile row-major (the MFMA A operand is 8
// consecutive k of one row per lane), the B tile row-major and read back
// transposed (ds_read_b64_tr_b16) into the B operand.  Wavefront w computes
// columns 16 w .. 16 w + 15 for all 64 rows (four 16x16x32 bf16 MFMA tiles).
// The next step's global loads are issued before the current step's MFMAs.
#include "kernels.hpp"

namespace dsa {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

constexpr int kAbBM = 64, kAbBN = 64, kAbBK = 32;
constexpr int kAbThreads = 256;
constexpr int kAStride = kAbBK + 8;          // bf16 per LDS row of the A tile (padded)
constexpr int kBStrideBytes = kAbBN * 2 + 16;  // bytes per LDS row of the B tile (padded)

struct AbsorbArgs {
  const void *a;        // [M][H][K], bf16 or f32
  const uint16_t *b;    // [H][K][N] bf16
  void *c;              // [M][H][ldc] (bf16 or f32), columns [0, N)
  int M, H, K, N, ldc;
  const uint16_t *rope;  // [M][H][R] bf16, copied to C columns [N, N + R) (query absorption only)
  int R;
};

__device__ __forceinline__ i16x4 lds_tr(const uint8_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(reinterpret_cast<uintptr_t>(p)));
}

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Rope columns of the MLA query for rows [m0, m0 + rows) of head h, in 16-byte
// chunks whose loads are all issued before the (non-temporal) stores (R is a
// multiple of 8).
__device__ __forceinline__ void copy_rope(const AbsorbArgs &a, int h, int m0, int rows) {
  const int cpr = a.R / 8;
  const int nch = rows * cpr;
  for (int base = 0; base < nch; base += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ch = min(base + (int)threadIdx.x + 256 * j, nch - 1);
      const int r = ch / cpr, c = ch - r * cpr;
      const int m = min(m0 + r, a.M - 1);
      v[j] = *reinterpret_cast<const u32x4 *>(a.rope + ((int64_t)m * a.H + h) * a.R + 8 * c);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ch = base + (int)threadIdx.x + 256 * j;
      const int r = ch / cpr, c = ch - r * cpr;
      if (ch < nch && m0 + r < a.M)
        __builtin_nontemporal_store(
            v[j], reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.c) + ((int64_t)(m0 + r) * a.H + h) * a.ldc +
                                            a.N + 8 * c));
    }
  }
}

template <bool A_F32, bool C_BF16>
__global__ __launch_bounds__(kAbThreads) void absorb_kernel(AbsorbArgs a) {
  __shared__ __align__(16) uint16_t la[2][kAbBM * kAStride];   // A tile: hi, lo (lo only for fp32 A)
  __shared__ __align__(16) uint8_t lb[kAbBK * kBStrideBytes];

  const int nblk = a.N / kAbBN;
  const int nb = blockIdx.x % nblk;
  const int rest = blockIdx.x / nblk;
  const int h = rest % a.H;
  const int m0 = (rest / a.H) * kAbBM;
  const int n0 = nb * kAbBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t arow = (int64_t)a.H * a.K;   // elements between consecutive rows of A

  // global -> register staging: A 64 x 32 (thread t: row t / 4, k 8 (t % 4) .. + 8),
  // B 32 x 64 (thread t: row t / 8, columns 8 (t % 8) .. + 8)
  const int ar = tid >> 2, ak = 8 * (tid & 3);
  const int br = tid >> 3, bc = 8 * (tid & 7);
  const bool arow_ok = m0 + ar < a.M;
  u32x4 ra0{}, ra1{}, rb{};
  auto load = [&](int k0) {
    if (A_F32) {
      const float *src = static_cast<const float *>(a.a) + (int64_t)(m0 + ar) * arow + (int64_t)h * a.K + k0 + ak;
      ra0 = arow_ok ? *reinterpret_cast<const u32x4 *>(src) : u32x4{};
      ra1 = arow_ok ? *reinterpret_cast<const u32x4 *>(src + 4) : u32x4{};
    } else {
      const uint16_t *src =
          static_cast<const uint16_t *>(a.a) + (int64_t)(m0 + ar) * arow + (int64_t)h * a.K + k0 + ak;
      ra0 = arow_ok ? *reinterpret_cast<const u32x4 *>(src) : u32x4{};
    }
    rb = *reinterpret_cast<const u32x4 *>(a.b + ((int64_t)h * a.K + k0 + br) * a.N + n0 + bc);
  };
  auto stage = [&]() {
    if (A_F32) {
      uint16_t hi[8], lo[8];
      const float f[8] = {__uint_as_float(ra0[0]), __uint_as_float(ra0[1]), __uint_as_float(ra0[2]),
                          __uint_as_float(ra0[3]), __uint_as_float(ra1[0]), __uint_as_float(ra1[1]),
                          __uint_as_float(ra1[2]), __uint_as_float(ra1[3])};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = to_bf16_rne(f[e]);
        lo[e] = to_bf16_rne(f[e] - __uint_as_float((uint32_t)hi[e] << 16));
      }
      u32x4 vh, vl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vh[e] = (uint32_t)hi[2 * e] | ((uint32_t)hi[2 * e + 1] << 16);
        vl[e] = (uint32_t)lo[2 * e] | ((uint32_t)lo[2 * e + 1] << 16);
      }
      *reinterpret_cast<u32x4 *>(&la[0][ar * kAStride + ak]) = vh;
      *reinterpret_cast<u32x4 *>(&la[1][ar * kAStride + ak]) = vl;
    } else {
      *reinterpret_cast<u32x4 *>(&la[0][ar * kAStride + ak]) = ra0;
    }
    *reinterpret_cast<u32x4 *>(lb + br * kBStrideBytes + bc * 2) = rb;
  };

  f32x4 acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / kAbBK;
  load(0);
  for (int ks = 0; ks < nk; ++ks) {
    __syncthreads();                   // the previous step's LDS reads are done
    stage();
    __syncthreads();
    if (ks + 1 < nk) load((ks + 1) * kAbBK);
    // B operand: rows (k) 8 g4 .. 8 g4 + 7 of column 16 wave + l16, two transposed reads
    const uint8_t *vb = lb + (8 * g4 + (l16 >> 2)) * kBStrideBytes + (16 * wave + 4 * (l16 & 3)) * 2;
    const i16x4 v0 = lds_tr(vb), v1 = lds_tr(vb + 4 * kBStrideBytes);
    const bf16x8 bop = __builtin_bit_cast(
        bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1],
                                                                             v1[2], v1[3]});
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                         &la[0][(16 * rt + l16) * kAStride + 8 * g4]));
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bop, acc[rt], 0, 0, 0);
      if (A_F32) {
        const bf16x8 alo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                           &la[1][(16 * rt + l16) * kAStride + 8 * g4]));
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bop, acc[rt], 0, 0, 0);
      }
    }
  }

  // epilogue: acc[rt][i] is C[row 16 rt + 4 g4 + i][column 16 wave + l16]
  const int col = n0 + 16 * wave + l16;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * rt + 4 * g4 + i;
      if (m < a.M) {
        const int64_t off = ((int64_t)m * a.H + h) * a.ldc + col;
        if (C_BF16)
          static_cast<uint16_t *>(a.c)[off] = to_bf16_rne(acc[rt][i]);
        else
          static_cast<float *>(a.c)[off] = acc[rt][i];
      }
    }
  }
  // rope columns of the MLA query, copied by the workgroups of the first column block
  if (a.rope && nb == 0) copy_rope(a, h, m0, kAbBM);
}


__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Few rows (decode): the weights dominate, so the kernel is a GEMV streaming
// them.  A workgroup owns one head and a block of 8 CPR columns; thread t reads
// 16-byte chunk t % CPR of rows t / CPR + (256 / CPR) p, with every load of a
// batch of 8 rows in flight, and accumulates all M rows in float32 (A from
// LDS).  Partial sums over rows are reduced across the lanes of a wavefront
// (xor shuffles) and then across the 4 wavefronts in a fixed order.
constexpr int kGemvMaxM = 8;
constexpr int kGemvMaxA = 8192;   // M * K floats in LDS

template <bool A_F32, bool C_BF16, int CPR, int MQ>
__global__ __launch_bounds__(256) void absorb_gemv_kernel(AbsorbArgs a) {
  constexpr int BN = 8 * CPR;
  constexpr int RG = 256 / CPR;           // rows in flight per pass
  constexpr int EPC = A_F32 ? 4 : 8;      // A elements per 16-byte chunk
  __shared__ __align__(16) float la[kGemvMaxA];
  __shared__ float red[4][MQ][BN];
  const int nblk = a.N / BN;
  const int nb = blockIdx.x % nblk;
  const int h = blockIdx.x / nblk;
  const int n0 = nb * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const int c = tid % CPR, g = tid / CPR;
  const int passes = K / RG;
  // issue order: A chunks, weight rows, the rope chunk; the A staging waits for the first only
  const int cpr = K / EPC;
  const int nch = MQ * cpr;               // <= 2048: at most 8 per thread
  u32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int ch = min(tid + 256 * j, nch - 1);
    const int i = ch / cpr, kc = ch - i * cpr;
    v[j] = *reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(a.a) +
                                            (((int64_t)i * a.H + h) * K + kc * EPC) * (A_F32 ? 4 : 2));
  }
  const uint16_t *wb = a.b + (int64_t)h * K * a.N + n0 + 8 * c;
  u32x4 w[8];
  auto load_w = [&](int p0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = min(p0 + j, passes - 1);
      w[j] = *reinterpret_cast<const u32x4 *>(wb + (int64_t)(g + RG * p) * a.N);
    }
  };
  load_w(0);
  const bool rope = a.rope && nb == 0;
  const int rcpr = a.R / 8;               // rope chunks per row (MQ * rcpr <= 1024)
  u32x4 rv[4];
  if (rope) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = min(tid + 256 * j, MQ * rcpr - 1);
      const int i = ch / rcpr, rc = ch - i * rcpr;
      rv[j] = *reinterpret_cast<const u32x4 *>(a.rope + ((int64_t)i * a.H + h) * a.R + 8 * rc);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int ch = tid + 256 * j;
    if (ch < nch) {
      const int i = ch / cpr, kc = ch - i * cpr;
      float *dst = la + i * K + kc * EPC;
      if (A_F32) {
        *reinterpret_cast<u32x4 *>(dst) = v[j];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[2 * e] = bf16_lo(v[j][e]);
          dst[2 * e + 1] = bf16_hi(v[j][e]);
        }
      }
    }
  }
  __syncthreads();
  float acc[MQ][8];
#pragma unroll
  for (int i = 0; i < MQ; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
  for (int p0 = 0; p0 < passes; p0 += 8) {
    if (p0 > 0) load_w(p0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (p0 + j < passes) {
        const int k = g + RG * (p0 + j);
        const float wf[8] = {bf16_lo(w[j][0]), bf16_hi(w[j][0]), bf16_lo(w[j][1]), bf16_hi(w[j][1]),
                             bf16_lo(w[j][2]), bf16_hi(w[j][2]), bf16_lo(w[j][3]), bf16_hi(w[j][3])};
#pragma unroll
        for (int i = 0; i < MQ; ++i) {
          const float av = la[i * K + k];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(av, wf[e], acc[i][e]);
        }
      }
    }
  }
  // lanes l, l + CPR, l + 2 CPR, ... of a wavefront hold the same columns
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[i][e];
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1) x += __shfl_xor(x, o);
      acc[i][e] = x;
    }
  }
  if (lane < CPR) {
#pragma unroll
    for (int i = 0; i < MQ; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][i][8 * lane + e] = acc[i][e];
  }
  __syncthreads();
  for (int o = tid; o < MQ * BN; o += 256) {
    const int i = o / BN, col = o - i * BN;
    const float x = ((red[0][i][col] + red[1][i][col]) + red[2][i][col]) + red[3][i][col];
    const int64_t off = ((int64_t)i * a.H + h) * a.ldc + n0 + col;
    if (C_BF16)
      static_cast<uint16_t *>(a.c)[off] = to_bf16_rne(x);
    else
      static_cast<float *>(a.c)[off] = x;
  }
  if (rope) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = tid + 256 * j;
      if (ch < MQ * rcpr) {
        const int i = ch / rcpr, rc = ch - i * rcpr;
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.c) + ((int64_t)i * a.H + h) * a.ldc + a.N + 8 * rc) =
            rv[j];
      }
    }
  }
}

template <bool A_F32, bool C_BF16, int CPR>
hipError_t launch_gemv(const AbsorbArgs &args, dim3 grid, hipStream_t stream) {
  switch (args.M) {
#define DSA_GEMV(MQV) \
  case MQV: hipLaunchKernelGGL((absorb_gemv_kernel<A_F32, C_BF16, CPR, MQV>), grid, dim3(256), 0, stream, args); break;
    DSA_GEMV(1) DSA_GEMV(2) DSA_GEMV(3) DSA_GEMV(4) DSA_GEMV(5) DSA_GEMV(6) DSA_GEMV(7) DSA_GEMV(8)
#undef DSA_GEMV
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Many rows (prefill): 128 x 128 tiles of one head, K steps of 32 through a
// two-stage LDS ring (one barrier per step; the step after next is loaded into
// registers while a step is computed).  Wavefront w owns rows 64 (w / 2) .. + 64
// and columns 64 (w % 2) .. + 64: 4 x 4 MFMA 16x16x32 tiles.
constexpr int kGmBM = 128, kGmBN = 128, kGmBK = 32;
constexpr int kGmAS = kGmBK + 8;            // bf16 per LDS row of an A tile
constexpr int kGmBS = kGmBN * 2 + 16;       // bytes per LDS row of a B tile

// NK > 0: K = 32 NK with the step loop fully unrolled (a loop back-edge makes
// the compiler wait for every load in flight, which would void the prefetch);
// NK = 0: any K, rolled.  A bf16 output tile leaves through LDS as 16-byte rows.
constexpr int kGmCS = kGmBN * 2 + 16;       // bytes per LDS row of a bf16 output tile

template <bool A_F32, bool C_BF16, int NK>
__global__ __launch_bounds__(256) void absorb_gemm_kernel(AbsorbArgs a) {
  constexpr int NA = A_F32 ? 2 : 1;
  constexpr int kMainBytes = 2 * NA * kGmBM * kGmAS * 2 + 2 * kGmBK * kGmBS;
  constexpr int kOutBytes = C_BF16 ? kGmBM * kGmCS : 0;
  __shared__ __align__(16) uint8_t smem[kMainBytes > kOutBytes ? kMainBytes : kOutBytes];
  typedef uint16_t ATile[NA][kGmBM * kGmAS];
  typedef uint8_t BTile[kGmBK * kGmBS];
  ATile *la = reinterpret_cast<ATile *>(smem);
  BTile *lb = reinterpret_cast<BTile *>(smem + 2 * sizeof(ATile));
  // When the (row block, head) pairs come in whole groups of 8, the nblk column
  // blocks of one pair are workgroups b, b + 8, b + 16, ...: dispatched together
  // on one XCD, so the A tile they share is read from memory once and then from
  // that XCD's L2.  Otherwise consecutive workgroups take its column blocks.
  const int nblk = a.N / kGmBN;
  const bool by_xcd = ((a.M + kGmBM - 1) / kGmBM) * a.H % 8 == 0;
  const int b8 = blockIdx.x % 8, bq = blockIdx.x / 8;
  const int nb = by_xcd ? bq % nblk : blockIdx.x % nblk;
  const int rest = by_xcd ? b8 + 8 * (bq / nblk) : blockIdx.x / nblk;
  const int h = rest % a.H;
  const int m0 = (rest / a.H) * kGmBM;
  const int n0 = nb * kGmBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t arow = (int64_t)a.H * a.K;
  constexpr int ACH = A_F32 ? 4 : 2;        // 16-byte A chunks per thread per step
  u32x4 ra[ACH], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      const int ch = tid + 256 * j;
      const int r = A_F32 ? ch >> 3 : ch >> 2;
      const int kk = A_F32 ? 4 * (ch & 7) : 8 * (ch & 3);
      const int64_t off = (int64_t)(m0 + r) * arow + (int64_t)h * a.K + k0 + kk;
      const bool ok = m0 + r < a.M;
      if (A_F32)   // (the fp32 attention output: every element read once, non-temporal)
        ra[j] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(static_cast<const float *>(a.a) + off))
                   : u32x4{};
      else
        ra[j] = ok ? *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.a) + off) : u32x4{};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ch = tid + 256 * j;
      rb[j] = *reinterpret_cast<const u32x4 *>(a.b + ((int64_t)h * a.K + k0 + (ch >> 4)) * a.N + n0 + 8 * (ch & 15));
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      const int ch = tid + 256 * j;
      if (A_F32) {
        const int r = ch >> 3, kk = 4 * (ch & 7);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = __uint_as_float(ra[j][e]);
          hi[e] = to_bf16_rne(f);
          lo[e] = to_bf16_rne(f - __uint_as_float(hi[e] << 16));
        }
        typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
        *reinterpret_cast<u32x2 *>(&la[buf][0][r * kGmAS + kk]) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
        *reinterpret_cast<u32x2 *>(&la[buf][NA - 1][r * kGmAS + kk]) =
            u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
      } else {
        const int r = ch >> 2, kk = 8 * (ch & 3);
        *reinterpret_cast<u32x4 *>(&la[buf][0][r * kGmAS + kk]) = ra[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ch = tid + 256 * j;
      *reinterpret_cast<u32x4 *>(lb[buf] + (ch >> 4) * kGmBS + 16 * (ch & 15)) = rb[j];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int wr = 64 * (wave >> 1), wc = 64 * (wave & 1);
  const int nk = NK > 0 ? NK : a.K / kGmBK;
  auto step = [&](int ks) {
    const int buf = ks & 1;
    bf16x8 bop[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const uint8_t *vb = lb[buf] + (8 * g4 + (l16 >> 2)) * kGmBS + (wc + 16 * ct + 4 * (l16 & 3)) * 2;
      const i16x4 v0 = lds_tr(vb), v1 = lds_tr(vb + 4 * kGmBS);
      bop[ct] = __builtin_bit_cast(bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){
                                               v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int part = 0; part < NA; ++part) {
        const bf16x8 aop = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4 *>(&la[buf][part][(wr + 16 * rt + l16) * kGmAS + 8 * g4]));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[ct], acc[rt][ct], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) {
      stage(buf ^ 1);                   // step ks + 1, loaded during the previous step
      if (ks + 2 < nk) load((ks + 2) * kGmBK);
    }
    __syncthreads();
  };
  load(0);
  if (a.rope && nb == 0) copy_rope(a, h, m0, kGmBM);   // its loads overlap the first step's
  stage(0);
  if (nk > 1) load(kGmBK);
  __syncthreads();
  if (NK > 0) {
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) step(ks);
  } else {
    for (int ks = 0; ks < nk; ++ks) step(ks);
  }
  if (C_BF16) {
    // the tile as bf16 into LDS (the last step's barrier has retired every
    // operand read), then 16-byte row pieces to memory
    uint8_t *lc = smem;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          *reinterpret_cast<uint16_t *>(lc + (wr + 16 * rt + 4 * g4 + i) * kGmCS + (wc + 16 * ct + l16) * 2) =
              to_bf16_rne(acc[rt][ct][i]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kGmBM * kGmBN * 2 / 16 / 256; ++j) {
      const int ch = tid + 256 * j;
      const int r = ch >> 4, cc = ch & 15;
      const int m = m0 + r;
      if (m < a.M)
        // written once and read by a later kernel: non-temporal (8 % faster at 2048 queries)
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x4 *>(lc + r * kGmCS + 16 * cc),
            reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.c) + ((int64_t)m * a.H + h) * a.ldc + n0 + 8 * cc));
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wr + 16 * rt + 4 * g4 + i;
        if (m < a.M) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            __builtin_nontemporal_store(
                acc[rt][ct][i], &static_cast<float *>(a.c)[((int64_t)m * a.H + h) * a.ldc + n0 + wc + 16 * ct + l16]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_absorb(void *c, int c_bf16, int ldc, const void *a, int a_f32, const uint16_t *b, int M, int H,
                         int K, int N, const uint16_t *rope, int R, hipStream_t stream) {
  AbsorbArgs args{a, b, c, M, H, K, N, ldc, rope, R};
  if (!((a_f32 && !c_bf16) || (!a_f32 && c_bf16))) return hipErrorInvalidValue;
  if (M <= kGemvMaxM && M * K <= kGemvMaxA && K % 32 == 0 && (R == 0 || M * R / 8 <= 1024)) {
    // 32-column blocks when 64-column ones would leave the chip half empty
    const bool narrow = (N / 64) * H < 256 && K % 64 == 0;
    const dim3 grid((unsigned)(H * (N / (narrow ? 32 : 64))));
    if (a_f32) return narrow ? launch_gemv<true, false, 4>(args, grid, stream)
                             : launch_gemv<true, false, 8>(args, grid, stream);
    return narrow ? launch_gemv<false, true, 4>(args, grid, stream) : launch_gemv<false, true, 8>(args, grid, stream);
  }
  if (N % kGmBN == 0) {
    const dim3 grid((unsigned)((M + kGmBM - 1) / kGmBM) * H * (N / kGmBN));
#define DSA_GEMM(AF, CB, NKV) hipLaunchKernelGGL((absorb_gemm_kernel<AF, CB, NKV>), grid, dim3(256), 0, stream, args)
    const int nk = K / kGmBK;
    if (a_f32) {
      switch (nk) {
        case 4: DSA_GEMM(true, false, 4); break;
        case 8: DSA_GEMM(true, false, 8); break;
        case 16: DSA_GEMM(true, false, 16); break;
        default: DSA_GEMM(true, false, 0); break;
      }
    } else {
      switch (nk) {
        case 4: DSA_GEMM(false, true, 4); break;
        case 6: DSA_GEMM(false, true, 6); break;
        case 8: DSA_GEMM(false, true, 8); break;
        default: DSA_GEMM(false, true, 0); break;
      }
    }
#undef DSA_GEMM
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((M + kAbBM - 1) / kAbBM) * H * (N / kAbBN));
  if (a_f32) hipLaunchKernelGGL((absorb_kernel<true, false>), grid, dim3(kAbThreads), 0, stream, args);
  else hipLaunchKernelGGL((absorb_kernel<false, true>), grid, dim3(kAbThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace dsa
