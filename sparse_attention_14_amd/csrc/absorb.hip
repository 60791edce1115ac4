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
  if (a.rope && nb == 0) {
    for (int e = tid; e < kAbBM * a.R; e += kAbThreads) {
      const int r = e / a.R, c = e - r * a.R;
      const int m = m0 + r;
      if (m < a.M)
        static_cast<uint16_t *>(a.c)[((int64_t)m * a.H + h) * a.ldc + a.N + c] =
            a.rope[((int64_t)m * a.H + h) * a.R + c];
    }
  }
}

}  // namespace

hipError_t launch_absorb(void *c, int c_bf16, int ldc, const void *a, int a_f32, const uint16_t *b, int M, int H,
                         int K, int N, const uint16_t *rope, int R, hipStream_t stream) {
  AbsorbArgs args{a, b, c, M, H, K, N, ldc, rope, R};
  const dim3 grid((unsigned)((M + kAbBM - 1) / kAbBM) * H * (N / kAbBN));
  if (a_f32 && !c_bf16)
    hipLaunchKernelGGL((absorb_kernel<true, false>), grid, dim3(kAbThreads), 0, stream, args);
  else if (!a_f32 && c_bf16)
    hipLaunchKernelGGL((absorb_kernel<false, true>), grid, dim3(kAbThreads), 0, stream, args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dsa
