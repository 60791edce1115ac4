// Sparse absorbed-MLA attention over the kept latent rows.
//
// For a query and head: z_j = scale * <q, row_j> over the whole latent row
// (kv_lora latent + rope), softmax over the kept rows, output = weighted sum of
// the rows' first kv_lora entries, lse = ln sum exp z ("GLM on an A100, in Vx",
// section "The model": each query attends only to its kept tokens' latent
// vectors; "Self-contained GLM-5 serving stack": absorbed MLA decode, stable
// softmax, split online-softmax compressed MLA).
//
// bf16 (576-wide rows, 512 latent): a workgroup owns one query, 16 heads and a
// split of the index slots.  Per 64-slot tile the selected rows are gathered
// once into LDS (padded rows against bank conflicts) and shared by all heads of
// the group (MLA rows are per token, not per head):
//   QK^T : v_mfma_f32_16x16x32_bf16, M = 16 heads, N = 16 rows per wavefront, K = 576;
//   online softmax in the exp2 domain, maxima and sums reduced in a fixed order;
//   PV   : M = 16 heads, N = 128 latent columns per wavefront, K = 64 rows.  The
//          probabilities are split into bf16 hi + lo parts (two MFMAs), so the
//          rounding of P adds ~2^-17 relative error instead of bf16's 2^-9.
// Splits write unnormalised partial outputs with their (max, sum); a merge
// kernel combines them in split order (deterministic).  The four head groups
// of one (query, split) are placed on the same XCD so that their identical
// row gathers hit one L2.
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ bf16 path
constexpr int kW = 576, kL = 512, kTile = 64, kHG = 16;
constexpr int kRowBytes = kW * 2 + 16;          // padded LDS row
constexpr int kChunks = kW * 2 / 16;            // 16-byte chunks per row (72)

struct AttArgs {
  float *out;
  float *lse;
  const uint16_t *q;
  CacheDev latent;
  const int32_t *indices;
  const int32_t *q_seq;
  float *part_o;   // [n_q][S][H][L]
  float *part_ml;  // [n_q][S][H][2]
  int k, n_q, n_heads, splits, rows_per_split, n_hg, pairs, seq_ident;
  float scale_log2;  // softmax_scale * log2(e)
};

template <bool SPLIT>
__global__ __launch_bounds__(256) void attend_bf16_kernel(AttArgs a) {
  __shared__ __align__(16) uint8_t lrows[kTile * kRowBytes];
  __shared__ __align__(16) uint16_t lp[2][kHG * kTile];  // P hi / lo, [head][row]
  __shared__ float red[2][4][kHG];
  __shared__ const uint8_t *lptr[kTile];
  __shared__ int lidx[kTile];

  // XCD-aware mapping: workgroup ids i, i+8, i+16, ... run on one XCD; give the
  // n_hg head groups of a (query, split) pair ids 8 apart.
  const int lin = blockIdx.x;
  const int group = lin / (8 * a.n_hg);
  const int rem = lin - group * 8 * a.n_hg;
  const int hg = rem >> 3;
  const int pair = group * 8 + (rem & 7);
  if (pair >= a.pairs) return;
  const int qi = pair / a.splits;
  const int sp = pair - qi * a.splits;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int H = a.n_heads;
  const int h0 = hg * kHG;
  const int seq = seq_of(a.q_seq, qi, a.seq_ident);

  // q operand: head h0 + l16, dims 32*ks + 8*g4 + [0, 8)
  bf16x8 qa[kW / 32];
  {
    const uint16_t *qr = a.q + ((int64_t)qi * H + h0 + l16) * kW + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < kW / 32; ++ks) qa[ks] = as_bf16x8(load16(qr + 32 * ks));
  }

  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }
  f32x4 o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0, 0, 0, 0};

  const int j0 = sp * a.rows_per_split;
  const int j1 = min(j0 + a.rows_per_split, a.k);
  const int32_t *idx_row = a.indices + (int64_t)qi * a.k;

  for (int tb = j0; tb < j1; tb += kTile) {
    if (tid < kTile) {
      const int j = tb + tid;
      const int t = j < j1 ? idx_row[j] : -1;
      lidx[tid] = t;
      const uint8_t *p = nullptr;
      if (t >= 0) {
        int slot;
        const int64_t blk = cache_block(a.latent, seq, t, slot);
        p = cache_row(a.latent, blk, slot);
      }
      lptr[tid] = p;
    }
    __syncthreads();
    // gather the tile's rows into LDS (zeros for empty slots)
    {
      constexpr int kPer = kTile * kChunks / 256;  // 18
      u32x4 v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int c = tid + 256 * i;
        const int r = c / kChunks, cc = c - r * kChunks;
        const uint8_t *p = lptr[r];
        v[i] = p ? load16(p + cc * 16) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int c = tid + 256 * i;
        const int r = c / kChunks, cc = c - r * kChunks;
        *reinterpret_cast<u32x4 *>(lrows + r * kRowBytes + cc * 16) = v[i];
      }
    }
    __syncthreads();

    // QK^T: this wavefront's 16 rows
    const int row = wave * 16 + l16;
    f32x4 sacc = {0, 0, 0, 0};
    {
      const uint8_t *rp = lrows + row * kRowBytes + 16 * g4;
#pragma unroll
      for (int ks = 0; ks < kW / 32; ++ks) {
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4 *>(rp + 64 * ks));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], b, sacc, 0, 0, 0);
      }
    }
    const bool valid = lidx[row] >= 0;
    float z[4], mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = valid ? sacc[i] * a.scale_log2 : -INFINITY;
      mx[i] = z[i];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], off, 64));
    if (l16 == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[0][wave][4 * g4 + i] = mx[i];
    __syncthreads();

    float m_new[4], alpha[4], p[4], ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
      float tm = fmaxf(fmaxf(red[0][0][h], red[0][1][h]), fmaxf(red[0][2][h], red[0][3][h]));
      m_new[i] = fmaxf(m_run[i], tm);
      const float mu = m_new[i] == -INFINITY ? 0.0f : m_new[i];
      alpha[i] = exp2f(m_run[i] - mu);
      p[i] = exp2f(z[i] - mu);
      const uint16_t hi = float_to_bf16_bits(p[i]);
      const uint16_t lo = float_to_bf16_bits(p[i] - bf16_bits_to_float(hi));
      lp[0][h * kTile + row] = hi;
      lp[1][h * kTile + row] = lo;
      ps[i] = p[i];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) ps[i] += __shfl_xor(ps[i], off, 64);
    if (l16 == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[1][wave][4 * g4 + i] = ps[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
      const float tsum = ((red[1][0][h] + red[1][1][h]) + red[1][2][h]) + red[1][3][h];
      l_run[i] = l_run[i] * alpha[i] + tsum;
      m_run[i] = m_new[i];
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nt][i] *= alpha[i];

    // PV: rows 32*ks2 + 8*g4 + e, columns 128*wave + 16*nt + l16
#pragma unroll
    for (int ks2 = 0; ks2 < kTile / 32; ++ks2) {
      const bf16x8 ahi = as_bf16x8(*reinterpret_cast<const u32x4 *>(&lp[0][l16 * kTile + 32 * ks2 + 8 * g4]));
      const bf16x8 alo = as_bf16x8(*reinterpret_cast<const u32x4 *>(&lp[1][l16 * kTile + 32 * ks2 + 8 * g4]));
      const uint8_t *vb = lrows + (32 * ks2 + 8 * g4) * kRowBytes + (128 * wave + l16) * 2;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x0 = *reinterpret_cast<const uint16_t *>(vb + (2 * e) * kRowBytes + 32 * nt);
          const uint32_t x1 = *reinterpret_cast<const uint16_t *>(vb + (2 * e + 1) * kRowBytes + 32 * nt);
          u[e] = x0 | (x1 << 16);
        }
        const bf16x8 b = as_bf16x8(u32x4{u[0], u[1], u[2], u[3]});
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, o[nt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds heads h0 + 4*g4 + i, columns 128*wave + 16*nt + l16
  if (!SPLIT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = h0 + 4 * g4 + i;
      const float inv = l_run[i] > 0.0f ? 1.0f / l_run[i] : 0.0f;
      float *orow = a.out + ((int64_t)qi * H + head) * kL + 128 * wave + l16;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) orow[16 * nt] = o[nt][i] * inv;
      if (wave == 0 && l16 == 0 && a.lse)
        a.lse[(int64_t)qi * H + head] = l_run[i] > 0.0f ? (m_run[i] + log2f(l_run[i])) * kLn2 : -INFINITY;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = h0 + 4 * g4 + i;
      const int64_t base = ((int64_t)(qi * a.splits + sp) * H + head);
      float *orow = a.part_o + base * kL + 128 * wave + l16;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) orow[16 * nt] = o[nt][i];
      if (wave == 0 && l16 == 0) {
        a.part_ml[base * 2 + 0] = m_run[i];
        a.part_ml[base * 2 + 1] = l_run[i];
      }
    }
  }
}

// Combine split partials in split order.  One workgroup per (query, head).
__global__ __launch_bounds__(128) void merge_kernel(float *__restrict__ out, float *__restrict__ lse,
                                                    const float *__restrict__ part_o,
                                                    const float *__restrict__ part_ml, int splits, int H, int L) {
  const int qi = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[(((int64_t)qi * splits + s) * H + h) * 2]);
  float *orow = out + ((int64_t)qi * H + h) * L;
  if (M == -INFINITY) {
    for (int c = threadIdx.x; c < L; c += 128) orow[c] = 0.0f;
    if (threadIdx.x == 0 && lse) lse[(int64_t)qi * H + h] = -INFINITY;
    return;
  }
  float Ls = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const int64_t b = ((int64_t)qi * splits + s) * H + h;
    Ls += exp2f(part_ml[b * 2] - M) * part_ml[b * 2 + 1];
  }
  const float inv = 1.0f / Ls;
  for (int c = threadIdx.x; c < L; c += 128) {
    float acc = 0.0f;
    for (int s = 0; s < splits; ++s) {
      const int64_t b = ((int64_t)qi * splits + s) * H + h;
      acc += exp2f(part_ml[b * 2] - M) * part_o[b * L + c];
    }
    orow[c] = acc * inv;
  }
  if (threadIdx.x == 0 && lse) lse[(int64_t)qi * H + h] = (M + log2f(Ls)) * kLn2;
}

// ------------------------------------------------------------------- f32 path
// One workgroup per (query, head); fixed-order reductions.
__device__ float block_reduce_max(float v, float *sh) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, sh[i]);
  __syncthreads();
  return r;
}
__device__ float block_reduce_sum(float v, float *sh) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r += sh[i];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void attend_f32_kernel(float *__restrict__ out, float *__restrict__ lse,
                                                         const float *__restrict__ q, CacheDev latent, int kv_lora,
                                                         const int32_t *__restrict__ indices, int k,
                                                         const int32_t *__restrict__ q_seq, int seq_ident, int H,
                                                         float scale_log2) {
  __shared__ float lq[1024];
  __shared__ float lz[2048];
  __shared__ const float *lrow[2048];
  __shared__ float sh[8];
  const int qi = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int W = latent.width;
  const int seq = seq_of(q_seq, qi, seq_ident);
  for (int c = threadIdx.x; c < W; c += 256) lq[c] = q[((int64_t)qi * H + h) * W + c];
  __syncthreads();
  float mloc = -INFINITY;
  for (int j = threadIdx.x; j < k; j += 256) {
    const int t = indices[(int64_t)qi * k + j];
    float z = -INFINITY;
    const float *rp = nullptr;
    if (t >= 0) {
      int slot;
      const int64_t blk = cache_block(latent, seq, t, slot);
      rp = reinterpret_cast<const float *>(cache_row(latent, blk, slot));
      float dot = 0.0f;
      for (int c = 0; c < W; ++c) dot = fmaf(lq[c], rp[c], dot);
      z = dot * scale_log2;
    }
    lz[j] = z;
    lrow[j] = rp;
    mloc = fmaxf(mloc, z);
  }
  const float m = block_reduce_max(mloc, sh);
  const float mu = m == -INFINITY ? 0.0f : m;
  float sloc = 0.0f;
  for (int j = threadIdx.x; j < k; j += 256) {
    const float p = exp2f(lz[j] - mu);
    lz[j] = p;
    sloc += p;
  }
  const float l = block_reduce_sum(sloc, sh);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  for (int c = threadIdx.x; c < kv_lora; c += 256) {
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      const float *rp = lrow[j];
      if (rp) acc = fmaf(lz[j], rp[c], acc);
    }
    out[((int64_t)qi * H + h) * kv_lora + c] = acc * inv;
  }
  if (threadIdx.x == 0 && lse) lse[(int64_t)qi * H + h] = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

AttendPlan plan_attend(int n_q, int n_heads, int kv_lora, int width, int k, int dtype) {
  AttendPlan p{};
  p.n_q = n_q;
  p.n_heads = n_heads;
  p.kv_lora = kv_lora;
  p.width = width;
  p.k = k;
  p.splits = 1;
  p.rows_per_split = (k + kTile - 1) / kTile * kTile;
  if (dtype == kBF16 && n_heads >= kHG) {
    const int n_hg = n_heads / kHG;
    const int tiles = (k + kTile - 1) / kTile;
    // ~256 workgroups, but at least two tiles per split so the partial outputs
    // (H x L floats per split) stay below the rows they summarise.
    int s = (256 + n_q * n_hg - 1) / (n_q * n_hg);
    const int most = (tiles + 1) / 2;
    if (s > most) s = most;
    if (s < 1) s = 1;
    const int tps = (tiles + s - 1) / s;
    p.rows_per_split = tps * kTile;
    p.splits = (tiles + tps - 1) / tps;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  if (p.splits > 1) {
    p.off_part_o = take((size_t)n_q * p.splits * n_heads * kv_lora * 4);
    p.off_part_ml = take((size_t)n_q * p.splits * n_heads * 2 * 4);
  }
  p.total = off;
  return p;
}

hipError_t launch_attend(float *out, float *lse, const void *q, int dt, const CacheDev &latent, int kv_lora,
                         const int32_t *indices, int k, const int32_t *q_seq, int seq_ident, int n_q, int n_heads,
                         float scale, const AttendPlan &plan, void *workspace, hipStream_t stream) {
  if (dt == kF32) {
    hipLaunchKernelGGL(attend_f32_kernel, dim3(n_q * n_heads), dim3(256), 0, stream, out, lse,
                       static_cast<const float *>(q), latent, kv_lora, indices, k, q_seq, seq_ident, n_heads,
                       scale * kLog2e);
    return hipGetLastError();
  }
  AttArgs a{};
  a.out = out;
  a.lse = lse;
  a.q = static_cast<const uint16_t *>(q);
  a.latent = latent;
  a.indices = indices;
  a.q_seq = q_seq;
  a.seq_ident = seq_ident;
  a.k = k;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.splits = plan.splits;
  a.rows_per_split = plan.rows_per_split;
  a.n_hg = n_heads / kHG;
  a.pairs = n_q * plan.splits;
  a.scale_log2 = scale * kLog2e;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const int groups = (a.pairs + 7) / 8;
  const dim3 grid(groups * 8 * a.n_hg);
  if (plan.splits > 1) {
    a.part_o = reinterpret_cast<float *>(ws + plan.off_part_o);
    a.part_ml = reinterpret_cast<float *>(ws + plan.off_part_ml);
    hipLaunchKernelGGL(attend_bf16_kernel<true>, grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel, dim3(n_q * n_heads), dim3(128), 0, stream, out, lse, a.part_o, a.part_ml,
                       plan.splits, n_heads, kv_lora);
  } else {
    hipLaunchKernelGGL(attend_bf16_kernel<false>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

__global__ void fill_zero_kernel(uint32_t *p, size_t words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_fill_zero(uint32_t *p, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, words);
  return hipGetLastError();
}

}  // namespace dsa
