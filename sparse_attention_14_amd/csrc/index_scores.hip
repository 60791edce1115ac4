// Lightning-indexer score kernels.
//
// score[s] = sum_h w[h] * max(0, <q_h, khat_s>)  -- an indexer that scores every
// earlier token, with a ReLU per head before the heads are combined ("GLM on an
// A100, in Vx", sections "The model" and "How do we know it is right?").
//
// bf16 / fp8 keys: one wavefront takes 32 keys per step and computes the
// [heads x 32 keys] block with v_mfma_f32_32x32x16_bf16 (heads are the M
// dimension, so one query per wavefront already fills the matrix core); fp8
// bytes are converted to bf16 exactly in registers.  The ReLU, the per-key
// fp8 scale, the head weights and the head sum are applied to the accumulator
// in registers: each lane holds 16 heads of one key, its partner lane (l ^ 32)
// the other 16, so one cross-lane add finishes a key.  The summation order is
// the same for every key, so byte-identical keys score bit-identically.
//
// The K dimension is permuted: lane half h (= lane / 32) holds dims
// [h*D/2, (h+1)*D/2) of its key, which is one contiguous run of the key row, and
// the q operand uses the same permutation, so the dot product is unchanged.
//
// Optionally the kernel also counts order_key(score) >> 20 per query into a
// global histogram (the first radix level of the top-k), workgroup-local in
// LDS first, then one atomic per non-empty bin.
#include "kernels.hpp"

namespace dsa {
namespace {

template <bool FP8, int D, int MT, bool HIST>
__global__ __launch_bounds__(256) void scores_mfma_kernel(float *__restrict__ scores, int64_t ld,
                                                          const uint16_t *__restrict__ q, const float *__restrict__ w,
                                                          CacheDev keys, const int32_t *__restrict__ q_seq,
                                                          int seq_ident, const int32_t *__restrict__ q_len,
                                                          int n_heads, int tiles_per_wave,
                                                          uint32_t *__restrict__ hist) {
  constexpr int KS = D / 16;                 // 32x32x16 K-steps
  constexpr int HALF = D / 2;                // dims held by one lane half
  constexpr int EB = FP8 ? 1 : 2;            // key element bytes
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];

  const int qi = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int n = q_len[qi];
  if (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
    __syncthreads();
  }
  const int tile_begin = (blockIdx.x * 4 + wave) * tiles_per_wave;
  const int seq = seq_of(q_seq, qi, seq_ident);

  if (tile_begin * 32 < n) {
    // q as the A operand: lane (col, half) holds head 32*mt + col, dims half*HALF + 8*ks + [0, 8).
    bf16x8 a[MT][KS];
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int head = 32 * mt + col;
      const uint16_t *qrow = q + ((int64_t)qi * n_heads + (head < n_heads ? head : 0)) * D + half * HALF;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = load16(qrow + 8 * ks);
        if (head >= n_heads) v = u32x4{0, 0, 0, 0};
        a[mt][ks] = as_bf16x8(v);
      }
      // Accumulator element r of this lane is head 32*mt + 8*(r/4) + 4*half + r%4.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * mt + 8 * (r >> 2) + 4 * half + (r & 3);
        wr[mt][r] = m < n_heads ? w[(int64_t)qi * n_heads + m] : 0.0f;
      }
    }

    for (int it = 0; it < tiles_per_wave; ++it) {
      const int t0 = (tile_begin + it) * 32;
      if (t0 >= n) break;
      const int t = t0 + col;
      const int tl = t < n ? t : n - 1;
      const int bi = t0 / keys.block_size;   // a 32-token tile never straddles a block
      const int64_t blk = keys.table ? (int64_t)keys.table[(int64_t)seq * keys.max_blocks + bi] : (int64_t)seq;
      const int slot = tl - bi * keys.block_size;
      const uint8_t *row = cache_row(keys, blk, slot) + half * HALF * EB;

      bf16x8 b[KS];
      if (FP8) {
#pragma unroll
        for (int j = 0; j < HALF / 16; ++j) {
          u32x4 v = load16_nt(row + 16 * j);
          b[2 * j] = fp8x8_to_bf16x8(v[0], v[1]);
          b[2 * j + 1] = fp8x8_to_bf16x8(v[2], v[3]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) b[ks] = as_bf16x8(load16_nt(row + 16 * ks));
      }
      const float sc = FP8 ? keys.scale[blk * keys.scale_block_stride + slot] : 1.0f;

      float s = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][ks], b[ks], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = FP8 ? acc[r] * sc : acc[r];
          v = fmaxf(v, 0.0f);
          s = fmaf(wr[mt][r], v, s);
        }
      }
      s += __shfl_xor(s, 32, 64);
      if (half == 0 && t < n) {
        scores[(int64_t)qi * ld + t] = s;
        if (HIST) atomicAdd(&lhist[order_key(s) >> kHistShift], 1u);
      }
    }
  }
  if (HIST) {
    __syncthreads();
    uint32_t *gh = hist + (int64_t)qi * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
      const uint32_t c = lhist[i];
      if (c) atomic_add_agent(gh + i, c);
    }
  }
}

// fp32 queries and keys: one thread per key, fp32 FMA chains in a fixed order
// (dims ascending, then heads ascending).
template <int D, bool HIST>
__global__ __launch_bounds__(256) void scores_f32_kernel(float *__restrict__ scores, int64_t ld,
                                                         const float *__restrict__ q, const float *__restrict__ w,
                                                         CacheDev keys, const int32_t *__restrict__ q_seq,
                                                         int seq_ident, const int32_t *__restrict__ q_len,
                                                         int n_heads, uint32_t *__restrict__ hist) {
  __shared__ float lq[64 * D];
  __shared__ float lw[64];
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];
  const int qi = blockIdx.y;
  const int n = q_len[qi];
  for (int i = threadIdx.x; i < n_heads * D; i += 256) lq[i] = q[(int64_t)qi * n_heads * D + i];
  for (int i = threadIdx.x; i < n_heads; i += 256) lw[i] = w[(int64_t)qi * n_heads + i];
  if (HIST)
    for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < n) {
    const int seq = seq_of(q_seq, qi, seq_ident);
    int slot;
    const int64_t blk = cache_block(keys, seq, t, slot);
    const float *row = reinterpret_cast<const float *>(cache_row(keys, blk, slot));
    float k[D];
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      u32x4 v = load16_nt(row + d);
      k[d] = __uint_as_float(v[0]);
      k[d + 1] = __uint_as_float(v[1]);
      k[d + 2] = __uint_as_float(v[2]);
      k[d + 3] = __uint_as_float(v[3]);
    }
    float s = 0.0f;
    for (int h = 0; h < n_heads; ++h) {
      float dot = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(lq[h * D + d], k[d], dot);
      s = fmaf(lw[h], fmaxf(dot, 0.0f), s);
    }
    scores[(int64_t)qi * ld + t] = s;
    if (HIST) atomicAdd(&lhist[order_key(s) >> kHistShift], 1u);
  }
  if (HIST) {
    __syncthreads();
    uint32_t *gh = hist + (int64_t)qi * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
      const uint32_t c = lhist[i];
      if (c) atomic_add_agent(gh + i, c);
    }
  }
}

template <bool FP8, int D, int MT, bool HIST>
hipError_t run_mfma(float *scores, int64_t ld, const void *q, const float *w, const CacheDev &keys,
                    const int32_t *q_seq, int seq_ident, const int32_t *q_len, int n_q, int n_heads, int max_len,
                    uint32_t *hist, hipStream_t stream) {
  const int tiles = (max_len + 31) / 32;
  // Aim at ~1024 workgroups of 4 wavefronts; each wavefront streams tiles_per_wave
  // consecutive 32-key tiles so that its q fragment load is amortised.
  const int64_t total = (int64_t)tiles * n_q;
  int tpw = (int)((total + 4 * 1024 - 1) / (4 * 1024));
  tpw = tpw < 1 ? 1 : (tpw > 64 ? 64 : tpw);
  const int gx = (tiles + 4 * tpw - 1) / (4 * tpw);
  dim3 grid(gx, n_q);
  hipLaunchKernelGGL((scores_mfma_kernel<FP8, D, MT, HIST>), grid, dim3(256), 0, stream, scores, ld,
                     static_cast<const uint16_t *>(q), w, keys, q_seq, seq_ident, q_len, n_heads, tpw, hist);
  return hipGetLastError();
}

template <int D, bool HIST>
hipError_t run_f32(float *scores, int64_t ld, const void *q, const float *w, const CacheDev &keys,
                   const int32_t *q_seq, int seq_ident, const int32_t *q_len, int n_q, int n_heads, int max_len,
                   uint32_t *hist, hipStream_t stream) {
  dim3 grid((max_len + 255) / 256, n_q);
  hipLaunchKernelGGL((scores_f32_kernel<D, HIST>), grid, dim3(256), 0, stream, scores, ld,
                     static_cast<const float *>(q), w, keys, q_seq, seq_ident, q_len, n_heads, hist);
  return hipGetLastError();
}

template <bool HIST>
hipError_t dispatch(float *scores, int64_t ld, const void *q, int q_dt, const float *w, const CacheDev &keys,
                    int key_dt, const int32_t *q_seq, int seq_ident, const int32_t *q_len, int n_q, int n_heads,
                    int max_len, uint32_t *hist, hipStream_t s) {
  const int D = keys.width;
  if (q_dt == kF32) {
    switch (D) {
      case 32: return run_f32<32, HIST>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, hist, s);
      case 64: return run_f32<64, HIST>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, hist, s);
      case 96: return run_f32<96, HIST>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, hist, s);
      case 128: return run_f32<128, HIST>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, hist, s);
      default: return hipErrorInvalidValue;
    }
  }
  const bool fp8 = key_dt == kFP8;
  const bool two = n_heads > 32;
#define DSA_SC(F, DD, M)                                                                                    \
  return run_mfma<F, DD, M, HIST>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, hist, s)
  if (D == 128) {
    if (fp8) { if (two) DSA_SC(true, 128, 2); DSA_SC(true, 128, 1); }
    if (two) DSA_SC(false, 128, 2);
    DSA_SC(false, 128, 1);
  }
  if (D == 64) {
    if (fp8) { if (two) DSA_SC(true, 64, 2); DSA_SC(true, 64, 1); }
    if (two) DSA_SC(false, 64, 2);
    DSA_SC(false, 64, 1);
  }
#undef DSA_SC
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_index_scores(float *scores, int64_t ld, const void *q, int q_dt, const float *w,
                               const CacheDev &keys, int key_dt, const int32_t *q_seq, int seq_ident,
                               const int32_t *q_len, int n_q, int n_heads, int max_len, uint32_t *hist,
                               hipStream_t stream) {
  if (hist)
    return dispatch<true>(scores, ld, q, q_dt, w, keys, key_dt, q_seq, seq_ident, q_len, n_q, n_heads, max_len, hist,
                          stream);
  return dispatch<false>(scores, ld, q, q_dt, w, keys, key_dt, q_seq, seq_ident, q_len, n_q, n_heads, max_len,
                         nullptr, stream);
}

}  // namespace dsa
