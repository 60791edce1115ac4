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
// [h*D/2, (h+1)*D/2) of its key, and the q operand uses the same permutation,
// so the dot product is unchanged.  Keys are fetched with fully coalesced
// loads and redistributed through a per-wavefront LDS tile.
#include "kernels.hpp"

namespace dsa {
namespace {

// max(x, 0) on the bits: IEEE floats order like sign-magnitude integers, so a
// signed-integer max with 0 is the float ReLU (-0 becomes +0, a negative NaN 0),
// in one instruction.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sum of a value over lanes l and l ^ 32, the same in both lanes and formed in
// the same order (lower half first) in both.
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kMaxTilesPerWave = 8;
constexpr int kPrefillMinQueries = 64;   // the GEMM-shaped kernel (prefill_scores.hip) takes over from here


// One wavefront scores TPW consecutive 32-key tiles.  The tile loop is fully
// unrolled and every tile load is issued unconditionally (tiles past the row's
// end reload its last tile and their scores are dropped), so the code is
// straight-line and the compiler waits for exactly the tile it needs while the
// next P tiles stay in flight.  Tile positions, block-table lookups and tile
// base addresses are wavefront-uniform (scalar); a lane adds one precomputed
// 32-bit offset per load.
//
// QW = 2: the M tiles are two queries of one sequence (rows 2 y and 2 y + 1,
// up to 32 heads each), e.g. neighbouring queries of a multi-token decode
// window: every key tile is loaded once for both, each query keeps its own
// visible count, score row and candidate bounds.  QW = 1: the M tiles are
// heads 0-31 and 32-63 of one query (row y).
//
// window > 0: rows are the queries of multi-token windows, row i the (i % window)-th
// of sequence i / window, whose visible count is q_len[i / window] - window + 1 +
// i % window (at least 0; q_len then holds the sequences' lengths).  The
// workgroups of the first key range write each row's count to row_len_out.
template <bool FP8, int D, int MT, int TPW, int QW>
__global__ __launch_bounds__(256) void scores_mfma_kernel(float *__restrict__ scores, int64_t ld,
                                                          const uint16_t *__restrict__ q, const float *__restrict__ w,
                                                          CacheDev keys, const int32_t *__restrict__ q_seq,
                                                          int seq_ident, const int32_t *__restrict__ q_len,
                                                          int n_heads, uint32_t *__restrict__ bounds, int topk,
                                                          int window, int32_t *__restrict__ row_len_out) {
  constexpr int KS = D / 16;            // 32x32x16 K-steps
  constexpr int HALF = D / 2;           // dims held by one lane half
  constexpr int EB = FP8 ? 1 : 2;       // key element bytes
  constexpr int ROWB = D * EB;          // key row bytes
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  constexpr int HALFC = CPR / 2;        // chunks per lane half
  constexpr int TILEB = 32 * ROWB;      // bytes of a 32-key tile
  constexpr int NLD = TILEB / 1024;     // 1 KB wavefront loads per tile
  constexpr int P = TPW < 2 ? TPW : 2;  // tiles in flight ahead of the one being scored
  static_assert(64 % CPR == 0, "a 1 KB load must cover whole rows");
  static_assert(QW == 1 || MT == QW, "a group of queries uses one M tile each");
  constexpr bool MULTI = QW > 1;
  constexpr int NQ = QW;                // queries (score rows) of the wavefront
  __shared__ __align__(16) uint8_t stage_all[4][TILEB];

  // Fetch every kernel argument at once: the compiler would otherwise load each
  // one just before its first use, one dependent round trip after another.  The
  // statement reads the arguments (so they are loaded before it) and yields a
  // zero that the wavefront index depends on (so it runs first); it touches no
  // memory.
  int zero;
  asm("s_mov_b32 %0, 0"
      : "=s"(zero)
      : "s"(scores), "s"(ld), "s"(q), "s"(w), "s"(keys.rows), "s"(keys.scale), "s"(keys.row_stride),
        "s"(keys.block_stride), "s"(keys.scale_block_stride), "s"(keys.table), "s"(keys.block_size),
        "s"(keys.max_blocks), "s"(q_seq), "s"(seq_ident), "s"(q_len), "s"(n_heads), "s"(bounds), "s"(topk),
        "s"(window), "s"(row_len_out));
  const int qi = QW * blockIdx.y;   // first score row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  int nq[NQ];   // visible tokens of each row
  if (window > 0) {
    const int sl = q_len[qi / window], j0 = qi % window;
#pragma unroll
    for (int u = 0; u < NQ; ++u) nq[u] = max(sl - window + 1 + j0 + u, 0);
  } else {
#pragma unroll
    for (int u = 0; u < NQ; ++u) nq[u] = q_len[qi + u];
  }
  int n = nq[0];
#pragma unroll
  for (int u = 1; u < NQ; ++u) n = max(n, nq[u]);
  const int ntile = (n + 31) / 32;
  const int wid = blockIdx.x * 4 + wave + zero;
  const int tile_begin = wid * TPW;
  float lane_best[NQ];   // largest score of this lane's keys, per row (bounds only)
#pragma unroll
  for (int u = 0; u < NQ; ++u) lane_best[u] = -__builtin_inff();

  if (tile_begin < ntile) {
    const int seq = window > 0 ? qi / window : seq_of(q_seq, qi, seq_ident);
    uint8_t *stage = stage_all[wave];
    // First row, first scale and last visible row of every tile (a 32-key tile
    // never straddles a block).  All of it is wavefront-uniform; the block
    // lookups are issued together, before any vector load.
    int bi[TPW], slot[TPW], tlast[TPW];
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      int tile = tile_begin + it;
      tile = tile < ntile ? tile : ntile - 1;
      const int t0 = tile * 32;
      bi[it] = t0 / keys.block_size;
      slot[it] = t0 - bi[it] * keys.block_size;
      tlast[it] = n - 1 - t0;
    }
    int blk[kMaxTilesPerWave] = {};
    if (keys.table) {
      const int32_t *trow = keys.table + (int64_t)seq * keys.max_blocks;
#pragma unroll
      for (int it = 0; it < TPW; ++it) blk[it] = trow[bi[it]];
      // every lookup is in flight before the first is used
      asm("" : "+s"(blk[0]), "+s"(blk[1]), "+s"(blk[2]), "+s"(blk[3]), "+s"(blk[4]), "+s"(blk[5]), "+s"(blk[6]),
          "+s"(blk[7]));
    } else {
#pragma unroll
      for (int it = 0; it < TPW; ++it) blk[it] = seq;
    }
    const uint8_t *tbase[TPW];
    const float *sbase[TPW];
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      tbase[it] = keys.rows + (int64_t)blk[it] * keys.block_stride + (int64_t)slot[it] * keys.row_stride;
      sbase[it] = FP8 ? keys.scale + (int64_t)blk[it] * keys.scale_block_stride + slot[it] : nullptr;
    }

    // Loads are coalesced: 16-byte piece j*64 + lane of the tile's rows (1 KB per
    // wavefront instruction), i.e. row (64 j + lane) / CPR, chunk lane % CPR.
    // A row past the last visible one is replaced by the last visible row, by a
    // min() on the byte offsets (the row stride is positive and below 2^24).
    // They go through a wavefront-private LDS tile (chunk slots XOR-swizzled by
    // the row against bank conflicts) into the MFMA operand layout.  Keys are
    // read once per call: non-temporal loads.
    const uint32_t rs = (uint32_t)keys.row_stride;
    const uint32_t ch16 = 16u * (uint32_t)(lane % CPR);
    uint32_t loff[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) loff[j] = (uint32_t)((64 * j + lane) / CPR) * rs + ch16;
    struct Raw {
      u32x4 v[NLD];
      float sc;
    };
    auto issue = [&](int it, Raw &r) {
      const uint32_t lim = (uint32_t)tlast[it] * rs + ch16;
#pragma unroll
      for (int j = 0; j < NLD; ++j) r.v[j] = load16_nt(tbase[it] + (loff[j] < lim ? loff[j] : lim));
      if (FP8) r.sc = sbase[it][col < tlast[it] ? col : tlast[it]];
    };
    Raw buf[P];
#pragma unroll
    for (int p = 0; p < P; ++p) issue(p, buf[p]);

    // q as the A operand: lane (col, half) holds head 32*mt + col, dims
    // half*HALF + 8*ks + [0, 8); head weights per accumulator element.  Loaded
    // after the first key tiles and unconditionally (clamped, then zeroed), so
    // that no branch separates the key loads from their use.
    bf16x8 a[MT][KS];
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int qm = MULTI ? qi + mt : qi;         // the tile's query
      const int head = MULTI ? col : 32 * mt + col;
      const uint16_t *qrow = q + ((int64_t)qm * n_heads + (head < n_heads ? head : n_heads - 1)) * D + half * HALF;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = load16(qrow + 8 * ks);
        if (head >= n_heads) v = u32x4{0, 0, 0, 0};
        a[mt][ks] = as_bf16x8(v);
      }
      // Accumulator element r of this lane is head (MULTI ? 0 : 32*mt) + 8*(r/4) + 4*half + r%4.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = (MULTI ? 0 : 32 * mt) + 8 * (r >> 2) + 4 * half + (r & 3);
        const float x = w[(int64_t)qm * n_heads + (m < n_heads ? m : n_heads - 1)];
        wr[mt][r] = m < n_heads ? x : 0.0f;
      }
    }
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      Raw &cur = buf[it % P];
      // stage the tile, then read this lane's operand chunks back
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int kk = (64 * j + lane) / CPR, ch = lane % CPR;
        *reinterpret_cast<u32x4 *>(stage + kk * ROWB + 16 * (ch ^ (kk & (CPR - 1)))) = cur.v[j];
      }
      const float sc = FP8 ? cur.sc : 1.0f;
      if (it + P < TPW) issue(it + P, cur);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      bf16x8 b[KS];
#pragma unroll
      for (int j = 0; j < HALFC; ++j) {
        const int ch = half * HALFC + j;
        const u32x4 x = *reinterpret_cast<const u32x4 *>(stage + col * ROWB + 16 * (ch ^ (col & (CPR - 1))));
        if (FP8) {
          b[2 * j] = fp8x8_to_bf16x8(x[0], x[1]);
          b[2 * j + 1] = fp8x8_to_bf16x8(x[2], x[3]);
        } else {
          b[j] = as_bf16x8(x);
        }
      }
      // Epilogue.  fp8: sum_h w_h ReLU(acc_h * sc) = |sc| * sum_h w_h ReLU(acc_h * sign(sc)),
      // the sign applied by flipping the accumulator's sign bit: one multiply per
      // key instead of one per head, and the same summation order for every key.
      const uint32_t flip = FP8 ? (__float_as_uint(sc) & 0x80000000u) : 0u;
      float s[NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) s[u] = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][ks], b[ks], acc, 0, 0, 0);
        float &su = s[MULTI ? mt : 0];
#pragma unroll
        for (int r = 0; r < 16; ++r) su = fmaf(wr[mt][r], relu(__uint_as_float(__float_as_uint(acc[r]) ^ flip)), su);
      }
      const int t = (tile_begin + it) * 32 + col;
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        float x = FP8 ? s[u] * fabsf(sc) : s[u];
        x = halves_sum(x);
        if (half == 0 && t < nq[u]) scores[(int64_t)(qi + u) * ld + t] = x;
        // only wavefronts whose keys are all visible to the row report a
        // bound, so every score reaches the maximum unmasked
        lane_best[u] = fmaxf(lane_best[u], x);
      }
    }
  }

  // Candidate bound for the top-k: a full wavefront (all TPW * 32 of its
  // tokens visible) reports the r-th largest of its lanes' maxima,
  // r = bound_rank(k, G, 32) with G full wavefronts in the row; each lane
  // maximum is the score of a distinct token.  Other wavefronts report 0.
  if (bounds) {
    constexpr int per_wave = TPW * 32;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int gfull = nq[u] / per_wave;
      const int rank = bound_rank(topk, gfull, 32);
      uint32_t T = 0;
      if ((wid + 1) * per_wave <= nq[u] && rank >= 1) {
        // rank-th largest of the 32 lane maxima (lanes 32..63 hold 0): extract
        // the maximum rank times
        uint32_t v = half == 0 ? order_key(lane_best[u]) : 0u;
        for (int i = 0; i < rank; ++i) {
          T = wave_max_u32(v);
          const uint64_t hit = __ballot(v == T);
          if (lane == __ffsll((unsigned long long)hit) - 1) v = 0;
        }
      }
      if (lane == 0) bounds[(int64_t)(qi + u) * gridDim.x * 4 + wid] = T;
    }
  }
  // window rows: the visible counts for the kernels that follow (last, so that
  // no lane-dependent branch precedes the scalar code above)
  if (window > 0 && row_len_out && blockIdx.x == 0 && wave == 0) {
    int v = nq[0];
#pragma unroll
    for (int u = 1; u < NQ; ++u) v = lane == u ? nq[u] : v;
    if (lane < NQ) row_len_out[qi + lane] = v;
  }
}

// fp32 queries and keys: one thread per key, fp32 FMA chains in a fixed order
// (dims ascending, then heads ascending).
template <int D>
__global__ __launch_bounds__(256) void scores_f32_kernel(float *__restrict__ scores, int64_t ld,
                                                         const float *__restrict__ q, const float *__restrict__ w,
                                                         CacheDev keys, const int32_t *__restrict__ q_seq,
                                                         int seq_ident, const int32_t *__restrict__ q_len,
                                                         int n_heads) {
  __shared__ float lq[64 * D];
  __shared__ float lw[64];
  const int qi = blockIdx.y;
  const int n = q_len[qi];
  for (int i = threadIdx.x; i < n_heads * D; i += 256) lq[i] = q[(int64_t)qi * n_heads * D + i];
  for (int i = threadIdx.x; i < n_heads; i += 256) lw[i] = w[(int64_t)qi * n_heads + i];
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
  }
}

template <bool FP8, int D, int MT, int QW>
hipError_t run_mfma(float *scores, int64_t ld, const void *q, const float *w, const CacheDev &keys,
                    const int32_t *q_seq, int seq_ident, const int32_t *q_len, int n_q, int n_heads, int max_len,
                    const ScoreBounds &sb, int window, int32_t *row_len_out, hipStream_t stream) {
  const int rows = n_q / QW;   // workgroup rows of the grid
  const int tiles = (max_len + 31) / 32;
  const int tpw = score_tiles_per_wave(rows, max_len);
  const int gx = (tiles + 4 * tpw - 1) / (4 * tpw);
  dim3 grid(gx, rows);
  const uint16_t *qb = static_cast<const uint16_t *>(q);
#define DSA_SK(T)                                                                                                  \
  hipLaunchKernelGGL((scores_mfma_kernel<FP8, D, MT, T, QW>), grid, dim3(256), 0, stream, scores, ld, qb, w, keys, \
                     q_seq, seq_ident, q_len, n_heads, sb.bounds, sb.topk, window, row_len_out)
  switch (tpw) {
    case 1: DSA_SK(1); break;
    case 2: DSA_SK(2); break;
    case 4: DSA_SK(4); break;
    default: DSA_SK(8); break;
  }
#undef DSA_SK
  return hipGetLastError();
}

template <int D>
hipError_t run_f32(float *scores, int64_t ld, const void *q, const float *w, const CacheDev &keys,
                   const int32_t *q_seq, int seq_ident, const int32_t *q_len, int n_q, int n_heads, int max_len,
                   hipStream_t stream) {
  dim3 grid((max_len + 255) / 256, n_q);
  hipLaunchKernelGGL((scores_f32_kernel<D>), grid, dim3(256), 0, stream, scores, ld,
                     static_cast<const float *>(q), w, keys, q_seq, seq_ident, q_len, n_heads);
  return hipGetLastError();
}

hipError_t dispatch(float *scores, int64_t ld, const void *q, int q_dt, const float *w, const CacheDev &keys,
                    int key_dt, const int32_t *q_seq, int seq_ident, const int32_t *q_len, int n_q, int n_heads,
                    int max_len, const ScoreBounds &sb, int qw, int window, int32_t *row_len_out, hipStream_t s) {
  const int D = keys.width;
  if (q_dt == kF32) {
    switch (D) {
      case 32: return run_f32<32>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, s);
      case 64: return run_f32<64>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, s);
      case 96: return run_f32<96>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, s);
      case 128: return run_f32<128>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, s);
      default: return hipErrorInvalidValue;
    }
  }
  const bool fp8 = key_dt == kFP8;
  const bool two = n_heads > 32;
  // the GEMM-shaped kernel: contiguous caches, or paged ones with a power-of-two block size
  int block_shift = 0;
  while ((1 << block_shift) < keys.block_size && block_shift < 30) ++block_shift;
  const bool pow2_blocks = !keys.table || (1 << block_shift) == keys.block_size;
  if (!fp8 && D == 128 && !two && n_q >= kPrefillMinQueries && !sb.bounds && !seq_ident && window == 0 &&
      pow2_blocks) {
    return launch_prefill_scores(scores, ld, static_cast<const uint16_t *>(q), w, keys, q_seq, q_len, n_q,
                                 n_heads, max_len, block_shift, s);
  }
#define DSA_SC(F, DD, M, QWV)                                                                              \
  return run_mfma<F, DD, M, QWV>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, sb, window, \
                                 row_len_out, s)
  if (qw == 2 && !two && D == 128) {
    if (fp8) DSA_SC(true, 128, 2, 2);
    DSA_SC(false, 128, 2, 2);
  }
  if (qw != 1) return hipErrorInvalidValue;
  if (D == 128) {
    if (fp8) { if (two) DSA_SC(true, 128, 2, 1); DSA_SC(true, 128, 1, 1); }
    if (two) DSA_SC(false, 128, 2, 1);
    DSA_SC(false, 128, 1, 1);
  }
  if (D == 64) {
    if (fp8) { if (two) DSA_SC(true, 64, 2, 1); DSA_SC(true, 64, 1, 1); }
    if (two) DSA_SC(false, 64, 2, 1);
    DSA_SC(false, 64, 1, 1);
  }
#undef DSA_SC
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_index_scores(float *scores, int64_t ld, const void *q, int q_dt, const float *w,
                               const CacheDev &keys, int key_dt, const int32_t *q_seq, int seq_ident,
                               const int32_t *q_len, int n_q, int n_heads, int max_len, const ScoreBounds &sb,
                               hipStream_t stream, int qw, int window, int32_t *row_len_out) {
  if (qw != 1 && qw != 2) return hipErrorInvalidValue;
  if (qw > 1 && (n_q % qw || keys.width != 128 || n_heads > 32 || q_dt == kF32)) return hipErrorInvalidValue;
  if (window > 0 && (q_dt == kF32 || q_seq || n_q % window || window % qw)) return hipErrorInvalidValue;
  return dispatch(scores, ld, q, q_dt, w, keys, key_dt, q_seq, seq_ident, q_len, n_q, n_heads, max_len, sb, qw,
                  window, row_len_out, stream);
}

int score_tiles_per_wave(int n_q, int max_len) {
  // ~512 workgroups of 4 wavefronts; each wavefront streams 1, 2, 4 or 8
  // consecutive 32-key tiles so its q fragment load is amortised.
  const int64_t total = (int64_t)((max_len + 31) / 32) * n_q;
  const int64_t want = (total + 4 * 512 - 1) / (4 * 512);
  int tpw = 1;
  while (tpw < kMaxTilesPerWave && tpw < want) tpw *= 2;
  return tpw;
}

int score_group_tokens(int n_q, int max_len) { return 32 * score_tiles_per_wave(n_q, max_len); }

int score_groups_per_row(int n_q, int max_len) {
  const int tpw = score_tiles_per_wave(n_q, max_len);
  return 4 * (((max_len + 31) / 32 + 4 * tpw - 1) / (4 * tpw));
}

}  // namespace dsa
