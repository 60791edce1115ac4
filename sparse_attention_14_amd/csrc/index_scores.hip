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
constexpr int kMaxPairTiles = 16;
constexpr int kPrefillMinQueries = 64;   // the GEMM-shaped kernel (prefill_scores.hip) takes over from here


// One wavefront scores TPW consecutive 32-key tiles.  The tile loop is fully
// unrolled and every tile load is issued unconditionally (tiles past the row's
// end reload its last tile and their scores are dropped), so the code is
// straight-line and the compiler waits for exactly the tile it needs while the
// next P tiles stay in flight.  Tile positions, block-table lookups and tile
// base addresses are wavefront-uniform (scalar); a lane adds one precomputed
// 32-bit offset per load.
//
// One query per workgroup row (row y); MT = 2: the M tiles are heads 0-31 and
// 32-63 of it.
//
// window > 0: rows are the queries of multi-token windows, row i the (i % window)-th
// of sequence i / window, whose visible count is q_len[i / window] - window + 1 +
// i % window (at least 0; q_len then holds the sequences' lengths).  The
// workgroups of the first key range write each row's count to row_len_out.
template <bool FP8, int D, int MT, int TPW>
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
  const int qi = blockIdx.y;   // score row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  // visible tokens of the row
  const int n = window > 0 ? max(q_len[qi / window] - window + 1 + qi % window, 0) : q_len[qi];
  const int ntile = (n + 31) / 32;
  const int wid = blockIdx.x * 4 + wave + zero;
  const int tile_begin = wid * TPW;
  float lane_best = -__builtin_inff();   // largest score of this lane's keys (bounds only)

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
      const int head = 32 * mt + col;
      const uint16_t *qrow = q + ((int64_t)qi * n_heads + (head < n_heads ? head : n_heads - 1)) * D + half * HALF;
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
        const float x = w[(int64_t)qi * n_heads + (m < n_heads ? m : n_heads - 1)];
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
      float su = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][ks], b[ks], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) su = fmaf(wr[mt][r], relu(__uint_as_float(__float_as_uint(acc[r]) ^ flip)), su);
      }
      const int t = (tile_begin + it) * 32 + col;
      float x = FP8 ? su * fabsf(sc) : su;
      x = halves_sum(x);
      if (half == 0 && t < n) scores[(int64_t)qi * ld + t] = x;
      // only wavefronts whose keys are all visible to the row report a
      // bound, so every score reaches the maximum unmasked
      lane_best = fmaxf(lane_best, x);
    }
  }

  // Candidate bound for the top-k: a full wavefront (all TPW * 32 of its
  // tokens visible) reports the r-th largest of its lanes' maxima,
  // r = bound_rank(k, G, 32) with G full wavefronts in the row; each lane
  // maximum is the score of a distinct token.  Other wavefronts report 0.
  if (bounds) {
    constexpr int per_wave = TPW * 32;
    const int gfull = n / per_wave;
    const int rank = bound_rank(topk, gfull, 32);
    uint32_t T = 0;
    if ((wid + 1) * per_wave <= n && rank >= 1) {
      // rank-th largest of the 32 lane maxima (lanes 32..63 hold 0): extract
      // the maximum rank times
      uint32_t v = half == 0 ? order_key(lane_best) : 0u;
      for (int i = 0; i < rank; ++i) {
        T = wave_max_u32(v);
        const uint64_t hit = __ballot(v == T);
        if (lane == __ffsll((unsigned long long)hit) - 1) v = 0;
      }
    }
    if (lane == 0) bounds[(int64_t)qi * gridDim.x * 4 + wid] = T;
  }
  // window rows: the visible counts for the kernels that follow (last, so that
  // no lane-dependent branch precedes the scalar code above)
  if (window > 0 && row_len_out && blockIdx.x == 0 && wave == 0 && lane == 0) row_len_out[qi] = n;
}

// Query pairs of multi-token decode windows: rows 2 y and 2 y + 1 (neighbouring
// queries of one sequence, up to 32 heads each) are the two M tiles of the MFMA,
// so every key tile serves both.  The result of every score is the same as in
// scores_mfma_kernel (the same products, accumulation order and epilogue).
//
// The key tiles go from memory straight into LDS (direct-to-LDS copies, no
// registers in between): each wavefront keeps P tiles in flight in stage
// buffers of its own (P + 1 of them).  The head weights of the pair are read
// from LDS in the epilogue, or held in registers when the stage buffers already
// limit the CU to two workgroups.  Each 16-byte chunk of the tile is converted
// and multiplied in turn, so the conversion of one chunk overlaps the MFMAs of
// the previous one.
//
// Stage layout: tile row kk at kk * ROWB, its chunk c in slot c ^ (kk % CPR)
// (against LDS bank conflicts when 32 lanes read 32 rows).  A copy writes 64
// consecutive slots, so lane l of copy j fetches the chunk that belongs in slot
// 64 j + l: a permutation of 16-byte chunks within each row, still one 128-byte
// line per 8 lanes.  fp8: the tile's 32 scales follow the tile (lanes 32-63
// load them again).
//
// Waits: a wavefront waits for the copies of tile it (its own vmcnt) with the
// later tiles' copies still in flight, counting copies only: a store issued
// in between can only lengthen the wait.  The scores of tile it are stored
// after the wait of tile it + 1, a whole tile before the next wait they could
// lengthen.
template <bool FP8, int TPW, int P>
__global__ __launch_bounds__(256) void scores_pair_kernel(float *__restrict__ scores, int64_t ld,
                                                          const uint16_t *__restrict__ q, const float *__restrict__ w,
                                                          CacheDev keys, const int32_t *__restrict__ seq_len,
                                                          int n_heads, uint32_t *__restrict__ bounds, int topk,
                                                          int window, int32_t *__restrict__ row_len_out) {
  constexpr int D = 128, KS = D / 16, HALF = D / 2;
  constexpr int ROWB = FP8 ? D : 2 * D;     // key row bytes
  constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  constexpr int HALFC = CPR / 2;            // chunks per lane half
  constexpr int TILEB = 32 * ROWB;
  constexpr int NLD = TILEB / 1024;         // 1 KB copies per tile
  constexpr int OPS = NLD + (FP8 ? 1 : 0);  // copy instructions per tile (keys, scales)
  constexpr int NB = P + 1;                 // P tiles in flight ahead of the one being scored
  constexpr int BUFB = TILEB + (FP8 ? 256 : 0);
  // head weights in registers when the stage buffers already limit the CU to
  // two workgroups (registers to spare), else read from LDS in the epilogue
  constexpr bool WREG = 3 * 4 * NB * BUFB > 160 * 1024;
  __shared__ __align__(16) uint8_t stage_all[4 * NB * BUFB];
  __shared__ __align__(16) float wl[2][32];

  int zero;
  asm("s_mov_b32 %0, 0"
      : "=s"(zero)
      : "s"(scores), "s"(ld), "s"(q), "s"(w), "s"(keys.rows), "s"(keys.scale), "s"(keys.row_stride),
        "s"(keys.block_stride), "s"(keys.scale_block_stride), "s"(keys.table), "s"(keys.block_size),
        "s"(keys.max_blocks), "s"(seq_len), "s"(n_heads), "s"(bounds), "s"(topk), "s"(window), "s"(row_len_out));
  const int qi = 2 * blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int seq = qi / window;
  const int sl = seq_len[seq], j0 = qi % window;
  int nq[2];
  nq[0] = max(sl - window + 1 + j0, 0);
  nq[1] = max(sl - window + 2 + j0, 0);
  const int n = nq[1];
  const int ntile = (n + 31) / 32;
  const int wid = blockIdx.x * 4 + wave + zero;
  const int tile_begin = wid * TPW;
  const bool active = tile_begin < ntile;
  float lane_best[2] = {-__builtin_inff(), -__builtin_inff()};
  uint8_t *stage = stage_all + wave * NB * BUFB;

  // Tile bases (wavefront-uniform): a 32-key tile never straddles a block.
  const uint8_t *tbase[TPW];
  const uint8_t *sbase[TPW];
  uint32_t tlim[TPW];   // byte offset of the last chunk of the tile's last visible row
  int tlast[TPW];
  {
    int bi[TPW], slot[TPW];
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      int tile = tile_begin + it;
      tile = tile < ntile ? tile : ntile - 1;
      tile = tile > 0 ? tile : 0;
      const int t0 = tile * 32;
      bi[it] = t0 / keys.block_size;
      slot[it] = t0 - bi[it] * keys.block_size;
      tlast[it] = n - 1 - t0;
    }
    int blk[(TPW + 7) / 8 * 8] = {};
    if (keys.table && active) {
      const int32_t *trow = keys.table + (int64_t)seq * keys.max_blocks;
#pragma unroll
      for (int it = 0; it < TPW; ++it) blk[it] = trow[bi[it]];
      // every lookup is in flight before the first is used
#pragma unroll
      for (int c = 0; c < TPW; c += 8)
        asm("" : "+s"(blk[c]), "+s"(blk[c + 1]), "+s"(blk[c + 2]), "+s"(blk[c + 3]), "+s"(blk[c + 4]),
            "+s"(blk[c + 5]), "+s"(blk[c + 6]), "+s"(blk[c + 7]));
    } else if (!keys.table) {
#pragma unroll
      for (int it = 0; it < TPW; ++it) blk[it] = seq;
    }
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      tbase[it] = keys.rows + (int64_t)blk[it] * keys.block_stride + (int64_t)slot[it] * keys.row_stride;
      sbase[it] = FP8 ? reinterpret_cast<const uint8_t *>(keys.scale + (int64_t)blk[it] * keys.scale_block_stride +
                                                           slot[it])
                      : nullptr;
      tlim[it] = (uint32_t)tlast[it] * (uint32_t)keys.row_stride + (ROWB - 16);
    }
  }
  // This lane's source offset for copy j (rows past the last visible one are
  // replaced by that row: min() with tlim), and its scale's offset.
  const uint32_t rs = (uint32_t)keys.row_stride;
  uint32_t coff[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int kk = (64 * j + lane) / CPR, sl16 = lane % CPR;
    coff[j] = (uint32_t)kk * rs + 16u * (uint32_t)(sl16 ^ (kk & (CPR - 1)));
  }
  auto issue = [&](int it) {
    uint8_t *buf = stage + (it % NB) * BUFB;
#pragma unroll
    for (int j = 0; j < NLD; ++j) copy16_to_lds(tbase[it], min(coff[j], tlim[it]), buf + 1024 * j);
    if (FP8) copy4_to_lds(sbase[it], 4u * (uint32_t)min(col, tlast[it]), buf + TILEB);
  };
  if (active) {
#pragma unroll
    for (int p = 0; p < P && p < TPW; ++p) issue(p);
  }

  // The q fragments into registers (lane (col, half) holds head col, dims
  // half*HALF + 8*ks + [0, 8)), then the head weights of the pair into LDS (the
  // wait for the weights is then also the wait for the fragments).
  bf16x8 a[2][KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int head = col < n_heads ? col : n_heads - 1;
    const uint16_t *qrow = q + ((int64_t)(qi + mt) * n_heads + head) * D + half * HALF;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = load16(qrow + 8 * ks);
      if (col >= n_heads) v = u32x4{0, 0, 0, 0};
      a[mt][ks] = as_bf16x8(v);
    }
  }
  if (threadIdx.x < 64) {
    const int u = threadIdx.x >> 5, h = threadIdx.x & 31;
    wl[u][h] = h < n_heads ? w[(int64_t)(qi + u) * n_heads + h] : 0.0f;
  }
  __syncthreads();
  f32x4 wr[2][4];
  if (WREG) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) wr[u][g] = *reinterpret_cast<const f32x4 *>(&wl[u][8 * g + 4 * half]);
  }

  if (active) {
    // this lane's stage offsets: row col, chunks half*HALFC + j
    uint32_t roff[HALFC];
#pragma unroll
    for (int j = 0; j < HALFC; ++j) roff[j] = col * ROWB + 16 * ((half * HALFC + j) ^ (col & (CPR - 1)));
    float xs[2] = {0.0f, 0.0f};
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      // copy groups issued after tile it's: tiles it+1 .. it+P-1 (those that exist)
      static_assert(P >= 1 && P <= 3, "up to two later copy groups");
      const int later = (TPW - 1 - it) < (P - 1) ? (TPW - 1 - it) : (P - 1);
      // (and the reads of the previous tile done: its buffer takes the copies below)
      if (later >= 2) wait_vm_lds<2 * OPS>();
      else if (later == 1) wait_vm_lds<OPS>();
      else wait_vm_lds<0>();
      const uint8_t *buf = stage + (it % NB) * BUFB;
      u32x4 raw[HALFC];
#pragma unroll
      for (int j = 0; j < HALFC; ++j) raw[j] = *reinterpret_cast<const u32x4 *>(buf + roff[j]);
      const float sc = FP8 ? *reinterpret_cast<const float *>(buf + TILEB + 4 * col) : 1.0f;
      // the previous tile's scores (stored here, after the wait)
      if (it > 0) {
        const int tp = (tile_begin + it - 1) * 32 + col;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (half == 0 && tp < nq[u]) scores[(int64_t)(qi + u) * ld + tp] = xs[u];
      }
      if (it + P < TPW) issue(it + P);
      f32x16 acc0 = {}, acc1 = {};
#pragma unroll
      for (int j = 0; j < HALFC; ++j) {
        if (FP8) {
          const bf16x8 b0 = fp8x8_to_bf16x8(raw[j][0], raw[j][1]);
          const bf16x8 b1 = fp8x8_to_bf16x8(raw[j][2], raw[j][3]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][2 * j], b0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][2 * j], b0, acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][2 * j + 1], b1, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][2 * j + 1], b1, acc1, 0, 0, 0);
        } else {
          const bf16x8 b = as_bf16x8(raw[j]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][j], b, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][j], b, acc1, 0, 0, 0);
        }
      }
      // Epilogue as in scores_mfma_kernel: accumulator element r of this lane is
      // head 8*(r/4) + 4*half + r%4; fp8 scale sign by flipping the accumulator's.
      const uint32_t flip = FP8 ? (__float_as_uint(sc) & 0x80000000u) : 0u;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x16 &acc = u ? acc1 : acc0;
        float su = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 wv = WREG ? wr[u][g] : *reinterpret_cast<const f32x4 *>(&wl[u][8 * g + 4 * half]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            su = fmaf(wv[i], relu(__uint_as_float(__float_as_uint(acc[4 * g + i]) ^ flip)), su);
        }
        float x = FP8 ? su * fabsf(sc) : su;
        x = halves_sum(x);
        xs[u] = x;
        lane_best[u] = fmaxf(lane_best[u], x);
      }
    }
    {
      const int tp = (tile_begin + TPW - 1) * 32 + col;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (half == 0 && tp < nq[u]) scores[(int64_t)(qi + u) * ld + tp] = xs[u];
    }
  }

  // candidate bounds, as in scores_mfma_kernel
  if (bounds) {
    constexpr int per_wave = TPW * 32;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int gfull = nq[u] / per_wave;
      const int rank = bound_rank(topk, gfull, 32);
      uint32_t T = 0;
      if ((wid + 1) * per_wave <= nq[u] && rank >= 1) {
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
  if (row_len_out && blockIdx.x == 0 && wave == 0) {
    const int v = lane == 0 ? nq[0] : nq[1];
    if (lane < 2) row_len_out[qi + lane] = v;
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

template <bool FP8, int D, int MT>
hipError_t run_mfma(float *scores, int64_t ld, const void *q, const float *w, const CacheDev &keys,
                    const int32_t *q_seq, int seq_ident, const int32_t *q_len, int n_q, int n_heads, int max_len,
                    const ScoreBounds &sb, int window, int32_t *row_len_out, hipStream_t stream) {
  const int rows = n_q;   // workgroup rows of the grid
  const int tiles = (max_len + 31) / 32;
  const int tpw = score_tiles_per_wave(rows, max_len);
  const int gx = (tiles + 4 * tpw - 1) / (4 * tpw);
  dim3 grid(gx, rows);
  const uint16_t *qb = static_cast<const uint16_t *>(q);
#define DSA_SK(T)                                                                                                  \
  hipLaunchKernelGGL((scores_mfma_kernel<FP8, D, MT, T>), grid, dim3(256), 0, stream, scores, ld, qb, w, keys, \
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

template <bool FP8>
hipError_t run_pair(float *scores, int64_t ld, const void *q, const float *w, const CacheDev &keys,
                    const int32_t *seq_len, int n_q, int n_heads, int max_len, const ScoreBounds &sb, int window,
                    int32_t *row_len_out, hipStream_t stream) {
  const int rows = n_q / 2;
  const int tiles = (max_len + 31) / 32;
  const int tpw = score_tiles_per_wave(rows, max_len, true);
  const int gx = (tiles + 4 * tpw - 1) / (4 * tpw);
  dim3 grid(gx, rows);
  const uint16_t *qb = static_cast<const uint16_t *>(q);
  // fp8: two tiles in flight (three stage buffers, 52 KB: three workgroups per
  // CU), three for the longest rows (69 KB: two per CU, as many as that grid
  // has); bf16 tiles are twice as large: one in flight
#define DSA_SP(T, PP)                                                                                              \
  hipLaunchKernelGGL((scores_pair_kernel<FP8, T, PP>), grid, dim3(256), 0, stream, scores, ld, qb, w, keys, seq_len, \
                     n_heads, sb.bounds, sb.topk, window, row_len_out)
  switch (tpw) {
    case 1: DSA_SP(1, 1); break;
    case 2: DSA_SP(2, FP8 ? 2 : 1); break;
    case 4: DSA_SP(4, FP8 ? 2 : 1); break;
    case 8: DSA_SP(8, FP8 ? 2 : 1); break;
    default: DSA_SP(16, FP8 ? 3 : 1); break;
  }
#undef DSA_SP
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
#define DSA_SC(F, DD, M)                                                                                   \
  return run_mfma<F, DD, M>(scores, ld, q, w, keys, q_seq, seq_ident, q_len, n_q, n_heads, max_len, sb, window, \
                                 row_len_out, s)
  if (qw == 2) {
    if (two || D != 128 || window <= 0) return hipErrorInvalidValue;
    if (fp8) return run_pair<true>(scores, ld, q, w, keys, q_len, n_q, n_heads, max_len, sb, window, row_len_out, s);
    return run_pair<false>(scores, ld, q, w, keys, q_len, n_q, n_heads, max_len, sb, window, row_len_out, s);
  }
  if (qw != 1) return hipErrorInvalidValue;
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
                               const int32_t *q_len, int n_q, int n_heads, int max_len, const ScoreBounds &sb,
                               hipStream_t stream, int qw, int window, int32_t *row_len_out) {
  if (qw != 1 && qw != 2) return hipErrorInvalidValue;
  if (qw > 1 && (n_q % qw || keys.width != 128 || n_heads > 32 || q_dt == kF32 || window <= 0))
    return hipErrorInvalidValue;
  if (window > 0 && (q_dt == kF32 || q_seq || n_q % window || window % qw)) return hipErrorInvalidValue;
  return dispatch(scores, ld, q, q_dt, w, keys, key_dt, q_seq, seq_ident, q_len, n_q, n_heads, max_len, sb, qw,
                  window, row_len_out, stream);
}

int score_tiles_per_wave(int n_q, int max_len, bool pair) {
  // ~512 workgroups of 4 wavefronts; each wavefront streams 1, 2, 4 or 8
  // consecutive 32-key tiles (query pairs: up to 16, so that the longest rows
  // fill the chip in one round) so its q fragment load is amortised.
  const int64_t total = (int64_t)((max_len + 31) / 32) * n_q;
  const int64_t want = (total + 4 * 512 - 1) / (4 * 512);
  const int most = pair ? kMaxPairTiles : kMaxTilesPerWave;
  int tpw = 1;
  while (tpw < most && tpw < want) tpw *= 2;
  return tpw;
}

int score_group_tokens(int n_q, int max_len, bool pair) { return 32 * score_tiles_per_wave(n_q, max_len, pair); }

int score_groups_per_row(int n_q, int max_len, bool pair) {
  const int tpw = score_tiles_per_wave(n_q, max_len, pair);
  return 4 * (((max_len + 31) / 32 + 4 * tpw - 1) / (4 * tpw));
}

}  // namespace dsa
