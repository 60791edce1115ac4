// Lightning-indexer scores for many queries (chunked prefill): the
// GEMM-shaped kernel.
//
// score[i][s] = sum_h w[i][h] * max(0, <q_ih, k_s>) for every key s a query
// sees ("GLM on an A100, in Vx", sections "The model" and "How do we know it
// is right?": every earlier token is scored, ReLU per head before the heads
// are combined), as a bf16 GEMM of (query, head) rows against key columns with
// K = 128, fp32 accumulation, and the ReLU, head weights and head sum applied
// to the accumulators in registers.  Each score is the same fp32 sum in the
// same order as in the decode score kernel (index_scores.hip), so the two
// agree bit for bit.
#include "kernels.hpp"

namespace dsa {
namespace {

// max(x, 0) on the bits (one signed-integer max).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sum over lanes l and l ^ 32, formed in the same order in both.
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Many queries (chunked prefill), bf16 q and keys, 128-wide keys, up to 32
// heads: a GEMM over (query, head) rows and key columns with K = 128.  A
// workgroup owns kPQ consecutive queries and one range of keys; 128-key steps
// are staged in LDS once and shared by its 8 wavefronts, each scoring 2
// queries x 4 key tiles per step (8 MFMAs 32x32x16 per query and tile), so a
// wavefront reads a key tile from LDS once for both of its queries, one tile
// ahead of its MFMAs.  The next step's keys are loaded into registers while
// a step is scored and written to the other slot of a 2-slot LDS ring: one
// barrier per step.  Queries of a block that belong to different sequences are
// processed one sequence at a time.
constexpr int kPQ = 16;            // queries per workgroup
constexpr int kPStepKeys = 128;    // keys per step (four 32-key tiles)
constexpr int kPTiles = kPStepKeys / 32;   // 4 (the block lookups below name four)
constexpr int kPThreads = 512;
constexpr int kPRowB = 256;        // bf16 key row bytes (128 dims)
constexpr int kPLdsRow = kPRowB + 16;   // padded LDS row: conflict-free 16-byte operand reads

// PAGED: keys through a block table whose block size is 1 << block_shift;
// otherwise a contiguous cache (token t of a sequence at slot t of its block).
template <bool PAGED>
__global__ __launch_bounds__(kPThreads) void scores_prefill_kernel(float *__restrict__ scores, int64_t ld,
                                                                   const uint16_t *__restrict__ q,
                                                                   const float *__restrict__ w, CacheDev keys,
                                                                   const int32_t *__restrict__ q_seq,
                                                                   const int32_t *__restrict__ q_len, int n_q,
                                                                   int n_heads, int keys_per_split, int block_shift) {
  constexpr int D = 128, KS = D / 16, HALF = D / 2, CPR = kPRowB / 16;   // 16 chunks per row
  __shared__ __align__(16) uint8_t ring[2][kPStepKeys * kPLdsRow];          // 2 x 34 KB
  __shared__ int32_t sseq[kPQ], slen[kPQ];
  __shared__ int32_t groups[kPQ + 1];

  const int qb = blockIdx.x, split = blockIdx.y;
  // the wavefront index as a scalar: everything derived from it (the wavefront's
  // queries, their lengths, score rows) stays in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int qbase = qb * kPQ;
  if (tid < kPQ) {
    const int qi = qbase + tid;
    sseq[tid] = qi < n_q ? (q_seq ? q_seq[qi] : 0) : -1;
    slen[tid] = qi < n_q ? q_len[qi] : 0;
  }
  __syncthreads();
  if (tid == 0) {   // distinct sequences of the block, in order of first appearance
    int ng = 0;
    for (int i = 0; i < kPQ; ++i) {
      if (sseq[i] < 0) continue;
      bool seen = false;
      for (int j = 0; j < i; ++j) seen = seen || sseq[j] == sseq[i];
      if (!seen) groups[ng++] = sseq[i];
    }
    groups[kPQ] = ng;
  }

  // this wavefront's two queries: A operands (lane half h holds dims
  // 64 h + 8 ks + [0, 8) of head col, the key operand uses the same order) and
  // head weights (accumulator element r is head 8 (r / 4) + 4 half + r % 4)
  bf16x8 a[2][KS];
  float wr[2][16];
  int qn[2], qs[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int qi = qbase + 2 * wave + u;
    const bool ok = qi < n_q;
    const int head = col < n_heads ? col : 0;
    const uint16_t *qrow = q + ((int64_t)(ok ? qi : 0) * n_heads + head) * D + half * HALF;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = load16(qrow + 8 * ks);
      if (!ok || col >= n_heads) v = u32x4{0, 0, 0, 0};
      a[u][ks] = as_bf16x8(v);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      wr[u][r] = (ok && m < n_heads) ? w[(int64_t)qi * n_heads + m] : 0.0f;
    }
  }
  __syncthreads();
  float *orow[2];   // this wavefront's score rows
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    qn[u] = slen[2 * wave + u];
    qs[u] = sseq[2 * wave + u];
    const int qi = qbase + 2 * wave + u;
    orow[u] = scores + (int64_t)(qi < n_q ? qi : 0) * ld;
  }
  const int ngroups = groups[kPQ];

  for (int gi = 0; gi < ngroups; ++gi) {
    const int seq = groups[gi];
    int nmax = 0;
    for (int i = 0; i < kPQ; ++i) nmax = sseq[i] == seq ? max(nmax, slen[i]) : nmax;
    const int k0 = split * keys_per_split;
    const int k1 = min(k0 + keys_per_split, nmax);
    if (k0 >= k1) continue;   // uniform over the workgroup
    const int nsteps = (k1 - k0 + kPStepKeys - 1) / kPStepKeys;

    // key step loads: thread t takes 16-byte chunk lch = t % 16 of rows
    // lrow + 32 x (x < 4) of the step, lrow = t / 16; rows past k1 are clamped
    // to k1 - 1.  Steps start on multiples of 32 tokens and blocks hold a
    // multiple of 32, so each 32-row group lies in one block: one uniform
    // lookup per group (the block index a shift), a scalar group base address
    // and a 32-bit lane offset (the row stride is below 2^24), no branch.
    const int lrow = tid / CPR, lch = tid % CPR;
    const uint32_t rs32 = (uint32_t)keys.row_stride;
    auto load_step = [&](int st, u32x4 (&r)[kPTiles]) {
      const int sc = st < nsteps ? st : nsteps - 1;
      const int t0 = k0 + sc * kPStepKeys;
      int gl[kPTiles], blk[kPTiles], slot0[kPTiles];
#pragma unroll
      for (int x = 0; x < kPTiles; ++x) {
        const int g0 = t0 + 32 * x;
        gl[x] = g0 < k1 ? g0 : ((k1 - 1) & ~31);   // the group's first row (in range)
      }
      // all lookups in flight together, then all key loads (no branch between
      // a load and the next)
      if (PAGED) {
        // the block table is read-only here: read it through the constant
        // address space, so the uniform lookups are scalar loads
        const auto trow = reinterpret_cast<const __attribute__((address_space(4))) int32_t *>(
            reinterpret_cast<uintptr_t>(keys.table + (int64_t)seq * keys.max_blocks));
#pragma unroll
        for (int x = 0; x < kPTiles; ++x) {
          blk[x] = trow[gl[x] >> block_shift];
          slot0[x] = gl[x] & ((1 << block_shift) - 1);
        }
        asm("" : "+s"(blk[0]), "+s"(blk[1]), "+s"(blk[2]), "+s"(blk[3]));   // all four before any use
      } else {
#pragma unroll
        for (int x = 0; x < kPTiles; ++x) {
          blk[x] = seq;
          slot0[x] = gl[x];
        }
      }
#pragma unroll
      for (int x = 0; x < kPTiles; ++x) {
        const uint8_t *gbase = keys.rows + (int64_t)blk[x] * keys.block_stride + (int64_t)slot0[x] * keys.row_stride;
        const uint32_t row = (uint32_t)min(lrow, k1 - 1 - gl[x]);
        r[x] = load16_nt(gbase + (row * rs32 + 16u * (uint32_t)lch));
      }
    };
    auto store_step = [&](int st, const u32x4 (&r)[kPTiles]) {
      uint8_t *buf = ring[st & 1] + lrow * kPLdsRow + 16 * lch;
#pragma unroll
      for (int x = 0; x < kPTiles; ++x) *reinterpret_cast<u32x4 *>(buf + 32 * x * kPLdsRow) = r[x];
    };
    // key operand of tile tl: lane (col, half) reads 128 contiguous bytes of row
    // 32 tl + col from byte 128 half (the padded rows keep 16 lanes on distinct banks)
    const int bofs = col * kPLdsRow + 128 * half;
    auto read_b = [&](int st, int tl, bf16x8 (&b)[KS]) {
      const uint8_t *rp = ring[st & 1] + tl * 32 * kPLdsRow + bofs;
#pragma unroll
      for (int j = 0; j < KS; ++j) b[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(rp + 16 * j));
    };
    // Epilogue of one (query u, key tile) combination: ReLU, head weights, head
    // sum.  The store is predicated once: every key of the tile visible to
    // query u (both lane halves hold the same sum and store it), or this
    // lane's key visible (lower half).
    auto head_sum = [&](const f32x16 &acc, int u) {
      float s = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) s = fmaf(wr[u][r], relu(acc[r]), s);
      return halves_sum(s);
    };
    // keys below lim[u] are visible to query u in this key range (0: the query
    // belongs to another sequence).  Both lane halves hold the same sums and
    // store them to the same addresses.
    int lim[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) lim[u] = qs[u] == seq ? min(qn[u], k1) : 0;
    auto store_score = [&](float s, int u, int key) {   // key -1 (nothing pending) fails the unsigned test
      if ((uint32_t)key < (uint32_t)lim[u]) orow[u][(uint32_t)key] = s;
    };
    // Per step: 8 (tile, query) combinations.  The 8 MFMAs of one combination
    // are interleaved (scheduling groups of 1 MFMA + 5 VALU) with the epilogue
    // of the one before it, across steps too: the last combination's epilogue
    // runs past the barrier, under the next step's first MFMAs.
    f32x16 acc[2] = {f32x16{}, f32x16{}};   // query u accumulates in acc[u]
    int pend_key = -1;                        // key of the pending (tile, query 1) epilogue; -1: none
    auto compute_step = [&](int st) {
      const int kb = k0 + st * kPStepKeys;
      bf16x8 b[2][KS];
      read_b(st, 0, b[0]);
#pragma unroll
      for (int tl = 0; tl < kPTiles; ++tl) {
        if (tl + 1 < kPTiles) read_b(st, tl + 1, b[(tl + 1) & 1]);
        const int key0 = kb + 32 * tl;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u][0], b[tl & 1][0], f32x16{}, 0, 0, 0);
#pragma unroll
          for (int ks = 1; ks < KS; ++ks)
            acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u][ks], b[tl & 1][ks], acc[u], 0, 0, 0);
          // the previous combination (query u ^ 1): (tile tl - 1, query 1) or (tile tl, query 0)
          const float sp = head_sum(acc[u ^ 1], u ^ 1);
#pragma unroll
          for (int i = 0; i < KS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // 5 VALU
          }
          if (u == 0) store_score(sp, 1, pend_key);
          else store_score(sp, 0, key0 + col);
        }
        pend_key = key0 + col;
      }
    };

    u32x4 rn[kPTiles];
    load_step(0, rn);
    store_step(0, rn);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      load_step(st + 1, rn);
      compute_step(st);
      store_step(st + 1, rn);
      __syncthreads();
    }
    store_score(head_sum(acc[1], 1), 1, pend_key);
    pend_key = -1;
  }
}

}  // namespace

hipError_t launch_prefill_scores(float *scores, int64_t ld, const uint16_t *q, const float *w, const CacheDev &keys,
                                 const int32_t *q_seq, const int32_t *q_len, int n_q, int n_heads, int max_len,
                                 int block_shift, hipStream_t stream) {
  const int blocks = (n_q + kPQ - 1) / kPQ;
  // split the keys so that about 512 workgroups run
  int splits = (512 + blocks - 1) / blocks;
  int per = (max_len + splits - 1) / splits;
  per = (per + kPStepKeys - 1) / kPStepKeys * kPStepKeys;
  splits = (max_len + per - 1) / per;
  if (keys.table)
    hipLaunchKernelGGL(scores_prefill_kernel<true>, dim3(blocks, splits), dim3(kPThreads), 0, stream, scores, ld, q,
                       w, keys, q_seq, q_len, n_q, n_heads, per, block_shift);
  else
    hipLaunchKernelGGL(scores_prefill_kernel<false>, dim3(blocks, splits), dim3(kPThreads), 0, stream, scores, ld, q,
                       w, keys, q_seq, q_len, n_q, n_heads, per, 0);
  return hipGetLastError();
}

}  // namespace dsa
