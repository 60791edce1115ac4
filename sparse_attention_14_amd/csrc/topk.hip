// Exact top-k selection.
//
// Keeps the first min(k, n) entries of a stable descending sort of a score row:
// the best k, everything when n <= k, ties to the lower token index ("GLM on an
// A100, in Vx", sections "The model" and "How do we know it is right?").  The
// kept token indices are written in ascending order.
//
// All decisions are integer comparisons of order_key(score), so the result is
// exact and deterministic.  Method:
//  1. Candidate bound.  The row is cut into G groups; each full group reports a
//     lower bound on its ceil(k / G)-th largest key (the score kernel does this
//     as it writes the scores; otherwise bound_kernel does).  At least k keys of
//     the row are >= T_lo = the minimum of these, and in practice only ~1.5-3 k.
//     Rows that fit the candidate buffer use T_lo = 0 (every score).
//  2. Filter.  The workgroups of a row scan their chunks, reserve room in the
//     row's candidate array with one atomic each, and write the (key, token)
//     pairs with key >= T_lo there.
//  3. The last workgroup of the row (one atomic per workgroup) loads the
//     candidates into registers and finds the exact k-th key T and the tie quota
//     r = k - #(> T) with up to three 12-bit radix levels over a window that
//     spans the candidates' keys.  If the candidates do not fit, the same
//     selection runs over the whole row in memory instead: exact, slower.
//  4. Ordered emission: candidates above T set a "sel" bit and candidates equal
//     to T an "eq" bit in per-row LDS bitmaps; one pass over the bitmap words in
//     token order keeps all sel bits and the first r eq bits (a block-wide
//     prefix count of eq bits gives each word its quota).
// When one workgroup owns a row (many rows, or short rows) it does all of this
// alone, with candidates in LDS and no global state.  The last workgroup leaves
// the row's counters zeroed for the next call.
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int kSelThreads = 512;
constexpr int kPerThread = 8;              // scores loaded per thread per pass
constexpr int kCandPerThread = 24;         // candidates held per thread
constexpr int kGroup = 1024;               // tokens per bound group (bound_kernel)
constexpr int kSamples = 1024;

__device__ __forceinline__ uint32_t lowest_bits(uint32_t e, uint32_t take) {
  uint32_t r = 0;
  for (uint32_t i = 0; i < take; ++i) {
    const uint32_t lb = e & (~e + 1u);
    r |= lb;
    e ^= lb;
  }
  return r;
}

// One histogram increment; a wavefront whose active lanes all hit the same bin
// (ties, narrow windows) adds once instead of serialising on one LDS address.
__device__ __forceinline__ void hist_add(uint32_t *h, uint32_t bin) {
  const uint64_t act = __ballot(1);
  const uint32_t first = (uint32_t)__builtin_amdgcn_readfirstlane((int)bin);
  if (__ballot(bin == first) == act) {
    if ((int)(threadIdx.x & 63) == __ffsll((unsigned long long)act) - 1) atomicAdd(&h[first], (uint32_t)__popcll(act));
  } else {
    atomicAdd(&h[bin], 1u);
  }
}

// Among h[0..nbins), find the highest bin b whose suffix count (bins >= b)
// reaches `need` (1 <= need <= total).  out[0] = b, out[1] = count of bins > b.
__device__ void find_from_top(const uint32_t *h, int nbins, uint32_t need, uint32_t *scratch, uint32_t *out) {
  const int per = nbins >= kSelThreads ? nbins / kSelThreads : 1;
  const int t = threadIdx.x;
  const bool owns = t * per < nbins;
  const int hi = nbins - t * per;  // thread t owns bins [hi - per, hi), counted from the top
  uint32_t hv[kHistBins / kSelThreads];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < kHistBins / kSelThreads; ++j) {
    hv[j] = (owns && j < per) ? h[hi - 1 - j] : 0u;
    local += hv[j];
  }
  uint32_t tot;
  const uint32_t before = block_exclusive_scan(local, scratch, &tot);
  if (owns && before < need && before + local >= need) {
    uint32_t run = before;
#pragma unroll
    for (int j = 0; j < kHistBins / kSelThreads; ++j) {
      if (j < per && run < need && run + hv[j] >= need) {
        out[0] = (uint32_t)(hi - 1 - j);
        out[1] = run;
      }
      run += hv[j];
    }
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t *scratch) {
  const uint32_t m = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = max(r, scratch[i]);
  __syncthreads();
  return r;
}

struct SelectArgs {
  int32_t *indices;
  int32_t *counts;
  const float *scores;
  int64_t ld;
  const int32_t *q_len;
  const uint32_t *bounds;  // [n_q][n_bounds] group bounds, or nullptr
  int n_bounds;
  int k;
  int chunk;       // tokens per workgroup (multiple of 64)
  int chunks;      // workgroups per row
  int words;       // bitmap words allocated per row (LDS)
  int cand_cap;    // candidate capacity per row
  uint32_t *ctrl;  // [n_q][4]: done counter, candidate counter
  uint2 *cand;     // [n_q][cand_cap]  (key, token)
};

// Calls f(key, token) for every score of the row (the exact path when the
// candidates do not fit); loads are issued kPerThread at a time.
template <typename F>
__device__ __forceinline__ void for_each_in_row(const float *row, int n, F &&f) {
  for (int g0 = 0; g0 < n; g0 += kPerThread * kSelThreads) {
    float v[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int t = g0 + threadIdx.x + kSelThreads * i;
      v[i] = t < n ? row[t] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int t = g0 + threadIdx.x + kSelThreads * i;
      if (t < n) f(order_key(v[i]), (uint32_t)t);
    }
  }
}

// Exact selection of the k best, then emission of the ascending index list.
// When `in_regs`, this thread's candidates are ck/ct[0..nc), every key >= the
// k-th key of the row is among the block's candidates, and all of them are
// >= lo; otherwise the whole row is read from memory (lo = 0).
__device__ void finish_row(const SelectArgs &a, int qi, int n, bool in_regs, const uint32_t *ck, const uint32_t *ct,
                           int nc, uint32_t lo, const float *row, uint32_t *lh, uint32_t *scratch, uint32_t *shv,
                           uint32_t *sel_l, uint32_t *eq_l) {
  const int tid = threadIdx.x;
  const int k = a.k;
  const int n_words = (n + 31) >> 5;
  for (int w = tid; w < n_words; w += kSelThreads) {
    sel_l[w] = 0;
    eq_l[w] = 0;
  }
  auto visit = [&](auto &&f) {
    if (in_regs) {
#pragma unroll
      for (int m = 0; m < kCandPerThread; ++m)
        if (m < nc) f(ck[m], ct[m]);
    } else {
      for_each_in_row(row, n, f);
    }
  };
  uint32_t r = 0;
  if (n <= k) {
    // every token is kept
    for (int w = tid; w < n_words; w += kSelThreads) {
      const int rem = n - 32 * w;
      sel_l[w] = rem >= 32 ? 0xFFFFFFFFu : ((1u << rem) - 1u);
    }
    __syncthreads();
  } else {
    if (!in_regs) lo = 0;
    // key window [lo, hi] of the source; levels of 12 bits from its top
    uint32_t mx = 0;
    visit([&](uint32_t key, uint32_t) { mx = max(mx, key); });
    const uint32_t range = block_max(mx, scratch) - lo;
    const int width = range ? 32 - __clz(range) : 0;   // bits of (key - lo)
    // level i histograms bits [sh, prev) of (key - lo) among the keys whose
    // bits >= prev match the prefix selected so far
    int prev = 32;
    int sh = width > 12 ? width - 12 : 0;
    uint32_t base = 0;       // selected bits of (key - lo) at and above prev
    uint32_t need = (uint32_t)k;
    while (true) {
      for (int i = tid; i < kHistBins; i += kSelThreads) lh[i] = 0;
      __syncthreads();
      const uint32_t mask = prev - sh >= 12 ? 0xFFFu : ((1u << (prev - sh)) - 1u);
      visit([&](uint32_t key, uint32_t) {
        const uint32_t off = key - lo;
        if (prev == 32 || (off >> prev) == (base >> prev)) hist_add(lh, (off >> sh) & mask);
      });
      __syncthreads();
      find_from_top(lh, kHistBins, need, scratch, shv);
      base |= (shv[0] & 0xFFFu) << sh;
      need -= shv[1];
      __syncthreads();
      if (sh == 0) break;
      prev = sh;
      sh = sh > 12 ? sh - 12 : 0;
    }
    const uint32_t T = lo + base;
    r = need;
    // classify
    visit([&](uint32_t key, uint32_t t) {
      if (key > T) atomicOr(&sel_l[t >> 5], 1u << (t & 31));
      else if (key == T) atomicOr(&eq_l[t >> 5], 1u << (t & 31));
    });
    __syncthreads();
  }

  // ordered emission: all sel bits, and the first r eq bits in token order
  constexpr int kWordsPerThread = 16;  // words <= 8192
  const int per = (n_words + kSelThreads - 1) / kSelThreads;
  const int w0 = min(tid * per, n_words), w1 = min(w0 + per, n_words);
  uint32_t ev[kWordsPerThread], sv[kWordsPerThread];
  uint32_t eqc = 0;
#pragma unroll
  for (int j = 0; j < kWordsPerThread; ++j) {
    const bool ok = w0 + j < w1;
    ev[j] = ok ? eq_l[w0 + j] : 0u;
    sv[j] = ok ? sel_l[w0 + j] : 0u;
    eqc += __popc(ev[j]);
  }
  uint32_t dummy;
  uint32_t eq_before = block_exclusive_scan(eqc, scratch, &dummy);
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < kWordsPerThread; ++j) {
    const uint32_t pe = __popc(ev[j]);
    // quota left for this word, clamped to [0, pe] in signed arithmetic (an
    // unsigned "a >= b ? 0 : b - a" form has been folded into a wrapping subtract)
    const int left = (int)r - (int)eq_before;
    const uint32_t take = (uint32_t)min(max(left, 0), (int)pe);
    eq_before += pe;
    if (take) sv[j] |= lowest_bits(ev[j], take);
    cnt += __popc(sv[j]);
  }
  uint32_t total;
  uint32_t pos = block_exclusive_scan(cnt, scratch, &total);
  int32_t *out = a.indices + (int64_t)qi * k;
#pragma unroll
  for (int j = 0; j < kWordsPerThread; ++j) {
    uint32_t f = sv[j];
    while (f) {
      const int b = __ffs(f) - 1;
      if (pos < (uint32_t)k) out[pos] = (int32_t)((w0 + j) * 32 + b);
      ++pos;
      f &= f - 1;
    }
  }
  for (int p = (int)total + tid; p < k; p += kSelThreads) out[p] = -1;
  if (tid == 0 && a.counts) a.counts[qi] = (int32_t)(total < (uint32_t)k ? total : (uint32_t)k);
}

// Lower bound (top 16 bits) on the key of rank `need` among kSamples strided
// samples of the row; used when one workgroup owns a row and no group bounds
// were given.  Called by one whole wavefront.
__device__ uint32_t sample_bound_wave(const float *row, int n, uint32_t need) {
  const int lane = threadIdx.x & 63;
  uint32_t x[kSamples / 64];
#pragma unroll
  for (int i = 0; i < kSamples / 64; ++i) x[i] = order_key(row[(int)(((int64_t)(lane + 64 * i) * n) / kSamples)]);
  return wave_rank_bound(x, need, 16);
}

template <bool LOCAL>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  uint32_t *lh = lds;                                   // [4096] histogram
  uint32_t *scratch = lh + kHistBins;                   // [32]
  uint32_t *shv = scratch + 32;                         // [32] shared scalars
  uint32_t *sel_l = shv + 32;                           // [words]
  uint32_t *eq_l = sel_l + a.words;                     // [words]
  uint2 *cand_l = reinterpret_cast<uint2 *>(eq_l + a.words);  // [cand_cap]  (one workgroup per row only)

  const int qi = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.q_len[qi];
  const int k = a.k;
  const float *row = a.scores + (int64_t)qi * a.ld;

  // ---- 1. candidate bound (identical in every workgroup of the row)
  const bool bounded = n > k && n > a.cand_cap;
  uint32_t t_lo = 0;
  if (bounded) {
    if (a.bounds) {
      uint32_t m = 0xFFFFFFFFu;
      for (int g = lane; g < a.n_bounds; g += 64) m = min(m, a.bounds[(int64_t)qi * a.n_bounds + g]);
      t_lo = wave_min_u32(m);
      if (t_lo == 0xFFFFFFFFu) t_lo = 0;  // no full group: no bound
    } else if (wave == 0) {
      const uint64_t want = (uint64_t)5 * (uint64_t)k * kSamples / (2 * (uint64_t)n) + 4;
      const uint32_t t = sample_bound_wave(row, n, (uint32_t)(want < kSamples ? want : kSamples));
      if (lane == 0) shv[4] = t;
    }
  }

  // ---- 2. filter this workgroup's tokens into (key, token) candidates
  const int c0 = LOCAL ? 0 : blockIdx.x * a.chunk;
  const int c1 = LOCAL ? n : min(c0 + a.chunk, n);
  uint32_t found = 0;
  // first pass: count, to reserve room (multi-workgroup rows)
  uint32_t key[kPerThread];
  int g0 = c0;
  bool loaded = false;
  if (!LOCAL) {
    // a chunk is at most kPerThread * kSelThreads tokens: one pass
    float v[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int t = c0 + tid + kSelThreads * i;
      v[i] = t < c1 ? row[t] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) key[i] = order_key(v[i]);
    loaded = true;
  }
  if (bounded && !a.bounds) {
    __syncthreads();
    t_lo = shv[4];
  }
  uint2 *gdst = nullptr;
  if (!LOCAL) {
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) mine += (c0 + tid + kSelThreads * i < c1 && key[i] >= t_lo) ? 1u : 0u;
    uint32_t tot;
    uint32_t pos = block_exclusive_scan(mine, scratch, &tot);
    if (tid == 0) shv[5] = tot ? atomic_add_agent(&a.ctrl[qi * 4 + 1], tot) : 0u;
    __syncthreads();
    pos += shv[5];
    found = tot;
    gdst = a.cand + (int64_t)qi * a.cand_cap;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int t = c0 + tid + kSelThreads * i;
      if (t < c1 && key[i] >= t_lo) {
        if (pos < (uint32_t)a.cand_cap) {
          // device-coherent store (written through to the coherence point), read
          // by the row's last workgroup, which may sit on another XCD
          const uint64_t pk = ((uint64_t)(uint32_t)t << 32) | key[i];
          __hip_atomic_store(reinterpret_cast<uint64_t *>(gdst + pos), pk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        ++pos;
      }
    }
  } else {
    for (; g0 < c1; g0 += kPerThread * kSelThreads) {
      float v[kPerThread];
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        const int t = g0 + tid + kSelThreads * i;
        v[i] = t < c1 ? row[t] : 0.0f;
      }
      uint32_t mine = 0;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        key[i] = order_key(v[i]);
        mine += (g0 + tid + kSelThreads * i < c1 && key[i] >= t_lo) ? 1u : 0u;
      }
      uint32_t tot;
      uint32_t pos = found + block_exclusive_scan(mine, scratch, &tot);
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        const int t = g0 + tid + kSelThreads * i;
        if (t < c1 && key[i] >= t_lo) {
          if (pos < (uint32_t)a.cand_cap) cand_l[pos] = make_uint2(key[i], (uint32_t)t);
          ++pos;
        }
      }
      found += tot;
    }
  }
  (void)loaded;

  uint32_t total = found;
  if (!LOCAL) {
    // ---- handshake: the last workgroup of the row finishes it.  Every store
    // this workgroup made for the finisher is device-coherent and has completed
    // (waitcnt 0) before the counter increment, so no L2 write-back is needed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t prev = __hip_atomic_fetch_add(&a.ctrl[qi * 4], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = prev == (uint32_t)(a.chunks - 1);
      shv[9] = last ? 1u : 0u;
      if (last) {
        // drop stale copies of other workgroups' lines from this L1/L2 once
        // (agent-scope acquire), then read them with ordinary loads
        fence_acquire_agent();
        shv[10] = __hip_atomic_load(&a.ctrl[qi * 4 + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (shv[9] == 0) return;
    total = shv[10];
  } else {
    __syncthreads();
  }

  // ---- 3. this thread's candidates g = tid + 512 m, into registers
  const bool in_regs = n <= k || (total >= (uint32_t)k && total <= (uint32_t)a.cand_cap);
  uint32_t ck[kCandPerThread], ct[kCandPerThread];
  int nc = 0;
  if (in_regs && n > k) {
    nc = total > (uint32_t)tid ? (int)((total - 1 - tid) / kSelThreads) + 1 : 0;
    const uint2 *src = LOCAL ? cand_l : a.cand + (int64_t)qi * a.cand_cap;
    uint2 c[kCandPerThread];
#pragma unroll
    for (int m = 0; m < kCandPerThread; ++m)
      if (m < nc) c[m] = src[tid + kSelThreads * m];
#pragma unroll
    for (int m = 0; m < kCandPerThread; ++m)
      if (m < nc) {
        ck[m] = c[m].x;
        ct[m] = c[m].y;
      }
  }
  finish_row(a, qi, n, in_regs, ck, ct, nc, t_lo, row, lh, scratch, shv, sel_l, eq_l);
  if (!LOCAL && tid == 0) {
    a.ctrl[qi * 4] = 0;       // leave the counters zeroed for the next call
    a.ctrl[qi * 4 + 1] = 0;
  }
}

// Group bounds from a score row (when the scores did not come with them): for
// group g of kGroup tokens, a lower bound on its ceil(k / G)-th largest key
// (G = full groups of the row), or 0xFFFFFFFF when the group is not full.
__global__ __launch_bounds__(256) void bound_kernel(const float *__restrict__ scores, int64_t ld,
                                                    const int32_t *__restrict__ q_len, int k,
                                                    uint32_t *__restrict__ bounds) {
  __shared__ uint32_t keys[kGroup];
  const int qi = blockIdx.y, g = blockIdx.x;
  const int n = q_len[qi];
  const int gfull = n / kGroup;
  const int rank = gfull > 0 ? (k + gfull - 1) / gfull : 0;
  const bool full = (g + 1) * kGroup <= n && rank <= kGroup;
  if (full) {
    const float *row = scores + (int64_t)qi * ld + (int64_t)g * kGroup;
    float v[kGroup / 256];
#pragma unroll
    for (int i = 0; i < kGroup / 256; ++i) v[i] = row[threadIdx.x + 256 * i];
#pragma unroll
    for (int i = 0; i < kGroup / 256; ++i) keys[threadIdx.x + 256 * i] = order_key(v[i]);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    uint32_t x[kGroup / 64];
#pragma unroll
    for (int i = 0; i < kGroup / 64; ++i) x[i] = full ? keys[threadIdx.x + 64 * i] : 0u;
    const uint32_t T = full ? wave_rank_bound(x, (uint32_t)rank, 16) : 0xFFFFFFFFu;
    if (threadIdx.x == 0) bounds[(int64_t)qi * gridDim.x + g] = T;
  }
}

}  // namespace

TopkPlan plan_topk(int n_q, int k, int max_len) {
  TopkPlan p{};
  p.n_q = n_q;
  p.k = k;
  p.max_len = max_len;
  // Many rows, or short rows: one workgroup per row.  Few long rows: spread each
  // row over several workgroups (about 256 in all) so the whole chip takes part.
  int chunks = 1;
  if (n_q < 128 && max_len > 8192) {
    chunks = 256 / (n_q > 0 ? n_q : 1);
    const int fewest = (max_len + kPerThread * kSelThreads - 1) / (kPerThread * kSelThreads);
    const int most = (max_len + 1023) / 1024;
    if (chunks > most) chunks = most;
    if (chunks < fewest) chunks = fewest;   // a chunk is one pass of kPerThread per thread
    if (chunks < 2) chunks = 2;
  }
  int chunk = (max_len + chunks - 1) / chunks;
  chunk = (chunk + 63) / 64 * 64;
  chunks = (max_len + chunk - 1) / chunk;
  p.chunks = chunks;
  p.chunk = chunk;
  p.group = kGroup;
  p.groups = (max_len + kGroup - 1) / kGroup;
  p.words = ((max_len + 31) / 32 + 3) / 4 * 4;
  // LDS: 4096-word histogram + 64 words, two bitmaps, and (one workgroup per
  // row) the candidate list, which takes what is left of 160 KiB.
  const size_t fixed = (size_t)(kHistBins + 64) * 4 + (size_t)2 * p.words * 4;
  size_t cap = (size_t)kCandPerThread * kSelThreads;  // 12288: the register budget
  if (chunks == 1) {
    const size_t room = fixed < 160 * 1024 ? (160 * 1024 - fixed) / 8 : 0;
    if (room < cap) cap = room / kSelThreads * kSelThreads;
  }
  p.cand_cap = (int)cap;
  p.lds_bytes = fixed + (chunks == 1 ? cap * 8 : 0);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  if (chunks > 1) {
    p.off_ctrl = take((size_t)n_q * 16);
    p.off_bounds = take((size_t)n_q * p.groups * 4);
    p.off_cand = take((size_t)n_q * cap * 8);
  }
  p.total = off;
  return p;
}

hipError_t launch_topk(int32_t *indices, int32_t *counts, const float *scores, int64_t ld, const int32_t *q_len,
                       const TopkPlan &plan, void *workspace, const uint32_t *bounds, int n_bounds,
                       hipStream_t stream) {
  // The select kernel uses up to 160 KiB of dynamic LDS.
  static const bool lds_ok = [] {
    const int most = 160 * 1024;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel<true>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, most) == hipSuccess &&
           hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel<false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, most) == hipSuccess;
  }();
  if (!lds_ok) return hipErrorInvalidConfiguration;
  if (plan.lds_bytes > 160 * 1024 || plan.cand_cap < kSamples) return hipErrorInvalidValue;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  SelectArgs a{};
  a.indices = indices;
  a.counts = counts;
  a.scores = scores;
  a.ld = ld;
  a.q_len = q_len;
  a.k = plan.k;
  a.chunk = plan.chunk;
  a.chunks = plan.chunks;
  a.words = plan.words;
  a.cand_cap = plan.cand_cap;
  a.bounds = bounds;
  a.n_bounds = n_bounds;
  if (plan.chunks > 1) {
    a.ctrl = reinterpret_cast<uint32_t *>(ws + plan.off_ctrl);
    a.cand = reinterpret_cast<uint2 *>(ws + plan.off_cand);
    if (!bounds) {
      uint32_t *b = reinterpret_cast<uint32_t *>(ws + plan.off_bounds);
      hipLaunchKernelGGL(bound_kernel, dim3(plan.groups, plan.n_q), dim3(256), 0, stream, scores, ld, q_len, plan.k,
                         b);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      a.bounds = b;
      a.n_bounds = plan.groups;
    }
    hipLaunchKernelGGL(select_kernel<false>, dim3(plan.chunks, plan.n_q), dim3(kSelThreads), plan.lds_bytes, stream,
                       a);
  } else {
    hipLaunchKernelGGL(select_kernel<true>, dim3(1, plan.n_q), dim3(kSelThreads), plan.lds_bytes, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
