// Exact top-k selection.
//
// Keeps the first min(k, n) entries of a stable descending sort of a score row:
// the best k, everything when n <= k, ties to the lower token index ("GLM on an
// A100, in Vx", sections "The model" and "How do we know it is right?").
//
// Method (integer only, on order_key(score), so exact and deterministic):
//  1. first radix level: a 4096-bin histogram of key >> 20, either global (built
//     by the score kernel or by hist_kernel, many workgroups per row) or built
//     in LDS by the one workgroup that owns the row;
//  2. threshold bin b*: the highest bin whose suffix count reaches k.  Every
//     key in a higher bin is kept (a "sel" bit in a per-row bitmap); keys in
//     b* are candidates, appended to a list;
//  3. the last workgroup of a row (atomic counter) finishes: two more radix
//     levels over the candidates (bits 19..8, then 7..0) give the exact
//     threshold key T and the tie quota r = (k - #keys > T); candidates above T
//     get sel bits, candidates equal to T get "eq" bits;
//  4. ordered emission: one pass over the bitmap words in token order keeps all
//     sel bits and the first r eq bits (a block-wide prefix count of eq bits
//     gives the quota per word), and writes the kept token indices ascending.
// If more candidates arrive than fit, the finisher runs the same two levels
// over the whole row in memory instead (exact, slower).
//
// The finisher leaves the global histogram and counters zeroed for the next call.
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int kSelThreads = 512;
constexpr int kModeAll = 0, kModeBinAll = 1, kModeRefine = 2;

__device__ __forceinline__ uint32_t lane_prefix_count(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t lowest_bits(uint32_t e, uint32_t take) {
  uint32_t r = 0;
  for (uint32_t i = 0; i < take; ++i) {
    const uint32_t lb = e & (~e + 1u);
    r |= lb;
    e ^= lb;
  }
  return r;
}

// Among h[0..nbins), find the highest bin b whose suffix count (bins >= b)
// reaches `need` (need >= 1 and <= total).  Writes b to out[0] and the count of
// bins > b to out[1].  scratch: >= 18 words.  All threads must call it.
__device__ void find_from_top(const uint32_t *h, int nbins, uint32_t need, uint32_t *scratch, uint32_t *out) {
  const int per = nbins >= kSelThreads ? nbins / kSelThreads : 1;
  const int t = threadIdx.x;
  const bool owns = t * per < nbins;
  // thread t owns bins [hi - per, hi) counted from the top
  const int hi = nbins - t * per;
  uint32_t local = 0;
  if (owns)
    for (int j = 0; j < per; ++j) local += h[hi - 1 - j];
  uint32_t tot;
  uint32_t before = block_exclusive_scan(local, scratch, &tot);
  if (owns && before < need && before + local >= need) {
    uint32_t run = before;
    for (int j = 0; j < per; ++j) {
      const int b = hi - 1 - j;
      if (run + h[b] >= need) {
        out[0] = (uint32_t)b;
        out[1] = run;
        break;
      }
      run += h[b];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void hist_kernel(const float *__restrict__ scores, int64_t ld,
                                                   const int32_t *__restrict__ q_len, int chunk,
                                                   uint32_t *__restrict__ hist) {
  __shared__ uint32_t lh[kHistBins];
  const int qi = blockIdx.y;
  const int n = q_len[qi];
  for (int i = threadIdx.x; i < kHistBins; i += 256) lh[i] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * chunk;
  const int c1 = min(c0 + chunk, n);
  const float *row = scores + (int64_t)qi * ld;
  for (int t = c0 + threadIdx.x; t < c1; t += 256) atomicAdd(&lh[order_key(row[t]) >> kHistShift], 1u);
  __syncthreads();
  uint32_t *gh = hist + (int64_t)qi * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t c = lh[i];
    if (c) atomic_add_agent(gh + i, c);
  }
}

struct SelectArgs {
  int32_t *indices;
  int32_t *counts;
  const float *scores;
  int64_t ld;
  const int32_t *q_len;
  int k;
  int chunk;
  int chunks;
  int words;       // allocated bitmap words per row
  int cand_cap;
  uint32_t *hist;  // [n_q][4096]      (multi-workgroup rows)
  uint32_t *ctrl;  // [n_q][4]         done, n_cand
  uint2 *cand;     // [n_q][cand_cap]  (key, token)
  uint32_t *sel;   // [n_q][words]
};

// LOCAL: one workgroup owns each row (no global state at all).
template <bool LOCAL>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  uint32_t *lh = lds;                                   // [4096]
  uint32_t *scratch = lh + kHistBins;                   // [32]
  uint32_t *shv = scratch + 32;                         // [32] shared scalars
  uint2 *cand_l = reinterpret_cast<uint2 *>(shv + 32);  // [cand_cap]
  uint32_t *sel_l = reinterpret_cast<uint32_t *>(cand_l + a.cand_cap);  // [words]
  uint32_t *eq_l = sel_l + a.words;                     // [words]

  const int qi = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kSelThreads / 64;
  const int n = a.q_len[qi];
  const int k = a.k;
  const float *row = a.scores + (int64_t)qi * a.ld;

  if (tid < 32) shv[tid] = 0;
  // ---- 1. first radix level
  if (LOCAL) {
    for (int i = tid; i < kHistBins; i += kSelThreads) lh[i] = 0;
    __syncthreads();  // shv[8] is the local candidate counter
    for (int t = tid; t < n; t += kSelThreads) atomicAdd(&lh[order_key(row[t]) >> kHistShift], 1u);
  } else {
    const uint32_t *gh = a.hist + (int64_t)qi * kHistBins;
    for (int i = tid; i < kHistBins; i += kSelThreads) lh[i] = gh[i];
  }
  __syncthreads();

  // ---- 2. threshold bin
  int mode;
  uint32_t bstar = 0, above = 0;
  if (n <= k) {
    mode = kModeAll;
  } else {
    find_from_top(lh, kHistBins, (uint32_t)k, scratch, shv);
    bstar = shv[0] & (kHistBins - 1);
    above = shv[1];
    mode = (k - above == lh[bstar]) ? kModeBinAll : kModeRefine;
  }

  // ---- 3. scan this workgroup's tokens: sel bits and candidates
  const int c0 = LOCAL ? 0 : blockIdx.x * a.chunk;
  const int c1 = LOCAL ? n : min(c0 + a.chunk, n);
  uint32_t *sel_dst = LOCAL ? sel_l : a.sel + (int64_t)qi * a.words;
  uint2 *cand_dst = LOCAL ? cand_l : a.cand + (int64_t)qi * a.cand_cap;
  uint32_t *cand_ctr = LOCAL ? &shv[8] : &a.ctrl[qi * 4 + 1];
  for (int g0 = c0; g0 < c1; g0 += 64 * kWaves) {
    const int gw = g0 + wave * 64;
    const int t = gw + lane;
    const bool in = t < c1;
    const uint32_t key = in ? order_key(row[t]) : 0u;
    const uint32_t bin = key >> kHistShift;
    const bool s = in && (mode == kModeAll || bin > bstar || (mode == kModeBinAll && bin == bstar));
    const bool c = in && mode == kModeRefine && bin == bstar;
    const uint64_t sm = __ballot(s);
    if (gw < c1 && lane == 0) {
      sel_dst[gw >> 5] = (uint32_t)sm;
      sel_dst[(gw >> 5) + 1] = (uint32_t)(sm >> 32);
    }
    const uint64_t cm = __ballot(c);
    if (cm) {
      uint32_t base = 0;
      if (lane == 0) base = LOCAL ? atomicAdd(cand_ctr, (uint32_t)__popcll(cm)) : atomic_add_agent(cand_ctr, (uint32_t)__popcll(cm));
      base = __shfl(base, 0, 64);
      const uint32_t pos = base + lane_prefix_count(cm);
      if (c && pos < (uint32_t)a.cand_cap) cand_dst[pos] = make_uint2(key, (uint32_t)t);
    }
  }

  // ---- handshake: the last workgroup of the row finishes it
  if (!LOCAL) {
    fence_release_agent();
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&a.ctrl[qi * 4 + 0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      shv[9] = (prev == (uint32_t)(a.chunks - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (shv[9] == 0) return;
    fence_acquire_agent();
  } else {
    __syncthreads();
  }

  // ---- 4. finish the row
  const int n_words = (n + 31) >> 5;
  uint32_t ncand;
  if (LOCAL) {
    ncand = shv[8];
  } else {
    ncand = __hip_atomic_load(&a.ctrl[qi * 4 + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t *gs = a.sel + (int64_t)qi * a.words;
    for (int w = tid; w < n_words; w += kSelThreads) sel_l[w] = gs[w];
    if (mode == kModeRefine && ncand <= (uint32_t)a.cand_cap) {
      const uint2 *gc = a.cand + (int64_t)qi * a.cand_cap;
      for (uint32_t i = tid; i < ncand; i += kSelThreads) cand_l[i] = gc[i];
    }
  }
  for (int w = tid; w < n_words; w += kSelThreads) eq_l[w] = 0;
  __syncthreads();

  uint32_t r = 0;
  if (mode == kModeRefine) {
    const uint32_t need = (uint32_t)k - above;
    const bool overflow = ncand > (uint32_t)a.cand_cap;
    // level 2: bits 19..8 within bin b*
    for (int i = tid; i < kHistBins; i += kSelThreads) lh[i] = 0;
    __syncthreads();
    if (!overflow) {
      for (uint32_t i = tid; i < ncand; i += kSelThreads) atomicAdd(&lh[(cand_l[i].x >> 8) & 0xFFFu], 1u);
    } else {
      for (int t = tid; t < n; t += kSelThreads) {
        const uint32_t key = order_key(row[t]);
        if ((key >> kHistShift) == bstar) atomicAdd(&lh[(key >> 8) & 0xFFFu], 1u);
      }
    }
    __syncthreads();
    find_from_top(lh, kHistBins, need, scratch, shv);
    const uint32_t b2 = shv[0] & 0xFFFu;
    const uint32_t need2 = need - shv[1];
    const uint32_t prefix = (bstar << 12) | b2;  // key >> 8 of the survivors
    __syncthreads();
    // level 3: bits 7..0
    for (int i = tid; i < 256; i += kSelThreads) lh[i] = 0;
    __syncthreads();
    if (!overflow) {
      for (uint32_t i = tid; i < ncand; i += kSelThreads) {
        const uint32_t key = cand_l[i].x;
        if ((key >> 8) == prefix) atomicAdd(&lh[key & 0xFFu], 1u);
      }
    } else {
      for (int t = tid; t < n; t += kSelThreads) {
        const uint32_t key = order_key(row[t]);
        if ((key >> 8) == prefix) atomicAdd(&lh[key & 0xFFu], 1u);
      }
    }
    __syncthreads();
    find_from_top(lh, 256, need2, scratch, shv);
    const uint32_t T = (prefix << 8) | (shv[0] & 0xFFu);
    r = need2 - shv[1];
    __syncthreads();
    // classify the threshold bin
    if (!overflow) {
      for (uint32_t i = tid; i < ncand; i += kSelThreads) {
        const uint2 ce = cand_l[i];
        if (ce.x > T) atomicOr(&sel_l[ce.y >> 5], 1u << (ce.y & 31));
        else if (ce.x == T) atomicOr(&eq_l[ce.y >> 5], 1u << (ce.y & 31));
      }
    } else {
      for (int t = tid; t < n; t += kSelThreads) {
        const uint32_t key = order_key(row[t]);
        if ((key >> kHistShift) != bstar) continue;
        if (key > T) atomicOr(&sel_l[t >> 5], 1u << (t & 31));
        else if (key == T) atomicOr(&eq_l[t >> 5], 1u << (t & 31));
      }
    }
    __syncthreads();
  }

  // ---- 5. ordered emission: all sel bits, and the first r eq bits in token order
  const int per = (n_words + kSelThreads - 1) / kSelThreads;
  const int w0 = min(tid * per, n_words), w1 = min(w0 + per, n_words);
  uint32_t eqc = 0;
  for (int w = w0; w < w1; ++w) eqc += __popc(eq_l[w]);
  uint32_t dummy;
  uint32_t eq_before = block_exclusive_scan(eqc, scratch, &dummy);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) {
    const uint32_t e = eq_l[w];
    const uint32_t pe = __popc(e);
    const uint32_t take = eq_before >= r ? 0u : min(r - eq_before, pe);
    eq_before += pe;
    const uint32_t f = sel_l[w] | lowest_bits(e, take);
    sel_l[w] = f;
    cnt += __popc(f);
  }
  uint32_t total;
  uint32_t pos = block_exclusive_scan(cnt, scratch, &total);
  int32_t *out = a.indices + (int64_t)qi * k;
  for (int w = w0; w < w1; ++w) {
    uint32_t f = sel_l[w];
    while (f) {
      const int b = __ffs(f) - 1;
      if (pos < (uint32_t)k) out[pos] = (int32_t)(w * 32 + b);
      ++pos;
      f &= f - 1;
    }
  }
  for (int p = (int)total + tid; p < k; p += kSelThreads) out[p] = -1;
  if (tid == 0 && a.counts) a.counts[qi] = (int32_t)(total < (uint32_t)k ? total : (uint32_t)k);

  // ---- 6. leave the global state zeroed for the next call
  if (!LOCAL) {
    uint32_t *gh = a.hist + (int64_t)qi * kHistBins;
    for (int i = tid; i < kHistBins; i += kSelThreads) gh[i] = 0;
    if (tid == 0) {
      a.ctrl[qi * 4 + 0] = 0;
      a.ctrl[qi * 4 + 1] = 0;
    }
  }
}

}  // namespace

TopkPlan plan_topk(int n_q, int k, int max_len) {
  TopkPlan p{};
  p.n_q = n_q;
  p.k = k;
  p.max_len = max_len;
  // Many rows, or short rows: one workgroup per row.  Few long rows: spread each
  // row over several workgroups so the whole chip takes part.
  int chunks = 1;
  if (n_q < 128 && max_len > 4096) {
    chunks = 256 / (n_q > 0 ? n_q : 1);
    const int most = (max_len + 1023) / 1024;
    if (chunks > most) chunks = most;
    if (chunks < 1) chunks = 1;
  }
  int chunk = (max_len + chunks - 1) / chunks;
  chunk = (chunk + 63) / 64 * 64;
  chunks = (max_len + chunk - 1) / chunk;
  p.chunks = chunks;
  p.chunk = chunk;
  p.words = ((max_len + 31) / 32 + 1) / 2 * 2;
  const int lim = (max_len + 63) / 64 * 64;
  p.cand_cap = lim < 8192 ? lim : 8192;
  p.lds_bytes = (size_t)(kHistBins + 64) * 4 + (size_t)p.cand_cap * 8 + (size_t)2 * p.words * 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  if (chunks > 1) {
    p.off_hist = take((size_t)n_q * kHistBins * 4);
    p.off_ctrl = take((size_t)n_q * 16);
    p.off_cand = take((size_t)n_q * p.cand_cap * 8);
    p.off_sel = take((size_t)n_q * p.words * 4);
  }
  p.total = off;
  return p;
}

hipError_t launch_topk(int32_t *indices, int32_t *counts, const float *scores, int64_t ld, const int32_t *q_len,
                       const TopkPlan &plan, void *workspace, bool hist_ready, hipStream_t stream) {
  // The select kernel may use more than 64 KiB of dynamic LDS (up to 144 KiB).
  static const bool lds_ok = [] {
    const int most = 160 * 1024;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel<true>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, most) == hipSuccess &&
           hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel<false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, most) == hipSuccess;
  }();
  if (!lds_ok) return hipErrorInvalidConfiguration;
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
  if (plan.chunks > 1) {
    a.hist = reinterpret_cast<uint32_t *>(ws + plan.off_hist);
    a.ctrl = reinterpret_cast<uint32_t *>(ws + plan.off_ctrl);
    a.cand = reinterpret_cast<uint2 *>(ws + plan.off_cand);
    a.sel = reinterpret_cast<uint32_t *>(ws + plan.off_sel);
    if (!hist_ready) {
      hipLaunchKernelGGL(hist_kernel, dim3(plan.chunks, plan.n_q), dim3(256), 0, stream, scores, ld, q_len,
                         plan.chunk, a.hist);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(select_kernel<false>, dim3(plan.chunks, plan.n_q), dim3(kSelThreads), plan.lds_bytes, stream,
                       a);
  } else {
    hipLaunchKernelGGL(select_kernel<true>, dim3(1, plan.n_q), dim3(kSelThreads), plan.lds_bytes, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
