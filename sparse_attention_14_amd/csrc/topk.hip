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
//     as it writes the scores; otherwise bound_kernel does, or one wavefront
//     estimates it from samples spread over the row).  With group bounds at
//     least k keys of the row are >= T_lo = their minimum; a sampled estimate
//     may miss, which only sends the row to the exact fallback below.  Rows
//     that fit the candidate budget use T_lo = 0.
//  2. Filter.  Workgroups scan the row in rounds of one score per thread and
//     compact the (key, token) pairs with key >= T_lo in token order (wavefront
//     ballots plus one prefix over the round totals).  For few long rows a
//     filter kernel spreads each row over many workgroups, each writing its
//     candidates and their count to a region of its own, and a finishing kernel
//     takes over; otherwise one workgroup per row does both in LDS.
//  3. Threshold.  Candidate j of the row (in token order) sits in thread
//     j % NT, register slot j / NT.  12-bit radix levels over the window
//     [T_lo, max key] give the exact k-th key T and the tie quota
//     r = k - #(key > T).
//  4. Ordered emission.  Keys > T, and the first r keys == T in token order,
//     are kept; one prefix over (#>T, #==T) in candidate order gives every kept
//     token its output slot.
// Rows whose candidates do not fit (or a sampled bound that keeps fewer than k)
// run steps 3-4 over the whole row in memory instead: exact, slower.
//
// The per-element code is branch-free (select instead of divergent branches,
// a dump bin for histogram entries that do not count): with few wavefronts per
// SIMD, divergent control flow per element costs far more than the arithmetic.
#include <atomic>

#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int kRegCap = 12288;                  // candidates per row held in registers
constexpr int kBins = kHistBins;                // 4096 (12-bit digits)
constexpr int kCoarse = kBins + 64;             // 64 super-bins of 64 bins each (summed from the bins);
                                                // before them, per-lane dump slots for elements that
                                                // do not count
constexpr int kHistWords = kCoarse + 128;
constexpr int kGroup = 1024;                    // tokens per bound group (bound_kernel)
constexpr int kSamples = 1024;
constexpr int kMaxChunks = 256;
constexpr int kFilterThreads = 512;
constexpr int kPassRounds = 8;                  // filter rounds per pass
constexpr int kPass = kFilterThreads * kPassRounds;   // 4096 scores per pass
constexpr int kFinishThreads = 1024;            // finishing kernel of a spread row
constexpr int kLocalThreads = 512;              // one workgroup per row
constexpr int kLocalCap = 14 * kLocalThreads;   // LDS candidates of a one-workgroup row (7168)

// LDS carve-up (32-bit words), the same for every kernel.
constexpr int kTotWords = 200;                  // >= rounds * waves + 1 for every use (192 + 1)
constexpr int kOffHist = 0;
constexpr int kOffScratch = kOffHist + kHistWords;
constexpr int kOffShv = kOffScratch + 64;
constexpr int kOffTot = kOffShv + 64;
constexpr int kOffCpre = kOffTot + 2 * kTotWords;
constexpr int kOffCmap = kOffCpre + kMaxChunks + 4;
constexpr int kOffCand = (kOffCmap + kRegCap / 64 + 4 + 3) / 4 * 4;   // uint2 array, 16-byte aligned
constexpr int kFixedWords = kOffCand;

struct Lds {
  uint32_t *hist, *scratch, *shv, *tot0, *tot1, *cpre, *cmap;
  uint2 *cand;
};

__device__ __forceinline__ Lds carve(uint32_t *lds) {
  Lds L;
  L.hist = lds + kOffHist;
  L.scratch = lds + kOffScratch;
  L.shv = lds + kOffShv;
  L.tot0 = lds + kOffTot;
  L.tot1 = lds + kOffTot + kTotWords;
  L.cpre = lds + kOffCpre;
  L.cmap = lds + kOffCmap;
  L.cand = reinterpret_cast<uint2 *>(lds + kOffCand);
  return L;
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
  int chunk;        // tokens per filter workgroup (<= kPass, multiple of 64)
  int chunks;       // filter workgroups per row
  int local_cap;    // LDS candidate capacity (one workgroup per row)
  int group_tokens; // tokens per bound group
  int bound_most;   // largest rank a bound group can report
  int max_len;      // allocated row length bound: every row holds at least this many scores
  uint32_t *ccount; // [n_q][chunks] candidates per chunk
  uint32_t *cmax;   // [n_q][chunks] largest candidate key per chunk
  uint32_t *tlo;    // [n_q] the row's candidate bound
  uint2 *cand;      // [n_q][chunks][chunk] (key, token) per chunk
};

// Fetches every argument in one round trip: the returned zero depends on all of
// them, so code indexed by it (the row, the chunk) waits for one batch of
// argument loads instead of one dependent scalar round trip per argument at
// its first use.
__device__ __forceinline__ int args_together(const SelectArgs &a) {
  int zero;
  asm("s_mov_b32 %0, 0"
      : "=s"(zero)
      : "s"(a.indices), "s"(a.counts), "s"(a.scores), "s"(a.ld), "s"(a.q_len), "s"(a.bounds), "s"(a.n_bounds),
        "s"(a.k), "s"(a.chunk), "s"(a.chunks), "s"(a.local_cap), "s"(a.group_tokens), "s"(a.bound_most),
        "s"(a.ccount), "s"(a.cmax), "s"(a.tlo), "s"(a.cand), "s"(a.max_len));
  return zero;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Waits for every outstanding memory operation of the wavefront: taken before
// an early return past loads issued ahead of the row-length check, so no load
// is still in flight when the wavefront ends.
__device__ __forceinline__ void drain_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Order-preserving prefix over `rounds` (uniform, <= R) rounds of one element per
// thread: element (m, tid) precedes (m', tid') when m < m' or (m == m' and
// tid < tid').  flag(m) returns 1 (counted in the low half), 1 << 16 (high half)
// or 0.  pre[m] receives the packed count of earlier elements (both halves); the
// packed total is returned.  Each half must stay below 65536.  tot: LDS of
// R * waves + 1 words, not written again before one more barrier.  Two barriers.
template <int NT, int R, typename F>
__device__ __forceinline__ uint32_t ordered_prefix(F &&flag, int rounds, uint32_t (&pre)[R], uint32_t *tot) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t totv = 0;   // lane m: packed total of round m in this wavefront
#pragma unroll
  for (int m = 0; m < R; ++m) {
    if (m < rounds) {
      const uint32_t v = flag(m);
      const uint64_t lo = __ballot((v & 0xFFFFu) != 0u);
      const uint64_t hi = __ballot((v >> 16) != 0u);
      pre[m] = lanes_below(lo) | (lanes_below(hi) << 16);
      const uint32_t t = (uint32_t)__popcll(lo) | ((uint32_t)__popcll(hi) << 16);
      totv = lane == m ? t : totv;
    }
  }
  if (lane < rounds) tot[lane * W + wave] = totv;
  __syncthreads();
  if (wave == 0) {
    const int E = rounds * W;
    constexpr int PL = (R * W + 63) / 64;
    uint32_t v[PL];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane * PL + i;
      v[i] = e < E ? tot[e] : 0u;
      s += v[i];
    }
    const uint32_t incl = wave_inclusive_scan(s);
    uint32_t run = incl - s;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane * PL + i;
      if (e < E) tot[e] = run;
      run += v[i];
    }
    if (lane == 63) tot[R * W] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < R; ++m)
    if (m < rounds) pre[m] += tot[m * W + wave];
  return tot[R * W];
}

template <int NT>
__device__ __forceinline__ void zero_hist(uint32_t *h) {
  uint4 *h4 = reinterpret_cast<uint4 *>(h);
#pragma unroll
  for (int i = 0; i < kBins / 4 / NT; ++i) h4[threadIdx.x + NT * i] = make_uint4(0, 0, 0, 0);
}

// Super-bin counts (64 bins each) summed from the finished fine histogram:
// thread t adds bins [t B, t B + B) (B = kBins / NT) and the B-bin partial sums
// of the 64 / B threads of one super-bin are added across their lanes.  Exact
// and order-independent; it replaces one LDS atomic per key on the 64 super-bin
// counters, which the keys just above the candidate bound all hit.  Called by
// every thread after the fine pass and a barrier; a barrier must follow.
template <int NT>
__device__ __forceinline__ void coarse_from_fine(uint32_t *h) {
  constexpr int B = kBins / NT;     // bins per thread (4 or 8)
  constexpr int TPS = 64 / B;       // threads per super-bin (16 or 8), aligned lane groups
  static_assert(B % 4 == 0 && TPS >= 1 && 64 % TPS == 0, "fine bins per thread");
  const uint4 *h4 = reinterpret_cast<const uint4 *>(h) + threadIdx.x * (B / 4);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < B / 4; ++i) {
    const uint4 v = h4[i];
    s += (v.x + v.y) + (v.z + v.w);
  }
#pragma unroll
  for (int off = 1; off < TPS; off <<= 1) s += (uint32_t)__shfl_xor((int)s, off, 64);
  if ((threadIdx.x & (TPS - 1)) == 0) h[kCoarse + threadIdx.x / TPS] = s;
}

// Highest bin b whose count of keys in bins >= b reaches `need` (1 <= need <=
// total): the first wavefront scans the 64 super-bins from the top, then the 64
// bins of the super-bin found.  Writes shv[0] = b, shv[1] = count in bins > b;
// the caller synchronises before reading them.
__device__ __forceinline__ void find_from_top(const uint32_t *h, uint32_t need, uint32_t *shv) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const uint32_t c = h[kCoarse + 63 - lane];   // lane 0: the highest super-bin
  const uint32_t ci = wave_inclusive_scan(c);
  const int l1 = __ffsll((unsigned long long)__ballot(ci >= need)) - 1;
  const uint32_t sb = 63u - (uint32_t)l1;
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(ci - c), l1);
  const uint32_t f = h[sb * 64 + 63 - lane];
  const uint32_t fi = wave_inclusive_scan(f) + above;
  const int l2 = __ffsll((unsigned long long)__ballot(fi >= need)) - 1;
  const uint32_t above2 = (uint32_t)__builtin_amdgcn_readlane((int)(fi - f), l2);
  if (lane == 0) {
    shv[0] = sb * 64 + 63u - (uint32_t)l2;
    shv[1] = above2;
  }
}

template <int NT>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t *scratch) {
  const uint32_t m = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r = max(r, scratch[i]);
  __syncthreads();
  return r;
}

// Exact k-th largest key T and tie quota r = k - #(key > T) among the keys that
// hist_pass(off_lo, himask, base, sh, mask) adds to L.hist (every thread its own
// share: bin ((key - lo) >> sh) & mask of the keys whose (key - lo) agrees with
// base on the bits in himask, the dump bin for the rest), all keys in [lo, mx],
// at least k of them.  Radix levels of 12 bits from the top of the window.
template <int NT, typename H>
__device__ void radix_threshold(H &&hist_pass, uint32_t lo, uint32_t mx, uint32_t k, const Lds &L, uint32_t &T,
                                uint32_t &r) {
  const uint32_t range = mx - lo;
  const int width = range ? 32 - __clz(range) : 0;   // bits of (key - lo)
  // each level histograms bits [sh, prev) of (key - lo) among the keys whose
  // bits >= prev equal the prefix chosen so far
  int prev = 32;
  int sh = width > 12 ? width - 12 : 0;
  uint32_t base = 0;
  uint32_t need = k;
  while (true) {
    zero_hist<NT>(L.hist);
    __syncthreads();
    const uint32_t mask = prev - sh >= 12 ? 0xFFFu : ((1u << (prev - sh)) - 1u);
    const uint32_t himask = prev >= 32 ? 0u : (0xFFFFFFFFu << prev);
    hist_pass(himask, base, sh, mask);
    __syncthreads();
    coarse_from_fine<NT>(L.hist);
    __syncthreads();
    find_from_top(L.hist, need, L.shv);
    __syncthreads();
    base |= L.shv[0] << sh;
    need -= L.shv[1];
    if (sh == 0) break;
    prev = sh;
    sh = sh > 12 ? sh - 12 : 0;
  }
  T = lo + base;
  r = need;
}

// Histogram increment of one key (branch-free): its bin, or this lane's dump
// slot when it does not count.
__device__ __forceinline__ void hist_add(uint32_t *h, bool valid, uint32_t key, uint32_t lo, uint32_t himask,
                                         uint32_t base, int sh, uint32_t mask) {
  const uint32_t off = key - lo;
  const bool in = valid && ((off ^ base) & himask) == 0u;
  const uint32_t bin = (off >> sh) & mask;
  const uint32_t lane = threadIdx.x & 63;
  atomicAdd(&h[in ? bin : kBins + lane], 1u);
}

// Rows with n <= k keep every token.
template <int NT>
__device__ void emit_all(const SelectArgs &a, int qi, int n) {
  int32_t *out = a.indices + (int64_t)qi * a.k;
  for (int p = threadIdx.x; p < a.k; p += NT) out[p] = p < n ? p : -1;
  if (threadIdx.x == 0 && a.counts) a.counts[qi] = n;
}

// Steps 3-4 on candidates held in registers: candidate j < C (token order) is
// ck/ct[j / NT] of thread j % NT; all keys in [lo, mx], C >= k, and every key
// of the row that ranks in the top k is among them.
template <int NT, int R>
__device__ void finish_regs(const SelectArgs &a, int qi, uint32_t C, uint32_t lo, uint32_t mx,
                            const uint32_t (&ck)[R], const uint32_t (&ct)[R], const Lds &L) {
  const int tid = threadIdx.x;
  const int rounds = (int)((C + NT - 1) / NT);
  uint32_t T, r;
  radix_threshold<NT>(
      [&](uint32_t himask, uint32_t base, int sh, uint32_t mask) {
#pragma unroll
        for (int m = 0; m < R; ++m)
          if (m < rounds)
            hist_add(L.hist, (uint32_t)(tid + NT * m) < C, ck[m], lo, himask, base, sh, mask);
      },
      lo, mx, (uint32_t)a.k, L, T, r);
  uint32_t pre[R];
  ordered_prefix<NT, R>(
      [&](int m) -> uint32_t {
        const bool valid = (uint32_t)(tid + NT * m) < C;
        return valid ? (ck[m] > T ? 1u : (ck[m] == T ? 0x10000u : 0u)) : 0u;
      },
      rounds, pre, L.tot0);
  int32_t *out = a.indices + (int64_t)qi * a.k;
#pragma unroll
  for (int m = 0; m < R; ++m) {
    if (m < rounds) {
      const bool valid = (uint32_t)(tid + NT * m) < C;
      const uint32_t sb = pre[m] & 0xFFFFu, eb = pre[m] >> 16;
      const bool gt = valid && ck[m] > T;
      const bool eq = valid && ck[m] == T && eb < r;
      const uint32_t pos = sb + (gt ? min(eb, r) : eb);
      if (gt || eq) out[pos] = (int32_t)ct[m];
    }
  }
  if (tid == 0 && a.counts) a.counts[qi] = a.k;
}

// Loads the rounds of scores of the pass at g0: token g0 + tid + NT i, clamped
// below `end` (<= the row's allocated length: a row holds at least max_len
// scores), so every load is unconditional and none waits for the row's
// visible count; scores past the visible count are masked by the caller.
template <int NT, int RP>
__device__ __forceinline__ void load_pass_clamped(const float *row, int g0, int end, float (&v)[RP]) {
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    const int t = g0 + (int)threadIdx.x + NT * i;
    v[i] = row[t < end ? t : end - 1];
  }
}

// Loads the rounds of scores of the pass at g0: token g0 + tid + NT i (< n).
template <int NT, int RP>
__device__ __forceinline__ void load_pass(const float *row, int g0, int n, float (&v)[RP]) {
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    const int t = g0 + (int)threadIdx.x + NT * i;
    v[i] = t < n ? row[t] : 0.0f;
  }
}

// Steps 3-4 over the whole row read from memory (n > k).
template <int NT>
__device__ void finish_row(const SelectArgs &a, int qi, int n, const float *row, const Lds &L) {
  constexpr int RP = kPass / NT;
  const int tid = threadIdx.x;
  uint32_t mx = 0;
  for (int g0 = 0; g0 < n; g0 += kPass) {
    float v[RP];
    load_pass<NT, RP>(row, g0, n, v);
#pragma unroll
    for (int i = 0; i < RP; ++i) mx = max(mx, g0 + tid + NT * i < n ? order_key(v[i]) : 0u);
  }
  mx = block_max<NT>(mx, L.scratch);
  uint32_t T, r;
  radix_threshold<NT>(
      [&](uint32_t himask, uint32_t base, int sh, uint32_t mask) {
        for (int g0 = 0; g0 < n; g0 += kPass) {
          float v[RP];
          load_pass<NT, RP>(row, g0, n, v);
#pragma unroll
          for (int i = 0; i < RP; ++i)
            hist_add(L.hist, g0 + tid + NT * i < n, order_key(v[i]), 0u, himask, base, sh, mask);
        }
      },
      0u, mx, (uint32_t)a.k, L, T, r);
  int32_t *out = a.indices + (int64_t)qi * a.k;
  uint32_t sel_base = 0, eq_base = 0;
  int parity = 0;
  for (int g0 = 0; g0 < n; g0 += kPass, parity ^= 1) {
    float v[RP];
    load_pass<NT, RP>(row, g0, n, v);
    uint32_t key[RP];
#pragma unroll
    for (int i = 0; i < RP; ++i) key[i] = order_key(v[i]);
    uint32_t pre[RP];
    const uint32_t tot = ordered_prefix<NT, RP>(
        [&](int i) -> uint32_t {
          if (g0 + tid + NT * i >= n) return 0u;
          return key[i] > T ? 1u : (key[i] == T ? 0x10000u : 0u);
        },
        RP, pre, parity ? L.tot1 : L.tot0);
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const int t = g0 + tid + NT * i;
      const uint32_t sb = sel_base + (pre[i] & 0xFFFFu), eb = eq_base + (pre[i] >> 16);
      const bool gt = t < n && key[i] > T;
      const bool eq = t < n && key[i] == T && eb < r;
      const uint32_t pos = sb + (gt ? min(eb, r) : eb);
      if (gt || eq) out[pos] = t;
    }
    sel_base += tot & 0xFFFFu;
    eq_base += tot >> 16;
  }
  if (tid == 0 && a.counts) a.counts[qi] = a.k;
}

// Lower bound (top 16 bits) on the key of rank `need` among kSamples samples
// of the row: 64 runs of 16 consecutive tokens spread evenly over it.  A run
// is one 64-byte segment, so the samples cost 4 KB of reads (one sample per
// cache line would read half of the row).  n >= 1024.  Called by one whole
// wavefront.
__device__ uint32_t sample_bound_wave(const float *row, int n, uint32_t need) {
  const int lane = threadIdx.x & 63;
  uint32_t x[kSamples / 64];
#pragma unroll
  for (int i = 0; i < kSamples / 64; ++i) {
    const int run = 4 * i + (lane >> 4);
    const int start = (int)(((int64_t)run * n) / 64) & ~15;
    x[i] = order_key(row[start + (lane & 15)]);
  }
  return wave_rank_bound(x, need, 16);
}

// Candidate bound of a row from its group reports: with r = bound_rank(k, G,
// most) for its G full groups, a lower bound (16-bit prefix) on the
// ceil(k / r)-th largest report; 0 when there is no bound.  The first
// wavefront computes it; the result is broadcast through LDS (one barrier).
template <int N>
__device__ __forceinline__ uint32_t report_quantile(const uint32_t *b, int nb, uint32_t need) {
  const int lane = threadIdx.x & 63;
  uint32_t x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int g = lane + 64 * i;
    x[i] = g < nb ? b[g] : 0u;
  }
  return wave_rank_bound(x, need, 16);
}

// The first wavefront's share of a row's bound reports, loaded before the row
// length is known (lane l holds reports l + 64 i; reports past n_bounds read
// as 0).  N = 8 covers up to 512 reports, N = 32 up to 2048.
template <int N>
__device__ __forceinline__ void load_reports(const SelectArgs &a, int qi, uint32_t (&x)[N]) {
  const int lane = threadIdx.x & 63;
  const uint32_t *b = a.bounds + (int64_t)qi * a.n_bounds;
  const int last = a.n_bounds - 1;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int g = lane + 64 * i;
    x[i] = b[g < last ? g : last];
  }
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = lane + 64 * i < a.n_bounds ? x[i] : 0u;
}

// row_bound from reports already loaded by the first wavefront (load_reports).
template <int N>
__device__ uint32_t row_bound_from(const SelectArgs &a, int n, const uint32_t (&x)[N], const Lds &L) {
  const int r = bound_rank(a.k, n / a.group_tokens, a.bound_most);
  if (r == 0) return 0u;
  const uint32_t need = (uint32_t)((a.k + r - 1) / r);
  if (threadIdx.x < 64) {
    const uint32_t t = wave_rank_bound(x, need, 16);
    if (threadIdx.x == 0) L.shv[6] = t;
  }
  __syncthreads();
  return L.shv[6];
}

__device__ uint32_t row_bound(const SelectArgs &a, int qi, int n, const Lds &L) {
  const int r = bound_rank(a.k, n / a.group_tokens, a.bound_most);
  if (r == 0) return 0u;
  const uint32_t need = (uint32_t)((a.k + r - 1) / r);
  if (threadIdx.x < 64) {
    const uint32_t *b = a.bounds + (int64_t)qi * a.n_bounds;
    uint32_t t;
    if (a.n_bounds <= 512) t = report_quantile<8>(b, a.n_bounds, need);
    else t = report_quantile<32>(b, a.n_bounds, need);
    if (threadIdx.x == 0) L.shv[6] = t;
  }
  __syncthreads();
  return L.shv[6];
}

// One workgroup per row.  Each wavefront filters a contiguous slice of the
// row into a region of LDS of its own, in token order, so the stream of
// scores needs no workgroup barrier and every wavefront keeps two batches of
// loads in flight; the regions taken in wavefront order hold the candidates
// in token order.  Then the exact finish on the candidates.
constexpr int kLocalWaves = kLocalThreads / 64;
constexpr int kWaveCap = kLocalCap / kLocalWaves;   // candidates per wavefront region (896)
constexpr int kWaveRounds = 16;                      // 64-token rounds per load batch (4 KB per wavefront)
// Cache policy of the score loads: non-temporal (each score is read once; 4 %
// faster on the 2048-row chunk at 64K)
constexpr int kCpolNT = 2;
static_assert(kWaveCap % 64 == 0, "a row of at most kLocalCap tokens fits the regions without a bound");

__global__ __launch_bounds__(kLocalThreads) void select_local_kernel(SelectArgs a) {
  constexpr int NT = kLocalThreads, W = kLocalWaves, RW = kWaveRounds;
  extern __shared__ __align__(16) uint32_t lds[];
  const Lds L = carve(lds);
  const int zero = args_together(a);
  const int qi = blockIdx.y + zero;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float *row = a.scores + (int64_t)qi * a.ld;
  const int n = a.q_len[qi];
  const int k = a.k;
  if (n <= k) {
    emit_all<NT>(a, qi, n);
    return;
  }

  // this wavefront's slice [t0, t1) (64-token multiples), read in batches of RW
  // rounds through a buffer resource that ends at the slice's end: loads past
  // it (the tail of the last batch, the batch after it) read 0 without
  // touching memory and are dropped, instead of reading the next slice
  const int span = ((n + W - 1) / W + 63) / 64 * 64;
  const int t0 = min(wave * span, n), t1 = min(t0 + span, n);
  const int pairs = (t1 - t0 + 2 * 64 * RW - 1) / (2 * 64 * RW);
  const __amdgpu_buffer_rsrc_t rrow =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), (short)0, t1 * 4, 0x00020000);
  auto load_batch = [&](int b, float (&v)[RW]) {
    const uint32_t off = (uint32_t)(t0 + 64 * RW * b + lane) * 4u;
#pragma unroll
    for (int i = 0; i < RW; ++i)
      v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rrow, off + 256u * i, 0, kCpolNT));
  };
  float va[RW], vb[RW];
  load_batch(0, va);   // in flight while the bound is found

  uint32_t t_lo = 0;
  if (n > a.local_cap) {
    if (a.bounds) {
      t_lo = row_bound(a, qi, n, L);
    } else {
      if (wave == 0) {
        // about 2k candidates expected: rank 2 k S / n among S samples (+4)
        const uint64_t want = (uint64_t)2 * (uint64_t)k * kSamples / (uint64_t)n + 4;
        const uint32_t t = sample_bound_wave(row, n, (uint32_t)(want < kSamples ? want : kSamples));
        if (lane == 0) L.shv[4] = t;
      }
      __syncthreads();
      t_lo = L.shv[4];
    }
  }
  // order_key(x) >= t_lo as one float comparison x >= f_lo (exact: fp32
  // denormals are not flushed): t_lo 0 takes every score, NaN included; a
  // bound at or below the key of -inf every score but NaN; a negative bound
  // the float whose key it is; a positive one likewise (above the key of +inf
  // that float is a NaN and nothing passes, as no key lies above it)
  const bool take_all = t_lo == 0u;
  const float f_lo = t_lo >= 0x80000000u ? __uint_as_float(t_lo & 0x7FFFFFFFu)
                     : t_lo > 0x007FFFFFu ? __uint_as_float(~t_lo)
                                         : -INFINITY;

  uint2 *region = L.cand + wave * kWaveCap;
  uint32_t cnt = 0;      // candidates of this wavefront (uniform)
  float fmx = -INFINITY;  // largest candidate of this lane (fmaxf skips NaN; see below)
  auto filter_batch = [&](int b, const float (&v)[RW]) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int t = t0 + 64 * (RW * b + i) + lane;
      const bool in = (t < t1) & ((v[i] >= f_lo) | take_all);   // (no short circuit: lane masks only)
      const uint64_t m = __ballot(in);
      const uint32_t pos = cnt + lanes_below(m);
      if (in && pos < (uint32_t)kWaveCap) region[pos] = make_uint2(__float_as_uint(v[i]), (uint32_t)t);
      cnt += (uint32_t)__popcll(m);
      fmx = fmaxf(fmx, in ? v[i] : -INFINITY);
    }
  };
  // two batches per iteration in alternating buffers: while one is filtered the
  // other is in flight (the batch after the slice's last is loaded and dropped)
  for (int p = 0; p < pairs; ++p) {
    load_batch(2 * p + 1, vb);
    filter_batch(2 * p, va);
    load_batch(2 * p + 2, va);
    filter_batch(2 * p + 1, vb);
  }
  drain_loads();
  // The window's top: the key of the largest candidate.  fmaxf skips NaN and
  // -0 and +0 share a key, so order_key(max) is the largest key unless every
  // candidate is NaN (key 0), when it is the key of -inf, still an upper bound.
  const uint32_t kmx = wave_max_u32(order_key(fmx));   // (order_key is monotone; fmx is never NaN)
  if (lane == 0) {
    L.scratch[wave] = cnt;
    L.scratch[W + wave] = kmx;
  }
  __syncthreads();   // (also publishes the regions)
  uint32_t off[W + 1];
  off[0] = 0;
  bool overflow = false;
  uint32_t mx = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint32_t c = L.scratch[w];
    overflow |= c > (uint32_t)kWaveCap;
    off[w + 1] = off[w] + c;
    if (c) mx = max(mx, L.scratch[W + w]);
  }
  const uint32_t C = off[W];
  if (overflow || C < (uint32_t)k) {
    __syncthreads();   // every thread has read the counts before finish_row reuses the scratch words
    finish_row<NT>(a, qi, n, row, L);
    return;
  }
  // candidate j (token order) is entry j - off[w] of region w, off[w] <= j < off[w + 1];
  // its key is formed here, once per candidate
  constexpr int R = kLocalCap / NT;   // 14 slots: the regions hold at most kLocalCap candidates
  static_assert(kLocalCap % NT == 0, "whole slots");
  uint32_t ck[R], ct[R];
#pragma unroll
  for (int m = 0; m < R; ++m) {
    const uint32_t j = tid + NT * m;
    uint32_t at = j;   // LDS entry: the last region whose offset is <= j (empty regions are skipped over)
#pragma unroll
    for (int i = 1; i < W; ++i) at = j >= off[i] ? (uint32_t)(i * kWaveCap) + (j - off[i]) : at;
    const uint2 c = j < C ? L.cand[at] : make_uint2(0u, 0u);
    ck[m] = j < C ? order_key(__uint_as_float(c.x)) : 0u;
    ct[m] = c.y;
  }
  finish_regs<NT, R>(a, qi, C, t_lo, mx, ck, ct, L);
}

// Few long rows, step 2: workgroup (chunk c, row) filters its chunk and writes
// the candidates and their count to its own region.
__global__ __launch_bounds__(kFilterThreads) void select_filter_kernel(SelectArgs a) {
  constexpr int NT = kFilterThreads;
  extern __shared__ __align__(16) uint32_t lds[];
  const Lds L = carve(lds);
  const int zero = args_together(a);
  const int qi = blockIdx.y + zero, c = blockIdx.x;
  const int tid = threadIdx.x;
  const float *row = a.scores + (int64_t)qi * a.ld;
  const int c0 = c * a.chunk;
  // in flight while the row length arrives: the chunk's scores and, in the
  // first wavefront, the row's bound reports
  float v[kPassRounds];
  // (clamped to the chunk's end: a pass may be longer than the chunk, and the
  // next chunk's scores are another workgroup's to read)
  load_pass_clamped<NT, kPassRounds>(row, c0, min(c0 + a.chunk, a.max_len), v);
  const bool few_reports = a.n_bounds <= 512;
  uint32_t rep8[8], rep32[32];
  if (a.bounds && tid < 64) {
    if (few_reports) load_reports<8>(a, qi, rep8);
    else load_reports<32>(a, qi, rep32);
  }
  const int n = a.q_len[qi];
  const int k = a.k;
  if (n <= k) {
    if (c == 0) emit_all<NT>(a, qi, n);
    drain_loads();
    return;
  }
  const int c1 = min(c0 + a.chunk, n);
  uint32_t t_lo = 0u;
  if (n > kRegCap)
    t_lo = a.bounds ? (few_reports ? row_bound_from<8>(a, n, rep8, L) : row_bound_from<32>(a, n, rep32, L))
                    : row_bound(a, qi, n, L);
  if (c == 0 && tid == 0) a.tlo[qi] = t_lo;
  uint32_t key[kPassRounds];
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < kPassRounds; ++i) {
    key[i] = order_key(v[i]);
    mx = max(mx, c0 + tid + NT * i < c1 ? key[i] : 0u);
  }
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) L.scratch[40 + (tid >> 6)] = mx;   // read after the prefix's barriers
  uint32_t pre[kPassRounds];
  const uint32_t found = ordered_prefix<NT, kPassRounds>(
      [&](int i) -> uint32_t { return (c0 + tid + NT * i < c1 && key[i] >= t_lo) ? 1u : 0u; }, kPassRounds, pre,
      L.tot0);
  uint2 *dst = a.cand + ((int64_t)qi * a.chunks + c) * a.chunk;
#pragma unroll
  for (int i = 0; i < kPassRounds; ++i) {
    const int t = c0 + tid + NT * i;
    if (t < c1 && key[i] >= t_lo) dst[pre[i]] = make_uint2(key[i], (uint32_t)t);
  }
  if (tid == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) m = max(m, L.scratch[40 + w]);
    a.ccount[(int64_t)qi * a.chunks + c] = found;
    a.cmax[(int64_t)qi * a.chunks + c] = found ? m : 0u;
  }
}

// Few long rows, steps 3-4: one workgroup per row gathers the chunks'
// candidates (in chunk order, i.e. token order) into registers and finishes.
__global__ __launch_bounds__(kFinishThreads) void select_finish_kernel(SelectArgs a) {
  constexpr int NT = kFinishThreads;
  constexpr int R = kRegCap / NT;
  extern __shared__ __align__(16) uint32_t lds[];
  const Lds L = carve(lds);
  const int zero = args_together(a);
  const int qi = blockIdx.y + zero;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *row = a.scores + (int64_t)qi * a.ld;
  const int chunks = a.chunks;
  // the row length, the row's bound and the chunk counts and maxima are all in
  // flight together (every row has its regions; rows the filter emitted whole
  // are not finished, so what they hold does not matter)
  const int n = a.q_len[qi];
  const uint32_t tlo_v = a.tlo[qi];
  constexpr int PL = kMaxChunks / 64;   // 4: one 16-byte load of each array per lane
  static_assert(PL == 4, "chunk counts are loaded as one uint4 per lane");
  uint4 c4 = make_uint4(0u, 0u, 0u, 0u), m4 = make_uint4(0u, 0u, 0u, 0u);
  if (wave == 0 && (chunks & 3) == 0) {
    // both loads of a lane in flight together (the counts and maxima of the
    // chunk regions are 16-byte aligned when chunks is a multiple of 4)
    const int cl = min(lane * PL, chunks - PL);
    c4 = *reinterpret_cast<const uint4 *>(a.ccount + (int64_t)qi * chunks + cl);
    m4 = *reinterpret_cast<const uint4 *>(a.cmax + (int64_t)qi * chunks + cl);
  }
  if (n <= a.k) {   // the filter kernel emitted the row
    drain_loads();
    return;
  }

  // the first wavefront: chunk counts -> exclusive prefix cpre[0..chunks],
  // cmap[b] = chunk of candidate 64 b, and the largest candidate key
  if (wave == 0) {
    uint32_t cc[PL];
    uint32_t s = 0, m = 0;
    if ((chunks & 3) == 0) {
      // both loads of a lane in flight together (the counts and maxima of the
      // chunk regions are 16-byte aligned when chunks is a multiple of 4)
      if (lane * PL >= chunks) {   // lanes past the last chunk loaded a clamped copy: they count nothing
        c4 = make_uint4(0u, 0u, 0u, 0u);
        m4 = make_uint4(0u, 0u, 0u, 0u);
      }
      cc[0] = c4.x;
      cc[1] = c4.y;
      cc[2] = c4.z;
      cc[3] = c4.w;
      m = max(max(m4.x, m4.y), max(m4.z, m4.w));
#pragma unroll
      for (int i = 0; i < PL; ++i) s += cc[i];
    } else {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int ch = lane * PL + i;
        cc[i] = ch < chunks ? a.ccount[(int64_t)qi * chunks + ch] : 0u;
        m = max(m, ch < chunks ? a.cmax[(int64_t)qi * chunks + ch] : 0u);
        s += cc[i];
      }
    }
    const uint32_t incl = wave_inclusive_scan(s);
    const bool fits = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) <= (uint32_t)kRegCap;
    m = wave_max_u32(m);
    uint32_t run = incl - s;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int ch = lane * PL + i;
      if (ch < chunks) {
        L.cpre[ch] = run;
        if (fits)
          for (uint32_t b = (run + 63u) >> 6; (b << 6) < run + cc[i]; ++b) L.cmap[b] = (uint32_t)ch;
      }
      run += cc[i];
    }
    if (lane == 63) {
      L.cpre[chunks] = incl;
      if (fits) L.cmap[(incl + 63u) >> 6] = (uint32_t)(chunks - 1);
      L.shv[1] = incl;
      L.shv[2] = tlo_v;
      L.shv[3] = m;
    }
  }
  __syncthreads();
  const uint32_t C = L.shv[1];
  const uint32_t t_lo = L.shv[2];
  const uint32_t mx = L.shv[3];
  if (C < (uint32_t)a.k || C > (uint32_t)kRegCap) {
    finish_row<NT>(a, qi, n, row, L);
    return;
  }
  const uint32_t nb = (C + 63u) >> 6;
  // Candidates 64 b .. 64 b + 63 are one wavefront's round (b uniform per
  // wavefront); their chunks lie in [cmap[b], cmap[b + 1]].
  const uint2 *cand_row = a.cand + (int64_t)qi * chunks * a.chunk;
  const int rounds = (int)((C + NT - 1) / NT);
  uint2 cv[R];
#pragma unroll
  for (int m = 0; m < R; ++m) {
    cv[m] = make_uint2(0u, 0u);
    if (m < rounds) {
      const uint32_t j = tid + NT * m;
      const uint32_t b = j >> 6;   // uniform per wavefront
      if (b < nb) {
        const uint32_t c0 = L.cmap[b], c1 = L.cmap[b + 1];
        uint32_t ch = c0;
        for (uint32_t x = c0 + 1; x <= c1; ++x) ch += L.cpre[x] <= j ? 1u : 0u;
        if (j < C) cv[m] = cand_row[(int64_t)ch * a.chunk + (j - L.cpre[ch])];
      }
    }
  }
  uint32_t ck[R], ct[R];
#pragma unroll
  for (int m = 0; m < R; ++m) {
    ck[m] = cv[m].x;
    ct[m] = cv[m].y;
  }
  finish_regs<NT, R>(a, qi, C, t_lo, mx, ck, ct, L);
}

// Group bounds from a score row (when the scores did not come with them): for
// group g of kGroup tokens, a lower bound (16-bit prefix) on its r-th largest
// key, r = bound_rank(k, G, kGroup) with G full groups in the row; 0 when the
// group is not full.
__global__ __launch_bounds__(256) void bound_kernel(const float *__restrict__ scores, int64_t ld,
                                                    const int32_t *__restrict__ q_len, int k,
                                                    uint32_t *__restrict__ bounds) {
  __shared__ uint32_t keys[kGroup];
  const int qi = blockIdx.y, g = blockIdx.x;
  const int n = q_len[qi];
  const int rank = bound_rank(k, n / kGroup, kGroup);
  const bool full = (g + 1) * kGroup <= n && rank >= 1;
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
    const uint32_t T = full ? wave_rank_bound(x, (uint32_t)rank, 16) : 0u;
    if (threadIdx.x == 0) bounds[(int64_t)qi * gridDim.x + g] = T;
  }
}

// Reorders each row's kept indices (ascending token order, count = min(k, n),
// -1 padding after them) into the stable argsort order of -scores: score
// descending, equal scores by ascending token index.  Every kept token becomes
// the 64-bit value (order_key(score) << 32) | ~token, which orders exactly that
// way (tokens are distinct, so no two values are equal), and a bitonic network
// in LDS sorts the values descending; padding values are 0, below every real
// one (~token >= 2^31).  One workgroup per row.
constexpr int kOrderThreads = 1024;
constexpr int kOrderMax = 2048;

__global__ __launch_bounds__(kOrderThreads) void order_by_score_kernel(int32_t *__restrict__ indices,
                                                                       const float *__restrict__ scores, int64_t ld,
                                                                       const int32_t *__restrict__ q_len, int k) {
  __shared__ uint64_t v[kOrderMax];
  const int qi = blockIdx.y;
  const int n = q_len[qi];
  const int cnt = n < k ? n : k;
  if (cnt <= 1) return;
  int lg = 0;
  while ((1 << lg) < cnt) ++lg;
  const int P = 1 << lg;
  int32_t *row = indices + (int64_t)qi * k;
  const float *srow = scores + (int64_t)qi * ld;
  for (int j = threadIdx.x; j < P; j += kOrderThreads) {
    uint64_t c = 0;
    if (j < cnt) {
      const uint32_t t = (uint32_t)row[j];
      c = ((uint64_t)order_key(srow[t]) << 32) | (uint64_t)(~t);
    }
    v[j] = c;
  }
  __syncthreads();
  for (int ls = 1; ls <= lg; ++ls) {            // blocks of 2^ls: descending when (i & 2^ls) == 0
    for (int lt = ls - 1; lt >= 0; --lt) {      // compare distance 2^lt
      for (int t = threadIdx.x; t < (P >> 1); t += kOrderThreads) {
        const int i = ((t >> lt) << (lt + 1)) | (t & ((1 << lt) - 1));
        const int j = i | (1 << lt);
        const uint64_t a = v[i], b = v[j];
        const bool desc = (i & (1 << ls)) == 0;
        if (desc ? a < b : a > b) {
          v[i] = b;
          v[j] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = threadIdx.x; j < cnt; j += kOrderThreads) row[j] = (int32_t)(~(uint32_t)v[j]);
}

}  // namespace

hipError_t launch_order_by_score(int32_t *indices, const float *scores, int64_t ld, const int32_t *q_len, int n_q,
                                 int k, hipStream_t stream) {
  if (k > kOrderMax || n_q > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(order_by_score_kernel, dim3(1, n_q), dim3(kOrderThreads), 0, stream, indices, scores, ld,
                     q_len, k);
  return hipGetLastError();
}

TopkPlan plan_topk(int n_q, int k, int max_len) {
  TopkPlan p{};
  p.n_q = n_q;
  p.k = k;
  p.max_len = max_len;
  // Many rows, or short rows: one workgroup per row.  Few long rows: spread each
  // row over several filter workgroups (about 256 in all) so the whole chip
  // takes part, then one finishing workgroup per row.
  int chunks = 1;
  if (n_q < 128 && max_len > 8192) {
    chunks = 256 / (n_q > 0 ? n_q : 1);
    const int fewest = (max_len + kPass - 1) / kPass;
    const int most = (max_len + 1023) / 1024;
    if (chunks > most) chunks = most;
    if (chunks < fewest) chunks = fewest;   // a chunk is one filter pass
    if (chunks < 2) chunks = 2;
  }
  int chunk = (max_len + chunks - 1) / chunks;
  chunk = (chunk + 63) / 64 * 64;
  chunks = (max_len + chunk - 1) / chunk;
  p.chunks = chunks;
  p.chunk = chunk;
  p.group = kGroup;
  p.groups = (max_len + kGroup - 1) / kGroup;
  p.local_cap = chunks == 1 ? kLocalCap : 0;
  p.lds_bytes = (size_t)kFixedWords * 4 + (size_t)p.local_cap * 8;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  if (chunks > 1) {
    p.off_tlo = take((size_t)n_q * 4);
    p.off_count = take((size_t)n_q * chunks * 4);
    p.off_cmax = take((size_t)n_q * chunks * 4);
    p.off_bounds = take((size_t)n_q * p.groups * 4);
    p.off_cand = take((size_t)n_q * chunks * chunk * 8);
  }
  p.total = off;
  return p;
}

hipError_t launch_topk(int32_t *indices, int32_t *counts, const float *scores, int64_t ld, const int32_t *q_len,
                       const TopkPlan &plan, void *workspace, const uint32_t *bounds, int n_bounds,
                       int group_tokens, hipStream_t stream) {
  // the one-workgroup-per-row kernel may use up to 160 KB of dynamic LDS; the
  // attribute is set once per device (the current one)
  static std::atomic<uint64_t> lds_set{0};
  int dev = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return de;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (!bit || !(lds_set.load(std::memory_order_acquire) & bit)) {
    de = hipFuncSetAttribute(reinterpret_cast<const void *>(&select_local_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (de != hipSuccess) return de;
    lds_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (plan.lds_bytes > 160 * 1024 || plan.chunks > kMaxChunks || (plan.chunks > 1 && plan.chunk > kPass))
    return hipErrorInvalidValue;
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
  a.local_cap = plan.local_cap;
  a.bounds = bounds;
  a.n_bounds = n_bounds;
  a.group_tokens = group_tokens > 0 ? group_tokens : 1;
  a.bound_most = 32;
  a.max_len = plan.max_len;
  if (plan.chunks > 1) {
    a.tlo = reinterpret_cast<uint32_t *>(ws + plan.off_tlo);
    a.ccount = reinterpret_cast<uint32_t *>(ws + plan.off_count);
    a.cmax = reinterpret_cast<uint32_t *>(ws + plan.off_cmax);
    a.cand = reinterpret_cast<uint2 *>(ws + plan.off_cand);
    if (!bounds) {
      uint32_t *b = reinterpret_cast<uint32_t *>(ws + plan.off_bounds);
      hipLaunchKernelGGL(bound_kernel, dim3(plan.groups, plan.n_q), dim3(256), 0, stream, scores, ld, q_len, plan.k,
                         b);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      a.bounds = b;
      a.n_bounds = plan.groups;
      a.group_tokens = kGroup;
      a.bound_most = kGroup;
    }
    hipLaunchKernelGGL(select_filter_kernel, dim3(plan.chunks, plan.n_q), dim3(kFilterThreads),
                       (size_t)kFixedWords * 4, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_finish_kernel, dim3(1, plan.n_q), dim3(kFinishThreads), (size_t)kFixedWords * 4,
                       stream, a);
  } else {
    hipLaunchKernelGGL(select_local_kernel, dim3(1, plan.n_q), dim3(kLocalThreads), plan.lds_bytes, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
