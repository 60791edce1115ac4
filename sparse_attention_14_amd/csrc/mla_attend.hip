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
// row gathers hit one L2.  Many queries (prefill chunks, decode windows) take
// the 64-head kernel further below, which gathers each kept row once for all
// heads of a query.
#include "kernels.hpp"

#include <atomic>
#include <utility>

namespace dsa {
namespace {

// Sequence of query qi: q_seq[qi], else qi / per (per queries per sequence),
// or 0 when per is 0.
__device__ __forceinline__ int attend_seq(const int32_t *q_seq, int qi, int per) {
  return q_seq ? q_seq[qi] : (per > 0 ? qi / per : 0);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ bf16 path
constexpr int kW = 576, kL = 512, kTile = 64, kHG = 16;
constexpr int kRowBytes = kW * 2 + 16;          // padded LDS row
constexpr int kChunks = kW * 2 / 16;            // 16-byte chunks per row (72)
constexpr int kMaxSplits = 32;
// Lazy softmax maximum: a head's reference maximum moves only when a step's
// maximum exceeds it by more than 2^kSlack (in the exp2 domain) or it is still
// -inf, so the weights stay <= 2^kSlack and the running output is rescaled only
// in the rare steps where some reference moved (alpha is exactly 1 otherwise).
constexpr float kSlack = 8.0f;
constexpr int kAttTargetWGs = 256;   // workgroups aimed at by the split count
constexpr int kWideMinRows = 16;     // (query, 64-head block) pairs from which the 64-head kernel is used

struct AttArgs {
  float *out;
  float *lse;
  const uint16_t *q;
  CacheDev latent;
  const int32_t *indices;
  const int32_t *q_seq;
  float *part_o;   // [n_q][S][H][L]
  float *part_ml;  // [n_q][S][H][2]
  int k, n_q, n_heads, splits, rows_per_split, n_hg, pairs, seq_per;
  float scale_log2;  // softmax_scale * log2(e)
};

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// Fetches every argument in one round trip: the returned zero depends on all of
// them, so code indexed by it waits for one batch of argument loads instead of
// one dependent scalar round trip per argument at its first use.
__device__ __forceinline__ int args_together(const AttArgs &a) {
  int zero;
  asm("s_mov_b32 %0, 0"
      : "=s"(zero)
      : "s"(a.out), "s"(a.lse), "s"(a.q), "s"(a.latent.rows), "s"(a.latent.scale), "s"(a.latent.row_stride),
        "s"(a.latent.block_stride), "s"(a.latent.scale_block_stride), "s"(a.latent.table), "s"(a.latent.block_size),
        "s"(a.latent.max_blocks), "s"(a.indices), "s"(a.q_seq), "s"(a.part_o), "s"(a.part_ml), "s"(a.k),
        "s"(a.n_q), "s"(a.n_heads), "s"(a.splits), "s"(a.rows_per_split), "s"(a.n_hg), "s"(a.pairs),
        "s"(a.seq_per), "s"(a.scale_log2));
  return zero;
}

// Allreduce over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1).
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
  return x;
}

// 2^x as the hardware instruction (v_exp_f32, about 1 ulp): the softmax
// weights and rescale factors have x <= 8, and results below 2^-126 of the
// running maximum are negligible next to it however they are rounded.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two weights split into bf16 hi + lo parts (hi = rne(x), lo = rne(x - hi)),
// packed two per word (first weight in the low half), by the packed
// round-to-nearest-even conversion.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}
__device__ __forceinline__ void split_hi_lo(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = bf16x2_rne(a, b);
  lo = bf16x2_rne(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// Transposed LDS read (ds_read_b64_tr_b16): in each 16-lane group, lane p
// names 4 bf16 of row base + p / 4 at columns col + 4 (p % 4); lane i of the
// group receives rows base .. base + 3 of column col + i.
__device__ __forceinline__ i16x4 lds_read_tr(const uint8_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(reinterpret_cast<uintptr_t>(p)));
}

// Two teams of four wavefronts: per step the workgroup gathers 128 kept rows
// (thread t copies 18 16-byte chunks of row t / 4 from one base address), and
// team t scores rows [64 t, 64 t + 64) with its own online softmax; the teams'
// states are combined at the end.
constexpr int kTeams = 2;
constexpr int kStepRows = kTile * kTeams;    // 128
constexpr int kAttThreads = 256 * kTeams;    // 512

// F8: e4m3fn latent rows with a float32 scale per token.  The bytes are
// decoded exactly to bf16 on their way into LDS; the token's scale multiplies
// its logit (after the QK^T MFMA) and its probability as a PV weight.
template <bool SPLIT, bool F8>
__global__ __launch_bounds__(kAttThreads) void attend_bf16_kernel(AttArgs a) {
  __shared__ __align__(16) uint8_t lrows[kTeams][kTile * kRowBytes];
  __shared__ __align__(16) uint16_t lp[kTeams][2][kHG * kTile];  // P hi / lo, [head][row]
  __shared__ float red[kTeams][2][4][kHG];
  __shared__ uint8_t lvalid[kStepRows];
  __shared__ float lscale[F8 ? kStepRows : 1];

  // XCD-aware mapping: workgroup ids i, i+8, i+16, ... run on one XCD; give the
  // n_hg head groups of a (query, split) pair ids 8 apart.
  const int lin = blockIdx.x + args_together(a);
  const int group = lin / (8 * a.n_hg);
  const int rem = lin - group * 8 * a.n_hg;
  const int hg = rem >> 3;
  const int pair = group * 8 + (rem & 7);
  if (pair >= a.pairs) return;
  const int qi = pair / a.splits;
  const int sp = pair - qi * a.splits;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int team = wave >> 2, tw = wave & 3;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int H = a.n_heads;
  const int h0 = hg * kHG;
  const int seq = attend_seq(a.q_seq, qi, a.seq_per);

  const int j0 = sp * a.rows_per_split;
  const int j1 = min(j0 + a.rows_per_split, a.k);
  const int nsteps = (j1 - j0 + kStepRows - 1) / kStepRows;

  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }
  f32x4 o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0, 0, 0, 0};

  // q operand (head h0 + l16, dims 32*ks + 8*g4 + [0, 8)): loaded after the
  // first step's index and row loads are issued, so those are not queued
  // behind it
  bf16x8 qa[kW / 32];
  const uint16_t *qr = a.q + ((int64_t)qi * H + h0 + l16) * kW + 8 * g4;

  uint8_t *my_rows = lrows[team];
  uint16_t *my_p = lp[team][0];
  for (int step = 0; step < nsteps; ++step) {
    {
      // 8 lanes per row, so every load instruction covers whole 128-byte lines:
      // rows gr8 and gr8 + kTile, 16-byte chunks gq8 + 8 i (bf16: 72 chunks,
      // i < 9; fp8: 36 chunks, i < 5, the last only for gq8 < 4)
      const int gr8 = tid >> 3, gq8 = tid & 7;
      constexpr int NV8 = F8 ? 5 : kChunks / 8;
      u32x4 w[kTeams][NV8];
      float sc[kTeams];
      bool ok[kTeams];
      // both rows' indices, then both rows' addresses, then all row loads, so
      // the second row does not wait behind the first row's data; an empty
      // slot loads the cache's first row and is zeroed when written to LDS
      int tok[kTeams];
#pragma unroll
      for (int r = 0; r < kTeams; ++r) {
        const int j = j0 + step * kStepRows + gr8 + kTile * r;
        tok[r] = j < j1 ? a.indices[(int64_t)qi * a.k + min(j, a.k - 1)] : -1;
      }
      const uint8_t *src[kTeams];
      int64_t sblk[kTeams];
      int sslot[kTeams];
#pragma unroll
      for (int r = 0; r < kTeams; ++r) {
        ok[r] = tok[r] >= 0;
        sblk[r] = cache_block(a.latent, seq, ok[r] ? tok[r] : 0, sslot[r]);
        src[r] = ok[r] ? cache_row(a.latent, sblk[r], sslot[r]) : a.latent.rows;
      }
#pragma unroll
      for (int r = 0; r < kTeams; ++r) {
#pragma unroll
        for (int i = 0; i < NV8; ++i)
          w[r][i] = load16(src[r] + (F8 ? min(16 * gq8 + 128 * i, kW - 16) : 16 * gq8 + 128 * i));
        sc[r] = F8 && ok[r] ? a.latent.scale[sblk[r] * a.latent.scale_block_stride + sslot[r]] : 0.0f;
      }
      if (__ballot(!(ok[0] && ok[1])))   // (only a split's last step has empty slots)
#pragma unroll
        for (int r = 0; r < kTeams; ++r)
#pragma unroll
          for (int i = 0; i < NV8; ++i) w[r][i] = ok[r] ? w[r][i] : u32x4{0, 0, 0, 0};
      if (step == 0) {
#pragma unroll
        for (int ks = 0; ks < kW / 32; ++ks) qa[ks] = as_bf16x8(load16(qr + 32 * ks));
      }
#pragma unroll
      for (int r = 0; r < kTeams; ++r) {
        if (gq8 == 0) {
          lvalid[gr8 + kTile * r] = ok[r] ? 1 : 0;
          if (F8) lscale[gr8 + kTile * r] = sc[r];
        }
        uint8_t *row_base = lrows[r] + gr8 * kRowBytes;
        if (F8) {
          // fp8 chunk gq8 + 8 i -> 16 bf16 at LDS bytes 32 (gq8 + 8 i) ..
#pragma unroll
          for (int i = 0; i < NV8; ++i) {
            if (i < NV8 - 1 || gq8 < 4) {
              uint8_t *dst = row_base + 32 * gq8 + 256 * i;
              *reinterpret_cast<bf16x8 *>(dst) = fp8x8_to_bf16x8(w[r][i][0], w[r][i][1]);
              *reinterpret_cast<bf16x8 *>(dst + 16) = fp8x8_to_bf16x8(w[r][i][2], w[r][i][3]);
            }
          }
        } else {
          uint8_t *dst = row_base + 16 * gq8;
#pragma unroll
          for (int i = 0; i < NV8; ++i) *reinterpret_cast<u32x4 *>(dst + 128 * i) = w[r][i];
        }
      }
    }
    __syncthreads();

    // QK^T: this wavefront's 16 rows of its team's tile; each row operand is
    // read two MFMAs ahead (the scheduling barriers keep the reads from being
    // hoisted further, which would not fit the registers)
    const int row = tw * 16 + l16;
    f32x4 sacc = {0, 0, 0, 0};
    {
      const uint8_t *rp = my_rows + row * kRowBytes + 16 * g4;
      auto qk_read = [&](int ks) { return as_bf16x8(*reinterpret_cast<const u32x4 *>(rp + 64 * ks)); };
      bf16x8 br[2] = {qk_read(0), qk_read(1)};
#pragma unroll
      for (int ks = 0; ks < kW / 32; ++ks) {
        const bf16x8 b = br[ks & 1];
        if (ks + 2 < kW / 32) br[ks & 1] = qk_read(ks + 2);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], b, sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const bool valid = lvalid[team * kTile + row] != 0;
    const float rs = F8 ? lscale[team * kTile + row] : 1.0f;   // the row's dequantization scale
    float z[4], mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = valid ? (F8 ? sacc[i] * rs : sacc[i]) * a.scale_log2 : -INFINITY;
      mx[i] = row16_max(z[i]);
    }
    if (l16 == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[team][0][tw][4 * g4 + i] = mx[i];
    __syncthreads();

    // lazy reference maximum, as in the 64-head kernel below
    float m_new[4], alpha[4], ps[4], pv[4];
    bool moved = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
      const float tm =
          fmaxf(fmaxf(red[team][0][0][h], red[team][0][1][h]), fmaxf(red[team][0][2][h], red[team][0][3][h]));
      const bool grow = tm > m_run[i] + kSlack;
      moved |= grow;
      m_new[i] = grow ? tm : m_run[i];
      const float mu = m_new[i] == -INFINITY ? 0.0f : m_new[i];
      alpha[i] = grow ? fast_exp2(m_run[i] - mu) : 1.0f;
      const float p = fast_exp2(z[i] - mu);
      pv[i] = F8 ? p * rs : p;                // weight of the decoded (unscaled) row
      ps[i] = row16_sum(p);
    }
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const int h = 4 * g4 + i;
      uint32_t hi, lo;
      split_hi_lo(pv[i], pv[i + 1], hi, lo);
      my_p[h * kTile + row] = (uint16_t)hi;
      my_p[(h + 1) * kTile + row] = (uint16_t)(hi >> 16);
      my_p[kHG * kTile + h * kTile + row] = (uint16_t)lo;
      my_p[kHG * kTile + (h + 1) * kTile + row] = (uint16_t)(lo >> 16);
    }
    if (l16 == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[team][1][tw][4 * g4 + i] = ps[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
      const float tsum = ((red[team][1][0][h] + red[team][1][1][h]) + red[team][1][2][h]) + red[team][1][3][h];
      l_run[i] = l_run[i] * alpha[i] + tsum;
      m_run[i] = m_new[i];
    }
    if (step > 0 && __ballot(moved))   // (before the first step o is 0)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= alpha[i];

    // PV: rows 32*ks2 + 8*g4 + e, columns 128*tw + 16*nt + l16; the V operand
    // comes from two transposed LDS reads of 4 rows each
#pragma unroll
    for (int ks2 = 0; ks2 < kTile / 32; ++ks2) {
      const bf16x8 ahi = as_bf16x8(*reinterpret_cast<const u32x4 *>(&my_p[l16 * kTile + 32 * ks2 + 8 * g4]));
      const bf16x8 alo =
          as_bf16x8(*reinterpret_cast<const u32x4 *>(&my_p[kHG * kTile + l16 * kTile + 32 * ks2 + 8 * g4]));
      const uint8_t *vb = my_rows + (32 * ks2 + 8 * g4 + (l16 >> 2)) * kRowBytes + (128 * tw + 4 * (l16 & 3)) * 2;
      auto pv_read = [&](int nt) {
        const i16x4 v0 = lds_read_tr(vb + 32 * nt);
        const i16x4 v1 = lds_read_tr(vb + 4 * kRowBytes + 32 * nt);
        return __builtin_bit_cast(bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){
                                              v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
      };
      bf16x8 vr[2] = {pv_read(0), pv_read(1)};   // V operands one tile ahead
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bf16x8 b = vr[nt & 1];
        if (nt + 2 < 8) vr[nt & 1] = pv_read(nt + 2);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, o[nt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  }

  // combine the teams: team 1 hands its state to team 0 through LDS
  float *xo = reinterpret_cast<float *>(lrows[1]);              // [16 heads][512]
  float *xml = reinterpret_cast<float *>(lrows[1]) + kHG * kL;  // [16 heads][2]
  if (team == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) xo[h * kL + 128 * tw + 16 * nt + l16] = o[nt][i];
      if (tw == 0 && l16 == 0) {
        xml[2 * h] = m_run[i];
        xml[2 * h + 1] = l_run[i];
      }
    }
  }
  __syncthreads();
  if (team == 1) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g4 + i;
    const float m1 = xml[2 * h], l1 = xml[2 * h + 1];
    const float m = fmaxf(m_run[i], m1);
    const float mu = m == -INFINITY ? 0.0f : m;
    const float a0 = fast_exp2(m_run[i] - mu), a1 = fast_exp2(m1 - mu);
    l_run[i] = a0 * l_run[i] + a1 * l1;
    m_run[i] = m;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt][i] = a0 * o[nt][i] + a1 * xo[h * kL + 128 * tw + 16 * nt + l16];
  }

  // epilogue: lane holds heads h0 + 4*g4 + i, columns 128*tw + 16*nt + l16
  if (!SPLIT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = h0 + 4 * g4 + i;
      const float inv = l_run[i] > 0.0f ? 1.0f / l_run[i] : 0.0f;
      float *orow = a.out + ((int64_t)qi * H + head) * kL + 128 * tw + l16;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) orow[16 * nt] = o[nt][i] * inv;
      if (tw == 0 && l16 == 0 && a.lse)
        a.lse[(int64_t)qi * H + head] = l_run[i] > 0.0f ? (m_run[i] + log2f(l_run[i])) * kLn2 : -INFINITY;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = h0 + 4 * g4 + i;
      const int64_t base = ((int64_t)(qi * a.splits + sp) * H + head);
      float *orow = a.part_o + base * kL + 128 * tw + l16;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) orow[16 * nt] = o[nt][i];
      if (tw == 0 && l16 == 0) {
        a.part_ml[base * 2 + 0] = m_run[i];
        a.part_ml[base * 2 + 1] = l_run[i];
      }
    }
  }
}

// Many queries (decode windows, prefill): a workgroup owns one query, a block
// of 64 heads and a split of whole 64-slot steps of the index list, so each
// kept row is gathered once for all 64 heads (the 16-head kernel above spreads
// few queries over more workgroups, at the price of gathering every row once
// per head group).
constexpr int kWideHeads = 64;
constexpr int kWideStep = 64;

// The 64-head kernel (prefill chunks, decode windows; bf16 or fp8 rows): a workgroup of
// four wavefronts owns one query, a block of 64 heads and a split of the index
// slots, and wavefront w owns heads 16 w .. 16 w + 15 of the block for the
// whole split, so its softmax needs no other wavefront.  Per 32-slot step the
// kept rows are copied from memory straight into LDS (global_load_lds_dwordx4,
// no registers), one step ahead into the other of two buffers; one barrier per
// step and two workgroups per CU.  The 16-byte chunk c of row r sits at slot
// c ^ h(r) of the row (h below), which keeps both operand reads free of bank
// conflicts:
//   QK^T : v_mfma_f32_16x16x32_bf16 with A = 16 rows (LDS) and B = q (16 heads,
//          registers), so D leaves lane (head l16, g4) with rows 4 g4 + i of
//          both 16-row halves: 8 rows of one head;
//   softmax in the exp2 domain (lazy reference maximum): 8 rows in the lane,
//          the 4 lanes of a head combined by two lane exchanges;
//   PV   : A = P exactly as the lane holds it (K = its 8 rows, bf16 hi + lo),
//          B = V read transposed from LDS in the same row order (two 4-row
//          reads), 32 tiles of 16 columns.
// fp8 rows (e4m3fn bytes and a float32 scale per token) are copied as they are
// stored, half the bytes, into a staging area inside each wavefront's part of
// the next step's image and converted to bf16 there at the end of the step
// (exactly: every e4m3fn value is a bf16 value); the scales multiply the scores
// and the weights of P instead of the rows.
constexpr int kW4Step = 32;                               // rows per step
constexpr int kW4Threads = 256;
constexpr int kW4RowB = kW * 2;                           // 1152 bytes per row, no padding
constexpr int kW4Chunks = kW4RowB / 16;                   // 72
constexpr int kW4PerThread = kW4Step * kW4Chunks / kW4Threads;   // 9 chunk copies per thread and step
constexpr int kW4BufB = kW4Step * kW4RowB;                // 36864
// fp8 rows: a step's 32 row scales follow its bf16 image in the buffer
constexpr int kW4ScaleOfs = kW4BufB;
template <bool F8>
constexpr int kW4BufStride = kW4BufB + (F8 ? 4 * kW4Step : 0);
template <bool F8>
constexpr size_t kW4LdsBytes = 2 * (size_t)kW4BufStride<F8>;   // two buffers: 73728 (+ 256)
// fp8 rows (576 bytes, 36 chunks): wavefront w copies its rows 8 w .. 8 w + 7
// (288 chunks) into the second half of their bf16 image (bytes 4608 ..), five
// instructions, the last for 32 lanes
constexpr int kW4F8Chunks = kW / 16;                      // 36
constexpr int kW4F8WaveChunks = 8 * kW4F8Chunks;          // 288
constexpr int kW4F8Copies = (kW4F8WaveChunks + 63) / 64;  // 5
constexpr int kW4F8Stage = 8 * kW4RowB / 2;               // 4608: staging offset in the wavefront's 9216 bytes
static_assert(kW4Step * kW4Chunks == kW4PerThread * kW4Threads, "whole chunk copies per thread");
constexpr int kW4QkAhead = 2;   // row operands in flight ahead of the QK^T MFMAs
constexpr int kW4PvAhead = 2;   // V operands in flight ahead of the PV MFMAs

// Chunk swizzle of row r: slot = chunk ^ h(r % 16), h a 3-bit value per row.
// The row stride (1152 bytes) is a multiple of the bank width, so only h
// separates rows: h is distinct over any 8 aligned rows and over the even and
// the odd rows of 16 (16-byte reads, 8 or 16 lanes per cycle), and h >> 1 is
// distinct over any 4 aligned rows and over the same-parity rows of 8 (the
// transposed reads: 4 or 8 rows at 2 adjacent chunks), so both operand reads
// are free of bank conflicts with 32 or with 64 banks.
__device__ __forceinline__ int w4_swz(int r) {
  constexpr uint64_t kH = 0x4602753157136420ull;   // h(i) in nibble i: 0 2 4 6 3 1 7 5 1 3 5 7 2 0 6 4
  return (int)((kH >> (4 * (r & 15))) & 7u);
}

// Lanes l and l ^ 16 (l ^ 32) combined by the VALU lane swaps (no LDS round
// trip): v_permlane16_swap / v_permlane32_swap of x with itself leave the two
// partners' values in the two results of every lane.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool SPLIT, bool F8>
__global__ __launch_bounds__(kW4Threads, 2) void attend_w4_kernel(AttArgs a) {
  extern __shared__ __align__(16) uint8_t w4lds[];
  const int H = a.n_heads;
  const int n_hb = H / kWideHeads;
  const int wg = blockIdx.x + args_together(a);
  const int qi = wg / (a.splits * n_hb);
  const int rem = wg - qi * a.splits * n_hb;
  const int hb = rem / a.splits, sp = rem - hb * a.splits;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int h0 = hb * kWideHeads + wave * kHG;
  const int seq = attend_seq(a.q_seq, qi, a.seq_per);
  const int j0 = sp * a.rows_per_split;
  const int j1 = min(j0 + a.rows_per_split, a.k);
  const int nsteps = (j1 - j0 + kW4Step - 1) / kW4Step;
  const int32_t *idx_row = a.indices + (int64_t)qi * a.k;

  // Step copies: this wavefront's 9 instructions write LDS bytes
  // [1024 (9 wave + u), +1024) of a buffer; lane l's 16 bytes there are entry
  // q = 64 (9 wave + u) + l = row q / 72, slot q % 72, i.e. chunk (q % 72) ^ h(row).
  // (recomputed where used: hoisted out of the step loop they would not fit the registers)
  auto fresh_lane = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  auto copy_row = [&](int u, int l) { return (64 * (kW4PerThread * wave + u) + l) / kW4Chunks; };
  // Lanes 0..31 each hold the token of one row of a step; the rows' validity is
  // a 32-bit mask (uniform).
  auto step_token = [&](int st) {
    const int j = j0 + st * kW4Step + lane;
    return (lane < kW4Step && j < j1) ? idx_row[j] : -1;
  };
  // The wavefront's entries cover its rows 8 wave .. 8 wave + 7: instruction u
  // starts in row 8 wave + (64 u) / 72 at slot (64 u) % 72, so a lane's row is
  // that one or the next; the eight row addresses are read from their lanes
  // into scalar registers once per step (no lane exchange through LDS).
  // fp8 rows: a lane's 16 bytes are chunk e % 36 of the wavefront's row e / 36,
  // e = 64 i + l, for instruction i; the rows' scales are loaded by lanes 0..31
  // (returned, 0 for an empty slot) and stored with the converted rows.
  auto issue_copies = [&](int tok, uint8_t *buf) {
    int slot;
    const int64_t blk = cache_block(a.latent, seq, tok >= 0 ? tok : 0, slot);
    const uint8_t *rp = tok >= 0 ? cache_row(a.latent, blk, slot) : a.latent.rows;
    const uint64_t rp64 = reinterpret_cast<uint64_t>(rp);
    uint64_t row_addr[10];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      row_addr[k] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(rp64 >> 32), 8 * wave + k) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)rp64, 8 * wave + k);
    row_addr[8] = row_addr[9] = row_addr[7];   // (never selected: past the wavefront's last row)
    const int l = fresh_lane();
    if (F8) {
#pragma unroll
      for (int i = 0; i < kW4F8Copies; ++i) {
        const int e = 64 * i + l;
        const int k0 = (64 * i) / kW4F8Chunks;
        const int k = e / kW4F8Chunks, c = e - kW4F8Chunks * k;
        const uint64_t base = k == k0 ? row_addr[k0] : k == k0 + 1 ? row_addr[k0 + 1] : row_addr[k0 + 2];
        if (e < kW4F8WaveChunks)
          copy16_to_lds(reinterpret_cast<const uint8_t *>(base) + 16 * c,
                        buf + 8 * kW4RowB * wave + kW4F8Stage + 1024 * i);
      }
      return (tok >= 0 && lane < kW4Step) ? a.latent.scale[blk * a.latent.scale_block_stride + slot] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kW4PerThread; ++u) {
      const int k0 = (64 * u) / kW4Chunks, b0 = (64 * u) % kW4Chunks;
      const int t = b0 + l;
      const bool next = t >= kW4Chunks;
      const int slot_in_row = next ? t - kW4Chunks : t;
      const int h = next ? w4_swz(8 * wave + k0 + 1) : w4_swz(8 * wave + k0);
      const uint64_t base = next ? row_addr[k0 + 1] : row_addr[k0];
      const uint8_t *src = reinterpret_cast<const uint8_t *>(base) + 16 * (slot_in_row ^ h);
      copy16_to_lds(src, buf + 1024 * (kW4PerThread * wave + u));
    }
    return 0.0f;
  };
  // fp8 rows, after the wavefront's copies have landed: its eight rows are read
  // from the staging area into registers, then written as bf16 (exact) into the
  // swizzled image (empty rows as zeros); lanes 0..31 of wavefront 0 store the
  // step's row scales.
  auto convert_rows = [&](uint32_t valid, float rscale, uint8_t *buf) {
    const int l = fresh_lane();
    u32x4 raw[kW4F8Copies];
#pragma unroll
    for (int i = 0; i < kW4F8Copies; ++i)
      raw[i] = 64 * i + l < kW4F8WaveChunks
                   ? *reinterpret_cast<const u32x4 *>(buf + 8 * kW4RowB * wave + kW4F8Stage + 1024 * i + 16 * l)
                   : u32x4{0, 0, 0, 0};
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): every staging read done before the image is written
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < kW4F8Copies; ++i) {
      const int e = 64 * i + l;
      if (e < kW4F8WaveChunks) {
        const int k = e / kW4F8Chunks, c = e - kW4F8Chunks * k;
        const int r = 8 * wave + k;
        const bool ok = (valid >> r) & 1u;
        const u32x4 x = ok ? raw[i] : u32x4{0, 0, 0, 0};
        const int h = w4_swz(r);
        uint8_t *row = buf + kW4RowB * r;
        *reinterpret_cast<bf16x8 *>(row + 16 * ((2 * c) ^ h)) = fp8x8_to_bf16x8(x[0], x[1]);
        *reinterpret_cast<bf16x8 *>(row + 16 * ((2 * c + 1) ^ h)) = fp8x8_to_bf16x8(x[2], x[3]);
      }
    }
    if (wave == 0 && l < kW4Step) reinterpret_cast<float *>(buf + kW4ScaleOfs)[l] = rscale;
  };
  // After a wavefront's copies have landed: its entries of invalid rows become
  // zeros (their weight is 0, but 0 times a non-finite value would not be).
  auto clear_invalid = [&](uint32_t valid, uint8_t *buf) {
    const int l = fresh_lane();
#pragma unroll
    for (int u = 0; u < kW4PerThread; ++u)
      if (!((valid >> copy_row(u, l)) & 1u))
        *reinterpret_cast<u32x4 *>(buf + 1024 * (kW4PerThread * wave + u) + 16 * lane) = u32x4{0, 0, 0, 0};
  };

  // first step's copies, then q (head h0 + l16, dims 8 g4 + 32 ks + [0, 8))
  int tok = step_token(0);
  uint32_t valid = (uint32_t)__ballot(tok >= 0);
  float rs_first = 0.0f;
  if (nsteps > 0) rs_first = issue_copies(tok, w4lds);
  bf16x8 qa[kW / 32];
  {
    const uint16_t *qr = a.q + ((int64_t)qi * H + h0 + l16) * kW + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < kW / 32; ++ks) qa[ks] = as_bf16x8(load16(qr + 32 * ks));
  }
  int tok_next = step_token(1);
  wait_copies();
  if (F8) {
    if (nsteps > 0) convert_rows(valid, rs_first, w4lds);
  } else if (valid != 0xFFFFFFFFu) {
    clear_invalid(valid, w4lds);
  }
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.0f;   // head l16: reference maximum, this lane's partial sum
  f32x4 o[kL / 16];                        // column tile nt: heads 4 g4 + i, column 16 nt + l16
#pragma unroll
  for (int nt = 0; nt < kL / 16; ++nt) o[nt] = f32x4{0, 0, 0, 0};

  // per-lane LDS offsets (h(r + 16) = h(r)): QK reads rows 16 t + l16 at chunk
  // 4 ks + g4, slot 8 (ks >> 1) + ((4 (ks & 1) + g4) ^ h), by ks's parity; PV's
  // transposed reads take rows 4 g4 + l16 / 4 (+ 16) at columns 16 nt + 4 (l16 % 4),
  // chunk 2 nt + (l16 % 4) / 2, slot 8 (nt >> 2) + ((2 (nt & 3) + (l16 % 4) / 2) ^ h), by nt % 4
  // (formed in every step from the lane index: held across the loop they would
  // push a value out to scratch, and its reload would wait for the copies in flight)
  auto lds_offsets = [&](int (&qk_off)[2], int (&pv_off)[4]) {
    const int l = fresh_lane();
    const int lq = l & 15, gq = l >> 4;
    const int hq = w4_swz(lq);
#pragma unroll
    for (int par = 0; par < 2; ++par) qk_off[par] = kW4RowB * lq + 16 * ((4 * par + gq) ^ hq);
    const int pr = 4 * gq + (lq >> 2);
    const int hp = w4_swz(pr);
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4)
      pv_off[m4] = kW4RowB * pr + 16 * ((2 * m4 + ((lq & 3) >> 1)) ^ hp) + 8 * (lq & 1);
  };

  for (int st = 0; st < nsteps; ++st) {
    int qk_off[2], pv_off[4];
    lds_offsets(qk_off, pv_off);
    uint8_t *cur = w4lds + (st & 1) * kW4BufStride<F8>;
    uint8_t *nxt = w4lds + ((st + 1) & 1) * kW4BufStride<F8>;
    // next step's copies into the other buffer (read by no one since the barrier)
    const uint32_t valid_next = (uint32_t)__ballot(tok_next >= 0);
    const bool more = st + 1 < nsteps;
    float rs_next = 0.0f;
    if (more) rs_next = issue_copies(tok_next, nxt);
    const int tok_after = step_token(st + 2);

    // QK^T: D[row 16 t + 4 g4 + i][head l16].  The two row tiles alternate
    // (n = 2 ks + t) and each row operand is read kW4QkAhead MFMAs ahead; the
    // scheduling barriers keep the compiler from hoisting the reads further,
    // which would not fit the registers.
    f32x4 acc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
    {
      auto qk_read = [&](int n) {
        return as_bf16x8(*reinterpret_cast<const u32x4 *>(cur + kW4RowB * 16 * (n & 1) + qk_off[(n >> 1) & 1] +
                                                          128 * (n >> 2)));
      };
      bf16x8 ar[kW4QkAhead];
#pragma unroll
      for (int i = 0; i < kW4QkAhead; ++i) ar[i] = qk_read(i);
#pragma unroll
      for (int n = 0; n < 2 * (kW / 32); ++n) {
        const bf16x8 av = ar[n % kW4QkAhead];
        if (n + kW4QkAhead < 2 * (kW / 32)) ar[n % kW4QkAhead] = qk_read(n + kW4QkAhead);
        acc[n & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qa[n >> 1], acc[n & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // fp8 rows: the score of the decoded row is its scale times the product with
    // the stored bytes (row scales of rows 16 t + 4 g4 + i)
    f32x4 rsc[2] = {f32x4{1, 1, 1, 1}, f32x4{1, 1, 1, 1}};
    if (F8) {
#pragma unroll
      for (int t = 0; t < 2; ++t) rsc[t] = *reinterpret_cast<const f32x4 *>(cur + kW4ScaleOfs + 4 * (16 * t + 4 * g4));
    }
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t + 4 * g4 + i;
        z[t][i] = ((valid >> r) & 1u) ? (F8 ? acc[t][i] * rsc[t][i] : acc[t][i]) * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, z[t][i]);
      }
    mx = max_xor32(max_xor16(mx));
    // lazy reference maximum (kSlack)
    const bool grow = mx > m_run + kSlack;
    const float m_new = grow ? mx : m_run;
    const float mu = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = grow ? fast_exp2(m_run - mu) : 1.0f;
    m_run = m_new;
    float p[2][4];
    float ps = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t][i] = fast_exp2(z[t][i] - mu);
        ps += p[t][i];
      }
    l_run = l_run * alpha + ps;
    if (st > 0 && __ballot(grow)) {   // (before the first step o is 0)
      // o's lane holds heads 4 g4 + i: their factors come from lanes 4 g4 + i
      float ao[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ao[i] = __shfl(alpha, 4 * g4 + i, 64);
#pragma unroll
      for (int nt = 0; nt < kL / 16; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= ao[i];
    }
    // P as the PV A operand: k = 8 g4 + e is row 4 g4 + e (e < 4) or 16 + 4 g4 + e - 4;
    // fp8 rows weigh the stored bytes by P times the row scale
    if (F8) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[t][i] *= rsc[t][i];
    }
    uint32_t ph[4], pl[4];
    split_hi_lo(p[0][0], p[0][1], ph[0], pl[0]);
    split_hi_lo(p[0][2], p[0][3], ph[1], pl[1]);
    split_hi_lo(p[1][0], p[1][1], ph[2], pl[2]);
    split_hi_lo(p[1][2], p[1][3], ph[3], pl[3]);
    const bf16x8 ahi = as_bf16x8(u32x4{ph[0], ph[1], ph[2], ph[3]});
    const bf16x8 alo = as_bf16x8(u32x4{pl[0], pl[1], pl[2], pl[3]});

    // PV: 32 column tiles, each V operand read kW4PvAhead - 1 tiles ahead
    {
      auto pv_read = [&](int nt) {
        const uint8_t *vb = cur + pv_off[nt & 3] + 128 * (nt >> 2);
        const i16x4 v0 = lds_read_tr(vb);
        const i16x4 v1 = lds_read_tr(vb + 16 * kW4RowB);
        return __builtin_bit_cast(bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){
                                              v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
      };
      bf16x8 vr[kW4PvAhead];
#pragma unroll
      for (int i = 0; i < kW4PvAhead; ++i) vr[i] = pv_read(i);
#pragma unroll
      for (int nt = 0; nt < kL / 16; ++nt) {
        const bf16x8 b = vr[nt % kW4PvAhead];
        if (nt + kW4PvAhead < kL / 16) vr[nt % kW4PvAhead] = pv_read(nt + kW4PvAhead);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, o[nt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // the next step's rows have landed (this wavefront's copies), invalid ones
    // cleared, and every wavefront is done with this buffer before it is refilled
    wait_copies();
    if (F8) {
      if (more) convert_rows(valid_next, rs_next, nxt);
    } else if (more && valid_next != 0xFFFFFFFFu) {
      clear_invalid(valid_next, nxt);
    }
    valid = valid_next;
    tok_next = tok_after;
    __syncthreads();
  }

  // epilogue: the head's sum over its 4 lanes; o's lane holds heads 4 g4 + i
  l_run = sum_xor32(sum_xor16(l_run));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * g4 + i;
    const float li = __shfl(l_run, hl, 64), mi = __shfl(m_run, hl, 64);
    const int head = h0 + hl;
    if (!SPLIT) {
      const float inv = li > 0.0f ? 1.0f / li : 0.0f;
      float *orow = a.out + ((int64_t)qi * H + head) * kL + l16;
#pragma unroll
      // (written once, read by a later kernel: non-temporal)
      for (int nt = 0; nt < kL / 16; ++nt) __builtin_nontemporal_store(o[nt][i] * inv, &orow[16 * nt]);
      if (l16 == 0 && a.lse) a.lse[(int64_t)qi * H + head] = li > 0.0f ? (mi + log2f(li)) * kLn2 : -INFINITY;
    } else {
      const int64_t base = ((int64_t)(qi * a.splits + sp) * H + head);
      float *orow = a.part_o + base * kL + l16;
#pragma unroll
      for (int nt = 0; nt < kL / 16; ++nt) orow[16 * nt] = o[nt][i];
      if (l16 == 0) {
        a.part_ml[base * 2 + 0] = mi;
        a.part_ml[base * 2 + 1] = li;
      }
    }
  }
}

// Combine split partials in split order.  One workgroup per (query, head), one
// thread per 4 output columns.  Every thread issues all of its loads at once
// (the splits' (max, sum) pairs and its 4 columns of every split; padding
// splits reload the last one and get weight 0), then forms the weights and the
// weighted sum in split order.
template <int NS>   // splits, rounded up to a multiple of 8
__global__ __launch_bounds__(128) void merge_kernel(float *__restrict__ out, float *__restrict__ lse,
                                                    const float *__restrict__ part_o,
                                                    const float *__restrict__ part_ml, int splits, int H) {
  const int qh = blockIdx.x;
  const int qi = qh / H, h = qh - qi * H;
  const int c = threadIdx.x * 4;
  f32x4 v[NS];
  float m[NS], l[NS];
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    const int s = sp < splits ? sp : splits - 1;
    const int64_t b = ((int64_t)qi * splits + s) * H + h;
    v[sp] = *reinterpret_cast<const f32x4 *>(part_o + b * kL + c);
    const auto x = *reinterpret_cast<const float2 *>(part_ml + b * 2);
    m[sp] = x.x;
    l[sp] = x.y;
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) M = sp < splits ? fmaxf(M, m[sp]) : M;
  float w[NS], Ls = 0.0f;
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    w[sp] = (sp < splits && M != -INFINITY) ? exp2f(m[sp] - M) : 0.0f;
    Ls = fmaf(w[sp], l[sp], Ls);
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    const float ws = w[sp] * inv;
    acc[0] = fmaf(ws, v[sp][0], acc[0]);
    acc[1] = fmaf(ws, v[sp][1], acc[1]);
    acc[2] = fmaf(ws, v[sp][2], acc[2]);
    acc[3] = fmaf(ws, v[sp][3], acc[3]);
  }
  *reinterpret_cast<f32x4 *>(out + (int64_t)qh * kL + c) = acc;
  if (threadIdx.x == 0 && lse) lse[qh] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
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
                                                         const int32_t *__restrict__ q_seq, int seq_per, int H,
                                                         float scale_log2) {
  __shared__ float lq[1024];
  __shared__ float lz[2048];
  __shared__ const float *lrow[2048];
  __shared__ float4 pv[256];
  __shared__ float sh[8];
  const int qi = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int W = latent.width;
  const int seq = attend_seq(q_seq, qi, seq_per);
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
      // 16-byte loads (W is a multiple of 4, rows 16-byte aligned), summed in column order
      const float4 *rp4 = reinterpret_cast<const float4 *>(rp);
      float dot = 0.0f;
#pragma unroll 4
      for (int c4 = 0; c4 < W / 4; ++c4) {
        const float4 r = rp4[c4];
        dot = fmaf(lq[4 * c4], r.x, dot);
        dot = fmaf(lq[4 * c4 + 1], r.y, dot);
        dot = fmaf(lq[4 * c4 + 2], r.z, dot);
        dot = fmaf(lq[4 * c4 + 3], r.w, dot);
      }
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
  // PV: thread (jg, cg) sums columns c0 + 4 cg .. + 3 (one 16-byte load per
  // row) over the slots j = jg (mod JG), four slots per round with their loads
  // issued together; the JG partial sums are added in jg order through LDS.
  // CG = the smallest power of two >= kv_lora / 4, at most 64; JG = 256 / CG.
  int CG = 1;
  while (CG < 64 && 4 * CG < kv_lora) CG *= 2;
  const int JG = 256 / CG;
  const int cg = threadIdx.x & (CG - 1), jg = threadIdx.x / CG;
  for (int c0 = 0; c0 < kv_lora; c0 += 4 * CG) {
    const int c = c0 + 4 * cg;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (c < kv_lora) {
      const float4 zero = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      int j = jg;
      for (; j + 3 * JG < k; j += 4 * JG) {
        const float *r[4] = {lrow[j], lrow[j + JG], lrow[j + 2 * JG], lrow[j + 3 * JG]};
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = r[u] ? *reinterpret_cast<const float4 *>(r[u] + c) : zero;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float pz = lz[j + u * JG];
          acc.x = fmaf(pz, v[u].x, acc.x);
          acc.y = fmaf(pz, v[u].y, acc.y);
          acc.z = fmaf(pz, v[u].z, acc.z);
          acc.w = fmaf(pz, v[u].w, acc.w);
        }
      }
      for (; j < k; j += JG) {
        const float *r = lrow[j];
        if (r) {
          const float4 v = *reinterpret_cast<const float4 *>(r + c);
          const float pz = lz[j];
          acc.x = fmaf(pz, v.x, acc.x);
          acc.y = fmaf(pz, v.y, acc.y);
          acc.z = fmaf(pz, v.z, acc.z);
          acc.w = fmaf(pz, v.w, acc.w);
        }
      }
    }
    pv[threadIdx.x] = acc;
    __syncthreads();
    if (jg == 0 && c < kv_lora) {
      float4 t = pv[cg];
      for (int g = 1; g < JG; ++g) {
        const float4 u = pv[g * CG + cg];
        t.x += u.x;
        t.y += u.y;
        t.z += u.z;
        t.w += u.w;
      }
      float *o = out + ((int64_t)qi * H + h) * kv_lora + c;
      o[0] = t.x * inv;
      o[1] = t.y * inv;
      o[2] = t.z * inv;
      o[3] = t.w * inv;
    }
    __syncthreads();
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
  p.wide = 0;
  p.rows_per_split = (k + kStepRows - 1) / kStepRows * kStepRows;
  if (dtype == kBF16 && n_heads % kWideHeads == 0 && n_q * (n_heads / kWideHeads) >= kWideMinRows) {
    // one workgroup per (query, 64 heads, split): ~256 workgroups, whole 64-row steps
    p.wide = 1;
    const int n_hb = n_heads / kWideHeads;
    const int steps = (k + kWideStep - 1) / kWideStep;
    int s = (kAttTargetWGs + n_q * n_hb - 1) / (n_q * n_hb);
    if (s > steps) s = steps;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < 1) s = 1;
    const int sps = (steps + s - 1) / s;
    p.rows_per_split = sps * kWideStep;
    p.splits = (steps + sps - 1) / sps;
  } else if (dtype == kBF16 && n_heads >= kHG) {
    const int n_hg = n_heads / kHG;
    const int steps = (k + kStepRows - 1) / kStepRows;
    // ~256 workgroups; each split is a whole number of 128-row steps
    int s = (kAttTargetWGs + n_q * n_hg - 1) / (n_q * n_hg);
    if (s > steps) s = steps;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < 1) s = 1;
    const int sps = (steps + s - 1) / s;
    p.rows_per_split = sps * kStepRows;
    p.splits = (steps + sps - 1) / sps;
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
                         const int32_t *indices, int k, const int32_t *q_seq, int seq_per, int n_q, int n_heads,
                         float scale, const AttendPlan &plan, void *workspace, hipStream_t stream) {
  if (dt == kF32) {
    hipLaunchKernelGGL(attend_f32_kernel, dim3(n_q * n_heads), dim3(256), 0, stream, out, lse,
                       static_cast<const float *>(q), latent, kv_lora, indices, k, q_seq, seq_per, n_heads,
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
  a.seq_per = seq_per;
  a.k = k;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.splits = plan.splits;
  a.rows_per_split = plan.rows_per_split;
  a.n_hg = n_heads / kHG;
  a.pairs = n_q * plan.splits;
  a.scale_log2 = scale * kLog2e;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  if (plan.wide) {
    // the 64-head kernel takes 72 KB of dynamic LDS: allowed once per device (the current one)
    static std::atomic<uint64_t> lds_set{0};
    int dev = 0;
    hipError_t de = hipGetDevice(&dev);
    if (de != hipSuccess) return de;
    const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
    if (!bit || !(lds_set.load(std::memory_order_acquire) & bit)) {
      const std::pair<const void *, size_t> fs[] = {
          {reinterpret_cast<const void *>(&attend_w4_kernel<true, false>), kW4LdsBytes<false>},
          {reinterpret_cast<const void *>(&attend_w4_kernel<false, false>), kW4LdsBytes<false>},
          {reinterpret_cast<const void *>(&attend_w4_kernel<true, true>), kW4LdsBytes<true>},
          {reinterpret_cast<const void *>(&attend_w4_kernel<false, true>), kW4LdsBytes<true>}};
      for (const auto &f : fs) {
        de = hipFuncSetAttribute(f.first, hipFuncAttributeMaxDynamicSharedMemorySize, (int)f.second);
        if (de != hipSuccess) return de;
      }
      lds_set.fetch_or(bit, std::memory_order_acq_rel);
    }
  }
  const int groups = (a.pairs + 7) / 8;
  const dim3 grid(groups * 8 * a.n_hg);
  const dim3 wide_grid(n_q * (n_heads / kWideHeads) * plan.splits);
  const bool f8 = dt == kFP8;
#define DSA_ATTEND(SP)                                                                                        \
  do {                                                                                                        \
    if (plan.wide) {                                                                                          \
      if (f8) hipLaunchKernelGGL((attend_w4_kernel<SP, true>), wide_grid, dim3(kW4Threads), kW4LdsBytes<true>,   \
                                 stream, a);                                                                  \
      else hipLaunchKernelGGL((attend_w4_kernel<SP, false>), wide_grid, dim3(kW4Threads), kW4LdsBytes<false>,   \
                              stream, a);                                                                     \
    } else {                                                                                                  \
      if (f8) hipLaunchKernelGGL((attend_bf16_kernel<SP, true>), grid, dim3(kAttThreads), 0, stream, a);       \
      else hipLaunchKernelGGL((attend_bf16_kernel<SP, false>), grid, dim3(kAttThreads), 0, stream, a);         \
    }                                                                                                         \
  } while (0)
  if (plan.splits > 1) {
    a.part_o = reinterpret_cast<float *>(ws + plan.off_part_o);
    a.part_ml = reinterpret_cast<float *>(ws + plan.off_part_ml);
    DSA_ATTEND(true);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
#define DSA_MERGE(NS)                                                                                         \
  hipLaunchKernelGGL(merge_kernel<NS>, dim3(n_q * n_heads), dim3(kL / 4), 0, stream, out, lse, a.part_o, a.part_ml, \
                     plan.splits, n_heads)
    if (plan.splits <= 8) DSA_MERGE(8);
    else if (plan.splits <= 16) DSA_MERGE(16);
    else if (plan.splits <= 24) DSA_MERGE(24);
    else DSA_MERGE(32);
#undef DSA_MERGE
  } else {
    DSA_ATTEND(false);
  }
#undef DSA_ATTEND
  return hipGetLastError();
}

__global__ void fill_zero_kernel(uint32_t *p, size_t words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void window_rows_kernel(const int32_t *__restrict__ seq_len, int batch, int window,
                                   int32_t *__restrict__ q_seq, int32_t *__restrict__ q_len) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch * window) return;
  const int b = i / window, j = i - b * window;
  const int n = seq_len[b] - window + j + 1;
  q_seq[i] = b;
  q_len[i] = n > 0 ? n : 0;
}

hipError_t launch_window_rows(const int32_t *seq_len, int batch, int window, int32_t *q_seq, int32_t *q_len,
                              hipStream_t stream) {
  const int n = batch * window;
  hipLaunchKernelGGL(window_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, seq_len, batch, window, q_seq,
                     q_len);
  return hipGetLastError();
}

hipError_t launch_fill_zero(uint32_t *p, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, words);
  return hipGetLastError();
}

}  // namespace dsa
