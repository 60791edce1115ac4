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
  const int lin = blockIdx.x;
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
#pragma unroll
      for (int r = 0; r < kTeams; ++r)
        if (!ok[r])
#pragma unroll
          for (int i = 0; i < NV8; ++i) w[r][i] = u32x4{0, 0, 0, 0};
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

    // QK^T: this wavefront's 16 rows of its team's tile
    const int row = tw * 16 + l16;
    f32x4 sacc = {0, 0, 0, 0};
    {
      const uint8_t *rp = my_rows + row * kRowBytes + 16 * g4;
#pragma unroll
      for (int ks = 0; ks < kW / 32; ++ks) {
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4 *>(rp + 64 * ks));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], b, sacc, 0, 0, 0);
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

    float m_new[4], alpha[4], ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
      const float tm =
          fmaxf(fmaxf(red[team][0][0][h], red[team][0][1][h]), fmaxf(red[team][0][2][h], red[team][0][3][h]));
      m_new[i] = fmaxf(m_run[i], tm);
      const float mu = m_new[i] == -INFINITY ? 0.0f : m_new[i];
      alpha[i] = exp2f(m_run[i] - mu);
      const float p = exp2f(z[i] - mu);
      const float pv = F8 ? p * rs : p;       // weight of the decoded (unscaled) row
      const uint16_t hi = float_to_bf16_bits(pv);
      const uint16_t lo = float_to_bf16_bits(pv - bf16_bits_to_float(hi));
      my_p[h * kTile + row] = hi;
      my_p[kHG * kTile + h * kTile + row] = lo;
      ps[i] = row16_sum(p);
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
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const i16x4 v0 = lds_read_tr(vb + 32 * nt);
        const i16x4 v1 = lds_read_tr(vb + 4 * kRowBytes + 32 * nt);
        const bf16x8 b = __builtin_bit_cast(
            bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){v0[0], v0[1], v0[2], v0[3], v1[0],
                                                                                 v1[1], v1[2], v1[3]});
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, o[nt], 0, 0, 0);
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
    const float a0 = exp2f(m_run[i] - mu), a1 = exp2f(m1 - mu);
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
// of 64 heads and a split of the index slots, so each kept row is gathered
// once for all 64 heads (the 16-head kernel above spreads few queries over
// more workgroups, at the price of gathering every row once per head group).
// Per 64-slot step the rows sit in LDS (8 threads per row, 128 contiguous
// bytes per load); wavefront w takes head group w / 2 (16 heads) and half
// w % 2 of the rows for QK^T and of the 512 value columns for PV.  The next
// step's rows are loaded into registers while a step is computed.
constexpr int kWideHeads = 64;
constexpr int kWideStep = 64;
constexpr int kWideThreads = 512;
constexpr int kWidePer = kW * 2 / 16 / 8;   // 16-byte chunks per thread and row (9)

template <bool SPLIT, bool F8>
__global__ __launch_bounds__(kWideThreads) void attend_wide_kernel(AttArgs a) {
  __shared__ __align__(16) uint8_t rows[kWideStep * kRowBytes];
  __shared__ __align__(16) uint16_t lp[4][2][kHG * kWideStep];   // per head group: P hi / lo, [head][row]
  __shared__ float red[4][2][2][kHG];                             // [head group][max | sum][row half][head]
  __shared__ uint8_t lvalid[kWideStep];
  __shared__ float lscale[F8 ? kWideStep : 1];

  const int H = a.n_heads;
  const int n_hb = H / kWideHeads;
  const int wg = blockIdx.x;
  const int qi = wg / (a.splits * n_hb);
  const int rem = wg - qi * a.splits * n_hb;
  const int hb = rem / a.splits, sp = rem - (rem / a.splits) * a.splits;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave >> 1, wr = wave & 1;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int h0 = hb * kWideHeads + hg * kHG;
  const int seq = attend_seq(a.q_seq, qi, a.seq_per);
  const int j0 = sp * a.rows_per_split;
  const int j1 = min(j0 + a.rows_per_split, a.k);
  const int nsteps = (j1 - j0 + kWideStep - 1) / kWideStep;

  // gather role: row gr of a step, chunks gq + 8 i (i < 9), 128 contiguous bytes per load
  // (fp8 rows: 36 chunks, i < 5, the last only for gq < 4)
  const int gr = tid >> 3, gq = tid & 7;
  constexpr int NV = F8 ? 5 : kWidePer;
  u32x4 v[NV];
  float v_sc = 0.0f;
  bool v_ok;
  auto load_rows = [&](int step) {
    const int j = j0 + step * kWideStep + gr;
    const int raw = a.indices[(int64_t)qi * a.k + (j < a.k ? j : a.k - 1)];
    const int t = j < j1 ? raw : -1;
    v_ok = t >= 0;
    int slot;
    const int64_t blk = cache_block(a.latent, seq, v_ok ? t : 0, slot);
    const uint8_t *src = v_ok ? cache_row(a.latent, blk, slot) : a.latent.rows;
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = load16(src + (F8 ? min(16 * gq + 128 * i, kW - 16) : 16 * gq + 128 * i));
    if (F8) v_sc = v_ok ? a.latent.scale[blk * a.latent.scale_block_stride + slot] : 0.0f;
  };
  load_rows(0);

  // q operand (head h0 + l16, dims 32 ks + 8 g4 + [0, 8))
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
  constexpr int NT = kL / 2 / 16;   // 16 value-column tiles per wavefront
  f32x4 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0, 0, 0, 0};
  uint16_t *my_p = lp[hg][0];

  for (int step = 0; step < nsteps; ++step) {
    {
      if (F8) {
        // fp8 chunk gq + 8 i -> 16 bf16 at LDS bytes 32 (gq + 8 i) ..
        // an empty slot (the cache's first row was loaded) is written as zeros:
        // its P is 0, but 0 times a non-finite value would not be
        uint8_t *dst = rows + gr * kRowBytes + 32 * gq;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          if (i < NV - 1 || gq < 4) {
            const u32x4 x = v_ok ? v[i] : u32x4{0, 0, 0, 0};
            *reinterpret_cast<bf16x8 *>(dst + 256 * i) = fp8x8_to_bf16x8(x[0], x[1]);
            *reinterpret_cast<bf16x8 *>(dst + 256 * i + 16) = fp8x8_to_bf16x8(x[2], x[3]);
          }
        }
        if (gq == 0) lscale[gr] = v_sc;
      } else {
        uint8_t *dst = rows + gr * kRowBytes + 16 * gq;
#pragma unroll
        for (int i = 0; i < NV; ++i) *reinterpret_cast<u32x4 *>(dst + 128 * i) = v_ok ? v[i] : u32x4{0, 0, 0, 0};
      }
      if (gq == 0) lvalid[gr] = v_ok ? 1 : 0;
    }
    __syncthreads();
    load_rows(step + 1);   // past the split's end: empty slots (the cache's first row, unused)

    // QK^T: 16 heads x rows 32 wr + 16 nt + l16
    float z[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = 32 * wr + 16 * nt + l16;
      const uint8_t *rp = rows + row * kRowBytes + 16 * g4;
      f32x4 sacc = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < kW / 32; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            qa[ks], as_bf16x8(*reinterpret_cast<const u32x4 *>(rp + 64 * ks)), sacc, 0, 0, 0);
      const bool valid = lvalid[row] != 0;
      const float rs = F8 ? lscale[row] : 1.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) z[nt][i] = valid ? (F8 ? sacc[i] * rs : sacc[i]) * a.scale_log2 : -INFINITY;
    }
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = row16_max(fmaxf(z[0][i], z[1][i]));
    if (l16 == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[hg][0][wr][4 * g4 + i] = mx[i];
    __syncthreads();

    float alpha[4], ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
      const float tm = fmaxf(red[hg][0][0][h], red[hg][0][1][h]);
      const float m_new = fmaxf(m_run[i], tm);
      const float mu = m_new == -INFINITY ? 0.0f : m_new;
      alpha[i] = exp2f(m_run[i] - mu);
      float pr[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = 32 * wr + 16 * nt + l16;
        const float p = exp2f(z[nt][i] - mu);
        const float pv = F8 ? p * lscale[row] : p;   // weight of the decoded (unscaled) row
        const uint16_t hi = float_to_bf16_bits(pv);
        const uint16_t lo = float_to_bf16_bits(pv - bf16_bits_to_float(hi));
        my_p[h * kWideStep + row] = hi;
        my_p[kHG * kWideStep + h * kWideStep + row] = lo;
        pr[nt] = p;
      }
      ps[i] = row16_sum(pr[0]) + row16_sum(pr[1]);
      m_run[i] = m_new;
    }
    if (l16 == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[hg][1][wr][4 * g4 + i] = ps[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
      l_run[i] = l_run[i] * alpha[i] + (red[hg][1][0][h] + red[hg][1][1][h]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nt][i] *= alpha[i];

    // PV: rows 32 ks2 + 8 g4 + e, columns 256 wr + 16 nt + l16; the V operand
    // comes from two transposed LDS reads of 4 rows each
#pragma unroll
    for (int ks2 = 0; ks2 < kWideStep / 32; ++ks2) {
      const bf16x8 ahi = as_bf16x8(*reinterpret_cast<const u32x4 *>(&my_p[l16 * kWideStep + 32 * ks2 + 8 * g4]));
      const bf16x8 alo = as_bf16x8(
          *reinterpret_cast<const u32x4 *>(&my_p[kHG * kWideStep + l16 * kWideStep + 32 * ks2 + 8 * g4]));
      const uint8_t *vb = rows + (32 * ks2 + 8 * g4 + (l16 >> 2)) * kRowBytes + (256 * wr + 4 * (l16 & 3)) * 2;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const i16x4 v0 = lds_read_tr(vb + 32 * nt);
        const i16x4 v1 = lds_read_tr(vb + 4 * kRowBytes + 32 * nt);
        const bf16x8 b = __builtin_bit_cast(
            bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){v0[0], v0[1], v0[2], v0[3], v1[0],
                                                                                 v1[1], v1[2], v1[3]});
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, o[nt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds heads h0 + 4 g4 + i, columns 256 wr + 16 nt + l16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = h0 + 4 * g4 + i;
    if (!SPLIT) {
      const float inv = l_run[i] > 0.0f ? 1.0f / l_run[i] : 0.0f;
      float *orow = a.out + ((int64_t)qi * H + head) * kL + 256 * wr + l16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) orow[16 * nt] = o[nt][i] * inv;
      if (wr == 0 && l16 == 0 && a.lse)
        a.lse[(int64_t)qi * H + head] = l_run[i] > 0.0f ? (m_run[i] + log2f(l_run[i])) * kLn2 : -INFINITY;
    } else {
      const int64_t base = ((int64_t)(qi * a.splits + sp) * H + head);
      float *orow = a.part_o + base * kL + 256 * wr + l16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) orow[16 * nt] = o[nt][i];
      if (wr == 0 && l16 == 0) {
        a.part_ml[base * 2 + 0] = m_run[i];
        a.part_ml[base * 2 + 1] = l_run[i];
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
  const int groups = (a.pairs + 7) / 8;
  const dim3 grid(groups * 8 * a.n_hg);
  const dim3 wide_grid(n_q * (n_heads / kWideHeads) * plan.splits);
  const bool f8 = dt == kFP8;
#define DSA_ATTEND(SP)                                                                                        \
  do {                                                                                                        \
    if (plan.wide) {                                                                                          \
      if (f8) hipLaunchKernelGGL((attend_wide_kernel<SP, true>), wide_grid, dim3(kWideThreads), 0, stream, a); \
      else hipLaunchKernelGGL((attend_wide_kernel<SP, false>), wide_grid, dim3(kWideThreads), 0, stream, a);   \
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
