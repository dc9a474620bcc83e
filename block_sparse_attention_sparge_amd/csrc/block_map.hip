// Stage 1 of SpargeAttn-style block-sparse attention on gfx950: the block map.
//
// "Sparge Attention (Composable Kernel)" page, "Status vs Upstream": per-block
// mean pool, cosine similarity, pooled QK, top-k / cdfthreshd selection into a
// BlockMap LUT, with per-head topk / simthreshd1 / cdfthreshd.  The same page
// lists sort-based top-k as the replacement for an O(nk^2) argmax that hurts
// at long sequences.  Here the top-k count needs no full sort: the n-th
// largest probability is found by a radix select on its bits (four rounds of
// 8-bit histograms), and ties at it go to the lower block index; the cdf rule
// needs the order itself and sorts each row with a bitonic network held in
// the registers of one wavefront.
//
// Two kernels:
//   pool_sim     one wavefront per 64-token block of Q or K: reads the block
//                once (HBM bound), writes its fp32 mean and the gate flag
//                (mean pairwise cosine of the block's tokens > simthreshd1).
//   score_select one workgroup per 16 Q-tiles of one (b, h): pooled scores
//                against every K block mean with fp32 MFMA fed straight from
//                memory, fp32 softmax, then the selection in the order
//                (probability descending, block index ascending), the four
//                rows of each wavefront interleaved step by step:
//                top-k finds the n-th largest probability by a radix select
//                on its bits and takes ties at it by ascending index; cdf
//                needs the order itself and sorts the row with a 64-bit-key
//                bitonic network.  The ascending LUT is written by a prefix
//                scan (no atomic slot assignment, so the output is
//                deterministic).
#include "common.h"
#include "kernels.h"

namespace sparge {

// ---------------------------------------------------------------------------
// key_mean: partial sums of K over the sequence (K smoothing)
// ---------------------------------------------------------------------------
// CK page, not-yet-ported list: K smoothing subtracts km = mean_s(k) before
// pooling.  One workgroup sums kKmChunkRows consecutive K rows of one (b, h);
// pool_sim adds the chunks in a fixed order, so km is deterministic.
template <class E, int D>
__global__ __launch_bounds__(256) void key_mean_kernel(PoolArgs a) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int RPP = 256 / CH;      // rows per pass
  __shared__ float s_part[RPP][D];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / a.km_chunks;
  const int chunk = (int)(blockIdx.x % a.km_chunks);
  const int hh = (int)(bh % a.h_kv), bb = (int)(bh / a.h_kv);
  const int r0 = chunk * kKmChunkRows;
  const int rows = min(kKmChunkRows, a.sk - r0);
  const int c = tid % CH, rsub = tid / CH;
  const typename E::T* base = reinterpret_cast<const typename E::T*>(a.k) + bb * a.ks[0] + hh * a.ks[1] + c * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll 8
  for (int r = rsub; r < rows; r += RPP) {
    const u32x4 w = load16(base + (int64_t)(r0 + r) * a.ks[2]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += E::lo(w[j]);
      acc[2 * j + 1] += E::hi(w[j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s_part[rsub][c * 8 + i] = acc[i];
  __syncthreads();
  for (int dd = tid; dd < D; dd += 256) {
    float sum = 0.f;
    for (int j = 0; j < RPP; ++j) sum += s_part[j][dd];
    a.km_part[(bh * a.km_chunks + chunk) * D + dd] = sum;
  }
}

// ---------------------------------------------------------------------------
// pool_sim
// ---------------------------------------------------------------------------
// A sequence whose length is not a multiple of 64 ends in a partial block: it
// loads only its own tokens, and its mean and mean pairwise cosine divide by
// its token count (for a full block, by the exact powers of two 64 and 4096).
template <class E, int D, bool SMOOTH, bool QUANT>
__global__ __launch_bounds__(256) void pool_sim_kernel(PoolArgs a) {
  constexpr int CH = D / 8;          // 16-byte chunks per token
  constexpr int TPP = kWave / CH;    // tokens per pass of the wave
  constexpr int NP = 64 / TPP;       // passes over the 64-token block
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nqb = (int64_t)a.b * a.h * a.nq;
  const int64_t total = nqb + (int64_t)a.b * a.h_kv * a.nk;
  if (gw >= total) return;

  const bool is_k = gw >= nqb;
  const int64_t idx = is_k ? gw - nqb : gw;
  const int nb = is_k ? a.nk : a.nq;
  const int64_t bh = idx / nb;            // (b, head) over the Q heads or the K heads
  const int blk = (int)(idx % nb);
  const int nh = is_k ? a.h_kv : a.h;
  const int hh = (int)(bh % nh);
  const int bb = (int)(bh / nh);
  const int64_t* st = is_k ? a.ks : a.qs;
  const typename E::T* base = reinterpret_cast<const typename E::T*>(is_k ? a.k : a.q);
  const int ntok = is_k ? a.sk : a.sq;
  const int cnt = min(64, ntok - blk * 64);   // tokens in this block

  const int c = lane % CH;
  const int t0 = lane / CH;
  const typename E::T* p0 = base + bb * st[0] + hh * st[1] + (int64_t)(blk * 64 + t0) * st[2] + c * 8;

  u32x4 raw[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    raw[p] = u32x4{0u, 0u, 0u, 0u};
    if (p * TPP + t0 < cnt) raw[p] = load16(p0 + (int64_t)(p * TPP) * st[2]);
  }

  // K smoothing: this lane's 8 entries of km (zero when not smoothing).
  float kmv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) kmv[i] = 0.f;
  if (SMOOTH && is_k) {
    const float* kp = a.km_part + bh * a.km_chunks * D + c * 8;
    for (int ch = 0; ch < a.km_chunks; ++ch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) kmv[i] += kp[(int64_t)ch * D + i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) kmv[i] *= a.km_scale;
  }

  float sx[8], sh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { sx[i] = 0.f; sh[i] = 0.f; }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float x[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = E::lo(raw[p][w]) - kmv[2 * w];
      x[2 * w + 1] = E::hi(raw[p][w]) - kmv[2 * w + 1];
    }
    if (SMOOTH && p * TPP + t0 >= cnt) {   // a missing token of a partial block
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    float n2 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) n2 = fmaf(x[i], x[i], n2);
    if constexpr (CH == 16) n2 = row16_sum(n2);
    else n2 = row8_sum(n2);
    const float inv = n2 > 0.f ? __builtin_amdgcn_rsqf(n2) : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sx[i] += x[i];
      sh[i] = fmaf(x[i], inv, sh[i]);
    }
  }
  // Sum over the tokens held by lanes that share the chunk index.
#pragma unroll
  for (int m = CH; m < kWave; m <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sx[i] += __shfl_xor(sx[i], m, kWave);
      sh[i] += __shfl_xor(sh[i], m, kWave);
    }
  }
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) dot = fmaf(sh[i], sh[i], dot);
  if constexpr (CH == 16) dot = row16_sum(dot);
  else dot = row8_sum(dot);

  float* mean = (is_k ? a.k_mean : a.q_mean) + (bh * nb + blk) * D;
  if (t0 == 0) {
    const float r = 1.0f / (float)cnt;
    floatx4 m0 = {sx[0] * r, sx[1] * r, sx[2] * r, sx[3] * r};
    floatx4 m1 = {sx[4] * r, sx[5] * r, sx[6] * r, sx[7] * r};
    *reinterpret_cast<floatx4*>(mean + c * 8) = m0;
    *reinterpret_cast<floatx4*>(mean + c * 8 + 4) = m1;
  }
  if (lane == 0) {
    // Q blocks are gated here; a K block's similarity is kept for the query
    // heads that read it, each with its own threshold.
    const float sim = dot * (1.0f / (float)(cnt * cnt));
    if (is_k) a.k_sim[bh * nb + blk] = sim;
    else a.sim_q[bh * nb + blk] = sim > a.thr[hh] ? 1 : 0;
  }

  if constexpr (QUANT) {
    // int8 codes of the block as given (not smoothed): scale = absmax / 127,
    // code = round-half-even(x * (127 / absmax)), both divisions correctly
    // rounded in fp32; an all-zero block gets scale 0 and codes 0.  With
    // quant_fp8 the codes are OCP fp8 e4m3 instead: scale = absmax / 448 and
    // code = x * (448 / absmax) rounded to the e4m3 grid, to nearest even
    // (v_cvt_pk_fp8_f32; its inputs stay within 448 * (1 + 2^-23), which
    // rounds to 448).
    // Convert again below rather than keep the 8 NP floats of the statistics
    // loop alive (the compiler would otherwise reuse them).
#pragma unroll
    for (int p = 0; p < NP; ++p) asm volatile("" : "+v"(raw[p]));
    // The absolute maximum is taken on the 16-bit patterns: with the sign
    // cleared they order like the values (inputs are finite).
    uint32_t amax_bits = 0;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        amax_bits = max(amax_bits, max(raw[p][w] & 0x7FFFu, (raw[p][w] >> 16) & 0x7FFFu));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, m, kWave));
    const float amax = E::lo(amax_bits);
    const bool fp8 = a.quant_fp8 != 0;
    const float qmax = fp8 ? 448.0f : 127.0f;
    const float inv = amax > 0.f ? qmax / amax : 0.f;
    int8_t* codes = (is_k ? a.k_i8 : a.q_i8) + (bh * ntok + blk * 64 + t0) * (int64_t)D + c * 8;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint32_t wd[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t acc = 0;
        if (fp8) {
          // Element j of the four goes to byte j: bytes 0-1 from the low
          // word of the conversion, bytes 2-3 from the high word.
          const uint32_t w0 = raw[p][2 * half], w1 = raw[p][2 * half + 1];
          acc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(E::lo(w0) * inv, E::hi(w0) * inv, 0, false);
          acc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(E::lo(w1) * inv, E::hi(w1) * inv, (int)acc, true);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t wv = raw[p][2 * half + j / 2];
            const float x = (j & 1) ? E::hi(wv) : E::lo(wv);
            const float t = fminf(fmaxf(rintf(x * inv), -127.f), 127.f);
            acc |= ((uint32_t)(int)t & 0xFFu) << (8 * j);
          }
        }
        wd[half] = acc;
      }
      if (p * TPP + t0 < cnt) *reinterpret_cast<u32x2*>(codes + (int64_t)(p * TPP) * D) = u32x2{wd[0], wd[1]};
    }
    if (lane == 0) (is_k ? a.k_i8_scale : a.q_i8_scale)[bh * nb + blk] = amax / qmax;
  }
}

// ---------------------------------------------------------------------------
// score_select
// ---------------------------------------------------------------------------
constexpr int kSelRows = 16;   // Q-tiles per workgroup (4 per wavefront)

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Sort the wave's 64*KPL keys into descending order; lane L holds elements
// L*KPL .. L*KPL+KPL-1 in key[0..KPL).
template <int KPL>
__device__ __forceinline__ void bitonic_desc(uint64_t (&key)[KPL], int lane) {
  constexpr int N = 64 * KPL;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj >= KPL) {
        const int lm = jj / KPL;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int e = lane * KPL + j;
          const uint64_t other = shfl_xor_u64(key[j], lm);
          const bool lower = (e & jj) == 0;
          const bool desc = (e & k) == 0;
          const bool take_max = lower == desc;
          const uint64_t mx = key[j] > other ? key[j] : other;
          const uint64_t mn = key[j] > other ? other : key[j];
          key[j] = take_max ? mx : mn;
        }
      } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          if ((j & jj) != 0) continue;
          const int e = lane * KPL + j;
          const bool desc = (e & k) == 0;
          const uint64_t x = key[j], y = key[j | jj];
          const bool swap = desc ? (x < y) : (x > y);
          key[j] = swap ? y : x;
          key[j | jj] = swap ? x : y;
        }
      }
    }
  }
}

template <int D, int KPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void score_select_kernel(SelectArgs a) {
  constexpr int NKP = 64 * KPL;
  constexpr int SP = NKP + 4;            // padded pitch of a score row (floats)
  constexpr int NG = D / 16;             // 16-wide slices of the head dimension
  static_assert(kSelRows == 16, "one 16-row MFMA tile per group");
  __shared__ __attribute__((aligned(16))) float s_score[kSelRows][SP];
  __shared__ uint8_t s_sel[kSelRows][NKP];
  __shared__ float s_sorted[4][NKP];
  // Radix-select histograms of rows too short to hold 256 bins in their own
  // s_score row (nk <= 128).
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[KPL < 4 ? kSelRows : 1][KPL < 4 ? 256 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int groups = (a.nq + kSelRows - 1) / kSelRows;
  // The groups of one (b, h) share its K means: keep them on one XCD's L2.
  const int64_t lin = xcd_remap(blockIdx.x, gridDim.x);
  if (lin >= (int64_t)a.b * a.h * groups) return;
  const int64_t bh = lin / groups;
  const int qb0 = (int)(lin % groups) * kSelRows;
  const int rows = min(kSelRows, a.nq - qb0);
  const int hh = (int)(bh % a.h);
  const int64_t bkv = (bh / a.h) * a.h_kv + hh / (a.h / a.h_kv);   // the K head query head hh reads
  const int nk = a.nk;
  const float thr = a.thr[hh];

  // Pooled scores with fp32 MFMA (16x16x4: exact products, fp32 sums).  The
  // contraction over the head dimension may visit it in any order as long as
  // both operands agree, so lane (m16, k4) feeds, at step t of slice g,
  // element d = 16g + 4k4 + t: each operand is then one 16-byte load per
  // slice, straight from memory into registers.  Wave w computes the columns
  // 64c + 16w .. +15 of the 16 x nk score tile.
  //
  // Every load below is unconditional: indices past the end are clamped to
  // the last row or block, whose finite copies are then masked or never
  // written.  A load under a branch would make the compiler wait for it at
  // the join, and so would the copy of a prefetched operand into the
  // registers the MFMAs read; the column chunks therefore alternate between
  // two operand sets, and chunk c+1's means load during chunk c's MFMAs.
  const int m16 = lane & 15, k4 = lane >> 4;
  floatx4 qf[NG];
  {
    const float* qrow = a.q_mean + (bh * a.nq + qb0 + min(m16, rows - 1)) * D + 4 * k4;
#pragma unroll
    for (int g = 0; g < NG; ++g) qf[g] = *reinterpret_cast<const floatx4*>(qrow + 16 * g);
  }
  const float* km = a.k_mean + bkv * nk * D;
  const float* ksim = a.k_sim + bkv * nk;
  auto ksim_at = [&](int kb) { return ksim[min(kb, nk - 1)]; };
  // Chunk c's operand: the means of K blocks 64c + 16 wave + m16 and the gate
  // value of the column this lane scores.
  auto load_k = [&](floatx4 (&kf)[NG], float& ks, int c) {
    const int kb = min(64 * c + 16 * wave + m16, nk - 1);
    const float* krow = km + (int64_t)kb * D + 4 * k4;
#pragma unroll
    for (int g = 0; g < NG; ++g) kf[g] = *reinterpret_cast<const floatx4*>(krow + 16 * g);
    ks = ksim[kb];
  };
  auto score_chunk = [&](const floatx4 (&kf)[NG], float ks, int c) {
    const int kb = 64 * c + 16 * wave + m16;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[g][t], kf[g][t], acc, 0, 0, 0);
    }
    // C: lane holds column kb for rows 4*k4 .. 4*k4+3.  Causal: block kb is
    // in the future of Q-tile qb0 + row when kb > qb0 + row.
    const bool live = kb < nk && ks > thr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = live && (!a.causal || kb <= qb0 + 4 * k4 + i);
      s_score[4 * k4 + i][kb] = ok ? acc[i] * a.scale : -INFINITY;
    }
  };
  // The scheduling barriers keep each chunk's loads issued ahead of the
  // MFMAs of the chunk before it (left alone, the scheduler sinks them to
  // their first use).
  floatx4 k0[NG], k1[NG];
  float ks0, ks1;
  load_k(k0, ks0, 0);
#pragma unroll
  for (int c = 0; c < KPL; c += 2) {
    if (c + 1 < KPL) load_k(k1, ks1, c + 1);
    __builtin_amdgcn_sched_barrier(0);
    score_chunk(k0, ks0, c);
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < KPL) {
      if (c + 2 < KPL) load_k(k0, ks0, c + 2);
      __builtin_amdgcn_sched_barrier(0);
      score_chunk(k1, ks1, c + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Inputs only the selection needs, requested now (they land during the
  // softmax): the K gate values of the row elements this lane selects and
  // the Q gate flag of row `lane`.
  float ksim_el[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) ksim_el[j] = ksim_at(lane * KPL + j);
  const uint8_t qflag_raw = a.sim_q[bh * a.nq + qb0 + min(lane, rows - 1)];
  __syncthreads();

  const int nsel_h = a.nsel[hh];
  const double cdf_h = (double)a.cdf[hh];
  constexpr int RW = kSelRows / 4;       // rows per wave: 4i + wave, i < RW
  bool valid[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) valid[j] = lane * KPL + j < nk;
  // Blocks a row may select: all nk, or kb <= qb when causal.  Future blocks
  // have probability 0 and a larger index than any allowed block, so the
  // first `limit` of the order are allowed ones.
  int limit[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) limit[i] = a.causal ? min(nk, qb0 + 4 * i + wave + 1) : nk;

  // The RW rows of a wave go through every step side by side, so that their
  // reduction and ballot chains overlap instead of running one after another.
  // Softmax of each pooled row (fp32).
  float p[RW][KPL];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int r = 4 * i + wave;          // rows past the end hold finite scores of zero Q rows
    const floatx4* src = reinterpret_cast<const floatx4*>(&s_score[r][lane * KPL]);
#pragma unroll
    for (int j4 = 0; j4 < KPL / 4 + (KPL < 4); ++j4) {
      const floatx4 v = src[j4];
#pragma unroll
      for (int t = 0; t < 4 && 4 * j4 + t < KPL; ++t) p[i][4 * j4 + t] = valid[4 * j4 + t] ? v[t] : -INFINITY;
    }
  }
  float mx[RW], sum[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    mx[i] = p[i][0];
#pragma unroll
    for (int j = 1; j < KPL; ++j) mx[i] = fmaxf(mx[i], p[i][j]);
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) mx[i] = wave_max_dpp(mx[i]);
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    sum[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      p[i][j] = mx[i] == -INFINITY ? 0.f : expf(p[i][j] - mx[i]);
      sum[i] += p[i][j];
    }
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) sum[i] = wave_sum_dpp(sum[i]);
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < KPL; ++j) p[i][j] = sum[i] > 0.f ? p[i][j] / sum[i] : 0.f;

  if (a.prob) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if (4 * i + wave >= rows) continue;
      const int64_t row = bh * a.nq + qb0 + 4 * i + wave;
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (valid[j]) a.prob[row * nk + lane * KPL + j] = p[i][j];
    }
  }

  // chosen[i][j]: element lane*KPL + j of row i is among the first n of the
  // order (probability descending, block index ascending).  Probabilities are
  // >= +0, so their bit patterns order like their values.
  bool chosen[RW][KPL];
  if (nsel_h > 0) {
    // top-k: T = the n-th largest probability (bits).  Probabilities are >= +0,
    // so their bit patterns order like their values.
    uint32_t thr_bits[RW];
    // Radix select from the most significant byte, four rounds: a histogram
    // of the next byte over the keys that share the bytes decided so far,
    // then a prefix count over the 256 bins, largest byte first, finds the
    // byte of the n-th largest and how many keys lie above it.  Each wave
    // keeps its rows' histograms in its own rows of s_score when 256 bins fit
    // there (nk > 128; in this mode the scores are in registers by now), in
    // s_hist otherwise, built with LDS atomics; bin 255 - byte, so lane l
    // holds the bins of bytes 255 - 4l .. 252 - 4l and the count from the top
    // is a prefix sum over the lanes (DPP row shifts and row broadcasts, no
    // LDS traffic).
    auto hist_row = [&](int i) -> uint32_t* {
      if constexpr (KPL >= 4) return reinterpret_cast<uint32_t*>(&s_score[4 * i + wave][0]);
      else return &s_hist[4 * i + wave][0];
    };
    uint32_t rank[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      thr_bits[i] = 0u;
      rank[i] = (uint32_t)min(nsel_h, limit[i]);
    }
#pragma unroll 1
    for (int rnd = 0; rnd < 4; ++rnd) {
      const int shift = 24 - 8 * rnd;
      const uint32_t pmask = rnd == 0 ? 0u : 0xFFFFFFFFu << (shift + 8);
#pragma unroll
      for (int i = 0; i < RW; ++i)
        reinterpret_cast<u32x4*>(hist_row(i))[lane] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        uint32_t* hist = hist_row(i);
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const uint32_t pb = __builtin_bit_cast(uint32_t, p[i][j]);
          if (valid[j] && (pb & pmask) == thr_bits[i]) atomicAdd(&hist[255u - ((pb >> shift) & 255u)], 1u);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const u32x4 h = reinterpret_cast<const u32x4*>(hist_row(i))[lane];
        const int lsum = (int)(h[0] + h[1] + h[2] + h[3]);
        const int pre = wave_prefix_sum_dpp(lsum);          // keys with byte >= 252 - 4 lane
        // The first lane whose prefix reaches the rank holds the byte.
        const int L = (int)__builtin_amdgcn_readfirstlane(
            (int)__builtin_ctzll(__ballot(pre >= (int)rank[i])));
        int cum = pre - lsum, byte = 0, above = 0;
        if (cum + (int)h[0] >= (int)rank[i]) {
          byte = 255 - 4 * lane;
          above = cum;
        } else if (cum + (int)(h[0] + h[1]) >= (int)rank[i]) {
          byte = 254 - 4 * lane;
          above = cum + (int)h[0];
        } else if (cum + (int)(h[0] + h[1] + h[2]) >= (int)rank[i]) {
          byte = 253 - 4 * lane;
          above = cum + (int)(h[0] + h[1]);
        } else {
          byte = 252 - 4 * lane;
          above = cum + (int)(h[0] + h[1] + h[2]);
        }
        thr_bits[i] |= (uint32_t)__builtin_amdgcn_readlane(byte, L) << shift;
        rank[i] -= (uint32_t)__builtin_amdgcn_readlane(above, L);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const uint32_t t = thr_bits[i];
      int above = 0, ties = 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const uint32_t pb = __builtin_bit_cast(uint32_t, p[i][j]);
        above += __popcll(__ballot(valid[j] && pb > t));      // strictly greater than T
        ties += (valid[j] && pb == t) ? 1 : 0;
      }
      const int need = min(nsel_h, limit[i]) - above;            // ties at T to take
      int tie_rank = wave_prefix_sum_dpp(ties) - ties;           // ties before this lane
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const uint32_t pb = __builtin_bit_cast(uint32_t, p[i][j]);
        const bool tie = valid[j] && pb == t;
        chosen[i][j] = valid[j] && (pb > t || (tie && tie_rank < need));
        tie_rank += tie ? 1 : 0;
      }
    }
  } else {
    // cdf: per row, sort into the order, then a running fp64 sum one block
    // at a time.  Keys: (probability bits, ~block index), descending;
    // padding keys (0) sort last.  Rows go one at a time through LDS (each
    // wave owns its rows of s_score and s_sel), which keeps every register
    // array statically indexed.
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int j = 0; j < KPL; ++j) s_score[4 * i + wave][lane * KPL + j] = p[i][j];
#pragma unroll 1
    for (int i = 0; i < RW; ++i) {
      const int r = 4 * i + wave;
      uint64_t key[KPL];
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = lane * KPL + j;
        key[j] = valid[j] ? (((uint64_t)__builtin_bit_cast(uint32_t, s_score[r][e]) << 32) |
                             (uint64_t)(~(uint32_t)e))
                          : 0ull;
      }
      bitonic_desc<KPL>(key, lane);
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        s_sorted[wave][lane * KPL + j] = __builtin_bit_cast(float, (uint32_t)(key[j] >> 32));
#pragma unroll
      for (int j = 0; j < KPL; ++j) s_sel[r][lane * KPL + j] = 0;
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      int found = nk;
      if (lane == 0) {
        double c = 0.0;
        for (int q = 0; q < nk; ++q) {
          c += (double)s_sorted[wave][q];
          if (c >= cdf_h) { found = q + 1; break; }
        }
      }
      const int n = min(__shfl(found, 0, kWave), a.causal ? min(nk, qb0 + r + 1) : nk);
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (lane * KPL + j < n) s_sel[r][~(uint32_t)key[j]] = 1;
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int j = 0; j < KPL; ++j) chosen[i][j] = s_sel[4 * i + wave][lane * KPL + j] != 0;
  }

  // Gate flags used by every row of the group, read once (their loads were issued
  // before the softmax).
  bool kgate[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = lane * KPL + j;
    kgate[j] = e < nk && !(ksim_el[j] > thr);          // K block forced on
  }
  if (a.sim_k && qb0 == 0 && wave == 0) {
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (lane * KPL + j < nk) a.sim_k[bh * nk + lane * KPL + j] = kgate[j] ? 0 : 1;
  }
  const uint64_t qflags = __ballot(lane < rows && qflag_raw != 0);

  // OR in the gate (within the allowed blocks) and the sink, then write the
  // ascending LUT by a prefix scan.
  int cnt[RW], incl[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const bool simq = (qflags >> (4 * i + wave < rows ? 4 * i + wave : 0)) & 1ull;
    cnt[i] = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int e = lane * KPL + j;
      chosen[i][j] = (valid[j] && e < limit[i] && (!simq || chosen[i][j] || kgate[j])) ||
                     (a.sink && e == 0);
      cnt[i] += chosen[i][j] ? 1 : 0;
    }
    incl[i] = cnt[i];
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) incl[i] = wave_prefix_sum_dpp(incl[i]);
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    if (4 * i + wave >= rows) continue;
    const int64_t row = bh * a.nq + qb0 + 4 * i + wave;
    const int total = __builtin_amdgcn_readlane(incl[i], kWave - 1);
    int32_t* lrow = a.lut + row * nk;
    int pos = incl[i] - cnt[i];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int e = lane * KPL + j;
      if (chosen[i][j]) lrow[pos++] = e;
      if (valid[j] && e >= total) lrow[e] = -1;
      if (valid[j] && a.bmap) a.bmap[row * nk + e] = chosen[i][j] ? 1 : 0;
    }
    if (lane == 0) a.count[row] = total;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class E, bool QUANT>
static void launch_pool_v(const PoolArgs& a, int d, dim3 grid, hipStream_t st) {
  if (a.km_part) {
    if (d == 128) hipLaunchKernelGGL((pool_sim_kernel<E, 128, true, QUANT>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((pool_sim_kernel<E, 64, true, QUANT>), grid, dim3(256), 0, st, a);
  } else {
    if (d == 128) hipLaunchKernelGGL((pool_sim_kernel<E, 128, false, QUANT>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((pool_sim_kernel<E, 64, false, QUANT>), grid, dim3(256), 0, st, a);
  }
}

template <class E>
static hipError_t launch_pool_t(const PoolArgs& a, int d, hipStream_t st) {
  const int64_t waves = (int64_t)a.b * (a.h * a.nq + a.h_kv * a.nk);
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (a.q_i8) launch_pool_v<E, true>(a, d, grid, st);
  else launch_pool_v<E, false>(a, d, grid, st);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_key_mean_t(const PoolArgs& a, int d, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.b * a.h_kv * a.km_chunks));
  if (d == 128) hipLaunchKernelGGL((key_mean_kernel<E, 128>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((key_mean_kernel<E, 64>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_key_mean(const PoolArgs& a, sparge_dtype dt, int d, hipStream_t st) {
  return dt == SPARGE_F16 ? launch_key_mean_t<F16>(a, d, st) : launch_key_mean_t<BF16>(a, d, st);
}

hipError_t launch_pool_sim(const PoolArgs& a, sparge_dtype dt, int d, hipStream_t st) {
  return dt == SPARGE_F16 ? launch_pool_t<F16>(a, d, st) : launch_pool_t<BF16>(a, d, st);
}

template <int D>
static hipError_t launch_select_d(const SelectArgs& a, hipStream_t st) {
  const int groups = (a.nq + kSelRows - 1) / kSelRows;
  const dim3 grid((unsigned)(((int64_t)a.b * a.h * groups + 7) / 8 * 8));
  const int nk = a.nk;
  if (nk <= 64) hipLaunchKernelGGL((score_select_kernel<D, 1>), grid, dim3(256), 0, st, a);
  else if (nk <= 128) hipLaunchKernelGGL((score_select_kernel<D, 2>), grid, dim3(256), 0, st, a);
  else if (nk <= 256) hipLaunchKernelGGL((score_select_kernel<D, 4>), grid, dim3(256), 0, st, a);
  else if (nk <= 512) hipLaunchKernelGGL((score_select_kernel<D, 8>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((score_select_kernel<D, 16>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_score_select(const SelectArgs& a, int d, hipStream_t st) {
  return d == 128 ? launch_select_d<128>(a, st) : launch_select_d<64>(a, st);
}

}  // namespace sparge
