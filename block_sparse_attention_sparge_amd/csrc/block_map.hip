// Stage 1 of SpargeAttn-style block-sparse attention on gfx950: the block map.
//
// "Sparge Attention (Composable Kernel)" page, "Status vs Upstream": per-block
// mean pool, cosine similarity, pooled QK, top-k / cdfthreshd selection into a
// BlockMap LUT, with per-head topk / simthreshd1 / cdfthreshd.  The same page
// lists sort-based top-k as the replacement for an O(nk^2) argmax that hurts
// at long sequences; the selector here sorts each row with a bitonic network
// held in the registers of one wavefront.
//
// Two kernels:
//   pool_sim     one wavefront per 64-token block of Q or K: reads the block
//                once (HBM bound), writes its fp32 mean and the gate flag
//                (mean pairwise cosine of the block's tokens > simthreshd1).
//   score_select one workgroup per 16 Q-tiles of one (b, h): pooled scores
//                against every K block mean, fp32 softmax, a 64-bit-key bitonic
//                sort per row (probability descending, block index ascending),
//                top-k or cdf count, and an ascending LUT written by a prefix
//                scan (no atomics, so the output is deterministic).
#include "common.h"
#include "kernels.h"

namespace sparge {

// ---------------------------------------------------------------------------
// pool_sim
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void pool_sim_kernel(PoolArgs a) {
  constexpr int CH = D / 8;          // 16-byte chunks per token
  constexpr int TPP = kWave / CH;    // tokens per pass of the wave
  constexpr int NP = 64 / TPP;       // passes over the 64-token block
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nqb = (int64_t)a.b * a.h * a.nq;
  const int64_t total = nqb + (int64_t)a.b * a.h * a.nk;
  if (gw >= total) return;

  const bool is_k = gw >= nqb;
  const int64_t idx = is_k ? gw - nqb : gw;
  const int nb = is_k ? a.nk : a.nq;
  const int64_t bh = idx / nb;
  const int blk = (int)(idx % nb);
  const int hh = (int)(bh % a.h);
  const int bb = (int)(bh / a.h);
  const int64_t* st = is_k ? a.ks : a.qs;
  const typename E::T* base = reinterpret_cast<const typename E::T*>(is_k ? a.k : a.q);

  const int c = lane % CH;
  const int t0 = lane / CH;
  const typename E::T* p0 = base + bb * st[0] + hh * st[1] + (int64_t)(blk * 64 + t0) * st[2] + c * 8;

  u32x4 raw[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) raw[p] = load16(p0 + (int64_t)(p * TPP) * st[2]);

  float sx[8], sh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { sx[i] = 0.f; sh[i] = 0.f; }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float x[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = E::lo(raw[p][w]);
      x[2 * w + 1] = E::hi(raw[p][w]);
    }
    float n2 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) n2 = fmaf(x[i], x[i], n2);
#pragma unroll
    for (int m = 1; m < CH; m <<= 1) n2 += __shfl_xor(n2, m, kWave);
    const float inv = n2 > 0.f ? 1.0f / sqrtf(n2) : 0.f;
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
#pragma unroll
  for (int m = 1; m < CH; m <<= 1) dot += __shfl_xor(dot, m, kWave);

  float* mean = (is_k ? a.k_mean : a.q_mean) + (bh * nb + blk) * D;
  if (t0 == 0) {
    const float r = 1.0f / 64.0f;
    floatx4 m0 = {sx[0] * r, sx[1] * r, sx[2] * r, sx[3] * r};
    floatx4 m1 = {sx[4] * r, sx[5] * r, sx[6] * r, sx[7] * r};
    *reinterpret_cast<floatx4*>(mean + c * 8) = m0;
    *reinterpret_cast<floatx4*>(mean + c * 8 + 4) = m1;
  }
  if (lane == 0) {
    const float sim = dot * (1.0f / 4096.0f);
    uint8_t* flags = is_k ? a.sim_k : a.sim_q;
    flags[bh * nb + blk] = sim > a.thr[hh] ? 1 : 0;
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
__global__ __launch_bounds__(256) void score_select_kernel(SelectArgs a) {
  constexpr int NKP = 64 * KPL;
  __shared__ float s_qm[kSelRows][D];
  __shared__ float s_score[kSelRows][NKP];
  __shared__ uint8_t s_sel[4][NKP];
  __shared__ float s_sorted[4][NKP];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int groups = (a.nq + kSelRows - 1) / kSelRows;
  const int64_t bh = blockIdx.x / groups;
  const int qb0 = (int)(blockIdx.x % groups) * kSelRows;
  const int rows = min(kSelRows, a.nq - qb0);
  const int hh = (int)(bh % a.h);
  const int nk = a.nk;

  // Pooled Q rows of this group into LDS.
  const float* qm = a.q_mean + (bh * a.nq + qb0) * D;
  for (int i = tid; i < kSelRows * D / 4; i += 256) {
    const int r = (i * 4) / D;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (r < rows) v = *reinterpret_cast<const floatx4*>(qm + i * 4);
    *reinterpret_cast<floatx4*>(&s_qm[0][0] + i * 4) = v;
  }
  __syncthreads();

  // Pooled scores: one K block per thread, all 16 rows.
  const float* km = a.k_mean + bh * nk * D;
  const uint8_t* simk = a.sim_k + bh * nk;
  for (int kb = tid; kb < NKP; kb += 256) {
    float acc[kSelRows];
#pragma unroll
    for (int r = 0; r < kSelRows; ++r) acc[r] = 0.f;
    const bool live = kb < nk && simk[kb] != 0;
    if (live) {
      const float* kr = km + (int64_t)kb * D;
      for (int d0 = 0; d0 < D; d0 += 4) {
        const floatx4 kv = *reinterpret_cast<const floatx4*>(kr + d0);
#pragma unroll
        for (int r = 0; r < kSelRows; ++r) {
          const floatx4 qv = *reinterpret_cast<const floatx4*>(&s_qm[r][d0]);
          acc[r] = fmaf(qv[0], kv[0], acc[r]);
          acc[r] = fmaf(qv[1], kv[1], acc[r]);
          acc[r] = fmaf(qv[2], kv[2], acc[r]);
          acc[r] = fmaf(qv[3], kv[3], acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kSelRows; ++r) s_score[r][kb] = live ? acc[r] * a.scale : -INFINITY;
  }
  __syncthreads();

  const int nsel_h = a.nsel[hh];
  const double cdf_h = (double)a.cdf[hh];
#pragma unroll 1
  for (int it = 0; it < kSelRows / 4; ++it) {
    const int r = it * 4 + wave;
    const bool active = r < rows;
    const int qb = qb0 + (active ? r : 0);
    const int64_t row = bh * a.nq + qb;

    // Softmax of the pooled row (fp32).
    float sc[KPL];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int e = lane * KPL + j;
      sc[j] = e < nk ? s_score[active ? r : 0][e] : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    mx = wave_max(mx);
    float p[KPL];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      p[j] = mx == -INFINITY ? 0.f : expf(sc[j] - mx);
      sum += p[j];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int j = 0; j < KPL; ++j) p[j] = sum > 0.f ? p[j] / sum : 0.f;

    if (active && a.prob) {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = lane * KPL + j;
        if (e < nk) a.prob[row * nk + e] = p[j];
      }
    }

    // Rank: 64-bit keys (probability bits, ~block index), sorted descending.
    // Probabilities are >= +0, so their bit patterns order like their values;
    // ~kb makes the lower block index win ties; padding keys (0) sort last.
    uint64_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int e = lane * KPL + j;
      key[j] = e < nk ? (((uint64_t)__builtin_bit_cast(uint32_t, p[j]) << 32) |
                         (uint64_t)(~(uint32_t)e))
                      : 0ull;
    }
    bitonic_desc<KPL>(key, lane);

    int n = nsel_h;
    if (n <= 0) {
      // cdf mode: running fp64 sum in sorted order, one block at a time.
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        s_sorted[wave][lane * KPL + j] = __builtin_bit_cast(float, (uint32_t)(key[j] >> 32));
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      int found = nk;
      if (lane == 0) {
        double c = 0.0;
        for (int i = 0; i < nk; ++i) {
          c += (double)s_sorted[wave][i];
          if (c >= cdf_h) { found = i + 1; break; }
        }
      }
      n = __shfl(found, 0, kWave);
    }

    // Mark the first n sorted blocks, then OR in the gate.
#pragma unroll
    for (int j = 0; j < KPL; ++j) s_sel[wave][lane * KPL + j] = 0;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int pos = lane * KPL + j;
      if (pos < n) s_sel[wave][~(uint32_t)key[j]] = 1;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();

    const bool simq = a.sim_q[row] != 0;
    bool sel[KPL];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int e = lane * KPL + j;
      sel[j] = e < nk && (!simq || s_sel[wave][e] != 0 || simk[e] == 0);
      cnt += sel[j] ? 1 : 0;
    }
    const int incl = wave_inclusive_scan(cnt);
    const int total = __shfl(incl, kWave - 1, kWave);
    if (active) {
      int32_t* lrow = a.lut + row * nk;
      int pos = incl - cnt;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = lane * KPL + j;
        if (sel[j]) lrow[pos++] = e;
        if (e < nk && e >= total) lrow[e] = -1;
        if (e < nk && a.bmap) a.bmap[row * nk + e] = sel[j] ? 1 : 0;
      }
      if (lane == 0) a.count[row] = total;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class E>
static hipError_t launch_pool_t(const PoolArgs& a, int d, hipStream_t st) {
  const int64_t waves = (int64_t)a.b * a.h * (a.nq + a.nk);
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (d == 128) hipLaunchKernelGGL((pool_sim_kernel<E, 128>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((pool_sim_kernel<E, 64>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pool_sim(const PoolArgs& a, sparge_dtype dt, int d, hipStream_t st) {
  return dt == SPARGE_F16 ? launch_pool_t<F16>(a, d, st) : launch_pool_t<BF16>(a, d, st);
}

template <int D>
static hipError_t launch_select_d(const SelectArgs& a, hipStream_t st) {
  const int groups = (a.nq + kSelRows - 1) / kSelRows;
  const dim3 grid((unsigned)((int64_t)a.b * a.h * groups));
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
