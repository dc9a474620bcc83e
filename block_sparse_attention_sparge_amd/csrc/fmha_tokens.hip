// Stage 2 of SpargeAttn-style block-sparse attention on gfx950, token-list
// mode (blk_q = blk_k = 1, decode).
//
// One workgroup per (group of up to 8 query rows, batch, KV head, split)
// serves query heads of that KV head (aiter 6841 page: query head j reads KV
// head j / ratio) over an index list in which -1 entries are skipped (aiter
// 4919 page).  Keys are gathered 64 at a time; scores and the PV update run
// on the vector ALUs in fp32.
//
// The K and V rows are gathered with buffer loads: one resource per (batch,
// KV head) slice and a 32-bit byte offset per row (the host keeps a slice
// below 2^31 bytes; aiter 4919 page: the 32-bit offset limit of buffer
// loads).  A -1 entry takes the offset 2^31, past the slice, which the
// buffer range check turns into zeros (aiter 6841 page: an out-of-range read
// clamped by the descriptor's record count), so the loaded data needs no
// select.
#include "attn_common.h"
#include "common.h"
#include "kernels.h"

namespace sparge {

// ---------------------------------------------------------------------------
// token-list kernel (decode)
// ---------------------------------------------------------------------------
template <class E, int D, int R, bool OUT_F32>
__global__ __launch_bounds__(256) void fmha_tokens_kernel(FmhaArgs a) {
  typedef typename E::T T;
  constexpr int QW = D / 4;          // d values per thread (QK phase)
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int NS = 256 / CPR;      // key subsets (PV phase)
  constexpr int KPS = 64 / NS;       // keys per subset per chunk
  __shared__ uint32_t s_q[R][D / 2];   // query rows as packed input-type pairs
  __shared__ float s_p[R][64];
  __shared__ float s_alpha[R];
  __shared__ float s_ml[R][2];
  __shared__ __attribute__((aligned(16))) float s_red[NS][R * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // (row group, kv head, b, split)
  int64_t lin = blockIdx.x;
  const int grp = (int)(lin % a.tok_groups);
  lin /= a.tok_groups;
  const int hk = (int)(lin % a.hkv);
  lin /= a.hkv;
  const int bb = (int)(lin % a.b);
  const int split = (int)(lin / a.b);
  const int sq = a.sq;

  const int hlut = a.lut_heads == a.hq ? hk * a.ratio : hk;   // rows are per KV head
  const int32_t* list = a.lut + ((int64_t)bb * a.lut_heads + hlut) * a.lut_row_len;
  const int L = a.lut_row_len;
  const int chunk = (L + a.splits - 1) / a.splits;
  const int beg = split * chunk;
  const int end = min(L, beg + chunk);

  // Query rows rg = g * sq + sp for query head hk*ratio + g, position sp; this
  // workgroup serves rows row0 .. row0 + rows - 1 as its rows r = rg - row0.
  // The template row count R may exceed rows; the extra rows stay zero.
  const int row0 = grp * 8;
  const int rows = min(R, a.ratio * sq - row0);
  for (int i = tid; i < R * D / 2; i += 256) {
    const int r = i / (D / 2), d2 = i % (D / 2);
    uint32_t x = 0u;
    if (r < rows) {
      const int g = (row0 + r) / sq, sp = (row0 + r) % sq;
      const T* qp = reinterpret_cast<const T*>(a.q) + bb * a.qs[0] + (int64_t)(hk * a.ratio + g) * a.qs[1] +
                    (int64_t)sp * a.qs[2] + 2 * d2;
      x = *reinterpret_cast<const uint32_t*>(qp);
    }
    s_q[r][d2] = x;
  }
  float m_run[2], l_run[2];    // rows wave and wave + 4 (R <= 8)
#pragma unroll
  for (int i = 0; i < 2; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  float acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;

  const T* kbase = reinterpret_cast<const T*>(a.k) + bb * a.ks[0] + hk * a.ks[1];
  const T* vbase = reinterpret_cast<const T*>(a.v) + bb * a.vs[0] + hk * a.vs[1];
  // Raw buffer resources over the slice (records counted in bytes).
  const uint32_t krow_b = (uint32_t)(a.ks[2] * (int64_t)sizeof(T)), vrow_b = (uint32_t)(a.vs[2] * (int64_t)sizeof(T));
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(kbase), (short)0, (int)(krow_b * (uint32_t)a.sk), kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(vbase), (short)0, (int)(vrow_b * (uint32_t)a.sk), kBufferWord3);
  const float c2 = a.scale_log2;
  const int qj = tid >> 2, qq = tid & 3;        // QK phase: key slot, quarter
  const int pc = tid % CPR, ps = tid / CPR;     // PV phase: d chunk, key subset

  // Pipeline over 64-token chunks: the token indices of chunk c+2 and the K/V
  // rows of chunk c+1 are in flight while chunk c is scored and accumulated.
  // Each thread reads only the list entries it gathers: key slot qj for K and
  // key slots ps + NS*i for V.
  auto tok = [&](int pos) { return pos < end ? list[pos] : -1; };
  auto row_off = [](int t, uint32_t row_b) { return t >= 0 ? (uint32_t)t * row_b : 0x80000000u; };
  auto load_chunk = [&](int tk, const int (&tv)[KPS], u32x4 (&kr)[QW / 8], u32x4 (&vr)[KPS]) {
    const uint32_t ko = row_off(tk, krow_b) + 16u * qq;
#pragma unroll
    for (int i = 0; i < QW / 8; ++i)
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(ko + 64u * i), 0, 0);
#pragma unroll
    for (int i = 0; i < KPS; ++i)
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)(row_off(tv[i], vrow_b) + 16u * pc), 0, 0);
  };
  int tk_cur = tok(beg + qj), tv_cur[KPS];
#pragma unroll
  for (int i = 0; i < KPS; ++i) tv_cur[i] = tok(beg + ps + NS * i);
  int tk_nxt = tok(beg + 64 + qj), tv_nxt[KPS];
#pragma unroll
  for (int i = 0; i < KPS; ++i) tv_nxt[i] = tok(beg + 64 + ps + NS * i);
  u32x4 kr[QW / 8], vr[KPS];
  load_chunk(tk_cur, tv_cur, kr, vr);
  __syncthreads();                   // s_q is complete

#pragma unroll 1
  for (int pos0 = beg; pos0 < end; pos0 += 64) {
    // Next chunk's rows and the chunk after's indices.
    u32x4 kn[QW / 8], vn[KPS];
    load_chunk(pos0 + 64 < end ? tk_nxt : -1, tv_nxt, kn, vn);
    const int tk_far = tok(pos0 + 128 + qj);
    int tv_far[KPS];
#pragma unroll
    for (int i = 0; i < KPS; ++i) tv_far[i] = tok(pos0 + 128 + ps + NS * i);

    // Scores: each thread dots a quarter of one key with every query row.
    // Load i of the four threads of a key covers one contiguous 64-byte
    // segment of its row (thread qq holds d = 32i + 8qq .. +7), so each
    // segment is requested once (measured 5% faster than contiguous quarters,
    // whose loads touched four segments of every row per instruction).
    // Rows two at a time: the query words of at most two rows are live (all
    // of them at once would hold 16 registers per row).
    float part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      part[r] = 0.f;
#pragma unroll
      for (int i = 0; i < QW / 8; ++i) {
#pragma unroll
        for (int w = 0; w < 4; ++w) part[r] = E::dot2(s_q[r][16 * i + 4 * qq + w], kr[i][w], part[r]);
      }
      if (r & 1) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      part[r] += __shfl_xor(part[r], 1, kWave);
      part[r] += __shfl_xor(part[r], 2, kWave);
    }
    __syncthreads();                 // the previous chunk's PV has read s_p
    if (qq == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) s_p[r][qj] = tk_cur >= 0 ? part[r] * c2 : -INFINITY;
    }
    __syncthreads();

    // Online softmax: wave w owns rows w and w + 4.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wave + 4 * i;
      if (r < R) {
        const float x = s_p[r][lane];
        const float cm = wave_max_dpp(x);
        const float m_new = fmaxf(m_run[i], cm);
        float alpha, p;
        if (m_new == -INFINITY) {
          alpha = 1.f;
          p = 0.f;
        } else {
          alpha = __builtin_amdgcn_exp2f(m_run[i] - m_new);
          p = __builtin_amdgcn_exp2f(x - m_new);
        }
        m_run[i] = m_new;
        l_run[i] = fmaf(l_run[i], alpha, wave_sum_dpp(p));
        s_p[r][lane] = p;
        if (lane == 0) s_alpha[r] = alpha;
      }
    }
    __syncthreads();

    // PV: thread (d chunk pc, key subset ps) accumulates its keys.
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float al = s_alpha[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < KPS; ++i) {
      const int j = ps + NS * i;
      float v[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = E::lo(vr[i][w]);
        v[2 * w + 1] = E::hi(vr[i][w]);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float p = s_p[r][j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(p, v[e], acc[r][e]);
      }
    }

#pragma unroll
    for (int i = 0; i < QW / 8; ++i) kr[i] = kn[i];
#pragma unroll
    for (int i = 0; i < KPS; ++i) {
      vr[i] = vn[i];
      tv_nxt[i] = tv_far[i];
    }
    tk_cur = tk_nxt;
    tk_nxt = tk_far;
  }

  // Publish each row's (max, sum), then reduce the PV partials over key subsets.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wave + 4 * i;
    if (r < R && lane == 0) {
      s_ml[r][0] = m_run[i];
      s_ml[r][1] = l_run[i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    floatx4 lo4 = {acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
    floatx4 hi4 = {acc[r][4], acc[r][5], acc[r][6], acc[r][7]};
    *reinterpret_cast<floatx4*>(&s_red[ps][r * D + pc * 8]) = lo4;
    *reinterpret_cast<floatx4*>(&s_red[ps][r * D + pc * 8 + 4]) = hi4;
  }
  __syncthreads();
  for (int i = tid; i < rows * D; i += 256) {
    const int r = i / D, d = i % D;
    float sum = 0.f;
#pragma unroll 8
    for (int j = 0; j < NS; ++j) sum += s_red[j][i];
    const float m = s_ml[r][0], l = s_ml[r][1];
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int g = (row0 + r) / sq, sp = (row0 + r) % sq;
    const int hq = hk * a.ratio + g;
    const int64_t off = (int64_t)split * a.o_split_stride + bb * a.os[0] + (int64_t)hq * a.os[1] +
                        (int64_t)sp * a.os[2] + d;
    const float val = l > 0.f ? sum * inv : 0.f;
    if constexpr (OUT_F32) reinterpret_cast<float*>(a.o)[off] = val;
    else reinterpret_cast<T*>(a.o)[off] = E::from_f(val);
    if (d == 0 && a.lse) {
      a.lse[(((int64_t)split * a.b + bb) * a.hq + hq) * sq + sp] =
          l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <class E, int D, int R>
static hipError_t launch_tokens_r(const FmhaArgs& a, bool out_f32, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.tok_groups * a.b * a.hkv * a.splits));
  if (out_f32) hipLaunchKernelGGL((fmha_tokens_kernel<E, D, R, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((fmha_tokens_kernel<E, D, R, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_tokens_d(const FmhaArgs& a, bool out_f32, int rows, hipStream_t st) {
  switch (rows) {
    case 1: return launch_tokens_r<E, D, 1>(a, out_f32, st);
    case 2: return launch_tokens_r<E, D, 2>(a, out_f32, st);
    case 3: case 4: return launch_tokens_r<E, D, 4>(a, out_f32, st);
    default: return launch_tokens_r<E, D, 8>(a, out_f32, st);
  }
}

hipError_t launch_fmha_tokens(const FmhaArgs& a, sparge_dtype dt, sparge_dtype o_dt, int d,
                              int rows_per_group, hipStream_t st) {
  const bool f32 = o_dt == SPARGE_F32;
  if (dt == SPARGE_F16)
    return d == 128 ? launch_tokens_d<F16, 128>(a, f32, rows_per_group, st)
                    : launch_tokens_d<F16, 64>(a, f32, rows_per_group, st);
  return d == 128 ? launch_tokens_d<BF16, 128>(a, f32, rows_per_group, st)
                  : launch_tokens_d<BF16, 64>(a, f32, rows_per_group, st);
}

}  // namespace sparge
