// Stage 2 of SpargeAttn-style block-sparse attention with int8 Q and K on
// gfx950 (CK page, "Status vs Upstream", not-yet-ported list: Q/K int8
// quantisation in the pool kernel feeding an int8 QK product in the
// attention kernel).
//
// The same walk as the fp16 / bf16 block kernel: one workgroup of four
// wavefronts per (Q-tile, head, batch, split), wave (qh, kh) owning 32 query
// rows and 32 keys of every listed 64-key block, K and V arriving by direct
// global->LDS loads into double buffers, one barrier per block, the two key
// halves merged by the LSE rule at the end.  What changes:
//   * S^T = K Q^T runs on v_mfma_i32_32x32x32_i8 from the int8 codes: four
//     MFMAs per block for d = 128 instead of eight, and the integer product is
//     exact (|sum| <= 128 * 127^2 < 2^24, so its conversion to fp32 is exact
//     too); the score is that integer times scale * q_scale * k_scale, one
//     fp32 multiply folded into the base-2 softmax FMA;
//   * a K block is 64 rows of d bytes in LDS, half the bytes of fp16, so the
//     direct loads write half as much into LDS and the operand reads of K
//     halve;
//   * the K scale of every block comes through the scalar cache, requested
//     one step ahead next to a LUT entry, after the block's last LDS wait.
// V and P stay in fp16 / bf16 and the PV product is the one of the fp16 / bf16
// kernel, and ragged lengths are handled as there: a partial last Q-tile
// repeats its last row and stores only its own rows; the MASKED kernel
// (causal, or a ragged K sequence) repeats the last K/V row in a partial last
// block and removes keys by position.
//
// With fp8 (e4m3) codes instead of int8 (the FP8 instantiation), S^T runs on
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales: two MFMAs per block for
// d = 128, each lane feeding 32 consecutive codes of its K row and of its Q
// row (any assignment of the 64 codes of a step to the two half-waves gives
// the same product as long as K and Q use the same one), accumulated in fp32.
// The codes occupy the same bytes as int8 codes, so the loads, the LDS layout
// and everything after the scores are shared.
#include <type_traits>

#include "attn_common.h"
#include "common.h"
#include "kernels.h"

namespace sparge {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ i32x16 mfma_i8(const u32x4& a, const u32x4& b, const i32x16& c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c,
                                               0, 0, 0);
}

// 32x32x64 fp8 (e4m3, format 0) MFMA with unit E8M0 scales (127 = 2^0).
__device__ __forceinline__ floatx16 mfma_f8(const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1,
                                            const floatx16& c) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// K rows are d bytes: GK 16-byte granules.  Row r's granule g sits in slot
// g ^ ((r / (16 / GK)) % GK): the 16 rows that 16 consecutive lanes read for
// one k-step then fall on 16 different 16-byte bank groups.
template <int GK>
__device__ __forceinline__ int k8_swz(int r) {
  return (r / (16 / GK)) % GK;
}

template <class E, int D, bool OUT_F32, bool MASKED, bool FP8>
// Three waves per SIMD at d = 128 (168 VGPRs), four at d = 64.  The hint
// shapes the compiler's schedule as well as its register budget: d = 64 runs
// 3-13% faster for (4, 4) than for (3, 3) at the same register count.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 3, D == 64 ? 4 : 3)))
void fmha_qk8_kernel(FmhaArgs a) {
  typedef typename E::T T;
  constexpr int G16 = D / 8;                 // 16-byte granules per V row
  constexpr int GK = D / 16;                 // 16-byte granules per int8 K row
  constexpr int NKK = D / 32;                // k-steps of S^T (32 codes each)
  constexpr int NMD = D / 32;                // M-tiles of O^T
  constexpr int TILE = 64 * D;               // elements of a V buffer, bytes of a K buffer
  constexpr int NDMA_V = 64 * G16 / 256;     // direct loads per thread per V tile
  constexpr int NDMA_K = 64 * GK / 256;      // and per K tile
  constexpr int VSW = G16 / 4;
  __shared__ __attribute__((aligned(16))) int8_t sK[2 * TILE];
  __shared__ __attribute__((aligned(16))) T sV[2 * TILE];
  __shared__ float s_ml[128];                // (m, l) of the kh = 1 waves, per query half

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int qh = wave & 1;
  const int kh = wave >> 1;

  // Row order across the XCDs: block_row_of().  Causal rows are taken last
  // tile first (measured 1.6% faster sparse, 2.0% dense, at b2 h32 s16384
  // d128).
  int qt;
  int64_t lin;
  if (!block_row_of(a.nqt, (int64_t)a.hq * a.b * a.splits, MASKED && a.causal, qt, lin)) return;
  const int hh = (int)(lin % a.hq);
  lin /= a.hq;
  const int bb = (int)(lin % a.b);
  const int split = (int)(lin / a.b);
  const int hk = hh / a.ratio;

  int n;
  const int32_t* list = nullptr;
  if (a.lut) {
    const int hlut = a.lut_heads == a.hq ? hh : hk;
    const int64_t row = ((int64_t)bb * a.lut_heads + hlut) * a.nqt + qt;
    list = a.lut + row * a.lut_row_len;
    n = a.cnt ? a.cnt[row] : first_negative(list, a.lut_row_len, lane);
  } else {
    n = MASKED && a.causal ? min(a.nkb, qt + 1) : a.nkb;
  }
  n = __builtin_amdgcn_readfirstlane(n);
  const int chunk = (n + a.splits - 1) / a.splits;
  const int beg = split * chunk;
  const int nloc = max(0, min(n, beg + chunk) - beg);

  const int q0 = qt * 64 + qh * 32;
  const bool row_ok = q0 + l32 < a.sq;       // false past the end of a ragged last tile
  const int64_t orow = (int64_t)split * a.o_split_stride + bb * a.os[0] + hh * a.os[1] +
                       (int64_t)(q0 + l32) * a.os[2];
  float* lse_row = a.lse ? a.lse + (((int64_t)split * a.b + bb) * a.hq + hh) * a.sq : nullptr;

  if (nloc == 0) {
    if (kh == 0 && row_ok) {
      for (int d0 = hl * (D / 2); d0 < (hl + 1) * (D / 2); d0 += 4)
        store4<E, OUT_F32>(a.o, orow + d0, 0.f, 0.f, 0.f, 0.f);
      if (lse_row && hl == 0) lse_row[q0 + l32] = -INFINITY;
    }
    return;
  }

  // Scales: the tile's Q scale and the softmax scale are folded once; the K
  // scale of each block joins them per block.
  const __attribute__((address_space(4))) float* ksc =
      (const __attribute__((address_space(4))) float*)(a.k_scale + ((int64_t)bb * a.hkv + hk) * a.nkb);
  const float c2q = a.scale_log2 * a.q_scale[((int64_t)bb * a.hq + hh) * a.nqt + qt];

  const char* kbase = reinterpret_cast<const char*>(a.k) + bb * a.ks[0] + hk * a.ks[1];
  const char* vbase = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + bb * a.vs[0] + hk * a.vs[1]);
  const int64_t kblk = 64 * a.ks[2], vblk = 64 * a.vs[2] * (int64_t)sizeof(T);
  const uint32_t sk_lds = (uint32_t)(uintptr_t)((SPARGE_LDS void*)sK);
  const uint32_t sv_lds = (uint32_t)(uintptr_t)((SPARGE_LDS void*)sV);

  // V's swizzle depends only on r mod 4, so V's lane offsets differ between
  // load instructions by whole rows, which go into the scalar offset.
  constexpr int RPI_V = 64 / G16;              // V rows per load instruction
  static_assert(RPI_V % 4 == 0, "V swizzle must repeat every load instruction");
  uint32_t koff[NDMA_K], voff;
#pragma unroll
  for (int j = 0; j < NDMA_K; ++j) {
    const int gi = 64 * (wave * NDMA_K + j) + lane;
    const int r = gi / GK, sl = gi % GK;
    koff[j] = (uint32_t)(r * a.ks[2] + (sl ^ k8_swz<GK>(r)) * 16);
  }
  {
    const int r0 = RPI_V * wave * NDMA_V + lane / G16, sl = lane % G16;
    voff = (uint32_t)((r0 * a.vs[2] + (sl ^ ((VSW * r0) % G16)) * 8) * (int64_t)sizeof(T));
  }
  const int krow_b = (int)a.ks[2], vrow_b = (int)(a.vs[2] * (int64_t)sizeof(T));
  // K codes of block kb into K buffer `buf`, V into V buffer `buf`, through
  // buffer resources that cover the block's existing rows: rows past the end
  // of a ragged K sequence read as zeros (their scores are removed below).
  auto issue_block = [&](int kb, int buf) {
    int krec = (int)kblk, vrec = (int)vblk;
    if constexpr (MASKED) {
      const int rows = min(64, a.sk - 64 * kb);
      krec = rows * krow_b;
      vrec = rows * vrow_b;
    }
    const i32x4 kr = raw_rsrc(kbase + kb * kblk, krec), vr = raw_rsrc(vbase + kb * vblk, vrec);
#pragma unroll
    for (int j = 0; j < NDMA_K; ++j)
      dma16_buf(kr, koff[j], 0u, sk_lds + (uint32_t)(buf * TILE + (wave * NDMA_K + j) * 64 * 16));
#pragma unroll
    for (int j = 0; j < NDMA_V; ++j)
      dma16_buf(vr, voff, (uint32_t)(RPI_V * j * vrow_b),
                sv_lds + (uint32_t)((buf * TILE + (wave * NDMA_V + j) * 64 * 8) * sizeof(T)));
  };
  const __attribute__((address_space(4))) int32_t* clist = (const __attribute__((address_space(4))) int32_t*)list;
  auto kb_of = [&](int i) { return list ? clist[beg + i] : beg + i; };

  floatx16 acc_o[NMD];
#pragma unroll
  for (int i = 0; i < NMD; ++i) acc_o[i] = floatx16{};
  float m_run = -INFINITY;   // reference maximum in base-2 units
  float l_run = 0.f;
  const int krow = 32 * kh + l32;
  const int kswz = k8_swz<GK>(krow);
  const int vs16 = lane & 15, vgrp = lane >> 4;
  const int vrow0 = 32 * kh + 4 * (vgrp >> 1) + (vs16 >> 2);
  const int vcol0 = 16 * (vgrp & 1) + 4 * (vs16 & 3);

  // Block 0 in LDS; the LUT entry of block 1 and the K scale of block 0 read.
  // Block it+1's K/V loads are issued in the middle of step it (as in the
  // fp16 / bf16 kernel).
  // The Q codes arrive by direct loads into K buffer 1 (refilled only after
  // the second barrier below), in K's layout, with the rows of a partial
  // last tile repeating its last row; each instruction then moves whole rows.
  {
    const char* qbase = reinterpret_cast<const char*>(a.q) + bb * a.qs[0] + hh * a.qs[1] + (int64_t)(64 * qt) * a.qs[2];
    const int last = a.sq - 1 - 64 * qt;
#pragma unroll
    for (int j = 0; j < NDMA_K; ++j) {
      const int gi = 64 * (wave * NDMA_K + j) + lane;
      const int r = gi / GK, sl = gi % GK, rc = min(r, last);
      dma16(qbase, (uint32_t)(rc * a.qs[2] + (sl ^ k8_swz<GK>(r)) * 16),
            sk_lds + (uint32_t)(TILE + (wave * NDMA_K + j) * 64 * 16));
    }
  }
  issue_block(kb_of(0), 0);
  wait_dma();
  __syncthreads();
  // Q^T codes (B operand): lane (query l32, half hl) holds d = 32kk + 16hl .. +15
  // of tile row 32 qh + l32 (for fp8, k-step kk / 2 takes granules 2kk + hl
  // and 2kk + 2 + hl: codes 64(kk/2) + 16hl .. +15 and + 32 .. +47).
  u32x4 qf[NKK];
  {
    const int qrow = 32 * qh + l32, qsw = k8_swz<GK>(qrow);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = *reinterpret_cast<const u32x4*>(&sK[TILE + qrow * D + ((2 * kk + hl) ^ qsw) * 16]);
  }
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qf[kk]));
  __syncthreads();
  int kb_ahead = nloc > 1 ? kb_of(1) : 0;
  float sk_cur = ksc[kb_of(0)];
  int kb_cur = MASKED ? kb_of(0) : 0;

  auto step = [&](int it, auto cur_tag) {
    constexpr int cur = decltype(cur_tag)::value;
    const int8_t* kt = &sK[cur * TILE];
    const SPARGE_LDS T* vt = (const SPARGE_LDS T*)&sV[cur * TILE];

    // The scalar loads of the previous step (or of the prologue) have landed.
    asm volatile("" ::"s"(kb_ahead), "s"(sk_cur));
    u32x4 kf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int g = (2 * kk + hl) ^ kswz;
      kf[kk] = *reinterpret_cast<const u32x4*>(&kt[krow * D + g * 16]);
    }
    u32x4 vf[2][NMD];
    auto read_vt = [&](int ks) {
#pragma unroll
      for (int md = 0; md < NMD; ++md) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int r = vrow0 + 16 * ks + 8 * c;
          const int col = 32 * md + vcol0;
          const int slot = (col >> 3) ^ ((VSW * r) % G16);
          const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (SPARGE_LDS short4v*)(vt + r * D + slot * 8 + (col & 7)));
          const u32x2 w2 = __builtin_bit_cast(u32x2, x);
          vf[ks][md][2 * c] = w2[0];
          vf[ks][md][2 * c + 1] = w2[1];
        }
      }
    };
    read_vt(0);
    __builtin_amdgcn_sched_barrier(0);

    // S^T (32 keys x 32 queries) = K Q^T on the codes, exact in int32.  These
    // MFMAs are issued at raised wave priority (of the two wavefronts on a
    // SIMD, the one starting a block goes first; measured 1.8% faster at topk
    // 0.4 and 2.5% at topk 0.1, bit-identical.  The fp16 / bf16 kernel, with
    // twice the S^T MFMAs, gains instead from raising it for PV).
    // fp8: step j of 64 codes pairs the reads kk = 2j and 2j + 1.
    typedef typename std::conditional<FP8, floatx16, i32x16>::type SAcc;
    SAcc si = SAcc{};
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < NKK / 2; ++j) si = mfma_f8(kf[2 * j], kf[2 * j + 1], qf[2 * j], qf[2 * j + 1], si);
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) si = mfma_i8(kf[kk], qf[kk], si);
    }
    read_vt(1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    // The other buffer held block it-1, released by the last barrier.
    if (it + 1 < nloc) issue_block(kb_ahead, 1 - cur);

    float s[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (float)si[r];
    if constexpr (MASKED) {
      if (64 * kb_cur + 64 > a.sk || (a.causal && kb_cur >= qt)) {
        const int qpos = 64 * qt + 32 * qh + l32;
        const int lim = a.causal ? min(qpos + 1, a.sk) : a.sk;   // first removed key
        // Register r holds key base + 8 (r / 4) + r % 4: one value per lane
        // against immediate offsets.
        const int rel = lim - (64 * kb_cur + 32 * kh + 4 * hl);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) >= rel) s[r] = -INFINITY;
      }
    }

    // This block's factor from code product to base-2 score.  It is 0 when a
    // scale is 0 (an all-zero block, whose codes and products are all 0); the
    // masked kernel lifts it to the least normal float so that a removed key
    // (-inf) still scores -inf and not -inf * 0.  The unmasked scores it then
    // gives, at most 2^21 * 2^-126, vanish next to any score that matters.
    const float c2 = MASKED ? fmaxf(c2q * sk_cur, 1.17549435e-38f) : c2q * sk_cur;
    float rmax = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) rmax = fmaxf(rmax, s[r]);
    rmax = half_swap_max(rmax);
    const float m_cand = rmax * c2;
    const bool need = m_cand > m_run + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? m_cand : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NMD; ++i) acc_o[i] *= alpha;
    }
    const float mref = MASKED && m_run == -INFINITY ? 0.f : m_run;
    u32x4 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * ks + 2 * w], c2, -mref));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * ks + 2 * w + 1], c2, -mref));
        pf[ks][w] = E::pack2(p0, p1);
        l_run += p0 + p1;   // fp32 row sum, as in the fp16 / bf16 kernel
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int md = 0; md < NMD; ++md) acc_o[md] = mfma32<E>(vf[ks][md], pf[ks], acc_o[md]);
    }

    // After the last LDS wait: the LUT entry of block it+2 and the K scale of
    // block it+1 (kb_ahead), both consumed first thing in the next step.
    __builtin_amdgcn_sched_barrier(0);
    const int kb_next = it + 2 < nloc ? kb_of(it + 2) : 0;
    const float sk_next = it + 1 < nloc ? ksc[kb_ahead] : 0.f;

    // Block it+1 must have landed before the barrier hands the buffers over.
    wait_dma();
    __syncthreads();
    if constexpr (MASKED) kb_cur = kb_ahead;
    sk_cur = sk_next;
    kb_ahead = kb_next;
  };

#pragma unroll 1
  for (int it = 0; it < nloc; it += 2) {
    step(it, Buf<0>{});
    if (it + 1 == nloc) break;
    step(it + 1, Buf<1>{});
  }

  // Merge the two key halves (as in the fp16 / bf16 kernel; the partial O^T
  // goes to the V buffers, the larger ones here).  A 16-bit O tile is then
  // staged in the K buffers (exactly its size) and stored as whole rows, as in
  // the fp16 / bf16 kernel; fp32 partials are stored from the fragments.
  const float l_w = l_run + __shfl_xor(l_run, 32, kWave);
  float* mrg = reinterpret_cast<float*>(sV) + qh * (NMD * 16 * 64);
  float* ml = s_ml + qh * 64;
  constexpr int OG = D * 2 / 16;                 // 16-byte granules per 16-bit O row
  char* stg = reinterpret_cast<char*>(sK);
  if (kh == 1) {
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) mrg[(md * 16 + r) * 64 + lane] = acc_o[md][r];
    if (hl == 0) {
      ml[l32] = m_run;
      ml[32 + l32] = l_w;
    }
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = ml[l32], l1 = ml[32 + l32];
    float m = fmaxf(m_run, m1);
    const bool empty = MASKED && m == -INFINITY;
    if (empty) m = 0.f;
    const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float l_tot = l_w * a0 + l1 * a1;
    const float inv = empty ? 0.f : 1.0f / l_tot;
    const float s0 = a0 * inv, s1 = a1 * inv;
    const int tr = 32 * qh + l32;
    char* srow = stg + tr * (OG * 16);
#pragma unroll
    for (int md = 0; md < NMD; ++md) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          x[i] = acc_o[md][r] * s0 + mrg[(md * 16 + r) * 64 + lane] * s1;
        }
        const int d0 = 32 * md + 8 * g + 4 * hl;
        if constexpr (OUT_F32) {
          if (row_ok) store4<E, true>(a.o, orow + d0, x[0], x[1], x[2], x[3]);
        } else {
          const int gr = 4 * md + g;
          *reinterpret_cast<u32x2*>(srow + ((gr ^ (tr % OG)) * 16) + 8 * hl) =
              u32x2{E::pack2(x[0], x[1]), E::pack2(x[2], x[3])};
        }
      }
    }
    if (lse_row && hl == 0 && row_ok) lse_row[q0 + l32] = empty ? -INFINITY : (m + __log2f(l_tot)) * kLn2;
  }
  if constexpr (!OUT_F32) {
    __syncthreads();
    const int nrows = min(64, a.sq - 64 * qt);
    T* obase = reinterpret_cast<T*>(a.o) + (int64_t)split * a.o_split_stride + bb * a.os[0] + hh * a.os[1] +
               (int64_t)(64 * qt) * a.os[2];
#pragma unroll
    for (int k = 0; k < OG / 4; ++k) {
      const int idx = tid + 256 * k;
      const int r = idx / OG, gs = idx % OG;
      if (r < nrows) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * (OG * 16) + ((gs ^ (r % OG)) * 16));
        store16(obase + (int64_t)r * a.os[2] + gs * 8, v);
      }
    }
  }
}

template <class E, int D, bool FP8>
static hipError_t launch_qk8_t(const FmhaArgs& a, bool out_f32, hipStream_t st) {
  const int64_t nwg = block_grid(a.nqt, (int64_t)a.hq * a.b * a.splits, a.causal != 0);
  if (nwg > 0xFFFFFFFFll) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nwg);
  if (a.causal || a.sk % 64) {
    if (out_f32) hipLaunchKernelGGL((fmha_qk8_kernel<E, D, true, true, FP8>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((fmha_qk8_kernel<E, D, false, true, FP8>), grid, dim3(256), 0, st, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((fmha_qk8_kernel<E, D, true, false, FP8>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((fmha_qk8_kernel<E, D, false, false, FP8>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <bool FP8>
static hipError_t launch_qk8_c(const FmhaArgs& a, sparge_dtype v_dt, bool f32, int d, hipStream_t st) {
  if (v_dt == SPARGE_F16)
    return d == 128 ? launch_qk8_t<F16, 128, FP8>(a, f32, st) : launch_qk8_t<F16, 64, FP8>(a, f32, st);
  return d == 128 ? launch_qk8_t<BF16, 128, FP8>(a, f32, st) : launch_qk8_t<BF16, 64, FP8>(a, f32, st);
}

hipError_t launch_fmha_qk8(const FmhaArgs& a, sparge_dtype v_dt, sparge_dtype o_dt, int d, bool fp8,
                           hipStream_t st) {
  const bool f32 = o_dt == SPARGE_F32;
  return fp8 ? launch_qk8_c<true>(a, v_dt, f32, d, st) : launch_qk8_c<false>(a, v_dt, f32, d, st);
}

}  // namespace sparge
