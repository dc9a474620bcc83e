// Stage 2 of SpargeAttn-style block-sparse attention on gfx950: sparse flash
// attention forward over a per-Q-tile list of K/V blocks, with LSE export.
//
// What is computed ("Updating Log -- Speculative Sparse Attention" page,
// Stage 3, and the aiter 6841 page): for each query row, an online softmax
// over the keys of the listed blocks; O = sum_j softmax_j v_j and the
// natural-log LSE; a list with no block writes O = 0 and LSE = -inf.
//
// Block kernel (blk_q = blk_k = 64), one workgroup of four wavefronts per
// (Q-tile, head, batch, split); each wavefront owns 32 query rows and 32 keys
// of every block and works in the transposed orientation S^T = K Q^T,
// O^T += V^T P^T on the 32x32x16 fp16/bf16 MFMA:
//   * Q^T stays in registers as the B operand for the whole row; the Q tile
//     itself arrives by direct global->LDS loads, whole rows per instruction;
//   * K and V blocks arrive by direct global->LDS loads, K into one buffer and
//     V into two; K is read row-major (A operand of S^T), V through the
//     transposing LDS read (A operand of O^T);
//   * the S^T accumulator already has the layout of the P^T B operand, so P
//     goes from softmax to the PV MFMA without leaving registers, and every
//     row reduction is in-lane plus one exchange with the partner half-wave;
//   * the softmax runs in base 2 with the scale folded in once (aiter 4919
//     page: one FMA per score, exp2), and the row sum is finished only at the
//     end (one reciprocal per row);
//   * the two key halves of a tile are merged at the end with the LSE rule,
//     and the finished tile leaves through LDS as whole rows;
//   * with a pv_threshold (CK page, "Status vs Upstream": a per-Q-tile skip
//     in the attention kernel), the workgroup drops the PV product of a whole
//     listed block when every one of the tile's 64 query rows scores, over
//     the block's 64 keys, more than the threshold below that row's running
//     maximum over the blocks already visited; its P still count in the row
//     sum.  The four wavefronts post their row maxima to LDS before the
//     block's first barrier, which publishes them; every wave then takes the
//     same decision, and a dropped block skips its V^T reads and PV MFMAs,
//     so the test adds no barrier;
//   * rows are dealt to the 8 XCDs (which receive workgroups round-robin by
//     linear id, aiter 4919 page) so that each gets an equal share of every
//     head; causal and one-round launches give each XCD contiguous heads
//     instead, causal ones last tile first (block_row_of in attn_common.h).
// The token-list (decode) kernel is in fmha_tokens.hip.
#include "attn_common.h"
#include "common.h"
#include "kernels.h"

namespace sparge {

// ---------------------------------------------------------------------------
// block-LUT kernel
// ---------------------------------------------------------------------------
// One workgroup of 4 wavefronts per (Q-tile, head, batch, split).  Wave w owns
// query rows 32*(w&1) .. +31 of the tile and keys 32*(w>>1) .. +31 of every
// 64-key block, keeping its own running maximum, row sum and O^T; the two
// key halves are merged in LDS at the end (the LSE combine of two partials).
//
// Three workgroups share a CU (168 VGPRs, 48.5 KB of LDS each; measured 4-10%
// faster than two workgroups with both K and V double-buffered, bit-identical).
// K blocks arrive in one LDS buffer and V blocks in two, by direct loads from
// memory into LDS (no registers on the way; on gfx950 this path moves
// gathered blocks out of L2 much faster than loads into VGPRs, and it stays
// faster than loads into VGPRs followed by LDS writes).  Each block has two
// barriers: the first, right after the S^T MFMAs, says every wave has read
// the block's K, and the loads of block i+1 (K into the one K buffer, V into
// the V buffer that block i-1 used) are issued there; the second ends the
// block once those loads have landed.  The loads go through buffer resources
// that end at the block's last existing row, so the rows past the end of a
// ragged K sequence read as zeros.  They are issued from inline assembly so
// the compiler does not guard every LDS read with a wait for them; the kernel
// waits for them itself (vmcnt) before the closing barrier.
//   * K is stored row-major with the 16-byte granules of row r XOR-swizzled
//     by r mod G16 (G16 = granules per row: 16 for d = 128), so S^T operand
//     reads of consecutive rows hit distinct banks.
//   * V is stored row-major with granules XOR-swizzled by (G16/4) r (4r for
//     d = 128, 2r for d = 64), and the V^T operand of O^T += V^T P^T is read
//     with the gfx950 transposing LDS read (ds_read_b64_tr_b16): within each
//     16-lane group, lane j receives element j%4 of the 4-element chunks
//     addressed by lanes j/4 + 4t, t = 0..3.  These reads are served 32 lanes
//     per clock; the swizzle puts the four rows one such half-wave touches on
//     four different sets of banks.
// The running maximum is only moved when a row's new maximum exceeds it by
// more than 2^8 (base-2 units), so most blocks skip rescaling O; the exported
// LSE and O are exact for any reference maximum, and P stays below 2^8.
//
// Lengths need not be multiples of 64.  A partial last Q-tile loads its
// missing rows as copies of its last row and stores only its own rows.  The
// MASKED kernel removes keys by position: past the query (causal) and past
// the end of a ragged K sequence, whose last block has zeros in its missing
// rows (finite values whose scores are then -inf, with P = 0 against zero V).
// Element type of O: fp32 partials or the input type.
template <class T, bool F32>
struct OutType {
  typedef T type;
};
template <class T>
struct OutType<T, true> {
  typedef float type;
};

template <class E, int D, bool OUT_F32, bool MASKED, bool PVSKIP>
// Three waves per SIMD at d = 128 (168 VGPRs), four at d = 64.  The hint
// shapes the compiler's schedule as well as its register budget: d = 64 runs
// 3-13% faster for (4, 4) than for (3, 3) at the same register count.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 3, D == 64 ? 4 : 3)))
void fmha_block_kernel(FmhaArgs a) {
  typedef typename E::T T;
  constexpr int G16 = D / 8;                 // 16-byte granules per K/V row
  constexpr int NKK = D / 16;                // k-steps of S^T
  constexpr int NMD = D / 32;                // M-tiles of O^T
  constexpr int TILE = 64 * D;               // elements per K or V buffer
  constexpr int NDMA = 64 * G16 / 256;       // direct loads per thread per tile
  constexpr int VSW = G16 / 4;               // V row r's granules are XOR-swizzled by VSW * r
  __shared__ __attribute__((aligned(16))) T sK[TILE];
  __shared__ __attribute__((aligned(16))) T sV[2 * TILE];
  __shared__ float s_ml[128];                // (m, l) of the kh = 1 waves, per query half
  // pv_threshold votes: (block maximum, running maximum) of each wave's 32
  // query rows over its 32 keys, scaled base-2 units.  A block's votes are
  // written before its first barrier and read before its closing one.
  __shared__ float2v s_vote[PVSKIP ? 128 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int qh = wave & 1;                   // query half of the tile
  const int kh = wave >> 1;                  // key half of every block

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
    n = MASKED && a.causal ? min(a.nkb, qt + 1) : a.nkb;   // dense causal: blocks 0..qt
  }
  // The row length is the same for every lane; saying so keeps the loop
  // uniform and lets the LUT entries come through scalar loads.
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

  const char* kbase = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + bb * a.ks[0] + hk * a.ks[1]);
  const char* vbase = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + bb * a.vs[0] + hk * a.vs[1]);
  const int64_t kblk = 64 * a.ks[2] * (int64_t)sizeof(T), vblk = 64 * a.vs[2] * (int64_t)sizeof(T);
  const uint32_t sk_lds = (uint32_t)(uintptr_t)((SPARGE_LDS void*)sK);
  const uint32_t sv_lds = (uint32_t)(uintptr_t)((SPARGE_LDS void*)sV);

  // Direct-load instruction J of a tile fills LDS granules 64J .. 64J+63;
  // granule (row r, slot sl) holds global granule sl ^ swz(r).  The byte
  // offsets inside a block are the same for every block (the host keeps a
  // block's span below 2^31 bytes).
  // Instruction j covers rows RPI (wave NDMA + j) .. +RPI-1.  V's swizzle
  // depends only on r mod 4, so its offsets differ between instructions by
  // whole rows, which go into the scalar offset; so do K's when each
  // instruction covers a multiple of G16 rows (d = 64).  For d = 128 K's
  // swizzle changes with j and each instruction keeps its own lane offset.
  constexpr int RPI = 64 / G16;                // rows per load instruction
  constexpr bool K_ROWSTEP = RPI % G16 == 0;
  static_assert(RPI % 4 == 0, "V swizzle must repeat every load instruction");
  uint32_t koff[K_ROWSTEP ? 1 : NDMA], voff;
  {
    const int r0 = RPI * wave * NDMA + lane / G16, sl = lane % G16;
    voff = (uint32_t)((r0 * a.vs[2] + (sl ^ ((VSW * r0) % G16)) * 8) * (int64_t)sizeof(T));
#pragma unroll
    for (int j = 0; j < (K_ROWSTEP ? 1 : NDMA); ++j) {
      const int r = r0 + RPI * j;
      koff[j] = (uint32_t)((r * a.ks[2] + (sl ^ (r % G16)) * 8) * (int64_t)sizeof(T));
    }
  }
  const int krow_b = (int)(a.ks[2] * (int64_t)sizeof(T)), vrow_b = (int)(a.vs[2] * (int64_t)sizeof(T));
  // K of block kb into the K buffer, V into V buffer `buf`.  The resources
  // cover the block's existing rows, so rows past the end of a ragged K
  // sequence read as zeros.
  auto issue_block = [&](int kb, int buf) {
    int krec = (int)kblk, vrec = (int)vblk;
    if constexpr (MASKED) {
      const int rows = min(64, a.sk - 64 * kb);
      krec = rows * krow_b;
      vrec = rows * vrow_b;
    }
    const i32x4 kr = raw_rsrc(kbase + kb * kblk, krec), vr = raw_rsrc(vbase + kb * vblk, vrec);
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const uint32_t off = (uint32_t)((wave * NDMA + j) * 64 * 8 * sizeof(T));
      if constexpr (K_ROWSTEP) dma16_buf(kr, koff[0], (uint32_t)(RPI * j * krow_b), sk_lds + off);
      else dma16_buf(kr, koff[j], 0u, sk_lds + off);
      dma16_buf(vr, voff, (uint32_t)(RPI * j * vrow_b), sv_lds + off + (uint32_t)(buf * TILE * sizeof(T)));
    }
  };

  // LUT entries come through the scalar cache (the LUT is read-only here).
  const __attribute__((address_space(4))) int32_t* clist = (const __attribute__((address_space(4))) int32_t*)list;
  auto kb_of = [&](int i) { return list ? clist[beg + i] : beg + i; };

  floatx16 acc_o[NMD];
#pragma unroll
  for (int i = 0; i < NMD; ++i) acc_o[i] = floatx16{};
  float m_run = -INFINITY;   // reference maximum, already times scale*log2(e)
  float l_run = 0.f;         // this lane's share of the row sum
  float m_top = -INFINITY;   // exact running maximum (pv_threshold test), same units
  const float c2 = a.scale_log2;
  const int krow = 32 * kh + l32;                  // K row this lane feeds to S^T
  const int kswz = krow % G16;
  // V^T operand (transposing read): lane (s = lane%16, group g16 = lane/16)
  // points at row 32kh + 16ks + 8c + 4(g16/2) + s/4, column
  // 32md + 16(g16%2) + 4(s%4), for PV k-step ks and half c of the 8 keys.
  const int vs16 = lane & 15, vgrp = lane >> 4;
  const int vrow0 = 32 * kh + 4 * (vgrp >> 1) + (vs16 >> 2);
  const int vcol0 = 16 * (vgrp & 1) + 4 * (vs16 & 3);

  // Prologue: the Q tile and block 0 by direct loads.  Q goes to V buffer 1,
  // which the first step refills only after every wave has taken its Q^T
  // fragments (the second barrier).  Loaded this way each instruction moves
  // whole rows; loads of the fragments straight from memory would touch 32
  // rows with 32 bytes each.  Q uses K's layout (granule g of row r at slot
  // g ^ (r mod G16)) and the rows of a partial last tile repeat its last row.
  // Q and O are touched once, so their loads and stores are non-temporal and
  // leave more of the caches to the K/V blocks that other rows reuse
  // (measured 1.0-1.3% faster at topk 0.1, bit-identical); split partials
  // small enough to stay in the last-level cache for the combine that reads
  // them next are the exception (o_nt = 0, set by the host).
  {
    const char* qbase = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.q) + bb * a.qs[0] +
                                                      hh * a.qs[1] + (int64_t)(64 * qt) * a.qs[2]);
    const int last = a.sq - 1 - 64 * qt;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int gi = 64 * (wave * NDMA + j) + lane;
      const int r = gi / G16, sl = gi % G16, rc = min(r, last);
      const uint32_t off = (uint32_t)((TILE + (wave * NDMA + j) * 64 * 8) * sizeof(T));
      dma16_nt(qbase, (uint32_t)((rc * a.qs[2] + (sl ^ (r % G16)) * 8) * (int64_t)sizeof(T)), sv_lds + off);
    }
  }
  issue_block(kb_of(0), 0);
  wait_dma();
  __syncthreads();
  // Q^T fragments (B operand): lane (query l32, half hl) holds d = 16kk + 8hl .. +7
  // of tile row 32 qh + l32.
  u32x4 qf[NKK];
  {
    const int qrow = 32 * qh + l32, qsw = qrow % G16;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = *reinterpret_cast<const u32x4*>(&sV[TILE + (qrow * G16 + ((2 * kk + hl) ^ qsw)) * 8]);
  }
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qf[kk]));
  __syncthreads();
  int kb_ahead = nloc > 1 ? kb_of(1) : 0;
  int kb_cur = MASKED ? kb_of(0) : 0;

  // pv_threshold: the decision on the current block: query row i of the
  // tile (lane i) has r_i = its maximum over the block's 64 keys and M_i its
  // running maximum over the blocks visited so far, this one included; the
  // block is dropped when r_i < M_i - tau for all 64 rows.  Every wave reads
  // the same values and takes the same decision.
  auto pv_keep_block = [&]() {
    const int vq = lane >> 5, vr = lane & 31;
    const float2v h0 = s_vote[vq * 32 + vr], h1 = s_vote[(2 + vq) * 32 + vr];
    const float r_i = fmaxf(h0[0], h1[0]), m_i = fmaxf(h0[1], h1[1]);
    return __any(!(r_i < m_i - a.pv_tau2));
  };

  // One 64-key block out of LDS buffer `cur` (a compile-time constant, so
  // every LDS address is a fixed register plus an immediate offset).
  auto step = [&](int it, auto cur_tag) {
    constexpr int cur = decltype(cur_tag)::value;
    const T* kt = &sK[0];
    const SPARGE_LDS T* vt = (const SPARGE_LDS T*)&sV[cur * TILE];

    asm volatile("" ::"s"(kb_ahead));   // the LUT load of the previous step has landed

    // The 8 K reads go out together, ahead of the S^T MFMAs; the V^T reads
    // follow once the next block's loads are issued (first half) and just
    // before the first PV MFMAs (second half), which keeps the registers
    // within three waves per SIMD.
    u32x4 kf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int g = (2 * kk + hl) ^ kswz;
      kf[kk] = *reinterpret_cast<const u32x4*>(&kt[(krow * G16 + g) * 8]);
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
    __builtin_amdgcn_sched_barrier(0);

    // S^T (32 keys x 32 queries) = K Q^T.
    floatx16 s = floatx16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s = mfma32<E>(kf[kk], qf[kk], s);
    __builtin_amdgcn_sched_barrier(0);

    // The block's row maximum of this lane's 16 scores (scaled, base 2),
    // after the position mask.
    auto block_max = [&]() {
      if constexpr (MASKED) {
        // Key 64 kb + 32 kh + 8 (r/4) + 4 hl + r%4 of register r against query
        // 64 qt + 32 qh + l32: keys past the query (causal) and keys past the
        // end of the sequence are removed.  Only the diagonal block, blocks
        // past it (listed by hand) and a partial last block can hold any.
        if (64 * kb_cur + 64 > a.sk || (a.causal && kb_cur >= qt)) {
          const int qpos = 64 * qt + 32 * qh + l32;
          const int lim = a.causal ? min(qpos + 1, a.sk) : a.sk;   // first removed key
          if constexpr (!PVSKIP) {
            // One value per lane against immediate offsets: this form left
            // the masked kernel 20 fewer bytes of spills (outside the loop)
            // and ran 0.5-3% faster; with a pv_threshold it spilled inside
            // the loop, so that variant keeps the per-key form below.
            const int rel = lim - (64 * kb_cur + 32 * kh + 4 * hl);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (8 * (r >> 2) + (r & 3) >= rel) s[r] = -INFINITY;
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = 64 * kb_cur + 32 * kh + 8 * (r >> 2) + 4 * hl + (r & 3);
              if (key >= lim) s[r] = -INFINITY;
            }
          }
        }
      }

      float rmax = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) rmax = fmaxf(rmax, s[r]);
      rmax = half_swap_max(rmax);
      return rmax * c2;
    };
    // Online softmax in base 2.  With a pv_threshold the row maxima are
    // needed before the first barrier, which publishes them as votes;
    // without one they are taken after it (measured 1% faster).
    float m_cand = 0.f;
    if constexpr (PVSKIP) {
      m_cand = block_max();
      // This wave's votes on the block, for its 32 query rows over its 32
      // keys: the block maximum and the running maximum, this block
      // included; the barrier below publishes them.
      m_top = fmaxf(m_top, m_cand);
      if (hl == 0) s_vote[wave * 32 + l32] = float2v{m_cand, m_top};
    }
    // Every wave has read this block's K: the K buffer, and the V buffer of
    // block it-1 (released by the last closing barrier), take block it+1.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (it + 1 < nloc) issue_block(kb_ahead, 1 - cur);
    // With a pv_threshold a dropped block reads no V^T and runs no PV MFMA.
    bool keep = true;
    if constexpr (PVSKIP) keep = pv_keep_block();
    if (keep) read_vt(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!PVSKIP) m_cand = block_max();

    const bool need = m_cand > m_run + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? m_cand : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NMD; ++i) acc_o[i] *= alpha;
    }
    // P^T fragments (k-step ks uses registers 8ks .. 8ks+7), rounded to the
    // input type for PV.  The row sum adds the fp32 values: rounding to the
    // input type moves a term by up to 2^-8 of itself (bf16), which on a row
    // carried by one key would move the LSE by up to 4e-3 nats.
    // Masked rows may still have no key (m_run = -inf): their P is 0.
    //
    // O^T += V^T P^T over this wave's 32 keys (unless a pv_threshold drops
    // the block for the tile).  The four
    // PV MFMAs of k-step 0 are issued as soon as its 8 P values exist, so the
    // exponentials of k-step 1 run in their shadow.  From the first PV MFMA to
    // the last the wave runs at raised priority: of the wavefronts sharing a
    // SIMD (one from each resident workgroup), the one about to finish its
    // block goes first and the others' softmax fills the MFMA shadows
    // (measured, bit-identical: the priority 1.5-2.4% at topk 0.4 and about 4%
    // at topk 0.1; the split issue 1% and 2% more; priority on the S MFMAs as
    // well gains nothing).
    const float mref = MASKED && m_run == -INFINITY ? 0.f : m_run;
    u32x4 pf[2];
    float p[16];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        p[8 * ks + 2 * w] = __builtin_amdgcn_exp2f(fmaf(s[8 * ks + 2 * w], c2, -mref));
        p[8 * ks + 2 * w + 1] = __builtin_amdgcn_exp2f(fmaf(s[8 * ks + 2 * w + 1], c2, -mref));
        pf[ks][w] = E::pack2(p[8 * ks + 2 * w], p[8 * ks + 2 * w + 1]);
        l_run += p[8 * ks + 2 * w] + p[8 * ks + 2 * w + 1];
      }
      __builtin_amdgcn_sched_barrier(0);
      if (ks == 0) {
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
        if (keep) read_vt(1);
      }
      if (keep) {
#pragma unroll
        for (int md = 0; md < NMD; ++md) acc_o[md] = mfma32<E>(vf[ks][md], pf[ks], acc_o[md]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);

    // The LUT entry of block it+2 is requested only now, after this block's
    // last LDS wait: scalar loads share the LDS wait counter but may return
    // out of order, so one in flight would turn every partial LDS wait above
    // into a full one.  The next step consumes it first thing.
    __builtin_amdgcn_sched_barrier(0);
    const int kb_next = it + 2 < nloc ? kb_of(it + 2) : 0;

    // Block it+1 must have landed before the barrier hands the buffers over.
    wait_dma();
    __syncthreads();
    if constexpr (MASKED) kb_cur = kb_ahead;
    kb_ahead = kb_next;
  };

#pragma unroll 1
  for (int it = 0; it < nloc; it += 2) {
    step(it, Buf<0>{});
    if (it + 1 == nloc) break;
    step(it + 1, Buf<1>{});
  }

  // Merge the two key halves: waves kh = 1 publish (m, l, O^T); waves kh = 0
  // combine and write the finished tile, in the output type, to LDS; then all
  // four waves store it with 16 bytes per lane, whole rows per instruction
  // (storing from the O^T fragments directly writes 8 or 16 bytes into each
  // of 32 rows per instruction).  Staged rows are [64][OG] 16-byte granules,
  // granule g of row r at slot g ^ (r mod OG), so neither the fragment writes
  // (32 rows, one column) nor the row reads meet the same banks.
  typedef typename OutType<T, OUT_F32>::type OT;
  constexpr int OG = D * (int)sizeof(OT) / 16;   // 16-byte granules per O row
  const float l_w = l_run + __shfl_xor(l_run, 32, kWave);
  float* mrg = reinterpret_cast<float*>(sV) + qh * (NMD * 16 * 64);
  float* ml = s_ml + qh * 64;
  // 16-bit rows are staged in the K buffer while the merge reads the V
  // buffers; fp32 rows (32 KB) go to the V buffers once it has read them.
  char* stg = OUT_F32 ? reinterpret_cast<char*>(sV) : reinterpret_cast<char*>(sK);
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
    // Causal: a query row whose listed keys all lie past it has no key at all
    // (both halves at -inf): O = 0, LSE = -inf.
    const bool empty = MASKED && m == -INFINITY;
    if (empty) m = 0.f;
    const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float l_tot = l_w * a0 + l1 * a1;
    const float inv = empty ? 0.f : 1.0f / l_tot;
    const float s0 = a0 * inv, s1 = a1 * inv;
    const int tr = 32 * qh + l32;                  // row of the tile
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
        // Columns 32 md + 8 g + 4 hl .. +3.
        if constexpr (OUT_F32) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_o[md][4 * g + i] = x[i];
        } else {
          const int gr = 4 * md + g;
          *reinterpret_cast<u32x2*>(srow + ((gr ^ (tr % OG)) * 16) + 8 * hl) =
              u32x2{E::pack2(x[0], x[1]), E::pack2(x[2], x[3])};
        }
      }
    }
    if (lse_row && hl == 0 && row_ok) lse_row[q0 + l32] = empty ? -INFINITY : (m + __log2f(l_tot)) * kLn2;
  }
  if constexpr (OUT_F32) {
    __syncthreads();
    if (kh == 0) {
      const int tr = 32 * qh + l32;
      char* srow = stg + tr * (OG * 16);
#pragma unroll
      for (int md = 0; md < NMD; ++md)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // Columns 32 md + 8 g + 4 hl .. +3.
          const int gr = 8 * md + 2 * g + hl;
          *reinterpret_cast<floatx4*>(srow + ((gr ^ (tr % OG)) * 16)) =
              floatx4{acc_o[md][4 * g], acc_o[md][4 * g + 1], acc_o[md][4 * g + 2], acc_o[md][4 * g + 3]};
        }
    }
  }
  __syncthreads();
  const int nrows = min(64, a.sq - 64 * qt);     // rows of a partial last tile
  OT* obase = reinterpret_cast<OT*>(a.o) + (int64_t)split * a.o_split_stride + bb * a.os[0] + hh * a.os[1] +
              (int64_t)(64 * qt) * a.os[2];
  auto store_rows = [&](auto nt_tag) {
#pragma unroll
    for (int k = 0; k < OG / 4; ++k) {
      const int idx = tid + 256 * k;
      const int r = idx / OG, gs = idx % OG;
      if (r < nrows) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * (OG * 16) + ((gs ^ (r % OG)) * 16));
        u32x4* dst = reinterpret_cast<u32x4*>(obase + (int64_t)r * a.os[2] + gs * (16 / (int)sizeof(OT)));
        if constexpr (decltype(nt_tag)::value) __builtin_nontemporal_store(v, dst);
        else *dst = v;
      }
    }
    // Ends the two store sequences differently, so the compiler does not
    // merge their last stores (which would drop the non-temporal hint).
    if constexpr (decltype(nt_tag)::value) asm volatile("" ::: "memory");
  };
  if (a.o_nt) store_rows(std::true_type{});
  else store_rows(std::false_type{});
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class E, int D, bool PVSKIP>
static void launch_block_v(const FmhaArgs& a, bool out_f32, dim3 grid, hipStream_t st) {
  if (a.causal || a.sk % 64) {
    if (out_f32) hipLaunchKernelGGL((fmha_block_kernel<E, D, true, true, PVSKIP>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((fmha_block_kernel<E, D, false, true, PVSKIP>), grid, dim3(256), 0, st, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((fmha_block_kernel<E, D, true, false, PVSKIP>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((fmha_block_kernel<E, D, false, false, PVSKIP>), grid, dim3(256), 0, st, a);
  }
}

template <class E, int D>
static hipError_t launch_block_t(const FmhaArgs& a, bool out_f32, hipStream_t st) {
  const int64_t nwg = block_grid(a.nqt, (int64_t)a.hq * a.b * a.splits, a.causal != 0);
  if (nwg > 0xFFFFFFFFll) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nwg);
  if (a.pv_tau2 > 0.f) launch_block_v<E, D, true>(a, out_f32, grid, st);
  else launch_block_v<E, D, false>(a, out_f32, grid, st);
  return hipGetLastError();
}

hipError_t launch_fmha_block(const FmhaArgs& a, sparge_dtype dt, sparge_dtype o_dt, int d,
                             hipStream_t st) {
  const bool f32 = o_dt == SPARGE_F32;
  if (dt == SPARGE_F16) return d == 128 ? launch_block_t<F16, 128>(a, f32, st) : launch_block_t<F16, 64>(a, f32, st);
  return d == 128 ? launch_block_t<BF16, 128>(a, f32, st) : launch_block_t<BF16, 64>(a, f32, st);
}

}  // namespace sparge
