// Internal kernel-argument structs and launchers of the gfx950 block-sparse
// attention library.  Host entry points (abi.hip) validate arguments and call
// these; each launcher enqueues its kernels on the given stream and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparge.h"

namespace sparge {

struct PoolArgs {
  const void* q;
  const void* k;
  int64_t qs[3];
  int64_t ks[3];
  int b, h, nq, nk;
  int h_kv;          // K heads (h is a multiple)
  int sq, sk;        // tokens; the last block of each may be partial
  float* q_mean;     // [b, h, nq, d]
  float* k_mean;     // [b, h_kv, nk, d]
  uint8_t* sim_q;    // [b, h, nq] Q gate flags
  float* k_sim;      // [b, h_kv, nk] K block similarity (each query head gates it)
  // K smoothing: per-chunk sums of K over the sequence, [b, h, km_chunks, d];
  // km = (sum over chunks) * km_scale.  Null when K is pooled as given.
  float* km_part;
  int km_chunks;
  float km_scale;    // 1 / s_k
  // int8 codes of Q and K per 64-token block ([b, h, s, d] contiguous) and
  // their scales ([b, h, nq], [b, h, nk]); null when not requested.
  int8_t* q_i8;
  int8_t* k_i8;
  float* q_i8_scale;
  float* k_i8_scale;
  int quant_fp8;     // the codes are fp8 e4m3 bytes (scale absmax / 448), not int8
  float thr[SPARGE_MAX_HEADS];
};

// K rows summed per partial of the K sequence mean (16 blocks of 64).
constexpr int kKmChunkRows = 1024;

struct SelectArgs {
  const float* q_mean;
  const float* k_mean;     // [b, h_kv, nk, d]
  const uint8_t* sim_q;
  const float* k_sim;      // [b, h_kv, nk]
  uint8_t* sim_k;          // [b, h, nk] K gate flags as each query head sees them, or null
  int b, h, nq, nk;
  int h_kv;
  float scale;
  int32_t* lut;      // [b, h, nq, nk]
  int32_t* count;    // [b, h, nq]
  uint8_t* bmap;     // [b, h, nq, nk] or null
  float* prob;       // [b, h, nq, nk] or null
  int causal;        // blocks kb > qb masked, counts clamped to qb + 1
  int sink;          // block 0 forced on
  int nsel[SPARGE_MAX_HEADS];   // > 0: top-k count; <= 0: cdf mode
  float cdf[SPARGE_MAX_HEADS];
  float thr[SPARGE_MAX_HEADS];  // simthreshd1
};

struct FmhaArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs[3], ks[3], vs[3], os[3];
  int b, hq, hkv, sq, sk;
  int ratio;               // hq / hkv
  const int32_t* lut;      // null => dense
  const int32_t* cnt;      // null => up to the first -1
  int lut_row_len;
  int lut_heads;
  int nqt;                 // rows per (b, lut head): q tiles, or query positions
  int nkb;                 // K blocks (block mode)
  float scale_log2;        // softmax scale * log2(e)
  int splits;
  int64_t o_split_stride;  // elements
  int o_nt;                // block kernel: O rows leave with non-temporal stores
  int causal;              // block mode: key j > query i masked
  float pv_tau2;           // block mode: pv_threshold * log2(e); 0 = no PV skip
  // int8-QK block kernel: q and k hold int8 codes; their per-block scales.
  const float* q_scale;    // [b, hq, nqt]
  const float* k_scale;    // [b, hkv, nkb]
  // Token-list mode: the query rows of a KV head are served in groups of up
  // to 8, one workgroup per group.
  int tok_groups;
};

struct CombineArgs {
  const void* parts;
  const float* lse_parts;
  int n_parts;
  int64_t rows;            // b * h * s
  int64_t part_stride;     // elements
  void* o;
  float* lse_out;
};

hipError_t launch_key_mean(const PoolArgs& a, sparge_dtype dt, int d, hipStream_t st);
hipError_t launch_pool_sim(const PoolArgs& a, sparge_dtype dt, int d, hipStream_t st);
hipError_t launch_score_select(const SelectArgs& a, int d, hipStream_t st);
hipError_t launch_fmha_block(const FmhaArgs& a, sparge_dtype dt, sparge_dtype o_dt, int d,
                             hipStream_t st);
hipError_t launch_fmha_qk8(const FmhaArgs& a, sparge_dtype v_dt, sparge_dtype o_dt, int d, bool fp8,
                           hipStream_t st);
hipError_t launch_fmha_tokens(const FmhaArgs& a, sparge_dtype dt, sparge_dtype o_dt, int d,
                              int rows_per_group, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, sparge_dtype part_dt, sparge_dtype out_dt,
                          int d, hipStream_t st);
hipError_t launch_validate_lut(const int32_t* lut, const int32_t* cnt, int64_t rows,
                               int row_len, int n_blocks, int32_t* bad, hipStream_t st);

}  // namespace sparge
