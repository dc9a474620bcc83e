// Device helpers shared by the gfx950 kernels of the block-sparse attention
// library: element types, conversions, 64-lane wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparge.h"

namespace sparge {

typedef _Float16 half_t;
typedef __bf16 bf16_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Input element types: 16-bit storage with fp32 arithmetic.
struct F16 {
  typedef half_t T;
  typedef half8 V8;
  static __device__ __forceinline__ float to_f(T x) { return (float)x; }
  static __device__ __forceinline__ T from_f(float x) { return (T)x; }
  // Convert the low / high 16-bit lane of a packed word.
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(half_t, (uint16_t)(w & 0xFFFFu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(half_t, (uint16_t)(w >> 16));
  }
  // Pack two floats (round to nearest even) into one word, a in the low half
  // (one v_cvt_pk_f16_f32).
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v{a, b}), half2v));
  }
  // acc + lo(x) lo(y) + hi(x) hi(y), products exact, in fp32.
  static __device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, x), __builtin_bit_cast(half2v, y), acc, false);
  }
};

struct BF16 {
  typedef bf16_t T;
  typedef bf16x8 V8;
  static __device__ __forceinline__ float to_f(T x) { return (float)x; }
  static __device__ __forceinline__ T from_f(float x) { return (T)x; }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return __builtin_bit_cast(float, w << 16);
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xFFFF0000u);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v{a, b}), bf16x2v));
  }
  static __device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, x), __builtin_bit_cast(bf16x2v, y), acc, false);
  }
};

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP: shifts by
// 1, 2, 4 and 8 inside each row of 16 lanes (lanes without a source add 0),
// then the last lane of row 0 added to row 1 and of row 2 to row 3, then the
// last lane of row 1 (rows 0 + 1 by now) to rows 2 and 3.
__device__ __forceinline__ int wave_prefix_sum_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Maximum and sum over the 64 lanes of a wavefront, the same DPP steps (a
// lane without a source keeps -inf, or adds 0), read from the last lane.
__device__ __forceinline__ float wave_max_dpp(float x) {
  const int ninf = __builtin_bit_cast(int, -INFINITY);
#define SPARGE_MAX_STEP(ctrl, rows)                                                                      \
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), ctrl, \
                                                                     rows, 0xF, false)))
  SPARGE_MAX_STEP(0x111, 0xF);
  SPARGE_MAX_STEP(0x112, 0xF);
  SPARGE_MAX_STEP(0x114, 0xF);
  SPARGE_MAX_STEP(0x118, 0xF);
  SPARGE_MAX_STEP(0x142, 0xA);
  SPARGE_MAX_STEP(0x143, 0xC);
#undef SPARGE_MAX_STEP
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ __forceinline__ float wave_sum_dpp(float x) {
#define SPARGE_SUM_STEP(ctrl, rows, bc) \
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, rows, 0xF, bc))
  SPARGE_SUM_STEP(0x111, 0xF, true);
  SPARGE_SUM_STEP(0x112, 0xF, true);
  SPARGE_SUM_STEP(0x114, 0xF, true);
  SPARGE_SUM_STEP(0x118, 0xF, true);
  SPARGE_SUM_STEP(0x142, 0xA, false);
  SPARGE_SUM_STEP(0x143, 0xC, false);
#undef SPARGE_SUM_STEP
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Workgroups are dispatched to the 8 XCDs round-robin by linear id; give every
// XCD a contiguous range of logical ids (grid is a multiple of 8).
__device__ __forceinline__ int64_t xcd_remap(int64_t pid, int64_t grid) {
  const int64_t per = grid >> 3;
  return (pid & 7) * per + (pid >> 3);
}

// Sum over each group of 8 lanes (aligned), left in every lane of the group.
__device__ __forceinline__ float row8_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}

// Sum over each row of 16 lanes, left in every lane of the row, by data-parallel
// primitives (no LDS round trip): swap neighbours, swap pairs, mirror within
// 8, mirror within 16.  Each step adds a lane whose partial covers a disjoint
// set of the row's lanes.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

}  // namespace sparge
