// Device helpers shared by the attention kernels (fp16 / bf16 and 8-bit-QK
// block kernels, token-list kernel): constants, the 32x32 MFMA wrappers, the
// output store, the loads from memory straight into LDS, the half-wave
// maximum, and the order in which the block kernels take their rows.
#pragma once

#include "common.h"

namespace sparge {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Index of the first negative entry of a LUT row (or its length), by one wave.
__device__ __forceinline__ int first_negative(const int32_t* row, int len, int lane) {
  int first = len;
  for (int i = lane; i < len; i += kWave) {
    if (row[i] < 0) { first = i; break; }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) first = min(first, __shfl_xor(first, m, kWave));
  return first;
}

template <class E>
__device__ __forceinline__ floatx16 mfma32(const u32x4& a, const u32x4& b, const floatx16& c);

template <>
__device__ __forceinline__ floatx16 mfma32<F16>(const u32x4& a, const u32x4& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ floatx16 mfma32<BF16>(const u32x4& a, const u32x4& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <class E, bool OUT_F32>
__device__ __forceinline__ void store4(void* base, int64_t off, float x0, float x1, float x2, float x3) {
  if constexpr (OUT_F32) {
    floatx4 v = {x0, x1, x2, x3};
    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(base) + off) = v;
  } else {
    u32x2 v = {E::pack2(x0, x1), E::pack2(x2, x3)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<typename E::T*>(base) + off) = v;
  }
}

// The running maximum is only moved when a row's new maximum exceeds it by
// more than 2^8 (base-2 units); see the block kernels.
constexpr float kRescaleSlack = 8.0f;

typedef short short4v __attribute__((ext_vector_type(4)));
#define SPARGE_LDS __attribute__((address_space(3)))

// 16 bytes from global memory at (wave-uniform base) + (per-lane 32-bit
// offset) into LDS at (wave-uniform base) + 16 * lane.  The global base is a
// scalar register pair, so moving to another block costs no vector ALU work.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t goff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base), "v"(goff), "s"(gbase)
               : "memory", "m0");
}

// The same load marked non-temporal, for data read once (a Q tile): it then
// displaces less of the K/V blocks that other rows reuse from the caches.
__device__ __forceinline__ void dma16_nt(const void* gbase, uint32_t goff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds_base), "v"(goff), "s"(gbase)
               : "memory", "m0");
}

// Word 3 of a raw buffer resource on gfx9-family parts (gfx950): 32-bit
// data format, no swizzle, so offsets count bytes and an access at or past
// the record count reads zero.
constexpr int kBufferWord3 = 0x00020000;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A raw buffer resource over `bytes` bytes from `base` (wave-uniform).
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)p, (int)(uint32_t)(p >> 32), bytes, kBufferWord3};
}

// 16 bytes through a buffer resource at (per-lane 32-bit offset) + (wave-
// uniform offset) into LDS at (wave-uniform base) + 16 * lane; an offset at
// or past the resource's record count delivers zeros.
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, uint32_t off, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(off), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// max(x, x of lane l ^ 32).  v_permlane32_swap exchanges lanes 32..63 of its
// first operand with lanes 0..31 of its second; with x in both, every lane
// then holds its own value in one register and its partner's in the other.
// Written in assembly because both outputs are needed (the s_nop covers the
// VALU-write-to-permlane hazard).
__device__ __forceinline__ float half_swap_max(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// The order in which the block kernels take their rows.  A row is one Q-tile
// of one row group (batch, head, split); the 8 XCDs receive workgroups
// round-robin by id (aiter 4919 page), and each XCD has its own L2.
//   * Contiguous: each XCD takes a contiguous range of row groups, so its
//     concurrent rows are tiles of one head, which share that head's K/V in
//     its L2.  Causal launches take each group's tiles last first: causal
//     rows grow with the tile index, so an XCD ends on short rows.
//   * Interleaved: XCD x takes tiles x, x + 8, x + 16, ... of every row group
//     in turn, so every XCD gets an equal share of each head whatever its
//     list lengths (a per-head topk).  With whole heads per XCD the heads of
//     the per-head topk sweep loaded the XCDs unevenly (measured 0-2.9%
//     faster on that sweep over three boxes, within 1% elsewhere).
// Launches of at least kInterleaveRows rows (several rounds of resident
// workgroups) are interleaved, unless causal: dealt like the others, causal
// launches ran 7-20% slower, and so did a one-round launch (b1 h8 s4096,
// 512 rows: 9%), whose balance across XCDs does not matter and whose L2
// then holds eight heads' K/V instead of one.
constexpr int64_t kInterleaveRows = 4096;

__host__ __device__ inline bool block_interleaved(int nqt, int64_t groups, bool causal) {
  return !causal && (int64_t)nqt * groups >= kInterleaveRows;
}

// block_grid() is the grid size for the order; block_row_of() returns false
// for a workgroup past the end.
__host__ __device__ inline int64_t block_grid(int nqt, int64_t groups, bool causal) {
  return block_interleaved(nqt, groups, causal) ? 8 * (int64_t)((nqt + 7) / 8) * groups
                                                : ((int64_t)nqt * groups + 7) / 8 * 8;
}

__device__ __forceinline__ bool block_row_of(int nqt, int64_t groups, bool causal, int& qt, int64_t& group) {
  if (!block_interleaved(nqt, groups, causal)) {
    const int64_t lin = xcd_remap(blockIdx.x, gridDim.x);
    if (lin >= (int64_t)nqt * groups) return false;
    const int t = (int)(lin % nqt);
    qt = causal ? nqt - 1 - t : t;
    group = lin / nqt;
    return true;
  }
  const int per_xcd = (nqt + 7) >> 3;
  const int64_t j = blockIdx.x >> 3;
  group = j / per_xcd;
  qt = (int)(blockIdx.x & 7) + 8 * (int)(j % per_xcd);
  return group < groups && qt < nqt;
}

// Compile-time buffer index for the two-way unrolled block loop.
template <int N>
struct Buf {
  static constexpr int value = N;
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace sparge
