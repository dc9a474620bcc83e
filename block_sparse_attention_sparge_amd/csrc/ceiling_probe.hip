// Throughput probes that put the block FMHA's roofline fraction in context.
// They are not part of the attention path: they build into their own
// library, which only the benchmark loads.
//
// Both kernels run a fixed number of iterations per wavefront and touch no
// global memory in their loop; each lane stores one float at the end, so
// `out` must hold workgroups * 256 floats.  Each iteration issues 16
// v_mfma_f32_32x32x16_f16 (32768 flops each) per wavefront.
//
//   kind 0 (mfma): the MFMAs alone, on fp16 operands held in registers and
//     drawn from a zero-mean bell-shaped distribution (like attention
//     inputs).  This is the rate the matrix pipes sustain under the part's
//     power limit on such data; with all-zero operands the same loop runs
//     at the nominal peak, with random ones well below it.
//   kind 1 (loop volume): the per-wavefront instruction volume of one
//     64-key block of the block FMHA at d = 128 (a wavefront owns 32 queries
//     and 32 keys), without its dependences:
//       - 8 ds_read_b128 and 16 ds_read_b64_tr_b16 (16 KB) whose results are
//         the A operands of the 16 MFMAs (K for S, V^T for PV);
//       - 8 ds_write_b128 (8 KB: one wavefront's share of the 32 KB of K and
//         V that a block's loads write into LDS);
//       - the softmax's VALU work on registers of its own: 7 max3 and a max,
//         16 fma, 16 exp2, 8 cvt_pk and 16 add.
//     No barriers, no global memory, and no MFMA waits for the softmax.
//     The FMHA runs the same volume with all of those, so its throughput
//     over this one says how much its dependences and memory cost.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sparge_probe.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
#define PROBE_LDS __attribute__((address_space(3)))

// A 32-bit integer hash (two multiply-xorshift rounds) for operand values.
__device__ inline uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Sum of four uniforms on [-1, 1), scaled to standard deviation 1.5.
__device__ inline float bell(uint32_t seed) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (float)((int)(mix(seed * 4u + i) & 0xFFFFFFu) - 8388608) * (1.0f / 8388608);
  return s * 1.299f;
}

__device__ inline uint32_t pack_half2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v{a, b}), half2v));
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void mfma_probe(float* out, int iters) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  half8 a[4], b[4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 8; ++j) {
      a[i][j] = (_Float16)bell(t * 64u + i * 8u + j);
      b[i][j] = (_Float16)bell(t * 64u + i * 8u + j + 0x40000000u);
    }
  floatx16 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        c[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(m + r) & 3], b[r], c[m], 0, 0, 0);
  }
  float s = 0.f;
  for (int m = 0; m < 4; ++m)
    for (int i = 0; i < 16; ++i) s += c[m][i];
  out[t] = s;
}

// LDS: a 24 KB read region (each iteration reads 16 KB from a base that
// moves by 2 KB, so the largest byte offset read is 6144 + 16384 - 1) and an
// 8 KB write region that the four wavefronts overwrite in turn (only the
// timing matters).  32 KB per workgroup: three fit on a CU, as in the FMHA.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void loop_volume_probe(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t rd[6144];
  __shared__ __attribute__((aligned(16))) uint32_t wr[2048];
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 6144; i += 256)
    rd[i] = pack_half2(bell(2u * i + 0x10000000u), bell(2u * i + 0x10000001u));
  __syncthreads();

  half8 b[4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 8; ++j) b[i][j] = (_Float16)bell(t * 64u + i * 8u + j + 0x40000000u);
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = 0.5f + 0.25f * bell(t * 16u + i + 0x20000000u) / 3.9f;
  float l = 0.f;
  floatx16 c[4] = {};
  const uint32_t wbase = (uint32_t)(uintptr_t)((PROBE_LDS void*)&wr[4 * lane]);

  for (int it = 0; it < iters; ++it) {
    const PROBE_LDS uint32_t* base = (const PROBE_LDS uint32_t*)rd + 512 * (it & 3);
    // S: 8 MFMAs on K fragments, one ds_read_b128 (1 KB per wavefront) each.
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 k = *reinterpret_cast<const PROBE_LDS u32x4*>(base + 256 * kk + 4 * lane);
      c[kk & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, k), b[kk & 3], c[kk & 3], 0, 0, 0);
    }
    // Softmax volume on registers the MFMAs do not use.
    float m = x[0];
#pragma unroll
    for (int i = 1; i < 15; i += 2) m = fmaxf(fmaxf(m, x[i]), x[i + 1]);
    m = fmaxf(m, x[15]);
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(fmaf(x[i], 1.0009765625f, -m));
#pragma unroll
    for (int i = 0; i < 8; ++i) pk[i] = pack_half2(x[2 * i], x[2 * i + 1]);
#pragma unroll
    for (int i = 0; i < 16; ++i) l += x[i];
    // PV: 8 MFMAs on V^T fragments, two ds_read_b64_tr_b16 (512 B each) per
    // fragment, from the upper 8 KB of this iteration's 16 KB.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const PROBE_LDS uint32_t* vp = base + 2048 + 256 * j + 2 * lane;
      const short4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PROBE_LDS short4v*)vp);
      const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PROBE_LDS short4v*)(vp + 128));
      const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
      const u32x4 v = {w0[0], w0[1], w1[0], w1[1]};
      c[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, v), b[(j + 1) & 3], c[j & 3], 0, 0, 0);
    }
    // 8 KB of LDS writes per wavefront; two of them carry the packed P.
    const u32x4 w0 = {pk[0], pk[1], pk[2], pk[3]}, w1 = {pk[4], pk[5], pk[6], pk[7]};
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t addr = wbase + 1024u * w;   // < 8192: inside wr
      const u32x4 val = w == 0 ? w0 : w == 1 ? w1 : u32x4{(uint32_t)it, (uint32_t)w, 0u, 0u};
      asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(val));
    }
  }
  __syncthreads();
  float s = l + (float)(wr[threadIdx.x] & 1u);
  for (int mm = 0; mm < 4; ++mm)
    for (int i = 0; i < 16; ++i) s += c[mm][i];
  out[t] = s;
}

}  // namespace

extern "C" int sparge_probe_launch(int kind, int workgroups, int iters, float* out, void* stream) {
  if (kind != SPARGE_PROBE_MFMA && kind != SPARGE_PROBE_LOOP_VOLUME) return (int)hipErrorInvalidValue;
  if (workgroups < 1 || workgroups > SPARGE_PROBE_MAX_WORKGROUPS) return (int)hipErrorInvalidValue;
  if (iters < 1 || iters > SPARGE_PROBE_MAX_ITERS || out == nullptr) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (kind == SPARGE_PROBE_MFMA)
    hipLaunchKernelGGL(mfma_probe, dim3(workgroups), dim3(256), 0, s, out, iters);
  else
    hipLaunchKernelGGL(loop_volume_probe, dim3(workgroups), dim3(256), 0, s, out, iters);
  return (int)hipGetLastError();
}

extern "C" double sparge_probe_flops(int workgroups, int iters) {
  return (double)workgroups * 4.0 * (double)iters * 16.0 * 32768.0;
}
