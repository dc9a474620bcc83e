// LSE combine of partial attention results, and a LUT checker, on gfx950.
//
// Combine ("Updating Log -- Speculative Sparse Attention" page, Stage 1:
// FA(A u B) = Combine(FA(A), FA(B)) with the running-maximum trick; aiter 4919
// page: the reduce is pure bandwidth, partials with a -inf maximum are masked
// before the exponential, and one reciprocal per row replaces a divide per
// element).  Per row: m = max_i LSE_i, w_i = exp(LSE_i - m) (0 for -inf),
// O = sum_i w_i O_i / sum_i w_i, LSE = m + ln sum_i w_i; all parts -inf gives
// O = 0, LSE = -inf.
//
// Layout: each thread owns 8 consecutive d values of one row (16 or 32 bytes
// per part), so a wavefront reads whole rows of every part with 16-byte loads.
#include "common.h"
#include "kernels.h"

namespace sparge {

template <class P>
struct PartLoad;

template <>
struct PartLoad<float> {
  static __device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
    const floatx4* p = reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(base) + off);
    const floatx4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  }
};

template <class E>
struct PartLoadE {
  static __device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
    const u32x4 w = load16(reinterpret_cast<const typename E::T*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = E::lo(w[i]); x[2 * i + 1] = E::hi(w[i]); }
  }
};
template <> struct PartLoad<F16> : PartLoadE<F16> {};
template <> struct PartLoad<BF16> : PartLoadE<BF16> {};

template <class O>
struct OutStore;

template <>
struct OutStore<float> {
  static __device__ __forceinline__ void store8(void* base, int64_t off, const float (&x)[8]) {
    floatx4* p = reinterpret_cast<floatx4*>(reinterpret_cast<float*>(base) + off);
    p[0] = floatx4{x[0], x[1], x[2], x[3]};
    p[1] = floatx4{x[4], x[5], x[6], x[7]};
  }
};

template <class E>
struct OutStoreE {
  static __device__ __forceinline__ void store8(void* base, int64_t off, const float (&x)[8]) {
    u32x4 w = {E::pack2(x[0], x[1]), E::pack2(x[2], x[3]), E::pack2(x[4], x[5]), E::pack2(x[6], x[7])};
    store16(reinterpret_cast<typename E::T*>(base) + off, w);
  }
};
template <> struct OutStore<F16> : OutStoreE<F16> {};
template <> struct OutStore<BF16> : OutStoreE<BF16> {};

template <class P, class O, int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int TPR = D / 8;   // threads per row
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gt / TPR;
  if (row >= a.rows) return;
  const int c = (int)(gt % TPR);

  float m = -INFINITY;
  for (int i = 0; i < a.n_parts; ++i) m = fmaxf(m, a.lse_parts[(int64_t)i * a.rows + row]);

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m > -INFINITY) {
    for (int i = 0; i < a.n_parts; ++i) {
      const float li = a.lse_parts[(int64_t)i * a.rows + row];
      if (!(li > -INFINITY)) continue;
      const float w = expf(li - m);
      float x[8];
      PartLoad<P>::load8(a.parts, (int64_t)i * a.part_stride + row * D + c * 8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[e], acc[e]);
      wsum += w;
    }
  }
  const bool live = wsum > 0.f;
  const float inv = live ? 1.0f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  OutStore<O>::store8(a.o, row * D + c * 8, acc);
  if (a.lse_out && c == 0) a.lse_out[row] = live ? m + logf(wsum) : -INFINITY;
}

// The same combine for grids too small to hide memory latency by occupancy
// (split-K decode: a few thousand rows).  The kernel above walks the parts one
// dependent load at a time, twice; here every LSE is requested at once, then
// every live part's 8 values, so a thread waits about two memory latencies
// instead of 2 * n_parts.  The arithmetic is the same, in the same order, so
// the results are bit-identical.  n_parts <= PN.
template <class P, class O, int D, int PN>
__global__ __launch_bounds__(256) void combine_small_kernel(CombineArgs a) {
  constexpr int TPR = D / 8;   // threads per row
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gt / TPR;
  if (row >= a.rows) return;
  const int c = (int)(gt % TPR);

  float l[PN];
#pragma unroll
  for (int i = 0; i < PN; ++i) l[i] = i < a.n_parts ? a.lse_parts[(int64_t)i * a.rows + row] : -INFINITY;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < PN; ++i) m = fmaxf(m, l[i]);

  float x[PN][8];
#pragma unroll
  for (int i = 0; i < PN; ++i) {
    if (l[i] > -INFINITY) {
      PartLoad<P>::load8(a.parts, (int64_t)i * a.part_stride + row * D + c * 8, x[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
    }
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m > -INFINITY) {
#pragma unroll
    for (int i = 0; i < PN; ++i) {
      if (!(l[i] > -INFINITY)) continue;
      const float w = expf(l[i] - m);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[i][e], acc[e]);
      wsum += w;
    }
  }
  const bool live = wsum > 0.f;
  const float inv = live ? 1.0f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  OutStore<O>::store8(a.o, row * D + c * 8, acc);
  if (a.lse_out && c == 0) a.lse_out[row] = live ? m + logf(wsum) : -INFINITY;
}

// Grids of at most this many workgroups (8 per CU) take the small-grid kernel
// when the parts fit its registers.
constexpr int64_t kCombineSmallGrid = 2048;

template <class P, class O, int D>
static void launch_combine_pod(const CombineArgs& a, dim3 grid, hipStream_t st) {
  if ((int64_t)grid.x <= kCombineSmallGrid && a.n_parts <= 4)
    hipLaunchKernelGGL((combine_small_kernel<P, O, D, 4>), grid, dim3(256), 0, st, a);
  else if ((int64_t)grid.x <= kCombineSmallGrid && a.n_parts <= 16)
    hipLaunchKernelGGL((combine_small_kernel<P, O, D, 16>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((combine_kernel<P, O, D>), grid, dim3(256), 0, st, a);
}

template <class P, class O>
static hipError_t launch_combine_po(const CombineArgs& a, int d, hipStream_t st) {
  const int64_t threads = a.rows * (d / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (d == 128) launch_combine_pod<P, O, 128>(a, grid, st);
  else launch_combine_pod<P, O, 64>(a, grid, st);
  return hipGetLastError();
}

template <class P>
static hipError_t launch_combine_p(const CombineArgs& a, sparge_dtype out_dt, int d, hipStream_t st) {
  switch (out_dt) {
    case SPARGE_F32: return launch_combine_po<P, float>(a, d, st);
    case SPARGE_F16: return launch_combine_po<P, F16>(a, d, st);
    default: return launch_combine_po<P, BF16>(a, d, st);
  }
}

hipError_t launch_combine(const CombineArgs& a, sparge_dtype part_dt, sparge_dtype out_dt, int d,
                          hipStream_t st) {
  switch (part_dt) {
    case SPARGE_F32: return launch_combine_p<float>(a, out_dt, d, st);
    case SPARGE_F16: return launch_combine_p<F16>(a, out_dt, d, st);
    default: return launch_combine_p<BF16>(a, out_dt, d, st);
  }
}

// ---------------------------------------------------------------------------
// LUT checker: one workgroup walks every row and counts the bad ones.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void validate_lut_kernel(const int32_t* lut, const int32_t* cnt,
                                                            int64_t rows, int row_len, int n_blocks,
                                                            int32_t* bad) {
  __shared__ int partial[1024];
  int my_bad = 0;
  for (int64_t r = threadIdx.x; r < rows; r += blockDim.x) {
    const int32_t* row = lut + r * row_len;
    int n;
    bool ok = true;
    if (cnt) {
      n = cnt[r];
      if (n < 0 || n > row_len) { ok = false; n = 0; }
    } else {
      n = row_len;
      for (int i = 0; i < row_len; ++i)
        if (row[i] < 0) { n = i; break; }
    }
    int prev = -1;
    for (int i = 0; i < n && ok; ++i) {
      const int x = row[i];
      if (x <= prev || x >= n_blocks) ok = false;
      prev = x;
    }
    for (int i = n; i < row_len && ok; ++i)
      if (row[i] != -1) ok = false;
    my_bad += ok ? 0 : 1;
  }
  partial[threadIdx.x] = my_bad;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) partial[threadIdx.x] += partial[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) bad[0] = partial[0];
}

hipError_t launch_validate_lut(const int32_t* lut, const int32_t* cnt, int64_t rows, int row_len,
                               int n_blocks, int32_t* bad, hipStream_t st) {
  hipLaunchKernelGGL(validate_lut_kernel, dim3(1), dim3(1024), 0, st, lut, cnt, rows, row_len,
                     n_blocks, bad);
  return hipGetLastError();
}

}  // namespace sparge
