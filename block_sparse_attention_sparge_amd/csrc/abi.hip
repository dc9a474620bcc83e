// Host entry points of the C ABI declared in include/sparge.h.
//
// Every call validates its arguments on the host first; on any error nothing is
// enqueued, the status is returned and the message is kept per thread for
// sparge_last_error().  Valid calls only enqueue kernels on the caller's stream:
// the library never allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include <algorithm>

#include "common.h"
#include "kernels.h"

using namespace sparge;

namespace {

thread_local std::string g_error;

sparge_status fail(sparge_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

sparge_status ok() {
  g_error.clear();
  return SPARGE_OK;
}

sparge_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(SPARGE_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Strides of a [b, h, s, d] tensor: non-negative, rows 16-byte aligned.
sparge_status check_strides(const char* name, const int64_t* st) {
  if (!st) return fail(SPARGE_ERR_INVALID, "%s strides are null", name);
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(SPARGE_ERR_INVALID, "%s stride %d is negative", name, i);
    if (st[i] % 8 != 0)
      return fail(SPARGE_ERR_INVALID, "%s stride %d (%lld elements) does not keep rows 16-byte aligned",
                  name, i, (long long)st[i]);
  }
  return SPARGE_OK;
}

bool is_half(sparge_dtype dt) { return dt == SPARGE_F16 || dt == SPARGE_BF16; }
int dtype_size(sparge_dtype dt) { return dt == SPARGE_F32 ? 4 : 2; }
// Split partials of at most this many bytes are stored through the caches.
constexpr int64_t kSplitCachedBytes = int64_t(128) << 20;

struct BlockMapLayout {
  size_t q_mean, k_mean, sim_q, k_sim, km_part, total;
  int km_chunks;
};

BlockMapLayout block_map_layout(int b, int h, int s_q, int s_k, int d) {
  const size_t nq = ((size_t)s_q + 63) / 64, nk = ((size_t)s_k + 63) / 64, bh = (size_t)b * h;
  BlockMapLayout l;
  l.km_chunks = (s_k + sparge::kKmChunkRows - 1) / sparge::kKmChunkRows;
  size_t off = 0;
  l.q_mean = off; off = align256(off + bh * nq * d * sizeof(float));
  l.k_mean = off; off = align256(off + bh * nk * d * sizeof(float));
  l.sim_q = off;  off = align256(off + bh * nq);
  l.k_sim = off;  off = align256(off + bh * nk * sizeof(float));
  l.km_part = off; off = align256(off + bh * (size_t)l.km_chunks * d * sizeof(float));
  l.total = off;
  return l;
}

// Device scratch of sparge_build_block_map_noalloc: one copy per GPU, held
// until the process ends.  In host code `scratch` is only a host-side handle;
// its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[SPARGE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of this device's scratch array (looked up on the first call made
// with that device current; no allocation).
sparge_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SPARGE_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(SPARGE_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPARGE_OK;
}

}  // namespace

extern "C" {

int sparge_abi_version(void) { return 7; }

const char* sparge_last_error(void) { return g_error.c_str(); }

size_t sparge_build_block_map_workspace(int b, int h, int s_q, int s_k, int d, int blk_q, int blk_k) {
  if (b <= 0 || h <= 0 || s_q <= 0 || s_k <= 0 || (d != 64 && d != 128)) return 0;
  if (blk_q != 64 || blk_k != 64) return 0;
  return block_map_layout(b, h, s_q, s_k, d).total;
}

}  // extern "C"

namespace {

// Both block-map entry points.  With use_scratch the workspace arguments are
// ignored and, once every argument has passed the host checks, this device's
// scratch array serves as the workspace.
sparge_status block_map_impl(
    const void* q, const void* k, sparge_dtype dt, int b, int h, int h_kv, int s_q, int s_k, int d,
    const int64_t q_strides[3], const int64_t k_strides[3], int blk_q, int blk_k,
    const float* topk, const float* cdfthreshd, const float* simthreshd1, float softmax_scale,
    unsigned flags, int32_t* lut, int32_t* lut_count, uint8_t* block_map, float* pooled_prob, uint8_t* sim_q,
    uint8_t* sim_k, float* q_mean, float* k_mean, int8_t* q_i8, float* q_i8_scale, int8_t* k_i8,
    float* k_i8_scale, void* workspace, size_t workspace_bytes, bool use_scratch, void* stream) {
  if (!q || !k) return fail(SPARGE_ERR_INVALID, "q and k must be non-null");
  if (!lut || !lut_count) return fail(SPARGE_ERR_INVALID, "lut and lut_count must be non-null");
  if (!topk || !simthreshd1) return fail(SPARGE_ERR_INVALID, "topk and simthreshd1 must be non-null");
  if (!is_half(dt)) return fail(SPARGE_ERR_UNSUPPORTED, "q/k dtype must be F16 or BF16");
  if (b <= 0 || h <= 0 || h_kv <= 0 || s_q <= 0 || s_k <= 0 || d <= 0)
    return fail(SPARGE_ERR_INVALID, "sizes must be positive (b=%d h=%d h_kv=%d s_q=%d s_k=%d d=%d)", b, h, h_kv,
                s_q, s_k, d);
  if (h % h_kv) return fail(SPARGE_ERR_INVALID, "h=%d is not a multiple of h_kv=%d", h, h_kv);
  if (d != 64 && d != 128) return fail(SPARGE_ERR_UNSUPPORTED, "head dim %d not built (64, 128)", d);
  if (blk_q != 64 || blk_k != 64)
    return fail(SPARGE_ERR_UNSUPPORTED, "block map needs blk_q = blk_k = 64 (got %d, %d)", blk_q, blk_k);
  if (h > SPARGE_MAX_HEADS) return fail(SPARGE_ERR_UNSUPPORTED, "h=%d exceeds %d", h, SPARGE_MAX_HEADS);
  const int nq = (s_q + 63) / 64, nk = (s_k + 63) / 64;   // a partial last block counts
  if (nk > SPARGE_MAX_KBLOCKS)
    return fail(SPARGE_ERR_UNSUPPORTED, "nk=%d K blocks exceeds %d", nk, SPARGE_MAX_KBLOCKS);
  sparge_status st;
  if ((st = check_strides("q", q_strides)) != SPARGE_OK) return st;
  if ((st = check_strides("k", k_strides)) != SPARGE_OK) return st;
  if (!aligned16(q) || !aligned16(k)) return fail(SPARGE_ERR_INVALID, "q/k must be 16-byte aligned");
  if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
    return fail(SPARGE_ERR_INVALID, "softmax_scale must be finite and >= 0");
  if (flags & ~(SPARGE_FLAG_SMOOTH_K | SPARGE_FLAG_CAUSAL | SPARGE_FLAG_ATTN_SINK | SPARGE_FLAG_QUANT_FP8))
    return fail(SPARGE_ERR_INVALID, "unknown flag bits 0x%x", flags);
  const bool causal = (flags & SPARGE_FLAG_CAUSAL) != 0;
  if (causal && s_q != s_k)
    return fail(SPARGE_ERR_UNSUPPORTED, "causal block map needs s_q = s_k (got %d, %d)", s_q, s_k);
  const BlockMapLayout lay = block_map_layout(b, h, s_q, s_k, d);
  if (use_scratch) {
    if (lay.total > (size_t)SPARGE_NOALLOC_SCRATCH_BYTES)
      return fail(SPARGE_ERR_UNSUPPORTED,
                  "these sizes need %zu bytes of scratch; the allocation-free entry point holds %zu "
                  "(use sparge_build_block_map with a workspace)",
                  lay.total, (size_t)SPARGE_NOALLOC_SCRATCH_BYTES);
  } else {
    if (!workspace || workspace_bytes < lay.total)
      return fail(SPARGE_ERR_INVALID, "workspace of %zu bytes needed (got %zu)", lay.total, workspace_bytes);
    if (((uintptr_t)workspace & 255u) != 0) return fail(SPARGE_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  if ((q_mean && ((uintptr_t)q_mean & 15u)) || (k_mean && ((uintptr_t)k_mean & 15u)))
    return fail(SPARGE_ERR_INVALID, "q_mean/k_mean must be 16-byte aligned");
  const int n_i8 = (q_i8 != nullptr) + (q_i8_scale != nullptr) + (k_i8 != nullptr) + (k_i8_scale != nullptr);
  if (n_i8 != 0 && n_i8 != 4)
    return fail(SPARGE_ERR_INVALID, "q_i8, q_i8_scale, k_i8 and k_i8_scale go together (all or none)");
  if (n_i8 && (!aligned16(q_i8) || !aligned16(k_i8)))
    return fail(SPARGE_ERR_INVALID, "q_i8/k_i8 must be 16-byte aligned");
  if ((flags & SPARGE_FLAG_QUANT_FP8) && n_i8 != 4)
    return fail(SPARGE_ERR_INVALID, "SPARGE_FLAG_QUANT_FP8 needs the four code outputs");

  PoolArgs pa;
  SelectArgs sa;
  for (int i = 0; i < h; ++i) {
    const float tk = topk[i], thr = simthreshd1[i];
    if (!isfinite(tk) || tk > 1.f) return fail(SPARGE_ERR_INVALID, "topk[%d]=%g must be finite and <= 1", i, tk);
    if (!isfinite(thr)) return fail(SPARGE_ERR_INVALID, "simthreshd1[%d] is not finite", i);
    pa.thr[i] = thr;
    sa.thr[i] = thr;
    if (tk > 0.f) {
      long n = (long)floor((double)tk * (double)nk);
      if (n < 1) n = 1;
      if (n > nk) n = nk;
      sa.nsel[i] = (int)n;
      sa.cdf[i] = 0.f;
    } else {
      if (!cdfthreshd) return fail(SPARGE_ERR_INVALID, "topk[%d] <= 0 needs cdfthreshd", i);
      const float c = cdfthreshd[i];
      if (!isfinite(c) || !(c > 0.f) || c > 1.f)
        return fail(SPARGE_ERR_INVALID, "cdfthreshd[%d]=%g must be in (0, 1]", i, c);
      sa.nsel[i] = 0;
      sa.cdf[i] = c;
    }
  }
  for (int i = h; i < SPARGE_MAX_HEADS; ++i) { pa.thr[i] = 0.f; sa.thr[i] = 0.f; sa.nsel[i] = 1; sa.cdf[i] = 0.f; }
  if (use_scratch) {
    // Every argument is valid: only now touch the device.
    const sparge_status sst = scratch_for_current_device(&workspace);
    if (sst != SPARGE_OK) return sst;
  }

  char* ws = reinterpret_cast<char*>(workspace);
  pa.q = q;
  pa.k = k;
  for (int i = 0; i < 3; ++i) { pa.qs[i] = q_strides[i]; pa.ks[i] = k_strides[i]; }
  pa.b = b; pa.h = h; pa.h_kv = h_kv; pa.nq = nq; pa.nk = nk; pa.sq = s_q; pa.sk = s_k;
  pa.q_mean = q_mean ? q_mean : reinterpret_cast<float*>(ws + lay.q_mean);
  pa.k_mean = k_mean ? k_mean : reinterpret_cast<float*>(ws + lay.k_mean);
  pa.sim_q = sim_q ? sim_q : reinterpret_cast<uint8_t*>(ws + lay.sim_q);
  pa.k_sim = reinterpret_cast<float*>(ws + lay.k_sim);
  const bool smooth = (flags & SPARGE_FLAG_SMOOTH_K) != 0;
  pa.km_part = smooth ? reinterpret_cast<float*>(ws + lay.km_part) : nullptr;
  pa.km_chunks = lay.km_chunks;
  pa.km_scale = 1.0f / (float)s_k;
  pa.q_i8 = q_i8; pa.k_i8 = k_i8; pa.q_i8_scale = q_i8_scale; pa.k_i8_scale = k_i8_scale;
  pa.quant_fp8 = (flags & SPARGE_FLAG_QUANT_FP8) ? 1 : 0;

  sa.q_mean = pa.q_mean; sa.k_mean = pa.k_mean; sa.sim_q = pa.sim_q; sa.k_sim = pa.k_sim;
  sa.sim_k = sim_k;
  sa.b = b; sa.h = h; sa.h_kv = h_kv; sa.nq = nq; sa.nk = nk;
  sa.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
  sa.lut = lut; sa.count = lut_count; sa.bmap = block_map; sa.prob = pooled_prob;
  sa.causal = causal ? 1 : 0;
  sa.sink = (flags & SPARGE_FLAG_ATTN_SINK) ? 1 : 0;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (smooth) {
    e = launch_key_mean(pa, dt, d, s);
    if (e != hipSuccess) return hip_status(e, "key_mean launch");
  }
  e = launch_pool_sim(pa, dt, d, s);
  if (e != hipSuccess) return hip_status(e, "pool_sim launch");
  e = launch_score_select(sa, d, s);
  return hip_status(e, "score_select launch");
}

}  // namespace

extern "C" {

sparge_status sparge_build_block_map(
    const void* q, const void* k, sparge_dtype dt, int b, int h, int h_kv, int s_q, int s_k, int d,
    const int64_t q_strides[3], const int64_t k_strides[3], int blk_q, int blk_k,
    const float* topk, const float* cdfthreshd, const float* simthreshd1, float softmax_scale,
    unsigned flags, int32_t* lut, int32_t* lut_count, uint8_t* block_map, float* pooled_prob, uint8_t* sim_q,
    uint8_t* sim_k, float* q_mean, float* k_mean, int8_t* q_i8, float* q_i8_scale, int8_t* k_i8,
    float* k_i8_scale, void* workspace, size_t workspace_bytes, void* stream) {
  return block_map_impl(q, k, dt, b, h, h_kv, s_q, s_k, d, q_strides, k_strides, blk_q, blk_k, topk, cdfthreshd,
                        simthreshd1, softmax_scale, flags, lut, lut_count, block_map, pooled_prob, sim_q, sim_k,
                        q_mean, k_mean, q_i8, q_i8_scale, k_i8, k_i8_scale, workspace, workspace_bytes, false,
                        stream);
}

sparge_status sparge_build_block_map_noalloc(
    const void* q, const void* k, sparge_dtype dt, int b, int h, int h_kv, int s_q, int s_k, int d,
    const int64_t q_strides[3], const int64_t k_strides[3], int blk_q, int blk_k,
    const float* topk, const float* cdfthreshd, const float* simthreshd1, float softmax_scale,
    unsigned flags, int32_t* lut, int32_t* lut_count, uint8_t* block_map, float* pooled_prob, uint8_t* sim_q,
    uint8_t* sim_k, float* q_mean, float* k_mean, int8_t* q_i8, float* q_i8_scale, int8_t* k_i8,
    float* k_i8_scale, void* stream) {
  return block_map_impl(q, k, dt, b, h, h_kv, s_q, s_k, d, q_strides, k_strides, blk_q, blk_k, topk, cdfthreshd,
                        simthreshd1, softmax_scale, flags, lut, lut_count, block_map, pooled_prob, sim_q, sim_k,
                        q_mean, k_mean, q_i8, q_i8_scale, k_i8, k_i8_scale, nullptr, 0, true, stream);
}

sparge_status sparse_fmha_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              sparge_dtype dt, sparge_dtype o_dt, int b, int h_q, int h_kv, int s_q,
                              int s_k, int d, const int64_t q_strides[3], const int64_t k_strides[3],
                              const int64_t v_strides[3], const int64_t o_strides[3], int blk_q,
                              int blk_k, const int32_t* lut, const int32_t* lut_count, int lut_row_len,
                              int lut_heads, float softmax_scale, unsigned flags, float pv_threshold,
                              int num_splits, int64_t o_split_stride, void* stream) {
  if (!q || !k || !v || !o) return fail(SPARGE_ERR_INVALID, "q, k, v and o must be non-null");
  if (!is_half(dt)) return fail(SPARGE_ERR_UNSUPPORTED, "input dtype must be F16 or BF16");
  if (o_dt != dt && o_dt != SPARGE_F32)
    return fail(SPARGE_ERR_UNSUPPORTED, "output dtype must equal the input dtype or be F32");
  if (b <= 0 || h_q <= 0 || h_kv <= 0 || s_q <= 0 || s_k <= 0 || d <= 0)
    return fail(SPARGE_ERR_INVALID, "sizes must be positive");
  if (h_q % h_kv != 0) return fail(SPARGE_ERR_INVALID, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  if (d != 64 && d != 128) return fail(SPARGE_ERR_UNSUPPORTED, "head dim %d not built (64, 128)", d);
  sparge_status st;
  if ((st = check_strides("q", q_strides)) != SPARGE_OK) return st;
  if ((st = check_strides("k", k_strides)) != SPARGE_OK) return st;
  if ((st = check_strides("v", v_strides)) != SPARGE_OK) return st;
  if ((st = check_strides("o", o_strides)) != SPARGE_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SPARGE_ERR_INVALID, "q/k/v/o must be 16-byte aligned");
  if (num_splits < 1 || num_splits > 1024) return fail(SPARGE_ERR_INVALID, "num_splits=%d out of [1, 1024]", num_splits);
  if (num_splits > 1 && !lse) return fail(SPARGE_ERR_INVALID, "split partials need an lse output");
  if (num_splits > 1 && (o_split_stride <= 0 || o_split_stride % 8))
    return fail(SPARGE_ERR_INVALID, "o_split_stride must be a positive multiple of 8 elements");
  if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
    return fail(SPARGE_ERR_INVALID, "softmax_scale must be finite and >= 0");
  const bool token_mode = blk_q == 1 && blk_k == 1;
  const bool block_mode = blk_q == 64 && blk_k == 64;
  if (!token_mode && !block_mode)
    return fail(SPARGE_ERR_UNSUPPORTED, "blocks (%d, %d) not built: use (64, 64) or (1, 1)", blk_q, blk_k);
  if (flags & ~SPARGE_FLAG_CAUSAL)
    return fail(SPARGE_ERR_INVALID, "sparse_fmha_fwd takes only SPARGE_FLAG_CAUSAL (flags 0x%x)", flags);
  const bool causal = (flags & SPARGE_FLAG_CAUSAL) != 0;
  if (!(pv_threshold >= 0.f) || !isfinite(pv_threshold))
    return fail(SPARGE_ERR_INVALID, "pv_threshold must be finite and >= 0");
  if (pv_threshold > 0.f && token_mode)
    return fail(SPARGE_ERR_UNSUPPORTED, "pv_threshold applies to block mode only");
  // The skip test compares each block with the maximum over the blocks of
  // the row visited before it; a split would start without that maximum.
  if (pv_threshold > 0.f && num_splits > 1)
    return fail(SPARGE_ERR_UNSUPPORTED, "pv_threshold decides over a row's whole list in one pass: "
                "it needs num_splits = 1 (got %d)", num_splits);
  if (causal && token_mode) return fail(SPARGE_ERR_INVALID, "causal masking applies to block mode only");
  if (causal && s_q != s_k)
    return fail(SPARGE_ERR_UNSUPPORTED, "causal attention needs s_q = s_k (got %d, %d)", s_q, s_k);
  if (lut) {
    if (lut_row_len <= 0) return fail(SPARGE_ERR_INVALID, "lut_row_len must be positive");
    if (lut_heads != h_q && lut_heads != h_kv)
      return fail(SPARGE_ERR_INVALID, "lut_heads=%d must be h_q=%d or h_kv=%d", lut_heads, h_q, h_kv);
  }

  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
  FmhaArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = q_strides[i]; a.ks[i] = k_strides[i]; a.vs[i] = v_strides[i]; a.os[i] = o_strides[i];
  }
  a.b = b; a.hq = h_q; a.hkv = h_kv; a.sq = s_q; a.sk = s_k;
  a.ratio = h_q / h_kv;
  a.lut = lut; a.cnt = lut_count; a.lut_row_len = lut_row_len; a.lut_heads = lut_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.splits = num_splits;
  a.o_split_stride = num_splits > 1 ? o_split_stride : 0;
  // O is written once and, as a finished output, not read again here, so
  // its rows bypass the caches.  Split partials are re-read at once by
  // attn_combine: when all of them fit well inside the 256 MB last-level
  // cache they are stored normally and the combine finds them there
  // (split + combine at b1 h8 s4096 with 2-8 splits measured 0-2.3% faster
  // over two runs); larger sets stay non-temporal (plain stores measured
  // 0.5-4.7% slower at b2 h32 s16384).
  const int64_t o_bytes = (int64_t)num_splits * b * h_q * s_q * d * dtype_size(o_dt);
  a.o_nt = num_splits == 1 || o_bytes > kSplitCachedBytes;
  a.causal = causal ? 1 : 0;
  a.pv_tau2 = pv_threshold * 1.4426950408889634f;
  a.q_scale = nullptr; a.k_scale = nullptr;
  a.tok_groups = 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  if (block_mode) {
    a.nqt = (s_q + 63) / 64;   // a partial last tile / block counts
    a.nkb = (s_k + 63) / 64;
    // The kernel addresses a 64-row Q tile or K/V block with 32-bit byte offsets.
    const int64_t elem = 2, span = 64 * std::max({q_strides[2], k_strides[2], v_strides[2]}) * elem;
    if (span >= (int64_t(1) << 31))
      return fail(SPARGE_ERR_UNSUPPORTED, "a 64-row Q/K/V block spans %lld bytes (limit 2^31)", (long long)span);
    if (!lut && lut_count) return fail(SPARGE_ERR_INVALID, "lut_count given without lut");
    return hip_status(launch_fmha_block(a, dt, o_dt, d, s), "sparse_fmha launch");
  }
  // token-list mode
  if (!lut) return fail(SPARGE_ERR_INVALID, "token-list mode needs an index list");
  {
    // Rows are gathered with 32-bit byte offsets into one (b, KV head) slice.
    const int64_t kspan = (int64_t)s_k * k_strides[2] * 2, vspan = (int64_t)s_k * v_strides[2] * 2;
    if (std::max(kspan, vspan) >= (int64_t(1) << 31))
      return fail(SPARGE_ERR_UNSUPPORTED, "token-list mode: a (b, KV head) slice of K or V spans %lld bytes "
                  "(limit 2^31)", (long long)std::max(kspan, vspan));
  }
  if (lut_count) return fail(SPARGE_ERR_INVALID, "token-list mode takes no lut_count");
  if (lut_heads != h_kv)
    return fail(SPARGE_ERR_UNSUPPORTED, "token-list mode needs one list per KV head (lut_heads = h_kv)");
  const int64_t rows = (int64_t)a.ratio * s_q;
  if (rows > 65536)
    return fail(SPARGE_ERR_UNSUPPORTED, "token-list mode serves at most 65536 query rows per KV head (got %lld)",
                (long long)rows);
  a.tok_groups = (int)((rows + 7) / 8);
  a.nqt = s_q;
  a.nkb = s_k;
  return hip_status(launch_fmha_tokens(a, dt, o_dt, d, (int)std::min<int64_t>(rows, 8), s),
                    "sparse_fmha token launch");
}

}  // extern "C"

namespace {

// Both 8-bit Q/K entry points: int8 codes, or fp8 e4m3 codes (fp8).
sparge_status fmha_qk8_impl(const void* q, const float* q_scale, const void* k, const float* k_scale,
                            const void* v, void* o, float* lse, sparge_dtype v_dt, sparge_dtype o_dt, int b,
                            int h_q, int h_kv, int s_q, int s_k, int d, const int64_t q_strides[3],
                            const int64_t k_strides[3], const int64_t v_strides[3], const int64_t o_strides[3],
                            const int32_t* lut, const int32_t* lut_count, int lut_row_len, int lut_heads,
                            float softmax_scale, unsigned flags, int num_splits, int64_t o_split_stride,
                            bool fp8, void* stream) {
  const char* entry = fp8 ? "sparse_fmha_fwd_qk_fp8" : "sparse_fmha_fwd_qk_int8";
  if (!q || !k || !v || !o || !q_scale || !k_scale)
    return fail(SPARGE_ERR_INVALID, "q, q_scale, k, k_scale, v and o must be non-null");
  if (!is_half(v_dt)) return fail(SPARGE_ERR_UNSUPPORTED, "v dtype must be F16 or BF16");
  if (o_dt != v_dt && o_dt != SPARGE_F32)
    return fail(SPARGE_ERR_UNSUPPORTED, "output dtype must equal the v dtype or be F32");
  if (b <= 0 || h_q <= 0 || h_kv <= 0 || s_q <= 0 || s_k <= 0 || d <= 0)
    return fail(SPARGE_ERR_INVALID, "sizes must be positive");
  if (h_q % h_kv != 0) return fail(SPARGE_ERR_INVALID, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  if (d != 64 && d != 128) return fail(SPARGE_ERR_UNSUPPORTED, "head dim %d not built (64, 128)", d);
  sparge_status st;
  if ((st = check_strides("q", q_strides)) != SPARGE_OK) return st;
  if ((st = check_strides("k", k_strides)) != SPARGE_OK) return st;
  if ((st = check_strides("v", v_strides)) != SPARGE_OK) return st;
  if ((st = check_strides("o", o_strides)) != SPARGE_OK) return st;
  if (q_strides[2] % 16 || k_strides[2] % 16)
    return fail(SPARGE_ERR_INVALID, "int8 q/k row strides must be multiples of 16 bytes");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SPARGE_ERR_INVALID, "q/k/v/o must be 16-byte aligned");
  if (num_splits < 1 || num_splits > 1024) return fail(SPARGE_ERR_INVALID, "num_splits=%d out of [1, 1024]", num_splits);
  if (num_splits > 1 && !lse) return fail(SPARGE_ERR_INVALID, "split partials need an lse output");
  if (num_splits > 1 && (o_split_stride <= 0 || o_split_stride % 8))
    return fail(SPARGE_ERR_INVALID, "o_split_stride must be a positive multiple of 8 elements");
  if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
    return fail(SPARGE_ERR_INVALID, "softmax_scale must be finite and >= 0");
  if (flags & ~SPARGE_FLAG_CAUSAL)
    return fail(SPARGE_ERR_INVALID, "%s takes only SPARGE_FLAG_CAUSAL (flags 0x%x)", entry, flags);
  const bool causal = (flags & SPARGE_FLAG_CAUSAL) != 0;
  if (causal && s_q != s_k)
    return fail(SPARGE_ERR_UNSUPPORTED, "causal attention needs s_q = s_k (got %d, %d)", s_q, s_k);
  if (lut) {
    if (lut_row_len <= 0) return fail(SPARGE_ERR_INVALID, "lut_row_len must be positive");
    if (lut_heads != h_q && lut_heads != h_kv)
      return fail(SPARGE_ERR_INVALID, "lut_heads=%d must be h_q=%d or h_kv=%d", lut_heads, h_q, h_kv);
  } else if (lut_count) {
    return fail(SPARGE_ERR_INVALID, "lut_count given without lut");
  }
  const int64_t span = std::max({64 * q_strides[2], 64 * k_strides[2], 64 * v_strides[2] * 2});
  if (span >= (int64_t(1) << 31))
    return fail(SPARGE_ERR_UNSUPPORTED, "a 64-row Q/K/V block spans %lld bytes (limit 2^31)", (long long)span);

  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
  FmhaArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = q_strides[i]; a.ks[i] = k_strides[i]; a.vs[i] = v_strides[i]; a.os[i] = o_strides[i];
  }
  a.b = b; a.hq = h_q; a.hkv = h_kv; a.sq = s_q; a.sk = s_k;
  a.ratio = h_q / h_kv;
  a.lut = lut; a.cnt = lut_count; a.lut_row_len = lut_row_len; a.lut_heads = lut_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.splits = num_splits;
  a.o_split_stride = num_splits > 1 ? o_split_stride : 0;
  a.o_nt = 1;                 // not used by the 8-bit kernels
  a.causal = causal ? 1 : 0;
  a.pv_tau2 = 0.f;
  a.q_scale = q_scale; a.k_scale = k_scale;
  a.tok_groups = 1;
  a.nqt = (s_q + 63) / 64;
  a.nkb = (s_k + 63) / 64;
  return hip_status(launch_fmha_qk8(a, v_dt, o_dt, d, fp8, reinterpret_cast<hipStream_t>(stream)), entry);
}

}  // namespace

extern "C" {

sparge_status sparse_fmha_fwd_qk_int8(const int8_t* q, const float* q_scale, const int8_t* k,
                                      const float* k_scale, const void* v, void* o, float* lse,
                                      sparge_dtype v_dt, sparge_dtype o_dt, int b, int h_q, int h_kv, int s_q,
                                      int s_k, int d, const int64_t q_strides[3], const int64_t k_strides[3],
                                      const int64_t v_strides[3], const int64_t o_strides[3], const int32_t* lut,
                                      const int32_t* lut_count, int lut_row_len, int lut_heads,
                                      float softmax_scale, unsigned flags, int num_splits,
                                      int64_t o_split_stride, void* stream) {
  return fmha_qk8_impl(q, q_scale, k, k_scale, v, o, lse, v_dt, o_dt, b, h_q, h_kv, s_q, s_k, d, q_strides,
                       k_strides, v_strides, o_strides, lut, lut_count, lut_row_len, lut_heads, softmax_scale,
                       flags, num_splits, o_split_stride, false, stream);
}

sparge_status sparse_fmha_fwd_qk_fp8(const uint8_t* q, const float* q_scale, const uint8_t* k,
                                     const float* k_scale, const void* v, void* o, float* lse,
                                     sparge_dtype v_dt, sparge_dtype o_dt, int b, int h_q, int h_kv, int s_q,
                                     int s_k, int d, const int64_t q_strides[3], const int64_t k_strides[3],
                                     const int64_t v_strides[3], const int64_t o_strides[3], const int32_t* lut,
                                     const int32_t* lut_count, int lut_row_len, int lut_heads,
                                     float softmax_scale, unsigned flags, int num_splits,
                                     int64_t o_split_stride, void* stream) {
  return fmha_qk8_impl(q, q_scale, k, k_scale, v, o, lse, v_dt, o_dt, b, h_q, h_kv, s_q, s_k, d, q_strides,
                       k_strides, v_strides, o_strides, lut, lut_count, lut_row_len, lut_heads, softmax_scale,
                       flags, num_splits, o_split_stride, true, stream);
}

sparge_status attn_combine(const void* o_parts, sparge_dtype part_dt, const float* lse_parts, int n_parts,
                           int b, int h, int s, int d, int64_t part_stride, void* o, sparge_dtype out_dt,
                           float* lse_out, void* stream) {
  if (!o_parts || !lse_parts || !o) return fail(SPARGE_ERR_INVALID, "o_parts, lse_parts and o must be non-null");
  if (n_parts < 1 || n_parts > 1024) return fail(SPARGE_ERR_INVALID, "n_parts=%d out of [1, 1024]", n_parts);
  if (b <= 0 || h <= 0 || s <= 0 || d <= 0) return fail(SPARGE_ERR_INVALID, "sizes must be positive");
  if (d != 64 && d != 128) return fail(SPARGE_ERR_UNSUPPORTED, "head dim %d not built (64, 128)", d);
  if (part_dt != SPARGE_F32 && !is_half(part_dt)) return fail(SPARGE_ERR_INVALID, "bad part dtype");
  if (out_dt != SPARGE_F32 && !is_half(out_dt)) return fail(SPARGE_ERR_INVALID, "bad output dtype");
  const int64_t rows = (int64_t)b * h * s;
  if (part_stride < rows * d) return fail(SPARGE_ERR_INVALID, "part_stride smaller than one part");
  if (part_stride % 8) return fail(SPARGE_ERR_INVALID, "part_stride must be a multiple of 8 elements");
  if (!aligned16(o_parts) || !aligned16(o)) return fail(SPARGE_ERR_INVALID, "o_parts/o must be 16-byte aligned");
  CombineArgs a;
  a.parts = o_parts; a.lse_parts = lse_parts; a.n_parts = n_parts; a.rows = rows;
  a.part_stride = part_stride; a.o = o; a.lse_out = lse_out;
  return hip_status(launch_combine(a, part_dt, out_dt, d, reinterpret_cast<hipStream_t>(stream)),
                    "attn_combine launch");
}

sparge_status sparge_validate_lut(const int32_t* lut, const int32_t* lut_count, int64_t rows, int row_len,
                                  int n_blocks, int32_t* bad_rows, void* stream) {
  if (!lut || !bad_rows) return fail(SPARGE_ERR_INVALID, "lut and bad_rows must be non-null");
  if (rows <= 0 || row_len <= 0 || n_blocks <= 0) return fail(SPARGE_ERR_INVALID, "sizes must be positive");
  return hip_status(launch_validate_lut(lut, lut_count, rows, row_len, n_blocks, bad_rows,
                                        reinterpret_cast<hipStream_t>(stream)),
                    "validate_lut launch");
}

}  // extern "C"
