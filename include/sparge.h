/*
 * sparge.h -- C ABI of the gfx950 (MI355X) block-sparse attention library.
 *
 * The library implements the forward pass of SpargeAttn-style block-sparse
 * attention in two stages, as the "Sparge Attention (Composable Kernel)" page
 * describes it ("Status vs Upstream"): a block map (per-block mean pool of Q
 * and K, an intra-block cosine-similarity gate, a softmax over pooled QK
 * scores, and top-k / cdfthreshd selection into a per-Q-tile LUT), then a
 * sparse flash attention over the selected K/V blocks that exports the
 * natural-log LSE (an empty row gives O = 0, LSE = -inf: aiter pull request
 * 6841 page; "Updating Log -- Speculative Sparse Attention" page, Stage 3),
 * plus the LSE combine that merges partial results (Updating Log page,
 * Stage 1: FA(A u B) = Combine(FA(A), FA(B))).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *   never allocates, frees or synchronises; it only enqueues kernels on the
 *   given stream (a hipStream_t passed as void*; NULL = the null stream).
 *   Outputs are valid once the stream has run the work.
 * - Small per-head parameter arrays (topk, cdfthreshd, simthreshd1) are HOST
 *   memory, read during the call only.
 * - Tensors of shape [b, h, s, d] are addressed with element strides for the
 *   b, h and s dimensions; the d dimension must be contiguous (stride 1) and
 *   every row must start 16-byte aligned.
 * - Arguments are checked on the host before anything is enqueued.  On any
 *   error nothing is enqueued and the call returns a non-zero status;
 *   sparge_last_error() then gives a message (per calling thread).
 * - The device does not check LUT / index-list entries: an entry outside
 *   [0, n_blocks) (or [0, s_k) for token lists), other than -1 padding, is
 *   undefined behaviour.  sparge_validate_lut() checks a LUT on the device.
 * - Supported: d in {64, 128}; fp16 or bf16 inputs; 64-token blocks (block
 *   mode) or 1-token granularity (token-list mode, see sparse_fmha_fwd).
 */
#ifndef SPARGE_H
#define SPARGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARGE_OK = 0,
  SPARGE_ERR_INVALID = 1,      /* null pointer, bad size, stride or parameter   */
  SPARGE_ERR_UNSUPPORTED = 2,  /* valid but not built: head dim, block, causal  */
  SPARGE_ERR_HIP = 3           /* a HIP runtime error at launch (see message)   */
} sparge_status;

typedef enum {
  SPARGE_F16 = 0,
  SPARGE_BF16 = 1,
  SPARGE_F32 = 2
} sparge_dtype;

/* Largest head count accepted by sparge_build_block_map (per-head parameters
 * travel in the kernel arguments). */
#define SPARGE_MAX_HEADS 128
/* Largest number of K blocks per row accepted by sparge_build_block_map
 * (s_k <= 64 * 1024 tokens with 64-token blocks). */
#define SPARGE_MAX_KBLOCKS 1024

/* Option bits for the `flags` arguments.  (CK page, "Status vs Upstream",
 * not-yet-ported list: K smoothing before pooling, the is_causal mask in the
 * pooled score, attention_sink with column 0 forced on.) */
#define SPARGE_FLAG_SMOOTH_K 1u   /* block map: pool and gate k - mean_s(k)        */
#define SPARGE_FLAG_CAUSAL 2u     /* block map and block-mode FMHA: causal masks   */
#define SPARGE_FLAG_ATTN_SINK 4u  /* block map: K block 0 selected in every row    */
#define SPARGE_FLAG_QUANT_FP8 8u  /* block map: the Q/K codes are fp8 e4m3, not int8 */

/* Device scratch held by sparge_build_block_map_noalloc on each GPU it runs
 * on (32 MiB: enough for the block map of b2 h32 s16384 d128, which needs
 * 16.6 MiB). */
#define SPARGE_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Library ABI version (this header: 7). */
int sparge_abi_version(void);

/* Message for the last failed call on this thread ("" if none). */
const char* sparge_last_error(void);

/*
 * Stage 1: block map.  (CK page, "Status vs Upstream": mean-pool, cosine
 * similarity, pooled QK, top-k / cdfthreshd selection, per-head knobs.)
 *
 * q [b, h, s_q, d], k [b, h_kv, s_k, d] in `dt` (F16 or BF16), strides in
 * elements for (b, h, s); h is a multiple of h_kv.  With h_kv < h (grouped
 * query attention) query head j pools against K head j / (h / h_kv), the
 * mapping attention uses (aiter 6841 page), and gates that head's K blocks
 * with its own simthreshd1[j]; h_kv = h is the plain per-head map.
 * blk_q = blk_k = 64; nq = ceil(s_q / 64), nk = ceil(s_k / 64) <=
 * SPARGE_MAX_KBLOCKS; h <= SPARGE_MAX_HEADS.  Lengths need not be multiples
 * of 64: the last block then holds n < 64 tokens and pools only those (the
 * plain reading of a per-block mean pool).
 *
 * For every block x_1..x_n of Q and of K (n = 64 but for a partial last one):
 *   mean  = (1/n) sum_i x_i                     (fp32)
 *   sim   = |sum_i x_i/|x_i| |^2 / n^2           (mean pairwise cosine, i = j
 *                                                 included; zero rows add 0)
 *   flag  = sim > simthreshd1[head]
 * Then per row (b, head, qb):
 *   S[kb] = scale * <q_mean[qb], k_mean[kb]>, -inf where the K flag is 0;
 *   P     = softmax_kb(S) in fp32 (a row of all -inf gives P = 0);
 *   order kb by P descending, ties to the lower kb;
 *   n     = clamp(floor(fp64(topk[head]) * nk), 1, nk) if topk[head] > 0,
 *           else the fewest leading blocks whose fp64 running sum of P (added
 *           one at a time in that order) reaches cdfthreshd[head] (nk if never);
 *   selected = all kb if the Q flag is 0, else the first n of the order plus
 *           every kb whose K flag is 0.
 *
 * flags (SPARGE_FLAG_*; other bits are rejected):
 *   SMOOTH_K   K is replaced by k - km before pooling and gating, km the fp32
 *              mean over all s_k positions of the (b, h) slice; k_mean is then
 *              the mean of the smoothed block.  Attention is unaffected.
 *   CAUSAL     needs s_q = s_k.  S[kb] = -inf for kb > qb; n is clamped to
 *              qb + 1; "all kb" and the forced blocks are limited to kb <= qb.
 *   ATTN_SINK  kb = 0 is added to every row.
 *   QUANT_FP8  needs the four code outputs: they receive OCP fp8 e4m3 codes
 *              (bytes) instead of int8, with scale = absmax / 448 and code =
 *              x * (448 / absmax) rounded to the e4m3 grid to nearest even,
 *              each step in fp32.  Input to sparse_fmha_fwd_qk_fp8.
 *
 * Inputs:
 *   topk        host float[h]; > 0 selects top-k mode for that head, must be <= 1.
 *   cdfthreshd  host float[h] or NULL; used for heads with topk <= 0, must be
 *               finite and in (0, 1].  NULL requires topk > 0 for every head.
 *   simthreshd1 host float[h], finite.
 *   softmax_scale  0 => 1/sqrt(d).
 *   flags      SPARGE_FLAG_* bits (above).
 * Outputs (device, caller-owned; optional ones may be NULL):
 *   lut        int32 [b, h, nq, nk]: selected kb ascending, then -1.
 *   lut_count  int32 [b, h, nq]: number of selected blocks.
 *   block_map  uint8 [b, h, nq, nk] or NULL: 1 = selected.
 *   pooled_prob float [b, h, nq, nk] or NULL: P exactly as the selection saw it.
 *   sim_q, sim_k uint8 [b, h, nq] / [b, h, nk] or NULL: gate flags (sim_k
 *              as query head j sees its K head's blocks).
 *   q_mean, k_mean float [b, h, nq, d] / [b, h_kv, nk, d] or NULL.
 *   q_i8, k_i8 int8 [b, h, s_q, d] / [b, h_kv, s_k, d] contiguous, 16-byte
 *              aligned, with q_i8_scale, k_i8_scale float [b, h, nq] /
 *              [b, h_kv, nk]: all four or none.  (CK page, "Status vs Upstream",
 *              not-yet-ported list: Q/K int8 quantisation fused into the pool
 *              kernel, for an int8 QK product in the attention kernel.)  Per
 *              64-token block of the inputs as given (K not smoothed):
 *              scale = absmax / 127 and code = round-half-even(x * (127 /
 *              absmax)) clamped to [-127, 127], in fp32 with correctly
 *              rounded divisions; an all-zero block gets scale 0, codes 0.
 *              Input to sparse_fmha_fwd_qk_int8.
 *   workspace  device scratch of at least sparge_build_block_map_workspace()
 *              bytes, 256-byte aligned; contents on entry are ignored.
 */
sparge_status sparge_build_block_map(
    const void* q, const void* k, sparge_dtype dt,
    int b, int h, int h_kv, int s_q, int s_k, int d,
    const int64_t q_strides[3], const int64_t k_strides[3],
    int blk_q, int blk_k,
    const float* topk, const float* cdfthreshd, const float* simthreshd1,
    float softmax_scale, unsigned flags,
    int32_t* lut, int32_t* lut_count, uint8_t* block_map, float* pooled_prob,
    uint8_t* sim_q, uint8_t* sim_k, float* q_mean, float* k_mean,
    int8_t* q_i8, float* q_i8_scale, int8_t* k_i8, float* k_i8_scale,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparge_build_block_map without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Arguments, outputs and results
 * are those of sparge_build_block_map; the scratch it needs lives in a
 * static device array of SPARGE_NOALLOC_SCRATCH_BYTES held by the library on
 * each GPU until the process ends.  The call allocates nothing: the first
 * call with a given device current looks the array's address up
 * (hipGetSymbolAddress) and keeps it.  Sizes whose workspace
 * (sparge_build_block_map_workspace) exceeds SPARGE_NOALLOC_SCRATCH_BYTES
 * return SPARGE_ERR_UNSUPPORTED with nothing enqueued.  Every call on one GPU
 * shares that array: calls whose work overlaps on one GPU (other streams,
 * other threads) race and give undefined results; calls ordered on one stream
 * are safe.  The array's contents on entry are ignored.
 */
sparge_status sparge_build_block_map_noalloc(
    const void* q, const void* k, sparge_dtype dt,
    int b, int h, int h_kv, int s_q, int s_k, int d,
    const int64_t q_strides[3], const int64_t k_strides[3],
    int blk_q, int blk_k,
    const float* topk, const float* cdfthreshd, const float* simthreshd1,
    float softmax_scale, unsigned flags,
    int32_t* lut, int32_t* lut_count, uint8_t* block_map, float* pooled_prob,
    uint8_t* sim_q, uint8_t* sim_k, float* q_mean, float* k_mean,
    int8_t* q_i8, float* q_i8_scale, int8_t* k_i8, float* k_i8_scale,
    void* stream);

/* Bytes of device workspace sparge_build_block_map needs for these sizes
 * (0 if the sizes are invalid); enough for any h_kv dividing h. */
size_t sparge_build_block_map_workspace(int b, int h, int s_q, int s_k, int d,
                                        int blk_q, int blk_k);

/*
 * Stage 2: sparse flash attention forward.  (Updating Log page, Stage 3: the
 * kernel walks the listed K/V blocks with an online softmax, an empty list
 * writes O = 0 and LSE = -inf; aiter 6841 page: LSE export and GQA mapping,
 * query head j reads KV head j / (h_q / h_kv).)
 *
 * q [b, h_q, s_q, d]; k, v [b, h_kv, s_k, d]; all in `dt` (F16 or BF16).
 * For every query row i the kernel computes, over the keys J the LUT selects,
 *   s_j = scale * <q_i, k_j>,  LSE_i = ln sum_j exp(s_j),
 *   O_i = sum_j exp(s_j - LSE_i) v_j;   J empty => O_i = 0, LSE_i = -inf.
 *
 * Block mode (blk_q = blk_k = 64): 64 rows of Q, K or V must span less than
 * 2^31 bytes (SPARGE_ERR_UNSUPPORTED otherwise; the LUT is read-only for the
 * duration of the call).  A LUT row belongs to (b, lut head, q tile of 64
 * rows) and lists K blocks kb in [0, nk), nk = ceil(s_k / 64) (keys
 * [64 kb, min(64 kb + 64, s_k))); nq = ceil(s_q / 64) tiles, the last one
 * partial when s_q is not a multiple of 64 (it writes only rows < s_q):
 *   lut        int32 [b, lut_heads, nq, lut_row_len], or NULL = dense
 *              (every block, in order; the dense baseline);
 *   lut_count  int32 [b, lut_heads, nq], or NULL = entries up to the
 *              first -1 (or the whole row).
 * Token-list mode (blk_q = blk_k = 1): a LUT row belongs to (b, lut head) and
 *   lists token positions in [0, s_k); -1 entries are skipped wherever they
 *   are; the same list serves every query position (decode: s_q = 1);
 *   lut_count must be NULL; lut_heads must be h_kv (one list per KV head,
 *   shared by its query heads).  The h_q / h_kv * s_q query rows of a KV
 *   head (at most 65536) are served in groups of 8, each group gathering the
 *   listed keys once.  s_k rows of one (b, KV head) slice of K or V must
 *   span less than 2^31 bytes (SPARGE_ERR_UNSUPPORTED otherwise).
 * In block mode lut_heads is h_q (one row per query head) or h_kv (a row
 * shared by the query heads of one KV head).
 *
 * num_splits >= 1 divides every row's list into num_splits contiguous chunks
 * of ceil(n / num_splits) entries; chunk c writes partial results to
 * o + c * o_split_stride and lse + c * b * h_q * s_q (a chunk with no entry
 * writes O = 0, LSE = -inf).  Merge them with attn_combine.
 *
 * Outputs: o [.., b, h_q, s_q, d] in o_dt (= dt, or F32 for partials), with
 * o_strides for (b, h, s); lse float [.., b, h_q, s_q] contiguous, or NULL
 * when num_splits = 1.
 * softmax_scale 0 => 1/sqrt(d).
 * flags: 0 or SPARGE_FLAG_CAUSAL (block mode, s_q = s_k): query position i
 * attends only to keys j <= i; listed blocks past the tile add nothing, and a
 * row left with no key gives O = 0, LSE = -inf.  In dense mode (lut = NULL)
 * the tile of rows [64 qt, 64 qt + 64) reads blocks 0..qt.
 *
 * pv_threshold (block mode; CK page, "Status vs Upstream": pv_threshold, a
 * per-Q-tile skip in the attention kernel): 0 = off.  A value tau > 0 drops
 * P.V products that cannot matter much.  The unit is one Q-tile (64 query
 * rows, fewer in a partial last tile) against one listed block (64 keys).
 * The row's blocks are visited in list order; for each block and each query
 * row i of the tile, r_i is the maximum of s over the block's keys (-inf
 * where masked) and M_i the running maximum of s over the blocks visited so
 * far, this one included.  The block's P.V product is skipped for the whole
 * tile when r_i < M_i - tau for every row i.  Skipped keys still count in the
 * softmax denominator and in LSE: LSE is the exact one, and O_i moves by at
 * most (skipped keys of row i) * exp(-tau) * max |v|.  The decision is taken
 * in fp32.  tau must be finite and >= 0; token-list mode takes 0 only, and a
 * tau > 0 needs num_splits = 1 (SPARGE_ERR_UNSUPPORTED otherwise: a split
 * would not know the maximum of the blocks before it).
 */
sparge_status sparse_fmha_fwd(
    const void* q, const void* k, const void* v, void* o, float* lse,
    sparge_dtype dt, sparge_dtype o_dt,
    int b, int h_q, int h_kv, int s_q, int s_k, int d,
    const int64_t q_strides[3], const int64_t k_strides[3],
    const int64_t v_strides[3], const int64_t o_strides[3],
    int blk_q, int blk_k,
    const int32_t* lut, const int32_t* lut_count, int lut_row_len, int lut_heads,
    float softmax_scale, unsigned flags, float pv_threshold,
    int num_splits, int64_t o_split_stride, void* stream);

/*
 * Stage 2 with int8 Q and K (CK page, "Status vs Upstream", not-yet-ported
 * list: an int8 QK product in the attention kernel, fed by the pool kernel's
 * quantisation).  Block mode only (64 x 64).  The same computation as
 * sparse_fmha_fwd, with every score taken from the codes:
 *   s_j = scale * q_scale[tile] * k_scale[block of j] * <q_code_i, k_code_j>
 * (the integer product is exact; the scores are then fp32).  V, O, the LUT,
 * num_splits, o_split_stride and flags (0 or SPARGE_FLAG_CAUSAL) are as in
 * sparse_fmha_fwd; v_dt is F16 or BF16 and o_dt is v_dt or F32.
 *   q        int8 [b, h_q, s_q, d], strides (elements) for (b, h, s);
 *   q_scale  float [b, h_q, ceil(s_q / 64)] contiguous;
 *   k        int8 [b, h_kv, s_k, d], strides for (b, h, s);
 *   k_scale  float [b, h_kv, ceil(s_k / 64)] contiguous.
 * A partial last block has its own scale (as the block map writes it).
 * d is 64 or 128; q, k, v, o 16-byte aligned; 64 rows of Q, K or V must span
 * less than 2^31 bytes.
 */
sparge_status sparse_fmha_fwd_qk_int8(
    const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
    const void* v, void* o, float* lse, sparge_dtype v_dt, sparge_dtype o_dt,
    int b, int h_q, int h_kv, int s_q, int s_k, int d,
    const int64_t q_strides[3], const int64_t k_strides[3],
    const int64_t v_strides[3], const int64_t o_strides[3],
    const int32_t* lut, const int32_t* lut_count, int lut_row_len, int lut_heads,
    float softmax_scale, unsigned flags, int num_splits, int64_t o_split_stride,
    void* stream);

/*
 * Stage 2 with fp8 (e4m3) Q and K codes, as sparge_build_block_map writes
 * them with SPARGE_FLAG_QUANT_FP8 (CK page, "Status vs Upstream", not-yet-ported
 * list: Q/K quantisation in the pool kernel for a low-precision QK product;
 * aiter 6841 page: fp8 Q/K recipes).  Arguments, layouts, limits and errors
 * as sparse_fmha_fwd_qk_int8, with q and k holding OCP e4m3 bytes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits); every score is
 *   s_j = scale * q_scale[tile] * k_scale[block of j] * <q_code_i, k_code_j>,
 * the code product accumulated in fp32 by the fp8 MFMA.
 */
sparge_status sparse_fmha_fwd_qk_fp8(
    const uint8_t* q, const float* q_scale, const uint8_t* k, const float* k_scale,
    const void* v, void* o, float* lse, sparge_dtype v_dt, sparge_dtype o_dt,
    int b, int h_q, int h_kv, int s_q, int s_k, int d,
    const int64_t q_strides[3], const int64_t k_strides[3],
    const int64_t v_strides[3], const int64_t o_strides[3],
    const int32_t* lut, const int32_t* lut_count, int lut_row_len, int lut_heads,
    float softmax_scale, unsigned flags, int num_splits, int64_t o_split_stride,
    void* stream);

/*
 * LSE combine of n_parts partial results.  (Updating Log page, Stage 1:
 * online-softmax merge with the running maximum; aiter 4919 page: partials
 * whose LSE is -inf are masked before the exponential.)
 *
 * Per row r and part i:  m = max_i LSE_i;  w_i = exp(LSE_i - m), 0 where
 * LSE_i = -inf;  O = sum_i w_i O_i / sum_i w_i;  LSE = m + ln sum_i w_i.
 * Every part -inf => O = 0, LSE = -inf.
 *
 * o_parts   [n_parts][b, h, s, d] in part_dt (F32, F16 or BF16), each part
 *           contiguous, part_stride elements apart (>= b*h*s*d).
 * lse_parts float [n_parts][b, h, s] contiguous.
 * o         [b, h, s, d] contiguous in out_dt (F32, F16 or BF16).
 * lse_out   float [b, h, s] or NULL.
 * 1 <= n_parts <= 1024 (the most splits sparse_fmha_fwd makes); d in {64, 128}.
 */
sparge_status attn_combine(
    const void* o_parts, sparge_dtype part_dt, const float* lse_parts,
    int n_parts, int b, int h, int s, int d, int64_t part_stride,
    void* o, sparge_dtype out_dt, float* lse_out, void* stream);

/*
 * Debug check of a LUT on the device.  For `rows` rows of `row_len` entries
 * (and per-row counts, or NULL = up to the first -1), counts the rows whose
 * listed entries are not strictly ascending, fall outside [0, n_blocks), or
 * whose count exceeds row_len, and whose tail after the count is not all -1.
 * Writes that number of bad rows to bad_rows (device int32[1]).
 */
sparge_status sparge_validate_lut(const int32_t* lut, const int32_t* lut_count,
                                  int64_t rows, int row_len, int n_blocks,
                                  int32_t* bad_rows, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARGE_H */
