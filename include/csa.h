/*
 * csa.h -- C ABI of the MI355X (gfx950) library for one layer of compressed
 * sparse attention (CSA) and heavily compressed attention (HCA).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer to dense row-major data owned
 *    by the caller; the library never allocates, frees or keeps a pointer
 *    after the call returns.  Inputs are never written.
 *  - `dtype` (csa_dtype) is the element type of every floating-point tensor
 *    argument except `w`, `sink` and `score`, which are always float32.
 *    Arithmetic is float32 in every mode; bfloat16 results are rounded to
 *    nearest-even when stored.
 *  - Positions are 0-based token positions.  A query at position t may read
 *    compressed entry s only if s < (t + 1) / m (integer division): entry s
 *    is complete once its m tokens are (cooking-agi "DeepSeek-V4: 压缩历史以后，
 *    还能读到什么？", section 3).
 *  - `*_bstride` arguments give the distance, in elements, between two
 *    consecutive sequences of a batched cache, so that a cache may be larger
 *    than the part in use; 0 means "dense" (rows-in-use * row length).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns without synchronising.
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued.  A negative return code means nothing was launched, except
 *    CSA_EHIP, which reports a launch failure from the HIP runtime.  No call
 *    aborts the process.  csa_strerror() names a code.
 *  - Results are bitwise reproducible from run to run: every reduction has a
 *    fixed order and no floating-point atomics are used.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* CSA_FP8 is the 8-bit E4M3 floating-point format of the OCP 8-bit floating
 * point specification (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * no infinities; 0x7F and 0xFF are NaN; largest finite value 448).  Only
 * csa_index_topk accepts it (for qI and KIcomp: the low-precision indexer);
 * every other entry point returns CSA_ENOTSUP for it. */
typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8 = 2 } csa_dtype;

enum {
  CSA_OK = 0,
  CSA_EINVAL = -1,  /* an argument is out of range or inconsistent      */
  CSA_ENOTSUP = -2, /* valid, but no kernel handles this shape / dtype  */
  CSA_ENOSPC = -3,  /* the workspace given is smaller than required     */
  CSA_EHIP = -4     /* the HIP runtime reported an error at launch      */
};

/* Library version string, e.g. "csa-mi355x 0.1.0". */
const char* csa_version(void);

/* Human-readable name of a return code. */
const char* csa_strerror(int code);

/*
 * csa_compress -- token-level KV compressor, CSA (overlap = 1) or HCA
 * (overlap = 0).
 *
 * Overlapped form (polysight "06-formulas" section B9; songhuiming
 * "DeepSeek-V4 百万 token 上下文" section 4.1, Eq. 11-12): for entry i and
 * each dimension d, softmax over the 2m scores
 *     Za[m*i + j][d] + Ba[j][d]        (j < m, block i, stream a)
 *     Zb[m*(i-1) + j][d] + Bb[j][d]    (j < m, block i-1, stream b)
 * and Ccomp[i][d] = sum of those weights times Ca / Cb of the same rows.
 * Block -1 is padded with -inf scores and zero values, unless prev_Cb /
 * prev_Zb ([b, m, c]) supply the block that precedes row 0 (continuing a
 * sequence, e.g. in decode).
 *
 * Pooling form (same pages, section B9 / section 5.1): overlap = 0, one
 * stream: softmax over the m rows Za[m*i + j][d] + Ba[j][d] and the weighted
 * sum of Ca.  Cb, Zb, Bb, prev_Cb and prev_Zb must then be NULL.
 *
 *  Ca, Cb, Za, Zb  [b, n, c]   input streams
 *  Ba, Bb          [m, c]      intra-block position bias
 *  Ccomp           out, entry i of sequence s at Ccomp + s*out_bstride + i*c,
 *                  i < n/m  (a ragged tail of n % m rows emits nothing)
 *
 * Errors: CSA_EINVAL for b, n, c or m < 1, NULL required pointers, pointers
 * given that must be NULL, out_bstride < (n/m)*c when non-zero, or only one
 * of prev_Cb / prev_Zb.  CSA_ENOTSUP for an unknown dtype.
 */
int csa_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb,
                 const void* Ba, const void* Bb, const void* prev_Cb, const void* prev_Zb,
                 int64_t b, int64_t n, int64_t c, int64_t m, int overlap, int dtype,
                 void* Ccomp, int64_t out_bstride, void* stream);

/*
 * csa_index_topk -- lightning-indexer scores and top-k selection
 * (polysight "06-formulas" section B9; AirCoding "deepseek-paper-analysis"
 * section 7.1):
 *     I[t][s] = sum_h w[t][h] * ReLU(qI[t][h] . KIcomp[s]),  s < (t+1)/m,
 * then the k entries of largest score.  If fewer than k entries are visible,
 * all of them are taken.  Ties at the k-th score go to the lower index.
 *
 *  qI      [b, n_q, n_hI, c_I]  indexer queries; row r is at position t0 + r
 *  w       [b, n_q, n_hI]       float32 per-head weights (any sign)
 *  KIcomp  [b, *, c_I]          compressed indexer keys (comp_bstride)
 *  idx     out [b, n_q, k] int32, selected entries in ascending order,
 *          padded with -1
 *  score   out [b, n_q, k] float32 scores of idx (0 at padding), or NULL
 *  workspace  device scratch of at least csa_index_topk_workspace_size()
 *          bytes, 256-byte aligned; its contents on return are unspecified.
 *
 * dtype: CSA_F32, CSA_BF16 or CSA_FP8 for qI and KIcomp.  With CSA_FP8 the
 * scores are the same weighted ReLU sums of the decoded E4M3 values,
 * accumulated in float32 (any scaling of the codes is the caller's: a
 * positive factor on all keys, or on one head's queries folded into that
 * head's w, leaves the selection unchanged).
 *
 * Errors: CSA_EINVAL for sizes < 1 (n_comp may be 0), t0 < 0, NULL required
 * pointers, or n_comp > (t0 + n_q)/m (entries that no query could have
 * completed).  CSA_ENOSPC if ws_bytes is too small.
 */
int csa_index_topk(const void* qI, const float* w, const void* KIcomp, int64_t comp_bstride,
                   int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_hI,
                   int64_t c_I, int64_t m, int64_t k, int dtype, int32_t* idx, float* score,
                   void* workspace, size_t ws_bytes, void* stream);

size_t csa_index_topk_workspace_size(int64_t b, int64_t n_q, int64_t n_comp, int64_t k);

/*
 * csa_index_topk_mxfp4 -- csa_index_topk with the indexer queries and keys
 * in OCP MXFP4 (songhuiming "DeepSeek-V4 百万 token 上下文" section 13.3 and
 * AirCoding "deepseek-paper-analysis" section 7, FP4 quantization-aware
 * training: the indexer's query/key path is cached, loaded and multiplied
 * in FP4; the element and scale formats are those of the OCP Microscaling
 * (MX) specification v1.0, which the pages name for the expert weights).
 * The scores are the weighted ReLU sums of the values the codes stand for,
 * accumulated in float32; selection, ties and output are as for
 * csa_index_topk.
 *
 *  qI        [b, n_q, n_hI, c_I/2] uint8  E2M1 codes, two per byte: byte j
 *            holds element 2j in its low nibble, 2j+1 in its high nibble
 *  qI_scale  [b, n_q, n_hI, c_I/32] uint8  E8M0 scale of each block of 32
 *            elements: value = e2m1(code) * 2^(scale - 127)
 *  w         [b, n_q, n_hI] float32
 *  KIcomp    [b, *, c_I/2] uint8 codes and KI_scale [b, *, c_I/32] uint8
 *            scales of the compressed keys, laid out the same way
 *  comp_bstride  entries (rows) from one sequence's first key to the next's,
 *            for both KIcomp and KI_scale (0 = n_comp)
 *  idx, score, workspace: as for csa_index_topk (same workspace size).
 *
 * Scale 255 (NaN in the MX specification) is not supported.  All pointers
 * are device memory owned by the caller; nothing is allocated.
 * Errors: CSA_EINVAL as for csa_index_topk, also for NULL scale pointers or
 * c_I not a multiple of 32; CSA_ENOTSUP for shapes without a kernel (the
 * streaming kernel takes fewer than 4 queries with c_I = 128 and 32, 64 or
 * 128 heads; every other shape needs n_hI * c_I <= 8192); CSA_ENOSPC if
 * ws_bytes is too small.
 */
int csa_index_topk_mxfp4(const void* qI, const void* qI_scale, const float* w, const void* KIcomp,
                         const void* KI_scale, int64_t comp_bstride, int64_t b, int64_t n_q, int64_t t0,
                         int64_t n_comp, int64_t n_hI, int64_t c_I, int64_t m, int64_t k, int32_t* idx,
                         float* score, void* workspace, size_t ws_bytes, void* stream);

/*
 * csa_norm_rope -- RMSNorm and partial rotary position embedding of query
 * heads, KV entries and attention outputs (songhuiming "DeepSeek-V4 百万
 * token 上下文" section 4.5; AirCoding "deepseek-paper-analysis" section
 * 7.1): before the core attention every query head and every KV entry is
 * RMS-normalised, and the last 64 dimensions of queries and entries carry a
 * rotary embedding at their positions; the attention output's last 64
 * dimensions are then turned back by -t so that only relative positions
 * remain in it.
 *
 * For each of `rows` rows holding `heads` vectors of c values:
 *   y = x / sqrt(mean(x^2) + eps) * gamma     (skipped when gamma is NULL)
 *   then for i < rope_dims/2 the pair (y[c-rope_dims+2i], y[c-rope_dims+2i+1])
 *   = (a, b) becomes (a cos A - b sin A, a sin A + b cos A) with
 *   A = pos * base^(-2i/rope_dims), pos = pos0 + row * pos_step.
 * Computed in float32 (angles in float64), stored in the storage type with
 * round-to-nearest-even.
 *
 *  x        [rows][x_rstride] float32 (CSA_F32) or bf16 (CSA_BF16); row r
 *           holds heads * c values: vector h at x + r*x_rstride + h*c
 *  out      [rows][out_rstride], same layout; may be x itself (same
 *           stride) for an in-place update, otherwise must not overlap x
 *  gamma    [c] float32 per-dimension gain, or NULL for no normalisation
 *  eps      >= 0, added to the mean square
 *  rope_dims  even, 0 (no rotation) .. min(c, 512)
 *  base     > 0, the rotary base (only read when rope_dims > 0)
 *  pos0, pos_step  positions of the rows, |value| <= 2^40 for every row
 * Typical calls: query heads of a prefill block (heads = n_h, pos0 = t0,
 * pos_step = 1); compressed entries (heads = 1, pos_step = m); raw window
 * rows (heads = 1, pos0 = their first position); the attention output
 * (gamma NULL, pos0 = -t0, pos_step = -1); one decode step of b sequences
 * (rows = b, pos_step = 0).
 * x, out and gamma must be 16-byte aligned and the row strides times the
 * element size multiples of 16.  All pointers are device memory owned by
 * the caller; nothing is allocated.
 * Errors: CSA_EINVAL for negative rows, heads or c < 1, odd or out-of-range
 * rope_dims, eps < 0, base <= 0, positions out of range, strides below
 * heads * c, misalignment, NULL x/out with rows > 0, or partial overlap of x
 * and out; CSA_ENOTSUP for other dtypes, c not a multiple of 8 (bf16) or 4
 * (float32), c above 2048 (bf16) or 1024 (float32), rope_dims > 512, or more
 * than 2^31 - 1 rows.
 */
int csa_norm_rope(const void* x, int64_t x_rstride, void* out, int64_t out_rstride, const float* gamma,
                  float eps, int64_t rows, int64_t heads, int64_t c, int64_t rope_dims, double base,
                  int64_t pos0, int64_t pos_step, int dtype, void* stream);

/*
 * csa_grouped_out_proj -- grouped output projection of the attention outputs
 * (songhuiming "DeepSeek-V4 百万 token 上下文" section 4.4; AirCoding
 * "deepseek-paper-analysis" section 7.1, which gives g = 8, d_g = 1024,
 * d = 4096 for the Flash model): the n_h heads of a token form g groups of
 * n_h/g consecutive heads; group j's outputs, concatenated in head order,
 * are projected to d_g values by W^G_j; the g results, concatenated in group
 * order, are projected to d by W^O:
 *   mid[t, j*d_g + r] = sum_q WG[j][r][q] * o[t, j*(n_h/g) + q/c, q%c]
 *   out[t, e]         = sum_p WO[e][p] * mid[t, p]
 * bf16 operands, float32 accumulation (MFMA), bf16 results; mid is stored in
 * bf16 and the second projection reads it back.
 *
 *  o    [n, n_h, c] bf16 (the attention output)
 *  WG   [g, d_g, (n_h/g)*c] bf16, input dimension contiguous
 *  WO   [d, g*d_g] bf16, input dimension contiguous
 *  mid  out [n, g*d_g] bf16 (the intermediate; caller-owned)
 *  out  out [n, d] bf16
 * o, WG, WO and mid must be 16-byte aligned.  All pointers are device memory
 * owned by the caller; nothing is allocated.  Results are reproducible run to
 * run (fixed accumulation order).
 * Errors: CSA_EINVAL for negative n, sizes < 1, n_h not a multiple of g,
 * NULL pointers with n > 0, or misalignment; CSA_ENOTSUP for a dtype other
 * than CSA_BF16, (n_h/g)*c or g*d_g not a multiple of 64, or sizes beyond
 * the launch limits.
 */
int csa_grouped_out_proj(const void* o, const void* WG, const void* WO, int64_t n, int64_t n_h, int64_t c,
                         int64_t g, int64_t d_g, int64_t d, int dtype, void* mid, void* out, void* stream);

/*
 * csa_quantize_mxfp4 -- OCP MXFP4 encoding of `rows` rows of c values, for
 * the indexer's FP4 query/key cache (songhuiming "DeepSeek-V4 百万 token
 * 上下文" section 13.3; AirCoding "deepseek-paper-analysis" section 7, FP4
 * quantization-aware training): the layout csa_index_topk_mxfp4 reads.
 * OCP Microscaling (MX) specification v1.0 conversion: each block of 32
 * values gets the E8M0 scale 2^(floor(log2 max|v|) - 2); each value divided
 * by it is rounded to the nearest E2M1 value, ties to the even code, and
 * saturated at 6.  An all-zero block gets scale byte 0; the sign bit is set
 * for every v < 0.
 *
 *  x       [rows][x_rstride] float32 (CSA_F32) or bf16 (CSA_BF16); the first
 *          c of each row are encoded; 16-byte aligned, x_rstride * element
 *          size a multiple of 16
 *  codes   out [rows][codes_rstride] bytes, c/2 used per row (element 2j in
 *          the low nibble of byte j); 16-byte aligned, codes_rstride a
 *          multiple of 16
 *  scales  out [rows][scales_rstride] bytes, c/32 used per row
 * Strides let a call write rows into a cache in place (one row per sequence
 * at entry e: x, codes and scales offset to entry e, strides = the batch
 * strides).  NaN or infinite inputs are not supported.
 * Errors: CSA_EINVAL for NULL pointers, rows < 1, c not a positive multiple of
 * 32, strides below the row size or misaligned; CSA_ENOTSUP for another dtype.
 */
int csa_quantize_mxfp4(const void* x, int64_t x_rstride, int64_t rows, int64_t c, int dtype, void* codes,
                       int64_t codes_rstride, void* scales, int64_t scales_rstride, void* stream);

/*
 * csa_attend -- shared key/value multi-query attention over the selected
 * compressed entries plus the causal sliding window, with one softmax whose
 * denominator also holds the per-head sink (AirCoding
 * "deepseek-paper-analysis" section 7.1; songhuiming "DeepSeek-V4 百万
 * token 上下文" sections 4.3, 4.5 and 7.3; polysight "06-formulas" B9):
 *   E_t   = { Ccomp[s] : s in idx[t], 0 <= s < (t+1)/m }
 *           U { kv_raw row at position p : max(0, t-n_win+1) <= p <= t }
 *   l_j   = scale * (q[t][h] . e_j)
 *   out[t][h] = sum_j exp(l_j) e_j / (sum_j exp(l_j) + exp(sink[h]))
 * Every entry is both key and value.  Indices outside [0, (t+1)/m) are
 * skipped (padding, or a guard against reading the future).
 *
 *  q       [b, n_q, n_h, c]   row r at position t0 + r
 *  Ccomp   [b, *, c]          compressed entries (comp_bstride)
 *  idx     [b, n_q, k] int32  from csa_index_topk (or any caller choice)
 *  kv_raw  [b, *, c]          raw rows (raw_bstride); row j is at position
 *                             raw_pos0 + j; n_raw rows are valid
 *  sink    [n_h] float32      per-head sink logits (not scaled)
 *  out     [b, n_q, n_h, c]
 *
 *  workspace  device scratch of csa_attend_workspace_size() bytes, 256-byte
 *          aligned (may be NULL when that size is 0)
 *
 * Errors: CSA_EINVAL for sizes < 1 (n_comp and k may be 0), NULL required
 * pointers, a scale that is not a finite positive number, or a window
 * that kv_raw does not cover:
 * rows max(0, t0-n_win+1) .. t0+n_q-1 must lie in [raw_pos0, raw_pos0 +
 * n_raw).  CSA_ENOSPC if ws_bytes is too small.  CSA_ENOTSUP for c > 1024
 * outside the bf16 64-head c = 512 kernel.
 */
int csa_attend(const void* q, const void* Ccomp, int64_t comp_bstride, const int32_t* idx,
               const void* kv_raw, int64_t raw_bstride, int64_t raw_pos0, const float* sink,
               int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw,
               int64_t n_h, int64_t c, int64_t k, int64_t m, int64_t n_win, float scale,
               int dtype, void* workspace, size_t ws_bytes, void* out, void* stream);

/* Device scratch csa_attend needs for these shapes (0 = none; then workspace
 * may be NULL).  Few queries (decode) split each query's entries over
 * several workgroups and merge the partial softmax states in a fixed order;
 * the scratch holds those partials. */
size_t csa_attend_workspace_size(int64_t b, int64_t n_q, int64_t t0, int64_t n_comp,
                                 int64_t n_h, int64_t c, int64_t k, int64_t m, int64_t n_win,
                                 int dtype);

/*
 * hca_attend -- HCA dense attention: every completed compressed entry
 * (s < (t+1)/m_prime) plus the causal window, one softmax with the sink
 * (polysight "06-formulas" B9; songhuiming section 5.2; AirCoding section
 * 7.2).  Arguments as in csa_attend, without idx/k.
 */
int hca_attend(const void* q, const void* Ccomp, int64_t comp_bstride, const void* kv_raw,
               int64_t raw_bstride, int64_t raw_pos0, const float* sink, int64_t b,
               int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h,
               int64_t c, int64_t m_prime, int64_t n_win, float scale, int dtype,
               void* workspace, size_t ws_bytes, void* out, void* stream);

size_t hca_attend_workspace_size(int64_t b, int64_t n_q, int64_t t0, int64_t n_comp,
                                 int64_t n_h, int64_t c, int64_t m_prime, int64_t n_win,
                                 int dtype);

/*
 * hca_layer -- one HCA prefill layer over whole sequences: the pooling
 * compressor (csa_compress, overlap = 0) writes Ccomp [b, n/m_prime, c],
 * then hca_attend runs every position 0..n-1 against it, with kv_raw = the
 * window source [b, n, c].
 *
 *  C, Z [b, n, c]; B [m_prime, c]; q [b, n, n_h, c]; sink [n_h] float32
 *  Ccomp  out (also read by the attention step) [b, n/m_prime, c]
 *  workspace  as for hca_attend (hca_layer_workspace_size() bytes)
 *  out    [b, n, n_h, c]
 */
int hca_layer(const void* C, const void* Z, const void* B, const void* q, const void* kv_raw,
              const float* sink, int64_t b, int64_t n, int64_t c, int64_t m_prime, int64_t n_h,
              int64_t n_win, float scale, int dtype, void* Ccomp, void* workspace,
              size_t ws_bytes, void* out, void* stream);

size_t hca_layer_workspace_size(int64_t b, int64_t n, int64_t n_h, int64_t c, int64_t m_prime,
                                int64_t n_win, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
