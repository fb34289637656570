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
 *  - Alignment: every pointer must be aligned to its element size.  Rows
 *    whose length in bytes is a multiple of 16 are moved with 16-byte vector
 *    loads and stores; their pointers must then be 16-byte aligned and their
 *    row and batch strides multiples of 16 bytes (csa_attend / hca_attend:
 *    on the bf16 c = 512 path, for q, Ccomp, kv_raw and out; csa_compress:
 *    every stream, bias, state and output; csa_index_topk: qI and KIcomp).
 *    Violations return CSA_EINVAL before anything is enqueued.
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
 * no infinities; 0x7F and 0xFF are NaN; largest finite value 448).  As a
 * dtype only csa_index_topk accepts it (for qI and KIcomp: the
 * low-precision indexer); the FP8 KV entries have entry points of their own
 * (csa_quantize_kv_fp8, csa_attend_fp8kv). */
typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8 = 2 } csa_dtype;

enum {
  CSA_OK = 0,
  CSA_EINVAL = -1,  /* an argument is out of range or inconsistent      */
  CSA_ENOTSUP = -2, /* valid, but no kernel handles this shape / dtype  */
  CSA_ENOSPC = -3,  /* the workspace given is smaller than required     */
  CSA_EHIP = -4,    /* the HIP runtime reported an error at launch      */
  CSA_EBOUNDS = -5  /* debug builds only: a gather's bounds check failed */
};

/* Library version string, e.g. "csa-mi355x 0.1.0". */
const char* csa_version(void);

/* Human-readable name of a return code. */
const char* csa_strerror(int code);

/*
 * Debug builds.  libcsa_debug.so is the library compiled with CSA_DEBUG=1:
 * csa_attend and hca_attend check every row their kernels gather from flat
 * caches (a compressed entry s must satisfy 0 <= s < n_comp, a window row
 * must lie between the query's first window row and its own row).  A row
 * outside those bounds is not read; the call waits for its stream and
 * returns CSA_EBOUNDS instead of CSA_OK.  Paged calls are not checked.
 * Release builds export the same two functions: csa_debug_enabled returns
 * 0 and csa_debug_set_entry_limit returns CSA_ENOTSUP.
 *
 * csa_debug_enabled -- 1 in a debug build, else 0.
 * csa_debug_set_entry_limit -- a tighter bound on compressed entry rows
 *   (rows >= limit fail the check; INT64_MAX restores the default), for
 *   tests that exercise the check with valid inputs.  limit < 0 is
 *   CSA_EINVAL.  Affects every later call on the current device.
 */
int csa_debug_enabled(void);
int csa_debug_set_entry_limit(int64_t limit);

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
/* CSA_SCORE_BF16 may be OR-ed into csa_index_topk's dtype when it is CSA_F32
 * or CSA_BF16 (also for csa_index_topk_noalloc): every score is rounded to
 * bfloat16 (nearest even) before the selection, the BF16 index scores of
 * AirCoding "deepseek-paper-analysis" section 7.8 (the pages report 99.7%
 * recall against float32 scores).  Ties among equal rounded scores go to
 * the lower index, as always; `score` returns the rounded values. */
#define CSA_SCORE_BF16 0x100

int csa_index_topk(const void* qI, const float* w, const void* KIcomp, int64_t comp_bstride,
                   int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_hI,
                   int64_t c_I, int64_t m, int64_t k, int dtype, int32_t* idx, float* score,
                   void* workspace, size_t ws_bytes, void* stream);

size_t csa_index_topk_workspace_size(int64_t b, int64_t n_q, int64_t n_comp, int64_t k);

/*
 * csa_index_topk_noalloc -- csa_index_topk for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same operation, arguments
 * and results as csa_index_topk without `workspace` / `ws_bytes`; its
 * scratch is a device array of CSA_NOALLOC_SCRATCH_BYTES that the library's
 * code object holds on each GPU it runs on until the process ends (no
 * allocation call is made, on the first call or any other).
 *
 *  - Uses the scratch of the device current at the call; `stream` must
 *    belong to that device.
 *  - Every call on one GPU shares that GPU's array: calls that may overlap
 *    in time on one GPU (other streams, other host threads) race and must
 *    be serialised by the caller.  The kernels write every scratch word they
 *    read before reading it, so nothing is carried from one call to the next.
 *
 * Errors: as csa_index_topk; CSA_ENOSPC when
 * csa_index_topk_workspace_size(b, n_q, n_comp, k) exceeds
 * CSA_NOALLOC_SCRATCH_BYTES (80 MiB: e.g. 8 or 16 sequences of a 2^20-token
 * decode, or a 8192-token prefill block with 2048 entries); CSA_EHIP if the
 * scratch address cannot be obtained on the current device.
 */
#define CSA_NOALLOC_SCRATCH_BYTES (80u * 1024u * 1024u)
int csa_index_topk_noalloc(const void* qI, const float* w, const void* KIcomp, int64_t comp_bstride,
                           int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_hI,
                           int64_t c_I, int64_t m, int64_t k, int dtype, int32_t* idx, float* score,
                           void* stream);

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

/*
 * csa_attend_norm_rope -- csa_attend with the query side of the norm and
 * partial RoPE folded in (songhuiming "DeepSeek-V4 百万 token 上下文"
 * section 4.5; AirCoding "deepseek-paper-analysis" section 7.1): q holds the
 * raw query heads; each head vector is RMS-normalised and its last rope_dims
 * dimensions rotated at the query's position t, as csa_norm_rope does
 * (y = x / sqrt(mean(x^2) + eps) * gamma_q, then the pair (y[c-rope_dims+2i],
 * y[c-rope_dims+2i+1]) turned by t * base^(-2i/rope_dims), angles in
 * float64), and rounded to bf16 before the products; the output's last
 * rope_dims dimensions are turned back by -t in float32 and stored once in
 * bf16.  The compressed entries and raw rows are read as given (normalise
 * and rotate them with csa_norm_rope when they are stored).
 *
 *  gamma_q  [c] float32 per-dimension gain, 16-byte aligned
 *  eps      >= 0;  rope_dims  even, 0 .. c;  base > 0 when rope_dims > 0
 *  every other argument and the workspace as for csa_attend (the workspace
 *  size is csa_attend_workspace_size()).
 *
 * Errors: as csa_attend, plus CSA_EINVAL for a NULL or misaligned gamma_q, a
 * negative or non-finite eps, an odd or negative rope_dims or one above c, a
 * bad base, or a position beyond 2^40; CSA_ENOTSUP outside bf16, c = 512,
 * n_h a multiple of 64 and k <= 2048.
 */
int csa_attend_norm_rope(const void* q, const float* gamma_q, float eps, int64_t rope_dims, double base,
                         const void* Ccomp, int64_t comp_bstride, const int32_t* idx, const void* kv_raw,
                         int64_t raw_bstride, int64_t raw_pos0, const float* sink, int64_t b, int64_t n_q,
                         int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c, int64_t k, int64_t m,
                         int64_t n_win, float scale, int dtype, void* workspace, size_t ws_bytes, void* out,
                         void* stream);

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

/*
 * hca_attend_norm_rope -- hca_attend with the query side of the norm and
 * partial RoPE folded in, as csa_attend_norm_rope does for CSA (songhuiming
 * "DeepSeek-V4 百万 token 上下文" sections 4.5 and 5.2; AirCoding
 * "deepseek-paper-analysis" sections 7.1-7.2): q holds the raw query heads,
 * each RMS-normalised with gain gamma_q and its last rope_dims dimensions
 * rotated at the query's position as it is loaded (rounded to bf16 once);
 * the output's rotated dimensions are turned back by -t in float32 and
 * stored once in bf16.  gamma_q, eps, rope_dims and base as in
 * csa_attend_norm_rope; every other argument and the workspace (size
 * hca_attend_workspace_size()) as in hca_attend.
 * Errors: as hca_attend, plus the gain, eps, rope_dims, base and position
 * checks of csa_attend_norm_rope; CSA_ENOTSUP outside bf16, c = 512 and n_h
 * a multiple of 64.
 */
int hca_attend_norm_rope(const void* q, const float* gamma_q, float eps, int64_t rope_dims, double base,
                         const void* Ccomp, int64_t comp_bstride, const void* kv_raw, int64_t raw_bstride,
                         int64_t raw_pos0, const float* sink, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp,
                         int64_t n_raw, int64_t n_h, int64_t c, int64_t m_prime, int64_t n_win, float scale,
                         int dtype, void* workspace, size_t ws_bytes, void* out, void* stream);

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

/* ------------------------------------------------------------------------
 * FP8 KV entries (AirCoding "deepseek-paper-analysis" section 7.3, KV mixed
 * precision storage; polysight "06-formulas" B9): compressed entries keep
 * their RoPE dimensions (the last rope_dims) in BF16 and store the others
 * as OCP E4M3 codes with one power-of-two scale per entry.
 * ------------------------------------------------------------------------ */

/*
 * csa_quantize_kv_fp8 -- encode `rows` entries x [rows][x_rstride] (float32
 * or bf16, the first c values of a row): scale[i] = the smallest 2^e with
 * max |x[i][d]| / 2^e <= 448 over the non-RoPE dims d < c - rope_dims (2^0
 * for an all-zero row); codes[i][d] = the E4M3 code nearest to
 * x[i][d] / scale[i] (ties to the even code, sign kept);
 * rope[i][d] = bf16(x[i][c - rope_dims + d]).
 *  codes [rows][codes_rstride] uint8, rope [rows][rope_rstride] bf16,
 *  scale [rows] float32.  rope_dims and c - rope_dims multiples of 8.
 * Errors: CSA_EINVAL for NULL pointers, rows < 1, sizes or strides out of
 * range, misalignment; CSA_ENOTSUP for another dtype.
 */
int csa_quantize_kv_fp8(const void* x, int64_t x_rstride, int64_t rows, int64_t c, int64_t rope_dims, int dtype,
                        void* codes, int64_t codes_rstride, void* rope, int64_t rope_rstride, float* scale,
                        void* stream);

/*
 * csa_attend_fp8kv -- csa_attend (bf16 queries, window rows and output)
 * with the compressed entries stored by csa_quantize_kv_fp8: codes
 * [b][*][c - rope_dims], rope [b][*][rope_dims], scale [b][*], dense rows,
 * comp_bstride entries from one sequence's first entry to the next (0 =
 * n_comp).  The attention reads the values the stored entries stand for: it
 * decodes the entries the call reads into bf16 rows in the workspace (every
 * entry for a block of queries; for one query per sequence with more
 * entries than k, only the selected ones) and attends over them.  Workspace:
 * csa_attend_fp8kv_workspace_size() bytes, 256-byte aligned.
 * Errors: as csa_attend; CSA_ENOTSUP for k > 2048.
 */
int csa_attend_fp8kv(const void* q, const void* codes, const void* rope, const float* scale, int64_t comp_bstride,
                     const int32_t* idx, const void* kv_raw, int64_t raw_bstride, int64_t raw_pos0, const float* sink,
                     int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c,
                     int64_t rope_dims, int64_t k, int64_t m, int64_t n_win, float sm_scale, void* workspace,
                     size_t ws_bytes, void* out, void* stream);
size_t csa_attend_fp8kv_workspace_size(int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h, int64_t c,
                                       int64_t k, int64_t m, int64_t n_win);

/* ------------------------------------------------------------------------
 * Backward pass (training needs the layer's gradients; AirCoding
 * "deepseek-paper-analysis" section 7.6 asks that the attention backward's
 * reductions be deterministic: per-unit accumulation buffers summed in a
 * fixed order, no floating-point atomics).  Gradients are float32 whatever
 * the storage type of the inputs.
 * ------------------------------------------------------------------------ */

/*
 * csa_attend_backward -- gradients of csa_attend (same arguments, same entry
 * sets) given dout = dL/dout [b, n_q, n_h, c] in the storage type:
 *   dl_j = p_j (g . e_j - g . o),  dz_h = -p_sink (g . o),
 *   dq = scale sum_j dl_j e_j,     de_j = p_j g + scale dl_j q
 * (p the softmax weights, g = dout of the head, o its output; each entry is
 * both key and value, so its gradient sums both roles over every head and
 * every query that read it).
 *  dq      out [b, n_q, n_h, c] float32
 *  dCcomp  out [b, *, c] float32 (dcomp_bstride, 0 = dense): rows of entries
 *          no query of the block selected get 0
 *  dkv_raw out [b, n_raw, c] float32 (draw_bstride): window rows
 *  dsink   out [n_h] float32, summed over sequences and queries
 *  accumulate  0: write the gradients; 1: add them to dCcomp, dkv_raw and
 *          dsink (process the queries of a long sequence in blocks, in
 *          order; dq is always written)
 * Each idx row must list its valid entries in ascending order without
 * repeats (as csa_index_topk returns them).  Workspace:
 * csa_attend_backward_workspace_size() bytes, 256-byte aligned: the
 * per-(query, slot) contributions, 4 (k + n_win) c bytes per query plus
 * 8 n_h (k + n_win) bytes per query.  The sums run over queries in order.
 * Errors: as csa_attend; CSA_ENOTSUP for c > 1024 or n_h > 512.
 */
int csa_attend_backward(const void* q, const void* Ccomp, int64_t comp_bstride, const int32_t* idx,
                        const void* kv_raw, int64_t raw_bstride, int64_t raw_pos0, const float* sink, const void* dout,
                        int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c,
                        int64_t k, int64_t m, int64_t n_win, float scale, int dtype, int accumulate, float* dq,
                        float* dCcomp, int64_t dcomp_bstride, float* dkv_raw, int64_t draw_bstride, float* dsink,
                        void* workspace, size_t ws_bytes, void* stream);
size_t csa_attend_backward_workspace_size(int64_t b, int64_t n_q, int64_t n_h, int64_t c, int64_t k, int64_t n_win);

/* hca_attend_backward -- the same for hca_attend (every completed entry
 * read; workspace grows with n_comp instead of k). */
int hca_attend_backward(const void* q, const void* Ccomp, int64_t comp_bstride, const void* kv_raw,
                        int64_t raw_bstride, int64_t raw_pos0, const float* sink, const void* dout, int64_t b,
                        int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c,
                        int64_t m_prime, int64_t n_win, float scale, int dtype, int accumulate, float* dq,
                        float* dCcomp, int64_t dcomp_bstride, float* dkv_raw, int64_t draw_bstride, float* dsink,
                        void* workspace, size_t ws_bytes, void* stream);
size_t hca_attend_backward_workspace_size(int64_t b, int64_t n_q, int64_t n_h, int64_t c, int64_t n_comp,
                                          int64_t n_win);

/*
 * csa_compress_backward -- gradients of csa_compress (same inputs) given
 * dCcomp [b, n/m, c] float32 (dense): with S the weights of entry i and
 * Cc_i its value, every row j the entry reads gets dC_j = S_j dCcomp_i and
 * dZ_j = S_j (C_j - Cc_i) dCcomp_i; rows no entry reads (the last block's
 * stream-b rows, a ragged tail) get 0; dBa / dBb [m, c] sum dZ of each
 * in-block row over entries and sequences, in order.  dCa, dCb, dZa, dZb
 * [b, n, c] float32; dprev_Cb, dprev_Zb [b, m, c] float32, required when
 * prev_Cb / prev_Zb are given (else may be NULL).  overlap = 0: the pooling
 * form (Cb, Zb, Bb, dCb, dZb, dBb NULL).  Workspace:
 * csa_compress_backward_workspace_size() bytes, 256-byte aligned.
 */
int csa_compress_backward(const void* Ca, const void* Cb, const void* Za, const void* Zb, const void* Ba,
                          const void* Bb, const void* prev_Cb, const void* prev_Zb, const float* dCcomp, int64_t b,
                          int64_t n, int64_t c, int64_t m, int overlap, int dtype, float* dCa, float* dCb, float* dZa,
                          float* dZb, float* dBa, float* dBb, float* dprev_Cb, float* dprev_Zb, void* workspace,
                          size_t ws_bytes, void* stream);
size_t csa_compress_backward_workspace_size(int64_t n, int64_t c, int64_t m);

/* ------------------------------------------------------------------------
 * Heterogeneous decode cache (AirCoding "deepseek-paper-analysis" section
 * 7.6, Inference KV Cache) for one CSA layer and one HCA layer, batched over
 * requests of different lengths.
 *
 * Classical cache: a pool of blocks in one device array; block j starts at
 * blocks + j * csa_paged_block_bytes().  A block covers L = lcm(m, m')
 * tokens and holds, in bf16, [L/m][c] CSA entries, [L/m][c_I] indexer keys
 * and [L/m'][c] HCA entries, in that order (m = 4, m' = 128: 32, 32 and 1;
 * 41 KiB at c = 512, c_I = 128).  CSA entry s of a request lives in block
 * block_table[req][s / (L/m)], at slot s % (L/m); HCA entry s in block
 * block_table[req][s / (L/m')].  The caller owns the table
 * ([requests][bt_stride] int32, device) and fills it from a block pool
 * (csa_block_pool_*): block floor(t / L) must be in place before token t is
 * appended.  Block ids are clamped into [0, n_blocks) before use.
 *
 * State cache: csa_paged_state_bytes() per request, fixed whatever the
 * request's length: the CSA window ring [n_win][c] (rows C^a at slot
 * t % n_win), the open CSA block [4][m][c] (C^a, C^b, Z^a, Z^b at slot
 * t % m), the previous block's [2][m][c] (C^b, Z^b), the same two for the
 * indexer-key streams with c_I, the HCA window ring [n_win][c] (rows C) and
 * the open HCA block [2][m'][c] (C, Z).  Request r's state starts at
 * state + r * csa_paged_state_bytes(); its contents are private to the
 * library; it needs no initialisation (every word is written before it is
 * read), so a slot can be reused for a new request as it is.
 *
 * Batches: row i of a call is request req_slot[i] (req_slot NULL: request
 * i), whose newest token is at position pos[i] (int64, device).  Queries
 * are one per row, at pos[i].  n_comp_max / n_hca_max bound every row's
 * completed entries ((pos+1)/m, (pos+1)/m'); rows are clamped to them.
 * dtype must be CSA_BF16; c and c_I multiples of 8; L/m a power of two of
 * at least 32 and L/m' a power of two; c_I * L/m a multiple of c.
 * ------------------------------------------------------------------------ */

/* Bytes of one classical-cache block, and of one request's state (0 for
 * sizes without a layout). */
size_t csa_paged_block_bytes(int64_t c, int64_t c_I, int64_t m, int64_t m_prime);
size_t csa_paged_state_bytes(int64_t c, int64_t c_I, int64_t m, int64_t m_prime, int64_t n_win);

/*
 * csa_paged_append -- add each row's newest token (position pos[i]) to its
 * request: the token's rows of the CSA streams (Ca, Cb, Za, Zb [b][c]), the
 * indexer-key streams (ICa, ICb, IZa, IZb [b][c_I]) and the HCA streams
 * (C_h, Z_h [b][c]) go into the state cache; when position pos[i] completes
 * a CSA block ((pos+1) % m == 0) the overlapped compressor (biases Ba, Bb
 * [m][c] and IBa, IBb [m][c_I]; block -1 padded) writes CSA entry and
 * indexer key (pos+1)/m - 1 into the request's block, and when it completes
 * an HCA block ((pos+1) % m' == 0) the pooling compressor (bias B_h [m'][c])
 * writes HCA entry (pos+1)/m' - 1.  Positions must be appended in order,
 * 0, 1, 2, ... per request.  All tensors 16-byte aligned.
 * Errors: CSA_EINVAL for NULL or misaligned pointers and sizes < 1;
 * CSA_ENOTSUP for other dtypes or geometries without a layout.
 */
int csa_paged_append(void* state, void* blocks, int64_t n_blocks, const int32_t* block_table, int64_t bt_stride,
                     const int32_t* req_slot, const int64_t* pos, int64_t b, const void* Ca, const void* Cb,
                     const void* Za, const void* Zb, const void* ICa, const void* ICb, const void* IZa,
                     const void* IZb, const void* C_h, const void* Z_h, const void* Ba, const void* Bb,
                     const void* IBa, const void* IBb, const void* B_h, int64_t c, int64_t c_I, int64_t m,
                     int64_t m_prime, int64_t n_win, int dtype, void* stream);

/*
 * csa_paged_index_topk -- csa_index_topk for one query per row (qI
 * [b][n_hI][c_I], w [b][n_hI]) at position pos[i], over the request's
 * (pos+1)/m indexer keys in its blocks.  idx [b][k] holds entry numbers s
 * (ascending, -1 padded), as csa_paged_attend takes them.  Workspace:
 * csa_index_topk_workspace_size(b, 1, n_comp_max, k) bytes, 256-byte
 * aligned.  n_hI in {32, 64, 128}, c_I in {64, 128}.
 * Errors: as csa_index_topk; CSA_EINVAL if n_comp_max exceeds the entries
 * bt_stride blocks hold.
 */
int csa_paged_index_topk(const void* qI, const float* w, const void* blocks, int64_t n_blocks,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* req_slot, const int64_t* pos,
                         int64_t b, int64_t n_comp_max, int64_t n_hI, int64_t c_I, int64_t c, int64_t m,
                         int64_t m_prime, int64_t k, int dtype, int32_t* idx, float* score, void* workspace,
                         size_t ws_bytes, void* stream);

/*
 * csa_paged_attend -- csa_attend for one query per row (q [b][n_h][c]) at
 * position pos[i]: the selected CSA entries (idx [b][k], entry numbers;
 * indices outside [0, (pos+1)/m) skipped) from the request's blocks plus the
 * window rows of positions max(0, pos-n_win+1) .. pos from its CSA window
 * ring, one softmax with the sink.  out [b][n_h][c].  c = 512, n_h a
 * multiple of 64, k <= 2048.  Workspace: csa_paged_attend_workspace_size()
 * bytes (0: none).
 */
int csa_paged_attend(const void* q, const void* blocks, int64_t n_blocks, const int32_t* block_table,
                     int64_t bt_stride, const int32_t* req_slot, const int64_t* pos, const int32_t* idx,
                     const void* state, const float* sink, int64_t b, int64_t n_comp_max, int64_t n_h, int64_t c,
                     int64_t c_I, int64_t k, int64_t m, int64_t m_prime, int64_t n_win, float scale, int dtype,
                     void* workspace, size_t ws_bytes, void* out, void* stream);
size_t csa_paged_attend_workspace_size(int64_t b, int64_t n_h, int64_t k, int64_t n_win);

/*
 * hca_paged_attend -- hca_attend for one query per row at position pos[i]:
 * every completed HCA entry ((pos+1)/m') of the request's blocks plus the
 * window from its HCA window ring.  As csa_paged_attend otherwise;
 * CSA_ENOTSUP also when n_hca_max + n_win exceeds 2^25 entries (the list is
 * split at least every 2048 entries, and the split merge takes at most
 * 16384 splits).
 */
int hca_paged_attend(const void* q, const void* blocks, int64_t n_blocks, const int32_t* block_table,
                     int64_t bt_stride, const int32_t* req_slot, const int64_t* pos, const void* state,
                     const float* sink, int64_t b, int64_t n_hca_max, int64_t n_h, int64_t c, int64_t c_I, int64_t m,
                     int64_t m_prime, int64_t n_win, float scale, int dtype, void* workspace, size_t ws_bytes,
                     void* out, void* stream);
size_t hca_paged_attend_workspace_size(int64_t b, int64_t n_h, int64_t n_hca_max, int64_t n_win);

/*
 * Block pool (host memory only): hands out the ids 0 .. n_blocks-1 of one
 * device block array and takes them back; thread-safe.
 *  csa_block_pool_create   NULL if n_blocks < 1 or out of host memory
 *  csa_block_pool_alloc    n ids into ids[] (host array); CSA_ENOSPC, with
 *                          nothing taken, if fewer than n are free
 *  csa_block_pool_release  CSA_EINVAL, with nothing released, if an id is
 *                          not allocated or appears twice
 *  csa_block_pool_available  free ids (-1 for a NULL pool)
 */
typedef struct csa_block_pool csa_block_pool;
csa_block_pool* csa_block_pool_create(int64_t n_blocks);
void csa_block_pool_destroy(csa_block_pool* pool);
int csa_block_pool_alloc(csa_block_pool* pool, int64_t n, int32_t* ids);
int csa_block_pool_release(csa_block_pool* pool, int64_t n, const int32_t* ids);
int64_t csa_block_pool_available(csa_block_pool* pool);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
