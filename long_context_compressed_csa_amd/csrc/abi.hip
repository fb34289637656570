// C ABI of the CSA/HCA library: host-side argument validation, then kernel
// launches on the caller's stream.  Nothing here allocates device memory or
// synchronises.  The operations are defined in include/csa.h.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "csa.h"
#include "kernels.hpp"

namespace {

inline bool dtype_ok(int dt) { return dt == CSA_F32 || dt == CSA_BF16; }
inline int64_t elem_bytes(int dt) { return dt == CSA_F32 ? 4 : dt == CSA_BF16 ? 2 : 1; }

// NULL, or a multiple of `a` bytes
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Rows whose byte length is a multiple of 16 are moved with 16-byte vector
// loads and stores: their pointers must then be 16-byte aligned and every
// row/batch stride a multiple of 16 bytes; other rows need only the
// element's natural alignment.
inline uintptr_t row_align(int64_t row_bytes, int64_t es) { return row_bytes % 16 == 0 ? 16 : (uintptr_t)es; }
inline bool stride_ok(int64_t stride_elems, int64_t es, uintptr_t a) { return (stride_elems * es) % (int64_t)a == 0; }
inline int launched(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_EHIP; }

// Debug builds: a launch that went through turns into CSA_EBOUNDS when a
// gather's bounds check failed (this waits for the stream).
#if CSA_DEBUG
inline int debug_checked(int rc, void* stream) {
  return rc == CSA_OK && csa::debug_take_oob((hipStream_t)stream) ? CSA_EBOUNDS : rc;
}
#else
inline int debug_checked(int rc, void*) { return rc; }
#endif

inline int64_t visible(int64_t t, int64_t m) { return (t + 1) / m; }

// Window rows of queries t0..t0+n_q-1 must lie inside kv_raw.
inline bool window_covered(int64_t t0, int64_t n_q, int64_t n_win, int64_t raw_pos0, int64_t n_raw) {
  const int64_t lo = t0 - n_win + 1 > 0 ? t0 - n_win + 1 : 0;
  const int64_t hi = t0 + n_q - 1;
  return lo >= raw_pos0 && hi < raw_pos0 + n_raw;
}

int64_t attend_nmax(int dense, int64_t t0, int64_t n_q, int64_t n_comp, int64_t k, int64_t m,
                    int64_t n_win) {
  int64_t v = visible(t0 + n_q - 1, m);
  if (v > n_comp) v = n_comp;
  return (dense ? v : k) + n_win;
}

int check_attend(const void* q, const void* Ccomp, int64_t cbs, const void* kv_raw, int64_t rbs,
                 int64_t raw_pos0, const float* sink, int64_t b, int64_t n_q, int64_t t0,
                 int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c, int64_t m, int64_t n_win,
                 float scale, int dtype, const void* out) {
  if (!dtype_ok(dtype)) return CSA_ENOTSUP;
  if (!q || !kv_raw || !sink || !out) return CSA_EINVAL;
  if (n_comp > 0 && !Ccomp) return CSA_EINVAL;
  if (b < 1 || n_q < 1 || n_h < 1 || c < 1 || m < 1 || n_win < 1 || n_raw < 1) return CSA_EINVAL;
  if (t0 < 0 || n_comp < 0 || !isfinite(scale) || !(scale > 0.f)) return CSA_EINVAL;
  if (cbs < 0 || rbs < 0) return CSA_EINVAL;
  if (cbs > 0 && cbs < n_comp * c) return CSA_EINVAL;
  if (rbs > 0 && rbs < n_raw * c) return CSA_EINVAL;
  if (!window_covered(t0, n_q, n_win, raw_pos0, n_raw)) return CSA_EINVAL;
  // the MFMA path (bf16, c = 512) gathers and stores whole rows 16 bytes per lane
  const int64_t es = elem_bytes(dtype);
  const uintptr_t a = (dtype == CSA_BF16 && c == 512 && n_h % 64 == 0) ? 16 : (uintptr_t)es;
  if (!aligned(q, a) || !aligned(Ccomp, a) || !aligned(kv_raw, a) || !aligned(out, a) || !aligned(sink, 4))
    return CSA_EINVAL;
  if (!stride_ok(cbs, es, a) || !stride_ok(rbs, es, a)) return CSA_EINVAL;
  return CSA_OK;
}

}  // namespace

extern "C" {

const char* csa_version(void) { return "csa-mi355x 0.1.0"; }

const char* csa_strerror(int code) {
  switch (code) {
    case CSA_OK: return "ok";
    case CSA_EINVAL: return "invalid argument";
    case CSA_ENOTSUP: return "unsupported shape or dtype";
    case CSA_ENOSPC: return "workspace too small";
    case CSA_EHIP: return "HIP launch error";
    case CSA_EBOUNDS: return "bounds check failed (debug build)";
    default: return "unknown error";
  }
}

int csa_debug_enabled(void) { return CSA_DEBUG ? 1 : 0; }

int csa_debug_set_entry_limit(int64_t limit) {
#if CSA_DEBUG
  if (limit < 0) return CSA_EINVAL;
  return launched(csa::debug_set_entry_limit(limit));
#else
  (void)limit;
  return CSA_ENOTSUP;
#endif
}

int csa_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb, const void* Ba,
                 const void* Bb, const void* prev_Cb, const void* prev_Zb, int64_t b, int64_t n,
                 int64_t c, int64_t m, int overlap, int dtype, void* Ccomp, int64_t out_bstride,
                 void* stream) {
  if (!dtype_ok(dtype)) return CSA_ENOTSUP;
  if (b < 1 || n < 1 || c < 1 || m < 1) return CSA_EINVAL;
  if (overlap != 0 && overlap != 1) return CSA_EINVAL;
  if (!Ca || !Za || !Ba || !Ccomp) return CSA_EINVAL;
  if (overlap) {
    if (!Cb || !Zb || !Bb) return CSA_EINVAL;
    if ((prev_Cb == nullptr) != (prev_Zb == nullptr)) return CSA_EINVAL;
  } else {
    if (Cb || Zb || Bb || prev_Cb || prev_Zb) return CSA_EINVAL;
  }
  const int64_t ne = n / m;
  if (out_bstride < 0 || (out_bstride > 0 && out_bstride < ne * c)) return CSA_EINVAL;
  {
    const int64_t es = elem_bytes(dtype);
    const uintptr_t a = row_align(c * es, es);
    const void* ps[] = {Ca, Cb, Za, Zb, Ba, Bb, prev_Cb, prev_Zb, Ccomp};
    for (const void* p : ps)
      if (!aligned(p, a)) return CSA_EINVAL;
    if (!stride_ok(out_bstride, es, a)) return CSA_EINVAL;
  }
  if (b > 65535) return CSA_ENOTSUP;
  const int64_t obs = out_bstride > 0 ? out_bstride : ne * c;
  return launched(csa::launch_compress(Ca, Cb, Za, Zb, Ba, Bb, prev_Cb, prev_Zb, b, n, c, m,
                                       overlap, dtype, Ccomp, obs, (hipStream_t)stream));
}

size_t csa_index_topk_workspace_size(int64_t b, int64_t n_q, int64_t n_comp, int64_t k) {
  if (b < 1 || n_q < 1 || n_comp < 0 || k < 1) return 0;
  return csa::index_topk_workspace_bytes(b, n_q, n_comp, k);
}

}  // extern "C"

namespace {

int check_index_topk(const void* qI, const float* w, const void* KIcomp, int64_t comp_bstride, int64_t b,
                     int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_hI, int64_t c_I, int64_t m, int64_t k,
                     int dtype_flags, const int32_t* idx, const float* score) {
  // the element type, and CSA_SCORE_BF16 for float32 / bf16 queries and keys
  const int dtype = dtype_flags & 0xff;
  if ((dtype_flags & ~0x1ff) != 0) return CSA_ENOTSUP;
  if ((dtype_flags & CSA_SCORE_BF16) && dtype == CSA_FP8) return CSA_ENOTSUP;
  if (!dtype_ok(dtype) && dtype != CSA_FP8) return CSA_ENOTSUP;
  if (!qI || !w || !idx) return CSA_EINVAL;
  if (n_comp > 0 && !KIcomp) return CSA_EINVAL;
  if (b < 1 || n_q < 1 || n_hI < 1 || c_I < 1 || m < 1 || k < 1 || t0 < 0 || n_comp < 0)
    return CSA_EINVAL;
  if (n_comp > visible(t0 + n_q - 1, m)) return CSA_EINVAL;
  if (comp_bstride < 0 || (comp_bstride > 0 && comp_bstride < n_comp * c_I)) return CSA_EINVAL;
  {
    const int64_t es = elem_bytes(dtype);
    const uintptr_t a = row_align(c_I * es, es);
    if (!aligned(qI, a) || !aligned(KIcomp, a) || !stride_ok(comp_bstride, es, a)) return CSA_EINVAL;
    if (!aligned(w, 4) || !aligned(idx, 4) || !aligned(score, 4)) return CSA_EINVAL;
  }
  if (n_q > 65535 || b > 65535) return CSA_ENOTSUP;
  if (!csa::index_topk_supported(n_comp, k)) return CSA_ENOTSUP;
  return CSA_OK;
}

// Scratch of csa_index_topk_noalloc: one array per GPU, placed by the loader
// with the code object (no allocation call at any time).  In host code the
// array's name stands for a host-side shadow, not a device address: kernels
// get the address hipGetSymbolAddress returns for the current device, looked
// up on the first call on each device and kept here.
static_assert(CSA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CSA_EHIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return CSA_OK;
}

}  // namespace

extern "C" {

int csa_index_topk(const void* qI, const float* w, const void* KIcomp, int64_t comp_bstride,
                   int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_hI, int64_t c_I,
                   int64_t m, int64_t k, int dtype, int32_t* idx, float* score, void* workspace,
                   size_t ws_bytes, void* stream) {
  int rc = check_index_topk(qI, w, KIcomp, comp_bstride, b, n_q, t0, n_comp, n_hI, c_I, m, k, dtype, idx, score);
  if (rc != CSA_OK) return rc;
  if (!workspace || ((uintptr_t)workspace & 255u) != 0) return CSA_EINVAL;
  if (ws_bytes < csa::index_topk_workspace_bytes(b, n_q, n_comp, k)) return CSA_ENOSPC;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp * c_I;
  return launched(csa::launch_index_topk(qI, w, KIcomp, cbs, b, n_q, t0, n_comp, n_hI, c_I, m, k,
                                         dtype, idx, score, workspace, (hipStream_t)stream));
}

int csa_index_topk_noalloc(const void* qI, const float* w, const void* KIcomp, int64_t comp_bstride, int64_t b,
                           int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_hI, int64_t c_I, int64_t m,
                           int64_t k, int dtype, int32_t* idx, float* score, void* stream) {
  int rc = check_index_topk(qI, w, KIcomp, comp_bstride, b, n_q, t0, n_comp, n_hI, c_I, m, k, dtype, idx, score);
  if (rc != CSA_OK) return rc;
  if (csa::index_topk_workspace_bytes(b, n_q, n_comp, k) > (size_t)CSA_NOALLOC_SCRATCH_BYTES) return CSA_ENOSPC;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != CSA_OK) return rc;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp * c_I;
  return launched(csa::launch_index_topk(qI, w, KIcomp, cbs, b, n_q, t0, n_comp, n_hI, c_I, m, k,
                                         dtype, idx, score, ws, (hipStream_t)stream));
}

int csa_index_topk_mxfp4(const void* qI, const void* qI_scale, const float* w, const void* KIcomp,
                         const void* KI_scale, int64_t comp_bstride, int64_t b, int64_t n_q, int64_t t0,
                         int64_t n_comp, int64_t n_hI, int64_t c_I, int64_t m, int64_t k, int32_t* idx,
                         float* score, void* workspace, size_t ws_bytes, void* stream) {
  if (!qI || !qI_scale || !w || !idx || !workspace) return CSA_EINVAL;
  if (n_comp > 0 && (!KIcomp || !KI_scale)) return CSA_EINVAL;
  if (b < 1 || n_q < 1 || n_hI < 1 || c_I < 1 || m < 1 || k < 1 || t0 < 0 || n_comp < 0)
    return CSA_EINVAL;
  if (c_I % 32 != 0) return CSA_EINVAL;
  if (n_comp > visible(t0 + n_q - 1, m)) return CSA_EINVAL;
  if (comp_bstride < 0 || (comp_bstride > 0 && comp_bstride < n_comp)) return CSA_EINVAL;
  // code rows (c_I/2 bytes, a multiple of 16) are loaded 16 bytes at a time,
  // a head's or key's scales (c_I/32 bytes) 4 at a time when they fill words
  {
    const uintptr_t as = (c_I / 32) % 4 == 0 ? 4 : 1;
    if (!aligned(qI, 16) || !aligned(KIcomp, 16) || !aligned(qI_scale, as) || !aligned(KI_scale, as))
      return CSA_EINVAL;
    if (((comp_bstride * (c_I / 32)) % (int64_t)as) != 0) return CSA_EINVAL;
    if (!aligned(w, 4) || !aligned(idx, 4) || !aligned(score, 4)) return CSA_EINVAL;
  }
  if (n_q > 65535 || b > 65535) return CSA_ENOTSUP;
  if (!csa::index_topk_supported(n_comp, k) || !csa::index_topk_mx_supported(n_q, n_hI, c_I)) return CSA_ENOTSUP;
  if (((uintptr_t)workspace & 255u) != 0) return CSA_EINVAL;
  if (ws_bytes < csa::index_topk_workspace_bytes(b, n_q, n_comp, k)) return CSA_ENOSPC;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp;
  return launched(csa::launch_index_topk_mx(qI, qI_scale, w, KIcomp, KI_scale, cbs, b, n_q, t0, n_comp, n_hI, c_I,
                                            m, k, idx, score, workspace, (hipStream_t)stream));
}

int csa_quantize_mxfp4(const void* x, int64_t x_rstride, int64_t rows, int64_t c, int dtype, void* codes,
                       int64_t codes_rstride, void* scales, int64_t scales_rstride, void* stream) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return CSA_ENOTSUP;
  if (!x || !codes || !scales) return CSA_EINVAL;
  if (rows < 1 || c < 32 || c % 32 != 0) return CSA_EINVAL;
  if (x_rstride < c || codes_rstride < c / 2 || scales_rstride < c / 32) return CSA_EINVAL;
  const int64_t es = dtype == CSA_F32 ? 4 : 2;
  // 16-byte loads of the values and stores of the codes
  if (((uintptr_t)x & 15u) != 0 || (x_rstride * es) % 16 != 0 || ((uintptr_t)codes & 15u) != 0 ||
      codes_rstride % 16 != 0)
    return CSA_EINVAL;
  return launched(csa::launch_quantize_mxfp4(x, x_rstride, rows, c, dtype, codes, codes_rstride, scales,
                                             scales_rstride, (hipStream_t)stream));
}

int csa_norm_rope(const void* x, int64_t x_rstride, void* out, int64_t out_rstride, const float* gamma,
                  float eps, int64_t rows, int64_t heads, int64_t c, int64_t rope_dims, double base,
                  int64_t pos0, int64_t pos_step, int dtype, void* stream) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return CSA_ENOTSUP;
  if (rows < 0 || heads < 1 || c < 1) return CSA_EINVAL;
  if (rope_dims < 0 || rope_dims > c || (rope_dims & 1)) return CSA_EINVAL;
  if (!(eps >= 0.f) || !isfinite(eps)) return CSA_EINVAL;
  if (rope_dims > 0 && !(base > 0.0 && isfinite(base))) return CSA_EINVAL;
  const int64_t es = dtype == CSA_F32 ? 4 : 2, V = 16 / es;
  if (x_rstride < heads * c || out_rstride < heads * c) return CSA_EINVAL;
  // positions stay far inside the range where float64 holds them and their angles exactly
  const int64_t kPosMax = 1LL << 40;
  if (pos0 > kPosMax || pos0 < -kPosMax || pos_step > kPosMax || pos_step < -kPosMax) return CSA_EINVAL;
  if (rows > 0) {
    const int64_t last = pos0 + (rows - 1) * pos_step;
    if (rows > kPosMax || last > kPosMax || last < -kPosMax) return CSA_EINVAL;
  }
  if (c % V != 0 || c > 256 * V || rope_dims > 512) return CSA_ENOTSUP;
  if (rows > 2147483647LL || heads * c > 2147483647LL) return CSA_ENOTSUP;
  if (rows == 0) return CSA_OK;
  if (!x || !out) return CSA_EINVAL;
  // 16-byte loads and stores
  if (((uintptr_t)x & 15u) != 0 || ((uintptr_t)out & 15u) != 0 || (x_rstride * es) % 16 != 0 ||
      (out_rstride * es) % 16 != 0 || ((uintptr_t)gamma & 15u) != 0)
    return CSA_EINVAL;
  // in place (same pointer and stride) or disjoint
  const uintptr_t xa = (uintptr_t)x, oa = (uintptr_t)out;
  const uintptr_t xe = xa + (uintptr_t)(((rows - 1) * x_rstride + heads * c) * es);
  const uintptr_t oe = oa + (uintptr_t)(((rows - 1) * out_rstride + heads * c) * es);
  if (!(xa == oa && x_rstride == out_rstride) && xa < oe && oa < xe) return CSA_EINVAL;
  return launched(csa::launch_norm_rope(x, x_rstride, out, out_rstride, gamma, eps, rows, heads, c, rope_dims,
                                        base, pos0, pos_step, dtype, (hipStream_t)stream));
}

int csa_grouped_out_proj(const void* o, const void* WG, const void* WO, int64_t n, int64_t n_h, int64_t c,
                         int64_t g, int64_t d_g, int64_t d, int dtype, void* mid, void* out, void* stream) {
  if (n < 0 || n_h < 1 || c < 1 || g < 1 || d_g < 1 || d < 1) return CSA_EINVAL;
  if (n_h % g != 0) return CSA_EINVAL;
  if (dtype != CSA_BF16) return CSA_ENOTSUP;
  const int64_t K1 = (n_h / g) * c, K2 = g * d_g;
  // K advances 64 values at a time; rows are gathered 16 bytes per lane
  if (K1 % 64 != 0 || K2 % 64 != 0) return CSA_ENOTSUP;
  if (n > 2147483647LL || d_g > 2147483647LL || d > 2147483647LL || g > 65535 || K1 > 2147483647LL ||
      K2 > 2147483647LL)
    return CSA_ENOTSUP;
  if ((int64_t)((n + 255) / 256) * ((d_g + 127) / 128) > 2147483647LL ||
      (int64_t)((n + 255) / 256) * ((d + 127) / 128) > 2147483647LL)
    return CSA_ENOTSUP;
  if (n == 0) return CSA_OK;
  if (!o || !WG || !WO || !mid || !out) return CSA_EINVAL;
  if (((uintptr_t)o & 15u) != 0 || ((uintptr_t)WG & 15u) != 0 || ((uintptr_t)WO & 15u) != 0 ||
      ((uintptr_t)mid & 15u) != 0)
    return CSA_EINVAL;
  return launched(csa::launch_grouped_out_proj(o, WG, WO, n, n_h, c, g, d_g, d, mid, out, (hipStream_t)stream));
}

size_t csa_attend_workspace_size(int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h,
                                 int64_t c, int64_t k, int64_t m, int64_t n_win, int dtype) {
  if (b < 1 || n_q < 1 || m < 1 || t0 < 0 || k < 0 || n_win < 1) return 0;
  return csa::attend_workspace_bytes(dtype, b, n_q, n_h, c, attend_nmax(0, t0, n_q, n_comp, k, m, n_win));
}

size_t hca_attend_workspace_size(int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h,
                                 int64_t c, int64_t m_prime, int64_t n_win, int dtype) {
  if (b < 1 || n_q < 1 || m_prime < 1 || t0 < 0 || n_win < 1) return 0;
  return csa::attend_workspace_bytes(dtype, b, n_q, n_h, c,
                                     attend_nmax(1, t0, n_q, n_comp, 0, m_prime, n_win));
}

int csa_attend(const void* q, const void* Ccomp, int64_t comp_bstride, const int32_t* idx,
               const void* kv_raw, int64_t raw_bstride, int64_t raw_pos0, const float* sink,
               int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h,
               int64_t c, int64_t k, int64_t m, int64_t n_win, float scale, int dtype,
               void* workspace, size_t ws_bytes, void* out, void* stream) {
  int rc = check_attend(q, Ccomp, comp_bstride, kv_raw, raw_bstride, raw_pos0, sink, b, n_q, t0,
                        n_comp, n_raw, n_h, c, m, n_win, scale, dtype, out);
  if (rc != CSA_OK) return rc;
  if (k < 0 || (k > 0 && !idx)) return CSA_EINVAL;
  if (n_q > 2147483647LL || b > 65535 || n_h > 65535) return CSA_ENOTSUP;
  if (!csa::attend_supported(dtype, n_h, c, k)) return CSA_ENOTSUP;
  const size_t need = csa_attend_workspace_size(b, n_q, t0, n_comp, n_h, c, k, m, n_win, dtype);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) != 0)) return CSA_EINVAL;
  if (ws_bytes < need) return CSA_ENOSPC;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp * c;
  const int64_t rbs = raw_bstride > 0 ? raw_bstride : n_raw * c;
  return debug_checked(launched(csa::launch_attend(0, q, Ccomp, cbs, idx, kv_raw, rbs, raw_pos0, sink, b, n_q, t0,
                                     n_comp, n_h, c, k, m, n_win, scale, dtype, workspace, out,
                                     (hipStream_t)stream)), stream);
}

int csa_attend_norm_rope(const void* q, const float* gamma_q, float eps, int64_t rope_dims, double base,
                         const void* Ccomp, int64_t comp_bstride, const int32_t* idx, const void* kv_raw,
                         int64_t raw_bstride, int64_t raw_pos0, const float* sink, int64_t b, int64_t n_q,
                         int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c, int64_t k, int64_t m,
                         int64_t n_win, float scale, int dtype, void* workspace, size_t ws_bytes, void* out,
                         void* stream) {
  int rc = check_attend(q, Ccomp, comp_bstride, kv_raw, raw_bstride, raw_pos0, sink, b, n_q, t0,
                        n_comp, n_raw, n_h, c, m, n_win, scale, dtype, out);
  if (rc != CSA_OK) return rc;
  if (k < 0 || (k > 0 && !idx)) return CSA_EINVAL;
  if (!gamma_q || !aligned(gamma_q, 16) || !(eps >= 0.f) || !isfinite(eps)) return CSA_EINVAL;
  if (rope_dims < 0 || (rope_dims & 1) || rope_dims > c || (rope_dims > 0 && (!(base > 0.0) || !isfinite(base))))
    return CSA_EINVAL;
  if (t0 + n_q - 1 > (1LL << 40)) return CSA_EINVAL;
  if (dtype != CSA_BF16 || c != 512 || n_h % 64 != 0 || k > 2048) return CSA_ENOTSUP;
  if (n_q > 2147483647LL || b > 65535 || n_h > 65535) return CSA_ENOTSUP;
  const size_t need = csa_attend_workspace_size(b, n_q, t0, n_comp, n_h, c, k, m, n_win, dtype);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) != 0)) return CSA_EINVAL;
  if (ws_bytes < need) return CSA_ENOSPC;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp * c;
  const int64_t rbs = raw_bstride > 0 ? raw_bstride : n_raw * c;
  return launched(csa::launch_attend_norm_rope(0, q, gamma_q, eps, rope_dims, base, Ccomp, cbs, idx, kv_raw, rbs,
                                               raw_pos0, sink, b, n_q, t0, n_comp, n_h, k, m, n_win, scale,
                                               workspace, out, (hipStream_t)stream));
}

int hca_attend_norm_rope(const void* q, const float* gamma_q, float eps, int64_t rope_dims, double base,
                         const void* Ccomp, int64_t comp_bstride, const void* kv_raw, int64_t raw_bstride,
                         int64_t raw_pos0, const float* sink, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp,
                         int64_t n_raw, int64_t n_h, int64_t c, int64_t m_prime, int64_t n_win, float scale,
                         int dtype, void* workspace, size_t ws_bytes, void* out, void* stream) {
  int rc = check_attend(q, Ccomp, comp_bstride, kv_raw, raw_bstride, raw_pos0, sink, b, n_q, t0,
                        n_comp, n_raw, n_h, c, m_prime, n_win, scale, dtype, out);
  if (rc != CSA_OK) return rc;
  if (!gamma_q || !aligned(gamma_q, 16) || !(eps >= 0.f) || !isfinite(eps)) return CSA_EINVAL;
  if (rope_dims < 0 || (rope_dims & 1) || rope_dims > c || (rope_dims > 0 && (!(base > 0.0) || !isfinite(base))))
    return CSA_EINVAL;
  if (t0 + n_q - 1 > (1LL << 40)) return CSA_EINVAL;
  if (dtype != CSA_BF16 || c != 512 || n_h % 64 != 0) return CSA_ENOTSUP;
  if (n_q > 2147483647LL || b > 65535 || n_h > 65535) return CSA_ENOTSUP;
  const size_t need = hca_attend_workspace_size(b, n_q, t0, n_comp, n_h, c, m_prime, n_win, dtype);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) != 0)) return CSA_EINVAL;
  if (ws_bytes < need) return CSA_ENOSPC;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp * c;
  const int64_t rbs = raw_bstride > 0 ? raw_bstride : n_raw * c;
  return launched(csa::launch_attend_norm_rope(1, q, gamma_q, eps, rope_dims, base, Ccomp, cbs, nullptr, kv_raw, rbs,
                                               raw_pos0, sink, b, n_q, t0, n_comp, n_h, 0, m_prime, n_win, scale,
                                               workspace, out, (hipStream_t)stream));
}

int hca_attend(const void* q, const void* Ccomp, int64_t comp_bstride, const void* kv_raw,
               int64_t raw_bstride, int64_t raw_pos0, const float* sink, int64_t b, int64_t n_q,
               int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c, int64_t m_prime,
               int64_t n_win, float scale, int dtype, void* workspace, size_t ws_bytes, void* out,
               void* stream) {
  int rc = check_attend(q, Ccomp, comp_bstride, kv_raw, raw_bstride, raw_pos0, sink, b, n_q, t0,
                        n_comp, n_raw, n_h, c, m_prime, n_win, scale, dtype, out);
  if (rc != CSA_OK) return rc;
  if (n_q > 2147483647LL || b > 65535 || n_h > 65535) return CSA_ENOTSUP;
  if (!csa::attend_supported(dtype, n_h, c, 0)) return CSA_ENOTSUP;
  const size_t need = hca_attend_workspace_size(b, n_q, t0, n_comp, n_h, c, m_prime, n_win, dtype);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) != 0)) return CSA_EINVAL;
  if (ws_bytes < need) return CSA_ENOSPC;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp * c;
  const int64_t rbs = raw_bstride > 0 ? raw_bstride : n_raw * c;
  return debug_checked(launched(csa::launch_attend(1, q, Ccomp, cbs, nullptr, kv_raw, rbs, raw_pos0, sink, b, n_q,
                                     t0, n_comp, n_h, c, 0, m_prime, n_win, scale, dtype, workspace,
                                     out, (hipStream_t)stream)), stream);
}

size_t hca_layer_workspace_size(int64_t b, int64_t n, int64_t n_h, int64_t c, int64_t m_prime,
                                int64_t n_win, int dtype) {
  if (b < 1 || n < 1 || m_prime < 1) return 0;
  return hca_attend_workspace_size(b, n, 0, n / m_prime, n_h, c, m_prime, n_win, dtype);
}

int hca_layer(const void* C, const void* Z, const void* B, const void* q, const void* kv_raw,
              const float* sink, int64_t b, int64_t n, int64_t c, int64_t m_prime, int64_t n_h,
              int64_t n_win, float scale, int dtype, void* Ccomp, void* workspace, size_t ws_bytes,
              void* out, void* stream) {
  if (!dtype_ok(dtype)) return CSA_ENOTSUP;
  if (!C || !Z || !B || !q || !kv_raw || !sink || !Ccomp || !out) return CSA_EINVAL;
  if (b < 1 || n < 1 || c < 1 || m_prime < 1 || n_h < 1 || n_win < 1 || !isfinite(scale) || !(scale > 0.f))
    return CSA_EINVAL;
  const int64_t ne = n / m_prime;
  // validate the attention step before enqueuing the compressor
  int rc = check_attend(q, Ccomp, 0, kv_raw, 0, 0, sink, b, n, 0, ne, n, n_h, c, m_prime, n_win,
                        scale, dtype, out);
  if (rc != CSA_OK) return rc;
  {
    const int64_t es = elem_bytes(dtype);
    const uintptr_t a = row_align(c * es, es);
    if (!aligned(C, a) || !aligned(Z, a) || !aligned(B, a) || !aligned(Ccomp, a)) return CSA_EINVAL;
  }
  if (b > 65535 || n_h > 65535) return CSA_ENOTSUP;
  if (!csa::attend_supported(dtype, n_h, c, 0)) return CSA_ENOTSUP;
  const size_t need = hca_layer_workspace_size(b, n, n_h, c, m_prime, n_win, dtype);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) != 0)) return CSA_EINVAL;
  if (ws_bytes < need) return CSA_ENOSPC;
  hipStream_t st = (hipStream_t)stream;
  if (ne > 0) {
    hipError_t e = csa::launch_compress(C, nullptr, Z, nullptr, B, nullptr, nullptr, nullptr, b, n,
                                        c, m_prime, 0, dtype, Ccomp, ne * c, st);
    if (e != hipSuccess) return CSA_EHIP;
  }
  return launched(csa::launch_attend(1, q, Ccomp, ne * c, nullptr, kv_raw, n * c, 0, sink, b, n, 0,
                                     ne, n_h, c, 0, m_prime, n_win, scale, dtype, workspace, out, st));
}

// ---------------------------------------------------------------------------
// Heterogeneous decode cache (paged)
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

struct PagedGeom {
  int64_t L, e1, e2;        // tokens per block, CSA entries and HCA entries per block
  int64_t blk_elems;        // bf16 elements per block
  int l1, l2;               // log2 of e1, e2
};

int ilog2_exact(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return (int64_t(1) << l) == x ? l : -1;
}

int64_t gcd64(int64_t a, int64_t b) {
  while (b) { const int64_t t = a % b; a = b; b = t; }
  return a;
}

// Geometry of the block layout [e1][c] CSA entries, [e1][c_I] keys, [e2][c]
// HCA entries; CSA_ENOTSUP unless e1 and e2 are powers of two, e1 a
// multiple of 32 (a key tile never spans two blocks) and every array starts
// on a whole c-element row.
int paged_geom(int64_t c, int64_t cI, int64_t m, int64_t mp, PagedGeom* g) {
  if (c < 8 || cI < 8 || m < 1 || mp < 1 || c % 8 || cI % 8) return CSA_EINVAL;
  if (m > (int64_t(1) << 20) || mp > (int64_t(1) << 20)) return CSA_ENOTSUP;
  g->L = m / gcd64(m, mp) * mp;
  g->e1 = g->L / m;
  g->e2 = g->L / mp;
  g->l1 = ilog2_exact(g->e1);
  g->l2 = ilog2_exact(g->e2);
  if (g->l1 < 5 || g->l2 < 0) return CSA_ENOTSUP;
  if ((g->e1 * cI) % c != 0) return CSA_ENOTSUP;
  g->blk_elems = g->e1 * (c + cI) + g->e2 * c;
  return CSA_OK;
}

csa::Rows paged_rows(const int32_t* table, int64_t bt_stride, const int32_t* slot, const PagedGeom& g,
                     int64_t n_blocks, int64_t off, int lg) {
  return csa::Rows{0, table, slot, bt_stride, g.blk_elems, off, n_blocks, lg};
}

int check_paged_common(const void* blocks, int64_t n_blocks, const int32_t* table, int64_t bt_stride,
                       const int64_t* pos, int64_t b, int dtype) {
  if (dtype != CSA_BF16) return CSA_ENOTSUP;
  if (!blocks || !table || !pos || b < 1 || n_blocks < 1 || bt_stride < 1) return CSA_EINVAL;
  if (!aligned(blocks, 16) || !aligned(table, 4) || !aligned(pos, 8)) return CSA_EINVAL;
  if (b > 2147483647LL || n_blocks > 2147483647LL) return CSA_ENOTSUP;
  return CSA_OK;
}

}  // namespace

extern "C" {

size_t csa_paged_block_bytes(int64_t c, int64_t c_I, int64_t m, int64_t m_prime) {
  PagedGeom g;
  if (paged_geom(c, c_I, m, m_prime, &g) != CSA_OK) return 0;
  return (size_t)g.blk_elems * 2;
}

size_t csa_paged_state_bytes(int64_t c, int64_t c_I, int64_t m, int64_t m_prime, int64_t n_win) {
  if (c < 8 || c_I < 8 || m < 1 || m_prime < 1 || n_win < 1 || c % 8 || c_I % 8) return 0;
  return (size_t)csa::paged_state_layout(c, c_I, m, m_prime, n_win).stride * 2;
}

int csa_paged_append(void* state, void* blocks, int64_t n_blocks, const int32_t* block_table, int64_t bt_stride,
                     const int32_t* req_slot, const int64_t* pos, int64_t b, const void* Ca, const void* Cb,
                     const void* Za, const void* Zb, const void* ICa, const void* ICb, const void* IZa,
                     const void* IZb, const void* C_h, const void* Z_h, const void* Ba, const void* Bb,
                     const void* IBa, const void* IBb, const void* B_h, int64_t c, int64_t c_I, int64_t m,
                     int64_t m_prime, int64_t n_win, int dtype, void* stream) {
  int rc = check_paged_common(blocks, n_blocks, block_table, bt_stride, pos, b, dtype);
  if (rc != CSA_OK) return rc;
  PagedGeom g;
  rc = paged_geom(c, c_I, m, m_prime, &g);
  if (rc != CSA_OK) return rc;
  if (!state || n_win < 1 || !aligned(state, 16) || !aligned(req_slot, 4)) return CSA_EINVAL;
  const void* tok[10] = {Ca, Cb, Za, Zb, ICa, ICb, IZa, IZb, C_h, Z_h};
  const void* bias[5] = {Ba, Bb, IBa, IBb, B_h};
  for (const void* p : tok)
    if (!p || !aligned(p, 16)) return CSA_EINVAL;
  for (const void* p : bias)
    if (!p || !aligned(p, 16)) return CSA_EINVAL;
  if (c > 2048 || c_I > 2048 || n_win > (int64_t(1) << 20)) return CSA_ENOTSUP;
  const csa::PagedState L = csa::paged_state_layout(c, c_I, m, m_prime, n_win);
  const csa::Rows er = paged_rows(block_table, bt_stride, req_slot, g, n_blocks, 0, g.l1);
  const csa::Rows kr = paged_rows(block_table, bt_stride, req_slot, g, n_blocks, g.e1 * c, g.l1);
  const csa::Rows hr = paged_rows(block_table, bt_stride, req_slot, g, n_blocks, g.e1 * (c + c_I), g.l2);
  return launched(csa::launch_paged_append(state, L, blocks, er, kr, hr, pos, b, tok, bias, (hipStream_t)stream));
}

int csa_paged_index_topk(const void* qI, const float* w, const void* blocks, int64_t n_blocks,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* req_slot, const int64_t* pos,
                         int64_t b, int64_t n_comp_max, int64_t n_hI, int64_t c_I, int64_t c, int64_t m,
                         int64_t m_prime, int64_t k, int dtype, int32_t* idx, float* score, void* workspace,
                         size_t ws_bytes, void* stream) {
  int rc = check_paged_common(blocks, n_blocks, block_table, bt_stride, pos, b, dtype);
  if (rc != CSA_OK) return rc;
  PagedGeom g;
  rc = paged_geom(c, c_I, m, m_prime, &g);
  if (rc != CSA_OK) return rc;
  if (!qI || !w || !idx || !workspace || n_comp_max < 0 || n_hI < 1 || k < 1) return CSA_EINVAL;
  if (!aligned(qI, 16) || !aligned(w, 4) || !aligned(idx, 4) || !aligned(score, 4) || !aligned(req_slot, 4) ||
      !aligned(workspace, 256))
    return CSA_EINVAL;
  if (n_comp_max > bt_stride * g.e1) return CSA_EINVAL;   // more entries than the table's blocks hold
  if (!csa::index_topk_paged_supported(n_hI, c_I) || !csa::index_topk_supported(n_comp_max, k)) return CSA_ENOTSUP;
  if (b > 65535) return CSA_ENOTSUP;
  if (ws_bytes < csa::index_topk_workspace_bytes(b, 1, n_comp_max, k)) return CSA_ENOSPC;
  const csa::Rows kr = paged_rows(block_table, bt_stride, req_slot, g, n_blocks, g.e1 * c, g.l1);
  return launched(csa::launch_index_topk_paged(qI, w, blocks, kr, pos, b, n_comp_max, n_hI, c_I, m, k, idx, score,
                                               workspace, (hipStream_t)stream));
}

size_t csa_paged_attend_workspace_size(int64_t b, int64_t n_h, int64_t k, int64_t n_win) {
  if (b < 1 || n_h < 64 || n_h % 64 || k < 0 || n_win < 1) return 0;
  return csa::attend_paged_workspace_bytes(0, b, n_h, k + n_win);
}

size_t hca_paged_attend_workspace_size(int64_t b, int64_t n_h, int64_t n_hca_max, int64_t n_win) {
  if (b < 1 || n_h < 64 || n_h % 64 || n_hca_max < 0 || n_win < 1) return 0;
  return csa::attend_paged_workspace_bytes(1, b, n_h, n_hca_max + n_win);
}

}  // extern "C"

namespace {

int paged_attend_common(int dense, const void* q, const void* blocks, int64_t n_blocks, const int32_t* block_table,
                        int64_t bt_stride, const int32_t* req_slot, const int64_t* pos, const int32_t* idx,
                        const void* state, const float* sink, int64_t b, int64_t n_max, int64_t n_h, int64_t c,
                        int64_t c_I, int64_t k, int64_t m, int64_t m_prime, int64_t n_win, float scale, int dtype,
                        void* workspace, size_t ws_bytes, void* out, void* stream) {
  int rc = check_paged_common(blocks, n_blocks, block_table, bt_stride, pos, b, dtype);
  if (rc != CSA_OK) return rc;
  PagedGeom g;
  rc = paged_geom(c, c_I, m, m_prime, &g);
  if (rc != CSA_OK) return rc;
  if (!q || !state || !sink || !out || (!dense && !idx) || n_win < 1 || n_h < 1 || n_max < 0 || (!dense && k < 0))
    return CSA_EINVAL;
  if (!isfinite(scale) || !(scale > 0.f)) return CSA_EINVAL;
  if (!aligned(q, 16) || !aligned(state, 16) || !aligned(out, 16) || !aligned(sink, 4) || !aligned(idx, 4) ||
      !aligned(req_slot, 4))
    return CSA_EINVAL;
  if (n_max > bt_stride * (dense ? g.e2 : g.e1)) return CSA_EINVAL;
  // the MFMA path only: c = 512, 64-head groups, at most 2048 selected entries
  if (c != 512 || n_h % 64 != 0 || (!dense && k > 2048) || b > 65535 || n_h > 65535) return CSA_ENOTSUP;
  if (!csa::attend_paged_supported(dense, b, n_h, (dense ? n_max : k) + n_win)) return CSA_ENOTSUP;
  const size_t need = csa::attend_paged_workspace_bytes(dense, b, n_h, (dense ? n_max : k) + n_win);
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return CSA_EINVAL;
  if (ws_bytes < need) return CSA_ENOSPC;
  const csa::PagedState L = csa::paged_state_layout(c, c_I, m, m_prime, n_win);
  const csa::Rows er = dense ? paged_rows(block_table, bt_stride, req_slot, g, n_blocks, g.e1 * (c + c_I), g.l2)
                             : paged_rows(block_table, bt_stride, req_slot, g, n_blocks, 0, g.l1);
  const uint16_t* win = (const uint16_t*)state + (dense ? L.hca_win : L.csa_win);
  return launched(csa::launch_attend_paged(dense, q, blocks, er, idx, win, L.stride, n_win, pos, sink, b, n_max, n_h,
                                           k, dense ? m_prime : m, n_win, scale, workspace, out,
                                           (hipStream_t)stream));
}

}  // namespace

extern "C" {

int csa_paged_attend(const void* q, const void* blocks, int64_t n_blocks, const int32_t* block_table,
                     int64_t bt_stride, const int32_t* req_slot, const int64_t* pos, const int32_t* idx,
                     const void* state, const float* sink, int64_t b, int64_t n_comp_max, int64_t n_h, int64_t c,
                     int64_t c_I, int64_t k, int64_t m, int64_t m_prime, int64_t n_win, float scale, int dtype,
                     void* workspace, size_t ws_bytes, void* out, void* stream) {
  return paged_attend_common(0, q, blocks, n_blocks, block_table, bt_stride, req_slot, pos, idx, state, sink, b,
                             n_comp_max, n_h, c, c_I, k, m, m_prime, n_win, scale, dtype, workspace, ws_bytes, out,
                             stream);
}

int hca_paged_attend(const void* q, const void* blocks, int64_t n_blocks, const int32_t* block_table,
                     int64_t bt_stride, const int32_t* req_slot, const int64_t* pos, const void* state,
                     const float* sink, int64_t b, int64_t n_hca_max, int64_t n_h, int64_t c, int64_t c_I, int64_t m,
                     int64_t m_prime, int64_t n_win, float scale, int dtype, void* workspace, size_t ws_bytes,
                     void* out, void* stream) {
  return paged_attend_common(1, q, blocks, n_blocks, block_table, bt_stride, req_slot, pos, nullptr, state, sink, b,
                             n_hca_max, n_h, c, c_I, 0, m, m_prime, n_win, scale, dtype, workspace, ws_bytes, out,
                             stream);
}

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------
size_t csa_attend_backward_workspace_size(int64_t b, int64_t n_q, int64_t n_h, int64_t c, int64_t k, int64_t n_win) {
  if (b < 1 || n_q < 1 || n_h < 1 || c < 1 || k < 0 || n_win < 1) return 0;
  return csa::attend_backward_workspace_bytes(b, n_q, n_h, c, k, n_win);
}

size_t hca_attend_backward_workspace_size(int64_t b, int64_t n_q, int64_t n_h, int64_t c, int64_t n_comp,
                                          int64_t n_win) {
  if (b < 1 || n_q < 1 || n_h < 1 || c < 1 || n_comp < 0 || n_win < 1) return 0;
  return csa::attend_backward_workspace_bytes(b, n_q, n_h, c, n_comp, n_win);
}

}  // extern "C"

namespace {

int attend_backward_common(int dense, const void* q, const void* Ccomp, int64_t cbs, const int32_t* idx,
                           const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink, const void* dout,
                           int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c,
                           int64_t k, int64_t m, int64_t n_win, float scale, int dtype, int accumulate, float* dq,
                           float* dCcomp, int64_t dcbs, float* dkv_raw, int64_t drbs, float* dsink, void* workspace,
                           size_t ws_bytes, void* stream) {
  int rc = check_attend(q, Ccomp, cbs, kv_raw, rbs, raw_pos0, sink, b, n_q, t0, n_comp, n_raw, n_h, c, m, n_win, scale,
                        dtype, q);
  if (rc != CSA_OK) return rc;
  if (!dout || !dq || !dkv_raw || !dsink || (n_comp > 0 && !dCcomp) || (accumulate != 0 && accumulate != 1))
    return CSA_EINVAL;
  if (!dense && (k < 0 || (k > 0 && !idx))) return CSA_EINVAL;
  const int64_t es = elem_bytes(dtype);
  if (!aligned(dout, (uintptr_t)es) || !aligned(dq, 4) || !aligned(dCcomp, 4) || !aligned(dkv_raw, 4) ||
      !aligned(dsink, 4) || !aligned(idx, 4) || !aligned(workspace, 256))
    return CSA_EINVAL;
  if (dcbs < 0 || drbs < 0 || (dcbs > 0 && dcbs < n_comp * c) || (drbs > 0 && drbs < n_raw * c)) return CSA_EINVAL;
  if (c > 1024 || n_h > 512 || n_q > 65535 || b > 65535 || n_comp > 2147483647LL || n_raw > 2147483647LL)
    return CSA_ENOTSUP;
  const int64_t ks = dense ? n_comp : k;
  if (ks + n_win > 2147483647LL) return CSA_ENOTSUP;
  if (!workspace) return CSA_EINVAL;
  if (ws_bytes < csa::attend_backward_workspace_bytes(b, n_q, n_h, c, ks, n_win)) return CSA_ENOSPC;
  const int64_t cb = cbs > 0 ? cbs : n_comp * c;
  const int64_t rb = rbs > 0 ? rbs : n_raw * c;
  return launched(csa::launch_attend_backward(dense, q, Ccomp, cb, idx, kv_raw, rb, raw_pos0, sink, dout, b, n_q, t0,
                                              n_comp, n_raw, n_h, c, k, m, n_win, scale, dtype, accumulate, dq, dCcomp,
                                              dcbs > 0 ? dcbs : n_comp * c, dkv_raw, drbs > 0 ? drbs : n_raw * c,
                                              dsink, workspace, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int csa_attend_backward(const void* q, const void* Ccomp, int64_t comp_bstride, const int32_t* idx,
                        const void* kv_raw, int64_t raw_bstride, int64_t raw_pos0, const float* sink, const void* dout,
                        int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c,
                        int64_t k, int64_t m, int64_t n_win, float scale, int dtype, int accumulate, float* dq,
                        float* dCcomp, int64_t dcomp_bstride, float* dkv_raw, int64_t draw_bstride, float* dsink,
                        void* workspace, size_t ws_bytes, void* stream) {
  return attend_backward_common(0, q, Ccomp, comp_bstride, idx, kv_raw, raw_bstride, raw_pos0, sink, dout, b, n_q, t0,
                                n_comp, n_raw, n_h, c, k, m, n_win, scale, dtype, accumulate, dq, dCcomp,
                                dcomp_bstride, dkv_raw, draw_bstride, dsink, workspace, ws_bytes, stream);
}

int hca_attend_backward(const void* q, const void* Ccomp, int64_t comp_bstride, const void* kv_raw,
                        int64_t raw_bstride, int64_t raw_pos0, const float* sink, const void* dout, int64_t b,
                        int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c,
                        int64_t m_prime, int64_t n_win, float scale, int dtype, int accumulate, float* dq,
                        float* dCcomp, int64_t dcomp_bstride, float* dkv_raw, int64_t draw_bstride, float* dsink,
                        void* workspace, size_t ws_bytes, void* stream) {
  return attend_backward_common(1, q, Ccomp, comp_bstride, nullptr, kv_raw, raw_bstride, raw_pos0, sink, dout, b, n_q,
                                t0, n_comp, n_raw, n_h, c, 0, m_prime, n_win, scale, dtype, accumulate, dq, dCcomp,
                                dcomp_bstride, dkv_raw, draw_bstride, dsink, workspace, ws_bytes, stream);
}

size_t csa_compress_backward_workspace_size(int64_t n, int64_t c, int64_t m) {
  if (n < 1 || c < 1 || m < 1) return 0;
  return csa::compress_backward_workspace_bytes(n, c, m);
}

int csa_compress_backward(const void* Ca, const void* Cb, const void* Za, const void* Zb, const void* Ba,
                          const void* Bb, const void* prev_Cb, const void* prev_Zb, const float* dCcomp, int64_t b,
                          int64_t n, int64_t c, int64_t m, int overlap, int dtype, float* dCa, float* dCb, float* dZa,
                          float* dZb, float* dBa, float* dBb, float* dprev_Cb, float* dprev_Zb, void* workspace,
                          size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CSA_ENOTSUP;
  if (b < 1 || n < 1 || c < 1 || m < 1 || (overlap != 0 && overlap != 1)) return CSA_EINVAL;
  if (!Ca || !Za || !Ba || !dCa || !dZa || !dBa || !workspace || (n / m > 0 && !dCcomp)) return CSA_EINVAL;
  if (overlap) {
    if (!Cb || !Zb || !Bb || !dCb || !dZb || !dBb) return CSA_EINVAL;
    if ((prev_Cb == nullptr) != (prev_Zb == nullptr)) return CSA_EINVAL;
    // the previous block's gradients are needed for stream b's bias
    if (prev_Cb && (!dprev_Cb || !dprev_Zb)) return CSA_EINVAL;
  } else if (Cb || Zb || Bb || prev_Cb || prev_Zb) {
    return CSA_EINVAL;
  }
  const int64_t es = elem_bytes(dtype);
  const void* in[] = {Ca, Cb, Za, Zb, Ba, Bb, prev_Cb, prev_Zb};
  for (const void* p : in)
    if (!aligned(p, (uintptr_t)es)) return CSA_EINVAL;
  const void* outs[] = {dCcomp, dCa, dCb, dZa, dZb, dBa, dBb, dprev_Cb, dprev_Zb};
  for (const void* p : outs)
    if (!aligned(p, 4)) return CSA_EINVAL;
  if (!aligned(workspace, 256)) return CSA_EINVAL;
  if (b > 65535 || n > 2147483647LL || c > 65535) return CSA_ENOTSUP;
  if (ws_bytes < csa::compress_backward_workspace_bytes(n, c, m)) return CSA_ENOSPC;
  return launched(csa::launch_compress_backward(Ca, Cb, Za, Zb, Ba, Bb, prev_Cb, prev_Zb, dCcomp, b, n, c, m, overlap,
                                                dtype, dCa, dCb, dZa, dZb, dBa, dBb, dprev_Cb, dprev_Zb, workspace,
                                                (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// FP8 KV entries
// ---------------------------------------------------------------------------
int csa_quantize_kv_fp8(const void* x, int64_t x_rstride, int64_t rows, int64_t c, int64_t rope_dims, int dtype,
                        void* codes, int64_t codes_rstride, void* rope, int64_t rope_rstride, float* scale,
                        void* stream) {
  if (!dtype_ok(dtype)) return CSA_ENOTSUP;
  if (!x || !codes || !rope || !scale || rows < 1 || c < 16) return CSA_EINVAL;
  if (rope_dims < 8 || rope_dims % 8 || (c - rope_dims) < 8 || (c - rope_dims) % 8) return CSA_EINVAL;
  if (x_rstride < c || codes_rstride < c - rope_dims || rope_rstride < rope_dims) return CSA_EINVAL;
  const int64_t es = elem_bytes(dtype);
  if (!aligned(x, (uintptr_t)es) || !aligned(rope, 2) || !aligned(scale, 4)) return CSA_EINVAL;
  if (c > 65535 || rows > 2147483647LL * 4) return CSA_ENOTSUP;
  return launched(csa::launch_quantize_kv_fp8(x, x_rstride, rows, c, rope_dims, dtype, codes, codes_rstride, rope,
                                              rope_rstride, scale, (hipStream_t)stream));
}

size_t csa_attend_fp8kv_workspace_size(int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h, int64_t c,
                                       int64_t k, int64_t m, int64_t n_win) {
  if (b < 1 || n_q < 1 || t0 < 0 || n_comp < 0 || n_h < 1 || c < 1 || k < 0 || m < 1 || n_win < 1) return 0;
  return csa::attend_fp8kv_workspace_bytes(b, n_q, t0, n_comp, n_h, c, k, m, n_win);
}

int csa_attend_fp8kv(const void* q, const void* codes, const void* rope, const float* scale, int64_t comp_bstride,
                     const int32_t* idx, const void* kv_raw, int64_t raw_bstride, int64_t raw_pos0, const float* sink,
                     int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_raw, int64_t n_h, int64_t c,
                     int64_t rope_dims, int64_t k, int64_t m, int64_t n_win, float sm_scale, void* workspace,
                     size_t ws_bytes, void* out, void* stream) {
  int rc = check_attend(q, codes, 0, kv_raw, raw_bstride, raw_pos0, sink, b, n_q, t0, n_comp, n_raw, n_h, c, m,
                        n_win, sm_scale, CSA_BF16, out);
  if (rc != CSA_OK) return rc;
  if (n_comp > 0 && (!rope || !scale)) return CSA_EINVAL;
  if (k < 0 || (k > 0 && !idx)) return CSA_EINVAL;
  if (rope_dims < 8 || rope_dims % 8 || c - rope_dims < 8 || (c - rope_dims) % 8) return CSA_EINVAL;
  if (comp_bstride < 0 || (comp_bstride > 0 && comp_bstride < n_comp)) return CSA_EINVAL;
  if (!aligned(codes, 8) || !aligned(rope, 16) || !aligned(scale, 4) || !aligned(idx, 4)) return CSA_EINVAL;
  if (n_q > 2147483647LL || b > 65535 || n_h > 65535 || k > 2048) return CSA_ENOTSUP;
  if (!csa::attend_supported(CSA_BF16, n_h, c, k)) return CSA_ENOTSUP;
  const size_t need = csa::attend_fp8kv_workspace_bytes(b, n_q, t0, n_comp, n_h, c, k, m, n_win);
  if (!workspace || !aligned(workspace, 256)) return CSA_EINVAL;
  if (ws_bytes < need) return CSA_ENOSPC;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp;
  const int64_t rbs = raw_bstride > 0 ? raw_bstride : n_raw * c;
  return launched(csa::launch_attend_fp8kv(q, codes, rope, scale, cbs, idx, kv_raw, rbs, raw_pos0, sink, b, n_q, t0,
                                           n_comp, n_h, c, rope_dims, k, m, n_win, sm_scale, workspace, out,
                                           (hipStream_t)stream));
}

}  // extern "C"
