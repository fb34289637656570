// C ABI of the CSA/HCA library: host-side argument validation, then kernel
// launches on the caller's stream.  Nothing here allocates device memory or
// synchronises.  The operations are defined in include/csa.h.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "csa.h"
#include "kernels.hpp"

namespace {

inline bool dtype_ok(int dt) { return dt == CSA_F32 || dt == CSA_BF16; }
inline int launched(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_EHIP; }

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
    default: return "unknown error";
  }
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
  if (b > 65535) return CSA_ENOTSUP;
  const int64_t obs = out_bstride > 0 ? out_bstride : ne * c;
  return launched(csa::launch_compress(Ca, Cb, Za, Zb, Ba, Bb, prev_Cb, prev_Zb, b, n, c, m,
                                       overlap, dtype, Ccomp, obs, (hipStream_t)stream));
}

size_t csa_index_topk_workspace_size(int64_t b, int64_t n_q, int64_t n_comp, int64_t k) {
  if (b < 1 || n_q < 1 || n_comp < 0 || k < 1) return 0;
  return csa::index_topk_workspace_bytes(b, n_q, n_comp, k);
}

int csa_index_topk(const void* qI, const float* w, const void* KIcomp, int64_t comp_bstride,
                   int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_hI, int64_t c_I,
                   int64_t m, int64_t k, int dtype, int32_t* idx, float* score, void* workspace,
                   size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) && dtype != CSA_FP8) return CSA_ENOTSUP;
  if (!qI || !w || !idx || !workspace) return CSA_EINVAL;
  if (n_comp > 0 && !KIcomp) return CSA_EINVAL;
  if (b < 1 || n_q < 1 || n_hI < 1 || c_I < 1 || m < 1 || k < 1 || t0 < 0 || n_comp < 0)
    return CSA_EINVAL;
  if (n_comp > visible(t0 + n_q - 1, m)) return CSA_EINVAL;
  if (comp_bstride < 0 || (comp_bstride > 0 && comp_bstride < n_comp * c_I)) return CSA_EINVAL;
  if (n_q > 65535 || b > 65535) return CSA_ENOTSUP;
  if (!csa::index_topk_supported(n_comp, k)) return CSA_ENOTSUP;
  if (((uintptr_t)workspace & 255u) != 0) return CSA_EINVAL;
  if (ws_bytes < csa::index_topk_workspace_bytes(b, n_q, n_comp, k)) return CSA_ENOSPC;
  const int64_t cbs = comp_bstride > 0 ? comp_bstride : n_comp * c_I;
  return launched(csa::launch_index_topk(qI, w, KIcomp, cbs, b, n_q, t0, n_comp, n_hI, c_I, m, k,
                                         dtype, idx, score, workspace, (hipStream_t)stream));
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
  return launched(csa::launch_attend(0, q, Ccomp, cbs, idx, kv_raw, rbs, raw_pos0, sink, b, n_q, t0,
                                     n_comp, n_h, c, k, m, n_win, scale, dtype, workspace, out,
                                     (hipStream_t)stream));
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
  return launched(csa::launch_attend(1, q, Ccomp, cbs, nullptr, kv_raw, rbs, raw_pos0, sink, b, n_q,
                                     t0, n_comp, n_h, c, 0, m_prime, n_win, scale, dtype, workspace,
                                     out, (hipStream_t)stream));
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

}  // extern "C"
