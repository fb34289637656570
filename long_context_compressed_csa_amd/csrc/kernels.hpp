// Host-side launchers of the CSA/HCA kernels.  Arguments are validated by
// the C ABI before any of these is called; each only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace csa {

hipError_t launch_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb,
                           const void* Ba, const void* Bb, const void* pCb, const void* pZb,
                           int64_t b, int64_t n, int64_t c, int64_t m, int overlap, int dtype,
                           void* out, int64_t obs, hipStream_t st);

size_t index_topk_workspace_bytes(int64_t b, int64_t n_q, int64_t n_comp, int64_t k);
bool index_topk_supported(int64_t n_comp, int64_t k);
bool index_topk_mx_supported(int64_t n_q, int64_t nh, int64_t cI);
hipError_t launch_quantize_mxfp4(const void* x, int64_t xrs, int64_t rows, int64_t c, int dtype, void* codes,
                                 int64_t crs, void* scales, int64_t srs, hipStream_t st);
hipError_t launch_index_topk_mx(const void* qI, const void* qS, const float* w, const void* KI, const void* KS,
                                int64_t cbs, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t nh,
                                int64_t cI, int64_t m, int64_t k, int32_t* idx, float* score, void* ws,
                                hipStream_t st);
hipError_t launch_index_topk(const void* qI, const float* w, const void* KI, int64_t cbs, int64_t b,
                             int64_t n_q, int64_t t0, int64_t n_comp, int64_t nh, int64_t cI,
                             int64_t m, int64_t k, int dtype, int32_t* idx, float* score,
                             void* ws, hipStream_t st);

size_t attend_workspace_bytes(int dtype, int64_t b, int64_t n_q, int64_t n_h, int64_t c,
                              int64_t nmax);
bool attend_supported(int dtype, int64_t n_h, int64_t c, int64_t k);
hipError_t launch_attend(int dense, const void* q, const void* Ccomp, int64_t cbs, const int32_t* idx,
                         const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink,
                         int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h,
                         int64_t c, int64_t k, int64_t m, int64_t n_win, float scale, int dtype,
                         void* ws, void* out, hipStream_t st);

hipError_t launch_norm_rope(const void* x, int64_t xrs, void* out, int64_t ors, const float* gamma, float eps,
                            int64_t rows, int64_t heads, int64_t c, int64_t rope_dims, double base, int64_t pos0,
                            int64_t pos_step, int dtype, hipStream_t st);

hipError_t launch_grouped_out_proj(const void* o, const void* WG, const void* WO, int64_t n, int64_t n_h, int64_t c,
                                   int64_t g, int64_t d_g, int64_t d, void* mid, void* out, hipStream_t st);

}  // namespace csa
