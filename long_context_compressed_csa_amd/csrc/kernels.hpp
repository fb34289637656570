// Host-side launchers of the CSA/HCA kernels.  Arguments are validated by
// the C ABI before any of these is called; each only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "common.hpp"

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
hipError_t launch_attend_norm_rope(int dense, const void* q, const float* gq, float eps, int64_t rope_dims,
                                   double base, const void* Ccomp, int64_t cbs, const int32_t* idx,
                                   const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink, int64_t b,
                                   int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h, int64_t k, int64_t m,
                                   int64_t n_win, float scale, void* ws, void* out, hipStream_t st);
#if CSA_DEBUG
bool debug_take_oob(hipStream_t st);
hipError_t debug_set_entry_limit(int64_t limit);
#endif
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

// ---- heterogeneous decode cache (paged) ----
// Per-request state cache layout (bf16 elements from the request's start).
struct PagedState {
  int64_t stride;                                  // elements per request (a multiple of 128)
  int64_t csa_win, csa_open, csa_prev;             // [n_win][c], [4][m][c] (C^a, C^b, Z^a, Z^b), [2][m][c] (C^b, Z^b)
  int64_t key_open, key_prev;                      // [4][m][c_I], [2][m][c_I]
  int64_t hca_win, hca_open;                       // [n_win][c], [2][m'][c] (C, Z)
  int c, c_I, m, m_prime, n_win;
};
inline PagedState paged_state_layout(int64_t c, int64_t cI, int64_t m, int64_t mp, int64_t n_win) {
  PagedState L{};
  int64_t off = 0;
  L.csa_win = off; off += n_win * c;
  L.csa_open = off; off += 4 * m * c;
  L.csa_prev = off; off += 2 * m * c;
  L.key_open = off; off += 4 * m * cI;
  L.key_prev = off; off += 2 * m * cI;
  L.hca_win = off; off += n_win * c;
  L.hca_open = off; off += 2 * mp * c;
  L.stride = (off + 127) / 128 * 128;
  L.c = (int)c; L.c_I = (int)cI; L.m = (int)m; L.m_prime = (int)mp; L.n_win = (int)n_win;
  return L;
}
hipError_t launch_paged_append(void* state, const PagedState& L, void* pool, const Rows& csa_rows,
                               const Rows& key_rows, const Rows& hca_rows, const int64_t* pos, int64_t b,
                               const void* const* tok, const void* const* bias, hipStream_t st);
bool index_topk_paged_supported(int64_t nh, int64_t cI);
hipError_t launch_index_topk_paged(const void* qI, const float* w, const void* pool, const Rows& kr,
                                   const int64_t* pos, int64_t b, int64_t n_comp_max, int64_t nh, int64_t cI,
                                   int64_t m, int64_t k, int32_t* idx, float* score, void* ws, hipStream_t st);
// whether the split combine can take a paged list of nmax entries (its
// split weights fill at most 64 KiB of LDS)
bool attend_paged_supported(int dense, int64_t b, int64_t n_h, int64_t nmax);
size_t attend_paged_workspace_bytes(int dense, int64_t b, int64_t n_h, int64_t nmax);
hipError_t launch_attend_paged(int dense, const void* q, const void* pool, const Rows& er, const int32_t* idx,
                               const void* state, int64_t state_elems, int64_t ring, const int64_t* pos,
                               const float* sink, int64_t b, int64_t n_comp_max, int64_t n_h, int64_t k, int64_t m,
                               int64_t n_win, float scale, void* ws, void* out, hipStream_t st);

// ---- FP8 KV entries ----
hipError_t launch_quantize_kv_fp8(const void* x, int64_t xrs, int64_t rows, int64_t c, int64_t r, int dtype,
                                  void* codes, int64_t crs, void* rope, int64_t rrs, float* scale, hipStream_t st);
size_t attend_fp8kv_workspace_bytes(int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h, int64_t c,
                                    int64_t k, int64_t m, int64_t n_win);
hipError_t launch_attend_fp8kv(const void* q, const void* codes, const void* rope, const float* scale, int64_t cbs,
                               const int32_t* idx, const void* kv_raw, int64_t rbs, int64_t raw_pos0,
                               const float* sink, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h,
                               int64_t c, int64_t r, int64_t k, int64_t m, int64_t n_win, float sc, void* ws,
                               void* out, hipStream_t st);

// ---- backward pass ----
bool attend_bwd_mfma_ok(int dtype, int64_t n_h, int64_t c, int64_t k);
hipError_t launch_attend_bwd_mfma(int dense, const void* q, const void* Ccomp, int64_t cbs, const int32_t* idx,
                                  const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink,
                                  const void* dout, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h,
                                  int64_t k, int64_t m, int64_t n_win, int64_t ks, int64_t nslot, float scale,
                                  float* P, float* DL, float* dq, float* dz, hipStream_t st);
bool attend_bwd_contrib_mfma_ok(int dtype, int64_t n_h, int64_t c);
hipError_t launch_attend_bwd_contrib_mfma(const void* q, const void* dout, const float* P, const float* DL, int64_t b,
                                          int64_t n_q, int64_t nslot, float scale, float* contrib, hipStream_t st);
size_t attend_backward_workspace_bytes(int64_t b, int64_t n_q, int64_t n_h, int64_t c, int64_t ks, int64_t n_win);
hipError_t launch_attend_backward(int dense, const void* q, const void* Ccomp, int64_t cbs, const int32_t* idx,
                                  const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink,
                                  const void* dout, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp,
                                  int64_t n_raw, int64_t n_h, int64_t c, int64_t k, int64_t m, int64_t n_win,
                                  float scale, int dtype, int accumulate, float* dq, float* dC, int64_t dcbs,
                                  float* dR, int64_t drbs, float* dsink, void* ws, hipStream_t st);
size_t compress_backward_workspace_bytes(int64_t n, int64_t c, int64_t m);
hipError_t launch_compress_backward(const void* Ca, const void* Cb, const void* Za, const void* Zb, const void* Ba,
                                    const void* Bb, const void* pCb, const void* pZb, const float* dCc, int64_t b,
                                    int64_t n, int64_t c, int64_t m, int overlap, int dtype, float* dCa, float* dCb,
                                    float* dZa, float* dZb, float* dBa, float* dBb, float* dpCb, float* dpZb,
                                    void* ws, hipStream_t st);

}  // namespace csa
