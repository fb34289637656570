// Backward pass of the CSA / HCA attention and of both compressors, with
// deterministic reductions (AirCoding "deepseek-paper-analysis" section 7.6:
// the attention backward accumulates into buffers of its own and sums them
// in a fixed order, instead of floating-point atomics).
//
// Attention (one query t, head h; entries e_j = selected compressed rows,
// then the window rows; logits l_j = scale q.e_j; sink logit z; weights p_j
// and p_z of one softmax; o = sum_j p_j e_j; g = dL/do):
//   dl_j = p_j (g.e_j - g.o)     dz = -p_z g.o     dq = scale sum_j dl_j e_j
//   de_j = p_j g + scale dl_j q, summed over the heads and the queries that
//   read entry j (each entry is both key and value).
// Steps, each with a fixed summation order:
//   attend_bwd_query    per (t, h): softmax statistics, p_j and dl_j of
//                       every entry slot, dq, dz
//   attend_bwd_contrib  per (t, slot): sum over heads of p g + scale dl q
//   attend_bwd_reduce_* per compressed entry / raw row / head: the sum of
//                       its contributions over the queries, in query order
// Compressors (entry i = sum_j S_j C_j over its rows, S the per-dimension
// softmax of Z + B; g = dL/dC^Comp_i):
//   dC_j = S_j g,  dZ_j = S_j (C_j - C^Comp_i) g,
//   dB (per in-block row) = sum over entries and sequences of dZ, in order.
//
// Gradients are float32 whatever the storage type of the inputs.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int kBwdT = 256;       // threads per workgroup
constexpr int kBwdMaxC = 1024;   // largest row length

// Entry slots of query t: [0, ks) compressed (CSA: idx positions; HCA:
// entry numbers), then [ks, ks + n_win) window rows wlo(t) + (slot - ks).
struct BwdGeom {
  int64_t n_q, t0, n_comp, k, m, n_win, ks, nslot;
  int n_h, c, dense;
  float scale;
  __device__ __forceinline__ int64_t t_of(int64_t r) const { return t0 + r; }
  __device__ __forceinline__ int64_t vis(int64_t t) const {
    const int64_t v = (t + 1) / m;
    return v < n_comp ? v : n_comp;
  }
  __device__ __forceinline__ int64_t wlo(int64_t t) const { return t - n_win + 1 > 0 ? t - n_win + 1 : 0; }
};

template <typename T>
__device__ __forceinline__ const T* bwd_entry_row(const BwdGeom& G, int64_t bi, int64_t r, int64_t j,
                                                  const T* Ccomp, int64_t cbs, const int32_t* idx,
                                                  const T* kv_raw, int64_t rbs, int64_t raw_pos0) {
  const int64_t t = G.t_of(r);
  if (j < G.ks) {
    int64_t s;
    if (G.dense) {
      s = j;
    } else {
      s = idx[(bi * G.n_q + r) * G.k + j];
    }
    if (s < 0 || s >= G.vis(t)) return nullptr;
    return Ccomp + bi * cbs + s * (int64_t)G.c;
  }
  const int64_t p = G.wlo(t) + (j - G.ks);
  if (p > t) return nullptr;
  return kv_raw + bi * rbs + (p - raw_pos0) * (int64_t)G.c;
}

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  v = wave_max(v);
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  v = wave_sum(v);
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// One workgroup per (query, head).  P and DL [b][n_q][n_h][nslot] receive
// p_j and dl_j (0 at unused slots); dq [b][n_q][n_h][c]; dz [b][n_q][n_h].
template <typename T>
__global__ __launch_bounds__(kBwdT) void attend_bwd_query(
    BwdGeom G, const T* __restrict__ q, const T* __restrict__ Ccomp, int64_t cbs, const int32_t* __restrict__ idx,
    const T* __restrict__ kv_raw, int64_t rbs, int64_t raw_pos0, const float* __restrict__ sink,
    const T* __restrict__ dout, float* __restrict__ P, float* __restrict__ DL, float* __restrict__ dq,
    float* __restrict__ dz) {
  __shared__ float qs[kBwdMaxC], gs[kBwdMaxC];
  __shared__ float pl[kBwdT];
  __shared__ const T* rows[kBwdT];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x, bi = blockIdx.z;
  const int h = blockIdx.y;
  const int c = G.c;
  const int64_t qoff = ((bi * G.n_q + r) * G.n_h + h) * (int64_t)c;
  for (int d = tid; d < c; d += kBwdT) {
    qs[d] = Elem<T>::ld(q + qoff + d);
    gs[d] = Elem<T>::ld(dout + qoff + d);
  }
  const int64_t prow = ((bi * G.n_q + r) * G.n_h + h) * G.nslot;
  float* Pr = P + prow;
  float* DLr = DL + prow;
  __syncthreads();
  // pass 1: logits and g.e of every slot (kept in P / DL), running maximum,
  // denominator and sum of weights times g.e; the sink (value 0) starts them
  const float z = sink[h];
  float M = z, D = 1.f, A = 0.f;
  for (int64_t j0 = 0; j0 < G.nslot; j0 += kBwdT) {
    const int64_t j = j0 + tid;
    float lg = -INFINITY, ge = 0.f;
    if (j < G.nslot) {
      const T* row = bwd_entry_row<T>(G, bi, r, j, Ccomp, cbs, idx, kv_raw, rbs, raw_pos0);
      if (row) {
        float a = 0.f, b2 = 0.f;
        for (int x = 0; x < c; ++x) {
          const float e = Elem<T>::ld(row + x);
          a = fmaf(qs[x], e, a);
          b2 = fmaf(gs[x], e, b2);
        }
        lg = G.scale * a;
        ge = b2;
      }
      Pr[j] = lg;
      DLr[j] = ge;
    }
    const float cm = block_reduce_max(lg, red);
    const float nm = fmaxf(M, cm);
    const float w = lg == -INFINITY ? 0.f : __expf(lg - nm);
    const float sw = block_reduce_sum(w, red);
    const float swg = block_reduce_sum(w * ge, red);
    const float al = __expf(M - nm);
    D = D * al + sw;
    A = A * al + swg;
    M = nm;
  }
  const float go = A / D;   // g . o
  if (tid == 0) dz[(bi * G.n_q + r) * G.n_h + h] = -(__expf(z - M) / D) * go;
  // pass 2: weights and logit gradients of every slot, then dq
  float acc[kBwdMaxC / kBwdT] = {};
  for (int64_t j0 = 0; j0 < G.nslot; j0 += kBwdT) {
    const int64_t j = j0 + tid;
    float p = 0.f, dl = 0.f;
    const T* row = nullptr;
    if (j < G.nslot) {
      const float lg = Pr[j];
      if (lg != -INFINITY) {
        p = __expf(lg - M) / D;
        dl = p * (DLr[j] - go);
        row = bwd_entry_row<T>(G, bi, r, j, Ccomp, cbs, idx, kv_raw, rbs, raw_pos0);
      }
      Pr[j] = p;
      DLr[j] = dl;
    }
    __syncthreads();
    pl[tid] = dl;
    rows[tid] = row;
    __syncthreads();
    const int cnt = (int)(G.nslot - j0 < kBwdT ? G.nslot - j0 : kBwdT);
    for (int jj = 0; jj < cnt; ++jj) {
      const float d2 = pl[jj];
      const T* rj = rows[jj];
      if (rj == nullptr || d2 == 0.f) continue;
#pragma unroll
      for (int i = 0; i < kBwdMaxC / kBwdT; ++i) {
        const int d = tid + kBwdT * i;
        if (d < c) acc[i] = fmaf(d2, Elem<T>::ld(rj + d), acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kBwdMaxC / kBwdT; ++i) {
    const int d = tid + kBwdT * i;
    if (d < c) dq[qoff + d] = G.scale * acc[i];
  }
}

// contrib[b][n_q][nslot][c] = sum over heads h (in order) of
//   P[h][slot] g_h + scale DL[h][slot] q_h, for 16 slots per workgroup.
constexpr int kSlotsPerWG = 16;
// P and DL are [b][n_q][n_h][nslot] (slot_major = 0, the vector path's
// layout) or [b][n_q][nslot][n_h] (slot_major = 1, the MFMA path's).
template <typename T>
__global__ __launch_bounds__(kBwdT) void attend_bwd_contrib(BwdGeom G, const T* __restrict__ q,
                                                            const T* __restrict__ dout, const float* __restrict__ P,
                                                            const float* __restrict__ DL, int slot_major,
                                                            float* __restrict__ contrib) {
  extern __shared__ float pd[];   // [n_h][2][kSlotsPerWG]
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x, bi = blockIdx.z;
  const int64_t s0 = (int64_t)blockIdx.y * kSlotsPerWG;
  const int c = G.c, nh = G.n_h;
  const int ns = (int)(G.nslot - s0 < kSlotsPerWG ? G.nslot - s0 : kSlotsPerWG);
  const int64_t prow0 = (bi * G.n_q + r) * nh;
  for (int e = tid; e < nh * kSlotsPerWG; e += kBwdT) {
    const int h = e / kSlotsPerWG, s = e % kSlotsPerWG;
    const bool ok = s < ns;
    const int64_t at = slot_major ? ((bi * G.n_q + r) * G.nslot + s0 + s) * nh + h : (prow0 + h) * G.nslot + s0 + s;
    pd[(h * 2 + 0) * kSlotsPerWG + s] = ok ? P[at] : 0.f;
    pd[(h * 2 + 1) * kSlotsPerWG + s] = ok ? G.scale * DL[at] : 0.f;
  }
  __syncthreads();
  for (int d0 = 0; d0 < c; d0 += kBwdT) {
    const int d = d0 + tid;
    float acc[kSlotsPerWG] = {};
    if (d < c) {
      for (int h = 0; h < nh; ++h) {
        const int64_t off = (prow0 + h) * (int64_t)c + d;
        const float gv = Elem<T>::ld(dout + off);
        const float qv = Elem<T>::ld(q + off);
#pragma unroll
        for (int s = 0; s < kSlotsPerWG; ++s)
          acc[s] = fmaf(pd[(h * 2 + 0) * kSlotsPerWG + s], gv, fmaf(pd[(h * 2 + 1) * kSlotsPerWG + s], qv, acc[s]));
      }
      for (int s = 0; s < ns; ++s) contrib[((bi * G.n_q + r) * G.nslot + s0 + s) * (int64_t)c + d] = acc[s];
    }
  }
}

// Slot of compressed entry s in query t's list, or -1: CSA lists are the
// idx row, ascending among its valid entries (binary search); HCA lists are
// the entries themselves.
__device__ __forceinline__ int64_t bwd_slot_of(const BwdGeom& G, const int32_t* __restrict__ idx, int64_t bi,
                                               int64_t r, int64_t s) {
  const int64_t t = G.t_of(r);
  if (s >= G.vis(t)) return -1;
  if (G.dense) return s;
  const int32_t* row = idx + (bi * G.n_q + r) * G.k;
  int64_t lo = 0, hi = G.k;   // first position whose value is >= s, -1 read as past every entry
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    const int32_t v = row[mid];
    if (v >= 0 && v < s) lo = mid + 1; else hi = mid;
  }
  return (lo < G.k && row[lo] == s) ? lo : -1;
}

// Inverse slot table of a CSA backward call: inv[b][s][r] = the slot of
// entry s in query r's list (the lowest, should a row list it twice), or a
// value >= k where r does not read s.  Built by a fill and a scatter of
// every valid listed entry (atomicMin: the result does not depend on the
// order of the writes).
__global__ __launch_bounds__(kBwdT) void bwd_inv_fill(int32_t* __restrict__ inv, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * kBwdT + threadIdx.x; i < count; i += (int64_t)gridDim.x * kBwdT)
    inv[i] = 0x7fffffff;
}
__global__ __launch_bounds__(kBwdT) void bwd_inv_scatter(BwdGeom G, const int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ inv) {
  const int64_t r = blockIdx.x, bi = blockIdx.y;
  const int64_t vis = G.vis(G.t_of(r));
  const int32_t* row = idx + (bi * G.n_q + r) * G.k;
  for (int64_t j = threadIdx.x; j < G.k; j += kBwdT) {
    const int32_t s = row[j];
    if (s >= 0 && s < vis) atomicMin(&inv[(bi * G.n_comp + s) * G.n_q + r], (int32_t)j);
  }
}

// dCcomp[b][s] (+)= sum over the block's queries t (ascending) of
// contrib[t][slot(t, s)].  One workgroup per (entry, sequence); the queries
// are looked up 256 at a time (in the inverse table when there is one, else
// by a search of each query's list), the found ones compacted in query
// order and their contributions summed in that order.
__global__ __launch_bounds__(kBwdT) void attend_bwd_reduce_comp(BwdGeom G, const int32_t* __restrict__ idx,
                                                                const int32_t* __restrict__ inv,
                                                                const float* __restrict__ contrib, int accumulate,
                                                                float* __restrict__ dC, int64_t dcbs) {
  __shared__ int32_t fr[kBwdT], fj[kBwdT];
  __shared__ int32_t wcnt[kBwdT / 64];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int64_t s = blockIdx.x, bi = blockIdx.y;
  const int c = G.c;
  float acc[kBwdMaxC / kBwdT] = {};
  // the first query that can read entry s completes it: t = m (s + 1) - 1
  int64_t r_first = G.m * (s + 1) - 1 - G.t0;
  if (r_first < 0) r_first = 0;
  for (int64_t r0 = r_first; r0 < G.n_q; r0 += kBwdT) {
    const int64_t r = r0 + tid;
    int32_t j = -1;
    if (r < G.n_q) {
      if (inv) {
        const int32_t v = inv[(bi * G.n_comp + s) * G.n_q + r];
        j = v < G.k ? v : -1;
      } else {
        j = (int32_t)bwd_slot_of(G, idx, bi, r, s);
      }
    }
    const uint64_t mk = __builtin_amdgcn_ballot_w64(j >= 0);
    __syncthreads();   // the previous round's list has been read
    if (l == 0) wcnt[wave] = __popcll(mk);
    __syncthreads();
    int pos = __popcll(mk & ((l == 0) ? 0ull : (~0ull >> (64 - l))));
    int nf = 0;
#pragma unroll
    for (int w = 0; w < kBwdT / 64; ++w) {
      pos += w < wave ? wcnt[w] : 0;
      nf += wcnt[w];
    }
    if (j >= 0) {
      fr[pos] = (int32_t)(r - r0);
      fj[pos] = j;
    }
    __syncthreads();
    // eight rows' loads in flight at a time, added in list order
    constexpr int B8 = 8;
    for (int i0 = 0; i0 < nf; i0 += B8) {
      float v[B8][kBwdMaxC / kBwdT];
#pragma unroll
      for (int b8 = 0; b8 < B8; ++b8) {
        const int i = i0 + b8 < nf ? i0 + b8 : i0;
        const float* src = contrib + ((bi * G.n_q + r0 + fr[i]) * G.nslot + fj[i]) * (int64_t)c;
#pragma unroll
        for (int u = 0; u < kBwdMaxC / kBwdT; ++u) {
          const int d = tid + kBwdT * u;
          v[b8][u] = d < c ? src[d] : 0.f;
        }
      }
#pragma unroll
      for (int b8 = 0; b8 < B8; ++b8)
        if (i0 + b8 < nf)
#pragma unroll
          for (int u = 0; u < kBwdMaxC / kBwdT; ++u) acc[u] += v[b8][u];
    }
  }
#pragma unroll
  for (int u = 0; u < kBwdMaxC / kBwdT; ++u) {
    const int d = tid + kBwdT * u;
    if (d < c) {
      float* o = dC + bi * dcbs + s * (int64_t)c + d;
      *o = accumulate ? *o + acc[u] : acc[u];
    }
  }
}

// dkv_raw[b][i] (+)= sum over the queries t whose window holds position
// p = raw_pos0 + i (t = p .. p + n_win - 1), ascending.
__global__ __launch_bounds__(kBwdT) void attend_bwd_reduce_raw(BwdGeom G, int64_t raw_pos0,
                                                               const float* __restrict__ contrib, int accumulate,
                                                               float* __restrict__ dR, int64_t drbs) {
  const int tid = threadIdx.x;
  const int64_t i = blockIdx.x, bi = blockIdx.y;
  const int64_t p = raw_pos0 + i;
  const int c = G.c;
  float acc[kBwdMaxC / kBwdT] = {};
  // the queries t = p .. p + n_win - 1 inside this block, ascending, eight
  // rows' loads in flight at a time
  int64_t tlo = p, thi = p + G.n_win;   // [tlo, thi)
  if (tlo < G.t0) tlo = G.t0;
  if (thi > G.t0 + G.n_q) thi = G.t0 + G.n_q;
  constexpr int B8 = 8;
  for (int64_t t0 = tlo; t0 < thi; t0 += B8) {
    float v[B8][kBwdMaxC / kBwdT];
#pragma unroll
    for (int b8 = 0; b8 < B8; ++b8) {
      const int64_t t = t0 + b8 < thi ? t0 + b8 : t0;
      const int64_t j = G.ks + (p - G.wlo(t));
      const float* src = contrib + ((bi * G.n_q + (t - G.t0)) * G.nslot + j) * (int64_t)c;
#pragma unroll
      for (int u = 0; u < kBwdMaxC / kBwdT; ++u) {
        const int d = tid + kBwdT * u;
        v[b8][u] = d < c ? src[d] : 0.f;
      }
    }
#pragma unroll
    for (int b8 = 0; b8 < B8; ++b8)
      if (t0 + b8 < thi)
#pragma unroll
        for (int u = 0; u < kBwdMaxC / kBwdT; ++u) acc[u] += v[b8][u];
  }
#pragma unroll
  for (int u = 0; u < kBwdMaxC / kBwdT; ++u) {
    const int d = tid + kBwdT * u;
    if (d < c) {
      float* o = dR + bi * drbs + i * (int64_t)c + d;
      *o = accumulate ? *o + acc[u] : acc[u];
    }
  }
}

// dsink[h] (+)= sum over sequences and queries of dz, in a fixed order:
// thread i sums rows i, i + 256, ...; then a fixed tree.
__global__ __launch_bounds__(kBwdT) void attend_bwd_reduce_sink(int64_t rows, int n_h, const float* __restrict__ dz,
                                                                int accumulate, float* __restrict__ dsink) {
  __shared__ float red[4];
  const int h = blockIdx.x;
  float a = 0.f;
  for (int64_t r = threadIdx.x; r < rows; r += kBwdT) a += dz[r * n_h + h];
  a = block_reduce_sum(a, red);
  if (threadIdx.x == 0) dsink[h] = accumulate ? dsink[h] + a : a;
}

size_t attend_backward_workspace_bytes(int64_t b, int64_t n_q, int64_t n_h, int64_t c, int64_t ks, int64_t n_win) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nslot = (size_t)(ks + n_win);
  const size_t rows = (size_t)b * n_q;
  return 2 * al(rows * n_h * nslot * 4) + al(rows * n_h * 4) + al(rows * nslot * c * 4);
}

hipError_t launch_attend_backward(int dense, const void* q, const void* Ccomp, int64_t cbs, const int32_t* idx,
                                  const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink,
                                  const void* dout, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp,
                                  int64_t n_raw, int64_t n_h, int64_t c, int64_t k, int64_t m, int64_t n_win,
                                  float scale, int dtype, int accumulate, float* dq, float* dC, int64_t dcbs,
                                  float* dR, int64_t drbs, float* dsink, void* ws, hipStream_t st) {
  BwdGeom G{n_q, t0, n_comp, k, m, n_win, dense ? n_comp : k, 0, (int)n_h, (int)c, dense, scale};
  G.nslot = G.ks + n_win;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)b * n_q;
  unsigned char* W = (unsigned char*)ws;
  float* P = (float*)W;
  float* DL = (float*)(W + al(rows * n_h * G.nslot * 4));
  float* dz = (float*)(W + 2 * al(rows * n_h * G.nslot * 4));
  float* contrib = (float*)(W + 2 * al(rows * n_h * G.nslot * 4) + al(rows * n_h * 4));
  const dim3 qgrid((unsigned)n_q, (unsigned)n_h, (unsigned)b);
  const dim3 cgrid((unsigned)n_q, (unsigned)((G.nslot + kSlotsPerWG - 1) / kSlotsPerWG), (unsigned)b);
  const size_t csh = (size_t)n_h * 2 * kSlotsPerWG * 4;
  if (attend_bwd_mfma_ok(dtype, n_h, c, dense ? 0 : k)) {
    // bf16, c = 512, 64-head groups: the per-query step on MFMA
    const hipError_t e = launch_attend_bwd_mfma(dense, q, Ccomp, cbs, idx, kv_raw, rbs, raw_pos0, sink, dout, b, n_q,
                                                t0, n_comp, n_h, k, m, n_win, G.ks, G.nslot, scale, P, DL, dq, dz, st);
    if (e != hipSuccess) return e;
    if (attend_bwd_contrib_mfma_ok(dtype, n_h, c)) {
      const hipError_t e2 = launch_attend_bwd_contrib_mfma(q, dout, P, DL, b, n_q, G.nslot, scale, contrib, st);
      if (e2 != hipSuccess) return e2;
    } else {
      hipLaunchKernelGGL(attend_bwd_contrib<bf16_t>, cgrid, dim3(kBwdT), csh, st, G, (const bf16_t*)q,
                         (const bf16_t*)dout, P, DL, 1, contrib);
    }
  } else if (dtype == 1) {
    hipLaunchKernelGGL(attend_bwd_query<bf16_t>, qgrid, dim3(kBwdT), 0, st, G, (const bf16_t*)q, (const bf16_t*)Ccomp,
                       cbs, idx, (const bf16_t*)kv_raw, rbs, raw_pos0, sink, (const bf16_t*)dout, P, DL, dq, dz);
    hipLaunchKernelGGL(attend_bwd_contrib<bf16_t>, cgrid, dim3(kBwdT), csh, st, G, (const bf16_t*)q,
                       (const bf16_t*)dout, P, DL, 0, contrib);
  } else {
    hipLaunchKernelGGL(attend_bwd_query<float>, qgrid, dim3(kBwdT), 0, st, G, (const float*)q, (const float*)Ccomp,
                       cbs, idx, (const float*)kv_raw, rbs, raw_pos0, sink, (const float*)dout, P, DL, dq, dz);
    hipLaunchKernelGGL(attend_bwd_contrib<float>, cgrid, dim3(kBwdT), csh, st, G, (const float*)q,
                       (const float*)dout, P, DL, 0, contrib);
  }
  if (n_comp > 0) {
    // CSA: the inverse slot table, in the P and DL arrays (read only by the
    // contribution step, done by now) when it fits there
    int32_t* inv = nullptr;
    const size_t inv_n = (size_t)b * n_comp * n_q;
    if (!dense && inv_n * 4 <= 2 * al(rows * n_h * G.nslot * 4)) {
      inv = (int32_t*)P;
      const int64_t blocks = (int64_t)((inv_n + kBwdT - 1) / kBwdT);
      hipLaunchKernelGGL(bwd_inv_fill, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(kBwdT), 0, st, inv,
                         (int64_t)inv_n);
      hipLaunchKernelGGL(bwd_inv_scatter, dim3((unsigned)n_q, (unsigned)b), dim3(kBwdT), 0, st, G, idx, inv);
    }
    hipLaunchKernelGGL(attend_bwd_reduce_comp, dim3((unsigned)n_comp, (unsigned)b), dim3(kBwdT), 0, st, G, idx,
                       (const int32_t*)inv, contrib, accumulate, dC, dcbs);
  }
  hipLaunchKernelGGL(attend_bwd_reduce_raw, dim3((unsigned)n_raw, (unsigned)b), dim3(kBwdT), 0, st, G, raw_pos0,
                     contrib, accumulate, dR, drbs);
  hipLaunchKernelGGL(attend_bwd_reduce_sink, dim3((unsigned)n_h), dim3(kBwdT), 0, st, (int64_t)rows, (int)n_h, dz,
                     accumulate, dsink);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compressors
// ---------------------------------------------------------------------------
// One thread per (sequence, entry, dimension): recompute the entry's weights
// and value, write the gradients of its rows (each row of each stream feeds
// exactly one entry), and zero the rows no entry reads.
template <typename T>
__global__ __launch_bounds__(kBwdT) void compress_bwd_rows(
    const T* __restrict__ Ca, const T* __restrict__ Cb, const T* __restrict__ Za, const T* __restrict__ Zb,
    const T* __restrict__ Ba, const T* __restrict__ Bb, const T* __restrict__ pCb, const T* __restrict__ pZb,
    const float* __restrict__ dCc, int64_t b, int64_t n, int c, int m, int overlap, float* __restrict__ dCa,
    float* __restrict__ dCb, float* __restrict__ dZa, float* __restrict__ dZb, float* __restrict__ dpCb,
    float* __restrict__ dpZb) {
  const int64_t ne = n / m;
  const int64_t total = b * (ne + 1) * c;   // the extra "entry" zeroes rows no entry reads
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int d = (int)(u % c);
    const int64_t rest = u / c;
    const int64_t e = rest % (ne + 1);
    const int64_t s = rest / (ne + 1);
    const int64_t sq = s * n * (int64_t)c;
    if (e == ne) {
      // the ragged tail of every stream, and the last block's stream-b rows
      for (int64_t row = ne * m; row < n; ++row) {
        dCa[sq + row * c + d] = 0.f;
        dZa[sq + row * c + d] = 0.f;
        if (overlap) { dCb[sq + row * c + d] = 0.f; dZb[sq + row * c + d] = 0.f; }
      }
      if (overlap && ne > 0)
        for (int j = 0; j < m; ++j) {
          const int64_t row = (ne - 1) * m + j;
          dCb[sq + row * c + d] = 0.f;
          dZb[sq + row * c + d] = 0.f;
        }
      if (overlap && ne == 0 && dpCb)
        for (int j = 0; j < m; ++j) { dpCb[(s * m + j) * c + d] = 0.f; dpZb[(s * m + j) * c + d] = 0.f; }
      continue;
    }
    const bool hasb = overlap && (e > 0 || pZb != nullptr);
    // scores and values of the entry's rows (stream a of block e, stream b of block e - 1)
    float mx = -INFINITY;
    for (int j = 0; j < m; ++j) {
      mx = fmaxf(mx, Elem<T>::ld(Za + sq + (m * e + j) * c + d) + Elem<T>::ld(Ba + j * c + d));
      if (hasb) {
        const float zb = e > 0 ? Elem<T>::ld(Zb + sq + (m * (e - 1) + j) * c + d) : Elem<T>::ld(pZb + (s * m + j) * c + d);
        mx = fmaxf(mx, zb + Elem<T>::ld(Bb + j * c + d));
      }
    }
    float den = 0.f, num = 0.f;
    for (int j = 0; j < m; ++j) {
      const float pa = __expf(Elem<T>::ld(Za + sq + (m * e + j) * c + d) + Elem<T>::ld(Ba + j * c + d) - mx);
      den += pa;
      num = fmaf(pa, Elem<T>::ld(Ca + sq + (m * e + j) * c + d), num);
      if (hasb) {
        const int64_t rb = (m * (e - 1) + j);
        const float zb = e > 0 ? Elem<T>::ld(Zb + sq + rb * c + d) : Elem<T>::ld(pZb + (s * m + j) * c + d);
        const float cb = e > 0 ? Elem<T>::ld(Cb + sq + rb * c + d) : Elem<T>::ld(pCb + (s * m + j) * c + d);
        const float pb = __expf(zb + Elem<T>::ld(Bb + j * c + d) - mx);
        den += pb;
        num = fmaf(pb, cb, num);
      }
    }
    const float cc = num / den;
    const float g = dCc[(s * ne + e) * c + d];
    for (int j = 0; j < m; ++j) {
      const int64_t ra = m * e + j;
      const float sa = __expf(Elem<T>::ld(Za + sq + ra * c + d) + Elem<T>::ld(Ba + j * c + d) - mx) / den;
      dCa[sq + ra * c + d] = sa * g;
      dZa[sq + ra * c + d] = sa * (Elem<T>::ld(Ca + sq + ra * c + d) - cc) * g;
      if (hasb) {
        const int64_t rb = m * (e - 1) + j;
        const float zb = e > 0 ? Elem<T>::ld(Zb + sq + rb * c + d) : Elem<T>::ld(pZb + (s * m + j) * c + d);
        const float cb = e > 0 ? Elem<T>::ld(Cb + sq + rb * c + d) : Elem<T>::ld(pCb + (s * m + j) * c + d);
        const float sb = __expf(zb + Elem<T>::ld(Bb + j * c + d) - mx) / den;
        if (e > 0) {
          dCb[sq + rb * c + d] = sb * g;
          dZb[sq + rb * c + d] = sb * (cb - cc) * g;
        } else if (dpCb) {
          dpCb[(s * m + j) * c + d] = sb * g;
          dpZb[(s * m + j) * c + d] = sb * (cb - cc) * g;
        }
      } else if (overlap && e == 0 && dpCb) {
        dpCb[(s * m + j) * c + d] = 0.f;
        dpZb[(s * m + j) * c + d] = 0.f;
      }
    }
  }
}

// The same per (sequence, entry, group of Vec16<T>::N dimensions): 16-byte
// loads and stores (c a multiple of N, rows 16-byte aligned).
template <typename T>
__global__ __launch_bounds__(kBwdT) void compress_bwd_rows_v(
    const T* __restrict__ Ca, const T* __restrict__ Cb, const T* __restrict__ Za, const T* __restrict__ Zb,
    const T* __restrict__ Ba, const T* __restrict__ Bb, const T* __restrict__ pCb, const T* __restrict__ pZb,
    const float* __restrict__ dCc, int64_t b, int64_t n, int c, int m, int overlap, float* __restrict__ dCa,
    float* __restrict__ dCb, float* __restrict__ dZa, float* __restrict__ dZb, float* __restrict__ dpCb,
    float* __restrict__ dpZb) {
  constexpr int N = Vec16<T>::N;
  typedef Vec16<float> F;
  const int cv = c / N;
  const int64_t ne = n / m;
  const int64_t total = b * (ne + 1) * cv;
  auto st_f = [](float* p, const float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float w[4] = {v[i], v[i + 1], v[i + 2], v[i + 3]};
      F::st(p + i, w);
    }
  };
  auto st_zero = [](float* p) {
#pragma unroll
    for (int i = 0; i < N; i += 4) *reinterpret_cast<float4*>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  };
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int d = (int)(u % cv) * N;
    const int64_t rest = u / cv;
    const int64_t e = rest % (ne + 1);
    const int64_t s = rest / (ne + 1);
    const int64_t sq = s * n * (int64_t)c;
    if (e == ne) {
      for (int64_t row = ne * m; row < n; ++row) {
        st_zero(dCa + sq + row * c + d);
        st_zero(dZa + sq + row * c + d);
        if (overlap) { st_zero(dCb + sq + row * c + d); st_zero(dZb + sq + row * c + d); }
      }
      if (overlap && ne > 0)
        for (int j = 0; j < m; ++j) {
          const int64_t row = (ne - 1) * m + j;
          st_zero(dCb + sq + row * c + d);
          st_zero(dZb + sq + row * c + d);
        }
      if (overlap && ne == 0 && dpCb)
        for (int j = 0; j < m; ++j) { st_zero(dpCb + (s * m + j) * c + d); st_zero(dpZb + (s * m + j) * c + d); }
      continue;
    }
    const bool hasb = overlap && (e > 0 || pZb != nullptr);
    auto zb_row = [&](int j) { return e > 0 ? Zb + sq + (m * (e - 1) + j) * c + d : pZb + (s * m + j) * c + d; };
    auto cb_row = [&](int j) { return e > 0 ? Cb + sq + (m * (e - 1) + j) * c + d : pCb + (s * m + j) * c + d; };
    float mx[N], den[N], num[N], g[N], cc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) { mx[i] = -INFINITY; den[i] = 0.f; num[i] = 0.f; }
    for (int j = 0; j < m; ++j) {
      float z[N], bb[N];
      Vec16<T>::ld(Za + sq + (m * e + j) * c + d, z);
      Vec16<T>::ld(Ba + j * c + d, bb);
#pragma unroll
      for (int i = 0; i < N; ++i) mx[i] = fmaxf(mx[i], z[i] + bb[i]);
      if (hasb) {
        Vec16<T>::ld(zb_row(j), z);
        Vec16<T>::ld(Bb + j * c + d, bb);
#pragma unroll
        for (int i = 0; i < N; ++i) mx[i] = fmaxf(mx[i], z[i] + bb[i]);
      }
    }
    for (int j = 0; j < m; ++j) {
      float z[N], bb[N], cv8[N];
      Vec16<T>::ld(Za + sq + (m * e + j) * c + d, z);
      Vec16<T>::ld(Ba + j * c + d, bb);
      Vec16<T>::ld(Ca + sq + (m * e + j) * c + d, cv8);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float pa = __expf(z[i] + bb[i] - mx[i]);
        den[i] += pa;
        num[i] = fmaf(pa, cv8[i], num[i]);
      }
      if (hasb) {
        Vec16<T>::ld(zb_row(j), z);
        Vec16<T>::ld(Bb + j * c + d, bb);
        Vec16<T>::ld(cb_row(j), cv8);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float pb = __expf(z[i] + bb[i] - mx[i]);
          den[i] += pb;
          num[i] = fmaf(pb, cv8[i], num[i]);
        }
      }
    }
    {
      float gg[4];
#pragma unroll
      for (int i = 0; i < N; i += 4) {
        F::ld(dCc + (s * ne + e) * c + d + i, gg);
        g[i] = gg[0]; g[i + 1] = gg[1]; g[i + 2] = gg[2]; g[i + 3] = gg[3];
      }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) cc[i] = num[i] / den[i];
    for (int j = 0; j < m; ++j) {
      const int64_t ra = m * e + j;
      float z[N], bb[N], cv8[N], o1[N], o2[N];
      Vec16<T>::ld(Za + sq + ra * c + d, z);
      Vec16<T>::ld(Ba + j * c + d, bb);
      Vec16<T>::ld(Ca + sq + ra * c + d, cv8);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float sa = __expf(z[i] + bb[i] - mx[i]) / den[i];
        o1[i] = sa * g[i];
        o2[i] = sa * (cv8[i] - cc[i]) * g[i];
      }
      st_f(dCa + sq + ra * c + d, o1);
      st_f(dZa + sq + ra * c + d, o2);
      if (hasb) {
        Vec16<T>::ld(zb_row(j), z);
        Vec16<T>::ld(Bb + j * c + d, bb);
        Vec16<T>::ld(cb_row(j), cv8);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float sb = __expf(z[i] + bb[i] - mx[i]) / den[i];
          o1[i] = sb * g[i];
          o2[i] = sb * (cv8[i] - cc[i]) * g[i];
        }
        if (e > 0) {
          const int64_t rb = m * (e - 1) + j;
          st_f(dCb + sq + rb * c + d, o1);
          st_f(dZb + sq + rb * c + d, o2);
        } else if (dpCb) {
          st_f(dpCb + (s * m + j) * c + d, o1);
          st_f(dpZb + (s * m + j) * c + d, o2);
        }
      } else if (overlap && e == 0 && dpCb) {
        st_zero(dpCb + (s * m + j) * c + d);
        st_zero(dpZb + (s * m + j) * c + d);
      }
    }
  }
}

// The same for m = 4 with the bias gradients folded in: a grid of at most
// kBiasWGs workgroups walks the (sequence, entry, 8-dimension group) units
// with a stride that is a multiple of c / 8, so a thread keeps one group of
// dimensions and sums its rows' dZ per in-block row j for both streams
// (stream b: the rows of block e - 1, or the previous-block state for
// e = 0); the four threads of a workgroup that share a group add their sums
// in thread order and the workgroup writes one partial [stream][j][c]; the
// final kernel adds the partials in workgroup order.  Deterministic for a
// given shape.
constexpr int kBiasWGs = 512;
template <typename T>
__global__ __launch_bounds__(kBwdT) void compress_bwd_rows_v4b(
    const T* __restrict__ Ca, const T* __restrict__ Cb, const T* __restrict__ Za, const T* __restrict__ Zb,
    const T* __restrict__ Ba, const T* __restrict__ Bb, const T* __restrict__ pCb, const T* __restrict__ pZb,
    const float* __restrict__ dCc, int64_t b, int64_t n, int c, float* __restrict__ dCa, float* __restrict__ dCb,
    float* __restrict__ dZa, float* __restrict__ dZb, float* __restrict__ dpCb, float* __restrict__ dpZb,
    float* __restrict__ part) {
  constexpr int N = Vec16<T>::N;
  constexpr int M = 4;
  typedef Vec16<float> F;
  __shared__ float red[kBwdT][2 * M][N];
  const int cv = c / N;
  const int64_t ne = n / M;
  const int64_t total = b * (ne + 1) * cv;
  auto st_f = [](float* p, const float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float w[4] = {v[i], v[i + 1], v[i + 2], v[i + 3]};
      F::st(p + i, w);
    }
  };
  auto st_zero = [](float* p) {
#pragma unroll
    for (int i = 0; i < N; i += 4) *reinterpret_cast<float4*>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  };
  float accA[M][N], accB[M][N];
#pragma unroll
  for (int j = 0; j < M; ++j)
#pragma unroll
    for (int i = 0; i < N; ++i) { accA[j][i] = 0.f; accB[j][i] = 0.f; }
  const int64_t u0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int d = (int)(u0 % cv) * N;   // the stride keeps it
  for (int64_t u = u0; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rest = u / cv;
    const int64_t e = rest % (ne + 1);
    const int64_t s = rest / (ne + 1);
    const int64_t sq = s * n * (int64_t)c;
    if (e == ne) {
      for (int64_t row = ne * M; row < n; ++row) {
        st_zero(dCa + sq + row * c + d);
        st_zero(dZa + sq + row * c + d);
        st_zero(dCb + sq + row * c + d);
        st_zero(dZb + sq + row * c + d);
      }
      if (ne > 0)
        for (int j = 0; j < M; ++j) {
          const int64_t row = (ne - 1) * M + j;
          st_zero(dCb + sq + row * c + d);
          st_zero(dZb + sq + row * c + d);
        }
      if (ne == 0 && dpCb)
        for (int j = 0; j < M; ++j) { st_zero(dpCb + (s * M + j) * c + d); st_zero(dpZb + (s * M + j) * c + d); }
      continue;
    }
    const bool hasb = e > 0 || pZb != nullptr;
    auto zb_row = [&](int j) { return e > 0 ? Zb + sq + (M * (e - 1) + j) * c + d : pZb + (s * M + j) * c + d; };
    auto cb_row = [&](int j) { return e > 0 ? Cb + sq + (M * (e - 1) + j) * c + d : pCb + (s * M + j) * c + d; };
    float mx[N], den[N], num[N], g[N], cc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) { mx[i] = -INFINITY; den[i] = 0.f; num[i] = 0.f; }
    for (int j = 0; j < M; ++j) {
      float z[N], bb[N];
      Vec16<T>::ld(Za + sq + (M * e + j) * c + d, z);
      Vec16<T>::ld(Ba + j * c + d, bb);
#pragma unroll
      for (int i = 0; i < N; ++i) mx[i] = fmaxf(mx[i], z[i] + bb[i]);
      if (hasb) {
        Vec16<T>::ld(zb_row(j), z);
        Vec16<T>::ld(Bb + j * c + d, bb);
#pragma unroll
        for (int i = 0; i < N; ++i) mx[i] = fmaxf(mx[i], z[i] + bb[i]);
      }
    }
    for (int j = 0; j < M; ++j) {
      float z[N], bb[N], cv8[N];
      Vec16<T>::ld(Za + sq + (M * e + j) * c + d, z);
      Vec16<T>::ld(Ba + j * c + d, bb);
      Vec16<T>::ld(Ca + sq + (M * e + j) * c + d, cv8);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float pa = __expf(z[i] + bb[i] - mx[i]);
        den[i] += pa;
        num[i] = fmaf(pa, cv8[i], num[i]);
      }
      if (hasb) {
        Vec16<T>::ld(zb_row(j), z);
        Vec16<T>::ld(Bb + j * c + d, bb);
        Vec16<T>::ld(cb_row(j), cv8);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float pb = __expf(z[i] + bb[i] - mx[i]);
          den[i] += pb;
          num[i] = fmaf(pb, cv8[i], num[i]);
        }
      }
    }
    {
      float gg[4];
#pragma unroll
      for (int i = 0; i < N; i += 4) {
        F::ld(dCc + (s * ne + e) * c + d + i, gg);
        g[i] = gg[0]; g[i + 1] = gg[1]; g[i + 2] = gg[2]; g[i + 3] = gg[3];
      }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) cc[i] = num[i] / den[i];
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const int64_t ra = M * e + j;
      float z[N], bb[N], cv8[N], o1[N], o2[N];
      Vec16<T>::ld(Za + sq + ra * c + d, z);
      Vec16<T>::ld(Ba + j * c + d, bb);
      Vec16<T>::ld(Ca + sq + ra * c + d, cv8);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float sa = __expf(z[i] + bb[i] - mx[i]) / den[i];
        o1[i] = sa * g[i];
        o2[i] = sa * (cv8[i] - cc[i]) * g[i];
        accA[j][i] += o2[i];
      }
      st_f(dCa + sq + ra * c + d, o1);
      st_f(dZa + sq + ra * c + d, o2);
      if (hasb) {
        Vec16<T>::ld(zb_row(j), z);
        Vec16<T>::ld(Bb + j * c + d, bb);
        Vec16<T>::ld(cb_row(j), cv8);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float sb = __expf(z[i] + bb[i] - mx[i]) / den[i];
          o1[i] = sb * g[i];
          o2[i] = sb * (cv8[i] - cc[i]) * g[i];
          accB[j][i] += o2[i];
        }
        if (e > 0) {
          const int64_t rb = M * (e - 1) + j;
          st_f(dCb + sq + rb * c + d, o1);
          st_f(dZb + sq + rb * c + d, o2);
        } else {
          st_f(dpCb + (s * M + j) * c + d, o1);
          st_f(dpZb + (s * M + j) * c + d, o2);
        }
      } else if (e == 0 && dpCb) {
        st_zero(dpCb + (s * M + j) * c + d);
        st_zero(dpZb + (s * M + j) * c + d);
      }
    }
  }
  // the threads sharing this group of dimensions: t % cv, in thread order
#pragma unroll
  for (int j = 0; j < M; ++j)
#pragma unroll
    for (int i = 0; i < N; ++i) {
      red[threadIdx.x][j][i] = accA[j][i];
      red[threadIdx.x][M + j][i] = accB[j][i];
    }
  __syncthreads();
  if ((int)threadIdx.x < cv) {
    float* pw = part + (int64_t)blockIdx.x * 2 * M * c;
    for (int r = 0; r < 2 * M; ++r) {
      float v[N];
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = 0.f;
      for (int t = threadIdx.x; t < kBwdT; t += cv)
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += red[t][r][i];
      st_f(pw + (int64_t)r * c + d, v);
    }
  }
}
// dB_stream[j][d] = sum over the workgroups' partials, in workgroup order:
// one workgroup per 64 outputs, wave w adding a quarter of the partials
// eight loads at a time, the quarters added in wave order.
__global__ __launch_bounds__(kBwdT) void compress_bwd_bias4_final(const float* __restrict__ part, int nwg, int c,
                                                                  float* __restrict__ dBa, float* __restrict__ dBb) {
  __shared__ float ws4[4][64];
  constexpr int M = 4;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t mc2 = (int64_t)2 * M * c;
  const int64_t u = (int64_t)blockIdx.x * 64 + l;
  const int qn = (nwg + 3) / 4;
  const int w0 = wave * qn, w1 = w0 + qn < nwg ? w0 + qn : nwg;
  float a = 0.f;
  if (u < mc2) {
    for (int w = w0; w < w1; w += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = w + i < w1 ? part[(int64_t)(w + i) * mc2 + u] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (w + i < w1) a += v[i];
    }
  }
  ws4[wave][l] = a;
  __syncthreads();
  if (wave == 0 && u < mc2) {
    const float r = ((ws4[0][l] + ws4[1][l]) + ws4[2][l]) + ws4[3][l];
    if (u < (int64_t)M * c) dBa[u] = r; else dBb[u - (int64_t)M * c] = r;
  }
}

// Bias gradient, stage 1: per (chunk of 64 entries, in-block row j,
// dimension d) the sum of dZ over the chunk's entries in order (over every
// sequence); stage 2 adds the chunks in order.  stream b: entry e's rows
// are those of block e - 1 (the previous-block state for e = 0).
constexpr int kBiasChunk = 64;
__global__ __launch_bounds__(kBwdT) void compress_bwd_bias_partial(const float* __restrict__ dZ,
                                                                   const float* __restrict__ dpZ, int64_t b, int64_t n,
                                                                   int c, int m, int shift, float* __restrict__ part) {
  const int64_t ne = n / m;
  const int64_t nch = (ne + kBiasChunk - 1) / kBiasChunk;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= nch * m * (int64_t)c) return;
  const int d = (int)(u % c);
  const int j = (int)((u / c) % m);
  const int64_t ch = u / ((int64_t)c * m);
  float a = 0.f;
  for (int64_t s = 0; s < b; ++s)
    for (int64_t e = ch * kBiasChunk; e < ne && e < (ch + 1) * kBiasChunk; ++e) {
      if (shift && e == 0) {
        if (dpZ) a += dpZ[(s * m + j) * c + d];
        continue;
      }
      const int64_t row = m * (e - shift) + j;
      a += dZ[(s * n + row) * c + d];
    }
  part[u] = a;
}
// One workgroup per 64 (row, dimension) outputs: wave w sums the chunks
// w * q .. (w + 1) * q - 1 (q = nch / 4 rounded up) in order, eight loads in
// flight, then the four wave sums are added in wave order.
__global__ __launch_bounds__(kBwdT) void compress_bwd_bias_final(const float* __restrict__ part, int64_t nch, int c,
                                                                 int m, float* __restrict__ dB) {
  __shared__ float ws4[4][64];
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t mc = (int64_t)m * c;
  const int64_t u = (int64_t)blockIdx.x * 64 + l;
  const int64_t qn = (nch + 3) / 4;
  const int64_t c0 = wave * qn, c1 = c0 + qn < nch ? c0 + qn : nch;
  float a = 0.f;
  if (u < mc) {
    for (int64_t ch = c0; ch < c1; ch += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ch + i < c1 ? part[(ch + i) * mc + u] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (ch + i < c1) a += v[i];
    }
  }
  ws4[wave][l] = a;
  __syncthreads();
  if (wave == 0 && u < mc) dB[u] = ((ws4[0][l] + ws4[1][l]) + ws4[2][l]) + ws4[3][l];
}

// the m = 4 path with 16-byte rows whose dimension groups divide a workgroup
static bool compress_bwd_v4b_ok(int64_t c, int64_t m) { return m == 4 && c % 8 == 0 && kBwdT % (c / 8) == 0; }

size_t compress_backward_workspace_bytes(int64_t n, int64_t c, int64_t m) {
  const int64_t ne = n / m;
  const int64_t nch = (ne + kBiasChunk - 1) / kBiasChunk;
  size_t bytes = (size_t)((nch > 0 ? nch : 1) * m * c * 4 + 255) & ~(size_t)255;
  if (compress_bwd_v4b_ok(c, m)) bytes = std::max(bytes, (size_t)kBiasWGs * 2 * 4 * c * 4);
  return bytes;
}

hipError_t launch_compress_backward(const void* Ca, const void* Cb, const void* Za, const void* Zb, const void* Ba,
                                    const void* Bb, const void* pCb, const void* pZb, const float* dCc, int64_t b,
                                    int64_t n, int64_t c, int64_t m, int overlap, int dtype, float* dCa, float* dCb,
                                    float* dZa, float* dZb, float* dBa, float* dBb, float* dpCb, float* dpZb,
                                    void* ws, hipStream_t st) {
  const int64_t ne = n / m;
  const int64_t total = b * (ne + 1) * c;
  const unsigned grid = (unsigned)std::min<int64_t>((total + kBwdT - 1) / kBwdT, 65535 * 4);
  // bf16 with 16-byte rows and aligned arrays: 8 dimensions per thread
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const bool vec_ok = dtype == 1 && c % 8 == 0 && a16(Ca) && a16(Za) && a16(Ba) && a16(dCc) && a16(dCa) && a16(dZa) &&
                      (!overlap || (a16(Cb) && a16(Zb) && a16(Bb) && a16(dCb) && a16(dZb))) && a16(pCb) && a16(pZb) &&
                      a16(dpCb) && a16(dpZb);
  const unsigned grid_v = (unsigned)std::min<int64_t>((b * (ne + 1) * (c / 8) + kBwdT - 1) / kBwdT, 65535 * 4);
  if (vec_ok && overlap && compress_bwd_v4b_ok(c, m)) {
    const int nwg = (int)std::min<int64_t>((b * (ne + 1) * (c / 8) + kBwdT - 1) / kBwdT, kBiasWGs);
    hipLaunchKernelGGL(compress_bwd_rows_v4b<bf16_t>, dim3((unsigned)nwg), dim3(kBwdT), 0, st, (const bf16_t*)Ca,
                       (const bf16_t*)Cb, (const bf16_t*)Za, (const bf16_t*)Zb, (const bf16_t*)Ba, (const bf16_t*)Bb,
                       (const bf16_t*)pCb, (const bf16_t*)pZb, dCc, b, n, (int)c, dCa, dCb, dZa, dZb, dpCb, dpZb,
                       (float*)ws);
    hipLaunchKernelGGL(compress_bwd_bias4_final, dim3((unsigned)((2 * 4 * c + 63) / 64)), dim3(kBwdT), 0, st,
                       (const float*)ws, nwg, (int)c, dBa, dBb);
    return hipGetLastError();
  }
  if (vec_ok)
    hipLaunchKernelGGL(compress_bwd_rows_v<bf16_t>, dim3(grid_v), dim3(kBwdT), 0, st, (const bf16_t*)Ca,
                       (const bf16_t*)Cb, (const bf16_t*)Za, (const bf16_t*)Zb, (const bf16_t*)Ba, (const bf16_t*)Bb,
                       (const bf16_t*)pCb, (const bf16_t*)pZb, dCc, b, n, (int)c, (int)m, overlap, dCa, dCb, dZa, dZb,
                       dpCb, dpZb);
  else if (dtype == 1)
    hipLaunchKernelGGL(compress_bwd_rows<bf16_t>, dim3(grid), dim3(kBwdT), 0, st, (const bf16_t*)Ca,
                       (const bf16_t*)Cb, (const bf16_t*)Za, (const bf16_t*)Zb, (const bf16_t*)Ba, (const bf16_t*)Bb,
                       (const bf16_t*)pCb, (const bf16_t*)pZb, dCc, b, n, (int)c, (int)m, overlap, dCa, dCb, dZa, dZb,
                       dpCb, dpZb);
  else
    hipLaunchKernelGGL(compress_bwd_rows<float>, dim3(grid), dim3(kBwdT), 0, st, (const float*)Ca, (const float*)Cb,
                       (const float*)Za, (const float*)Zb, (const float*)Ba, (const float*)Bb, (const float*)pCb,
                       (const float*)pZb, dCc, b, n, (int)c, (int)m, overlap, dCa, dCb, dZa, dZb, dpCb, dpZb);
  const int64_t nch = (ne + kBiasChunk - 1) / kBiasChunk;
  float* part = (float*)ws;
  const int64_t pu = nch * m * c;
  for (int stream = 0; stream < (overlap ? 2 : 1); ++stream) {
    float* dB = stream == 0 ? dBa : dBb;
    if (nch > 0)
      hipLaunchKernelGGL(compress_bwd_bias_partial, dim3((unsigned)((pu + kBwdT - 1) / kBwdT)), dim3(kBwdT), 0, st,
                         stream == 0 ? dZa : dZb, stream == 0 ? (const float*)nullptr : (const float*)dpZb, b, n,
                         (int)c, (int)m, stream, part);
    hipLaunchKernelGGL(compress_bwd_bias_final, dim3((unsigned)((m * c + 63) / 64)), dim3(kBwdT), 0, st, part, nch,
                       (int)c, (int)m, dB);
  }
  return hipGetLastError();
}

}  // namespace csa
