// RMSNorm and partial rotary embedding of query heads, KV entries and
// attention outputs (songhuiming "DeepSeek-V4 百万 token 上下文" section 4.5;
// AirCoding "deepseek-paper-analysis" section 7.1).
//
// Each vector of c values (one query head, one KV entry) is divided by the
// root of its mean square plus eps and multiplied by a per-dimension gain;
// then the last rope_dims dimensions, taken as adjacent pairs (2i, 2i+1) of
// that slice, turn by pos * base^(-2i / rope_dims) radians.  The vectors of
// one row share the row's position pos0 + row * pos_step, so a workgroup
// serves one row and builds its rotation table once, in float64: positions
// reach 2^20 and beyond, where a float32 product would lose the angle.  The
// back-rotation of an attention output by -t is the same kernel with no gain
// and negative positions.
//
// The mean square is a fixed-order butterfly over the wave, so results are
// reproducible.  HBM-bound: every value is read and written once, except that
// a rotation-only update in place (no gain, out == x) touches only the chunks
// holding rotated dimensions.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int kNrMaxPairs = 256;   // rotation pairs (rope_dims <= 512)

// Rotation table of one row: (cos, sin) of pos * base^(-2i / rope_dims) for
// i < rope_dims / 2, in float64, written by the first rope_dims / 2 threads.
// The caller issues its loads next and then waits at a barrier before the
// first read: the other waves' loads overlap the table's float64 work, and
// no loaded values are held across it.
__device__ __forceinline__ void rotation_table(float2* rot, int rope_dims, double base, int64_t pos) {
  const int npair = rope_dims >> 1;
  if ((int)threadIdx.x < npair) {
    const double theta = pow(base, -2.0 * (double)threadIdx.x / (double)rope_dims);
    double s, co;
    sincos((double)pos * theta, &s, &co);
    rot[threadIdx.x] = make_float2((float)co, (float)s);
  }
}

// Turn the pairs of one 16-byte chunk (dims d0 .. d0 + V - 1) that lie in the
// rotated part (dims >= lo).
template <int V>
__device__ __forceinline__ void rotate_chunk(float (&v)[V], int d0, int lo, const float2* rot) {
#pragma unroll
  for (int i = 0; i < V; i += 2) {
    const int d = d0 + i;
    if (d >= lo) {
      const float2 r = rot[(d - lo) >> 1];
      const float a = v[i], b = v[i + 1];
      v[i] = a * r.x - b * r.y;
      v[i + 1] = a * r.y + b * r.x;
    }
  }
}

// Norm (optional) and rotation of whole vectors.  One workgroup per row; a
// wave owns vectors wave*VPP + 4*VPP*j .. +VPP-1 and loads all of a pass's
// vectors before using any.  MC: 16-byte chunks per lane and vector (c up to
// 64 * MC chunks); VPP * MC = 4 chunks per lane in flight.
template <typename T, int MC>
__global__ __launch_bounds__(256) void norm_rope(const T* x, int64_t xrs, T* out, int64_t ors,
                                                 const float* __restrict__ gamma, float eps, int heads,
                                                 int c, int rope_dims, double base, int64_t pos0,
                                                 int64_t pos_step) {
  constexpr int V = Vec16<T>::N;
  constexpr int VPP = MC == 4 ? 1 : 4 / MC;   // vectors per wave and pass
  __shared__ float2 rot[kNrMaxPairs];
  const int64_t row = blockIdx.x;
  const int lo = c - rope_dims;
  const int nch = c / V;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const T* xr = x + row * xrs;
  T* orow = out + row * ors;
  uint4 raw[VPP][MC];
  auto load = [&](int h0) {
#pragma unroll
    for (int hb = 0; hb < VPP; ++hb)
#pragma unroll
      for (int j = 0; j < MC; ++j) {
        const int ch = l + 64 * j;
        raw[hb][j] = make_uint4(0u, 0u, 0u, 0u);
        if (h0 + hb < heads && ch < nch)
          raw[hb][j] = *reinterpret_cast<const uint4*>(xr + (int64_t)(h0 + hb) * c + ch * V);
      }
  };
  rotation_table(rot, rope_dims, base, pos0 + row * pos_step);
  int h0 = wave * VPP;
  load(h0);
  __syncthreads();   // the table is complete
  for (; h0 < heads; h0 += 4 * VPP) {
    if (h0 != wave * VPP) load(h0);
    float inv[VPP];
#pragma unroll
    for (int hb = 0; hb < VPP; ++hb) {
      inv[hb] = 1.f;
      if (gamma) {   // uniform: every lane joins the reduction
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < MC; ++j)
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const float v = Vec16<T>::get(raw[hb][j], i);
            ss = fmaf(v, v, ss);
          }
        ss = wave_sum(ss);
        inv[hb] = 1.f / sqrtf(ss / (float)c + eps);
      }
    }
#pragma unroll
    for (int hb = 0; hb < VPP; ++hb)
#pragma unroll
      for (int j = 0; j < MC; ++j) {
        const int ch = l + 64 * j;
        if (h0 + hb >= heads || ch >= nch) continue;
        const int d0 = ch * V;
        float v[V];
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] = Vec16<T>::get(raw[hb][j], i) * inv[hb];
        if (gamma) {
#pragma unroll
          for (int i = 0; i < V; i += 4) {
            const float4 g = *reinterpret_cast<const float4*>(gamma + d0 + i);
            v[i] *= g.x; v[i + 1] *= g.y; v[i + 2] *= g.z; v[i + 3] *= g.w;
          }
        }
        rotate_chunk<V>(v, d0, lo, rot);
        Vec16<T>::st(orow + (int64_t)(h0 + hb) * c + d0, v);
      }
  }
}

// Norm (optional) and rotation of rows holding one or two vectors (KV
// entries, window rows): one wave per row and four rows per workgroup, each
// wave with its own rotation table, so that no wave of a workgroup idles.
// Same arithmetic, in the same order, as norm_rope.
template <typename T, int MC>
__global__ __launch_bounds__(256) void norm_rope_rows(const T* x, int64_t xrs, T* out, int64_t ors,
                                                      const float* __restrict__ gamma, float eps, int64_t rows,
                                                      int heads, int c, int rope_dims, double base, int64_t pos0,
                                                      int64_t pos_step) {
  constexpr int V = Vec16<T>::N;
  __shared__ float2 rot_all[4][kNrMaxPairs];
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= rows) return;   // a whole wave; there is no workgroup barrier below
  float2* rot = rot_all[wave];
  const int lo = c - rope_dims;
  const int nch = c / V;
  const T* xr = x + row * xrs;
  T* orow = out + row * ors;
  for (int h = 0; h < heads; ++h) {
    uint4 raw[MC];
#pragma unroll
    for (int j = 0; j < MC; ++j) {
      const int ch = l + 64 * j;
      raw[j] = ch < nch ? *reinterpret_cast<const uint4*>(xr + (int64_t)h * c + ch * V) : make_uint4(0u, 0u, 0u, 0u);
    }
    if (h == 0) {
      // the wave's table while its first vector is in flight; the LDS
      // executes one wave's accesses in order, so the reads below see it
      const int64_t pos = pos0 + row * pos_step;
      for (int i = l; i < (rope_dims >> 1); i += 64) {
        const double theta = pow(base, -2.0 * (double)i / (double)rope_dims);
        double sn, co;
        sincos((double)pos * theta, &sn, &co);
        rot[i] = make_float2((float)co, (float)sn);
      }
    }
    float inv = 1.f;
    if (gamma) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < MC; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const float v = Vec16<T>::get(raw[j], i);
          ss = fmaf(v, v, ss);
        }
      ss = wave_sum(ss);
      inv = 1.f / sqrtf(ss / (float)c + eps);
    }
#pragma unroll
    for (int j = 0; j < MC; ++j) {
      const int ch = l + 64 * j;
      if (ch >= nch) continue;
      const int d0 = ch * V;
      float v[V];
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = Vec16<T>::get(raw[j], i) * inv;
      if (gamma) {
#pragma unroll
        for (int i = 0; i < V; i += 4) {
          const float4 g = *reinterpret_cast<const float4*>(gamma + d0 + i);
          v[i] *= g.x; v[i + 1] *= g.y; v[i + 2] *= g.z; v[i + 3] *= g.w;
        }
      }
      rotate_chunk<V>(v, d0, lo, rot);
      Vec16<T>::st(orow + (int64_t)h * c + d0, v);
    }
  }
}

// Rotation only, in place: just the 16-byte chunks holding rotated dims,
// spread over the workgroup's threads across all vectors of the row (an
// attention output's 64 rotated dims of 512 are 8 chunks per head).
template <typename T>
__global__ __launch_bounds__(256) void rope_in_place(T* x, int64_t xrs, int heads, int c, int rope_dims,
                                                     double base, int64_t pos0, int64_t pos_step) {
  constexpr int V = Vec16<T>::N;
  constexpr int U = 4;   // chunks per thread and round, loaded before use
  __shared__ float2 rot[kNrMaxPairs];
  const int64_t row = blockIdx.x;
  const int lo = c - rope_dims;
  const int ch0 = lo / V, nrc = c / V - ch0;   // chunks from the first holding a rotated dim
  const int items = heads * nrc;
  T* xr = x + row * xrs;
  bool first = true;
  rotation_table(rot, rope_dims, base, pos0 + row * pos_step);
  for (int b0 = 0; b0 < items; b0 += 256 * U) {   // uniform over the workgroup
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = b0 + u * 256 + (int)threadIdx.x;
      raw[u] = make_uint4(0u, 0u, 0u, 0u);
      if (it < items) raw[u] = *reinterpret_cast<const uint4*>(xr + (int64_t)(it / nrc) * c + (ch0 + it % nrc) * V);
    }
    if (first) __syncthreads();   // the table is complete
    first = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = b0 + u * 256 + (int)threadIdx.x;
      if (it >= items) continue;
      const int d0 = (ch0 + it % nrc) * V;
      float v[V];
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = Vec16<T>::get(raw[u], i);
      rotate_chunk<V>(v, d0, lo, rot);
      Vec16<T>::st(xr + (int64_t)(it / nrc) * c + d0, v);
    }
  }
}

hipError_t launch_norm_rope(const void* x, int64_t xrs, void* out, int64_t ors, const float* gamma, float eps,
                            int64_t rows, int64_t heads, int64_t c, int64_t rope_dims, double base, int64_t pos0,
                            int64_t pos_step, int dtype, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  // no gain and an in-place update: only the rotated dimensions change
  if (gamma == nullptr && x == out && xrs == ors) {
    if (rope_dims == 0) return hipSuccess;
    if (dtype == 1)
      hipLaunchKernelGGL(rope_in_place<bf16_t>, dim3((unsigned)rows), dim3(256), 0, st, (bf16_t*)out, ors,
                         (int)heads, (int)c, (int)rope_dims, base, pos0, pos_step);
    else
      hipLaunchKernelGGL(rope_in_place<float>, dim3((unsigned)rows), dim3(256), 0, st, (float*)out, ors, (int)heads,
                         (int)c, (int)rope_dims, base, pos0, pos_step);
    return hipGetLastError();
  }
  const int64_t nch = c / (dtype == 1 ? 8 : 4);
  const int mc = nch <= 64 ? 1 : nch <= 128 ? 2 : 4;
  // rows of one or two vectors: a wave per row
  const bool per_wave = heads <= 2;
#define CSA_NR_LAUNCH(T, MCV)                                                                                  \
  if (per_wave)                                                                                                \
    hipLaunchKernelGGL((norm_rope_rows<T, MCV>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,          \
                       (const T*)x, xrs, (T*)out, ors, gamma, eps, rows, (int)heads, (int)c, (int)rope_dims, base, \
                       pos0, pos_step);                                                                       \
  else                                                                                                         \
    hipLaunchKernelGGL((norm_rope<T, MCV>), dim3((unsigned)rows), dim3(256), 0, st, (const T*)x, xrs, (T*)out,  \
                       ors, gamma, eps, (int)heads, (int)c, (int)rope_dims, base, pos0, pos_step)
  if (dtype == 1) {
    if (mc == 1) CSA_NR_LAUNCH(bf16_t, 1);
    else if (mc == 2) CSA_NR_LAUNCH(bf16_t, 2);
    else CSA_NR_LAUNCH(bf16_t, 4);
  } else {
    if (mc == 1) CSA_NR_LAUNCH(float, 1);
    else if (mc == 2) CSA_NR_LAUNCH(float, 2);
    else CSA_NR_LAUNCH(float, 4);
  }
#undef CSA_NR_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
