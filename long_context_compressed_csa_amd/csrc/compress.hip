// Token-level KV compressor (CSA overlapped form and HCA pooling form).
//
// Definition: polysight "06-formulas" section B9 and songhuiming
// "DeepSeek-V4 百万 token 上下文" section 4.1 (Eq. 11-12) for the overlapped
// form -- entry i takes a per-dimension softmax over the m rows of block i
// of stream a and the m rows of block i-1 of stream b, each score plus its
// intra-block bias, and sums the element-wise products with the values;
// block -1 is padded with -inf scores and zero values.  Section 5.1 of the
// same page (and AirCoding "deepseek-paper-analysis" section 7.2) for the
// pooling form: one stream, the m' rows of the block, no overlap.
//
// The operation is a pure HBM stream: every input row is read exactly once
// (entry i reads only block i of stream a and block i-1 of stream b), with
// ~1 flop per byte.  Threads therefore own 16-byte slices of a row so that a
// wave reads whole rows with 16-byte loads, and all loads of an entry are
// issued before any arithmetic.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// One thread per (sequence, entry, 16-byte dimension slice), M rows per
// block known at compile time (the CSA ratio m = 4).  Stream-b rows come
// from block e-1, or from the caller's previous-block state for e == 0.
template <typename T, int M>
__global__ __launch_bounds__(256) void compress_overlap_fixed(
    const T* __restrict__ Ca, const T* __restrict__ Cb, const T* __restrict__ Za,
    const T* __restrict__ Zb, const T* __restrict__ Ba, const T* __restrict__ Bb,
    const T* __restrict__ pCb, const T* __restrict__ pZb, int64_t n, int c, int64_t ne,
    int64_t total, T* __restrict__ out, int64_t obs) {
  constexpr int V = Vec16<T>::N;
  const int CH = c / V;
  // grid-stride over (sequence, entry, channel) units.  When the stride is a
  // multiple of CH (c = 512 and 128: 256 threads per block), a thread keeps
  // its channel and loads that channel's bias rows once.
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  float ba[M][V], bb[M][V];
  int chb = -1;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += stride) {
    const int ch = (int)(u % CH);
    const int d0 = ch * V;
    if (ch != chb) {
#pragma unroll
      for (int j = 0; j < M; ++j) {
        Vec16<T>::ld(Ba + j * (int64_t)c + d0, ba[j]);
        Vec16<T>::ld(Bb + j * (int64_t)c + d0, bb[j]);
      }
      chb = ch;
    }
    const int64_t rest = u / CH;
    const int64_t e = rest % ne;
    const int64_t s = rest / ne;
    const int64_t seq = s * n * (int64_t)c;
    float za[M][V], ca[M][V], zb[M][V], cb[M][V];
    const T* zap = Za + seq + (M * e) * (int64_t)c + d0;
    const T* cap = Ca + seq + (M * e) * (int64_t)c + d0;
    // block e-1 of stream b, or the caller's previous block; at the sequence
    // start with no previous block, rows of block e stand in (weight 0)
    const bool hasb = (e > 0) || (pZb != nullptr);
    const T* zbp = e > 0 ? Zb + seq + (M * (e - 1)) * (int64_t)c + d0
                         : (pZb != nullptr ? pZb + s * M * (int64_t)c + d0 : zap);
    const T* cbp = e > 0 ? Cb + seq + (M * (e - 1)) * (int64_t)c + d0
                         : (pCb != nullptr ? pCb + s * M * (int64_t)c + d0 : cap);
#pragma unroll
    for (int j = 0; j < M; ++j) {
      Vec16<T>::ld(zap + j * (int64_t)c, za[j]);
      Vec16<T>::ld(cap + j * (int64_t)c, ca[j]);
      Vec16<T>::ld(zbp + j * (int64_t)c, zb[j]);
      Vec16<T>::ld(cbp + j * (int64_t)c, cb[j]);
    }
    float res[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        za[j][v] += ba[j][v];
        mx = fmaxf(mx, za[j][v]);
        zb[j][v] = hasb ? zb[j][v] + bb[j][v] : -INFINITY;
        mx = fmaxf(mx, zb[j][v]);
      }
      float sum = 0.f, acc = 0.f;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const float p = fast_exp(za[j][v] - mx);
        sum += p;
        acc = fmaf(p, ca[j][v], acc);
      }
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const float p = fast_exp(zb[j][v] - mx);   // 0 for the padded block -1
        sum += p;
        acc = fmaf(p, cb[j][v], acc);
      }
      res[v] = acc / sum;
    }
    Vec16<T>::st(out + s * obs + e * (int64_t)c + d0, res);
  }
}

// Row access for the generic kernel: VEC = Vec16<T>::N with 16-byte loads,
// or 1 with scalar loads when c is not a multiple of the vector width.
template <typename T, int V> struct RowIO {
  static __device__ __forceinline__ void ld(const T* p, float (&o)[V]) {
    if constexpr (V == 1) {
      o[0] = Elem<T>::ld(p);
    } else {
      Vec16<T>::ld(p, o);
    }
  }
  static __device__ __forceinline__ void st(T* p, const float (&o)[V]) {
    if constexpr (V == 1) {
      Elem<T>::st(p, o[0]);
    } else {
      Vec16<T>::st(p, o);
    }
  }
};

// Any m, either form.  A workgroup owns one entry and CHB dimension slices;
// its P parts split the entry's rows (interleaved) and keep a running
// max / sum / weighted sum each, merged in part order through LDS.
// Virtual rows 0..m-1 are block e of stream a; rows m..2m-1 (overlap only)
// are block e-1 of stream b (or the caller's previous block).
template <typename T, int V>
__global__ __launch_bounds__(256) void compress_generic(
    const T* __restrict__ Ca, const T* __restrict__ Cb, const T* __restrict__ Za,
    const T* __restrict__ Zb, const T* __restrict__ Ba, const T* __restrict__ Bb,
    const T* __restrict__ pCb, const T* __restrict__ pZb, int64_t n, int c, int64_t m,
    int overlap, int P, T* __restrict__ out, int64_t obs) {
  __shared__ float sm_state[256 * 3 * V];
  const int CHB = 256 / P;
  const int tid = threadIdx.x;
  const int part = tid / CHB;
  const int cl = tid % CHB;
  const int64_t e = blockIdx.x;
  const int ch = blockIdx.y * CHB + cl;
  const int64_t s = blockIdx.z;
  const int CH = c / V;
  const bool active = ch < CH;
  const int d0 = ch * V;
  const int64_t seq = s * n * (int64_t)c;
  const bool hasb = overlap && ((e > 0) || (pZb != nullptr));
  const int64_t R = hasb ? 2 * m : m;

  float mx[V], sum[V], acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) { mx[v] = -INFINITY; sum[v] = 0.f; acc[v] = 0.f; }

  if (active) {
    for (int64_t r0 = part; r0 < R; r0 += 4 * (int64_t)P) {
      float z[4][V], cv[4][V], bv[4][V];
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t r = r0 + (int64_t)q * P;
        if (r < R) {
          const T *zp, *cp, *bp;
          if (r < m) {
            zp = Za + seq + (m * e + r) * (int64_t)c;
            cp = Ca + seq + (m * e + r) * (int64_t)c;
            bp = Ba + r * (int64_t)c;
          } else {
            const int64_t j = r - m;
            if (e > 0) {
              zp = Zb + seq + (m * (e - 1) + j) * (int64_t)c;
              cp = Cb + seq + (m * (e - 1) + j) * (int64_t)c;
            } else {
              zp = pZb + (s * m + j) * (int64_t)c;
              cp = pCb + (s * m + j) * (int64_t)c;
            }
            bp = Bb + j * (int64_t)c;
          }
          RowIO<T, V>::ld(zp + d0, z[q]);
          RowIO<T, V>::ld(cp + d0, cv[q]);
          RowIO<T, V>::ld(bp + d0, bv[q]);
          cnt = q + 1;
        }
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float bm = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < cnt) {
            z[q][v] += bv[q][v];
            bm = fmaxf(bm, z[q][v]);
          }
        const float nm = fmaxf(mx[v], bm);
        const float sc = fast_exp(mx[v] - nm);
        float sd = sum[v] * sc, ad = acc[v] * sc;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < cnt) {
            const float p = fast_exp(z[q][v] - nm);
            sd += p;
            ad = fmaf(p, cv[q][v], ad);
          }
        mx[v] = nm;
        sum[v] = sd;
        acc[v] = ad;
      }
    }
  }
  if (P > 1) {
    // publish this part's running state; part 0 merges parts 1..P-1 in order
    float* st = sm_state + (size_t)tid * 3 * V;
#pragma unroll
    for (int v = 0; v < V; ++v) { st[v] = mx[v]; st[V + v] = sum[v]; st[2 * V + v] = acc[v]; }
    __syncthreads();
    if (part == 0 && active) {
      for (int p = 1; p < P; ++p) {
        const float* o = sm_state + (size_t)(p * CHB + cl) * 3 * V;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const float om = o[v];
          if (om == -INFINITY) continue;  // that part saw no rows
          const float nm = fmaxf(mx[v], om);
          const float a = fast_exp(mx[v] - nm), b = fast_exp(om - nm);
          sum[v] = sum[v] * a + o[V + v] * b;
          acc[v] = acc[v] * a + o[2 * V + v] * b;
          mx[v] = nm;
        }
      }
    }
  }
  if (part == 0 && active) {
    float res[V];
#pragma unroll
    for (int v = 0; v < V; ++v) res[v] = acc[v] / sum[v];
    RowIO<T, V>::st(out + s * obs + e * (int64_t)c + d0, res);
  }
}

// ---------------------------------------------------------------------------
// Pooling compressor (no overlap), for blocks of many rows (HCA, m' = 128):
// one workgroup per entry and CPW channels of V values.  Thread t takes
// channel t % CPW and rows p, p+P, ... of the block (part p = t / CPW, P =
// 256 / CPW parts), so the lanes of a wave read whole contiguous row
// segments; NR rows per round are loaded together (row indices clamped, rows
// past the block weighted 0) before any is used, with one running max / sum
// / weighted sum per value.  The parts' states merge in part order through
// LDS.
// ---------------------------------------------------------------------------
template <typename T, int V, int NR, int CPW>
__global__ __launch_bounds__(256) void compress_pool(const T* __restrict__ C, const T* __restrict__ Z,
                                                     const T* __restrict__ B, int64_t n, int c, int64_t m,
                                                     T* __restrict__ out, int64_t obs) {
  constexpr int P = 256 / CPW;
  __shared__ float st[P - 1][3 * V][CPW];   // parts 1..P-1: max, sum, acc per value and channel
  const int part = threadIdx.x / CPW, cl = threadIdx.x % CPW;
  const int64_t e = blockIdx.x, s = blockIdx.z;
  const int ch = blockIdx.y * CPW + cl;
  const bool active = ch < c / V;
  const int d0 = (active ? ch : 0) * V;
  const T* zrow = Z + (s * n + m * e) * (int64_t)c + d0;
  const T* crow = C + (s * n + m * e) * (int64_t)c + d0;
  const T* brow = B + d0;
  float mx[V], sum[V], acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) { mx[v] = -INFINITY; sum[v] = 0.f; acc[v] = 0.f; }
  for (int64_t r0 = part; r0 < m; r0 += P * NR) {
    // the round's rows stay packed (16 bytes each) until they are used
    uint4 zr[NR], cr[NR], br[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      int64_t r = r0 + P * q;
      r = r < m ? r : m - 1;
      zr[q] = *reinterpret_cast<const uint4*>(zrow + r * (int64_t)c);
      cr[q] = *reinterpret_cast<const uint4*>(crow + r * (int64_t)c);
      br[q] = *reinterpret_cast<const uint4*>(brow + r * (int64_t)c);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float z[NR];
      float bm = mx[v];
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        z[q] = (r0 + P * q < m) ? Vec16<T>::get(zr[q], v) + Vec16<T>::get(br[q], v) : -INFINITY;
        bm = fmaxf(bm, z[q]);
      }
      const float sc = fast_exp(mx[v] - bm);   // bm is finite: row r0 < m exists
      float sd = sum[v] * sc, ad = acc[v] * sc;
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const float p = fast_exp(z[q] - bm);
        sd += p;
        ad = fmaf(p, Vec16<T>::get(cr[q], v), ad);
      }
      mx[v] = bm;
      sum[v] = sd;
      acc[v] = ad;
    }
  }
  if (part > 0) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      st[part - 1][v][cl] = mx[v];
      st[part - 1][V + v][cl] = sum[v];
      st[part - 1][2 * V + v][cl] = acc[v];
    }
  }
  __syncthreads();
  if (part == 0 && active) {
    for (int w = 0; w < P - 1; ++w) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float om = st[w][v][cl];
        if (om == -INFINITY) continue;   // that part saw no rows
        const float nm = fmaxf(mx[v], om);
        const float a = fast_exp(mx[v] - nm), b = fast_exp(om - nm);
        sum[v] = sum[v] * a + st[w][V + v][cl] * b;
        acc[v] = acc[v] * a + st[w][2 * V + v][cl] * b;
        mx[v] = nm;
      }
    }
    float res[V];
#pragma unroll
    for (int v = 0; v < V; ++v) res[v] = acc[v] / sum[v];
    RowIO<T, V>::st(out + s * obs + e * (int64_t)c + d0, res);
  }
}

}  // namespace csa

namespace csa {

constexpr int kOverlapWGsPerCU = 16;  // grid cap of the overlapped compressor: workgroups per CU
constexpr int kPoolChannels = 64;   // channels (of 16 bytes) per workgroup of the pooling kernel
constexpr int kPoolRows = 4;        // rows per thread and round

template <typename T>
static hipError_t launch_compress_t(const void* Ca, const void* Cb, const void* Za, const void* Zb,
                                    const void* Ba, const void* Bb, const void* pCb,
                                    const void* pZb, int64_t b, int64_t n, int64_t c, int64_t m,
                                    int overlap, void* out, int64_t obs, hipStream_t st) {
  const int64_t ne = n / m;
  if (ne == 0 || b == 0) return hipSuccess;
  constexpr int V = Vec16<T>::N;
  const T* ca = (const T*)Ca; const T* cb = (const T*)Cb;
  const T* za = (const T*)Za; const T* zb = (const T*)Zb;
  const T* ba = (const T*)Ba; const T* bb = (const T*)Bb;
  const T* pcb = (const T*)pCb; const T* pzb = (const T*)pZb;
  T* o = (T*)out;
  if (overlap && m == 4 && c % V == 0) {
    const int64_t total = b * ne * (c / V);
    // kOverlapWGsPerCU workgroups per CU of the 256, each thread looping over
    // the units of one channel
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * kOverlapWGsPerCU);
    hipLaunchKernelGGL((compress_overlap_fixed<T, 4>), dim3((unsigned)blocks), dim3(256), 0, st,
                       ca, cb, za, zb, ba, bb, pcb, pzb, n, (int)c, ne, total, o, obs);
    return hipGetLastError();
  }
  if (!overlap && m >= 32 && c % V == 0) {
    const int CH = (int)(c / V);
    constexpr int CPW = kPoolChannels;
    dim3 grid((unsigned)ne, (unsigned)((CH + CPW - 1) / CPW), (unsigned)b);
    hipLaunchKernelGGL((compress_pool<T, V, kPoolRows, CPW>), grid, dim3(256), 0, st, ca, za, ba, n, (int)c, m,
                       o, obs);
    return hipGetLastError();
  }
  // generic path: rows split over P parts of one workgroup
  const int64_t R = overlap ? 2 * m : m;
  int P = 1;
  while (P < 16 && (int64_t)P * 8 < R) P *= 2;
  const int CHB = 256 / P;
  if (c % V == 0) {
    const int CH = (int)(c / V);
    dim3 grid((unsigned)ne, (unsigned)((CH + CHB - 1) / CHB), (unsigned)b);
    hipLaunchKernelGGL((compress_generic<T, V>), grid, dim3(256), 0, st, ca, cb, za, zb, ba, bb,
                       pcb, pzb, n, (int)c, m, overlap, P, o, obs);
  } else {
    const int CH = (int)c;
    dim3 grid((unsigned)ne, (unsigned)((CH + CHB - 1) / CHB), (unsigned)b);
    hipLaunchKernelGGL((compress_generic<T, 1>), grid, dim3(256), 0, st, ca, cb, za, zb, ba, bb,
                       pcb, pzb, n, (int)c, m, overlap, P, o, obs);
  }
  return hipGetLastError();
}

hipError_t launch_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb,
                           const void* Ba, const void* Bb, const void* pCb, const void* pZb,
                           int64_t b, int64_t n, int64_t c, int64_t m, int overlap, int dtype,
                           void* out, int64_t obs, hipStream_t st) {
  if (dtype == 1)
    return launch_compress_t<bf16_t>(Ca, Cb, Za, Zb, Ba, Bb, pCb, pZb, b, n, c, m, overlap, out, obs, st);
  return launch_compress_t<float>(Ca, Cb, Za, Zb, Ba, Bb, pCb, pZb, b, n, c, m, overlap, out, obs, st);
}

}  // namespace csa
