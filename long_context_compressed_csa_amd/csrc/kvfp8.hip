// Mixed-precision KV entries (AirCoding "deepseek-paper-analysis" section
// 7.3, KV mixed precision storage; polysight "06-formulas" B9): the RoPE
// dimensions of a compressed entry stay BF16, the others are stored as FP8.
// Layout of n entries of c dims with r RoPE dims (the last r):
//   codes [n][c - r] uint8   OCP E4M3 codes of x / scale
//   rope  [n][r]     bf16    the RoPE dims as given
//   scale [n]        float32 one power of two per entry: the smallest 2^e
//                            with max |x| / 2^e <= 448 (the E4M3 maximum);
//                            2^0 for an all-zero entry
// quantize_kv_fp8 encodes (round to nearest even); the attention reads the
// entries back through dequant_* kernels that gather the entries one call
// reads -- all of them for a block of queries, the selected ones for a
// single query -- into bf16 rows (exact: an E4M3 value times a power of two
// has at most 4 significant bits), then runs the bf16 attention on them.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// E4M3 code of a finite |v| <= 448, round to nearest even, sign kept.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0x1p-6f) {
    // subnormals (and zero): multiples of 2^-9; 8 * 2^-9 is the smallest normal
    code = (uint32_t)rintf(a * 0x1p9f);
  } else {
    int e;
    const float mant = frexpf(a, &e) * 2.f;   // a = mant * 2^(e-1), mant in [1, 2)
    int ex = e - 1;
    float f = rintf((mant - 1.f) * 8.f);       // exact products; rintf ties to even
    if (f == 8.f) { f = 0.f; ++ex; }
    code = (uint32_t)((ex + 7) << 3) | (uint32_t)f;
  }
  return sign | code;
}

// E4M3 value (finite codes)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, f = c & 7;
  const float mag = e == 0 ? (float)f * 0x1p-9f : ldexpf(1.f + (float)f * 0.125f, (int)e - 7);
  return (c & 0x80) ? -mag : mag;
}

// One wave per row: scale from the row's largest magnitude, then codes.
template <typename T>
__global__ __launch_bounds__(256) void quantize_kv_fp8(const T* __restrict__ x, int64_t xrs, int64_t rows, int c,
                                                       int r, uint8_t* __restrict__ codes, int64_t crs,
                                                       bf16_t* __restrict__ rope, int64_t rrs,
                                                       float* __restrict__ scale) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= rows) return;
  const T* xr = x + row * xrs;
  const int h = c - r;
  float amax = 0.f;
  for (int d = l; d < h; d += 64) amax = fmaxf(amax, fabsf(Elem<T>::ld(xr + d)));
  amax = wave_max(amax);
  // smallest e with amax <= 448 * 2^e (448 = 1.75 * 2^8)
  int e = 0;
  if (amax > 0.f) {
    int ea;
    const float mant = frexpf(amax, &ea) * 2.f;   // amax = mant * 2^(ea-1)
    e = (ea - 1) - 8 + (mant > 1.75f ? 1 : 0);
  }
  const float inv = ldexpf(1.f, -e);
  if (l == 0) scale[row] = ldexpf(1.f, e);
  for (int d = l; d < h; d += 64) codes[row * crs + d] = (uint8_t)e4m3_rne(Elem<T>::ld(xr + d) * inv);
  for (int d = l; d < r; d += 64) rope[row * rrs + d] = f2bf(Elem<T>::ld(xr + h + d));
}

// 8 consecutive values (chunk ch) of a stored entry, decoded to bf16: the
// codes part and the RoPE part are both multiples of 8 values long
__device__ __forceinline__ void dequant_chunk(const uint8_t* __restrict__ cr, const bf16_t* __restrict__ rr, float sc,
                                              int h, int ch, bf16_t* __restrict__ out) {
  const int d = 8 * ch;
  if (d < h) {
    const uint2 w = *reinterpret_cast<const uint2*>(cr + d);
    float v[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = e4m3_value((w.x >> (8 * u)) & 255u) * sc;
      v[4 + u] = e4m3_value((w.y >> (8 * u)) & 255u) * sc;
    }
    Vec16<bf16_t>::st(out + d, v);
  } else {
    *reinterpret_cast<uint4*>(out + d) = *reinterpret_cast<const uint4*>(rr + (d - h));
  }
}

// all entries of every sequence into [b][n_comp][c]: one thread per chunk
__global__ __launch_bounds__(256) void dequant_all(const uint8_t* __restrict__ codes, const bf16_t* __restrict__ rope,
                                                   const float* __restrict__ scale, int64_t cbs, int64_t n_comp, int c,
                                                   int r, bf16_t* __restrict__ out) {
  const int nch = c / 8;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t bi = blockIdx.y;
  if (u >= n_comp * nch) return;
  const int64_t e = u / nch;
  const int ch = (int)(u % nch);
  const int64_t row = bi * cbs + e;
  dequant_chunk(codes + row * (c - r), rope + row * r, scale[row], c - r, ch, out + (bi * n_comp + e) * (int64_t)c);
}

// One query per sequence: its valid selected entries (0 <= s < (t0+1)/m),
// compacted in list order, into [b][k][c]; idx2 [b][k] = 0 .. nv-1, then
// -1.  A workgroup takes 16 list slots; it counts the valid slots before
// its own and in the whole row, then decodes its entries chunk-parallel.
constexpr int kDqSlots = 16;
__global__ __launch_bounds__(256) void dequant_selected(const uint8_t* __restrict__ codes,
                                                        const bf16_t* __restrict__ rope,
                                                        const float* __restrict__ scale, int64_t cbs,
                                                        const int32_t* __restrict__ idx, int64_t k, int64_t t0,
                                                        int64_t n_comp, int64_t m, int c, int r,
                                                        bf16_t* __restrict__ out, int32_t* __restrict__ idx2) {
  __shared__ int32_t red[2][4];
  __shared__ int32_t s_ent[kDqSlots];
  __shared__ int32_t s_pos[kDqSlots];
  const int64_t bi = blockIdx.x;
  const int64_t j0 = (int64_t)blockIdx.y * kDqSlots;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  int64_t vis = (t0 + 1) / m;
  if (vis > n_comp) vis = n_comp;
  const int32_t* ir = idx + bi * k;
  int before = 0, total = 0;
  for (int64_t j = tid; j < k; j += 256) {
    const int32_t s = ir[j];
    const int ok = s >= 0 && s < vis;
    total += ok;
    before += (ok && j < j0) ? 1 : 0;
  }
  before = (int)wave_sum_u32((uint32_t)before);
  total = (int)wave_sum_u32((uint32_t)total);
  if (l == 0) { red[0][w] = before; red[1][w] = total; }
  __syncthreads();
  before = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  total = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  if (w == 0) {
    const int64_t j = j0 + l;
    const int32_t s = (l < kDqSlots && j < k) ? ir[j] : -1;
    const bool ok = s >= 0 && s < vis;
    const uint64_t mk = __builtin_amdgcn_ballot_w64(ok);
    const int pos = before + __popcll(mk & ((l == 0) ? 0ull : (~0ull >> (64 - l))));
    if (l < kDqSlots) {
      s_ent[l] = ok ? s : -1;
      s_pos[l] = pos;
      if (ok) idx2[bi * k + pos] = pos;
      if (j < k && j >= total) idx2[bi * k + j] = -1;
    }
  }
  __syncthreads();
  const int nch = c / 8;
  for (int u = tid; u < kDqSlots * nch; u += 256) {
    const int e = u / nch, ch = u % nch;
    const int32_t s = s_ent[e];
    if (s < 0) continue;
    const int64_t row = bi * cbs + s;
    dequant_chunk(codes + row * (c - r), rope + row * r, scale[row], c - r, ch, out + (bi * k + s_pos[e]) * (int64_t)c);
  }
}

hipError_t launch_quantize_kv_fp8(const void* x, int64_t xrs, int64_t rows, int64_t c, int64_t r, int dtype,
                                  void* codes, int64_t crs, void* rope, int64_t rrs, float* scale, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (dtype == 1)
    hipLaunchKernelGGL(quantize_kv_fp8<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)x, xrs, rows, (int)c,
                       (int)r, (uint8_t*)codes, crs, (bf16_t*)rope, rrs, scale);
  else
    hipLaunchKernelGGL(quantize_kv_fp8<float>, dim3(grid), dim3(256), 0, st, (const float*)x, xrs, rows, (int)c,
                       (int)r, (uint8_t*)codes, crs, (bf16_t*)rope, rrs, scale);
  return hipGetLastError();
}

// Selected-entry mode for one query per sequence when the sequences hold
// more entries than they select; every entry otherwise.
static bool fp8kv_selected_mode(int64_t n_q, int64_t n_comp, int64_t k) { return n_q == 1 && n_comp > k; }

size_t attend_fp8kv_workspace_bytes(int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h, int64_t c,
                                    int64_t k, int64_t m, int64_t n_win) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  if (fp8kv_selected_mode(n_q, n_comp, k)) {
    const size_t att = attend_workspace_bytes(1, b, n_q, n_h, c, k + n_win);
    return al((size_t)b * k * c * 2) + al((size_t)b * k * 4) + att;
  }
  int64_t vmax = (t0 + n_q) / m;
  if (vmax > n_comp) vmax = n_comp;
  return al((size_t)b * n_comp * c * 2) + attend_workspace_bytes(1, b, n_q, n_h, c, k + n_win);
}

hipError_t launch_attend_fp8kv(const void* q, const void* codes, const void* rope, const float* scale, int64_t cbs,
                               const int32_t* idx, const void* kv_raw, int64_t rbs, int64_t raw_pos0,
                               const float* sink, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h,
                               int64_t c, int64_t r, int64_t k, int64_t m, int64_t n_win, float sc, void* ws,
                               void* out, hipStream_t st) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  unsigned char* W = (unsigned char*)ws;
  if (fp8kv_selected_mode(n_q, n_comp, k)) {
    bf16_t* ent = (bf16_t*)W;
    int32_t* idx2 = (int32_t*)(W + al((size_t)b * k * c * 2));
    void* aws = W + al((size_t)b * k * c * 2) + al((size_t)b * k * 4);
    hipLaunchKernelGGL(dequant_selected, dim3((unsigned)b, (unsigned)((k + kDqSlots - 1) / kDqSlots)), dim3(256), 0,
                       st, (const uint8_t*)codes,
                       (const bf16_t*)rope, scale, cbs, idx, k, t0, n_comp, m, (int)c, (int)r, ent, idx2);
    // the gathered entries are entries 0 .. k-1 of a k-entry cache, all
    // complete for the query (their number is at most its visible count)
    return launch_attend(0, q, ent, k * c, idx2, kv_raw, rbs, raw_pos0, sink, b, n_q, t0, k, n_h, c, k, 1, n_win,
                         sc, 1, aws, out, st);
  }
  bf16_t* ent = (bf16_t*)W;
  void* aws = W + al((size_t)b * n_comp * c * 2);
  if (n_comp > 0)
    hipLaunchKernelGGL(dequant_all, dim3((unsigned)((n_comp * (c / 8) + 255) / 256), (unsigned)b), dim3(256), 0, st,
                       (const uint8_t*)codes, (const bf16_t*)rope, scale, cbs, n_comp, (int)c, (int)r, ent);
  return launch_attend(0, q, ent, n_comp * c, idx, kv_raw, rbs, raw_pos0, sink, b, n_q, t0, n_comp, n_h, c, k, m,
                       n_win, sc, 1, aws, out, st);
}

}  // namespace csa
