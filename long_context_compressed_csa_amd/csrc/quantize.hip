// OCP MXFP4 encoding of rows of values, for the indexer's FP4 query/key path
// (songhuiming "DeepSeek-V4 百万 token 上下文" section 13.3; AirCoding
// "deepseek-paper-analysis" section 7, FP4 quantization-aware training).
//
// OCP Microscaling Formats (MX) specification v1.0, conversion to an MX
// format: each block of 32 consecutive values takes the shared E8M0 scale
// X = 2^(floor(log2 max|v|) - 2), 2 being the largest E2M1 exponent; each
// value v / X is rounded to the nearest E2M1 magnitude (0, 0.5, 1, 1.5, 2, 3,
// 4, 6), ties to the even code, and saturated at 6.  An all-zero block gets
// scale byte 0; the sign bit is set for v < 0 also when the magnitude rounds
// to 0.  Codes are packed two per byte, element 2j in the low nibble of byte
// j.  X is a power of two, so v / X is exact and so is every decision.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// E2M1 magnitude code of y >= 0: the number of midpoints below y, where a
// value on the midpoint after an odd code (0.75, 1.75, 3.5) rounds up to the
// even code and one on any other midpoint rounds down; 7 above 5 (saturated)
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  return (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) + (uint32_t)(y >= 1.75f) +
         (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) + (uint32_t)(y > 5.0f);
}

template <typename T> struct Block32;
template <> struct Block32<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[32]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
  }
};
template <> struct Block32<float> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[32]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 u = reinterpret_cast<const float4*>(p)[q];
      v[4 * q] = u.x;
      v[4 * q + 1] = u.y;
      v[4 * q + 2] = u.z;
      v[4 * q + 3] = u.w;
    }
  }
};

// One thread per block of 32 values (consecutive threads take consecutive
// blocks of a row), grid-stride over rows x c/32 blocks.
template <typename T>
__global__ __launch_bounds__(256) void quantize_mxfp4(const T* __restrict__ x, int64_t xrs, int64_t rows, int nb,
                                                      uint8_t* __restrict__ codes, int64_t crs,
                                                      uint8_t* __restrict__ scales, int64_t srs) {
  const int64_t total = rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / nb;
    const int bl = (int)(i % nb);
    float v[32];
    Block32<T>::load(x + r * xrs + 32 * bl, v);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    int e = -127;
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);   // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
      e = max(ex - 3, -127);
    }
    const float inv = ldexpf(1.f, -e);   // 1 / X, a power of two within float range
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t c = e2m1_code(fabsf(v[j]) * inv) | (v[j] < 0.f ? 8u : 0u);
      w[j >> 3] |= c << (4 * (j & 7));
    }
    *reinterpret_cast<uint4*>(codes + r * crs + 16 * bl) = make_uint4(w[0], w[1], w[2], w[3]);
    scales[r * srs + bl] = (uint8_t)(e + 127);
  }
}

hipError_t launch_quantize_mxfp4(const void* x, int64_t xrs, int64_t rows, int64_t c, int dtype, void* codes,
                                 int64_t crs, void* scales, int64_t srs, hipStream_t st) {
  const int nb = (int)(c / 32);
  const int64_t total = rows * nb;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 16);
  if (dtype == 1)
    hipLaunchKernelGGL(quantize_mxfp4<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, st, (const bf16_t*)x, xrs,
                       rows, nb, (uint8_t*)codes, crs, (uint8_t*)scales, srs);
  else
    hipLaunchKernelGGL(quantize_mxfp4<float>, dim3((unsigned)blocks), dim3(256), 0, st, (const float*)x, xrs,
                       rows, nb, (uint8_t*)codes, crs, (uint8_t*)scales, srs);
  return hipGetLastError();
}

}  // namespace csa
