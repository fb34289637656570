// Device helpers shared by the CSA/HCA kernels (gfx950 / CDNA4).
#pragma once

// CSA_DEBUG=1 builds the bounds-checked debug library (libcsa_debug.so).
#ifndef CSA_DEBUG
#define CSA_DEBUG 0
#endif
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

typedef uint16_t bf16_t;
typedef uint8_t fp8_t;   // OCP E4M3 code

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// float32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Scalar element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
};
// 8-bit E4M3 (OCP), read only: the hardware conversion decodes every code
// exactly (NaN codes to NaN).
template <> struct Elem<fp8_t> {
  static __device__ __forceinline__ float ld(const fp8_t* p) { return __builtin_amdgcn_cvt_f32_fp8((int)*p, 0); }
};

// 16-byte vector loads/stores: VEC = 16 / sizeof(T) elements widened to float.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  // element i of a 16-byte vector loaded raw
  static __device__ __forceinline__ float get(const uint4& r, int i) {
    return __uint_as_float(i == 0 ? r.x : i == 1 ? r.y : i == 2 ? r.z : r.w);
  }
  static __device__ __forceinline__ void ld(const float* p, float (&o)[4]) {
    float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  static __device__ __forceinline__ void st(float* p, const float (&o)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ float get(const uint4& r, int i) {
    const uint32_t w = (i >> 1) == 0 ? r.x : (i >> 1) == 1 ? r.y : (i >> 1) == 2 ? r.z : r.w;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  static __device__ __forceinline__ void ld(const bf16_t* p, float (&o)[8]) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void st(bf16_t* p, const float (&o)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(o[2 * i]) | ((uint32_t)f2bf(o[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// Order-preserving map float32 -> uint32 (larger float <=> larger key).
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Wave-wide (64-lane) sum / max with a fixed butterfly order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Position of query row r of batch row s: t0 + r for one block of
// consecutive queries shared by the batch, or pos[s] + r when every batch row
// carries a position of its own (variable-length batched decode).
struct QPos {
  int64_t t0;
  const int64_t* pos;
  __device__ __forceinline__ int64_t at(int64_t s, int64_t r) const { return (pos ? pos[s] : t0) + r; }
};

// Where row i of one cached array (compressed entries, indexer keys, HCA
// entries) of batch row s lives.  Dense: at s * bstride + i * rowlen
// elements.  Paged: row i sits in block table[req(s)][i >> pb_log2] (clamped
// into [0, n_blocks)), at off + (i & (per_block - 1)) * rowlen elements from
// that block's start; req(s) maps a batch row to its request slot.
struct Rows {
  int64_t bstride;
  const int32_t* table;
  const int32_t* slot;
  int64_t table_stride, blk_elems, off, n_blocks;
  int pb_log2;
  __device__ __forceinline__ int64_t req(int64_t s) const { return slot ? (int64_t)slot[s] : s; }
  __device__ __forceinline__ int64_t at(int64_t s, int64_t i, int64_t rowlen) const {
    if (table == nullptr) return s * bstride + i * rowlen;
    int64_t b = table[req(s) * table_stride + (i >> pb_log2)];
    b = b < 0 ? 0 : (b >= n_blocks ? n_blocks - 1 : b);
    return b * blk_elems + off + (i & ((1 << pb_log2) - 1)) * rowlen;
  }
};

inline Rows dense_rows(int64_t bstride) { return Rows{bstride, nullptr, nullptr, 0, 0, 0, 1, 0}; }

}  // namespace csa
