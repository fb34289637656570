// Heterogeneous decode cache: per-request state cache plus a pool of
// classical-cache blocks (AirCoding "deepseek-paper-analysis" section 7.6,
// "Inference KV Cache").
//
// The state cache of a request has a fixed size: the sliding-window segment
// (the n_win most recent uncompressed rows of each layer, a ring indexed by
// position) and the compressor segments (the rows of each layer's open block
// waiting for compression, plus, for CSA, the stream-b rows of the previous
// block that the overlapped compressor needs).  The classical cache is a
// list of blocks per request, each covering lcm(m, m') tokens and holding
// lcm/m CSA entries, their lcm/m indexer keys and lcm/m' HCA entries.
//
// paged_append adds one token per batch row: it stores the token's rows in
// the state, and when the token completes a CSA block (every m tokens) or an
// HCA block (every m' tokens) it compresses that block -- the overlapped
// form of polysight "06-formulas" B9 / songhuiming "DeepSeek-V4 百万 token
// 上下文" section 4.1 for CSA entries and keys, the pooling form of section
// 5.1 for HCA -- and writes the entry into the request's block.  A thread
// owns the same 16-byte column slice of every row of a request in every
// launch, so the rows a compression reads were written by that thread (in
// this launch or an earlier one) and no synchronisation is needed.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// softmax over the rows' scores per dimension (scores Z + bias, values C)
// accumulated with a running maximum; `first` starts a new entry
struct ColSoftmax {
  float mx[8], sum[8], acc[8];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int v = 0; v < 8; ++v) { mx[v] = -INFINITY; sum[v] = 0.f; acc[v] = 0.f; }
  }
  __device__ __forceinline__ void add(const float (&z)[8], const float (&bias)[8], const float (&cv)[8]) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float s = z[v] + bias[v];
      const float nm = fmaxf(mx[v], s);
      const float a = fast_exp(mx[v] - nm);   // 0 while mx is -inf
      const float p = fast_exp(s - nm);
      sum[v] = sum[v] * a + p;
      acc[v] = acc[v] * a + p * cv[v];
      mx[v] = nm;
    }
  }
  __device__ __forceinline__ void result(float (&o)[8]) const {
#pragma unroll
    for (int v = 0; v < 8; ++v) o[v] = acc[v] / sum[v];
  }
};

__device__ __forceinline__ void ld8(const bf16_t* p, float (&o)[8]) { Vec16<bf16_t>::ld(p, o); }
__device__ __forceinline__ void st8(bf16_t* p, const float (&o)[8]) { Vec16<bf16_t>::st(p, o); }
__device__ __forceinline__ void cp8(bf16_t* d, const bf16_t* s) {
  *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
}

// One column slice (8 values) of one overlapped-compressor stream set: store
// the token's rows in the open block, and on block completion emit entry e
// from the open block (stream a) and the previous block (stream b; none for
// e = 0), then keep this block's stream-b rows as the next previous block.
__device__ __forceinline__ void overlap_slice(const bf16_t* Ca, const bf16_t* Cb, const bf16_t* Za,
                                              const bf16_t* Zb, const bf16_t* Ba, const bf16_t* Bb,
                                              bf16_t* open, bf16_t* prev, int width, int m, int64_t t,
                                              bf16_t* entry_out) {
  const int64_t blk = (int64_t)m * width;   // elements of one stream's open block
  const int slot = (int)(t % m);
  cp8(open + 0 * blk + slot * width, Ca);
  cp8(open + 1 * blk + slot * width, Cb);
  cp8(open + 2 * blk + slot * width, Za);
  cp8(open + 3 * blk + slot * width, Zb);
  if (entry_out == nullptr) return;
  const int64_t e = (t + 1) / m - 1;
  ColSoftmax sm;
  sm.reset();
  float z[8], bias[8], cv[8];
  for (int j = 0; j < m; ++j) {   // block e, stream a
    ld8(open + 2 * blk + j * width, z);
    ld8(Ba + j * width, bias);
    ld8(open + 0 * blk + j * width, cv);
    sm.add(z, bias, cv);
  }
  if (e > 0) {                    // block e - 1, stream b (block -1: nothing)
    for (int j = 0; j < m; ++j) {
      ld8(prev + 1 * blk + j * width, z);
      ld8(Bb + j * width, bias);
      ld8(prev + 0 * blk + j * width, cv);
      sm.add(z, bias, cv);
    }
  }
  float res[8];
  sm.result(res);
  st8(entry_out, res);
  for (int j = 0; j < m; ++j) {
    cp8(prev + 0 * blk + j * width, open + 1 * blk + j * width);
    cp8(prev + 1 * blk + j * width, open + 3 * blk + j * width);
  }
}

__global__ __launch_bounds__(256) void paged_append(
    bf16_t* __restrict__ state, PagedState L, bf16_t* __restrict__ pool, Rows csa_rows, Rows key_rows,
    Rows hca_rows, const int64_t* __restrict__ pos, const bf16_t* __restrict__ Ca, const bf16_t* __restrict__ Cb,
    const bf16_t* __restrict__ Za, const bf16_t* __restrict__ Zb, const bf16_t* __restrict__ ICa,
    const bf16_t* __restrict__ ICb, const bf16_t* __restrict__ IZa, const bf16_t* __restrict__ IZb,
    const bf16_t* __restrict__ Ch, const bf16_t* __restrict__ Zh, const bf16_t* __restrict__ Ba,
    const bf16_t* __restrict__ Bb, const bf16_t* __restrict__ IBa, const bf16_t* __restrict__ IBb,
    const bf16_t* __restrict__ Bh) {
  const int64_t r = blockIdx.x;
  const int64_t t = pos[r];
  bf16_t* S = state + csa_rows.req(r) * L.stride;
  const int c = L.c, cI = L.c_I, m = L.m, mp = L.m_prime;
  const bool csa_done = (t + 1) % m == 0;
  const bool hca_done = (t + 1) % mp == 0;
  const int nc = c / 8, nci = cI / 8;
  for (int u = threadIdx.x; u < 2 * nc + nci; u += blockDim.x) {
    if (u < nc) {
      // CSA main streams and the CSA window row (C^a)
      const int d = 8 * u;
      const int64_t ro = r * c + d;
      cp8(S + L.csa_win + (t % L.n_win) * c + d, Ca + ro);
      bf16_t* eo = csa_done ? pool + csa_rows.at(r, (t + 1) / m - 1, c) + d : nullptr;
      overlap_slice(Ca + ro, Cb + ro, Za + ro, Zb + ro, Ba + d, Bb + d, S + L.csa_open + d, S + L.csa_prev + d, c,
                    m, t, eo);
    } else if (u < 2 * nc) {
      // HCA stream (its window row is C) and the pooling compressor
      const int d = 8 * (u - nc);
      const int64_t ro = r * c + d;
      cp8(S + L.hca_win + (t % L.n_win) * c + d, Ch + ro);
      const int64_t blk = (int64_t)mp * c;
      cp8(S + L.hca_open + (t % mp) * c + d, Ch + ro);
      cp8(S + L.hca_open + blk + (t % mp) * c + d, Zh + ro);
      if (hca_done) {
        ColSoftmax sm;
        sm.reset();
        float z[8], bias[8], cv[8];
        for (int j = 0; j < mp; ++j) {
          ld8(S + L.hca_open + blk + j * c + d, z);
          ld8(Bh + j * c + d, bias);
          ld8(S + L.hca_open + j * c + d, cv);
          sm.add(z, bias, cv);
        }
        float res[8];
        sm.result(res);
        st8(pool + hca_rows.at(r, (t + 1) / mp - 1, c) + d, res);
      }
    } else {
      // indexer-key streams
      const int d = 8 * (u - 2 * nc);
      const int64_t ro = r * cI + d;
      bf16_t* eo = csa_done ? pool + key_rows.at(r, (t + 1) / m - 1, cI) + d : nullptr;
      overlap_slice(ICa + ro, ICb + ro, IZa + ro, IZb + ro, IBa + d, IBb + d, S + L.key_open + d,
                    S + L.key_prev + d, cI, m, t, eo);
    }
  }
}

hipError_t launch_paged_append(void* state, const PagedState& L, void* pool, const Rows& csa_rows,
                               const Rows& key_rows, const Rows& hca_rows, const int64_t* pos, int64_t b,
                               const void* const* tok, const void* const* bias, hipStream_t st) {
  if (b == 0) return hipSuccess;
  const bf16_t* const* T = (const bf16_t* const*)tok;
  const bf16_t* const* Bs = (const bf16_t* const*)bias;
  hipLaunchKernelGGL(paged_append, dim3((unsigned)b), dim3(256), 0, st, (bf16_t*)state, L, (bf16_t*)pool,
                     csa_rows, key_rows, hca_rows, pos, T[0], T[1], T[2], T[3], T[4], T[5], T[6], T[7], T[8], T[9],
                     Bs[0], Bs[1], Bs[2], Bs[3], Bs[4]);
  return hipGetLastError();
}

}  // namespace csa
