// Shared key/value multi-query attention with sliding window and sink, for
// CSA (selected compressed entries) and HCA (every completed entry).
//
// Definition: AirCoding "deepseek-paper-analysis" section 7.1 (each
// compressed entry is both key and value, all query heads share it);
// songhuiming "DeepSeek-V4 百万 token 上下文" sections 4.5 and 7.2-7.3 (the
// window of the n_win most recent raw entries joins the compressed entries
// in one softmax, whose denominator also holds exp of a learned per-head
// sink logit); section 5.2 and polysight "06-formulas" B9 for the dense HCA
// read.
//
// MFMA path (bf16, 64 heads x c = 512): one workgroup per (query, 64-head
// group, entry split).  The four waves split the 512 dimensions: wave w
// holds q[:, 128w:128w+128] in registers and owns O[:, 128w:128w+128] in
// accumulators.  Per tile of 32 entries each wave gathers its 128-dim slice
// of the 32 rows straight from global memory into MFMA B registers (S = Q E^T
// needs entries with dimensions contiguous, which is how they are stored),
// the four partial S tiles are summed through LDS, the wave that owns a head
// runs the online softmax for it, and P V uses each wave's own slice of the
// tile re-read from LDS with rows as the contraction index.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// ---------------------------------------------------------------------------
// Generic path: any dtype, head count and c <= 1024.  One workgroup per
// (query, head); 256 entries per chunk, online softmax across chunks.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attend_generic(
    const T* __restrict__ q, const T* __restrict__ Ccomp, int64_t cbs,
    const int32_t* __restrict__ idx, const T* __restrict__ kv_raw, int64_t rbs, int64_t raw_pos0,
    const float* __restrict__ sink, int64_t n_q, int64_t t0, int64_t n_comp, int n_h, int c,
    int64_t k, int64_t m, int64_t n_win, float scale, int dense, T* __restrict__ out) {
  __shared__ float qs[1024];
  __shared__ float ps[256];
  __shared__ const T* rows[256];
  __shared__ float red[4];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int64_t r = blockIdx.x, bi = blockIdx.z;
  const int h = blockIdx.y;
  const int64_t t = t0 + r;
  int64_t vis = (t + 1) / m;
  if (vis > n_comp) vis = n_comp;
  const int64_t nsel = dense ? vis : k;
  const int64_t wlo = t - n_win + 1 > 0 ? t - n_win + 1 : 0;
  const int64_t N = nsel + (t - wlo + 1);
  const T* qrow = q + ((bi * n_q + r) * n_h + h) * (int64_t)c;
  for (int d = tid; d < c; d += 256) qs[d] = Elem<T>::ld(qrow + d);
  float M = -INFINITY, Lsum = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int64_t j0 = 0; j0 < N; j0 += 256) {
    const int64_t j = j0 + tid;
    float logit = -INFINITY;
    const T* row = nullptr;
    if (j < N) {
      if (j < nsel) {
        const int64_t s = dense ? j : (int64_t)idx[(bi * n_q + r) * k + j];
        if (s >= 0 && s < vis) row = Ccomp + bi * cbs + s * (int64_t)c;
      } else {
        row = kv_raw + bi * rbs + (wlo + (j - nsel) - raw_pos0) * (int64_t)c;
      }
      if (row) {
        float d = 0.f;
        for (int x = 0; x < c; ++x) d = fmaf(qs[x], Elem<T>::ld(row + x), d);
        logit = scale * d;
      }
    }
    rows[tid] = row;
    float cm = wave_max(logit);
    if (l == 0) red[wave] = cm;
    __syncthreads();
    cm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float nm = fmaxf(M, cm);
    __syncthreads();
    if (nm == -INFINITY) continue;  // nothing valid yet (uniform)
    const float p = row ? fast_exp(logit - nm) : 0.f;
    ps[tid] = p;
    float cs = wave_sum(p);
    if (l == 0) red[wave] = cs;
    __syncthreads();
    cs = (red[0] + red[1]) + (red[2] + red[3]);
    const float alpha = fast_exp(M - nm);
    Lsum = Lsum * alpha + cs;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    const int cnt = (int)(N - j0 < 256 ? N - j0 : 256);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = ps[jj];
      const T* rj = rows[jj];
      if (pj == 0.f || rj == nullptr) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = tid + 256 * i;
        if (d < c) acc[i] = fmaf(pj, Elem<T>::ld(rj + d), acc[i]);
      }
    }
    M = nm;
    __syncthreads();
  }
  const float z = sink[h];
  T* orow = out + ((bi * n_q + r) * n_h + h) * (int64_t)c;
  const float Mf = fmaxf(M, z);
  const float fac = (M == -INFINITY) ? 0.f : fast_exp(M - Mf);
  const float den = Lsum * fac + fast_exp(z - Mf);
  const float g = fac / den;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = tid + 256 * i;
    if (d < c) Elem<T>::st(orow + d, acc[i] * g);
  }
}

// ---------------------------------------------------------------------------
// MFMA path.  Layout constants for one workgroup (4 waves, 64 heads, c=512).
// ---------------------------------------------------------------------------
constexpr int kC = 512;
constexpr int kHG = 64;              // heads per workgroup
constexpr int kDW = kC / 4;          // dimensions per wave (128)
constexpr int kT = 32;               // entries per tile
constexpr int kERow = kDW * 2 + 8;   // LDS row of a wave's E slice, bytes (264)
constexpr int kSStr = 33;            // S partial row stride, floats
constexpr int kPRow = kT * 2 + 16;   // P row (one head), bytes (80)
constexpr int kMaxSel = 2048;        // selected entries staged in LDS

struct AttnSmem {
  unsigned char E[4][kT * kERow];        // 33 KiB
  float S[4][kHG * kSStr];               // 33 KiB
  unsigned char P[kHG * kPRow];          // 5 KiB
  float alpha[kHG];
  float fin[kHG];
  int32_t sel[kMaxSel];                  // 8 KiB
  int32_t nsel_part[4];
};

template <int DENSE>
__global__ __launch_bounds__(256) void attend_mfma_c512(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Ccomp, int64_t cbs,
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ kv_raw, int64_t rbs,
    int64_t raw_pos0, const float* __restrict__ sink, int64_t n_q, int64_t t0, int64_t n_comp,
    int n_h, int64_t k, int64_t m, int64_t n_win, float scale, int nsplit,
    float* __restrict__ part_o, float* __restrict__ part_ml, bf16_t* __restrict__ out) {
  __shared__ AttnSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int64_t r = (int64_t)gridDim.x - 1 - blockIdx.x;   // later queries (more work) first
  const int hg = blockIdx.y / nsplit;
  const int split = blockIdx.y % nsplit;
  const int64_t bi = blockIdx.z;
  const int64_t t = t0 + r;
  int64_t vis = (t + 1) / m;
  if (vis > n_comp) vis = n_comp;
  const int64_t wlo = t - n_win + 1 > 0 ? t - n_win + 1 : 0;
  const int64_t nwin = t - wlo + 1;

  // ---- entry list: selected compressed rows (compacted), then window rows
  int64_t nsel;
  if (DENSE) {
    nsel = vis;
  } else {
    // stable compaction of valid indices (0 <= s < vis) in list order
    const int32_t* ir = idx + (bi * n_q + r) * k;
    int64_t base = 0;
    for (int64_t j0 = 0; j0 < k; j0 += 256) {
      const int64_t j = j0 + tid;
      const int32_t s = j < k ? ir[j] : -1;
      const bool ok = s >= 0 && s < vis;
      const uint64_t mk = __ballot(ok);
      if (l == 0) sm.nsel_part[wave] = __popcll(mk);
      __syncthreads();
      int64_t pos = base;
      for (int w2 = 0; w2 < wave; ++w2) pos += sm.nsel_part[w2];
      pos += __popcll(mk & ((l == 0) ? 0ull : (~0ull >> (64 - l))));
      if (ok && pos < kMaxSel) sm.sel[pos] = s;
      base += sm.nsel_part[0] + sm.nsel_part[1] + sm.nsel_part[2] + sm.nsel_part[3];
      __syncthreads();
    }
    nsel = base < kMaxSel ? base : kMaxSel;
  }
  const int64_t N = nsel + nwin;
  // this split's entry range
  const int64_t per = (N + nsplit - 1) / nsplit;
  const int64_t jb = split * per;
  const int64_t je = jb + per < N ? jb + per : N;

  // ---- query operand: heads 64*hg + 32*mb + l%32, dims 128*wave + 16*ks + 8*(l/32)
  bf16x8 qa[2][8];
  {
    const bf16_t* qb = q + ((bi * n_q + r) * n_h + kHG * hg) * (int64_t)kC + kDW * wave + 8 * (l >> 5);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qa[mb][ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(qb + (mb * 32 + (l & 31)) * (int64_t)kC + ks * 16));
  }
  f32x16 o[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) o[mb][nb] = (f32x16){};

  // softmax state of head 16*wave + l/4 (replicated over 4 lanes)
  float m_run = -INFINITY, l_run = 0.f;
  const int own_h = 16 * wave + (l >> 2);
  const int own_r0 = (l & 3) * 8;

  const bf16_t* cbase = Ccomp + bi * cbs;
  const bf16_t* rbase = kv_raw + bi * rbs + (wlo - raw_pos0) * (int64_t)kC;
  unsigned char* Ew = sm.E[wave];

  for (int64_t j0 = jb; j0 < je; j0 += kT) {
    // (a) row of entry j0 + l%32
    const int64_t j = j0 + (l & 31);
    const bool jvalid = j < je;
    const int64_t jc = jvalid ? j : jb;   // any valid entry for padding lanes
    const bf16_t* row = jc < nsel ? cbase + (int64_t)(DENSE ? jc : sm.sel[jc]) * kC
                                  : rbase + (jc - nsel) * (int64_t)kC;
    row += kDW * wave + 8 * (l >> 5);
    // (b) B operand of S: 8 k-steps x 8 dims of that row
    bf16x8 eb[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      eb[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + ks * 16));
    // (c) partial S over this wave's 128 dims
    f32x16 sacc[2];
    sacc[0] = (f32x16){};
    sacc[1] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][ks], eb[ks], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][ks], eb[ks], sacc[1], 0, 0, 0);
    }
    // (d) keep the slice in LDS for P V (row-major, 8-byte stores)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 v = __builtin_bit_cast(uint4, eb[ks]);
      uint2* dst = reinterpret_cast<uint2*>(Ew + (l & 31) * kERow + (ks * 16 + 8 * (l >> 5)) * 2);
      dst[0] = make_uint2(v.x, v.y);
      dst[1] = make_uint2(v.z, v.w);
    }
    // (e) partial S to LDS: S[w][head][entry]
    {
      float* Sw = sm.S[wave];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int head = mb * 32 + 8 * (rr >> 2) + 4 * (l >> 5) + (rr & 3);
          Sw[head * kSStr + (l & 31)] = sacc[mb][rr];
        }
    }
    __syncthreads();
    // (g) online softmax for the 16 heads this wave owns
    {
      float s[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = own_r0 + i;
        float v = sm.S[0][own_h * kSStr + e] + sm.S[1][own_h * kSStr + e];
        v += sm.S[2][own_h * kSStr + e] + sm.S[3][own_h * kSStr + e];
        s[i] = (j0 + e < je) ? v * scale : -INFINITY;
      }
      float tm = s[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tm = fmaxf(tm, s[i]);
      tm = fmaxf(tm, __shfl_xor(tm, 1, 64));
      tm = fmaxf(tm, __shfl_xor(tm, 2, 64));
      const float m_new = fmaxf(m_run, tm);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp(m_run - m_new);
      float rs = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float p0 = (s[i] == -INFINITY) ? 0.f : fast_exp(s[i] - m_new);
        const float p1 = (s[i + 1] == -INFINITY) ? 0.f : fast_exp(s[i + 1] - m_new);
        const uint16_t b0 = f2bf(p0), b1 = f2bf(p1);
        // the row sum uses the rounded weights that P V multiplies
        rs += bf2f(b0) + bf2f(b1);
        pk[i / 2] = (uint32_t)b0 | ((uint32_t)b1 << 16);
      }
      rs += __shfl_xor(rs, 1, 64);
      rs += __shfl_xor(rs, 2, 64);
      l_run = l_run * alpha + rs;
      m_run = m_new;
      *reinterpret_cast<uint4*>(sm.P + own_h * kPRow + own_r0 * 2) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      if ((l & 3) == 0) sm.alpha[own_h] = alpha;
    }
    __syncthreads();
    // (i) rescale O, then O += P E over this wave's dims
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = *reinterpret_cast<const float4*>(&sm.alpha[mb * 32 + 8 * g + 4 * (l >> 5)]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          o[mb][nb][4 * g + 0] *= a.x;
          o[mb][nb][4 * g + 1] *= a.y;
          o[mb][nb][4 * g + 2] *= a.z;
          o[mb][nb][4 * g + 3] *= a.w;
        }
      }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      bf16x8 pa[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        pa[mb] = *reinterpret_cast<const bf16x8*>(sm.P + (mb * 32 + (l & 31)) * kPRow + (ks2 * 16 + 8 * (l >> 5)) * 2);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        // B[k = entry][n = dim]: 8 consecutive entries of one dimension
        const unsigned char* src = Ew + (ks2 * 16 + 8 * (l >> 5)) * kERow + (nb * 32 + (l & 31)) * 2;
        uint16_t e8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e8[i] = *reinterpret_cast<const uint16_t*>(src + i * kERow);
        const uint4 pkd = make_uint4((uint32_t)e8[0] | ((uint32_t)e8[1] << 16), (uint32_t)e8[2] | ((uint32_t)e8[3] << 16),
                                     (uint32_t)e8[4] | ((uint32_t)e8[5] << 16), (uint32_t)e8[6] | ((uint32_t)e8[7] << 16));
        const bf16x8 bv = __builtin_bit_cast(bf16x8, pkd);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          o[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[mb], bv, o[mb][nb], 0, 0, 0);
      }
    }
  }

  // ---- finish: either normalise with the sink, or publish the split's partials
  if (nsplit == 1) {
    if ((l & 3) == 0) {
      const float z = sink[kHG * hg + own_h];
      const float Mf = fmaxf(m_run, z);
      const float fac = (m_run == -INFINITY) ? 0.f : fast_exp(m_run - Mf);
      sm.fin[own_h] = fac / (l_run * fac + fast_exp(z - Mf));
    }
    __syncthreads();
    bf16_t* ob = out + ((bi * n_q + r) * n_h + kHG * hg) * (int64_t)kC + kDW * wave + (l & 31);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int head = mb * 32 + 8 * (rr >> 2) + 4 * (l >> 5) + (rr & 3);
        const float g = sm.fin[head];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) ob[head * (int64_t)kC + nb * 32] = f2bf(o[mb][nb][rr] * g);
      }
  } else {
    const int64_t slot = ((bi * n_q + r) * (n_h / kHG) + hg) * nsplit + split;
    float* po = part_o + slot * (int64_t)kHG * kC + kDW * wave + (l & 31);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int head = mb * 32 + 8 * (rr >> 2) + 4 * (l >> 5) + (rr & 3);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) po[head * (int64_t)kC + nb * 32] = o[mb][nb][rr];
      }
    if ((l & 3) == 0) {
      part_ml[(slot * kHG + own_h) * 2 + 0] = m_run;
      part_ml[(slot * kHG + own_h) * 2 + 1] = l_run;
    }
  }
}

// Merge the splits of one (query, 64-head group) in split order, then apply
// the sink: out = sum_s O_s e^{m_s - M} / (sum_s l_s e^{m_s - M} + e^{z - M}).
__global__ __launch_bounds__(256) void attend_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const float* __restrict__ sink, int n_h,
                                                      int nsplit, bf16_t* __restrict__ out) {
  const int64_t qh = blockIdx.x;  // (b*n_q + r) * (n_h/64) + hg
  const int hgn = n_h / kHG;
  const int hg = (int)(qh % hgn);
  const int64_t br = qh / hgn;
  for (int hh = 0; hh < kHG; ++hh) {
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((qh * nsplit + s) * kHG + hh) * 2]);
    const float z = sink[kHG * hg + hh];
    const float Mf = fmaxf(M, z);
    float L = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = part_ml[((qh * nsplit + s) * kHG + hh) * 2];
      const float ls = part_ml[((qh * nsplit + s) * kHG + hh) * 2 + 1];
      const float f = (ms == -INFINITY) ? 0.f : fast_exp(ms - Mf);
      L = fmaf(ls, f, L);
      const float* po = part_o + ((qh * nsplit + s) * kHG + hh) * (int64_t)kC;
      acc0 = fmaf(po[threadIdx.x], f, acc0);
      acc1 = fmaf(po[threadIdx.x + 256], f, acc1);
    }
    const float den = L + fast_exp(z - Mf);
    bf16_t* ob = out + (br * n_h + kHG * hg + hh) * (int64_t)kC;
    ob[threadIdx.x] = f2bf(acc0 / den);
    ob[threadIdx.x + 256] = f2bf(acc1 / den);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static bool attend_mfma_ok(int dtype, int64_t n_h, int64_t c, int64_t k) {
  return dtype == 1 && c == kC && n_h % kHG == 0 && k <= kMaxSel;
}

static int attend_nsplit(int64_t b, int64_t n_q, int64_t n_h, int64_t nmax) {
  const int64_t items = b * n_q * (n_h / kHG);
  if (items >= 512) return 1;
  int64_t ns = (1024 + items - 1) / items;
  const int64_t cap = (nmax + 2 * kT - 1) / (2 * kT);  // at least two tiles per split
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  if (ns > 64) ns = 64;
  return (int)ns;
}

size_t attend_workspace_bytes(int dtype, int64_t b, int64_t n_q, int64_t n_h, int64_t c,
                              int64_t nmax) {
  if (!attend_mfma_ok(dtype, n_h, c, 0)) return 0;
  const int ns = attend_nsplit(b, n_q, n_h, nmax);
  if (ns == 1) return 0;
  const int64_t slots = b * n_q * (n_h / kHG) * ns;
  const size_t o = (size_t)slots * kHG * kC * 4;
  return ((o + 255) & ~(size_t)255) + (size_t)slots * kHG * 2 * 4;
}

bool attend_supported(int dtype, int64_t n_h, int64_t c, int64_t k) {
  return attend_mfma_ok(dtype, n_h, c, k) || c <= 1024;
}

hipError_t launch_attend(int dense, const void* q, const void* Ccomp, int64_t cbs, const int32_t* idx,
                         const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink,
                         int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h,
                         int64_t c, int64_t k, int64_t m, int64_t n_win, float scale, int dtype,
                         void* ws, void* out, hipStream_t st) {
  if (b == 0 || n_q == 0) return hipSuccess;
  if (attend_mfma_ok(dtype, n_h, c, dense ? 0 : k)) {
    int64_t vmax = (t0 + n_q) / m;
    if (vmax > n_comp) vmax = n_comp;
    const int64_t nmax = (dense ? vmax : k) + n_win;
    const int ns = attend_nsplit(b, n_q, n_h, nmax);
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (ns > 1) {
      const int64_t slots = b * n_q * (n_h / kHG) * ns;
      const size_t osz = ((size_t)slots * kHG * kC * 4 + 255) & ~(size_t)255;
      part_o = (float*)ws;
      part_ml = (float*)((unsigned char*)ws + osz);
    }
    dim3 grid((unsigned)n_q, (unsigned)((n_h / kHG) * ns), (unsigned)b);
    if (dense)
      hipLaunchKernelGGL((attend_mfma_c512<1>), grid, dim3(256), 0, st, (const bf16_t*)q,
                         (const bf16_t*)Ccomp, cbs, idx, (const bf16_t*)kv_raw, rbs, raw_pos0, sink,
                         n_q, t0, n_comp, (int)n_h, k, m, n_win, scale, ns, part_o, part_ml,
                         (bf16_t*)out);
    else
      hipLaunchKernelGGL((attend_mfma_c512<0>), grid, dim3(256), 0, st, (const bf16_t*)q,
                         (const bf16_t*)Ccomp, cbs, idx, (const bf16_t*)kv_raw, rbs, raw_pos0, sink,
                         n_q, t0, n_comp, (int)n_h, k, m, n_win, scale, ns, part_o, part_ml,
                         (bf16_t*)out);
    if (ns > 1)
      hipLaunchKernelGGL(attend_combine, dim3((unsigned)(b * n_q * (n_h / kHG))), dim3(256), 0, st,
                         part_o, part_ml, sink, (int)n_h, ns, (bf16_t*)out);
    return hipGetLastError();
  }
  dim3 grid((unsigned)n_q, (unsigned)n_h, (unsigned)b);
  if (dtype == 1)
    hipLaunchKernelGGL((attend_generic<bf16_t>), grid, dim3(256), 0, st, (const bf16_t*)q,
                       (const bf16_t*)Ccomp, cbs, idx, (const bf16_t*)kv_raw, rbs, raw_pos0, sink, n_q,
                       t0, n_comp, (int)n_h, (int)c, k, m, n_win, scale, dense, (bf16_t*)out);
  else
    hipLaunchKernelGGL((attend_generic<float>), grid, dim3(256), 0, st, (const float*)q,
                       (const float*)Ccomp, cbs, idx, (const float*)kv_raw, rbs, raw_pos0, sink, n_q,
                       t0, n_comp, (int)n_h, (int)c, k, m, n_win, scale, dense, (float*)out);
  return hipGetLastError();
}

}  // namespace csa
