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
// The MFMA path (bf16, c = 512, 64-head groups) is described above its
// kernel; the generic path covers every other shape and float32.
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
// MFMA path (bf16, c = 512, 64-head groups).
//
// A workgroup serves G consecutive queries of one 64-head group; two waves
// per query, each owning 32 heads over all 512 dimensions (Q^T operand in
// 128 VGPRs, O accumulator in 256 AGPRs).  Entries are processed in tiles of
// 32 rows that all waves of the workgroup share: the rows are gathered from
// HBM/L2 straight into LDS (global_load_lds_dwordx4, one 1 KiB row per wave
// instruction), double-buffered with one barrier per tile.
//
// Per tile and wave:
//   S^T = E Q^T      v_mfma_f32_32x32x16_bf16, A = E rows from LDS
//                    (ds_read_b128), B = Q^T from registers.  The result
//                    has one head per lane column and 16 entries per lane,
//                    so the softmax over entries needs only in-lane work and
//                    one exchange between the two lane halves.
//   O += P E         A = P taken straight from the S^T accumulators (the
//                    contraction index is permuted to match their row
//                    layout), B = E^T read with ds_read_b64_tr_b16, which
//                    returns a 4-row x 16-column block column-per-lane.
// LDS rows are 1 KiB with the 16-byte chunks of row r XOR-swizzled by
// f(r) = 2(r%4) + (r/4)%2, which keeps both the b128 row reads (8 rows, one
// chunk) and the transposed reads (4 rows, two chunks) free of bank
// conflicts.
// ---------------------------------------------------------------------------
constexpr int kC = 512;
constexpr int kHG = 64;              // heads per head group
constexpr int kHW = 32;              // heads per wave
constexpr int kT = 32;               // entries per tile
constexpr int kRowB = kC * 2;        // LDS bytes per entry row
constexpr int kTileB = kT * kRowB;   // 32 KiB
constexpr int kMaxSel = 2048;        // selected entries staged in LDS
constexpr int kStageRowB = 256 * 2;  // output staging row (256 dims), XOR-swizzled

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ int swz(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }

template <int DENSE, int G>
struct AttnSmem {
  unsigned char E[2][kTileB];       // 64 KiB, reused for output staging
  int32_t sel[DENSE ? 1 : kMaxSel];
  float bc[2 * G][kHW];             // per-wave broadcast of per-head factors
  int32_t cnt[2 * G];
  int32_t gen;                      // restart generation (see the softmax note)
};

template <int DENSE, int G>
__global__ __launch_bounds__(128 * G) void attend_mfma_c512(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Ccomp, int64_t cbs,
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ kv_raw, int64_t rbs,
    int64_t raw_pos0, const float* __restrict__ sink, int64_t n_q, int64_t t0, int64_t n_comp,
    int n_h, int64_t k, int64_t m, int64_t n_win, float scale, int nsplit,
    float* __restrict__ part_o, float* __restrict__ part_ml, bf16_t* __restrict__ out) {
  constexpr int NW = 2 * G;  // waves per workgroup
  __shared__ AttnSmem<DENSE, G> sm;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int half = l >> 5;
  const int qw = wave >> 1;          // query slot in the group
  const int hw = wave & 1;           // which 32 heads of the group
  const int64_t grp = (int64_t)gridDim.x - 1 - blockIdx.x;   // later queries (more work) first
  const int hg = blockIdx.y / nsplit;
  const int split = blockIdx.y % nsplit;
  const int64_t bi = blockIdx.z;
  const int64_t r0 = grp * G;
  const int64_t rlast = (r0 + G - 1 < n_q) ? r0 + G - 1 : n_q - 1;
  const int64_t rq = r0 + qw;
  const bool qvalid = rq < n_q;
  const int64_t t_first = t0 + r0, t_last = t0 + rlast;
  const int64_t t_q = t0 + (qvalid ? rq : rlast);

  // ---- entry list: compressed part (selected or dense), then the union of
  //      the group's causal windows
  int64_t nsel, vis_q;
  if (DENSE) {
    nsel = (t_last + 1) / m;
    if (nsel > n_comp) nsel = n_comp;
    vis_q = (t_q + 1) / m;
    if (vis_q > n_comp) vis_q = n_comp;
  } else {
    // G == 1: stable compaction of the valid indices (0 <= s < visible)
    int64_t vis = (t_first + 1) / m;
    if (vis > n_comp) vis = n_comp;
    const int32_t* ir = idx + (bi * n_q + r0) * k;
    int64_t base = 0;
    for (int64_t j0 = 0; j0 < k; j0 += 64 * NW) {
      const int64_t j = j0 + tid;
      const int32_t sv = j < k ? ir[j] : -1;
      const bool ok = sv >= 0 && sv < vis;
      const uint64_t mk = __ballot(ok);
      if (l == 0) sm.cnt[wave] = __popcll(mk);
      __syncthreads();
      int64_t pos = base;
      for (int w2 = 0; w2 < wave; ++w2) pos += sm.cnt[w2];
      pos += __popcll(mk & ((l == 0) ? 0ull : (~0ull >> (64 - l))));
      if (ok && pos < kMaxSel) sm.sel[pos] = sv;
      for (int w2 = 0; w2 < NW; ++w2) base += sm.cnt[w2];
      __syncthreads();
    }
    nsel = base < kMaxSel ? base : kMaxSel;
    vis_q = nsel;
  }
  const int64_t wlo = t_first - n_win + 1 > 0 ? t_first - n_win + 1 : 0;
  const int64_t N = nsel + (t_last - wlo + 1);
  const int64_t per = (N + nsplit - 1) / nsplit;
  const int64_t jb = (int64_t)split * per;
  const int64_t je = jb + per < N ? jb + per : N;
  const int ntiles = je > jb ? (int)((je - jb + kT - 1) / kT) : 0;

  const bf16_t* cbase = Ccomp + bi * cbs;
  const bf16_t* rbase = kv_raw + bi * rbs + (wlo - raw_pos0) * (int64_t)kC;
  // gather one tile into LDS.  Lane l (< 32) resolves the address of tile
  // row l; wave w then loads rows w, w+NW, ... with the row base broadcast
  // to scalar registers, lane l fetching chunk l ^ f(row) so that LDS chunk
  // position c holds row chunk c ^ f(row).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue_tile = [&](int64_t jt, int buf) {
    int64_t j = jt + (l & 31);
    if (j >= je) j = jb;  // tail padding rows: any real row (its weight is 0)
    const bf16_t* p = j < nsel ? cbase + (int64_t)(DENSE ? j : sm.sel[j]) * kC
                               : rbase + (j - nsel) * (int64_t)kC;
    const uint64_t pv = reinterpret_cast<uint64_t>(p);
    const uint32_t plo = (uint32_t)pv, phi = (uint32_t)(pv >> 32);
#pragma unroll
    for (int rr = 0; rr < kT / NW; ++rr) {
      const int row = wave_u + rr * NW;
      // readlane returns a signed int: zero-extend both halves
      const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(phi, row) << 32) |
                            (uint64_t)(uint32_t)__builtin_amdgcn_readlane(plo, row);
      const unsigned char* src = reinterpret_cast<const unsigned char*>(base) + ((l ^ swz(row)) << 4);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(&sm.E[buf][row * kRowB]), 16, 0, 0);
    }
  };

  // ---- Q^T operand: head 64*hg + 32*hw + l%32, dims 16*ks + 8*half + (0..7)
  bf16x8 qT[32];
  {
    const int64_t qrow = qvalid ? rq : rlast;
    const bf16_t* qp = q + ((bi * n_q + qrow) * n_h + kHG * hg + kHW * hw + (l & 31)) * (int64_t)kC + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks)
      qT[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 16));
  }
  // Softmax without rescaling O.  VALU instructions cannot operate on the
  // accumulation registers, so an online max that rescales O every time it
  // grows would force O out of them.  Instead each head keeps a fixed
  // reference m_ref (log2 domain), set from its first valid logits; weights
  // 2^(s - m_ref) are exact relative values and may exceed 1.  Should a later
  // logit exceed m_ref by more than kLogHeadroom (weights up to 2^64; the
  // float32 range stops at 2^128), the workgroup runs this query's entries
  // again with m_ref raised to the largest logit seen -- a rare, exact
  // fallback.
  constexpr float kLogHeadroom = 64.f;
  f32x16 o[16];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;   // head l%32
  const float sl2 = scale * kLog2e;
  const int srow = l & 31;                // entry row this lane feeds in S^T
  const int s16 = l & 15;
  const int colh = 16 * ((l >> 4) & 1);
  if (tid == 0) sm.gen = 0;
  __syncthreads();
  int gen = 0;
  for (;;) {
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) o[nb] = (f32x16){};
    l_run = 0.f;
    if (ntiles > 0) issue_tile(jb, 0);
    for (int it = 0; it < ntiles; ++it) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (it + 1 < ntiles) issue_tile(jb + (int64_t)(it + 1) * kT, (it + 1) & 1);
      const unsigned char* Eb = sm.E[it & 1];
      const int64_t j0 = jb + (int64_t)it * kT;

      // S^T[entry][head] over 512 dims
      f32x16 st = (f32x16){};
      {
        const unsigned char* er = Eb + srow * kRowB;
        const int f = swz(srow);
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(er + (((2 * ks + half) ^ f) << 4));
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qT[ks], st, 0, 0, 0);
          if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // bound the operands in flight
        }
      }
      // weights of head l%32 for the tile's entries
      uint32_t pk[8];
      {
        float sv[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t e = j0 + 8 * (r >> 2) + 4 * half + (r & 3);
          bool valid = e < je;
          if (DENSE) {
            if (e < nsel) {
              valid = valid && e < vis_q;
            } else {
              const int64_t p = wlo + (e - nsel);
              valid = valid && p > t_q - n_win && p <= t_q;
            }
          }
          sv[r] = valid ? st[r] * sl2 : -INFINITY;
          tmax = fmaxf(tmax, sv[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        m_seen = fmaxf(m_seen, tmax);
        if (m_ref == -INFINITY) m_ref = tmax;            // first valid logits of this head
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = (sv[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m_ref);
          const float p1 = (sv[r + 1] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sv[r + 1] - m_ref);
          const uint16_t b0 = f2bf(p0), b1 = f2bf(p1);
          rs += bf2f(b0) + bf2f(b1);   // normalise with the weights P V multiplies
          pk[r >> 1] = (uint32_t)b0 | ((uint32_t)b1 << 16);
        }
        rs += __shfl_xor(rs, 32, 64);
        l_run += rs;
      }
      // O[head][dim] += P[head][entry] E[entry][dim]
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(pk[4 * ks2], pk[4 * ks2 + 1], pk[4 * ks2 + 2],
                                                                pk[4 * ks2 + 3]));
        const int rowA = 16 * ks2 + 4 * half + (s16 >> 2);
        const int rowB = rowA + 8;
        const unsigned char* ea = Eb + rowA * kRowB;
        const unsigned char* eb2 = Eb + rowB * kRowB;
        const int fa = swz(rowA), fb = swz(rowB);
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
          const int col = 32 * nb + colh + 4 * (s16 & 3);
          const int chunk = col >> 3, off = (col & 7) * 2;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4_t*)(ea + ((chunk ^ fa) << 4) + off));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4_t*)(eb2 + ((chunk ^ fb) << 4) + off));
          const bf16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, bv, o[nb], 0, 0, 0);
          if ((nb & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // an attempt whose weights may have overflowed is discarded as a whole;
    // the decision is workgroup-wide because the waves share the tiles
    if (m_seen > m_ref + kLogHeadroom) sm.gen = gen + 1;
    __syncthreads();
    if (sm.gen == gen) break;
    ++gen;
    m_ref = m_seen;
  }
  const float m_run = m_ref;

  const int head0 = kHG * hg + kHW * hw;   // first head of this wave
  if (nsplit == 1) {
    // final per-head factor e^{-M} / (sum + e^{z - M}), broadcast over the O rows
    if (l < 32) {
      const float z2 = sink[head0 + l] * kLog2e;
      const float Mf = fmaxf(m_run, z2);
      const float fac = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - Mf);
      sm.bc[wave][l] = fac / (l_run * fac + __builtin_amdgcn_exp2f(z2 - Mf));
    }
    float4 g4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) g4[g] = *reinterpret_cast<const float4*>(&sm.bc[wave][8 * g + 4 * half]);
    __syncthreads();   // every wave is done with the tile buffers
    unsigned char* stg = &sm.E[0][0] + wave * (kHW * kStageRowB);
    bf16_t* ob = out + ((bi * n_q + (qvalid ? rq : rlast)) * n_h + head0) * (int64_t)kC;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int nb8 = 0; nb8 < 8; ++nb8) {
        const int nb = pass * 8 + nb8;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float gv[4] = {g4[g].x, g4[g].y, g4[g].z, g4[g].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int hr = 8 * g + 4 * half + i;
            // rows 4 apart would share banks: flip the 64-byte half for odd row quads
            const int byte = ((nb8 * 32 + (l & 31)) * 2) ^ (((hr >> 2) & 1) << 6);
            *reinterpret_cast<bf16_t*>(stg + hr * kStageRowB + byte) = f2bf(o[nb][4 * g + i] * gv[i]);
          }
        }
      }
      // the staging area is private to this wave: its own writes are ordered
      // before its reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cidx = l + 64 * i;            // 16-byte chunk of the 32 x 512 B block
        const int hr = cidx >> 5, c16 = cidx & 31;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + hr * kStageRowB + ((c16 * 16) ^ (((hr >> 2) & 1) << 6)));
        if (qvalid)
          *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(ob + hr * (int64_t)kC + pass * 256) + c16 * 16) = v;
      }
    }
  } else if (qvalid) {
    const int64_t slot = ((bi * n_q + rq) * (n_h / kHG) + hg) * nsplit + split;
    float* po = part_o + slot * (int64_t)kHG * kC + (int64_t)kHW * hw * kC + (l & 31);
#pragma unroll
    for (int nb = 0; nb < 16; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hr = 8 * (r >> 2) + 4 * half + (r & 3);
        po[hr * (int64_t)kC + nb * 32] = o[nb][r];
      }
    if (l < 32) {
      part_ml[(slot * kHG + kHW * hw + l) * 2 + 0] = m_run;
      part_ml[(slot * kHG + kHW * hw + l) * 2 + 1] = l_run;
    }
  }
}

// Merge the splits of one (query, head) in split order (log2-domain maxima),
// then apply the sink: out = sum_s O_s 2^{m_s - M} / (sum_s l_s 2^{m_s - M} + 2^{z - M}).
__global__ __launch_bounds__(128) void attend_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const float* __restrict__ sink, int n_h,
                                                      int nsplit, bf16_t* __restrict__ out) {
  const int64_t qr = blockIdx.x;   // b * n_q + r
  const int h = blockIdx.y;
  const int hg = h / kHG, hh = h % kHG;
  const int64_t base = (qr * (n_h / kHG) + hg) * nsplit;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((base + s) * kHG + hh) * 2]);
  const float z2 = sink[h] * kLog2e;
  const float Mf = fmaxf(M, z2);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; ++s) {
    const float ms = part_ml[((base + s) * kHG + hh) * 2];
    const float ls = part_ml[((base + s) * kHG + hh) * 2 + 1];
    const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - Mf);
    L = fmaf(ls, f, L);
    const float4 v = reinterpret_cast<const float4*>(part_o + ((base + s) * kHG + hh) * (int64_t)kC)[threadIdx.x];
    acc.x = fmaf(v.x, f, acc.x);
    acc.y = fmaf(v.y, f, acc.y);
    acc.z = fmaf(v.z, f, acc.z);
    acc.w = fmaf(v.w, f, acc.w);
  }
  const float inv = 1.f / (L + __builtin_amdgcn_exp2f(z2 - Mf));
  bf16_t* ob = out + (qr * n_h + h) * (int64_t)kC + 4 * threadIdx.x;
  const uint2 pk = make_uint2((uint32_t)f2bf(acc.x * inv) | ((uint32_t)f2bf(acc.y * inv) << 16),
                              (uint32_t)f2bf(acc.z * inv) | ((uint32_t)f2bf(acc.w * inv) << 16));
  *reinterpret_cast<uint2*>(ob) = pk;
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
    const int G = dense ? 2 : 1;
    dim3 grid((unsigned)((n_q + G - 1) / G), (unsigned)((n_h / kHG) * ns), (unsigned)b);
    if (dense)
      hipLaunchKernelGGL((attend_mfma_c512<1, 2>), grid, dim3(256), 0, st, (const bf16_t*)q,
                         (const bf16_t*)Ccomp, cbs, idx, (const bf16_t*)kv_raw, rbs, raw_pos0, sink,
                         n_q, t0, n_comp, (int)n_h, k, m, n_win, scale, ns, part_o, part_ml,
                         (bf16_t*)out);
    else
      hipLaunchKernelGGL((attend_mfma_c512<0, 1>), grid, dim3(128), 0, st, (const bf16_t*)q,
                         (const bf16_t*)Ccomp, cbs, idx, (const bf16_t*)kv_raw, rbs, raw_pos0, sink,
                         n_q, t0, n_comp, (int)n_h, k, m, n_win, scale, ns, part_o, part_ml,
                         (bf16_t*)out);
    if (ns > 1)
      hipLaunchKernelGGL(attend_combine, dim3((unsigned)(b * n_q), (unsigned)n_h), dim3(128), 0, st,
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
