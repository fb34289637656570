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
// LDS rows are 1024 + 64 bytes apart and the four 16-byte chunks of every
// 64-byte column block of row r are XOR-permuted by (r/4)%4.  With gfx950's
// 64 LDS banks this keeps both access patterns conflict-free: the b128 row
// reads (16 lanes = 16 consecutive rows, one chunk each) and the transposed
// reads (32 lanes = 4 consecutive rows x one 64-byte block each), and the
// offset of column block nb stays a constant 64*nb, so each lane needs only
// two base addresses per phase.
// ---------------------------------------------------------------------------
constexpr int kC = 512;
constexpr int kHG = 64;              // heads per head group
constexpr int kHW = 32;              // heads per wave
constexpr int kT = 32;               // entries per tile
constexpr int kRowB = kC * 2 + 64;   // LDS bytes per entry row (64-byte skew)
constexpr int kTileB = kT * kRowB;   // 34 KiB
constexpr int kMaxSel = 2048;        // selected entries staged in LDS
constexpr int kStageRowB = 256 * 2;  // output staging row (256 dims), XOR-swizzled

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// max / sum of a value and its copy in the other 32-lane half
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

template <int DENSE, int G>
struct AttnSmem {
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
  // the two tile buffers (double buffering: gather one while computing the other)
  __shared__ __attribute__((aligned(16))) unsigned char E0[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char E1[kTileB];
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
  // entries of the group list this wave's query may not read (-1: none)
  int64_t exA_abs = -1, exW_abs = -1;
  if (DENSE) {
    if (vis_q < nsel) exA_abs = vis_q;                       // at most one: vis differs by <= 1
    const int64_t wq_lo = t_q - n_win + 1;                   // this query's window starts here
    if (wlo < wq_lo) exW_abs = nsel;                         // union starts one row earlier
    if (t_q < t_last) exW_abs = nsel + (t_last - wlo);       // union ends one row later
  }

  const bf16_t* cbase = Ccomp + bi * cbs;
  const bf16_t* rbase = kv_raw + bi * rbs + (wlo - raw_pos0) * (int64_t)kC;
  // gather one tile into LDS.  Lane l (< 32) resolves the address of tile
  // row l; wave w then loads rows w, w+NW, ... with the row base broadcast
  // to scalar registers, lane l fetching chunk l ^ f(row) so that LDS chunk
  // position c holds row chunk c ^ f(row).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue_tile = [&](int64_t jt, unsigned char* buf) {
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
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(buf + row * kRowB), 16, 0, 0);
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
  // per-lane LDS byte offsets inside a tile buffer
  //   S^T A operand: row l%32, chunk 2ks + half -> 16*((2(ks%2) + half) ^ g) + 64*(ks/2)
  const int srow = l & 31;
  const int sb0 = srow * kRowB + 16 * (half ^ swz(srow));
  const int sb1 = srow * kRowB + 16 * ((half ^ swz(srow)) ^ 2);
  //   P V B operand (transposed read): rows 16ks2 + 8q + 4half + (l%16)/4,
  //   column block nb, chunk 2*((l/16)%2) + (l%4)/2 of the block, byte 8*(l%2)
  const int s16 = l & 15;
  const int cpart = 2 * ((l >> 4) & 1) + ((s16 & 3) >> 1);
  const int boff = 8 * (s16 & 1);
  auto trbase = [&](int row) { return row * kRowB + 16 * (cpart ^ swz(row)) + boff; };
  const int tbA0 = trbase(4 * half + (s16 >> 2)), tbB0 = trbase(8 + 4 * half + (s16 >> 2));
  const int tbA1 = trbase(16 + 4 * half + (s16 >> 2)), tbB1 = trbase(24 + 4 * half + (s16 >> 2));
  if (tid == 0) sm.gen = 0;
  __syncthreads();
  int gen = 0;
  for (;;) {
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) o[nb] = (f32x16){};
    l_run = 0.f;
    // one tile: wait for its gather, start the next gather into the other
    // buffer, then S^T, weights and P V from this buffer
    auto tile = [&](const int it, unsigned char* const Eb, unsigned char* const En) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (it + 1 < ntiles) issue_tile(jb + (int64_t)(it + 1) * kT, En);
      const int64_t j0 = jb + (int64_t)it * kT;

      // S^T[entry][head] over 512 dims: two independent accumulation chains,
      // LDS operands fetched two steps ahead of the MFMAs that use them
      f32x16 st0 = (f32x16){}, st1 = (f32x16){};
      {
        const unsigned char* e0 = Eb + sb0;
        const unsigned char* e1 = Eb + sb1;
        bf16x8 a[3][2];
        a[0][0] = *reinterpret_cast<const bf16x8*>(e0);
        a[0][1] = *reinterpret_cast<const bf16x8*>(e1);
        a[1][0] = *reinterpret_cast<const bf16x8*>(e0 + 64);
        a[1][1] = *reinterpret_cast<const bf16x8*>(e1 + 64);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (u + 2 < 16) {
            a[(u + 2) % 3][0] = *reinterpret_cast<const bf16x8*>(e0 + 64 * (u + 2));
            a[(u + 2) % 3][1] = *reinterpret_cast<const bf16x8*>(e1 + 64 * (u + 2));
          }
          st0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u % 3][0], qT[2 * u], st0, 0, 0, 0);
          st1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u % 3][1], qT[2 * u + 1], st1, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // first P V operands, independent of the weights: fetch them now
      bf16x4 tr[3][2];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        tr[q2][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Eb + tbA0 + 64 * q2));
        tr[q2][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Eb + tbB0 + 64 * q2));
      }
      // weights of head l%32 for the tile's entries (entry = j0 + local)
      uint32_t pk[8];
      {
        const int rem = (int)(je - j0 < kT ? je - j0 : kT);   // real entries in this tile
        // the group's entry list is the union over its G consecutive queries:
        // this query excludes at most one compressed entry (completed only at
        // the group's last position) and one window row (outside its window)
        int exA = -1, exW = -1;
        if (DENSE) {
          const int64_t cap = 1 << 20;
          auto rel = [&](int64_t e) { const int64_t x = e - j0; return (int)(x < -1 || x > cap ? -1 : x); };
          exA = rel(exA_abs);
          exW = rel(exW_abs);
        }
        float sv[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int loc = 8 * (r >> 2) + 4 * half + (r & 3);
          bool valid = loc < rem;
          if (DENSE) valid = valid & (loc != exA) & (loc != exW);
          sv[r] = valid ? (st0[r] + st1[r]) * sl2 : -INFINITY;
          tmax = fmaxf(tmax, sv[r]);
        }
        tmax = half_max(tmax);
        m_seen = fmaxf(m_seen, tmax);
        if (m_ref == -INFINITY) m_ref = tmax;            // first valid logits of this head
        const float mb = (m_ref == -INFINITY) ? 0.f : m_ref;
        const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(sv[r] - mb);
          const float p1 = __builtin_amdgcn_exp2f(sv[r + 1] - mb);
          const bf16x2_t b = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);   // round to nearest even
          rs = __builtin_amdgcn_fdot2_f32_bf16(b, ones, rs, false);   // sum of the weights P V multiplies
          pk[r >> 1] = __builtin_bit_cast(uint32_t, b);
        }
        l_run += half_sum(rs);
      }
      // O[head][dim] += P[head][entry] E[entry][dim]; step i = (ks2, nb) = (i/16, i%16),
      // its transposed operands fetched two steps ahead
      {
        bf16x8 pa[2];
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
          pa[ks2] = __builtin_bit_cast(bf16x8, make_uint4(pk[4 * ks2], pk[4 * ks2 + 1], pk[4 * ks2 + 2],
                                                          pk[4 * ks2 + 3]));
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (i + 2 < 32) {
            const int i2 = i + 2, k2 = i2 >> 4, n2 = i2 & 15;
            tr[i2 % 3][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4_t*)(Eb + (k2 ? tbA1 : tbA0) + 64 * n2));
            tr[i2 % 3][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4_t*)(Eb + (k2 ? tbB1 : tbB0) + 64 * n2));
          }
          const bf16x8 bv = __builtin_shufflevector(tr[i % 3][0], tr[i % 3][1], 0, 1, 2, 3, 4, 5, 6, 7);
          o[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i >> 4], bv, o[i & 15], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    if (ntiles > 0) issue_tile(jb, E0);
    for (int it = 0; it < ntiles; ++it) {
      unsigned char* const Eb = (it & 1) ? E1 : E0;
      unsigned char* const En = (it & 1) ? E0 : E1;
      tile(it, Eb, En);
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
    unsigned char* stg = ((wave < 2) ? E0 : E1) + (wave & 1) * (kHW * kStageRowB);
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
