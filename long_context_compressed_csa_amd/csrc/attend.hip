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
// MFMA path (bf16, c = 512, 64-head groups): attend_ds.
//
// A workgroup serves one query and one 64-head group with four waves; wave
// w owns heads 32 (w & 1) .. +31 and dimensions 256 (w >> 1) .. +255, so a
// wave holds the Q operand of its heads over its dimensions (64 VGPRs) and
// the O accumulator of its heads over its dimensions (128 AGPRs), and two
// waves share each SIMD, each hiding the other's LDS, barrier and softmax
// latencies.  Entries stream through LDS in tiles of 16 rows that all four
// waves share, gathered from HBM/L2 straight into LDS (global_load_lds_dwordx4,
// one 64-byte column block of 16 rows per wave instruction) two tiles ahead
// of use, into three statically distinct buffers.
//
// Per tile and wave:
//   S^T = E Q^T        v_mfma_f32_16x16x32_bf16 over the wave's 256
//                      dimensions, A = 16 entry rows from LDS (ds_read_b128),
//                      B = Q^T (16 heads) from registers; two head blocks.  A
//                      lane ends up with 4 entries of each of two heads.
//   exchange           the partial S^T goes to LDS; after a barrier the wave
//                      adds its partner's (same heads, other dimensions), so
//                      both hold the same scores, maxima and weights
//   O += P E           v_mfma_f32_32x32x16_bf16 over the 16 entries, B = E^T
//                      read with ds_read_b64_tr_b16 (4 rows x 16 columns,
//                      column-per-lane) for the wave's 8 column blocks, A = P
//                      in registers.
// A lane's 32x32 A operand (head l%32, entries 8(l/32)..+7) is its own 4
// weights of that head plus the 4 held by lane l^16, exchanged with one
// v_permlane16_swap per register.  A tile is stored column-block major: the
// 64-byte column block b of all 16 rows fills 1 KiB at b * 1024, and inside
// it chunk c of row r sits at c * 256 + (r ^ x_c) * 16 with x_c = -4c mod 16
// (0, 12, 8, 4).  One gather instruction then fills one block with 16 B per
// lane.  gfx950's LDS (64 banks) serves a b128 read in four cycles of 16
// lanes that are not 16 consecutive lanes (LDS counters on read patterns fit
// lanes sharing a cycle when lane bit 5 and the parity of lane bits 2..4
// agree): with x_c = 4c the row reads (lane l: row l % 16 of chunk l / 16)
// ran at half rate, with x_c above they are conflict-free, and so are the
// transposed reads (16 lanes = 4 rows x 4 chunks, the four chunks' rows in
// disjoint bank quarters).
// ---------------------------------------------------------------------------
constexpr int kC = 512;
constexpr int kHG = 64;              // heads per head group
constexpr int kHW = 32;              // heads per wave
constexpr int kT = 16;               // entries per tile
constexpr int kBlkB = kT * 64;       // one 64-byte column block of all 16 rows
constexpr int kTileB = kT * kC * 2;  // 16 KiB: 16 column blocks
constexpr int kMaxSel = 2048;        // selected entries staged in LDS
constexpr int kStageRowB = 256 * 2;  // output staging row (256 dims), XOR-swizzled
static_assert(kHW * kStageRowB <= kTileB, "a wave's output staging must fit one tile buffer");
// row permutation x_c of chunk c inside a tile's column block
__device__ __forceinline__ int tile_swz(int c) { return (16 - 4 * c) & 15; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// max / sum of a value and its copy in the other 32-lane half
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// the value held by lane l ^ 16
__device__ __forceinline__ uint32_t from_lane_xor16(uint32_t x, bool upper16) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);   // {x[l & ~16], x[l | 16]}
  return upper16 ? r[0] : r[1];
}

// barrier among the workgroup's waves that does not drain outstanding LDS
// gathers (a __syncthreads fence would wait for every one of them)
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// O += A B on the 32x32x16 bf16 MFMA with O pinned to accumulation registers.
// This file is compiled with MFMA results in VGPRs (the S^T accumulators are
// read by VALU code); O alone, 128 registers per lane, is kept in AGPRs by
// issuing its products as asm (the first product of a query with C = 0, so
// O needs no zeroing).  The compiler sees only asm statements, so it neither
// checks their hazards nor pads for them: compiled code reading O after the
// last product pads with o_hazard_pad, and VALU-written operands wait before
// the first product that reads them and stay unchanged until a wait after
// the last (see pv_part).
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8 a, const bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// O = A B (the first product of an accumulation: C is the inline constant 0,
// so no register holds the zeros)
__device__ __forceinline__ void mfma_first(f32x16& acc, const bf16x8 a, const bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void o_hazard_pad() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// LDS-DMA of 16 bytes per lane (lane l's bytes land at LDS byte address
// lds + 16 l; lds is wave-uniform, passed in M0) issued as inline assembly:
// the compiler does not track these LDS writes, so it adds no wait of its
// own before the operand reads of other tile buffers; the kernel orders them
// with explicit vmcnt waits and barriers.  M0 is restored afterwards, since
// the compiler does not accept it as a clobber.  No register results.
__device__ __forceinline__ void attn_dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds) : "memory");
}

struct DsSmem {
  int32_t sel[kMaxSel];
  int32_t cnt[kMaxSel / 256][4];
  float bc[4][kHW];
  int32_t gen;
};
constexpr int kXB = 64 * 8 * 4;   // one wave's partial S^T: 64 lanes x 8 floats

// SPLIT = 1: the entry list is split over nsplit workgroups that write
// partial states for attend_combine; SPLIT = 0: nsplit is 1 and the output is
// written here.  PG = 1 (paged decode cache): the query of batch row b sits
// at pos[b], compressed entries are pool rows found through the block table
// of `er` (translated during the compaction), window rows live in a ring of
// `ring` slots per request.  DENSE = 1 (HCA): the entry list is every
// completed entry, s < (t+1)/m, with no index list (paged: a split's entries
// are translated to pool rows in LDS before its tiles, so a split holds at
// most kMaxSel of them).  NRQ = 1: q holds the raw query heads; each is
// RMS-normalised (gain gq, eps), its last rope_dims dimensions turned by
// t * base^(-2i / rope_dims), and rounded to bf16 as it becomes the MFMA
// operand; the output's last rope_dims dimensions are turned back by -t in
// float32 before the bf16 store (split partial states are turned before
// they are written: the merge is linear).
#if CSA_DEBUG
// Debug builds: every row the attention gathers (flat caches) is checked
// against the bounds the call implies -- a compressed entry below n_comp
// (and below a host-set limit, which tests lower to force the check), a
// window row between the window's first row and the query's own.  A row
// outside them is not read (the query's own window row is gathered in its
// place) and the flag is raised; the host reports it after the launch.
__device__ unsigned int csa_dbg_oob = 0;
__device__ long long csa_dbg_entry_limit = 0x7fffffffffffffffLL;
#endif

template <int SPLIT, int PG, int DENSE, int NRQ>
__global__ __launch_bounds__(256, 2) void attend_ds(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Ccomp, int64_t cbs,
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ kv_raw, int64_t rbs,
    int64_t raw_pos0, const float* __restrict__ sink, int64_t n_q, int64_t t0, int64_t n_comp,
    int n_h, int64_t k, int64_t m, int64_t n_win, float scale, int nsplit, float* __restrict__ part_o,
    float* __restrict__ part_ml, bf16_t* __restrict__ out, Rows er, int64_t ring,
    const int64_t* __restrict__ pos, const float* __restrict__ gq, float eps, int rope_dims, double base) {
  constexpr int NW = 4;
  constexpr int R = kT / NW;   // gather loads per wave and tile
  __shared__ DsSmem sm;
  // NRQ: per-dimension coefficients (A, B) of the normalised, rotated
  // query, q'[d] = inv (q[d] A_d + q[d ^ 1] B_d) with inv the head's
  // 1 / rms (gains and rotation folded in); per pair of dimensions the
  // rotation (cos, sin) for the output; the waves' partial sums of squares
  __shared__ __attribute__((aligned(16))) float2 nr_ab[NRQ ? kC : 2];
  __shared__ __attribute__((aligned(16))) float2 nr_pr[NRQ ? kC / 2 : 1];
  __shared__ float nr_ss[NRQ ? NW : 1][NRQ ? kHW : 1];
  __shared__ __attribute__((aligned(16))) unsigned char T0[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char T1[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char T2[kTileB];
  // partial S^T exchange of the four waves; also wave 3's output staging
  __shared__ __attribute__((aligned(16))) unsigned char XB[NW * kXB];
  static_assert(NW * kXB >= kHW * kStageRowB / 2, "half a wave's staging must fit the exchange buffer");
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int half = l >> 5;
  const int g4 = l >> 4;
  const bool up16 = (l & 16) != 0;
  const int s16 = l & 15;
  const int hw = wave & 1;           // which 32 heads of the group
  const int dh = wave >> 1;          // which 256 dimensions
  const int64_t rq = (int64_t)gridDim.x - 1 - blockIdx.x;   // later queries (more work) first
  const int hg = blockIdx.y / nsplit;
  const int split = blockIdx.y % nsplit;
  const int64_t bi = blockIdx.z;
  const int64_t t = (PG ? pos[bi] : t0) + rq;
  const int head0 = kHG * hg + kHW * hw;

  // Q operand, this wave's dimensions: lane holds head head0 + 16 hb + l%16,
  // dims 256 dh + 32 ks + 8 (l/16) + (0..7)
  bf16x8 qB[8][2];
  // NRQ: whether this wave's 32-dimension block blk (dimensions 256 dh +
  // 32 blk ..) holds rotated dimensions (uniform over the wave)
  const int dh_u = __builtin_amdgcn_readfirstlane(dh);
  auto rotated_block = [&](int blk) -> bool { return NRQ && 256 * dh_u + 32 * blk + 31 >= kC - rope_dims; };
  // stable compaction of the valid indices (0 <= s < visible); every index
  // load is issued before the first is used
  constexpr int NT = 64 * NW;
  constexpr int NR = kMaxSel / NT;
  int64_t vis = (t + 1) / m;
  if (vis > n_comp) vis = n_comp;
  // the index list and Q are loaded together, the index list first: the
  // compaction waits only for it, and Q's latency overlaps the compaction
  int32_t sv[NR];
  if (!DENSE) {
    const int32_t* ir = idx + (bi * n_q + rq) * k;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int64_t j = (int64_t)u * NT + tid;
      sv[u] = j < k ? ir[j] : -1;
    }
  }
  // NRQ: this thread's pair of gains, loaded ahead of Q so that waiting
  // for it does not wait for Q
  float2 gv = make_float2(0.f, 0.f);
  if (NRQ) {
    static_assert(2 * 64 * NW == kC, "one pair of dimensions per thread");
    gv = reinterpret_cast<const float2*>(gq)[tid];
  }
  {
    const bf16_t* qp = q + ((bi * n_q + rq) * n_h + head0 + s16) * (int64_t)kC + 256 * dh + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) qB[ks][hb] = *reinterpret_cast<const bf16x8*>(qp + hb * 16 * kC + ks * 32);
  }
  if (DENSE) {
    sm.gen = 0;   // every thread writes the same value; read after a later barrier
  } else {
    uint64_t mk[NR];
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      mk[u] = __builtin_amdgcn_ballot_w64(sv[u] >= 0 && sv[u] < vis);
      if (l == 0) sm.cnt[u][wave] = __popcll(mk[u]);
    }
    if (PG) {
      // a selected entry becomes its row number in the block pool
#pragma unroll
      for (int u = 0; u < NR; ++u)
        if ((mk[u] >> l) & 1) sv[u] = (int32_t)(er.at(bi, sv[u], kC) / kC);
    }
    __syncthreads();
    const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
    int64_t base = 0;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      int pre = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) pre += w < wave ? sm.cnt[u][w] : 0;
      const int64_t pos = base + pre + __popcll(mk[u] & below);
      if (((mk[u] >> l) & 1) && pos < kMaxSel) sm.sel[pos] = sv[u];
      base += sm.cnt[u][0] + sm.cnt[u][1] + sm.cnt[u][2] + sm.cnt[u][3];
    }
    __syncthreads();
    sm.gen = 0;   // every thread writes the same value; read after the next barrier
  }
  {
    if (NRQ) {
      // the tables while Q is in flight, angles in float64 (positions reach
      // 2^20 and beyond).  Thread tid: the pair of dimensions (2 tid,
      // 2 tid + 1), rotated pair tid - lo/2 when 2 tid >= lo = c - rope_dims;
      // the normalised pair (a, b) turns into (a cos - b sin, a sin + b cos)
      const int lo2 = (kC - rope_dims) >> 1;
      float c1 = 1.f, s1 = 0.f;
      if (tid >= lo2) {
        const double theta = pow(base, -2.0 * (double)(tid - lo2) / (double)rope_dims);
        double sn, cs;
        sincos((double)t * theta, &sn, &cs);
        c1 = (float)cs;
        s1 = (float)sn;
      }
      reinterpret_cast<float4*>(nr_ab)[tid] = make_float4(c1 * gv.x, -s1 * gv.y, c1 * gv.y, s1 * gv.x);
      nr_pr[tid] = make_float2(c1, s1);
    }
    // Q must have arrived before the first gather is issued: the compiler
    // does not count the gathers (inline asm), so a wait it placed for Q
    // later on would also drain every gather in flight
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) asm volatile("" ::"v"(qB[ks][hb]));
  }
  // NRQ: the back-rotation by -t of this lane's output column in block nb
  // (dimension d = 256 dh + 32 nb + l % 32, the accumulator's column) as
  // x' = x c + x_partner s', the pair partner held by lane l ^ 1: (c, s') =
  // (cos, +sin) on the pair's first dimension, (cos, -sin) on its second,
  // (1, 0) outside the rotated dimensions
  auto rot_coef = [&](int nb) -> float2 {
    // the lane number recomputed here (mbcnt), so that nothing derived from
    // it stays live through the main loop for this use
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const float2 r = nr_pr[128 * dh_u + 16 * nb + ((ln & 31) >> 1)];
    return make_float2(r.x, (ln & 1) ? -r.y : r.y);
  };
  auto unrotate = [](float x, float2 cs) -> float {
    // quad permutation (1, 0, 3, 2): the value of lane l ^ 1
    const float y = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
    return fmaf(y, cs.y, x * cs.x);
  };
  int64_t nsel = 0;
  if (DENSE) {
    nsel = vis;
  } else {
#pragma unroll
    for (int u = 0; u < NR; ++u) nsel += sm.cnt[u][0] + sm.cnt[u][1] + sm.cnt[u][2] + sm.cnt[u][3];
    if (nsel > kMaxSel) nsel = kMaxSel;
  }
  const int64_t wlo = t - n_win + 1 > 0 ? t - n_win + 1 : 0;
  const int64_t N = nsel + (t - wlo + 1);
  // this workgroup's part of the entry list (all of it when nsplit = 1)
  const int64_t per = (N + nsplit - 1) / nsplit;
  const int64_t jb = (int64_t)split * per;
  const int64_t je = jb + per < N ? jb + per : N;
  const int ntiles = je > jb ? (int)((je - jb + kT - 1) / kT) : 0;
  if (DENSE && PG) {
    // this split's compressed entries as pool rows (the host keeps a split
    // within kMaxSel entries)
    int64_t ce = je < nsel ? je : nsel;
    if (ce > jb + kMaxSel) ce = jb + kMaxSel;
    for (int64_t j = jb + tid; j < ce; j += 64 * NW) sm.sel[j - jb] = (int32_t)(er.at(bi, j, kC) / kC);
  }

  const bf16_t* cbase = PG ? Ccomp : Ccomp + bi * cbs;
  const bf16_t* rbase = PG ? kv_raw + er.req(bi) * rbs : kv_raw + bi * rbs + (wlo - raw_pos0) * (int64_t)kC;
  // paged: ring slot of the first window row; window row e (< n_win <= ring)
  // sits at slot wslot0 + e, wrapped once
  const int ring_i = PG ? (int)ring : 1;
  const int wslot0 = PG ? (int)(wlo % ring) : 0;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int jbi = (int)jb, jei = (int)je, nseli = (int)nsel;
  const int grow = s16 ^ tile_swz(g4);   // tile row this lane fetches
  auto issue_tile = [&](int ti, unsigned char* buf) {
    const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)buf);
    int j = jbi + ti * kT + grow;
    if (j >= jei) j = jbi;
    int selj = j;
    if (!DENSE || PG) {
      const int si = j < nseli ? (DENSE ? j - jbi : j) : 0;
      const uint32_t a = (uint32_t)(uintptr_t)&sm.sel[si];
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(selj) : "v"(a));
    }
    const int e = j < nseli ? selj : j - nseli;
    int we = e;
    if (PG) {
      we = wslot0 + e;
      we = we >= ring_i ? we - ring_i : we;
    }
    const bf16_t* p = (j < nseli ? cbase + (int64_t)e * kC : rbase + (int64_t)we * kC) + 8 * g4;
#if CSA_DEBUG
    if (!PG) {
      const bool bad = j < nseli ? (e < 0 || e >= n_comp || e >= csa_dbg_entry_limit) : (we < 0 || we > t - wlo);
      if (bad) {
        atomicOr(&csa_dbg_oob, 1u);
        p = rbase + (t - wlo) * (int64_t)kC + 8 * g4;
      }
    }
#endif
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int b = wave_u + rr * NW;
      attn_dma16(p + 32 * b, lbase + (uint32_t)(b * kBlkB));
    }
  };

  const int sA = g4 * 256 + ((s16 ^ tile_swz(g4)) * 16) + kBlkB * 8 * dh;
  const int cpart = 2 * (g4 & 1) + ((s16 & 3) >> 1);
  auto trbase = [&](int row) { return cpart * 256 + ((row ^ tile_swz(cpart)) * 16) + 8 * (s16 & 1); };
  const int trB0 = trbase(8 * half + (s16 >> 2)) + kBlkB * 8 * dh;
  const int trB1 = trbase(8 * half + 4 + (s16 >> 2)) + kBlkB * 8 * dh;

  constexpr float kLogHeadroom = 64.f;
  const float sl2 = scale * kLog2e;
  f32x16 o[8];
  float m_ref[2] = {-INFINITY, -INFINITY}, m_seen[2] = {-INFINITY, -INFINITY};
  float l_part = 0.f;

  // partial S^T of one tile over this wave's 256 dimensions
  auto s_part = [&](const unsigned char* B, f32x4 (&sp)[2]) {
    f32x4 c0 = (f32x4){}, c1 = (f32x4){};
    const unsigned char* a = B + sA;
    constexpr int D = 2;
    bf16x8 av[D + 1];
#pragma unroll
    for (int u = 0; u < D; ++u) av[u] = *reinterpret_cast<const bf16x8*>(a + kBlkB * u);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + D < 8) av[(ks + D) % (D + 1)] = *reinterpret_cast<const bf16x8*>(a + kBlkB * (ks + D));
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks % (D + 1)], qB[ks][0], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks % (D + 1)], qB[ks][1], c1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
#pragma unroll
    for (int ks = 0; ks < 8 - D; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * D, 0);
    sp[0] = c0;
    sp[1] = c1;
  };
  auto put_part = [&](const f32x4 (&sp)[2]) {
    unsigned char* x = XB + wave * kXB + 16 * l;
    *reinterpret_cast<f32x4*>(x) = sp[0];
    *reinterpret_cast<f32x4*>(x + 1024) = sp[1];
  };
  auto add_partner = [&](f32x4 (&sp)[2]) {
    const unsigned char* x = XB + (wave ^ 2) * kXB + 16 * l;
    sp[0] += *reinterpret_cast<const f32x4*>(x);
    sp[1] += *reinterpret_cast<const f32x4*>(x + 1024);
  };
  // Softmax without rescaling O.  VALU instructions cannot operate on the
  // accumulation registers, so an online max that rescales O every time it
  // grows would force O out of them.  Instead each head keeps a fixed
  // reference m_ref (log2 domain), set from its first valid logits; weights
  // 2^(s - m_ref) are exact relative values and may exceed 1.  Should a later
  // logit exceed m_ref by more than kLogHeadroom (weights up to 2^64; the
  // float32 range stops at 2^128), the workgroup runs this query's entries
  // again with m_ref raised to the largest logit seen -- a rare, exact
  // fallback.  A lane holds logits of two heads (16-head blocks hb = 0, 1);
  // all four lanes that hold a head agree on its m_ref.
  // Weights of tile ti from its full S^T:
  auto weights = [&](int ti, const f32x4 (&sacc)[2]) -> bf16x8 {
    const int rem0 = jei - (jbi + ti * kT);
    const int rem = rem0 < 0 ? 0 : (rem0 < kT ? rem0 : kT);
    float sv[2][4], tmax[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      tmax[hb] = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int loc = 4 * g4 + r;
        sv[hb][r] = loc < rem ? sacc[hb][r] * sl2 : -INFINITY;
        tmax[hb] = fmaxf(tmax[hb], sv[hb][r]);
      }
      m_seen[hb] = fmaxf(m_seen[hb], tmax[hb]);
    }
    if (__builtin_amdgcn_ballot_w64(m_ref[0] == -INFINITY || m_ref[1] == -INFINITY)) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float x = fmaxf(tmax[hb], __uint_as_float(from_lane_xor16(__float_as_uint(tmax[hb]), up16)));
        x = half_max(x);
        if (m_ref[hb] == -INFINITY) m_ref[hb] = x;
      }
    }
    uint32_t pk[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float mb = (m_ref[hb] == -INFINITY) ? 0.f : m_ref[hb];
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sv[hb][r] - mb);
        const float p1 = __builtin_amdgcn_exp2f(sv[hb][r + 1] - mb);
        pk[hb][r >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t));
      }
    }
    uint32_t own[2], lo[2], hi[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      own[i] = up16 ? pk[1][i] : pk[0][i];
      const uint32_t recv = from_lane_xor16(up16 ? pk[0][i] : pk[1][i], up16);
      lo[i] = up16 ? recv : own[i];
      hi[i] = up16 ? own[i] : recv;
    }
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float rs = l_part;
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lo[0]), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lo[1]), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hi[0]), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hi[1]), ones, rs, false);
    l_part = rs;
    return __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], hi[0], hi[1]));
  };
  // O[head][dim] += P E over this wave's 8 column blocks
  auto pv_part = [&](const unsigned char* B, bf16x8 pa, bool first) {
    // pa may come straight from VALU code (the last step has no S product
    // in between) and the asm MFMAs below are opaque to the compiler's
    // hazard checks: wait out the VALU-write / MFMA-read hazard here (pa is
    // an operand, so its producers stay above the wait)
    asm volatile("s_nop 4" : "+v"(pa));
    bf16x4 tr[3][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      tr[u][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(B + trB0 + kBlkB * u));
      tr[u][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(B + trB1 + kBlkB * u));
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      if (nb + 2 < 8) {
        tr[(nb + 2) % 3][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(B + trB0 + kBlkB * (nb + 2)));
        tr[(nb + 2) % 3][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(B + trB1 + kBlkB * (nb + 2)));
      }
      const bf16x8 bv = __builtin_shufflevector(tr[nb % 3][0], tr[nb % 3][1], 0, 1, 2, 3, 4, 5, 6, 7);
      if (first)
        mfma_first(o[nb], pa, bv);
      else
        mfma_acc(o[nb], pa, bv);
    }
    // the queued products may still read pa: keep its registers until they have
    asm volatile("s_nop 7" ::"v"(pa));
  };
  // step i: tile i in Bc (waited for here), tile i+1 in flight, tile i+2
  // gathered into Bf, whose previous tile (i-1) every wave has finished once
  // past the first barrier; the second barrier publishes the partial S^T
  // (first: the first tile, whose P V product starts O; a constant at each
  // call, so that O's first definition is one asm statement)
  auto step = [&](int i, const unsigned char* Bc, unsigned char* Bf, bool first) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<R>();
    tile_barrier();
    issue_tile(i + 2, Bf);
    f32x4 sp[2];
    s_part(Bc, sp);
    put_part(sp);
    tile_barrier();
    add_partner(sp);
    const bf16x8 pa = weights(i, sp);
    pv_part(Bc, pa, first);
    __builtin_amdgcn_sched_barrier(0);
  };

  __syncthreads();
  int gen = 0;
  issue_tile(0, T0);
  issue_tile(1, T1);
  if (NRQ) {
    // the query's norm and rotation while the first two tiles are gathered:
    // this wave's sum of squares of each of its heads over its 256 dimensions
    // (bf16 pairs squared and summed in float32 by the dot instruction)
    float ss[2] = {0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const uint4 w = __builtin_bit_cast(uint4, qB[ks][hb]);
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2_t pr = __builtin_bit_cast(bf16x2_t, wv[i]);
          ss[hb] = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss[hb], false);
        }
      }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      ss[hb] += __uint_as_float(from_lane_xor16(__float_as_uint(ss[hb]), up16));
      ss[hb] = half_sum(ss[hb]);
      if (g4 == 0) nr_ss[wave][16 * hb + s16] = ss[hb];
    }
    tile_barrier();   // not a fence: the first gathers stay in flight
    float inv[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      // both dimension halves' sums, in a fixed order
      const float tot = nr_ss[hw][16 * hb + s16] + nr_ss[hw + 2][16 * hb + s16];
      inv[hb] = 1.f / sqrtf(tot / (float)kC + eps);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int d0 = 256 * dh + 32 * ks + 8 * g4;
      // this lane's eight dimensions' coefficients, read in one batch
      // (issued in order: the compiler would hoist every group's reads ahead
      // of the products and run out of registers)
      f32x4 ab[4];
      const uint32_t ta = (uint32_t)(uintptr_t)&nr_ab[d0];
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %4 offset:16\n\t"
          "ds_read_b128 %2, %4 offset:32\n\t"
          "ds_read_b128 %3, %4 offset:48\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(ab[0]), "=&v"(ab[1]), "=&v"(ab[2]), "=&v"(ab[3])
          : "v"(ta)
          : "memory");
      // q'[d] = inv (q[d] A_d + q[d ^ 1] B_d); B = 0 outside the rotated
      // dimensions, whose blocks skip that product
      auto norm_rot = [&](auto rot) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          float u[8], v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = (float)qB[ks][hb][i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (decltype(rot)::value) {
              v[2 * j] = inv[hb] * fmaf(u[2 * j + 1], ab[j][1], u[2 * j] * ab[j][0]);
              v[2 * j + 1] = inv[hb] * fmaf(u[2 * j], ab[j][3], u[2 * j + 1] * ab[j][2]);
            } else {
              v[2 * j] = inv[hb] * (u[2 * j] * ab[j][0]);
              v[2 * j + 1] = inv[hb] * (u[2 * j + 1] * ab[j][2]);
            }
          }
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){v[2 * i], v[2 * i + 1]}, bf16x2_t));
          qB[ks][hb] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
      };
      if (rotated_block(ks))
        norm_rot(std::true_type{});
      else
        norm_rot(std::false_type{});
    }
  }
  for (;;) {
    l_part = 0.f;
    if (ntiles > 0) step(0, T0, T2, true);
    for (int it = 1; it < ntiles; it += 3) {
      step(it, T1, T0, false);
      if (it + 1 >= ntiles) break;
      step(it + 1, T2, T1, false);
      if (it + 2 >= ntiles) break;
      step(it + 2, T0, T2, false);
    }
    wait_vm<0>();   // the look-ahead gathers past the last tile
    o_hazard_pad();
    bool over = false;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float x = fmaxf(m_seen[hb], __uint_as_float(from_lane_xor16(__float_as_uint(m_seen[hb]), up16)));
      x = half_max(x);
      m_seen[hb] = x;
      over |= x > m_ref[hb] + kLogHeadroom;
    }
    if (over) sm.gen = gen + 1;
    __syncthreads();
    if (sm.gen == gen) break;
    ++gen;
    m_ref[0] = m_seen[0];
    m_ref[1] = m_seen[1];
    // again from the first tile
    issue_tile(0, T0);
    issue_tile(1, T1);
  }
  const float m_run = up16 ? m_ref[1] : m_ref[0];
  const float l_run = half_sum(l_part);
  if (SPLIT) {
    // partial state of this split: O over this wave's dimensions, and (once
    // per head, from the first dimension half) the maximum and the sum
    const int64_t slot = ((bi * n_q + rq) * (n_h / kHG) + hg) * nsplit + split;
    float* po = part_o + slot * (int64_t)kHG * kC + (int64_t)kHW * hw * kC + 256 * dh + (l & 31);
    // an empty split (no tiles: O was never written) leaves O = 0 and a
    // maximum of -inf, which the combine weighs with 0
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const float2 cs = NRQ ? rot_coef(nb) : make_float2(1.f, 0.f);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hr = 8 * (r >> 2) + 4 * half + (r & 3);
        const float x = rotated_block(nb) ? unrotate(o[nb][r], cs) : o[nb][r];
        po[hr * (int64_t)kC + nb * 32] = ntiles > 0 ? x : 0.f;
      }
    }
    if (dh == 0 && l < 32) {
      part_ml[(slot * kHG + kHW * hw + l) * 2 + 0] = m_run;
      part_ml[(slot * kHG + kHW * hw + l) * 2 + 1] = l_run;
    }
    return;
  }
  if (l < 32) {
    const float z2 = sink[head0 + l] * kLog2e;
    const float Mf = fmaxf(m_run, z2);
    const float fac = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - Mf);
    sm.bc[wave][l] = fac / (l_run * fac + __builtin_amdgcn_exp2f(z2 - Mf));
  }
  __syncthreads();   // every wave is done with the tile and exchange buffers; bc is visible
  float4 g4v[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) g4v[g] = *reinterpret_cast<const float4*>(&sm.bc[wave][8 * g + 4 * half]);
  unsigned char* stg = wave == 0 ? T0 : wave == 1 ? T1 : wave == 2 ? T2 : XB;
  bf16_t* ob = out + ((bi * n_q + rq) * n_h + head0) * (int64_t)kC + 256 * dh;
  // two passes of 16 head rows (8 KiB of staging each)
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int nb8 = 0; nb8 < 8; ++nb8) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * pass + gg;
        const float gv[4] = {g4v[g].x, g4v[g].y, g4v[g].z, g4v[g].w};
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int hr = 8 * g + 4 * half + i;   // head row; staged at hr - 16 pass
          float x0 = o[nb8][4 * g + i] * gv[i], x1 = o[nb8][4 * g + i + 1] * gv[i + 1];
          if (rotated_block(nb8)) {
            // read where used: coefficients held across the passes would
            // push live values to scratch
            const float2 cs = rot_coef(nb8);
            x0 = unrotate(x0, cs);
            x1 = unrotate(x1, cs);
          }
          const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x0, x1}, bf16x2_t));
          const int byte = ((nb8 * 32 + (l & 31)) * 2) ^ (((hr >> 2) & 1) << 6);
          *reinterpret_cast<uint16_t*>(stg + (hr - 16 * pass) * kStageRowB + byte) = (uint16_t)pk;
          *reinterpret_cast<uint16_t*>(stg + (hr + 1 - 16 * pass) * kStageRowB + byte) = (uint16_t)(pk >> 16);
        }
      }
    }
    // the staging area is private to this wave: its own writes are ordered
    // before its reads
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cidx = l + 64 * i;
      const int hs = cidx >> 5, c16 = cidx & 31;   // staged row, 16-byte chunk
      const int hr = hs + 16 * pass;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + hs * kStageRowB + ((c16 * 16) ^ (((hr >> 2) & 1) << 6)));
      *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(ob + hr * (int64_t)kC) + c16 * 16) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Backward of the attention, per query (bf16, c = 512, 64-head groups): the
// softmax statistics, p_j and dl_j of every entry slot, dq and the sink's dz
// (the entry gradients follow from p and dl in a separate step; p and dl
// are stored [row][slot][head]).  With l_j =
// scale q.e_j, dP_j = g.e_j, o = sum_j p_j e_j and g.o = sum_j p_j dP_j:
//   dl_j = p_j (dP_j - g.o),  dq = scale sum_j dl_j e_j,  dz = -p_z g.o.
// Same workgroup shape, tiles and gathers as attend_ds: four waves, wave w
// owning heads 32 (w & 1) .. +31 and dimensions 256 (w >> 1) .. +255.  Each
// wave holds Q and G (= dL/do) of its heads over its dimensions as MFMA
// operands; per tile it forms partial S^T = E Q^T and dP^T = E G^T over its
// dimensions and adds its partner's through LDS.  Slots are taken in order,
// 16 per tile (slot j < ks: the j-th listed entry -- CSA: idx[t][j], valid
// when 0 <= idx < visible; HCA: entry j, valid when j < visible --; slot
// ks + i: window row wlo(t) + i, valid when <= t); invalid slots get p = dl
// = 0 and gather the query's own row.  Pass 1 accumulates the maximum, the
// denominator and sum_j exp(l_j - max) dP_j per head; pass 2 forms p and dl,
// stores them and accumulates dq on the 32x32x16 MFMA, dl split into a bf16
// high part and a bf16 remainder so that the product keeps about 16 bits.
// ---------------------------------------------------------------------------
struct BwdSmem {
  int32_t sel[kMaxSel];   // CSA: idx[t][j], or -1 where not a valid entry
};
constexpr int kXB2 = 2 * kXB;   // one wave's partial S^T and dP^T

template <int DENSE>
__global__ __launch_bounds__(256) void attend_bwd_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Ccomp, int64_t cbs, const int32_t* __restrict__ idx,
    const bf16_t* __restrict__ kv_raw, int64_t rbs, int64_t raw_pos0, const float* __restrict__ sink,
    const bf16_t* __restrict__ dout, int64_t n_q, int64_t t0, int64_t n_comp, int n_h, int64_t k, int64_t m,
    int64_t n_win, int64_t ks, int64_t nslot, float scale, float* __restrict__ P, float* __restrict__ DL,
    float* __restrict__ dq, float* __restrict__ dz) {
  constexpr int NW = 4;
  constexpr int R = kT / NW;
  __shared__ BwdSmem sm;
  __shared__ __attribute__((aligned(16))) unsigned char T0[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char T1[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char T2[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char XB[NW * kXB2];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int half = l >> 5;
  const int g4 = l >> 4;
  const bool up16 = (l & 16) != 0;
  const int s16 = l & 15;
  const int hw = wave & 1;
  const int dh = wave >> 1;
  const int64_t rq = blockIdx.x;
  const int hg = blockIdx.y;
  const int64_t bi = blockIdx.z;
  const int64_t t = t0 + rq;
  const int head0 = kHG * hg + kHW * hw;
  int64_t vis = (t + 1) / m;
  if (vis > n_comp) vis = n_comp;
  const int64_t wlo = t - n_win + 1 > 0 ? t - n_win + 1 : 0;
  if (!DENSE) {
    const int32_t* ir = idx + (bi * n_q + rq) * k;
    for (int64_t j = tid; j < k; j += 64 * NW) {
      const int32_t v = ir[j];
      sm.sel[j] = (v >= 0 && v < vis) ? v : -1;
    }
  }
  bf16x8 qB[8][2], gB[8][2];
  {
    const int64_t off = ((bi * n_q + rq) * n_h + head0 + s16) * (int64_t)kC + 256 * dh + 8 * g4;
#pragma unroll
    for (int ks2 = 0; ks2 < 8; ++ks2)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        qB[ks2][hb] = *reinterpret_cast<const bf16x8*>(q + off + hb * 16 * kC + ks2 * 32);
        gB[ks2][hb] = *reinterpret_cast<const bf16x8*>(dout + off + hb * 16 * kC + ks2 * 32);
      }
    // the operands must have arrived before the first gather is issued (the
    // compiler does not count the gathers)
#pragma unroll
    for (int ks2 = 0; ks2 < 8; ++ks2)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) asm volatile("" ::"v"(qB[ks2][hb]), "v"(gB[ks2][hb]));
  }
  __syncthreads();   // sel

  const int ntiles = (int)((nslot + kT - 1) / kT);
  const bf16_t* cbase = Ccomp + bi * cbs;
  const bf16_t* rbase = kv_raw + bi * rbs;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int grow = s16 ^ tile_swz(g4);
  // the row slot j reads, or -1 for an invalid slot
  auto slot_row = [&](int64_t j, bool& comp) -> int64_t {
    comp = j < ks;
    if (j >= nslot) return -1;
    if (comp) {
      if (DENSE) return j < vis ? j : -1;
      return (int64_t)sm.sel[j];
    }
    const int64_t p = wlo + (j - ks);
    return p <= t ? p : -1;
  };
  auto issue_tile = [&](int ti, unsigned char* buf) {
    const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)buf);
    bool comp;
    const int64_t e = slot_row((int64_t)ti * kT + grow, comp);
    const bf16_t* p = (e < 0 ? rbase + (t - raw_pos0) * (int64_t)kC
                             : (comp ? cbase + e * kC : rbase + (e - raw_pos0) * (int64_t)kC)) + 8 * g4;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int b = wave_u + rr * NW;
      attn_dma16(p + 32 * b, lbase + (uint32_t)(b * kBlkB));
    }
  };

  const int sA = g4 * 256 + ((s16 ^ tile_swz(g4)) * 16) + kBlkB * 8 * dh;
  const int cpart = 2 * (g4 & 1) + ((s16 & 3) >> 1);
  auto trbase = [&](int row) { return cpart * 256 + ((row ^ tile_swz(cpart)) * 16) + 8 * (s16 & 1); };
  const int trB0 = trbase(8 * half + (s16 >> 2)) + kBlkB * 8 * dh;
  const int trB1 = trbase(8 * half + 4 + (s16 >> 2)) + kBlkB * 8 * dh;
  const float sl2 = scale * kLog2e;
  f32x16 o[8];

  // partial S^T and dP^T of one tile over this wave's 256 dimensions
  auto sd_part = [&](const unsigned char* B, f32x4 (&sp)[2], f32x4 (&dp)[2]) {
    f32x4 c0 = (f32x4){}, c1 = (f32x4){}, c2 = (f32x4){}, c3 = (f32x4){};
    const unsigned char* a = B + sA;
    constexpr int D = 2;
    bf16x8 av[D + 1];
#pragma unroll
    for (int u = 0; u < D; ++u) av[u] = *reinterpret_cast<const bf16x8*>(a + kBlkB * u);
#pragma unroll
    for (int ks2 = 0; ks2 < 8; ++ks2) {
      if (ks2 + D < 8) av[(ks2 + D) % (D + 1)] = *reinterpret_cast<const bf16x8*>(a + kBlkB * (ks2 + D));
      const bf16x8 x = av[ks2 % (D + 1)];
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qB[ks2][0], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qB[ks2][1], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, gB[ks2][0], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, gB[ks2][1], c3, 0, 0, 0);
    }
    sp[0] = c0;
    sp[1] = c1;
    dp[0] = c2;
    dp[1] = c3;
  };
  auto exchange = [&](f32x4 (&sp)[2], f32x4 (&dp)[2]) {
    unsigned char* x = XB + wave * kXB2 + 16 * l;
    *reinterpret_cast<f32x4*>(x) = sp[0];
    *reinterpret_cast<f32x4*>(x + 1024) = sp[1];
    *reinterpret_cast<f32x4*>(x + 2048) = dp[0];
    *reinterpret_cast<f32x4*>(x + 3072) = dp[1];
    tile_barrier();
    const unsigned char* y = XB + (wave ^ 2) * kXB2 + 16 * l;
    sp[0] += *reinterpret_cast<const f32x4*>(y);
    sp[1] += *reinterpret_cast<const f32x4*>(y + 1024);
    dp[0] += *reinterpret_cast<const f32x4*>(y + 2048);
    dp[1] += *reinterpret_cast<const f32x4*>(y + 3072);
  };
  // validity of this lane's 4 slots of tile ti (slots 16 ti + 4 (l/16) + r)
  auto valid4 = [&](int ti, bool (&v)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bool comp;
      v[r] = slot_row((int64_t)ti * kT + 4 * g4 + r, comp) >= 0;
    }
  };
  // one pass over the tiles; body(i, Bc, sp, dp, first) runs after the
  // exchange (first: a constant at each call, true for tile 0 only)
  auto run_pass = [&](auto&& body) {
    issue_tile(0, T0);
    issue_tile(1, T1);
    auto step = [&](int i, const unsigned char* Bc, unsigned char* Bf, bool first) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<R>();
      tile_barrier();
      issue_tile(i + 2, Bf);
      f32x4 sp[2], dp[2];
      sd_part(Bc, sp, dp);
      exchange(sp, dp);
      body(i, Bc, sp, dp, first);
      __builtin_amdgcn_sched_barrier(0);
    };
    step(0, T0, T2, true);   // ntiles >= 1: the query's own window row
    for (int it = 1; it < ntiles; it += 3) {
      step(it, T1, T0, false);
      if (it + 1 >= ntiles) break;
      step(it + 1, T2, T1, false);
      if (it + 2 >= ntiles) break;
      step(it + 2, T0, T2, false);
    }
    wait_vm<0>();
    tile_barrier();   // every wave is done with the buffers before they are reused
  };

  // pass 1: per lane and head block, running max (log2 domain), sum of
  // weights and sum of weights times dP over the lane's slots
  float mx[2] = {-INFINITY, -INFINITY}, den[2] = {0.f, 0.f}, acc[2] = {0.f, 0.f};
  run_pass([&](int i, const unsigned char*, f32x4 (&sp)[2], f32x4 (&dp)[2], bool) {
    bool v[4];
    valid4(i, v);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float lg[4], tm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lg[r] = v[r] ? sp[hb][r] * sl2 : -INFINITY;
        tm = fmaxf(tm, lg[r]);
      }
      const float nm = fmaxf(mx[hb], tm);
      if (nm != -INFINITY) {
        const float f = __builtin_amdgcn_exp2f(mx[hb] - nm);   // 0 while mx is -inf
        float sw = 0.f, swd = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float w = __builtin_amdgcn_exp2f(lg[r] - nm);
          sw += w;
          swd = fmaf(w, dp[hb][r], swd);
        }
        den[hb] = den[hb] * f + sw;
        acc[hb] = acc[hb] * f + swd;
        mx[hb] = nm;
      }
    }
  });
  // combine the four lanes that hold a head (l, l ^ 16, l ^ 32, l ^ 48),
  // then add the sink: final max Mf, denominator Lt, g.o per head block
  float Mf[2], Lt[2], go[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float m2, d2, a2;
      if (st == 0) {
        m2 = __uint_as_float(from_lane_xor16(__float_as_uint(mx[hb]), up16));
        d2 = __uint_as_float(from_lane_xor16(__float_as_uint(den[hb]), up16));
        a2 = __uint_as_float(from_lane_xor16(__float_as_uint(acc[hb]), up16));
      } else {
        const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[hb]), __float_as_uint(mx[hb]), false, false);
        const auto rd = __builtin_amdgcn_permlane32_swap(__float_as_uint(den[hb]), __float_as_uint(den[hb]), false, false);
        const auto ra = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[hb]), __float_as_uint(acc[hb]), false, false);
        // {x[l & ~32], x[l | 32]}: the other half's value
        m2 = __uint_as_float(half ? rm[0] : rm[1]);
        d2 = __uint_as_float(half ? rd[0] : rd[1]);
        a2 = __uint_as_float(half ? ra[0] : ra[1]);
      }
      const float nm = fmaxf(mx[hb], m2);
      const float f1 = nm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx[hb] - nm);
      const float f2 = nm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - nm);
      den[hb] = den[hb] * f1 + d2 * f2;
      acc[hb] = acc[hb] * f1 + a2 * f2;
      mx[hb] = nm;
    }
    const float z2 = sink[head0 + 16 * hb + s16] * kLog2e;
    Mf[hb] = fmaxf(mx[hb], z2);
    const float f = mx[hb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx[hb] - Mf[hb]);
    const float pz = __builtin_amdgcn_exp2f(z2 - Mf[hb]);
    Lt[hb] = den[hb] * f + pz;
    go[hb] = acc[hb] * f / Lt[hb];
    if (dh == 0 && g4 == 0)
      dz[(bi * n_q + rq) * n_h + head0 + 16 * hb + s16] = -(pz / Lt[hb]) * go[hb];
  }

  // pass 2: p and dl of every slot, stored, and dq += dl E
  const float inv[2] = {1.f / Lt[0], 1.f / Lt[1]};
  auto pack2 = [](float a, float b) -> uint32_t {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
  };
  // A operand of the 32x32x16 MFMA (head l%32, entries 8(l/32)..+7) from this
  // lane's values of its 4 entries of both head blocks (as in attend_ds)
  auto a_operand = [&](const uint32_t (&pk)[2][2]) -> bf16x8 {
    uint32_t own[2], lo[2], hi[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      own[i] = up16 ? pk[1][i] : pk[0][i];
      const uint32_t recv = from_lane_xor16(up16 ? pk[0][i] : pk[1][i], up16);
      lo[i] = up16 ? recv : own[i];
      hi[i] = up16 ? own[i] : recv;
    }
    return __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], hi[0], hi[1]));
  };
  run_pass([&](int i, const unsigned char* Bc, f32x4 (&sp)[2], f32x4 (&dp)[2], bool first) {
    bool v[4];
    valid4(i, v);
    uint32_t hiw[2][2], low[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float pr[4], dl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = v[r] ? __builtin_amdgcn_exp2f(sp[hb][r] * sl2 - Mf[hb]) * inv[hb] : 0.f;
        dl[r] = pr[r] * (dp[hb][r] - go[hb]);
      }
      if (dh == 0) {
        // [row][slot][head]: the heads of a slot are contiguous
        const int64_t slot0 = (int64_t)i * kT + 4 * g4;
        const int64_t base = (bi * n_q + rq) * nslot;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (slot0 + r < nslot) {
            P[(base + slot0 + r) * n_h + head0 + 16 * hb + s16] = pr[r];
            DL[(base + slot0 + r) * n_h + head0 + 16 * hb + s16] = dl[r];
          }
      }
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const uint32_t h2 = pack2(dl[r], dl[r + 1]);
        hiw[hb][r >> 1] = h2;
        low[hb][r >> 1] = pack2(dl[r] - __uint_as_float(h2 << 16), dl[r + 1] - __uint_as_float(h2 & 0xffff0000u));
      }
    }
    bf16x8 ah = a_operand(hiw), al = a_operand(low);
    // the operands come from VALU code just above, and the asm MFMAs below
    // are opaque to the compiler's hazard checks
    asm volatile("s_nop 4" : "+v"(ah), "+v"(al));
    bf16x4 tr[3][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      tr[u][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Bc + trB0 + kBlkB * u));
      tr[u][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Bc + trB1 + kBlkB * u));
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      if (nb + 2 < 8) {
        tr[(nb + 2) % 3][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Bc + trB0 + kBlkB * (nb + 2)));
        tr[(nb + 2) % 3][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Bc + trB1 + kBlkB * (nb + 2)));
      }
      const bf16x8 bv = __builtin_shufflevector(tr[nb % 3][0], tr[nb % 3][1], 0, 1, 2, 3, 4, 5, 6, 7);
      if (first)
        mfma_first(o[nb], ah, bv);
      else
        mfma_acc(o[nb], ah, bv);
      mfma_acc(o[nb], al, bv);
    }
    // the queued products may still read ah and al
    asm volatile("s_nop 7" ::"v"(ah), "v"(al));
  });
  o_hazard_pad();
  // dq = scale * O over this wave's heads and dimensions
  float* dqp = dq + ((bi * n_q + rq) * n_h + head0) * (int64_t)kC + 256 * dh + (l & 31);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hr = 8 * (r >> 2) + 4 * half + (r & 3);
      dqp[hr * (int64_t)kC + nb * 32] = scale * o[nb][r];
    }
}

// Entry contributions of one query (64 heads, bf16, c = 512):
//   contrib[t][j][:] = sum_h p[t][j][h] g_h + scale dl[t][j][h] q_h
// for every slot j, a product over the heads: A = p (and scale dl) of 32
// slots x 16 heads, split into a bf16 high part and remainder; B = G (and
// Q) of 16 heads x 32 dimensions, bf16 as given.  One workgroup per query;
// wave w owns dimensions 128 w .. +127 and keeps its B operands of all 64
// heads in registers (loaded once through LDS, transposed by the tile read
// of the attention's P V product), then walks the slots 32 at a time.
__global__ __launch_bounds__(256) void attend_bwd_contrib_mfma(const bf16_t* __restrict__ q,
                                                               const bf16_t* __restrict__ dout,
                                                               const float* __restrict__ P,
                                                               const float* __restrict__ DL, int64_t nslot,
                                                               float scale, float* __restrict__ contrib) {
  constexpr int NW = 4;
  constexpr int R = kT / NW;
  __shared__ __attribute__((aligned(16))) unsigned char GQ[8][kTileB];   // heads 16 i .. +15 of G (i < 4), Q (i >= 4)
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int half = l >> 5;
  const int g4 = l >> 4;
  const int s16 = l & 15;
  const int64_t row = (int64_t)blockIdx.z * gridDim.x + blockIdx.x;   // b * n_q + r
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int grow = s16 ^ tile_swz(g4);
  // stage: tile i holds head rows 16 (i % 4) + 0..15 of G (i < 4) or Q
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bf16_t* src = (i < 4 ? dout : q) + (row * kHG + 16 * (i & 3) + grow) * (int64_t)kC + 8 * g4;
    const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&GQ[i][0]);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int b = wave_u + rr * NW;
      attn_dma16(src + 32 * b, lbase + (uint32_t)(b * kBlkB));
    }
  }
  wait_vm<0>();
  __syncthreads();
  // B operands: column block cb = 4 w + c, heads 16 kb + 8 (l/32) .. +7
  const int cpart = 2 * (g4 & 1) + ((s16 & 3) >> 1);
  auto trbase = [&](int r) { return cpart * 256 + ((r ^ tile_swz(cpart)) * 16) + 8 * (s16 & 1); };
  const int trB0 = trbase(8 * half + (s16 >> 2)), trB1 = trbase(8 * half + 4 + (s16 >> 2));
  bf16x8 Bg[4][4], Bq[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int cb = 4 * wave + c;
      const bf16x4 g0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(&GQ[kb][0] + trB0 + kBlkB * cb));
      const bf16x4 g1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(&GQ[kb][0] + trB1 + kBlkB * cb));
      const bf16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(&GQ[4 + kb][0] + trB0 + kBlkB * cb));
      const bf16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(&GQ[4 + kb][0] + trB1 + kBlkB * cb));
      Bg[kb][c] = __builtin_shufflevector(g0, g1, 0, 1, 2, 3, 4, 5, 6, 7);
      Bq[kb][c] = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  auto split8 = [](const float (&v)[8], bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){v[2 * i], v[2 * i + 1]}, bf16x2_t));
      r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                              (f32x2_t){v[2 * i] - __uint_as_float(h[i] << 16),
                                                        v[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u)},
                                              bf16x2_t));
    }
    hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(bf16x8, make_uint4(r[0], r[1], r[2], r[3]));
  };
  for (int64_t s0 = 0; s0 < nslot; s0 += 32) {
    // A operands: slot s0 + l%32, heads 16 kb + 8 (l/32) .. +7
    const int64_t slot = s0 + (l & 31);
    const bool ok = slot < nslot;
    const float* pr = P + (row * nslot + (ok ? slot : 0)) * kHG + 8 * half;
    const float* dr = DL + (row * nslot + (ok ? slot : 0)) * kHG + 8 * half;
    f32x16 acc[4] = {};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float pv[8], dv[8];
      const float4 p0 = *reinterpret_cast<const float4*>(pr + 16 * kb);
      const float4 p1 = *reinterpret_cast<const float4*>(pr + 16 * kb + 4);
      const float4 d0 = *reinterpret_cast<const float4*>(dr + 16 * kb);
      const float4 d1 = *reinterpret_cast<const float4*>(dr + 16 * kb + 4);
      pv[0] = p0.x; pv[1] = p0.y; pv[2] = p0.z; pv[3] = p0.w; pv[4] = p1.x; pv[5] = p1.y; pv[6] = p1.z; pv[7] = p1.w;
      dv[0] = d0.x; dv[1] = d0.y; dv[2] = d0.z; dv[3] = d0.w; dv[4] = d1.x; dv[5] = d1.y; dv[6] = d1.z; dv[7] = d1.w;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = ok ? pv[i] : 0.f;
        dv[i] = ok ? scale * dv[i] : 0.f;
      }
      bf16x8 ph, pl, dh, dlo;
      split8(pv, ph, pl);
      split8(dv, dh, dlo);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, Bg[kb][c], acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl, Bg[kb][c], acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dh, Bq[kb][c], acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dlo, Bq[kb][c], acc[c], 0, 0, 0);
      }
    }
    // rows (slots) 8 (r/4) + 4 (l/32) + r%4 of column (dimension) 32 cb + l%32
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t sl = s0 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (sl < nslot) contrib[(row * nslot + sl) * kC + 32 * (4 * wave + c) + (l & 31)] = acc[c][r];
      }
  }
}

bool attend_bwd_contrib_mfma_ok(int dtype, int64_t n_h, int64_t c) { return dtype == 1 && c == kC && n_h == kHG; }

hipError_t launch_attend_bwd_contrib_mfma(const void* q, const void* dout, const float* P, const float* DL, int64_t b,
                                          int64_t n_q, int64_t nslot, float scale, float* contrib, hipStream_t st) {
  hipLaunchKernelGGL(attend_bwd_contrib_mfma, dim3((unsigned)n_q, 1u, (unsigned)b), dim3(256), 0, st,
                     (const bf16_t*)q, (const bf16_t*)dout, P, DL, nslot, scale, contrib);
  return hipGetLastError();
}

bool attend_bwd_mfma_ok(int dtype, int64_t n_h, int64_t c, int64_t k) {
  return dtype == 1 && c == kC && n_h % kHG == 0 && k <= kMaxSel;
}

hipError_t launch_attend_bwd_mfma(int dense, const void* q, const void* Ccomp, int64_t cbs, const int32_t* idx,
                                  const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink,
                                  const void* dout, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h,
                                  int64_t k, int64_t m, int64_t n_win, int64_t ks, int64_t nslot, float scale,
                                  float* P, float* DL, float* dq, float* dz, hipStream_t st) {
  const dim3 grid((unsigned)n_q, (unsigned)(n_h / kHG), (unsigned)b);
  if (dense)
    hipLaunchKernelGGL(attend_bwd_mfma<1>, grid, dim3(256), 0, st, (const bf16_t*)q, (const bf16_t*)Ccomp, cbs, idx,
                       (const bf16_t*)kv_raw, rbs, raw_pos0, sink, (const bf16_t*)dout, n_q, t0, n_comp, (int)n_h, k,
                       m, n_win, ks, nslot, scale, P, DL, dq, dz);
  else
    hipLaunchKernelGGL(attend_bwd_mfma<0>, grid, dim3(256), 0, st, (const bf16_t*)q, (const bf16_t*)Ccomp, cbs, idx,
                       (const bf16_t*)kv_raw, rbs, raw_pos0, sink, (const bf16_t*)dout, n_q, t0, n_comp, (int)n_h, k,
                       m, n_win, ks, nslot, scale, P, DL, dq, dz);
  return hipGetLastError();
}

// Merge the splits of one (query, head), then apply the sink:
//   out = sum_s O_s 2^{m_s - M} / (sum_s l_s 2^{m_s - M} + 2^{z - M}),
// M the largest of the m_s and z (log2 domain).  The first wave loads every
// split's (m_s, l_s) at once (lane s, s + 64, ...), reduces M and the
// denominator over the wave in a fixed order and leaves each split's weight
// 2^{m_s - M} in LDS (nsplit floats of dynamic LDS); then the workgroup's
// 128 threads stream the partial rows, 4 values each, in split order.
__global__ __launch_bounds__(128) void attend_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const float* __restrict__ sink, int n_h,
                                                      int nsplit, bf16_t* __restrict__ out) {
  extern __shared__ float split_w[];   // nsplit weights
  __shared__ float den_sh;
  const int tx = threadIdx.x;
  const int64_t qr = blockIdx.x;   // b * n_q + r
  const int h = blockIdx.y;
  const int hg = h / kHG, hh = h % kHG;
  const int64_t base = (qr * (n_h / kHG) + hg) * nsplit;
  const float2* ml = reinterpret_cast<const float2*>(part_ml);
  if (tx < 64) {
    float M = -INFINITY;
    for (int s = tx; s < nsplit; s += 64) M = fmaxf(M, ml[(base + s) * kHG + hh].x);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float z2 = sink[h] * kLog2e;
    const float Mf = fmaxf(M, z2);
    float L = 0.f;
    for (int s = tx; s < nsplit; s += 64) {
      const float2 v = ml[(base + s) * kHG + hh];
      // an empty split (maximum -inf) has weight 0
      const float f = (v.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(v.x - Mf);
      L = fmaf(v.y, f, L);
      split_w[s] = f;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o, 64);
    if (tx == 0) den_sh = L + __builtin_amdgcn_exp2f(z2 - Mf);
  }
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float f = split_w[s];
    const float4 v = reinterpret_cast<const float4*>(part_o + ((base + s) * kHG + hh) * (int64_t)kC)[tx];
    acc.x = fmaf(v.x, f, acc.x);
    acc.y = fmaf(v.y, f, acc.y);
    acc.z = fmaf(v.z, f, acc.z);
    acc.w = fmaf(v.w, f, acc.w);
  }
  const float inv = 1.f / den_sh;
  bf16_t* ob = out + (qr * n_h + h) * (int64_t)kC + 4 * tx;
  const uint2 pk = make_uint2((uint32_t)f2bf(acc.x * inv) | ((uint32_t)f2bf(acc.y * inv) << 16),
                              (uint32_t)f2bf(acc.z * inv) | ((uint32_t)f2bf(acc.w * inv) << 16));
  *reinterpret_cast<uint2*>(ob) = pk;
}
// splits a combine takes: its weights fill at most 64 KiB of LDS
constexpr int kCombineMaxSplits = 16384;

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static bool attend_mfma_ok(int dtype, int64_t n_h, int64_t c, int64_t k) {
  return dtype == 1 && c == kC && n_h % kHG == 0 && k <= kMaxSel;
}

#ifndef CSA_SPLIT_MIN_TILES
#define CSA_SPLIT_MIN_TILES 4
#endif
constexpr int64_t kSplitMinTiles = CSA_SPLIT_MIN_TILES;
static int attend_nsplit(int64_t b, int64_t n_q, int64_t n_h, int64_t nmax) {
  const int64_t items = b * n_q * (n_h / kHG);
  if (items >= 512) return 1;
  // about one workgroup per CU: every split also writes (and the combine
  // reads) a 128 KiB float partial, which more splits would multiply
  int64_t ns = (256 + items - 1) / items;
  // at least kSplitMinTiles tiles per split: a split pays a fixed cost (index
  // compaction, the first gathers, a 128 KiB float partial written and
  // merged again) that fewer tiles do not amortise
  const int64_t cap = (nmax + kSplitMinTiles * kT - 1) / (kSplitMinTiles * kT);
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
    // one query per workgroup (attend_ds), selected or dense lists
    const Rows none = dense_rows(cbs);
    const dim3 grid((unsigned)n_q, (unsigned)((n_h / kHG) * ns), (unsigned)b);
#define CSA_ATTEND_DS(S, D)                                                                                          \
  hipLaunchKernelGGL((attend_ds<S, 0, D, 0>), grid, dim3(256), 0, st, (const bf16_t*)q, (const bf16_t*)Ccomp, cbs,    \
                     idx, (const bf16_t*)kv_raw, rbs, raw_pos0, sink, n_q, t0, n_comp, (int)n_h, k, m, n_win, scale, \
                     ns, part_o, part_ml, (bf16_t*)out, none, (int64_t)0, (const int64_t*)nullptr,                   \
                     (const float*)nullptr, 0.f, 0, 0.0)
    if (ns == 1) {
      if (dense) CSA_ATTEND_DS(0, 1); else CSA_ATTEND_DS(0, 0);
    } else {
      if (dense) CSA_ATTEND_DS(1, 1); else CSA_ATTEND_DS(1, 0);
    }
#undef CSA_ATTEND_DS
    if (ns > 1)
      hipLaunchKernelGGL(attend_combine, dim3((unsigned)(b * n_q), (unsigned)n_h), dim3(128), ns * sizeof(float), st,
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

// CSA (dense = 0) or HCA (dense = 1) attention with the query heads' RMSNorm
// and partial RoPE applied as Q is loaded and the output turned back by -t
// before it is stored (bf16, c = 512, 64-head groups, rope_dims even and
// <= 512; the caller checked).
hipError_t launch_attend_norm_rope(int dense, const void* q, const float* gq, float eps, int64_t rope_dims,
                                   double base, const void* Ccomp, int64_t cbs, const int32_t* idx,
                                   const void* kv_raw, int64_t rbs, int64_t raw_pos0, const float* sink, int64_t b,
                                   int64_t n_q, int64_t t0, int64_t n_comp, int64_t n_h, int64_t k, int64_t m,
                                   int64_t n_win, float scale, void* ws, void* out, hipStream_t st) {
  if (b == 0 || n_q == 0) return hipSuccess;
  // the split count launch_attend takes for the same list
  int64_t vmax = (t0 + n_q) / m;
  if (vmax > n_comp) vmax = n_comp;
  const int ns = attend_nsplit(b, n_q, n_h, (dense ? vmax : k) + n_win);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (ns > 1) {
    const int64_t slots = b * n_q * (n_h / kHG) * ns;
    const size_t osz = ((size_t)slots * kHG * kC * 4 + 255) & ~(size_t)255;
    part_o = (float*)ws;
    part_ml = (float*)((unsigned char*)ws + osz);
  }
  const Rows none = dense_rows(cbs);
  const dim3 grid((unsigned)n_q, (unsigned)((n_h / kHG) * ns), (unsigned)b);
#define CSA_ATTEND_NRQ(S, D)                                                                                         \
  hipLaunchKernelGGL((attend_ds<S, 0, D, 1>), grid, dim3(256), 0, st, (const bf16_t*)q, (const bf16_t*)Ccomp, cbs,    \
                     idx, (const bf16_t*)kv_raw, rbs, raw_pos0, sink, n_q, t0, n_comp, (int)n_h, k, m, n_win, scale, \
                     ns, part_o, part_ml, (bf16_t*)out, none, (int64_t)0, (const int64_t*)nullptr, gq, eps,          \
                     (int)rope_dims, base)
  if (ns == 1) {
    if (dense) CSA_ATTEND_NRQ(0, 1); else CSA_ATTEND_NRQ(0, 0);
  } else {
    if (dense) CSA_ATTEND_NRQ(1, 1); else CSA_ATTEND_NRQ(1, 0);
  }
#undef CSA_ATTEND_NRQ
  if (ns > 1)
    hipLaunchKernelGGL(attend_combine, dim3((unsigned)(b * n_q), (unsigned)n_h), dim3(128), ns * sizeof(float), st, part_o, part_ml,
                       sink, (int)n_h, ns, (bf16_t*)out);
  return hipGetLastError();
}

// Paged decode: one query per batch row at its own position, entries via
// the block table, window rows from the request's ring.  bf16, c = 512,
// 64-head groups (the caller checked).
// Paged HCA translates a split's compressed entries into kMaxSel LDS slots,
// so it takes at least nmax / kMaxSel splits.
static int attend_paged_nsplit(int dense, int64_t b, int64_t n_h, int64_t nmax) {
  int ns = attend_nsplit(b, 1, n_h, nmax);
  const int64_t need = dense ? (nmax + kMaxSel - 1) / kMaxSel : 1;
  return ns < need ? (int)need : ns;
}

bool attend_paged_supported(int dense, int64_t b, int64_t n_h, int64_t nmax) {
  return attend_paged_nsplit(dense, b, n_h, nmax) <= kCombineMaxSplits;
}

size_t attend_paged_workspace_bytes(int dense, int64_t b, int64_t n_h, int64_t nmax) {
  const int ns = attend_paged_nsplit(dense, b, n_h, nmax);
  if (ns == 1) return 0;
  const int64_t slots = b * (n_h / kHG) * ns;
  return ((((size_t)slots * kHG * kC * 4) + 255) & ~(size_t)255) + (size_t)slots * kHG * 2 * 4;
}

hipError_t launch_attend_paged(int dense, const void* q, const void* pool, const Rows& er, const int32_t* idx,
                               const void* state, int64_t state_elems, int64_t ring, const int64_t* pos,
                               const float* sink, int64_t b, int64_t n_comp_max, int64_t n_h, int64_t k, int64_t m,
                               int64_t n_win, float scale, void* ws, void* out, hipStream_t st) {
  if (b == 0) return hipSuccess;
  const int64_t nmax = (dense ? n_comp_max : k) + n_win;
  const int ns = attend_paged_nsplit(dense, b, n_h, nmax);
  if (ns > kCombineMaxSplits) return hipErrorInvalidValue;   // the entry point rejects these first
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (ns > 1) {
    const int64_t slots = b * (n_h / kHG) * ns;
    const size_t osz = ((size_t)slots * kHG * kC * 4 + 255) & ~(size_t)255;
    part_o = (float*)ws;
    part_ml = (float*)((unsigned char*)ws + osz);
  }
  const dim3 grid(1u, (unsigned)((n_h / kHG) * ns), (unsigned)b);
#define CSA_ATTEND_DS_PG(S, D)                                                                                        \
  hipLaunchKernelGGL((attend_ds<S, 1, D, 0>), grid, dim3(256), 0, st, (const bf16_t*)q, (const bf16_t*)pool,          \
                     (int64_t)0, idx, (const bf16_t*)state, state_elems, (int64_t)0, sink, (int64_t)1, (int64_t)0,    \
                     n_comp_max, (int)n_h, k, m, n_win, scale, ns, part_o, part_ml, (bf16_t*)out, er, ring, pos,      \
                     (const float*)nullptr, 0.f, 0, 0.0)
  if (ns == 1) {
    if (dense) CSA_ATTEND_DS_PG(0, 1); else CSA_ATTEND_DS_PG(0, 0);
  } else {
    if (dense) CSA_ATTEND_DS_PG(1, 1); else CSA_ATTEND_DS_PG(1, 0);
  }
#undef CSA_ATTEND_DS_PG
  if (ns > 1)
    hipLaunchKernelGGL(attend_combine, dim3((unsigned)b, (unsigned)n_h), dim3(128), ns * sizeof(float), st, part_o, part_ml, sink,
                       (int)n_h, ns, (bf16_t*)out);
  return hipGetLastError();
}

#if CSA_DEBUG
// Wait for the stream, then read and clear the bounds flag of the gathers.
bool debug_take_oob(hipStream_t st) {
  unsigned int v = 0, z = 0;
  if (hipStreamSynchronize(st) != hipSuccess) return true;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(csa_dbg_oob), sizeof v) != hipSuccess) return true;
  if (v != 0 && hipMemcpyToSymbol(HIP_SYMBOL(csa_dbg_oob), &z, sizeof z) != hipSuccess) return true;
  return v != 0;
}
hipError_t debug_set_entry_limit(int64_t limit) {
  const long long v = (long long)limit;
  return hipMemcpyToSymbol(HIP_SYMBOL(csa_dbg_entry_limit), &v, sizeof v);
}
#endif

}  // namespace csa
