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
// per query, each owning 32 heads over all 512 dimensions (the Q operand in
// 128 VGPRs, the O accumulator in 256 AGPRs).  Entries stream through LDS in
// tiles of 16 rows that all waves of the workgroup share, gathered from
// HBM/L2 straight into LDS (global_load_lds_dwordx4, one 1 KiB row per wave
// instruction) three tiles ahead of use, into four statically distinct
// buffers, with one barrier per tile.
//
// Per tile step i and wave the work is software-pipelined:
//   S^T(i+1) = E Q^T   v_mfma_f32_16x16x32_bf16, A = 16 entry rows from LDS
//                      (ds_read_b128), B = Q^T (16 heads) from registers; two
//                      head blocks.  A lane ends up with 4 entries of each of
//                      two heads.
//   O += P(i) E(i)     v_mfma_f32_32x32x16_bf16 over the 16 entries of tile
//                      i, B = E^T read with ds_read_b64_tr_b16 (4 rows x 16
//                      columns, column-per-lane), A = P(i) in registers;
//                      the weights of tile i+1 are computed between these
//                      MFMAs, which do not depend on them.
// A lane's 32x32 A operand (head l%32, entries 8(l/32)..+7) is its own 4
// weights of that head plus the 4 held by lane l^16, exchanged with one
// v_permlane16_swap per register.  A tile is stored column-block major: the
// 64-byte column block b of all 16 rows fills 1 KiB at b * 1024, and inside
// it chunk c of row r sits at c * 256 + (r ^ 4c) * 16.  One gather
// instruction then fills one block with 16 B per lane, and with gfx950's 64
// LDS banks both the b128 row reads (16 lanes = 16 rows of one chunk) and the
// transposed reads (16 lanes = 4 rows x 4 chunks) are conflict-free.
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

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

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
// read by VALU code); O alone, 256 registers per lane, is kept in AGPRs by
// issuing its product here.  The compiler sees only an asm statement, so
// every place where compiled code touches O next to these instructions
// (zeroing before the first, reading after the last) pads with o_hazard_pad.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8 a, const bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void o_hazard_pad() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

template <int DENSE, int G>
struct AttnSmem {
  int32_t sel[DENSE ? 1 : kMaxSel];
  int32_t cnt[DENSE ? 1 : kMaxSel / 128][2];   // per-round valid counts of the compaction
  float bc[2 * G][kHW];                          // per-wave broadcast of per-head factors
  int32_t gen;                                   // restart generation (see the softmax note)
};

template <int DENSE, int G>
__global__ __launch_bounds__(128 * G) void attend_mfma_c512(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Ccomp, int64_t cbs,
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ kv_raw, int64_t rbs,
    int64_t raw_pos0, const float* __restrict__ sink, int64_t n_q, int64_t t0, int64_t n_comp,
    int n_h, int64_t k, int64_t m, int64_t n_win, float scale, int nsplit,
    float* __restrict__ part_o, float* __restrict__ part_ml, bf16_t* __restrict__ out) {
  constexpr int NW = 2 * G;        // waves per workgroup
  constexpr int R = kT / NW;       // gathered rows per wave and tile
  __shared__ AttnSmem<DENSE, G> sm;
  // four tile buffers: tile i lives in buffer i % 4
  __shared__ __attribute__((aligned(16))) unsigned char T0[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char T1[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char T2[kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char T3[kTileB];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int half = l >> 5;
  const int g4 = l >> 4;             // 16-lane group
  const bool up16 = (l & 16) != 0;   // odd 16-lane group
  const int s16 = l & 15;
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
  const int head0 = kHG * hg + kHW * hw;   // first head of this wave

  // ---- Q operand (B of the 16x16x32 MFMA): lane holds head
  //      head0 + 16*hb + l%16, dims 32*ks + 8*(l/16) + (0..7)
  bf16x8 qB[16][2];
  auto load_q = [&]() {
    const int64_t qrow = qvalid ? rq : rlast;
    const bf16_t* qp = q + ((bi * n_q + qrow) * n_h + head0 + s16) * (int64_t)kC + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        qB[ks][hb] = *reinterpret_cast<const bf16x8*>(qp + hb * 16 * kC + ks * 32);
  };

  // ---- entry list: compressed part (selected or dense), then the union of
  //      the group's causal windows
  int64_t nsel, vis_q;
  if (DENSE) {
    load_q();
    nsel = (t_last + 1) / m;
    if (nsel > n_comp) nsel = n_comp;
    vis_q = (t_q + 1) / m;
    if (vis_q > n_comp) vis_q = n_comp;
  } else {
    // G == 1: stable compaction of the valid indices (0 <= s < visible);
    // every index load is issued before the first is used
    constexpr int NT = 64 * NW;
    constexpr int NR = kMaxSel / NT;
    int64_t vis = (t_first + 1) / m;
    if (vis > n_comp) vis = n_comp;
    const int32_t* ir = idx + (bi * n_q + r0) * k;
    int32_t sv[NR];
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int64_t j = (int64_t)u * NT + tid;
      sv[u] = j < k ? ir[j] : -1;
    }
    load_q();   // in flight while the indices are compacted
    uint64_t mk[NR];
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      mk[u] = __builtin_amdgcn_ballot_w64(sv[u] >= 0 && sv[u] < vis);
      if (l == 0) sm.cnt[u][wave] = __popcll(mk[u]);
    }
    __syncthreads();
    const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
    int64_t base = 0;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int64_t pos = base + (wave ? sm.cnt[u][0] : 0) + __popcll(mk[u] & below);
      if (((mk[u] >> l) & 1) && pos < kMaxSel) sm.sel[pos] = sv[u];
      base += sm.cnt[u][0] + sm.cnt[u][1];
    }
    __syncthreads();
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
  // Gather tile ti into a buffer.  Lane l (< 16) resolves the address of
  // tile row l (rows past the split's end repeat its first entry, weight 0);
  // wave w loads rows w, w+NW, ... with the row base broadcast to scalar
  // registers, lane l fetching chunk l ^ f(row), so LDS chunk position c
  // holds row chunk c ^ f(row).  Always exactly R loads per wave.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int jbi = (int)jb, jei = (int)je, nseli = (int)nsel;
  // Tile layout in LDS (column-block major): 64-byte column block b of
  // tile row r, 16-byte chunk c of that block, lives at
  //   b * 1024 + c * 256 + ((r ^ 4c) * 16).
  // Gather: one wave instruction loads column block b of all 16 rows (lane
  // l: row (l%16) ^ 4(l/16), chunk l/16, i.e. LDS bytes b*1024 + 16 l); wave
  // w loads blocks w, w+NW, ...  Rows past the split's end repeat its first
  // entry (weight 0).  Always exactly R loads per wave and tile.
  const int grow = s16 ^ (4 * g4);   // tile row this lane fetches
  auto issue_tile = [&](int ti, unsigned char* buf) {
    int j = jbi + ti * kT + grow;
    if (j >= jei) j = jbi;
    // The selected entry is read with a self-contained asm load (it waits
    // for its own result): left to the compiler, these per-tile LDS reads
    // are hoisted across the unrolled steps, and the live ranges that
    // creates push the Q operand out of registers.  The index is clamped so
    // that every lane reads, with no branch around the load.
    int selj = j;
    if (!DENSE) {
      const uint32_t a = (uint32_t)(uintptr_t)&sm.sel[j < nseli ? j : 0];
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(selj) : "v"(a));
    }
    const int e = j < nseli ? selj : j - nseli;
    const bf16_t* p = (j < nseli ? cbase : rbase) + (int64_t)e * kC + 8 * g4;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int b = wave_u + rr * NW;
      __builtin_amdgcn_global_load_lds((const void*)(p + 32 * b), (lds_void_t*)(buf + b * kBlkB), 16, 0, 0);
    }
  };

  // per-lane LDS byte offsets inside a tile buffer (add b * 1024 for column block b)
  //   S A operand: row l%16, chunk l/16
  const int sA = g4 * 256 + ((s16 ^ (4 * g4)) * 16);
  //   P V B operand (transposed read): rows 8*half + 4*u + (l%16)/4, columns
  //   32*nb + 16*((l/16)%2) + 4*(l%4): chunk 2*((l/16)%2) + (l%4)/2 of the
  //   block, byte 8*(l%2) of the chunk
  const int cpart = 2 * (g4 & 1) + ((s16 & 3) >> 1);
  auto trbase = [&](int row) { return cpart * 256 + ((row ^ (4 * cpart)) * 16) + 8 * (s16 & 1); };
  const int trB0 = trbase(8 * half + (s16 >> 2)), trB1 = trbase(8 * half + 4 + (s16 >> 2));

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
  constexpr float kLogHeadroom = 64.f;
  const float sl2 = scale * kLog2e;
  f32x16 o[16];
  float m_ref[2] = {-INFINITY, -INFINITY}, m_seen[2] = {-INFINITY, -INFINITY};
  float l_part = 0.f;   // sum of this lane's weights of head l%32

  // S^T of one tile: 16 entries x (2 blocks of 16 heads), 4 accumulation
  // chains, row operands fetched three column blocks ahead
  auto s_tile = [&](const unsigned char* B, f32x4 (&sacc)[2]) {
    f32x4 c[2][2] = {{(f32x4){}, (f32x4){}}, {(f32x4){}, (f32x4){}}};
    const unsigned char* a = B + sA;
    constexpr int D = 3;   // column blocks read ahead
    bf16x8 av[D + 1];
#pragma unroll
    for (int u = 0; u < D; ++u) av[u] = *reinterpret_cast<const bf16x8*>(a + kBlkB * u);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (ks + D < 16) av[(ks + D) % (D + 1)] = *reinterpret_cast<const bf16x8*>(a + kBlkB * (ks + D));
      c[0][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks % (D + 1)], qB[ks][0], c[0][ks & 1], 0, 0, 0);
      c[1][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks % (D + 1)], qB[ks][1], c[1][ks & 1], 0, 0, 0);
    }
    // keep the operand reads ahead of the MFMAs that use them: left alone,
    // the scheduler sinks every read next to its use and waits on it
    __builtin_amdgcn_sched_group_barrier(0x100, D, 0);   // D LDS reads
#pragma unroll
    for (int ks = 0; ks < 16 - D; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * D, 0);
    sacc[0] = c[0][0] + c[0][1];
    sacc[1] = c[1][0] + c[1][1];
  };
  // weights of tile ti from its S^T: the A operand of the P V product
  auto weights = [&](int ti, const f32x4 (&sacc)[2]) -> bf16x8 {
    const int64_t j0 = jb + (int64_t)ti * kT;
    const int64_t remv = je - j0;
    const int rem = (int)(remv < 0 ? 0 : (remv < kT ? remv : kT));   // real entries in this tile
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
    float sv[2][4], tmax[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      tmax[hb] = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int loc = 4 * g4 + r;
        bool valid = loc < rem;
        if (DENSE) valid = valid & (loc != exA) & (loc != exW);
        sv[hb][r] = valid ? sacc[hb][r] * sl2 : -INFINITY;
        tmax[hb] = fmaxf(tmax[hb], sv[hb][r]);
      }
      m_seen[hb] = fmaxf(m_seen[hb], tmax[hb]);
    }
    if (__builtin_amdgcn_ballot_w64(m_ref[0] == -INFINITY || m_ref[1] == -INFINITY)) {
      // first valid logits of a head: its maximum over the four lanes holding it
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
    // own head block (head l%32) and the block lane l^16 needs
    uint32_t own[2], lo[2], hi[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      own[i] = up16 ? pk[1][i] : pk[0][i];
      const uint32_t recv = from_lane_xor16(up16 ? pk[0][i] : pk[1][i], up16);
      lo[i] = up16 ? recv : own[i];   // entries 8*half + 0..3
      hi[i] = up16 ? own[i] : recv;   // entries 8*half + 4..7
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
  // O[head][dim] += P[head][entry] E[entry][dim] over one tile: 16 column
  // blocks, transposed operands fetched two blocks ahead
  auto pv_tile = [&](const unsigned char* B, const bf16x8 pa) {
    bf16x4 tr[3][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      tr[u][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(B + trB0 + kBlkB * u));
      tr[u][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(B + trB1 + kBlkB * u));
    }
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      if (nb + 2 < 16) {
        tr[(nb + 2) % 3][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(B + trB0 + kBlkB * (nb + 2)));
        tr[(nb + 2) % 3][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(B + trB1 + kBlkB * (nb + 2)));
      }
      const bf16x8 bv = __builtin_shufflevector(tr[nb % 3][0], tr[nb % 3][1], 0, 1, 2, 3, 4, 5, 6, 7);
      mfma_acc(o[nb], pa, bv);
    }
  };
  // one pipeline step: tile i is in Bc with its weights in pa; tile i+1 in
  // Bn (its gather waited for here); tile i+3 is gathered into Bf, whose
  // previous tile (i-1) every wave has finished once past the barrier
  auto step = [&](int i, const unsigned char* Bc, const unsigned char* Bn, unsigned char* Bf, bf16x8& pa) {
    wait_vm<R>();
    tile_barrier();
    issue_tile(i + 3, Bf);
    f32x4 sn[2];
    s_tile(Bn, sn);
    pv_tile(Bc, pa);
    pa = weights(i + 1, sn);
  };

  if (tid == 0) sm.gen = 0;
  __syncthreads();
  int gen = 0;
  for (;;) {
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) o[nb] = (f32x16){};
    o_hazard_pad();
    l_part = 0.f;
    if (ntiles > 0) {
      issue_tile(0, T0);
      issue_tile(1, T1);
      issue_tile(2, T2);
      wait_vm<2 * R>();
      tile_barrier();
      f32x4 s0[2];
      s_tile(T0, s0);
      bf16x8 pa = weights(0, s0);
      for (int it = 0; it < ntiles; it += 4) {
        step(it, T0, T1, T3, pa);
        if (it + 1 >= ntiles) break;
        step(it + 1, T1, T2, T0, pa);
        if (it + 2 >= ntiles) break;
        step(it + 2, T2, T3, T1, pa);
        if (it + 3 >= ntiles) break;
        step(it + 3, T3, T0, T2, pa);
      }
      wait_vm<0>();   // the look-ahead gathers past the last tile
      o_hazard_pad();
    }
    // an attempt whose weights may have overflowed is discarded as a whole;
    // the decision is workgroup-wide because the waves share the tiles
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
  }
  // head l%32: block (l/16)%2 of this lane; both 32-lane halves hold half of its weights
  const float m_run = up16 ? m_ref[1] : m_ref[0];
  const float l_run = half_sum(l_part);

  if (nsplit == 1) {
    // final per-head factor e^{-M} / (sum + e^{z - M}), broadcast over the O rows
    if (l < 32) {
      const float z2 = sink[head0 + l] * kLog2e;
      const float Mf = fmaxf(m_run, z2);
      const float fac = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - Mf);
      sm.bc[wave][l] = fac / (l_run * fac + __builtin_amdgcn_exp2f(z2 - Mf));
    }
    __syncthreads();   // every wave is done with the tile buffers; bc is visible
    float4 g4v[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) g4v[g] = *reinterpret_cast<const float4*>(&sm.bc[wave][8 * g + 4 * half]);
    unsigned char* stg = wave == 0 ? T0 : wave == 1 ? T1 : wave == 2 ? T2 : T3;
    bf16_t* ob = out + ((bi * n_q + (qvalid ? rq : rlast)) * n_h + head0) * (int64_t)kC;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int nb8 = 0; nb8 < 8; ++nb8) {
        const int nb = pass * 8 + nb8;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float gv[4] = {g4v[g].x, g4v[g].y, g4v[g].z, g4v[g].w};
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            // rows hr and hr + 1 of this column, rounded to bf16 as one pair
            const int hr = 8 * g + 4 * half + i;
            const uint32_t pk = __builtin_bit_cast(
                uint32_t, __builtin_convertvector((f32x2_t){o[nb][4 * g + i] * gv[i], o[nb][4 * g + i + 1] * gv[i + 1]},
                                                  bf16x2_t));
            // rows 4 apart would share banks: flip the 64-byte half for odd row quads
            const int byte = ((nb8 * 32 + (l & 31)) * 2) ^ (((hr >> 2) & 1) << 6);
            *reinterpret_cast<uint16_t*>(stg + hr * kStageRowB + byte) = (uint16_t)pk;
            *reinterpret_cast<uint16_t*>(stg + (hr + 1) * kStageRowB + byte) = (uint16_t)(pk >> 16);
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
#pragma unroll 4
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
  // about one workgroup per CU: every split also writes (and the combine
  // reads) a 128 KiB float partial, which more splits would multiply
  int64_t ns = (256 + items - 1) / items;
  // at least eight tiles per split: a split pays a fixed cost (index
  // compaction, the first gathers, a 128 KiB float partial written and
  // merged again) that fewer tiles do not amortise
  const int64_t cap = (nmax + 8 * kT - 1) / (8 * kT);
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
    // dense lists: two consecutive queries share each workgroup's tiles (a
    // single query leaves the second pair of waves redundant; a one-query
    // instance of the kernel spills and is no faster)
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
