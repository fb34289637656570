// Lightning-indexer scoring and top-k selection.
//
// Definition: polysight "06-formulas" section B9 and AirCoding
// "deepseek-paper-analysis" section 7.1 -- for query t and compressed
// indexer key s, I[t][s] = sum over indexer heads h of
// w[t][h] * ReLU(qI[t][h] . KIcomp[s]); the query reads the k entries with
// the largest scores among those completed before it (s < (t+1)/m,
// cooking-agi "DeepSeek-V4: 压缩历史以后，还能读到什么？" section 3).
//
// Scoring is a GEMM (query heads x keys, contracted over c_I) with a fused
// ReLU * w reduction over the heads, so it runs on the MFMA unit -- bf16,
// 8-bit E4M3, or block-scaled MXFP4 operands for the low-precision indexer
// (songhuiming "DeepSeek-V4 百万 token 上下文" section 13.3, AirCoding
// section 7: the indexer's query/key path in FP4): each wave keeps its
// query's 32*NHB x c_I operand in registers and streams key tiles through
// LDS.  Selection searches the k-th largest of the
// order-preserving 32-bit images of the scores bit by bit, then compacts the
// taken elements in list order, with a fixed reduction order everywhere.
// Prefill (four or more queries, at most 2048 candidates) selects inside the
// scoring kernel; decode (few queries, long lists) bounds each row's k-th
// score from group maxima, filters, and merges; other shapes take a general
// multi-stage selection.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// LDS DMA of 16 bytes per lane: lane l's bytes land at LDS byte address
// lds + 16 l (lds is wave-uniform, passed in M0).  Written as inline asm so
// that the compiler does not track these writes: the kernels that use it
// order them with explicit vmcnt waits (wait_vmem) before reading the LDS.
// M0 is restored afterwards, since the compiler does not accept it as a
// clobber.
__device__ __forceinline__ void dma_chunk16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds) : "memory");
}
// wait until at most N vector-memory operations of this wave are in flight
// (loads, stores and LDS-DMA leave the counter in issue order on this
// architecture, so a pending store only makes such a wait stricter)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------
// Generic scoring (any dtype, any head count / dimension): one thread per
// (query, key).  Used for float32 and for shapes the MFMA kernel does not
// cover.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void index_scores_generic(
    const T* __restrict__ qI, const float* __restrict__ w, const T* __restrict__ KI,
    int64_t comp_bs, int64_t n_q, int64_t t0, int64_t n_comp, int nh, int cI, int64_t m,
    float* __restrict__ scores, int sbf) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = blockIdx.y;
  const int64_t bi = blockIdx.z;
  int64_t vis = (t0 + r + 1) / m;
  if (vis > n_comp) vis = n_comp;
  if (s >= vis) return;
  const T* q = qI + (bi * n_q + r) * (int64_t)nh * cI;
  const float* wr = w + (bi * n_q + r) * (int64_t)nh;
  const T* key = KI + bi * comp_bs + s * (int64_t)cI;
  float tot = 0.f;
  for (int h = 0; h < nh; ++h) {
    float d = 0.f;
    for (int j = 0; j < cI; ++j) d = fmaf(Elem<T>::ld(q + h * cI + j), Elem<T>::ld(key + j), d);
    tot = fmaf(wr[h], fmaxf(d, 0.f), tot);
  }
  scores[(bi * n_q + r) * n_comp + s] = sbf ? bf2f(f2bf(tot)) : tot;
}

// ---------------------------------------------------------------------------
// MFMA scoring, bf16.  NHB = heads / 32, KS = c_I / 16.  A workgroup has 4
// waves, one query each.  Key tiles of 64 rows (c_I x 2 bytes each, one
// contiguous block in HBM) stream through a three-slot LDS ring filled with
// 1 KiB LDS-DMA loads (global_load_lds_dwordx4, a quarter of each tile per
// wave) two tiles ahead, with one barrier per tile; each wave multiplies its
// query block by the 64 keys with v_mfma_f32_32x32x16_bf16 and reduces over
// heads in registers.  LDS chunk p of key row r holds source chunk p ^ f(r),
// which keeps the B operand reads free of bank conflicts.
//
// Operand layouts of the 32x32x16 MFMA (lane l, j < 8):
//   A[i][k] : lane holds A[l%32][8*(l/32) + j]
//   B[k][n] : lane holds B[8*(l/32) + j][l%32]
//   D[i][n] : lane holds D[8*(r/4) + 4*(l/32) + r%4][l%32] in register r
//
// FUSED (at most 2048 candidates): the workgroup holds every score
// of its four queries, in LDS rather than HBM, and each wave then selects
// its query's top k from there and writes the final indices (and scores), as
// the single-wave selection stage would from the score rows.
// ---------------------------------------------------------------------------
constexpr int kFusedMaxKeys = 2048;

// ---------------------------------------------------------------------------
// Single-wave selection.  The wave holds a list of up to 64 R elements: slot r
// of lane l is element 64 r + l; its key (the order-preserving image of a
// score) is 0 for an empty slot, and every finite score's key is >= 1.
// Counts are per-lane VALU sums reduced with six bit ballots, and selections
// are per-lane bit masks, so that nothing of size R lives in scalar
// registers.
// ---------------------------------------------------------------------------
// Wave sum of a per-lane count below 64.
__device__ __forceinline__ uint32_t wave_sum_small(uint32_t c) {
  uint32_t t = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b) t += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64((c >> b) & 1u)) << b;
  return t;
}
// Keys >= cand over the wave (cand >= 1, so empty slots never count).
template <int R>
__device__ __forceinline__ uint32_t wave_count_ge(const uint32_t (&key)[R], uint32_t cand) {
  static_assert(R < 64, "per-lane counts must stay below 64");
  uint32_t c = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) c += key[r] >= cand ? 1u : 0u;
  return wave_sum_small(c);
}
// A threshold T of the list (more than k non-empty slots) with at least k
// keys >= T, found bit by bit from the top below the common prefix of the
// largest and smallest key: the k-th largest key, unless a candidate with
// exactly k keys at or above it turns up first (then *exact is set and those
// k keys are the selection, ties included).
template <int R>
__device__ __forceinline__ uint32_t wave_kth(const uint32_t (&key)[R], int k, bool* exact) {
  *exact = false;
  uint32_t hi = 0, lo = 0xffffffffu;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (key[r] != 0u) { hi = max(hi, key[r]); lo = min(lo, key[r]); }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
  }
  const uint32_t diff = hi ^ lo;
  if (diff == 0) return hi;
  const int top = 31 - __clz(diff);
  uint32_t T = top == 31 ? 0u : (hi >> (top + 1)) << (top + 1);
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    const uint32_t c = wave_count_ge(key, cand);
    if (c >= (uint32_t)k) {
      T = cand;
      if (c == (uint32_t)k) {
        *exact = true;
        break;
      }
    }
  }
  return T;
}
// The top k of the list (nval non-empty slots, the same in every lane): keys
// above the k-th largest T, then keys equal to T in list order until k are
// taken (ties go to the lower index).  Returns the lane's slots as a bit mask.
template <int R>
__device__ __forceinline__ uint32_t wave_select(const uint32_t (&key)[R], int nval, int k) {
  static_assert(R <= 32, "one mask bit per slot");
  uint32_t sel = 0;
  if (nval <= k) {
#pragma unroll
    for (int r = 0; r < R; ++r) sel |= (key[r] != 0u ? 1u : 0u) << r;
    return sel;
  }
  bool exact;
  const uint32_t T = wave_kth(key, k, &exact);
  if (exact) {   // exactly k keys are >= T
#pragma unroll
    for (int r = 0; r < R; ++r) sel |= (key[r] >= T ? 1u : 0u) << r;
    return sel;
  }
  const uint32_t gt = T == 0xffffffffu ? 0u : wave_count_ge(key, T + 1);
  const uint32_t eq = wave_count_ge(key, T) - gt;
  const uint32_t need = (uint32_t)k - gt;
#pragma unroll
  for (int r = 0; r < R; ++r) sel |= (key[r] > T ? 1u : 0u) << r;
  if (eq <= need) {   // every tie is taken (the usual case: T is one key)
#pragma unroll
    for (int r = 0; r < R; ++r) sel |= (key[r] == T ? 1u : 0u) << r;
  } else {
    uint32_t run = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(key[r] == T);
      const uint32_t before = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (key[r] == T && before < need) sel |= 1u << r;
      run += (uint32_t)__popcll(m);
    }
  }
  return sel;
}
// Output positions of the selected slots, compacted in list order.
template <int R>
__device__ __forceinline__ void wave_positions(uint32_t sel, uint32_t (&pos)[R]) {
  uint32_t run = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint64_t m = __builtin_amdgcn_ballot_w64((sel >> r) & 1u);
    pos[r] = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    run += (uint32_t)__popcll(m);
  }
}

// Two workgroups per CU: the register budget this asks for (256 per lane)
// fits the 64-head, 128-dimension form without spills, and its 80 KiB of
// LDS fits twice.
template <int NHB, int KS, int FUSED>
__global__ __launch_bounds__(256, 2) void index_scores_mfma(
    const bf16_t* __restrict__ qI, const float* __restrict__ w, const bf16_t* __restrict__ KI,
    int64_t comp_bs, int64_t n_q, int64_t t0, int64_t n_comp, int64_t m, int64_t cand_per_wg,
    int64_t n_qblocks, float* __restrict__ scores, int64_t k, int32_t* __restrict__ idx,
    float* __restrict__ score_out, int sbf) {
  constexpr int CI = KS * 16;
  constexpr int NH = NHB * 32;
  constexpr int TN = 64;                 // keys per tile
  constexpr int NCH = 2 * KS;            // 16-byte chunks per key row
  constexpr int KPI = 64 / NCH;          // key rows per 1 KiB DMA instruction
  constexpr int DPW = TN / KPI / 4;      // DMA instructions per wave and tile
  constexpr int SDIV = 16 / NCH;         // f(r) = (r / SDIV) % NCH spreads 16 rows over 64 banks
  static_assert(NCH == 8 || NCH == 16, "c_I must be 64 or 128");
  __shared__ uint4 ring[3][TN * NCH];
  __shared__ float ssc[FUSED ? 4 : 1][FUSED ? kFusedMaxKeys : 1];   // FUSED: the queries' scores

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  // heaviest (latest) query blocks first: causal work grows with position
  const int64_t qb = n_qblocks - 1 - blockIdx.x;
  const int64_t bi = blockIdx.z;
  const int64_t qrow = qb * 4 + wave;
  const bool qvalid = qrow < n_q;

  int64_t vis_q = qvalid ? (t0 + qrow + 1) / m : 0;
  if (vis_q > n_comp) vis_q = n_comp;
  int64_t last = qb * 4 + 3;
  if (last > n_q - 1) last = n_q - 1;
  int64_t vis_wg = (t0 + last + 1) / m;
  if (vis_wg > n_comp) vis_wg = n_comp;
  const int64_t c0 = (int64_t)blockIdx.y * cand_per_wg;
  int64_t c1 = c0 + cand_per_wg;
  if (c1 > vis_wg) c1 = vis_wg;
  if (!FUSED && c0 >= c1) return;
  const int ntl = c0 < c1 ? (int)((c1 - c0 + TN - 1) / TN) : 0;   // uniform over the workgroup

  const bf16_t* kbase = KI + bi * comp_bs;
  const int64_t lastkey = c1 - 1;
  // DMA of tile j into a ring slot: this wave's instructions i = DPW*wave ..
  // +DPW; lane l fills chunk l % NCH of row i*KPI + l/NCH from source chunk
  // (l % NCH) ^ f(row).  Rows past the last key re-read it (in bounds; their
  // scores are not stored), and so does a tile wholly past the end.
  int src_off[DPW];
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int r = (DPW * wave + d) * KPI + l / NCH;
    src_off[d] = r * CI + (((l % NCH) ^ ((r / SDIV) % NCH)) * 8);
  }
  auto issue = [&](int j, int slot) {
    int64_t kb = c0 + (int64_t)TN * j;
    kb = kb < lastkey ? kb : lastkey;
    const int room = (int)(lastkey - kb < TN ? lastkey - kb : TN);
    const uint32_t lds = (uint32_t)(uintptr_t)&ring[slot][0];
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int i = DPW * wave + d;
      const int r = i * KPI + l / NCH;
      const bf16_t* src = kbase + kb * CI + (r <= room ? src_off[d] : room * CI + (src_off[d] - r * CI));
      dma_chunk16(src, lds + 1024 * i);
    }
  };
  if (ntl > 0) {
    issue(0, 0);
    issue(1, 1);
  }

  // query operand and head weights in registers
  bf16x8 qa[NHB][KS];
  float wv[NHB][16];
  const int64_t qoff = (bi * n_q + (qvalid ? qrow : 0)) * (int64_t)NH;
#pragma unroll
  for (int mb = 0; mb < NHB; ++mb) {
    const bf16_t* qp = qI + (qoff + mb * 32 + (l & 31)) * CI + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qa[mb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 16));
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wv[mb][r] = qvalid ? w[qoff + mb * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3)] : 0.f;
  }
  // Consume the operand loads here, so that the compiler waits for them once,
  // before the key loop: a wait it placed inside the loop would also drain
  // the DMA loads in flight, which it does not count.
#pragma unroll
  for (int mb = 0; mb < NHB; ++mb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qa[mb][ks]));
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(wv[mb][r]));
  }

  float* srow = scores + (bi * n_q + (qvalid ? qrow : 0)) * n_comp;
  // B operand of step (ks, nb): lane l holds dims 16 ks + 8 (l / 32) .. +8 of
  // key row 32 nb + l % 32
  int rd_off[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = nb * 32 + (l & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rd_off[nb][ks] = r * NCH + ((2 * ks + (l >> 5)) ^ ((r / SDIV) % NCH));
  }
  // Step j: this wave's part of tile j has landed once at most the DPW loads
  // of tile j + 1 are in flight (loads complete in order; a pending score
  // store only makes the wait stricter); after the barrier every wave's part
  // has, and every wave is done with tile j - 1, whose slot receives tile
  // j + 2.
  int slot = 0;
  for (int j = 0; j < ntl; ++j) {
    wait_vmem<DPW>();
    __syncthreads();
    issue(j + 2, slot == 0 ? 2 : slot - 1);
    const int64_t kb = c0 + (int64_t)TN * j;
    if (qvalid && kb < vis_q) {
      f32x16 acc[NHB][2];
#pragma unroll
      for (int mb = 0; mb < NHB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const bf16x8 bv = __builtin_bit_cast(bf16x8, ring[slot][rd_off[nb][ks]]);
#pragma unroll
          for (int mb = 0; mb < NHB; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], bv, acc[mb][nb], 0, 0, 0);
        }
      }
      float s2[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float s = 0.f;
#pragma unroll
        for (int mb = 0; mb < NHB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s = fmaf(fmaxf(acc[mb][nb][r], 0.f), wv[mb][r], s);
        s2[nb] = s + __shfl_xor(s, 32, 64);
      }
      const int64_t cand = kb + l;
      if (cand < vis_q) {
        const float v = (l < 32) ? s2[0] : s2[1];
        const float vs = sbf ? bf2f(f2bf(v)) : v;   // bf16 index scores: rounded before the selection
        if constexpr (FUSED) ssc[wave][cand] = vs;
        else srow[cand] = vs;
      }
    }
    slot = slot == 2 ? 0 : slot + 1;
  }
  wait_vmem<0>();   // the look-ahead tiles past the end
  if constexpr (FUSED) {
    // Each wave selects over its own query's scores (slot r, lane l holds
    // entry 64 r + l): the top k, ties to the lower index, written in
    // ascending index order and padded with -1.  The wave wrote these LDS
    // words itself, so no barrier is needed.
    constexpr int R = kFusedMaxKeys / 64;
    const int len = (int)vis_q;
    uint32_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) key[r] = r * 64 + l < len ? f2key(ssc[wave][r * 64 + l]) : 0u;
    const uint32_t sel = wave_select<R>(key, len, (int)k);
    uint32_t pos[R];
    wave_positions<R>(sel, pos);
    if (qvalid) {
      const int64_t row = bi * n_q + qrow;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if ((sel >> r) & 1u) {
          idx[row * k + pos[r]] = r * 64 + l;
          if (score_out) score_out[row * k + pos[r]] = key2f(key[r]);
        }
      for (int64_t p = (len < k ? len : k) + l; p < k; p += 64) {
        idx[row * k + p] = -1;
        if (score_out) score_out[row * k + p] = 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming MFMA scoring for few queries (decode), bf16.  Each wave keeps its
// query's 32*NHB x c_I operand in registers and walks 32-key tiles of its
// workgroup's keys on its own, with no barrier until the end.  A tile's 32
// key rows are one contiguous block in HBM; the wave copies it whole into an
// LDS ring of its own with 1 KiB LDS-DMA loads (global_load_lds_dwordx4),
// D - 1 tiles ahead of the MFMAs, and reads the B operands back from LDS.
// (Loading the operands straight into registers makes every load instruction
// touch 32 rows x 32 bytes, which HBM serves well below its contiguous
// rate.)  The DMA writes 16-byte chunks in lane order, so the permutation that
// keeps the operand reads free of bank conflicts is applied on the global
// side: LDS chunk p of key r holds source chunk p ^ f(r).
// Per key the only traffic is its c_I bf16 values and one float score; the
// scores collect in LDS and leave in one pass at the end.  The kernel also
// records, per group of up to 512 keys, the largest score (as an
// order-preserving key): the k-th largest of these group maxima bounds the
// k-th largest score from below, which lets selection discard almost every
// key in one pass.
// ---------------------------------------------------------------------------
// One lane's operand of a 32x32x16 MFMA step (8 elements: 16 bytes of bf16,
// 8 of E4M3) and the MFMA itself, per key element type.
template <typename E> struct ScoreOps;
template <> struct ScoreOps<bf16_t> {
  typedef bf16x8 op_t;
  static __device__ __forceinline__ op_t ld(const void* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ f32x16 mfma(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct ScoreOps<fp8_t> {
  typedef long op_t;
  static __device__ __forceinline__ op_t ld(const void* p) { return *reinterpret_cast<const long*>(p); }
  static __device__ __forceinline__ f32x16 mfma(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
  }
};

template <int NHB, int KS, int D, typename E, int SBK>
__global__ __launch_bounds__(256) void index_scores_stream(
    const E* __restrict__ qI, const float* __restrict__ w, const E* __restrict__ KI,
    Rows kr, int64_t n_q, QPos qp, int64_t n_comp, int64_t m,
    float* __restrict__ scores, uint32_t* __restrict__ gmax, int64_t ld_gmax, int sbf) {
  typedef ScoreOps<E> Ops;
  constexpr int CI = KS * 16;
  constexpr int NH = NHB * 32;
  constexpr int ES = (int)sizeof(E);
  constexpr int ROWB = CI * ES;      // bytes per key row
  constexpr int NCH = ROWB / 16;     // 16-byte chunks per key row
  constexpr int KPI = 64 / NCH;      // key rows per 1 KiB DMA instruction
  constexpr int NDMA = NCH / 2;      // 1 KiB DMA instructions per 32-key tile
  constexpr int SDIV = 16 / NCH;     // f(r) = (r / SDIV) % NCH spreads 16 rows over 64 banks
  constexpr int TU4 = 32 * NCH;      // 16-byte chunks per tile
  static_assert(NCH == 4 || NCH == 8 || NCH == 16, "c_I must be 64 or 128");
  __shared__ uint4 ring[4][D][TU4];
  // SBK > 0: the workgroup's scores (at most SBK) collect here and leave in
  // one burst at the end; SBK == 0: each tile's 128 bytes are stored as made
  __shared__ float sbuf[SBK > 0 ? SBK : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int64_t qrow = blockIdx.x;
  const int64_t bi = blockIdx.z;
  int64_t vis = (qp.at(bi, qrow) + 1) / m;
  if (vis > n_comp) vis = n_comp;
  // The row's keys are dealt to the gridDim.y workgroups in 128-key chunks,
  // round robin (chunk c goes to workgroup c % gridDim.y), so that the
  // workgroups in flight read neighbouring chunks rather than the same
  // offset of distant ranges; within a chunk, wave w takes keys 32 w .. +32.
  const int64_t first = 128 * (int64_t)blockIdx.y + 32 * wave;  // the wave's first key
  const int64_t kstep = 128 * (int64_t)gridDim.y;                // distance between its tiles
  const int64_t c1 = vis;
  // group maxima (order-preserving keys, 0 = no key): lanes 4q..4q+3 of a
  // wave form one group, i.e. 4 keys of each of its 32-key tiles; every
  // group of the grid is written, empty ones as 0.  Any partition of the keys
  // into groups gives a valid bound.
  uint32_t gm = 0;
  auto write_gmax = [&]() {
    if (gmax == nullptr) return;
    gm = max(gm, (uint32_t)__shfl_xor((int)gm, 1, 64));
    gm = max(gm, (uint32_t)__shfl_xor((int)gm, 2, 64));
    if (l < 32 && (l & 3) == 0)
      gmax[(bi * n_q + qrow) * ld_gmax + (int64_t)blockIdx.y * 32 + wave * 8 + (l >> 2)] = gm;
  };
  if (vis <= 0) {  // uniform over the workgroup
    write_gmax();
    return;
  }
  // SBK > 0: at most SBK / 128 tiles per wave (the host splits each row over
  // enough workgroups)
  const int ntiles = first >= c1 ? 0 : (int)((c1 - first + kstep - 1) / kstep);

  const int64_t lastkey = c1 - 1;
  // DMA: instruction i, lane l fills LDS chunk 64 i + l of the tile = chunk
  // l % NCH of row i * KPI + l / NCH, from source chunk (l % NCH) ^ f(row)
  int src_off[NDMA];   // elements from the tile's first row
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = i * KPI + l / NCH;
    src_off[i] = r * CI + (((l % NCH) ^ ((r / SDIV) % NCH)) * (16 / ES));
  }
  // Paged keys (SBK > 0: at most SBK / 128 tiles per wave): the block of
  // every tile of the wave is looked up before the stream starts, tile j's
  // in lane j % 64 of blk[j / 64] (tiles past the end: the last key's
  // block).  Looked up as each tile is issued, the block-table load's wait
  // would also drain the tiles already in flight.
  constexpr int NBR = SBK > 0 ? (SBK / 128 + 63) / 64 : 1;
  const bool paged = SBK > 0 && kr.table != nullptr;
  int blk[NBR];
  int blk_last = 0;
  if (paged) {
    const int32_t* trow = kr.table + kr.req(bi) * kr.table_stride;
    auto block_of = [&](int64_t key) {
      int64_t b = trow[key >> kr.pb_log2];
      return (int)(b < 0 ? 0 : (b >= kr.n_blocks ? kr.n_blocks - 1 : b));
    };
#pragma unroll
    for (int r = 0; r < NBR; ++r) {
      const int64_t kb = first + kstep * (int64_t)(64 * r + l);
      blk[r] = block_of(kb < lastkey ? kb : lastkey);
    }
    blk_last = block_of(lastkey);
  }
  auto issue = [&](int j, int slot) {
    // rows past the last key re-read the last key (in bounds; their scores
    // are dropped), and so does a tile wholly past the end
    int64_t kb = first + kstep * j;
    kb = kb < lastkey ? kb : lastkey;
    const int room = (int)(lastkey - kb < 32 ? lastkey - kb : 32);
    const uint32_t lds = (uint32_t)(uintptr_t)&ring[wave][slot][0];
    // the tile's rows kb .. kb + room lie in one block when paged (blocks
    // hold a multiple of 32 keys, and kb is a multiple of 32 or the last key)
    const E* tb;
    if (paged) {
      int b = blk_last;
#pragma unroll
      for (int r = 0; r < NBR; ++r)
        if ((j >> 6) == r) b = __builtin_amdgcn_readlane(blk[r], j & 63);
      tb = KI + (int64_t)b * kr.blk_elems + kr.off + (kb & ((1 << kr.pb_log2) - 1)) * CI;
    } else {
      tb = KI + kr.at(bi, kb, CI);
    }
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int r = i * KPI + l / NCH;
      const E* src = tb + (r <= room ? src_off[i] : room * CI + (src_off[i] - r * CI));
      dma_chunk16(src, lds + 1024 * i);
    }
  };
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, j);

  typename Ops::op_t qa[NHB][KS];
  float wv[NHB][16];
  const int64_t qoff = (bi * n_q + qrow) * (int64_t)NH;
#pragma unroll
  for (int mb = 0; mb < NHB; ++mb) {
    const E* qp = qI + (qoff + mb * 32 + (l & 31)) * CI + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = Ops::ld(qp + ks * 16);
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[mb][r] = w[qoff + mb * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3)];
  }

  float* srow = scores + (bi * n_q + qrow) * n_comp;
  // B operand of 32x32x16 step ks: lane l holds elements 16 ks + 8 (l / 32)
  // .. +8 of key l % 32: byte b = ES (16 ks + 8 (l / 32)) of the row, in
  // 16-byte chunk b / 16 at byte b % 16
  const int rr = l & 31;
  int rd_off[KS];   // bytes from the slot's start
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int bb = ES * (16 * ks + 8 * (l >> 5));
    rd_off[ks] = rr * ROWB + (((bb >> 4) ^ ((rr / SDIV) % NCH)) << 4) + (bb & 15);
  }
  auto compute = [&](int j, int slot) {
    const unsigned char* tile = reinterpret_cast<const unsigned char*>(&ring[wave][slot][0]);
    f32x16 acc[NHB];
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb) acc[mb] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const typename Ops::op_t bv = Ops::ld(tile + rd_off[ks]);
#pragma unroll
      for (int mb = 0; mb < NHB; ++mb) acc[mb] = Ops::mfma(qa[mb][ks], bv, acc[mb]);
    }
    float sc = 0.f;
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc = fmaf(fmaxf(acc[mb][r], 0.f), wv[mb][r], sc);
    sc += __shfl_xor(sc, 32, 64);
    if (sbf) sc = bf2f(f2bf(sc));   // bf16 index scores: rounded before the selection
    const int64_t key = first + kstep * j + l;
    if constexpr (SBK > 0) {
      if (l < 32) sbuf[128 * j + 32 * wave + l] = sc;
    } else {
      if (l < 32 && key < c1) srow[key] = sc;
    }
    if (l < 32 && key < c1) gm = max(gm, f2key(sc));
  };
  // tile j sits in slot j % D; step j first issues tile j + D - 1 into the
  // slot step j - 1 has finished reading.  Every step issues exactly one tile
  // (those past the last tile re-read the last key row: they keep the wait
  // counts static and cost no HBM traffic), so before step j's reads the
  // D - 1 tiles issued after tile j ((D - 1) NDMA loads) may still be in
  // flight; loads complete in order, and a pending score store only makes the
  // wait stricter.
  int slot = 0;
  for (int j = 0; j < ntiles; ++j) {
    issue(j + D - 1, slot == 0 ? D - 1 : slot - 1);
    wait_vmem<(D - 1) * NDMA>();
    compute(j, slot);
    slot = slot == D - 1 ? 0 : slot + 1;
  }
  wait_vmem<0>();
  write_gmax();
  // SBK > 0: the scores leave in one pass of full-line stores per workgroup
  // (for bf16 keys, storing each tile's 128 bytes as it is scored costs about
  // a tenth of the kernel's time; for narrower keys the LDS the buffer takes
  // is worth more as ring slots)
  if constexpr (SBK > 0) {
    __syncthreads();
    const int64_t nch = (c1 - 128 * (int64_t)blockIdx.y + kstep - 1) / kstep;  // the workgroup's chunks
    for (int e = threadIdx.x; e < nch * 128; e += 256) {
      const int64_t key = 128 * ((int64_t)blockIdx.y + (int64_t)gridDim.y * (e >> 7)) + (e & 127);
      if (key < c1) srow[key] = sbuf[e];
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP4 scoring (OCP MX: E2M1 elements, one E8M0 scale per 32 dimensions).
//
// Streaming form (decode; c_I = 128): the layout of index_scores_stream with
// 64-byte code rows, on the block-scaled MFMA v_mfma_scale_f32_32x32x64
// (E2M1 x E2M1, float32 accumulation).  Per 64-dimension step a lane's
// operand is 16 bytes = 32 consecutive dimensions of its row, i.e. exactly one
// MX block, and the MFMA takes one scale byte per lane and operand (chosen by
// an immediate byte select from a 32-bit register).  Queries and keys are
// read in the same storage order, so the products pair the right elements
// whatever order the unit uses inside a lane.  A tile's 32 scale words (4
// bytes per key) reach LDS by one dword LDS-DMA next to the code DMA.
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void dma_dword(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds) : "memory");
}

// 16 code bytes in the low half of the 32-byte operand (the E2M1 form reads
// only that half)
__device__ __forceinline__ i32x8 mx_operand(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

template <int NHB, int D, int SBK>
__global__ __launch_bounds__(256) void index_scores_stream_mx(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qS, const float* __restrict__ w,
    const uint8_t* __restrict__ KI, const uint8_t* __restrict__ KS, int64_t comp_bs, int64_t n_q, int64_t t0,
    int64_t n_comp, int64_t m, float* __restrict__ scores, uint32_t* __restrict__ gmax, int64_t ld_gmax) {
  constexpr int CI = 128;
  constexpr int NH = NHB * 32;
  constexpr int ROWB = CI / 2;       // code bytes per key row
  constexpr int NB = CI / 32;        // scale bytes per key (one 32-bit word)
  constexpr int NCH = ROWB / 16;     // 16-byte chunks per row
  constexpr int KPI = 64 / NCH;      // rows per 1 KiB DMA instruction
  constexpr int NDMA = NCH / 2;      // 1 KiB DMA instructions per 32-key tile
  constexpr int SDIV = 16 / NCH;     // f(r) = (r / SDIV) % NCH spreads rows over the banks
  constexpr int TU4 = 32 * NCH;      // 16-byte chunks per tile
  static_assert(NB == 4, "one scale word per key");
  __shared__ uint4 ring[4][D][TU4];
  // a tile's 32 scale words (dword LDS-DMA writes lane l's word at 4 l)
  __shared__ uint32_t sring[4][D][32];
  // SBK > 0: the scores collect in LDS and leave in one burst at the end;
  // SBK == 0: each tile's 32 scores (128 bytes) are stored as they are made
  __shared__ float sbuf[SBK > 0 ? SBK : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int h = l >> 5;
  const int64_t qrow = blockIdx.x;
  const int64_t bi = blockIdx.z;
  int64_t vis = (t0 + qrow + 1) / m;
  if (vis > n_comp) vis = n_comp;
  // 128-key chunks dealt to the gridDim.y workgroups round robin; wave w
  // takes keys 32 w .. +32 of each chunk
  const int64_t first = 128 * (int64_t)blockIdx.y + 32 * wave;
  const int64_t kstep = 128 * (int64_t)gridDim.y;
  const int64_t c1 = vis;
  uint32_t gm = 0;
  auto write_gmax = [&]() {
    if (gmax == nullptr) return;
    gm = max(gm, (uint32_t)__shfl_xor((int)gm, 1, 64));
    gm = max(gm, (uint32_t)__shfl_xor((int)gm, 2, 64));
    if (l < 32 && (l & 3) == 0)
      gmax[(bi * n_q + qrow) * ld_gmax + (int64_t)blockIdx.y * 32 + wave * 8 + (l >> 2)] = gm;
  };
  if (vis <= 0) {
    write_gmax();
    return;
  }
  // SBK > 0: at most SBK / 128 tiles per wave (the host splits each row over
  // enough workgroups)
  const int ntiles = first >= c1 ? 0 : (int)((c1 - first + kstep - 1) / kstep);
  const uint8_t* kbase = KI + bi * comp_bs * ROWB;
  const uint8_t* sbase = KS + bi * comp_bs * NB;
  const int64_t lastkey = c1 - 1;
  int src_off[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = i * KPI + l / NCH;
    src_off[i] = r * ROWB + (((l % NCH) ^ ((r / SDIV) % NCH)) * 16);
  }
  auto issue = [&](int j, int slot) {
    // rows past the last key re-read the last key (in bounds; their scores
    // are dropped), and so does a tile wholly past the end
    int64_t kb = first + kstep * j;
    kb = kb < lastkey ? kb : lastkey;
    const int room = (int)(lastkey - kb < 32 ? lastkey - kb : 32);
    const uint32_t lds = (uint32_t)(uintptr_t)&ring[wave][slot][0];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int r = i * KPI + l / NCH;
      const uint8_t* src = kbase + kb * ROWB + (r <= room ? src_off[i] : room * ROWB + (src_off[i] - r * ROWB));
      dma_chunk16(src, lds + 1024 * i);
    }
    if (l < 32) {
      const int r = l <= room ? l : room;
      dma_dword(sbase + (kb + r) * NB, (uint32_t)(uintptr_t)&sring[wave][slot][0]);
    }
  };
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, j);

  // query operands and scale words (shifted so that byte 0 / byte 2 select
  // blocks h / 2 + h, the dimensions this lane's half holds in steps 0 / 1)
  i32x8 qa[NHB][2];
  uint32_t qsw[NHB];
  float wv[NHB][16];
  const int64_t qoff = (bi * n_q + qrow) * (int64_t)NH;
#pragma unroll
  for (int mb = 0; mb < NHB; ++mb) {
    const int64_t hr = qoff + mb * 32 + (l & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qa[mb][ks] = mx_operand(qI + hr * ROWB + 32 * ks + 16 * h);
    qsw[mb] = *reinterpret_cast<const uint32_t*>(qS + hr * NB) >> (8 * h);
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[mb][r] = w[qoff + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3)];
  }

  float* srow = scores + (bi * n_q + qrow) * n_comp;
  const int rr = l & 31;
  int rd_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd_off[ks] = rr * ROWB + ((((2 * ks + h)) ^ ((rr / SDIV) % NCH)) << 4);
  auto compute = [&](int j, int slot) {
    const unsigned char* tile = reinterpret_cast<const unsigned char*>(&ring[wave][slot][0]);
    const uint32_t ksw = sring[wave][slot][rr] >> (8 * h);
    const i32x8 b0 = mx_operand(tile + rd_off[0]);
    const i32x8 b1 = mx_operand(tile + rd_off[1]);
    f32x16 acc[NHB];
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb) {
      acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][0], b0, (f32x16){}, 4, 4, 0, (int)qsw[mb], 0,
                                                                 (int)ksw);
      acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][1], b1, acc[mb], 4, 4, 2, (int)qsw[mb], 2,
                                                                 (int)ksw);
    }
    float sc = 0.f;
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc = fmaf(fmaxf(acc[mb][r], 0.f), wv[mb][r], sc);
    sc += __shfl_xor(sc, 32, 64);
    const int64_t key = first + kstep * j + l;
    if constexpr (SBK > 0) {
      if (l < 32) sbuf[128 * j + 32 * wave + l] = sc;
    } else {
      if (l < 32 && key < c1) srow[key] = sc;
    }
    if (l < 32 && key < c1) gm = max(gm, f2key(sc));
  };
  // as in index_scores_stream, with NDMA + 1 loads per tile: before step j's
  // reads the D - 1 tiles issued after tile j may still be in flight
  int slot = 0;
  for (int j = 0; j < ntiles; ++j) {
    issue(j + D - 1, slot == 0 ? D - 1 : slot - 1);
    wait_vmem<(D - 1) * (NDMA + 1)>();
    compute(j, slot);
    slot = slot == D - 1 ? 0 : slot + 1;
  }
  wait_vmem<0>();
  write_gmax();
  if constexpr (SBK > 0) {
    __syncthreads();
    const int64_t nch = (c1 - 128 * (int64_t)blockIdx.y + kstep - 1) / kstep;
    for (int e = threadIdx.x; e < nch * 128; e += 256) {
      const int64_t key = 128 * ((int64_t)blockIdx.y + (int64_t)gridDim.y * (e >> 7)) + (e & 127);
      if (key < c1) srow[key] = sbuf[e];
    }
  }
}

// Many-query low-precision scoring (prefill; c_I = 128): index_scores_mfma's
// layout -- four queries per workgroup, one per wave, sharing 64-key tiles
// that reach a 3-slot LDS ring by LDS-DMA two tiles ahead, one barrier per
// tile -- on the block-scaled MFMA v_mfma_scale_f32_32x32x64.  FMT 4: MXFP4
// (64-byte code rows; the tile's 64 scale words DMA'd beside them, 16 per
// wave; a lane's operand is 16 bytes, one MX block); FMT 0: E4M3 codes
// without scales (128-byte rows, 32-byte lane operands, unit scales).
// FUSED: every list fits one workgroup (at most kFusedMaxKeys keys) and each
// wave selects its query's top k from LDS as in index_scores_mfma; else the
// scores are written.
template <int NHB, int FUSED, int FMT>
__global__ __launch_bounds__(256) void index_scores_mfma_mx(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qS, const float* __restrict__ w,
    const uint8_t* __restrict__ KI, const uint8_t* __restrict__ KS, int64_t comp_bs, int64_t n_q, int64_t t0,
    int64_t n_comp, int64_t m, int64_t n_qblocks, float* __restrict__ scores, int64_t k,
    int32_t* __restrict__ idx, float* __restrict__ score_out) {
  static_assert(FMT == 4 || FMT == 0, "E2M1 or E4M3 operands");
  constexpr bool MX = FMT == 4;
  constexpr int CI = 128;
  constexpr int NH = NHB * 32;
  constexpr int TN = 64;                 // keys per tile
  constexpr int ROWB = MX ? CI / 2 : CI; // code bytes per key
  constexpr int OPB = MX ? 16 : 32;      // operand bytes per lane and 64-dimension step
  constexpr int NB = CI / 32;            // MXFP4 scale bytes per key (one word)
  constexpr int NCH = ROWB / 16;         // 16-byte chunks per row
  constexpr int KPI = 64 / NCH;          // rows per 1 KiB DMA instruction
  constexpr int DPW = TN / KPI / 4;      // code DMAs per wave and tile
  constexpr int SDIV = 16 / NCH;
  constexpr int LPT = DPW + (MX ? 1 : 0);   // vector-memory loads per wave and tile
  __shared__ uint4 ring[3][TN * NCH];
  __shared__ uint32_t sring[MX ? 3 : 1][MX ? TN : 1];
  __shared__ float ssc[FUSED ? 4 : 1][FUSED ? kFusedMaxKeys : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int h = l >> 5;
  const int64_t qb = n_qblocks - 1 - blockIdx.x;   // heaviest (latest) query blocks first
  const int64_t bi = blockIdx.z;
  const int64_t qrow = qb * 4 + wave;
  const bool qvalid = qrow < n_q;
  int64_t vis_q = qvalid ? (t0 + qrow + 1) / m : 0;
  if (vis_q > n_comp) vis_q = n_comp;
  int64_t last = qb * 4 + 3;
  if (last > n_q - 1) last = n_q - 1;
  int64_t c1 = (t0 + last + 1) / m;   // the workgroup's keys: 0 .. c1-1
  if (c1 > n_comp) c1 = n_comp;
  const int ntl = (int)((c1 + TN - 1) / TN);   // uniform over the workgroup

  const uint8_t* kbase = KI + bi * comp_bs * ROWB;
  const uint8_t* sbase = MX ? KS + bi * comp_bs * NB : nullptr;
  const int64_t lastkey = c1 - 1;
  int dr[DPW], src_off[DPW];   // tile row each of this lane's code DMAs fills, and its source
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    dr[d] = (DPW * wave + d) * KPI + l / NCH;
    src_off[d] = dr[d] * ROWB + (((l % NCH) ^ ((dr[d] / SDIV) % NCH)) * 16);
  }
  auto issue = [&](int j, int slot) {
    int64_t kb = (int64_t)TN * j;
    kb = kb < lastkey ? kb : lastkey;
    const int room = (int)(lastkey - kb < TN ? lastkey - kb : TN);
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const uint8_t* src =
          kbase + kb * ROWB + (dr[d] <= room ? src_off[d] : room * ROWB + (src_off[d] - dr[d] * ROWB));
      dma_chunk16(src, (uint32_t)(uintptr_t)&ring[slot][0] + 1024 * (DPW * wave + d));
    }
    if constexpr (MX) {
      if (l < 16) {
        const int r = 16 * wave + l;
        dma_dword(sbase + (kb + (r <= room ? r : room)) * NB, (uint32_t)(uintptr_t)&sring[slot][16 * wave]);
      }
    }
  };
  if (ntl > 0) {
    issue(0, 0);
    issue(1, 1);
  }

  // an operand: this lane's 32 dimensions of a 64-dimension step
  auto operand = [&](const uint8_t* p) -> i32x8 {
    if constexpr (MX) {
      return mx_operand(p);
    } else {
      const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
      return (i32x8){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
  };
  // query operands (two 64-dimension steps); MXFP4: scale words shifted so
  // that bytes 0 / 2 select the blocks this lane's half holds (E4M3: the unit
  // scale 2^0 in every byte); head weights
  i32x8 qa[NHB][2];
  uint32_t qsw[NHB];
  float wv[NHB][16];
  const int64_t qoff = (bi * n_q + (qvalid ? qrow : 0)) * (int64_t)NH;
#pragma unroll
  for (int mb = 0; mb < NHB; ++mb) {
    const int64_t hr = qoff + mb * 32 + (l & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qa[mb][ks] = operand(qI + hr * ROWB + 2 * OPB * ks + OPB * h);
    if constexpr (MX) qsw[mb] = *reinterpret_cast<const uint32_t*>(qS + hr * NB) >> (8 * h);
    else qsw[mb] = 0x7f7f7f7fu;
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[mb][r] = qvalid ? w[qoff + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3)] : 0.f;
  }
  // consume the operand loads before the key loop (see index_scores_mfma)
#pragma unroll
  for (int mb = 0; mb < NHB; ++mb) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {   // the loaded dwords (a 32-byte vector has no host-side constraint)
      asm volatile("" ::"v"(qa[mb][ks][0]), "v"(qa[mb][ks][1]), "v"(qa[mb][ks][2]), "v"(qa[mb][ks][3]));
      if constexpr (!MX)
        asm volatile("" ::"v"(qa[mb][ks][4]), "v"(qa[mb][ks][5]), "v"(qa[mb][ks][6]), "v"(qa[mb][ks][7]));
    }
    asm volatile("" ::"v"(qsw[mb]));
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(wv[mb][r]));
  }

  float* srow = scores + (bi * n_q + (qvalid ? qrow : 0)) * n_comp;
  // bytes from the slot's start of the 16-byte chunks of key row 32 nb + l % 32
  // holding this lane's operand of step ks (OPB / 16 chunks from chunk
  // (2 ks + h) OPB / 16)
  constexpr int CPO = OPB / 16;
  int rd_off[2][2][CPO];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = nb * 32 + (l & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int u = 0; u < CPO; ++u)
        rd_off[nb][ks][u] = r * ROWB + ((((2 * ks + h) * CPO + u) ^ ((r / SDIV) % NCH)) << 4);
  }
  auto tile_operand = [&](const unsigned char* tile, int nb, int ks) -> i32x8 {
    if constexpr (MX) {
      return mx_operand(tile + rd_off[nb][ks][0]);
    } else {
      const uint4 a = *reinterpret_cast<const uint4*>(tile + rd_off[nb][ks][0]);
      const uint4 b = *reinterpret_cast<const uint4*>(tile + rd_off[nb][ks][CPO - 1]);
      return (i32x8){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
  };
  int slot = 0;
  for (int j = 0; j < ntl; ++j) {
    // this wave's part of tile j has landed once at most tile j + 1's LPT
    // loads are in flight; after the barrier every wave's part has
    wait_vmem<LPT>();
    __syncthreads();
    issue(j + 2, slot == 0 ? 2 : slot - 1);
    const int64_t kb = (int64_t)TN * j;
    if (qvalid && kb < vis_q) {
      const unsigned char* tile = reinterpret_cast<const unsigned char*>(&ring[slot][0]);
      f32x16 acc[NHB][2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        uint32_t ksw = 0x7f7f7f7fu;
        if constexpr (MX) ksw = sring[slot][32 * nb + (l & 31)] >> (8 * h);
        const i32x8 b0 = tile_operand(tile, nb, 0);
        const i32x8 b1 = tile_operand(tile, nb, 1);
#pragma unroll
        for (int mb = 0; mb < NHB; ++mb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][0], b0, (f32x16){}, FMT, FMT, 0,
                                                                       (int)qsw[mb], 0, (int)ksw);
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][1], b1, acc[mb][nb], FMT, FMT, 2,
                                                                       (int)qsw[mb], 2, (int)ksw);
        }
      }
      float s2[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float sacc = 0.f;
#pragma unroll
        for (int mb = 0; mb < NHB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc = fmaf(fmaxf(acc[mb][nb][r], 0.f), wv[mb][r], sacc);
        s2[nb] = sacc + __shfl_xor(sacc, 32, 64);
      }
      const int64_t cand = kb + l;
      if (cand < vis_q) {
        if constexpr (FUSED) ssc[wave][cand] = (l < 32) ? s2[0] : s2[1];
        else srow[cand] = (l < 32) ? s2[0] : s2[1];
      }
    }
    slot = slot == 2 ? 0 : slot + 1;
  }
  wait_vmem<0>();   // the look-ahead tiles past the end
  if constexpr (FUSED) {
    constexpr int R = kFusedMaxKeys / 64;
    const int len = (int)vis_q;
    uint32_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) key[r] = r * 64 + l < len ? f2key(ssc[wave][r * 64 + l]) : 0u;
    const uint32_t sel = wave_select<R>(key, len, (int)k);
    uint32_t pos[R];
    wave_positions<R>(sel, pos);
    if (qvalid) {
      const int64_t row = bi * n_q + qrow;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if ((sel >> r) & 1u) {
          idx[row * k + pos[r]] = r * 64 + l;
          if (score_out) score_out[row * k + pos[r]] = key2f(key[r]);
        }
      for (int64_t p = (len < k ? len : k) + l; p < k; p += 64) {
        idx[row * k + p] = -1;
        if (score_out) score_out[row * k + p] = 0.f;
      }
    }
  }
}

// Generic MXFP4 scoring (any head count, c_I a multiple of 32, n_hI * c_I
// at most kMxGenericMaxQ): one thread per (key, query row); the row's query
// values are decoded into LDS once; each key's values are decoded on the fly
// (E2M1 times the block's E8M0 scale, both exact in float32) and the
// products summed in dimension order.
constexpr int kMxGenericMaxQ = 8192;
__device__ __forceinline__ float e2m1_value(uint32_t nib) {
  const uint32_t e = (nib >> 1) & 3, f = nib & 1;
  const float mag = e == 0 ? 0.5f * (float)f : (1.f + 0.5f * (float)f) * (float)(1u << (e - 1));
  return (nib & 8) ? -mag : mag;
}
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  return s == 0 ? 0x1p-127f : __uint_as_float(s << 23);   // 2^(s - 127) (s = 255 gives inf, not NaN)
}
__global__ __launch_bounds__(256) void index_scores_generic_mx(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qS, const float* __restrict__ w,
    const uint8_t* __restrict__ KI, const uint8_t* __restrict__ KS, int64_t comp_bs, int64_t n_q, int64_t t0,
    int64_t n_comp, int nh, int cI, int64_t m, float* __restrict__ scores) {
  __shared__ float qv[kMxGenericMaxQ];
  const int64_t r = blockIdx.y, bi = blockIdx.z;
  const int64_t qoff = (bi * n_q + r) * (int64_t)nh;
  const int half = cI / 2, nb = cI / 32;
  for (int e = threadIdx.x; e < nh * cI; e += 256) {
    const int hh = e / cI, d = e % cI;
    const uint8_t byte = qI[(qoff + hh) * half + d / 2];
    qv[e] = e2m1_value((d & 1) ? (byte >> 4) : (byte & 15)) * e8m0_value(qS[(qoff + hh) * nb + d / 32]);
  }
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= n_comp) return;
  int64_t vis = (t0 + r + 1) / m;
  if (vis > n_comp) vis = n_comp;
  if (s >= vis) return;
  float* out = scores + (bi * n_q + r) * n_comp + s;
  const uint8_t* krow = KI + (bi * comp_bs + s) * half;
  const uint8_t* srow = KS + (bi * comp_bs + s) * nb;
  float acc = 0.f;
  for (int hh = 0; hh < nh; ++hh) {
    float dot = 0.f;
    for (int d = 0; d < cI; d += 2) {
      const uint8_t byte = krow[d / 2];
      const float sc = e8m0_value(srow[d / 32]);
      dot = fmaf(qv[hh * cI + d], e2m1_value(byte & 15) * sc, dot);
      dot = fmaf(qv[hh * cI + d + 1], e2m1_value(byte >> 4) * sc, dot);
    }
    acc = fmaf(w[qoff + hh], fmaxf(dot, 0.f), acc);
  }
  *out = acc;
}

// ---------------------------------------------------------------------------
// Top-k selection.  A segment (one query's candidate list, or one chunk of
// it) is held in registers by NT threads (one wave or a 256-thread
// workgroup), R keys each; element e of the segment sits in thread e % NT,
// slot e / NT, so slot-major order is list order.  Keys are order-preserving
// 32-bit images of the float scores.
//
// The k-th largest key T is found bit by bit from the top, starting below the
// common prefix of the segment's smallest and largest key; each step counts
// the keys >= a candidate with wave ballots and scalar popcounts (plus one LDS
// exchange per step in the workgroup form, where a step settles two bits).  Keys > T are taken, then keys
// == T in list order until k are taken (ties go to the lower index), and the
// taken elements are compacted in list order.
// ---------------------------------------------------------------------------
template <int NT>
struct SegReduce {
  // Exchanges alternate between two halves of the buffer (parity), so one
  // exchange's writes never meet the previous exchange's reads; each half
  // holds three values per wave.
  static constexpr int kStride = 3 * (NT / 64);
  static constexpr int kRedSize = 2 * kStride + 1;
  // sum of a wave-uniform count over the NT/64 waves (LDS exchange when NT > 64)
  static __device__ __forceinline__ uint32_t sum(uint32_t c, uint32_t* red, int wave, int& parity) {
    if constexpr (NT == 64) {
      return c;
    } else {
      uint32_t* slot = red + parity * kStride;
      parity ^= 1;
      if ((threadIdx.x & 63) == 0) slot[wave] = c;
      __syncthreads();
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) t += slot[w];
      return t;
    }
  }
  // three counts at once (one exchange)
  static __device__ __forceinline__ void sum3(uint32_t (&c)[3], uint32_t* red, int wave, int& parity) {
    if constexpr (NT > 64) {
      uint32_t* slot = red + parity * kStride;
      parity ^= 1;
      if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int j = 0; j < 3; ++j) slot[j * (NT / 64) + wave] = c[j];
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) t += slot[j * (NT / 64) + w];
        c[j] = t;
      }
    }
  }
  static __device__ __forceinline__ uint32_t umax(uint32_t v, uint32_t* red, int wave, int& parity) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    if constexpr (NT == 64) {
      return v;
    } else {
      uint32_t* slot = red + parity * kStride;
      parity ^= 1;
      if ((threadIdx.x & 63) == 0) slot[wave] = v;
      __syncthreads();
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) t = max(t, slot[w]);
      return t;
    }
  }
};

// Select the top k of the segment held in key[] (valid where val[]; nval
// of them, the same value in every lane; the caller zeroes the keys of
// invalid slots, so that no candidate threshold, which is always >= 1,
// counts them); writes the selection flags into sel[].  `red` is LDS
// scratch of 2 * NT/64 words (unused for NT == 64); `pre` is LDS scratch of
// R * NT/64 words used for list-order ranks.
template <int NT, int R>
__device__ __forceinline__ void segment_take(const uint32_t (&key)[R], const bool (&val)[R], int k, uint32_t T,
                                             bool (&sel)[R], uint32_t* red, uint32_t* pre, int parity);
template <int NT, int R>
__device__ __forceinline__ void segment_select(const uint32_t (&key)[R], const bool (&val)[R], int nval, int k,
                                               bool (&sel)[R], uint32_t* red, uint32_t* pre) {
  const int tid = threadIdx.x % NT, wave = tid >> 6, l = tid & 63;
  int parity = 0;
  if (nval <= k) {
#pragma unroll
    for (int r = 0; r < R; ++r) sel[r] = val[r];
    return;
  }
  // common prefix of the largest and smallest key bounds the search
  uint32_t hi = 0, lo = 0xffffffffu;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (val[r]) { hi = max(hi, key[r]); lo = min(lo, key[r]); }
  hi = SegReduce<NT>::umax(hi, red, wave, parity);
  lo = ~SegReduce<NT>::umax(~lo, red, wave, parity);
  const uint32_t diff = hi ^ lo;
  uint32_t T = 0;
  // a candidate with exactly k keys at or above it settles the selection
  // (ties included); the counts are the same in every lane, so the exit is
  // uniform
  bool exact = false;
  if (diff == 0) {
    T = hi;
  } else {
    const int top = 31 - __clz(diff);
    T = top == 31 ? 0u : (hi >> (top + 1)) << (top + 1);
    int bit = top;
    if constexpr (NT > 64) {
      // two bits per exchange: the counts >= T + u, T + 2u, T + 3u (u the
      // lower of the two bits, both clear in T) settle both at once
      for (; bit >= 1; bit -= 2) {
        const uint32_t u = 1u << (bit - 1);
        uint32_t c[3] = {0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int r = 0; r < R; ++r)
            c[j] += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(key[r] >= T + (uint32_t)(j + 1) * u));
        SegReduce<NT>::sum3(c, red, wave, parity);
        const int js = c[2] >= (uint32_t)k ? 3 : c[1] >= (uint32_t)k ? 2 : c[0] >= (uint32_t)k ? 1 : 0;
        if (js > 0) {
          T += (uint32_t)js * u;
          if (c[js - 1] == (uint32_t)k) {
            exact = true;
            break;
          }
        }
      }
    }
    for (; !exact && bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t c = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) c += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(key[r] >= cand));
      c = SegReduce<NT>::sum(c, red, wave, parity);
      if (c >= (uint32_t)k) {
        T = cand;
        exact = c == (uint32_t)k;
      }
    }
  }
  if (exact) {
#pragma unroll
    for (int r = 0; r < R; ++r) sel[r] = val[r] && key[r] >= T;
    return;
  }
  segment_take<NT, R>(key, val, k, T, sel, red, pre, parity);
}

// Given T, the k-th largest key of the segment, flag the elements taken: keys
// above T, then keys equal to T in list order until k are taken.
template <int NT, int R>
__device__ __forceinline__ void segment_take(const uint32_t (&key)[R], const bool (&val)[R], int k, uint32_t T,
                                             bool (&sel)[R], uint32_t* red, uint32_t* pre, int parity) {
  const int tid = threadIdx.x % NT, wave = tid >> 6, l = tid & 63;
  uint32_t gt = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) gt += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(val[r] && key[r] > T));
  gt = SegReduce<NT>::sum(gt, red, wave, parity);
  const uint32_t need_eq = (uint32_t)k - gt;
  // rank of each tie in list order: wave-local ballot prefix, plus earlier
  // waves (per slot) and earlier slots
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
  uint64_t meq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    meq[r] = __builtin_amdgcn_ballot_w64(val[r] && key[r] == T);
    if (NT > 64 && l == 0) pre[r * (NT / 64) + wave] = (uint32_t)__popcll(meq[r]);
  }
  if (NT > 64) __syncthreads();
  uint32_t run = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    uint32_t before = run + (uint32_t)__popcll(meq[r] & below);
    uint32_t slot_total = (uint32_t)__popcll(meq[r]);
    if constexpr (NT > 64) {
      slot_total = 0;
#pragma unroll
      for (int w2 = 0; w2 < NT / 64; ++w2) {
        const uint32_t cw = pre[r * (NT / 64) + w2];
        if (w2 < wave) before += cw;
        slot_total += cw;
      }
    }
    const bool eq = val[r] && key[r] == T;
    sel[r] = (val[r] && key[r] > T) || (eq && before < need_eq);
    run += slot_total;
  }
  if (NT > 64) __syncthreads();   // pre[] is reused by the caller's compaction
}

// Compact the selected elements in list order: returns each element's output
// position (valid where sel) through pos[].
template <int NT, int R>
__device__ __forceinline__ void segment_positions(const bool (&sel)[R], uint32_t (&pos)[R], uint32_t* pre) {
  const int tid = threadIdx.x % NT, wave = tid >> 6, l = tid & 63;
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
  uint64_t ms[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ms[r] = __builtin_amdgcn_ballot_w64(sel[r]);
    if (NT > 64 && l == 0) pre[r * (NT / 64) + wave] = (uint32_t)__popcll(ms[r]);
  }
  if (NT > 64) __syncthreads();
  uint32_t run = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    uint32_t p = run + (uint32_t)__popcll(ms[r] & below);
    uint32_t slot_total = (uint32_t)__popcll(ms[r]);
    if constexpr (NT > 64) {
      slot_total = 0;
#pragma unroll
      for (int w2 = 0; w2 < NT / 64; ++w2) {
        const uint32_t cw = pre[r * (NT / 64) + w2];
        if (w2 < wave) p += cw;
        slot_total += cw;
      }
    }
    pos[r] = p;
    run += slot_total;
  }
}

// One segment per wave (NT = 64, four segments per workgroup) or per
// workgroup (NT = 256).  Segment s of row `row` covers list elements
// [s*CH, s*CH + CH) with CH = NT*R.
//   from_scores: keys come from scores[row][e] (idx = e); otherwise from the
//                previous stage's (key, idx) pairs.
//   final_stage: write idx (ascending, -1 padded) and scores; otherwise write
//                min(k, len) pairs at slot s*k of the next list.
template <int NT, int R>
__global__ __launch_bounds__(256) void topk_stage(
    int from_scores, int final_stage, const float* __restrict__ scores, int64_t ld_scores,
    const uint32_t* __restrict__ kin, const int32_t* __restrict__ iin, int64_t ld_in,
    uint32_t* __restrict__ kout, int32_t* __restrict__ iout, int64_t ld_out, int32_t* __restrict__ idx,
    float* __restrict__ score_out, int64_t n_rows, int64_t n_q, QPos qp, int64_t n_comp, int64_t m,
    int64_t k, const int64_t* __restrict__ len_in, int64_t nseg) {
  constexpr int CH = NT * R;
  constexpr int SEGS = 256 / NT;   // segments per workgroup
  __shared__ uint32_t red_all[SEGS][SegReduce<NT>::kRedSize];
  __shared__ uint32_t pre_all[SEGS][R * (NT / 64) + 1];
  const int sub = threadIdx.x / NT;
  const int tid = threadIdx.x % NT;
  const int64_t gseg = (int64_t)blockIdx.x * SEGS + sub;   // global segment id over (row, seg)
  const bool active = gseg < n_rows * nseg;
  const int64_t row = active ? gseg / nseg : 0;
  const int64_t seg = active ? gseg % nseg : 0;
  int64_t L;
  if (from_scores) {
    L = (qp.at(row / n_q, row % n_q) + 1) / m;
    if (L > n_comp) L = n_comp;
  } else {
    L = len_in[row];
  }
  const int64_t base = seg * CH;
  int64_t len64 = L - base;
  if (len64 > CH) len64 = CH;
  if (len64 < 0 || !active) len64 = 0;
  const int len = (int)len64;
  // a wave with nothing to do still runs the uniform code when NT == 256.
  // Loads are unconditional (index clamped into the segment) so that all R
  // of them are in flight before the first wait.
  uint32_t key[R];
  int32_t ix[R];
  const int lastc = len > 0 ? len - 1 : 0;
  if (len > 0) {
    if (from_scores) {
      const float* src = scores + row * ld_scores + base;
      float raw[R];
#pragma unroll
      for (int r = 0; r < R; ++r) raw[r] = src[min(r * NT + tid, lastc)];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        key[r] = r * NT + tid < len ? f2key(raw[r]) : 0u;
        ix[r] = (int32_t)(base + r * NT + tid);
      }
    } else {
      const uint32_t* ks = kin + row * ld_in + base;
      const int32_t* is = iin + row * ld_in + base;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = min(r * NT + tid, lastc);
        key[r] = r * NT + tid < len ? ks[e] : 0u;
        ix[r] = is[e];
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) { key[r] = 0u; ix[r] = -1; }
  }
  bool val[R], sel[R];
#pragma unroll
  for (int r = 0; r < R; ++r) val[r] = r * NT + tid < len;
  segment_select<NT, R>(key, val, len, (int)k, sel, red_all[sub], pre_all[sub]);
  uint32_t pos[R];
  segment_positions<NT, R>(sel, pos, pre_all[sub]);
  if (!active) return;
  if (final_stage) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (sel[r]) {
        idx[row * k + pos[r]] = ix[r];
        if (score_out) score_out[row * k + pos[r]] = key2f(key[r]);
      }
    const int64_t take = len64 < k ? len64 : k;
    for (int64_t p = take + tid; p < k; p += NT) {
      idx[row * k + p] = -1;
      if (score_out) score_out[row * k + p] = 0.f;
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (sel[r]) {
        kout[row * ld_out + seg * k + pos[r]] = key[r];
        iout[row * ld_out + seg * k + pos[r]] = ix[r];
      }
  }
}

// ---------------------------------------------------------------------------
// Threshold path for long candidate lists (the decode scorer's group maxima)
// ---------------------------------------------------------------------------
// Count of valid slots over NT threads (a ballot sum; NT == 64 only here).
template <int R>
__device__ __forceinline__ int wave_count(const bool (&val)[R]) {
  int c = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) c += (int)__popcll(__builtin_amdgcn_ballot_w64(val[r]));
  return c;
}

// A lower bound tau on the k-th largest score of a row, from its first
// min(G, 256 R) group maxima (src): their k-th largest, or 1 (every valid
// key) when fewer than k are non-empty.  Each maximum is a distinct key of
// the row, so at least k keys are >= tau.  The k-th largest is found to
// kThresholdBits bits below the common prefix of the largest and smallest
// maximum: the bit search keeps count(>= T) >= k at every step, so stopping
// it early still gives a valid bound, one that lets through only the keys
// within 2^-12 of the maxima's range below the exact value.  Every thread of
// a 256-thread workgroup calls it (R maxima each).
constexpr int kThresholdBits = 12;
template <int R>
__device__ __forceinline__ uint32_t row_threshold(const uint32_t* __restrict__ src, int64_t G, int64_t k,
                                                  uint32_t* red) {
  constexpr int NT = 256;   // the whole workgroup takes part
  const int tid = threadIdx.x, wave = tid >> 6;
  const int g = (int)(G < NT * R ? G : NT * R);
  uint32_t key[R];
  uint32_t c = 0, hi = 0, lo = 0xffffffffu;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * NT + tid;
    const uint32_t v = src[min(e, g - 1)];
    key[r] = e < g ? v : 0u;   // 0 = empty
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    c += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(key[r] != 0u));
    if (key[r] != 0u) { hi = max(hi, key[r]); lo = min(lo, key[r]); }
  }
  int parity = 0;
  const uint32_t nval = SegReduce<NT>::sum(c, red, wave, parity);
  if (nval <= (uint32_t)k) return 1u;   // every valid key (uniform)
  hi = SegReduce<NT>::umax(hi, red, wave, parity);
  lo = ~SegReduce<NT>::umax(~lo, red, wave, parity);
  const uint32_t diff = hi ^ lo;
  uint32_t T = hi;
  if (diff != 0) {
    const int top = 31 - __clz(diff);
    T = top == 31 ? 0u : (hi >> (top + 1)) << (top + 1);   // <= lo: count(>= T) = nval >= k
    const int last = max(0, top - (kThresholdBits - 1));
    for (int bit = top; bit >= last; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t cc = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) cc += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(key[r] >= cand));
      cc = SegReduce<NT>::sum(cc, red, wave, parity);
      if (cc >= (uint32_t)k) {
        T = cand;
        if (cc == (uint32_t)k) break;   // the exact k-th largest maximum bounds it as well
      }
    }
  }
  return max(T, 1u);
}

// Threshold and filter in one launch: a workgroup takes four 2048-key
// segments of one row, one per wave.  Its 256 threads first find the row's
// bound from the group maxima (the search above; each of the row's
// workgroups repeats it), then each wave keeps the top k of its segment's
// scores at or above the bound (usually all of them: only a few keys pass),
// written in list order at slot seg*k of the row's pair list, their count in
// cnt[row][seg].  The segment's score loads are issued before the search, so
// their latency overlaps it.  Every count of the grid is written.
template <int RT>
__global__ __launch_bounds__(256) void topk_threshold_filter(
    const float* __restrict__ scores, int64_t ld_scores, const uint32_t* __restrict__ gmax, int64_t ld_gmax,
    int64_t G, int64_t n_q, QPos qp, int64_t n_comp, int64_t m, int64_t k, int64_t nseg,
    uint32_t* __restrict__ kout, int32_t* __restrict__ iout, int64_t ld_out, int32_t* __restrict__ cnt) {
  constexpr int R = 32, CH = 64 * R;
  __shared__ uint32_t red[SegReduce<256>::kRedSize];
  const int sub = threadIdx.x >> 6, tid = threadIdx.x & 63;
  const int64_t row = blockIdx.x;                          // rows on x: up to 2^31 of them
  const int64_t seg = (int64_t)blockIdx.y * 4 + sub;      // at most kMergeMaxSeg / 4 groups on y
  const bool active = seg < nseg;   // a wave past the row's last segment only helps the search
  int64_t L = (qp.at(row / n_q, row % n_q) + 1) / m;
  if (L > n_comp) L = n_comp;
  const int64_t base = seg * CH;
  int64_t len64 = L - base;
  if (len64 > CH) len64 = CH;
  if (len64 < 0 || !active) len64 = 0;
  const int len = (int)len64;
  float raw[R];
  if (len > 0) {
    const float* src = scores + row * ld_scores + base;
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = src[min(r * 64 + tid, len - 1)];
  }
  const uint32_t th = row_threshold<RT>(gmax + row * ld_gmax, G, k, red);   // >= 1
  if (!active) return;   // whole wave, after the workgroup's last barrier
  uint32_t key[R];
  if (len > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t kk = f2key(raw[r]);
      key[r] = r * 64 + tid < len && kk >= th ? kk : 0u;
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) key[r] = 0u;
  }
  const int nval = (int)wave_count_ge(key, 1u);
  const uint32_t sel = wave_select<R>(key, nval, (int)k);
  uint32_t pos[R];
  wave_positions<R>(sel, pos);
#pragma unroll
  for (int r = 0; r < R; ++r)
    if ((sel >> r) & 1u) {
      kout[row * ld_out + seg * k + pos[r]] = key[r];
      iout[row * ld_out + seg * k + pos[r]] = (int32_t)(base + r * 64 + tid);
    }
  if (tid == 0) cnt[row * nseg + seg] = nval < k ? nval : (int)k;
}

// One workgroup per row: the row's pair list is the concatenation, in
// segment order, of cnt[row][s] pairs at slot s*k.  The list is taken in
// chunks of up to 2048 - run entries after the running top k (run of them,
// earlier in list order), each chunk reduced to its top k; the final set is
// written in ascending index order, -1 padded.  Usually one chunk.
constexpr int kMergeMaxSeg = 4096;
__global__ __launch_bounds__(256) void topk_merge(const uint32_t* __restrict__ kin, const int32_t* __restrict__ iin,
                                                  int64_t ld_in, const int32_t* __restrict__ cnt, int64_t nseg,
                                                  int64_t k, int32_t* __restrict__ idx, float* __restrict__ score_out) {
  constexpr int NT = 256, R = 8, C = NT * R;
  __shared__ int32_t pref[kMergeMaxSeg + 1];
  __shared__ uint32_t runK[1024];
  __shared__ int32_t runI[1024];
  __shared__ uint32_t red[SegReduce<NT>::kRedSize];
  __shared__ uint32_t pre[R * (NT / 64) + 1];
  __shared__ int32_t part[NT / 64];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int ns = (int)nseg;
  // exclusive prefix of the segment counts
  const int per = (ns + NT - 1) / NT;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int sgi = tid * per + i;
    if (sgi < ns) local += cnt[row * nseg + sgi];
  }
  {
    // exclusive scan of the per-thread sums: wave scans, then wave totals
    const int lane = tid & 63, wv = tid >> 6;
    int v = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(v, o, 64);
      if (lane >= o) v += y;
    }
    if (lane == 63) part[wv] = v;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < NT / 64; ++w2) {
      const int t = part[w2];
      if (w2 < wv) before += t;
      total += t;
    }
    if (tid == 0) pref[ns] = total;
    local = before + v - local;   // exclusive prefix of this thread's segments
  }
  {
    int acc = local;
    for (int i = 0; i < per; ++i) {
      const int sgi = tid * per + i;
      if (sgi < ns) { pref[sgi] = acc; acc += cnt[row * nseg + sgi]; }
    }
  }
  __syncthreads();
  const int N = pref[ns];
  int run = 0, P = 0;
  while (true) {
    const int fill = min(C - run, N - P);
    const int len = run + fill;
    uint32_t key[R];
    int32_t ix[R];
    bool val[R], sel[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = r * NT + tid;
      val[r] = e < len;
      key[r] = 0u;
      ix[r] = -1;
      if (e < run) {
        key[r] = runK[e];
        ix[r] = runI[e];
      } else if (e < len) {
        const int p = P + (e - run);
        int lo = 0, hi = ns;   // last segment s with pref[s] <= p
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pref[mid] <= p) lo = mid; else hi = mid;
        }
        const int64_t off = row * ld_in + (int64_t)lo * k + (p - pref[lo]);
        key[r] = kin[off];
        ix[r] = iin[off];
      }
    }
    __syncthreads();   // the running set is read; it may be rewritten below
    segment_select<NT, R>(key, val, len, (int)k, sel, red, pre);
    uint32_t pos[R];
    segment_positions<NT, R>(sel, pos, pre);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (sel[r]) { runK[pos[r]] = key[r]; runI[pos[r]] = ix[r]; }
    run = len < k ? len : (int)k;
    P += fill;
    __syncthreads();
    if (P >= N) break;
  }
  for (int p = tid; p < k; p += NT) {
    idx[row * k + p] = p < run ? runI[p] : -1;
    if (score_out) score_out[row * k + p] = p < run ? key2f(runK[p]) : 0.f;
  }
}

// Next-stage list length per row: (nseg - 1) * k + min(k, last segment).
__global__ void topk_next_len(int64_t n_rows, int64_t n_q, QPos qp, int64_t n_comp, int64_t m,
                              int64_t k, int64_t chunk, const int64_t* __restrict__ len_in,
                              int64_t* __restrict__ len_out) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= n_rows) return;
  int64_t L;
  if (len_in == nullptr) {
    L = (qp.at(row / n_q, row % n_q) + 1) / m;
    if (L > n_comp) L = n_comp;
  } else {
    L = len_in[row];
  }
  if (L <= 0) { len_out[row] = 0; return; }
  const int64_t nch = (L + chunk - 1) / chunk;
  const int64_t last = L - (nch - 1) * chunk;
  len_out[row] = (nch - 1) * k + (last < k ? last : k);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int kWaveR = 32;                        // wave segment: 64 x 32 = 2048 keys
constexpr int64_t kWaveChunk = 64 * kWaveR;
constexpr int kBlockR = 32;                       // workgroup segment: 256 x 32 = 8192 keys
constexpr int64_t kBlockChunk = 256 * kBlockR;

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The streaming (decode) scoring kernel: at most StreamPolicy::keys keys per
// workgroup (its LDS score buffer), 32 group maxima per workgroup (4 waves x
// 8 groups).  bf16: a 3-slot ring of 8 KiB tiles per wave plus a 64 KiB score
// buffer fill a CU (160 KiB of LDS), so each row's keys are split over
// enough workgroups for about one per CU of the 256 on the chip; E4M3: a
// 3-slot ring of 4 KiB tiles plus a 32 KiB buffer leave room for two per CU.
// More splits when the buffer requires them, fewer when the row has fewer
// 128-key chunks: a grid just above the CU slots would run a nearly empty
// second round.
constexpr int64_t kStreamGroupsPerWG = 32;
template <int ES> struct StreamPolicy;
template <> struct StreamPolicy<2> { static constexpr int64_t keys = 16384, wgs = 256; static constexpr int ring = 3; };
template <> struct StreamPolicy<1> { static constexpr int64_t keys = 8192, wgs = 512; static constexpr int ring = 3; };
static int64_t stream_splits(int64_t b, int64_t n_q, int64_t vmax, int64_t keys, int64_t wgs) {
  if (keys <= 0) keys = (int64_t)1 << 40;   // no score buffer: any split
  const int64_t need = (vmax + keys - 1) / keys;
  const int64_t want = wgs / std::max<int64_t>(1, b * n_q);
  const int64_t chunks = (vmax + 127) / 128;
  return std::max<int64_t>(1, std::min(chunks, std::max(need, want)));
}
// MXFP4 codes: a tile is 2 KiB of codes and 128 bytes of scales, so what a
// CU keeps in flight is bounded by its ring slots.  keys == 0: no score
// buffer (each tile's 128 bytes of scores are stored as they are made), so
// a 4-slot ring still fits four workgroups per CU, and a row may be split
// over any number of workgroups; about four per CU are launched.
struct StreamPolicyMx { static constexpr int64_t keys = 0, wgs = 1024; static constexpr int ring = 4; };
static int64_t stream_splits_for(int dtype, int64_t b, int64_t n_q, int64_t vmax) {
  if (dtype == 3) return stream_splits(b, n_q, vmax, StreamPolicyMx::keys, StreamPolicyMx::wgs);
  return dtype == 2 ? stream_splits(b, n_q, vmax, StreamPolicy<1>::keys, StreamPolicy<1>::wgs)
                    : stream_splits(b, n_q, vmax, StreamPolicy<2>::keys, StreamPolicy<2>::wgs);
}

// Workspace: scores [rows, n_comp] f32 | len A, len B [rows] i64 |
//            pairs A, pairs B [rows, cap] (u32 key + i32 idx each) |
//            group maxima [rows, gcap] u32 | tau [rows] u32 | counts [rows, nseg] i32
struct TopkLayout {
  size_t scores, lenA, lenB, kA, iA, kB, iB, gmax, tau, cnt, total;
  int64_t cap, gcap, nseg;
};
static TopkLayout topk_layout(int64_t b, int64_t n_q, int64_t n_comp, int64_t k) {
  TopkLayout L{};
  const int64_t rows = b * n_q;
  const int64_t nch = (n_comp + kWaveChunk - 1) / kWaveChunk;
  L.nseg = nch;
  L.cap = nch > 1 ? nch * k : 0;
  // grows with n_comp; the largest of the element types' splits
  L.gcap = nch > 1 ? std::max({stream_splits_for(1, b, n_q, n_comp), stream_splits_for(2, b, n_q, n_comp),
                               stream_splits_for(3, b, n_q, n_comp)}) *
                         kStreamGroupsPerWG
                   : 0;
  size_t off = 0;
  L.scores = off; off = align256(off + (size_t)rows * n_comp * 4);
  L.lenA = off; off = align256(off + (size_t)rows * 8);
  L.lenB = off; off = align256(off + (size_t)rows * 8);
  L.kA = off; off = align256(off + (size_t)rows * L.cap * 4);
  L.iA = off; off = align256(off + (size_t)rows * L.cap * 4);
  L.kB = off; off = align256(off + (size_t)rows * L.cap * 4);
  L.iB = off; off = align256(off + (size_t)rows * L.cap * 4);
  L.gmax = off; off = align256(off + (size_t)rows * L.gcap * 4);
  L.tau = off; off = align256(off + (size_t)rows * 4);
  L.cnt = off; off = align256(off + (size_t)rows * (nch > 1 ? nch : 0) * 4);
  L.total = off;
  return L;
}

size_t index_topk_workspace_bytes(int64_t b, int64_t n_q, int64_t n_comp, int64_t k) {
  return topk_layout(b, n_q, n_comp, k).total;
}

bool index_topk_supported(int64_t n_comp, int64_t k) {
  // multi-stage selection needs each stage to shrink the list at least 2x,
  // and the merge of the threshold path holds at most 1024 pairs and
  // kMergeMaxSeg segment counts
  if (n_comp <= kWaveChunk) return true;
  return k <= kWaveChunk / 2 && (n_comp + kWaveChunk - 1) / kWaveChunk <= kMergeMaxSeg;
}

// Streaming scoring for few queries (decode): each query's keys split over
// many workgroups.  Writes the group maxima when gmax is given.
template <int NHB, int KS, typename E>
static hipError_t launch_scores_stream(const void* qI, const float* w, const void* KI, const Rows& kr, int64_t b,
                                       int64_t n_q, QPos qp, int64_t vmax, int64_t n_comp, int64_t m,
                                       float* scores, uint32_t* gmax, int64_t ld_gmax, bool* gmax_used,
                                       hipStream_t st, int sbf = 0) {
  typedef StreamPolicy<(int)sizeof(E)> Pol;
  const int64_t nsplit = stream_splits(b, n_q, vmax, Pol::keys, Pol::wgs);
  dim3 grid((unsigned)n_q, (unsigned)nsplit, (unsigned)b);
  hipLaunchKernelGGL((index_scores_stream<NHB, KS, Pol::ring, E, (int)Pol::keys>), grid, dim3(256), 0, st,
                     (const E*)qI, w,
                     (const E*)KI, kr, n_q, qp, n_comp, m, scores, gmax, ld_gmax, sbf);
  *gmax_used = gmax != nullptr;
  return hipGetLastError();
}

// Scoring on MFMA.  Returns through *gmax_used whether the group maxima
// were written (the streaming kernel writes them when gmax is given).
template <int NHB, int KS>
static hipError_t launch_scores_mfma(const void* qI, const float* w, const void* KI, int64_t cbs,
                                     int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t m,
                                     float* scores, uint32_t* gmax, int64_t ld_gmax, bool* gmax_used,
                                     int64_t k, int32_t* idx, float* score_out, hipStream_t st, int sbf) {
  const int64_t vmax = std::min<int64_t>((t0 + n_q) / m, n_comp);
  *gmax_used = false;
  if (n_q >= 4) {
    const int64_t nqb = (n_q + 3) / 4;
    const int64_t cpw = ((vmax + 63) / 64) * 64;
    dim3 grid((unsigned)nqb, 1, (unsigned)b);
    if (idx != nullptr)   // every list fits one workgroup: selection fused (the caller checked)
      hipLaunchKernelGGL((index_scores_mfma<NHB, KS, 1>), grid, dim3(256), 0, st, (const bf16_t*)qI, w,
                         (const bf16_t*)KI, cbs, n_q, t0, n_comp, m, cpw, nqb, scores, k, idx, score_out, sbf);
    else
      hipLaunchKernelGGL((index_scores_mfma<NHB, KS, 0>), grid, dim3(256), 0, st, (const bf16_t*)qI, w,
                         (const bf16_t*)KI, cbs, n_q, t0, n_comp, m, cpw, nqb, scores, k, nullptr, nullptr, sbf);
  } else {
    return launch_scores_stream<NHB, KS, bf16_t>(qI, w, KI, dense_rows(cbs), b, n_q, QPos{t0, nullptr}, vmax,
                                                 n_comp, m, scores, gmax, ld_gmax, gmax_used, st, sbf);
  }
  return hipGetLastError();
}

// Selection from the score rows in the workspace (every path's scoring
// kernel leaves them there): the threshold path when the scorer recorded
// group maxima, else wave segments and workgroup segments until one is left.
static hipError_t finish_topk(const TopkLayout& L, unsigned char* W, float* scores, uint32_t* gmax,
                              bool gmax_used, int dtype, int64_t b, int64_t n_q, QPos t0, int64_t lmax,
                              int64_t n_comp, int64_t m, int64_t k, int32_t* idx, float* score, hipStream_t st) {
  const int64_t rows = b * n_q;
  int64_t nseg = std::max<int64_t>(1, (lmax + kWaveChunk - 1) / kWaveChunk);
  // one wave per row when every list fits one segment
  if (nseg == 1) {
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL((topk_stage<64, kWaveR>), dim3((unsigned)blocks), dim3(256), 0, st, 1, 1, scores,
                       n_comp, nullptr, nullptr, 0, nullptr, nullptr, 0, idx, score, rows, n_q, t0, n_comp,
                       m, k, nullptr, (int64_t)1);
    return hipGetLastError();
  }
  uint32_t* kbuf[2] = {(uint32_t*)(W + L.kA), (uint32_t*)(W + L.kB)};
  int32_t* ibuf[2] = {(int32_t*)(W + L.iA), (int32_t*)(W + L.iB)};
  if (gmax_used) {
    // threshold path: a lower bound on each row's k-th largest score from the
    // group maxima, a filtering pass per 2048-key segment, one exact merge
    int32_t* cnt = (int32_t*)(W + L.cnt);
    const int64_t G = stream_splits_for(dtype, b, n_q, lmax) * kStreamGroupsPerWG;
    // every maximum counts (up to 4096 per row: more of them, a tighter bound)
    const dim3 fgrid((unsigned)rows, (unsigned)((nseg + 3) / 4));
    if (G > 2048)
      hipLaunchKernelGGL(topk_threshold_filter<16>, fgrid, dim3(256), 0, st, scores, n_comp, gmax, L.gcap, G, n_q,
                         t0, n_comp, m, k, nseg, kbuf[0], ibuf[0], L.cap, cnt);
    else
      hipLaunchKernelGGL(topk_threshold_filter<8>, fgrid, dim3(256), 0, st, scores, n_comp, gmax, L.gcap, G, n_q,
                         t0, n_comp, m, k, nseg, kbuf[0], ibuf[0], L.cap, cnt);
    hipLaunchKernelGGL(topk_merge, dim3((unsigned)rows), dim3(256), 0, st, kbuf[0], ibuf[0], L.cap, cnt, nseg, k,
                       idx, score);
    return hipGetLastError();
  }
  // general path: wave segments first, then workgroup segments until one
  // segment is left
  int64_t* lbuf[2] = {(int64_t*)(W + L.lenA), (int64_t*)(W + L.lenB)};
  const unsigned lgrid = (unsigned)((rows + 255) / 256);
  {
    const int64_t blocks = (rows * nseg + 3) / 4;
    hipLaunchKernelGGL((topk_stage<64, kWaveR>), dim3((unsigned)blocks), dim3(256), 0, st, 1, 0, scores,
                       n_comp, nullptr, nullptr, 0, kbuf[0], ibuf[0], L.cap, nullptr, nullptr, rows, n_q, t0,
                       n_comp, m, k, nullptr, nseg);
    hipLaunchKernelGGL(topk_next_len, dim3(lgrid), dim3(256), 0, st, rows, n_q, t0, n_comp, m, k,
                       kWaveChunk, nullptr, lbuf[0]);
  }
  lmax = (nseg - 1) * k + std::min<int64_t>(k, kWaveChunk);   // bound on every next list
  int cur = 0;
  while (true) {
    const int64_t nseg2 = std::max<int64_t>(1, (lmax + kBlockChunk - 1) / kBlockChunk);
    const int fin = nseg2 == 1 ? 1 : 0;
    hipLaunchKernelGGL((topk_stage<256, kBlockR>), dim3((unsigned)(rows * nseg2)), dim3(256), 0, st, 0, fin,
                       nullptr, 0, kbuf[cur], ibuf[cur], L.cap, kbuf[cur ^ 1], ibuf[cur ^ 1], L.cap, idx, score,
                       rows, n_q, t0, n_comp, m, k, lbuf[cur], nseg2);
    if (fin) break;
    hipLaunchKernelGGL(topk_next_len, dim3(lgrid), dim3(256), 0, st, rows, n_q, t0, n_comp, m, k,
                       kBlockChunk, lbuf[cur], lbuf[cur ^ 1]);
    lmax = (nseg2 - 1) * k + std::min<int64_t>(k, kBlockChunk);
    cur ^= 1;
  }
  return hipGetLastError();
}

hipError_t launch_index_topk(const void* qI, const float* w, const void* KI, int64_t cbs, int64_t b,
                             int64_t n_q, int64_t t0, int64_t n_comp, int64_t nh, int64_t cI,
                             int64_t m, int64_t k, int dtype_flags, int32_t* idx, float* score,
                             void* ws, hipStream_t st) {
  const int dtype = dtype_flags & 0xff;
  const int sbf = (dtype_flags & 0x100) ? 1 : 0;   // bf16 index scores
  const TopkLayout L = topk_layout(b, n_q, n_comp, k);
  unsigned char* W = (unsigned char*)ws;
  float* scores = (float*)(W + L.scores);
  uint32_t* gmax = L.gcap > 0 ? (uint32_t*)(W + L.gmax) : nullptr;
  bool gmax_used = false;
  hipError_t err = hipSuccess;
  // four or more queries whose lists fit one 2048-key segment: the scoring
  // kernel selects as well (also when n_comp == 0: it writes the padding)
  const bool mfma_shape = dtype == 1 && (nh == 32 || nh == 64 || nh == 128) && (cI == 64 || cI == 128);
  const bool fused = mfma_shape && n_q >= 4 && n_comp <= kFusedMaxKeys;
  if (n_comp > 0 || fused) {
    bool done = false;
    if (dtype == 1 && nh % 32 == 0 && cI % 16 == 0) {
      const int nhb = (int)(nh / 32), ks = (int)(cI / 16);
#define CSA_SCORES_CASE(A, B)                                                                       \
  if (!done && nhb == A && ks == B) {                                                               \
    err = launch_scores_mfma<A, B>(qI, w, KI, cbs, b, n_q, t0, n_comp, m, scores, gmax, L.gcap,     \
                                   &gmax_used, k, fused ? idx : nullptr, score, st, sbf);           \
    done = true;                                                                                    \
  }
      CSA_SCORES_CASE(1, 4) CSA_SCORES_CASE(1, 8) CSA_SCORES_CASE(2, 4) CSA_SCORES_CASE(2, 8)
      CSA_SCORES_CASE(4, 4) CSA_SCORES_CASE(4, 8)
#undef CSA_SCORES_CASE
    }
    // E4M3 keys and queries, few queries: the streaming kernel on the FP8 MFMA
    if (dtype == 2 && n_q < 4 && nh % 32 == 0 && cI % 16 == 0) {
      const int nhb = (int)(nh / 32), ks = (int)(cI / 16);
#define CSA_STREAM8_CASE(A, B)                                                                          \
  if (!done && nhb == A && ks == B) {                                                                   \
    err = launch_scores_stream<A, B, fp8_t>(qI, w, KI, dense_rows(cbs), b, n_q, QPos{t0, nullptr},      \
                                            std::min<int64_t>((t0 + n_q) / m, n_comp), n_comp, m, scores, \
                                            gmax, L.gcap, &gmax_used, st, sbf);                         \
    done = true;                                                                                        \
  }
      CSA_STREAM8_CASE(1, 4) CSA_STREAM8_CASE(1, 8) CSA_STREAM8_CASE(2, 4) CSA_STREAM8_CASE(2, 8)
      CSA_STREAM8_CASE(4, 4) CSA_STREAM8_CASE(4, 8)
#undef CSA_STREAM8_CASE
    }
    // E4M3 codes, four or more queries: the block-scaled MFMA scorer with
    // unit scales (selection fused when every list fits one workgroup)
    if (!done && dtype == 2 && n_q >= 4 && cI == 128 && (nh == 32 || nh == 64 || nh == 128)) {
      const bool f8fused = n_comp <= kFusedMaxKeys;
      const int64_t nqb = (n_q + 3) / 4;
      dim3 grid((unsigned)nqb, 1, (unsigned)b);
      const uint8_t* q8 = (const uint8_t*)qI;
      const uint8_t* k8 = (const uint8_t*)KI;
      const int64_t cbe = cbs / cI;   // the stride in entries
#define CSA_F8_MFMA(NHB_)                                                                                         \
  if (f8fused)                                                                                                     \
    hipLaunchKernelGGL((index_scores_mfma_mx<NHB_, 1, 0>), grid, dim3(256), 0, st, q8, nullptr, w, k8, nullptr,      \
                       cbe, n_q, t0, n_comp, m, nqb, scores, k, idx, score);                                       \
  else                                                                                                             \
    hipLaunchKernelGGL((index_scores_mfma_mx<NHB_, 0, 0>), grid, dim3(256), 0, st, q8, nullptr, w, k8, nullptr,      \
                       cbe, n_q, t0, n_comp, m, nqb, scores, k, nullptr, nullptr);
      if (nh == 32) {
        CSA_F8_MFMA(1)
      } else if (nh == 64) {
        CSA_F8_MFMA(2)
      } else {
        CSA_F8_MFMA(4)
      }
#undef CSA_F8_MFMA
      err = hipGetLastError();
      if (err != hipSuccess || f8fused) return err;
      done = true;
    }
    if (!done) {
      dim3 grid((unsigned)((n_comp + 255) / 256), (unsigned)n_q, (unsigned)b);
      if (dtype == 1)
        hipLaunchKernelGGL((index_scores_generic<bf16_t>), grid, dim3(256), 0, st, (const bf16_t*)qI,
                           w, (const bf16_t*)KI, cbs, n_q, t0, n_comp, (int)nh, (int)cI, m, scores, sbf);
      else if (dtype == 2)
        hipLaunchKernelGGL((index_scores_generic<fp8_t>), grid, dim3(256), 0, st, (const fp8_t*)qI,
                           w, (const fp8_t*)KI, cbs, n_q, t0, n_comp, (int)nh, (int)cI, m, scores, sbf);
      else
        hipLaunchKernelGGL((index_scores_generic<float>), grid, dim3(256), 0, st, (const float*)qI,
                           w, (const float*)KI, cbs, n_q, t0, n_comp, (int)nh, (int)cI, m, scores, sbf);
      err = hipGetLastError();
    }
    if (err != hipSuccess) return err;
    if (fused && done) return hipSuccess;
  }
  return finish_topk(L, W, scores, gmax, gmax_used, dtype, b, n_q, QPos{t0, nullptr},
                     std::min<int64_t>((t0 + n_q) / m, n_comp), n_comp, m, k, idx, score, st);
}

// MXFP4 queries and keys: the streaming scorer for few queries at c_I = 128
// and 32-head multiples, generic scoring otherwise; the same selection.
static bool mx_stream_shape(int64_t n_q, int64_t nh, int64_t cI) {
  return n_q < 4 && cI == 128 && (nh == 32 || nh == 64 || nh == 128);
}

bool index_topk_mx_supported(int64_t n_q, int64_t nh, int64_t cI) {
  if (cI < 32 || cI % 32 != 0) return false;
  return (cI == 128 && (nh == 32 || nh == 64 || nh == 128)) || nh * cI <= kMxGenericMaxQ;
}

hipError_t launch_index_topk_mx(const void* qI, const void* qS, const float* w, const void* KI, const void* KS,
                                int64_t cbs, int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t nh,
                                int64_t cI, int64_t m, int64_t k, int32_t* idx, float* score, void* ws,
                                hipStream_t st) {
  const TopkLayout L = topk_layout(b, n_q, n_comp, k);
  unsigned char* W = (unsigned char*)ws;
  float* scores = (float*)(W + L.scores);
  uint32_t* gmax = L.gcap > 0 ? (uint32_t*)(W + L.gmax) : nullptr;
  bool gmax_used = false;
  const uint8_t* q8 = (const uint8_t*)qI;
  const uint8_t* qs8 = (const uint8_t*)qS;
  const uint8_t* k8 = (const uint8_t*)KI;
  const uint8_t* ks8 = (const uint8_t*)KS;
  const bool mfma_shape = cI == 128 && (nh == 32 || nh == 64 || nh == 128);
  if (mfma_shape && n_q >= 4) {
    // four queries per workgroup, every key of the block's lists in one
    // workgroup; the selection is fused when every list fits it (also when
    // n_comp == 0: the kernel writes the padding)
    const bool fused = n_comp <= kFusedMaxKeys;
    const int64_t nqb = (n_q + 3) / 4;
    dim3 grid((unsigned)nqb, 1, (unsigned)b);
    int32_t* fi = fused ? idx : nullptr;
    float* fs = fused ? score : nullptr;
#define CSA_MX_MFMA(NHB_)                                                                                        \
  if (fused)                                                                                                      \
    hipLaunchKernelGGL((index_scores_mfma_mx<NHB_, 1, 4>), grid, dim3(256), 0, st, q8, qs8, w, k8, ks8, cbs, n_q, t0, \
                       n_comp, m, nqb, scores, k, fi, fs);                                                         \
  else                                                                                                            \
    hipLaunchKernelGGL((index_scores_mfma_mx<NHB_, 0, 4>), grid, dim3(256), 0, st, q8, qs8, w, k8, ks8, cbs, n_q, t0, \
                       n_comp, m, nqb, scores, k, nullptr, nullptr);
    if (nh == 32) {
      CSA_MX_MFMA(1)
    } else if (nh == 64) {
      CSA_MX_MFMA(2)
    } else {
      CSA_MX_MFMA(4)
    }
#undef CSA_MX_MFMA
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || fused) return err;
    return finish_topk(L, W, scores, gmax, false, 3, b, n_q, QPos{t0, nullptr},
                       std::min<int64_t>((t0 + n_q) / m, n_comp), n_comp, m, k, idx, score, st);
  }
  if (n_comp > 0) {
    if (mx_stream_shape(n_q, nh, cI)) {
      const int64_t vmax = std::min<int64_t>((t0 + n_q) / m, n_comp);
      const int64_t nsplit = stream_splits(b, n_q, vmax, StreamPolicyMx::keys, StreamPolicyMx::wgs);
      dim3 grid((unsigned)n_q, (unsigned)nsplit, (unsigned)b);
      constexpr int D = StreamPolicyMx::ring, SBK = (int)StreamPolicyMx::keys;
      if (nh == 32)
        hipLaunchKernelGGL((index_scores_stream_mx<1, D, SBK>), grid, dim3(256), 0, st, q8, qs8, w, k8, ks8, cbs,
                           n_q, t0, n_comp, m, scores, gmax, L.gcap);
      else if (nh == 64)
        hipLaunchKernelGGL((index_scores_stream_mx<2, D, SBK>), grid, dim3(256), 0, st, q8, qs8, w, k8, ks8, cbs,
                           n_q, t0, n_comp, m, scores, gmax, L.gcap);
      else
        hipLaunchKernelGGL((index_scores_stream_mx<4, D, SBK>), grid, dim3(256), 0, st, q8, qs8, w, k8, ks8, cbs,
                           n_q, t0, n_comp, m, scores, gmax, L.gcap);
      gmax_used = gmax != nullptr;
    } else {
      dim3 grid((unsigned)((n_comp + 255) / 256), (unsigned)n_q, (unsigned)b);
      hipLaunchKernelGGL(index_scores_generic_mx, grid, dim3(256), 0, st, q8, qs8, w, k8, ks8, cbs, n_q, t0,
                         n_comp, (int)nh, (int)cI, m, scores);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return finish_topk(L, W, scores, gmax, gmax_used, 3, b, n_q, QPos{t0, nullptr},
                     std::min<int64_t>((t0 + n_q) / m, n_comp), n_comp, m, k, idx, score, st);
}

// Paged decode: one query per batch row at its own position pos[b], keys
// located through the block table (a block holds a multiple of 32 keys, so
// every 32-key tile lies in one block); the streaming scorer, then the same
// selection as csa_index_topk.  bf16 keys, 32/64/128 heads, c_I = 64 or 128.
bool index_topk_paged_supported(int64_t nh, int64_t cI) {
  return (nh == 32 || nh == 64 || nh == 128) && (cI == 64 || cI == 128);
}

hipError_t launch_index_topk_paged(const void* qI, const float* w, const void* pool, const Rows& kr,
                                   const int64_t* pos, int64_t b, int64_t n_comp_max, int64_t nh, int64_t cI,
                                   int64_t m, int64_t k, int32_t* idx, float* score, void* ws, hipStream_t st) {
  const TopkLayout L = topk_layout(b, 1, n_comp_max, k);
  unsigned char* W = (unsigned char*)ws;
  float* scores = (float*)(W + L.scores);
  uint32_t* gmax = L.gcap > 0 ? (uint32_t*)(W + L.gmax) : nullptr;
  bool gmax_used = false;
  hipError_t err = hipSuccess;
  const QPos qp{0, pos};
  if (n_comp_max > 0) {
    const int nhb = (int)(nh / 32);
    if (cI == 128) {
      if (nhb == 1) err = launch_scores_stream<1, 8, bf16_t>(qI, w, pool, kr, b, 1, qp, n_comp_max, n_comp_max, m,
                                                             scores, gmax, L.gcap, &gmax_used, st);
      else if (nhb == 2) err = launch_scores_stream<2, 8, bf16_t>(qI, w, pool, kr, b, 1, qp, n_comp_max, n_comp_max,
                                                                  m, scores, gmax, L.gcap, &gmax_used, st);
      else err = launch_scores_stream<4, 8, bf16_t>(qI, w, pool, kr, b, 1, qp, n_comp_max, n_comp_max, m, scores,
                                                    gmax, L.gcap, &gmax_used, st);
    } else {
      if (nhb == 1) err = launch_scores_stream<1, 4, bf16_t>(qI, w, pool, kr, b, 1, qp, n_comp_max, n_comp_max, m,
                                                             scores, gmax, L.gcap, &gmax_used, st);
      else if (nhb == 2) err = launch_scores_stream<2, 4, bf16_t>(qI, w, pool, kr, b, 1, qp, n_comp_max, n_comp_max,
                                                                  m, scores, gmax, L.gcap, &gmax_used, st);
      else err = launch_scores_stream<4, 4, bf16_t>(qI, w, pool, kr, b, 1, qp, n_comp_max, n_comp_max, m, scores,
                                                    gmax, L.gcap, &gmax_used, st);
    }
    if (err != hipSuccess) return err;
  }
  return finish_topk(L, W, scores, gmax, gmax_used, 1, b, 1, qp, n_comp_max, n_comp_max, m, k, idx, score, st);
}

}  // namespace csa
