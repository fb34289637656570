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
// ReLU * w reduction over the heads, so it runs on the bf16 MFMA unit: each
// wave keeps its query's 32*NHB x c_I operand in registers and streams key
// tiles that the workgroup stages once in LDS.  Selection is a radix-style
// threshold search over order-preserving 32-bit keys, then an ordered
// compaction, with a fixed reduction order everywhere.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// ---------------------------------------------------------------------------
// Generic scoring (any dtype, any head count / dimension): one thread per
// (query, key).  Used for float32 and for shapes the MFMA kernel does not
// cover.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void index_scores_generic(
    const T* __restrict__ qI, const float* __restrict__ w, const T* __restrict__ KI,
    int64_t comp_bs, int64_t n_q, int64_t t0, int64_t n_comp, int nh, int cI, int64_t m,
    float* __restrict__ scores) {
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
  scores[(bi * n_q + r) * n_comp + s] = tot;
}

// ---------------------------------------------------------------------------
// MFMA scoring, bf16.  NHB = heads / 32, KS = c_I / 16.  A workgroup has 4
// waves; QW of them (1 or 4) carry distinct queries and the 4/QW waves that
// share a query split each key tile.  The workgroup stages TN = 64*(4/QW)
// keys per tile in LDS; each wave multiplies its query block by 64 keys with
// v_mfma_f32_32x32x16_bf16 and reduces over heads in registers.
//
// Operand layouts of the 32x32x16 MFMA (lane l, j < 8):
//   A[i][k] : lane holds A[l%32][8*(l/32) + j]
//   B[k][n] : lane holds B[8*(l/32) + j][l%32]
//   D[i][n] : lane holds D[8*(r/4) + 4*(l/32) + r%4][l%32] in register r
// ---------------------------------------------------------------------------
template <int NHB, int KS, int QW>
__global__ __launch_bounds__(256) void index_scores_mfma(
    const bf16_t* __restrict__ qI, const float* __restrict__ w, const bf16_t* __restrict__ KI,
    int64_t comp_bs, int64_t n_q, int64_t t0, int64_t n_comp, int64_t m, int64_t cand_per_wg,
    int64_t n_qblocks, float* __restrict__ scores) {
  constexpr int CI = KS * 16;
  constexpr int NH = NHB * 32;
  constexpr int SUB = 4 / QW;            // waves sharing one query
  constexpr int TN = 64 * SUB;           // keys per LDS tile
  constexpr int ROWB = CI * 2 + 16;      // padded LDS row (bytes): conflict-free b128 reads
  constexpr int U4_PER_ROW = CI / 8;     // 16-byte pieces per key row
  constexpr int LOADS = TN * U4_PER_ROW / 256;
  static_assert(LOADS >= 1 && (TN * U4_PER_ROW) % 256 == 0, "tile must split over 256 threads");
  __shared__ __attribute__((aligned(16))) unsigned char lds[TN * ROWB];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  // heaviest (latest) query blocks first: causal work grows with position
  const int64_t qb = n_qblocks - 1 - blockIdx.x;
  const int64_t bi = blockIdx.z;
  const int64_t qrow = qb * QW + (wave % QW);
  const int sub = wave / QW;
  const bool qvalid = qrow < n_q;

  int64_t vis_q = qvalid ? (t0 + qrow + 1) / m : 0;
  if (vis_q > n_comp) vis_q = n_comp;
  int64_t last = qb * QW + QW - 1;
  if (last > n_q - 1) last = n_q - 1;
  int64_t vis_wg = (t0 + last + 1) / m;
  if (vis_wg > n_comp) vis_wg = n_comp;
  const int64_t c0 = (int64_t)blockIdx.y * cand_per_wg;
  int64_t c1 = c0 + cand_per_wg;
  if (c1 > vis_wg) c1 = vis_wg;
  if (c0 >= c1) return;

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

  const bf16_t* kbase = KI + bi * comp_bs;
  float* srow = scores + (bi * n_q + (qvalid ? qrow : 0)) * n_comp;
  uint4 pre[LOADS];
  auto load_tile = [&](int64_t tb) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int p = i * 256 + tid;
      const int row = p / U4_PER_ROW, col = p % U4_PER_ROW;
      const int64_t key = tb + row;
      pre[i] = key < n_comp ? *reinterpret_cast<const uint4*>(kbase + key * CI + col * 8)
                            : make_uint4(0, 0, 0, 0);
    }
  };
  load_tile(c0);
  for (int64_t tb = c0; tb < c1; tb += TN) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int p = i * 256 + tid;
      const int row = p / U4_PER_ROW, col = p % U4_PER_ROW;
      *reinterpret_cast<uint4*>(lds + row * ROWB + col * 16) = pre[i];
    }
    __syncthreads();
    if (tb + TN < c1) load_tile(tb + TN);

    const int64_t kb = tb + sub * 64;  // this wave's 64 keys
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
          const int row = sub * 64 + nb * 32 + (l & 31);
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(lds + row * ROWB + ks * 32 + 16 * (l >> 5));
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
      if (cand < vis_q) srow[cand] = (l < 32) ? s2[0] : s2[1];
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming MFMA scoring for few queries (decode), bf16.  Nothing is shared
// between waves, so there is no LDS and no barrier: each wave keeps its
// query's 32*NHB x c_I operand in registers and walks 32-key tiles of its
// workgroup's key range (tiles wave, wave+4, ...), loading the B operand of
// the next tile straight from HBM while the MFMAs of the current one run.
// Per key the only traffic is its c_I bf16 values and one float score.
// ---------------------------------------------------------------------------
template <int NHB, int KS>
__global__ __launch_bounds__(256) void index_scores_stream(
    const bf16_t* __restrict__ qI, const float* __restrict__ w, const bf16_t* __restrict__ KI,
    int64_t comp_bs, int64_t n_q, int64_t t0, int64_t n_comp, int64_t m, int64_t cand_per_wg,
    float* __restrict__ scores) {
  constexpr int CI = KS * 16;
  constexpr int NH = NHB * 32;
  const int wave = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int64_t qrow = blockIdx.x;
  const int64_t bi = blockIdx.z;
  int64_t vis = (t0 + qrow + 1) / m;
  if (vis > n_comp) vis = n_comp;
  const int64_t c0 = (int64_t)blockIdx.y * cand_per_wg;
  int64_t c1 = c0 + cand_per_wg;
  if (c1 > vis) c1 = vis;
  const int64_t first = c0 + 32 * wave;
  if (first >= c1) return;

  bf16x8 qa[NHB][KS];
  float wv[NHB][16];
  const int64_t qoff = (bi * n_q + qrow) * (int64_t)NH;
#pragma unroll
  for (int mb = 0; mb < NHB; ++mb) {
    const bf16_t* qp = qI + (qoff + mb * 32 + (l & 31)) * CI + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qa[mb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 16));
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[mb][r] = w[qoff + mb * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3)];
  }

  const bf16_t* kbase = KI + bi * comp_bs;
  float* srow = scores + (bi * n_q + qrow) * n_comp;
  const int64_t lastkey = c1 - 1;
  // lane's 16-byte slice of key (tile + l % 32), dims 8 * (l / 32) + 16 * ks
  auto load_tile = [&](int64_t kb, uint4 (&dst)[KS]) {
    int64_t key = kb + (l & 31);
    key = key < lastkey ? key : lastkey;
    const bf16_t* kp = kbase + key * CI + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = *reinterpret_cast<const uint4*>(kp + ks * 16);
  };
  uint4 cur[KS], nxt[KS];
  load_tile(first, cur);
  for (int64_t kb = first; kb < c1; kb += 128) {
    const bool more = kb + 128 < c1;
    if (more) load_tile(kb + 128, nxt);
    f32x16 acc[NHB];
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb) acc[mb] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 bv = __builtin_bit_cast(bf16x8, cur[ks]);
#pragma unroll
      for (int mb = 0; mb < NHB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], bv, acc[mb], 0, 0, 0);
    }
    float sc = 0.f;
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc = fmaf(fmaxf(acc[mb][r], 0.f), wv[mb][r], sc);
    sc += __shfl_xor(sc, 32, 64);
    const int64_t key = kb + l;
    if (l < 32 && key < c1) srow[key] = sc;
    if (more) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) cur[ks] = nxt[ks];
    }
  }
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
// exchange per step in the workgroup form).  Keys > T are taken, then keys
// == T in list order until k are taken (ties go to the lower index), and the
// taken elements are compacted in list order.
// ---------------------------------------------------------------------------
template <int NT>
struct SegReduce {
  // sum of a wave-uniform count over the NT/64 waves (LDS exchange when NT > 64)
  static __device__ __forceinline__ uint32_t sum(uint32_t c, uint32_t* red, int wave, int& parity) {
    if constexpr (NT == 64) {
      return c;
    } else {
      uint32_t* slot = red + parity * (NT / 64);
      parity ^= 1;
      if ((threadIdx.x & 63) == 0) slot[wave] = c;
      __syncthreads();
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) t += slot[w];
      return t;
    }
  }
  static __device__ __forceinline__ uint32_t umax(uint32_t v, uint32_t* red, int wave, int& parity) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    if constexpr (NT == 64) {
      return v;
    } else {
      uint32_t* slot = red + parity * (NT / 64);
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

// Select the top k of the segment held in key[] (valid where e < len; the
// caller zeroes the keys of invalid slots, so that no candidate threshold,
// which is always >= 1, counts them);
// writes the selection flags into sel[].  `red` is LDS scratch of
// 2 * NT/64 words (unused for NT == 64); `pre` is LDS scratch of R * NT/64
// words used for list-order ranks.
template <int NT, int R>
__device__ __forceinline__ void segment_select(const uint32_t (&key)[R], int len, int k, bool (&sel)[R],
                                               uint32_t* red, uint32_t* pre) {
  const int tid = threadIdx.x % NT, wave = tid >> 6, l = tid & 63;
  int parity = 0;
  bool val[R];
#pragma unroll
  for (int r = 0; r < R; ++r) val[r] = r * NT + tid < len;
  if (len <= k) {
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
  if (diff == 0) {
    T = hi;
  } else {
    const int top = 31 - __clz(diff);
    T = top == 31 ? 0u : (hi >> (top + 1)) << (top + 1);
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t c = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) c += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(key[r] >= cand));
      c = SegReduce<NT>::sum(c, red, wave, parity);
      if (c >= (uint32_t)k) T = cand;
    }
  }
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
    float* __restrict__ score_out, int64_t n_rows, int64_t n_q, int64_t t0, int64_t n_comp, int64_t m,
    int64_t k, const int64_t* __restrict__ len_in, int64_t nseg) {
  constexpr int CH = NT * R;
  constexpr int SEGS = 256 / NT;   // segments per workgroup
  __shared__ uint32_t red_all[SEGS][2 * (NT / 64) + 1];
  __shared__ uint32_t pre_all[SEGS][R * (NT / 64) + 1];
  const int sub = threadIdx.x / NT;
  const int tid = threadIdx.x % NT;
  const int64_t gseg = (int64_t)blockIdx.x * SEGS + sub;   // global segment id over (row, seg)
  const bool active = gseg < n_rows * nseg;
  const int64_t row = active ? gseg / nseg : 0;
  const int64_t seg = active ? gseg % nseg : 0;
  int64_t L;
  if (from_scores) {
    L = (t0 + row % n_q + 1) / m;
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
  bool sel[R];
  segment_select<NT, R>(key, len, (int)k, sel, red_all[sub], pre_all[sub]);
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

// Next-stage list length per row: (nseg - 1) * k + min(k, last segment).
__global__ void topk_next_len(int64_t n_rows, int64_t n_q, int64_t t0, int64_t n_comp, int64_t m,
                              int64_t k, int64_t chunk, const int64_t* __restrict__ len_in,
                              int64_t* __restrict__ len_out) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= n_rows) return;
  int64_t L;
  if (len_in == nullptr) {
    L = (t0 + row % n_q + 1) / m;
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

// Workspace: scores [rows, n_comp] f32 | len A, len B [rows] i64 |
//            pairs A, pairs B [rows, cap] (u32 key + i32 idx each)
struct TopkLayout {
  size_t scores, lenA, lenB, kA, iA, kB, iB, total;
  int64_t cap;
};
static TopkLayout topk_layout(int64_t b, int64_t n_q, int64_t n_comp, int64_t k) {
  TopkLayout L{};
  const int64_t rows = b * n_q;
  const int64_t nch = (n_comp + kWaveChunk - 1) / kWaveChunk;
  L.cap = nch > 1 ? nch * k : 0;
  size_t off = 0;
  L.scores = off; off = align256(off + (size_t)rows * n_comp * 4);
  L.lenA = off; off = align256(off + (size_t)rows * 8);
  L.lenB = off; off = align256(off + (size_t)rows * 8);
  L.kA = off; off = align256(off + (size_t)rows * L.cap * 4);
  L.iA = off; off = align256(off + (size_t)rows * L.cap * 4);
  L.kB = off; off = align256(off + (size_t)rows * L.cap * 4);
  L.iB = off; off = align256(off + (size_t)rows * L.cap * 4);
  L.total = off;
  return L;
}

size_t index_topk_workspace_bytes(int64_t b, int64_t n_q, int64_t n_comp, int64_t k) {
  return topk_layout(b, n_q, n_comp, k).total;
}

bool index_topk_supported(int64_t n_comp, int64_t k) {
  // multi-stage selection needs each stage to shrink the list at least 2x
  return n_comp <= kWaveChunk || k <= kWaveChunk / 2;
}

// keys per workgroup of the streaming (decode) scoring kernel
constexpr int64_t kStreamKeysPerWG = 4096;

template <int NHB, int KS>
static hipError_t launch_scores_mfma(const void* qI, const float* w, const void* KI, int64_t cbs,
                                     int64_t b, int64_t n_q, int64_t t0, int64_t n_comp, int64_t m,
                                     float* scores, hipStream_t st) {
  const int64_t vmax = std::min<int64_t>((t0 + n_q) / m, n_comp);
  if (n_q >= 4) {
    const int64_t nqb = (n_q + 3) / 4;
    const int64_t cpw = ((vmax + 63) / 64) * 64;
    dim3 grid((unsigned)nqb, 1, (unsigned)b);
    hipLaunchKernelGGL((index_scores_mfma<NHB, KS, 4>), grid, dim3(256), 0, st, (const bf16_t*)qI, w,
                       (const bf16_t*)KI, cbs, n_q, t0, n_comp, m, cpw, nqb, scores);
  } else {
    // few queries (decode): split each query's keys over many workgroups
    const int64_t cpw = kStreamKeysPerWG;
    const int64_t nsplit = std::max<int64_t>(1, (vmax + cpw - 1) / cpw);
    dim3 grid((unsigned)n_q, (unsigned)nsplit, (unsigned)b);
    hipLaunchKernelGGL((index_scores_stream<NHB, KS>), grid, dim3(256), 0, st, (const bf16_t*)qI, w,
                       (const bf16_t*)KI, cbs, n_q, t0, n_comp, m, cpw, scores);
  }
  return hipGetLastError();
}

hipError_t launch_index_topk(const void* qI, const float* w, const void* KI, int64_t cbs, int64_t b,
                             int64_t n_q, int64_t t0, int64_t n_comp, int64_t nh, int64_t cI,
                             int64_t m, int64_t k, int dtype, int32_t* idx, float* score,
                             void* ws, hipStream_t st) {
  const TopkLayout L = topk_layout(b, n_q, n_comp, k);
  unsigned char* W = (unsigned char*)ws;
  float* scores = (float*)(W + L.scores);
  hipError_t err = hipSuccess;
  if (n_comp > 0) {
    bool done = false;
    if (dtype == 1 && nh % 32 == 0 && cI % 16 == 0) {
      const int nhb = (int)(nh / 32), ks = (int)(cI / 16);
#define CSA_SCORES_CASE(A, B)                                                                   \
  if (!done && nhb == A && ks == B) {                                                           \
    err = launch_scores_mfma<A, B>(qI, w, KI, cbs, b, n_q, t0, n_comp, m, scores, st);         \
    done = true;                                                                                \
  }
      CSA_SCORES_CASE(1, 4) CSA_SCORES_CASE(1, 8) CSA_SCORES_CASE(2, 4) CSA_SCORES_CASE(2, 8)
      CSA_SCORES_CASE(4, 4) CSA_SCORES_CASE(4, 8)
#undef CSA_SCORES_CASE
    }
    if (!done) {
      dim3 grid((unsigned)((n_comp + 255) / 256), (unsigned)n_q, (unsigned)b);
      if (dtype == 1)
        hipLaunchKernelGGL((index_scores_generic<bf16_t>), grid, dim3(256), 0, st, (const bf16_t*)qI,
                           w, (const bf16_t*)KI, cbs, n_q, t0, n_comp, (int)nh, (int)cI, m, scores);
      else
        hipLaunchKernelGGL((index_scores_generic<float>), grid, dim3(256), 0, st, (const float*)qI,
                           w, (const float*)KI, cbs, n_q, t0, n_comp, (int)nh, (int)cI, m, scores);
      err = hipGetLastError();
    }
    if (err != hipSuccess) return err;
  }
  // selection: one wave per row when every list fits one segment; otherwise
  // wave segments first, then workgroup segments until one segment is left
  const int64_t rows = b * n_q;
  int64_t lmax = std::min<int64_t>((t0 + n_q) / m, n_comp);
  int64_t nseg = std::max<int64_t>(1, (lmax + kWaveChunk - 1) / kWaveChunk);
  if (nseg == 1) {
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL((topk_stage<64, kWaveR>), dim3((unsigned)blocks), dim3(256), 0, st, 1, 1, scores,
                       n_comp, nullptr, nullptr, 0, nullptr, nullptr, 0, idx, score, rows, n_q, t0, n_comp,
                       m, k, nullptr, (int64_t)1);
    return hipGetLastError();
  }
  uint32_t* kbuf[2] = {(uint32_t*)(W + L.kA), (uint32_t*)(W + L.kB)};
  int32_t* ibuf[2] = {(int32_t*)(W + L.iA), (int32_t*)(W + L.iB)};
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

}  // namespace csa
