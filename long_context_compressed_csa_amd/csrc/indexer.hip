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
// Top-k selection over one list segment with 256 threads x R keys.
// Element e of the segment sits in thread e % 256, slot e / 256, so slot
// order then thread order is list order.
//
// mode 0: keys come from scores[row][base + e], idx = base + e
// mode 1: keys/idx come from (kin, iin) pairs
// final:  write idx (int32, ascending list order, -1 padded to k) and the
//         scores; otherwise write the selected pairs compactly to
//         (kout, iout) at slot offset chunk * k.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void topk_select_kernel(
    int mode, int final_stage, const float* __restrict__ scores, int64_t ld_scores,
    const uint32_t* __restrict__ kin, const int32_t* __restrict__ iin, int64_t ld_in,
    uint32_t* __restrict__ kout, int32_t* __restrict__ iout, int64_t ld_out, int32_t* __restrict__ idx,
    float* __restrict__ score_out, int64_t n_q, int64_t t0, int64_t n_comp, int64_t m, int64_t k,
    const int64_t* __restrict__ len_override) {
  constexpr int CHUNK = 256 * R;
  __shared__ uint32_t red[2][4];
  __shared__ uint32_t cnt_eq[R][4];
  __shared__ uint32_t cnt_sel[R][4];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int64_t row = blockIdx.y + (int64_t)blockIdx.z * n_q;  // (b, query)
  const int64_t chunk = blockIdx.x;
  // length of this query's full list
  int64_t L;
  if (mode == 0) {
    L = (t0 + blockIdx.y + 1) / m;
    if (L > n_comp) L = n_comp;
  } else {
    L = len_override[row];
  }
  const int64_t base = chunk * CHUNK;
  if (base >= L && !(final_stage && chunk == 0)) return;
  int64_t len = L - base;
  if (len > CHUNK) len = CHUNK;
  if (len < 0) len = 0;

  uint32_t key[R];
  int32_t ix[R];
  bool val[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t e = (int64_t)r * 256 + tid;
    val[r] = e < len;
    if (mode == 0) {
      key[r] = val[r] ? f2key(scores[row * ld_scores + base + e]) : 0u;
      ix[r] = (int32_t)(base + e);
    } else {
      key[r] = val[r] ? kin[row * ld_in + base + e] : 0u;
      ix[r] = val[r] ? iin[row * ld_in + base + e] : -1;
    }
  }

  const int64_t take = len < k ? len : k;
  bool sel[R];
  if (len <= k) {
#pragma unroll
    for (int r = 0; r < R; ++r) sel[r] = val[r];
  } else {
    // largest T with #{key >= T} >= k, one bit at a time from the top
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t c = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) c += (val[r] && key[r] >= cand) ? 1u : 0u;
      c = wave_sum_u32(c);
      const int slot = bit & 1;
      if (l == 0) red[slot][wave] = c;
      __syncthreads();
      const uint32_t tot = red[slot][0] + red[slot][1] + red[slot][2] + red[slot][3];
      if (tot >= (uint32_t)k) T = cand;
    }
    uint32_t gt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) gt += (val[r] && key[r] > T) ? 1u : 0u;
    gt = wave_sum_u32(gt);
    if (l == 0) red[0][wave] = gt;
    // exclusive rank of each tie (key == T) in list order
    uint64_t meq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      meq[r] = __ballot(val[r] && key[r] == T);
      if (l == 0) cnt_eq[r][wave] = (uint32_t)__popcll(meq[r]);
    }
    __syncthreads();
    const uint32_t gt_tot = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const uint32_t need_eq = (uint32_t)k - gt_tot;
    uint32_t run = 0;
    const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t before = run;
      for (int w2 = 0; w2 < wave; ++w2) before += cnt_eq[r][w2];
      before += (uint32_t)__popcll(meq[r] & below);
      const bool eq = val[r] && key[r] == T;
      sel[r] = (val[r] && key[r] > T) || (eq && before < need_eq);
      run += cnt_eq[r][0] + cnt_eq[r][1] + cnt_eq[r][2] + cnt_eq[r][3];
    }
  }
  // ordered compaction of the selected elements
  uint64_t msel[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    msel[r] = __ballot(sel[r]);
    if (l == 0) cnt_sel[r][wave] = (uint32_t)__popcll(msel[r]);
  }
  __syncthreads();
  {
    uint32_t run = 0;
    const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t pos = run;
      for (int w2 = 0; w2 < wave; ++w2) pos += cnt_sel[r][w2];
      pos += (uint32_t)__popcll(msel[r] & below);
      if (sel[r]) {
        if (final_stage) {
          idx[row * k + pos] = ix[r];
          if (score_out) score_out[row * k + pos] = key2f(key[r]);
        } else {
          kout[row * ld_out + chunk * k + pos] = key[r];
          iout[row * ld_out + chunk * k + pos] = ix[r];
        }
      }
      run += cnt_sel[r][0] + cnt_sel[r][1] + cnt_sel[r][2] + cnt_sel[r][3];
    }
  }
  if (final_stage) {
    for (int64_t p = take + tid; p < k; p += 256) {
      idx[row * k + p] = -1;
      if (score_out) score_out[row * k + p] = 0.f;
    }
  }
}

// Next-stage list length per query: (nchunks - 1) * k + min(k, last chunk).
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
constexpr int kTopkR = 16;
constexpr int64_t kTopkChunk = 256 * kTopkR;

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
  const int64_t nch = (n_comp + kTopkChunk - 1) / kTopkChunk;
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
  // multi-stage selection needs each stage to shrink the list
  return n_comp <= kTopkChunk || k <= kTopkChunk / 2;
}

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
    const int64_t cpw = 1024;
    const int64_t nsplit = std::max<int64_t>(1, (vmax + cpw - 1) / cpw);
    dim3 grid((unsigned)n_q, (unsigned)nsplit, (unsigned)b);
    hipLaunchKernelGGL((index_scores_mfma<NHB, KS, 1>), grid, dim3(256), 0, st, (const bf16_t*)qI, w,
                       (const bf16_t*)KI, cbs, n_q, t0, n_comp, m, cpw, n_q, scores);
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
  // selection: stage 1 reads scores; further stages shrink the candidate list
  const int64_t rows = b * n_q;
  int64_t nch = std::max<int64_t>(1, (n_comp + kTopkChunk - 1) / kTopkChunk);
  if (nch == 1) {
    dim3 grid(1, (unsigned)n_q, (unsigned)b);
    hipLaunchKernelGGL((topk_select_kernel<kTopkR>), grid, dim3(256), 0, st, 0, 1, scores, n_comp,
                       nullptr, nullptr, 0, nullptr, nullptr, 0, idx, score, n_q, t0, n_comp, m, k,
                       nullptr);
    return hipGetLastError();
  }
  uint32_t* kbuf[2] = {(uint32_t*)(W + L.kA), (uint32_t*)(W + L.kB)};
  int32_t* ibuf[2] = {(int32_t*)(W + L.iA), (int32_t*)(W + L.iB)};
  int64_t* lbuf[2] = {(int64_t*)(W + L.lenA), (int64_t*)(W + L.lenB)};
  const unsigned lgrid = (unsigned)((rows + 255) / 256);
  {
    dim3 grid((unsigned)nch, (unsigned)n_q, (unsigned)b);
    hipLaunchKernelGGL((topk_select_kernel<kTopkR>), grid, dim3(256), 0, st, 0, 0, scores, n_comp,
                       nullptr, nullptr, 0, kbuf[0], ibuf[0], L.cap, nullptr, nullptr, n_q, t0,
                       n_comp, m, k, nullptr);
    hipLaunchKernelGGL(topk_next_len, dim3(lgrid), dim3(256), 0, st, rows, n_q, t0, n_comp, m, k,
                       kTopkChunk, nullptr, lbuf[0]);
  }
  // an upper bound of every list length after stage 1
  int64_t lmax = (nch - 1) * k + std::min<int64_t>(k, kTopkChunk);
  int cur = 0;
  while (true) {
    const int64_t nch2 = std::max<int64_t>(1, (lmax + kTopkChunk - 1) / kTopkChunk);
    const int fin = nch2 == 1 ? 1 : 0;
    dim3 grid((unsigned)nch2, (unsigned)n_q, (unsigned)b);
    hipLaunchKernelGGL((topk_select_kernel<kTopkR>), grid, dim3(256), 0, st, 1, fin, nullptr,
                       0, kbuf[cur], ibuf[cur], L.cap, kbuf[cur ^ 1], ibuf[cur ^ 1], L.cap, idx, score,
                       n_q, t0, n_comp, m, k, lbuf[cur]);
    if (fin) break;
    hipLaunchKernelGGL(topk_next_len, dim3(lgrid), dim3(256), 0, st, rows, n_q, t0, n_comp, m, k,
                       kTopkChunk, lbuf[cur], lbuf[cur ^ 1]);
    lmax = (nch2 - 1) * k + std::min<int64_t>(k, kTopkChunk);
    cur ^= 1;
  }
  return hipGetLastError();
}

}  // namespace csa
