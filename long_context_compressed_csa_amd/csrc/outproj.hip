// Grouped output projection (songhuiming "DeepSeek-V4 百万 token 上下文"
// section 4.4; AirCoding "deepseek-paper-analysis" section 7.1): the n_h head
// outputs of a token split into g groups of consecutive heads; group j's
// concatenated output is projected to d_g values by W^G_j, and the g results,
// concatenated in group order, are projected to d by W^O.
//
// Both projections are one kernel: C[b] (M x N) = A[b] (M x K) B[b]^T, where
// B[b] is N x K, bf16 operands with K contiguous, float32 accumulation on
// v_mfma_f32_32x32x16_bf16, bf16 results.  The first projection is a batch
// of g products (A = the group's columns of the head outputs, B = W^G_j, C =
// the group's columns of the intermediate), the second a single product.
//
// A workgroup (4 waves) computes a 256 x 256 tile of C; wave w owns rows
// 128*(w/2) .. +127 and columns 128*(w%2) .. +127 as 4 x 4 blocks of 32 x 32
// (256 accumulators, in the accumulation registers), so every 16-byte
// operand read from LDS feeds four MFMAs: the LDS port, shared by the
// gathers and the operand reads, stays below the MFMA rate.  K advances 32
// at a time through a ring of four LDS stages (32 KiB each: 256 A rows and
// 256 B rows of 64 bytes), filled by LDS-DMA three stages ahead
// (global_load_lds_dwordx4, 16 rows of 64 B per wave instruction); each
// step's barrier also covers the next stage, whose operands are read into a
// second register set while the current stage's MFMAs run.  Chunk c
// (16 B) of tile row r sits at position c ^ ((r >> 2) & 3) of its row, so the
// operand reads of 16 consecutive rows at one chunk hit 16 distinct bank
// groups.  The tile grid is split into an xr x xc grid of blocks, one per
// XCD (dispatch index mod 8), the split chosen to read the least from HBM
// (A once per column group, B once per row group): tiles sharing A rows or
// B rows share that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int kGBM = 256, kGBN = 256, kGBK = 32;
constexpr int kGRowB = kGBK * 2;                   // bytes per tile row
constexpr int kGCPR = kGBK / 8;                    // 16-byte chunks per tile row
constexpr int kGRPI = 1024 / kGRowB;               // tile rows per gather instruction
constexpr int kGSwzShift = kGCPR == 8 ? 1 : 2;     // rows sharing one chunk permutation: 2 or 4
constexpr int kGStageB = (kGBM + kGBN) * kGRowB;   // 32 KiB
constexpr int kGDmaPerWave = (kGBM + kGBN) / kGRPI / 4;   // gathers per wave and stage (8)

// LDS-DMA of 16 bytes per lane (lane l to LDS address lds + 16 l) issued as
// inline assembly: the compiler then does not treat the pending LDS writes as
// aliasing the operand reads and inserts no wait of its own (with the builtin
// it drains every gather at the top of the K loop); the waits are explicit
// (gemm_wait_vm before the barrier of each step).  M0 is restored
// afterwards, since the compiler does not accept it as a clobber.  No
// register results: nothing is left for a later instruction to overwrite.
__device__ __forceinline__ void gemm_dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void gemm_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// barrier that leaves later gathers in flight (a full fence would drain them)
__device__ __forceinline__ void gemm_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int gemm_pos(int r, int c) { return c ^ ((r >> kGSwzShift) & (kGCPR - 1)); }

// acc += a b on the 32x32x16 bf16 MFMA with acc pinned to accumulation
// registers: the 256 accumulators of a wave fill them exactly.  The compiler
// sees only an asm statement, so where compiled code touches acc next to
// these instructions (zeroing before the first, reading after the last) the
// kernel pads with gemm_acc_pad.
__device__ __forceinline__ void gemm_mfma(f32x16& acc, const bf16x8 a, const bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void gemm_acc_pad() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

__global__ __launch_bounds__(256) void gemm_nt_bf16(const bf16_t* __restrict__ A, int64_t lda, int64_t sa,
                                                    const bf16_t* __restrict__ B, int64_t ldb, int64_t sb,
                                                    bf16_t* __restrict__ C, int64_t ldc, int64_t sc, int M, int N,
                                                    int K, int tiles_m, int tiles_n, int xr) {
  __shared__ __attribute__((aligned(16))) unsigned char S0[kGStageB];
  __shared__ __attribute__((aligned(16))) unsigned char S1[kGStageB];
  __shared__ __attribute__((aligned(16))) unsigned char S2[kGStageB];
  __shared__ __attribute__((aligned(16))) unsigned char S3[kGStageB];
  const int T = tiles_m * tiles_n;
  const int L = blockIdx.x;
  // XCD x (dispatch index mod 8) takes block (x / xc, x % xc) of an xr x xc
  // grid of tile blocks (xr xc = 8), row-major inside its block; xr = 0:
  // no such split (dispatch order)
  int tm_, tn_;
  if (xr > 0) {
    const int xc = 8 / xr, bm = tiles_m / xr, bn = tiles_n / xc;
    const int x = L & 7, loc = L >> 3;
    tm_ = (x / xc) * bm + loc / bn;
    tn_ = (x % xc) * bn + loc % bn;
  } else {
    // contiguous ranges of tiles per XCD, row-block major
    const int t = (T & 7) == 0 ? (L & 7) * (T >> 3) + (L >> 3) : L;
    tm_ = t / tiles_n;
    tn_ = t % tiles_n;
  }
  const int m0 = tm_ * kGBM, n0 = tn_ * kGBN;
  const int64_t bz = blockIdx.y;
  A += bz * sa;
  B += bz * sb;
  C += bz * sc;
  const int l = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = K / kGBK;

  // gather stage kt: instruction `ins` fills tile rows kGRPI*ins .. +kGRPI-1,
  // lane l row kGRPI*ins + l/kGCPR at position l%kGCPR, i.e. the row's chunk
  // (l%kGCPR) ^ f(row)
  const int lrow = l / kGCPR, lpos = l % kGCPR;
  auto issue = [&](int kt, unsigned char* buf) {
    const int k0 = kt * kGBK;
#pragma unroll
    for (int i = 0; i < kGBM / kGRPI / 4; ++i) {
      const int ins = wave + 4 * i;
      const int r = ins * kGRPI + lrow;
      const int gr = m0 + r < M ? m0 + r : M - 1;
      const bf16_t* p = A + (int64_t)gr * lda + k0 + 8 * gemm_pos(r, lpos);
      gemm_dma16(p, (uint32_t)(uintptr_t)buf + ins * 1024);
    }
#pragma unroll
    for (int i = 0; i < kGBN / kGRPI / 4; ++i) {
      const int ins = wave + 4 * i;
      const int r = ins * kGRPI + lrow;
      const int gr = n0 + r < N ? n0 + r : N - 1;
      const bf16_t* p = B + (int64_t)gr * ldb + k0 + 8 * gemm_pos(r, lpos);
      gemm_dma16(p, (uint32_t)(uintptr_t)buf + kGBM * kGRowB + ins * 1024);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = (f32x16){};
  gemm_acc_pad();

  // 32 values of K from one stage, in 2 steps of 16: lane l reads row l%32
  // of each block at chunk 2*ks + l/32 (K values 16 ks + 8 (l/32) .. +7);
  // the wave owns rows 128 wm .. +127 and columns 128 wn .. +127 as 4 x 4
  // blocks, so each operand read feeds four MFMAs.
  auto read_stage = [&](const unsigned char* buf, bf16x8 (&av)[2][4], bf16x8 (&bv)[2][4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 2 * ks + (l >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wm * 128 + 32 * i + (l & 31);
        av[ks][i] = *reinterpret_cast<const bf16x8*>(buf + ra * kGRowB + 16 * gemm_pos(ra, ch));
        const int rb = wn * 128 + 32 * i + (l & 31);
        bv[ks][i] = *reinterpret_cast<const bf16x8*>(buf + kGBM * kGRowB + rb * kGRowB + 16 * gemm_pos(rb, ch));
      }
    }
  };
  auto mma = [&](const bf16x8 (&av)[2][4], const bf16x8 (&bv)[2][4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) gemm_mfma(acc[mi][ni], av[ks][mi], bv[ks][ni]);
  };
  // One K step.  The operands of stage kt are already in registers (pa, pb);
  // past the barrier stages kt and kt + 1 have landed (each wave waited for
  // its own gathers up to kt + 1; kt + 2 may still be in flight), so the wave
  // reads stage kt + 1's operands into (qa, qb) while stage kt's MFMAs run.
  // Stage kt + 3 goes to `ahead`, the buffer of stage kt - 1, whose operands
  // every wave read during step kt - 2.
  auto step = [&](int kt, const unsigned char* nxt, unsigned char* ahead, const bf16x8 (&pa)[2][4],
                  const bf16x8 (&pb)[2][4], bf16x8 (&qa)[2][4], bf16x8 (&qb)[2][4]) {
    if (kt + 2 < nk) gemm_wait_vm<kGDmaPerWave>();
    else gemm_wait_vm<0>();
    gemm_barrier();
    if (kt + 3 < nk) issue(kt + 3, ahead);
    if (kt + 1 < nk) read_stage(nxt, qa, qb);
    mma(pa, pb);
  };

  bf16x8 xa[2][4], xb[2][4], ya[2][4], yb[2][4];
  issue(0, S0);
  if (nk > 1) issue(1, S1);
  if (nk > 2) issue(2, S2);
  if (nk > 2) gemm_wait_vm<2 * kGDmaPerWave>();
  else if (nk > 1) gemm_wait_vm<kGDmaPerWave>();
  else gemm_wait_vm<0>();
  gemm_barrier();
  read_stage(S0, xa, xb);
  // whole rounds of the four stages, then at most three more steps (a loop
  // with early exits costs moves of the accumulators at every exit)
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {
    step(kt, S1, S3, xa, xb, ya, yb);
    step(kt + 1, S2, S0, ya, yb, xa, xb);
    step(kt + 2, S3, S1, xa, xb, ya, yb);
    step(kt + 3, S0, S2, ya, yb, xa, xb);
  }
  if (kt < nk) step(kt, S1, S3, xa, xb, ya, yb);
  if (kt + 1 < nk) step(kt + 1, S2, S0, ya, yb, xa, xb);
  if (kt + 2 < nk) step(kt + 2, S3, S1, xa, xb, ya, yb);
  gemm_acc_pad();

  // D layout of the 32 x 32 MFMA: register r of lane l is row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int col = n0 + wn * 128 + 32 * ni + (l & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + 32 * mi + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (row < M && col < N) C[(int64_t)row * ldc + col] = f2bf(acc[mi][ni][r]);
      }
    }
}

static hipError_t launch_gemm_nt(const bf16_t* A, int64_t lda, int64_t sa, const bf16_t* B, int64_t ldb,
                                 int64_t sb, bf16_t* C, int64_t ldc, int64_t sc, int64_t M, int64_t N, int64_t K,
                                 int64_t batch, hipStream_t st) {
  const int tm = (int)((M + kGBM - 1) / kGBM), tn = (int)((N + kGBN - 1) / kGBN);
  // the split of the tile grid over the 8 XCDs (each with its own L2) that
  // reads the least: A is read once per column group, B once per row group
  int xr = 0;
  double best = 0.0;
  for (int r = 1; r <= 8; r *= 2) {
    const int c = 8 / r;
    if (tm % r || tn % c) continue;
    const double bytes = (double)M * K * c + (double)N * K * r;
    if (xr == 0 || bytes < best) { xr = r; best = bytes; }
  }
  hipLaunchKernelGGL(gemm_nt_bf16, dim3((unsigned)(tm * tn), (unsigned)batch), dim3(256), 0, st, A, lda, sa, B, ldb,
                     sb, C, ldc, sc, (int)M, (int)N, (int)K, tm, tn, xr);
  return hipGetLastError();
}

hipError_t launch_grouped_out_proj(const void* o, const void* WG, const void* WO, int64_t n, int64_t n_h, int64_t c,
                                   int64_t g, int64_t d_g, int64_t d, void* mid, void* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t K1 = (n_h / g) * c, K2 = g * d_g;
  hipError_t e = launch_gemm_nt((const bf16_t*)o, n_h * c, K1, (const bf16_t*)WG, K1, d_g * K1, (bf16_t*)mid, K2,
                                d_g, n, d_g, K1, g, st);
  if (e != hipSuccess) return e;
  return launch_gemm_nt((const bf16_t*)mid, K2, 0, (const bf16_t*)WO, K2, 0, (bf16_t*)out, d, 0, n, d, K2, 1, st);
}

}  // namespace csa
