// bf16 GEMM with fp32 accumulate on gfx950 matrix cores:
//   C[M, N] = A[M, K] * B[N, K]^T  (+ bias, GELU-tanh or SwiGLU, bf16 store | fp32 store |
//   fp32 accumulate)
//
// This is the colwise projection (output features = weight dim 0) and the
// rowwise partial projection (input features = weight dim 1) of the Diffusers
// tensor-parallelism page, §"Colwise e rowwise": in both cases the rank's
// weight slice is an nn.Linear [out, in] matrix, so both operands are
// K-contiguous and the kernel is one "NT" GEMM with different epilogues.
//
// Design (gfx950, 64-wide waves, 160 KB LDS per CU).  Two kernels: a
// 4-wave register-staged one for small and ragged shapes, and the 8-wave
// ping-pong kernel further down for large ones (at least 128 tiles of
// 256x256, K % 64 == 0).  The 4-wave kernel:
//   * 256 threads = 4 waves in a WM x WN grid; each wave owns a
//     (BM/WM) x (BN/WN) block of C held in accumulation registers as
//     32x32 tiles of v_mfma_f32_32x32x16_bf16.
//   * K advances 64 elements (128 bytes per row) per tile.  A and B tiles are
//     fetched with 16-byte global loads into registers one tile ahead, then
//     written to a double-buffered LDS tile; one barrier per K tile.
// Both kernels:
//   * LDS rows are 128 bytes; the 16-byte chunk of k-group kc of row r lives
//     at chunk kc ^ (r & 7) ^ ((r >> 3) & 1), so the rows read by one
//     ds_read_b128 phase fall in distinct banks.
//   * Workgroup ids are renumbered so each of the 8 XCDs (own L2) walks a
//     contiguous stretch of a grouped tile order (8 tile rows per group), and
//     the A/B panels it streams are shared by its neighbours in L2.
//   * Rows past M / N are clamped on load and masked on store.  In the 4-wave
//     kernel a K that is not a multiple of 64 zero-fills the chunks past K
//     (K must be a multiple of 8).
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 64;        // K elements per tile
constexpr int kRowChunks = 8;  // 16-byte chunks per LDS tile row
constexpr int kGroupM = 8;     // tile rows per group in the tile order

__device__ __forceinline__ int swizzle(int row, int kc) {
  return kc ^ (row & 7) ^ ((row >> 3) & 1);
}

// GELU, tanh form: 0.5 u (1 + tanh(z)) = u * sigmoid(2 z) = u / (1 + exp(-2 z)),
// z = sqrt(2/pi) (u + 0.044715 u^3).  With the constants folded,
// exp(-2 z) = exp2(u (k1 + k2 u^2)), k1 = -2 sqrt(2/pi) log2(e),
// k2 = 0.044715 k1: three FMA-class operations, one exp2 and one hardware
// reciprocal (1 ulp), far below the bf16 rounding of the result.
__device__ __forceinline__ float gelu_tanh(float u) {
  const float k1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  const float k2 = 0.044715f * k1;
  const float t = u * fmaf(k2, u * u, k1);
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// SiLU: u * sigmoid(u) = u / (1 + exp(-u)) = u / (1 + exp2(-log2(e) u)).
__device__ __forceinline__ float silu(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * u));
}

// One 32-column block of a wave's accumulators: rows r(i, e) = 32 i + 8 (e / 4)
// + (e % 4) past the lane's first row (lane: column lane & 31, first row
// 4 (lane >> 5)), i.e. row steps +1, +1, +1, +5 repeating.  `p` points at
// the lane's first row and advances by the row stride, so no element needs
// a 64-bit multiply; `rows_left` (ROWCHECK only) bounds the rows stored.
enum class Mode : int { PLAIN, GELU, GLU };

template <OutKind KIND, Mode MODE, bool ROWCHECK, int TM, int TN>
__device__ __forceinline__ void store_block(const f32x16 (&acc)[TM][TN], int j, char* p,
                                            int64_t stride, int rows_left, float bias,
                                            float bias_up) {
  constexpr int ES = KIND == OutKind::BF16 ? 2 : 4;
  const int64_t stride5 = 5 * stride;
  if constexpr (KIND == OutKind::F32_ACC) {
    // read the 16 rows of tile i first, then add and store: one wait per tile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float old[16];
      char* q = p;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + (e & 3);
        old[e] = (!ROWCHECK || r < rows_left) ? *reinterpret_cast<const float*>(q) : 0.0f;
        q += (e & 3) == 3 ? stride5 : stride;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + (e & 3);
        if (!ROWCHECK || r < rows_left) *reinterpret_cast<float*>(p) = old[e] + acc[i][j][e];
        p += (e & 3) == 3 ? stride5 : stride;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 32 * i + 8 * (e >> 2) + (e & 3);
      // keeps each row test at its store: hoisted, the 64 tests' masks would
      // take registers the accumulators need
      if constexpr (ROWCHECK) asm volatile("" : "+v"(rows_left));
      if (!ROWCHECK || r < rows_left) {
        float v = acc[i][j][e] + bias;
        if constexpr (MODE == Mode::GLU) v = silu(v) * (acc[i][j | 1][e] + bias_up);
        if constexpr (MODE == Mode::GELU) v = gelu_tanh(v);
        if constexpr (ES == 2)
          *reinterpret_cast<bf16*>(p) = static_cast<bf16>(v);
        else
          *reinterpret_cast<float*>(p) = v;
      }
      p += (e & 3) == 3 ? stride5 : stride;
    }
  }
}

// Writes one wave's TM x TN accumulator tiles: tile (i, j) holds C rows
// row0 + 32 i + [0, 32) and columns col0 + 32 j + [0, 32) in the 32x32 MFMA
// layout (lane: column lane & 31, rows 8 (e / 4) + 4 (lane >> 5) + (e % 4)).
// Each store instruction writes 32 adjacent columns of two rows.  With
// FULL_ROWS_FAST, a wave whose rows all lie below M (row0 is wave-uniform)
// takes a copy without the row test (the 4-wave kernels, whose accumulators
// fill the register file, keep the one tested copy).  col0 is a multiple of
// 64, so under SWIGLU tile j (even) is a gate block and tile j + 1 its up
// block: the pair is combined in registers and stored as 32 output columns.
template <OutKind KIND, int TM, int TN, bool FULL_ROWS_FAST>
__device__ __forceinline__ void store_tiles(const f32x16 (&acc)[TM][TN], const GemmProblem& p,
                                            const GemmEpilogue& ep, int row0, int col0,
                                            int lane) {
  static_assert(TN % 2 == 0, "SwiGLU pairs tile j with tile j + 1");
  constexpr int ES = KIND == OutKind::BF16 ? 2 : 4;
  const int col_l = lane & 31;
  const int row_l = 4 * (lane >> 5);
  const int rows_left = p.M - row0 - row_l;           // rows of this lane's half below M
  const bool rows_full = row0 + 32 * TM <= p.M;       // wave-uniform
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = col0 + 32 * j + col_l;
    if (col >= p.N) continue;
    const bool active = KIND != OutKind::F32_ACC && col >= ep.act_from;
    const bool glu = active && ep.act == Act::SWIGLU;
    const bool gelu = active && ep.act == Act::GELU_TANH;
    if (glu && (j & 1)) continue;  // an up block, consumed with its gate block
    int ocol = glu ? ep.act_from + (((col - ep.act_from) >> 6) << 5) + col_l : col;
    float bias = 0.0f, bias_up = 0.0f;
    if constexpr (KIND != OutKind::F32_ACC) {
      if (ep.bias) {
        bias = ep.bias[col];
        if (glu) bias_up = ep.bias[col + 32];
      }
    }
    const bool second = ocol >= ep.split;
    if (second) ocol -= ep.split;
    const int64_t ld = second ? ep.ld1 : ep.ld0;
    char* base = static_cast<char*>(second ? ep.out1 : ep.out0) +
                 ((int64_t)(row0 + row_l) * ld + ocol) * ES;
    const int64_t stride = ld * ES;
#define TPK_STORE(MODE_)                                                                    \
  do {                                                                                       \
    if (FULL_ROWS_FAST && rows_full)                                                         \
      store_block<KIND, MODE_, false>(acc, j, base, stride, rows_left, bias, bias_up);       \
    else                                                                                     \
      store_block<KIND, MODE_, true>(acc, j, base, stride, rows_left, bias, bias_up);        \
  } while (0)
    if constexpr (KIND == OutKind::F32_ACC) {
      TPK_STORE(Mode::PLAIN);
    } else {
      if (glu) TPK_STORE(Mode::GLU);
      else if (gelu) TPK_STORE(Mode::GELU);
      else TPK_STORE(Mode::PLAIN);
    }
#undef TPK_STORE
  }
}

template <int BM, int BN, int WM, int WN, OutKind KIND, bool KTAIL>
__global__ void __launch_bounds__(kThreads)
gemm_bf16_nt(GemmProblem p, GemmEpilogue ep, int tiles_m, int tiles_n) {
  static_assert(WM * WN * 64 == kThreads, "4 waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  constexpr int A_LOADS = BM * kRowChunks / kThreads;
  constexpr int B_LOADS = BN * kRowChunks / kThreads;
  constexpr int BUF = (BM + BN) * kRowChunks;  // 16-byte chunks per stage
  static_assert(TM >= 1 && TN >= 1 && A_LOADS >= 1 && B_LOADS >= 1, "tile shape");

  __shared__ u32x4 smem[2 * BUF];

  // ---- tile coordinates: XCD-contiguous renumbering, then grouped order
  const int nb = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, per = nb >> 3, rem = nb & 7;
  const int id = xcd * per + min(xcd, rem) + (bid >> 3);
  const int group = id / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = id - group * kGroupM * tiles_n;
  const int m0 = (first_m + in_group % gm) * BM;
  const int n0 = (in_group / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bf16* __restrict__ A = static_cast<const bf16*>(p.A);
  const bf16* __restrict__ B = static_cast<const bf16*>(p.B);

  // ---- global -> register staging: thread loads chunk kc of rows r0 + 32 i
  const int ld_row = tid >> 3, ld_kc = tid & 7;
  int64_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i)
    a_off[i] = (int64_t)min(m0 + ld_row + 32 * i, p.M - 1) * p.lda + ld_kc * 8;
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i)
    b_off[i] = (int64_t)min(n0 + ld_row + 32 * i, p.N - 1) * p.ldb + ld_kc * 8;
  // the swizzle of rows ld_row + 32 i does not depend on i
  const int st_base = ld_row * kRowChunks + swizzle(ld_row, ld_kc);

  u32x4 ra[A_LOADS], rb[B_LOADS];
  auto gload = [&](int kt) {
    const int k = kt * kBK;
    const bool in = !KTAIL || (k + ld_kc * 8 < p.K);
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      ra[i] = in ? *reinterpret_cast<const u32x4*>(A + a_off[i] + k) : zero;
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      rb[i] = in ? *reinterpret_cast<const u32x4*>(B + b_off[i] + k) : zero;
  };
  auto sstore = [&](int buf) {
    u32x4* sa = smem + buf * BUF;
    u32x4* sb = sa + BM * kRowChunks;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) sa[st_base + 32 * kRowChunks * i] = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) sb[st_base + 32 * kRowChunks * i] = rb[i];
  };

  // ---- MFMA operand reads: lane holds row (lane & 31), k-group 2 s + (lane >> 5)
  const int wm = wave / WN, wn = wave % WN;
  const int a_row = wm * WTM + (lane & 31);
  const int b_row = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto compute = [&](int buf) {
    const u32x4* sa = smem + buf * BUF;
    const u32x4* sb = sa + BM * kRowChunks;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int kc = 2 * s + khalf;
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = __builtin_bit_cast(bf16x8, sa[(a_row + 32 * i) * kRowChunks + swizzle(a_row, kc)]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = __builtin_bit_cast(bf16x8, sb[(b_row + 32 * j) * kRowChunks + swizzle(b_row, kc)]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = (p.K + kBK - 1) / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    compute(kt & 1);
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }

  store_tiles<KIND, TM, TN, false>(acc, p, ep, m0 + wm * WTM, n0 + wn * WTN, lane);
}

// 256x256 tile (TM = 4; TM = 3 gives 192x256 for problems that one round
// of 256-row tiles would leave CUs idle in), 8 waves (2 per SIMD) in a
// ping-pong schedule; each wave owns a (32 TM)x64 block of C.  A and B tiles
// go global -> LDS directly (global_load_lds_dwordx4: each wave instruction
// fills 1 KB = 8 tile rows), so no registers stage them and no ds_write is
// issued; K % 64 == 0 (no zero-fill on this path).  Waves 0-3 (group 0) own
// C rows [0, 32 TM) and waves 4-7 (group 1) rows [32 TM, 64 TM).  The groups
// run one phase apart, separated by workgroup barriers: while one group reads
// a whole K tile of operand fragments from LDS into registers
// ((TM + 2) x 4 x 16 bytes per lane), the other issues the 8 TM MFMAs of the
// tile it read in the previous phase.  Phase 2k:
// group 0 reads tile k, group 1 multiplies tile k-1; phase 2k+1: group 0
// multiplies tile k, group 1 reads tile k.
//
// A wave that waits to issue a global load issues no MFMA meanwhile, so
// loads are issued only in read phases: group 0, after reading tile k in
// phase 2k, fetches the whole B tile k+1; group 1, after reading tile k in
// phase 2k+1, fetches the whole A tile k+2.  A has three LDS stages and B
// two (96 + 64 KB at TM = 4): the B tile k+1 goes into the stage of tile k-1 (last
// read in phase 2k-1) and is waited for by group 0 at the end of phase 2k+1;
// the A tile k+2 goes into the stage of tile k-1 too and is waited for by
// group 1 at the end of phase 2k+3.  Tile 0 and A tile 1 are fetched before
// the loop.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// all but the newest N loads of this wave have landed
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N == 8 || N == 6, "instantiated counts");
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <OutKind KIND, int TM>
__global__ void __launch_bounds__(512)
gemm_bf16_nt_pingpong(GemmProblem p, GemmEpilogue ep, int tiles_m, int tiles_n) {
  static_assert(TM == 4 || TM == 3, "256- or 192-row tiles");
  constexpr int BM = 64 * TM, BN = 256;
  constexpr int TN = 2;                         // 32 TM x 64 per wave
  constexpr int KS = kBK / 16;                  // 4 MFMA k-steps per tile
  constexpr int A_STAGE = BM * kRowChunks;      // 16-byte chunks per A stage
  constexpr int B_STAGE = BN * kRowChunks;
  constexpr int A_LOADS = 2 * TM;               // 8-row loads per wave per A tile

  __shared__ u32x4 smem[3 * A_STAGE + 2 * B_STAGE];   // 160 KB (136 KB at BM 192)

  const int nb = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, per = nb >> 3, rem = nb & 7;
  const int id = xcd * per + min(xcd, rem) + (bid >> 3);
  const int group = id / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = id - group * kGroupM * tiles_n;
  const int m0 = (first_m + in_group % gm) * BM;
  const int n0 = (in_group / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = wave >> 2, q = wave & 3;   // wave group (0: waves 0-3), place in it
  const bf16* __restrict__ A = static_cast<const bf16*>(p.A);
  const bf16* __restrict__ B = static_cast<const bf16*>(p.B);

  auto stage_a = [&](int kt) { return smem + (kt % 3) * A_STAGE; };
  auto stage_b = [&](int kt) { return smem + 3 * A_STAGE + (kt & 1) * B_STAGE; };

  // global -> LDS: wave q of the fetching group covers the operand rows
  // 8 n q + 8 i + (lane >> 3), i = 0..n-1 (n = 8 for B, 2 TM for A), one
  // instruction each; 8 n q is a multiple of 16, so the swizzle of a row
  // depends only on i & 1.
  const int kc_even = swizzle(lane >> 3, lane & 7) * 8, kc_odd = swizzle(8 + (lane >> 3), lane & 7) * 8;
  auto fetch = [&](const bf16* __restrict__ src, int ld, int first_row, int rows, int kt, u32x4* dst,
                   int n) {
    const int k = kt * kBK;
    const int wrow = 8 * n * q;
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int kc = (i & 1) ? kc_odd : kc_even;
      const int off = min(first_row + wrow + 8 * i + (lane >> 3), rows - 1) * ld + kc + k;
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(src + off),
          (void __attribute__((address_space(3)))*)(dst + (wrow + 8 * i) * kRowChunks), 16, 0, 0);
    }
  };
  auto fetch_a = [&](int kt) { fetch(A, (int)p.lda, m0, p.M, kt, stage_a(kt), A_LOADS); };
  auto fetch_b = [&](int kt) { fetch(B, (int)p.ldb, n0, p.N, kt, stage_b(kt), 8); };

  const int a_row = 32 * TM * g + (lane & 31);
  const int b_row = 64 * q + (lane & 31);
  const int khalf = lane >> 5;
  bf16x8 fa[KS][TM], fb[KS][TN];
  auto read_tile = [&](int kt) {
    const u32x4* sa = stage_a(kt);
    const u32x4* sb = stage_b(kt);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int kc = 2 * s + khalf;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[s][i] = __builtin_bit_cast(bf16x8, sa[(a_row + 32 * i) * kRowChunks + swizzle(a_row, kc)]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[s][j] = __builtin_bit_cast(bf16x8, sb[(b_row + 32 * j) * kRowChunks + swizzle(b_row, kc)]);
    }
  };
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto multiply = [&]() {
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
  };

  const int nk = p.K / kBK;
  if (g == 0) {
    fetch_b(0);
  } else {
    fetch_a(0);
    if (nk > 1) fetch_a(1);
  }
  wait_vmem();
  wg_barrier();
  if (g == 0) {
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      if (more) fetch_b(kt + 1);
      wg_barrier();                       // end of phase 2 kt
      multiply();
      if (more) wait_vmem();              // B tile kt + 1
      wg_barrier();                       // end of phase 2 kt + 1
    }
    wg_barrier();
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      if (kt > 0) multiply();             // tile kt - 1
      wg_barrier();                       // end of phase 2 kt
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 2 < nk) {
        fetch_a(kt + 2);
        wait_vmem_keep<A_LOADS>();        // A tile kt + 1
      } else {
        wait_vmem();
      }
      wg_barrier();                       // end of phase 2 kt + 1
    }
    multiply();
    wg_barrier();
  }

  store_tiles<KIND, TM, TN, true>(acc, p, ep, m0 + 32 * TM * g, n0 + 64 * q, lane);
}

// The 8-wave kernel with TM * 64-row tiles (TM 4: 256 x 256, TM 3: 192 x 256).
template <int TM>
hipError_t launch_8w(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind,
                     hipStream_t stream) {
  const int tm = (p.M + 64 * TM - 1) / (64 * TM), tn = (p.N + 255) / 256;
  const dim3 grid(tm * tn), block(512);
  switch (kind) {
    case OutKind::BF16:
      hipLaunchKernelGGL((gemm_bf16_nt_pingpong<OutKind::BF16, TM>), grid, block, 0, stream, p, ep, tm, tn);
      break;
    case OutKind::F32_STORE:
      hipLaunchKernelGGL((gemm_bf16_nt_pingpong<OutKind::F32_STORE, TM>), grid, block, 0, stream, p, ep, tm, tn);
      break;
    case OutKind::F32_ACC:
      hipLaunchKernelGGL((gemm_bf16_nt_pingpong<OutKind::F32_ACC, TM>), grid, block, 0, stream, p, ep, tm, tn);
      break;
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tile(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind,
                       hipStream_t stream) {
  const int tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
  const dim3 grid(tm * tn), block(kThreads);
  const bool ktail = (p.K % kBK) != 0;
#define TPK_LAUNCH(K_, T_) \
  hipLaunchKernelGGL((gemm_bf16_nt<BM, BN, WM, WN, K_, T_>), grid, block, 0, stream, p, ep, tm, tn)
  switch (kind) {
    case OutKind::BF16:
      if (ktail) TPK_LAUNCH(OutKind::BF16, true); else TPK_LAUNCH(OutKind::BF16, false);
      break;
    case OutKind::F32_STORE:
      if (ktail) TPK_LAUNCH(OutKind::F32_STORE, true); else TPK_LAUNCH(OutKind::F32_STORE, false);
      break;
    case OutKind::F32_ACC:
      if (ktail) TPK_LAUNCH(OutKind::F32_ACC, true); else TPK_LAUNCH(OutKind::F32_ACC, false);
      break;
  }
#undef TPK_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind,
                            hipStream_t stream) {
  // 256x256 tiles (or 192x256, below) when they fill at least half the 256
  // CUs (the 8-wave kernel beats four times as many 128x128 tiles even
  // then); 128x128 otherwise.
  const long big = (long)((p.M + 255) / 256) * ((p.N + 255) / 256);
  // the 8-wave kernel indexes operands with 32-bit element offsets
  const bool fits32 = (int64_t)p.M * p.lda < ((int64_t)1 << 31) &&
                      (int64_t)p.N * p.ldb < ((int64_t)1 << 31);
  if (big >= 128 && p.K % kBK == 0 && fits32) {
    // One partial round of 256-row tiles leaves CUs idle (e.g. 162 tiles at
    // M = 4608, N = 2304); if 192-row tiles still fit in one round, every
    // busy CU has 3/4 of the work.
    const long mid = (long)((p.M + 191) / 192) * ((p.N + 255) / 256);
    if (big < 256 && mid <= 256) return launch_8w<3>(p, ep, kind, stream);
    return launch_8w<4>(p, ep, kind, stream);
  }
  if (big >= 256) return launch_tile<256, 256, 2, 2>(p, ep, kind, stream);
  return launch_tile<128, 128, 2, 2>(p, ep, kind, stream);
}

}  // namespace tpk
