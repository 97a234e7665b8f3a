// GEMMs with fp32 accumulate on gfx950 matrix cores:
//   C[M, N] = A[M, K] * B[N, K]^T  (+ bias, GELU-tanh or SwiGLU, bf16 store | fp32 store |
//   fp32 accumulate), A and B both bf16 (v_mfma_f32_32x32x16_bf16 and
//   v_mfma_f32_16x16x32_bf16) or both fp32 (v_mfma_f32_32x32x2_f32).
//
// This is the colwise projection (output features = weight dim 0) and the
// rowwise partial projection (input features = weight dim 1) of the Diffusers
// tensor-parallelism page, §"Colwise e rowwise": in both cases the rank's
// weight slice is an nn.Linear [out, in] matrix, so both operands are
// K-contiguous and the kernel is one "NT" GEMM with different epilogues.
//
// Design (gfx950, 64-wide waves, 160 KB LDS per CU).  A 4-wave
// register-staged kernel for small and ragged bf16 shapes and for every fp32
// one; for large bf16 ones (at least 128 tiles, K % 64 == 0) direct-to-LDS
// kernels further down: 8-wave ping-pong kernels on 288x192 and 192x256
// tiles, and on 256x256 tiles a one-wave-per-SIMD kernel (persistent when
// there are more tiles than compute units), with the 8-wave kernel as its
// fallback (launch_gemm_bf16 chooses).  The register-staged kernel:
//   * 256 threads = 4 waves in a WM x WN grid; each wave owns a
//     (BM/WM) x (BN/WN) block of C held in accumulation registers as
//     32x32 MFMA tiles.
//   * K advances 128 bytes per row per tile (64 bf16 or 32 fp32 elements).
//     A and B tiles are fetched with 16-byte global loads into registers one
//     tile ahead, then written to a double-buffered LDS tile; one barrier per
//     K tile.
// All kernels:
//   * LDS rows are 128 bytes; the 16-byte chunk of k-group kc of row r lives
//     at chunk kc ^ (r & 7) ^ ((r >> 3) & 1), so the rows read by one
//     ds_read_b128 phase fall in distinct banks.
//   * Workgroup ids are renumbered so each of the 8 XCDs (own L2) walks a
//     contiguous stretch of a grouped tile order (8 tile rows per group), and
//     the A/B panels it streams are shared by its neighbours in L2.
//   * Rows past M / N are masked on store; on load the register-staged
//     kernel clamps them to the last row and the direct-to-LDS kernels read
//     them as zero (past their buffer descriptors' range).  In the
//     register-staged kernel a K that is not a whole number of tiles
//     zero-fills the chunks past K (K must be a multiple of the 8 bf16 or 4
//     fp32 elements of a chunk).
#include "tp_kernels.h"

#include <type_traits>

namespace tpk {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 64;        // bf16 K elements per tile (128 bytes per row)
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

// T = bf16: each 16-byte chunk holds 8 k; an MFMA step (32x32x16) takes
// chunk 2 s + (lane >> 5) of the lane's row, k-step s = 0..3 of the tile.
// T = float: a chunk holds 4 k; an MFMA step (32x32x2) takes one k per lane
// half, and the lane half h reads chunks 2 c + h (c = 0..3), so step 4 c + j
// reduces k = 8 c + j (half 0) and 8 c + 4 + j (half 1): the same k for A
// and B, each k of the tile once.
template <class T, int BM, int BN, int WM, int WN, OutKind KIND, bool KTAIL>
__global__ void __launch_bounds__(kThreads)
gemm_nt_staged(GemmProblem p, GemmEpilogue ep, int tiles_m, int tiles_n) {
  static_assert(std::is_same<T, bf16>::value || std::is_same<T, float>::value, "bf16 or fp32");
  constexpr int CE = 16 / sizeof(T);           // elements per 16-byte chunk
  constexpr int BKT = kRowChunks * CE;          // K elements per tile
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
  const T* __restrict__ A = static_cast<const T*>(p.A);
  const T* __restrict__ B = static_cast<const T*>(p.B);

  // ---- global -> register staging: thread loads chunk kc of rows r0 + 32 i
  const int ld_row = tid >> 3, ld_kc = tid & 7;
  int64_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i)
    a_off[i] = (int64_t)min(m0 + ld_row + 32 * i, p.M - 1) * p.lda + ld_kc * CE;
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i)
    b_off[i] = (int64_t)min(n0 + ld_row + 32 * i, p.N - 1) * p.ldb + ld_kc * CE;
  // the swizzle of rows ld_row + 32 i does not depend on i
  const int st_base = ld_row * kRowChunks + swizzle(ld_row, ld_kc);

  u32x4 ra[A_LOADS], rb[B_LOADS];
  auto gload = [&](int kt) {
    const int k = kt * BKT;
    const bool in = !KTAIL || (k + ld_kc * CE < p.K);
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
    for (int s = 0; s < kRowChunks / 2; ++s) {
      const int kc = 2 * s + khalf;
      u32x4 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = sa[(a_row + 32 * i) * kRowChunks + swizzle(a_row, kc)];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = sb[(b_row + 32 * j) * kRowChunks + swizzle(b_row, kc)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (std::is_same<T, bf16>::value) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
          } else {
            const f32x4 af = __builtin_bit_cast(f32x4, a[i]), bfv = __builtin_bit_cast(f32x4, b[j]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[q], bfv[q], acc[i][j], 0, 0, 0);
          }
        }
    }
  };

  const int nk = (p.K + BKT - 1) / BKT;
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
// ping-pong schedule; each wave owns a (32 TM)x64 block of C.  Waves 0-3
// (group 0) own C rows [0, 32 TM) and waves 4-7 (group 1) rows
// [32 TM, 64 TM).  The groups run one phase apart, separated by workgroup
// barriers: while one group reads a whole K tile of operand fragments from
// LDS into registers ((TM + 2) x 4 x 16 bytes per lane), the other issues
// the 8 TM MFMAs of the tile it read in the previous phase.  Phase 2k:
// group 0 reads tile k, group 1 multiplies tile k-1; phase 2k+1: group 0
// multiplies tile k, group 1 reads tile k.
//
// A and B tiles go global -> LDS directly with buffer loads
// (buffer_load_dwordx4 ... lds: each wave instruction fills 1 KB = 8 tile
// rows), so no registers stage them and no ds_write is issued; K % 64 == 0.
// A load's address is the operand's buffer descriptor, a per-lane 32-bit
// offset fixed for the whole kernel (row within the tile, swizzled chunk) and
// a wave-uniform K offset in a scalar register, so the loads of a tile cost
// one VGPR each and no address arithmetic.  Rows past M (or N) lie past the
// descriptor's byte range and read as zero (their results are not stored).
//
// Every wave fetches an equal share of every tile: the B tile k+1 (4 loads
// per wave) in phase 2k and the A tile k+2 (BM/64 loads per wave) in phase
// 2k+1.  The reading group issues its share after its fragment reads; the
// multiplying group spreads its share among its first MFMAs (one load per
// two), so a load that waits to issue delays only a few MFMAs.  A has three
// LDS stages and B two (96 + 64 KB at TM = 4): B tile k+1 goes into the stage
// of tile k-1 (last read in phase 2k-1) and A tile k+2 likewise; at the end
// of phase 2k+1 every wave waits for its B tile k+1 loads (the A tile k+2
// ones may stay in flight: they are needed two phases later), then the
// barrier publishes the tile to both groups.
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
  static_assert(N == 5 || N == 4 || N == 3, "instantiated counts");
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over [base, base + bytes): offsets at or past `bytes`
// read as zero.  Word 3 (0x00020000) selects 32-bit data with no swizzle.
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from byte offset voff + soff of the buffer into LDS at
// dst + 16 lane (dst wave-uniform).
__device__ __forceinline__ void lds_dma(rsrc_t r, const u32x4* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)voff,
                                           (int)soff, 0, 0);
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
  constexpr int AW = BM / 64;                   // 8-row A loads per wave per tile
  constexpr int BW = BN / 64;                   // 8-row B loads per wave per tile

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

  // Descriptors end right after the last row's K elements.
  const uint32_t lda2 = (uint32_t)p.lda * 2, ldb2 = (uint32_t)p.ldb * 2;
  const rsrc_t ra = buffer_rsrc(p.A, (uint32_t)(p.M - 1) * lda2 + (uint32_t)p.K * 2);
  const rsrc_t rb = buffer_rsrc(p.B, (uint32_t)(p.N - 1) * ldb2 + (uint32_t)p.K * 2);
  // Wave w fetches tile rows [w BM/8, (w+1) BM/8) of A and [32 w, 32 w + 32)
  // of B, 8 rows per load.  In the load of the 8 rows from R (R % 8 == 0)
  // lane l reads row R + (l >> 3) and fills physical chunk l & 7 of it, which
  // holds logical chunk (l & 7) ^ (l >> 3) ^ ((R >> 3) & 1) (the swizzle).
  const int lr = lane >> 3, lc = lane & 7;
  uint32_t voa[AW], vob[BW];
#pragma unroll
  for (int j = 0; j < AW; ++j) {
    const int R = wave * (BM / 8) + 8 * j;
    voa[j] = (uint32_t)(m0 + R + lr) * lda2 + (uint32_t)((lc ^ lr ^ ((R >> 3) & 1)) * 16);
  }
#pragma unroll
  for (int j = 0; j < BW; ++j) {
    const int R = wave * (BN / 8) + 8 * j;
    vob[j] = (uint32_t)(n0 + R + lr) * ldb2 + (uint32_t)((lc ^ lr ^ ((R >> 3) & 1)) * 16);
  }
  auto stage_a = [&](int kt) { return smem + (kt % 3) * A_STAGE; };
  auto stage_b = [&](int kt) { return smem + 3 * A_STAGE + (kt & 1) * B_STAGE; };
  auto load_a = [&](int kt, int j) {
    lds_dma(ra, stage_a(kt) + (wave * (BM / 8) + 8 * j) * kRowChunks, voa[j], (uint32_t)kt * (kBK * 2));
  };
  auto load_b = [&](int kt, int j) {
    lds_dma(rb, stage_b(kt) + (wave * (BN / 8) + 8 * j) * kRowChunks, vob[j], (uint32_t)kt * (kBK * 2));
  };
  auto a_loads = [&](int kt) {
#pragma unroll
    for (int j = 0; j < AW; ++j) load_a(kt, j);
  };
  auto b_loads = [&](int kt) {
#pragma unroll
    for (int j = 0; j < BW; ++j) load_b(kt, j);
  };

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
  // The tile's MFMAs, with load(l), l < nl, issued after MFMA 2 l.
  auto multiply = [&](auto&& load, int nl) {
    int idx = 0;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
          if ((idx & 1) == 0 && (idx >> 1) < nl) {
            __builtin_amdgcn_sched_barrier(0);
            load(idx >> 1);
            __builtin_amdgcn_sched_barrier(0);
          }
          ++idx;
        }
  };
  auto none = [](int) {};

  // The loop bodies carry no branch on the loads: the last two tiles, which
  // fetch less, are peeled by hand.
  const int nk = p.K / kBK;
  b_loads(0);
  a_loads(0);
  if (nk > 1) a_loads(1);
  wait_vmem();
  wg_barrier();
  if (g == 0) {
    int kt = 0;
    for (; kt + 2 < nk; ++kt) {
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      b_loads(kt + 1);
      wg_barrier();                       // end of phase 2 kt
      multiply([&](int j) { load_a(kt + 2, j); }, AW);
      wait_vmem_keep<AW>();               // B tile kt + 1 landed
      wg_barrier();                       // end of phase 2 kt + 1
    }
    if (kt + 1 < nk) {                    // kt = nk - 2
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      b_loads(kt + 1);
      wg_barrier();
      multiply(none, 0);
      wait_vmem();
      wg_barrier();
      ++kt;
    }
    read_tile(kt);                        // kt = nk - 1
    wg_barrier();
    multiply(none, 0);
    wg_barrier();
    wg_barrier();
  } else {
    if (nk > 1) b_loads(1);
    wg_barrier();                         // end of phase 0
    read_tile(0);
    __builtin_amdgcn_sched_barrier(0);
    if (nk > 2) {
      a_loads(2);
      wait_vmem_keep<AW>();
    } else {
      wait_vmem();
    }
    wg_barrier();                         // end of phase 1
    int kt = 1;
    for (; kt + 2 < nk; ++kt) {
      multiply([&](int j) { load_b(kt + 1, j); }, BW);   // tile kt - 1
      wg_barrier();                       // end of phase 2 kt
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      a_loads(kt + 2);
      wait_vmem_keep<AW>();
      wg_barrier();                       // end of phase 2 kt + 1
    }
    if (kt + 1 < nk) {                    // kt = nk - 2 >= 1
      multiply([&](int j) { load_b(kt + 1, j); }, BW);
      wg_barrier();
      read_tile(kt);
      wait_vmem();
      wg_barrier();
      ++kt;
    }
    if (kt < nk) {                        // kt = nk - 1 >= 1
      multiply(none, 0);
      wg_barrier();
      read_tile(kt);
      wg_barrier();
    }
    multiply(none, 0);                    // tile nk - 1
    wg_barrier();
  }

  store_tiles<KIND, TM, TN, true>(acc, p, ep, m0 + 32 * TM * g, n0 + 64 * q, lane);
}

// Epilogue of the 16x16 MFMA layout: accumulator (i, j) holds C rows
// row0 + 16 i + [0, 16) and columns col0 + 16 j + [0, 16); lane l holds
// column l & 15 of rows 4 (l >> 4) + e, e = 0..3.  A store instruction writes
// 16 adjacent columns of four rows.  act_from and split are multiples of 16,
// so a 16-column block lies wholly on one side of each (GELU or none; SwiGLU
// shapes stay on the 32x32 kernels).
template <OutKind KIND, bool GELU, bool ROWCHECK, int TM, int TN>
__device__ __forceinline__ void store_block16(const f32x4 (&acc)[TM][TN], int j, char* p,
                                              int64_t stride, int rows_left, float bias) {
  const int64_t stride13 = 13 * stride;
  if constexpr (KIND == OutKind::F32_ACC) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float old[4];
      char* q = p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        old[e] = (!ROWCHECK || 16 * i + e < rows_left) ? *reinterpret_cast<const float*>(q) : 0.0f;
        q += stride;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!ROWCHECK || 16 * i + e < rows_left) *reinterpret_cast<float*>(p) = old[e] + acc[i][j][e];
        p += e == 3 ? stride13 : stride;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (ROWCHECK) asm volatile("" : "+v"(rows_left));
      if (!ROWCHECK || 16 * i + e < rows_left) {
        float v = acc[i][j][e] + bias;
        if constexpr (GELU) v = gelu_tanh(v);
        if constexpr (KIND == OutKind::BF16)
          *reinterpret_cast<bf16*>(p) = static_cast<bf16>(v);
        else
          *reinterpret_cast<float*>(p) = v;
      }
      p += e == 3 ? stride13 : stride;
    }
  }
}

template <OutKind KIND, int TM, int TN>
__device__ __forceinline__ void store_tiles16(const f32x4 (&acc)[TM][TN], const GemmProblem& p,
                                              const GemmEpilogue& ep, int row0, int col0, int lane) {
  constexpr int ES = KIND == OutKind::BF16 ? 2 : 4;
  const int col_l = lane & 15;
  const int row_l = 4 * (lane >> 4);
  const int rows_left = p.M - row0 - row_l;
  const bool rows_full = row0 + 16 * TM <= p.M;       // wave-uniform
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = col0 + 16 * j + col_l;
    if (col >= p.N) continue;
    const bool gelu = KIND != OutKind::F32_ACC && col >= ep.act_from && ep.act == Act::GELU_TANH;
    const float bias = (KIND != OutKind::F32_ACC && ep.bias) ? ep.bias[col] : 0.0f;
    const bool second = col >= ep.split;
    const int ocol = second ? col - ep.split : col;
    const int64_t ld = second ? ep.ld1 : ep.ld0;
    char* base = static_cast<char*>(second ? ep.out1 : ep.out0) + ((int64_t)(row0 + row_l) * ld + ocol) * ES;
    const int64_t stride = ld * ES;
    if (rows_full) {
      if (gelu) store_block16<KIND, true, false>(acc, j, base, stride, rows_left, bias);
      else store_block16<KIND, false, false>(acc, j, base, stride, rows_left, bias);
    } else {
      if (gelu) store_block16<KIND, true, true>(acc, j, base, stride, rows_left, bias);
      else store_block16<KIND, false, true>(acc, j, base, stride, rows_left, bias);
    }
  }
}

// 288x192 tiles, for problems whose 256x256 tiling leaves CUs idle in its
// last round while this one fills them: at M = 4608 it gives exactly 256
// tiles per round for N = 3072, 6144 and 9216 (216, 432 and 648 tiles of
// 256x256 use 84 % of the CUs).  The ping-pong schedule of the 256x256 kernel
// above, with v_mfma_f32_16x16x32_bf16: group g owns C rows [144 g, 144 g +
// 144), wave q of a group columns [48 q, 48 q + 48), 9 x 3 accumulators of
// 16x16; a 64-deep K tile is two 32-deep k-steps.  Operand lane l holds row
// (l & 15) of its 16-row fragment and 8 K elements from 8 (l >> 4) of the
// k-step: chunk 4 s + (l >> 4) of the 128-byte LDS row.  A has three LDS
// stages and B two (108 + 48 KB).  Loads: B 24 per tile (3 per wave), A 36
// (5 per wave in group 0, 4 in group 1).
template <OutKind KIND>
__global__ void __launch_bounds__(512)
gemm_bf16_nt_pp288(GemmProblem p, GemmEpilogue ep, int tiles_m, int tiles_n) {
  constexpr int BM = 288, BN = 192;
  constexpr int TM = 9, TN = 3, KS = 2;
  constexpr int A_STAGE = BM * kRowChunks;
  constexpr int B_STAGE = BN * kRowChunks;
  constexpr int BW = 3;
  __shared__ u32x4 smem[3 * A_STAGE + 2 * B_STAGE];   // 156 KB

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, q = wave & 3;

  const uint32_t lda2 = (uint32_t)p.lda * 2, ldb2 = (uint32_t)p.ldb * 2;
  const rsrc_t ra = buffer_rsrc(p.A, (uint32_t)(p.M - 1) * lda2 + (uint32_t)p.K * 2);
  const rsrc_t rb = buffer_rsrc(p.B, (uint32_t)(p.N - 1) * ldb2 + (uint32_t)p.K * 2);
  // A rows of this wave's loads: group 0 waves 40 each from 40 q, group 1
  // waves 32 each from 160 + 32 q; B rows 24 from 24 wave.  8 rows per load;
  // lane l reads row R + (l >> 3) into physical chunk l & 7 (swizzled).
  const int lr = lane >> 3, lc = lane & 7;
  const int arow0 = g == 0 ? 40 * q : 160 + 32 * q;
  const int brow0 = 24 * wave;
  uint32_t voa[5], vob[BW];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int R = arow0 + 8 * j;
    voa[j] = (uint32_t)(m0 + R + lr) * lda2 + (uint32_t)((lc ^ lr ^ ((R >> 3) & 1)) * 16);
  }
#pragma unroll
  for (int j = 0; j < BW; ++j) {
    const int R = brow0 + 8 * j;
    vob[j] = (uint32_t)(n0 + R + lr) * ldb2 + (uint32_t)((lc ^ lr ^ ((R >> 3) & 1)) * 16);
  }
  auto stage_a = [&](int kt) { return smem + (kt % 3) * A_STAGE; };
  auto stage_b = [&](int kt) { return smem + 3 * A_STAGE + (kt & 1) * B_STAGE; };
  auto load_a = [&](int kt, int j) {
    lds_dma(ra, stage_a(kt) + (arow0 + 8 * j) * kRowChunks, voa[j], (uint32_t)kt * (kBK * 2));
  };
  auto load_b = [&](int kt, int j) {
    lds_dma(rb, stage_b(kt) + (brow0 + 8 * j) * kRowChunks, vob[j], (uint32_t)kt * (kBK * 2));
  };
  auto b_loads = [&](int kt) {
#pragma unroll
    for (int j = 0; j < BW; ++j) load_b(kt, j);
  };
  // group 0 issues 5 A loads per tile, group 1 four (AW is a template
  // constant on each group's code path)
  auto a_loads = [&](int kt, auto aw) {
    constexpr int AW = decltype(aw)::value;
#pragma unroll
    for (int j = 0; j < AW; ++j) load_a(kt, j);
  };

  const int a_row = 144 * g + (lane & 15);
  const int b_row = 48 * q + (lane & 15);
  const int kq = lane >> 4;
  bf16x8 fa[KS][TM], fb[KS][TN];
  auto read_tile = [&](int kt) {
    const u32x4* sa = stage_a(kt);
    const u32x4* sb = stage_b(kt);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int kc = 4 * s + kq;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[s][i] = __builtin_bit_cast(bf16x8, sa[(a_row + 16 * i) * kRowChunks + swizzle(a_row, kc)]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[s][j] = __builtin_bit_cast(bf16x8, sb[(b_row + 16 * j) * kRowChunks + swizzle(b_row, kc)]);
    }
  };
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
  // The tile's 54 MFMAs, with load(l), l < nl, issued after MFMA 2 l.
  auto multiply = [&](auto&& load, int nl) {
    int idx = 0;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
          if ((idx & 1) == 0 && (idx >> 1) < nl) {
            __builtin_amdgcn_sched_barrier(0);
            load(idx >> 1);
            __builtin_amdgcn_sched_barrier(0);
          }
          ++idx;
        }
  };
  auto none = [](int) {};
  using AW0 = std::integral_constant<int, 5>;
  using AW1 = std::integral_constant<int, 4>;

  const int nk = p.K / kBK;
  b_loads(0);
  if (g == 0) {
    a_loads(0, AW0{});
    if (nk > 1) a_loads(1, AW0{});
  } else {
    a_loads(0, AW1{});
    if (nk > 1) a_loads(1, AW1{});
  }
  wait_vmem();
  wg_barrier();
  if (g == 0) {
    int kt = 0;
    for (; kt + 2 < nk; ++kt) {
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      b_loads(kt + 1);
      wg_barrier();                       // end of phase 2 kt
      multiply([&](int j) { load_a(kt + 2, j); }, 5);
      wait_vmem_keep<5>();                // B tile kt + 1 landed
      wg_barrier();                       // end of phase 2 kt + 1
    }
    if (kt + 1 < nk) {                    // kt = nk - 2
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      b_loads(kt + 1);
      wg_barrier();
      multiply(none, 0);
      wait_vmem();
      wg_barrier();
      ++kt;
    }
    read_tile(kt);                        // kt = nk - 1
    wg_barrier();
    multiply(none, 0);
    wg_barrier();
    wg_barrier();
  } else {
    if (nk > 1) b_loads(1);
    wg_barrier();                         // end of phase 0
    read_tile(0);
    __builtin_amdgcn_sched_barrier(0);
    if (nk > 2) {
      a_loads(2, AW1{});
      wait_vmem_keep<4>();
    } else {
      wait_vmem();
    }
    wg_barrier();                         // end of phase 1
    int kt = 1;
    for (; kt + 2 < nk; ++kt) {
      multiply([&](int j) { load_b(kt + 1, j); }, BW);   // tile kt - 1
      wg_barrier();                       // end of phase 2 kt
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      a_loads(kt + 2, AW1{});
      wait_vmem_keep<4>();
      wg_barrier();                       // end of phase 2 kt + 1
    }
    if (kt + 1 < nk) {                    // kt = nk - 2 >= 1
      multiply([&](int j) { load_b(kt + 1, j); }, BW);
      wg_barrier();
      read_tile(kt);
      wait_vmem();
      wg_barrier();
      ++kt;
    }
    if (kt < nk) {                        // kt = nk - 1 >= 1
      multiply(none, 0);
      wg_barrier();
      read_tile(kt);
      wg_barrier();
    }
    multiply(none, 0);                    // tile nk - 1
    wg_barrier();
  }

  store_tiles16<KIND, TM, TN>(acc, p, ep, m0 + 144 * g, n0 + 48 * q, lane);
}

// 256x256 tile on 4 waves, one per SIMD: wave (wm, wn) owns the 128x128
// block of C at rows 128 wm, columns 128 wn as 16 accumulator tiles of 32x32
// (256 registers, held in AGPRs).  A fragment read from LDS feeds 4 MFMAs
// here against 2 in the 8-wave kernel (whose waves own 128x64), so a K tile
// costs a third fewer LDS bytes.  With one wave per SIMD that wave's
// instruction stream alone keeps the matrix core busy:
//   * a 64-deep K tile is 4 k-steps of 16 MFMAs; the 8 fragments of k-step
//     s + 1 (4 of A, 4 of B, 16 bytes per lane each) are read while the MFMAs
//     of k-step s run, one read after every second MFMA;
//   * A has three LDS stages and B two (96 + 64 KB).  Each wave loads a
//     quarter of every tile (8 rows per load, 16 loads per K tile), one load
//     after every fourth MFMA: in K tile k the second half of B tile k + 1
//     (k-step 0), A tile k + 2 (k-steps 1-2) and the first half of B tile
//     k + 2 (k-step 3);
//   * one barrier per K tile, after the first 4 MFMAs of k-step 3: the
//     fragments of k-step 3 (read during k-step 2) have landed by then, so
//     the LDS wait before the barrier stalls nothing.  Before it every wave
//     waits for its loads of B tile k + 1; after it the first fragments of
//     tile k + 1 are read (two per MFMA) and B tile k + 2 goes into the
//     stage of tile k.
// Operand loads take the same buffer descriptors as the 8-wave kernel (rows
// past M or N read as zero).  The accumulators are stored in place: bias,
// activation and bf16 rounding are applied in the accumulator registers,
// then every element goes out with a buffer store whose per-lane offset lies
// past the output buffer for rows at or past M and columns at or past N.
// Requires K % 64 == 0, act_from and split multiples of 32 (of 64 for
// SwiGLU), and (M + 256) ld ES < 2^31 for the outputs as for the operands.
__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t bf16bits(float x) {
  const bf16 b = static_cast<bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}

// all but the newest N loads of this wave have landed (N = 8 or 0)
template <int N>
__device__ __forceinline__ void wait_vmem_w128() {
  static_assert(N == 8 || N == 0, "instantiated counts");
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// this wave's LDS reads have landed, then every wave's (the barrier)
__device__ __forceinline__ void lds_wait_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// In-place epilogue of a wave's TM x TN accumulator tiles at (row0, col0).
// FIX selects the activation for all the wave's columns at compile time
// (1: none, 2: GELU-tanh, 3: SwiGLU) or, with 0, per 32-column block.
template <OutKind KIND, int TM, int TN, int FIX>
__device__ __forceinline__ void store_tiles_inplace(f32x16 (&acc)[TM][TN], const GemmProblem& p,
                                                    const GemmEpilogue& ep, int row0, int col0,
                                                    int lane) {
  constexpr int ES = KIND == OutKind::BF16 ? 2 : 4;
  const int col_l = lane & 31;
  const int row_l = 4 * (lane >> 5);
  const uint32_t ld0 = (uint32_t)ep.ld0 * ES, ld1 = (uint32_t)ep.ld1 * ES;
  const rsrc_t r0 = buffer_rsrc(ep.out0, (uint32_t)p.M * ld0);
  const rsrc_t r1 = buffer_rsrc(ep.out1, (uint32_t)p.M * ld1);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int cb = col0 + 32 * j;                // the block's first column (wave-uniform)
    if (cb >= p.N) continue;
    const bool active = FIX != 0 ? FIX != 1 : (KIND != OutKind::F32_ACC && cb >= ep.act_from);
    const bool glu = FIX != 0 ? FIX == 3 : (active && ep.act == Act::SWIGLU);
    const bool gelu = FIX != 0 ? FIX == 2 : (active && ep.act == Act::GELU_TANH);
    if (glu && (j & 1)) continue;                // an up block, consumed with its gate block
    const int col = cb + col_l;
    const int ocb = glu ? ep.act_from + ((cb - ep.act_from) >> 1) : cb;
    const bool second = ocb >= ep.split;
    const int ocol = (second ? ocb - ep.split : ocb) + col_l;
    const uint32_t ld = second ? ld1 : ld0;
    const rsrc_t r = second ? r1 : r0;
    const bool colok = col < p.N;
    float bias = 0.0f, bias_up = 0.0f;
    if constexpr (KIND != OutKind::F32_ACC) {
      if (ep.bias && colok) {
        bias = ep.bias[col];
        if (glu) bias_up = ep.bias[col + 32];
      }
    }
    // columns past N get an offset past every output buffer
    const uint32_t lane_off = colok ? (uint32_t)(row0 + row_l) * ld + (uint32_t)ocol * ES : 0xF0000000u;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      // each element computed in its own accumulator register and stored
      // from there: no store's data register is rewritten while the store
      // may be in flight
      if constexpr (KIND == OutKind::F32_ACC) {
        float old[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t rw = 32 * i + 8 * (e >> 2) + (e & 3);
          old[e] = bitsf(__builtin_amdgcn_raw_buffer_load_b32(r, lane_off + rw * ld, 0, 0));
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] += old[e];
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float v = acc[i][j][e] + bias;
          if (glu) v = silu(v) * (acc[i][j | 1][e] + bias_up);
          else if (gelu) v = gelu_tanh(v);
          acc[i][j][e] = ES == 2 ? bitsf(bf16bits(v)) : v;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t rw = 32 * i + 8 * (e >> 2) + (e & 3);
        const uint32_t x = fbits(acc[i][j][e]);
        if constexpr (ES == 2)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)x, r, lane_off + rw * ld, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(x, r, lane_off + rw * ld, 0, 0);
      }
    }
  }
}

template <OutKind KIND, bool PERSIST>
__global__ void __launch_bounds__(256, 1)
gemm_bf16_nt_w128(GemmProblem p, GemmEpilogue ep, int tiles_m, int tiles_n) {
  constexpr int TM = 4, TN = 4;
  constexpr int A_STAGE = 256 * kRowChunks, B_STAGE = 256 * kRowChunks;
  __shared__ u32x4 smem[3 * A_STAGE + 2 * B_STAGE];   // 160 KB

  // Persistent: workgroup b takes one tile per round of G tiles, the
  // (b >> 3)-th of its XCD's contiguous stretch of the round (XCD b & 7) in
  // the grouped tile order.
  const int ntiles = tiles_m * tiles_n;
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  auto tile_id = [&](int round) -> int {
    const int base = round * G;
    if (base >= ntiles) return -1;
    const int count = min(G, ntiles - base);
    const int per = count >> 3, rem = count & 7;
    if (slot >= per + (xcd < rem ? 1 : 0)) return -1;
    return base + xcd * per + min(xcd, rem) + slot;
  };
  auto origin = [&](int id, int& m0, int& n0) {
    const int group = id / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in_group = id - group * kGroupM * tiles_n;
    m0 = (first_m + in_group % gm) * 256;
    n0 = (in_group / gm) * 256;
  };
  const int full_rounds = ntiles / G;
  const int n_mine = PERSIST ? full_rounds + (tile_id(full_rounds) >= 0 ? 1 : 0) : 1;   // >= 1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lda2 = (uint32_t)p.lda * 2, ldb2 = (uint32_t)p.ldb * 2;
  const rsrc_t ra = buffer_rsrc(p.A, (uint32_t)(p.M - 1) * lda2 + (uint32_t)p.K * 2);
  const rsrc_t rb = buffer_rsrc(p.B, (uint32_t)(p.N - 1) * ldb2 + (uint32_t)p.K * 2);
  // Wave w loads tile rows [64 w, 64 w + 64) of A and of B, 8 per load; lane
  // l reads row R + (l >> 3) into physical chunk l & 7 (the swizzle).  The
  // per-lane offset is this part plus the tile's first row times the row
  // pitch, so rows past M or N lie past the descriptors and read as zero.
  const int lr = lane >> 3, lc = lane & 7;
  uint32_t voa[8], vob[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int R = wave * 64 + 8 * j;
    voa[j] = (uint32_t)(R + lr) * lda2 + (uint32_t)((lc ^ lr ^ ((R >> 3) & 1)) * 16);
    vob[j] = (uint32_t)(R + lr) * ldb2 + (uint32_t)((lc ^ lr ^ ((R >> 3) & 1)) * 16);
  }
  // origins of this workgroup's current and next tile
  int m0, n0, m0n = 0, n0n = 0;
  origin(tile_id(0), m0, n0);
  if (n_mine > 1) origin(tile_id(1), m0n, n0n);
  const int nk = p.K / kBK;
  // global K-tile u of this workgroup's stream: A stage u % 3, B stage u % 2
  auto stage_a = [&](int u) { return smem + (u % 3) * A_STAGE; };
  auto stage_b = [&](int u) { return smem + 3 * A_STAGE + (u & 1) * B_STAGE; };
  // loads of global K-tile u, K-tile kt of the current tile (kt >= nk: of the next)
  // (with one tile per workgroup the tile's rows are folded into the
  // per-lane offsets once)
  if constexpr (!PERSIST) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      voa[j] += (uint32_t)m0 * lda2;
      vob[j] += (uint32_t)n0 * ldb2;
    }
  }
  auto load_a = [&](int u, int kt, int j) {
    if constexpr (PERSIST) {
      const bool nxt = kt >= nk;
      const uint32_t row = (uint32_t)(nxt ? m0n : m0) * lda2;
      lds_dma(ra, stage_a(u) + (wave * 64 + 8 * j) * kRowChunks, voa[j] + row,
              (uint32_t)(nxt ? kt - nk : kt) * (kBK * 2));
    } else {
      lds_dma(ra, stage_a(u) + (wave * 64 + 8 * j) * kRowChunks, voa[j], (uint32_t)kt * (kBK * 2));
    }
  };
  auto load_b = [&](int u, int kt, int j) {
    if constexpr (PERSIST) {
      const bool nxt = kt >= nk;
      const uint32_t row = (uint32_t)(nxt ? n0n : n0) * ldb2;
      lds_dma(rb, stage_b(u) + (wave * 64 + 8 * j) * kRowChunks, vob[j] + row,
              (uint32_t)(nxt ? kt - nk : kt) * (kBK * 2));
    } else {
      lds_dma(rb, stage_b(u) + (wave * 64 + 8 * j) * kRowChunks, vob[j], (uint32_t)kt * (kBK * 2));
    }
  };
  const int a_row = 128 * wm + (lane & 31), b_row = 128 * wn + (lane & 31), khalf = lane >> 5;
  const int total = n_mine * nk;   // K tiles in this workgroup's stream
  // prologue: B and A of K-tile 0, A of K-tile 1, then the first half of B of K-tile 1
#pragma unroll
  for (int j = 0; j < 8; ++j) load_b(0, 0, j);
#pragma unroll
  for (int j = 0; j < 8; ++j) load_a(0, 0, j);
  if (total > 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) load_a(1, 1, j);
  }
  wait_vmem_w128<0>();
  __syncthreads();
  if (total > 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) load_b(1, 1, j);
  }
  using T_ = std::true_type;
  using F_ = std::false_type;
  int u = 0;
  for (int t = 0; t < n_mine; ++t) {
    // fragments and accumulators live within one tile, so none is carried
    // across the tile's stores into the next
    bf16x8 fa[2][TM], fb[2][TN];
    f32x16 acc[TM][TN];
    // fragment r of k-group kc of global K-tile u into buffer buf: A tile i
    // = r (r < 4), B tile j = r - 4
    auto read_frag = [&](int uu, int kc, int buf, int r) {
      if (r < TM) {
        const u32x4* sa = stage_a(uu);
        fa[buf][r] = __builtin_bit_cast(bf16x8, sa[(a_row + 32 * r) * kRowChunks + swizzle(a_row, kc)]);
      } else {
        const u32x4* sb = stage_b(uu);
        fb[buf][r - TM] = __builtin_bit_cast(bf16x8, sb[(b_row + 32 * (r - TM)) * kRowChunks + swizzle(b_row, kc)]);
      }
    };
    auto mfma = [&](int buf, int m) {
      acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][m >> 2], fb[buf][m & 3],
                                                                   acc[m >> 2][m & 3], 0, 0, 0);
    };
    // the tile's first k-step starts its accumulators from zero
    auto mfma0 = [&](int m) {
      const f32x16 zero = {};
      acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][m >> 2], fb[0][m & 3], zero, 0, 0, 0);
    };
    // Global K tile u = K tile kt of the current tile.  NEXT2: K tile u + 2
    // exists; NEXT1: u + 1 exists (either may be in the next tile); FRAG1:
    // u + 1's first fragments are read here (not in a tile's last K tile, so
    // that no fragment registers stay live across the tile's stores).
    auto ktile = [&](int u, int kt, auto next2_c, auto next1_c, auto frag1_c, auto first_c) {
      constexpr bool NEXT2 = decltype(next2_c)::value;
      constexpr bool NEXT1 = decltype(next1_c)::value;
      constexpr bool FRAG1 = decltype(frag1_c)::value;
      constexpr bool FIRST = decltype(first_c)::value;   // the tile's first K tile
      // k-steps 0-2: fragments of k-step s + 1 after MFMAs 0, 2, .., 14;
      // loads after MFMAs 0, 4, 8, 12
  #pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int buf = s & 1;
  #pragma unroll
        for (int m = 0; m < 16; ++m) {
          if (FIRST && s == 0) mfma0(m); else mfma(buf, m);
          __builtin_amdgcn_sched_barrier(0);
          if ((m & 1) == 0) read_frag(u, 2 * (s + 1) + khalf, buf ^ 1, m >> 1);
          if ((m & 3) == 0) {
            if (s == 0) {
              if constexpr (NEXT1) load_b(u + 1, kt + 1, 4 + (m >> 2));
            } else {
              if constexpr (NEXT2) load_a(u + 2, kt + 2, 4 * (s - 1) + (m >> 2));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // k-step 3 (buffer 1): the barrier after MFMA 3; then K-tile u + 1's
      // first fragments, two after each of MFMAs 4-7 (so they have landed well
      // before its first MFMAs), and the first half of B of u + 2 after MFMAs 8-11
  #pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma(1, m);
        __builtin_amdgcn_sched_barrier(0);
        if (m == 3) {
          if constexpr (NEXT2) wait_vmem_w128<8>(); else wait_vmem_w128<0>();
          lds_wait_barrier();
        }
        if (m >= 4 && m < 8) {
          if constexpr (FRAG1) {
            read_frag(u + 1, khalf, 0, 2 * (m - 4));
            read_frag(u + 1, khalf, 0, 2 * (m - 4) + 1);
          }
        }
        if (m >= 8 && m < 12) {
          if constexpr (NEXT2) load_b(u + 2, kt + 2, m - 8);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // the tile's first fragments (its first K tile was published by the
    // prologue's barrier or by the previous tile's last K tile)
#pragma unroll
    for (int r = 0; r < 8; ++r) read_frag(u, khalf, 0, r);
    int kt = 0;
    if (t + 1 < n_mine) {
      ktile(u, kt, T_{}, T_{}, T_{}, T_{});
      for (++kt, ++u; kt + 1 < nk; ++kt, ++u) ktile(u, kt, T_{}, T_{}, T_{}, F_{});
      ktile(u, kt, T_{}, T_{}, F_{}, F_{});
      ++u;
    } else if (nk == 1) {
      ktile(u, kt, F_{}, F_{}, F_{}, T_{});
      ++u;
    } else {
      if (nk == 2) ktile(u, kt, F_{}, T_{}, T_{}, T_{});
      else ktile(u, kt, T_{}, T_{}, T_{}, T_{});
      for (++kt, ++u; kt + 2 < nk; ++kt, ++u) ktile(u, kt, T_{}, T_{}, T_{}, F_{});
      if (kt + 1 < nk) {
        ktile(u, kt, F_{}, T_{}, T_{}, F_{});
        ++kt;
        ++u;
      }
      ktile(u, kt, F_{}, F_{}, F_{}, F_{});
      ++u;
    }
    // the tile's results (with several tiles per workgroup, the loads of the
    // next tile's first K tiles are in flight meanwhile); one activation for
    // the wave's 128 columns when they lie on one side of act_from
    const int c0 = n0 + 128 * wn, r0 = m0 + 128 * wm;
    if (KIND == OutKind::F32_ACC || c0 + 128 <= ep.act_from || ep.act == Act::NONE)
      store_tiles_inplace<KIND, TM, TN, 1>(acc, p, ep, r0, c0, lane);
    else if (c0 >= ep.act_from && ep.act == Act::GELU_TANH)
      store_tiles_inplace<KIND, TM, TN, 2>(acc, p, ep, r0, c0, lane);
    else if (c0 >= ep.act_from && ep.act == Act::SWIGLU)
      store_tiles_inplace<KIND, TM, TN, 3>(acc, p, ep, r0, c0, lane);
    else
      store_tiles_inplace<KIND, TM, TN, 0>(acc, p, ep, r0, c0, lane);
    m0 = m0n;
    n0 = n0n;
    if (t + 2 < n_mine) origin(tile_id(t + 2), m0n, n0n);
  }
}

hipError_t launch_288(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind, hipStream_t stream) {
  const int tm = (p.M + 287) / 288, tn = (p.N + 191) / 192;
  const dim3 grid(tm * tn), block(512);
  switch (kind) {
    case OutKind::BF16:
      hipLaunchKernelGGL((gemm_bf16_nt_pp288<OutKind::BF16>), grid, block, 0, stream, p, ep, tm, tn);
      break;
    case OutKind::F32_STORE:
      hipLaunchKernelGGL((gemm_bf16_nt_pp288<OutKind::F32_STORE>), grid, block, 0, stream, p, ep, tm, tn);
      break;
    case OutKind::F32_ACC:
      hipLaunchKernelGGL((gemm_bf16_nt_pp288<OutKind::F32_ACC>), grid, block, 0, stream, p, ep, tm, tn);
      break;
  }
  return hipGetLastError();
}

// Compute units of the current device (cached per device; 256 on MI355X).
int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// One workgroup per compute unit, each looping over its tiles, when there
// are more tiles than compute units: then the next tile's first loads overlap
// this tile's stores.  This holds also where an activation covers only part
// of the columns (the fused QKV + up projection), whose activated tiles'
// epilogues cost several times the others': a workgroup's share of them
// differs from another's by at most one, less than the overlap gains.  One
// tile per workgroup when K is a single K tile, which the stream's two-ahead
// loads would otherwise reach past the next tile.
hipError_t launch_w128(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind, hipStream_t stream) {
  const int tm = (p.M + 255) / 256, tn = (p.N + 255) / 256;
  const int ntiles = tm * tn;
  const bool persist = p.K / kBK >= 2 && ntiles > cu_count();
  const dim3 grid(persist ? cu_count() : ntiles), block(256);
  switch (kind) {
    case OutKind::BF16:
      if (persist)
        hipLaunchKernelGGL((gemm_bf16_nt_w128<OutKind::BF16, true>), grid, block, 0, stream, p, ep, tm, tn);
      else
        hipLaunchKernelGGL((gemm_bf16_nt_w128<OutKind::BF16, false>), grid, block, 0, stream, p, ep, tm, tn);
      break;
    case OutKind::F32_STORE:
      if (persist)
        hipLaunchKernelGGL((gemm_bf16_nt_w128<OutKind::F32_STORE, true>), grid, block, 0, stream, p, ep, tm, tn);
      else
        hipLaunchKernelGGL((gemm_bf16_nt_w128<OutKind::F32_STORE, false>), grid, block, 0, stream, p, ep, tm, tn);
      break;
    case OutKind::F32_ACC:
      if (persist)
        hipLaunchKernelGGL((gemm_bf16_nt_w128<OutKind::F32_ACC, true>), grid, block, 0, stream, p, ep, tm, tn);
      else
        hipLaunchKernelGGL((gemm_bf16_nt_w128<OutKind::F32_ACC, false>), grid, block, 0, stream, p, ep, tm, tn);
      break;
  }
  return hipGetLastError();
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

template <class T, int BM, int BN, int WM, int WN>
hipError_t launch_tile(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind,
                       hipStream_t stream) {
  const int tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
  const dim3 grid(tm * tn), block(kThreads);
  const bool ktail = (p.K % (kRowChunks * (16 / (int)sizeof(T)))) != 0;
#define TPK_LAUNCH(K_, T_) \
  hipLaunchKernelGGL((gemm_nt_staged<T, BM, BN, WM, WN, K_, T_>), grid, block, 0, stream, p, ep, tm, tn)
  switch (kind) {
    case OutKind::BF16:
      if constexpr (std::is_same<T, float>::value) return hipErrorInvalidValue;  // fp32 in, fp32 out
      else if (ktail) TPK_LAUNCH(OutKind::BF16, true); else TPK_LAUNCH(OutKind::BF16, false);
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
  // the 8-wave kernel addresses operands with 32-bit byte offsets, also for
  // the rows of a last partial tile (up to 256 past M or N)
  const bool fits32 = (int64_t)(p.M + 256) * p.lda < ((int64_t)1 << 31) &&
                      (int64_t)(p.N + 256) * p.ldb < ((int64_t)1 << 31);
  // 288x192 tiles when they fill the rounds of CUs at least 8 % better than
  // 256x256 ones (e.g. every M = 4608 shape with N a multiple of 3072), for
  // the epilogues the 16x16 layout serves (not SwiGLU)
  const long t288 = (long)((p.M + 287) / 288) * ((p.N + 191) / 192);
  const bool fits288 = (int64_t)(p.M + 288) * p.lda < ((int64_t)1 << 31) &&
                       (int64_t)(p.N + 192) * p.ldb < ((int64_t)1 << 31);
  auto fill = [](long t) { return (double)t / (double)(((t + 255) / 256) * 256); };
  const long mid = (long)((p.M + 191) / 192) * ((p.N + 255) / 256);   // 192x256 tiles
  const double fill_32x32 = big < 256 && mid <= 256 ? fill(mid) : fill(big);
  if (t288 >= 128 && p.K % kBK == 0 && fits288 && ep.act != Act::SWIGLU &&
      ep.act_from % 16 == 0 && ep.split % 16 == 0 && fill(t288) > 1.08 * fill_32x32)
    return launch_288(p, ep, kind, stream);
  if (big >= 128 && p.K % kBK == 0 && fits32) {
    // One partial round of 256-row tiles leaves CUs idle (e.g. 162 tiles at
    // M = 4608, N = 2304); if 192-row tiles still fit in one round, every
    // busy CU has 3/4 of the work.
    if (big < 256 && mid <= 256) return launch_8w<3>(p, ep, kind, stream);
    // the one-wave-per-SIMD kernel where its in-place epilogue applies: the
    // activation and the output split fall on 32-column blocks (64 for
    // SwiGLU) and every output offset fits 31 bits
    const int64_t es = kind == OutKind::BF16 ? 2 : 4;
    const bool out_fits = (int64_t)(p.M + 256) * ep.ld0 * es < ((int64_t)1 << 31) &&
                          (ep.out1 == nullptr || (int64_t)(p.M + 256) * ep.ld1 * es < ((int64_t)1 << 31));
    const bool blocks = ep.split % 32 == 0 && ep.act_from % (ep.act == Act::SWIGLU ? 64 : 32) == 0;
    if (out_fits && blocks) return launch_w128(p, ep, kind, stream);
    return launch_8w<4>(p, ep, kind, stream);
  }
  if (big >= 256) return launch_tile<bf16, 256, 256, 2, 2>(p, ep, kind, stream);
  return launch_tile<bf16, 128, 128, 2, 2>(p, ep, kind, stream);
}

// fp32 operands (the fp32 shards, parity workloads): the register-staged
// kernel with 128x128 tiles, fp32 out (store or accumulate).
hipError_t launch_gemm_f32(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind,
                           hipStream_t stream) {
  if (kind == OutKind::BF16) return hipErrorInvalidValue;
  return launch_tile<float, 128, 128, 2, 2>(p, ep, kind, stream);
}

}  // namespace tpk
