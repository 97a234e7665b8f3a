// Rowwise partial projection with few rows, bf16 in, fp32 out:
//   out[m, n] (+)= sum_k A[m, k] * B[n, k],   m < M <= 64, n < N, k < K
//
// The rowwise partial of the Diffusers TP page (§"Colwise e rowwise") when
// the input has only a handful of rows -- the replicated conditioning rows of
// an AdaLN modulation projection sharded "rowwise_split_input", or a short
// sequence.  The work is then a stream of the weight slice B (N x K bf16)
// past a tiny A: bound by HBM, not by the matrix cores.  Design:
//   * one workgroup = 4 waves = RG groups of 16 weight rows; wave w takes the
//     32-wide k-blocks kb = w, w + 4, ... of those rows, so the four waves'
//     loads of one row are neighbouring 64-byte segments;
//   * per k-block a lane loads 16 bytes of B per row group (row l % 16,
//     k-group l / 16) -- exactly the A-operand layout of
//     v_mfma_f32_16x16x32_bf16 -- and 16 bytes of A per 16-row block of M
//     (the B-operand layout), then one MFMA per (row group, row block):
//     D[n][m] accumulates over the wave's k-blocks;
//   * UN k-blocks of loads are issued before their MFMAs (up to 16: with a
//     1536-wide slice that is every load of the wave), which sets the bytes
//     in flight per CU; measured best at RG = 2, UN = 16 for M <= 16;
//   * the four waves' partial D tiles are summed through LDS in wave order
//     (deterministic) and stored as float4 rows of out (n contiguous).
// k-blocks past K read as zero (K % 8 == 0 keeps 16-byte chunks whole);
// A rows past M read as zero and are not stored; N % 16 == 0.
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kMaxMB = 4;     // 16-row blocks of A: M <= 64

template <int MB, int RG, int UN, bool ACC>
__global__ void __launch_bounds__(256)
skinny_bf16(const __bf16* __restrict__ A, int lda, const __bf16* __restrict__ B, int ldb, int M,
            int N, int K, float* __restrict__ out, int64_t ldo) {
  __shared__ f32x4 red[kWaves][RG * MB][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16 * RG;
  const int r = lane & 15, kg = lane >> 4;
  const __bf16* brow[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) brow[g] = B + (int64_t)(n0 + 16 * g + r) * ldb + 8 * kg;
  const __bf16* arow[MB];
  bool a_in[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = 16 * mb + r;
    a_in[mb] = m < M;
    arow[mb] = A + (int64_t)(a_in[mb] ? m : 0) * lda + 8 * kg;
  }

  f32x4 acc[RG][MB];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[g][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int nkb = (K + 31) / 32;
  for (int kb0 = wave; kb0 < nkb; kb0 += kWaves * UN) {
    u32x4 b[UN][RG], a[UN][MB];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int kb = kb0 + kWaves * u;
      const bool in = 32 * kb + 8 * kg < K;
#pragma unroll
      for (int g = 0; g < RG; ++g)
        b[u][g] = in ? *reinterpret_cast<const u32x4*>(brow[g] + 32 * kb) : zero;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[u][mb] = in && a_in[mb] ? *reinterpret_cast<const u32x4*>(arow[mb] + 32 * kb) : zero;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[g][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, b[u][g]), __builtin_bit_cast(bf16x8, a[u][mb]),
              acc[g][mb], 0, 0, 0);
  }

#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][g * MB + mb][lane] = acc[g][mb];
  __syncthreads();
  // tile t = (row group g, row block mb), stored by wave t % 4, summed in wave
  // order: D[n = 4 (lane / 16) + e][m = lane % 16]
  for (int t = wave; t < RG * MB; t += kWaves) {
    const int g = t / MB, mb = t % MB;
    f32x4 s = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[w][t][lane];
    const int m = 16 * mb + r;
    if (m < M) {
      f32x4* o = reinterpret_cast<f32x4*>(out + (int64_t)m * ldo + n0 + 16 * g + 4 * kg);
      if constexpr (ACC) s += *o;
      *o = s;
    }
  }
}

template <int MB, int RG, int UN>
void launch_cfg(const GemmProblem& p, float* out, int64_t ldo, bool acc, hipStream_t stream) {
  const dim3 grid(p.N / (16 * RG)), block(kWaves * 64);
  const __bf16* A = static_cast<const __bf16*>(p.A);
  const __bf16* B = static_cast<const __bf16*>(p.B);
  if (acc)
    hipLaunchKernelGGL((skinny_bf16<MB, RG, UN, true>), grid, block, 0, stream, A, (int)p.lda, B,
                       (int)p.ldb, p.M, p.N, p.K, out, ldo);
  else
    hipLaunchKernelGGL((skinny_bf16<MB, RG, UN, false>), grid, block, 0, stream, A, (int)p.lda, B,
                       (int)p.ldb, p.M, p.N, p.K, out, ldo);
}

// Deeper unroll for fewer row blocks keeps the register count in bounds.
template <int MB, int UN>
void launch_mb(const GemmProblem& p, float* out, int64_t ldo, bool acc, hipStream_t stream) {
  if (p.N % 32 == 0)
    launch_cfg<MB, 2, UN>(p, out, ldo, acc, stream);
  else
    launch_cfg<MB, 1, UN>(p, out, ldo, acc, stream);
}

}  // namespace

bool skinny_bf16_fits(const GemmProblem& p) {
  return p.M >= 1 && p.M <= 16 * kMaxMB && p.N % 16 == 0 && p.K % 8 == 0 &&
         (int64_t)p.N * p.ldb < ((int64_t)1 << 31) && (int64_t)p.M * p.lda < ((int64_t)1 << 31);
}

hipError_t launch_skinny_bf16(const GemmProblem& p, float* out, int64_t ldo, bool accumulate,
                              hipStream_t stream) {
  if (!skinny_bf16_fits(p)) return hipErrorInvalidValue;
  switch ((p.M + 15) / 16) {
    case 1: launch_mb<1, 16>(p, out, ldo, accumulate, stream); break;
    case 2: launch_mb<2, 8>(p, out, ldo, accumulate, stream); break;
    case 3: launch_mb<3, 4>(p, out, ldo, accumulate, stream); break;
    default: launch_mb<4, 4>(p, out, ldo, accumulate, stream); break;
  }
  return hipGetLastError();
}

}  // namespace tpk
