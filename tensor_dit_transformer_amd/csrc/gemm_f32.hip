// fp32 GEMM, C[M, N] = A[M, K] * B[N, K]^T with the same epilogues as the
// bf16 kernel (bias, GELU-tanh or SwiGLU on a column range, split output,
// fp32 accumulate).  It serves fp32 shards (colwise / rowwise projections of
// the Diffusers TP page, §"Colwise e rowwise"), which are small and
// correctness-oriented; it runs on the vector ALUs with plain fp32 FMA,
// 64x64 output tiles, 16-deep K tiles staged through LDS, 4x4 outputs per
// thread (columns 2 tx, 2 tx + 1, 32 + 2 tx, 33 + 2 tx of the tile, so a
// SwiGLU gate column and its up column, 32 apart, sit in one thread).
// Out-of-range rows are clamped on load and masked on store; K past the end
// is zero-filled (K is a multiple of 4).
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64, kBN = 64, kBK = 16;

__device__ __forceinline__ float gelu_tanh(float u) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float z = c * fmaf(0.044715f * u, u * u, u);
  return u / (1.0f + __expf(-2.0f * z));
}

__device__ __forceinline__ float silu(float u) { return u / (1.0f + __expf(-u)); }

// Tile column of a thread's j-th output column.
__device__ __forceinline__ int tile_col(int tx, int j) { return (j >> 1) * 32 + 2 * tx + (j & 1); }

template <OutKind KIND>
__global__ void __launch_bounds__(256) gemm_f32_nt(GemmProblem p, GemmEpilogue ep) {
  __shared__ float As[kBK][kBM + 4];  // transposed tiles: [k][row]
  __shared__ float Bs[kBK][kBN + 4];
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const float* __restrict__ A = static_cast<const float*>(p.A);
  const float* __restrict__ B = static_cast<const float*>(p.B);

  // loader: row tid/4 of the tile, k quad (tid%4)*4
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int64_t a_off = (int64_t)min(m0 + lr, p.M - 1) * p.lda + lk;
  const int64_t b_off = (int64_t)min(n0 + lr, p.N - 1) * p.ldb + lk;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += kBK) {
    const bool in = k0 + lk < p.K;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 a = in ? *reinterpret_cast<const f32x4*>(A + a_off + k0) : zero;
    const f32x4 b = in ? *reinterpret_cast<const f32x4*>(B + b_off + k0) : zero;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lk + i][lr] = a[i];
      Bs[lk + i][lr] = b[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tile_col(tx, j)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + tile_col(tx, j);
    if (col >= p.N) continue;
    const bool active = KIND != OutKind::F32_ACC && col >= ep.act_from;
    const bool glu = active && ep.act == Act::SWIGLU;
    const bool gelu = active && ep.act == Act::GELU_TANH;
    if (glu && j >= 2) continue;  // an up column, consumed with its gate (j - 2)
    int ocol = glu ? ep.act_from + (((col - ep.act_from) >> 6) << 5) + ((col - ep.act_from) & 31) : col;
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
    float* out = static_cast<float*>(second ? ep.out1 : ep.out0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + ty * 4 + i;
      if (row >= p.M) continue;
      float* o = out + (int64_t)row * ld + ocol;
      if constexpr (KIND == OutKind::F32_ACC) {
        *o = *o + acc[i][j];
      } else {
        float v = acc[i][j] + bias;
        if (glu) v = silu(v) * (acc[i][(j + 2) & 3] + bias_up);
        else if (gelu) v = gelu_tanh(v);
        *o = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind,
                           hipStream_t stream) {
  const dim3 grid((p.N + kBN - 1) / kBN, (p.M + kBM - 1) / kBM), block(256);
  switch (kind) {
    case OutKind::F32_ACC:
      hipLaunchKernelGGL(gemm_f32_nt<OutKind::F32_ACC>, grid, block, 0, stream, p, ep);
      break;
    case OutKind::F32_STORE:
      hipLaunchKernelGGL(gemm_f32_nt<OutKind::F32_STORE>, grid, block, 0, stream, p, ep);
      break;
    default:
      return hipErrorInvalidValue;  // fp32 inputs never produce bf16 outputs
  }
  return hipGetLastError();
}

}  // namespace tpk
