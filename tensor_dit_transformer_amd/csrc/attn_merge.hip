// Merge of partial attention results over disjoint key blocks -- the
// combination a Ring Attention rank applies to the outputs of its ring steps
// (Diffusers context-parallelism page, §"Ring Attention": after a full cycle
// every rank has attended its queries to every K/V block):
//   per (token t, head j):  lse = log sum_i exp(lse_i),
//                           o   = sum_i exp(lse_i - lse) o_i
// with the largest lse_i subtracted before the exponentials.
//
// HBM-bound: one thread per 4 consecutive output dims of one (t, j), so a
// row's threads read each partial's row as contiguous float4s and write the
// output row contiguously; the threads of a head recompute the n weights
// (n <= 16 exponentials, trivial next to the loads).  The grid's x index is
// the token and y the column block, so a thread finds its head with one
// 32-bit division.
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) attn_merge(MergeArgs a) {
  const int groups = a.head_dim / 4;
  const int col4 = blockIdx.y * blockDim.x + threadIdx.x;   // float4 column of the row
  if (col4 >= a.heads * groups) return;
  const int j = col4 / groups, c4 = col4 - j * groups;
  const int64_t t = blockIdx.x;

  float l[kMaxMergeParts];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i) {
    if (i < a.n) {
      l[i] = a.lse[i][t * a.ld_lse_in + j];
      m = fmaxf(m, l[i]);
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i) {
    if (i < a.n) {
      l[i] = __expf(l[i] - m);
      sum += l[i];
    }
  }
  const float inv = 1.0f / sum;
  const int64_t col = (int64_t)j * a.head_dim + 4 * c4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i) {
    if (i < a.n) acc += (l[i] * inv) * *reinterpret_cast<const f32x4*>(a.o[i] + t * a.ldo_in + col);
  }
  if (a.out_bf16) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[e]);
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.out) + t * a.ldo + col) = v;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + t * a.ldo + col) = acc;
  }
  if (a.lse_out && c4 == 0) a.lse_out[t * a.ld_lse_out + j] = m + __logf(sum);
}

}  // namespace

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  const int row4 = a.heads * (a.head_dim / 4);   // float4 columns per token
  const int threads = min(256, (row4 + 63) / 64 * 64);
  const dim3 grid((unsigned)a.T, (unsigned)((row4 + threads - 1) / threads)), block(threads);
  hipLaunchKernelGGL(attn_merge, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace tpk
