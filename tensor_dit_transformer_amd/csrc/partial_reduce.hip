// The layer-boundary AllReduce of the Diffusers TP page (intro; §"Colwise e
// rowwise": one AllReduce at the block boundary rebuilds the result), done on
// one GPU for ranks simulated one after another:
//   out[r, c] = ((p_0[r, c] + p_1[r, c]) + ... + p_{P-1}[r, c]) + b_0[c] + ...
// in fp32, rank order fixed, so the result is deterministic.
//
// Pure HBM streaming (0.2 FLOP/byte): one float4 (16-byte) element per
// thread and many small workgroups; each thread has its P loads in flight at
// once.  (Measured at 4 x 16384 x 6144: one element per thread streams
// ~6.6 TB/s alone, two ~6.5, four ~6.0, eight collapse.)  Partials are read and the output written with non-temporal hints:
// none of it is reused, so it should not displace L2 / MALL contents.
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 1;

template <bool CONTIG>
__global__ void __launch_bounds__(kThreads) partial_reduce_kernel(ReduceArgs a) {
  const int64_t cols4 = a.cols >> 2;
  const int64_t n = a.rows * cols4;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  int64_t poff[kUnroll], ooff[kUnroll], boff[kUnroll];
  bool live[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t idx = base + (int64_t)u * kThreads;
    live[u] = idx < n;
    if (CONTIG) {
      poff[u] = ooff[u] = idx << 2;
      boff[u] = (int64_t)((uint32_t)idx % (uint32_t)cols4) << 2;  // n < 2^31 (host-checked)
    } else {
      const int64_t r = (uint32_t)idx / (uint32_t)cols4, c = idx - r * cols4;
      poff[u] = r * a.ldp + (c << 2);
      ooff[u] = r * a.ldo + (c << 2);
      boff[u] = c << 2;
    }
  }
  f32x4 s[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    s[u] = live[u] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.partials[0] + poff[u]))
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 1; i < kMaxReducePartials; ++i) {
    if (i >= a.n_partials) break;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (live[u])
        s[u] += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.partials[i] + poff[u]));
  }
#pragma unroll
  for (int i = 0; i < kMaxReduceBiases; ++i) {
    if (i >= a.n_biases) break;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (live[u]) s[u] += *reinterpret_cast<const f32x4*>(a.biases[i] + boff[u]);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (live[u]) __builtin_nontemporal_store(s[u], reinterpret_cast<f32x4*>(a.out + ooff[u]));
}

}  // namespace

hipError_t launch_partial_reduce(const ReduceArgs& a, hipStream_t stream) {
  const int64_t n = a.rows * (a.cols >> 2);
  const int64_t blocks = (n + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  if (blocks == 0) return hipSuccess;
  const bool contig = a.ldp == a.cols && a.ldo == a.cols;
  if (contig)
    hipLaunchKernelGGL(partial_reduce_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(partial_reduce_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace tpk
