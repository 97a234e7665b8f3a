// Ulysses re-layouts on one GPU (Diffusers context-parallelism page,
// §"Ulysses Attention": a first all-to-all regroups the data so each GPU holds
// every token of a subset of heads; a second regroups the attention output by
// token).  With the u ranks' buffers all on one device, each all-to-all is a
// set of equal-shaped 2-D block copies:
//   sequence -> heads, for rank r: rows [s n, (s+1) n) of its output, column
//     block b (Q, K, V or a single tensor) = token chunk s's columns
//     [b H d + r W, + W), W = (H / u) d, for every source rank s;
//   heads -> sequence, for rank s: its columns [r W, + W) = rows
//     [s n, (s+1) n) of rank r's head-block output, for every r.
// One launch copies up to kMaxCopies such blocks; a thread moves 16 bytes,
// consecutive threads walk a row, so every block row is read and written
// as whole contiguous segments (HBM-bound: 2 x the bytes moved).
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) copy_blocks(CopyBlocksArgs a) {
  const int c = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.rows * a.chunks) return;
  const int64_t row = idx / a.chunks;
  const int ch = (int)(idx - row * a.chunks);
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.src[c] + row * a.src_ld + 16 * ch);
  *reinterpret_cast<u32x4*>(a.dst[c] + row * a.dst_ld + 16 * ch) = v;
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.rows * a.chunks;
  const dim3 grid((unsigned)((threads + 255) / 256), a.n), block(256);
  hipLaunchKernelGGL(copy_blocks, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace tpk
