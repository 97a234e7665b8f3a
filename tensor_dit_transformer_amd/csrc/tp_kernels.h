// Internal interface between the host layer (shard.hip) and the gfx950
// kernels.  Not part of the public ABI (include/tp_shard.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace tpk {

// What the GEMM epilogue does with each fp32 accumulator.
enum class OutKind : int {
  BF16 = 0,       // (+bias, activation on a column range) -> bf16 store
  F32_STORE = 1,  // (+bias, activation on a column range) -> fp32 store
  F32_ACC = 2,    // fp32 read-add-write (rowwise partial accumulate), no bias
};

// C[M, N] = A[M, K] * B[N, K]^T: both operands K-contiguous (x in [T, K],
// weights in the nn.Linear [out, in] layout).
struct GemmProblem {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int M, N, K;
};

// Activation applied by the colwise epilogue to columns n >= act_from, after
// the bias.
enum class Act : int {
  NONE = 0,
  GELU_TANH = 1,  // y[n] = gelu_tanh(c[n] + b[n])
  SWIGLU = 2,     // columns from act_from on come in 64-column pairs
                  // [gate 32 | up 32]; pair p's lane c < 32 gives the ONE
                  // output column act_from + 32 p + c = silu(gate + b) * (up + b)
};

// Output column o (after SwiGLU's pair -> column map) goes to out0[:, o] if
// o < split, else to out1[:, o - split] (two tensors written by one launch:
// the packed QKV + MLP-in colwise projection).  bias is fp32 [N] or nullptr.
// SWIGLU needs act_from and N - act_from to be multiples of 64 (the kernels'
// per-wave column blocks start at multiples of 64).
struct GemmEpilogue {
  const float* bias;
  int act_from;
  Act act;
  int split;
  void* out0;
  int64_t ld0;
  void* out1;
  int64_t ld1;
};

hipError_t launch_gemm_bf16(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind,
                            hipStream_t stream);
hipError_t launch_gemm_f32(const GemmProblem& p, const GemmEpilogue& ep, OutKind kind,
                           hipStream_t stream);

// Rowwise partial with few rows (bf16 in, fp32 out, store or accumulate):
// out[m, n] (+)= sum_k A[m, k] B[n, k].  Applies when 1 <= M <= 64,
// N % 16 == 0 and K % 8 == 0 (skinny_bf16_fits); an HBM-bound weight stream.
bool skinny_bf16_fits(const GemmProblem& p);
hipError_t launch_skinny_bf16(const GemmProblem& p, float* out, int64_t ldo, bool accumulate,
                              hipStream_t stream);

// Non-causal multi-head attention, bf16 in/out, head_dim 128, fp32 softmax.
// qkv: [T, 3*Dr] (Q | K | V, head j at columns j*128 of each block);
// o: [T, Dr].
hipError_t launch_attn_fwd_bf16_d128(const void* qkv, int64_t ldqkv, void* o, int64_t ldo,
                                     int T, int heads, hipStream_t stream);

// Attention of Tq queries against a block of Tkv keys/values (head j at
// columns j*128 of q, k and v, all bf16): the block's normalised output in
// fp32, o[t, j*128 + c], and the natural log-sum-exp of its scaled scores,
// lse[t * ld_lse + j].  With splits > 1 the keys are cut into that many
// contiguous ranges [floor(z Tkv / splits), floor((z+1) Tkv / splits)), all
// in one launch, range z writing at o + z o_split and lse + z lse_split
// (Tkv < splits is hipErrorInvalidValue).
struct AttnBlockArgs {
  const void* q;
  int64_t ldq;
  const void* k;
  const void* v;
  int64_t ldkv;
  int Tq, Tkv, heads;
  float* o;
  int64_t ldo;
  float* lse;
  int64_t ld_lse;
  int splits;
  int64_t o_split, lse_split;
};
hipError_t launch_attn_block_bf16_d128(const AttnBlockArgs& a, hipStream_t stream);
// Key splits (1..4) at which one launch over T queries and `heads` heads
// runs the pipelined kernel on enough workgroups; 1 when it already does or
// when no split up to 4 gets there.
int attn_split_hint(int T, int heads);

// Merge of partial attention results over disjoint key blocks, per (token t,
// head j): lse = log sum_i exp(lse_i), o = sum_i exp(lse_i - lse) o_i.
constexpr int kMaxMergeParts = 16;
struct MergeArgs {
  const float* o[kMaxMergeParts];
  const float* lse[kMaxMergeParts];
  int n;
  int64_t ldo_in, ld_lse_in;
  int T, heads, head_dim;    // head_dim % 4 == 0
  void* out;                 // bf16 or fp32 [T, heads*head_dim]
  bool out_bf16;
  int64_t ldo;
  float* lse_out;            // nullable
  int64_t ld_lse_out;
};
hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream);

// Up to kMaxCopies equal-shaped 2-D block copies in one launch: block c
// copies `rows` rows of `chunks` 16-byte chunks from src[c] (row stride
// src_ld bytes) to dst[c] (row stride dst_ld bytes).  All 16-byte aligned.
constexpr int kMaxCopies = 48;
struct CopyBlocksArgs {
  const char* src[kMaxCopies];
  char* dst[kMaxCopies];
  int n;
  int rows, chunks;
  int64_t src_ld, dst_ld;
};
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

constexpr int kMaxReducePartials = 16;
constexpr int kMaxReduceBiases = 4;

struct ReduceArgs {
  const float* partials[kMaxReducePartials];
  const float* biases[kMaxReduceBiases];
  int n_partials;
  int n_biases;
  int64_t rows;
  int64_t cols;      // multiple of 4
  int64_t ldp;
  int64_t ldo;
  float* out;
};

hipError_t launch_partial_reduce(const ReduceArgs& a, hipStream_t stream);

}  // namespace tpk
