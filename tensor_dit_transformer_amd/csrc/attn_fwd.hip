// Non-causal multi-head attention over one rank's heads, bf16 in/out,
// head_dim 128, fp32 online softmax, on gfx950 matrix cores.
//
// Colwise Q/K/V projections give each rank a subset of the heads (Diffusers
// TP page, §"Colwise e rowwise"), so attention needs nothing from other
// ranks: for local head j, O_j = softmax(Q_j K_j^T / sqrt(128)) V_j over all
// T keys, with Q_j, K_j, V_j the column blocks j*128 of the Q, K and V parts
// of the packed qkv tensor [T, 3*Dr].
//
// Design:
//   * grid = (ceil(T/128), heads); 4 waves per workgroup, 32 queries per wave,
//     <= 256 VGPRs so two workgroups share a CU (two waves per SIMD).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = a 32-key slab of K from LDS, B = the
//     wave's Q^T held in registers for the whole kernel).  In the 32x32
//     accumulator a lane owns one query column, so the running max / sum
//     of its query are lane-local (plus one exchange with lane ^ 32).
//   * Output is accumulated transposed too, O^T += V^T P^T: the bf16 P^T
//     B-operand is the score accumulator itself, converted in registers; the
//     A-operand is V^T, stored in LDS key-contiguous with the key order
//     inside every 16 keys permuted (bits 2 and 3 swapped) so that the 8
//     keys a lane needs are one 16-byte read.
//   * K and V tiles of 64 keys are fetched one tile ahead into registers and
//     written to a double-buffered LDS (padded rows, conflict-free reads);
//     one barrier per tile.
//   * Softmax runs in the exp2 domain with few vector instructions per
//     score: one FMA (scale folded in) and one exp2; the row sum is a bf16
//     dot2 over the packed weights; the accumulator is rescaled by
//     exp2(m_old - m_new) only when a row max outgrows the reference by 8
//     (log2 units).  Keys past T get -inf (last tile only); query rows past T
//     are clamped on load and not stored.
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;            // head dim
constexpr int kBQ = 128;           // queries per workgroup
constexpr int kBKV = 64;           // keys per tile
constexpr int kKPitch = kD + 8;    // bf16 per K row in LDS (272 bytes)
constexpr int kVPitch = kBKV + 8;  // bf16 per V^T row in LDS (144 bytes)

// Position of key k (0..63) in a V^T row: swap bits 2 and 3.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Slack (log2 domain) the running max may trail the true row max before the
// accumulator is rescaled.  Softmax is invariant to the reference value, so
// this only lets the unnormalised weights grow to at most 2^8; it skips almost
// every O rescale once the first tiles have set the max.
constexpr float kRescaleSlack = 8.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <bool MASKED>
__device__ __forceinline__ void attn_tile(const bf16* __restrict__ sKb, const bf16* __restrict__ sVb,
                                          const bf16x8 (&qf)[kD / 16], f32x16 (&acc_o)[kD / 32],
                                          float& m_ref, float& l_run, int key0, int T,
                                          float scale_log2, int l32, int half) {
  // S^T for keys 32 c .. 32 c + 31 of the tile (raw scores)
  f32x16 s[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[c][e] = 0.0f;
    const bf16* kb = sKb + (32 * c + l32) * kKPitch + 8 * half;
#pragma unroll
    for (int st = 0; st < kD / 16; ++st) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kb + 16 * st);
      s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s[c], 0, 0, 0);
    }
  }
  if constexpr (MASKED) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + 32 * c + 8 * (e >> 2) + 4 * half + (e & 3);
        if (key >= T) s[c][e] = -INFINITY;
      }
  }
  // tile max of this lane's 32 scores, then of the other half-wave's 32
  float mloc = s[0][0];
#pragma unroll
  for (int e = 1; e < 16; e += 2) mloc = fmaxf(mloc, fmaxf(s[0][e], s[0][e + 1]));
#pragma unroll
  for (int e = 0; e < 16; e += 2) mloc = fmaxf(mloc, fmaxf(s[1][e], s[1][e + 1]));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32)) * scale_log2;
  // rescale only when some row's max outgrew the reference by the slack
  if (__builtin_amdgcn_ballot_w64(mloc > m_ref + kRescaleSlack)) {
    const float m_new = fmaxf(m_ref, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    m_ref = m_new;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < kD / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[t][e] *= alpha;
  }
  // p = exp2(s * log2(e)/sqrt(d) - m_ref), packed to bf16 for the PV product;
  // the row sum adds the bf16 values the product actually uses
  bf16x8 pb[2][2];
  const bf16x2 ones = {static_cast<bf16>(1.0f), static_cast<bf16>(1.0f)};
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[c][e], scale_log2, -m_ref));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[c][e + 1], scale_log2, -m_ref));
      const bf16x2 pp = {static_cast<bf16>(p0), static_cast<bf16>(p1)};
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
      pb[c][e >> 3][e & 7] = pp[0];
      pb[c][e >> 3][(e & 7) + 1] = pp[1];
    }
  // O^T += V^T P^T over the tile's 4 steps of 16 keys
#pragma unroll
  for (int t = 0; t < kD / 32; ++t) {
    const bf16* vb = sVb + (32 * t + l32) * kVPitch + 8 * half;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vb + 32 * c + 16 * u);
        acc_o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c][u], acc_o[t], 0, 0, 0);
      }
  }
}

// Two workgroups per CU (<= 256 VGPRs per wave): each SIMD runs two waves, so
// one wave's softmax arithmetic overlaps the other's matrix instructions.
__global__ void __launch_bounds__(256, 2)
attn_fwd_bf16_d128(const bf16* __restrict__ qkv, int64_t ldqkv, bf16* __restrict__ o,
                   int64_t ldo, int T, int heads, float scale_log2) {
  __shared__ bf16 sK[2][kBKV * kKPitch];
  __shared__ bf16 sVt[2][kD * kVPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * kBQ + wave * 32;
  const int Dr = heads * kD;
  const bf16* Qg = qkv + head * kD;
  const bf16* Kg = qkv + Dr + head * kD;
  const bf16* Vg = qkv + 2 * Dr + head * kD;
  const int half = lane >> 5, l32 = lane & 31;

  // Q^T operand: lane holds query q0 + l32, dims 16 s + 8 half .. +7
  bf16x8 qf[kD / 16];
  {
    const int64_t row = min(q0 + l32, T - 1);
#pragma unroll
    for (int s = 0; s < kD / 16; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(Qg + row * ldqkv + 16 * s + 8 * half);
  }

  // K tile loader: chunk (row (tid >> 4) + 16 i, 16-byte column tid & 15)
  const int k_row = tid >> 4, k_c = tid & 15;
  // V tile loader: key pair (tid & 31), dim chunk (tid >> 5) + 8 i
  const int v_pair = tid & 31, v_c = tid >> 5;
  u32x4 rk[4];
  u32x4 rv[2][2];

  auto gload = [&](int kt) {
    const int k0 = kt * kBKV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = min(k0 + k_row + 16 * i, T - 1);
      rk[i] = *reinterpret_cast<const u32x4*>(Kg + row * ldqkv + 8 * k_c);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = v_c + 8 * i;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int64_t row = min(k0 + 2 * v_pair + t, T - 1);
        rv[i][t] = *reinterpret_cast<const u32x4*>(Vg + row * ldqkv + 8 * c);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&sK[buf][(k_row + 16 * i) * kKPitch + 8 * k_c]) = rk[i];
    const int pos = vt_pos(2 * v_pair);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = v_c + 8 * i;
      const u16x8 a = __builtin_bit_cast(u16x8, rv[i][0]);
      const u16x8 b = __builtin_bit_cast(u16x8, rv[i][1]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const unsigned int w = (unsigned int)a[jj] | ((unsigned int)b[jj] << 16);
        *reinterpret_cast<unsigned int*>(&sVt[buf][(8 * c + jj) * kVPitch + pos]) = w;
      }
    }
  };

  f32x16 acc_o[kD / 32];
#pragma unroll
  for (int t = 0; t < kD / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc_o[t][e] = 0.0f;
  float m_ref = -INFINITY, l_run = 0.0f;

  const int nkt = (T + kBKV - 1) / kBKV;
  const int nfull = T / kBKV;  // tiles with every key valid
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) gload(kt + 1);
    if (kt < nfull)
      attn_tile<false>(sK[buf], sVt[buf], qf, acc_o, m_ref, l_run, kt * kBKV, T, scale_log2, l32, half);
    else
      attn_tile<true>(sK[buf], sVt[buf], qf, acc_o, m_ref, l_run, kt * kBKV, T, scale_log2, l32, half);
    if (more) sstore(buf ^ 1);
    __syncthreads();
  }

  // normalise and store: lane holds query q0 + l32, dims 32 t + 8 (e/4) + 4 half + (e%4)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  const int q = q0 + l32;
  if (q < T) {
    bf16* orow = o + (int64_t)q * ldo + head * kD;
#pragma unroll
    for (int t = 0; t < kD / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(acc_o[t][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * half) = v;
      }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16_d128(const void* qkv, int64_t ldqkv, void* o, int64_t ldo,
                                     int T, int heads, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kD);
  const dim3 grid((T + kBQ - 1) / kBQ, heads), block(256);
  hipLaunchKernelGGL(attn_fwd_bf16_d128, grid, block, 0, stream,
                     static_cast<const bf16*>(qkv), ldqkv, static_cast<bf16*>(o), ldo, T, heads,
                     scale_log2);
  return hipGetLastError();
}

}  // namespace tpk
