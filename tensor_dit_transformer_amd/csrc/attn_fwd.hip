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
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = a 32-key slab of K from LDS, B = the
//     wave's Q^T held in registers for the whole kernel).  In the 32x32
//     accumulator a lane owns one query column, so the running max / sum
//     of its query are lane-local (plus one exchange with lane ^ 32).
//   * Output is accumulated transposed too, O^T += V^T P^T: the bf16 P^T
//     B-operand is the score accumulator itself, converted in registers; the
//     V^T A-operand is read from row-major V with the transposing LDS read
//     ds_read_b64_tr_b16 (in each 16-lane group, source lane 4 r + c points
//     at V[k + r][d + 4 c] and lane i receives V[k + e][d + i], e = 0..3).
//   * K and V tiles of 64 keys go global -> LDS directly into LDS rows of 256
//     bytes with an XOR chunk swizzle that keeps both the K reads and the
//     transposed V reads conflict-free.
//   * Softmax in the exp2 domain; the accumulator is rescaled only when a row
//     max outgrows the running reference by a slack, and the row max itself
//     is taken only for a tile whose weights, computed against the current
//     reference, lift a lane's row sum by more than a guard (any score past
//     the slack does).  Keys past T get -inf (last tile only); query rows
//     past T are clamped on load and not stored.
//   * Two kernels.  Short query sets: 4 waves of 32 queries per workgroup,
//     two workgroups per CU, two waves per SIMD.  Everything else: 4 waves
//     of 64 queries (one wave per SIMD, one workgroup per CU), in which each
//     wave interleaves the score MFMAs of the next tile, the PV MFMAs of the
//     previous one and the softmax of the current one (description below).
//   * Queries and keys/values may come from different tensors and lengths
//     (a K/V block of a longer sequence, the Ring Attention step of the
//     Diffusers context-parallelism page): the block form stores the
//     normalised output in fp32 and the natural log-sum-exp of the scaled
//     scores, lse = ln 2 * (m + log2 l), for the merge.
#include "tp_kernels.h"

#include <type_traits>

namespace tpk {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;            // head dim
constexpr int kBKV = 64;           // keys per tile
constexpr int kRowChunks = kD / 8; // 16-byte chunks per K or V row (256 bytes)

// LDS position of 16-byte chunk c of K/V tile row r: c ^ f(r), rows being
// 256 bytes (all 64 banks), so a chunk's banks depend on its position only.
// f is a bijection on 16 consecutive rows (conflict-free K reads: 16 lanes
// read one chunk of 16 rows) with f(4 a + b) = 4 b + a: a transposed V read
// serves 32 lanes at once, two 16-lane groups each reading 4 aligned rows at
// chunks {2 j, 2 j + 1} and {2 j + 2, 2 j + 3}; XOR with {0, 4, 8, 12} (+ a
// constant) sends the two groups to disjoint halves of the banks.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// x of lane l ^ 32: one v_permlane32_swap (lanes 32-63 of the first operand
// trade places with lanes 0-31 of the second) instead of an LDS permute.
__device__ __forceinline__ float other_half(float x, int half) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(half ? r[0] : r[1]);
}

// Slack (log2 domain) the running max may trail the true row max before the
// accumulator is rescaled.  Softmax is invariant to the reference value, so
// this only lets the unnormalised weights grow to at most 2^8; it skips almost
// every O rescale once the first tiles have set the max.
constexpr float kRescaleSlack = 8.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A score exceeds the reference by more than the slack exactly when its
// weight exp2(s * scale_log2 - m_ref) exceeds 2^8, which lifts its lane's
// row sum by more than 128 within the tile.  So each tile's weights are
// computed against the current reference first, and the row max -- needed
// only to apply the rule -- is taken only when some lane's sum grew by more
// than that, or on the first tile (m_ref still -inf, the same in every lane;
// its provisional weights are not finite).  Otherwise the weights and sum
// are already those the rule gives, bit for bit, since it would leave the
// reference unchanged.  After the first tile the reference is finite, so a
// weight is finite or +inf and the sum is never NaN: the check is an
// ordinary comparison (this file is built without NaN semantics).
constexpr float kSumGuard = 128.0f;

__device__ __forceinline__ bool sum_check(float m_ref, float l, float l_before) {
  return __builtin_amdgcn_ballot_w64(m_ref == -INFINITY || l > l_before + kSumGuard) != 0;
}

// Weight pair q (0..15) of a 64-key tile: scores (c, e), (c, e + 1) with
// c = q / 8, e = 2 (q % 8); packed to bf16 for the PV product, and the row
// sum adds the bf16 values the product uses.
__device__ __forceinline__ void weight_pair(const f32x16 (&s)[2], int q, float scale_log2, float m,
                                            float& l, bf16x8 (&pb)[2][2]) {
  const int c = q >> 3, e = 2 * (q & 7);
  const bf16x2 ones = {static_cast<bf16>(1.0f), static_cast<bf16>(1.0f)};
  const float p0 = __builtin_amdgcn_exp2f(fmaf(s[c][e], scale_log2, -m));
  const float p1 = __builtin_amdgcn_exp2f(fmaf(s[c][e + 1], scale_log2, -m));
  const bf16x2 pp = {static_cast<bf16>(p0), static_cast<bf16>(p1)};
  l = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l, false);
  pb[c][e >> 3][e & 7] = pp[0];
  pb[c][e >> 3][(e & 7) + 1] = pp[1];
}

// The reference rule, for a tile whose sum check fired: with the row max
// (this lane's 32 scores, then the other half-wave's), rescale when some
// row's max outgrew the reference by the slack -- the accumulator, the sum
// before the tile (l_before) and the tile's weights, recomputed against the
// new reference.  Otherwise l and pb stand.
__device__ __forceinline__ void reference_rule(const f32x16 (&s)[2], float scale_log2, int half,
                                               float& m_ref, float l_before, float& l,
                                               bf16x8 (&pb)[2][2], f32x16 (&acc_o)[kD / 32]) {
  float mloc = s[0][0];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, s[c][e]);
  mloc = fmaxf(mloc, other_half(mloc, half)) * scale_log2;
  if (__builtin_amdgcn_ballot_w64(mloc > m_ref + kRescaleSlack) == 0) return;
  const float m_new = fmaxf(m_ref, mloc);
  const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
  m_ref = m_new;
  l = l_before * alpha;
#pragma unroll
  for (int q = 0; q < 16; ++q) weight_pair(s, q, scale_log2, m_new, l, pb);
#pragma unroll
  for (int t = 0; t < kD / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc_o[t][e] *= alpha;
}

// Operands of one launch: head j's Q, K, V at columns j*128 of q, k, v.
// Key split z of kv_splits (the grid's z index; the pipelined kernel takes
// it from its work order) covers keys
// [floor(z Tkv / kv_splits), floor((z+1) Tkv / kv_splits)) -- never empty when
// Tkv >= kv_splits -- and writes its partial result at o + z o_split,
// lse + z lse_split.
struct AttnIO {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  int64_t ldq, ldkv;
  int Tq, Tkv, kv_splits;
  void* o;          // bf16 output, or fp32 with LSE
  int64_t ldo, o_split;
  float* lse;
  int64_t ld_lse, lse_split;
  float scale_log2;
};

// Epilogue of one wave's 32 queries (lane: query q = q0 + lane % 32, dims
// 32 t + 8 (e / 4) + 4 half + (e % 4)): normalise by the row sum, store bf16,
// or fp32 plus the row's log-sum-exp.
template <bool LSE>
__device__ __forceinline__ void store_rows(const AttnIO& a, int head, int z, int q, int half,
                                           const f32x16 (&acc_o)[kD / 32], float m_ref,
                                           float l_run) {
  const float l_tot = l_run + other_half(l_run, half);
  const float inv = 1.0f / l_tot;
  if (q >= a.Tq) return;
  if constexpr (LSE) {
    float* orow = static_cast<float*>(a.o) + z * a.o_split + (int64_t)q * a.ldo + head * kD;
#pragma unroll
    for (int t = 0; t < kD / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc_o[t][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * t + 8 * g + 4 * half) = v;
      }
    if (half == 0)
      a.lse[z * a.lse_split + (int64_t)q * a.ld_lse + head] =
          0.6931471805599453f * (m_ref + __log2f(l_tot));
  } else {
    bf16* orow = static_cast<bf16*>(a.o) + (int64_t)q * a.ldo + head * kD;
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

// One 64-key tile for one wave.  dma(j), j = 0..7, issues this wave's share
// of the next tile's global -> LDS loads; the calls are spread over the
// tile's 32 MFMAs (one per 4) so a load that waits at issue delays only a
// few MFMAs instead of the whole tile.
template <bool MASKED, class Dma>
__device__ __forceinline__ void attn_tile(const u32x4* __restrict__ sK, const u32x4* __restrict__ sV,
                                          const bf16x8 (&qf)[kD / 16], f32x16 (&acc_o)[kD / 32],
                                          float& m_ref, float& l_run, int key0, int T,
                                          float scale_log2, int lane, Dma&& dma) {
  const int half = lane >> 5, l32 = lane & 31;
  // S^T for keys 32 c .. 32 c + 31 of the tile (raw scores): A = K rows
  f32x16 s[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[c][e] = 0.0f;
    const int row = 32 * c + l32;
    const u32x4* kb = sK + row * kRowChunks;
    const int f = swz(row);
#pragma unroll
    for (int st = 0; st < kD / 16; ++st) {
      const bf16x8 ka = __builtin_bit_cast(bf16x8, kb[(2 * st + half) ^ f]);
      s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s[c], 0, 0, 0);
      if ((st & 3) == 3) {
        __builtin_amdgcn_sched_barrier(0);
        dma(2 * c + (st >> 2));
        __builtin_amdgcn_sched_barrier(0);
      }
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
  // weights against the current reference; the reference rule only when the
  // sum check fires (see kSumGuard)
  bf16x8 pb[2][2];
  const float l_before = l_run;
#pragma unroll
  for (int q = 0; q < 16; ++q) weight_pair(s, q, scale_log2, m_ref, l_run, pb);
  if (sum_check(m_ref, l_run, l_before))
    reference_rule(s, scale_log2, half, m_ref, l_before, l_run, pb, acc_o);
  // O^T += V^T P^T.  The P^T operand element j of this lane is key
  // 8 (j / 4) + 4 half + (j % 4) of each 16-key step; the V^T operand is read
  // transposed from row-major V: in each 16-lane group, source lane 4 r + cc
  // points at V[key0 + r][d0 + 4 cc], and lane i of the group receives
  // V[key0 + e][d0 + i], e = 0..3 -- keys 4 half .. + 3 (first read) and
  // 8 + 4 half .. + 3 (second read), dim = 32 t + (lane & 31).
  const int gi = lane & 15, r = gi >> 2, cc = gi & 3;
  const int keyA = 4 * half + r, keyB = keyA + 8;
  const int fA = swz(keyA), fB = swz(keyB);
  const int dsub = 16 * ((lane >> 4) & 1) + 4 * cc;      // dim within the 32-dim tile
  const int off8 = (dsub & 7) * 2;                        // byte offset in the chunk
#pragma unroll
  for (int t = 0; t < kD / 32; ++t) {
    const int lchunk = (32 * t + dsub) >> 3;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kb = 32 * c + 16 * u;
        const char* pa = reinterpret_cast<const char*>(sV + (kb + keyA) * kRowChunks + (lchunk ^ fA)) + off8;
        const char* pbp = reinterpret_cast<const char*>(sV + (kb + keyB) * kRowChunks + (lchunk ^ fB)) + off8;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(pa));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(pbp));
        const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc_o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), pb[c][u],
                                                          acc_o[t], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    dma(4 + t);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// NW waves x 32 queries per workgroup.  NW = 4: two workgroups per CU;
// NW = 8: one.  Either way <= 256 VGPRs per wave and two waves per SIMD, so
// one wave's softmax arithmetic overlaps another's matrix instructions.  The
// 8-wave form shares each K/V tile among 256 queries, halving the tile
// traffic per query; it is used when the sequence gives enough workgroups.
template <int NW, bool LSE>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
attn_fwd_bf16_d128(AttnIO a) {
  constexpr int BQ = 32 * NW;
  constexpr int PER_WAVE = 32 / NW;     // 1 KB K/V loads per wave per tile
  __shared__ u32x4 sK[2][kBKV * kRowChunks];
  __shared__ u32x4 sV[2][kBKV * kRowChunks];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * BQ + wave * 32;
  const int k0 = (int)((int64_t)blockIdx.z * a.Tkv / a.kv_splits);
  const int T = (int)((int64_t)(blockIdx.z + 1) * a.Tkv / a.kv_splits) - k0;   // >= 1
  const bf16* Qg = a.q + head * kD;
  const bf16* Kg = a.k + head * kD + (int64_t)k0 * a.ldkv;
  const bf16* Vg = a.v + head * kD + (int64_t)k0 * a.ldkv;
  const int half = lane >> 5, l32 = lane & 31;

  // Q^T operand: lane holds query q0 + l32, dims 16 s + 8 half .. +7
  bf16x8 qf[kD / 16];
  {
    const int64_t row = min(q0 + l32, a.Tq - 1);
#pragma unroll
    for (int s = 0; s < kD / 16; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(Qg + row * a.ldq + 16 * s + 8 * half);
  }

  // K and V tiles go global -> LDS directly.  Load n (0..31) of a tile fills
  // 1 KB = tile rows 4 (n & 15) .. + 3 of K (n < 16) or V; lane writes
  // physical chunk lane & 15 of its row, which holds logical chunk
  // (lane & 15) ^ swz(row).  Wave w issues loads w * PER_WAVE .. + PER_WAVE-1.
  auto load = [&](int kt, int buf, int n) {
    const int blk = n & 15;
    const int rr = 4 * blk + (lane >> 4);
    const int c = (lane & 15) ^ swz(rr);
    const int64_t row = min(kt * kBKV + rr, T - 1);
    const bf16* src = (n < 16 ? Kg : Vg) + row * a.ldkv + 8 * c;
    u32x4* dst = (n < 16 ? sK[buf] : sV[buf]) + 64 * blk;
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
  };

  f32x16 acc_o[kD / 32];
#pragma unroll
  for (int t = 0; t < kD / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc_o[t][e] = 0.0f;
  float m_ref = -INFINITY, l_run = 0.0f;

  const int nkt = (T + kBKV - 1) / kBKV;
  const int nfull = T / kBKV;  // tiles with every key valid
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) load(0, 0, wave * PER_WAVE + j);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    // slot j of 8 in the tile carries load j * PER_WAVE / 8 ... spread evenly
    auto dma = [&](int j) {
      if (!more) return;
      if constexpr (PER_WAVE == 8) {
        load(kt + 1, buf ^ 1, wave * 8 + j);
      } else {
        if ((j & 1) == 0) load(kt + 1, buf ^ 1, wave * PER_WAVE + (j >> 1));
      }
    };
    if (kt < nfull)
      attn_tile<false>(sK[buf], sV[buf], qf, acc_o, m_ref, l_run, kt * kBKV, T, a.scale_log2, lane, dma);
    else
      attn_tile<true>(sK[buf], sV[buf], qf, acc_o, m_ref, l_run, kt * kBKV, T, a.scale_log2, lane, dma);
    __syncthreads();  // tile kt + 1 landed (this wave's DMA) and every wave is done with buf
  }

  store_rows<LSE>(a, head, blockIdx.z, q0 + l32, half, acc_o, m_ref, l_run);
}

// ---------------------------------------------------------------------------
// Long query sets: 64 queries per wave, one wave per SIMD (4-wave workgroups
// of 256 queries, one per CU).  A K or V fragment read from LDS feeds two
// MFMAs (the wave's two 32-query blocks), half the LDS bytes per FLOP of 32
// queries per wave.
//
// Each wave's instruction stream alone has to keep the matrix core busy, so
// one key tile is one straight run of 32 slots, each holding one score MFMA,
// one PV MFMA and one weight pair:
//   * score MFMA p: key half 1 of tile kt (p < 16), then key half 0 of tile
//     kt + 1 (K fragment p / 2 of the 16, feeding both query blocks);
//   * PV MFMA p of tile kt - 1 (V fragment p / 2, query block p % 2);
//   * weight pair p of tile kt: blocks (query block 0, key half 0), (1, 0),
//     (0, 1), (1, 1) -- key half 1 of tile kt is complete by slot 16.
// A block's scores are thus consumed before the MFMAs of the next tile
// overwrite it, and one register set holds the scores of both tiles.
//
// A weight pair takes two FMAs (scale and reference), two exponentials, one
// pack and two adds.  The row sum adds the fp32 weights in two accumulators:
// the bf16 dot product the 4-wave kernel uses waits for the matrix core to
// drain before it issues, which left it idle for ~20 cycles per weight pair
// here.
//
// The MFMAs are issued from inline asm to pin their registers: the PV
// accumulators and Q in AGPRs (untouched by the vector code), the scores in
// VGPRs.  The compiler does not see these as MFMAs, so the fences below
// provide the wait states between an MFMA writing registers and any other
// instruction reading or rewriting them.
//
// Lazy rescale, as in the other kernels: a tile's weights are computed
// against the current reference, and only when some lane's row sum grew by
// more than kSumGuard does the rule run -- here at the end of the tile, from
// raw scores recomputed out of the tile still resident in LDS (its own
// registers hold the next tile's scores by then), after the tile's PV MFMAs
// have drained, so the accumulator rescale sees every earlier tile.

// Rescale slack of this kernel (log2 units) and the row-sum growth that
// triggers the rule.  Its rule recomputes a tile's scores, so it runs only
// when a weight may exceed 2^16 (any weight past the slack lifts its lane's
// sum by more than the guard); fp32 accumulators and bf16 weights hold such
// values with their full relative precision.
constexpr float kSlackQ64 = 16.0f;
constexpr float kGuardQ64 = 65536.0f;

// PV MFMA: accumulator in AGPRs.
__device__ __forceinline__ void mfma_pv(f32x16& acc, bf16x8 v, bf16x8 p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
}
// Score MFMAs: K fragment in VGPRs, Q in AGPRs, scores in VGPRs; the first
// k-step starts from zero.
__device__ __forceinline__ void mfma_s_zero(f32x16& s, bf16x8 k, bf16x8 q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_s_acc(f32x16& s, bf16x8 k, bf16x8 q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "a"(q));
}
// 24 wait states after the MFMAs writing these registers (an 8-pass MFMA
// needs fewer before a vector instruction may touch its result).
__device__ __forceinline__ void fence_s(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
// No wait states, only an ordering point: where the slot schedule already
// puts more than an MFMA's wait states of other instructions between the
// last MFMA writing these registers and the first instruction touching them.
__device__ __forceinline__ void order_s(f32x16& x, f32x16& y) {
  asm volatile("" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void fence_acc(f32x16 (&acc)[2][kD / 32]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                 "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]));
}
// After the vector writes of Q into AGPRs, before the first MFMA reads it.
__device__ __forceinline__ void fence_q(bf16x8 (&qf)[2][kD / 16]) {
  asm volatile("s_nop 7"
               : "+a"(qf[0][0]), "+a"(qf[0][1]), "+a"(qf[0][2]), "+a"(qf[0][3]),
                 "+a"(qf[0][4]), "+a"(qf[0][5]), "+a"(qf[0][6]), "+a"(qf[0][7]),
                 "+a"(qf[1][0]), "+a"(qf[1][1]), "+a"(qf[1][2]), "+a"(qf[1][3]),
                 "+a"(qf[1][4]), "+a"(qf[1][5]), "+a"(qf[1][6]), "+a"(qf[1][7]));
}
// After vector writes of P operands, before an MFMA reads them.
__device__ __forceinline__ void fence_p(bf16x8 (&p)[2][2][2]) {
  asm volatile("s_nop 1"
               : "+v"(p[0][0][0]), "+v"(p[0][0][1]), "+v"(p[0][1][0]), "+v"(p[0][1][1]),
                 "+v"(p[1][0][0]), "+v"(p[1][0][1]), "+v"(p[1][1][0]), "+v"(p[1][1][1]));
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over [base, base + bytes): per-lane offsets past it read as zero.
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from byte offset voff + soff of the buffer into LDS at
// dst + 16 lane (dst wave-uniform).
__device__ __forceinline__ void lds_dma(rsrc_t r, const u32x4* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)voff,
                                           (int)soff, 0, 0);
}

template <bool LSE>
__global__ void __launch_bounds__(256, 1)
attn_fwd_q64(AttnIO io) {
  constexpr int NSTAGE = 4;
  constexpr int BQ = 256;
  __shared__ u32x4 sK[NSTAGE][kBKV * kRowChunks];
  __shared__ u32x4 sV[NSTAGE][kBKV * kRowChunks];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-contiguous work order, as in the 8-wave kernel
  const int nqb = gridDim.x, nh = gridDim.y, nb = nqb * nh * gridDim.z;
  const int lin = blockIdx.x + nqb * (blockIdx.y + nh * blockIdx.z);
  const int xcd = lin & 7, per = nb >> 3, rem = nb & 7;
  const int w = xcd * per + min(xcd, rem) + (lin >> 3);
  const int qb = w % nqb, head = (w / nqb) % nh, z = w / (nqb * nh);
  const int q0 = qb * BQ + wave * 64;
  const int k0 = (int)((int64_t)z * io.Tkv / io.kv_splits);
  const int T = (int)((int64_t)(z + 1) * io.Tkv / io.kv_splits) - k0;   // >= 1
  const bf16* Qg = io.q + head * kD;
  const int half = lane >> 5, l32 = lane & 31;

  const float scale_log2 = io.scale_log2;
  // Q^T operands of the two query blocks (queries q0 + 32 a + l32)
  bf16x8 qf[2][kD / 16];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t row = min(q0 + 32 * a + l32, io.Tq - 1);
#pragma unroll
    for (int st = 0; st < kD / 16; ++st)
      qf[a][st] = *reinterpret_cast<const bf16x8*>(Qg + row * io.ldq + 16 * st + 8 * half);
  }
  fence_q(qf);

  const int nkt = (T + kBKV - 1) / kBKV;
  const int nfull = T / kBKV;
  const bool partial = nfull < nkt;
  // Loads of a tile: 32 of 1 KB (4 rows); wave w issues 8, all of K (w < 2)
  // or all of V, rows 32 (w & 1) + 4 j + (lane >> 4).  A whole tile's loads
  // take the tile's start as a scalar offset.  Only tiles below nfull are
  // loaded that way: the partial last tile puts its whole offset in the
  // per-lane register, with rows past key T clamped to row T - 1 (finite data,
  // whose scores are masked to -inf, so their weights are 0), and tiles past
  // the last are not loaded.  No load leaves the split's rows [0, T).
  const uint32_t ldkv2 = (uint32_t)io.ldkv * 2;
  const bf16* base = (wave < 2 ? io.k : io.v) + head * kD + (int64_t)k0 * io.ldkv;
  const rsrc_t rs = buffer_rsrc(base, (uint32_t)(T - 1) * ldkv2 + kD * 2);
  uint32_t loff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rr = 32 * (wave & 1) + 4 * j + (lane >> 4);
    loff[j] = (uint32_t)rr * ldkv2 + 16 * ((lane & 15) ^ swz(rr));
  }
  const uint32_t tile_bytes = (uint32_t)kBKV * ldkv2;
  auto load = [&](int kt, int stage, int j) {   // kt < nfull
    u32x4* dst = (wave < 2 ? sK[stage] : sV[stage]) + 64 * (8 * (wave & 1) + j);
    lds_dma(rs, dst, loff[j], (uint32_t)kt * tile_bytes);
  };
  auto load_any = [&](int kt, int stage, int j) {   // any kt >= 0
    if (kt < nfull) {
      load(kt, stage, j);
    } else if (kt < nkt) {
      const int rr = 32 * (wave & 1) + 4 * j + (lane >> 4);
      const int row = min(kt * kBKV + rr, T - 1);
      u32x4* dst = (wave < 2 ? sK[stage] : sV[stage]) + 64 * (8 * (wave & 1) + j);
      lds_dma(rs, dst, (uint32_t)row * ldkv2 + 16 * ((lane & 15) ^ swz(rr)), 0);
    }
  };

  // K operand of key half c, k-step st: rows 32 c + l32, dims 16 st + 8 half
  auto kread = [&](const u32x4* __restrict__ sKb, int c, int st) {
    const int row = 32 * c + l32;
    return __builtin_bit_cast(bf16x8, sKb[row * kRowChunks + ((2 * st + half) ^ swz(row))]);
  };
  // V^T operand of key step cu (16 keys), dim block t: two transposing reads
  const int gi = lane & 15, r = gi >> 2, cc = gi & 3;
  const int keyA = 4 * half + r, keyB = keyA + 8;
  const int fA = swz(keyA), fB = swz(keyB);
  const int dsub = 16 * ((lane >> 4) & 1) + 4 * cc;
  const int off8 = (dsub & 7) * 2;
  auto vread = [&](const u32x4* __restrict__ sVb, int cu, int t) {
    const int lchunk = (32 * t + dsub) >> 3;
    const int kb = 32 * (cu >> 1) + 16 * (cu & 1);
    const char* pa = reinterpret_cast<const char*>(sVb + (kb + keyA) * kRowChunks + (lchunk ^ fA)) + off8;
    const char* pbp = reinterpret_cast<const char*>(sVb + (kb + keyB) * kRowChunks + (lchunk ^ fB)) + off8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pa));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pbp));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  f32x16 s[2][2];   // scores, [query block][key half]
  // keys past T get -inf (last tile only)
  auto mask_half = [&](int kt, int c) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kt * kBKV + 32 * c + 8 * (e >> 2) + 4 * half + (e & 3);
        if (key >= T) s[a][c][e] = -INFINITY;
      }
  };

  f32x16 acc_o[2][kD / 32];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < kD / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[a][t][e] = 0.0f;
  float m_ref[2], l_run[2] = {0.0f, 0.0f};   // references in log2 units of the scaled scores
  bf16x8 kf[3], vf[3];
  bf16x8 pA[2][2][2], pB[2][2][2];

  // row max of query block a over the raw scores in s[a] (both lane halves),
  // scaled to log2 units
  auto row_max = [&](int a) {
    float m = s[a][0][0];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, s[a][c][e]);
    return fmaxf(m, other_half(m, half)) * scale_log2;
  };

  // Prologue: tiles 0 and 1 resident, raw scores of tile 0; the references
  // are their row maxima.
#pragma unroll
  for (int j = 0; j < 8; ++j) load_any(0, 0, j);
#pragma unroll
  for (int j = 0; j < 8; ++j) load_any(1, 1, j);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int st = 0; st < kD / 16; ++st)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 k = kread(sK[0], c, st);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        if (st == 0) mfma_s_zero(s[a][c], k, qf[a][0]);
        else mfma_s_acc(s[a][c], k, qf[a][st]);
      }
    }
  fence_s(s[0][0], s[0][1]);
  fence_s(s[1][0], s[1][1]);
  if (nkt == 1 && partial) {
    mask_half(0, 0);
    mask_half(0, 1);
  }
  m_ref[0] = row_max(0);
  m_ref[1] = row_max(1);
  kf[0] = kread(sK[0], 1, 0);
  kf[1] = kread(sK[0], 1, 1);

  // The reference rule for tile kt, after its sum check fired (see above).
  auto rule = [&](int kt, const u32x4* __restrict__ sKc, const u32x4* __restrict__ sKn, bool masked,
                  const float (&lb)[2], float (&l)[2], bf16x8 (&pcur)[2][2][2]) {
    // the last score MFMAs of the tile (into s[.][0]) land before these
    // registers take anything else
    fence_s(s[0][0], s[0][1]);
    fence_s(s[1][0], s[1][1]);
    fence_acc(acc_o);
#pragma unroll
    for (int st = 0; st < kD / 16; ++st)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 k = kread(sKc, c, st);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          if (st == 0) mfma_s_zero(s[a][c], k, qf[a][0]);
          else mfma_s_acc(s[a][c], k, qf[a][st]);
        }
      }
    fence_s(s[0][0], s[0][1]);
    fence_s(s[1][0], s[1][1]);
    if (masked) {
      mask_half(kt, 0);
      mask_half(kt, 1);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float mloc = row_max(a);
      if (__builtin_amdgcn_ballot_w64(mloc > m_ref[a] + kSlackQ64) == 0) continue;
      const float m_new = fmaxf(m_ref[a], mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_ref[a] - m_new);
      m_ref[a] = m_new;
      float la = lb[a] * alpha, lo = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int c = q >> 3, e = 2 * (q & 7);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[a][c][e], scale_log2, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[a][c][e + 1], scale_log2, -m_new));
        pcur[a][c][e >> 3][e & 7] = static_cast<bf16>(p0);
        pcur[a][c][e >> 3][(e & 7) + 1] = static_cast<bf16>(p1);
        la += p0;
        lo += p1;
      }
      l[a] = la + lo;
      // one accumulator at a time, each back in its AGPRs before the next
#pragma unroll
      for (int t = 0; t < kD / 32; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[a][t][e] *= alpha;
        asm volatile("" : "+a"(acc_o[a][t]));
      }
    }
    fence_acc(acc_o);
    // raw scores of S(kt + 1) key half 0 again
#pragma unroll
    for (int st = 0; st < kD / 16; ++st) {
      const bf16x8 k = kread(sKn, 0, st);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        if (st == 0) mfma_s_zero(s[a][0], k, qf[a][0]);
        else mfma_s_acc(s[a][0], k, qf[a][st]);
      }
    }
    // the next tile reads these right after its barrier
    fence_s(s[0][0], s[1][0]);
  };

  // Tile kt.  On entry: s[.][0] holds the raw scores of S(kt) key half 0,
  // kf[0..1] the first two K fragments of its key half 1 and
  // vf[0..1] the first two V fragments of tile kt - 1.  With whole_c true
  // the caller guarantees that tile kt + 2 is a whole tile (kt + 2 < nfull).
  auto step = [&](int kt, auto stage_c, bool has_prev, bool masked, bf16x8 (&pprev)[2][2][2],
                  bf16x8 (&pcur)[2][2][2], auto whole_c) {
    constexpr int J = decltype(stage_c)::value;
    constexpr bool WHOLE = decltype(whole_c)::value;
    const int cur = J >= 0 ? J : kt % NSTAGE;
    const u32x4* __restrict__ sKc = sK[cur];
    const u32x4* __restrict__ sKn = sK[(cur + 1) % NSTAGE];
    const u32x4* __restrict__ sVp = sV[(cur + 3) % NSTAGE];
    // this wave's loads of tile kt + 1 landed, then every wave's; every wave
    // is also done with tile kt - 2, whose stage the loads below refill
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // key half 0's last score MFMAs were in the previous tile's slots 30 and
    // 31 (the prologue and the rescale rule end with a fence instead)
    order_s(s[0][0], s[1][0]);
    if (masked) mask_half(kt, 0);
    const float lb[2] = {l_run[0], l_run[1]};
    float l[2] = {l_run[0], l_run[1]}, l2[2] = {0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      // score MFMA
      {
        const int st = (p & 15) >> 1, a = p & 1, c = p < 16 ? 1 : 0;
        const bf16x8 k = kf[(p >> 1) % 3];
        if (st == 0) mfma_s_zero(s[a][c], k, qf[a][0]);
        else mfma_s_acc(s[a][c], k, qf[a][st]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (p == 16) {
        // key half 1's last score MFMAs were in slots 14 and 15, at least a
        // slot of other instructions ago (tests/test_isa_hazards.py checks
        // the distance on every path)
        order_s(s[0][1], s[1][1]);
        if (masked) mask_half(kt, 1);
      }
      const int wa = (p >> 3) & 1, q = (p & 7) + 8 * (p >> 4);
      const int wc = q >> 3, we = 2 * (q & 7);
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[wa][wc][we], scale_log2, -m_ref[wa]));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[wa][wc][we + 1], scale_log2, -m_ref[wa]));
      __builtin_amdgcn_sched_barrier(0);
      // PV MFMA of tile kt - 1
      if (has_prev) {
        const int f = p >> 1, a = p & 1, cu = f >> 2, t = f & 3;
        mfma_pv(acc_o[a][t], vf[f % 3], pprev[a][cu >> 1][cu & 1]);
        if (a == 1 && f + 2 < 16) vf[(f + 2) % 3] = vread(sVp, (f + 2) >> 2, (f + 2) & 3);
      }
      // the 8 loads of tile kt + 2 in the even slots 0-14, one per two
      // slots; they land before the next tile's barrier waits on them
      if (p < 16 && (p & 1) == 0) {
        if constexpr (WHOLE) load(kt + 2, (cur + 2) % NSTAGE, p >> 1);
        else load_any(kt + 2, (cur + 2) % NSTAGE, p >> 1);
      }
      // the K fragment two ahead, in the even slots after the PV MFMA (the
      // odd slots read V there)
      if ((p & 1) == 0) {
        const int nf = (p >> 1) + 2;
        if (nf < 16) kf[nf % 3] = nf < 8 ? kread(sKc, 1, nf) : kread(sKn, 0, nf - 8);
      }
      __builtin_amdgcn_sched_barrier(0);
      pcur[wa][wc][we >> 3][we & 7] = static_cast<bf16>(e0);
      pcur[wa][wc][we >> 3][(we & 7) + 1] = static_cast<bf16>(e1);
      l[wa] += e0;
      l2[wa] += e1;
      // keeps the sums in their slots (sunk, they would queue up at the end)
      asm volatile("" : "+v"(l[wa]), "+v"(l2[wa]));
      __builtin_amdgcn_sched_barrier(0);
    }
    l[0] += l2[0];
    l[1] += l2[1];
    const bool fire =
        __builtin_amdgcn_ballot_w64(l[0] > lb[0] + kGuardQ64 || l[1] > lb[1] + kGuardQ64) != 0;
    if (__builtin_expect(fire, 0)) rule(kt, sKc, sKn, masked, lb, l, pcur);
    l_run[0] = l[0];
    l_run[1] = l[1];
    // the first operands of the next tile (both resident since this tile's barrier)
    kf[0] = kread(sKn, 1, 0);
    kf[1] = kread(sKn, 1, 1);
    vf[0] = vread(sV[cur], 0, 0);
    vf[1] = vread(sV[cur], 0, 1);
  };

  using Stage0 = std::integral_constant<int, 0>;
  using Stage1 = std::integral_constant<int, 1>;
  using Stage2 = std::integral_constant<int, 2>;
  using Stage3 = std::integral_constant<int, 3>;
  using StageR = std::integral_constant<int, -1>;
  using Whole = std::true_type;
  using Any = std::false_type;
  // tile t's weights go to pA when t is even, pB when odd; the unrolled loop
  // loads up to tile kt + 5, so it runs while that is a whole tile
  step(0, Stage0{}, false, nkt == 1 && partial, pB, pA, Any{});
  int kt = 1;
  for (; kt + 5 < nfull; kt += 4) {
    step(kt, Stage1{}, true, false, pA, pB, Whole{});
    step(kt + 1, Stage2{}, true, false, pB, pA, Whole{});
    step(kt + 2, Stage3{}, true, false, pA, pB, Whole{});
    step(kt + 3, Stage0{}, true, false, pB, pA, Whole{});
  }
  for (; kt + 1 < nkt; kt += 2) {
    step(kt, StageR{}, true, false, pA, pB, Any{});
    step(kt + 1, StageR{}, true, kt + 1 == nkt - 1 && partial, pB, pA, Any{});
  }
  if (kt < nkt) step(kt, StageR{}, true, partial, pA, pB, Any{});
  // the last iteration's scores of a tile past the end land before their
  // registers are reused
  fence_s(s[0][0], s[1][0]);
  // PV of the last tile
  {
    const bool odd = (nkt - 1) & 1;
    bf16x8 pl[2][2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int u = 0; u < 2; ++u) pl[a][c][u] = odd ? pB[a][c][u] : pA[a][c][u];
    fence_p(pl);
    const u32x4* __restrict__ sVb = sV[(nkt - 1) % NSTAGE];
#pragma unroll
    for (int f = 0; f < 16; ++f) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int cu = f >> 2;
        mfma_pv(acc_o[a][f & 3], vf[f % 3], pl[a][cu >> 1][cu & 1]);
      }
      if (f + 2 < 16) vf[(f + 2) % 3] = vread(sVb, (f + 2) >> 2, (f + 2) & 3);
    }
  }
  fence_acc(acc_o);
  // loads of tiles past the end may still be in flight
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int a = 0; a < 2; ++a)
    store_rows<LSE>(io, head, z, q0 + 32 * a + l32, half, acc_o[a], m_ref[a], l_run[a]);
}

}  // namespace

namespace {

// Workgroups of 256 queries: the 64-query-per-wave kernel runs when they
// number at least kQ64MinWorkgroups and its 32-bit buffer offsets reach every
// key row; otherwise 128-query workgroups of the 4-wave kernel, two per CU.
// Key splits are chosen (attn_split_hint) to reach kPipeMinWorkgroups.
constexpr long kPipeMinWorkgroups = 192;
constexpr long kQ64MinWorkgroups = 32;

long pipe_workgroups(int Tq, int heads, int splits) {
  return (long)((Tq + 255) / 256) * heads * splits;
}

template <bool LSE>
void launch_io(const AttnIO& io, int heads, int splits, hipStream_t stream) {
  const bool offsets32 = ((int64_t)io.Tkv + 4 * kBKV) * io.ldkv * 2 < ((int64_t)1 << 31);
  if (pipe_workgroups(io.Tq, heads, splits) >= kQ64MinWorkgroups && offsets32) {
    const dim3 grid((io.Tq + 255) / 256, heads, splits), block(256);
    hipLaunchKernelGGL((attn_fwd_q64<LSE>), grid, block, 0, stream, io);
  } else {
    const dim3 grid((io.Tq + 127) / 128, heads, splits), block(256);
    hipLaunchKernelGGL((attn_fwd_bf16_d128<4, LSE>), grid, block, 0, stream, io);
  }
}

constexpr float kScaleLog2 = 1.4426950408889634f / 11.313708498984761f;  // log2(e) / sqrt(128)

}  // namespace

int attn_split_hint(int T, int heads) {
  if (pipe_workgroups(T, heads, 1) >= kPipeMinWorkgroups) return 1;
  for (int s = 2; s <= 4; ++s)
    if (pipe_workgroups(T, heads, s) >= kPipeMinWorkgroups && T >= s) return s;
  return 1;
}

hipError_t launch_attn_fwd_bf16_d128(const void* qkv, int64_t ldqkv, void* o, int64_t ldo,
                                     int T, int heads, hipStream_t stream) {
  const bf16* base = static_cast<const bf16*>(qkv);
  const int64_t Dr = (int64_t)heads * kD;
  const AttnIO io{base, base + Dr, base + 2 * Dr, ldqkv, ldqkv, T, T, 1, o, ldo, 0, nullptr, 0, 0,
                  kScaleLog2};
  launch_io<false>(io, heads, 1, stream);
  return hipGetLastError();
}

hipError_t launch_attn_block_bf16_d128(const AttnBlockArgs& a, hipStream_t stream) {
  const int splits = a.splits < 1 ? 1 : a.splits;
  if (a.Tkv < splits) return hipErrorInvalidValue;   // a split would be empty
  const AttnIO io{static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                  static_cast<const bf16*>(a.v), a.ldq, a.ldkv, a.Tq, a.Tkv, splits, a.o, a.ldo,
                  a.o_split, a.lse, a.ld_lse, a.lse_split, kScaleLog2};
  launch_io<true>(io, a.heads, splits, stream);
  return hipGetLastError();
}

}  // namespace tpk
