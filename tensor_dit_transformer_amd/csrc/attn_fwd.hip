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
//   * 32 queries per wave, <= 256 VGPRs so two waves share each SIMD.  Short
//     sequences: 4-wave workgroups, two per CU.  Long sequences: the
//     software-pipelined form below, 8-wave workgroups sharing each K/V tile
//     among 256 queries, in which each wave overlaps the next tile's score
//     MFMAs with this tile's softmax.
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
//   * K and V tiles of 64 keys go global -> LDS directly
//     (global_load_lds_dwordx4) into LDS rows of 256 bytes with an XOR chunk
//     swizzle that keeps both the K reads and the transposed V reads
//     conflict-free; one barrier per tile.  The 4-wave kernel double-buffers
//     one tile ahead, the long-sequence kernel keeps four stages and fetches
//     three tiles ahead.
//   * Softmax runs in the exp2 domain with few vector instructions per
//     score: one FMA (scale folded in) and one exp2; the row sum is a bf16
//     dot2 over the packed weights; the accumulator is rescaled by
//     exp2(m_old - m_new) only when a row max outgrows the reference by 8
//     (log2 units).  The row max itself is taken only for a tile whose
//     weights, computed against the current reference, lift a lane's row
//     sum by more than 128 (any score past the slack does), so most tiles
//     skip it.  Keys past T get -inf (last tile only); query rows past T
//     are clamped on load and not stored.
//   * The long-sequence kernel's main loop covers four tiles per iteration,
//     one per LDS stage, so the stage offsets of its LDS reads are
//     instruction immediates rather than per-tile address arithmetic.
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
// Software-pipelined form for long query sets, launched as NW = 8 waves (two
// per SIMD, <= 256 VGPRs each) of NQ = 1 sub-tile of 32 queries.  (With NQ
// sub-tiles a K or V fragment read from LDS would feed NQ MFMAs, but the
// state of NQ = 2 does not fit the registers of two waves per SIMD, and at
// one wave per SIMD the compiler spills.)  Within key tile j a wave issues the
// score MFMAs of tile j+1 in the same straight-line block as the softmax of
// tile j, one MFMA before each slice of the softmax, so the matrix core and
// the vector ALU work at the same time inside one wave; then the PV MFMAs of
// tile j.  Four LDS stages: iteration j reads K of tile j+1
// and V of tile j, and fetches tile j+3 into the stage tile j-1 used, so
// every tile's loads have two iterations to land.  Loads past the last tile
// re-fetch the last tile (harmless, keeps the block branch-free), and the
// scores computed in the final iteration are discarded.
template <int N>
__device__ __forceinline__ void barrier_keep_newest_loads() {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int NQ, int NW, bool LSE>
__global__ void __launch_bounds__(64 * NW, 1)
attn_fwd_pipe(AttnIO io) {
  static_assert(NQ == 1, "one 32-query sub-tile per wave");
  constexpr int NSTAGE = 4;
  constexpr int BQ = NW * 32 * NQ;
  constexpr int PER_WAVE = 32 / NW;   // 1 KB loads per wave per tile
  __shared__ u32x4 sK[NSTAGE][kBKV * kRowChunks];
  __shared__ u32x4 sV[NSTAGE][kBKV * kRowChunks];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work order: workgroups are dispatched round-robin over the 8 XCDs (own
  // L2 each) in linear id order, so the linear id is renumbered to give each
  // XCD a contiguous run of (query block, head, key split) items, query block
  // fastest: the workgroups an XCD runs at once are query blocks of one or
  // two heads and share their K/V tiles in its L2.
  const int nqb = gridDim.x, nh = gridDim.y, nb = nqb * nh * gridDim.z;
  const int lin = blockIdx.x + nqb * (blockIdx.y + nh * blockIdx.z);
  const int xcd = lin & 7, per = nb >> 3, rem = nb & 7;
  const int w = xcd * per + min(xcd, rem) + (lin >> 3);
  const int qb = w % nqb, head = (w / nqb) % nh, z = w / (nqb * nh);
  const int q0 = qb * BQ + wave * 32 * NQ;
  const int k0 = (int)((int64_t)z * io.Tkv / io.kv_splits);
  const int T = (int)((int64_t)(z + 1) * io.Tkv / io.kv_splits) - k0;   // >= 1
  const bf16* Qg = io.q + head * kD;
  const bf16* Kg = io.k + head * kD + (int64_t)k0 * io.ldkv;
  const bf16* Vg = io.v + head * kD + (int64_t)k0 * io.ldkv;
  const float scale_log2 = io.scale_log2;
  const int half = lane >> 5, l32 = lane & 31;

  bf16x8 qf[NQ][kD / 16];
#pragma unroll
  for (int a = 0; a < NQ; ++a) {
    const int64_t row = min(q0 + 32 * a + l32, io.Tq - 1);
#pragma unroll
    for (int st = 0; st < kD / 16; ++st)
      qf[a][st] = *reinterpret_cast<const bf16x8*>(Qg + row * io.ldq + 16 * st + 8 * half);
  }

  const int nkt = (T + kBKV - 1) / kBKV;
  const int nfull = T / kBKV;   // tiles with every key valid
  // Load n (0..31) of tile kt: K rows (n < 16) or V rows 4 (n & 15) .. + 3;
  // wave w issues loads PER_WAVE w .. PER_WAVE (w + 1) - 1.  A load's
  // address is a wave-uniform tile base plus a loop-invariant per-lane 32-bit
  // offset (row within the tile, chunk); a partial last tile uses offsets
  // with its rows past T clamped to T - 1.
  uint32_t loff[PER_WAVE], loff_last[PER_WAVE];
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int n = PER_WAVE * wave + j;
    const int rr = 4 * (n & 15) + (lane >> 4);
    const int c = (lane & 15) ^ swz(rr);
    const int rlast = min(nfull * kBKV + rr, T - 1) - nfull * kBKV;
    loff[j] = (uint32_t)((int64_t)rr * io.ldkv * 2 + 16 * c);
    loff_last[j] = (uint32_t)((int64_t)rlast * io.ldkv * 2 + 16 * c);
  }
  const int64_t tile_bytes = (int64_t)kBKV * io.ldkv * 2;
  auto load_tile = [&](int kt, int buf) {   // buf = kt % NSTAGE
    const int tt = min(kt, nkt - 1);
    const bool full = tt < nfull;
    const int64_t toff = (int64_t)tt * tile_bytes;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int n = PER_WAVE * wave + j;
      const char* src = reinterpret_cast<const char*>(n < 16 ? Kg : Vg) + toff +
                        (full ? loff[j] : loff_last[j]);
      u32x4* dst = (n < 16 ? sK[buf] : sV[buf]) + 64 * (n & 15);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
    }
  };

  auto scores = [&](const u32x4* __restrict__ sKb, f32x16 (&s)[NQ][2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int a = 0; a < NQ; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[a][c][e] = 0.0f;
      const int row = 32 * c + l32;
      const u32x4* kb = sKb + row * kRowChunks;
      const int f = swz(row);
#pragma unroll
      for (int st = 0; st < kD / 16; ++st) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, kb[(2 * st + half) ^ f]);
#pragma unroll
        for (int a = 0; a < NQ; ++a)
          s[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[a][st], s[a][c], 0, 0, 0);
      }
    }
  };

  f32x16 acc_o[NQ][kD / 32];
#pragma unroll
  for (int a = 0; a < NQ; ++a)
#pragma unroll
    for (int t = 0; t < kD / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[a][t][e] = 0.0f;
  float m_ref[NQ], l_run[NQ];
#pragma unroll
  for (int a = 0; a < NQ; ++a) { m_ref[a] = -INFINITY; l_run[a] = 0.0f; }

  // V^T operand addressing (see attn_tile): per lane constants
  const int gi = lane & 15, r = gi >> 2, cc = gi & 3;
  const int keyA = 4 * half + r, keyB = keyA + 8;
  const int fA = swz(keyA), fB = swz(keyB);
  const int dsub = 16 * ((lane >> 4) & 1) + 4 * cc;
  const int off8 = (dsub & 7) * 2;

  // K operand of score MFMA i of a tile: key half c = i & 1, k-step
  // st = i >> 1, so neighbouring MFMAs feed different accumulators.
  auto kread = [&](const u32x4* __restrict__ sKb, int i) {
    const int row = 32 * (i & 1) + l32;
    return __builtin_bit_cast(bf16x8, sKb[row * kRowChunks + ((2 * (i >> 1) + half) ^ swz(row))]);
  };
  // V^T operand of PV MFMA (cu, t): keys 32 c + 16 u .. + 15 (cu = 2 c + u)
  // of dims 32 t .. + 31, two transposing reads.
  auto vread = [&](const u32x4* __restrict__ sVb, int cu, int t) {
    const int lchunk = (32 * t + dsub) >> 3;
    const int kb = 32 * (cu >> 1) + 16 * (cu & 1);
    const char* pa = reinterpret_cast<const char*>(sVb + (kb + keyA) * kRowChunks + (lchunk ^ fA)) + off8;
    const char* pbp = reinterpret_cast<const char*>(sVb + (kb + keyB) * kRowChunks + (lchunk ^ fB)) + off8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pa));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pbp));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // One key tile: s_cur holds the raw scores of tile kt; the scores of tile
  // kt + 1 go to s_nxt.  Score MFMA i (K read KPF MFMAs ahead) is followed by
  // slice i of the softmax of tile kt: slices 0-1 the row max, 2 the
  // reference update, 3-15 the exponentials, weights and row sum.  The
  // scheduling fences keep that order, so the matrix core and the vector ALU
  // of the wave work side by side.  Then the rare rescale of the accumulator
  // and the PV MFMAs, in (key block, dim block) order with the V reads two
  // key blocks ahead; the LDS pointers are __restrict__ so the compiler can
  // tell these reads from the LDS-bound loads in flight and adds no wait for
  // them (the vmcnt wait before each barrier orders every tile's loads before
  // its reads, and a tile's loads get two iterations to land).
  auto step = [&](int kt, auto stage_c, f32x16 (&s_cur)[NQ][2], f32x16 (&s_nxt)[NQ][2]) {
    // stage_c: kt % NSTAGE as a compile-time constant (the LDS addresses of
    // the tile's reads then fold into the instructions' offsets), or -1
    constexpr int J = decltype(stage_c)::value;
    const int cur = J >= 0 ? J : kt % NSTAGE;
    if (kt * kBKV + kBKV > T) {  // last, partial tile: mask keys past T
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt * kBKV + 32 * c + 8 * (e >> 2) + 4 * half + (e & 3);
          if (key >= T) s_cur[0][c][e] = -INFINITY;
        }
    }
    load_tile(kt + 3, (cur + 3) % NSTAGE);
    const u32x4* __restrict__ sKb = sK[(cur + 1) % NSTAGE];
    constexpr int KPF = 6;
    bf16x8 kf[16];
#pragma unroll
    for (int i = 0; i < KPF; ++i) kf[i] = kread(sKb, i);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) s_nxt[0][c][e] = 0.0f;
    // Score MFMAs 2j, 2j + 1, then weight pairs 2j, 2j + 1 of tile kt against
    // the current reference; the reference rule only when the sum check
    // fires (see kSumGuard), before the PV MFMAs.
    //
    // The two waves of a SIMD (w and w + 4) start each tile together at the
    // barrier, and the older one wins issue: it finishes the tile first and
    // then idles at the next barrier while the other finishes alone.  Waves
    // 4-7 therefore take the top issue priority for this phase (the one
    // with the vector work), which evens the two out.
    const float l_before = l_run[0];
    float l = l_before;
    bf16x8 pb[2][2];
    if (wave >= NW / 2) __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int i0 = 0; i0 < 16; i0 += 2) {
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) {
        s_nxt[0][i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[0][i >> 1], s_nxt[0][i & 1], 0, 0, 0);
        if (i + KPF < 16) kf[i + KPF] = kread(sKb, i + KPF);
      }
      __builtin_amdgcn_sched_barrier(0);
      weight_pair(s_cur[0], i0, scale_log2, m_ref[0], l, pb);
      weight_pair(s_cur[0], i0 + 1, scale_log2, m_ref[0], l, pb);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // the weights are used only after the check's branch; without this, IR
    // passes sink their computation into the PV block, away from the score
    // MFMAs it is interleaved with
    asm volatile("" :: "v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]), "v"(l));
    if (sum_check(m_ref[0], l, l_before))
      reference_rule(s_cur[0], scale_log2, half, m_ref[0], l_before, l, pb, acc_o[0]);
    l_run[0] = l;
    // O^T += V^T P^T
    const u32x4* __restrict__ sVb = sV[cur];
    bf16x8 vf[4][kD / 32];
#pragma unroll
    for (int cu = 0; cu < 2; ++cu)
#pragma unroll
      for (int t = 0; t < kD / 32; ++t) vf[cu][t] = vread(sVb, cu, t);
#pragma unroll
    for (int cu = 0; cu < 4; ++cu)
#pragma unroll
      for (int t = 0; t < kD / 32; ++t) {
        acc_o[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cu][t], pb[cu >> 1][cu & 1], acc_o[0][t], 0, 0, 0);
        if (cu + 2 < 4) vf[cu + 2][t] = vread(sVb, cu + 2, t);
      }
    barrier_keep_newest_loads<PER_WAVE>();
  };

  load_tile(0, 0);
  load_tile(1, 1);
  load_tile(2, 2);
  __syncthreads();
  f32x16 sa[NQ][2], sb[NQ][2];
  scores(sK[0], sa);
  // four tiles per iteration, one per LDS stage; the last nkt % 4 with the
  // stage computed at run time
  using Stage0 = std::integral_constant<int, 0>;
  using Stage1 = std::integral_constant<int, 1>;
  using Stage2 = std::integral_constant<int, 2>;
  using Stage3 = std::integral_constant<int, 3>;
  using StageR = std::integral_constant<int, -1>;
  int kt = 0;
  for (; kt + 3 < nkt; kt += 4) {
    step(kt, Stage0{}, sa, sb);
    step(kt + 1, Stage1{}, sb, sa);
    step(kt + 2, Stage2{}, sa, sb);
    step(kt + 3, Stage3{}, sb, sa);
  }
  for (; kt + 1 < nkt; kt += 2) {
    step(kt, StageR{}, sa, sb);
    step(kt + 1, StageR{}, sb, sa);
  }
  if (kt < nkt) step(kt, StageR{}, sa, sb);

#pragma unroll
  for (int a = 0; a < NQ; ++a)
    store_rows<LSE>(io, head, z, q0 + 32 * a + l32, half, acc_o[a], m_ref[a], l_run[a]);
}

}  // namespace

namespace {

// Long query sets: the software-pipelined form in 256-query workgroups (one
// per CU), when they cover at least three quarters of the 256 CUs;
// otherwise 128-query workgroups, two per CU.
// The pipelined kernel needs 256-query workgroups covering three quarters of
// the CUs.
constexpr long kPipeMinWorkgroups = 192;

long pipe_workgroups(int Tq, int heads, int splits) {
  return (long)((Tq + 255) / 256) * heads * splits;
}

template <bool LSE>
void launch_io(const AttnIO& io, int heads, int splits, hipStream_t stream) {
  if (pipe_workgroups(io.Tq, heads, splits) >= kPipeMinWorkgroups) {
    const dim3 grid((io.Tq + 255) / 256, heads, splits), block(512);
    hipLaunchKernelGGL((attn_fwd_pipe<1, 8, LSE>), grid, block, 0, stream, io);
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
