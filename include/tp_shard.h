/*
 * tp_shard.h -- C ABI of one tensor-parallel rank's share of a DiT block,
 * running on one AMD Instinct MI355X (gfx950).
 *
 * What it computes follows the Diffusers tensor-parallelism page
 * ("Paralelismo de tensor"; v0.43.0 Chinese twin "张量并行"), cited as
 * [TP page, §section]:
 *   - intro: each device holds a colwise or rowwise slice of each layer and
 *     computes a partial result; an AllReduce at the layer boundary combines
 *     the partials into the full output;
 *   - §"Colwise e rowwise" (列向和行向), style table: "colwise" shards output
 *     features (weight dim 0) and each rank computes a slice of the output
 *     (to_q, to_k, to_v, the FFN in-projection); "rowwise" shards input
 *     features (weight dim 1) and each rank computes a partial sum (to_out.0,
 *     the FFN out-projection); always colwise then rowwise, one AllReduce at
 *     the block boundary; colwise Q/K/V give each rank a subset of heads;
 *   - §"Projeções fundidas" (融合投影): a packed Linear is sharded block by
 *     block: [1, 1] for a SwiGLU gate/up projection, [1, 1, 1, 3, 3] for a
 *     fused Q, K, V, gate, up projection at mlp_ratio 3; a rowwise to_out may
 *     pack [inner_dim, mlp_hidden_dim];
 *   - style table, "rowwise_split_input", and §"O que deixar de fora": an
 *     independent projection whose input is replicated (a large AdaLN
 *     modulation projection reading the timestep embedding) is sharded by
 *     input features, each rank slicing its own copy of the input;
 *   - §"Restrições e verificação" (约束与验证): tp_degree divides the head
 *     count and each packed block on its own, checked before any weight is
 *     touched;
 *   - §"Limitações": unsupported combinations raise an error instead of
 *     silently doing something else.
 *
 * Context parallelism follows the Diffusers context-parallelism page
 * ("Paralelismo de contexto"), cited as [CP page, §section].
 *
 * Readings where the pages are silent: attention is softmax(Q K^T/sqrt(d)) V
 * per head, non-causal, unmasked; the MLP activation is GELU (tanh form) or
 * SwiGLU silu(gate) * up with the gate as the first packed half;
 * rank r owns heads [r*H/P, (r+1)*H/P) and the contiguous 1/P block of every
 * sharded feature dimension; the rowwise bias is added once, by the reduce.
 *
 * Conventions for every call below:
 *   - Matrices are row-major; "ld" arguments are row strides in ELEMENTS.
 *     Weights use the nn.Linear layout [out_features, in_features].
 *   - Device pointers must be 16-byte aligned and every row start too
 *     (ld * element size a multiple of 16 bytes).
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and is asynchronous: no call synchronises the host, except
 *     tp_block_shard_create (blocking host->device copies).
 *   - The calling thread's current HIP device must be the one the shard was
 *     created on.
 *   - The caller owns every activation, partial and output buffer, and the
 *     stream.  The library allocates device memory only in
 *     tp_block_shard_create (the rank's weight slices); no call allocates.
 *   - Every call validates all arguments before touching the device and
 *     returns a tp_status; on error nothing is enqueued and
 *     tp_last_error_detail() says why.  There is no fallback path.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stdint.h>

/* Symbols of this interface are the only ones the library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define TP_API __attribute__((visibility("default")))
#else
#define TP_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below is an int on the ABI.  In C++ it gets int32_t as its fixed
 * underlying type, so any int a C or Python caller passes is a value of the
 * type (the library rejects the ones it does not know); without a fixed type
 * an out-of-range value would be undefined behaviour in the library. */
#ifdef __cplusplus
#define TP_ENUM_INT : int32_t
#else
#define TP_ENUM_INT
#endif

typedef enum tp_status TP_ENUM_INT {
  TP_OK = 0,
  TP_ERR_ARG = -1,           /* NULL/misaligned pointer, bad size, wrong layer */
  TP_ERR_DIVISIBILITY = -2,  /* tp_degree does not divide heads / a packed block / ffn,
                                or num_heads*head_dim != hidden */
  TP_ERR_UNSUPPORTED = -3,   /* a valid request this library does not build */
  TP_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed */
  TP_ERR_OOM = -5,           /* device allocation failed */
  TP_ERR_IO = -6             /* a weight file is missing, unreadable or too short */
} tp_status;

typedef enum tp_dtype TP_ENUM_INT {
  TP_F32 = 0,                /* fp32 activations and weights */
  TP_BF16 = 1                /* bf16 activations and weights; fp32 accumulate */
} tp_dtype;

typedef enum tp_mlp_act TP_ENUM_INT {
  TP_MLP_GELU_TANH = 0,      /* h = GELU-tanh(x W_up^T + b_up); W_up is [F, D] */
  TP_MLP_SWIGLU = 1          /* h = silu(x W_gate^T + b_gate) * (x W_up^T + b_up); the
                                in-projection packs [W_gate; W_up] as one [2F, D]
                                weight (and [b_gate; b_up] as [2F]), sharded with
                                blocks [1, 1] */
} tp_mlp_act;

typedef enum tp_layer TP_ENUM_INT {
  TP_QKV = 0,                /* colwise: packed [Q_r; K_r; V_r], blocks [1, 1, 1] */
  TP_MLP_UP = 1,             /* colwise: FFN in-projection, fused bias + activation */
  TP_ATTN_OUT = 2,           /* rowwise: to_out.0 (attention out-projection) */
  TP_MLP_DOWN = 3,           /* rowwise: FFN out-projection */
  TP_BLOCK_OUT = 4,          /* rowwise, packed over [inner_dim, ffn]: [o_r | h_r] */
  TP_ADALN_MOD = 5           /* rowwise_split_input: AdaLN modulation projection */
} tp_layer;

/* UNSHARDED sizes of the block and this shard's place in the group.
 * num_heads == 0: no attention layers; ffn == 0: no MLP layers; mod_out == 0:
 * no modulation projection. */
typedef struct tp_block_config {
  int32_t tp_degree;         /* P >= 1 */
  int32_t rank;              /* 0 <= rank < P */
  int64_t hidden;            /* D */
  int64_t num_heads;         /* H; H * head_dim must equal D */
  int64_t head_dim;          /* d */
  int64_t ffn;               /* F */
  tp_dtype dtype;
  tp_mlp_act mlp_act;        /* 0 = GELU-tanh */
  int64_t mod_in;            /* input features of the AdaLN modulation projection (0: none) */
  int64_t mod_out;           /* its output features */
} tp_block_config;

/* UNSHARDED weights in HOST memory, element type = config dtype (bf16 as raw
 * 16-bit patterns), row-major nn.Linear layout.  Only this rank's slices are
 * read and copied to the device; the arrays are not retained.  Biases may be
 * NULL (zero).  The rowwise biases (b_o, b_down) are not sharded: they are
 * added once after the partial sum, by tp_partial_reduce.
 *
 * Packed checkpoints [TP page, §Projeções fundidas] need no copy: a fused
 * input projection W_in = [W_q; W_k; W_v; W_gate; W_up] (blocks [1, 1, 1, 3, 3]
 * at mlp_ratio 3 with SwiGLU) is passed as w_q = W_in, w_k = W_in + H*d*D,
 * w_v = W_in + 2*H*d*D, w_up = W_in + 3*H*d*D (elements; biases alike), and a
 * fused output projection W_out [D, H*d + F] over [inner_dim, mlp_hidden_dim]
 * as w_o = W_out, w_down = W_out + H*d with ld_o = ld_down = H*d + F. */
typedef struct tp_block_weights {
  const void *w_q, *w_k, *w_v;     /* [H*d, D] each */
  const void *b_q, *b_k, *b_v;     /* [H*d] each, nullable */
  const void *w_o;                 /* [D, H*d], row stride ld_o */
  const void *w_up;                /* [F, D]; SwiGLU: [2F, D] = [W_gate; W_up] */
  const void *b_up;                /* [F] (SwiGLU: [2F]), nullable */
  const void *w_down;              /* [D, F], row stride ld_down */
  int64_t ld_o;                    /* row stride of w_o in elements; 0 = H*d */
  int64_t ld_down;                 /* row stride of w_down in elements; 0 = F */
  const void *w_mod;               /* [mod_out, mod_in]; its bias goes to tp_partial_reduce */
} tp_block_weights;

typedef struct tp_block_shard tp_block_shard;  /* opaque; owns the device weight slices */

/* Validate `cfg` and `w`, then allocate and upload rank cfg->rank's slices on
 * the current HIP device [TP page, §Carregar um modelo fragmentado: each rank
 * reads only its own slice of each weight]:
 *   colwise (dim-0 rows):   W_qkv_r = [W_q[R_r,:]; W_k[R_r,:]; W_v[R_r,:]]  [3*D_r, D]
 *                           W_up_r  = W_up[C_r,:]                           [F_r, D]
 *                 (SwiGLU:  [W_gate[C_r,:]; W_up[C_r,:]] = rows C_r and F + C_r of
 *                           the packed [2F, D], stored with gate and up rows
 *                           interleaved in blocks of 32)
 *   rowwise (dim-1 cols):   W_o_r   = W_o[:, R_r]                           [D, D_r]
 *                           W_dn_r  = W_down[:, C_r]                        [D, F_r]
 *                           W_mod_r = W_mod[:, M_r]               [mod_out, mod_in/P]
 * with D_r = D/P, R_r = [r*D_r, (r+1)*D_r), F_r = F/P, C_r = [r*F_r, (r+1)*F_r),
 * M_r = [r*mod_in/P, (r+1)*mod_in/P).
 * Checks, in order, before any allocation [TP page, §Restrições e
 * verificação]: out != NULL (else TP_ERR_ARG); cfg, w != NULL; dtype and
 * mlp_act known; P >= 1 and 0 <= rank < P; D > 0, H >= 0, F >= 0, mod_in >= 0,
 * mod_out >= 0 (mod_in > 0 exactly when mod_out > 0), not all of H, F and
 * mod_out zero, d > 0 if H > 0 (TP_ERR_ARG); H*d == D, P | H, P | D (each
 * Q/K/V block), P | F (each gate/up block), P | mod_in (TP_ERR_DIVISIBILITY);
 * D, D_r, F_r, mod_in/P, mod_out multiples of 8, and of 32 for F_r with
 * SwiGLU (TP_ERR_UNSUPPORTED); the weights the enabled layers need are
 * non-NULL, ld_o is 0 or >= H*d, ld_down is 0 or >= F (TP_ERR_ARG).  On any error *out is set to NULL and nothing is allocated
 * (or everything allocated so far is freed). */
TP_API tp_status tp_block_shard_create(const tp_block_config *cfg, const tp_block_weights *w,
                                tp_block_shard **out);

/* One UNSHARDED weight in a raw file: the array exactly as in tp_block_weights
 * (row-major, config dtype, bf16 as 16-bit little-endian patterns), element
 * [0, 0] at byte `offset`.  path == NULL: the weight is absent. */
typedef struct tp_weight_file {
  const char *path;
  int64_t offset;
} tp_weight_file;

typedef struct tp_block_weight_files {
  tp_weight_file w_q, w_k, w_v, b_q, b_k, b_v, w_o, w_up, b_up, w_down, w_mod;
  int64_t ld_o, ld_down;     /* as in tp_block_weights (0 = dense) */
} tp_block_weight_files;

/* tp_block_shard_create reading the weights from files, shard-on-read
 * [TP page, §Carregar um modelo fragmentado: each rank reads only its own
 * slice of each weight, so no rank ever holds a full weight; §Desempenho de
 * carregamento: this is what bounds the per-rank CPU memory]: only rank
 * cfg->rank's byte ranges are read (pread), through one pinned host staging
 * buffer of staging_bytes (>= 1 MiB, else TP_ERR_ARG) split in two halves,
 * each copied to the device while the other is filled.  Host memory used:
 * the staging buffer plus the fp32 colwise bias (3*D_r + 2*F_r floats at
 * most), whatever the weights' size.  The resulting shard is identical to
 * tp_block_shard_create's for the same weights.  Same validation, in the same
 * order, before any file is opened; then TP_ERR_IO for a file that cannot be
 * opened or read or is too short. */
TP_API tp_status tp_block_shard_load(const tp_block_config *cfg, const tp_block_weight_files *files,
                                     int64_t staging_bytes, tp_block_shard **out);

/* Free the shard's device memory.  The caller must have synchronised every
 * stream that still uses it.  NULL is ignored. */
TP_API void tp_block_shard_destroy(tp_block_shard *shard);

/* Colwise projection [TP page, §Colwise e rowwise]:
 *   y[t, n] = act( sum_k x[t, k] * W_r[n, k] + b_r[n] ),  t < tokens, n < N_r
 * layer TP_QKV:    N_r = 3*D_r, columns [Q_r | K_r | V_r], act = identity;
 * layer TP_MLP_UP: N_r = F_r, act = GELU-tanh, or with SwiGLU
 *                  y[t, n] = silu(x W_gate_r[n]^T + b_gate_r[n]) * (x W_up_r[n]^T + b_up_r[n]).
 * x: device [tokens, D] (ldx >= D); y: device [tokens, N_r] (ldy >= N_r); both
 * in the config dtype.  tokens == 0 is a no-op; tokens < 0 is TP_ERR_ARG, as is
 * a layer that is not colwise or was not configured. */
TP_API tp_status tp_colwise_linear(tp_block_shard *shard, tp_layer layer, int64_t tokens,
                            const void *x, int64_t ldx, void *y, int64_t ldy, void *stream);

/* Both colwise projections of the block in one launch, over the packed
 * weight [W_qkv_r; W_up_r] ([TP page, §Projeções fundidas]: a fused
 * Q, K, V and MLP-in projection, sharded block by block):
 *   qkv[t, 0:3*D_r] = x W_qkv_r^T + b_qkv_r      (ldqkv >= 3*D_r)
 *   h  [t, 0:F_r]   = GELU-tanh(x W_up_r^T + b_up_r)  (ldh >= F_r)
 *                     (SwiGLU: silu(x W_gate_r^T + b_gate_r) * (x W_up_r^T + b_up_r);
 *                     with the [1, 1, 1, 3, 3]-style packing this is the whole
 *                     fused single-stream input projection)
 * Needs both attention and MLP configured (else TP_ERR_ARG).  Results are
 * identical to TP_QKV followed by TP_MLP_UP. */
TP_API tp_status tp_colwise_qkv_up(tp_block_shard *shard, int64_t tokens, const void *x, int64_t ldx,
                            void *qkv, int64_t ldqkv, void *h, int64_t ldh, void *stream);

/* Attention over this rank's H/P heads [TP page, §Colwise e rowwise: colwise
 * Q/K/V give each rank a subset of heads]: for local head j,
 *   o[:, j*d:(j+1)*d] = softmax(Q_j K_j^T / sqrt(d)) V_j   (non-causal, no mask)
 * with Q_j = qkv[:, j*d:(j+1)*d], K_j = qkv[:, D_r + j*d : ...],
 * V_j = qkv[:, 2*D_r + j*d : ...].  qkv: device [tokens, 3*D_r]
 * (ldqkv >= 3*D_r); o: device [tokens, D_r] (ldo >= D_r).  Softmax in fp32.
 * Built for bf16 and head_dim 128 only; other combinations return
 * TP_ERR_UNSUPPORTED.  Needs attention configured (else TP_ERR_ARG).
 * o must not overlap qkv. */
TP_API tp_status tp_attn_heads(tp_block_shard *shard, int64_t tokens, const void *qkv, int64_t ldqkv,
                        void *o, int64_t ldo, void *stream);

/* Attention of this rank's heads for the queries of one packed qkv buffer
 * against the keys and values of another -- one step of Ring Attention
 * [CP page, §Ring Attention: each rank attends its queries to the K/V block
 * it holds, then passes the block on], or one key split of a long
 * attention.  For local head j (d = 128):
 *   s      = Q_j K_j^T / sqrt(d)  over the kv_tokens keys of the block
 *   lse[t * ld_lse + j]  = log sum_k exp(s[t][k])            (natural log)
 *   o[t, j*d:(j+1)*d]    = sum_k exp(s[t][k] - lse) V_j[k]   (fp32, normalised)
 * Q_j = q_qkv[:, j*d : (j+1)*d] (only the Q columns [0, D_r) are read; ldq >=
 * D_r); K_j, V_j = columns D_r + j*d and 2*D_r + j*d of kv_qkv (ldkv >=
 * 3*D_r): both are packed [tokens, 3*D_r] buffers as tp_colwise_linear writes
 * them, or row ranges of one.  o: device fp32 [q_tokens, D_r], ldo >= D_r;
 * lse: device fp32, 4-byte aligned, ld_lse >= H/P.  q_tokens == 0 is a no-op;
 * kv_tokens must be >= 1.  bf16 and head_dim 128 only (TP_ERR_UNSUPPORTED);
 * o and lse must not overlap each other or the inputs.  tp_attn_merge
 * combines the blocks. */
TP_API tp_status tp_attn_heads_block(tp_block_shard *shard, int64_t q_tokens, const void *q_qkv,
                                     int64_t ldq, int64_t kv_tokens, const void *kv_qkv,
                                     int64_t ldkv, float *o, int64_t ldo, float *lse,
                                     int64_t ld_lse, void *stream);

/* tp_attn_heads with the keys cut into n_splits contiguous ranges
 * [floor(z*T/n_splits), floor((z+1)*T/n_splits)) processed in ONE launch, so
 * a short sequence over few heads still gives the GPU enough workgroups; each
 * range z writes its partial result like tp_attn_heads_block:
 *   o_parts + z * o_part_stride    fp32 [tokens, D_r], row stride ldo
 *   lse_parts + z * lse_part_stride fp32 [tokens, H/P], row stride ld_lse
 * (strides in elements; the parts must not overlap each other or qkv).
 * tp_attn_merge over the n_splits parts gives tp_attn_heads' result.
 * 1 <= n_splits <= 16 (else TP_ERR_ARG / TP_ERR_UNSUPPORTED) and
 * n_splits <= tokens; bf16 and head_dim 128 only. */
TP_API tp_status tp_attn_heads_split(tp_block_shard *shard, int64_t tokens, const void *qkv,
                                     int64_t ldqkv, int32_t n_splits, float *o_parts, int64_t ldo,
                                     int64_t o_part_stride, float *lse_parts, int64_t ld_lse,
                                     int64_t lse_part_stride, void *stream);

/* tp_attn_heads_block with the block's keys cut into n_splits contiguous
 * ranges [floor(z*kv_tokens/n_splits), floor((z+1)*kv_tokens/n_splits)) in
 * ONE launch -- one Ring Attention step [CP page, §Ring Attention] whose
 * query and key chunks are too short to fill the GPU in one piece.  Range z
 * writes its (o, lse) like tp_attn_heads_block at
 *   o_parts + z * o_part_stride     fp32 [q_tokens, D_r], row stride ldo
 *   lse_parts + z * lse_part_stride fp32 [q_tokens, H/P], row stride ld_lse
 * (strides in elements, o_part_stride a multiple of 4; the parts must not
 * overlap each other or the inputs).  The ranges are disjoint key blocks, so
 * tp_attn_merge over them (with the parts of the other ring steps) gives the
 * attention over all keys.  1 <= n_splits <= 16 (else TP_ERR_ARG /
 * TP_ERR_UNSUPPORTED), n_splits <= kv_tokens when q_tokens > 0; n_splits == 1
 * is tp_attn_heads_block.  tp_attn_split_hint(shard, q_tokens) gives a split
 * count that fills the GPU. */
TP_API tp_status tp_attn_heads_block_split(tp_block_shard *shard, int64_t q_tokens,
                                           const void *q_qkv, int64_t ldq, int64_t kv_tokens,
                                           const void *kv_qkv, int64_t ldkv, int32_t n_splits,
                                           float *o_parts, int64_t ldo, int64_t o_part_stride,
                                           float *lse_parts, int64_t ld_lse,
                                           int64_t lse_part_stride, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): tp_attn_heads_split
 * followed by tp_attn_merge in one call, writing tp_attn_heads' result
 * o[tokens, D_r] (bf16, ldo >= D_r) with the n_splits partial outputs and
 * log-sum-exps held in the library's own device scratch array instead of
 * caller buffers.  It allocates nothing and calls no allocating routine.
 * The array is 64 MiB, a file-scope device variable, so every GPU the
 * library runs on holds one copy until the process ends; a call needs
 * n_splits * tokens * (D_r + H/P) * 4 bytes of it and larger requests fail
 * with TP_ERR_ARG (the detail text gives both sizes).  Every call on a GPU
 * uses that GPU's one array, whose contents the next call overwrites: calls
 * that overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  1 <= n_splits <= 16 (else TP_ERR_ARG /
 * TP_ERR_UNSUPPORTED), n_splits <= tokens; bf16 and head_dim 128 only; o
 * must not overlap qkv; tokens == 0 is a no-op. */
TP_API tp_status tp_attn_heads_split_noalloc(tp_block_shard *shard, int64_t tokens, const void *qkv,
                                             int64_t ldqkv, int32_t n_splits, void *o, int64_t ldo,
                                             void *stream);

/* Host-only query: the n_splits (1..4) at which tp_attn_heads_split over
 * `tokens` tokens fills the GPU with its long-sequence kernel -- 1 when
 * tp_attn_heads already does (or the shard has no attention, or tokens < 1).
 * A split count above 1 pays for the merge's extra pass only when this says so. */
TP_API int32_t tp_attn_split_hint(const tp_block_shard *shard, int64_t tokens);

/* Merge of partial attention results over disjoint key blocks (the
 * combination that makes a full ring cycle equal attention over the whole
 * sequence [CP page, §Ring Attention]), per (token t, head j):
 *   lse = log sum_i exp(lse_i[t, j]),  o[t, j*hd + c] = sum_i exp(lse_i - lse) o_i[t, j*hd + c]
 * o_parts / lse_parts: HOST arrays of n_parts DEVICE pointers (1 <= n_parts
 * <= 16, else TP_ERR_ARG below / TP_ERR_UNSUPPORTED above), each o_i fp32
 * [tokens, heads*head_dim] with row stride ldo_parts, each lse_i fp32 with row
 * stride ld_lse_parts >= heads.  o: device, o_dtype (TP_BF16 or TP_F32),
 * ldo >= heads*head_dim.  lse_out: device fp32 (row stride ld_lse_out >=
 * heads) or NULL.  head_dim a positive multiple of 4.  The outputs must not
 * overlap the inputs.  Shard-independent; tokens == 0 is a no-op. */
TP_API tp_status tp_attn_merge(const float *const *o_parts, const float *const *lse_parts,
                               int32_t n_parts, int64_t ldo_parts, int64_t ld_lse_parts,
                               int64_t tokens, int64_t heads, int64_t head_dim, void *o,
                               int64_t ldo, tp_dtype o_dtype, float *lse_out, int64_t ld_lse_out,
                               void *stream);

/* Rowwise projection, partial sum [TP page, §Colwise e rowwise]:
 *   partial[t, n] (+)= sum_k x_local[t, k] * W_r[n, k],  n < D, k < K_r   (no bias)
 * layer TP_ATTN_OUT:  K_r = D_r (x_local = o_r);
 * layer TP_MLP_DOWN:  K_r = F_r (x_local = h_r);
 * layer TP_BLOCK_OUT: K_r = D_r + F_r, x_local = [o_r | h_r], W_r = [W_o_r | W_dn_r]
 *                     (a packed rowwise to_out over [inner_dim, mlp_hidden_dim],
 *                     [TP page, §Projeções fundidas]); equals ATTN_OUT + MLP_DOWN.
 * x_local: device, config dtype, ldx >= K_r; partial: device fp32 [tokens, D],
 * ldp >= D.  accumulate = 0 stores, 1 adds to what partial holds. */
TP_API tp_status tp_rowwise_linear_partial(tp_block_shard *shard, tp_layer layer, int64_t tokens,
                                    const void *x_local, int64_t ldx, float *partial,
                                    int64_t ldp, int accumulate, void *stream);

/* "rowwise_split_input" partial [TP page, style table; §O que deixar de
 * fora]: the input is REPLICATED (every rank holds all of it) and the rank
 * slices its own input features from it:
 *   partial[t, n] (+)= sum_{k in K_r} x_full[t, k] * W[n, k]      (no bias)
 * layer TP_ADALN_MOD: x_full [rows, mod_in], K_r = M_r, partial [rows, mod_out];
 * layer TP_ATTN_OUT:  x_full [rows, H*d] (all heads' output), K_r = R_r, partial [rows, D];
 * layer TP_MLP_DOWN:  x_full [rows, F], K_r = C_r, partial [rows, D];
 * layer TP_BLOCK_OUT: x_full [rows, H*d + F] = [o | h], K_r = R_r and H*d + C_r
 *                     (the packed row blocks), partial [rows, D].
 * x_full: device, config dtype, ldx >= its width; partial: device fp32, ldp >=
 * its width; accumulate = 0 stores, 1 adds.  rows == 0 is a no-op.  Results
 * equal tp_rowwise_linear_partial on the sliced columns.  The summed partials
 * plus the bias (tp_partial_reduce) give the unsharded projection. */
TP_API tp_status tp_rowwise_split_input_partial(tp_block_shard *shard, tp_layer layer, int64_t rows,
                                                const void *x_full, int64_t ldx, float *partial,
                                                int64_t ldp, int accumulate, void *stream);

/* The two all-to-alls of Ulysses Attention [CP page, §Ulysses Attention],
 * simulated with all `degree` (= u) ranks' buffers on one device.  H heads of
 * head_dim d, W = (H / u) * d; rank r owns heads [r*H/u, (r+1)*H/u) after the
 * first all-to-all and tokens [r*n, (r+1)*n) before it (n = tokens_per_rank).
 *
 * tp_ulysses_seq_to_heads -- rank `rank`'s view after the first all-to-all:
 *   out[s*n + t, b*W + c] = chunks[s][t, b*H*d + rank*W + c]
 * for every source rank s < u, column block b < blocks (1: one tensor [n, H*d];
 * 3: a packed Q | K | V [n, 3*H*d], giving a packed [u*n, 3*W] buffer that
 * tp_attn_heads reads directly), t < n, c < W.  chunks: HOST array of u
 * DEVICE pointers, row stride ld_in >= blocks*H*d; out: device, ldo >= blocks*W.
 *
 * tp_ulysses_heads_to_seq -- rank `rank`'s view after the second all-to-all:
 *   out[t, r*W + c] = parts[r][rank*n + t, c]
 * parts: HOST array of u DEVICE pointers to [u*n, W] (ld_in >= W); out:
 * device [n, H*d], ldo >= H*d.
 *
 * Both: element type dtype; 1 <= degree <= 16 (TP_ERR_ARG / TP_ERR_UNSUPPORTED);
 * u must divide H (TP_ERR_DIVISIBILITY; the sequence divides by construction,
 * u*n tokens); W*element size a multiple of 16 bytes (TP_ERR_UNSUPPORTED);
 * pointers and rows 16-byte aligned; out must not overlap the inputs.  Exact
 * copies; tokens_per_rank == 0 is a no-op. */
TP_API tp_status tp_ulysses_seq_to_heads(const void *const *chunks, int32_t degree, int64_t ld_in,
                                         int64_t tokens_per_rank, int64_t heads, int64_t head_dim,
                                         int32_t blocks, int32_t rank, tp_dtype dtype, void *out,
                                         int64_t ldo, void *stream);
TP_API tp_status tp_ulysses_heads_to_seq(const void *const *parts, int32_t degree, int64_t ld_in,
                                         int64_t tokens_per_rank, int64_t heads, int64_t head_dim,
                                         int32_t rank, tp_dtype dtype, void *out, int64_t ldo,
                                         void *stream);

/* The layer-boundary AllReduce of the TP page's intro, on one GPU: all
 * simulated ranks' partials summed in rank order, then the rowwise biases:
 *   out[t, c] = ((partials[0][t, c] + partials[1][t, c]) + ...) + biases[0][c] + ...
 * in fp32.  partials: HOST array of n_partials DEVICE pointers, each fp32
 * [tokens, hidden] with row stride ldp; biases: HOST array of n_biases DEVICE
 * pointers to fp32 [hidden] (may be NULL when n_biases == 0); out: device
 * fp32, ldo >= hidden.  1 <= n_partials <= 16, 0 <= n_biases <= 4 (else
 * TP_ERR_UNSUPPORTED beyond, TP_ERR_ARG below); hidden a multiple of 4.  out
 * may alias partials[0] exactly (same pointer and stride), nothing else. */
TP_API tp_status tp_partial_reduce(const float *const *partials, int32_t n_partials, int64_t ldp,
                            const float *const *biases, int32_t n_biases, int64_t tokens,
                            int64_t hidden, float *out, int64_t ldo, void *stream);

/* Static text naming a status code. */
TP_API const char *tp_status_string(tp_status status);

/* Text describing the last non-OK status returned to the calling thread
 * (thread-local; valid until that thread's next call). */
TP_API const char *tp_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H */
