"""Seeded synthetic inputs for the tensor-parallel DiT block shard.

This module only draws random tensors and states workload shapes.  It holds
none of the block's arithmetic: both the CPU oracle (``oracle/``) and the HIP
path (``tensor_dit_transformer_amd``) consume what it returns, and neither is
imported here.

Distributions and draw order (one ``numpy.random.default_rng(seed)`` stream,
float32 ``standard_normal`` scaled by the stated standard deviation):

    x ~ N(0, 1)                                [T, D]
    W_q, W_k, W_v ~ N(0, 0.02)                 [D, D]   (nn.Linear [out, in])
    b_q, b_k, b_v ~ N(0, 0.01)                 [D]
    W_o ~ N(0, 0.02)                           [D, H*d]
    b_o ~ N(0, 0.01)                           [D]
    W_up ~ N(0, 0.02)                          [F, D]  (SwiGLU: [2F, D] = [W_gate; W_up])
    b_up ~ N(0, 0.01)                          [F]     (SwiGLU: [2F])
    W_dn ~ N(0, 0.02)                          [D, F]
    b_dn ~ N(0, 0.01)                          [D]
    c ~ N(0, 1)                                [R, D]   (replicated conditioning input)
    W_mod ~ N(0, 0.02)                         [N_mod, D]
    b_mod ~ N(0, 0.01)                         [N_mod]

Tensors a workload lacks (no attention, or no MLP) are skipped, not drawn.
For bf16 workloads every array is rounded to bfloat16 with torch's
round-to-nearest-even conversion, so the GPU and the oracle read identical
bits; the arrays are handed out as float32 numpy arrays holding those
bf16-representable values, plus the raw uint16 bit patterns for upload.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

WEIGHT_STD = 0.02
BIAS_STD = 0.01

# Names in the order they are drawn.
DRAW_ORDER = ("x", "w_q", "w_k", "w_v", "b_q", "b_k", "b_v", "w_o", "b_o",
              "w_up", "b_up", "w_dn", "b_dn", "c", "w_mod", "b_mod")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one block-shard workload (unsharded sizes)."""
    name: str
    tokens: int
    hidden: int
    num_heads: int      # 0: no attention half
    head_dim: int
    ffn: int            # 0: no MLP half
    tp_degree: int
    dtype: str          # "f32" or "bf16"
    description: str = ""
    mlp_act: str = "gelu_tanh"   # or "swiglu" (packed gate/up, blocks [1, 1])
    mod_rows: int = 0            # rows R of the replicated modulation input
    mod_out: int = 0             # N_mod, output features of the modulation projection
    cp: str = ""                 # context-parallel attention only: "ring" or "ulysses"
    cp_degree: int = 0

    @property
    def has_attn(self) -> bool:
        return self.num_heads > 0

    @property
    def has_mlp(self) -> bool:
        return self.ffn > 0

    @property
    def has_mod(self) -> bool:
        return self.mod_out > 0


# The five workloads of the tensor-parallel block shard.  Token count 4608 is
# 4096 image latents plus 512 text tokens; 16384 is a video-like latent.
C1 = Workload("mlp_f32_T64_D256_F1024_P2", 64, 256, 0, 0, 1024, 2, "f32",
              "fp32 MLP block, both ranks of tp_degree 2")
C2 = Workload("mlp_bf16_T4608_D3072_F12288_P4", 4608, 3072, 0, 0, 12288, 4, "bf16",
              "bf16 DiT MLP shard, one rank of tp_degree 4")
C3 = Workload("attn_bf16_T4608_D3072_H24_P4", 4608, 3072, 24, 128, 0, 4, "bf16",
              "bf16 DiT attention shard, one rank of tp_degree 4")
C4 = Workload("block_bf16_T4608_D6144_H48_F18432_P4", 4608, 6144, 48, 128, 18432, 4,
              "bf16", "bf16 wide DiT block shard, one rank of tp_degree 4")
C5_P4 = Workload("block_bf16_T16384_D6144_H48_F18432_P4", 16384, 6144, 48, 128, 18432,
                 4, "bf16", "bf16 full block, all 4 rank shards then partial reduce")
C5_P2 = dataclasses.replace(C5_P4, name="block_bf16_T16384_D6144_H48_F18432_P2",
                            tp_degree=2,
                            description="bf16 full block, both rank shards then partial reduce")

# Single-stream block with fused projections and a SwiGLU MLP at mlp_ratio 3:
# the input projection packs Q, K, V, gate, up (blocks [1, 1, 1, 3, 3]) and the
# output projection reads [attention output | hidden] (row blocks [6144, 18432]).
C6 = Workload("single_swiglu_bf16_T4608_D6144_H48_F18432_P4", 4608, 6144, 48, 128, 18432, 4,
              "bf16", "bf16 single-stream SwiGLU block shard, one rank of tp_degree 4",
              mlp_act="swiglu")
C7 = Workload("single_swiglu_bf16_T16384_D6144_H48_F18432_P4", 16384, 6144, 48, 128, 18432,
              4, "bf16", "bf16 single-stream SwiGLU block, all 4 rank shards then partial reduce",
              mlp_act="swiglu")

# AdaLN modulation projection of the wide block (shift, scale and gate for
# attention and MLP: 6 x 6144 outputs) sharded "rowwise_split_input": every
# rank holds the replicated conditioning rows and a quarter of the input
# features.  8 rows: one conditioning vector per sample of a batch of 8.
C8 = Workload("adaln_mod_bf16_R8_D6144_N36864_P4", 0, 6144, 0, 0, 0, 4, "bf16",
              "bf16 AdaLN modulation projection, all 4 rank shards then partial reduce",
              mod_rows=8, mod_out=36864)

# Context-parallel attention of the CP page's benchmark model size (a
# 1024x1024 FLUX.1-like image: 4096 latents + 512 text tokens, 24 heads of
# 128) across 4 simulated GPUs; the attention input is a seeded packed qkv
# (std 1.5, like the projections' output), drawn by cp_qkv.
C9 = Workload("cp_ring_bf16_T4608_H24_R4", 4608, 3072, 24, 128, 0, 1, "bf16",
              "Ring Attention over 4 simulated GPUs", cp="ring", cp_degree=4)
C10 = Workload("cp_ulysses_bf16_T4608_H24_U4", 4608, 3072, 24, 128, 0, 1, "bf16",
               "Ulysses Attention over 4 simulated GPUs", cp="ulysses", cp_degree=4)

# Shard-on-read loading of the full block's weights (a 755 MB bf16
# checkpoint) by all 4 ranks, each reading only its slices.
C11 = Workload("load_block_bf16_D6144_H48_F18432_P4", 0, 6144, 48, 128, 18432, 4, "bf16",
               "every rank of tp_degree 4 loads its slices from one raw checkpoint file")

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5_P4, C5_P2, C6, C7, C8, C9, C10, C11)}


def cp_qkv(w: Workload, seed: int = 0, tokens: Optional[int] = None):
    """The packed [T, 3 H d] attention input of a context-parallel workload
    (values, bits)."""
    T = w.tokens if tokens is None else tokens
    return random_matrix((T, 3 * w.num_heads * w.head_dim), seed=seed, std=1.5)


def _shapes(w: Workload) -> Dict[str, tuple]:
    T, D, F = w.tokens, w.hidden, w.ffn
    HD = w.num_heads * w.head_dim
    shapes = {"x": (T, D)} if T > 0 else {}
    if w.has_attn:
        shapes.update(w_q=(HD, D), w_k=(HD, D), w_v=(HD, D),
                      b_q=(HD,), b_k=(HD,), b_v=(HD,),
                      w_o=(D, HD), b_o=(D,))
    if w.has_mlp:
        U = 2 * F if w.mlp_act == "swiglu" else F
        shapes.update(w_up=(U, D), b_up=(U,), w_dn=(D, F), b_dn=(D,))
    if w.has_mod:
        shapes.update(c=(w.mod_rows, D), w_mod=(w.mod_out, D), b_mod=(w.mod_out,))
    return shapes


def _std(name: str) -> float:
    if name in ("x", "c"):
        return 1.0
    return WEIGHT_STD if name.startswith("w_") else BIAS_STD


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of a float32 array, rounded by torch
    (round-to-nearest-even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """float32 values of bfloat16 bit patterns (exact widening)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    values: Dict[str, np.ndarray]          # float32 arrays (bf16-representable if bf16)
    bits: Optional[Dict[str, np.ndarray]]  # uint16 bf16 patterns (bf16 workloads only)

    def __getitem__(self, k: str) -> np.ndarray:
        return self.values[k]


def make_inputs(w: Workload, seed: int = 0, tokens: Optional[int] = None) -> Inputs:
    """Draw every tensor of workload ``w`` from ``default_rng(seed)``.

    ``tokens`` overrides the token count (the weights are unchanged in shape and
    drawn identically only when ``tokens`` equals ``w.tokens``)."""
    if tokens is not None:
        w = dataclasses.replace(w, tokens=tokens)
    rng = np.random.default_rng(seed)
    shapes = _shapes(w)
    values: Dict[str, np.ndarray] = {}
    for name in DRAW_ORDER:
        if name not in shapes:
            continue
        a = rng.standard_normal(shapes[name], dtype=np.float32)
        if _std(name) != 1.0:
            a *= np.float32(_std(name))
        values[name] = a
    bits = None
    if w.dtype == "bf16":
        bits = {k: bf16_bits(v) for k, v in values.items()}
        values = {k: bits_to_f32(b) for k, b in bits.items()}
    return Inputs(w, values, bits)


def random_matrix(shape, seed: int, std: float = 1.0, dtype: str = "bf16"):
    """A seeded N(0, std^2) matrix for single-kernel cases (a rowwise GEMM fed a
    seeded activation, attention fed a seeded packed QKV, the reduce fed seeded
    partials).  Returns (float32 values, uint16 bits or None)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == "bf16":
        b = bf16_bits(a)
        return bits_to_f32(b), b
    return a, None


def sample_rows(tokens: int, n: int, seed: int = 1) -> np.ndarray:
    """Sorted distinct row indices for row-sampled checks; always includes the
    first and last row (the ragged tail)."""
    rng = np.random.default_rng(seed)
    n = min(n, tokens)
    rows = set(rng.choice(tokens, size=n, replace=False).tolist())
    rows.update({0, tokens - 1})
    return np.array(sorted(rows), dtype=np.int64)


# Structured packed qkv [T, 3 H d] for the attention edge cases (input
# construction only; both sides read the same bf16 bits):
#   "growing":  per head a random unit direction u; query row i has component
#               beta_i * 4 along u (beta_i cycles 1, 0, 0.5, -1 with the row),
#               key t has component 24 * (t // 64) along u, so for beta = 1 a
#               row's scores rise by about 12 log2 units from one 64-key tile
#               to the next (6 for beta = 0.5; flat or falling otherwise);
#               plus N(0, 0.5^2) noise on q and N(0, 1) on k and v.
#   "dominant": every query has component 4 along u; one key, at row
#               5 T / 8 + 17, is 80 u, over 20 log2 units above every other
#               score of every query; the rest N(0, 1.5^2).
#   "zero_q":   Q = 0 (every score 0), K and V N(0, 1.5^2).
EDGE_KINDS = ("growing", "dominant", "zero_q")


def attention_edge_qkv(T: int, heads: int, kind: str, seed: int = 0, head_dim: int = 128):
    if kind not in EDGE_KINDS:
        raise ValueError(kind)
    rng = np.random.default_rng(seed)
    W = heads * head_dim
    u = rng.standard_normal((heads, head_dim)).astype(np.float64)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    u = u.reshape(W)
    if kind == "growing":
        q = 0.5 * rng.standard_normal((T, W))
        k = rng.standard_normal((T, W))
        v = rng.standard_normal((T, W))
        beta = np.array([1.0, 0.0, 0.5, -1.0])[np.arange(T) % 4]
        q += 4.0 * beta[:, None] * u[None, :]
        k += 24.0 * (np.arange(T) // 64)[:, None] * u[None, :]
    elif kind == "dominant":
        q = 0.5 * rng.standard_normal((T, W)) + 4.0 * u[None, :]
        k = 1.5 * rng.standard_normal((T, W))
        v = 1.5 * rng.standard_normal((T, W))
        k[dominant_key(T)] = 80.0 * u
    else:
        q = np.zeros((T, W))
        k = 1.5 * rng.standard_normal((T, W))
        v = 1.5 * rng.standard_normal((T, W))
    a = np.concatenate([q, k, v], axis=1).astype(np.float32)
    b = bf16_bits(a)
    return bits_to_f32(b), b


def dominant_key(T: int) -> int:
    """Row of the dominant key in attention_edge_qkv(kind="dominant")."""
    return min(T - 1, 5 * T // 8 + 17)
