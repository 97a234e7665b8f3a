"""Plain float64 oracle of one tensor-parallel rank's share of a DiT block.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU-baseline leg).

Sources (the Diffusers tensor-parallelism pages, Portuguese "Paralelismo de
tensor" and its v0.43.0 Chinese twin "张量并行"; cited below as [TP page]):

* intro: each device holds a colwise or rowwise slice of each layer and computes
  a partial result; an AllReduce at the layer boundary forms the full output.
* §"Colwise e rowwise" (列向和行向), style table: "colwise" shards output
  features (weight dim 0) and each rank computes a slice of the output;
  "rowwise" shards input features (weight dim 1) and each rank computes a
  partial sum.  The pair is always colwise then rowwise, with one AllReduce at
  the block boundary.  Colwise Q/K/V give each rank a subset of heads.
* §"Projeções fundidas" (融合投影): a packed Linear is sharded block by block,
  never by one plain slice across the concatenation.
* §"Restrições e verificação" (约束与验证): tp_degree divides the head count;
  every packed block is divisible by tp_degree on its own; both are checked
  before any weight is touched.

Readings where the pages are silent (all stated again in the design notes):
* attention is softmax(Q K^T / sqrt(d)) V per head, non-causal, no mask;
* the MLP activation is GELU with the tanh approximation;
* a rank owns the contiguous head block [r*H/P, (r+1)*H/P) and the contiguous
  feature blocks [r*N/P, (r+1)*N/P) of each sharded dimension;
* the rowwise bias is added once, after the partial sum;
* the DiT block is y = attn_branch(x) + mlp_branch(x) (both branches read x),
  the single-stream layout implied by a packed rowwise to_out over
  [inner_dim, mlp_hidden_dim] (§"Projeções fundidas");
* bf16 workloads store x, weights, biases, qkv_r, o_r and h_r as bfloat16
  (round to nearest even); partials and y stay unrounded.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "ShardConfigError", "to_bf16_rne", "linear", "gelu_tanh", "softmax_rows",
    "attention_head", "attention_heads", "check_config", "colwise_range",
    "rowwise_range", "packed_colwise_rows", "shard_weights", "rank_forward",
    "block_unsharded", "partial_reduce", "rowwise_bias",
    "attention_rows", "colwise_rows_sampled",
]


class ShardConfigError(ValueError):
    """A configuration the TP page's constraints reject.  ``kind`` is
    'divisibility' or 'argument'."""

    def __init__(self, kind: str, msg: str):
        super().__init__(msg)
        self.kind = kind


# --------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------

def to_bf16_rne(a) -> np.ndarray:
    """Round to bfloat16 (8-bit significand), round-to-nearest-even, returned
    as float64.  The value is first rounded to float32 (numpy, RNE), then the
    low 16 bits of the float32 pattern are rounded away: add 0x7FFF plus the
    lowest kept bit, truncate.  NaN stays NaN; finite values that overflow
    become +-inf, as for any RNE narrowing."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    out = np.where(np.isnan(f), np.float32(np.nan), out)
    return out.astype(np.float64)


# --------------------------------------------------------------------------
# The three operations of the block
# --------------------------------------------------------------------------

def linear(x, w, b=None) -> np.ndarray:
    """nn.Linear with weight in [out_features, in_features] layout:
    y[t, n] = sum_k x[t, k] * w[n, k] (+ b[n])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = x @ w.T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)
    return y


_GELU_C = math.sqrt(2.0 / math.pi)
_GELU_A = 0.044715


def gelu_tanh(u) -> np.ndarray:
    """GELU, tanh approximation (Hendrycks & Gimpel):
    0.5 * u * (1 + tanh(sqrt(2/pi) * (u + 0.044715 u^3)))."""
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(_GELU_C * (u + _GELU_A * u * u * u)))


def softmax_rows(s) -> np.ndarray:
    """Row softmax, with the row maximum subtracted before exp."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_head(q, k, v, scale: Optional[float] = None) -> np.ndarray:
    """One head: softmax(q k^T * scale) v, non-causal and unmasked; scale
    defaults to 1/sqrt(head_dim)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return softmax_rows((q @ k.T) * scale) @ v


def attention_heads(q, k, v, num_heads: int, head_dim: int) -> np.ndarray:
    """Multi-head attention over feature-major [T, num_heads*head_dim] Q, K, V:
    head h is the column block [h*d, (h+1)*d) of each, and its output lands in
    the same column block of the result.  [TP page, §Colwise e rowwise: colwise
    Q/K/V give each rank a subset of heads, so attention is head-local.]"""
    out = np.zeros((q.shape[0], num_heads * head_dim), dtype=np.float64)
    for h in range(num_heads):
        c = slice(h * head_dim, (h + 1) * head_dim)
        out[:, c] = attention_head(q[:, c], k[:, c], v[:, c])
    return out


# --------------------------------------------------------------------------
# Sharding: constraints and slices
# --------------------------------------------------------------------------

def check_config(tp_degree: int, rank: int, hidden: int, num_heads: int,
                 head_dim: int, ffn: int) -> None:
    """[TP page, §Restrições e verificação] tp_degree must divide the head
    count, and each packed block (Q, K, V of width H*d, and the FFN width) must
    be divisible by tp_degree on its own; checked before any weight is used.
    Argument sanity (positive sizes, rank in range, H*d == hidden) is checked
    first."""
    if tp_degree < 1 or not (0 <= rank < tp_degree):
        raise ShardConfigError("argument", f"rank {rank} not in [0, {tp_degree})")
    if hidden <= 0 or num_heads < 0 or ffn < 0 or (num_heads > 0 and head_dim <= 0):
        raise ShardConfigError("argument", "sizes must be positive")
    if num_heads == 0 and ffn == 0:
        raise ShardConfigError("argument", "neither attention nor MLP")
    if num_heads > 0:
        if num_heads * head_dim != hidden:
            raise ShardConfigError("divisibility",
                                   f"num_heads*head_dim={num_heads * head_dim} != hidden={hidden}")
        if num_heads % tp_degree:
            raise ShardConfigError("divisibility",
                                   f"tp_degree {tp_degree} does not divide {num_heads} heads")
        for name, width in (("q", hidden), ("k", hidden), ("v", hidden)):
            if width % tp_degree:
                raise ShardConfigError("divisibility", f"packed block {name} not divisible")
    if ffn > 0 and ffn % tp_degree:
        raise ShardConfigError("divisibility", f"tp_degree {tp_degree} does not divide ffn {ffn}")


def colwise_range(n_out: int, tp_degree: int, rank: int) -> slice:
    """[TP page, §Colwise e rowwise] colwise: this rank's contiguous block of
    output features = rows of weight dim 0."""
    n = n_out // tp_degree
    return slice(rank * n, (rank + 1) * n)


def rowwise_range(n_in: int, tp_degree: int, rank: int) -> slice:
    """[TP page, §Colwise e rowwise] rowwise: this rank's contiguous block of
    input features = columns of weight dim 1."""
    n = n_in // tp_degree
    return slice(rank * n, (rank + 1) * n)


def packed_colwise_rows(block_sizes: Sequence[int], tp_degree: int, rank: int) -> np.ndarray:
    """[TP page, §Projeções fundidas] dim-0 row indices a rank takes from a
    packed Linear whose output is the concatenation of blocks of the given
    absolute sizes: its own slice of every block, in block order."""
    rows: List[np.ndarray] = []
    start = 0
    for size in block_sizes:
        if size % tp_degree:
            raise ShardConfigError("divisibility", f"packed block {size} not divisible by {tp_degree}")
        s = colwise_range(size, tp_degree, rank)
        rows.append(np.arange(start + s.start, start + s.stop))
        start += size
    return np.concatenate(rows)


def shard_weights(wts: Dict[str, np.ndarray], tp_degree: int, rank: int,
                  num_heads: int, head_dim: int) -> Dict[str, np.ndarray]:
    """One rank's weight slices.  Colwise (dim 0): the packed Q|K|V weight with
    blocks [1, 1, 1] and the MLP up-projection.  Rowwise (dim 1): the attention
    out-projection and the MLP down-projection.  Rowwise biases are not
    sharded (added once after the sum).  [TP page, §Colwise e rowwise;
    §Projeções fundidas]"""
    out: Dict[str, np.ndarray] = {}
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    if "w_q" in wts:
        HD = num_heads * head_dim
        w_qkv = np.concatenate([f64(wts["w_q"]), f64(wts["w_k"]), f64(wts["w_v"])], axis=0)
        b_qkv = np.concatenate([f64(wts["b_q"]), f64(wts["b_k"]), f64(wts["b_v"])])
        rows = packed_colwise_rows([HD, HD, HD], tp_degree, rank)
        out["w_qkv"] = w_qkv[rows]
        out["b_qkv"] = b_qkv[rows]
        out["w_o"] = f64(wts["w_o"])[:, rowwise_range(HD, tp_degree, rank)]
    if "w_up" in wts:
        F = wts["w_up"].shape[0]
        c = colwise_range(F, tp_degree, rank)
        out["w_up"] = f64(wts["w_up"])[c]
        out["b_up"] = f64(wts["b_up"])[c]
        out["w_dn"] = f64(wts["w_dn"])[:, rowwise_range(F, tp_degree, rank)]
    return out


# --------------------------------------------------------------------------
# One rank's forward, the reduce, and the unsharded block
# --------------------------------------------------------------------------

def rank_forward(x, wts: Dict[str, np.ndarray], tp_degree: int, rank: int,
                 num_heads: int, head_dim: int, bf16: bool) -> Dict[str, np.ndarray]:
    """Everything rank ``rank`` computes, in order:

    qkv_r   = x W_qkv_r^T + b_qkv_r                  colwise  [T, 3*D_r]
    o_r     = attention over the rank's H/P heads     [T, D_r]
    h_r     = gelu_tanh(x W_up_r^T + b_up_r)          colwise  [T, F_r]
    p_attn  = o_r W_o_r^T                            rowwise partial [T, D]
    p_mlp   = h_r W_dn_r^T                           rowwise partial [T, D]
    p_block = p_attn + p_mlp                          (= [o_r | h_r] [W_o_r | W_dn_r]^T)

    [TP page, intro and §Colwise e rowwise.]  Rowwise partials carry no bias.
    With ``bf16`` the stored activations qkv_r, o_r, h_r are rounded to
    bfloat16 (inputs are assumed bf16-representable already)."""
    rnd = to_bf16_rne if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    s = shard_weights(wts, tp_degree, rank, num_heads, head_dim)
    x = np.asarray(x, dtype=np.float64)
    res: Dict[str, np.ndarray] = {}
    parts = []
    if "w_qkv" in s:
        Hr = num_heads // tp_degree
        Dr = Hr * head_dim
        qkv = rnd(linear(x, s["w_qkv"], s["b_qkv"]))
        o = rnd(attention_heads(qkv[:, :Dr], qkv[:, Dr:2 * Dr], qkv[:, 2 * Dr:], Hr, head_dim))
        res["qkv_r"] = qkv
        res["o_r"] = o
        res["p_attn"] = linear(o, s["w_o"])
        parts.append(res["p_attn"])
    if "w_up" in s:
        h = rnd(gelu_tanh(linear(x, s["w_up"], s["b_up"])))
        res["h_r"] = h
        res["p_mlp"] = linear(h, s["w_dn"])
        parts.append(res["p_mlp"])
    res["p_block"] = parts[0] if len(parts) == 1 else parts[0] + parts[1]
    return res


def rowwise_bias(wts: Dict[str, np.ndarray]) -> np.ndarray:
    """The bias added once after the rowwise sum: b_o, b_dn, or both."""
    b = None
    for k in ("b_o", "b_dn"):
        if k in wts:
            v = np.asarray(wts[k], dtype=np.float64)
            b = v if b is None else b + v
    return b


def partial_reduce(partials: Sequence[np.ndarray], bias=None) -> np.ndarray:
    """The layer-boundary AllReduce, on one host: y = sum_r partial_r (+ bias),
    summed in rank order.  [TP page, intro; §Colwise e rowwise: one AllReduce
    at the block boundary.]"""
    y = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        y = y + np.asarray(p, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


def block_unsharded(x, wts: Dict[str, np.ndarray], num_heads: int, head_dim: int,
                    bf16: bool) -> Dict[str, np.ndarray]:
    """The same block on one device, no sharding: the result tensor parallelism
    must reproduce.  [TP page, §Restrições e verificação: compare single-device
    output with the tensor-parallel output.]"""
    rnd = to_bf16_rne if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    x = np.asarray(x, dtype=np.float64)
    res: Dict[str, np.ndarray] = {}
    ys = []
    if "w_q" in wts:
        q = rnd(linear(x, wts["w_q"], wts["b_q"]))
        k = rnd(linear(x, wts["w_k"], wts["b_k"]))
        v = rnd(linear(x, wts["w_v"], wts["b_v"]))
        o = rnd(attention_heads(q, k, v, num_heads, head_dim))
        res.update(q=q, k=k, v=v, o=o)
        res["y_attn"] = linear(o, wts["w_o"], wts["b_o"])
        ys.append(res["y_attn"])
    if "w_up" in wts:
        g = rnd(gelu_tanh(linear(x, wts["w_up"], wts["b_up"])))
        res["g"] = g
        res["y_mlp"] = linear(g, wts["w_dn"], wts["b_dn"])
        ys.append(res["y_mlp"])
    res["y"] = ys[0] if len(ys) == 1 else ys[0] + ys[1]
    return res


# --------------------------------------------------------------------------
# Row-sampled pieces for full-size checks (same definitions, fewer rows)
# --------------------------------------------------------------------------

def colwise_rows_sampled(x_rows, w, b=None, gelu: bool = False, bf16: bool = True) -> np.ndarray:
    """A colwise projection evaluated only on some rows of x (each output row
    depends only on its own input row)."""
    y = linear(x_rows, w, b)
    if gelu:
        y = gelu_tanh(y)
    return to_bf16_rne(y) if bf16 else y


def attention_rows(q_rows, k, v, num_heads: int, head_dim: int) -> np.ndarray:
    """Attention for some query rows against all keys/values (each output row
    depends only on its own query row and on every key and value)."""
    return attention_heads(q_rows, k, v, num_heads, head_dim)
