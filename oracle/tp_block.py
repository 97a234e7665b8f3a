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
  never by one plain slice across the concatenation; blocks [1, 1] for a
  SwiGLU gate/up projection with equal halves, [1, 1, 1, 3, 3] for a fused
  Q, K, V, gate, up projection at mlp_ratio 3, and stored row blocks
  [inner_dim, mlp_hidden_dim] for a rowwise output projection over the
  concatenated attention output and MLP hidden (the single-stream block).
* §"Restrições e verificação" (约束与验证): tp_degree divides the head count;
  every packed block is divisible by tp_degree on its own; both are checked
  before any weight is touched.

Readings where the pages are silent (all stated again in the design notes):
* attention is softmax(Q K^T / sqrt(d)) V per head, non-causal, no mask;
* the MLP activation is GELU with the tanh approximation, or SwiGLU
  silu(gate) * up with gate the first half of the packed gate/up output;
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
    "attention_rows", "colwise_rows_sampled", "silu", "swiglu", "MLP_ACTS",
    "mlp_hidden", "packed_rowwise_cols", "single_stream_block",
    "single_stream_rank", "single_stream_as_block", "split_input_rank",
    "block_keys_values", "block_rows_sampled",
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


def silu(u) -> np.ndarray:
    """SiLU (swish): u * sigmoid(u) = u / (1 + exp(-u))."""
    u = np.asarray(u, dtype=np.float64)
    return u / (1.0 + np.exp(-u))


def swiglu(gate, up) -> np.ndarray:
    """SwiGLU combination of a gate and an up projection: silu(gate) * up."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


# MLP activations: "gelu_tanh" (W_up is [F, D]) or "swiglu" (W_up packs the
# gate and up projections as [W_gate; W_up], [2F, D], the [1, 1] packed
# projection of [TP page, §Projeções fundidas]).
MLP_ACTS = ("gelu_tanh", "swiglu")


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
                 head_dim: int, ffn: int, mod_in: int = 0) -> None:
    """[TP page, §Restrições e verificação] tp_degree must divide the head
    count, and each packed block (Q, K, V of width H*d, and the FFN width) must
    be divisible by tp_degree on its own; checked before any weight is used.
    Argument sanity (positive sizes, rank in range, H*d == hidden) is checked
    first."""
    if tp_degree < 1 or not (0 <= rank < tp_degree):
        raise ShardConfigError("argument", f"rank {rank} not in [0, {tp_degree})")
    if hidden <= 0 or num_heads < 0 or ffn < 0 or (num_heads > 0 and head_dim <= 0):
        raise ShardConfigError("argument", "sizes must be positive")
    if mod_in < 0:
        raise ShardConfigError("argument", "sizes must be positive")
    if num_heads == 0 and ffn == 0 and mod_in == 0:
        raise ShardConfigError("argument", "neither attention nor MLP nor modulation")
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
    if mod_in > 0 and mod_in % tp_degree:
        raise ShardConfigError("divisibility",
                               f"tp_degree {tp_degree} does not divide the modulation input {mod_in}")


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


def packed_rowwise_cols(block_sizes: Sequence[int], tp_degree: int, rank: int) -> np.ndarray:
    """[TP page, §Projeções fundidas] dim-1 column indices a rank takes from
    a rowwise Linear whose input is the concatenation of blocks of the given
    absolute sizes (the stored packed row blocks, e.g. [inner_dim,
    mlp_hidden_dim] for an output projection over attention output and MLP
    hidden): its own slice of every block, in block order."""
    cols: List[np.ndarray] = []
    start = 0
    for size in block_sizes:
        if size % tp_degree:
            raise ShardConfigError("divisibility", f"packed block {size} not divisible by {tp_degree}")
        s = rowwise_range(size, tp_degree, rank)
        cols.append(np.arange(start + s.start, start + s.stop))
        start += size
    return np.concatenate(cols)


def shard_weights(wts: Dict[str, np.ndarray], tp_degree: int, rank: int,
                  num_heads: int, head_dim: int, mlp_act: str = "gelu_tanh") -> Dict[str, np.ndarray]:
    """One rank's weight slices.  Colwise (dim 0): the packed Q|K|V weight with
    blocks [1, 1, 1] and the MLP up-projection (for SwiGLU the packed
    [W_gate; W_up] with blocks [1, 1], so the slice is [gate_r; up_r]).
    Rowwise (dim 1): the attention out-projection and the MLP
    down-projection.  Rowwise biases are not sharded (added once after the
    sum).  [TP page, §Colwise e rowwise; §Projeções fundidas]"""
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
        F = wts["w_dn"].shape[1]
        if mlp_act == "swiglu":
            rows = packed_colwise_rows([F, F], tp_degree, rank)
        else:
            c = colwise_range(F, tp_degree, rank)
            rows = np.arange(c.start, c.stop)
        out["w_up"] = f64(wts["w_up"])[rows]
        out["b_up"] = f64(wts["b_up"])[rows]
        out["w_dn"] = f64(wts["w_dn"])[:, rowwise_range(F, tp_degree, rank)]
    return out


def mlp_hidden(x, w_up, b_up, mlp_act: str) -> np.ndarray:
    """The MLP hidden activation from an (unsharded or colwise-sharded) up
    projection: gelu_tanh(x W^T + b), or for SwiGLU with W = [W_gate; W_up]
    (equal halves) silu(x W_gate^T + b_gate) * (x W_up^T + b_up)."""
    u = linear(x, w_up, b_up)
    if mlp_act == "swiglu":
        n = u.shape[1] // 2
        return swiglu(u[:, :n], u[:, n:])
    if mlp_act != "gelu_tanh":
        raise ValueError(mlp_act)
    return gelu_tanh(u)


# --------------------------------------------------------------------------
# One rank's forward, the reduce, and the unsharded block
# --------------------------------------------------------------------------

def rank_forward(x, wts: Dict[str, np.ndarray], tp_degree: int, rank: int,
                 num_heads: int, head_dim: int, bf16: bool,
                 mlp_act: str = "gelu_tanh") -> Dict[str, np.ndarray]:
    """Everything rank ``rank`` computes, in order:

    qkv_r   = x W_qkv_r^T + b_qkv_r                  colwise  [T, 3*D_r]
    o_r     = attention over the rank's H/P heads     [T, D_r]
    h_r     = gelu_tanh(x W_up_r^T + b_up_r)          colwise  [T, F_r]
              (SwiGLU: silu(x G_r^T + b_g) * (x U_r^T + b_u))
    p_attn  = o_r W_o_r^T                            rowwise partial [T, D]
    p_mlp   = h_r W_dn_r^T                           rowwise partial [T, D]
    p_block = p_attn + p_mlp                          (= [o_r | h_r] [W_o_r | W_dn_r]^T)

    [TP page, intro and §Colwise e rowwise.]  Rowwise partials carry no bias.
    With ``bf16`` the stored activations qkv_r, o_r, h_r are rounded to
    bfloat16 (inputs are assumed bf16-representable already)."""
    rnd = to_bf16_rne if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    s = shard_weights(wts, tp_degree, rank, num_heads, head_dim, mlp_act)
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
        h = rnd(mlp_hidden(x, s["w_up"], s["b_up"], mlp_act))
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
                    bf16: bool, mlp_act: str = "gelu_tanh") -> Dict[str, np.ndarray]:
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
        g = rnd(mlp_hidden(x, wts["w_up"], wts["b_up"], mlp_act))
        res["g"] = g
        res["y_mlp"] = linear(g, wts["w_dn"], wts["b_dn"])
        ys.append(res["y_mlp"])
    res["y"] = ys[0] if len(ys) == 1 else ys[0] + ys[1]
    return res


# --------------------------------------------------------------------------
# "rowwise_split_input" [TP page, §Colwise e rowwise; §O que deixar de fora]
# --------------------------------------------------------------------------

def split_input_rank(c, w, tp_degree: int, rank: int) -> np.ndarray:
    """An independent projection whose input c [R, K] is replicated on every
    rank (e.g. an AdaLN modulation projection reading the timestep
    embedding), sharded by input features: the rank takes its contiguous
    block K_r of columns from its own copy of c and of W [N, K] (weight dim
    1) and returns the partial sum c[:, K_r] W[:, K_r]^T [R, N].  No bias:
    it is added once, after the partials are summed."""
    w = np.asarray(w, dtype=np.float64)
    K = w.shape[1]
    if K % tp_degree:
        raise ShardConfigError("divisibility", f"tp_degree {tp_degree} does not divide {K} input features")
    cols = rowwise_range(K, tp_degree, rank)
    return linear(np.asarray(c, dtype=np.float64)[:, cols], w[:, cols])


# --------------------------------------------------------------------------
# Single-stream block with fused projections [TP page, §Projeções fundidas]
#
# One input Linear W_in [3 HD + 2 F, D] packs Q, K, V, gate and up (blocks
# [1, 1, 1, 3, 3] when F = 3 D); one output Linear W_out [D, HD + F] reads the
# concatenation [attention output | SwiGLU hidden] (row blocks [HD, F]).
# --------------------------------------------------------------------------

def _single_stream_parts(u, sizes, num_heads_local, head_dim, rnd):
    """Split the fused projection output by block sizes and run both halves
    (attention over the heads present, SwiGLU over gate/up).  The stored
    activations are q, k, v (the attention input), o and h; gate and up are
    only the SwiGLU's operands."""
    q_w, k_w, v_w, g_w, u_w = sizes
    edges = np.cumsum([0, q_w, k_w, v_w, g_w, u_w])
    q, k, v, gate, up = (u[:, edges[i]:edges[i + 1]] for i in range(5))
    qkv = rnd(np.concatenate([q, k, v], axis=1))
    q, k, v = qkv[:, :q_w], qkv[:, q_w:q_w + k_w], qkv[:, q_w + k_w:]
    o = rnd(attention_heads(q, k, v, num_heads_local, head_dim))
    h = rnd(swiglu(gate, up))
    return qkv, o, h


def single_stream_block(x, w_in, b_in, w_out, b_out, num_heads: int, head_dim: int,
                        ffn: int, bf16: bool) -> Dict[str, np.ndarray]:
    """The unsharded single-stream block: u = x W_in^T + b_in split into
    q, k, v, gate, up; o = attention over all heads; h = silu(gate) * up;
    y = [o | h] W_out^T + b_out.  With bf16 the stored activations q, k, v,
    o, h are rounded to bfloat16."""
    rnd = to_bf16_rne if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    HD = num_heads * head_dim
    u = linear(x, w_in, b_in)
    qkv, o, h = _single_stream_parts(u, (HD, HD, HD, ffn, ffn), num_heads, head_dim, rnd)
    y = linear(np.concatenate([o, h], axis=1), w_out, b_out)
    return {"qkv": qkv, "o": o, "h": h, "y": y}


def single_stream_rank(x, w_in, b_in, w_out, tp_degree: int, rank: int, num_heads: int,
                       head_dim: int, ffn: int, bf16: bool) -> Dict[str, np.ndarray]:
    """One rank of the single-stream block under PackedColwiseParallel on
    W_in (its slice of each of the five blocks) and PackedRowwiseParallel on
    W_out (its slice of each of the two row blocks): the rank's fused
    q/k/v slice qkv_r, its heads' attention o_r, its SwiGLU hidden h_r and
    its fp32 partial [o_r | h_r] W_out_r^T (no bias: added once after the
    sum)."""
    check_config(tp_degree, rank, num_heads * head_dim, num_heads, head_dim, ffn)
    rnd = to_bf16_rne if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    HD = num_heads * head_dim
    rows = packed_colwise_rows([HD, HD, HD, ffn, ffn], tp_degree, rank)
    cols = packed_rowwise_cols([HD, ffn], tp_degree, rank)
    w_in = np.asarray(w_in, dtype=np.float64)
    u = linear(x, w_in[rows], np.asarray(b_in, dtype=np.float64)[rows])
    Dr, Fr = HD // tp_degree, ffn // tp_degree
    qkv, o, h = _single_stream_parts(u, (Dr, Dr, Dr, Fr, Fr), num_heads // tp_degree, head_dim, rnd)
    w_out_r = np.asarray(w_out, dtype=np.float64)[:, cols]
    return {"qkv_r": qkv, "o_r": o, "h_r": h,
            "partial": linear(np.concatenate([o, h], axis=1), w_out_r)}


def single_stream_as_block(w_in, b_in, w_out, b_out, num_heads: int, head_dim: int,
                           ffn: int) -> Dict[str, np.ndarray]:
    """The single-stream weights in the separate-projection form of the block
    (w_q, w_k, w_v, w_up = [W_gate; W_up], w_o, w_dn) with the output bias
    carried as b_o and a zero b_dn."""
    HD = num_heads * head_dim
    e = np.cumsum([0, HD, HD, HD, 2 * ffn])
    w_in, b_in, w_out = (np.asarray(a) for a in (w_in, b_in, w_out))
    return {"w_q": w_in[e[0]:e[1]], "w_k": w_in[e[1]:e[2]], "w_v": w_in[e[2]:e[3]],
            "b_q": b_in[e[0]:e[1]], "b_k": b_in[e[1]:e[2]], "b_v": b_in[e[2]:e[3]],
            "w_up": w_in[e[3]:e[4]], "b_up": b_in[e[3]:e[4]],
            "w_o": w_out[:, :HD], "b_o": np.asarray(b_out),
            "w_dn": w_out[:, HD:], "b_dn": np.zeros_like(np.asarray(b_out))}


# --------------------------------------------------------------------------
# Row-sampled pieces for full-size checks (same definitions, fewer rows)
# --------------------------------------------------------------------------

def colwise_rows_sampled(x_rows, w, b=None, gelu: bool = False, bf16: bool = True,
                         mlp_act: Optional[str] = None) -> np.ndarray:
    """A colwise projection evaluated only on some rows of x (each output row
    depends only on its own input row); with mlp_act, the MLP hidden
    activation of it."""
    if mlp_act is not None:
        y = mlp_hidden(x_rows, w, b, mlp_act)
    else:
        y = linear(x_rows, w, b)
        if gelu:
            y = gelu_tanh(y)
    return to_bf16_rne(y) if bf16 else y


def attention_rows(q_rows, k, v, num_heads: int, head_dim: int) -> np.ndarray:
    """Attention for some query rows against all keys/values (each output row
    depends only on its own query row and on every key and value)."""
    return attention_heads(q_rows, k, v, num_heads, head_dim)


def block_keys_values(x, wts: Dict[str, np.ndarray], bf16: bool):
    """K and V of every token over all heads (unsharded), rounded where the
    ABI stores them: what every sampled attention row reads.  Returned
    separately so several tp_degrees can share one (costly) evaluation."""
    rnd = to_bf16_rne if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    x = np.asarray(x, dtype=np.float64)
    return rnd(linear(x, wts["w_k"], wts["b_k"])), rnd(linear(x, wts["w_v"], wts["b_v"]))


def block_rows_sampled(x, wts: Dict[str, np.ndarray], rows, tp_degree: int, num_heads: int,
                       head_dim: int, bf16: bool, mlp_act: str = "gelu_tanh",
                       kv=None) -> Dict[str, object]:
    """``rank_forward`` for every rank and the reduce, on some token rows only.

    Each output row of the block depends on its own input row, plus every
    key and value for attention, so the rows are exact at any sequence
    length.  Per rank r the stored activations are the column slices of the
    unsharded ones (colwise shards concatenate to the unsharded output, and
    attention is head-local: [TP page, §Colwise e rowwise]): qkv_r = [Q_r |
    K_r | V_r], o_r = O[:, R_r], h_r = G[:, C_r]; the rank's partial is
    o_r W_o[:, R_r]^T + h_r W_dn[:, C_r]^T (no bias), and y = sum over ranks
    in order, plus the rowwise biases once ([TP page, intro]).

    Returns {"ranks": [{"qkv_r", "o_r", "h_r", "p_block"} per rank, on the
    rows], "y": [len(rows), D]}; ``kv`` = block_keys_values(...) if already
    computed."""
    rnd = to_bf16_rne if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    rows = np.asarray(rows)
    xr = np.asarray(x, dtype=np.float64)[rows]
    P = tp_degree
    has_attn = "w_q" in wts
    has_mlp = "w_up" in wts
    if has_attn:
        HD = num_heads * head_dim
        K, V = block_keys_values(x, wts, bf16) if kv is None else kv
        Q = rnd(linear(xr, wts["w_q"], wts["b_q"]))
        o = rnd(attention_heads(Q, K, V, num_heads, head_dim))
        Kr, Vr = K[rows], V[rows]
    if has_mlp:
        F = np.asarray(wts["w_dn"]).shape[1]
        g = rnd(mlp_hidden(xr, wts["w_up"], wts["b_up"], mlp_act))
    ranks = []
    for r in range(P):
        res: Dict[str, np.ndarray] = {}
        part = 0.0
        if has_attn:
            R = colwise_range(HD, P, r)
            res["qkv_r"] = np.concatenate([Q[:, R], Kr[:, R], Vr[:, R]], axis=1)
            res["o_r"] = o[:, R]
            part = part + linear(res["o_r"], np.asarray(wts["w_o"])[:, rowwise_range(HD, P, r)])
        if has_mlp:
            C = colwise_range(F, P, r)
            res["h_r"] = g[:, C]
            part = part + linear(res["h_r"], np.asarray(wts["w_dn"])[:, rowwise_range(F, P, r)])
        res["p_block"] = part
        ranks.append(res)
    y = partial_reduce([res["p_block"] for res in ranks], rowwise_bias(wts))
    return {"ranks": ranks, "y": y}
