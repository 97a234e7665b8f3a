"""Harness shared by the GPU tests, the smoke check and the benchmark: upload
seeded inputs, create the P rank shards through the C ABI, and run one rank's
hot path (all through tensor_dit_transformer_amd; no arithmetic here)."""
from __future__ import annotations

from typing import Dict, List

import numpy as np
import torch

import tensor_dit_transformer_amd as tp
import tp_inputs


def to_device(inp: tp_inputs.Inputs, name: str) -> torch.Tensor:
    if inp.bits is not None:
        return torch.from_numpy(inp.bits[name].view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(inp.values[name])).cuda()


def host_weights(inp: tp_inputs.Inputs) -> Dict[str, np.ndarray]:
    src = inp.bits if inp.bits is not None else inp.values
    out = {k: v for k, v in src.items() if k not in ("x", "c")}
    if "w_dn" in out:
        out["w_down"] = out.pop("w_dn")
    return out


def config(w: tp_inputs.Workload, rank: int) -> tp.TpBlockConfig:
    dt = tp.TP_BF16 if w.dtype == "bf16" else tp.TP_F32
    act = tp.TP_MLP_SWIGLU if w.mlp_act == "swiglu" else tp.TP_MLP_GELU_TANH
    return tp.make_config(w.tp_degree, rank, w.hidden, w.num_heads, w.head_dim, w.ffn, dt, act,
                          w.hidden if w.has_mod else 0, w.mod_out)


def packed_host_weights(inp: tp_inputs.Inputs) -> Dict[str, np.ndarray]:
    """The same weights as one fused input projection w_in = [W_q; W_k; W_v;
    W_up-block] (+ b_in) and one fused output projection w_out = [W_o | W_dn]
    (a packed checkpoint's layout; concatenation only)."""
    h = host_weights(inp)
    return {"w_in": np.concatenate([h["w_q"], h["w_k"], h["w_v"], h["w_up"]]),
            "b_in": np.concatenate([h["b_q"], h["b_k"], h["b_v"], h["b_up"]]),
            "w_out": np.ascontiguousarray(np.concatenate([h["w_o"], h["w_down"]], axis=1))}


def write_weights(path, weights: Dict[str, np.ndarray]) -> Dict[str, tuple]:
    """Append the arrays to one raw file (a checkpoint of unsharded weights,
    each row-major in the workload's dtype) and return {name: (path, byte
    offset)} for the shard-on-read loader.  Data movement only."""
    out, off = {}, 0
    with open(path, "wb") as f:
        for name, a in weights.items():
            a = np.ascontiguousarray(a)
            out[name] = (str(path), off)
            f.write(a.tobytes())
            off += a.nbytes
    return out


def create_shards(w: tp_inputs.Workload, inp: tp_inputs.Inputs, ranks=None,
                  packed: bool = False) -> List[tp.TpBlockShard]:
    hw = packed_host_weights(inp) if packed else host_weights(inp)
    ranks = range(w.tp_degree) if ranks is None else ranks
    return [tp.tp_block_shard_create(config(w, r), hw) for r in ranks]


def f32_device(a: np.ndarray) -> torch.Tensor:
    """An fp32 device copy of a host array (exact widening of bf16 values)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def rowwise_biases(w: tp_inputs.Workload, inp: tp_inputs.Inputs) -> List[torch.Tensor]:
    """fp32 device copies of the rowwise biases (exact widening of bf16)."""
    out = []
    for k in ("b_o", "b_dn"):
        if k in inp.values:
            out.append(torch.from_numpy(np.ascontiguousarray(inp.values[k], dtype=np.float32)).cuda())
    return out


class RankBuffers:
    """Activation buffers of one rank: qkv [T, 3Dr], oh = [o_r | h_r]
    [T, Dr + Fr], partial fp32 [T, D]; and, when the library's split hint
    asks for key splits, their fp32 partial outputs and log-sum-exps."""

    def __init__(self, shard: tp.TpBlockShard, T: int, partial: torch.Tensor = None):
        dt = torch.bfloat16 if shard.dtype == tp.TP_BF16 else torch.float32
        Dr, Fr, D = shard.d_r, shard.f_r, shard.hidden
        self.qkv = torch.empty((T, 3 * Dr), dtype=dt, device="cuda") if Dr else None
        self.oh = torch.empty((T, Dr + Fr), dtype=dt, device="cuda")
        self.o = self.oh[:, :Dr] if Dr else None
        self.h = self.oh[:, Dr:] if Fr else None
        self.partial = partial if partial is not None else torch.empty((T, D), dtype=torch.float32,
                                                                      device="cuda")
        self.splits = tp.tp_attn_split_hint(shard, T) if Dr and shard.dtype == tp.TP_BF16 else 1
        if self.splits > 1:
            self.o_parts = torch.empty((self.splits, T, Dr), dtype=torch.float32, device="cuda")
            self.lse_parts = torch.empty((self.splits, T, shard.heads_r), dtype=torch.float32,
                                         device="cuda")


def attention(shard: tp.TpBlockShard, T: int, buf: RankBuffers) -> None:
    """The rank's attention: one call, or key splits in one launch plus the
    merge when the split hint says the single launch leaves the GPU idle."""
    if buf.splits > 1:
        tp.tp_attn_heads_split(shard, T, buf.qkv, buf.o_parts, buf.lse_parts)
        tp.tp_attn_merge(list(buf.o_parts), list(buf.lse_parts), buf.o, shard.heads_r, shard.head_dim)
    else:
        tp.tp_attn_heads(shard, T, buf.qkv, buf.o)


def run_rank(shard: tp.TpBlockShard, x: torch.Tensor, buf: RankBuffers, fused: bool = True) -> None:
    """One rank's hot path: colwise projection(s), attention, rowwise partial."""
    T = x.shape[0]
    attn, mlp = shard.d_r > 0, shard.f_r > 0
    if attn and mlp:
        if fused:
            tp.tp_colwise_qkv_up(shard, T, x, buf.qkv, buf.h)
        else:
            tp.tp_colwise_linear(shard, tp.TP_QKV, T, x, buf.qkv)
            tp.tp_colwise_linear(shard, tp.TP_MLP_UP, T, x, buf.h)
        attention(shard, T, buf)
        tp.tp_rowwise_linear_partial(shard, tp.TP_BLOCK_OUT, T, buf.oh, buf.partial)
    elif attn:
        tp.tp_colwise_linear(shard, tp.TP_QKV, T, x, buf.qkv)
        attention(shard, T, buf)
        tp.tp_rowwise_linear_partial(shard, tp.TP_ATTN_OUT, T, buf.o, buf.partial)
    else:
        tp.tp_colwise_linear(shard, tp.TP_MLP_UP, T, x, buf.h)
        tp.tp_rowwise_linear_partial(shard, tp.TP_MLP_DOWN, T, buf.h, buf.partial)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref|, the parity metric."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


TOL = {"f32": 1e-4, "bf16": 2e-2}
