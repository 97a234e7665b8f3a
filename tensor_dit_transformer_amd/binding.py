"""ctypes binding of libtp_shard.so (include/tp_shard.h).

Argument marshalling only: torch tensors supply device pointers and row
strides, ``torch.cuda.current_stream()`` supplies the hipStream_t, numpy arrays
supply the host weights for shard creation.  Every computation runs in the HIP
library; there is no fallback of any kind.  If the library is missing, every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

# TP_SHARD_LIB names another build of the same library (the host-sanitizer
# build the CPU tests run the ABI checks under); the default is the in-tree one.
LIB_PATH = os.environ.get("TP_SHARD_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libtp_shard.so")

# tp_status
TP_OK = 0
TP_ERR_ARG = -1
TP_ERR_DIVISIBILITY = -2
TP_ERR_UNSUPPORTED = -3
TP_ERR_HIP = -4
TP_ERR_OOM = -5
TP_ERR_IO = -6
# tp_dtype
TP_F32 = 0
TP_BF16 = 1
# tp_mlp_act
TP_MLP_GELU_TANH = 0
TP_MLP_SWIGLU = 1
# tp_layer
TP_QKV = 0
TP_MLP_UP = 1
TP_ATTN_OUT = 2
TP_MLP_DOWN = 3
TP_BLOCK_OUT = 4
TP_ADALN_MOD = 5

EXPORTED = (
    "tp_block_shard_create", "tp_block_shard_destroy", "tp_colwise_linear",
    "tp_colwise_qkv_up", "tp_attn_heads", "tp_rowwise_linear_partial",
    "tp_partial_reduce", "tp_status_string", "tp_last_error_detail",
    "tp_rowwise_split_input_partial", "tp_attn_heads_block", "tp_attn_merge",
    "tp_attn_heads_split", "tp_attn_split_hint", "tp_ulysses_seq_to_heads",
    "tp_ulysses_heads_to_seq", "tp_block_shard_load", "tp_attn_heads_block_split",
    "tp_attn_heads_split_noalloc",
)


class TpBlockConfig(ctypes.Structure):
    _fields_ = [("tp_degree", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("hidden", ctypes.c_int64), ("num_heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("dtype", ctypes.c_int), ("mlp_act", ctypes.c_int),
                ("mod_in", ctypes.c_int64), ("mod_out", ctypes.c_int64)]


_WEIGHT_FIELDS = ("w_q", "w_k", "w_v", "b_q", "b_k", "b_v", "w_o", "w_up", "b_up", "w_down",
                  "w_mod")


class TpBlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS[:10]] + [
        ("ld_o", ctypes.c_int64), ("ld_down", ctypes.c_int64), ("w_mod", ctypes.c_void_p)]


class TpWeightFile(ctypes.Structure):
    _fields_ = [("path", ctypes.c_char_p), ("offset", ctypes.c_int64)]


class TpBlockWeightFiles(ctypes.Structure):
    _fields_ = [(n, TpWeightFile) for n in _WEIGHT_FIELDS] + [
        ("ld_o", ctypes.c_int64), ("ld_down", ctypes.c_int64)]


class TpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)} ({detail})")
        self.status = status
        self.detail = detail


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is missing: build it with "
                               "`python -m tensor_dit_transformer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.tp_block_shard_create.argtypes = [ctypes.POINTER(TpBlockConfig),
                                            ctypes.POINTER(TpBlockWeights), ctypes.POINTER(vp)]
        L.tp_block_shard_load.argtypes = [ctypes.POINTER(TpBlockConfig),
                                          ctypes.POINTER(TpBlockWeightFiles), i64, ctypes.POINTER(vp)]
        L.tp_block_shard_destroy.argtypes = [vp]
        L.tp_block_shard_destroy.restype = None
        L.tp_colwise_linear.argtypes = [vp, ctypes.c_int, i64, vp, i64, vp, i64, vp]
        L.tp_colwise_qkv_up.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp]
        L.tp_attn_heads.argtypes = [vp, i64, vp, i64, vp, i64, vp]
        L.tp_rowwise_linear_partial.argtypes = [vp, ctypes.c_int, i64, vp, i64, vp, i64,
                                                ctypes.c_int, vp]
        L.tp_rowwise_split_input_partial.argtypes = [vp, ctypes.c_int, i64, vp, i64, vp, i64,
                                                     ctypes.c_int, vp]
        L.tp_attn_heads_block.argtypes = [vp, i64, vp, i64, i64, vp, i64, vp, i64, vp, i64, vp]
        L.tp_attn_heads_split.argtypes = [vp, i64, vp, i64, i32, vp, i64, i64, vp, i64, i64, vp]
        L.tp_attn_heads_split_noalloc.argtypes = [vp, i64, vp, i64, i32, vp, i64, vp]
        L.tp_attn_heads_block_split.argtypes = [vp, i64, vp, i64, i64, vp, i64, i32, vp, i64, i64,
                                                vp, i64, i64, vp]
        L.tp_ulysses_seq_to_heads.argtypes = [ctypes.POINTER(vp), i32, i64, i64, i64, i64, i32, i32,
                                              ctypes.c_int, vp, i64, vp]
        L.tp_ulysses_heads_to_seq.argtypes = [ctypes.POINTER(vp), i32, i64, i64, i64, i64, i32,
                                              ctypes.c_int, vp, i64, vp]
        L.tp_attn_split_hint.argtypes = [vp, i64]
        L.tp_attn_split_hint.restype = ctypes.c_int32
        L.tp_attn_merge.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i64, i64, i64, i64,
                                    i64, vp, i64, ctypes.c_int, vp, i64, vp]
        L.tp_partial_reduce.argtypes = [ctypes.POINTER(vp), i32, i64, ctypes.POINTER(vp), i32,
                                        i64, i64, vp, i64, vp]
        for f in ("tp_block_shard_create", "tp_block_shard_load", "tp_colwise_linear", "tp_colwise_qkv_up",
                  "tp_attn_heads", "tp_rowwise_linear_partial", "tp_partial_reduce",
                  "tp_rowwise_split_input_partial", "tp_attn_heads_block", "tp_attn_merge",
                  "tp_attn_heads_split", "tp_attn_heads_block_split", "tp_ulysses_seq_to_heads",
                  "tp_attn_heads_split_noalloc",
                  "tp_ulysses_heads_to_seq"):
            getattr(L, f).restype = ctypes.c_int
        L.tp_status_string.argtypes = [ctypes.c_int]
        L.tp_status_string.restype = ctypes.c_char_p
        L.tp_last_error_detail.argtypes = []
        L.tp_last_error_detail.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tp_status_string(status).decode()


def tp_status_string(status: int) -> str:
    return status_string(status)


def tp_last_error_detail() -> str:
    return lib().tp_last_error_detail().decode()


def _check(status: int) -> None:
    if status != TP_OK:
        raise TpError(status, tp_last_error_detail())


# ------------------------------------------------------------------ marshalling

def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _mat(t, name: str, rows: int = 0, cols: int = 0, dtype: Optional[int] = None):
    """(device pointer, row stride in elements) of a 2-D row-major torch
    tensor that holds at least rows x cols elements of the given dtype code."""
    if dtype is not None and _dtype_code(t) != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, the shard's dtype code is {dtype}")
    if t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, needs at least ({rows}, {cols})")
    return t.data_ptr(), t.stride(0)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


class TpBlockShard:
    """Handle of a created shard (owns the rank's device weight slices)."""

    def __init__(self, handle: int, cfg: TpBlockConfig):
        self.handle = handle
        self.tp_degree = cfg.tp_degree
        self.rank = cfg.rank
        self.hidden = cfg.hidden
        self.num_heads = cfg.num_heads
        self.head_dim = cfg.head_dim
        self.ffn = cfg.ffn
        self.dtype = cfg.dtype
        self.mlp_act = cfg.mlp_act
        self.mod_in = cfg.mod_in
        self.mod_out = cfg.mod_out
        P = cfg.tp_degree
        self.d_r = cfg.hidden // P if cfg.num_heads > 0 else 0
        self.f_r = cfg.ffn // P
        self.heads_r = cfg.num_heads // P

    def close(self) -> None:
        if self.handle:
            lib().tp_block_shard_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        import torch
        torch.cuda.synchronize()
        self.close()


def make_config(tp_degree: int, rank: int, hidden: int, num_heads: int, head_dim: int,
                ffn: int, dtype: int, mlp_act: int = TP_MLP_GELU_TANH, mod_in: int = 0,
                mod_out: int = 0) -> TpBlockConfig:
    return TpBlockConfig(tp_degree, rank, hidden, num_heads, head_dim, ffn, dtype, mlp_act,
                         mod_in, mod_out)


def _weight_shapes(cfg: TpBlockConfig):
    D, HD, F = cfg.hidden, cfg.num_heads * cfg.head_dim, cfg.ffn
    U = 2 * F if cfg.mlp_act == TP_MLP_SWIGLU else F
    return {"w_q": (HD, D), "w_k": (HD, D), "w_v": (HD, D), "b_q": (HD,), "b_k": (HD,),
            "b_v": (HD,), "w_o": (D, HD), "w_up": (U, D), "b_up": (U,), "w_down": (D, F),
            "w_in": (3 * HD + U, D), "b_in": (3 * HD + U,), "w_out": (D, HD + F),
            "w_mod": (cfg.mod_out, cfg.mod_in)}


def _host_weights(weights: Dict[str, np.ndarray], cfg: TpBlockConfig):
    """TpBlockWeights pointing at contiguous host arrays (kept alive by the
    returned list).  bf16 arrays are uint16 bit patterns.

    Besides the separate projections, a packed checkpoint may be given as
    ``w_in`` [3 H d + U, D] = [W_q; W_k; W_v; W_up-block] (with ``b_in``) and
    ``w_out`` [D, H d + F] = [W_o | W_down]: the pointers then address the
    blocks inside them (rows for w_in, columns with ld = H d + F for w_out)."""
    keep = []
    w = TpBlockWeights()
    want = np.uint16 if cfg.dtype == TP_BF16 else np.float32
    es = np.dtype(want).itemsize
    shapes = _weight_shapes(cfg)
    D, HD, F = cfg.hidden, cfg.num_heads * cfg.head_dim, cfg.ffn

    def host(name, key=None):
        a = np.ascontiguousarray(weights[key or name])
        if a.dtype != want:
            raise ValueError(f"{name}: host weights must be {np.dtype(want).name} for this dtype")
        if a.size != int(np.prod(shapes[name])):
            raise ValueError(f"{name}: {a.size} elements, expected shape {shapes[name]}")
        keep.append(a)
        return a.ctypes.data

    if "w_in" in weights:
        base = host("w_in")
        w.w_q, w.w_k, w.w_v, w.w_up = (base + i * HD * D * es for i in range(4))
        if weights.get("b_in") is not None:
            bb = host("b_in")
            w.b_q, w.b_k, w.b_v, w.b_up = (bb + i * HD * es for i in range(4))
    if "w_out" in weights:
        base = host("w_out")
        w.w_o, w.w_down = base, base + HD * es
        w.ld_o = w.ld_down = HD + F
    for name in _WEIGHT_FIELDS:
        if getattr(w, name):
            continue
        key = "w_dn" if name == "w_down" and name not in weights else name
        if weights.get(key) is None:
            continue
        setattr(w, name, host(name, key))
    return w, keep


# ------------------------------------------------------------------ entry points

def tp_block_shard_create(cfg: TpBlockConfig, weights: Dict[str, np.ndarray]) -> TpBlockShard:
    w, keep = _host_weights(weights, cfg)
    out = ctypes.c_void_p()
    st = lib().tp_block_shard_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(out))
    del keep
    _check(st)
    return TpBlockShard(out.value, cfg)


def tp_block_shard_load(cfg: TpBlockConfig, files: Dict[str, tuple], staging_bytes: int = 64 << 20,
                        ld_o: int = 0, ld_down: int = 0) -> TpBlockShard:
    """Create a shard reading only its slices from raw weight files: `files`
    maps a weight name (w_q, ..., w_down, w_mod) to (path, byte offset)."""
    f = TpBlockWeightFiles()
    for name, (path, offset) in files.items():
        if name not in _WEIGHT_FIELDS:
            raise ValueError(f"unknown weight {name}")
        setattr(f, name, TpWeightFile(str(path).encode(), int(offset)))
    f.ld_o, f.ld_down = ld_o, ld_down
    out = ctypes.c_void_p()
    _check(lib().tp_block_shard_load(ctypes.byref(cfg), ctypes.byref(f), staging_bytes,
                                     ctypes.byref(out)))
    return TpBlockShard(out.value, cfg)


def tp_block_shard_destroy(shard: TpBlockShard) -> None:
    shard.close()


def tp_colwise_linear(shard: TpBlockShard, layer: int, tokens: int, x, y, stream=None) -> None:
    n = {TP_QKV: 3 * shard.d_r, TP_MLP_UP: shard.f_r}.get(layer, 0)
    xp, ldx = _mat(x, "x", tokens, shard.hidden, shard.dtype)
    yp, ldy = _mat(y, "y", tokens, n, shard.dtype)
    _check(lib().tp_colwise_linear(shard.handle, layer, tokens, xp, ldx, yp, ldy, _stream(stream)))


def tp_colwise_qkv_up(shard: TpBlockShard, tokens: int, x, qkv, h, stream=None) -> None:
    xp, ldx = _mat(x, "x", tokens, shard.hidden, shard.dtype)
    qp, ldq = _mat(qkv, "qkv", tokens, 3 * shard.d_r, shard.dtype)
    hp, ldh = _mat(h, "h", tokens, shard.f_r, shard.dtype)
    _check(lib().tp_colwise_qkv_up(shard.handle, tokens, xp, ldx, qp, ldq, hp, ldh,
                                   _stream(stream)))


def tp_attn_heads(shard: TpBlockShard, tokens: int, qkv, o, stream=None) -> None:
    qp, ldq = _mat(qkv, "qkv", tokens, 3 * shard.d_r, shard.dtype)
    op, ldo = _mat(o, "o", tokens, shard.d_r, shard.dtype)
    _check(lib().tp_attn_heads(shard.handle, tokens, qp, ldq, op, ldo, _stream(stream)))


def tp_attn_heads_block(shard: TpBlockShard, q_tokens: int, q_qkv, kv_tokens: int, kv_qkv, o, lse,
                        stream=None) -> None:
    """One key block of attention: fp32 normalised o [q_tokens, D_r] and the
    natural log-sum-exp lse [q_tokens, H/P] (fp32)."""
    qp, ldq = _mat(q_qkv, "q_qkv", q_tokens, shard.d_r, shard.dtype)
    kp, ldk = _mat(kv_qkv, "kv_qkv", kv_tokens, 3 * shard.d_r, shard.dtype)
    op, ldo = _mat(o, "o", q_tokens, shard.d_r, TP_F32)
    lp, ldl = _mat(lse, "lse", q_tokens, shard.heads_r, TP_F32)
    _check(lib().tp_attn_heads_block(shard.handle, q_tokens, qp, ldq, kv_tokens, kp, ldk, op, ldo,
                                     lp, ldl, _stream(stream)))


def tp_attn_heads_block_split(shard: TpBlockShard, q_tokens: int, q_qkv, kv_tokens: int, kv_qkv,
                              o_parts, lse_parts, stream=None) -> None:
    """tp_attn_heads_block with the block's keys split len-wise into
    o_parts.shape[0] ranges in one launch: o_parts fp32 [S, q_tokens, D_r],
    lse_parts fp32 [S, q_tokens, H/P] (3-D device tensors; each part a 2-D
    row-major slice)."""
    S = o_parts.shape[0]
    if o_parts.dim() != 3 or lse_parts.dim() != 3 or lse_parts.shape[0] != S:
        raise ValueError("o_parts / lse_parts must be 3-D with one part per split")
    qp, ldq = _mat(q_qkv, "q_qkv", q_tokens, shard.d_r, shard.dtype)
    kp, ldk = _mat(kv_qkv, "kv_qkv", kv_tokens, 3 * shard.d_r, shard.dtype)
    op, ldo = _mat(o_parts[0], "o_parts[0]", q_tokens, shard.d_r, TP_F32)
    lp, ldl = _mat(lse_parts[0], "lse_parts[0]", q_tokens, shard.heads_r, TP_F32)
    _check(lib().tp_attn_heads_block_split(shard.handle, q_tokens, qp, ldq, kv_tokens, kp, ldk, S,
                                           op, ldo, o_parts.stride(0), lp, ldl, lse_parts.stride(0),
                                           _stream(stream)))


def tp_attn_heads_split(shard: TpBlockShard, tokens: int, qkv, o_parts, lse_parts,
                        stream=None) -> None:
    """Attention with the keys split len-wise into o_parts.shape[0] ranges in
    one launch: o_parts fp32 [S, tokens, D_r], lse_parts fp32 [S, tokens, H/P]
    (3-D device tensors; each part a 2-D row-major slice)."""
    S = o_parts.shape[0]
    if o_parts.dim() != 3 or lse_parts.dim() != 3 or lse_parts.shape[0] != S:
        raise ValueError("o_parts / lse_parts must be 3-D with one part per split")
    qp, ldq = _mat(qkv, "qkv", tokens, 3 * shard.d_r, shard.dtype)
    op, ldo = _mat(o_parts[0], "o_parts[0]", tokens, shard.d_r, TP_F32)
    lp, ldl = _mat(lse_parts[0], "lse_parts[0]", tokens, shard.heads_r, TP_F32)
    _check(lib().tp_attn_heads_split(shard.handle, tokens, qp, ldq, S, op, ldo, o_parts.stride(0),
                                     lp, ldl, lse_parts.stride(0), _stream(stream)))


def tp_attn_heads_split_noalloc(shard: TpBlockShard, tokens: int, qkv, o, n_splits: int,
                                stream=None) -> None:
    """tp_attn_heads_split + tp_attn_merge in one call, the partial results in
    the library's per-GPU scratch array (no allocation; calls overlapping on
    one GPU race)."""
    qp, ldq = _mat(qkv, "qkv", tokens, 3 * shard.d_r, shard.dtype)
    op, ldo = _mat(o, "o", tokens, shard.d_r, shard.dtype)
    _check(lib().tp_attn_heads_split_noalloc(shard.handle, tokens, qp, ldq, int(n_splits), op, ldo,
                                             _stream(stream)))


def tp_attn_split_hint(shard: TpBlockShard, tokens: int) -> int:
    return int(lib().tp_attn_split_hint(shard.handle, tokens))


def _same_ld(mats, name):
    lds = {ld for _, ld in mats}
    if len(lds) != 1:
        raise ValueError(f"{name} must share one row stride")
    return mats[0][1]


def tp_ulysses_seq_to_heads(chunks: Sequence, heads: int, head_dim: int, blocks: int, rank: int,
                            out, stream=None) -> None:
    """Rank `rank`'s buffer after Ulysses' first all-to-all, from every rank's
    token chunk ([n, blocks*H*d] each) into out [u*n, blocks*W]."""
    u, n = len(chunks), chunks[0].shape[0]
    dt = _dtype_code(out)
    mats = [_mat(c, "chunk", n, blocks * heads * head_dim, dt) for c in chunks]
    ld = _same_ld(mats, "chunks")
    op, ldo = _mat(out, "out", u * n, blocks * heads // u * head_dim, dt)
    C = (ctypes.c_void_p * u)(*[p for p, _ in mats])
    _check(lib().tp_ulysses_seq_to_heads(C, u, ld, n, heads, head_dim, blocks, rank, dt, op, ldo,
                                         _stream(stream)))


def tp_ulysses_heads_to_seq(parts: Sequence, heads: int, head_dim: int, rank: int, out,
                            stream=None) -> None:
    """Rank `rank`'s token chunk after Ulysses' second all-to-all, from every
    rank's head-block output ([u*n, W] each) into out [n, H*d]."""
    u = len(parts)
    n = parts[0].shape[0] // u
    dt = _dtype_code(out)
    mats = [_mat(p, "part", u * n, heads // u * head_dim, dt) for p in parts]
    ld = _same_ld(mats, "parts")
    op, ldo = _mat(out, "out", n, heads * head_dim, dt)
    Pp = (ctypes.c_void_p * u)(*[p for p, _ in mats])
    _check(lib().tp_ulysses_heads_to_seq(Pp, u, ld, n, heads, head_dim, rank, dt, op, ldo,
                                         _stream(stream)))


def tp_attn_merge(o_parts: Sequence, lse_parts: Sequence, o, heads: int, head_dim: int,
                  lse_out=None, stream=None) -> None:
    """o = merge of the partial results (o_i fp32 [T, heads*head_dim], lse_i
    fp32 [T, heads]); o is bf16 or fp32; lse_out optional fp32 [T, heads]."""
    if len(o_parts) != len(lse_parts) or not o_parts:
        raise ValueError("need as many lse parts as output parts, at least one")
    T = o.shape[0]
    W = heads * head_dim
    ops = [_mat(p, "o_part", T, W, TP_F32) for p in o_parts]
    lps = [_mat(p, "lse_part", T, heads, TP_F32) for p in lse_parts]
    if any(ld != ops[0][1] for _, ld in ops) or any(ld != lps[0][1] for _, ld in lps):
        raise ValueError("parts must share one row stride each")
    od = _dtype_code(o)
    op, ldo = _mat(o, "o", T, W, od)
    lo, ldl = (None, 0) if lse_out is None else _mat(lse_out, "lse_out", T, heads, TP_F32)
    OP = (ctypes.c_void_p * len(ops))(*[p for p, _ in ops])
    LP = (ctypes.c_void_p * len(lps))(*[p for p, _ in lps])
    _check(lib().tp_attn_merge(OP, LP, len(ops), ops[0][1], lps[0][1], T, heads, head_dim, op, ldo,
                               od, lo, ldl, _stream(stream)))


def tp_rowwise_linear_partial(shard: TpBlockShard, layer: int, tokens: int, x_local, partial,
                              accumulate: bool = False, stream=None) -> None:
    k = {TP_ATTN_OUT: shard.d_r, TP_MLP_DOWN: shard.f_r,
         TP_BLOCK_OUT: shard.d_r + shard.f_r}.get(layer, 0)
    xp, ldx = _mat(x_local, "x_local", tokens, k, shard.dtype)
    pp, ldp = _mat(partial, "partial", tokens, shard.hidden, TP_F32)
    _check(lib().tp_rowwise_linear_partial(shard.handle, layer, tokens, xp, ldx, pp, ldp,
                                           1 if accumulate else 0, _stream(stream)))


def tp_rowwise_split_input_partial(shard: TpBlockShard, layer: int, rows: int, x_full, partial,
                                   accumulate: bool = False, stream=None) -> None:
    HD = shard.d_r * shard.tp_degree
    width, n = {TP_ADALN_MOD: (shard.mod_in, shard.mod_out), TP_ATTN_OUT: (HD, shard.hidden),
                TP_MLP_DOWN: (shard.ffn, shard.hidden),
                TP_BLOCK_OUT: (HD + shard.ffn, shard.hidden)}.get(layer, (0, 0))
    xp, ldx = _mat(x_full, "x_full", rows, width, shard.dtype)
    pp, ldp = _mat(partial, "partial", rows, n, TP_F32)
    _check(lib().tp_rowwise_split_input_partial(shard.handle, layer, rows, xp, ldx, pp, ldp,
                                                1 if accumulate else 0, _stream(stream)))


def tp_partial_reduce(partials: Sequence, biases: Sequence, out, stream=None) -> None:
    """out = sum(partials) + sum(biases); partials [T, D] fp32 sharing one row
    stride, biases fp32 [D]."""
    if len(partials) == 0:
        raise ValueError("no partials")
    T, D = out.shape
    ptrs = [_mat(p, "partial", T, D, TP_F32) for p in partials]
    ldp = ptrs[0][1]
    if any(ld != ldp for _, ld in ptrs):
        raise ValueError("partials must share one row stride")
    for b in biases:
        if b.dim() != 1 or not b.is_cuda or b.stride(0) != 1 or b.shape[0] < D or _dtype_code(b) != TP_F32:
            raise ValueError("biases must be contiguous fp32 1-D device tensors of length >= hidden")
    P = (ctypes.c_void_p * max(1, len(partials)))(*[p for p, _ in ptrs])
    B = (ctypes.c_void_p * max(1, len(biases)))(*[b.data_ptr() for b in biases])
    op, ldo = _mat(out, "out", 0, 0, TP_F32)
    _check(lib().tp_partial_reduce(P, len(partials), ldp, B if biases else None, len(biases),
                                   T, D, op, ldo, _stream(stream)))
