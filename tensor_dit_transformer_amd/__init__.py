"""MI355X-native tensor-parallel DiT block shard.

One tensor-parallel rank's share of a diffusion-transformer block -- colwise
QKV and MLP-up projections, attention over the rank's heads, rowwise partial
projections, and the boundary partial-sum -- as hand-written HIP kernels for
gfx950 behind the C ABI of include/tp_shard.h.  This package is the thin
ctypes binding (same entry-point names as the C ABI) and the build script.
"""
from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, TP_ADALN_MOD, TP_ATTN_OUT, TP_BF16, TP_BLOCK_OUT, TP_ERR_ARG,
    TP_ERR_DIVISIBILITY, TP_ERR_HIP, TP_ERR_IO, TP_ERR_OOM, TP_ERR_UNSUPPORTED, TP_F32,
    TP_MLP_DOWN, TP_MLP_GELU_TANH, TP_MLP_SWIGLU, TP_MLP_UP, TP_OK, TP_QKV, TpBlockConfig, TpBlockShard,
    TpBlockWeights, TpError, lib, make_config, status_string, tp_attn_heads,
    tp_attn_heads_block, tp_attn_heads_block_split, tp_attn_heads_split, tp_attn_merge,
    tp_attn_heads_split_noalloc,
    tp_attn_split_hint,
    tp_block_shard_create, tp_block_shard_destroy, tp_block_shard_load, tp_colwise_linear,
    tp_colwise_qkv_up, tp_last_error_detail, tp_partial_reduce,
    tp_rowwise_linear_partial, tp_rowwise_split_input_partial, tp_status_string,
    tp_ulysses_heads_to_seq, tp_ulysses_seq_to_heads,
)
