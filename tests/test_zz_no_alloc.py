"""The allocation-free split attention (for callers that cannot allocate):
tp_attn_heads_split_noalloc, called through the C ABI, gives exactly what
tp_attn_heads_split + tp_attn_merge give with caller-owned partial buffers
(the same kernels in the same launch configuration, so bit for bit), on two
calls in a row -- the second smaller, over the scratch contents the first
left -- and matches the float64 oracle (per-head attention, Diffusers TP
page, §Colwise e rowwise) within the bf16 tolerance.  A request beyond the
scratch array's 64 MiB is rejected before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import tensor_dit_transformer_amd as tp
import tp_harness as H
import tp_inputs
from tp_inputs import Workload

pytestmark = pytest.mark.gpu


def shard(heads_r):
    w = Workload(f"attn_H{4 * heads_r}_P4", 8, 4 * heads_r * 128, 4 * heads_r, 128, 0, 4, "bf16")
    return H.create_shards(w, tp_inputs.make_inputs(w, seed=3), ranks=(1,))[0]


def with_caller_buffers(s, T, qkv, S):
    o_parts = torch.empty((S, T, s.d_r), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((S, T, s.heads_r), dtype=torch.float32, device="cuda")
    o = torch.empty((T, s.d_r), dtype=torch.bfloat16, device="cuda")
    tp.tp_attn_heads_split(s, T, qkv, o_parts, l_parts)
    tp.tp_attn_merge(list(o_parts), list(l_parts), o, s.heads_r, 128)
    return o


def noalloc_abi(s, T, qkv, S, o):
    """Straight through the C entry point (ctypes), no binding wrapper."""
    return tp.lib().tp_attn_heads_split_noalloc(s.handle, T, qkv.data_ptr(), qkv.stride(0), S,
                                                o.data_ptr(), o.stride(0), None)


def test_noalloc_split_attention_equals_caller_buffer_path():
    s = shard(6)
    Dr = s.d_r
    for T, S, seed in ((4608, 2, 61), (1000, 3, 62)):      # second call smaller
        qv, qb = tp_inputs.random_matrix((T, 3 * Dr), seed=seed, std=1.5)
        qkv = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).cuda()
        ref = with_caller_buffers(s, T, qkv, S)
        o = torch.full((T, Dr), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert noalloc_abi(s, T, qkv, S, o) == tp.TP_OK, tp.tp_last_error_detail()
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"T={T} S={S}"
        rows = tp_inputs.sample_rows(T, 48, seed=seed)
        q64 = qv.astype(np.float64)
        want = O.to_bf16_rne(O.attention_rows(q64[rows, :Dr], q64[:, Dr:2 * Dr], q64[:, 2 * Dr:],
                                              s.heads_r, 128))
        e = H.rel_err(H.as_f64(o[rows]), want)
        print(f"noalloc T={T} splits={S}: bitwise equal to the caller-buffer path; oracle {e:.2e}", flush=True)
        assert e <= H.TOL["bf16"]
        # the binding wrapper reaches the same entry point
        o2 = torch.empty_like(o)
        tp.tp_attn_heads_split_noalloc(s, T, qkv, o2, S)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref)
    torch.cuda.synchronize()
    s.close()


def test_noalloc_rejects_requests_beyond_the_scratch_array():
    s = shard(12)                                  # D_r = 1536
    T, S = 8192, 2                                 # 2 x 8192 x (1536 + 12) x 4 B = 101 MB > 64 MiB
    qkv = torch.zeros((T, 3 * s.d_r), dtype=torch.bfloat16, device="cuda")
    o = torch.full((T, s.d_r), 7.0, dtype=torch.bfloat16, device="cuda")
    assert noalloc_abi(s, T, qkv, S, o) == tp.TP_ERR_ARG
    assert "scratch" in tp.tp_last_error_detail() and "maximum" in tp.tp_last_error_detail()
    torch.cuda.synchronize()
    assert bool((o.float() == 7.0).all())          # nothing was launched
    s.close()
