"""GPU parity of attention on the inputs that force its special paths
(Diffusers TP page, §Colwise e rowwise: each rank runs plain per-head
attention over its own heads), against the float64 oracle:

* "growing": a row's scores rise by about 12 log2 units from each 64-key tile
  to the next (other rows of the same wave rise by 6, stay flat or fall), so
  every tile of the rising rows outgrows the running max by more than the
  kernels' 8-unit slack and the accumulator, already holding the earlier
  tiles, is rescaled -- an error in how the rescale is applied would leave
  the earlier tiles' weight about 2^12 too large;
* "dominant": one key scores over 20 log2 units above every other, in a
  middle tile, so the output is that key's value row;
* "zero_q": Q = 0, every score 0, so the output is the column mean of V.

Each runs through the 4-wave kernel (fewer than 192 workgroups of 256
queries) and the pipelined one (at least 192), key splits in one launch plus
the merge, and the block form (fp32 output and log-sum-exp, the Ring
Attention step) whole and split.  Outputs within 2e-2 of max|ref|,
log-sum-exps within 5e-3 absolute."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import tensor_dit_transformer_amd as tp
import tp_harness as H
import tp_inputs
from tp_inputs import Workload

pytestmark = pytest.mark.gpu
LSE_ATOL = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def attn_shard(heads_r):
    w = Workload(f"attn_H{2 * heads_r}_P2", 8, 2 * heads_r * 128, 2 * heads_r, 128, 0, 2, "bf16")
    return H.create_shards(w, tp_inputs.make_inputs(w, seed=2), ranks=(0,))[0]


def edge_qkv(T, heads, kind):
    v, b = tp_inputs.attention_edge_qkv(T, heads, kind, seed=7)
    return v.astype(np.float64), torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()


def rows_of(T):
    return np.arange(T) if T <= 1200 else tp_inputs.sample_rows(T, 64, seed=8)


def check_special(kind, o_rows, qkv, rows, Dr, heads):
    """The closed forms the cases are built for, on top of the oracle."""
    v = qkv[:, 2 * Dr:]
    if kind == "zero_q":
        np.testing.assert_allclose(o_rows, np.broadcast_to(v.mean(axis=0), o_rows.shape),
                                   atol=2e-2 * np.max(np.abs(v.mean(axis=0))))
    if kind == "dominant":
        j = tp_inputs.dominant_key(qkv.shape[0])
        np.testing.assert_allclose(o_rows, np.broadcast_to(v[j], o_rows.shape),
                                   atol=2e-2 * np.max(np.abs(v[j])))


@pytest.mark.parametrize("kind", tp_inputs.EDGE_KINDS)
@pytest.mark.parametrize("T,heads", [(1000, 3), (4000, 12)], ids=["4wave", "pipelined"])
def test_attn_heads_edge_cases(kind, T, heads):
    s = attn_shard(heads)
    Dr = s.d_r
    qv, qd = edge_qkv(T, heads, kind)
    o = torch.empty((T, Dr), dtype=torch.bfloat16, device="cuda")
    tp.tp_attn_heads(s, T, qd, o)
    torch.cuda.synchronize()
    rows = rows_of(T)
    ref = O.to_bf16_rne(O.attention_rows(qv[rows, :Dr], qv[:, Dr:2 * Dr], qv[:, 2 * Dr:], heads, 128))
    got = H.as_f64(o[rows])
    e = H.rel_err(got, ref)
    say(f"{kind} T={T} heads={heads}: {e:.2e}")
    assert e <= H.TOL["bf16"]
    check_special(kind, got, qv, rows, Dr, heads)
    torch.cuda.synchronize()
    s.close()


@pytest.mark.parametrize("kind", tp_inputs.EDGE_KINDS)
def test_attn_heads_split_edge_cases(kind):
    T, heads = 4608, 6           # the split hint gives 2 key ranges (216 workgroups)
    s = attn_shard(heads)
    Dr = s.d_r
    S = tp.tp_attn_split_hint(s, T)
    assert S == 2
    qv, qd = edge_qkv(T, heads, kind)
    o_parts = torch.empty((S, T, Dr), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((S, T, heads), dtype=torch.float32, device="cuda")
    o = torch.empty((T, Dr), dtype=torch.bfloat16, device="cuda")
    tp.tp_attn_heads_split(s, T, qd, o_parts, l_parts)
    tp.tp_attn_merge(list(o_parts), list(l_parts), o, heads, 128)
    torch.cuda.synchronize()
    rows = rows_of(T)
    q, k, v = qv[rows, :Dr], qv[:, Dr:2 * Dr], qv[:, 2 * Dr:]
    for z in range(S):           # each key range on its own
        a, b = z * T // S, (z + 1) * T // S
        o_ref, l_ref = O.attention_block(q, k[a:b], v[a:b], heads, 128)
        e_o = H.rel_err(H.as_f64(o_parts[z][rows]), o_ref)
        e_l = float(np.max(np.abs(H.as_f64(l_parts[z][rows]) - l_ref)))
        say(f"{kind} split {z}: o {e_o:.2e} lse {e_l:.2e}")
        assert e_o <= H.TOL["bf16"] and e_l <= LSE_ATOL
    ref = O.to_bf16_rne(O.attention_rows(q, k, v, heads, 128))
    e = H.rel_err(H.as_f64(o[rows]), ref)
    say(f"{kind} merged: {e:.2e}")
    assert e <= H.TOL["bf16"]
    check_special(kind, H.as_f64(o[rows]), qv, rows, Dr, heads)
    torch.cuda.synchronize()
    s.close()


@pytest.mark.parametrize("kind", tp_inputs.EDGE_KINDS)
@pytest.mark.parametrize("Tq,Tkv,heads,S", [(777, 3000, 3, 1), (4096, 2000, 12, 1),
                                            (1000, 3000, 6, 3), (2048, 4000, 12, 2)],
                         ids=["4wave", "pipelined", "4wave_split3", "pipelined_split2"])
def test_block_attention_edge_cases(kind, Tq, Tkv, heads, S):
    s = attn_shard(heads)
    Dr = s.d_r
    # queries and keys from two packed tensors of their own lengths, drawn with
    # the same per-head directions (same seed)
    qv, qd = edge_qkv(Tq, heads, kind)
    kv, kd = edge_qkv(Tkv, heads, kind)
    rows = rows_of(Tq)
    q, k, v = qv[rows, :Dr], kv[:, Dr:2 * Dr], kv[:, 2 * Dr:]
    if S == 1:
        o = torch.empty((Tq, Dr), dtype=torch.float32, device="cuda")
        lse = torch.empty((Tq, heads), dtype=torch.float32, device="cuda")
        tp.tp_attn_heads_block(s, Tq, qd, Tkv, kd, o, lse)
        parts = [(o, lse, 0, Tkv)]
    else:
        o_parts = torch.empty((S, Tq, Dr), dtype=torch.float32, device="cuda")
        l_parts = torch.empty((S, Tq, heads), dtype=torch.float32, device="cuda")
        tp.tp_attn_heads_block_split(s, Tq, qd, Tkv, kd, o_parts, l_parts)
        parts = [(o_parts[z], l_parts[z], z * Tkv // S, (z + 1) * Tkv // S) for z in range(S)]
    torch.cuda.synchronize()
    for i, (o_, l_, a, b) in enumerate(parts):
        o_ref, l_ref = O.attention_block(q, k[a:b], v[a:b], heads, 128)
        e_o = H.rel_err(H.as_f64(o_[rows]), o_ref)
        e_l = float(np.max(np.abs(H.as_f64(l_[rows]) - l_ref)))
        say(f"{kind} block Tq={Tq} keys [{a},{b}) heads={heads}: o {e_o:.2e} lse {e_l:.2e}")
        assert e_o <= H.TOL["bf16"] and e_l <= LSE_ATOL
        if kind != "growing" and S == 1:
            check_special(kind, H.as_f64(o_[rows]), kv, np.arange(Tkv), Dr, heads)
    torch.cuda.synchronize()
    s.close()
