"""GPU parity of the "rowwise_split_input" partial (Diffusers TP page, style
table; §O que deixar de fora: a large AdaLN modulation projection reading
the replicated timestep embedding) against the float64 oracle: every rank of
a modulation-only shard on the few-row kernel (1..64 rows, with and without
a K tail) and on the GEMM (more rows, or an output width the few-row kernel
does not take), the summed partials plus bias against the unsharded
projection, accumulate mode, the full-size modulation projection of the
wide block, and the split-input form of the block's rowwise layers against
the rowwise partial of the sliced input.  Tolerances: 1e-4 (fp32) and 2e-2
(bf16) of max|ref|."""
import dataclasses
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def mod_workload(rows, D, N, P=4, dtype="bf16"):
    return Workload(f"mod_R{rows}_D{D}_N{N}_P{P}_{dtype}", 0, D, 0, 0, 0, P, dtype,
                    mod_rows=rows, mod_out=N)


def run_mod(w, inp, accumulate_twice=False):
    shards = H.create_shards(w, inp)
    c = H.to_device(inp, "c")
    parts = []
    for s in shards:
        p = torch.empty((w.mod_rows, w.mod_out), dtype=torch.float32, device="cuda")
        tp.tp_rowwise_split_input_partial(s, tp.TP_ADALN_MOD, w.mod_rows, c, p)
        if accumulate_twice:
            tp.tp_rowwise_split_input_partial(s, tp.TP_ADALN_MOD, w.mod_rows, c, p, accumulate=True)
        parts.append(p)
    torch.cuda.synchronize()
    return shards, parts


def close(shards):
    torch.cuda.synchronize()
    for s in shards:
        s.close()


@pytest.mark.parametrize("rows,D,N,dtype", [
    (1, 512, 1536, "bf16"), (5, 512, 1536, "bf16"), (16, 512, 1536, "bf16"),
    (17, 512, 1536, "bf16"), (40, 512, 1536, "bf16"),
    (64, 512, 1536, "bf16"),                                  # few-row kernel
    (8, 512, 1552, "bf16"),                                   # N % 32 != 0: one row group
    (8, 160, 1536, "bf16"),                                   # K_r = 40: a k-block tail
    (8, 512, 16 * 773, "bf16"),                               # 773 row groups: more than the
                                                              # workgroup slots, so a few loop twice
    (65, 512, 1536, "bf16"), (200, 512, 1536, "bf16"),        # GEMM
    (8, 512, 264, "bf16"),                                    # N % 16 != 0: GEMM
    (8, 256, 512, "f32"), (70, 256, 512, "f32"),              # fp32 GEMM
])
def test_modulation_ranks_and_reduce(rows, D, N, dtype):
    w = mod_workload(rows, D, N, dtype=dtype)
    inp = tp_inputs.make_inputs(w, seed=13)
    v = inp.values
    tol = H.TOL[dtype]
    shards, parts = run_mod(w, inp)
    for r, p in enumerate(parts):
        e = H.rel_err(H.as_f64(p), O.split_input_rank(v["c"], v["w_mod"], w.tp_degree, r))
        assert e <= tol, f"rank {r}: {e:.3e}"
    y = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    b = torch.from_numpy(np.ascontiguousarray(v["b_mod"], dtype=np.float32)).cuda()
    tp.tp_partial_reduce(parts, [b], y)
    torch.cuda.synchronize()
    ref = O.linear(v["c"], v["w_mod"], v["b_mod"])
    e = H.rel_err(H.as_f64(y), ref)
    say(f"modulation rows={rows} D={D} N={N} {dtype}: y vs unsharded {e:.2e}")
    assert e <= tol
    close(shards)


@pytest.mark.parametrize("rows", [8, 100])
def test_modulation_accumulate_doubles_exactly(rows):
    w = mod_workload(rows, 512, 1536)
    inp = tp_inputs.make_inputs(w, seed=14)
    shards, once = run_mod(w, inp)
    close(shards)
    shards, twice = run_mod(w, inp, accumulate_twice=True)
    for a, b in zip(once, twice):
        assert torch.equal(2 * a, b)
    close(shards)


def test_full_size_modulation_projection():
    """AdaLN modulation of the wide block: 8 conditioning rows, hidden 6144,
    6 x 6144 outputs, tp_degree 4, every rank and the reduce."""
    w = tp_inputs.C8
    inp = tp_inputs.make_inputs(w, seed=0)
    v = inp.values
    shards, parts = run_mod(w, inp)
    for r, p in enumerate(parts):
        e = H.rel_err(H.as_f64(p), O.split_input_rank(v["c"], v["w_mod"], w.tp_degree, r))
        say(f"[modulation 8 x 6144 -> 36864] rank {r}: {e:.2e}")
        assert e <= H.TOL["bf16"]
    y = torch.empty((w.mod_rows, w.mod_out), dtype=torch.float32, device="cuda")
    b = torch.from_numpy(np.ascontiguousarray(v["b_mod"], dtype=np.float32)).cuda()
    tp.tp_partial_reduce(parts, [b], y)
    torch.cuda.synchronize()
    e = H.rel_err(H.as_f64(y), O.linear(v["c"], v["w_mod"], v["b_mod"]))
    say(f"[modulation 8 x 6144 -> 36864] y vs unsharded: {e:.2e}")
    assert e <= H.TOL["bf16"]
    close(shards)


BLOCK = Workload("split_block_T300_D512_H4_F1024_P2", 300, 512, 4, 128, 1024, 2, "bf16")


@pytest.mark.parametrize("T", [40, 300])
def test_block_rowwise_layers_from_replicated_input(T):
    """The block's rowwise layers in split-input form: the rank slices its
    head columns (and hidden columns) out of a replicated full activation.
    Against the oracle's split-input partial, and bitwise against the
    rowwise partial given the same columns as a strided view."""
    w = dataclasses.replace(BLOCK, tokens=T)
    inp = tp_inputs.make_inputs(w, seed=15)
    v = inp.values
    HD, F, D, P = w.num_heads * w.head_dim, w.ffn, w.hidden, w.tp_degree
    full_v, full_b = tp_inputs.random_matrix((T, HD + F), seed=33)
    full = torch.from_numpy(full_b.view(np.int16)).view(torch.bfloat16).cuda()
    w_block = np.concatenate([v["w_o"], v["w_dn"]], axis=1)
    shards = H.create_shards(w, inp)
    for r, s in enumerate(shards):
        outs = {}
        for name, layer, xs, wt in (
                ("attn_out", tp.TP_ATTN_OUT, full[:, :HD], v["w_o"]),
                ("mlp_down", tp.TP_MLP_DOWN, full[:, HD:], v["w_dn"]),
                ("block_out", tp.TP_BLOCK_OUT, full, None)):
            p = torch.empty((T, D), dtype=torch.float32, device="cuda")
            tp.tp_rowwise_split_input_partial(s, layer, T, xs, p)
            torch.cuda.synchronize()
            if layer == tp.TP_BLOCK_OUT:
                cols = O.packed_rowwise_cols([HD, F], P, r)
                ref = O.linear(full_v[:, cols], w_block[:, cols])
            else:
                lo = 0 if layer == tp.TP_ATTN_OUT else HD
                ref = O.split_input_rank(full_v[:, lo:lo + wt.shape[1]], wt, P, r)
            e = H.rel_err(H.as_f64(p), ref)
            say(f"T={T} rank {r} split-input {name}: {e:.2e}")
            assert e <= H.TOL["bf16"]
            outs[name] = p
        # the same columns through the rowwise partial (a strided view)
        p = torch.empty((T, D), dtype=torch.float32, device="cuda")
        tp.tp_rowwise_linear_partial(s, tp.TP_ATTN_OUT, T, full[:, r * s.d_r:(r + 1) * s.d_r], p)
        torch.cuda.synchronize()
        assert torch.equal(p, outs["attn_out"])
    close(shards)
