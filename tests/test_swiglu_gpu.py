"""GPU parity of the SwiGLU MLP and the packed (fused) projections against the
float64 oracle: [1, 1] gate/up colwise with the in-register SwiGLU epilogue,
the single-stream block created from one packed input projection
(Q, K, V, gate, up; blocks [1, 1, 1, 3, 3] at mlp_ratio 3) and one packed
output projection over [inner_dim, mlp_hidden_dim] (Diffusers TP page,
§Projeções fundidas), on every GEMM path (fp32 VALU, bf16 128x128 with a K
tail, bf16 256x256 8-wave), ragged token counts, and the two-launch form of
the fused call.  Tolerances: 1e-4 (fp32), 2e-2 (bf16) relative to max|ref|."""
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


def rank_refs(w: Workload, inp):
    v = inp.values
    return [O.rank_forward(v["x"], v, w.tp_degree, r, w.num_heads, w.head_dim,
                           w.dtype == "bf16", mlp_act="swiglu") for r in range(w.tp_degree)]


def run(w: Workload, inp, fused=True, packed=False):
    shards = H.create_shards(w, inp, packed=packed)
    x = H.to_device(inp, "x")
    outs = []
    for s in shards:
        b = H.RankBuffers(s, w.tokens)
        H.run_rank(s, x, b, fused=fused)
        outs.append(b)
    torch.cuda.synchronize()
    return shards, outs


def close(shards):
    torch.cuda.synchronize()
    for s in shards:
        s.close()


def check(buf, ref, tol, what):
    errs = {}
    if buf.qkv is not None:
        errs["qkv_r"] = H.rel_err(H.as_f64(buf.qkv), ref["qkv_r"])
        errs["o_r"] = H.rel_err(H.as_f64(buf.o), ref["o_r"])
    errs["h_r"] = H.rel_err(H.as_f64(buf.h), ref["h_r"])
    errs["partial_r"] = H.rel_err(H.as_f64(buf.partial), ref["p_block"])
    say(what, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= tol, f"{what} {k}: {v:.3e} > {tol}"


F32_MLP = Workload("swiglu_mlp_f32_T70_D256_F1024_P2", 70, 256, 0, 0, 1024, 2, "f32",
                   mlp_act="swiglu")


def test_fp32_swiglu_mlp_both_ranks_and_reduce():
    w = F32_MLP
    inp = tp_inputs.make_inputs(w, seed=5)
    refs = rank_refs(w, inp)
    shards, outs = run(w, inp)
    for r, (b, ref) in enumerate(zip(outs, refs)):
        check(b, ref, H.TOL["f32"], f"f32 SwiGLU rank {r}")
    y = torch.empty((w.tokens, w.hidden), dtype=torch.float32, device="cuda")
    tp.tp_partial_reduce([b.partial for b in outs], H.rowwise_biases(w, inp), y)
    torch.cuda.synchronize()
    full = O.block_unsharded(inp["x"], inp.values, 0, 0, bf16=False, mlp_act="swiglu")["y"]
    e = H.rel_err(H.as_f64(y), full)
    say("f32 SwiGLU y vs unsharded", f"{e:.2e}")
    assert e <= H.TOL["f32"]
    close(shards)


# 3 * D_r = 48 is not a multiple of 64: the fused call runs as two launches.
F32_UNALIGNED = Workload("swiglu_f32_T65_D32_H4d8_F128_P2", 65, 32, 4, 8, 128, 2, "f32",
                         mlp_act="swiglu")


def test_fp32_fused_colwise_two_launch_form():
    w = F32_UNALIGNED
    inp = tp_inputs.make_inputs(w, seed=6)
    refs = rank_refs(w, inp)
    shards = H.create_shards(w, inp)
    x = H.to_device(inp, "x")
    for r, s in enumerate(shards):
        qkv = torch.empty((w.tokens, 3 * s.d_r), dtype=torch.float32, device="cuda")
        h = torch.empty((w.tokens, s.f_r), dtype=torch.float32, device="cuda")
        tp.tp_colwise_qkv_up(s, w.tokens, x, qkv, h)
        torch.cuda.synchronize()
        e_q = H.rel_err(H.as_f64(qkv), refs[r]["qkv_r"])
        e_h = H.rel_err(H.as_f64(h), refs[r]["h_r"])
        say(f"f32 unaligned fused rank {r}: qkv {e_q:.2e} h {e_h:.2e}")
        assert e_q <= H.TOL["f32"] and e_h <= H.TOL["f32"]
    close(shards)


MID = Workload("swiglu_block_T777_D512_H4_F1536_P2", 777, 512, 4, 128, 1536, 2, "bf16",
               mlp_act="swiglu")


@pytest.mark.parametrize("fused", [True, False])
def test_mid_bf16_swiglu_block_ragged(fused):
    w = MID
    inp = tp_inputs.make_inputs(w, seed=7)
    refs = rank_refs(w, inp)
    shards, outs = run(w, inp, fused=fused)
    for r, (b, ref) in enumerate(zip(outs, refs)):
        check(b, ref, H.TOL["bf16"], f"MID SwiGLU rank {r} fused={fused}")
    close(shards)


def test_fused_swiglu_bitwise_equal_to_separate_calls():
    w = MID
    inp = tp_inputs.make_inputs(w, seed=8)
    shards, a = run(w, inp, fused=True)
    close(shards)
    shards, b = run(w, inp, fused=False)
    for x, z in zip(a, b):
        assert torch.equal(x.qkv, z.qkv) and torch.equal(x.oh, z.oh)
    close(shards)


@pytest.mark.parametrize("T", [1, 63, 65, 300])
def test_bf16_swiglu_mlp_k_tail_small_tokens(T):
    """hidden 200 is not a multiple of 64 (the K tail of the 128x128 kernel)."""
    w = Workload(f"swiglu_mlp_T{T}_D200_F256_P2", T, 200, 0, 0, 256, 2, "bf16", mlp_act="swiglu")
    inp = tp_inputs.make_inputs(w, seed=9)
    refs = rank_refs(w, inp)
    shards, outs = run(w, inp)
    for r, (b, ref) in enumerate(zip(outs, refs)):
        check(b, ref, H.TOL["bf16"], f"T={T} D=200 SwiGLU rank {r}")
    close(shards)


BIG = Workload("swiglu_block_T2048_D1024_H8_F4096_P2", 2048, 1024, 8, 128, 4096, 2, "bf16",
               mlp_act="swiglu")


def test_bf16_swiglu_block_on_the_8wave_path():
    """Fused colwise N = 3*512 + 2*2048 = 5632 columns, 8 x 22 tiles of 256:
    the 8-wave ping-pong kernel with the SwiGLU epilogue."""
    w = BIG
    inp = tp_inputs.make_inputs(w, seed=10)
    refs = rank_refs(w, inp)
    shards, outs = run(w, inp)
    for r, (b, ref) in enumerate(zip(outs, refs)):
        check(b, ref, H.TOL["bf16"], f"BIG SwiGLU rank {r}")
    close(shards)


def test_bf16_swiglu_persistent_gemm_all_columns():
    """MLP-only, P = 1, T = 2248: the gate/up projection has N = 2 x 8192
    columns, all SwiGLU (9 x 64 = 576 tiles of 256 x 256), so the
    one-wave-per-SIMD kernel runs persistent (256 workgroups, a last round of
    64 tiles) with the SwiGLU epilogue; the ragged last tile row stores 200
    of its 256 rows."""
    w = Workload("swiglu_mlp_T2248_D1024_F8192_P1", 2248, 1024, 0, 0, 8192, 1, "bf16",
                 mlp_act="swiglu")
    inp = tp_inputs.make_inputs(w, seed=12)
    refs = rank_refs(w, inp)
    shards, outs = run(w, inp)
    for r, (b, ref) in enumerate(zip(outs, refs)):
        check(b, ref, H.TOL["bf16"], f"persistent SwiGLU rank {r}")
    close(shards)


@pytest.mark.parametrize("T", [2100, 2300])
def test_bf16_swiglu_8wave_ragged_rows(T):
    """The same block at T = 2100 (9 x 22 = 198 tiles of 256 rows, 242 of
    192: 192-row tiles, the second wave group of the last tile row holds 84
    of its 96 rows) and T = 2300 (264 tiles of 192 rows would need two
    rounds: 256-row tiles, 124 of 128 rows): the SwiGLU epilogue's row test."""
    w = Workload(f"swiglu_block_T{T}_D1024_H8_F4096_P2", T, 1024, 8, 128, 4096, 2, "bf16",
                 mlp_act="swiglu")
    inp = tp_inputs.make_inputs(w, seed=11)
    refs = rank_refs(w, inp)
    shards, outs = run(w, inp)
    for r, (b, ref) in enumerate(zip(outs, refs)):
        check(b, ref, H.TOL["bf16"], f"SwiGLU T={T} rank {r}")
    close(shards)


def test_single_stream_from_packed_checkpoint():
    """Shards created from one fused input projection and one fused output
    projection (pointers into the blocks, the output projection's row
    stride): every rank against the oracle's packed single-stream rank, and
    the reduced output against the unsharded single-stream block."""
    w = dataclasses.replace(MID, name="single_T777_D512_H4_F1536_P2", tokens=777)
    inp = tp_inputs.make_inputs(w, seed=11)
    v = inp.values
    packed = H.packed_host_weights(inp)
    widen = tp_inputs.bits_to_f32
    w_in, b_in, w_out = widen(packed["w_in"]), widen(packed["b_in"]), widen(packed["w_out"])
    HD, F = w.num_heads * w.head_dim, w.ffn
    shards, outs = run(w, inp, packed=True)
    for r, b in enumerate(outs):
        ref = O.single_stream_rank(v["x"], w_in, b_in, w_out, w.tp_degree, r, w.num_heads,
                                   w.head_dim, F, bf16=True)
        check(b, {"qkv_r": ref["qkv_r"], "o_r": ref["o_r"], "h_r": ref["h_r"],
                  "p_block": ref["partial"]}, H.TOL["bf16"], f"packed single-stream rank {r}")
    y = torch.empty((w.tokens, w.hidden), dtype=torch.float32, device="cuda")
    b_out = torch.from_numpy(np.ascontiguousarray(v["b_o"])).cuda()
    tp.tp_partial_reduce([b.partial for b in outs], [b_out], y)
    torch.cuda.synchronize()
    full = O.single_stream_block(v["x"], w_in, b_in, w_out, v["b_o"], w.num_heads, w.head_dim, F,
                                 bf16=True)["y"]
    e = H.rel_err(H.as_f64(y), full)
    say(f"packed single-stream y vs unsharded: {e:.2e}")
    assert e <= H.TOL["bf16"]
    close(shards)


def test_packed_and_separate_creation_give_identical_results():
    w = MID
    inp = tp_inputs.make_inputs(w, seed=12)
    shards, a = run(w, inp, packed=True)
    close(shards)
    shards, b = run(w, inp, packed=False)
    for x, z in zip(a, b):
        assert torch.equal(x.qkv, z.qkv) and torch.equal(x.oh, z.oh)
        assert torch.equal(x.partial, z.partial)
    close(shards)
