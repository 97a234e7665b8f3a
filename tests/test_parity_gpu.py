"""GPU parity: every output of the C ABI (qkv_r, o_r, h_r, partial_r and the
reduced y) against the float64 CPU oracle on the same seeded inputs, at the
tolerance max|gpu - ref| / max|ref| <= 1e-4 (fp32) or 2e-2 (bf16).

The check recipe is the Diffusers TP page's own (§Restrições e verificação):
run the same seeded inputs unsharded and under tensor parallelism and compare
numerically, since a misplaced colwise/rowwise still runs.
"""
import os
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


def full_oracle(w: Workload, inp):
    vals = inp.values
    bf16 = w.dtype == "bf16"
    ranks = [O.rank_forward(vals["x"], vals, w.tp_degree, r, w.num_heads, w.head_dim, bf16)
             for r in range(w.tp_degree)]
    y = O.partial_reduce([r["p_block"] for r in ranks], O.rowwise_bias(vals))
    return ranks, y


def run_all_ranks(w: Workload, inp, fused=True):
    shards = H.create_shards(w, inp)
    x = H.to_device(inp, "x")
    T = w.tokens
    outs = []
    partials = []
    for s in shards:
        buf = H.RankBuffers(s, T)
        H.run_rank(s, x, buf, fused=fused)
        partials.append(buf.partial)
        outs.append(buf)
    y = torch.empty((T, w.hidden), dtype=torch.float32, device="cuda")
    tp.tp_partial_reduce(partials, H.rowwise_biases(w, inp), y)
    torch.cuda.synchronize()
    return shards, outs, y


def close_all(shards):
    torch.cuda.synchronize()
    for s in shards:
        s.close()


def check_rank(w, buf, ref, tol, what=""):
    errs = {}
    if buf.qkv is not None:
        errs["qkv_r"] = H.rel_err(H.as_f64(buf.qkv), ref["qkv_r"])
        errs["o_r"] = H.rel_err(H.as_f64(buf.o), ref["o_r"])
    if buf.h is not None:
        errs["h_r"] = H.rel_err(H.as_f64(buf.h), ref["h_r"])
    errs["partial_r"] = H.rel_err(H.as_f64(buf.partial), ref["p_block"])
    say(what, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= tol, f"{what} {k}: {v:.3e} > {tol}"


# ------------------------------------------------------------------ small/mid, full compare

def test_c1_fp32_mlp_both_ranks_reduce_equals_unsharded():
    w = tp_inputs.C1
    inp = tp_inputs.make_inputs(w, seed=0)
    ranks, y_ref = full_oracle(w, inp)
    unsharded = O.block_unsharded(inp["x"], inp.values, 0, 0, bf16=False)["y"]
    shards, outs, y = run_all_ranks(w, inp)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["f32"], f"C1 rank {r}")
    e = H.rel_err(H.as_f64(y), unsharded)
    say("C1 y vs unsharded", e)
    assert e <= H.TOL["f32"]
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["f32"]
    close_all(shards)


MID = Workload("mid_block_T777_D512_H4_F2048_P2", 777, 512, 4, 128, 2048, 2, "bf16")


@pytest.mark.parametrize("fused", [True, False])
def test_mid_bf16_block_ragged_all_outputs(fused):
    w = MID
    inp = tp_inputs.make_inputs(w, seed=3)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp, fused=fused)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["bf16"], f"MID rank {r} fused={fused}")
    unsharded = O.block_unsharded(inp["x"], inp.values, w.num_heads, w.head_dim, bf16=True)["y"]
    e = H.rel_err(H.as_f64(y), unsharded)
    say("MID y vs unsharded", e)
    assert e <= H.TOL["bf16"]
    close_all(shards)


def test_fused_qkv_up_is_bitwise_equal_to_separate_calls():
    w = MID
    inp = tp_inputs.make_inputs(w, seed=4)
    shards, a, _ = run_all_ranks(w, inp, fused=True)
    close_all(shards)
    shards, b, _ = run_all_ranks(w, inp, fused=False)
    for x, z in zip(a, b):
        assert torch.equal(x.qkv, z.qkv)
        assert torch.equal(x.oh, z.oh)
    close_all(shards)


def test_block_out_equals_attn_out_plus_mlp_down_accumulate():
    w = MID
    inp = tp_inputs.make_inputs(w, seed=5)
    shards, outs, _ = run_all_ranks(w, inp)
    s, buf = shards[1], outs[1]
    T = w.tokens
    p2 = torch.empty_like(buf.partial)
    tp.tp_rowwise_linear_partial(s, tp.TP_ATTN_OUT, T, buf.o, p2)
    tp.tp_rowwise_linear_partial(s, tp.TP_MLP_DOWN, T, buf.h, p2, accumulate=True)
    torch.cuda.synchronize()
    assert H.rel_err(H.as_f64(p2), H.as_f64(buf.partial)) < 1e-5
    close_all(shards)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 129, 300])
def test_small_and_ragged_token_counts(T):
    w = Workload(f"small_T{T}", T, 256, 2, 128, 512, 2, "bf16")
    inp = tp_inputs.make_inputs(w, seed=T)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["bf16"], f"T={T} rank {r}")
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    if T == 1:  # one token attends to itself: o = v exactly (softmax weight 1)
        Dr = shards[0].d_r
        assert torch.equal(outs[0].o, outs[0].qkv[:, 2 * Dr:])
    close_all(shards)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_k_not_multiple_of_tile_and_single_rank(dtype):
    # MLP-only, P = 1 (the shard is the whole layer), K = 264 and 520: both
    # GEMMs take the zero-filled K-tail path.
    w = Workload(f"ktail_{dtype}", 200, 264, 0, 0, 520, 1, dtype)
    inp = tp_inputs.make_inputs(w, seed=11)
    ranks, y_ref = full_oracle(w, inp)
    unsharded = O.block_unsharded(inp["x"], inp.values, 0, 0, bf16=dtype == "bf16")["y"]
    shards, outs, y = run_all_ranks(w, inp)
    check_rank(w, outs[0], ranks[0], H.TOL[dtype], f"ktail {dtype}")
    assert H.rel_err(H.as_f64(y), unsharded) <= H.TOL[dtype]
    close_all(shards)


# Shapes large enough (>= 256 output tiles of 256 x 256, K % 64 == 0) for the
# 8-wave direct-to-LDS GEMM, with a ragged token count.
BIG_FUSED = Workload("big_fused_T2125_D1024_H8_F16384_P2", 2125, 1024, 8, 128, 16384, 2, "bf16")


def test_large_fused_colwise_and_attention_paths():
    w = BIG_FUSED   # fused QKV+up: N = 3*512 + 8192 = 9728 -> 9 x 38 tiles
    inp = tp_inputs.make_inputs(w, seed=21)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["bf16"], f"BIG_FUSED rank {r}")
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    close_all(shards)


def test_large_ragged_rows_in_the_second_wave_group():
    # T = 2248 = 8 x 256 + 200: in the last tile row of the 8-wave GEMM the
    # first wave group (rows 0-127) is whole and takes the untested store
    # copy, the second (rows 128-199 of 256) stores only its rows below M.
    # Fused colwise (bf16 + GELU, split output) and packed rowwise (fp32).
    w = Workload("big_fused_T2248_D1024_H8_F16384_P2", 2248, 1024, 8, 128, 16384, 2, "bf16")
    inp = tp_inputs.make_inputs(w, seed=24)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["bf16"], f"T2248 rank {r}")
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    close_all(shards)


def test_192_row_tiles_with_ragged_rows():
    # M = 4000, N = 2304 (QKV of 6 heads of 128): 16 x 9 = 144 tiles of 256
    # rows leave CUs idle in one round, so the GEMM takes 192-row tiles (21 x 9
    # = 189); 4000 = 20 x 192 + 160, so in the last tile row group 0 (rows
    # 0-95) is whole and group 1 stores 64 of its 96 rows.  The attention-out
    # GEMM (N = 3072, K = 768) takes them too (21 x 12 = 252 tiles).
    w = Workload("qkv_T4000_D3072_H24_P4", 4000, 3072, 24, 128, 0, 4, "bf16")
    inp = tp_inputs.make_inputs(w, seed=25)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["bf16"], f"T4000 rank {r}")
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    # fp32 accumulate form of the same 192-row out-projection, twice onto zeros
    p2 = torch.zeros_like(outs[0].partial)
    o = outs[0].o
    for _ in range(2):
        tp.tp_rowwise_linear_partial(shards[0], tp.TP_ATTN_OUT, w.tokens, o, p2, accumulate=True)
    torch.cuda.synchronize()
    assert H.rel_err(H.as_f64(p2), 2 * ranks[0]["p_block"]) <= H.TOL["bf16"]
    close_all(shards)


def test_192_row_tiles_with_gelu_epilogue():
    # MLP up-projection M = 4000, N = 9216 / 4 = 2304: 144 tiles of 256 rows,
    # 189 of 192, so the GELU epilogue runs on 192-row tiles with a ragged
    # last tile row.
    w = Workload("mlp_T4000_D1024_F9216_P4", 4000, 1024, 0, 0, 9216, 4, "bf16")
    inp = tp_inputs.make_inputs(w, seed=26)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["bf16"], f"T4000 MLP rank {r}")
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    close_all(shards)


def test_288_row_tiles_gelu_store_and_accumulate_with_ragged_edges():
    # MLP shard M = 4408 = 15 x 288 + 88, up N = 12032 / 4 = 3008 = 15 x 192
    # + 128, down N = 3072, K = 3072 / 3008: 16 x 16 = 256 tiles of 288 x 192
    # against 216 of 256 x 256, so both GEMMs take the 16x16-MFMA 288-row
    # kernel.  In the last tile row wave group 0 stores 88 of its 144 rows
    # and group 1 none; in the up-projection's last tile column waves 0-1
    # store all 48 columns, wave 2 32 and wave 3 none.  GELU bf16 store, fp32
    # store, and the fp32 accumulate form twice onto zeros.
    w = Workload("mlp288_T4408_D3072_F12032_P4", 4408, 3072, 0, 0, 12032, 4, "bf16")
    inp = tp_inputs.make_inputs(w, seed=28)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["bf16"], f"{w.name} rank {r}")
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    p2 = torch.zeros_like(outs[1].partial)
    for _ in range(2):
        tp.tp_rowwise_linear_partial(shards[1], tp.TP_MLP_DOWN, w.tokens, outs[1].h, p2, accumulate=True)
    torch.cuda.synchronize()
    assert H.rel_err(H.as_f64(p2), 2 * ranks[1]["p_block"]) <= H.TOL["bf16"]
    close_all(shards)


def test_288_row_tiles_fused_colwise_split_and_block_out():
    # Block shard at M = 4408: the fused colwise launch (N = 2304 + 3008 =
    # 5312, 448 tiles of 288 x 192 against 378 of 256 x 256 in two rounds)
    # splits its output at column 2304 (qkv | h, GELU from there on), and the
    # packed rowwise out (N = 3072, K = 768 + 3008 = 3776) takes the same
    # kernel with the fp32 store.
    w = Workload("block288_T4408_D3072_H24_F12032_P4", 4408, 3072, 24, 128, 12032, 4, "bf16")
    inp = tp_inputs.make_inputs(w, seed=29)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    for r, (buf, ref) in enumerate(zip(outs, ranks)):
        check_rank(w, buf, ref, H.TOL["bf16"], f"{w.name} rank {r}")
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    close_all(shards)


def test_persistent_gemm_several_tiles_per_workgroup_gelu_all_columns():
    # MLP-only, P = 1: the up-projection (N = 16384, M = 2248 = 8 x 256 + 200,
    # K = 1024) has 9 x 64 = 576 tiles of 256 x 256 with GELU on every
    # column, so the one-wave-per-SIMD kernel runs persistent: 256
    # workgroups, two full rounds and a last one of 64 tiles, each workgroup
    # loading its next tile's first K tiles before storing the current one.
    w = Workload("persist_mlp_T2248_D1024_F16384_P1", 2248, 1024, 0, 0, 16384, 1, "bf16")
    inp = tp_inputs.make_inputs(w, seed=31)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    check_rank(w, outs[0], ranks[0], H.TOL["bf16"], w.name)
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    close_all(shards)


@pytest.mark.parametrize("tokens", [2048, 2248])
@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_one_wave_gemm_activation_boundary_inside_a_wave(act, tokens):
    # Fused colwise with head_dim 32 and hidden 1088 (34 heads, P = 1): qkv
    # takes columns [0, 3264) and the activation starts at column 3264 =
    # 25.5 x 128, inside a 128-column wave block.  N = 3264 + 4928 (GELU) or
    # 3264 + 2 x 2464 (SwiGLU gate/up) = 8192 and K = 1088, so the
    # one-wave-per-SIMD kernel runs, and for that wave its epilogue chooses
    # the activation and the output (qkv or h) per 32-column block (SwiGLU: a
    # plain pair, then a gate/up pair).  M = 2048 gives exactly 256 tiles of
    # 256 x 256, one per workgroup; M = 2248 gives 288 (the last tile row
    # ragged) on the persistent grid.  Only the colwise call: attention is
    # built for head_dim 128.
    F = 4928 if act == "gelu_tanh" else 2464
    w = Workload(f"fix0_{act}_T{tokens}_D1088_H34d32_F{F}_P1", tokens, 1088, 34, 32, F, 1, "bf16",
                 mlp_act=act)
    inp = tp_inputs.make_inputs(w, seed=32)
    ref = O.rank_forward(inp.values["x"], inp.values, 1, 0, 34, 32, True, mlp_act=act)
    shards = H.create_shards(w, inp)
    x = H.to_device(inp, "x")
    s = shards[0]
    qkv = torch.empty((w.tokens, 3 * s.d_r), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((w.tokens, s.f_r), dtype=torch.bfloat16, device="cuda")
    tp.tp_colwise_qkv_up(s, w.tokens, x, qkv, h)
    torch.cuda.synchronize()
    e_q = H.rel_err(H.as_f64(qkv), ref["qkv_r"])
    e_h = H.rel_err(H.as_f64(h), ref["h_r"])
    say(w.name, f"qkv {e_q:.2e} h {e_h:.2e}")
    assert e_q <= H.TOL["bf16"] and e_h <= H.TOL["bf16"]
    close_all(shards)


def test_large_rowwise_store_and_accumulate_paths():
    # MLP-only, P = 1, hidden 8192: the down projection is N = 8192 -> 9 x 32 =
    # 288 tiles, on 256 persistent workgroups (a last round of 32 tiles)
    w = Workload("big_down_T2125_D8192_F1024_P1", 2125, 8192, 0, 0, 1024, 1, "bf16")
    inp = tp_inputs.make_inputs(w, seed=22)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    check_rank(w, outs[0], ranks[0], H.TOL["bf16"], "BIG_DOWN")
    p2 = torch.zeros_like(outs[0].partial)
    tp.tp_rowwise_linear_partial(shards[0], tp.TP_MLP_DOWN, w.tokens, outs[0].h, p2, accumulate=True)
    tp.tp_rowwise_linear_partial(shards[0], tp.TP_MLP_DOWN, w.tokens, outs[0].h, p2, accumulate=True)
    torch.cuda.synchronize()
    assert H.rel_err(H.as_f64(p2), 2 * ranks[0]["p_block"]) <= H.TOL["bf16"]
    close_all(shards)


def test_four_wave_256_tiles_with_k_tail():
    # hidden = ffn = 4104 = 64 x 64 + 8: K % 64 != 0 for both GEMMs, with
    # 18 x 17 = 306 tiles of 256 x 256 (at least 256), so both take the 4-wave
    # 256 x 256 register-staged kernel with the zero-filled K tail: the
    # up-projection's GELU bf16 store, the down-projection's fp32 store, and
    # the fp32 accumulate form.
    w = Workload("ktail256_T4608_D4104_F4104_P1", 4608, 4104, 0, 0, 4104, 1, "bf16")
    inp = tp_inputs.make_inputs(w, seed=27)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    check_rank(w, outs[0], ranks[0], H.TOL["bf16"], w.name)
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    p2 = torch.zeros_like(outs[0].partial)
    for _ in range(2):
        tp.tp_rowwise_linear_partial(shards[0], tp.TP_MLP_DOWN, w.tokens, outs[0].h, p2, accumulate=True)
    torch.cuda.synchronize()
    assert H.rel_err(H.as_f64(p2), 2 * ranks[0]["p_block"]) <= H.TOL["bf16"]
    close_all(shards)


@pytest.mark.parametrize("w", [
    # up-projection N = 8288 = 32 x 256 + 96: 9 x 33 tiles on the 8-wave kernel,
    # the last tile column partly past N
    Workload("ragged_up_T2125_D1024_F8288_P1", 2125, 1024, 0, 0, 8288, 1, "bf16"),
    # down-projection N = 8352 = 32 x 256 + 160 on the 8-wave kernel; the
    # up-projection's K = 8352 is not a multiple of 64 (zero-filled tail)
    Workload("ragged_down_T2125_D8352_F1024_P1", 2125, 8352, 0, 0, 1024, 1, "bf16"),
], ids=lambda w: w.name)
def test_large_ragged_n_paths(w):
    inp = tp_inputs.make_inputs(w, seed=23)
    ranks, y_ref = full_oracle(w, inp)
    shards, outs, y = run_all_ranks(w, inp)
    check_rank(w, outs[0], ranks[0], H.TOL["bf16"], w.name)
    assert H.rel_err(H.as_f64(y), y_ref) <= H.TOL["bf16"]
    close_all(shards)


@pytest.mark.parametrize("T,heads", [(5500, 24), (4608, 11), (4608, 6)])
def test_attention_long_sequences_both_workgroup_shapes(T, heads):
    """T=5500 x 24 heads takes the 256-query (8-wave) workgroups with a
    ragged last tile; 4608 x 11 takes them too, 198 workgroups, so the XCD
    work order gives six XCDs one item more than the other two; 4608 x 6
    takes the 128-query ones.  Seeded packed qkv, oracle on sampled query
    rows (each against all keys)."""
    w = Workload(f"attn_T{T}_H{heads}", T, heads * 128, heads, 128, 0, 1, "bf16")
    inp = tp_inputs.make_inputs(w, seed=12, tokens=8)      # weights only matter for create
    s = H.create_shards(dataclass_tokens(w, 8), inp)[0]
    Dr = s.d_r
    qkv_v, qkv_b = tp_inputs.random_matrix((T, 3 * Dr), seed=13, std=1.5)
    qkv = torch.from_numpy(qkv_b.view(np.int16)).view(torch.bfloat16).cuda()
    o = torch.empty((T, Dr), dtype=torch.bfloat16, device="cuda")
    tp.tp_attn_heads(s, T, qkv, o)
    torch.cuda.synchronize()
    rows = tp_inputs.sample_rows(T, 40, seed=14)
    q64 = qkv_v.astype(np.float64)
    ref = O.to_bf16_rne(O.attention_rows(q64[rows, :Dr], q64[:, Dr:2 * Dr], q64[:, 2 * Dr:], heads, 128))
    e = H.rel_err(H.as_f64(o[rows]), ref)
    say(f"attention T={T} heads={heads}: {e:.2e}")
    assert e <= H.TOL["bf16"]
    close_all([s])


def test_zero_tokens_is_a_no_op():
    w = Workload("zero", 8, 256, 2, 128, 512, 2, "bf16")
    inp = tp_inputs.make_inputs(w, seed=1)
    shards = H.create_shards(w, inp)
    x = H.to_device(inp, "x")
    buf = H.RankBuffers(shards[0], 8)
    for t in (buf.qkv, buf.oh, buf.partial):
        t.fill_(7)
    tp.tp_colwise_qkv_up(shards[0], 0, x, buf.qkv, buf.h)
    tp.tp_colwise_linear(shards[0], tp.TP_QKV, 0, x, buf.qkv)
    tp.tp_attn_heads(shards[0], 0, buf.qkv, buf.o)
    tp.tp_rowwise_linear_partial(shards[0], tp.TP_BLOCK_OUT, 0, buf.oh, buf.partial)
    import ctypes
    parts = (ctypes.c_void_p * 1)(buf.partial.data_ptr())
    st = tp.lib().tp_partial_reduce(parts, 1, 256, None, 0, 0, 256, buf.partial.data_ptr(), 256, None)
    assert st == tp.TP_OK
    torch.cuda.synchronize()
    for t in (buf.qkv, buf.oh, buf.partial):
        assert bool((t.float() == 7).all())
    close_all(shards)


def test_reduce_fp32_exact_rank_order_and_aliasing():
    rng = np.random.default_rng(9)
    T, D, P = 1000, 768, 3
    parts = [rng.standard_normal((T, D)).astype(np.float32) for _ in range(P)]
    bias = [rng.standard_normal(D).astype(np.float32) * 0.01 for _ in range(2)]
    ref = O.partial_reduce(parts, bias[0].astype(np.float64) + bias[1])
    dp = [torch.from_numpy(p).cuda() for p in parts]
    db = [torch.from_numpy(b).cuda() for b in bias]
    out = torch.empty((T, D), device="cuda")
    tp.tp_partial_reduce(dp, db, out)
    torch.cuda.synchronize()
    assert H.rel_err(H.as_f64(out), ref) < 1e-6
    # the fp32 rank-order sum is reproduced exactly by numpy in float32
    f32 = ((parts[0] + parts[1]) + parts[2]) + bias[0] + bias[1]
    assert np.array_equal(out.cpu().numpy(), f32)
    # strided partials and output, and in-place into partials[0]
    big = torch.zeros((T, D + 64), device="cuda")
    big[:, :D] = dp[0]
    tp.tp_partial_reduce([big[:, :D]], db[:1], big[:, :D])
    torch.cuda.synchronize()
    assert np.array_equal(big[:, :D].cpu().numpy(), parts[0] + bias[0])
    assert bool((big[:, D:] == 0).all())


def test_deterministic_repeats():
    w = MID
    inp = tp_inputs.make_inputs(w, seed=6)
    shards, first, y0 = run_all_ranks(w, inp)
    x = H.to_device(inp, "x")
    for _ in range(10):
        for s, b0 in zip(shards, first):
            b = H.RankBuffers(s, w.tokens)
            H.run_rank(s, x, b)
            torch.cuda.synchronize()
            assert torch.equal(b.qkv, b0.qkv) and torch.equal(b.oh, b0.oh)
            assert torch.equal(b.partial, b0.partial)
    close_all(shards)


def test_side_stream_gives_identical_results():
    w = MID
    inp = tp_inputs.make_inputs(w, seed=7)
    shards, outs, y = run_all_ranks(w, inp)
    x = H.to_device(inp, "x")
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        b = H.RankBuffers(shards[0], w.tokens)
        H.run_rank(shards[0], x, b)
    st.synchronize()
    assert torch.equal(b.partial, outs[0].partial)
    close_all(shards)


def test_call_errors_enqueue_nothing():
    w = MID
    inp = tp_inputs.make_inputs(w, seed=8, tokens=64)
    shards = H.create_shards(dataclass_tokens(w, 64), inp)
    s = shards[0]
    x = H.to_device(inp, "x")
    buf = H.RankBuffers(s, 64)
    buf.partial.fill_(3)
    with pytest.raises(tp.TpError) as e:             # colwise call with a rowwise layer
        tp.tp_colwise_linear(s, tp.TP_BLOCK_OUT, 64, x, buf.qkv)
    assert e.value.status == tp.TP_ERR_ARG
    raw = torch.empty(64 * 512 + 8, dtype=torch.bfloat16, device="cuda")
    mis = raw[1:1 + 64 * 512].view(64, 512)          # 2-byte offset: misaligned
    with pytest.raises(tp.TpError) as e:
        tp.tp_colwise_linear(s, tp.TP_QKV, 64, mis, buf.qkv)
    assert e.value.status == tp.TP_ERR_ARG
    narrow = torch.empty((64, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):                  # the binding checks shapes
        tp.tp_rowwise_linear_partial(s, tp.TP_BLOCK_OUT, 64, narrow, buf.partial)
    st = tp.lib().tp_rowwise_linear_partial(s.handle, tp.TP_BLOCK_OUT, 64, narrow.data_ptr(), 16,
                                            buf.partial.data_ptr(), buf.partial.stride(0), 0, None)
    assert st == tp.TP_ERR_ARG                       # ld (16) < K_r
    with pytest.raises(tp.TpError) as e:             # o overlapping qkv
        tp.tp_attn_heads(s, 64, buf.qkv, buf.qkv[:, :s.d_r])
    assert e.value.status == tp.TP_ERR_ARG
    with pytest.raises(tp.TpError) as e:             # tokens < 0
        tp.tp_attn_heads(s, -1, buf.qkv, buf.o)
    assert e.value.status == tp.TP_ERR_ARG
    torch.cuda.synchronize()
    assert bool((buf.partial == 3).all())
    f32 = tp_inputs.Workload("f32attn", 64, 256, 2, 128, 0, 1, "f32")
    i32 = tp_inputs.make_inputs(f32, seed=1)
    s32 = H.create_shards(f32, i32)[0]
    b32 = H.RankBuffers(s32, 64)
    with pytest.raises(tp.TpError) as e:             # fp32 attention is not built
        tp.tp_attn_heads(s32, 64, b32.qkv, b32.o)
    assert e.value.status == tp.TP_ERR_UNSUPPORTED
    close_all(shards + [s32])


def dataclass_tokens(w, T):
    import dataclasses
    return dataclasses.replace(w, tokens=T)
