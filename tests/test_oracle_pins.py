"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself -- a closed form, brute force over explicit index sums, an
independent library routine, or one of the tensor-parallel invariants the
Diffusers TP page states (§Colwise e rowwise, §Projeções fundidas,
§Restrições e verificação).  The pages print no worked numbers, so no check
compares against printed values.  CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn
from scipy.special import erf

import oracle as O

# ---------------------------------------------------------------- bf16 rounding


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(5)
    a = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.4e38, 1e-45], np.float32),
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.to_bf16_rne(a)
    np.testing.assert_array_equal(got, ref)


def test_bf16_rne_ties_go_to_even():
    # 1 + 2^-8 lies exactly halfway between 1 and 1 + 2^-7: rounds to 1 (even).
    assert O.to_bf16_rne(1 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: rounds to the even one.
    assert O.to_bf16_rne(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert O.to_bf16_rne(-(1 + 2.0 ** -8)) == -1.0
    # just above the tie rounds up
    assert O.to_bf16_rne(1 + 2.0 ** -8 + 2.0 ** -20) == 1 + 2.0 ** -7
    assert np.isnan(O.to_bf16_rne(np.nan))
    # already representable values are unchanged
    v = np.array([1.0, -2.5, 0.15625, 3.0 * 2 ** 100])
    np.testing.assert_array_equal(O.to_bf16_rne(v), v)


# ---------------------------------------------------------------- linear


def test_linear_brute_force_index_sum():
    rng = np.random.default_rng(1)
    T, K, N = 4, 8, 6          # non-square so a transposed operand cannot pass
    x = rng.standard_normal((T, K))
    w = rng.standard_normal((N, K))
    b = rng.standard_normal(N)
    got = O.linear(x, w, b)
    assert got.shape == (T, N)
    for t in range(T):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(x[t, k]) * float(w[n, k])
            assert abs(got[t, n] - (acc + b[n])) < 1e-12


def test_linear_matches_torch_linear_fp64():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((37, 50))
    w = rng.standard_normal((23, 50))
    b = rng.standard_normal(23)
    ref = Fnn.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(O.linear(x, w, b), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.linear(x, w), ref - b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- GELU (tanh)


def test_gelu_closed_forms():
    assert O.gelu_tanh(0.0) == 0.0
    u = np.linspace(-9, 9, 2001)
    # tanh is odd, so gelu(u) - gelu(-u) = u exactly (up to rounding)
    np.testing.assert_allclose(O.gelu_tanh(u) - O.gelu_tanh(-u), u, atol=1e-14)
    # asymptotes
    assert abs(O.gelu_tanh(30.0) - 30.0) < 1e-12
    assert abs(O.gelu_tanh(-30.0)) < 1e-12
    # slope 1/2 at the origin: gelu(u) = u/2 + O(u^2)
    eps = 1e-7
    assert abs(O.gelu_tanh(eps) / eps - 0.5) < 1e-6


def test_gelu_matches_torch_tanh_gelu_fp64():
    u = torch.linspace(-12, 12, 100_001, dtype=torch.float64)
    ref = Fnn.gelu(u, approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(u.numpy()), ref, rtol=1e-14, atol=1e-15)


def test_gelu_tanh_close_to_exact_gelu():
    # The tanh form approximates x*Phi(x) to within ~5e-4 absolute; a wrong
    # constant (or sign) in the cubic term breaks this bound.
    u = np.linspace(-8, 8, 20001)
    exact = 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))
    assert np.max(np.abs(O.gelu_tanh(u) - exact)) < 5e-4
    assert np.max(np.abs(O.gelu_tanh(u) - exact)) > 1e-5   # it is an approximation


# ---------------------------------------------------------------- attention


def _sdpa64(q, k, v):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return Fnn.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(3)
    for Tq, Tk, d in ((17, 17, 8), (5, 33, 16), (64, 64, 128)):
        q = rng.standard_normal((Tq, d)) * 2
        k = rng.standard_normal((Tk, d)) * 2
        v = rng.standard_normal((Tk, d))
        np.testing.assert_allclose(O.attention_head(q, k, v), _sdpa64(q, k, v),
                                   rtol=1e-12, atol=1e-12)


def test_attention_brute_force_loops():
    rng = np.random.default_rng(4)
    Tq, Tk, d = 3, 4, 2
    q, k, v = rng.standard_normal((Tq, d)), rng.standard_normal((Tk, d)), rng.standard_normal((Tk, 3))
    got = O.attention_head(q, k, v)
    for i in range(Tq):
        s = [sum(q[i, c] * k[j, c] for c in range(d)) / math.sqrt(d) for j in range(Tk)]
        e = [math.exp(x) for x in s]
        z = sum(e)
        for c in range(3):
            assert abs(got[i, c] - sum(e[j] * v[j, c] for j in range(Tk)) / z) < 1e-12


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    T, d = 9, 8
    k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    # Q = 0: uniform weights, each output row is the column mean of V
    np.testing.assert_allclose(O.attention_head(np.zeros((T, d)), k, v),
                               np.broadcast_to(v.mean(axis=0), (T, d)), atol=1e-13)
    # constant V gives that constant
    c = np.full((T, d), 0.75)
    np.testing.assert_allclose(O.attention_head(rng.standard_normal((T, d)), k, c), c, atol=1e-13)
    # one key with a dominant score selects its V row
    kk = np.zeros((T, d)); kk[4, 0] = 1.0
    qq = np.zeros((T, d)); qq[:, 0] = 1e4
    np.testing.assert_allclose(O.attention_head(qq, kk, v), np.broadcast_to(v[4], (T, d)), atol=1e-12)
    # a single token attends to itself: O = V
    np.testing.assert_allclose(O.attention_head(k[:1], k[:1], v[:1]), v[:1], atol=1e-15)
    # the scale is 1/sqrt(d): scaling q by sqrt(d) with scale 1 is the same
    q = rng.standard_normal((T, d))
    np.testing.assert_allclose(O.attention_head(q, k, v),
                               O.attention_head(q / math.sqrt(d), k, v, scale=1.0), atol=1e-13)


def test_softmax_rows_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((6, 11)) * 50
    p = O.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(O.softmax_rows(s + rng.standard_normal((6, 1)) * 100), p, atol=1e-13)


def test_multihead_layout_head_blocks():
    # head h reads and writes the column block [h*d, (h+1)*d) and nothing else
    rng = np.random.default_rng(8)
    T, H, d = 7, 3, 4
    q, k, v = (rng.standard_normal((T, H * d)) for _ in range(3))
    out = O.attention_heads(q, k, v, H, d)
    for h in range(H):
        c = slice(h * d, (h + 1) * d)
        np.testing.assert_allclose(out[:, c], _sdpa64(q[:, c], k[:, c], v[:, c]), atol=1e-12)


# ---------------------------------------------------------------- sharding invariants

T_, D_, H_, d_, F_ = 8, 32, 4, 8, 64


def _weights(seed=9):
    rng = np.random.default_rng(seed)
    w = dict(x=rng.standard_normal((T_, D_)))
    for n in ("w_q", "w_k", "w_v"):
        w[n] = rng.standard_normal((D_, D_)) * 0.2
    for n in ("b_q", "b_k", "b_v", "b_o", "b_dn"):
        w[n] = rng.standard_normal(D_) * 0.1
    w["w_o"] = rng.standard_normal((D_, D_)) * 0.2
    w["w_up"] = rng.standard_normal((F_, D_)) * 0.2
    w["b_up"] = rng.standard_normal(F_) * 0.1
    w["w_dn"] = rng.standard_normal((D_, F_)) * 0.2
    return w


@pytest.mark.parametrize("P", [1, 2, 4])
def test_I1_colwise_shards_concatenate_to_unsharded(P):
    w = _weights()
    full = O.block_unsharded(w["x"], w, H_, d_, bf16=False)
    Dr = D_ // P
    qs, ks, vs, hs = [], [], [], []
    for r in range(P):
        res = O.rank_forward(w["x"], w, P, r, H_, d_, bf16=False)
        qkv = res["qkv_r"]
        assert qkv.shape == (T_, 3 * Dr)
        qs.append(qkv[:, :Dr]); ks.append(qkv[:, Dr:2 * Dr]); vs.append(qkv[:, 2 * Dr:])
        hs.append(res["h_r"])
    np.testing.assert_allclose(np.concatenate(qs, 1), full["q"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(ks, 1), full["k"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(vs, 1), full["v"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(hs, 1), full["g"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P", [1, 2, 4])
def test_I2_I4_rowwise_partials_sum_to_unsharded(P):
    w = _weights()
    full = O.block_unsharded(w["x"], w, H_, d_, bf16=False)
    ranks = [O.rank_forward(w["x"], w, P, r, H_, d_, bf16=False) for r in range(P)]
    s_attn = O.partial_reduce([r["p_attn"] for r in ranks], w["b_o"])
    s_mlp = O.partial_reduce([r["p_mlp"] for r in ranks], w["b_dn"])
    np.testing.assert_allclose(s_attn, full["y_attn"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s_mlp, full["y_mlp"], rtol=1e-12, atol=1e-12)
    y = O.partial_reduce([r["p_block"] for r in ranks], O.rowwise_bias(w))
    np.testing.assert_allclose(y, full["y"], rtol=1e-12, atol=1e-12)
    # and each rank's partial alone is NOT the answer when P > 1
    if P > 1:
        assert np.max(np.abs(ranks[0]["p_block"] + O.rowwise_bias(w) - full["y"])) > 1e-3


@pytest.mark.parametrize("P", [1, 2, 4])
def test_I3_head_locality(P):
    w = _weights()
    full = O.block_unsharded(w["x"], w, H_, d_, bf16=False)
    for r in range(P):
        o_r = O.rank_forward(w["x"], w, P, r, H_, d_, bf16=False)["o_r"]
        np.testing.assert_allclose(o_r, full["o"][:, O.colwise_range(D_, P, r)], atol=1e-12)


def test_I5_divisibility_is_rejected_before_anything():
    with pytest.raises(O.ShardConfigError) as e:
        O.check_config(5, 0, 24 * 8, 24, 8, 0)
    assert e.value.kind == "divisibility"
    for P in (1, 2, 3, 4, 6, 8, 12, 24):
        O.check_config(P, P - 1, 24 * 8, 24, 8, 24 * 16)
    with pytest.raises(O.ShardConfigError) as e:      # P divides heads, not ffn
        O.check_config(4, 0, 24 * 8, 24, 8, 1022)
    assert e.value.kind == "divisibility"
    with pytest.raises(O.ShardConfigError) as e:      # heads * d != hidden
        O.check_config(2, 0, 100, 4, 8, 0)
    assert e.value.kind == "divisibility"
    for bad_rank in (-1, 4):
        with pytest.raises(O.ShardConfigError) as e:
            O.check_config(4, bad_rank, 32, 4, 8, 64)
        assert e.value.kind == "argument"
    with pytest.raises(O.ShardConfigError) as e:      # sum 12 divides by 4, block 2 does not
        O.packed_colwise_rows([2, 2, 8], 4, 0)
    assert e.value.kind == "divisibility"
    # blocks [1, 2] of sizes (4, 8): the sum 12 divides by 4 and so does each block
    np.testing.assert_array_equal(O.packed_colwise_rows([4, 8], 4, 1), [1, 6, 7])


def test_I6_single_rank_is_the_unsharded_block():
    w = _weights()
    full = O.block_unsharded(w["x"], w, H_, d_, bf16=False)
    r = O.rank_forward(w["x"], w, 1, 0, H_, d_, bf16=False)
    np.testing.assert_allclose(r["p_block"] + O.rowwise_bias(w), full["y"], atol=1e-12)
    np.testing.assert_allclose(r["o_r"], full["o"], atol=1e-12)


@pytest.mark.parametrize("P", [2, 4])
def test_I7_naive_slice_of_packed_qkv_differs(P):
    """§Projeções fundidas: a plain dim-0 slice of a fused [3D, D] QKV weight
    straddles the concatenation; the per-block slice does not."""
    w = _weights()
    w_qkv = np.concatenate([w["w_q"], w["w_k"], w["w_v"]])
    rows_packed = O.packed_colwise_rows([D_, D_, D_], P, 0)
    naive = O.colwise_range(3 * D_, P, 0)
    assert not np.array_equal(rows_packed, np.arange(naive.start, naive.stop))
    good = O.rank_forward(w["x"], w, P, 0, H_, d_, bf16=False)["qkv_r"]
    bad = O.linear(w["x"], w_qkv[naive])
    assert good.shape == bad.shape
    assert np.max(np.abs(good - bad - np.concatenate([w["b_q"], w["b_k"], w["b_v"]])[rows_packed])) > 1e-2
    # the packed slice is exactly [Q_r; K_r; V_r]
    Dr = D_ // P
    np.testing.assert_array_equal(rows_packed, np.concatenate(
        [np.arange(0, Dr), np.arange(D_, D_ + Dr), np.arange(2 * D_, 2 * D_ + Dr)]))


@pytest.mark.parametrize("P", [2, 4])
def test_I8_misplaced_style_breaks_the_sum(P):
    """§Restrições e verificação: a misplaced colwise/rowwise still runs but is
    wrong -- sharding the up-projection rowwise (then GELU of a partial) and
    the down-projection colwise does not reproduce the unsharded MLP."""
    w = _weights()
    x = w["x"]
    y_ref = O.linear(O.gelu_tanh(O.linear(x, w["w_up"], w["b_up"])), w["w_dn"], w["b_dn"])
    parts = []
    for r in range(P):
        ci = O.rowwise_range(D_, P, r)               # up-proj sharded on its input features
        u_partial = O.linear(x[:, ci], w["w_up"][:, ci])
        g = O.gelu_tanh(u_partial + w["b_up"] / P)
        co = O.colwise_range(D_, P, r)               # down-proj sharded on its output features
        y_slice = O.linear(g, w["w_dn"][co])
        full_width = np.zeros((T_, D_)); full_width[:, co] = y_slice
        parts.append(full_width)
    y_bad = O.partial_reduce(parts, w["b_dn"])
    assert y_bad.shape == y_ref.shape
    assert np.max(np.abs(y_bad - y_ref)) > 1e-2
    # the correct placement reproduces it
    good = O.partial_reduce([O.rank_forward(x, {k: w[k] for k in ("w_up", "b_up", "w_dn", "b_dn")},
                                            P, r, 0, 0, bf16=False)["p_mlp"] for r in range(P)], w["b_dn"])
    np.testing.assert_allclose(good, y_ref, atol=1e-12)


def test_block_out_is_packed_rowwise_over_o_and_h():
    """§Projeções fundidas: a rowwise to_out over [inner_dim, mlp_hidden_dim]
    equals the sum of the two separate rowwise partials."""
    w = _weights()
    P, r = 2, 1
    res = O.rank_forward(w["x"], w, P, r, H_, d_, bf16=False)
    s = O.shard_weights(w, P, r, H_, d_)
    packed = O.linear(np.concatenate([res["o_r"], res["h_r"]], 1), np.concatenate([s["w_o"], s["w_dn"]], 1))
    np.testing.assert_allclose(packed, res["p_block"], atol=1e-12)


def test_bf16_storage_points_only():
    """With bf16 storage, qkv_r/o_r/h_r are bf16-representable and partials are
    not rounded; the sharded result still matches the unsharded one closely."""
    w = {k: O.to_bf16_rne(v) for k, v in _weights().items()}
    ranks = [O.rank_forward(w["x"], w, 2, r, H_, d_, bf16=True) for r in range(2)]
    for res in ranks:
        for k in ("qkv_r", "o_r", "h_r"):
            np.testing.assert_array_equal(res[k], O.to_bf16_rne(res[k]))
    full = O.block_unsharded(w["x"], w, H_, d_, bf16=True)
    y = O.partial_reduce([r["p_block"] for r in ranks], O.rowwise_bias(w))
    assert np.max(np.abs(y - full["y"])) / np.max(np.abs(full["y"])) < 1e-2


def test_row_sampled_helpers_match_full():
    w = _weights()
    full = O.block_unsharded(w["x"], w, H_, d_, bf16=False)
    rows = np.array([0, 3, 7])
    np.testing.assert_allclose(O.attention_rows(full["q"][rows], full["k"], full["v"], H_, d_),
                               full["o"][rows], atol=1e-12)
    np.testing.assert_allclose(O.colwise_rows_sampled(w["x"][rows], w["w_up"], w["b_up"], gelu=True, bf16=False),
                               full["g"][rows], atol=1e-12)


def test_oracle_drift_against_golden_summary():
    """Regression only: the stored summary was written by the oracle itself
    (tests/golden/make_golden.py), so it detects unintended change, not error."""
    import json
    import os
    import sys
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, here)
    import make_golden
    with open(os.path.join(here, "c1_oracle_summary.json")) as f:
        want = json.load(f)
    got = make_golden.summary()
    assert got["shape"] == want["shape"]
    for k in ("sum", "sum_sq", "max_abs"):
        assert abs(got[k] - want[k]) <= 1e-9 * max(1.0, abs(want[k]))
    for (i, j, v), (i2, j2, v2) in zip(got["samples"], want["samples"]):
        assert (i, j) == (i2, j2) and abs(v - v2) <= 1e-12


@pytest.mark.parametrize("P", [1, 2, 4])
@pytest.mark.parametrize("mlp_act", ["gelu_tanh", "swiglu"])
@pytest.mark.parametrize("bf16", [False, True])
def test_block_rows_sampled_equals_full_rank_forward_rows(P, mlp_act, bf16):
    """The row-sampled whole block (every rank's stored activations and
    partial, and the reduced y, on some rows) equals the rows of the full
    per-rank forward and reduce, and y equals the unsharded block's rows:
    each output row depends only on its own input row plus every key/value."""
    rng = np.random.default_rng(31)
    T, D, H, d, F = 40, 64, 4, 16, 96
    w = dict(x=rng.standard_normal((T, D)))
    for n in ("w_q", "w_k", "w_v", "w_o"):
        w[n] = rng.standard_normal((D, D)) * 0.2
    for n in ("b_q", "b_k", "b_v", "b_o", "b_dn"):
        w[n] = rng.standard_normal(D) * 0.1
    U = 2 * F if mlp_act == "swiglu" else F
    w["w_up"] = rng.standard_normal((U, D)) * 0.2
    w["b_up"] = rng.standard_normal(U) * 0.1
    w["w_dn"] = rng.standard_normal((D, F)) * 0.2
    if bf16:
        w = {k: O.to_bf16_rne(v) for k, v in w.items()}
    rows = np.array([0, 5, 17, 39])
    got = O.block_rows_sampled(w["x"], w, rows, P, H, d, bf16, mlp_act=mlp_act)
    full = [O.rank_forward(w["x"], w, P, r, H, d, bf16, mlp_act=mlp_act) for r in range(P)]
    for r in range(P):
        for k in ("qkv_r", "o_r", "h_r", "p_block"):
            np.testing.assert_allclose(got["ranks"][r][k], full[r][k][rows], rtol=1e-12, atol=1e-12)
    y = O.partial_reduce([f["p_block"] for f in full], O.rowwise_bias(w))
    np.testing.assert_allclose(got["y"], y[rows], rtol=1e-12, atol=1e-12)
    un = O.block_unsharded(w["x"], w, H, d, bf16, mlp_act=mlp_act)["y"]
    np.testing.assert_allclose(got["y"], un[rows], rtol=1e-12, atol=1e-12)
    # a misplaced head block (rank 0 reading rank 1's heads) must not pass
    if P > 1:
        wrong = O.linear(got["ranks"][1]["o_r"], w["w_o"][:, O.rowwise_range(D, P, 0)])
        right = O.linear(got["ranks"][0]["o_r"], w["w_o"][:, O.rowwise_range(D, P, 0)])
        assert np.max(np.abs(wrong - right)) > 1e-3
