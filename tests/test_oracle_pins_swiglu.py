"""Pins for the SwiGLU MLP and the packed (fused) projections of the oracle:
SiLU against closed forms and torch's silu in float64, the [1, 1] gate/up
slice and the [1, 1, 1, 3, 3] / [inner_dim, mlp_hidden_dim] single-stream
slices against hand-listed indices, and the invariants of the Diffusers TP
page (§Projeções fundidas; §Restrições e verificação: the sharded result
equals the single-device one, a plain slice across a packed concatenation
does not).  CPU only."""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle as O

# ---------------------------------------------------------------- SiLU / SwiGLU


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    u = np.linspace(-30, 30, 6001)
    # sigmoid(u) + sigmoid(-u) = 1, so silu(u) - silu(-u) = u
    np.testing.assert_allclose(O.silu(u) - O.silu(-u), u, atol=1e-13)
    assert abs(O.silu(40.0) - 40.0) < 1e-12          # u -> +inf: silu(u) -> u
    assert abs(O.silu(-40.0)) < 1e-15                # u -> -inf: silu(u) -> 0
    assert abs(O.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    eps = 1e-7                                       # slope 1/2 at the origin
    assert abs(O.silu(eps) / eps - 0.5) < 1e-6
    # the minimum of silu is at u* with 1 + exp(-u*) + u* exp(-u*) = 0 ... i.e.
    # u* = -1.2784645; its value -0.2784645 (W0 closed form: u* = -1 - W(1/e))
    us = np.linspace(-1.4, -1.1, 300001)
    i = np.argmin(O.silu(us))
    assert abs(us[i] + 1.2784645427610738) < 2e-6
    assert abs(O.silu(us[i]) + 0.2784645427610738) < 1e-9


def test_silu_matches_torch_fp64():
    u = torch.linspace(-60, 60, 100_001, dtype=torch.float64)
    np.testing.assert_allclose(O.silu(u.numpy()), Fnn.silu(u).numpy(), rtol=1e-14, atol=1e-300)


def test_swiglu_is_gate_silu_times_up():
    rng = np.random.default_rng(3)
    g, u = rng.standard_normal((5, 7)), rng.standard_normal((5, 7))
    ref = (Fnn.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(O.swiglu(g, u), ref, rtol=1e-14)
    # the gate is the argument of silu, not the up half: swapping them differs
    assert np.max(np.abs(O.swiglu(u, g) - ref)) > 1e-2
    # zero gate kills the row whatever up is; zero up kills it whatever gate is
    assert np.all(O.swiglu(np.zeros(4), rng.standard_normal(4)) == 0.0)
    assert np.all(O.swiglu(rng.standard_normal(4), np.zeros(4)) == 0.0)


def test_mlp_hidden_swiglu_uses_first_half_as_gate():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 8))
    wg, wu = rng.standard_normal((5, 8)), rng.standard_normal((5, 8))
    bg, bu = rng.standard_normal(5), rng.standard_normal(5)
    h = O.mlp_hidden(x, np.concatenate([wg, wu]), np.concatenate([bg, bu]), "swiglu")
    # explicit loops over the definition
    ref = np.zeros((6, 5))
    for t in range(6):
        for j in range(5):
            gate = sum(x[t, k] * wg[j, k] for k in range(8)) + bg[j]
            up = sum(x[t, k] * wu[j, k] for k in range(8)) + bu[j]
            ref[t, j] = gate / (1.0 + np.exp(-gate)) * up
    np.testing.assert_allclose(h, ref, rtol=1e-12)
    with pytest.raises(ValueError):
        O.mlp_hidden(x, wg, bg, "relu")


# ---------------------------------------------------------------- packed slices


def test_packed_slices_hand_listed():
    # SwiGLU gate/up [1, 1] with F = 6, tp_degree 3, rank 1: gate rows 2..3, up rows 8..9
    np.testing.assert_array_equal(O.packed_colwise_rows([6, 6], 3, 1), [2, 3, 8, 9])
    # fused Q, K, V, gate, up with hidden 2 and mlp_ratio 3: blocks [2, 2, 2, 6, 6]
    np.testing.assert_array_equal(O.packed_colwise_rows([2, 2, 2, 6, 6], 2, 0),
                                  [0, 2, 4, 6, 7, 8, 12, 13, 14])
    np.testing.assert_array_equal(O.packed_colwise_rows([2, 2, 2, 6, 6], 2, 1),
                                  [1, 3, 5, 9, 10, 11, 15, 16, 17])
    # rowwise over [inner_dim 4 | mlp_hidden 8], tp_degree 2
    np.testing.assert_array_equal(O.packed_rowwise_cols([4, 8], 2, 0), [0, 1, 4, 5, 6, 7])
    np.testing.assert_array_equal(O.packed_rowwise_cols([4, 8], 2, 1), [2, 3, 8, 9, 10, 11])
    with pytest.raises(O.ShardConfigError):
        O.packed_rowwise_cols([4, 6], 4, 0)


T_, H_, d_ = 9, 4, 8
D_ = H_ * d_
F_ = 3 * D_          # mlp_ratio 3


def _single(seed=11):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T_, D_))
    w_in = rng.standard_normal((3 * D_ + 2 * F_, D_)) * 0.2
    b_in = rng.standard_normal(3 * D_ + 2 * F_) * 0.1
    w_out = rng.standard_normal((D_, D_ + F_)) * 0.2
    b_out = rng.standard_normal(D_) * 0.1
    return x, w_in, b_in, w_out, b_out


@pytest.mark.parametrize("P", [1, 2, 4])
def test_single_stream_sharded_sum_is_the_unsharded_block(P):
    x, w_in, b_in, w_out, b_out = _single()
    full = O.single_stream_block(x, w_in, b_in, w_out, b_out, H_, d_, F_, bf16=False)
    ranks = [O.single_stream_rank(x, w_in, b_in, w_out, P, r, H_, d_, F_, bf16=False)
             for r in range(P)]
    y = O.partial_reduce([r["partial"] for r in ranks], b_out)
    np.testing.assert_allclose(y, full["y"], rtol=1e-12, atol=1e-12)
    # each rank's SwiGLU hidden is its colwise slice of the full hidden, its
    # attention output its own heads
    for r, res in enumerate(ranks):
        np.testing.assert_allclose(res["h_r"], full["h"][:, O.colwise_range(F_, P, r)], atol=1e-12)
        np.testing.assert_allclose(res["o_r"], full["o"][:, O.colwise_range(D_, P, r)], atol=1e-12)


@pytest.mark.parametrize("P", [2, 4])
def test_single_stream_naive_slices_differ(P):
    """A plain dim-0 slice of the fused input weight, or a plain dim-1 slice of
    the fused output weight, still runs but is wrong."""
    x, w_in, b_in, w_out, b_out = _single()
    full = O.single_stream_block(x, w_in, b_in, w_out, b_out, H_, d_, F_, bf16=False)
    n = (3 * D_ + 2 * F_) // P
    Dr, Fr = D_ // P, F_ // P
    parts = []
    for r in range(P):
        u = O.linear(x, w_in[r * n:(r + 1) * n], b_in[r * n:(r + 1) * n])
        e = np.cumsum([0, Dr, Dr, Dr, Fr, Fr])
        o = O.attention_heads(u[:, e[0]:e[1]], u[:, e[1]:e[2]], u[:, e[2]:e[3]], H_ // P, d_)
        h = O.swiglu(u[:, e[3]:e[4]], u[:, e[4]:e[5]])
        c = (D_ + F_) // P
        parts.append(O.linear(np.concatenate([o, h], 1), w_out[:, r * c:(r + 1) * c]))
    assert np.max(np.abs(O.partial_reduce(parts, b_out) - full["y"])) > 1e-2


@pytest.mark.parametrize("P", [1, 2, 4])
def test_single_stream_equals_separate_projection_form(P):
    """The fused single-stream rank and the separate-projection rank (SwiGLU
    MLP, output bias carried as b_o) compute the same activations and partial."""
    x, w_in, b_in, w_out, b_out = _single()
    sep = O.single_stream_as_block(w_in, b_in, w_out, b_out, H_, d_, F_)
    for r in range(P):
        a = O.single_stream_rank(x, w_in, b_in, w_out, P, r, H_, d_, F_, bf16=True)
        b = O.rank_forward(x, sep, P, r, H_, d_, bf16=True, mlp_act="swiglu")
        np.testing.assert_allclose(b["qkv_r"], a["qkv_r"], atol=1e-12)
        np.testing.assert_allclose(b["o_r"], a["o_r"], atol=1e-12)
        np.testing.assert_allclose(b["h_r"], a["h_r"], atol=1e-12)
        np.testing.assert_allclose(b["p_block"], a["partial"], rtol=1e-12, atol=1e-12)
    full = O.block_unsharded(x, sep, H_, d_, bf16=False, mlp_act="swiglu")
    ref = O.single_stream_block(x, w_in, b_in, w_out, b_out, H_, d_, F_, bf16=False)
    np.testing.assert_allclose(full["y"], ref["y"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P", [2, 4])
def test_swiglu_gate_up_slice_pairs_gate_with_its_up(P):
    """[1, 1] on [W_gate; W_up]: rank r's hidden column j uses gate row j and
    up row j of its own blocks; the sharded hidden concatenates to the
    unsharded one, while a plain half-split of the rank's contiguous slice of
    [W_gate; W_up] pairs gate rows with gate rows (rank 0) and does not."""
    x, w_in, b_in, _, _ = _single()
    w_gu, b_gu = w_in[3 * D_:], b_in[3 * D_:]
    full = O.mlp_hidden(x, w_gu, b_gu, "swiglu")
    wts = {"w_up": w_gu, "b_up": b_gu, "w_dn": np.zeros((D_, F_))}
    hs = []
    for r in range(P):
        s = O.shard_weights(wts, P, r, 0, 0, mlp_act="swiglu")
        hs.append(O.mlp_hidden(x, s["w_up"], s["b_up"], "swiglu"))
    np.testing.assert_allclose(np.concatenate(hs, 1), full, rtol=1e-12, atol=1e-12)
    n = 2 * F_ // P
    bad = O.mlp_hidden(x, w_gu[:n], b_gu[:n], "swiglu")
    assert np.max(np.abs(bad - hs[0])) > 1e-2
