"""Pins for the oracle's context-parallel attention (Diffusers CP page,
§Ring Attention, §Ulysses Attention, variant table): the block log-sum-exp
against scipy's logsumexp, the block output against torch's SDPA in
float64, the merge over any partition of the keys against attention over
all keys, order invariance, ring and Ulysses against plain multi-head
attention, the all-to-all layouts against hand-listed placements, and the
divisibility rules.  CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn
from scipy.special import logsumexp

import oracle as O

H, d = 3, 8


def _qkv(T=24, Tk=None, seed=31):
    rng = np.random.default_rng(seed)
    Tk = T if Tk is None else Tk
    return (rng.standard_normal((T, H * d)), rng.standard_normal((Tk, H * d)) * 1.5,
            rng.standard_normal((Tk, H * d)))


def test_block_lse_and_output():
    q, k, v = _qkv(T=7, Tk=11)
    o, lse = O.attention_block(q, k, v, H, d)
    for h in range(H):
        c = slice(h * d, (h + 1) * d)
        s = q[:, c] @ k[:, c].T / math.sqrt(d)
        np.testing.assert_allclose(lse[:, h], logsumexp(s, axis=1), rtol=1e-14)
        ref = Fnn.scaled_dot_product_attention(torch.from_numpy(q[:, c])[None], torch.from_numpy(k[:, c])[None],
                                               torch.from_numpy(v[:, c])[None])[0].numpy()
        np.testing.assert_allclose(o[:, c], ref, rtol=1e-12, atol=1e-13)
    # one key: the output is that key's value, lse its scaled score
    o1, l1 = O.attention_block(q, k[:1], v[:1], H, d)
    np.testing.assert_allclose(o1, np.repeat(v[:1], 7, axis=0), atol=1e-14)
    np.testing.assert_allclose(l1[:, 0], q[:, :d] @ k[0, :d] / math.sqrt(d), atol=1e-14)


@pytest.mark.parametrize("cuts", [[24], [12, 12], [5, 7, 12], [1, 1, 22], [8, 8, 8]])
def test_merge_over_a_key_partition_is_full_attention(cuts):
    q, k, v = _qkv()
    full = O.attention_heads(q, k, v, H, d)
    edges = np.cumsum([0] + cuts)
    parts = [O.attention_block(q, k[a:b], v[a:b], H, d) for a, b in zip(edges[:-1], edges[1:])]
    o, lse = O.attention_merge([p[0] for p in parts], [p[1] for p in parts], d)
    np.testing.assert_allclose(o, full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, O.attention_block(q, k, v, H, d)[1], rtol=1e-13)
    # order does not matter
    o2, _ = O.attention_merge([p[0] for p in parts[::-1]], [p[1] for p in parts[::-1]], d)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)


def test_merge_weights_use_lse_not_plain_average():
    """A plain average of the partial outputs is not attention (wrong weights)."""
    q, k, v = _qkv()
    parts = [O.attention_block(q, k[:4], v[:4], H, d), O.attention_block(q, k[4:], v[4:], H, d)]
    full = O.attention_heads(q, k, v, H, d)
    assert np.max(np.abs(0.5 * (parts[0][0] + parts[1][0]) - full)) > 1e-2


@pytest.mark.parametrize("R", [1, 2, 3, 4, 6])
def test_ring_equals_attention(R):
    q, k, v = _qkv()
    outs = O.ring_attention(q, k, v, H, d, R)
    assert len(outs) == R and all(o.shape == (24 // R, H * d) for o in outs)
    np.testing.assert_allclose(np.concatenate(outs), O.attention_heads(q, k, v, H, d), rtol=1e-12, atol=1e-13)


def test_ring_divisibility():
    with pytest.raises(O.ShardConfigError):
        O.ring_attention(*_qkv(T=25), H, d, 4)


def test_ulysses_layouts_hand_listed():
    # 4 tokens, 2 heads of width 1, degree 2: rank s holds tokens 2s, 2s+1
    x = np.arange(8, dtype=float).reshape(4, 2)       # x[t, h] = 2 t + h
    chunks = [x[:2], x[2:]]
    heads = O.ulysses_seq_to_heads(chunks, 2, 1)
    np.testing.assert_array_equal(heads[0][:, 0], [0, 2, 4, 6])   # head 0, every token
    np.testing.assert_array_equal(heads[1][:, 0], [1, 3, 5, 7])   # head 1
    back = O.ulysses_heads_to_seq(heads, 2, 1)
    np.testing.assert_array_equal(back[0], x[:2])
    np.testing.assert_array_equal(back[1], x[2:])


@pytest.mark.parametrize("u", [1, 3])
def test_ulysses_equals_attention(u):
    q, k, v = _qkv()
    outs = O.ulysses_attention(q, k, v, H, d, u)
    np.testing.assert_allclose(np.concatenate(outs), O.attention_heads(q, k, v, H, d), rtol=1e-12, atol=1e-13)


def test_ulysses_divisibility():
    with pytest.raises(O.ShardConfigError):
        O.check_ulysses(24, 3, 2)       # heads do not divide
    with pytest.raises(O.ShardConfigError):
        O.check_ulysses(25, 6, 2)       # tokens do not divide
    O.check_ulysses(24, 6, 2)
