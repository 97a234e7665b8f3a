"""Pins for the oracle's "rowwise_split_input" projection (Diffusers TP page,
§Colwise e rowwise style table; §O que deixar de fora: a large AdaLN
modulation projection is sharded this way): brute-force index sums, the
tensor-parallel invariant that the summed partials plus the bias equal the
single-device projection, input locality (a rank reads only its own input
features), and the divisibility check.  CPU only."""
import numpy as np
import pytest

import oracle as O


def _case(seed=21, R=3, K=24, N=10):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((R, K)), rng.standard_normal((N, K)), rng.standard_normal(N)


def test_split_input_brute_force():
    c, w, _ = _case()
    P, r = 4, 2
    got = O.split_input_rank(c, w, P, r)
    ref = np.zeros((3, 10))
    for i in range(3):
        for n in range(10):
            ref[i, n] = sum(c[i, k] * w[n, k] for k in range(12, 18))   # K_r = [12, 18)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 6, 8])
def test_split_input_partials_sum_to_the_projection(P):
    c, w, b = _case()
    parts = [O.split_input_rank(c, w, P, r) for r in range(P)]
    y = O.partial_reduce(parts, b)
    ref = c @ w.T + b
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    if P > 1:    # one rank's partial alone is not the answer
        assert np.max(np.abs(parts[0] + b - ref)) > 1e-2


@pytest.mark.parametrize("P", [2, 4])
def test_split_input_reads_only_its_own_features(P):
    c, w, _ = _case()
    K = c.shape[1]
    for r in range(P):
        keep = np.zeros(K, bool)
        keep[O.rowwise_range(K, P, r)] = True
        c2 = np.where(keep, c, 1e6)          # garbage outside K_r
        w2 = np.where(keep, w, -1e6)
        np.testing.assert_array_equal(O.split_input_rank(c2, w2, P, r), O.split_input_rank(c, w, P, r))


def test_split_input_divisibility_and_config():
    c, w, _ = _case(K=24)
    with pytest.raises(O.ShardConfigError) as e:
        O.split_input_rank(c, w, 5, 0)
    assert e.value.kind == "divisibility"
    with pytest.raises(O.ShardConfigError) as e:
        O.check_config(4, 0, 64, 0, 0, 0, mod_in=30)
    assert e.value.kind == "divisibility"
    O.check_config(4, 0, 64, 0, 0, 0, mod_in=64)          # a modulation-only shard is valid
    with pytest.raises(O.ShardConfigError) as e:
        O.check_config(4, 0, 64, 0, 0, 0, mod_in=0)
    assert e.value.kind == "argument"
