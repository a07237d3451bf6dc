"""Pins for the log-sum-exp merge: a segmented softmax merged from its parts
equals one softmax over everything."""

import numpy as np

from oracle import attention_one_head, merge_partials


def test_partition_merge_equals_single_softmax():
    rng = np.random.default_rng(2)
    for trial in range(30):
        t, d = int(rng.integers(1, 400)), 16
        keys = rng.standard_normal((t, d)) * 3
        vals = rng.standard_normal((t, d))
        q = rng.standard_normal(d)
        whole, lse_whole = attention_one_head(keys, vals, q, 0.25)
        cuts = np.sort(rng.integers(0, t + 1, size=int(rng.integers(0, 8))))
        bounds = [0, *cuts.tolist(), t]  # repeated cuts give empty parts
        parts = [attention_one_head(keys[a:b], vals[a:b], q, 0.25) for a, b in zip(bounds[:-1], bounds[1:])]
        o, lse = merge_partials([p[0] for p in parts], [p[1] for p in parts])
        assert np.allclose(o, whole, rtol=1e-12, atol=1e-13)
        assert abs(lse - lse_whole) < 1e-12 * max(1, abs(lse_whole))


def test_all_empty_and_single_part():
    o, lse = merge_partials(np.ones((3, 4)), [-np.inf] * 3)
    assert np.all(o == 0) and lse == -np.inf
    o, lse = merge_partials(np.arange(4.0)[None], [2.5])
    assert np.array_equal(o, np.arange(4.0)) and lse == 2.5
    o, lse = merge_partials(np.array([[1.0, 0], [0, 1.0]]), [-np.inf, 0.0])
    assert np.array_equal(o, [0, 1.0])
