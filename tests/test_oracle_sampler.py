"""Pins of the sampling oracle (oracle/sampler.py) against things other than itself:
numpy's own Philox4x64-10 generator, argmax as the top_k = 1 special case, a
worked example whose draws follow from hand arithmetic, the penalty's closed form,
and the draw's distribution against the normalised weights."""
import math

import numpy as np
import pytest

from oracle import sampler


@pytest.mark.parametrize("key,ctr", [((5, 0), (0, 0, 0, 0)), ((0xDEADBEEF12345678, 0), (41, 7, 0, 0)),
                                     ((1, 2), ((1 << 64) - 1, 3, 9, 1 << 63))])
def test_philox_matches_numpy(key, ctr):
    # numpy's Philox (4x64, 10 rounds) raises its counter before computing a block,
    # so its first block is the block of ctr + 1
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    want = [int(x) for x in g.random_raw(8)]
    c = sum(int(w) << (64 * i) for i, w in enumerate(ctr))
    blocks = []
    for step in (1, 2):
        n = (c + step) % (1 << 256)
        blocks += sampler.philox4x64([(n >> (64 * i)) & ((1 << 64) - 1) for i in range(4)], key)
    assert blocks == want


def test_uniform_range_and_spread():
    us = np.array([sampler.uniform(1234, f, k) for f in range(400) for k in range(16)])
    assert us.min() >= 0.0 and us.max() < 1.0
    assert np.all(us * 2 ** 24 == np.floor(us * 2 ** 24))  # 24-bit, exact in float32
    hist, _ = np.histogram(us, bins=16, range=(0, 1))
    exp = len(us) / 16
    chi2 = float(np.sum((hist - exp) ** 2 / exp))
    assert chi2 < 45.0  # 15 degrees of freedom; p < 1e-4 beyond this
    # distinct (counter, codebook) give distinct draws; the seed changes them
    assert len(set(us.tolist())) > 0.99 * len(us)
    assert sampler.uniform(1, 5, 3) != sampler.uniform(2, 5, 3)


def test_top_k_one_is_argmax_lowest_index_on_ties():
    rng = np.random.default_rng(0)
    for _ in range(20):
        x = rng.normal(size=300).astype(np.float32)
        x[rng.integers(0, 300, size=3)] = x.max()  # ties at the top
        for u in (0.0, 0.5, 0.999):
            tok, _ = sampler.sample(x, u, temperature=0.7, top_k=1, top_p=0.9)
            assert tok == int(np.argmax(x))


def test_worked_example():
    # weights 1, 2, 3, 4 (logits ln w, T = 1): candidate order 3, 2, 1, 0 with
    # probabilities 0.4, 0.3, 0.2, 0.1 and running sums 0.4, 0.7, 0.9, 1.0
    x = np.log(np.array([1.0, 2.0, 3.0, 4.0])).astype(np.float32)
    for u, tok in ((0.05, 3), (0.39, 3), (0.45, 2), (0.75, 1), (0.95, 0)):
        assert sampler.sample(x, u, top_k=4)[0] == tok
    # top_p 0.5: 0.4 < 0.5 <= 0.7, so tokens 3 and 2 are kept (total 0.7):
    # r = 0.35 -> 3, r = 0.42 -> 2
    assert sampler.sample(x, 0.5, top_k=4, top_p=0.5)[0] == 3
    assert sampler.sample(x, 0.6, top_k=4, top_p=0.5)[0] == 2
    # top_k 2 keeps 3 and 2 as well: r = u * 0.7 as above
    assert sampler.sample(x, 0.6, top_k=2)[0] == 2
    # tiny top_p keeps the most probable token only
    assert sampler.sample(x, 0.99, top_k=4, top_p=1e-6)[0] == 3
    p = sampler.distribution(x, top_k=4, top_p=0.5)
    np.testing.assert_allclose(p, [0, 0, 3 / 7, 4 / 7], rtol=1e-6)  # logits rounded to float32


def test_repetition_penalty_closed_form():
    x = np.array([2.0, 1.5, -0.5, -0.4], dtype=np.float32)
    seen = np.array([True, False, True, False])
    z = sampler.process(x, temperature=1.0, penalty=2.0, seen=seen)
    f = float(np.float32(-0.4))
    np.testing.assert_array_equal(z, [1.0, 1.5, -1.0, f])
    # the penalty moves the greedy choice from 0 to 1
    assert sampler.sample(x, 0.0, top_k=1)[0] == 0
    assert sampler.sample(x, 0.0, top_k=1, penalty=2.0, seen=seen)[0] == 1
    # temperature divides after the penalty
    z = sampler.process(x, temperature=0.5, penalty=2.0, seen=seen)
    np.testing.assert_array_equal(z, [2.0, 3.0, -2.0, 2 * f])


def test_draws_follow_the_distribution():
    rng = np.random.default_rng(3)
    x = rng.normal(scale=1.5, size=64).astype(np.float32)
    seen = rng.random(64) < 0.3
    kw = dict(temperature=0.8, top_k=20, top_p=0.9, penalty=1.3, seen=seen)
    p = sampler.distribution(x, **kw)
    assert abs(p.sum() - 1) < 1e-12 and np.count_nonzero(p) <= 20
    # softmax of the processed scores over the kept set, computed independently
    z = sampler.process(x, kw["temperature"], kw["penalty"], seen)
    kept = np.flatnonzero(p)
    q = np.exp(z[kept] - z[kept].max())
    np.testing.assert_allclose(p[kept], q / q.sum(), rtol=1e-12)
    # a fine grid of u reproduces p (the inverse CDF hits each token in proportion)
    n = 20000
    counts = np.zeros(64)
    for i in range(n):
        counts[sampler.sample(x, (i + 0.5) / n, **kw)[0]] += 1
    np.testing.assert_allclose(counts / n, p, atol=2.0 / n)
    # the kept set is the shortest prefix reaching top_p of the top-k weight
    order = sorted(kept, key=lambda i: -p[i])
    full = sampler.distribution(x, temperature=0.8, top_k=20, top_p=1.0, penalty=1.3, seen=seen)
    mass = np.cumsum(sorted(full[full > 0], reverse=True))
    m = len(order)
    assert mass[m - 1] >= 0.9 - 1e-12 and (m == 1 or mass[m - 2] < 0.9)


def test_nan_scores_are_never_drawn():
    x = np.array([np.nan, 0.3, np.nan, 0.2], dtype=np.float32)
    for u in np.linspace(0, 0.999, 50):
        assert sampler.sample(x, float(u), top_k=4)[0] in (1, 3)
