"""Pins of oracle.distributions: library top-k/softmax, a library-built
inverse CDF, the closed form 1 - TV(p, q) of the acceptance rate, one-step
losslessness of accept-or-resample, the greedy verifier contract, ties."""
import json
import os

import numpy as np
import pytest
import torch
from scipy.stats import chisquare

from oracle import distributions as dist

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_topk_softmax_matches_torch():
    rng = np.random.default_rng(1)
    for V, k, T in [(256, 50, 0.9), (2048, 50, 0.9), (4096, 100, 0.8),
                    (64, 64, 1.3), (16, 1, 0.5)]:
        z = (rng.standard_normal(V) * 0.4).astype(np.float32)
        p, _ = dist.topk_softmax(z, T, k)
        zt = torch.from_numpy(z.astype(np.float64))
        vals, idx = torch.topk(zt, k)
        assert set(np.flatnonzero(p > 0)) == set(idx.tolist())
        ref = torch.softmax(vals / float(np.float32(T)), dim=0).numpy()
        np.testing.assert_allclose(p[idx.numpy()], ref, rtol=2e-7, atol=0)
        assert p.dtype == np.float32


def test_full_softmax_when_k_covers_vocab():
    z = np.linspace(-1, 1, 40).astype(np.float32)
    p, flag = dist.topk_softmax(z, 0.7, 40)
    ref = torch.softmax(torch.from_numpy(z.astype(np.float64)) /
                        float(np.float32(0.7)), 0).numpy()
    np.testing.assert_allclose(p, ref, rtol=2e-7)
    assert not flag
    p2, _ = dist.topk_softmax(z, 0.7, 1000)
    np.testing.assert_array_equal(p, p2)


def test_topk_ties_go_to_lower_id_and_flag():
    z = np.array([1.0, 2.0, 2.0, 2.0, 0.0, 3.0], np.float32)
    sup, flag = dist.topk_support(z, 3)
    assert list(sup) == [1, 2, 5] and flag
    sup, flag = dist.topk_support(z, 4)
    assert list(sup) == [1, 2, 3, 5] and not flag
    z = np.array([0.5, 0.50005, 0.0], np.float32)
    assert dist.topk_support(z, 1)[1]          # gap 5e-5 < 1e-4


def test_argmax_ties_and_gap():
    z = np.array([0.1, 0.7, 0.7, -1.0], np.float32)
    assert dist.argmax_with_gap(z) == (1, True)
    z = np.array([0.1, 0.7, 0.5, -1.0], np.float32)
    assert dist.argmax_with_gap(z) == (1, False)
    z = np.array([0.1, 0.70005, 0.7], np.float32)
    assert dist.argmax_with_gap(z) == (1, True)


def _searchsorted_sample(w, u):
    ids = np.flatnonzero(w > 0)
    cs = np.cumsum(w[ids], dtype=np.float32)        # sequential float32
    t = np.float32(np.float32(u) * cs[-1])
    j = int(np.searchsorted(cs, t, side="right"))
    return int(ids[min(j, ids.size - 1)])


def test_sample_is_the_inverse_cdf():
    rng = np.random.default_rng(2)
    for trial in range(30):
        V = int(rng.integers(2, 300))
        w = rng.random(V).astype(np.float32)
        w[rng.random(V) < 0.5] = 0
        if not np.any(w > 0):
            w[0] = 1
        us = rng.integers(0, 2**24, size=200) / 2**24
        # also exactly at the boundaries
        ids = np.flatnonzero(w > 0)
        cs = np.cumsum(w[ids], dtype=np.float32)
        us = np.concatenate([us, (cs / cs[-1])[:-1], [0.0, 1 - 2**-24]])
        for u in us:
            got, _ = dist.sample(w, np.float32(u))
            assert got == _searchsorted_sample(w, u), (trial, u)


def test_sample_cdf_flag():
    w = np.array([0.25, 0.25, 0.5], np.float32)
    assert dist.sample(w, 0.25)[0] == 1 and dist.sample(w, 0.25)[1]
    assert dist.sample(w, 0.1) == (0, False)
    assert dist.sample(w, 0.4999999)[1]
    assert dist.sample(w, 0.0) == (0, False)      # no boundary below entry 0
    with pytest.raises(ValueError):
        dist.sample(np.zeros(3, np.float32), 0.5)


def _explicit_pairs():
    return [
        (np.array([0.1, 0.2, 0.3, 0.4]), np.array([0.4, 0.3, 0.2, 0.1])),
        (np.array([0.7, 0.1, 0.1, 0.1]), np.array([0.25, 0.25, 0.25, 0.25])),
        (np.array([0.0, 0.5, 0.5, 0.0]), np.array([0.5, 0.0, 0.25, 0.25])),
    ]


def test_acceptance_rate_is_one_minus_tv():
    """Lesson 8, section 02: averaged over y ~ q the acceptance probability is
    sum_x min(p(x), q(x)) = 1 - TV(p, q)."""
    rng = np.random.default_rng(3)
    n = 30000
    for p, q in _explicit_pairs():
        p32, q32 = p.astype(np.float32), q.astype(np.float32)
        u = rng.integers(0, 2**24, size=(n, 2)) / 2**24
        acc = 0
        for i in range(n):
            y, _ = dist.sample(q32, np.float32(u[i, 0]))
            ok, _ = dist.accept_test(p32[y], q32[y], np.float32(u[i, 1]))
            acc += ok
        tv = 0.5 * np.abs(p - q).sum()
        expect = 1.0 - tv
        sigma = np.sqrt(expect * (1 - expect) / n)
        assert abs(acc / n - expect) < 5 * sigma + 1e-9, (acc / n, expect)


def test_accept_or_resample_is_lossless_one_step():
    """Accept y ~ q with min(1, p/q), else resample norm(max(0, p - q)):
    the result is distributed as p (Leviathan et al., restated in Lesson 8)."""
    rng = np.random.default_rng(4)
    n = 30000
    for p, q in _explicit_pairs():
        p32, q32 = p.astype(np.float32), q.astype(np.float32)
        u = rng.integers(0, 2**24, size=(n, 3)) / 2**24
        counts = np.zeros(4)
        for i in range(n):
            y, _ = dist.sample(q32, np.float32(u[i, 0]))
            ok, _ = dist.accept_test(p32[y], q32[y], np.float32(u[i, 1]))
            if not ok:
                y, _ = dist.sample(dist.residual_or_target(p32, q32),
                                   np.float32(u[i, 2]))
            counts[y] += 1
        live = p > 0
        assert counts[~live].sum() == 0
        assert chisquare(counts[live], p[live] * n).pvalue > 1e-3


def test_accept_test_edges():
    assert dist.accept_test(0.0, 0.3, 0.0) == (False, True)   # p(d)=0 rejects
    assert dist.accept_test(0.5, 0.25, 0.999)[0]              # ratio > 1
    ok, flag = dist.accept_test(np.float32(0.3), np.float32(0.6),
                                np.float32(0.5))
    assert not ok and flag                                    # u == p/q
    r = dist.residual(np.array([0.5, 0.5, 0], np.float32),
                      np.array([0.2, 0.6, 0.2], np.float32))
    np.testing.assert_array_equal(r, np.array([0.3, 0, 0], np.float32))
    same = np.array([0.5, 0.5], np.float32)
    np.testing.assert_array_equal(dist.residual_or_target(same, same), same)


def test_greedy_verifier_golden():
    g = json.load(open(os.path.join(GOLDEN, "greedy_verifier.json")))
    for c in g["cases"]:
        r = dist.verify_greedy(tuple(c["draft"]), tuple(c["target"]))
        assert r.accepted == tuple(c["accepted"])
        assert r.emitted == tuple(c["emitted"])
        assert r.rejected_at == c["rejected_at"]
    for c in g["errors"]:
        with pytest.raises(ValueError):
            dist.verify_greedy(tuple(c["draft"]), tuple(c["target"]))
