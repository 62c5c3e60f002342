"""Pins of the oracle's near-tie machinery (test infrastructure for the GPU
parity rule, which accepts a differing code stream only when the oracle,
re-run with one near-tie decision taken the other way, reproduces it):

* the alternative outcomes of each decision kind on hand-built cases: the
  neighbouring entry of a sample point that sits on a CDF boundary, the other
  member of a tied top-k boundary, the other code of a tied argmax;
* a forced flip equals decoding a model whose logits were nudged so that the
  decision really goes the other way (greedy argmax tie, sampled top-k tie),
  and an unforced run with a log equals the plain run.
"""
import numpy as np

from oracle import distributions as dist
from oracle import spec
from tablemodel import TableModel


def test_sample_alternatives_on_boundaries():
    w = np.array([0.25, 0.0, 0.25, 0.5], np.float32)
    # t = 0.5 sits on the boundary between codes 2 and 3: Sample takes 3
    # (first running sum above t), the other rounding takes 2
    code, near = dist.sample(w, 0.5)
    assert code == 3 and near
    assert dist.sample_alternatives(w, 0.5) == [2]
    # t = 0.25: boundary between codes 0 and 2 (code 1 has no weight)
    code, near = dist.sample(w, 0.25)
    assert code == 2 and near and dist.sample_alternatives(w, 0.25) == [0]
    # interior point: no alternative
    code, near = dist.sample(w, 0.6)
    assert code == 3 and not near and dist.sample_alternatives(w, 0.6) == []
    # just below a boundary: the next entry is the alternative
    u = np.float32(0.5) - np.float32(2**-24)
    code, near = dist.sample(w, u)
    assert code == 2 and near and dist.sample_alternatives(w, u) == [3]


def test_topk_alternatives_swap_the_tied_member():
    z = np.array([3.0, 1.0, 2.0, 1.0, 0.5, 1.00005], np.float32)
    p, near = dist.topk_softmax(z, 0.9, 3)
    # members: 0, 2 and the lowest id among the tied 1.0 / 1.00005 group
    # by value: 5 (1.00005) > 1 = 3 (1.0); members {0, 2, 5}
    assert list(np.flatnonzero(p > 0)) == [0, 2, 5] and near
    alts = dist.topk_alternatives(z, 0.9, 3)
    sets = [list(np.flatnonzero(a > 0)) for a in alts]
    assert [0, 1, 2] in sets and [0, 2, 3] in sets and len(sets) == 2
    for a, sup in zip(alts, sets):
        ref, _ = dist.topk_softmax(np.where(np.isin(np.arange(6), sup), z, -50.0).astype(np.float32),
                                   0.9, 3)
        np.testing.assert_allclose(a, ref, rtol=1e-6)
    assert dist.topk_alternatives(z, 0.9, 6) == []  # k = V: nothing to swap


def test_argmax_alternatives():
    z = np.array([0.1, 0.9, 0.9, 0.89995, 0.2], np.float32)
    code, near = dist.argmax_with_gap(z)
    assert code == 1 and near
    assert dist.argmax_alternatives(z) == [2, 3]


def test_forced_argmax_flip_equals_nudged_model():
    G, V = 6, 8
    dp = dict(verify_size=3, greedy=True, temperature=1.0, top_k=1)
    base = TableModel(G, V, seed=5)
    key = ("p", (3,))                       # the prefill's target row (c_1)
    z = base._logits(key, None)
    order = np.argsort(-z, kind="stable")
    a, b = int(order[0]), int(order[1])
    win, lose = min(a, b), max(a, b)
    tied = TableModel(G, V, seed=5, edits={key: {a: z[a], b: z[a]}})
    codes, flags = spec.decode_frame(tied, dp, np.zeros(1), 3, 11)
    assert codes[1] == win and flags & 2
    log = []
    again, _ = spec.decode_frame(tied, dp, np.zeros(1), 3, 11, log=log)
    np.testing.assert_array_equal(again, codes)
    assert log[0][:2] == (1, "argmax")
    forced, _ = spec.decode_frame(tied, dp, np.zeros(1), 3, 11, force=(0, 0))
    nudged = TableModel(G, V, seed=5, edits={key: {win: z[a], lose: z[a] + np.float32(1e-3)}})
    ref, rflags = spec.decode_frame(nudged, dp, np.zeros(1), 3, 11)
    assert ref[1] == lose and not rflags & 2
    np.testing.assert_array_equal(forced, ref)


def test_forced_topk_flip_equals_nudged_model():
    G, V, k = 6, 8, 3
    dp = dict(verify_size=3, greedy=False, temperature=0.9, top_k=k)
    base = TableModel(G, V, seed=9, scale=0.5)
    key = ("p", (3,))
    z = base._logits(key, None)
    order = np.argsort(-z, kind="stable")
    a, b = int(order[k - 1]), int(order[k])  # the boundary pair
    win, lose = min(a, b), max(a, b)
    v = z[a]
    tied = TableModel(G, V, seed=9, scale=0.5, edits={key: {a: v, b: v}})
    log = []
    codes, flags = spec.decode_frame(tied, dp, np.zeros(1), 3, 11, log=log)
    assert flags & 2 and log[0][:2] == (1, "topk")
    forced, _ = spec.decode_frame(tied, dp, np.zeros(1), 3, 11, force=(0, 0))
    nudged = TableModel(G, V, seed=9, scale=0.5,
                        edits={key: {win: v, lose: v + np.float32(2e-4)}})
    ref, rflags = spec.decode_frame(nudged, dp, np.zeros(1), 3, 11)
    assert not rflags & 2
    np.testing.assert_array_equal(forced, ref)
    # the flip matters here: the other set gives another frame
    assert not np.array_equal(forced, codes)
