"""Pins of oracle.tree (the tree-shaped verify window):

* a tree with one child per node is the chain window: the same codes, flags
  and counters as oracle.spec for stochastic and greedy decoding, with and
  without position-aware offsets;
* brute-force enumeration of every node's draw and every acceptance branch of
  a branching tree (vocabulary 4) gives the autoregressive joint to 1e-12 --
  the walk with residual updates between siblings is exact;
* greedy trees reproduce greedy autoregressive decoding;
* tree-decoded frames pass a chi-square test against the exact joint, and a
  planted error in the residual fails it.
"""
import itertools

import numpy as np
import pytest

import synth
from oracle import decoder as dec
from oracle import distributions as dist
from oracle import spec, tree
from tablemodel import TableModel
from test_oracle_spec import _ar_joint, _chi2_against, _copy_kv, _dp, _normalised


def _tiny(**kw):
    c = synth.custom(**kw)
    return c, dec.Model(c, synth.make_weights(c))


@pytest.mark.parametrize("greedy", [False, True])
@pytest.mark.parametrize("K", [0, 3])
def test_one_child_tree_is_the_chain(greedy, K):
    c = synth.config("tiny", draft_offsets=K, offset_scale=0.3)
    m = dec.Model(c, synth.make_weights(c))
    hf, c0, seeds = synth.make_inputs(c, frames=8, streams=1)
    dp = _dp(4, greedy=greedy, T=0.9, k=50)
    t = tree.Tree.chain(3)
    for f in range(8):
        a_st, b_st = spec.new_stats(), spec.new_stats()
        a = spec.decode_frame(m, dp, hf[f, 0], int(c0[f, 0]), int(seeds[f, 0]), a_st)
        b = tree.decode_frame_tree(m, dp, t, hf[f, 0], int(c0[f, 0]), int(seeds[f, 0]), b_st)
        np.testing.assert_array_equal(a[0], b[0])
        assert a[1] == b[1]
        assert a_st == b_st


def _tree_joint(m, dp, t, h_frame, c0):
    """Exact distribution of the tree window's frame, enumerated in float64:
    every node's draw from its depth's q, and every branch of the walk (each
    child tested with min(1, p'/q), p' replaced by norm(max(0, p' - q)) after a
    rejection, the final draw from p')."""
    out = {}
    T, k = dp["temperature"], dp["top_k"]
    kv = m.new_kv()
    hs = m.forward_rows([h_frame, m.embed_row(0, c0)], [0, 1], kv)
    G = m.G

    def dist_of(j, h):
        return _normalised(dist.topk_softmax(m.logits(j, h), T, k)[0])

    def rnd(s, h, kv, codes, prob):
        if s == G - 1:
            out[codes] = out.get(codes, 0.0) + prob
            return
        dmax = G - 2 - s
        nodes = [i for i in range(1, t.T + 1) if t.depth[i] <= dmax]
        kids = {v: [c for c in t.children[v] if c in nodes] for v in [0] + nodes}
        D = max([t.depth[i] for i in nodes], default=0)
        q = {d: dist_of(s + d, h) for d in range(1, D + 1)}
        supports = [np.flatnonzero(q[t.depth[i]] > 0) for i in nodes]
        for xs in itertools.product(*supports):
            code = dict(zip(nodes, (int(x) for x in xs)))
            pa = prob * np.prod([q[t.depth[i]][code[i]] for i in nodes])
            if pa == 0:
                continue
            hid, kvs = {}, {}
            kvs[0] = _copy_kv(kv)
            hid[0] = m.forward_rows([m.embed_row(s, codes[s])], [s + 1], kvs[0])[0]
            for i in nodes:
                kvs[i] = _copy_kv(kvs[t.parent[i]])
                hid[i] = m.forward_rows([m.embed_row(s + t.depth[i], code[i])],
                                        [s + 1 + t.depth[i]], kvs[i])[0]

            def walk(v, pw, emitted):
                d1 = t.depth[v] + 1
                p = dist_of(s + d1, hid[v])
                for c in kids[v]:
                    x = code[c]
                    a = min(1.0, p[x] / q[d1][x])
                    if a > 0:
                        walk(c, pw * a, emitted + (x,))
                    pw *= 1.0 - a
                    if pw == 0:
                        return
                    r = np.maximum(p - q[d1], 0.0)
                    p = r / r.sum() if r.sum() > 0 else p
                for x in np.flatnonzero(p > 0):
                    n = len(emitted) + 1
                    kv_next = _copy_kv(kvs[v])
                    kv_next.truncate(s + n + 1)
                    rnd(s + n, hid[v], kv_next, codes + emitted + (int(x),), pw * p[x])

            walk(0, pa, ())

    p1 = dist_of(1, hs[1])
    for x in np.flatnonzero(p1 > 0):
        rnd(1, hs[1], kv, (c0, int(x)), p1[x])
    return {key[1:]: v for key, v in out.items()}


def test_bruteforce_tree_equals_ar_joint():
    """Vocabulary 4, top-k 3 < V, T != 1; the root has two children, the
    first of which has one."""
    c, m = _tiny(layers=1, hidden=16, q_heads=2, kv_heads=1, head_dim=8,
                 ffn=24, groups=5, vocab=4, weight_scale=0.6)
    dp = _dp(0, T=0.7, k=3)
    h = np.random.default_rng(1).standard_normal(16)
    t = tree.Tree([0, 0, 1])
    ar = _ar_joint(m, dp, h, 2)
    tj = _tree_joint(m, dp, t, h, 2)
    assert abs(sum(tj.values()) - 1) < 1e-12
    keys = set(ar) | set(tj)
    assert max(abs(ar.get(key, 0) - tj.get(key, 0)) for key in keys) < 1e-12


@pytest.mark.parametrize("parents", [[0, 0, 1], [0, 0, 0, 1, 2], [0, 1, 1, 2, 3]])
def test_greedy_tree_is_greedy_ar(parents):
    c = synth.config("tiny")
    m = dec.Model(c, synth.make_weights(c))
    hf, c0, seeds = synth.make_inputs(c, frames=6, streams=1)
    ar, _ = spec.decode(m, _dp(0, greedy=True), hf, c0, seeds)
    t = tree.Tree(parents)
    st = spec.new_stats()
    for f in range(6):
        got, _ = tree.decode_frame_tree(m, _dp(0, greedy=True), t, hf[f, 0],
                                        int(c0[f, 0]), int(seeds[f, 0]), st)
        np.testing.assert_array_equal(got, ar[f, 0])
    assert st["rounds"] < 6 * (c["groups"] - 2)  # the tree did speculate


def _tree_counts(m, dp, t, n, seed0):
    counts = {}
    st = spec.new_stats()
    for i in range(n):
        codes, _ = tree.decode_frame_tree(m, dp, t, None, 1, seed0 + i, st)
        key = tuple(int(v) for v in codes[1:])
        counts[key] = counts.get(key, 0) + 1
    return counts, st


def test_chi_square_lossless_tree_table_model():
    m = TableModel(G=5, V=5, seed=3, scale=1.2)
    dp = _dp(0, T=1.3, k=4)
    t = tree.Tree([0, 0, 1, 2])
    n = 20000
    joint = _ar_joint(m, dp, None, 1)
    counts, st = _tree_counts(m, dp, t, n, 7000)
    assert _chi2_against(joint, counts, n) > 1e-3
    assert spec.codes_per_round(st) > 1.2


def test_chi_square_tree_detects_a_planted_error(monkeypatch):
    m = TableModel(G=4, V=4, seed=8, scale=1.5)
    dp = _dp(0, T=1.0, k=4)
    t = tree.Tree([0, 0, 1])
    joint = _ar_joint(m, dp, None, 1)
    monkeypatch.setattr(dist, "residual_or_target", lambda p, q: np.asarray(p, np.float32))
    n = 20000
    counts, _ = _tree_counts(m, dp, t, n, 100)
    assert _chi2_against(joint, counts, n) < 1e-6
