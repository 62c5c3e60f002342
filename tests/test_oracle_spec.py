"""Pins of oracle.spec (the frame loop and the round):

* greedy speculative decoding equals greedy autoregressive decoding exactly
  (Lesson 8, sections 02 and 08) for every window N = 2..8;
* brute-force enumeration of every draft outcome, with the acceptance
  probabilities min(1, p/q) and the residual masses, gives exactly the
  autoregressive joint distribution (to 1e-12, float64);
* speculative code sequences over many seeds pass a chi-square test against
  the exact autoregressive joint (losslessness, guide "How a round works");
* special cases: p == q accepts every draft; disjoint supports reject every
  draft and reproduce the autoregressive codes; top-k 1 is the greedy chain;
* one verify pass per round and the per-round commit bounds 1 <= n <= N.
"""
import itertools

import numpy as np
import pytest
from scipy.stats import chisquare

import synth
from oracle import decoder as dec
from oracle import distributions as dist
from oracle import spec
from tablemodel import TableModel


def _dp(N, greedy=False, T=0.9, k=50):
    return dict(verify_size=N, greedy=greedy, temperature=T, top_k=k)


def _tiny(**kw):
    c = synth.custom(**kw)
    return c, dec.Model(c, synth.make_weights(c))


@pytest.mark.parametrize("c", [
    synth.config("tiny"),
    synth.custom(layers=2, hidden=32, q_heads=4, kv_heads=2, head_dim=8,
                 ffn=48, groups=16, vocab=32, weight_scale=0.3),
], ids=["config1", "G16"])
def test_greedy_spec_equals_greedy_ar(c):
    m = dec.Model(c, synth.make_weights(c))
    h, c0, seeds = synth.make_inputs(c, frames=6, streams=1)
    ref, _ = spec.decode(m, _dp(0, greedy=True), h, c0, seeds)
    for N in range(2, 9):
        st = spec.new_stats()
        got, _ = spec.decode(m, _dp(N, greedy=True), h, c0, seeds, stats=st)
        np.testing.assert_array_equal(got, ref, err_msg=f"N={N}")
        assert st["rounds"] < 6 * (c["groups"] - 2) or N == 2


def _normalised(p):
    p = p.astype(np.float64)
    return p / p.sum()


def _ar_joint(m, dp, h_frame, c0):
    """Exact autoregressive joint over c_1..c_{G-1} by depth-first search."""
    out = {}
    kv = m.new_kv()
    hs = m.forward_rows([h_frame, m.embed_row(0, c0)], [0, 1], kv)

    def walk(j, h, kv, prefix, prob):
        p = _normalised(dist.topk_softmax(m.logits(j, h), dp["temperature"],
                                          dp["top_k"])[0])
        for x in np.flatnonzero(p > 0):
            pr = prob * p[x]
            if j == m.G - 1:
                out[prefix + (int(x),)] = out.get(prefix + (int(x),), 0) + pr
                continue
            kv2 = _copy_kv(kv)
            h2 = m.forward_rows([m.embed_row(j, int(x))], [j + 1], kv2)[0]
            walk(j + 1, h2, kv2, prefix + (int(x),), pr)

    walk(1, hs[1], kv, (), 1.0)
    return out


def _copy_kv(kv):
    import copy
    return copy.deepcopy(kv)


def _spec_joint(m, dp, h_frame, c0):
    """Exact distribution of the speculative frame loop by enumerating every
    draft tuple and every accept/reject outcome of every round."""
    out = {}
    kv = m.new_kv()
    hs = m.forward_rows([h_frame, m.embed_row(0, c0)], [0, 1], kv)
    p1 = _normalised(dist.topk_softmax(m.logits(1, hs[1]),
                                       dp["temperature"], dp["top_k"])[0])
    G, N = m.G, dp["verify_size"]

    def rnd(s, h, kv, codes, prob):
        if s == G - 1:
            out[codes] = out.get(codes, 0) + prob
            return
        gamma = min(N - 1, G - 2 - s)
        qs = [_normalised(dist.topk_softmax(m.logits(s + t, h),
                                            dp["temperature"],
                                            dp["top_k"])[0])
              for t in range(1, gamma + 1)]
        supports = [np.flatnonzero(q > 0) for q in qs]
        for d in itertools.product(*supports):
            pd = prob * np.prod([qs[t][d[t]] for t in range(gamma)])
            kv2 = _copy_kv(kv)
            rows = [m.embed_row(s, codes[s])]
            rows += [m.embed_row(s + t, d[t - 1]) for t in range(1, gamma + 1)]
            outs = m.forward_rows(rows, [s + 1 + r for r in range(gamma + 1)],
                                  kv2)
            ps = [_normalised(dist.topk_softmax(m.logits(s + 1 + r, outs[r]),
                                                dp["temperature"],
                                                dp["top_k"])[0])
                  for r in range(gamma + 1)]
            keep = 1.0
            for t in range(1, gamma + 1):
                a = min(1.0, ps[t - 1][d[t - 1]] / qs[t - 1][d[t - 1]])
                rej = keep * (1.0 - a)
                if rej > 0:
                    r = np.maximum(ps[t - 1] - qs[t - 1], 0.0)
                    r = r / r.sum()
                    for x in np.flatnonzero(r > 0):
                        kv3 = _copy_kv(kv2)
                        kv3.truncate(s + t + 1)
                        rnd(s + t, outs[t - 1], kv3,
                            codes + tuple(int(v) for v in d[: t - 1]) +
                            (int(x),), pd * rej * r[x])
                keep *= a
                if keep == 0:
                    break
            if keep > 0:
                for x in np.flatnonzero(ps[gamma] > 0):
                    kv3 = _copy_kv(kv2)
                    kv3.truncate(s + gamma + 2)
                    rnd(s + gamma + 1, outs[gamma], kv3,
                        codes + tuple(int(v) for v in d) + (int(x),),
                        pd * keep * ps[gamma][x])

    for x in np.flatnonzero(p1 > 0):
        rnd(1, hs[1], kv, (c0, int(x)), p1[x])
    return {k[1:]: v for k, v in out.items()}


def test_bruteforce_enumeration_equals_ar_joint():
    """Vocabulary 4, window N = 3, top-k 3 < V, T != 1."""
    c, m = _tiny(layers=1, hidden=16, q_heads=2, kv_heads=1, head_dim=8,
                 ffn=24, groups=5, vocab=4, weight_scale=0.6)
    dp = _dp(3, T=0.7, k=3)
    h = np.random.default_rng(1).standard_normal(16)
    ar = _ar_joint(m, dp, h, 2)
    sp = _spec_joint(m, dp, h, 2)
    assert abs(sum(ar.values()) - 1) < 1e-12
    assert abs(sum(sp.values()) - 1) < 1e-12
    keys = set(ar) | set(sp)
    assert max(abs(ar.get(k, 0) - sp.get(k, 0)) for k in keys) < 1e-12


def _chi2_against(joint, counts, n):
    keys = sorted(joint)
    exp = np.array([joint[k] * n for k in keys])
    obs = np.array([counts.get(k, 0) for k in keys], dtype=np.float64)
    assert sum(counts.values()) == obs.sum(), "sample outside the support"
    small = exp < 5
    if small.any():
        exp = np.append(exp[~small], exp[small].sum())
        obs = np.append(obs[~small], obs[small].sum())
    exp *= obs.sum() / exp.sum()
    return chisquare(obs, exp).pvalue


def test_chi_square_lossless_table_model():
    """10^5 seeds through the scripted table model, V = 5, G = 5, N = 4."""
    m = TableModel(G=5, V=5, seed=3, scale=1.2)
    dp = _dp(4, T=1.3, k=4)
    n = 100000
    joint = _ar_joint(m, dp, None, 1)
    counts = {}
    st = spec.new_stats()
    rng = np.random.default_rng(99)
    seeds = rng.integers(0, 2**63, size=n, dtype=np.int64)
    passes0 = m.calls["forward_rows"]
    for i in range(n):
        codes, _ = spec.decode_frame(m, dp, None, 1, int(seeds[i]), st)
        key = tuple(int(v) for v in codes[1:])
        counts[key] = counts.get(key, 0) + 1
    assert _chi2_against(joint, counts, n) > 1e-3
    # the window really speculated: more than one code per verify pass
    assert spec.codes_per_round(st) > 1.2
    # exactly one decoder pass per round, plus the prefill of each frame
    assert st["rounds"] == m.calls["forward_rows"] - passes0 - n


def test_chi_square_lossless_tiny_decoder():
    c, m = _tiny(layers=1, hidden=16, q_heads=2, kv_heads=1, head_dim=8,
                 ffn=24, groups=4, vocab=4, weight_scale=0.7)
    dp = _dp(3, T=0.8, k=3)
    h = np.random.default_rng(5).standard_normal(16)
    joint = _ar_joint(m, dp, h, 3)
    n = 12000
    seeds = np.random.default_rng(6).integers(0, 2**63, size=n, dtype=np.int64)
    counts = {}
    for i in range(n):
        codes, _ = spec.decode_frame(m, dp, h, 3, int(seeds[i]))
        key = tuple(int(v) for v in codes[1:])
        counts[key] = counts.get(key, 0) + 1
    assert _chi2_against(joint, counts, n) > 1e-3


def test_chi_square_detects_a_planted_error(monkeypatch):
    """The lossless test has power: resampling from p instead of the
    residual biases the output and must fail the same chi-square test."""
    m = TableModel(G=4, V=4, seed=8, scale=1.5)
    dp = _dp(3, T=1.0, k=4)
    joint = _ar_joint(m, dp, None, 0)
    monkeypatch.setattr(dist, "residual_or_target",
                        lambda p, q: np.asarray(p, np.float32))
    n = 20000
    counts = {}
    for i in range(n):
        codes, _ = spec.decode_frame(m, dp, None, 0, 1000 + i)
        key = tuple(int(v) for v in codes[1:])
        counts[key] = counts.get(key, 0) + 1
    assert _chi2_against(joint, counts, n) < 1e-6


def test_identical_distributions_accept_everything():
    """Zero attention/FFN outputs and one shared embedding row: every
    position's hidden state is the same, so q_t == p_{t-1} and every draft is
    accepted; each round commits gamma + 1 codes."""
    c = synth.custom(layers=1, hidden=16, q_heads=2, kv_heads=1, head_dim=8,
                     ffn=24, groups=8, vocab=16, weight_scale=0.5)
    w = synth.make_weights(c)
    for lw in w["layers"]:
        lw["wo"][:] = 0
        lw["w_down"][:] = 0
    w["embed"][:] = w["embed"][0, 0]
    m = dec.Model(c, w)
    st = spec.new_stats()
    h = np.asarray(w["embed"][0, 0], np.float64)
    for seed in range(20):
        spec.decode_frame(m, _dp(4, T=0.9, k=8), h, 3, seed, st)
    assert st["accepted"] == st["proposed"]
    assert st["bonus"] == st["rounds"]
    # G = 8, N = 4: s = 1 -> 5 (gamma 3) -> 7 (gamma 1): two rounds a frame
    assert st["rounds"] == 40


def test_disjoint_supports_reject_everything_and_match_ar():
    m = TableModel(G=6, V=6, seed=4, target_support=(0, 1, 2),
                   draft_support=(3, 4, 5))
    dp = _dp(4, T=1.0, k=3)
    for seed in range(200):
        st = spec.new_stats()
        a, _ = spec.decode_frame(m, dp, None, 2, seed, st)
        b, _ = spec.decode_frame(m, _dp(0, T=1.0, k=3), None, 2, seed)
        np.testing.assert_array_equal(a, b)
        assert sum(st["accepted"]) == 0
        assert st["rounds"] == 4             # one code per round


def test_top1_sampling_is_the_greedy_chain():
    c = synth.config("tiny")
    m = dec.Model(c, synth.make_weights(c))
    h, c0, seeds = synth.make_inputs(c, frames=3, streams=1)
    a, _ = spec.decode(m, _dp(3, T=0.9, k=1), h, c0, seeds)
    b, _ = spec.decode(m, _dp(3, greedy=True), h, c0, seeds)
    np.testing.assert_array_equal(a, b)


def test_round_bounds_and_first_code_matches_ar():
    c = synth.config("tiny")
    m = dec.Model(c, synth.make_weights(c))
    h, c0, seeds = synth.make_inputs(c, frames=8, streams=1)
    st = spec.new_stats()
    got, _ = spec.decode(m, _dp(3), h, c0, seeds, stats=st)
    ar, _ = spec.decode(m, _dp(0), h, c0, seeds)
    # c_1 comes from the prefill with U(1, target) in both modes
    np.testing.assert_array_equal(got[:, :, :2], ar[:, :, :2])
    assert np.all(got >= 0) and np.all(got < c["vocab"])
    G = c["groups"]
    assert st["codes"] == 8 * (G - 1) and st["prefill_passes"] == 8
    # every round commits between 1 and N codes
    assert 8 * 2 <= st["rounds"] <= 8 * (G - 2)
    assert st["accepted"][0] <= st["proposed"][0]
    for t in range(1, 8):
        assert st["accepted"][t] <= st["accepted"][t - 1]
