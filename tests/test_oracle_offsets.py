"""Pins of the position-aware draft offsets in oracle.spec ("RVQ Position
Aware Speculative Decoding ...", section 2.2 and Figure 3: draft offset t
drives head_{s+t} with h_s + b_t, the same K vectors for every s):

* an offset that moves h_s onto lambda * e_i turns the draft logits into
  lambda times column i of the head (a column read, no product), for each
  offset index t and a different i per t;
* with large one-hot offsets every greedy draft at offset t <= K is the
  argmax of its head's column i_t, and drafts past K see h_s unchanged;
* offsets change q only: greedy output equals the autoregressive output for
  N = 2..8 while the acceptance counts move, and stochastic output passes
  the chi-square test against the exact autoregressive joint.
"""
import numpy as np

import synth
from oracle import decoder as dec
from oracle import spec
from test_oracle_spec import _ar_joint, _chi2_against, _dp


def _model(K, scale=0.1, **kw):
    c = synth.custom(draft_offsets=K, offset_scale=scale, **kw)
    return c, dec.Model(c, synth.make_weights(c))


def test_offsets_come_from_their_own_generator():
    c = synth.custom()
    a = synth.make_weights(c)
    b = synth.make_weights(synth.custom(draft_offsets=3))
    assert "draft_offsets" not in a and b["draft_offsets"].shape == (3, 16)
    np.testing.assert_array_equal(a["heads"], b["heads"])
    np.testing.assert_array_equal(a["embed"], b["embed"])


def test_draft_logits_of_an_offset_onto_a_unit_vector():
    c, m = _model(3, groups=8, vocab=16)
    h = np.random.default_rng(2).standard_normal(m.H)
    cols = {1: 5, 2: 11, 3: 0}
    lam = {1: 2.0, 2: -0.75, 3: 3.5}
    m.draft_offsets = np.stack([lam[t] * np.eye(m.H)[cols[t]] - h
                                for t in (1, 2, 3)])
    for s in (1, 3):
        for t in (1, 2, 3):
            j = s + t
            got = spec.draft_logits(m, j, t, h)
            exp = (lam[t] * m.heads[j - 1][:, cols[t]]).astype(np.float32)
            np.testing.assert_array_max_ulp(got, exp, maxulp=1)
    # no b_4: offset 4 sees h_s itself
    np.testing.assert_array_equal(spec.draft_logits(m, 5, 4, h),
                                  m.logits(5, h))


def test_one_hot_offsets_steer_every_greedy_draft():
    c, m = _model(2, groups=10, vocab=32, layers=1, hidden=16, weight_scale=0.3)
    cols = (3, 9)
    lam = 1e4
    m.draft_offsets = np.stack([lam * np.eye(m.H)[i] for i in cols])
    mn = dec.Model(c, {**synth.make_weights(c), "draft_offsets": None})
    h, c0, seeds = synth.make_inputs(c, frames=4)
    checked = beyond = 0
    for f in range(4):
        trace = []
        spec.decode_frame(m, _dp(5, greedy=True), h[f, 0], int(c0[f, 0]),
                          int(seeds[f, 0]), trace=trace)
        for s, h_s, drafts, _ in trace:
            for t, d in enumerate(drafts, 1):
                if t <= 2:
                    assert d == int(np.argmax(m.heads[s + t - 1][:, cols[t - 1]]))
                    checked += 1
                else:
                    assert d == int(np.argmax(mn.logits(s + t, h_s)))
                    beyond += 1
    assert checked >= 8 and beyond >= 4


def test_greedy_output_unchanged_by_offsets():
    c = synth.config("tiny", draft_offsets=3, offset_scale=0.5)
    w = synth.make_weights(c)
    m = dec.Model(c, w)
    m0 = dec.Model(c, {**w, "draft_offsets": None})
    h, c0, seeds = synth.make_inputs(c, frames=4, streams=1)
    ref, _ = spec.decode(m0, _dp(0, greedy=True), h, c0, seeds)
    for N in range(2, 9):
        st, st0 = spec.new_stats(), spec.new_stats()
        got, _ = spec.decode(m, _dp(N, greedy=True), h, c0, seeds, stats=st)
        spec.decode(m0, _dp(N, greedy=True), h, c0, seeds, stats=st0)
        np.testing.assert_array_equal(got, ref, err_msg=f"N={N}")
        if N >= 3:  # the offsets did change the drafts
            assert st["accepted"] != st0["accepted"]


def test_chi_square_lossless_with_offsets():
    c, m = _model(2, scale=1.0, layers=1, hidden=16, q_heads=2, kv_heads=1,
                  head_dim=8, ffn=24, groups=4, vocab=4, weight_scale=0.7)
    dp = _dp(3, T=0.8, k=3)
    h = np.random.default_rng(5).standard_normal(16)
    joint = _ar_joint(m, dp, h, 3)
    n = 12000
    seeds = np.random.default_rng(7).integers(0, 2**63, size=n, dtype=np.int64)
    counts = {}
    st = spec.new_stats()
    for i in range(n):
        codes, _ = spec.decode_frame(m, dp, h, 3, int(seeds[i]), st)
        key = tuple(int(v) for v in codes[1:])
        counts[key] = counts.get(key, 0) + 1
    assert _chi2_against(joint, counts, n) > 1e-3
    # the offsets are large enough to reject some drafts
    assert sum(st["accepted"]) < sum(st["proposed"])
