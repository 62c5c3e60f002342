"""Pins of oracle.spec.talker_feedback (the codec part of the Talker's next
input, sum over code groups of E_g[c_g]; SGLang-Omni note, the Talker /
CodePredictor hand-off paragraph):

* the same vector from one-hot matrix products, sum_g onehot(c_g) @ E_g;
* replacing one group's code changes it by exactly the difference of the two
  embedding rows;
* a hand-sized table with small integers.
"""
import numpy as np
import pytest

import synth
from oracle import decoder as dec
from oracle import spec


@pytest.mark.parametrize("cid", ["tiny", "qwen3tts"])
def test_feedback_equals_one_hot_products(cid):
    c = synth.config(cid)
    w = synth.make_weights(c)
    m = dec.Model(c, w)
    rng = np.random.default_rng(7)
    G, V = c["groups"], c["vocab"]
    for _ in range(3):
        codes = rng.integers(0, V, size=G)
        got = spec.talker_feedback(m, codes)
        want = np.zeros(c["hidden"])
        for g in range(G):
            table = dec._f64(w["embed"][g], m.dtype)          # [V][H]
            onehot = np.zeros(V)
            onehot[codes[g]] = 1.0
            want = want + onehot @ table
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_feedback_replacing_one_code():
    c = synth.config("tiny")
    w = synth.make_weights(c)
    m = dec.Model(c, w)
    codes = np.arange(c["groups"]) * 17 % c["vocab"]
    base = spec.talker_feedback(m, codes)
    for g in (0, 3, c["groups"] - 1):
        alt = codes.copy()
        alt[g] = (alt[g] + 5) % c["vocab"]
        moved = spec.talker_feedback(m, alt)
        np.testing.assert_allclose(moved - base, m.embed_row(g, alt[g]) - m.embed_row(g, codes[g]),
                                   rtol=0, atol=1e-12)


class _Tables:
    """Three groups of two codes with two channels, integer entries."""
    G, H = 3, 2
    E = np.array([[[1, 2], [3, 4]], [[10, 20], [30, 40]], [[100, 200], [300, 400]]], dtype=np.float64)

    def embed_row(self, g, code):
        return self.E[g, code]


def test_feedback_hand_sized():
    m = _Tables()
    assert spec.talker_feedback(m, [1, 0, 1]).tolist() == [313.0, 424.0]
    assert spec.talker_feedback(m, [0, 1, 0]).tolist() == [131.0, 242.0]
