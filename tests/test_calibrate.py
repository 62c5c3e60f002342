"""Host logic of the per-device verify-window choice
(speculative_decoding_rvq_amd.calibrate): the expected codes per round
against a brute-force enumeration of acceptance patterns, and the choice
rule on hand-made profiles; the passes of a whole frame (prefill pass, the
frame's end cutting the window) against an enumeration of every round's
accept/reject path through the frame."""
import itertools

import pytest

from speculative_decoding_rvq_amd.calibrate import (choose_window, commit_distribution, expected_codes_per_round,
                                                     expected_passes_per_frame)


def _enumerate(cond, n):
    """Expected codes of one round with window n when draft t is accepted
    with probability cond[t-1] given that drafts 1..t-1 were: every
    accept/reject pattern of the n-1 drafts weighted by its probability, the
    round committing the accepted prefix plus one code."""
    total = 0.0
    for pattern in itertools.product((True, False), repeat=n - 1):
        p = 1.0
        alive = True
        prefix = 0
        for t, ok in enumerate(pattern):
            if alive:
                p *= cond[t] if ok else 1.0 - cond[t]
                if ok:
                    prefix += 1
                else:
                    alive = False
            else:
                # later drafts are never tested: count each rejected round once
                p *= 1.0 if ok else 0.0
        total += p * (prefix + 1)
    return total


@pytest.mark.parametrize("n", [1, 2, 3, 4, 6])
def test_expected_codes_matches_enumeration(n):
    cond = [0.62, 0.55, 0.5, 0.45, 0.4, 0.3, 0.2]
    share, run = [], 1.0
    for a in cond:
        run *= a
        share.append(run)
    assert expected_codes_per_round(share, n) == pytest.approx(_enumerate(cond, n), abs=1e-12)


def test_expected_codes_edges():
    assert expected_codes_per_round([], 4) == 1.0          # nothing measured past the window
    assert expected_codes_per_round([1.0, 1.0, 1.0], 4) == 4.0  # every draft accepted
    assert expected_codes_per_round([0.5, 0.2], 1) == 1.0  # no drafts
    with pytest.raises(ValueError):
        expected_codes_per_round([0.5], 0)


def test_choose_window_picks_best_rate():
    share = [0.62, 0.34, 0.18, 0.09, 0.04, 0.02, 0.01]
    # rates: 1.62/148, 1.96/163, 2.14/168, 2.23/192 -> N = 4
    assert choose_window(share, {2: 148.0, 3: 163.0, 4: 168.0, 5: 192.0}) == 4
    # a flat pass cost favours the widest window
    assert choose_window(share, {2: 100.0, 4: 100.0, 8: 100.0}) == 8
    # an expensive pass favours the narrowest
    assert choose_window(share, {2: 100.0, 3: 200.0, 4: 300.0}) == 2


def test_choose_window_ties_and_errors():
    # 1.5 / 150 == 2.0 / 200: the smaller window wins
    assert choose_window([0.5, 0.5], {2: 150.0, 3: 200.0}) == 2
    with pytest.raises(ValueError):
        choose_window([0.5], {})
    with pytest.raises(ValueError):
        choose_window([0.5], {2: 0.0})


def _shares(cond):
    share, run = [], 1.0
    for a in cond:
        run *= a
        share.append(run)
    return share


def _frame_passes(cond, n, G):
    """Expected passes of one frame, by walking every path: the prefill
    commits c_1; a round at depth s tests its min(n - 1, G - 2 - s) drafts
    one by one (draft t kept with probability cond[t-1] once drafts
    1..t-1 were) and commits the kept ones plus one code."""
    def rounds_from(s):
        if s >= G - 1:
            return 0.0
        gamma = min(n - 1, G - 2 - s)
        total = 0.0

        def walk(t, p):
            nonlocal total
            if t == gamma:
                total += p * (1.0 + rounds_from(s + gamma + 1))
                return
            walk(t + 1, p * cond[t])
            total += p * (1.0 - cond[t]) * (1.0 + rounds_from(s + t + 1))

        walk(0, 1.0)
        return total

    return 1.0 + rounds_from(1)


@pytest.mark.parametrize("n,G", [(2, 4), (3, 6), (4, 8), (8, 8), (5, 7)])
def test_frame_passes_match_enumeration(n, G):
    cond = [0.62, 0.55, 0.5, 0.45, 0.4, 0.3, 0.2]
    got = expected_passes_per_frame(_shares(cond), n, G)
    assert got == pytest.approx(_frame_passes(cond, n, G), abs=1e-12)


def test_frame_passes_edges():
    # every draft accepted: ceil((G - 2) / n) rounds after the prefill
    assert expected_passes_per_frame([1.0] * 7, 4, 16) == 1 + 4  # depths 1, 5, 9, 13, then one draft to 15
    # no draft ever accepted: one code per round
    assert expected_passes_per_frame([0.0] * 7, 4, 16) == 15.0
    # two groups: the prefill pass alone
    assert expected_passes_per_frame([0.5], 4, 2) == 1.0
    assert commit_distribution([0.5, 0.2], 0) == [1.0]
    assert sum(commit_distribution([0.62, 0.34, 0.18], 3)) == pytest.approx(1.0, abs=1e-15)
    with pytest.raises(ValueError):
        expected_passes_per_frame([0.5], 0, 16)


def test_choose_window_with_frame_ends():
    # the shares and pass times of a 64-stream run: the frame's end and the
    # prefill pass make N = 2 the best, as the decodes measured, where the
    # per-round rule alone says N = 4
    share = [0.617, 0.349, 0.180, 0.09, 0.045, 0.02, 0.01]
    us = {2: 253.7, 3: 301.3, 4: 326.2, 5: 447.4, 6: 475.0, 7: 502.3, 8: 531.7}
    assert choose_window(share, us) == 4
    assert choose_window(share, us, groups=16) == 2
    # one stream: both rules give N = 4
    us1 = {2: 125.1, 3: 137.7, 4: 142.5, 5: 170.0, 6: 174.3, 7: 183.5, 8: 184.2}
    assert choose_window(share, us1, groups=16) == 4
    # two groups: every window costs one pass, ties go to the smallest
    assert choose_window(share, {3: 100.0, 4: 100.0}, groups=2) == 3
