"""Host logic of the per-device verify-window choice
(speculative_decoding_rvq_amd.calibrate): the expected codes per round
against a brute-force enumeration of acceptance patterns, and the choice
rule on hand-made profiles."""
import itertools

import pytest

from speculative_decoding_rvq_amd.calibrate import choose_window, expected_codes_per_round


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
