"""Processed distributions and the discrete decisions of a round.

Every decision here is taken in float32, the precision the GPU takes it in:
the logits arrive as float32, probabilities leave as float32, and sampling
and acceptance use float32 sums, products, quotients and compares.

Definitions (TensorRT-Edge-LLM guide "CodePredictor Speculative Decoding",
"How a round works"; lab-artifacts "Lesson 8: Speculative Decoding, Beyond
Text", section 02 "Two exact algorithms"):

* TopKSoftmax(z; T, k): the k largest logits form the support (total order:
  larger logit first, lower code id first among equal logits); on it
  p_i = exp((z_i - max z) / T) / sum_j exp((z_j - max z) / T); p = 0 elsewhere.
  Temperature and top-k are applied to draft and target alike, as the exact
  stochastic algorithm requires both to be taken after every processor.
* Sample(w, u): inverse CDF over the entries with w_i > 0 in ascending code
  order, with a sequential float32 running sum: t = u * sum(w), return the
  first i whose running sum exceeds t.
* Acceptance of draft d: accept iff u < p(d) / q(d) (float32 quotient), which
  is "accept with probability min(1, p/q)" for u uniform in [0, 1).
* Residual: w = max(0, p - q) elementwise in float32, sampled with Sample; if
  every entry is zero (possible only through rounding) p itself is sampled.
* Greedy: argmax over the raw logits, ties to the lowest code id; the draft is
  accepted left to right while it equals the target argmax, the first mismatch
  emits the target argmax, a full match emits the bonus argmax.

Near-tie flags mark decisions whose outcome could flip under a different but
equally valid float32 rounding of the same quantities:
  accept  |u - p(d)/q(d)| < 1e-5
  argmax  top-2 logit gap < 1e-4
  topk    k-th minus (k+1)-th largest logit < 1e-4  (only when k < V)
  cdf     t within 1e-5 * sum(w) of an interior boundary of the chosen entry

Pins: tests/test_oracle_distributions.py (torch.topk/torch.softmax,
np.cumsum + np.searchsorted inverse CDF, the closed form 1 - TV(p, q) for the
acceptance rate, hand-built tie and degenerate cases, and the greedy
verifier tuples of tests/golden/greedy_verifier.json).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

EPS_ACCEPT = 1e-5
EPS_GAP = 1e-4
EPS_CDF = 1e-5


def topk_support(z: np.ndarray, k: int):
    """Top-k set of float32 logits ``z`` as ascending code ids, plus the
    near-tie flag of its boundary."""
    z = np.asarray(z, dtype=np.float32)
    V = z.shape[0]
    if k >= V:
        return np.arange(V), False
    # primary key: logit descending; secondary: code id ascending
    order = np.lexsort((np.arange(V), -z))
    gap = float(z[order[k - 1]]) - float(z[order[k]])
    return np.sort(order[:k]), gap < EPS_GAP


def _softmax_on(z: np.ndarray, support, temperature) -> np.ndarray:
    """exp((z_i - max) / T) normalised over ``support``, zero elsewhere."""
    zs = z[support].astype(np.float64)
    m = zs.max()
    e = np.exp((zs - m) / float(np.float32(temperature)))
    p = np.zeros(z.shape[0], dtype=np.float32)
    p[support] = (e / e.sum()).astype(np.float32)
    return p


def topk_softmax(z: np.ndarray, temperature, k: int):
    """TopKSoftmax(z; T, k) -> (dense float32 probabilities [V], topk flag)."""
    z = np.asarray(z, dtype=np.float32)
    support, flag = topk_support(z, k)
    return _softmax_on(z, support, temperature), flag


# ---- the other outcomes of near-tie decisions ----------------------------
# A decision flagged as a near tie may come out the other way under another,
# equally valid float32 rounding of its inputs.  These give the outcomes it
# could have had instead; tests re-run a frame with one of them to check that
# a code stream differing from this oracle's is such a rounding difference.

def topk_alternatives(z: np.ndarray, temperature, k: int, limit: int = 8):
    """TopKSoftmax with one set member a swapped for a non-member b, for the
    pairs whose logits differ by less than EPS_GAP (closest pairs first, at
    most ``limit``)."""
    z = np.asarray(z, dtype=np.float32)
    V = z.shape[0]
    if k >= V:
        return []
    support, _ = topk_support(z, k)
    inset = np.zeros(V, dtype=bool)
    inset[support] = True
    outside = np.flatnonzero(~inset)
    pairs = []
    for a in support:
        gaps = float(z[a]) - z[outside].astype(np.float64)
        for b in outside[gaps < EPS_GAP]:
            pairs.append((float(z[a]) - float(z[b]), int(a), int(b)))
    pairs.sort()
    out = []
    for _, a, b in pairs[:limit]:
        alt = np.sort(np.concatenate([support[support != a], [b]]))
        out.append(_softmax_on(z, alt, temperature))
    return out


def argmax_alternatives(z: np.ndarray):
    """Codes other than the argmax whose logit is within EPS_GAP of it."""
    z = np.asarray(z, dtype=np.float32)
    i = int(np.argmax(z))
    close = np.flatnonzero(float(z[i]) - z.astype(np.float64) < EPS_GAP)
    return [int(c) for c in close if c != i]


def sample_alternatives(w: np.ndarray, u):
    """The neighbours Sample(w, u) could have chosen instead when its CDF
    near-tie flag is set: the positive entry before the chosen one when t is
    within EPS_CDF * sum of their shared boundary, the one after it when the
    chosen entry's upper boundary is that close."""
    w = np.asarray(w, dtype=np.float32)
    u = np.float32(u)
    ids = np.flatnonzero(w > 0)
    tot = np.float32(0.0)
    for i in ids:
        tot = np.float32(tot + w[i])
    t = np.float32(u * tot)
    eps = float(tot) * EPS_CDF
    run = np.float32(0.0)
    before = run
    for pos, i in enumerate(ids):
        before = run
        run = np.float32(run + w[i])
        if t < run:
            out = []
            if pos > 0 and abs(float(t) - float(before)) < eps:
                out.append(int(ids[pos - 1]))
            if pos + 1 < ids.size and abs(float(run) - float(t)) < eps:
                out.append(int(ids[pos + 1]))
            return out
    if ids.size > 1 and abs(float(t) - float(before)) < eps:
        return [int(ids[-2])]
    return []


def argmax_with_gap(z: np.ndarray):
    """Greedy choice: (argmax with ties to the lowest id, top-2 near-tie flag)."""
    z = np.asarray(z, dtype=np.float32)
    i = int(np.argmax(z))
    if z.shape[0] == 1:
        return i, False
    rest = np.delete(z, i)
    gap = float(z[i]) - float(rest.max())
    return i, gap < EPS_GAP


def sample(w: np.ndarray, u) -> tuple[int, bool]:
    """Sample(w, u): sequential float32 inverse CDF over the positive entries
    of ``w`` in ascending code order.  Returns (code, cdf near-tie flag)."""
    w = np.asarray(w, dtype=np.float32)
    u = np.float32(u)
    ids = np.flatnonzero(w > 0)
    if ids.size == 0:
        raise ValueError("sample(): no positive weight")
    tot = np.float32(0.0)
    for i in ids:
        tot = np.float32(tot + w[i])
    t = np.float32(u * tot)
    eps = float(tot) * EPS_CDF
    run = np.float32(0.0)
    before = run
    for pos, i in enumerate(ids):
        before = run
        run = np.float32(run + w[i])
        if t < run:
            near_lo = pos > 0 and abs(float(t) - float(before)) < eps
            near_hi = pos + 1 < ids.size and abs(float(run) - float(t)) < eps
            return int(i), bool(near_lo or near_hi)
    # t == sum after rounding: the last positive entry owns the top end
    near = ids.size > 1 and abs(float(t) - float(before)) < eps
    return int(ids[-1]), bool(near)


def accept_test(p_d, q_d, u) -> tuple[bool, bool]:
    """min(1, p/q) acceptance: (accepted, accept near-tie flag)."""
    p_d, q_d, u = np.float32(p_d), np.float32(q_d), np.float32(u)
    ratio = np.float32(p_d / q_d)
    return bool(u < ratio), abs(float(u) - float(ratio)) < EPS_ACCEPT


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalised residual max(0, p - q) in float32 (Sample normalises)."""
    d = np.asarray(p, np.float32) - np.asarray(q, np.float32)
    return np.maximum(d, np.float32(0.0)).astype(np.float32)


def residual_or_target(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """The weights a rejected position is resampled from."""
    r = residual(p, q)
    return r if np.any(r > 0) else np.asarray(p, np.float32)


def _keep(kind, t, near, default, alternatives):
    return default


def accept_scan(drafts, qs, ps, u_accept, u_target, choose=_keep):
    """Stochastic accept scan of one round (guide, "How a round works",
    step 3).  ``drafts[t-1]`` was drawn from ``qs[t-1]``; ``ps[r]`` is the
    verified distribution of row r (row t-1 scores draft t, row gamma the
    bonus position).  ``u_accept(t)`` and ``u_target(t)`` give the uniforms
    of offset t.  Returns (emitted codes, drafts accepted, [(offset, kind)]
    near ties) where kind is 'accept' or 'cdf'.  ``choose(kind, t, near,
    outcome, alternatives)`` sees every decision and returns the outcome to
    use (by default the computed one)."""
    gamma = len(drafts)
    emitted, near = [], []
    for t in range(1, gamma + 1):
        d = drafts[t - 1]
        ok, f_acc = accept_test(ps[t - 1][d], qs[t - 1][d], u_accept(t))
        if f_acc:
            near.append((t, "accept"))
        ok = choose("accept", t, f_acc, ok, [not ok])
        if ok:
            emitted.append(d)
            continue
        w = residual_or_target(ps[t - 1], qs[t - 1])
        code, f_cdf = sample(w, u_target(t))
        if f_cdf:
            near.append((t, "cdf"))
            code = choose("cdf", t, f_cdf, code, sample_alternatives(w, u_target(t)))
        emitted.append(code)
        return emitted, t - 1, near
    code, f_cdf = sample(ps[gamma], u_target(gamma + 1))
    if f_cdf:
        near.append((gamma + 1, "cdf"))
        code = choose("cdf", gamma + 1, f_cdf, code,
                      sample_alternatives(ps[gamma], u_target(gamma + 1)))
    emitted.append(code)
    return emitted, gamma, near


@dataclass(frozen=True)
class GreedyRound:
    """Decision of one greedy verification block: the accepted draft prefix,
    the codes emitted this round, and the first rejected draft offset."""
    accepted: tuple
    emitted: tuple
    rejected_at: int | None


def verify_greedy(draft, target_argmax) -> GreedyRound:
    """Greedy argmax-equality verification of one block.

    ``target_argmax`` scores every drafted position plus the one after it, so
    it must be exactly one longer than ``draft``.  The matching prefix of the
    draft is kept; the first mismatch is replaced by the target's choice and
    ends the round; a full match is followed by the target's bonus choice.
    Pure function: no cache is touched here.
    """
    draft, target_argmax = tuple(draft), tuple(target_argmax)
    if len(target_argmax) != len(draft) + 1:
        raise ValueError("target_argmax must have one entry per drafted "
                         "position plus one for the bonus position")
    n_match = 0
    while n_match < len(draft) and draft[n_match] == target_argmax[n_match]:
        n_match += 1
    accepted = draft[:n_match]
    emitted = accepted + (target_argmax[n_match],)
    rejected = n_match if n_match < len(draft) else None
    return GreedyRound(accepted, emitted, rejected)
