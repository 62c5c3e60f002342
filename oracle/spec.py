"""Per-frame decode: prefill, then speculative rounds until the frame is full.

Frame state between rounds (plainest reading of the TensorRT-Edge-LLM guide,
"How a round works", and Lesson 8, sections 03 and 07): codes c_0..c_s are
committed, the KV holds positions 0..s, h_s is held, and c_s was drawn from
head_s(h_s) but has not been fed yet.

Prefill ("RVQ Position Aware ...", Figure 1 caption; SGLang-Omni note, MTP):
rows [h_frame, E_0[c_0]] at positions 0, 1 -> h_1; c_1 ~ TopKSoftmax(head_1
h_1) with U(1, target); s = 1.

Round, while s < G - 1, with gamma = min(N - 1, G - 2 - s) (0 when
speculation is off, which is exactly the autoregressive loop):
  draft   t = 1..gamma: q_t = TopKSoftmax(head_{s+t} (h_s + b_t)),
          d_t = Sample(q_t, U(s+t, draft))                  [greedy: argmax]
          b_t is the position-aware offset of draft offset t ("RVQ Position
          Aware ...", section 2.2 and Figure 3): K vectors shared by every
          starting depth s, none (b_t = 0) when the model has no offsets or
          t > K.  Only q depends on b, so the output distribution does not.
  verify  one causal pass over rows r = 0..gamma at positions s+1+r with
          inputs E_s[c_s] (r = 0) and E_{s+r}[d_r] (r >= 1); row r is scored
          by head_{s+1+r}, so row t-1 scores draft d_t (the logit shift of
          Lesson 8, section 07) and row gamma scores the bonus position.
  accept  t = 1..gamma: keep d_t iff U(s+t, accept) < p_{t-1}(d_t)/q_t(d_t);
          at the first rejection c_{s+t} = Sample(max(0, p_{t-1} - q_t),
          U(s+t, target)) and stop; if every draft is kept,
          c_{s+gamma+1} = Sample(p_gamma, U(s+gamma+1, target)).
          [greedy: Lesson 8's argmax-equality rule, verify_greedy]
  commit  n codes; KV truncated to positions 0..s+n; h_{s+n} = row n-1's
          output; s += n.

Uniforms are indexed by absolute depth, so a depth that was drafted and
discarded is redrafted in the next round with the same draft uniform; no
committed code ever depended on it, so the reuse is statistically safe.

Pins: tests/test_oracle_spec.py -- greedy speculative output equals greedy
autoregressive output exactly for N = 2..8; brute-force enumeration of every
draft outcome equals the autoregressive joint to 1e-12; chi-square of
speculative code sequences against the exact autoregressive joint; special
cases p == q (all accepted) and k = 1 (deterministic chain equals greedy).
tests/test_oracle_offsets.py -- draft logits of an offset that moves h_s onto
a scaled unit vector equal the scaled head column; with large one-hot offsets
every draft is the argmax of its head's column at offset t; greedy output and
the chi-square of stochastic output are unchanged by offsets.
"""
from __future__ import annotations

import numpy as np

from . import distributions as dist
from .philox import PURPOSE_ACCEPT, PURPOSE_DRAFT, PURPOSE_TARGET, uniform

MAX_OFFSETS = 8


def new_stats() -> dict:
    return {
        "frames": 0, "codes": 0, "prefill_passes": 0, "rounds": 0,
        "proposed": [0] * MAX_OFFSETS, "accepted": [0] * MAX_OFFSETS,
        "bonus": 0, "near_tie_accept": 0, "near_tie_argmax": 0,
        "near_tie_cdf": 0, "near_tie_topk": 0,
    }


class _Frame:
    """Book-keeping of one frame: codes, near-tie flags, counters, and the
    log of its near-tie decisions.

    Flags: bit j is set for a near tie at depth j in a decision the frame's
    outcome used (the prefill's; in a round, drafts 1..n_acc + 1 and target
    rows 0..n_acc, the accept tests that were made and the committed draw).
    Decisions of drafts and rows past the first rejection did not shape any
    committed code, so they are not flagged.

    Log: every decision flagged as a near tie, used or not, in the order the
    frame takes them, with the outcomes it could have had instead.  A frame
    re-run with ``force = (i, a)`` takes alternative a at near tie i and is
    otherwise the same computation; the tests use it to show that a code
    stream that differs from this oracle's is explained by one such
    rounding-level flip."""

    def __init__(self, G, c0, stats, force=None):
        self.codes = np.full(G, -1, dtype=np.int32)
        self.codes[0] = c0
        self.flags = 0
        self.stats = stats
        self.force = force
        self.log = []

    def flag(self, kind: str, depth: int, hit: bool):
        if hit:
            self.flags |= 1 << depth
            self.stats["near_tie_" + kind] += 1

    def choose(self, kind: str, depth: int, near: bool, outcome, alternatives):
        """The outcome of a decision; ``alternatives`` (a list, or a callable
        giving one) are its other outcomes when ``near``."""
        if not near:
            return outcome
        alts = alternatives() if callable(alternatives) else alternatives
        i = len(self.log)
        self.log.append((depth, kind, len(alts)))
        if self.force is not None and self.force[0] == i and self.force[1] < len(alts):
            return alts[self.force[1]]
        return outcome


def draft_logits(model, j: int, t: int, h) -> np.ndarray:
    """Draft logits of offset t from h_s for depth j = s + t: head_j applied
    to h_s + b_t ("RVQ Position Aware ...", section 2.2, Figure 3), or to
    h_s alone when there is no b_t."""
    b = getattr(model, "draft_offsets", None)
    if b is not None and t <= len(b):
        h = h + b[t - 1]
    return model.logits(j, h)


def _dist(model, fr, j, z, dp):
    """Processed distribution for depth j from logits z (stochastic mode):
    (p, top-k near-tie flag)."""
    T, k = dp["temperature"], dp["top_k"]
    p, f = dist.topk_softmax(z, T, k)
    f = bool(f and k < model.V)
    p = fr.choose("topk", j, f, p, lambda: dist.topk_alternatives(z, T, k))
    return p, f


def _greedy(fr, j, z):
    code, f = dist.argmax_with_gap(z)
    code = fr.choose("argmax", j, f, code, lambda: dist.argmax_alternatives(z))
    return code, f


def _draw(fr, w, seed, depth, purpose, index=0):
    u = uniform(seed, depth, purpose, index)
    code, f = dist.sample(w, u)
    code = fr.choose("cdf", depth, f, code, lambda: dist.sample_alternatives(w, u))
    return code, f


def _prefill(model, fr, dp, h_frame, c0, seed, stats):
    """Positions 0 (talker hidden state) and 1 (E_0[c_0]); c_1 from head_1."""
    kv = model.new_kv()
    outs = model.forward_rows([np.asarray(h_frame, np.float64),
                               model.embed_row(0, c0)], [0, 1], kv)
    stats["prefill_passes"] += 1
    h = outs[1]
    if model.G > 1:
        z = model.logits(1, h)
        if dp["greedy"]:
            fr.codes[1], f = _greedy(fr, 1, z)
            fr.flag("argmax", 1, f)
        else:
            p, f = _dist(model, fr, 1, z, dp)
            fr.flag("topk", 1, f)
            fr.codes[1], f = _draw(fr, p, seed, 1, PURPOSE_TARGET)
            fr.flag("cdf", 1, f)
    return kv, h


def decode_frame(model, dp: dict, h_frame, c0: int, seed: int,
                 stats: dict | None = None, trace: list | None = None,
                 force=None, log: list | None = None):
    """Decode one frame.  ``dp`` = {verify_size, greedy, temperature, top_k}.

    Returns (codes [G] int32 with codes[0] = c0, near-tie flag bitmask).
    ``trace``, if given, receives (s, h_s, drafts, n) for every round;
    ``log``, if given, receives the frame's near-tie decisions (depth, kind,
    number of alternatives); ``force`` = (i, a) takes alternative a at near
    tie i (see _Frame).
    """
    stats = new_stats() if stats is None else stats
    G = model.G
    N = int(dp["verify_size"])
    greedy = bool(dp["greedy"])
    fr = _Frame(G, c0, stats, force)
    kv, h = _prefill(model, fr, dp, h_frame, c0, seed, stats)
    s = 1

    while s < G - 1:
        gamma = 0 if N == 0 else min(N - 1, G - 2 - s)
        # (1) draft from h_s (+ b_t) with the later heads; flags wait for the
        # outcome (only the drafts it used are flagged)
        h_s = h
        drafts, qs, dflags = [], [], []
        for t in range(1, gamma + 1):
            z = draft_logits(model, s + t, t, h)
            if greedy:
                d, f = _greedy(fr, s + t, z)
                dflags.append(["argmax"] if f else [])
            else:
                q, f1 = _dist(model, fr, s + t, z, dp)
                qs.append(q)
                d, f2 = _draw(fr, q, seed, s + t, PURPOSE_DRAFT)
                dflags.append(["topk"] * f1 + ["cdf"] * f2)
            drafts.append(d)
        # (2) verify: one causal block over the committed depth + drafts
        rows = [model.embed_row(s, int(fr.codes[s]))]
        rows += [model.embed_row(s + t, d) for t, d in enumerate(drafts, 1)]
        outs = model.forward_rows(rows, [s + 1 + r for r in range(gamma + 1)],
                                  kv)
        # (3) accept
        rflags = []
        if greedy:
            target = []
            for r in range(gamma + 1):
                a, f = _greedy(fr, s + 1 + r, model.logits(s + 1 + r, outs[r]))
                target.append(a)
                rflags.append(["argmax"] if f else [])
            rnd = dist.verify_greedy(drafts, target)
            emitted = list(rnd.emitted)
            n_acc = len(rnd.accepted)
        else:
            ps = []
            for r in range(gamma + 1):
                p, f = _dist(model, fr, s + 1 + r,
                             model.logits(s + 1 + r, outs[r]), dp)
                ps.append(p)
                rflags.append(["topk"] if f else [])
            emitted, n_acc, near = dist.accept_scan(
                drafts, qs, ps,
                lambda t: uniform(seed, s + t, PURPOSE_ACCEPT),
                lambda t: uniform(seed, s + t, PURPOSE_TARGET),
                lambda kind, t, nr, out, alts: fr.choose(kind, s + t, nr, out, alts))
            for t, kind in near:
                fr.flag(kind, s + t, True)
        for t in range(1, min(n_acc + 1, gamma) + 1):
            for kind in dflags[t - 1]:
                fr.flag(kind, s + t, True)
        for r in range(n_acc + 1):
            for kind in rflags[r]:
                fr.flag(kind, s + 1 + r, True)
        # (4) commit and truncate
        n = len(emitted)
        fr.codes[s + 1: s + 1 + n] = emitted
        kv.truncate(s + n + 1)
        h = outs[n - 1]
        if trace is not None:
            trace.append((s, h_s, tuple(int(d) for d in drafts), n))
        stats["rounds"] += 1
        for t in range(1, gamma + 1):
            stats["proposed"][t - 1] += 1
            if t <= n_acc:
                stats["accepted"][t - 1] += 1
        if n_acc == gamma:
            stats["bonus"] += 1
        s += n

    stats["frames"] += 1
    stats["codes"] += G - 1
    if log is not None:
        log.extend(fr.log)
    return fr.codes, fr.flags


def decode(model, dp: dict, h_frame, c0, seeds, frames=None, streams=None,
           stats: dict | None = None):
    """Decode frames/streams of [F][B] inputs; returns codes [F][B][G] and
    flags [F][B].  ``frames``/``streams`` select a subset (index lists)."""
    F, B = c0.shape
    fsel = range(F) if frames is None else frames
    bsel = range(B) if streams is None else streams
    codes = np.full((F, B, model.G), -1, dtype=np.int32)
    flags = np.zeros((F, B), dtype=np.uint32)
    for f in fsel:
        for b in bsel:
            codes[f, b], flags[f, b] = decode_frame(
                model, dp, h_frame[f, b], int(c0[f, b]), int(seeds[f, b]),
                stats)
    return codes, flags


def talker_feedback(model, codes) -> np.ndarray:
    """The codec part of the Talker's next input for a finished frame
    (SGLang-Omni note, the Talker/CodePredictor hand-off paragraph; "RVQ
    Position Aware ...", section 2.1): the sum over the frame's code groups
    g = 0..G-1 of that group's embedding row E_g[c_g], in float64.  The text
    projection the Talker adds is not part of the CodePredictor.

    Pins: tests/test_oracle_feedback.py -- one-hot matrix products give the
    same vector, replacing one code changes it by the difference of the two
    rows, and a hand-sized table model."""
    acc = np.zeros(model.H, dtype=np.float64)
    for g in range(model.G):
        acc = acc + model.embed_row(g, int(codes[g]))
    return acc


def codes_per_round(stats: dict) -> float:
    """Committed codes per verify pass (a round commits 1 + accepted drafts;
    the autoregressive loop scores 1.0)."""
    return (stats["codes"] - stats["frames"]) / max(stats["rounds"], 1) \
        if stats["rounds"] else 0.0
