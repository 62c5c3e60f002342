"""Per-frame decode with a tree-shaped verify window.  Test infrastructure:
only tests/, the package's smoke check and the benchmark's CPU baseline use
the oracle.

Source: "RVQ Position Aware Speculative Decoding for On Device Text to
Speech", section 2.2 and Figure 2 (the draft heads propose several codes per
depth, arranged as a tree; the tree is packed with the committed code into one
verify block in which every node attends to its ancestors only; the standard
acceptance rule with residual resampling is applied along the tree), with
Medusa's tree attention as the pages cite it.

The pages fix the shape of the method, not every step; the readings taken
here (each kept as close to the chain window as the rule allows):
  * The tree is a fixed parent list.  Node 0 is the root: the committed code
    c_s, row 0 of the verify block.  Nodes 1..T are numbered so that a parent
    comes before its children; a node at depth d proposes the code of depth
    s + d and sits at position s + 1 + d.
  * Candidates, stochastic mode: every node draws its own code from its
    depth's draft distribution q_d = TopKSoftmax(head_{s+d}(h_s + b_d)) with
    U(s + d, draft, j), j = the node's number among the window's nodes of
    depth d.  Every draft head reads h_s, so the children of any node are
    independent draws from one q: the multi-candidate acceptance below is
    exact for such children.  Greedy mode: the k-th child (in node order) of
    any node proposes the k-th highest draft logit of its depth (ties to the
    lower code).
  * Verification walks down from the root.  At node v (depth d), with p' =
    TopKSoftmax(head_{s+d+1}(h_v)) and the children c_0, c_1, ... of v in
    node order: child c_k is accepted iff U(s+d+1, accept, k) <
    p'(x)/q_{d+1}(x) (x = its code); after each rejection p' becomes
    norm(max(0, p' - q_{d+1})), or stays p' when that is all zero
    (normalised with a sequential float32 sum in ascending code order when
    another child is tested on it; Sample normalises the last one itself).
    The first accepted child becomes v; when no child is accepted, or v has
    none, c_{s+d+1} = Sample(p', U(s+d+1, target)) ends the round.  Greedy: the
    first child whose code equals the argmax of head_{s+d+1}(h_v) is
    accepted, otherwise the argmax is committed and the round ends.
  * Ancestor-only attention: node v sees the committed prefix, the root and
    its ancestors, which is the chain computation over its root path; this
    oracle evaluates every node that way, from a copy of the committed cache.
  * Frame end: nodes deeper than G - 2 - s are left out of the round, as the
    chain's window is cut to gamma = min(N - 1, G - 2 - s).
  * The committed K/V after a round is that of the accepted path: positions
    0..s+n with n the codes committed.
With one child per node the tree is the chain window of oracle.spec, uniform
for uniform (the chain's draws and trials all have index 0).

Pins: tests/test_oracle_tree.py -- a one-child tree equals the chain decoder
code for code with the same flags and counters; brute-force enumeration of
every draft outcome and acceptance branch of a branching tree gives the
autoregressive joint to 1e-12; greedy trees equal greedy autoregressive
decoding; chi-square of tree-decoded frames against the exact joint.
"""
from __future__ import annotations

import copy

import numpy as np

from . import distributions as dist
from .philox import PURPOSE_ACCEPT, PURPOSE_DRAFT, PURPOSE_TARGET, uniform
from .spec import _Frame, _dist, _draw, _greedy, _prefill, draft_logits, new_stats


class Tree:
    """A verify tree from its parent list: ``parents[i - 1]`` is the parent
    of node i (i = 1..T), always lower than i; node 0 is the root."""

    def __init__(self, parents):
        self.parent = [-1] + [int(p) for p in parents]
        self.T = len(parents)
        self.depth = [0] * (self.T + 1)
        self.children = [[] for _ in range(self.T + 1)]
        for i in range(1, self.T + 1):
            p = self.parent[i]
            if not 0 <= p < i:
                raise ValueError(f"node {i}: parent {p} must precede it")
            self.depth[i] = self.depth[p] + 1
            self.children[p].append(i)
        self.max_depth = max(self.depth)

    @classmethod
    def chain(cls, length: int) -> "Tree":
        return cls(list(range(length)))


def normalise(r) -> np.ndarray:
    """r / (sequential float32 sum of its positive entries in ascending code
    order), element by element in float32."""
    r = np.asarray(r, dtype=np.float32)
    tot = np.float32(0.0)
    for w in r[r > 0]:
        tot = np.float32(tot + w)
    return (r / tot).astype(np.float32)


def _ranked(fr, depth, z, m):
    """The m highest draft logits' codes (logit descending, code ascending),
    and whether a gap under EPS_GAP separates two of the first m + 1 (then
    the ranking could come out with those two swapped)."""
    z = np.asarray(z, dtype=np.float32)
    order = np.lexsort((np.arange(z.shape[0]), -z))
    top = z[order[: m + 1]].astype(np.float64)
    near_at = [i for i in range(len(top) - 1) if top[i] - top[i + 1] < dist.EPS_GAP]
    ranked = [int(c) for c in order[: m + 1]]

    def alts():
        out = []
        for i in near_at:
            r = list(ranked)
            r[i], r[i + 1] = r[i + 1], r[i]
            out.append(r[:m])
        return out

    return fr.choose("argmax", depth, bool(near_at), ranked[:m], alts), bool(near_at)


def walk_step(p, q, children, u_accept, u_target, choose=None):
    """One node's step of the walk: the node's children (codes
    ``children[k]``, drawn from ``q``) are tested in order against the node's
    target distribution ``p``: child k is accepted iff u_accept(k) <
    p'(x)/q(x) (float32), p' = p for the first child; after a rejection p'
    becomes max(0, p' - q) (p' kept when that is all zero), divided by its
    sequential float32 sum when another child follows.  With none accepted
    the node draws Sample(p', u_target).  Returns (index of the accepted
    child or None, its code or the draw, [near-tie kinds]).  ``choose`` (as in
    accept_scan) sees every decision."""
    choose = choose or (lambda kind, k, near, out, alts: out)
    near = []
    p = np.asarray(p, np.float32)
    for k, x in enumerate(children):
        ok, f = dist.accept_test(p[x], q[x], u_accept(k))
        if f:
            near.append("accept")
        ok = choose("accept", k, f, ok, [not ok])
        if ok:
            return k, int(x), near
        p = dist.residual_or_target(p, q)
        if k + 1 < len(children):
            p = normalise(p)
    code, f = dist.sample(p, u_target)
    if f:
        near.append("cdf")
        code = choose("cdf", len(children), f, code, dist.sample_alternatives(p, u_target))
    return None, int(code), near


def decode_frame_tree(model, dp: dict, tree: Tree, h_frame, c0: int, seed: int,
                      stats: dict | None = None, trace: list | None = None,
                      force=None, log: list | None = None):
    """Decode one frame with a tree window.  ``dp`` = {greedy, temperature,
    top_k} (the tree replaces verify_size).  Returns (codes [G] int32,
    near-tie flag bitmask: the decisions of the walk's rows and of the draft
    depths it tested).  ``trace``, if given, receives (s, {node: code}, n)
    for every round; ``log`` and ``force`` as in spec.decode_frame."""
    stats = new_stats() if stats is None else stats
    G = model.G
    greedy = bool(dp["greedy"])
    fr = _Frame(G, c0, stats, force)
    kv, h = _prefill(model, fr, dp, h_frame, c0, seed, stats)
    s = 1

    while s < G - 1:
        dmax = G - 2 - s
        nodes = [i for i in range(1, tree.T + 1) if tree.depth[i] <= dmax]
        live = set(nodes)
        kids = {v: [c for c in tree.children[v] if c in live] for v in [0] + nodes}
        D = max([tree.depth[i] for i in nodes], default=0)
        # (1) candidates of every node from h_s (+ b_d); each depth's flags
        # wait for the walk
        q, code, dflags = {}, {}, {}
        for d in range(1, D + 1):
            z = draft_logits(model, s + d, d, h)
            at_d = [i for i in nodes if tree.depth[i] == d]
            if greedy:
                m = max(len(kids[tree.parent[i]]) for i in at_d)
                ranked, f = _ranked(fr, s + d, z, m)
                dflags[d] = ["argmax"] * f
                for i in at_d:
                    code[i] = ranked[kids[tree.parent[i]].index(i)]
            else:
                q[d], f = _dist(model, fr, s + d, z, dp)
                dflags[d] = ["topk"] * f
                fcdf = False
                for j, i in enumerate(at_d):
                    code[i], f = _draw(fr, q[d], seed, s + d, PURPOSE_DRAFT, j)
                    fcdf |= f
                dflags[d] += ["cdf"] * fcdf
        # (2) verify: the root row and every node, each over its root path
        hid, kvs = {}, {}
        kv0 = copy.deepcopy(kv)
        hid[0] = model.forward_rows([model.embed_row(s, int(fr.codes[s]))], [s + 1], kv0)[0]
        kvs[0] = kv0
        for i in nodes:
            d = tree.depth[i]
            kvi = copy.deepcopy(kvs[tree.parent[i]])
            hid[i] = model.forward_rows([model.embed_row(s + d, code[i])], [s + 1 + d], kvi)[0]
            kvs[i] = kvi
        stats["rounds"] += 1
        # (3) every row's target decision (argmax, or p with its top-k
        # flag), then the walk down the tree
        target, rflag = {}, {}
        for v in [0] + nodes:
            j = s + tree.depth[v] + 1
            z = model.logits(j, hid[v])
            if greedy:
                target[v], rflag[v] = _greedy(fr, j, z)
            else:
                target[v], rflag[v] = _dist(model, fr, j, z, dp)
        v, emitted = 0, []
        while True:
            d1 = tree.depth[v] + 1
            j = s + d1
            fr.flag("argmax" if greedy else "topk", j, rflag[v])
            if greedy:
                t = target[v]
                nxt = next((c for c in kids[v] if code[c] == t), None)
                emitted.append(t)
                if nxt is None:
                    break
                v = nxt
                continue
            k, x, near = walk_step(
                target[v], q.get(d1), [code[c] for c in kids[v]],
                lambda k: uniform(seed, j, PURPOSE_ACCEPT, k),
                uniform(seed, j, PURPOSE_TARGET, 0),
                lambda kind, k, nr, out, alts: fr.choose(kind, j, nr, out, alts))
            for kind in near:
                fr.flag(kind, j, True)
            emitted.append(x)
            if k is None:
                break
            v = kids[v][k]
        # (4) commit the path: codes, its K/V, h of its last node
        n = len(emitted)
        for d in range(1, min(n, D) + 1):
            for kind in dflags[d]:
                fr.flag(kind, s + d, True)
        fr.codes[s + 1: s + 1 + n] = emitted
        kv = kvs[v]
        kv.truncate(s + n + 1)
        h = hid[v]
        if trace is not None:
            trace.append((s, dict(code), n))
        for d in range(1, D + 1):
            stats["proposed"][d - 1] += 1
            if d <= n - 1:
                stats["accepted"][d - 1] += 1
        if not kids[v]:
            stats["bonus"] += 1
        s += n

    stats["frames"] += 1
    stats["codes"] += G - 1
    if log is not None:
        log.extend(fr.log)
    return fr.codes, fr.flags
