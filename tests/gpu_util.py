"""Shared helpers of the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import functools
import sys

import numpy as np

import synth


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def weights(cid: int):
    return synth.make_weights(synth.config(cid))


@functools.lru_cache(maxsize=3)
def oracle_model(cid: int):
    from oracle import decoder
    return decoder.Model(synth.config(cid), weights(cid))


@functools.lru_cache(maxsize=2)
def device_weights(cid: int):
    from speculative_decoding_rvq_amd import binding
    return binding.weights_to_device(weights(cid))


def handle(cid: int, max_streams: int | None = None, **cfg):
    """A library handle for workload ``cid`` with cfg fields overridden."""
    from speculative_decoding_rvq_amd import binding
    c = synth.config(cid)
    return binding.Handle(c, device_weights(cid), max_streams=max_streams,
                          cfg_overrides=cfg)


def decode_gpu(h, hf, c0, seeds):
    """Run cp_spec_decode_frames on numpy inputs; returns codes, flags, stats."""
    import torch
    from speculative_decoding_rvq_amd import binding
    F, B = c0.shape
    G = h.cfg.code_groups
    dh = torch.from_numpy(np.ascontiguousarray(hf)).cuda()
    dc = torch.from_numpy(np.ascontiguousarray(c0)).cuda()
    ds = torch.from_numpy(np.ascontiguousarray(seeds).view(np.int64)).cuda()
    out = torch.full((F, B, G), -7, dtype=torch.int32, device="cuda")
    fl = torch.zeros((F, B), dtype=torch.int32, device="cuda")
    st = binding.new_stats_tensor()
    h.decode_frames(dh, dc, ds, out, fl, st)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), fl.cpu().numpy().view(np.uint32),
            binding.get_stats(st))


# Per-workload parity counts of the session, printed by conftest at the end
# of the run: {workload: {"frames", "exact", "flip", "unexplained",
# "flagged", "flag_diff"}}.
PARITY = {}


def _record(tag, res):
    if tag is None:
        return
    acc = PARITY.setdefault(tag, {"frames": 0, "exact": 0, "flip": 0,
                                  "unexplained": 0, "flagged": 0, "flag_diff": 0})
    acc["flag_diff"] += res["flag_diff"]
    acc["frames"] += res["frames"]
    acc["exact"] += res["exact"]
    acc["flip"] += res["flip_explained"]
    acc["unexplained"] += len(res["unflagged"])
    acc["flagged"] += res["flagged_frames"]


def compare_frames(gc, gf, oc, of, rerun=None, tag=None):
    """Frame-level parity rule.

    A frame passes when its G codes equal the reference's.  Otherwise let j
    be the first differing depth:
      * with ``rerun`` (the reference is the oracle): the frame passes only
        if the oracle, re-run with one of its near-tie decisions at a depth
        <= j taken the other way, gives exactly the GPU's codes.
        ``rerun(i, force, log)`` decodes selected frame i again (force =
        (near-tie index, alternative) or None; log = a list receiving the
        frame's near-tie decisions (depth, kind, alternatives)).
      * without (two GPU runs): bit j of either side's near-tie flags must be
        set.
    Returns counts and the unexplained frames; ``tag`` adds the counts to the
    session's PARITY table."""
    gc = gc.reshape(-1, gc.shape[-1])
    oc = oc.reshape(-1, oc.shape[-1])
    gf = np.asarray(gf).reshape(-1).astype(np.uint64)
    of = np.asarray(of).reshape(-1).astype(np.uint64)
    res = {"frames": gc.shape[0], "exact": 0, "flip_explained": 0,
           "flagged_mismatch": 0, "unflagged": [], "flag_diff": 0,
           "flagged_frames": int(np.sum((gf | of) != 0))}
    for i in range(gc.shape[0]):
        diff = np.flatnonzero(gc[i] != oc[i])
        if diff.size == 0:
            res["exact"] += 1
            # same outcome, same decisions used: the near-tie bits agree
            # unless a margin straddles a threshold (rare)
            res["flag_diff"] += int(gf[i] != of[i])
            continue
        j = int(diff[0])
        if rerun is None:
            if (gf[i] | of[i]) & np.uint64(1 << j):
                res["flagged_mismatch"] += 1
                continue
        else:
            log = []
            rerun(i, None, log)
            hit = None
            for k, (depth, kind, nalt) in enumerate(log):
                if depth > j:
                    continue
                for a in range(nalt):
                    codes, _ = rerun(i, (k, a), None)
                    if np.array_equal(np.asarray(codes), gc[i]):
                        hit = (depth, kind)
                        break
                if hit:
                    break
            if hit:
                res["flip_explained"] += 1
                res["flagged_mismatch"] += 1
                log(f"frame {i}: first difference at depth {j}, "
                         f"reproduced by the oracle with its {hit[1]} near "
                         f"tie at depth {hit[0]} taken the other way")
                continue
        res["unflagged"].append((i, j, gc[i].tolist(), oc[i].tolist()))
    _record(tag, res)
    return res


def offsets_setup(cid: str, K: int, scale: float, **cfg):
    """Workload ``cid`` with K seeded position-aware draft offsets: (config,
    library handle, oracle model); the other weights are the cached ones."""
    import copy
    import torch
    from speculative_decoding_rvq_amd import binding
    c = synth.config(cid, draft_offsets=K, offset_scale=scale, **cfg)
    off = synth.make_offsets(c)
    wdev = {**device_weights(cid), "draft_offsets": torch.from_numpy(off).cuda()}
    h = binding.Handle(c, wdev)
    m = copy.copy(oracle_model(cid))
    m.draft_offsets = off.astype(np.float64)
    return c, h, m


def oracle_frames(cid, dp, hf, c0, seeds, pairs, model=None, tree=None):
    """Oracle codes/flags for the selected (frame, stream) pairs, the
    accumulated oracle stats, and a rerun(i, force, log) function for
    compare_frames (i indexes ``pairs``)."""
    from oracle import spec
    from oracle import tree as otree
    m = oracle_model(cid) if model is None else model

    def one(f, b, st, force=None, lg=None):
        if tree is not None:
            return otree.decode_frame_tree(m, dp, otree.Tree(tree), hf[f, b],
                                           int(c0[f, b]), int(seeds[f, b]), st,
                                           force=force, log=lg)
        return spec.decode_frame(m, dp, hf[f, b], int(c0[f, b]),
                                 int(seeds[f, b]), st, force=force, log=lg)

    st = spec.new_stats()
    codes, flags = [], []
    for f, b in pairs:
        c, fl = one(f, b, st)
        codes.append(c)
        flags.append(fl)

    def rerun(i, force, lg):
        f, b = pairs[i]
        return one(f, b, spec.new_stats(), force, lg)

    return np.array(codes), np.array(flags, dtype=np.uint32), st, rerun


def spread_pairs(F, B, n, seed):
    """n distinct (frame, stream) pairs covering every stream when n >= B:
    stream b gets frames drawn without replacement, the first and last frame
    of the run included."""
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (F - 1, B - 1)}
    b = 0
    while len(pairs) < min(n, F * B):
        pairs.add((int(rng.integers(0, F)), b % B))
        b += 1
    return sorted(pairs)


def dparams(c: dict, **over) -> dict:
    d = dict(verify_size=c["verify_size"], greedy=c["greedy"],
             temperature=c["temperature"], top_k=c["top_k"])
    d.update(over)
    return d
