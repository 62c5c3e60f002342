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


def compare_frames(gc, gf, oc, of):
    """Frame-level parity rule: a frame matches, or its first differing depth
    j has a near-tie flag (either side) at a depth <= j."""
    gc = gc.reshape(-1, gc.shape[-1])
    oc = oc.reshape(-1, oc.shape[-1])
    gf = np.asarray(gf).reshape(-1).astype(np.uint64)
    of = np.asarray(of).reshape(-1).astype(np.uint64)
    res = {"frames": gc.shape[0], "exact": 0, "flagged_mismatch": 0,
           "unflagged": [], "flagged_frames": int(np.sum((gf | of) != 0))}
    for i in range(gc.shape[0]):
        diff = np.flatnonzero(gc[i] != oc[i])
        if diff.size == 0:
            res["exact"] += 1
            continue
        j = int(diff[0])
        mask = np.uint64((1 << (j + 1)) - 1)
        if (gf[i] | of[i]) & mask:
            res["flagged_mismatch"] += 1
        else:
            res["unflagged"].append((i, j, gc[i].tolist(), oc[i].tolist()))
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


def oracle_frames(cid, dp, hf, c0, seeds, pairs, model=None):
    """Oracle codes/flags for the selected (frame, stream) pairs."""
    from oracle import spec
    m = oracle_model(cid) if model is None else model
    st = spec.new_stats()
    codes, flags = [], []
    for f, b in pairs:
        c, fl = spec.decode_frame(m, dp, hf[f, b], int(c0[f, b]),
                                  int(seeds[f, b]), st)
        codes.append(c)
        flags.append(fl)
    return np.array(codes), np.array(flags, dtype=np.uint32), st


def dparams(c: dict, **over) -> dict:
    d = dict(verify_size=c["verify_size"], greedy=c["greedy"],
             temperature=c["temperature"], top_k=c["top_k"])
    d.update(over)
    return d
