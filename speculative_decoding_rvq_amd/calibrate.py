"""Per-device choice of the verify window N.

Source: "RVQ Position Aware Speculative Decoding for On Device Text to
Speech", section 3.4 and Figure 4: how far the drafts get accepted does not
depend on the device, the verify call's cost at query length N does, so N is
calibrated once per device class from the acceptance and a profile of the
verify cost at each N.  "Speculative Decoding, Beyond Text", section 06,
states the same trade-off as a latency model (a round's cost split into
draft, verify and bookkeeping, acceptance reported per draft offset).

Here:
  * acceptance: share[t-1] = the fraction of rounds whose first t drafts were
    all accepted, read once from the stats of a decode at the widest window;
    a window of N then commits 1 + share[0] + ... + share[N-2] codes per
    round on average away from the frame's end;
  * passes per frame: a frame of G codes takes one prefill pass (c_1) and
    then rounds until c_{G-1} is committed; the round at committed depth s
    drafts gamma = min(N - 1, G - 2 - s) codes (the frame's end cuts the
    window) and commits k codes with the probability the shares give for
    gamma drafts, so the expected pass count follows by recursion over s;
  * cost: for every N, one decode on this GPU; one verify pass costs the
    decode's device time over its passes (rounds plus prefills; one graph
    replay advances every stream by one pass);
  * choice: the N with the fewest expected microseconds of passes per frame
    (the most codes per microsecond), ties to the smaller N.
The measured codes/s of each N's decode are returned beside the prediction.
"""
from __future__ import annotations


def expected_codes_per_round(share, n: int) -> float:
    """Codes a round with verify window n commits on average: 1 (the
    target's own draw) plus the share of rounds whose first t drafts were
    all accepted, for t = 1 .. n-1."""
    if n < 1:
        raise ValueError("verify window must be at least 1")
    return 1.0 + float(sum(share[: n - 1]))


def commit_distribution(share, gamma: int) -> list:
    """P(a round with gamma drafts commits k codes), k = 1 .. gamma + 1:
    k - 1 drafts accepted, then the first rejection (or every draft
    accepted and the row after the last one drawn)."""
    if gamma < 0:
        raise ValueError("gamma must be non-negative")
    full = [1.0] + [float(share[t]) if t < len(share) else 0.0 for t in range(gamma)]
    return [full[k - 1] - (full[k] if k <= gamma else 0.0) for k in range(1, gamma + 2)]


def expected_passes_per_frame(share, n: int, groups: int) -> float:
    """Expected decoder passes for one frame of `groups` codes with verify
    window n: the prefill pass plus the rounds from committed depth 1 until
    depth groups - 1, each round's window cut to min(n - 1, groups - 2 - s)
    drafts."""
    if n < 1:
        raise ValueError("verify window must be at least 1")
    if groups < 2:
        raise ValueError("a frame has at least two code groups")
    last = groups - 1
    rounds = [0.0] * (last + n + 1)  # expected rounds from depth s; zero from the last depth on
    for s in range(last - 1, 0, -1):
        gamma = min(n - 1, last - 1 - s)
        dist = commit_distribution(share, gamma)
        rounds[s] = 1.0 + sum(p * rounds[s + k] for k, p in enumerate(dist, start=1))
    return 1.0 + rounds[1]


def choose_window(share, us_per_pass: dict, groups: int | None = None) -> int:
    """The window with the most expected codes per microsecond of pass;
    ties go to the smaller window.  With `groups`, a frame's passes come
    from expected_passes_per_frame (the frame's end and its prefill pass
    counted), else from expected_codes_per_round alone."""
    if not us_per_pass:
        raise ValueError("no window sizes to choose from")
    best, best_rate = None, -1.0
    for n in sorted(us_per_pass):
        us = float(us_per_pass[n])
        if us <= 0.0:
            raise ValueError(f"window {n}: pass time must be positive")
        if groups is None:
            rate = expected_codes_per_round(share, n) / us
        else:
            rate = (groups - 1) / (expected_passes_per_frame(share, n, groups) * us)
        if rate > best_rate:
            best, best_rate = n, rate
    return best


def calibrate_window(c: dict, wdev: dict, h_frame, c0, seeds,
                     sizes=(2, 3, 4, 5, 6, 8), repeats: int = 2) -> dict:
    """Profile one verify pass at every window in `sizes` on the current
    GPU and choose N.  `c` is the decoder configuration (its verify_size is
    replaced per size), `wdev` the device weights, h_frame / c0 / seeds the
    frames to decode (device tensors, as for decode_frames).  Returns the
    chosen window, the per-offset acceptance shares and, per size, the pass
    time, the measured codes/s and codes per verify pass, and the expected
    codes per round."""
    import torch

    from .binding import Handle, get_stats, new_stats_tensor
    sizes = sorted(set(int(n) for n in sizes))
    if not sizes or sizes[0] < 2:
        raise ValueError("window sizes must be at least 2 (one draft)")
    if repeats < 1:
        raise ValueError("repeats must be at least 1")
    F, B = int(c0.shape[0]), int(c0.shape[1])
    G = int(c["groups"])
    out = torch.empty((F, B, G), dtype=torch.int32, device="cuda")
    rows = {}
    for n in sizes:
        h = Handle(dict(c, verify_size=n), wdev)
        try:
            st = new_stats_tensor()
            h.decode_frames(h_frame, c0, seeds, out)  # warm-up: graph capture, caches
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(repeats):
                h.decode_frames(h_frame, c0, seeds, out, None, st if i == 0 else None)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / repeats
        finally:
            h.close()
        s = get_stats(st)
        passes = max(s["rounds"] + s["prefill_passes"], 1)
        rows[n] = {"codes_per_s": F * B * (G - 1) / (ms / 1e3),
                   "codes_per_verify_pass": (s["codes"] - s["frames"]) / max(s["rounds"], 1),
                   "us_per_pass": 1e3 * ms / passes * B,
                   "stats": s}
    widest = rows[sizes[-1]]["stats"]
    share = [a / p for a, p in zip(widest["accepted"], widest["proposed"]) if p]
    for n in sizes:
        rows[n]["expected_codes_per_round"] = expected_codes_per_round(share, n)
        rows[n]["expected_passes_per_frame"] = expected_passes_per_frame(share, n, G)
        rows[n]["passes_per_frame"] = (rows[n]["stats"]["rounds"] + rows[n]["stats"]["prefill_passes"]) / max(
            rows[n]["stats"]["frames"], 1)
        del rows[n]["stats"]
    chosen = choose_window(share, {n: rows[n]["us_per_pass"] for n in sizes}, G)
    return {"verify_size": chosen,
            "measured_best": max(sizes, key=lambda n: rows[n]["codes_per_s"]),
            "accepted_share_by_offset": share,
            "by_verify_size": rows}
