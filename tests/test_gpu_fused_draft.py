"""GPU parity of the fused next-round drafts (cfg.fused_draft = 1; "RVQ
Position Aware Speculative Decoding ...", section 2.2 and Figure 3: one call
verifies a round and drafts the next): the drafts and committed codes are
the oracle's (oracle.spec, which drafts from h_s after acceptance), under the
frame rule of gpu_util.compare_frames, on the one-stream GEMV path (heads
grouped per block), the fp32 matrix-core heads (64 streams) and the packed
bf16 heads (64 streams), greedy and sampled, with and without position-aware
offsets (which enter as head . b_t added to the candidate rows' logits)."""
import numpy as np
import pytest

import synth
from gpu_util import (compare_frames, decode_gpu, dparams, handle, log, offsets_setup,
                      oracle_frames, spread_pairs)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _check(cid, c, hf, c0, seeds, pairs, got, model=None, exact_stats=False):
    gc, gf, gst = got
    oc, of, ost, rerun = oracle_frames(cid, dparams(c), hf, c0, seeds, pairs, model=model)
    res = compare_frames(np.array([gc[f, b] for f, b in pairs]),
                         np.array([gf[f, b] for f, b in pairs]), oc, of,
                         rerun=rerun, tag=f"{cid} fused drafts")
    log(f"{cid} fused N={c['verify_size']} K={c.get('draft_offsets', 0)}: "
        f"{res['frames']} frames, {res['exact']} exact, {res['flip_explained']} "
        f"explained by a near-tie flip, {len(res['unflagged'])} unexplained")
    assert not res["unflagged"], res["unflagged"][:3]
    if exact_stats and res["exact"] == res["frames"] == gst["frames"]:
        for k in ("frames", "codes", "prefill_passes", "rounds", "bonus", "proposed", "accepted"):
            assert gst[k] == ost[k], k


@pytest.mark.parametrize("N", [2, 3, 4, 8])
def test_fused_tiny_all_frames(N):
    c = synth.config("tiny", verify_size=N, frames=100, fused_draft=1)
    hf, c0, seeds = synth.make_inputs(c)
    h = handle("tiny", verify_size=N, fused_draft=1)
    log(f"decode tiny fused N={N} F=100")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 100
    _check("tiny", c, hf, c0, seeds, [(f, 0) for f in range(100)], got, exact_stats=True)


def test_fused_tiny_greedy_equals_ar():
    c = synth.config("tiny-greedy", frames=200, fused_draft=1)
    hf, c0, seeds = synth.make_inputs(c)
    h = handle("tiny-greedy", fused_draft=1)
    log("decode tiny-greedy fused F=200")
    got = decode_gpu(h, hf, c0, seeds)
    _check("tiny-greedy", c, hf, c0, seeds, [(f, 0) for f in range(0, 200, 2)], got)
    ar = decode_gpu(handle("tiny-greedy", verify_size=0), hf, c0, seeds)
    assert not compare_frames(got[0], got[1], ar[0], ar[1])["unflagged"]


def test_fused_tiny_64_streams():
    c = synth.config("tiny-64", frames=6, fused_draft=1)
    hf, c0, seeds = synth.make_inputs(c)
    h = handle("tiny-64", fused_draft=1)
    log("decode tiny-64 fused B=64 F=6")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 6 * 64
    _check("tiny-64", c, hf, c0, seeds, spread_pairs(6, 64, 96, seed=1), got)


def test_fused_few_streams():
    """Four streams on the one-stream GEMV path: a head's rows come from
    several streams."""
    c = synth.config("tiny-64", frames=5, streams=4, fused_draft=1)
    hf, c0, seeds = synth.make_inputs(c)
    h = handle("tiny-64", max_streams=4, fused_draft=1)
    log("decode tiny fused B=4 F=5")
    got = decode_gpu(h, hf, c0, seeds)
    _check("tiny-64", c, hf, c0, seeds, [(f, b) for f in range(5) for b in range(4)], got,
           exact_stats=True)


def test_fused_qwen3tts_sampled():
    """The one-stream benchmark configuration (qwen3tts, N = 4, drafts
    folded into the verify tail): 60 of 100 decoded frames against the
    oracle."""
    c = synth.config("qwen3tts", frames=100, fused_draft=1)
    hf, c0, seeds = synth.make_inputs(c)
    h = handle("qwen3tts", fused_draft=1)
    log("decode qwen3tts fused F=100")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 100
    _check("qwen3tts", c, hf, c0, seeds, spread_pairs(100, 1, 60, seed=2), got)


def test_fused_qwen3tts_64_streams_sampled():
    c = synth.config("qwen3tts-64", frames=6, fused_draft=1)
    hf, c0, seeds = synth.make_inputs(c)
    h = handle("qwen3tts-64", fused_draft=1)
    log("decode qwen3tts-64 fused B=64 F=6")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 6 * 64
    _check("qwen3tts-64", c, hf, c0, seeds, spread_pairs(6, 64, 24, seed=3), got)


@pytest.mark.parametrize("cid,K,scale,frames,pairs", [
    ("tiny", 2, 0.5, 100, None), ("qwen3tts", 3, 0.1, 40, 12), ("tiny-64", 3, 0.5, 4, 48)])
def test_fused_with_offsets(cid, K, scale, frames, pairs):
    c, h, m = offsets_setup(cid, K, scale, frames=frames, fused_draft=1)
    hf, c0, seeds = synth.make_inputs(c)
    log(f"decode {cid} fused K={K} F={frames}")
    got = decode_gpu(h, hf, c0, seeds)
    F, B = c["frames"], c["streams"]
    sel = [(f, 0) for f in range(F)] if pairs is None else spread_pairs(F, B, pairs, seed=K)
    _check(cid, c, hf, c0, seeds, sel, got, model=m, exact_stats=pairs is None)
