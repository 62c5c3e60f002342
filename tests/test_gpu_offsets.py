"""GPU parity of the position-aware draft offsets ("RVQ Position Aware
Speculative Decoding ...", section 2.2, Figure 3): draft offset t scores
head_{s+t} on h_s + b_t, over the
GEMV (1 stream), fp32 matrix-core (64 streams) and bf16 batched (64 streams)
head paths, with K equal to the window and K below it (drafts past K see h_s).
Frame rule of gpu_util.compare_frames (exact, or reproduced by the oracle
with one near-tie decision taken the other way).
"""
import numpy as np
import pytest

import synth
from gpu_util import (compare_frames, decode_gpu, dparams, handle, log,
                      offsets_setup, oracle_frames)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _check(cid, c, m, hf, c0, seeds, pairs, got, exact_stats):
    gc, gf, gst = got
    dp = dparams(c)
    oc, of, ost, rerun = oracle_frames(cid, dp, hf, c0, seeds, pairs, model=m)
    sel_c = np.array([gc[f, b] for f, b in pairs])
    sel_f = np.array([gf[f, b] for f, b in pairs])
    res = compare_frames(sel_c, sel_f, oc, of, rerun=rerun, tag=f"{cid} offsets")
    log(f"{cid} K={c['draft_offsets']} N={c['verify_size']}: {res['frames']} "
        f"frames, {res['exact']} exact, {res['flip_explained']} explained by "
        f"a near-tie flip, {len(res['unflagged'])} unexplained")
    assert not res["unflagged"], res["unflagged"][:3]
    if exact_stats and res["exact"] == res["frames"]:
        assert gst["proposed"] == ost["proposed"]
        assert gst["accepted"] == ost["accepted"]
        assert gst["rounds"] == ost["rounds"]
    return res


def test_offsets_tiny_all_frames():
    c, h, m = offsets_setup("tiny", 2, 0.5)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode tiny K=2 F=100")
    got = decode_gpu(h, hf, c0, seeds)
    _check("tiny", c, m, hf, c0, seeds, [(f, 0) for f in range(100)], got, True)
    # the offsets moved the acceptance counts away from the offset-free run
    base = decode_gpu(handle("tiny"), hf, c0, seeds)
    assert got[2]["accepted"] != base[2]["accepted"]


def test_offsets_below_the_window_greedy():
    """N = 8 with K = 3: offsets 4..7 draft from h_s alone; greedy output
    still equals the autoregressive output."""
    c, h, m = offsets_setup("tiny-greedy", 3, 0.5, verify_size=8, frames=60)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode tiny-greedy K=3 N=8 F=60")
    got = decode_gpu(h, hf, c0, seeds)
    _check("tiny-greedy", c, m, hf, c0, seeds, [(f, 0) for f in range(60)], got, True)
    ar = decode_gpu(handle("tiny-greedy", verify_size=0), hf, c0, seeds)
    assert not compare_frames(got[0], got[1], ar[0], ar[1])["unflagged"]


def test_zero_offsets_are_bit_identical_to_none():
    from speculative_decoding_rvq_amd import binding
    from gpu_util import device_weights
    c = synth.config("tiny-64", frames=3, draft_offsets=3)
    wdev = {**device_weights("tiny-64"),
            "draft_offsets": torch.zeros((3, c["hidden"]), device="cuda")}
    hf, c0, seeds = synth.make_inputs(c)
    log("decode tiny-64 zero offsets F=3")
    a = decode_gpu(binding.Handle(c, wdev), hf, c0, seeds)
    b = decode_gpu(handle("tiny-64"), hf, c0, seeds)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    assert a[2] == b[2]


def test_offsets_tiny_64_streams():
    c, h, m = offsets_setup("tiny-64", 3, 0.5, frames=4)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode tiny-64 K=3 B=64 F=4")
    got = decode_gpu(h, hf, c0, seeds)
    pairs = [(f, b) for f in range(4) for b in range(0, 64, 3)]
    _check("tiny-64", c, m, hf, c0, seeds, pairs, got, False)


def test_offsets_qwen3tts_sampled():
    c, h, m = offsets_setup("qwen3tts", 3, 0.1, frames=200)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode qwen3tts K=3 F=200")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 200
    _check("qwen3tts", c, m, hf, c0, seeds, [(f, 0) for f in range(0, 200, 10)], got, False)


def test_offsets_qwen3tts_64_streams_sampled():
    c, h, m = offsets_setup("qwen3tts-64", 3, 0.1, frames=12)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode qwen3tts-64 K=3 B=64 F=12")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 12 * 64
    from gpu_util import spread_pairs
    _check("qwen3tts-64", c, m, hf, c0, seeds, spread_pairs(12, 64, 24, seed=3), got, False)
