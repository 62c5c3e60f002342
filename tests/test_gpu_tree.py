"""GPU parity of the tree-shaped verify window ("RVQ Position Aware
Speculative Decoding ...", section 2.2 and Figure 2) against oracle.tree.
Frame rule as in the other decode tests (gpu_util.compare_frames): equal
codes, or the oracle re-run with one near-tie decision taken the other way
reproduces them.  A one-child tree runs the tree kernels
over the chain's computation and must equal the GPU chain window exactly.
"""
import numpy as np
import pytest

import synth
from gpu_util import compare_frames, decode_gpu, device_weights, handle, log, oracle_frames, oracle_model

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _tree_handle(cid, parents, max_streams=None, wdev=None, **cfg):
    from speculative_decoding_rvq_amd import binding
    c = synth.config(cid, tree=list(parents), **cfg)
    return c, binding.Handle(c, wdev or device_weights(cid), max_streams=max_streams)


def _check(name, c, m, parents, got, hf, c0, seeds, pairs):
    gc, gf, gst = got
    dp = dict(greedy=c["greedy"], temperature=c["temperature"], top_k=c["top_k"])
    oc, of, ost, rerun = oracle_frames(None, dp, hf, c0, seeds, pairs, model=m, tree=parents)
    res = compare_frames(np.array([gc[f, b] for f, b in pairs]),
                         np.array([gf[f, b] for f, b in pairs]), oc, of,
                         rerun=rerun, tag=f"{name} tree")
    log(f"{name} tree {parents}: {res['frames']} frames, {res['exact']} exact, "
        f"{res['flip_explained']} explained by a near-tie flip, "
        f"{len(res['unflagged'])} unexplained")
    assert not res["unflagged"], res["unflagged"][:3]
    if res["exact"] == res["frames"] == gst["frames"]:  # every frame compared
        for k in ("frames", "codes", "prefill_passes", "rounds", "bonus"):
            assert gst[k] == ost[k], k
        assert gst["proposed"] == ost["proposed"] and gst["accepted"] == ost["accepted"]
    return res


def widths_tree(widths, extra_root=0):
    """Parent list of a tree whose nodes at depth d each have widths[d]
    children (breadth-first numbering), plus extra_root more children of the
    root without children of their own."""
    par, level, nid = [], [0], 0
    for d, w in enumerate(widths):
        nxt = []
        for p in level:
            for _ in range(w):
                nid += 1
                par.append(p)
                nxt.append(nid)
        if d == 0:
            for _ in range(extra_root):
                nid += 1
                par.append(0)
        level = nxt
    return par


T15 = widths_tree((3, 2, 1))            # 15 nodes, depth 3
T31 = widths_tree((2, 2, 2, 2), 1)      # 31 nodes, depth 4
T63 = widths_tree((2, 2, 2, 2, 2), 1)   # 63 nodes, depth 5


@pytest.mark.parametrize("parents", [[0, 0, 1], [0, 0, 0, 1, 2], [0, 1, 1, 2, 3, 0, 6], T15, T31, T63],
                         ids=["3", "5", "7", "15", "31", "63"])
def test_tree_tiny_all_frames(parents):
    c, h = _tree_handle("tiny", parents, frames=60)
    hf, c0, seeds = synth.make_inputs(c)
    log(f"decode tiny tree {parents} F=60")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 60
    _check("tiny", c, oracle_model("tiny"), parents, got, hf, c0, seeds, [(f, 0) for f in range(60)])


@pytest.mark.parametrize("parents", [T15, T63], ids=["15", "63"])
def test_tree_thirty_two_groups(parents):
    """G = 32 (the most the library takes): the committed prefix reaches
    position 31, so the tree attention keys on up to 32 + 63 positions and
    nodes; the tiny decoder's shape with its own 32-group weights."""
    from oracle import decoder
    from speculative_decoding_rvq_amd import binding
    c = synth.config("tiny", groups=32, tree=list(parents), frames=8)
    w = synth.make_weights(c)
    h = binding.Handle(c, binding.weights_to_device(w))
    hf, c0, seeds = synth.make_inputs(c)
    log(f"decode tiny G=32 tree of {len(parents)} nodes F=8")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 8 and got[2]["codes"] == 8 * 31
    _check("tiny G=32", c, decoder.Model(c, w), parents, got, hf, c0, seeds, [(f, 0) for f in range(8)])


def test_one_child_tree_equals_gpu_chain():
    c, h = _tree_handle("tiny", [0, 1, 2], frames=60)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode tiny one-child tree vs chain N=4 F=60")
    a = decode_gpu(h, hf, c0, seeds)
    b = decode_gpu(handle("tiny", verify_size=4), hf, c0, seeds)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    for k in ("frames", "codes", "rounds", "bonus", "proposed", "accepted"):
        assert a[2][k] == b[2][k], k


def test_tree_with_offsets():
    from gpu_util import offsets_setup
    c, _, m = offsets_setup("tiny", 2, 0.5, frames=40)
    off = synth.make_offsets(c)
    wdev = {**device_weights("tiny"), "draft_offsets": torch.from_numpy(off).cuda()}
    parents = [0, 0, 1]
    ct, h = _tree_handle("tiny", parents, wdev=wdev, frames=40, draft_offsets=2, offset_scale=0.5)
    hf, c0, seeds = synth.make_inputs(ct)
    log("decode tiny tree + offsets F=40")
    got = decode_gpu(h, hf, c0, seeds)
    _check("tiny+offsets", ct, m, parents, got, hf, c0, seeds, [(f, 0) for f in range(40)])


def test_tree_four_streams():
    parents = [0, 0, 1, 2]
    c, h = _tree_handle("tiny", parents, max_streams=4, frames=6, streams=4)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode tiny tree B=4 F=6")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 24
    pairs = [(f, b) for f in range(6) for b in range(4)]
    _check("tiny B=4", c, oracle_model("tiny"), parents, got, hf, c0, seeds, pairs)


def test_tree_qwen3tts_sampled():
    parents = [0, 0, 1, 2]
    c, h = _tree_handle("qwen3tts", parents, frames=40)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode qwen3tts tree F=40")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 40
    _check("qwen3tts", c, oracle_model("qwen3tts"), parents, got, hf, c0, seeds,
           [(f, 0) for f in range(0, 40, 2)])


@pytest.mark.parametrize("parents", [[0, 0, 1, 1], T15, T31], ids=["4", "15", "31"])
def test_tree_greedy(parents):
    """Greedy trees: node k of a parent proposes the k-th highest draft
    logit; the codes equal the oracle's and the GPU's autoregressive greedy
    codes."""
    c, h = _tree_handle("tiny-greedy", parents, frames=120)
    hf, c0, seeds = synth.make_inputs(c)
    log(f"decode tiny-greedy tree {len(parents)} F=120")
    got = decode_gpu(h, hf, c0, seeds)
    _check("tiny-greedy", c, oracle_model("tiny-greedy"), parents, got, hf, c0, seeds,
           [(f, 0) for f in range(120)])
    ar = decode_gpu(handle("tiny-greedy", verify_size=0), hf, c0, seeds)
    assert not compare_frames(got[0], got[1], ar[0], ar[1])["unflagged"]


@pytest.mark.parametrize("B,parents", [(8, T15), (64, T31)], ids=["8x15", "64x31"])
def test_tree_many_streams(B, parents):
    """Tree windows on the batched path: matrix-core projections and lm_heads
    with the nodes of one depth sharing their head across streams."""
    c, h = _tree_handle("tiny-64", parents, max_streams=B, frames=4, streams=B)
    hf, c0, seeds = synth.make_inputs(c)
    log(f"decode tiny tree {len(parents)} B={B} F=4")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 4 * B
    from gpu_util import spread_pairs
    _check(f"tiny B={B}", c, oracle_model("tiny-64"), parents, got, hf, c0, seeds,
           spread_pairs(4, B, min(4 * B, 96), seed=B))


@pytest.mark.parametrize("parents", [T15, T31], ids=["15", "31"])
def test_tree_qwen3tts_large_sampled(parents):
    c, h = _tree_handle("qwen3tts", parents, frames=40)
    hf, c0, seeds = synth.make_inputs(c)
    log(f"decode qwen3tts tree {len(parents)} F=40")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 40
    _check("qwen3tts", c, oracle_model("qwen3tts"), parents, got, hf, c0, seeds,
           [(f, 0) for f in range(0, 40, 4)])


def test_tree_qwen3tts_64_streams_sampled():
    from gpu_util import spread_pairs
    c, h = _tree_handle("qwen3tts-64", T15, frames=3)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode qwen3tts-64 tree 15 F=3")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == 3 * 64
    _check("qwen3tts-64", c, oracle_model("qwen3tts-64"), T15, got, hf, c0, seeds,
           spread_pairs(3, 64, 12, seed=5))
