"""GPU parity at the edges of the method: the fewest code groups (G = 3: every
round is a single target draw; G = 2: the autoregressive fallback), the full
vocabulary as top-k set, top-k 1 (the deterministic chain), very low and very
high temperature, the most code groups (G = 32: attention over positions
16..31, heads up to 31), head dims 16 and 32, vocabularies of 512, 1024 and 4096 codes, and one handle decoding different stream counts in
turn (GEMV and matrix-core paths, a new graph per count).  Same frame rule as the
other decode tests: equal codes, or the oracle re-run with one near-tie
decision taken the other way reproduces the GPU's codes.
"""
import numpy as np
import pytest

import synth
from gpu_util import compare_frames, decode_gpu, dparams, log, oracle_frames

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_SHAPE = dict(layers=1, hidden=256, q_heads=4, kv_heads=2, head_dim=64,
              ffn=512, vocab=256, weight_scale=0.05)


def _setup(max_streams=None, **kw):
    from oracle import decoder
    from speculative_decoding_rvq_amd import binding
    c = synth.custom(**{**_SHAPE, **kw})
    w = synth.make_weights(c)
    h = binding.Handle(c, binding.weights_to_device(w), max_streams=max_streams)
    return c, h, decoder.Model(c, w)


def _check(name, c, m, got, hf, c0, seeds, pairs, dp=None):
    gc, gf, gst = got
    oc, of, ost, rerun = oracle_frames(None, dp or dparams(c), hf, c0, seeds, pairs, model=m)
    res = compare_frames(np.array([gc[f, b] for f, b in pairs]),
                         np.array([gf[f, b] for f, b in pairs]), oc, of,
                         rerun=rerun, tag="edge cases")
    log(f"{name}: {res['frames']} frames, {res['exact']} exact, "
        f"{res['flip_explained']} explained by a near-tie flip, "
        f"{len(res['unflagged'])} unexplained")
    assert not res["unflagged"], res["unflagged"][:3]
    return res, ost


def test_three_groups_single_draw_rounds():
    c, h, m = _setup(groups=3, verify_size=4, top_k=50, frames=30)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode G=3 F=30")
    got = decode_gpu(h, hf, c0, seeds)
    res, ost = _check("G3", c, m, got, hf, c0, seeds, [(f, 0) for f in range(30)])
    st = got[2]
    assert st["frames"] == 30 and st["codes"] == 60
    assert st["rounds"] == 30 and sum(st["proposed"]) == 0  # gamma is 0 at s = 1


def test_two_groups_autoregressive_fallback():
    c, h, m = _setup(groups=2, verify_size=4, top_k=50, frames=20)
    assert h.status == 1  # CP_SPEC_WARN_AR_FALLBACK: created, runs the AR loop
    hf, c0, seeds = synth.make_inputs(c)
    log("decode G=2 (fallback) F=20")
    got = decode_gpu(h, hf, c0, seeds)
    _check("G2", c, m, got, hf, c0, seeds, [(f, 0) for f in range(20)])
    assert got[2]["rounds"] == 0 and got[2]["prefill_passes"] == 20


def test_full_vocabulary_top_k():
    c, h, m = _setup(groups=8, verify_size=4, top_k=256, temperature=0.9, frames=40)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode top-k = V F=40")
    got = decode_gpu(h, hf, c0, seeds)
    _check("topk=V", c, m, got, hf, c0, seeds, [(f, 0) for f in range(40)])


def test_top1_sampling_equals_greedy_on_gpu():
    c, h, m = _setup(groups=8, verify_size=4, top_k=1, frames=30)
    cg, hg, _ = _setup(groups=8, verify_size=4, greedy=True, top_k=1, frames=30)
    hf, c0, seeds = synth.make_inputs(c)
    log("decode top-k 1 vs greedy F=30")
    a = decode_gpu(h, hf, c0, seeds)
    b = decode_gpu(hg, hf, c0, seeds)
    assert not compare_frames(a[0], a[1], b[0], b[1])["unflagged"]
    _check("topk=1", c, m, a, hf, c0, seeds, [(f, 0) for f in range(0, 30, 3)])


@pytest.mark.parametrize("T", [0.05, 5.0])
def test_temperature_extremes(T):
    c, h, m = _setup(groups=8, verify_size=4, top_k=50, temperature=T, frames=30)
    hf, c0, seeds = synth.make_inputs(c)
    log(f"decode T={T} F=30")
    got = decode_gpu(h, hf, c0, seeds)
    _check(f"T={T}", c, m, got, hf, c0, seeds, [(f, 0) for f in range(30)])


@pytest.mark.parametrize("B,fused,dtype", [(1, 0, synth.F32), (1, 1, synth.F32), (12, 1, synth.F32),
                                           (1, 1, synth.BF16), (12, 0, synth.BF16)])
def test_thirty_two_groups(B, fused, dtype):
    """G = 32, the most the library takes: a frame's positions reach 31, so
    the attention's scores take their second 16-position half, and the heads
    run up to 31; one stream (GEMV path, the folded accept step with fused
    drafts) and 12 streams (48 rows: matrix-core path), fp32 and bf16
    weights."""
    kw = dict(hidden=512, q_heads=8, ffn=1024) if dtype == synth.BF16 else {}
    c, h, m = _setup(max_streams=B, groups=32, verify_size=4, top_k=50, frames=6 if B == 1 else 2,
                     streams=B, fused_draft=fused, dtype=dtype, **kw)
    hf, c0, seeds = synth.make_inputs(c)
    F = c["frames"]
    log(f"decode G=32 B={B} fused={fused} {'bf16' if dtype == synth.BF16 else 'fp32'} F={F}")
    got = decode_gpu(h, hf, c0, seeds)
    assert got[2]["frames"] == F * B and got[2]["codes"] == F * B * 31
    _check(f"G32 B={B} fused={fused}", c, m, got, hf, c0, seeds, [(f, b) for f in range(F) for b in range(B)])


@pytest.mark.parametrize("d,B", [(16, 1), (32, 1), (16, 12), (32, 12)])
def test_small_head_dims(d, B):
    """Head dims 16 and 32 (16 and 8 query heads over a 256-wide model, two
    per KV head): the attention kernel's other instantiations, one stream
    and 12 streams."""
    c, h, m = _setup(max_streams=B, groups=8, verify_size=4, top_k=50, frames=8 if B == 1 else 2, streams=B,
                     head_dim=d, q_heads=256 // d, kv_heads=128 // d)
    hf, c0, seeds = synth.make_inputs(c)
    F = c["frames"]
    log(f"decode d={d} B={B} F={F}")
    got = decode_gpu(h, hf, c0, seeds)
    _check(f"d={d} B={B}", c, m, got, hf, c0, seeds, [(f, b) for f in range(F) for b in range(B)])


@pytest.mark.parametrize("V,B,greedy", [(512, 1, False), (1024, 1, False), (1024, 12, False), (512, 1, True),
                                        (4096, 1, False), (4096, 1, True)])
def test_vocabulary_sizes(V, B, greedy):
    """Vocabularies of 512, 1024 and 4096 codes (two, four and sixteen codes
    per thread in the top-k and sampling kernels), sampled and greedy."""
    c, h, m = _setup(max_streams=B, groups=8, verify_size=4, top_k=1 if greedy else 50, greedy=greedy,
                     vocab=V, frames=8 if B == 1 else 2, streams=B)
    hf, c0, seeds = synth.make_inputs(c)
    F = c["frames"]
    log(f"decode V={V} B={B} greedy={greedy} F={F}")
    got = decode_gpu(h, hf, c0, seeds)
    _check(f"V={V} B={B}", c, m, got, hf, c0, seeds, [(f, b) for f in range(F) for b in range(B)])


def test_one_handle_different_stream_counts():
    """B = 3 (GEMV path), 8 (matrix-core path) and 1 on one handle."""
    c, h, m = _setup(max_streams=8, groups=8, verify_size=4, top_k=50, frames=3, streams=8)
    hf, c0, seeds = synth.make_inputs(c)
    for B in (3, 8, 1):
        log(f"decode B={B} of max 8, F=3")
        got = decode_gpu(h, hf[:, :B], c0[:, :B], seeds[:, :B])
        assert got[2]["frames"] == 3 * B
        pairs = [(f, b) for f in range(3) for b in range(B)]
        _check(f"B={B}", c, m, got, hf[:, :B], c0[:, :B], seeds[:, :B], pairs)


def test_activation_outside_fp16_range_is_reported():
    """The matrix-core projections (bf16 weights, 32 or more rows) carry
    activations as two fp16 pieces.  A layer-0 norm gain of 1e5 pushes the
    normed inputs past fp16's range: the call must fail with EUNSUPPORTED,
    and the same handle must decode normally, code for code, once the gain
    is back to 1 (the flag starts clear in every call)."""
    from speculative_decoding_rvq_amd import binding
    c = synth.custom(**{**_SHAPE, "hidden": 512, "q_heads": 8, "ffn": 1024},
                     dtype=synth.BF16, groups=8, verify_size=4, top_k=50, frames=2,
                     streams=16)
    assert binding.workspace_bytes(binding.make_cfg(c, 16)) > 0  # a valid bf16 shape
    w = synth.make_weights(c)
    wd = binding.weights_to_device(w)
    h = binding.Handle(c, wd, max_streams=16)
    hf, c0, seeds = synth.make_inputs(c)
    log("bf16 B=16 N=4: reference call")
    ref = decode_gpu(h, hf, c0, seeds)
    gain = wd["layers"][0]["attn_norm"]
    gain.fill_(1e5)
    torch.cuda.synchronize()
    log("bf16 B=16 N=4: layer-0 gain 1e5")
    with pytest.raises(binding.CpSpecError) as err:
        decode_gpu(h, hf, c0, seeds)
    assert err.value.rc == binding.EUNSUPPORTED and "65504" in str(err.value)
    gain.fill_(1.0)
    torch.cuda.synchronize()
    log("bf16 B=16 N=4: gain back to 1")
    again = decode_gpu(h, hf, c0, seeds)
    assert np.array_equal(again[0], ref[0]) and np.array_equal(again[1], ref[1])
