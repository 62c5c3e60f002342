"""cp_spec_accept_noalloc (no handle, static per-GPU scratch) against
cp_spec_accept (the handle's workspace as scratch): identical committed
counts, codes and near-tie flags, bit for bit, on two calls in a row with
the second smaller, stochastic and greedy; the size bound is rejected on the
host before anything runs.  Runs last (its array keeps the previous call's
contents, which the second, smaller call must not see)."""
import numpy as np
import pytest

import synth
from gpu_util import handle, log
from oracle import distributions as odist

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _inputs(V, k, B, W, rng, greedy):
    gamma = rng.integers(0, W + 1, size=B).astype(np.int32)
    if greedy:
        p = (rng.standard_normal((B, W + 1, V)) * 0.4).astype(np.float32)
        draft = p[:, :W].argmax(-1).astype(np.int32)
        miss = rng.random((B, W)) < 0.3
        draft[miss] = (draft[miss] + 1) % V
        return gamma, draft, None, p, None, None
    z = (rng.standard_normal((B, W + 1, V)) * 0.8).astype(np.float32)
    p = np.array([[odist.topk_softmax(z[b, r], 0.9, k)[0] for r in range(W + 1)]
                  for b in range(B)], np.float32)
    zq = z[:, :W] + (rng.standard_normal((B, W, V)) * 0.3).astype(np.float32)
    q = np.array([[odist.topk_softmax(zq[b, t], 0.9, k)[0] for t in range(W)]
                  for b in range(B)], np.float32)
    draft = np.array([[odist.sample(q[b, t], rng.random())[0] for t in range(W)]
                      for b in range(B)], np.int32).reshape(B, W)
    ua = (rng.integers(0, 2**24, size=(B, W)) / 2**24).astype(np.float32)
    ut = (rng.integers(0, 2**24, size=(B, W + 1)) / 2**24).astype(np.float32)
    return gamma, draft, q, p, ua, ut


@pytest.mark.parametrize("cid,greedy", [("tiny", False), ("qwen3tts", False),
                                        ("tiny-greedy", True)])
def test_noalloc_accept_matches_accept(cid, greedy):
    from speculative_decoding_rvq_amd import binding
    c = synth.config(cid)
    V, k = c["vocab"], c["top_k"]
    h = handle(cid, max_streams=160, verify_size=8)
    rng = np.random.default_rng(80 + len(cid))
    for B, W in ((160, 7), (23, 3)):  # the second call is smaller
        log(f"accept_noalloc {cid} B={B} W={W}")
        gamma, draft, q, p, ua, ut = _inputs(V, k, B, W, rng, greedy)
        args = [_t(gamma), _t(draft), None if q is None else _t(q), _t(p),
                None if ua is None else _t(ua), None if ut is None else _t(ut)]
        outs = []
        for variant in ("accept", "noalloc"):
            n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
            codes = torch.full((B, W + 1), -7, dtype=torch.int32, device="cuda")
            flags = torch.full((B,), -7, dtype=torch.int32, device="cuda")
            if variant == "accept":
                h.accept(*args, n, codes, flags)
            else:
                binding.accept_noalloc(V, greedy, *args, n, codes, flags)
            torch.cuda.synchronize()
            outs.append((n.cpu().numpy(), codes.cpu().numpy(), flags.cpu().numpy()))
        for a, b in zip(*outs):
            np.testing.assert_array_equal(a, b)
        assert np.all(outs[0][0] >= 1) and np.all(outs[0][0] <= gamma + 1)


def test_noalloc_accept_rejects_oversize_and_bad_vocab():
    from speculative_decoding_rvq_amd import binding
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    zf = torch.zeros(1, dtype=torch.float32, device="cuda")
    dummy = torch.zeros((8193, 7), dtype=torch.int32, device="cuda")
    with pytest.raises(binding.CpSpecError, match="static scratch"):
        binding.accept_noalloc(256, False, z, dummy, zf, zf, zf, zf, z, z)
    with pytest.raises(binding.CpSpecError, match="vocab"):
        binding.accept_noalloc(300, False, z, dummy[:1], zf, zf, zf, zf, z, z)
