"""GPU parity of each step of the round, through the C ABI, against the oracle.

* stacked-head logits: rel 1e-3 / abs 2e-3 (same bf16 weights, fp32 sums);
* top-k softmax: identical support (unless the boundary is a flagged near
  tie), probabilities to float32 rounding; sampling bit-exact against the
  oracle's inverse CDF fed the GPU's own float32 probabilities;
* accept scan: bit-exact codes, counts and flags on fed p, q and uniforms;
* decoder pass: ragged multi-stream blocks, transactional truncation.
"""
import numpy as np
import pytest

import synth
from gpu_util import decode_gpu, device_weights, handle, log, oracle_model, weights
from oracle import decoder as odec
from oracle import distributions as odist

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _t(a, dtype=None):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    return (t if dtype is None else t.to(dtype)).cuda()


@pytest.mark.parametrize("cid,rows", [("tiny", 6), ("qwen3tts", 8),
                                      ("qwen3tts", 24), ("tiny", 31),
                                      ("tiny", 77), ("qwen3tts", 133),
                                      ("wide-256", 70), ("tiny", 4100)])
@pytest.mark.parametrize("norm", [0, 1])
def test_head_logits(cid, rows, norm):
    """Fewer than 32 rows run the GEMV with the rows of a head in one block
    (24 and 31 rows share three heads: several blocks per head); 32 or more
    rows are grouped by head into matrix-core tiles (ragged last tile per
    head): 32 x 32 split-K tiles for few rows per head, 64 x 64 tiles for
    many."""
    log(f"head_logits {cid} rows={rows} norm={norm}")
    c = synth.config(cid)
    m = oracle_model(cid)
    R = max(c["verify_size"], 2)
    h = handle(cid, max_streams=(rows + R - 1) // R)
    rng = np.random.default_rng(10 + len(cid) + rows)
    x = rng.standard_normal((rows, c["hidden"])).astype(np.float32)
    heads = rng.integers(1, c["groups"], size=rows).astype(np.int32)
    if 16 < rows < 32:
        heads = rng.integers(1, 4, size=rows).astype(np.int32)
    heads[1] = 0                                   # a skipped row
    if rows > 64:
        heads[:70 if rows > 70 else 66] = 2        # one head spans two tiles
        heads[1] = 0
    out = torch.full((rows, c["vocab"]), 123.0, device="cuda")
    h.head_logits(_t(x), _t(heads), norm, out)
    got = out.cpu().numpy()
    for r in range(rows):
        if heads[r] == 0:
            assert np.all(got[r] == 123.0)
            continue
        xr = x[r].astype(np.float64)
        if norm:
            xr = odec.rmsnorm(xr, m.final_norm, m.eps)
        ref = m.logits(int(heads[r]), xr)
        np.testing.assert_allclose(got[r], ref, rtol=1e-3, atol=2e-3)
        # the achieved error is far inside the stated tolerance
        assert np.max(np.abs(got[r] - ref)) < 1e-4


def _logit_rows(V, n, rng, ties=False):
    """Rows of N(0, 0.4) logits.  ties=True / "ties": exact ties straddling
    the top-k boundary and the maximum; "mass": a third of the row tied at
    the boundary value; "outlier": one logit far above the rest, so that the
    rest crowd into one value bin; both of the last two exceed the 256
    entries the boundary bin is ranked by directly (for V >= 1024)."""
    z = (rng.standard_normal((n, V)) * 0.4).astype(np.float32)
    if ties is True or ties == "ties":
        for r in range(n):
            order = np.argsort(-z[r])
            z[r, order[45:55]] = z[r, order[49]]
            z[r, order[1]] = z[r, order[0]]
    elif ties == "mass":
        for r in range(n):
            order = np.argsort(-z[r])
            z[r, order[30:30 + V // 3]] = z[r, order[40]]
    elif ties == "outlier":
        z[:, 5] = 3.0e4
        z[1, :] = 1.0                              # one value everywhere
    return z


@pytest.mark.parametrize("cid,over", [
    ("tiny", {}), ("qwen3tts", {}), ("wide-256", {}),
    ("tiny", {"top_k": 256}),             # k = V: full softmax
    ("qwen3tts", {"top_k": 1}),           # k = 1: a point mass
    ("qwen3tts", {"temperature": 1.7, "top_k": 333}),
])
@pytest.mark.parametrize("ties", [False, True, "mass", "outlier"])
def test_topk_sample(cid, over, ties):
    log(f"topk_sample {cid} {over} ties={ties}")
    c = synth.config(cid)
    h = handle(cid, max_streams=1, **over)
    k = h.cfg.top_k
    T = h.cfg.temperature
    V = c["vocab"]
    rng = np.random.default_rng(20 + len(cid) + k)
    n = 24
    z = _logit_rows(V, n, rng, ties)
    u = (rng.integers(0, 2**24, size=n) / 2**24).astype(np.float32)
    u[0], u[1] = 0.0, 1 - 2**-24
    probs = torch.zeros((n, V), device="cuda")
    codes = torch.zeros(n, dtype=torch.int32, device="cuda")
    flags = torch.zeros(n, dtype=torch.int32, device="cuda")
    h.topk_sample(_t(z), _t(u), probs, codes, flags)
    P = probs.cpu().numpy()
    C = codes.cpu().numpy()
    Fl = flags.cpu().numpy().view(np.uint32)
    for r in range(n):
        ref, ftopk = odist.topk_softmax(z[r], T, k)
        assert bool(Fl[r] & 1) == (ftopk and k < V), r
        if not ftopk:
            assert np.array_equal(P[r] > 0, ref > 0), r
        np.testing.assert_allclose(P[r], ref, rtol=3e-6, atol=1e-8)
        # sampling: bit-exact on the same float32 probabilities
        code, fcdf = odist.sample(P[r], u[r])
        assert C[r] == code, (r, C[r], code)
        assert bool(Fl[r] & 4) == fcdf


@pytest.mark.parametrize("cid", ["tiny", "wide-256"])
def test_topk_greedy_argmax(cid):
    log(f"greedy argmax {cid}")
    c = synth.config(cid)
    h = handle(cid, max_streams=1, greedy=1)
    rng = np.random.default_rng(30)
    z = _logit_rows(c["vocab"], 16, rng, ties=True)
    z[3, :] = 0.25                                 # all equal: id 0 wins
    z[4, 7] = z[4].max() + 5e-5                    # near tie
    codes = torch.zeros(16, dtype=torch.int32, device="cuda")
    flags = torch.zeros(16, dtype=torch.int32, device="cuda")
    h.topk_sample(_t(z), None, None, codes, flags)
    C = codes.cpu().numpy()
    Fl = flags.cpu().numpy().view(np.uint32)
    for r in range(16):
        ref, near = odist.argmax_with_gap(z[r])
        assert C[r] == ref and bool(Fl[r] & 2) == near


def _dist_rows(V, n, k, rng, T=0.9):
    out = []
    for _ in range(n):
        z = (rng.standard_normal(V) * 0.8).astype(np.float32)
        out.append(odist.topk_softmax(z, T, k)[0])
    return np.array(out, dtype=np.float32)


@pytest.mark.parametrize("cid", ["tiny", "qwen3tts", "wide-256"])
def test_accept_bit_exact(cid):
    log(f"accept {cid}")
    c = synth.config(cid)
    V, k = c["vocab"], c["top_k"]
    W = 3
    B = 64
    h = handle(cid, max_streams=B)
    rng = np.random.default_rng(40 + len(cid))
    gamma = rng.integers(0, W + 1, size=B).astype(np.int32)
    q = _dist_rows(V, B * W, k, rng).reshape(B, W, V)
    p = _dist_rows(V, B * (W + 1), k, rng).reshape(B, W + 1, V)
    # special streams: p == q (accept all), disjoint supports (reject all),
    # draft outside p's support (p(d) = 0), and an exact ratio tie
    p[0, :W] = q[0]
    gamma[0] = W
    q[1] = 0
    q[1, :, :3] = np.float32(1 / 3)
    p[1, :, :3] = 0
    gamma[1] = W
    draft = np.zeros((B, W), np.int32)
    for b in range(B):
        for t in range(W):
            draft[b, t] = odist.sample(q[b, t], rng.random())[0]
    ua = (rng.integers(0, 2**24, size=(B, W)) / 2**24).astype(np.float32)
    ut = (rng.integers(0, 2**24, size=(B, W + 1)) / 2**24).astype(np.float32)
    d2 = draft[2, 0]
    ua[2, 0] = np.float32(p[2, 0, d2] / q[2, 0, d2]) if p[2, 0, d2] > 0 else 0
    gamma[2] = max(gamma[2], 1)
    # a draft outside p's support (p(d) = 0: always rejected), then the
    # residual draw
    gamma[3] = W
    off = np.flatnonzero(p[3, 0] == 0)[:2]
    q[3, 0] = 0
    q[3, 0, off] = np.float32(0.5)
    draft[3, 0] = off[0]
    # q >= p everywhere on p's support: the residual is all zero and the
    # draw falls back to p
    gamma[4] = 1
    q[4, 0] = p[4, 0]
    draft[4, 0] = int(np.flatnonzero(p[4, 0] > 0)[0])
    ua[4, 0] = np.float32(1.0 - 2**-24)     # ratio 1: u < 1 accepts ...
    p[4, 0, draft[4, 0]] = np.float32(p[4, 0, draft[4, 0]] * 0.5)  # ... unless p(d) < q(d)
    n_out = torch.zeros(B, dtype=torch.int32, device="cuda")
    codes = torch.zeros((B, W + 1), dtype=torch.int32, device="cuda")
    flags = torch.zeros(B, dtype=torch.int32, device="cuda")
    h.accept(_t(gamma), _t(draft), _t(q), _t(p), _t(ua), _t(ut), n_out, codes,
             flags)
    N = n_out.cpu().numpy()
    Cd = codes.cpu().numpy()
    Fl = flags.cpu().numpy().view(np.uint32)
    for b in range(B):
        g = int(gamma[b])
        em, n_acc, near = odist.accept_scan(
            list(draft[b, :g]), list(q[b, :g]), list(p[b, :g + 1]),
            lambda t: ua[b, t - 1], lambda t: ut[b, t - 1])
        assert N[b] == len(em), b
        assert list(Cd[b, :N[b]]) == em, b
        assert np.all(Cd[b, N[b]:] == -1)
        want = 0
        for t, _ in near:
            want |= 1 << (t - 1)
        assert Fl[b] == want, (b, Fl[b], want)
    assert N[0] == W + 1                      # p == q: everything accepted
    assert N[1] == 1                          # disjoint: first draft rejected


def test_accept_greedy():
    log("accept greedy")
    c = synth.config("tiny")
    V, W, B = c["vocab"], 4, 16
    h = handle("tiny-greedy", max_streams=B, verify_size=5)
    rng = np.random.default_rng(50)
    logits = (rng.standard_normal((B, W + 1, V)) * 0.4).astype(np.float32)
    amax = logits.argmax(-1)
    gamma = rng.integers(0, W + 1, size=B).astype(np.int32)
    draft = amax[:, :W].copy().astype(np.int32)
    for b in range(B):                         # a mismatch at a random offset
        t = rng.integers(0, W + 1)
        if t < W:
            draft[b, t] = (draft[b, t] + 1) % V
    n_out = torch.zeros(B, dtype=torch.int32, device="cuda")
    codes = torch.zeros((B, W + 1), dtype=torch.int32, device="cuda")
    h.accept(_t(gamma), _t(draft), None, _t(logits), None, None, n_out, codes)
    N = n_out.cpu().numpy()
    Cd = codes.cpu().numpy()
    for b in range(B):
        g = int(gamma[b])
        rnd = odist.verify_greedy(tuple(draft[b, :g]), tuple(amax[b, :g + 1]))
        assert tuple(Cd[b, :N[b]]) == rnd.emitted


def _schedule(G, R, rng, steps):
    """One stream's verify blocks: the prefill [0, 1], then blocks of 1..R
    consecutive positions, each after truncating 0..2 positions of the block
    before (never the committed prefix 0..1), until the frame is full; then
    empty blocks.  Returns [(positions, valid length before the block)]."""
    out = [([0, 1], 0)]
    valid, last = 2, 2
    for _ in range(steps):
        if valid >= G:
            out.append(([], valid))
            continue
        cut = int(rng.integers(0, min(2, last - 1) + 1)) if last > 1 else 0
        start = max(2, valid - cut)
        n = min(int(rng.integers(1, R + 1)), G - start)
        out.append((list(range(start, start + n)), start))
        valid, last = start + n, n
    return out


@pytest.mark.parametrize("cid,B,check", [("tiny", 3, None), ("qwen3tts", 3, None),
                                         ("tiny", 24, None), ("qwen3tts", 24, None),
                                         ("qwen3tts", 275, None), ("tiny", 400, None),
                                         ("wide-256", 260, (0, 1, 2, 100, 201, 259))])
def test_decoder_ragged_blocks_and_truncation(cid, B, check):
    """Every position of the frame (0..G-1) through ragged verify blocks with
    transactional truncation between them, for B streams (stream b follows
    schedule b % 3).  3 streams run the GEMV path; 24 streams the split-K
    matrix-core tiles (fp32) or the packed bf16 tiles; 275 qwen3tts streams
    (1100 rows: the last 128-row tile ragged) the LDS-staged 128 x 192 tiles
    for gate/up; 400 tiny streams the 64 x 64 tiles; 260 wide streams (1040
    rows) the 64 x 128 residual-add tiles with a ragged last row tile, the
    oracle following the streams in `check` (all when None)."""
    log(f"decoder_forward {cid} B={B}")
    c = synth.config(cid)
    m = oracle_model(cid)
    R = max(c["verify_size"], 2)
    h = handle(cid, max_streams=B)
    L, G, nkv, d, H = c["layers"], c["groups"], c["kv_heads"], c["head_dim"], \
        c["hidden"]
    kv = torch.zeros((B, L, 2, G, nkv, d), device="cuda")
    okv = [m.new_kv() for _ in range(B)]
    checked = set(range(B) if check is None else check)
    rng = np.random.default_rng(60 + len(cid))
    scheds = [_schedule(G, R, rng, G) for _ in range(3)]
    nsteps = max(len(sc) for sc in scheds)
    top = 0
    for k in range(nsteps):
        x = np.zeros((B, R, H), np.float32)
        pos = np.full((B, R), -1, np.int32)
        rows = []
        for b in range(B):
            sc = scheds[b % 3]
            plist, valid = sc[k] if k < len(sc) else ([], G)
            if plist and b in checked:
                okv[b].truncate(valid)
            for r, p_ in enumerate(plist):
                x[b, r] = (rng.standard_normal(H) if p_ == 0 else
                           m.embed_row((p_ - 1) % G, int(rng.integers(0, c["vocab"]))))
                pos[b, r] = p_
                top = max(top, p_)
            rows.append(plist)
        xt = _t(x)
        h.decoder_forward(xt, _t(pos), kv)
        got = xt.cpu().numpy()
        for b, plist in enumerate(rows):
            if not plist or b not in checked:
                continue
            ref = m.forward_rows([x[b, r].astype(np.float64)
                                  for r in range(len(plist))], plist, okv[b])
            for r in range(len(plist)):
                np.testing.assert_allclose(got[b, r], ref[r], rtol=1e-3,
                                           atol=2e-3)
                assert np.max(np.abs(got[b, r] - ref[r])) < 1e-4, (k, b, r)
    assert top == G - 1  # the last position of the frame was covered


@pytest.mark.parametrize("cid", ["tiny", "qwen3tts"])
def test_talker_feedback(cid):
    """Sum of the frame's embedding rows (Talker hand-off) against the oracle,
    on codes the GPU decoded; a row with an out-of-range code is NaN."""
    from oracle import spec as ospec
    log(f"talker feedback {cid}")
    c = synth.config(cid, frames=6)
    hf, c0, seeds = synth.make_inputs(c)
    h = handle(cid)
    gc, _, _ = decode_gpu(h, hf, c0, seeds)
    F, B, G = gc.shape
    codes = np.ascontiguousarray(gc.reshape(F * B, G)).astype(np.int32)
    codes = np.concatenate([codes, codes[:1]])
    codes[-1, G // 2] = c["vocab"]                  # out of range: NaN row
    out = torch.empty((codes.shape[0], c["hidden"]), dtype=torch.float32, device="cuda")
    h.talker_feedback(_t(codes), out)
    got = out.cpu().numpy()
    m = oracle_model(cid)
    for i in range(F * B):
        ref = ospec.talker_feedback(m, codes[i])
        np.testing.assert_allclose(got[i], ref, rtol=2e-6, atol=2e-6 * np.abs(ref).max())
    assert np.all(np.isnan(got[-1]))


def _walk_rows(V, k, n, maxc, rng):
    """Rows for the tree walk step: p, q (top-k softmax rows), children drawn
    from q, uniforms; special rows p == q, disjoint supports, children
    outside p's support, and an exact ratio tie."""
    z = (rng.standard_normal((n, V)) * 0.8).astype(np.float32)
    p = np.array([odist.topk_softmax(z[i] + (rng.standard_normal(V) * 0.3).astype(np.float32),
                                     0.9, k)[0] for i in range(n)], np.float32)
    q = np.array([odist.topk_softmax(z[i] + (rng.standard_normal(V) * 0.3).astype(np.float32),
                                     0.9, k)[0] for i in range(n)], np.float32)
    nch = rng.integers(0, maxc + 1, size=n).astype(np.int32)
    ch = np.zeros((n, maxc), np.int32)
    for i in range(n):
        for j in range(maxc):
            ch[i, j] = odist.sample(q[i], rng.random())[0]
    ua = (rng.integers(0, 2**24, size=(n, maxc)) / 2**24).astype(np.float32)
    ut = (rng.integers(0, 2**24, size=n) / 2**24).astype(np.float32)
    p[0] = q[0]                                  # p == q: the first child passes
    nch[0] = maxc
    p[1] = 0
    p[1, :5] = np.float32(0.2)                   # disjoint supports: all rejected
    q[1] = 0
    q[1, 8:11] = np.float32(1 / 3)
    ch[1] = 8 + np.arange(maxc) % 3
    nch[1] = maxc
    nch[2] = maxc                                # several rejections in a row
    ua[2] = np.float32(1 - 2**-24)
    nch[3] = 1                                   # exact tie u == p/q
    x = ch[3, 0]
    ua[3, 0] = np.float32(p[3, x] / q[3, x]) if p[3, x] > 0 else 0
    return p, q, nch, ch, ua, ut


@pytest.mark.parametrize("cid", ["tiny", "qwen3tts", "wide-256"])
def test_walk_step_bit_exact(cid):
    """cp_spec_walk_step (the tree rows' step in the decode round) against
    oracle.tree.walk_step: the accepted child, the code and the near-tie
    flags, bit for bit, for 0..3 children per row."""
    from oracle import tree as otree
    log(f"walk step {cid}")
    c = synth.config(cid)
    V, k = c["vocab"], c["top_k"]
    h = handle(cid, max_streams=1)
    rng = np.random.default_rng(70 + len(cid))
    n, maxc = 96, 3
    p, q, nch, ch, ua, ut = _walk_rows(V, k, n, maxc, rng)
    acc = torch.zeros(n, dtype=torch.int32, device="cuda")
    codes = torch.zeros(n, dtype=torch.int32, device="cuda")
    flags = torch.zeros(n, dtype=torch.int32, device="cuda")
    h.walk_step(_t(p), _t(q), _t(nch), _t(ch), _t(ua), _t(ut), acc, codes, flags)
    A = acc.cpu().numpy()
    Cd = codes.cpu().numpy()
    Fl = flags.cpu().numpy().view(np.uint32)
    kinds = {"accept": 8, "cdf": 4}
    for i in range(n):
        kk, code, near = otree.walk_step(p[i], q[i], list(ch[i, :nch[i]]),
                                         lambda j: ua[i, j], ut[i])
        assert A[i] == (-1 if kk is None else kk), i
        assert Cd[i] == code, (i, Cd[i], code)
        want = 0
        for kind in near:
            want |= kinds[kind]
        assert Fl[i] == want, (i, Fl[i], want)
    assert A[0] == 0 and A[1] == -1
