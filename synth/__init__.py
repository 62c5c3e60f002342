"""Seeded synthetic inputs for the CodePredictor speculative-decoding workloads.

This module is shared by the CPU oracle, the tests and the benchmark.  It only
draws numbers: model shapes, weights, per-frame inputs and per-frame Philox
seeds.  It holds none of the decoding method's arithmetic (no forward pass, no
softmax, no sampling, no acceptance rule).

Workloads (the real Qwen3-TTS CodePredictor is 5 layers, hidden 1024, 16
code groups of vocabulary 2048, per "RVQ Position Aware Speculative Decoding
for On Device TTS", section 2 and Figure 1):

  tiny         fp32: 2 layers, H 256, 4/4 heads of 64, FFN 768, G 8, V 256,
               1 stream x 100 frames, N 3
  qwen3tts     Qwen3-TTS-0.6B-shaped, bf16: 5 layers, H 1024, 16/8 heads of
               128, FFN 3072, G 16, V 2048, 1 stream x 1000 frames, N 4
  tiny-greedy  the tiny decoder, greedy, verify window swept 2..8
  tiny-64      the tiny decoder, 64 streams x 500 frames, top-k 50, N 4
  wide-256     wide Omni-talker-like, bf16: 8 layers, H 2048, 16/4 heads of
               128, FFN 6144, G 16, V 4096, heads correlated across depths,
               256 streams x 200 frames, N 4
  qwen3tts-64  the qwen3tts shape with 64 streams x 100 frames (batched rows
               large enough that the decoder's weights, not launches, set
               the pace)

Value recipe:
  * every weight matrix (projections, embedding tables, lm_heads) is drawn
    N(0, 0.02) in float32 from numpy's PCG64 seeded with ``1000 + n``, n the
    workload's number in WORKLOADS (1-based);
    bf16 configurations round each value to bfloat16 with round-to-nearest-
    even and hand the bit patterns over as uint16;
  * RMSNorm gains are 1 (float32);
  * wide-256's heads are W_j = B + 0.3 * N_j with B, N_j iid N(0, 0.02);
  * h_frame ~ N(0, 1) float32 and c0 ~ U{0..V-1}, from PCG64 seeded with
    ``2000 + n``;
  * the Philox key of frame f, stream b is SplitMix64(seed_base + f*B + b)
    with seed_base = ``3000 + n`` shifted left by 32 bits.
"""
from __future__ import annotations

import copy
import numpy as np

F32 = "f32"
BF16 = "bf16"

# Decoder/codebook shapes and decoding parameters of the workloads.
WORKLOADS = ("tiny", "qwen3tts", "tiny-greedy", "tiny-64", "wide-256", "qwen3tts-64")

_BASE = {
    "tiny": dict(name="tiny-fp32", layers=2, hidden=256, q_heads=4, kv_heads=4,
            head_dim=64, ffn=768, groups=8, vocab=256, dtype=F32,
            rope_theta=1e4, rms_eps=1e-6, greedy=False, temperature=0.9,
            top_k=50, verify_size=3, streams=1, frames=100, heads_corr=None),
    "qwen3tts": dict(name="qwen3-tts-0.6b-codepredictor", layers=5, hidden=1024,
            q_heads=16, kv_heads=8, head_dim=128, ffn=3072, groups=16,
            vocab=2048, dtype=BF16, rope_theta=1e4, rms_eps=1e-6,
            greedy=False, temperature=0.9, top_k=50, verify_size=4,
            streams=1, frames=1000, heads_corr=None),
    "tiny-greedy": dict(name="tiny-fp32-greedy", layers=2, hidden=256, q_heads=4,
            kv_heads=4, head_dim=64, ffn=768, groups=8, vocab=256, dtype=F32,
            rope_theta=1e4, rms_eps=1e-6, greedy=True, temperature=1.0,
            top_k=1, verify_size=4, verify_sweep=(2, 3, 4, 5, 6, 7, 8),
            streams=1, frames=1000, heads_corr=None),
    "tiny-64": dict(name="tiny-fp32-64streams", layers=2, hidden=256, q_heads=4,
            kv_heads=4, head_dim=64, ffn=768, groups=8, vocab=256, dtype=F32,
            rope_theta=1e4, rms_eps=1e-6, greedy=False, temperature=0.9,
            top_k=50, verify_size=4, streams=64, frames=500, heads_corr=None),
    "wide-256": dict(name="omni-talker-wide-codepredictor", layers=8, hidden=2048,
            q_heads=16, kv_heads=4, head_dim=128, ffn=6144, groups=16,
            vocab=4096, dtype=BF16, rope_theta=1e4, rms_eps=1e-6,
            greedy=False, temperature=0.8, top_k=100, verify_size=4,
            streams=256, frames=200, heads_corr=0.3),
    "qwen3tts-64": dict(name="qwen3-tts-0.6b-codepredictor-64streams", layers=5,
            hidden=1024, q_heads=16, kv_heads=8, head_dim=128, ffn=3072,
            groups=16, vocab=2048, dtype=BF16, rope_theta=1e4, rms_eps=1e-6,
            greedy=False, temperature=0.9, top_k=50, verify_size=4,
            streams=64, frames=100, heads_corr=None),
}


def config(wl: str, **overrides) -> dict:
    """Return a copy of workload ``wl`` (a name in WORKLOADS) with
    ``overrides`` applied.

    Keys: layers, hidden, q_heads, kv_heads, head_dim, ffn, groups (G),
    vocab (V), dtype ('f32'|'bf16'), rope_theta, rms_eps, greedy,
    temperature, top_k, verify_size (N; 0 = autoregressive), streams (B),
    frames (F), heads_corr (None or the noise scale of correlated heads),
    draft_offsets (K position-aware draft offset vectors, default 0),
    offset_scale (their standard deviation, default 0.1),
    plus 'id', 'weight_seed', 'input_seed', 'philox_base', 'offset_seed'.
    """
    n = WORKLOADS.index(wl) + 1
    c = copy.deepcopy(_BASE[wl])
    c["id"] = wl
    c["weight_seed"] = 1000 + n
    c["input_seed"] = 2000 + n
    c["philox_base"] = (3000 + n) << 32
    c["offset_seed"] = 4000 + n
    c.update(overrides)
    return c


def custom(**kw) -> dict:
    """A free-form configuration (used for tiny test models)."""
    c = dict(name="custom", layers=1, hidden=16, q_heads=2, kv_heads=1,
             head_dim=8, ffn=24, groups=4, vocab=8, dtype=F32,
             rope_theta=1e4, rms_eps=1e-6, greedy=False, temperature=0.9,
             top_k=4, verify_size=3, streams=1, frames=4, heads_corr=None,
             id=0, weight_seed=7, input_seed=8, philox_base=9 << 32,
             offset_seed=10, weight_scale=0.02)
    c.update(kw)
    return c


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Input values are finite normal draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng, shape, scale, dtype):
    w = rng.standard_normal(shape, dtype=np.float32)
    w *= np.float32(scale)
    return bf16_bits(w) if dtype == BF16 else w


def layer_shapes(c: dict) -> list[tuple[str, tuple[int, ...]]]:
    """Per-layer tensors in the order they are drawn and passed to the ABI.

    Matrices are row-major [out][in]; norm gains are vectors of H.
    """
    H, d, F = c["hidden"], c["head_dim"], c["ffn"]
    return [
        ("attn_norm", (H,)),
        ("wq", (c["q_heads"] * d, H)),
        ("wk", (c["kv_heads"] * d, H)),
        ("wv", (c["kv_heads"] * d, H)),
        ("wo", (H, c["q_heads"] * d)),
        ("ffn_norm", (H,)),
        ("w_gate", (F, H)),
        ("w_up", (F, H)),
        ("w_down", (H, F)),
    ]


def make_weights(c: dict) -> dict:
    """Draw the weights of configuration ``c``.

    Returns {'embed': [G][V][H], 'heads': [G-1][V][H] (head j at index j-1),
    'final_norm': [H] f32, 'layers': [ {name: array} ... ]} and, when the
    configuration asks for K > 0 draft offsets, 'draft_offsets': [K][H] f32
    from a generator of their own (so the other weights do not change).
    Matrices are float32 for 'f32' configurations and uint16 bf16 bit
    patterns for 'bf16'.
    """
    rng = np.random.Generator(np.random.PCG64(c["weight_seed"]))
    G, V, H, dt = c["groups"], c["vocab"], c["hidden"], c["dtype"]
    s = c.get("weight_scale", 0.02)
    w = {"embed": _draw(rng, (G, V, H), s, dt)}
    if c.get("heads_corr"):
        base = rng.standard_normal((V, H), dtype=np.float32) * np.float32(s)
        heads = []
        for _ in range(G - 1):
            n = rng.standard_normal((V, H), dtype=np.float32) * np.float32(s)
            hj = base + np.float32(c["heads_corr"]) * n
            heads.append(bf16_bits(hj) if dt == BF16 else hj)
            del n
        w["heads"] = np.stack(heads)
        del heads, base
    else:
        w["heads"] = _draw(rng, (G - 1, V, H), s, dt)
    w["final_norm"] = np.ones(H, np.float32)
    layers = []
    for _ in range(c["layers"]):
        lw = {}
        for name, shape in layer_shapes(c):
            if name.endswith("norm"):
                lw[name] = np.ones(shape, np.float32)
            else:
                lw[name] = _draw(rng, shape, s, dt)
        layers.append(lw)
    w["layers"] = layers
    off = make_offsets(c)
    if off is not None:
        w["draft_offsets"] = off
    return w


def make_offsets(c: dict):
    """The K position-aware draft offsets of ``c`` ([K][H] f32), or None:
    N(0, offset_scale^2) from a generator of their own."""
    K = int(c.get("draft_offsets", 0))
    if K <= 0:
        return None
    ro = np.random.Generator(np.random.PCG64(c["offset_seed"]))
    return (ro.standard_normal((K, c["hidden"]), dtype=np.float32) *
            np.float32(c.get("offset_scale", 0.1)))


def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output for state values ``x`` (uint64 array)."""
    with np.errstate(over="ignore"):
        z = (x.astype(np.uint64) + np.uint64(0x9E3779B97F4A7C15))
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def make_inputs(c: dict, frames: int | None = None, streams: int | None = None):
    """Per-frame inputs: h_frame [F][B][H] f32, c0 [F][B] i32, seeds [F][B] u64."""
    F = c["frames"] if frames is None else frames
    B = c["streams"] if streams is None else streams
    rng = np.random.Generator(np.random.PCG64(c["input_seed"]))
    h = rng.standard_normal((F, B, c["hidden"]), dtype=np.float32)
    c0 = rng.integers(0, c["vocab"], size=(F, B), dtype=np.int32)
    idx = np.arange(F * B, dtype=np.uint64).reshape(F, B)
    seeds = splitmix64(np.uint64(c["philox_base"]) + idx)
    return h, c0, seeds


def decoder_params(c: dict) -> int:
    """Number of decoder parameters (all layers, excluding tables and heads)."""
    n = 0
    for name, shape in layer_shapes(c):
        if not name.endswith("norm"):
            n += int(np.prod(shape))
    return n * c["layers"]
