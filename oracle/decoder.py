"""CodePredictor decoder, one position at a time, in float64.

Structure ("RVQ Position Aware Speculative Decoding for On Device TTS",
section 2.1; SGLang-Omni note, MTP paragraph): every RVQ depth has its own
input embedding table and its own lm_head; the decoder sees, within one
frame, position 0 = the talker hidden state h_frame (same width as the
decoder, no projection) and position j >= 1 = E_{j-1}[c_{j-1}].  The output
at position j, after the final RMSNorm, is h_j and head_j(h_j) scores c_j.

The block itself is not spelled out on the pages; the plainest reading (a
Qwen/Llama-style pre-norm block, no biases, no QK-norm) is used:
    n  = RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g
    q, k, v = Wq n, Wk n, Wv n;  q, k rotated by RoPE (rotate-half pairs
              (i, i + d/2), angle = position * theta^(-2i/d))
    query head h reads key/value head h // (n_q / n_kv)  (grouped-query)
    attention softmax(q k^T / sqrt(d)) over positions <= own position
    x += Wo attn;  n = RMSNorm(x);  x += Wdown (SiLU(Wgate n) * (Wup n))
    output = RMSNorm_final(x)

KV cache as a transaction (Lesson 8, section 07): a position may be written
only at the current committed length (append), and truncation marks every
position past the new length as NaN so that any read of stale state poisons
the result instead of passing silently.

A block of verify rows is processed row by row in order; row r sees the KV
of the committed prefix and of rows < r, which is exactly causal attention
over the block.

Pins: tests/test_oracle_decoder.py compares a whole frame's positions with
Hugging Face transformers' LlamaModel (float64) fed the same weights, and
checks RMSNorm/SiLU against torch, RoPE against its complex-number form and
its relative-position invariance, the transactional KV rules, and that a
multi-row block equals single-row steps.
"""
from __future__ import annotations

import math

import numpy as np

import synth


def _f64(a, dtype):
    if dtype == synth.BF16:
        return synth.bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    return x / math.sqrt(float(np.mean(x * x)) + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE of rows ``v`` [heads, d] at position ``pos``."""
    d = v.shape[-1]
    half = d // 2
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = pos * inv_freq
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


class KVCache:
    """Per-frame K/V of every layer, [L][G][n_kv][d], plus its valid length."""

    def __init__(self, layers, positions, kv_heads, head_dim):
        shape = (layers, positions, kv_heads, head_dim)
        self.k = np.full(shape, np.nan)
        self.v = np.full(shape, np.nan)
        self.valid = 0

    def truncate(self, length: int):
        """Keep positions [0, length); poison the rest."""
        if length > self.valid:
            raise ValueError("truncate() cannot extend the committed prefix")
        self.k[:, length:] = np.nan
        self.v[:, length:] = np.nan
        self.valid = length


class Model:
    """Decoder, tables and heads of one configuration (float64 copies)."""

    def __init__(self, c: dict, w: dict):
        self.c = c
        self.G, self.V, self.H = c["groups"], c["vocab"], c["hidden"]
        self.nq, self.nkv, self.d = c["q_heads"], c["kv_heads"], c["head_dim"]
        self.L = c["layers"]
        self.eps = float(np.float32(c["rms_eps"]))
        self.theta = float(np.float32(c["rope_theta"]))
        self.dtype = c["dtype"]
        self._embed = w["embed"]           # converted one row at a time
        self.heads = _f64(w["heads"], self.dtype)
        self.final_norm = np.asarray(w["final_norm"], np.float64)
        # position-aware draft offsets b_1..b_K (float32 vectors), or None
        off = w.get("draft_offsets")
        self.draft_offsets = (None if off is None or len(off) == 0 else
                              np.asarray(off, np.float32).astype(np.float64))
        self.layers = []
        for lw in w["layers"]:
            cv = {}
            for name, a in lw.items():
                if name.endswith("norm"):
                    cv[name] = np.asarray(a, np.float64)
                else:
                    cv[name] = _f64(a, self.dtype)
            self.layers.append(cv)

    # --- inputs and outputs --------------------------------------------
    def embed_row(self, table: int, code: int) -> np.ndarray:
        """E_table[code] as float64."""
        return _f64(self._embed[table, code], self.dtype)

    def logits(self, j: int, h: np.ndarray) -> np.ndarray:
        """head_j(h) rounded to float32 (j = 1 .. G-1)."""
        if not 1 <= j <= self.G - 1:
            raise IndexError(f"no lm_head for depth {j}")
        return (self.heads[j - 1] @ h).astype(np.float32)

    def new_kv(self) -> KVCache:
        return KVCache(self.L, self.G, self.nkv, self.d)

    # --- decoder --------------------------------------------------------
    def forward_row(self, x: np.ndarray, pos: int, kv: KVCache) -> np.ndarray:
        """One position through every layer; appends its K/V at ``pos``."""
        if pos != kv.valid:
            raise ValueError(f"KV append at {pos} but committed length is "
                             f"{kv.valid}")
        x = np.array(x, dtype=np.float64)
        group = self.nq // self.nkv
        scale = 1.0 / math.sqrt(self.d)
        for li, lw in enumerate(self.layers):
            n = rmsnorm(x, lw["attn_norm"], self.eps)
            q = (lw["wq"] @ n).reshape(self.nq, self.d)
            k = (lw["wk"] @ n).reshape(self.nkv, self.d)
            v = (lw["wv"] @ n).reshape(self.nkv, self.d)
            kv.k[li, pos] = rope(k, pos, self.theta)
            kv.v[li, pos] = v
            q = rope(q, pos, self.theta)
            att = np.empty((self.nq, self.d))
            for hq in range(self.nq):
                g = hq // group
                keys = kv.k[li, : pos + 1, g]
                vals = kv.v[li, : pos + 1, g]
                s = keys @ q[hq] * scale
                e = np.exp(s - s.max())
                att[hq] = (e / e.sum()) @ vals
            x = x + lw["wo"] @ att.reshape(-1)
            n = rmsnorm(x, lw["ffn_norm"], self.eps)
            x = x + lw["w_down"] @ (silu(lw["w_gate"] @ n) * (lw["w_up"] @ n))
        kv.valid = pos + 1
        return rmsnorm(x, self.final_norm, self.eps)

    def forward_rows(self, rows, positions, kv: KVCache) -> list:
        """A causal block: rows in order, each at its position."""
        return [self.forward_row(x, p, kv) for x, p in zip(rows, positions)]
