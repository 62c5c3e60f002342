"""Philox4x32-10 and the per-decision uniforms of a frame.

Philox4x32 is defined in Salmon, Moraes, Dror & Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11), section 4: a 4-word counter is passed
through ten rounds of a multiply/xor S-box keyed by a 2-word key that is
advanced by the Weyl constants between rounds.  The pages only say "a Philox
seed per frame"; the counter layout below is this library's choice.

Uniform of a frame decision:
    U(seed, depth, purpose, i) = (word0 >> 8) * 2**-24, a float32 in [0, 1),
    word0 = Philox4x32-10(counter=(depth, purpose, i, 0),
                          key=(seed & 0xffffffff, seed >> 32))[0]
    i = 0 for the chain window; a tree window numbers the draws and trials
    that share a depth and purpose.
    purpose 0 = draft sample, 1 = acceptance test, 2 = target sample
    (residual, bonus, prefill and every autoregressive draw).

Pinned by tests/test_oracle_philox.py against rocRAND's open-source
philox4x32_10 engine (compiled from its header on the host) and by
uniformity checks.
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
# Multipliers and Weyl key increments of Philox4x32 (SC'11, section 4).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_TARGET = 2


def philox4x32_10(counter, key):
    """Ten Philox4x32 rounds on ``counter`` (4 uint32) under ``key`` (2 uint32)."""
    x0, x1, x2, x3 = (int(v) & MASK32 for v in counter)
    k0, k1 = (int(v) & MASK32 for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        prod0 = PHILOX_M0 * x0
        prod1 = PHILOX_M1 * x2
        hi0, lo0 = prod0 >> 32, prod0 & MASK32
        hi1, lo1 = prod1 >> 32, prod1 & MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def word(seed: int, depth: int, purpose: int, index: int = 0) -> int:
    """First output word of Philox4x32-10 for one decision of a frame."""
    seed = int(seed)
    return philox4x32_10((depth, purpose, index, 0),
                         (seed & MASK32, (seed >> 32) & MASK32))[0]


def uniform(seed: int, depth: int, purpose: int, index: int = 0) -> np.float32:
    """U(seed, depth, purpose, index) as a float32 in [0, 1) with 24 random
    bits."""
    return np.float32((word(seed, depth, purpose, index) >> 8) * (1.0 / (1 << 24)))
