"""A scripted conditional-table CodePredictor for testing the round logic
apart from the decoder (Lesson 8, section 03: unit-test the acceptance math on
tiny scripted distributions before entangling it with model state).

It exposes the interface oracle.spec uses (G, V, new_kv, forward_rows,
embed_row, logits).  The "hidden state" at position j is the tuple of codes
c_0..c_{j-1} fed so far; head_j applied to the state at depth j gives the
target logits of c_j, applied to an earlier state (a draft) it gives logits
from a separate table keyed by (state, j).  ``edits`` overwrites single
logits of a table (by its key) to script ties.
"""
import zlib

import numpy as np


class _KV:
    def __init__(self):
        self.inputs = []

    @property
    def valid(self):
        return len(self.inputs)

    def truncate(self, length):
        if length > len(self.inputs):
            raise ValueError("cannot extend")
        del self.inputs[length:]


class TableModel:
    def __init__(self, G, V, seed=0, scale=1.5, draft_shift=0.0,
                 target_support=None, draft_support=None, edits=None):
        self.G, self.V = G, V
        self.edits = edits or {}  # table key -> {code: logit}
        self.seed = seed
        self.scale = scale
        self.draft_shift = draft_shift
        self.target_support = target_support
        self.draft_support = draft_support
        self.calls = {"forward_rows": 0, "rows": 0}
        self._cache = {}

    def _logits(self, key, support):
        if key in self._cache:
            return self._cache[key]
        h = zlib.crc32(repr((self.seed, key)).encode())
        z = np.random.default_rng(h).standard_normal(self.V) * self.scale
        if support is not None:
            mask = np.full(self.V, -30.0)
            mask[list(support)] = 0.0
            z = z + mask
        z = z.astype(np.float32)
        for code, value in self.edits.get(key, {}).items():
            z[code] = np.float32(value)
        self._cache[key] = z
        return self._cache[key]

    def new_kv(self):
        return _KV()

    def embed_row(self, table, code):
        return ("code", int(table), int(code))

    def forward_rows(self, rows, positions, kv):
        self.calls["forward_rows"] += 1
        outs = []
        for x, pos in zip(rows, positions):
            if pos != kv.valid:
                raise ValueError("append out of order")
            if pos > 0:
                assert x[0] == "code" and x[1] == pos - 1, (x, pos)
            kv.inputs.append(x)
            self.calls["rows"] += 1
            prefix = tuple(r[2] for r in kv.inputs[1:])
            outs.append(("h", prefix))
        return outs

    def logits(self, j, h):
        prefix = h[1]
        if len(prefix) == j:
            return self._logits(("p", prefix), self.target_support)
        assert len(prefix) < j
        z = self._logits(("q", prefix, j), self.draft_support)
        return (z + np.float32(self.draft_shift)).astype(np.float32)
