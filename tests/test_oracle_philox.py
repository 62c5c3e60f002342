"""Pins of oracle.philox: rocRAND's open-source Philox4x32-10 engine, built
from its header for the host, must produce the same words for the same key
and counter; the derived uniforms must be uniform."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox

ROCRAND_PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
// argv: seed subsequence offset -> the 4 words at that position
int main(int argc, char** argv) {
  for (int a = 1; a + 2 < argc; a += 3) {
    unsigned long long seed = strtoull(argv[a], 0, 0);
    unsigned long long sub = strtoull(argv[a + 1], 0, 0);
    unsigned long long off = strtoull(argv[a + 2], 0, 0);
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    uint4 r = e.next4();
    printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_probe():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists(
            "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "probe.cpp"), os.path.join(d, "probe")
    with open(src, "w") as f:
        f.write(ROCRAND_PROBE)
    subprocess.run([hipcc, "-O1", "-o", exe, src], check=True,
                   capture_output=True)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def _rocrand_words(exe, triples):
    args = []
    for seed, sub, off in triples:
        args += [str(seed), str(sub), str(off)]
    out = subprocess.run([exe] + args, check=True, capture_output=True,
                         text=True).stdout.split("\n")
    return [tuple(int(v) for v in line.split()) for line in out if line]


def test_philox_matches_rocrand(rocrand_probe):
    rng = np.random.default_rng(5)
    cases = []
    for _ in range(40):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        ctr = [int(v) for v in rng.integers(0, 2**32, size=4)]
        ctr[1] >>= 2            # rocRAND's 64-bit offset reaches 2^30 here
        cases.append((seed, ctr))
    cases.append((0, [0, 0, 0, 0]))
    cases.append((2**64 - 1, [2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1]))
    # rocRAND: key = seed (lo, hi); counter = (offset/4 as 64 bits) +
    # (subsequence as 64 bits in the upper two words)
    triples = []
    for seed, (c0, c1, c2, c3) in cases:
        triples.append((seed, c2 | (c3 << 32), 4 * (c0 | (c1 << 32))))
    got = _rocrand_words(rocrand_probe, triples)
    for (seed, ctr), ref in zip(cases, got):
        key = (seed & 0xFFFFFFFF, seed >> 32)
        assert philox.philox4x32_10(ctr, key) == ref


def test_frame_uniform_layout(rocrand_probe):
    # U(seed, depth, purpose) uses counter (depth, purpose, 0, 0)
    seed = 0x0123456789ABCDEF
    triples = [(seed, 0, 4 * (d | (p << 32))) for d in range(16)
               for p in range(3)]
    got = _rocrand_words(rocrand_probe, triples)
    k = 0
    for d in range(16):
        for p in range(3):
            assert philox.word(seed, d, p) == got[k][0]
            u = philox.uniform(seed, d, p)
            assert u == np.float32((got[k][0] >> 8) / 2**24)
            k += 1


def test_uniforms_are_uniform():
    n = 40000
    u = np.array([philox.uniform(s * 7919 + 13, s % 16, s % 3)
                  for s in range(n)], dtype=np.float64)
    assert u.min() >= 0.0 and u.max() < 1.0
    hist, _ = np.histogram(u, bins=50, range=(0.0, 1.0))
    from scipy.stats import chisquare
    assert chisquare(hist).pvalue > 1e-4
    # 24-bit resolution: every value is a multiple of 2^-24
    assert np.all((u * 2**24) == np.floor(u * 2**24))
