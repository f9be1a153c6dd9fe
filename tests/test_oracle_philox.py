"""Pins for oracle.philox.

Philox4x32-10 is cross-checked against two independently written installed
implementations that are compiled here from their public headers and run as
black boxes: ATen's ``at::philox_engine`` (PyTorch) and rocRAND's
``rocrand_state_philox4x32_10``.  Their (seed, subsequence, offset)
arguments map to key = (seed lo, seed hi) and counter = (offset lo, offset hi,
subsequence lo, subsequence hi) (rocRAND counts the offset in 32-bit words).
The mappings are pinned by their exact ranges and by distribution tests.
"""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

from oracle import philox

CASES = [(0, 0, 0), (1, 0, 0), (0, 1, 0), (0, 0, 1), (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFE),
         (0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0 & 0xFFFFFFFFFFFF),
         (12345, 67, 89), (2 ** 32 + 7, 2 ** 40 + 3, 2 ** 33 + 11)]

TORCH_PROBE = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  for (int a = 1; a + 2 < argc; a += 3) {
    unsigned long long s = strtoull(argv[a], 0, 0), q = strtoull(argv[a+1], 0, 0), o = strtoull(argv[a+2], 0, 0);
    at::Philox4_32 e(s, q, o);
    for (int i = 0; i < 8; ++i) printf("%u ", e());
    printf("\n");
  }
}
"""

ROCRAND_PROBE = r"""
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  for (int a = 1; a + 2 < argc; a += 3) {
    unsigned long long s = strtoull(argv[a], 0, 0), q = strtoull(argv[a+1], 0, 0), o = strtoull(argv[a+2], 0, 0);
    rocrand_state_philox4x32_10 st;
    rocrand_init(s, q, o * 4ull, &st);
    for (int i = 0; i < 2; ++i) { uint4 r = rocrand4(&st); printf("%u %u %u %u ", r.x, r.y, r.z, r.w); }
    printf("\n");
  }
}
"""


def _expected(cases):
    rows = []
    for s, q, o in cases:
        key = philox.seed_key(np.uint64(s))
        ctr = np.array([[(o + i) & 0xFFFFFFFF, ((o + i) >> 32) & 0xFFFFFFFF, q & 0xFFFFFFFF, (q >> 32) & 0xFFFFFFFF]
                        for i in range(2)], dtype=np.uint32)
        rows.append(philox.philox4x32_10(ctr, key).reshape(-1).tolist())
    return rows


def _run_probe(src, compiler_cmd, cases):
    with tempfile.TemporaryDirectory() as d:
        cpp = os.path.join(d, "p.cpp")
        exe = os.path.join(d, "p")
        with open(cpp, "w") as f:
            f.write(src)
        subprocess.run(compiler_cmd(cpp, exe), check=True, capture_output=True)
        args = [str(x) for c in cases for x in c]
        out = subprocess.run([exe] + args, check=True, capture_output=True, text=True).stdout
    return [[int(t) for t in line.split()] for line in out.strip().splitlines()]


def test_philox_matches_aten_engine():
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    got = _run_probe(TORCH_PROBE, lambda c, e: ["g++", "-O1", "-std=c++17", "-I" + inc, c, "-o", e], CASES)
    assert got == _expected(CASES)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not on PATH")
def test_philox_matches_rocrand():
    got = _run_probe(ROCRAND_PROBE, lambda c, e: ["hipcc", "-O1", "-std=c++17", "-x", "hip",
                                                   "--offload-arch=gfx950", c, "-o", e], CASES)
    assert got == _expected(CASES)


def test_uniform_mapping_range_and_exactness():
    w = np.array([0, 1, 511, 512, 0xFFFFFFFF, 0x80000000], dtype=np.uint32)
    u = philox.uniform_from_word(w)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24 and u[2] == 2.0 ** -24
    assert u[3] == 3 * 2.0 ** -24
    assert u[4] == 1.0 - 2.0 ** -24
    assert u[5] == 0.5 + 2.0 ** -24
    assert np.all(u.astype(np.float32).astype(np.float64) == u)      # exact in fp32
    assert np.all((u > 0) & (u < 1))


def test_gumbel_moments():
    ctr = np.zeros((200000, 4), np.uint32)
    ctr[:, 0] = np.arange(200000)
    ctr[:, 3] = 7
    words = philox.philox4x32_10(ctr, philox.seed_key(np.uint64(99))).reshape(-1)
    g = philox.gumbel_from_word(words)
    assert abs(g.mean() - 0.5772156649) < 0.01
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    # extreme values of the mapping
    assert philox.gumbel_from_word(np.uint32(0xFFFFFFFF)) == pytest.approx(-math.log(-math.log(1 - 2.0 ** -24)))
    assert philox.gumbel_from_word(np.uint32(0)) == pytest.approx(-math.log(24 * math.log(2)))


@pytest.mark.parametrize("V", [1024, 1000, 151936])
def test_token_mapping_uniform(V):
    pos = np.arange(200000)
    t = philox.random_tokens(5, 3, pos, V, philox.RENOISE)
    assert t.min() >= 0 and t.max() < V
    bins = np.bincount(t * 16 // V, minlength=16)
    assert stats.chisquare(bins).pvalue > 1e-4
    assert philox.token_from_word(np.uint32(0xFFFFFFFF), V) == V - 1
    assert philox.token_from_word(np.uint32(0), V) == 0


def test_streams_and_steps_differ():
    a = philox.random_tokens(1, 0, np.arange(256), 262144, philox.RENOISE)
    b = philox.random_tokens(1, 0, np.arange(256), 262144, philox.INIT)
    c = philox.random_tokens(1, 1, np.arange(256), 262144, philox.RENOISE)
    d = philox.random_tokens(1 | (1 << 32), 0, np.arange(256), 262144, philox.RENOISE)
    assert (a != b).mean() > 0.99 and (a != c).mean() > 0.99 and (a != d).mean() > 0.99
