"""Pins for the oracle's Philox4x32-10 and its transforms.

The generator's parity with the published definition is pinned against ROCm's
independent open-source rocRAND implementation (compiled for the host from its
header and run here), and the Weyl constants against their closed forms.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def test_weyl_constants_closed_form():
    # floor(2^32 * (phi - 1)) with phi - 1 = (sqrt(5) - 1) / 2
    assert philox.W0 == (math.isqrt(5 << 64) - (1 << 32)) // 2
    # floor(2^32 * (sqrt(3) - 1))
    assert philox.W1 == math.isqrt(3 << 64) - (1 << 32)


@pytest.fixture(scope="module")
def rocrand_probe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND cross-check")
    exe = str(tmp_path_factory.mktemp("rr") / "rr_check")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "rocrand_philox_check.cpp"), "-o", exe],
                   check=True, capture_output=True, cwd="/tmp")
    return exe


def test_philox_matches_rocrand(rocrand_probe):
    rng = np.random.default_rng(7)
    cases = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF,) * 6, (1, 2, 3, 4, 5, 6)]
    cases += [tuple(int(v) for v in rng.integers(0, 2 ** 32, 6, dtype=np.uint64))
              for _ in range(2000)]
    inp = "\n".join(" ".join("%x" % v for v in c) for c in cases) + "\n"
    out = subprocess.run([rocrand_probe], input=inp, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    for c, line in zip(cases, out):
        want = tuple(int(t, 16) for t in line.split())
        assert philox.philox4x32_10(c[:4], c[4:]) == want, c


def test_numpy_twin_matches_scalar():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 2 ** 32, (4, 300), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    vec = philox.philox4x32_10_np(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(300):
        assert tuple(int(v[i]) for v in vec) == philox.philox4x32_10(c[:, i], (k0, k1))


def test_word_layout():
    seed = 0x0123456789ABCDEF
    for draw in range(9):
        blk = philox.philox4x32_10((5, 7, draw >> 2, philox.RESIDUAL),
                                   (0x89ABCDEF, 0x01234567))
        assert philox.word(seed, 5, 7, draw, philox.RESIDUAL) == blk[draw & 3]
    w = philox.words_np(seed, 5, 7, np.arange(9), philox.RESIDUAL)
    assert [int(x) for x in w] == [philox.word(seed, 5, 7, d, philox.RESIDUAL) for d in range(9)]


def test_u24_exact_values():
    assert philox.u24(0) == 0.0
    assert philox.u24(0xFF) == 0.0
    assert philox.u24(0x100) == 2.0 ** -24
    assert philox.u24(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert philox.u24(0x80000000) == 0.5
    # every u24 value is a binary32 number
    for w in (0x12345678, 0xDEADBEEF, 0x00000100):
        u = philox.u24(w)
        assert float(np.float32(u)) == u


def test_uniformity_chi_square():
    w = philox.words_np(0, 1, 2, np.arange(200_000), philox.SAMPLE)
    u = philox.u24_np(w)
    counts = np.histogram(u, bins=64, range=(0.0, 1.0))[0]
    assert stats.chisquare(counts).pvalue > 1e-4
    # consecutive draws are uncorrelated
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 0.01


def test_domains_and_requests_are_distinct_streams():
    a = philox.words_np(0, 3, 0, np.arange(64), philox.SAMPLE)
    b = philox.words_np(0, 3, 0, np.arange(64), philox.ACCEPT)
    c = philox.words_np(0, 4, 0, np.arange(64), philox.SAMPLE)
    d = philox.words_np(1, 3, 0, np.arange(64), philox.SAMPLE)
    for other in (b, c, d):
        assert np.count_nonzero(a == other) <= 1


def test_gumbel_closed_forms():
    # tiny x: -log1p(-x) = x + x^2/2 + O(x^3), so g = -ln(x) - x/2 to ~1e-20 relative
    for w in (0, 1, 7):
        x = (w + 0.5) * 2.0 ** -32
        assert philox.gumbel(w) == pytest.approx(-math.log(x) - x / 2, rel=1e-15)
    # largest word: U = 2^-33 (0.5 * 2^-32 away from 0), E = 33 ln 2
    assert philox.gumbel(0xFFFFFFFF) == pytest.approx(-math.log(33 * math.log(2.0)), rel=1e-12)
    # the numpy twin agrees with the scalar version
    ws = np.array([0, 1, 12345, 2 ** 31, 2 ** 32 - 1], dtype=np.uint32)
    assert np.allclose(philox.gumbel_np(ws), [philox.gumbel(int(v)) for v in ws], rtol=1e-15)


def test_gumbel_moments():
    w = philox.words_np(9, 0, 0, np.arange(400_000), philox.GUMBEL)
    g = philox.gumbel_np(w)
    euler_gamma = 0.5772156649015329
    assert abs(g.mean() - euler_gamma) < 0.01
    assert abs(g.var() - math.pi ** 2 / 6) < 0.03
    # CDF exp(-exp(-x)) at a few points
    for x in (-1.0, 0.0, 1.0, 3.0):
        assert abs(np.mean(g <= x) - math.exp(-math.exp(-x))) < 0.005
