"""Pins for the oracle's Philox4x32-10 and its verify uniforms (CPU only).

* Library routine: rocRAND's installed Philox4x32-10 engine (host build of its
  header) must agree bit for bit with the oracle on random keys and counters.
* Scalar and vectorised oracle implementations agree.
* The uniform mapping is exact on the 2^-24 grid and passes a chi-square test.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("rr") / "rocrand_philox_ref")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def _run_ref(exe, rows):
    text = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return [tuple(int(x) for x in line.split()) for line in out.strip().splitlines()]


def test_philox_matches_rocrand_engine(rocrand_ref):
    rng = np.random.default_rng(12345)
    rows = [(0, 0, 0, 0, 0, 0), (2**32 - 1, 2**32 - 1, 2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1)]
    for _ in range(2000):
        k0, k1, c0, c2, c3 = (int(x) for x in rng.integers(0, 2**32, size=5))
        c1 = int(rng.integers(0, 2**30))
        rows.append((k0, k1, c0, c1, c2, c3))
    ref = _run_ref(rocrand_ref, rows)
    assert len(ref) == len(rows)
    for r, want in zip(rows, ref):
        got = philox.philox4x32_10((r[2], r[3], r[4], r[5]), (r[0], r[1]))
        assert got == want, (r, got, want)


def test_vectorised_equals_scalar():
    rng = np.random.default_rng(7)
    n = 500
    c = rng.integers(0, 2**32, size=(4, n), dtype=np.uint64)
    k = rng.integers(0, 2**32, size=(2, n), dtype=np.uint64)
    w = philox.philox4x32_10_np(c[0], c[1], c[2], c[3], k[0], k[1])
    for i in range(n):
        want = philox.philox4x32_10(tuple(int(x) for x in c[:, i]), tuple(int(x) for x in k[:, i]))
        assert tuple(int(x[i]) for x in w) == want


def test_verify_uniforms_vectorised_and_keying():
    seed = 0xDEADBEEF12345678
    sids = np.array([0, 1, 2**31 + 5, 2**40 + 3, -7], dtype=np.int64)
    pos = np.array([0, 17, 4096, 262147, 5])
    ua, us = philox.verify_uniforms_np(seed, sids, pos)
    for i in range(len(sids)):
        a, s = philox.verify_uniforms(seed, int(sids[i]), int(pos[i]))
        assert (a, s) == (ua[i], us[i])
        # the words come from counter (pos, sid_lo, sid_hi, 0) and key (seed_lo, seed_hi)
        sid = int(sids[i]) & (2**64 - 1)
        w = philox.philox4x32_10((int(pos[i]), sid & 0xFFFFFFFF, sid >> 32, 0),
                                 (seed & 0xFFFFFFFF, seed >> 32))
        assert a == (w[0] >> 8) / 2**24 and s == (w[1] >> 8) / 2**24


def test_uniform_grid_and_range():
    ua, us = philox.verify_uniforms_np(1, np.arange(20000), np.arange(20000) * 3 + 1)
    for u in (ua, us):
        assert u.min() >= 0.0 and u.max() <= 1.0 - 2**-24
        m = u * 2**24
        assert np.all(m == np.floor(m))


def test_uniforms_chi_square():
    n = 200_000
    sid = np.repeat(np.arange(400), n // 400)
    pos = np.tile(np.arange(n // 400) + 1000, 400)
    ua, us = philox.verify_uniforms_np(0x5EED0001, sid, pos)
    for u in (ua, us):
        counts = np.bincount((u * 64).astype(np.int64), minlength=64)
        p = stats.chisquare(counts).pvalue
        assert p > 1e-4, p
    # the two words of one block are not correlated
    r = np.corrcoef(ua, us)[0, 1]
    assert abs(r) < 5.0 / np.sqrt(n)


def test_distinct_positions_give_distinct_streams():
    a = philox.verify_uniforms_np(3, np.zeros(1000, np.int64), np.arange(1000))[0]
    b = philox.verify_uniforms_np(3, np.ones(1000, np.int64), np.arange(1000))[0]
    assert len(np.unique(a)) > 990 and np.mean(a == b) < 0.01
