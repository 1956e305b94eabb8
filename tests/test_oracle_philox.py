"""Pins for the oracle's Philox4x32-10 and uniform conversions.

External pin: rocRAND's Philox4x32-10 engine, compiled for the host from its
public header (tests/pins/rocrand_philox.cpp), evaluated at the same seeds and
counters.  The oracle and rocRAND share no code.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.fixture(scope="module")
def rocrand_pin(tmp_path_factory):
    if HIPCC is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("pin") / "rocrand_philox")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-w",
                    os.path.join(HERE, "pins", "rocrand_philox.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def _run_pin(exe, rows):
    text = "".join(f"{s} {a} {b} {c} {d}\n" for s, a, b, c, d in rows)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return np.array([[int(w, 16) for w in line.split()] for line in out.strip().splitlines()],
                    dtype=np.uint64)


def test_philox_matches_rocrand(rocrand_pin):
    g = np.random.default_rng(1234)
    rows = [(0, 0, 0, 0, 0), (0, 1, 0, 0, 0), (0, 0, 1, 0, 0), (0, 0, 0, 1, 0), (0, 0, 0, 0, 1),
            (2**64 - 1, 2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1)]
    for _ in range(200):
        rows.append((int(g.integers(0, 2**63)) * 2 + int(g.integers(0, 2)),
                     int(g.integers(0, 2**32)), int(g.integers(0, 2**30)),
                     int(g.integers(0, 2**32)), int(g.integers(0, 2**32))))
    # the verification step's own counters: (request, position, draw, step)
    for b in (0, 1, 255):
        for j in range(0, 10):
            for draw in (0, 1, 2):
                rows.append((0, b, j, draw, 7))
    ref = _run_pin(rocrand_pin, rows)
    arr = np.array(rows, dtype=object)
    seeds = np.array([int(s) for s in arr[:, 0]], dtype=np.uint64)
    out = philox.philox4x32_10(arr[:, 1].astype(np.uint64), arr[:, 2].astype(np.uint64),
                               arr[:, 3].astype(np.uint64), arr[:, 4].astype(np.uint64),
                               seeds & np.uint64(0xFFFFFFFF), seeds >> np.uint64(32))
    got = np.stack(out, axis=1)
    assert np.array_equal(got, ref)


def test_uniform_conversions_exact():
    w = np.array([0, 255, 256, 2**32 - 1], dtype=np.uint64)
    ua = philox.u_accept(w)
    ur = philox.u_resample(w)
    assert ua[0] == 2.0 ** -24 and ua[1] == 2.0 ** -24 and ua[2] == 2.0 ** -23
    assert ua[3] == 1.0                                    # u = 1 reachable, u = 0 not
    assert ur[0] == 0.0 and ur[3] == 1.0 - 2.0 ** -24      # [0, 1)
    # every value is a multiple of 2^-24 below 2^24 * 2^-24, so exact in fp32
    assert np.all(ua.astype(np.float32).astype(np.float64) == ua)
    assert np.all(ur.astype(np.float32).astype(np.float64) == ur)


def test_word_uniformity():
    # 2^16 draws of word 0 over consecutive requests: the top byte is uniform
    b = np.arange(1 << 16)
    w = philox.word(b, 3, philox.DRAW_ACCEPT, 0, 42)
    counts = np.bincount((w >> np.uint64(24)).astype(np.int64), minlength=256)
    from scipy.stats import chisquare
    assert chisquare(counts).pvalue > 1e-4
