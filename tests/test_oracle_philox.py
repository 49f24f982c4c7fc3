"""Pins for the oracle's Philox4x32-10 and Box-Muller normals."""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import normals, philox

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    if not os.path.exists(HIPCC) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    src = os.path.join(os.path.dirname(__file__), "philox_rocrand_check.cpp")
    exe = str(tmp_path_factory.mktemp("rr") / "philox_rocrand_check")
    subprocess.run([HIPCC, "-O1", "-x", "hip", "--offload-arch=gfx950", src, "-o", exe],
                   check=True, capture_output=True)

    def run(rows):
        inp = "".join(f"{c0} {c1} {c2} {c3} {seed}\n" for c0, c1, c2, c3, seed in rows)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(h, 16) for h in line.split()) for line in out.strip().splitlines()]

    return run


def _cases():
    rng = np.random.default_rng(12345)
    rows = [(0, 0, 0, 0, 0), (0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFFFFFFFFFF),
            (503, 531599, 1000, 0, 2), (0, 1, 1, 0, 1), (7, 0, 50, 0, 0x123456789ABCDEF0)]
    for _ in range(200):
        c = [int(v) for v in rng.integers(0, 2**32, size=4, dtype=np.uint64)]
        rows.append((c[0], c[1], c[2], c[3], int(rng.integers(0, 2**63, dtype=np.uint64)) * 2 + 1))
    return rows


def test_scalar_matches_rocrand(rocrand_philox):
    rows = _cases()
    want = rocrand_philox(rows)
    for (c0, c1, c2, c3, seed), w in zip(rows, want):
        assert philox.block((c0, c1, c2, c3), philox.key_from_seed(seed)) == w


def test_vectorised_matches_scalar():
    rows = _cases()
    for c0, c1, c2, c3, seed in rows[:50]:
        v = philox.blocks(np.uint64(c0), np.uint64(c1), np.uint64(c2), np.uint64(c3), philox.key_from_seed(seed))
        assert tuple(int(x) for x in v) == philox.block((c0, c1, c2, c3), philox.key_from_seed(seed))


def test_map_words_layout():
    # element e of trajectory t takes word e % 4 of block (e // 4, t, slot, 0)
    w = philox.map_words(2, [0, 17], slot=5)
    assert w.shape == (2, 2016) and w.dtype == np.uint32
    for t_i, t in enumerate([0, 17]):
        for e in (0, 1, 2, 3, 4, 1949, 1950, 2015):
            blk = philox.block((e // 4, t, 5, 0), philox.key_from_seed(2))
            assert int(w[t_i, e]) == blk[e % 4]


def test_words_uniform_and_bit_balance():
    w = philox.map_words(0, np.arange(64), slot=1).reshape(-1)
    # chi-square over 256 bins of the top byte
    counts = np.bincount((w >> 24).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4
    bits = np.unpackbits(w.view(np.uint8)).reshape(-1, 32)
    frac = bits.mean(axis=0)
    assert np.all(np.abs(frac - 0.5) < 0.01)


def test_uniforms_exact_and_in_range():
    words = np.array([0, 255, 256, 0xFFFFFFFF, 0x80000000], dtype=np.uint32)
    u1 = normals.uniform_open0(words)
    u2 = normals.uniform_open1(words)
    assert u1.min() > 0 and u1.max() == 1.0
    assert u2.min() == 0.0 and u2.max() < 1.0
    assert np.all(u1.astype(np.float32).astype(np.float64) == u1)
    assert np.all(u2.astype(np.float32).astype(np.float64) == u2)
    assert u1[0] == 2.0 ** -24 and u2[2] == 2.0 ** -24


def test_box_muller_handworked_block():
    # words (r0, r1, r2, r3) -> elements (cos from r0,r1; sin from r0,r1; cos from r2,r3; sin from r2,r3)
    # r0 = 0xffffffff -> u1 = 1 -> radius 0; r2 = 0 -> u1 = 2^-24 -> radius sqrt(48 ln 2);
    # r3 = 2^30 -> u2 = 1/4 -> angle pi/2.
    z = normals.words_to_normals(np.array([0xFFFFFFFF, 0x12345678, 0, 1 << 30], dtype=np.uint32))
    rad = math.sqrt(48.0 * math.log(2.0))
    assert z[0] == 0.0 and z[1] == 0.0
    assert abs(z[2]) < 1e-12 and z[3] == pytest.approx(rad, rel=1e-15)
    z = normals.words_to_normals(np.array([0, 0, 0, 0], dtype=np.uint32))
    assert z[0] == pytest.approx(rad, rel=1e-15) and z[1] == 0.0


def test_normals_are_standard_gaussian():
    z = normals.words_to_normals(philox.map_words(1, np.arange(200), slot=3)).reshape(-1)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    assert abs(z.mean()) < 5.0 / math.sqrt(z.size)
    assert abs(z.var() - 1.0) < 0.01
    blk = z.reshape(-1, 4)
    # the two members of a Box-Muller pair are uncorrelated; radius^2 ~ chi^2(2)
    assert abs(np.corrcoef(blk[:, 0], blk[:, 1])[0, 1]) < 0.01
    r2 = blk[:, 0] ** 2 + blk[:, 1] ** 2
    assert stats.kstest(r2, "expon", args=(0, 2)).pvalue > 1e-3
