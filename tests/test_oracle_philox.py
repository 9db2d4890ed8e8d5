"""Pins of the oracle's Philox4x32-10 and of the stochastic-rounding bit map.

* Word for word against rocRAND's Philox4x32-10 engine (its header source,
  compiled here for the host as ``tests/philox_rocrand_pin.cpp``), over many
  keys and counters, including carries in every counter word.
* The element -> (group, word, half) map, checked element by element on a
  tiny case with explicit Philox calls.
* A chi-squared uniformity check of the 16-bit values (sanity only).
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as o
from oracle.philox import STREAM_COL, STREAM_ROW

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_pin(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc or rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("philox") / "pin")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "philox_rocrand_pin.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(rows):
        text = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w) for w in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64)

    return run


def test_philox_matches_rocrand(rocrand_pin):
    rng = np.random.default_rng(2024)
    rows = [[0, 0, 0, 0, 0, 0], [0xFFFFFFFF] * 6, [7, 0, 5, 0, 0, 1], [7, 0, 0, 0, 0, 2]]
    rows += [[0x12345678, 0x9ABCDEF0, 0xFFFFFFFF, 0, 3, 0], [1, 2, 0xFFFFFFFF, 0xFFFFFFFF, 9, 1]]
    rows += rng.integers(0, 2 ** 32, size=(400, 6), dtype=np.uint64).tolist()
    want = rocrand_pin(rows)
    for r, w in zip(rows, want):
        got = o.philox4x32_10((r[0], r[1]), np.array(r[2:], dtype=np.uint64))
        assert got.astype(np.uint64).tolist() == w.tolist(), r


def test_philox_vectorised_equals_single_calls():
    key = (0xDEADBEEF, 0x01234567)
    ctr = np.random.default_rng(3).integers(0, 2 ** 32, size=(64, 4), dtype=np.uint64)
    batch = o.philox4x32_10(key, ctr)
    for i in range(64):
        assert np.array_equal(batch[i], o.philox4x32_10(key, ctr[i]))


@pytest.mark.parametrize("stream", [STREAM_ROW, STREAM_COL])
def test_sr_bit_map_element_by_element(stream):
    seed, offset = (5 << 32) | 11, 3
    e = np.arange(40, dtype=np.int64)
    got = o.sr_random_u16(seed, offset, stream, e)
    for i in range(40):
        g = i >> 3
        words = o.philox4x32_10((11, 5), np.array([g, 0, offset, stream], dtype=np.uint64))
        w = int(words[(i & 7) >> 1])
        want = (w >> 16) if (i & 1) else (w & 0xFFFF)
        assert int(got[i]) == want


def test_sr_bits_high_group_index_uses_both_counter_words():
    e = np.array([(1 << 35) + 5], dtype=np.int64)
    got = int(o.sr_random_u16(7, 0, 0, e)[0])
    g = int(e[0]) >> 3
    w = o.philox4x32_10((7, 0), np.array([g & 0xFFFFFFFF, g >> 32, 0, 0], dtype=np.uint64))
    assert got == int(w[2]) >> 16


def test_sr_u16_uniformity_chi2():
    u = o.sr_random_u16(7, 0, 0, np.arange(1 << 18, dtype=np.int64)).astype(np.int64)
    counts = np.bincount(u >> 8, minlength=256)
    exp = len(u) / 256
    chi2 = float(np.sum((counts - exp) ** 2 / exp))
    assert 160 < chi2 < 360  # 255 degrees of freedom, far tails excluded
