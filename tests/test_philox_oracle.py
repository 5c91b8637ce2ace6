"""Pin the oracle's Philox4x32-10 to an independent implementation.

PyTorch ships a header-only C++ Philox4x32-10 engine (ATen/core/PhiloxRNGEngine.h,
written from the same SC'11 paper).  This test compiles a tiny host program
against that header and compares its output words with the oracle's for many
keys and counters.  The engine's (seed, subsequence, offset) map to the key
(seed lo, seed hi) and the counter (offset lo, offset hi, subsequence lo,
subsequence hi); four successive calls return the four output words.
"""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox

SRC = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    at::philox_engine e(seed, sub, off);
    unsigned w[4];
    for (int k = 0; k < 4; ++k) w[k] = e();
    std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
  }
}
"""


@pytest.fixture(scope="module")
def aten_philox():
    torch = pytest.importorskip("torch")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if shutil.which("g++") is None or not os.path.exists(os.path.join(inc, "ATen/core/PhiloxRNGEngine.h")):
        pytest.skip("no g++ or no PyTorch headers")
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "p.cpp"), os.path.join(d, "p")
    with open(src, "w") as f:
        f.write(SRC)
    subprocess.run(["g++", "-O1", "-std=c++17", "-I" + inc, src, "-o", exe], check=True)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_independent_engine(aten_philox):
    rng = np.random.default_rng(0)
    cases = [(0, 0, 0), (2**64 - 1, 2**64 - 1, 2**64 - 1), (1, 2, 3)]
    cases += [tuple(int(x) for x in rng.integers(0, 2**63, 3, dtype=np.uint64)) for _ in range(200)]
    cases += [(int(s), int(b), int(o)) for s, b, o in rng.integers(0, 2**20, (200, 3))]
    inp = "".join(f"{s} {b} {o}\n" for s, b, o in cases)
    out = subprocess.run([aten_philox], input=inp, capture_output=True, text=True, check=True).stdout
    want = np.array([[int(w) for w in line.split()] for line in out.strip().splitlines()], dtype=np.uint64)
    for (seed, sub, off), w in zip(cases, want):
        ctr = (off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32)
        got = philox.philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32))
        assert [int(g) for g in got] == [int(x) for x in w], (seed, sub, off)


def test_keep_mask_uses_half_j_mod_2_of_word_j_mod_8_div_2_of_counter_j_div_8(aten_philox):
    seed, rho, lane = 0x1234_5678_9ABC, 0.1, 37
    rows, cols = np.arange(5, 9), np.arange(0, 21)
    keep = philox.keep_mask(seed, rho, lane, rows, cols)
    thr = philox.drop_threshold(rho)
    inp = "".join(f"{seed} {lane} {(i << 32) + j8}\n" for i in rows for j8 in range(3))
    out = subprocess.run([aten_philox], input=inp, capture_output=True, text=True, check=True).stdout
    words = np.array([[int(w) for w in l.split()] for l in out.strip().splitlines()]).reshape(len(rows), 3, 4)
    for a, i in enumerate(rows):
        for b, j in enumerate(cols):
            u = (words[a, j // 8, (j % 8) // 2] >> (16 * (j % 2))) & 0xFFFF
            assert keep[a, b] == (u >= thr)


def test_keep_rate_is_within_five_sigma():
    rho = 0.1
    keep = philox.keep_mask(0, rho, 3, np.arange(256), np.arange(1024))
    p = 1.0 - philox.drop_threshold(rho) / 2**16
    n = keep.size
    assert abs(keep.mean() - p) < 5 * np.sqrt(p * (1 - p) / n)


def test_both_halves_of_a_word_are_used_independently():
    # a plausible slip (one half read twice) would make keys 2w and 2w+1 agree
    keep = philox.keep_mask(7, 0.5, 1, np.arange(64), np.arange(512))
    assert (keep[:, 0::2] != keep[:, 1::2]).mean() > 0.45


def test_threshold_rule():
    assert philox.drop_threshold(0.0) == 0
    assert philox.drop_threshold(0.5) == 2**15
    assert philox.drop_threshold(float(np.float32(0.1))) == 6553
    assert philox.drop_threshold(0.99999) == 65535
    with pytest.raises(ValueError):
        philox.drop_threshold(1.0)
