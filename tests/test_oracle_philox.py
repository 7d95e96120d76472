"""Pins for the oracle's Philox4x32-10 (CPU only)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

from conftest import read_golden_rows
from oracle.philox import philox4x32_10, sr_uniform


def test_known_answer_vectors():
    for row in read_golden_rows("philox_kat.txt"):
        v = [int(t, 16) for t in row]
        got = philox4x32_10(*v[:6])
        assert [int(g) for g in got] == v[6:], row


def _torch_ref(queries):
    gxx = shutil.which("g++")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    src = os.path.join(os.path.dirname(__file__), "philox_torch_ref.cpp")
    if not gxx or not os.path.exists(os.path.join(inc, "ATen/core/PhiloxRNGEngine.h")):
        pytest.skip("g++ or torch headers missing")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "ref")
        subprocess.run([gxx, "-O1", "-std=c++17", "-I", inc, src, "-o", exe], check=True,
                       capture_output=True)
        inp = "".join(f"{s} {b} {o}\n" for s, b, o in queries)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return [[int(t) for t in line.split()] for line in out.strip().splitlines()]


def test_matches_pytorch_engine_stream_layout():
    # torch's engine: key = seed, counter = (offset lo, offset hi, subsequence lo, hi).
    # The codec's layout: counter = (i>>2 lo, i>>2 hi, step lo, step hi), key = seed.
    rng = np.random.default_rng(7)
    q = [(int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 40)), int(rng.integers(0, 2 ** 40)))
         for _ in range(64)]
    q += [(0, 0, 0), (4, 3, 12345), (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1)]
    ref = _torch_ref(q)
    for (seed, step, blk), words in zip(q, ref):
        got = philox4x32_10(blk & 0xFFFFFFFF, blk >> 32, step & 0xFFFFFFFF, step >> 32,
                            seed & 0xFFFFFFFF, seed >> 32)
        assert [int(g) for g in got] == words
        idx = np.array([4 * blk + k for k in range(4)], dtype=np.uint64) if blk < 2 ** 61 else None
        if idx is not None:
            u = sr_uniform(idx, seed, step)
            np.testing.assert_array_equal(u, [(w >> 8) * 2.0 ** -24 for w in words])


def test_uniform_statistics():
    u = sr_uniform(np.arange(1 << 20), seed=3, step=1)
    assert u.min() >= 0 and u.max() < 1
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / u.size)
    # different steps give different streams
    assert not np.array_equal(u[:1000], sr_uniform(np.arange(1000), seed=3, step=2))
