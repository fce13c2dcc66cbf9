"""Pins for the oracle's Philox4x32-10 (Salmon et al., SC'11)."""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def test_weyl_constants_closed_forms():
    # W0 = floor(2^32 * (sqrt(5) - 1) / 2), W1 = floor(2^32 * (sqrt(3) - 1)), exactly
    two32 = 2 ** 32
    s5 = math.isqrt(5 * two32 * two32)          # floor(2^32 * sqrt(5))
    s3 = math.isqrt(3 * two32 * two32)          # floor(2^32 * sqrt(3))
    assert philox.W0 == (s5 - two32) // 2
    assert philox.W1 == s3 - two32
    assert philox.ROUNDS == 10


def test_scalar_and_vectorized_agree():
    rng = np.random.default_rng(1234)
    n = 100_000
    c = rng.integers(0, 2 ** 32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    for key in [(0, 0), (0xFFFFFFFF, 0xFFFFFFFF), (0x12345678, 0x9ABCDEF0)]:
        vec = philox.blocks_np(c[:, 0], c[:, 1], c[:, 2], c[:, 3], *key)
        for i in list(range(200)) + list(rng.integers(0, n, size=300)):
            assert tuple(int(v) for v in vec[i]) == philox.block_scalar(c[i], key)


def test_vectorized_broadcasts_counter_words():
    c0 = np.arange(1000, dtype=np.uint32)
    a = philox.blocks_np(c0, 7, 0, 0, 5, 6)
    for i in (0, 1, 999):
        assert tuple(int(v) for v in a[i]) == philox.block_scalar((i, 7, 0, 0), (5, 6))


def _rocrand_exe(tmp_path_factory):
    cxx = shutil.which("g++")
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if cxx is None or not os.path.exists(hdr):
        pytest.skip("no host compiler or rocRAND header")
    out = tmp_path_factory.mktemp("kat") / "kat"
    cmd = [cxx, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(HERE, "philox_rocrand_kat.cpp"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("rocRAND header does not build for the host: " + r.stderr[-300:])
    return str(out)


def test_known_answers_against_rocrand(tmp_path_factory):
    """rocRAND ships Philox4x32-10 as header-only host code: an independent implementation."""
    exe = _rocrand_exe(tmp_path_factory)
    rng = np.random.default_rng(7)
    pairs = [(0, 0), (0, 1), (1, 0), (2 ** 64 - 1, 0), (0xDEADBEEFCAFEF00D, 2 ** 40 + 3),
             (4, 6_291_455), (3, 2 ** 33 + 17)]
    pairs += [(int(s), int(g)) for s, g in zip(rng.integers(0, 2 ** 63, 500, dtype=np.uint64),
                                               rng.integers(0, 2 ** 61, 500, dtype=np.uint64))]
    text = "".join(f"{s} {g} 0\n" for s, g in pairs)
    r = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
    lines = r.stdout.split("\n")
    for (s, g), line in zip(pairs, lines):
        want = tuple(int(w, 16) for w in line.split())
        got = philox.block_scalar((g & 0xFFFFFFFF, g >> 32, 0, 0), (s & 0xFFFFFFFF, s >> 32))
        assert got == want, (s, g)
    # non-zero counter words 2 and 3 (rocRAND's subsequence): the mask's stream offset
    trip = [(0, 0, 1), (5, 3, 2 ** 32), (2 ** 64 - 1, 2 ** 40 + 3, 2 ** 64 - 1),
            (0x5EED, 17, 0x0123456789ABCDEF)]
    trip += [(int(s), int(g), int(o)) for s, g, o in zip(rng.integers(0, 2 ** 63, 300, dtype=np.uint64),
                                                         rng.integers(0, 2 ** 61, 300, dtype=np.uint64),
                                                         rng.integers(0, 2 ** 63, 300, dtype=np.uint64))]
    r = subprocess.run([exe], input="".join(f"{s} {g} {o}\n" for s, g, o in trip),
                       capture_output=True, text=True, check=True)
    for (s, g, o), line in zip(trip, r.stdout.split("\n")):
        want = tuple(int(w, 16) for w in line.split())
        got = philox.block_scalar((g & 0xFFFFFFFF, g >> 32, o & 0xFFFFFFFF, o >> 32),
                                  (s & 0xFFFFFFFF, s >> 32))
        assert got == want, (s, g, o)
    # the vectorized form over a contiguous run of counters, seed 2
    g = np.arange(4096, dtype=np.uint64)
    vec = philox.blocks_np(g.astype(np.uint32), 0, 0, 0, 2, 0)
    r = subprocess.run([exe], input="".join(f"2 {i} 0\n" for i in range(4096)),
                       capture_output=True, text=True, check=True)
    want = np.array([[int(w, 16) for w in ln.split()] for ln in r.stdout.strip().split("\n")],
                    dtype=np.uint32)
    assert np.array_equal(vec, want)


def test_output_statistics():
    n = 1 << 18
    blk = philox.blocks_np(np.arange(n, dtype=np.uint32), 0, 0, 0, 99, 0).ravel()
    # every bit is set about half of the time
    bits = ((blk[:, None] >> np.arange(32, dtype=np.uint32)[None, :]) & 1).mean(axis=0)
    sigma = 0.5 / math.sqrt(blk.size)
    assert np.all(np.abs(bits - 0.5) < 6 * sigma)
    # top-4-bit buckets are uniform (chi-square, 15 dof; 99.99% quantile ~ 44.3)
    counts = np.bincount((blk >> 28).astype(np.int64), minlength=16)
    exp = blk.size / 16
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 44.3


def test_avalanche_on_counter_bit():
    base = philox.block_scalar((12345, 0, 0, 0), (1, 2))
    flips = []
    for bit in range(32):
        other = philox.block_scalar((12345 ^ (1 << bit), 0, 0, 0), (1, 2))
        flips.append(sum(bin(a ^ b).count("1") for a, b in zip(base, other)))
    assert 40 < np.mean(flips) < 88      # about half of the 128 output bits
