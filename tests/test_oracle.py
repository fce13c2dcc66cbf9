"""Pins for the fp64 oracle: each checks it against something other than itself."""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import philox
from workload import WORKLOADS, f32_to_bf16_bits, make_inputs, make_random_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ONE = 0x3F80            # bf16 bits of 1.0


def _bf16_to_float(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- bf16 generator
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # ties and near-ties around bf16 boundaries, both parities
    base = rng.integers(0, 2 ** 16, 5000).astype(np.uint32) << 16
    ties = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base | 0x18000 & 0xFFFFFFFF])
    ties = ties.view(np.float32)
    ties = ties[np.isfinite(ties)]
    a = np.concatenate([a, ties, np.array([0.0, -0.0, 1e-40, -1e-40, 3.0e38], np.float32)])
    ours = f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_widen_is_exact():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 16, 10000).astype(np.uint16)
    bits = bits[[math.isfinite(_bf16_to_float(b)) for b in bits]]
    w = oracle.widen(bits)
    assert all(w[i] == _bf16_to_float(b) for i, b in enumerate(bits[:3000]))


# ---------------------------------------------------------------- exact brute force
def _exact_block(X, W, bias, res, P, p32, seed):
    """Rational arithmetic, element by element; mask from the scalar Philox."""
    M, K = X.shape
    N = W.shape[1]
    Ks = K // P
    thr = math.floor(Fraction(float(p32)) * 2 ** 32)
    scale = None if p32 == 1 else 1 / (1 - Fraction(float(p32)))
    xf = [[Fraction(_bf16_to_float(X[m, k])) for k in range(K)] for m in range(M)]
    wf = [[Fraction(_bf16_to_float(W[k, n])) for n in range(N)] for k in range(K)]
    out = np.zeros((M, N), dtype=object)
    mag = np.zeros((M, N))
    keep = np.zeros((M, N), dtype=bool)
    for m in range(M):
        for n in range(N):
            e = m * N + n
            blk = philox.block_scalar((e >> 2 & 0xFFFFFFFF, e >> 34, 0, 0),
                                      (seed & 0xFFFFFFFF, seed >> 32))
            kp = thr < 2 ** 32 and blk[e & 3] >= thr
            tot = Fraction(0)
            absum = 0.0
            for p in range(P):
                s = sum((xf[m][k] * wf[k][n] for k in range(p * Ks, (p + 1) * Ks)), Fraction(0))
                tot += s
                absum += float(sum(abs(xf[m][k] * wf[k][n]) for k in range(p * Ks, (p + 1) * Ks)))
            b = Fraction(_bf16_to_float(bias[n]))
            r = Fraction(_bf16_to_float(res[m, n]))
            out[m, n] = r + ((tot + b) * scale if kp else 0)
            mag[m, n] = abs(float(r)) + (float(scale) * (absum + abs(float(b))) if kp else 0)
            keep[m, n] = kp
    return out, mag, keep


@pytest.mark.parametrize("M,K,N,P", [(3, 8, 5, 1), (4, 16, 4, 2), (5, 16, 6, 4), (2, 12, 7, 3),
                                     (6, 8, 8, 8)])
@pytest.mark.parametrize("p_drop", [0.0, 0.1, 0.5, 1.0])
def test_brute_force_exact(M, K, N, P, p_drop):
    inp = make_random_inputs(M, K, N, seed=M * 100 + K + N, sigma_w=0.5, sigma_bias=0.5)
    seed = 0x0123456789ABCDEF if P == 2 else P
    p32 = np.float32(p_drop)
    out, keep = oracle.run(inp["X"], inp["W"], inp["bias"], inp["residual"], P, p32, seed)
    ex, mag, kex = _exact_block(inp["X"], inp["W"], inp["bias"], inp["residual"], P, p32, seed)
    assert np.array_equal(keep, kex)
    err = np.abs(out - ex.astype(np.float64))
    bound = (K + 8) * 2.0 ** -53 * mag + 1e-300
    assert np.all(err <= bound), (err.max(), bound.min())


# ---------------------------------------------------------------- invariants & special cases
def test_slice_sum_equals_unsliced_product():
    inp = make_random_inputs(48, 384, 40, seed=5)
    X = oracle.widen(inp["X"])
    W = oracle.widen(inp["W"])
    full = X @ W
    absprod = np.abs(X) @ np.abs(W)
    for P in (1, 2, 3, 4, 6, 8, 16, 32):
        T = sum(oracle.slice_partials(inp["X"], inp["W"], P))
        assert np.all(np.abs(T - full) <= 1e-12 * absprod + 1e-300)


def test_p0_is_residual_plus_bias_plus_product():
    inp = make_random_inputs(40, 256, 72, seed=6)
    out, keep = oracle.run(inp["X"], inp["W"], inp["bias"], inp["residual"], 4, 0.0, 11)
    assert keep.all()
    X = oracle.widen(inp["X"])
    W = oracle.widen(inp["W"])
    direct = oracle.widen(inp["residual"]) + oracle.widen(inp["bias"])[None, :] + np.matmul(X, W)
    assert np.allclose(out, direct, rtol=0, atol=1e-12)


def test_p1_is_residual_exactly():
    inp = make_random_inputs(32, 64, 64, seed=7)
    out, keep = oracle.run(inp["X"], inp["W"], inp["bias"], inp["residual"], 2, 1.0, 3)
    assert not keep.any()
    assert np.array_equal(out, oracle.widen(inp["residual"]))


def test_dropped_elements_equal_residual():
    inp = make_random_inputs(64, 128, 96, seed=8)
    out, keep = oracle.run(inp["X"], inp["W"], inp["bias"], inp["residual"], 4, 0.3, 9)
    res = oracle.widen(inp["residual"])
    assert np.array_equal(out[~keep], res[~keep])
    assert 0.6 < keep.mean() < 0.8


def test_indexing_pins_bias_column_residual_row():
    """X = 0: out[m, n] = m + n + 1 exactly when bias[n] = n + 1, residual[m, n] = m."""
    M, N, K = 12, 20, 64
    X = np.zeros((M, K), np.uint16)
    W = f32_to_bf16_bits(np.ones((K, N), np.float32))
    bias = f32_to_bf16_bits(np.arange(1, N + 1, dtype=np.float32))
    res = f32_to_bf16_bits(np.repeat(np.arange(M, dtype=np.float32)[:, None], N, axis=1))
    out, _ = oracle.run(X, W, bias, res, 4, 0.0, 0)
    want = np.arange(M)[:, None] + np.arange(N)[None, :] + 1.0
    assert np.array_equal(out, want)


def test_permutation_pins_operand_orientation():
    """X = a permutation matrix: out = W with its rows permuted; W non-square."""
    K, N = 64, 48
    perm = np.random.default_rng(2).permutation(K)
    Xf = np.zeros((K, K), np.float32)
    Xf[np.arange(K), perm] = 1.0
    W = make_random_inputs(1, K, N, seed=3)["W"]
    out, _ = oracle.run(f32_to_bf16_bits(Xf), W, np.zeros(N, np.uint16),
                        np.zeros((K, N), np.uint16), 4, 0.0, 0)
    assert np.array_equal(out, oracle.widen(W)[perm])


def test_one_hot_slices_pin_slice_boundaries():
    """A single unit product in slice q lands in the output; the sum is over all slices."""
    M, N, K, P = 2, 8, 64, 4
    for q in range(P):
        for kk in (0, K // P - 1):
            k = q * (K // P) + kk
            X = np.zeros((M, K), np.uint16)
            W = np.zeros((K, N), np.uint16)
            X[1, k] = ONE
            W[k, 5] = f32_to_bf16_bits(np.float32([3.0]))[0]
            parts = list(oracle.slice_partials(X, W, P))
            for p, S in enumerate(parts):
                assert S[1, 5] == (3.0 if p == q else 0.0)
                assert np.count_nonzero(S) == (1 if p == q else 0)


def test_scale_closed_form_and_mask_readout():
    """X = 0, bias = 1, residual = 0: out is 0 (dropped) or exactly 1/(1-p) (kept)."""
    M, N, K = 64, 256, 256
    X = np.zeros((M, K), np.uint16)
    W = np.zeros((K, N), np.uint16)
    bias = np.full(N, ONE, np.uint16)
    res = np.zeros((M, N), np.uint16)
    out, keep = oracle.run(X, W, bias, res, 4, np.float32(0.1), 0)
    scale = 1.0 / (1.0 - float(np.float32(0.1)))
    assert np.array_equal(out != 0, keep)
    assert np.all(out[keep] == scale)


def test_threshold_closed_form():
    g = _load("structure_pins.json")
    assert oracle.drop_threshold(np.float32(0.1)) == g["threshold_p_0.1f"]["value"]
    assert oracle.drop_threshold(0.0) == 0
    assert oracle.drop_threshold(0.5) == 2 ** 31
    assert oracle.drop_threshold(1.0) == 2 ** 32
    # the smallest positive fp32 p drops only r = 0 ... floor(p * 2^32)
    assert oracle.drop_threshold(np.float32(2.0 ** -32)) == 1
    for bad in (-0.1, 1.5, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            oracle.check_p(bad)


def test_bad_slicing_rejected():
    with pytest.raises(ValueError):
        list(oracle.slice_partials(np.zeros((2, 10), np.uint16), np.zeros((10, 2), np.uint16), 3))


# ---------------------------------------------------------------- mask
def test_mask_matches_scalar_philox_per_element():
    M, N, seed, p = 96, 160, 0xFEEDFACE12345678, np.float32(0.25)
    keep = oracle.keep_mask(M, N, p, seed)
    thr = oracle.drop_threshold(p)
    rng = np.random.default_rng(4)
    for m, n in zip(rng.integers(0, M, 400), rng.integers(0, N, 400)):
        e = int(m) * N + int(n)
        w = philox.block_scalar((e >> 2, 0, 0, 0), (seed & 0xFFFFFFFF, seed >> 32))[e & 3]
        assert keep[m, n] == (w >= thr)


@pytest.mark.parametrize("offset", [1, 0xFFFFFFFF, 2 ** 32, 0x0123456789ABCDEF, 2 ** 64 - 1])
def test_mask_with_offset_matches_scalar_philox_per_element(offset):
    """A non-zero stream offset fills counter words 2 (low half) and 3 (high half)."""
    M, N, seed, p = 64, 96, 0x5EED, np.float32(0.3)
    keep = oracle.keep_mask(M, N, p, seed, offset=offset)
    thr = oracle.drop_threshold(p)
    rng = np.random.default_rng(5)
    for m, n in zip(rng.integers(0, M, 300), rng.integers(0, N, 300)):
        e = int(m) * N + int(n)
        w = philox.block_scalar((e >> 2, 0, offset & 0xFFFFFFFF, offset >> 32),
                                (seed & 0xFFFFFFFF, seed >> 32))[e & 3]
        assert keep[m, n] == (w >= thr)
    # the row-subset and element paths agree with the whole-output path
    rows = np.array([3, 0, 63])
    assert np.array_equal(oracle.keep_mask(M, N, p, seed, rows=rows, offset=offset), keep[rows])
    e = np.arange(M * N).reshape(M, N)
    assert np.array_equal(oracle.keep_elements(e, p, seed, offset), keep)


def test_offset_zero_is_the_default_and_offsets_give_independent_masks():
    a = oracle.keep_mask(128, 256, 0.1, 9)
    assert np.array_equal(oracle.keep_mask(128, 256, 0.1, 9, offset=0), a)
    for off in (1, 2 ** 32):
        b = oracle.keep_mask(128, 256, 0.1, 9, offset=off)
        assert abs((a != b).mean() - 2 * 0.1 * 0.9) < 0.02
    # run() threads the offset to the mask: dropped elements equal the residual exactly
    inp = make_random_inputs(32, 64, 32, 2)
    X, W, bias, res = inp["X"], inp["W"], inp["bias"], inp["residual"]
    out0, k0 = oracle.run(X, W, bias, res, 2, 0.5, 3)
    out1, k1 = oracle.run(X, W, bias, res, 2, 0.5, 3, offset=7)
    assert np.array_equal(k1, oracle.keep_mask(32, 32, 0.5, 3, offset=7))
    assert not np.array_equal(k0, k1)
    assert np.array_equal(out1[~k1], oracle.widen(res)[~k1])
    assert np.array_equal(out1[k1 & k0], out0[k1 & k0])


def test_mask_row_subsets_and_elements_agree():
    M, N = 64, 96
    full = oracle.keep_mask(M, N, 0.1, 77)
    rows = np.array([0, 5, 63, 17])
    assert np.array_equal(oracle.keep_mask(M, N, 0.1, 77, rows=rows), full[rows])
    e = np.arange(M * N).reshape(M, N)
    assert np.array_equal(oracle.keep_elements(e, 0.1, 77), full)
    # N not a multiple of 4: groups straddle rows, still by linear index
    full2 = oracle.keep_mask(7, 9, 0.5, 1)
    assert np.array_equal(full2, oracle.keep_elements(np.arange(63).reshape(7, 9), 0.5, 1))


def test_mask_depends_on_seed():
    a = oracle.keep_mask(128, 256, 0.1, 1)
    b = oracle.keep_mask(128, 256, 0.1, 2)
    frac = (a != b).mean()
    assert abs(frac - 2 * 0.1 * 0.9) < 0.02


@pytest.mark.parametrize("name", ["tiny", "gpt2_attn", "bert_mlp", "gpt3_mlp"])
def test_kept_fraction_within_binomial_spread(name):
    w = WORKLOADS[name]
    keep = oracle.keep_mask(w.M, w.N, np.float32(w.p_drop), w.seed)
    q = 1 - oracle.drop_threshold(np.float32(w.p_drop)) / 2 ** 32
    n = keep.size
    sigma = math.sqrt(q * (1 - q) / n)
    assert abs(keep.mean() - q) <= 5 * sigma
    if name != "tiny":
        # neighbouring elements are independent: P(keep_e and keep_e+1) ~ q^2
        both = (keep[:, :-1] & keep[:, 1:]).mean()
        assert abs(both - q * q) < 6 * math.sqrt(q * q * (1 - q * q) / both.size) + 1e-4


# ---------------------------------------------------------------- fp32 order model
def _structure_inputs(P, Ks, slice_values):
    """One output element; slice p is made of Ks products whose sum is slice_values[p]."""
    K = P * Ks
    X = np.zeros((1, K), np.uint16)
    W = np.zeros((K, 1), np.uint16)
    for p, kind in enumerate(slice_values):
        lo = p * Ks
        if kind == "big":          # Ks products of 2^18 -> 2^24 (Ks = 64)
            X[0, lo:lo + Ks] = ONE
            W[lo:lo + Ks, 0] = f32_to_bf16_bits(np.full(Ks, 2.0 ** 18, np.float32))
        elif kind == "-big":
            X[0, lo:lo + Ks] = ONE
            W[lo:lo + Ks, 0] = f32_to_bf16_bits(np.full(Ks, -(2.0 ** 18), np.float32))
        elif kind == "unit_per_32":   # one unit product in each 32-wide k block
            for b in range(0, Ks, 32):
                X[0, lo + b] = ONE
                W[lo + b, 0] = ONE
        elif kind == "one":
            X[0, lo] = ONE
            W[lo, 0] = ONE
    return X, W


def test_per_slice_accumulation_pin():
    g = _load("structure_pins.json")["per_slice_2p24"]
    X, W = _structure_inputs(2, 64, ["big", "unit_per_32"])
    z1 = np.zeros(1, np.uint16)
    parts = list(oracle.slice_partials(X, W, 2))
    assert parts[0][0, 0] == 2.0 ** 24 and parts[1][0, 0] == 2.0
    keep = np.ones((1, 1), bool)
    out32 = oracle.reduce_epilogue_fp32(parts, z1, np.zeros((1, 1), np.uint16), keep, 0.0)
    assert float(out32[0, 0]) == g["per_slice_fp32"]
    out64, _ = oracle.run(X, W, z1, np.zeros((1, 1), np.uint16), 2, 0.0, 0)
    assert out64[0, 0] == g["fp64"]
    # the alternative reading (one fp32 accumulator across the slices) gives another value
    acc = np.float32(2.0 ** 24)
    for _ in range(2):
        acc = np.float32(acc + np.float32(1.0))
    assert float(acc) == g["continuous_fp32"] != g["per_slice_fp32"]


def test_slice_order_pin():
    g = _load("structure_pins.json")["slice_order"]
    X, W = _structure_inputs(3, 64, ["big", "one", "-big"])
    parts = list(oracle.slice_partials(X, W, 3))
    z1 = np.zeros(1, np.uint16)
    zr = np.zeros((1, 1), np.uint16)
    keep = np.ones((1, 1), bool)
    assert float(oracle.reduce_epilogue_fp32(parts, z1, zr, keep, 0.0)[0, 0]) == g["left_to_right_fp32"]
    assert float(oracle.reduce_epilogue_fp32(parts[::-1], z1, zr, keep, 0.0)[0, 0]) == g["right_to_left_fp32"]
    out64, _ = oracle.run(X, W, z1, zr, 3, 0.0, 0)
    assert out64[0, 0] == g["fp64"]


def test_fp32_model_epilogue_closed_form():
    """T exact, bias 0.5, residual 0.25, p = 0.1: out = fl(0.25 + fl(fl(T + 0.5) * s32))."""
    T = np.array([[3.0, -7.0, 1.0e6, 0.0]])
    bias = f32_to_bf16_bits(np.full(4, 0.5, np.float32))
    res = f32_to_bf16_bits(np.full((1, 4), 0.25, np.float32))
    keep = np.array([[True, True, True, False]])
    out = oracle.reduce_epilogue_fp32([T], bias, res, keep, np.float32(0.1))
    s32 = np.float32(1.0 / (1.0 - float(np.float32(0.1))))
    for j in range(3):
        v = np.float32(np.float32(T[0, j]) + np.float32(0.5))
        assert out[0, j] == np.float32(np.float32(0.25) + np.float32(v * s32))
    assert out[0, 3] == np.float32(0.25)


# ---------------------------------------------------------------- stored oracle digest
@pytest.mark.parametrize("name", ["tiny", "gpt2_attn"])
def test_oracle_matches_stored_digest(name):
    import hashlib
    d = _load("oracle_digest.json")[name]
    inp = make_inputs(name)
    w = WORKLOADS[name]
    keep = oracle.keep_mask(w.M, w.N, inp["p_drop"], w.seed)
    assert hashlib.sha256(np.packbits(keep).tobytes()).hexdigest() == d["keep_sha256"]
    assert int(keep.sum()) == d["kept"]
    rows, cols = d["rows"], d["cols"]
    out, _ = oracle.run_inputs(inp, rows=rows, cols=cols)
    assert np.allclose(out, np.array(d["out"]), rtol=1e-12, atol=1e-12)


def test_threshold_tie_is_kept():
    """A word equal to floor(p * 2^32) is kept (drop iff r < threshold, strictly)."""
    # find a seed whose element-0 word has its low 8 bits clear, so r / 2^32 is an fp32
    for seed in range(100000):
        r = philox.block_scalar((0, 0, 0, 0), (seed, 0))[0]
        if r % 256 == 0 and r > 2 ** 24:
            break
    p = np.float32(r / 2 ** 32)
    assert oracle.drop_threshold(p) == r
    assert oracle.keep_elements(np.array([0]), p, seed)[0]
    assert oracle.keep_mask(1, 4, p, seed)[0, 0]
    p_up = np.nextafter(p, np.float32(1))
    assert oracle.drop_threshold(p_up) > r
    assert not oracle.keep_elements(np.array([0]), p_up, seed)[0]
    assert not oracle.keep_mask(1, 4, p_up, seed)[0, 0]
