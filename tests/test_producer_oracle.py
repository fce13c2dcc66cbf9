"""Pins of the producer oracle (column-parallel MatMul + GeLU in front of the block)."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import producer
from oracle.block import widen
from workload import f32_to_bf16_bits, make_random_inputs

torch = pytest.importorskip("torch")


def test_gelu_matches_torch_tanh_gelu():
    """A library routine with the same definition (PyTorch's tanh GeLU, fp64)."""
    v = np.concatenate([np.linspace(-9, 9, 4001), np.random.default_rng(0).standard_normal(5000) * 3])
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    assert np.max(np.abs(producer.gelu_tanh(v) - ref)) < 1e-14


def test_gelu_close_to_exact_erf_gelu():
    """The tanh form approximates v * Phi(v) to within a few 1e-4 everywhere."""
    v = np.linspace(-8, 8, 16001)
    exact = np.array([x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) for x in v])
    dev = np.abs(producer.gelu_tanh(v) - exact)
    assert dev.max() < 5e-4
    assert dev.max() > 1e-5          # it is the tanh form, not the erf form


def test_gelu_identities():
    v = np.linspace(-20, 20, 2001)
    g = producer.gelu_tanh(v)
    assert producer.gelu_tanh(0.0) == 0.0
    np.testing.assert_allclose(g - producer.gelu_tanh(-v), v, rtol=0, atol=1e-12)   # odd tanh
    assert np.all(np.abs(g[v >= 10] - v[v >= 10]) < 1e-12)
    assert np.all(np.abs(g[v <= -10]) < 1e-12)


def test_round_bf16_matches_torch_on_fp32_values():
    """For fp64 values that are fp32 values, direct rounding equals fp32 -> bf16."""
    rng = np.random.default_rng(1)
    x32 = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                          (rng.standard_normal(1000) * 1e-38).astype(np.float32),
                          np.array([0.0, -0.0, 1e38, -3.3e38, 3.39e38], np.float32)])
    _, bits = producer.round_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(bits, f32_to_bf16_bits(x32))


def test_round_bf16_ties_and_no_double_rounding():
    one = 1.0
    vals = np.array([one + 2.0 ** -8,            # midpoint of 1 and 1 + 2^-7: to even (1)
                     one + 3 * 2.0 ** -8,        # midpoint of 1 + 2^-7 and 1 + 2^-6: to even
                     one + 2.0 ** -8 + 2.0 ** -40,   # just above the midpoint: up (an fp32
                                                     # step would round to the midpoint first)
                     -(one + 2.0 ** -8 + 2.0 ** -40)])
    v, bits = producer.round_bf16(vals)
    assert v.tolist() == [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7)]
    assert bits.tolist() == [0x3F80, 0x3F82, 0x3F81, 0xBF81]
    # the fp32 route double-rounds the third value down
    assert f32_to_bf16_bits(np.array([vals[2]], np.float32))[0] == 0x3F80


def test_producer_matmul_is_exact_on_tiny_shapes():
    """v = X . W1 + b1 against exact rational arithmetic; h = gelu(v)."""
    inp = make_random_inputs(6, 8, 5, seed=3)
    X, W, b = inp["X"], inp["W"], inp["bias"]
    h, bits, bound = producer.producer(X, W, b)
    x, w, bb = widen(X), widen(W), widen(b)
    for i in range(6):
        for j in range(5):
            exact = sum(Fraction(float(x[i, k])) * Fraction(float(w[k, j])) for k in range(8)) + \
                Fraction(float(bb[j]))
            assert abs(h[i, j] - producer.gelu_tanh(float(exact))) <= 1e-15 * max(1.0, abs(h[i, j]))
    _, expect = producer.round_bf16(h)
    assert np.array_equal(bits, expect)
    assert np.all(bound > 0)


def test_one_hot_rows_pin_orientation_and_bias():
    """X row i = e_i picks row i of W1: h[i, :] = gelu(W1[i, :] + b1)."""
    rng = np.random.default_rng(4)
    W1 = f32_to_bf16_bits(rng.standard_normal((7, 9)).astype(np.float32))
    b1 = f32_to_bf16_bits(rng.standard_normal(9).astype(np.float32))
    X = np.zeros((7, 7), np.uint16)
    X[np.arange(7), np.arange(7)] = 0x3F80
    h, _, _ = producer.producer(X, W1, b1)
    np.testing.assert_array_equal(h, producer.gelu_tanh(widen(W1) + widen(b1)[None, :]))


def test_check_bf16_output_accepts_exact_and_rejects_one_ulp_off():
    inp = make_random_inputs(32, 64, 48, seed=5)
    h, bits, bound = producer.producer(inp["X"], inp["W"], inp["bias"])
    producer.check_bf16_output(bits, h, bound)
    tie = producer.near_tie(h, bound)
    i = np.argwhere(~tie)[0]
    bad = bits.copy()
    bad[tuple(i)] += 1
    with pytest.raises(AssertionError):
        producer.check_bf16_output(bad, h, bound)
    assert tie.mean() < 0.2


def test_check_bf16_output_near_zero_after_cancellation():
    """Where the fp32 error bound exceeds a bf16 spacing (|h| tiny), values a few
    spacings away are accepted, values beyond the bound are not."""
    h = np.array([4.977e-6, 1.0])
    bound = np.array([1e-6, 1e-9])
    _, exact = producer.round_bf16(h)
    g = exact.copy()
    g[0] += 2                                        # two spacings (~3e-8 each) away
    assert producer.check_bf16_output(g, h, bound) == 1
    g[0] = exact[0] + 200                            # ~6e-6 away: beyond the bound
    with pytest.raises(AssertionError):
        producer.check_bf16_output(g, h, bound)


def test_linear_without_activation_is_exact_on_tiny_shapes():
    """activation="none" (the QKV projection): v = X . W1 + b1 against exact rational
    arithmetic, rounded once to bf16."""
    inp = make_random_inputs(5, 12, 7, seed=8)
    X, W, b = inp["X"], inp["W"], inp["bias"]
    h, bits, bound = producer.producer(X, W, b, activation="none")
    x, w, bb = widen(X), widen(W), widen(b)
    for i in range(5):
        for j in range(7):
            exact = sum(Fraction(float(x[i, k])) * Fraction(float(w[k, j])) for k in range(12)) + \
                Fraction(float(bb[j]))
            assert abs(Fraction(h[i, j]) - exact) <= Fraction(2.0 ** -50) * max(1, abs(exact))
    _, expect = producer.round_bf16(h)
    assert np.array_equal(bits, expect)
    # the GeLU variant of the same inputs differs (the activation is really applied there)
    hg, _, _ = producer.producer(X, W, b)
    assert not np.allclose(hg, h)
    with pytest.raises(ValueError):
        producer.producer(X, W, b, activation="relu")


def test_linear_one_hot_rows_and_double_rounding_pin():
    """One-hot X rows copy W1 rows plus b1 exactly; a row whose sum lies just above a bf16
    midpoint rounds up (the direct fp64 rounding), and the GPU's fp32 sum, which lands on
    the midpoint and rounds to even, is accepted only as a near tie."""
    rng = np.random.default_rng(9)
    W1 = f32_to_bf16_bits(rng.standard_normal((4, 6)).astype(np.float32))
    b1 = f32_to_bf16_bits(rng.standard_normal(6).astype(np.float32))
    X = np.zeros((4, 4), np.uint16)
    X[np.arange(4), np.arange(4)] = 0x3F80
    h, _, _ = producer.producer(X, W1, b1, activation="none")
    np.testing.assert_array_equal(h, widen(W1) + widen(b1)[None, :])
    # 1 + 2^-8 + 2^-40: X row (1, 2^-8, 2^-40) against a column of ones, bias 0
    Xd = f32_to_bf16_bits(np.array([[1.0, 2.0 ** -8, 2.0 ** -40]], np.float32))
    Wd = f32_to_bf16_bits(np.ones((3, 1), np.float32))
    bd = np.zeros(1, np.uint16)
    h, bits, bound = producer.producer(Xd, Wd, bd, activation="none")
    assert h[0, 0] == 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert bits[0, 0] == 0x3F81
    assert producer.near_tie(h, bound)[0, 0]
    assert producer.check_bf16_output(np.array([[0x3F80]], np.uint16), h, bound) == 1
    with pytest.raises(AssertionError):
        producer.check_bf16_output(np.array([[0x3F82]], np.uint16), h, bound)
