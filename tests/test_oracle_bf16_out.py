"""Pins of the fp32 error bound that judges the block's bf16 output variant.

The bf16 output is the fp32 result rounded once more (to nearest even).  Its bits are
compared with the fp64 oracle rounded straight to bf16, except where the fp64 value lies
within the fp32 error bound of a rounding midpoint (``oracle.producer.near_tie``).  The
bound must hold for any fp32 computation of the block, so it is checked here against
two fp32 simulations that sum in different orders, and it must be tight enough that a
plausible mistake breaks it.
"""
import numpy as np
import pytest

import oracle
from oracle import producer
from oracle.block import widen
from workload import make_random_inputs


def _fp32_block(inp, keep, order):
    """The block in numpy fp32: each slice summed from zero (k ascending, or pairwise),
    slices reduced left to right, then the epilogue with separate roundings."""
    X = widen(inp["X"]).astype(np.float32)
    W = widen(inp["W"]).astype(np.float32)
    b = widen(inp["bias"]).astype(np.float32)
    R = widen(inp["residual"]).astype(np.float32)
    P, K = inp["P"], X.shape[1]
    Ks = K // P
    T = None
    for p in range(P):
        prods = X[:, p * Ks:(p + 1) * Ks, None] * W[None, p * Ks:(p + 1) * Ks, :]   # exact
        if order == "sequential":
            S = np.zeros((X.shape[0], W.shape[1]), np.float32)
            for k in range(Ks):
                S = (S + prods[:, k, :]).astype(np.float32)
        else:   # pairwise
            while prods.shape[1] > 1:
                h = prods.shape[1] // 2
                pairs = (prods[:, :h, :] + prods[:, h:2 * h, :]).astype(np.float32)
                prods = np.concatenate([pairs, prods[:, 2 * h:, :]], axis=1)   # odd one out
            S = prods[:, 0, :]
        T = S if T is None else (T + S).astype(np.float32)
    v = (T + b[None, :]).astype(np.float32)
    scale = np.float32(oracle.keep_scale(inp["p_drop"]))
    out = (R + (v * scale).astype(np.float32)).astype(np.float32)
    return np.where(keep, out, R)


@pytest.mark.parametrize("M,K,N,P,seed", [(16, 256, 24, 4, 1), (8, 1024, 16, 2, 2), (12, 768, 8, 8, 3)])
@pytest.mark.parametrize("order", ["sequential", "pairwise"])
def test_fp32_simulations_stay_within_the_bound(M, K, N, P, seed, order):
    inp = make_random_inputs(M, K, N, seed=seed)
    inp.update(P=P, p_drop=np.float32(0.1), seed=seed)
    out, keep = oracle.run_inputs(inp)
    bound = oracle.error_bound_fp32(inp["X"], inp["W"], inp["bias"], inp["residual"], P,
                                    inp["p_drop"], keep)
    out32 = _fp32_block(inp, keep, order).astype(np.float64)
    err = np.abs(out32 - out)
    assert np.all(err <= bound)
    assert np.all(bound[~keep] == 0) and np.all(err[~keep] == 0)   # dropped: the residual
    assert np.all(bound[keep] > 0)
    # the bound is generous but not vacuous: far below a bf16 spacing for most elements
    assert np.median(bound[keep] / producer.bf16_ulp(out[keep])) < 0.05


def test_a_wrong_bias_breaks_the_bound():
    """A plausible mistake (each column given its neighbour's bias) is far outside."""
    inp = make_random_inputs(16, 512, 32, seed=4)
    inp.update(P=4, p_drop=np.float32(0.0), seed=4)
    out, keep = oracle.run_inputs(inp)
    bound = oracle.error_bound_fp32(inp["X"], inp["W"], inp["bias"], inp["residual"], 4,
                                    inp["p_drop"], keep)
    shifted = dict(inp, bias=np.roll(inp["bias"], 1))
    wrong, _ = oracle.run_inputs(shifted)
    assert np.mean(np.abs(wrong - out) > bound) > 0.9


def test_bf16_rounding_of_the_fp32_simulation_passes_the_near_tie_rule():
    """The bf16 output of an fp32 computation (its fp32 result rounded to nearest even)
    satisfies check_bf16_output against the fp64 oracle; a one-spacing error off a near
    tie does not."""
    inp = make_random_inputs(32, 1024, 48, seed=5)
    inp.update(P=8, p_drop=np.float32(0.1), seed=5)
    out, keep = oracle.run_inputs(inp)
    bound = oracle.error_bound_fp32(inp["X"], inp["W"], inp["bias"], inp["residual"], 8,
                                    inp["p_drop"], keep)
    out32 = _fp32_block(inp, keep, "sequential")
    _, bits = producer.round_bf16(out32.astype(np.float64))
    ties = producer.check_bf16_output(bits, out, bound)
    assert ties < 0.1 * out.size
    tie = producer.near_tie(out, bound)
    i = np.argwhere(~tie)[0]
    bad = bits.copy()
    bad[tuple(i)] += 1
    with pytest.raises(AssertionError):
        producer.check_bf16_output(bad, out, bound)
