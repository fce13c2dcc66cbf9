"""The producer side of the block, computed plainly in fp64 (oracle side; test infrastructure).

What is computed.  The tensor-parallel MatMul-then-AllReduce block sits between two
matmuls of a transformer layer (practices record SOTA-059, "Where it stops being free";
CoCoNet record LIT-735, "Key takeaways", second bullet: the block of a GPT-2 MLP).  The
first of the two is the column-parallel MatMul with the MLP's GeLU: rank p holds the
column block N_p of W1 and computes H[:, N_p] = GeLU(X . W1[:, N_p] + b1[N_p]).  That
shard is exactly the K-slice p the row-parallel block consumes, so no collective sits
between the two; folded onto one device it is one MatMul with a bias + GeLU tail whose
bf16 output H is the block's X.

For the attention block the MatMul in front is the QKV projection: the same column-
parallel MatMul + bias with no activation (H = X . W + b), so ``producer`` takes the
activation as an argument ("gelu_tanh" or "none").

Readings (the pages name the MLP but give no formula):

* GeLU is the tanh form used by GPT-2: gelu(v) = v/2 * (1 + tanh(sqrt(2/pi) * (v +
  0.044715 v^3)));
* v = X . W1 + b1 in fp64 from the bf16 inputs (widened exactly);
* H is gelu(v) rounded once, from fp64, to bf16 (round to nearest, ties to even), the
  activation dtype of a bf16 model.

Parity of a bf16 output.  The GPU computes v and gelu(v) in fp32, so its value differs
from the fp64 one by a small amount; rounding to bf16 gives the same bits unless the
fp64 value lies within that amount of a rounding midpoint.  ``near_tie`` marks those
elements from a per-element error bound; there any bf16 value within the bound plus half
a bf16 spacing of the fp64 value is a correct result (usually one of the two
neighbours; a few spacings for a value near zero after cancellation).
"""
from __future__ import annotations

import math

import numpy as np

from .block import widen

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)


def gelu_tanh(v):
    """GeLU, tanh form, in fp64."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(_SQRT_2_OVER_PI * (v + 0.044715 * v * v * v)))


def round_bf16(x):
    """fp64 -> nearest bf16 (ties to even), directly from fp64 (no fp32 step).

    Returns (value as fp64, bits as uint16).  Values beyond the bf16 range become
    +-inf; NaN becomes the canonical quiet NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    finite = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[finite])                   # x = m * 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits for normal numbers (exponent >= -125 here: e - 1 >=
    # -126); below that the spacing is fixed at 2^-133
    e_eff = np.maximum(e, -125)
    q = np.rint(np.ldexp(x[finite], 8 - e_eff))  # exact scaling; rint = ties to even
    out[finite] = np.ldexp(q, e_eff - 8)
    out[~finite] = x[~finite]
    big = np.abs(out) > float(np.float32(3.3895313892515355e38))  # largest finite bf16
    out[big & np.isfinite(x)] = np.copysign(np.inf, x[big & np.isfinite(x)])
    f32 = out.astype(np.float32)                  # exact: every bf16 value is an fp32 value
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(x)] = np.uint16(0x7FC0)
    return out, bits


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (fp64), for finite x."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x == 0, 1.0, x))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


ACTIVATIONS = ("gelu_tanh", "none")


def producer(X, W1, b1, rows=None, activation="gelu_tanh"):
    """H = act(X . W1 + b1), act = GeLU (tanh form) or the identity ("none").  Returns
    (h fp64, H bf16 bits, bound fp64) for the listed rows (all by default); ``bound`` is
    the per-element error bound of an fp32 computation of h (see ``near_tie``)."""
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {ACTIVATIONS}")
    X = np.asarray(X)
    W1 = np.asarray(W1)
    b1 = np.asarray(b1)
    Xr = X if rows is None else X[np.asarray(rows)]
    x64, w64 = widen(Xr), widen(W1)
    v = x64 @ w64 + widen(b1)[None, :]
    # error of an fp32 sum of these products: a few units of 2^-24 times the sum of the
    # magnitudes (generous: 64 units), carried through gelu (|gelu'| < 1.13), plus a few
    # fp32 units of gelu itself
    mag = np.abs(x64) @ np.abs(w64) + np.abs(widen(b1))[None, :]
    if activation == "gelu_tanh":
        h = gelu_tanh(v)
        bound = 1.13 * 64.0 * 2.0 ** -24 * mag + 2.0 ** -20 * np.abs(h)
    else:
        h = v
        bound = 64.0 * 2.0 ** -24 * mag + 2.0 ** -22 * np.abs(h)
    _, bits = round_bf16(h)
    return h, bits, bound


def near_tie(h, bound):
    """True where h lies within ``bound`` of a bf16 rounding midpoint (or of a value
    whose neighbours straddle it), so that an fp32 computation may round either way."""
    h = np.asarray(h, dtype=np.float64)
    ulp = bf16_ulp(h)
    lo = np.floor(h / ulp) * ulp
    mid = lo + 0.5 * ulp
    return np.abs(h - mid) <= bound


def check_bf16_output(gpu_bits, h, bound):
    """Bits of a GPU bf16 output against the fp64 value: equal to round_bf16(h), or, at
    a near tie, a bf16 value within bound + half a bf16 spacing of h (what rounding an
    fp32 value within ``bound`` of h can give; where the bound exceeds a spacing, as for
    a value near zero after cancellation, that is more than the two neighbours).
    Returns the number of near-tie elements; raises AssertionError on a mismatch."""
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    _, exact = round_bf16(h)
    tie = near_tie(h, bound)
    ok = gpu_bits == exact
    if tie.any():
        g = widen(gpu_bits[tie])
        ht = h[tie]
        half = 0.5 * np.maximum(bf16_ulp(ht), bf16_ulp(g))
        ok[tie] = np.abs(g - ht) <= bound[tie] + half
    if not ok.all():
        i = np.unravel_index(np.argmin(ok), ok.shape)
        raise AssertionError(f"{int((~ok).sum())} bf16 outputs differ; first at {i}: "
                             f"gpu=0x{int(gpu_bits[i]):04x} exact=0x{int(exact[i]):04x} "
                             f"h={h[i]!r} near_tie={bool(tie[i])}")
    return int(tie.sum())
