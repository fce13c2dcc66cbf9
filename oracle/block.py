"""The block, computed plainly in fp64 on the CPU (oracle side; test infrastructure).

What is computed.  The tensor-parallel MatMul-then-AllReduce of a transformer layer
(CoCoNet record LIT-735, "Key takeaways", second bullet: the model-parallel MatMul whose
result an AllReduce sums, overlapped in chunks) with the pointwise work that follows it
fused in (same page, first bullet: fusing pointwise work into a collective).  Rank p of
a row-parallel layer holds the K-slice K_p of the contraction and produces the partial
product S_p = X[:, K_p] . W[K_p, :]; the AllReduce sums the P partials; the pointwise
tail adds the bias, applies dropout and adds the residual:

    out = residual + dropout_p( bias + sum_{p=0}^{P-1} X[:, K_p] . W[K_p, :] )

Folded onto one device, the P ranks become P K-slices of one contraction.  The pages
print no numeric example, so each choice they leave open is a stated reading:

* inputs are bf16 bit patterns, widened exactly (bf16 -> fp32 -> fp64);
* K_p = [p*K/P, (p+1)*K/P), P divides K;
* the partials are summed left to right, p = 0 .. P-1, starting from S_0;
* dropout is inverted dropout: a kept value is multiplied by 1/(1-p), a dropped one
  contributes zero;
* the keep decision for the element at row m, column n uses e = m*N + n: the
  Philox4x32-10 block with counter (lo32(e>>2), hi32(e>>2), lo32(offset), hi32(offset))
  and key (lo32(seed), hi32(seed)); r = word (e & 3) of that block; the element is
  dropped iff r < floor(p * 2^32), with p taken as an fp32 value; p = 1 drops
  everything.  The offset (counter words 2 and 3) is 0 unless a caller asks for a
  separate stream under the same seed (a layer or step index);
* p outside [0, 1] or not finite is an error.

Everything here is fp64 except the keep decision (integer) and ``reduce_epilogue_fp32``,
which models the fp32 rounding order of the reduction and epilogue for the structure
checks (partials summed in fp32 from S_0, left to right; bias add, scale multiply and
residual add each rounded to nearest even, with no fused multiply-add).
"""
from __future__ import annotations

import math

import numpy as np

from . import philox

_U32 = np.uint32
_TWO32 = 2 ** 32


# ---------------------------------------------------------------- inputs
def widen(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64, exactly (bits become the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << _U32(16)).view(np.float32).astype(np.float64)


def _widen32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << _U32(16)).view(np.float32)


# ---------------------------------------------------------------- dropout parameters
def check_p(p_drop) -> np.float32:
    p = np.float32(p_drop)
    if not np.isfinite(p) or p < 0 or p > 1:
        raise ValueError(f"dropout probability must be in [0, 1], got {p_drop!r}")
    return p


def drop_threshold(p_drop) -> int:
    """floor(p * 2^32) for the fp32 value p; exact (fp32 -> fp64 and * 2^32 are exact)."""
    p = check_p(p_drop)
    return int(math.floor(float(p) * _TWO32))


def keep_scale(p_drop) -> float:
    """1 / (1 - p) in fp64 for the fp32 value p (undefined, returned as 0, when p = 1)."""
    p = check_p(p_drop)
    return 0.0 if float(p) == 1.0 else 1.0 / (1.0 - float(p))


# ---------------------------------------------------------------- mask
def keep_elements(e, p_drop, seed, offset=0) -> np.ndarray:
    """Keep decision for linear output indices ``e`` (int64 array, e = m*N + n); ``offset``
    fills Philox counter words 2 and 3."""
    e = np.asarray(e, dtype=np.uint64)
    thr = drop_threshold(p_drop)
    if thr >= _TWO32:
        return np.zeros(e.shape, dtype=bool)
    g = e >> np.uint64(2)
    word = (e & np.uint64(3)).astype(np.intp)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    off = int(offset) & 0xFFFFFFFFFFFFFFFF
    blk = philox.blocks_np((g & np.uint64(0xFFFFFFFF)).astype(np.uint32).ravel(),
                           (g >> np.uint64(32)).astype(np.uint32).ravel(),
                           off & 0xFFFFFFFF, off >> 32, seed & 0xFFFFFFFF, seed >> 32)
    r = blk[np.arange(blk.shape[0]), word.ravel()].reshape(e.shape)
    return r.astype(np.int64) >= thr


def keep_mask(M, N, p_drop, seed, rows=None, offset=0) -> np.ndarray:
    """Keep mask of the [M, N] output (or of the listed rows only), bool; ``offset`` fills
    Philox counter words 2 and 3."""
    thr = drop_threshold(p_drop)
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    if thr >= _TWO32:
        return np.zeros((rows.size, N), dtype=bool)
    if rows.size == M and np.array_equal(rows, np.arange(M)) and (M * N) % 4 == 0:
        # whole output: one block per group of four consecutive linear indices
        G = (M * N) // 4
        g = np.arange(G, dtype=np.uint64)
        seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        off = int(offset) & 0xFFFFFFFFFFFFFFFF
        blk = philox.blocks_np((g & np.uint64(0xFFFFFFFF)).astype(np.uint32),
                               (g >> np.uint64(32)).astype(np.uint32),
                               off & 0xFFFFFFFF, off >> 32, seed & 0xFFFFFFFF, seed >> 32)
        return (blk.reshape(M, N).astype(np.int64) >= thr)
    e = rows[:, None].astype(np.int64) * N + np.arange(N, dtype=np.int64)[None, :]
    return keep_elements(e, p_drop, seed, offset)


# ---------------------------------------------------------------- the block
def slice_bounds(K, P):
    if P < 1 or K % P != 0:
        raise ValueError(f"P={P} must divide K={K}")
    Ks = K // P
    return [(p * Ks, (p + 1) * Ks) for p in range(P)]


def slice_partials(X_bits, W_bits, P, rows=None, cols=None):
    """Yield S_p = X[rows, K_p] . W[K_p, cols] in fp64 for p = 0 .. P-1 (numpy dgemm)."""
    X_bits = np.asarray(X_bits)
    W_bits = np.asarray(W_bits)
    K = X_bits.shape[1]
    if W_bits.shape[0] != K:
        raise ValueError("X is [M,K] and W is [K,N]")
    for k0, k1 in slice_bounds(K, P):
        Xp = X_bits[:, k0:k1] if rows is None else X_bits[rows, k0:k1]
        Wp = W_bits[k0:k1, :] if cols is None else W_bits[k0:k1][:, cols]
        yield widen(Xp) @ widen(Wp)


def run(X, W, bias, residual, P, p_drop, seed, rows=None, cols=None, offset=0):
    """The block in fp64.  Returns (out [M,N] fp64, keep [M,N] bool).  ``offset``: Philox
    counter words 2 and 3 of the mask.

    ``rows`` / ``cols`` restrict the computation to a sub-grid of the output (every
    output element depends only on its own row of X and column of W); the mask still
    uses the element's index in the full [M, N] output.
    """
    X = np.asarray(X)
    W = np.asarray(W)
    M, N = X.shape[0], W.shape[1]
    T = None
    for Sp in slice_partials(X, W, P, rows, cols):
        T = Sp if T is None else T + Sp          # left to right, starting from S_0
    b = widen(bias) if cols is None else widen(np.asarray(bias)[cols])
    v = T + b[None, :]
    rr = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    cc = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    if cols is None:
        keep = keep_mask(M, N, p_drop, seed, rows=None if rows is None else rr, offset=offset)
    else:
        e = rr[:, None] * N + cc[None, :]
        keep = keep_elements(e, p_drop, seed, offset)
    res = np.asarray(residual)
    res = res if rows is None else res[rr]
    res = res if cols is None else res[:, cc]
    out = widen(res) + np.where(keep, v * keep_scale(p_drop), 0.0)
    return out, keep


def error_bound_fp32(X, W, bias, residual, P, p_drop, keep, rows=None, cols=None):
    """Per-element bound on |out_fp32 - out| for an fp32 computation of the block (slice
    sums accumulated in fp32 from zero, reduced in fp32, fp32 epilogue), for the bf16
    output variant: there the fp32 result is rounded once more, to bf16, and an element
    may round either way only if out lies within this bound of a bf16 rounding midpoint.

    With u = 2^-24 and mag = |X| . |W| + |bias| (fp64): 64 u scale mag (the summation
    error, generous: an fp32 sum of n terms errs by about u sqrt(n) times its terms'
    typical size, far below u times the sum of their magnitudes), plus 4 u (|v scale| +
    |out|) for the bias add, the scale multiply and the residual add.  A dropped element
    is the residual exactly (bound 0).  Parity unpinned beyond the fp32 simulations of the
    tests: the pages fix no precision for the summation inside a slice."""
    X = np.asarray(X)
    W = np.asarray(W)
    Xr = X if rows is None else X[np.asarray(rows)]
    Wc = W if cols is None else W[:, np.asarray(cols)]
    b = widen(bias) if cols is None else widen(np.asarray(bias)[cols])
    res = np.asarray(residual)
    res = res if rows is None else res[np.asarray(rows)]
    res = res if cols is None else res[:, np.asarray(cols)]
    scale = keep_scale(p_drop)
    mag = np.abs(widen(Xr)) @ np.abs(widen(Wc)) + np.abs(b)[None, :]
    v = None
    for Sp in slice_partials(Xr, Wc, P):
        v = Sp if v is None else v + Sp
    v = (v + b[None, :]) * scale
    out = widen(res) + v
    u = 2.0 ** -24
    bound = 64.0 * u * scale * mag + 4.0 * u * (np.abs(v) + np.abs(out))
    return np.where(keep, bound, 0.0)


def run_inputs(inp, rows=None, cols=None):
    """``run`` on a dict with keys X, W, bias, residual, P, p_drop, seed (and optionally
    offset)."""
    return run(inp["X"], inp["W"], inp["bias"], inp["residual"], inp["P"], inp["p_drop"],
               inp["seed"], rows=rows, cols=cols, offset=inp.get("offset", 0))


# ---------------------------------------------------------------- fp32 order model
def reduce_epilogue_fp32(partials, bias, residual, keep, p_drop) -> np.ndarray:
    """fp32 model of the declared rounding order, for partials that fp32 holds exactly.

    ``partials`` is a sequence of P fp64 arrays [M, N] whose values are exactly
    representable in fp32 (checked).  T = S_0; T = fl32(T + S_p) for p = 1 .. P-1;
    v = fl32(T + bias); kept: out = fl32(residual + fl32(v * scale32)) with
    scale32 = fl32(1 / (1 - p)); dropped: out = residual.
    """
    T = None
    for Sp in partials:
        S32 = np.asarray(Sp, dtype=np.float64).astype(np.float32)
        if not np.array_equal(S32.astype(np.float64), np.asarray(Sp, dtype=np.float64)):
            raise ValueError("partials must be exactly representable in fp32")
        T = S32 if T is None else (T + S32).astype(np.float32)
    v = (T + _widen32(bias)[None, :]).astype(np.float32)
    scale32 = np.float32(keep_scale(p_drop))
    res32 = _widen32(residual)
    kept = (res32 + (v * scale32).astype(np.float32)).astype(np.float32)
    return np.where(keep, kept, res32).astype(np.float32)
