"""GPU parity of mmar_fused_strided: the block over row-strided views, with the dropout
mask's Philox counter words 2-3 set to a stream offset.

Bars as for the dense entry points: the mask bit-exact against the oracle (same offset),
fp32 output within 2e-3 * max(1, |oracle|), dropped elements equal to the residual bit
for bit; offset 0 over dense buffers reproduces mmar_fused's bits; nothing outside the
output view is written.
"""
import numpy as np
import pytest

import oracle
from workload import make_random_inputs
from helpers import assert_within_tol, dev, f32_bits, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import chunked_matmul_reduce_amd as mmar  # noqa: E402

SENTINEL = np.float32(-1234.5)


def _embed(bits, ld, col0):
    """A bf16 device view of ``bits`` [R, C] inside a zero buffer [R, ld] at column col0."""
    R, C = bits.shape
    big = np.zeros((R, ld), dtype=np.uint16)
    big[:, col0:col0 + C] = bits
    t = dev(big, torch)
    return t[:, col0:col0 + C], t


def _out_view(M, N, ldo, col0):
    big = torch.full((M, ldo), float(SENTINEL), dtype=torch.float32, device="cuda")
    return big[:, col0:col0 + N], big


def _strided_case(M, K, N, P, p, seed, offset, pads, plan=None):
    """Runs the strided entry on inputs embedded with the given (ld, col0) per operand and
    returns (inputs, out view on the host, whole out buffer on the host)."""
    inp = make_random_inputs(M, K, N, seed=seed)
    (ldx, cx), (ldw, cw), (ldr, cr), (ldo, co) = pads
    X, _ = _embed(inp["X"], ldx, cx)
    W, _ = _embed(inp["W"], ldw, cw)
    R, _ = _embed(inp["residual"], ldr, cr)
    b = dev(inp["bias"], torch)
    out, big = _out_view(M, N, ldo, co)
    assert X.stride() == (ldx, 1) and W.stride() == (ldw, 1) and out.stride() == (ldo, 1)
    if plan is not None:
        mmar.set_plan(M, N, K, P, "persistent", chunk=plan[0], w_mode="direct", tile=plan[1])
    try:
        mmar.fused_strided(X, W, b, R, P, p, seed, philox_offset=offset, out=out)
        torch.cuda.synchronize()
    finally:
        if plan is not None:
            mmar.set_plan(M, N, K, P, "auto")
    return inp, host(out), host(big)


def _check(inp, out, P, p, seed, offset):
    inp = dict(inp, P=P, p_drop=p, seed=seed, offset=offset)
    ora, keep = oracle.run_inputs(inp)
    assert_within_tol(out, ora, "strided")
    res32 = (inp["residual"].astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f32_bits(out[~keep]), f32_bits(res32[~keep]))
    return keep


# (ld, first column) of X, W, residual and out: rows padded past their length, views
# starting inside the row, all within the alignment the header asks for
PADS = [((768 + 40, 8), (416 + 24, 16), (416 + 12, 4), (416 + 8, 4)),
        ((768, 0), (416, 0), (416, 0), (416, 0))]


@pytest.mark.parametrize("offset", [0, 1, 0xFFFFFFFF00000001])
@pytest.mark.parametrize("pads", PADS)
def test_strided_views_against_oracle(pads, offset):
    # 544 x 416: two row tiles and a 32-row tail, three column tiles and a 32-column tail
    M, K, N, P, p, seed = 544, 768, 416, 4, 0.3, 11
    inp, out, big = _strided_case(M, K, N, P, p, seed, offset, pads)
    print(f"strided M={M} K={K} N={N} P={P} offset={offset} pads={pads}", flush=True)
    keep = _check(inp, out, P, p, seed, offset)
    assert np.array_equal(keep, oracle.keep_mask(M, N, p, seed, offset=offset))
    # the output's padding columns keep their sentinel
    ldo, co = pads[3]
    pad = np.ones(big.shape, dtype=bool)
    pad[:, co:co + N] = False
    assert np.all(big[pad] == SENTINEL)


@pytest.mark.parametrize("plan", [((0, 0), "256x192"), ((256, 384), "256x192"),
                                  ((256, 128), "256x128"), ((512, 192), "256x128")])
def test_strided_on_other_persistent_plans(plan):
    """The 256 x 192 tile and chunked persistent plans take the same leading dimensions."""
    M, K, N, P, p, seed, offset = 512, 512, 384, 2, 0.2, 5, 3
    inp, out, big = _strided_case(M, K, N, P, p, seed, offset, PADS[0][:2] + (
        (384 + 12, 4), (384 + 8, 4)), plan=plan)
    print(f"strided plan={plan}", flush=True)
    _check(inp, out, P, p, seed, offset)


def test_offset_zero_dense_matches_fused_bits():
    M, K, N, P, p, seed = 1024, 1536, 768, 6, 0.1, 2
    inp = make_random_inputs(M, K, N, seed=seed)
    d = {k: dev(inp[k], torch) for k in ("X", "W", "bias", "residual")}
    a = mmar.fused(d["X"], d["W"], d["bias"], d["residual"], P, p, seed)
    b = mmar.fused_strided(d["X"], d["W"], d["bias"], d["residual"], P, p, seed)
    c = mmar.fused_strided(d["X"], d["W"], d["bias"], d["residual"], P, p, seed, philox_offset=9)
    torch.cuda.synchronize()
    a, b, c = host(a), host(b), host(c)
    assert np.array_equal(f32_bits(a), f32_bits(b))
    # another offset: only the mask changes; elements kept under both offsets agree bitwise
    k0 = oracle.keep_mask(M, N, p, seed)
    k9 = oracle.keep_mask(M, N, p, seed, offset=9)
    assert np.array_equal(f32_bits(c[k0 & k9]), f32_bits(a[k0 & k9]))
    assert not np.array_equal(k0, k9)


def test_mask_readout_with_offset_is_exact():
    """X = 0, bias = 1, residual = 0: out is exactly 0 (dropped) or the scale (kept)."""
    M, K, N, P, p, seed, offset = 1024, 256, 1024, 2, 0.25, 0xFEEDFACE, 2 ** 63 + 5
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
    b = torch.ones((N,), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    out = host(mmar.fused_strided(X, W, b, r, P, p, seed, philox_offset=offset))
    scale = np.float32(1.0 / (1.0 - float(np.float32(p))))
    assert np.all((out == 0) | (out == scale))
    assert np.array_equal(out != 0, oracle.keep_mask(M, N, p, seed, offset=offset))
