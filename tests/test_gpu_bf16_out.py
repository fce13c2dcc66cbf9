"""GPU parity of the block's bf16 output variant (mmar_fused_bf16) through the C ABI.

Bars: every bf16 element equals the fp64 oracle rounded to bf16 (nearest even), except
where the fp64 value lies within the fp32 error bound (``oracle.error_bound_fp32``) of a
rounding midpoint, where a value within that bound plus half a bf16 spacing is accepted;
dropped elements equal the residual bit for bit; and the output equals the fp32 output
of mmar_fused on the same arguments rounded to bf16 (the documented relation between the
two entry points).
"""
import numpy as np
import pytest

import oracle
from oracle import producer
from workload import WORKLOADS, make_inputs, make_random_inputs
from helpers import dev, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import chunked_matmul_reduce_amd as mmar  # noqa: E402


def _bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


def _run_both(inp, P, p, seed):
    d = {k: dev(inp[k], torch) for k in ("X", "W", "bias", "residual")}
    ob = mmar.fused_bf16(d["X"], d["W"], d["bias"], d["residual"], P, p, seed)
    of = mmar.fused(d["X"], d["W"], d["bias"], d["residual"], P, p, seed)
    rounded = of.to(torch.bfloat16)          # fp32 -> bf16, nearest even
    torch.cuda.synchronize()
    return _bits(ob), _bits(rounded)


def _check(inp, P, p, seed, bits, rows=None):
    out, keep = oracle.run(inp["X"], inp["W"], inp["bias"], inp["residual"], P, p, seed,
                           rows=rows)
    bound = oracle.error_bound_fp32(inp["X"], inp["W"], inp["bias"], inp["residual"], P, p,
                                    keep, rows=rows)
    b = bits if rows is None else bits[rows]
    ties = producer.check_bf16_output(b, out, bound)
    res = inp["residual"] if rows is None else inp["residual"][rows]
    assert np.array_equal(b[~keep], res[~keep])
    return ties / out.size


# (M, K, N, P): tiny, ragged tiles with a 32-wide K step, several tiles, one slice
SHAPES = [(64, 256, 256, 4), (288, 480, 160, 5), (1056, 2048, 544, 8), (256, 96, 128, 1)]


@pytest.mark.parametrize("M,K,N,P", SHAPES)
def test_bf16_output_against_oracle(M, K, N, P):
    print("fused bf16", M, K, N, P, flush=True)
    inp = make_random_inputs(M, K, N, seed=M + K + N + P)
    p, seed = np.float32(0.1), 1234 + M
    bits, rounded = _run_both(inp, P, p, seed)
    assert np.array_equal(bits, rounded)
    frac = _check(inp, P, p, seed, bits)
    print("near-tie fraction", frac, flush=True)
    assert frac < 0.3


def test_bf16_output_edge_probabilities():
    inp = make_random_inputs(64, 256, 256, seed=9)
    for p in (np.float32(0.0), np.float32(1.0)):
        bits, rounded = _run_both(inp, 4, p, 77)
        assert np.array_equal(bits, rounded)
        _check(inp, 4, p, 77, bits)
    assert np.array_equal(bits, inp["residual"])        # p = 1: the residual, exactly


@pytest.mark.parametrize("name", ["gpt2_mlp"])
def test_bf16_output_full_size_all_rows(name):
    w = WORKLOADS[name]
    inp = make_inputs(name)
    bits, rounded = _run_both(inp, w.P, inp["p_drop"], w.seed)
    assert np.array_equal(bits, rounded)
    print(name, "bf16 output: oracle over all rows", flush=True)
    frac = _check(inp, w.P, inp["p_drop"], w.seed, bits)
    print(name, "near-tie fraction", frac, flush=True)
    torch.cuda.empty_cache()


def test_bf16_output_rejects_bad_arguments():
    X = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((64,), dtype=torch.bfloat16, device="cuda")
    R = torch.ones((64, 64), dtype=torch.bfloat16, device="cuda")
    O = torch.full((64, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    f = mmar.lib.mmar_fused_bf16
    assert f(X.data_ptr(), W.data_ptr(), b.data_ptr(), R.data_ptr(), R.data_ptr(),
             64, 64, 256, 4, 0.1, 1, None) == mmar.EINVAL          # out overlaps residual
    assert f(X.data_ptr(), W.data_ptr(), b.data_ptr(), R.data_ptr(), O.data_ptr(),
             64, 64, 250, 4, 0.1, 1, None) == mmar.EINVAL          # K not divisible
    assert f(X.data_ptr(), W.data_ptr(), b.data_ptr(), R.data_ptr(), O.data_ptr(),
             64, 64, 256, 4, 1.5, 1, None) == mmar.EINVAL          # p outside [0, 1]
    torch.cuda.synchronize()
    assert np.all(host(O.float()) == 3.0)                          # nothing was launched
