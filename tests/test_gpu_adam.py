"""GPU parity of the fused gradient-average + Adam step (mmar_adam_step) against the
fp64 oracle, through the C ABI.

Bar: parameters within 2e-6 relative (+ 1e-9 + 1e-5 lr per step absolute), moments within 1e-5 relative (+ an
absolute floor of a few fp32 units of their terms) after each step of an independent run of both sides from the same
seeded state; the bf16 parameter copy correctly rounded except near a rounding midpoint.
"""
import numpy as np
import pytest

from oracle import adam as oadam
from oracle import producer
from workload import ADAM_WORKLOADS, make_adam_inputs
from helpers import host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import chunked_matmul_reduce_amd as mmar  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _dev(inp):
    return {k: torch.from_numpy(inp[k]).to("cuda") for k in ("grads", "param", "m", "v")}


def _compare(d, pb, p, m, v, bits, lr, steps):
    gp, gm, gv = host(d["param"]), host(d["m"]), host(d["v"])
    # the normalized update m^/(sqrt(v^)+eps) is O(1) with an fp32 error up to ~1e-5 where
    # the moment update cancels; each step moves p by lr times it
    np.testing.assert_allclose(gp, p, rtol=2e-6, atol=1e-9 + 1e-5 * lr * steps)
    # absolute floors: a few fp32 units of the terms summed (m ~ 1e-3, v ~ 1e-6), which
    # matter where the two terms of the moment update cancel
    np.testing.assert_allclose(gm, m, rtol=1e-5, atol=1e-9)
    np.testing.assert_allclose(gv, v, rtol=1e-5, atol=1e-12)
    gb = host(pb.view(torch.int16)).view(np.uint16)
    bound = 2.0 ** -20 * np.abs(p) + 1e-9
    producer.check_bf16_output(gb, p, bound)


@pytest.mark.parametrize("P", [1, 3, 8])
@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_steps_against_oracle(P, wd):
    n = 4096 + 4 * P
    inp = make_adam_inputs(n, P, seed=40 + P)
    d = _dev(inp)
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    p, m, v = inp["param"], inp["m"], inp["v"]
    for t in range(1, 5):
        mmar.adam_step(d["grads"], d["param"], d["m"], d["v"], t, weight_decay=wd, param_bf16=pb,
                       **HP)
        torch.cuda.synchronize()
        p, m, v, bits = oadam.adam_step(inp["grads"], p, m, v, t, HP["lr"], HP["beta1"],
                                        HP["beta2"], HP["eps"], wd)
        _compare(d, pb, p, m, v, bits, HP["lr"], t)


def test_16m_parameters_one_step():
    w = ADAM_WORKLOADS["adam_16m"]
    inp = make_adam_inputs(w.n, w.P, w.seed)
    d = _dev(inp)
    pb = torch.empty(w.n, dtype=torch.bfloat16, device="cuda")
    mmar.adam_step(d["grads"], d["param"], d["m"], d["v"], w.step, w.lr, w.beta1, w.beta2, w.eps,
                   w.weight_decay, param_bf16=pb)
    torch.cuda.synchronize()
    p, m, v, bits = oadam.adam_step(inp["grads"], inp["param"], inp["m"], inp["v"], w.step, w.lr,
                                    w.beta1, w.beta2, w.eps, w.weight_decay)
    _compare(d, pb, p, m, v, bits, w.lr, 1)


def test_without_bf16_copy_and_bad_arguments():
    inp = make_adam_inputs(256, 2, seed=9)
    d = _dev(inp)
    mmar.adam_step(d["grads"], d["param"], d["m"], d["v"], 1, **HP)
    torch.cuda.synchronize()
    p, _, _, _ = oadam.adam_step(inp["grads"], inp["param"], inp["m"], inp["v"], 1, HP["lr"],
                                 HP["beta1"], HP["beta2"], HP["eps"])
    np.testing.assert_allclose(host(d["param"]), p, rtol=2e-6, atol=1e-9 + 1e-5 * HP["lr"])
    before = host(d["param"]).copy()
    with pytest.raises(mmar.MmarError):
        mmar.adam_step(d["grads"], d["param"], d["m"], d["v"], 0, **HP)          # step 0
    with pytest.raises(mmar.MmarError):
        mmar.adam_step(d["grads"], d["param"], d["m"], d["v"], 1, lr=1e-3, beta1=1.0)
    with pytest.raises(mmar.MmarError):
        mmar.adam_step(d["grads"], d["param"], d["param"], d["v"], 1, **HP)      # overlap
    torch.cuda.synchronize()
    assert np.array_equal(host(d["param"]), before)
