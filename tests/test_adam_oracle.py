"""Pins of the fused reduce + Adam oracle (the data-parallel side, folded)."""
import numpy as np
import pytest

from oracle import adam

torch = pytest.importorskip("torch")

# hyperparameters that are exact fp32 values, so the fp32-taking oracle and PyTorch (fp64
# floats) see the same numbers
B1, B2, LR, EPS = 0.875, 1.0 - 2.0 ** -10, 2.0 ** -10, 2.0 ** -20


def _torch_steps(opt_cls, p0, grads_per_step, **kw):
    p = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = opt_cls([p], lr=LR, betas=(B1, B2), eps=EPS, **kw)
    for g in grads_per_step:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("wd", [0.0, 0.25])
def test_matches_torch_adam_over_several_steps(wd):
    """A library routine with the same definition: torch.optim.Adam (wd = 0) / AdamW."""
    rng = np.random.default_rng(0)
    n = 1000
    p0 = rng.standard_normal(n) * 0.02
    steps = [rng.standard_normal(n) * 1e-2 for _ in range(5)]
    opt_cls = torch.optim.AdamW if wd else torch.optim.Adam
    kw = {"weight_decay": wd} if wd else {}
    tp, tm, tv = _torch_steps(opt_cls, p0, steps, **kw)
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for t, g in enumerate(steps, start=1):
        p, m, v, _ = adam.adam_step(g[None, :], p, m, v, t, LR, B1, B2, EPS, wd)
    np.testing.assert_allclose(p, tp, rtol=0, atol=1e-15)
    # torch forms m by interpolation (m + (1 - b1)(g - m)): equal up to fp64 rounding
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-18)


def test_constant_gradient_closed_form():
    """With a constant gradient c from zero moments, the bias-corrected moments are c and
    c^2 at every step, so each step moves p by lr * c / (|c| + eps)."""
    c = np.array([1e-3, -2.0, 0.5, -1e-6])
    p0 = np.array([0.1, -0.2, 0.3, 0.0])
    p, m, v = p0, np.zeros(4), np.zeros(4)
    T = 7
    for t in range(1, T + 1):
        p, m, v, _ = adam.adam_step(c[None, :], p, m, v, t, LR, B1, B2, EPS)
    np.testing.assert_allclose(p, p0 - T * LR * c / (np.abs(c) + EPS), rtol=0, atol=1e-14)


def test_replicas_are_averaged_in_order():
    rng = np.random.default_rng(1)
    G = rng.standard_normal((6, 64))
    p0, m0, v0 = rng.standard_normal(64), rng.standard_normal(64) * 1e-3, rng.random(64) * 1e-6
    a = adam.adam_step(G, p0, m0, v0, 3, LR, B1, B2, EPS)
    b = adam.adam_step(G.mean(axis=0)[None, :], p0, m0, v0, 3, LR, B1, B2, EPS)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-17)


def test_weight_decay_alone():
    p0 = np.array([1.0, -2.0, 0.5])
    p, m, v, _ = adam.adam_step(np.zeros((2, 3)), p0, np.zeros(3), np.zeros(3), 1, LR, B1, B2,
                                EPS, 0.25)
    np.testing.assert_array_equal(m, 0)
    np.testing.assert_array_equal(v, 0)
    np.testing.assert_allclose(p, p0 * (1 - LR * 0.25), rtol=0, atol=1e-16)


def test_bf16_copy_is_the_rounded_parameter():
    rng = np.random.default_rng(2)
    p, _, _, bits = adam.adam_step(rng.standard_normal((2, 100)), rng.standard_normal(100),
                                   np.zeros(100), np.zeros(100), 1, LR, B1, B2, EPS)
    ref = torch.from_numpy(p.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    # equal except where the fp32 step double-rounds (never for these values)
    assert np.array_equal(bits, ref.view(np.uint16))


def test_bad_arguments():
    with pytest.raises(ValueError):
        adam.adam_step(np.zeros(3), np.zeros(3), np.zeros(3), np.zeros(3), 1, LR)
    with pytest.raises(ValueError):
        adam.adam_step(np.zeros((1, 3)), np.zeros(3), np.zeros(3), np.zeros(3), 0, LR)
