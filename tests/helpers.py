"""Shared helpers for the GPU tests: device transfer and the output tolerance."""
import numpy as np

TOL = 2e-3      # |gpu - oracle| <= TOL * max(1, |oracle|) on the fp32 output


def dev(bits, torch):
    """uint16 bf16 bit patterns (numpy) -> bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def host(t):
    return t.detach().cpu().numpy()


def assert_within_tol(gpu, ora, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ora)
    bound = TOL * np.maximum(1.0, np.abs(ora))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside tolerance; worst at {i}: "
                             f"gpu={gpu[i]!r} oracle={ora[i]!r}")
    return float((err / np.maximum(1.0, np.abs(ora))).max())


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
