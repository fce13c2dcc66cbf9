"""The default (persistent) path under HIP graph capture: the call allocates nothing and
does not synchronize, so a serving loop can capture it once and replay it.  Every replay,
with eager work and synchronizations between replays, must give the eager result's bits.
"""
import numpy as np
import pytest

from workload import make_random_inputs
from helpers import dev, f32_bits, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import chunked_matmul_reduce_amd as mmar  # noqa: E402


@pytest.mark.parametrize("M,K,N,P", [(1024, 2048, 768, 8), (288, 480, 160, 5)])
def test_persistent_block_replays_from_a_graph(M, K, N, P):
    print("graph", M, K, N, P, flush=True)
    inp = make_random_inputs(M, K, N, seed=M + K + N)
    d = {k: dev(inp[k], torch) for k in ("X", "W", "bias", "residual")}
    args = (d["X"], d["W"], d["bias"], d["residual"], P, np.float32(0.1), 1234)
    plan = mmar.get_plan(M, N, K, P)            # one kernel, no workspace, no second stream
    assert plan["schedule"] == mmar.SCHED_PERSISTENT and plan["w_mode"] == mmar.W_DIRECT
    ref = mmar.fused(*args)                      # eager, also the first launch of the kernel
    torch.cuda.synchronize()
    ref_bits = f32_bits(host(ref))
    out = torch.full((M, N), float("nan"), device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                # warm-up on the capture stream
        mmar.fused(*args, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mmar.fused(*args, out=out)
    for rep in range(4):
        out.fill_(float("nan"))                  # eager work between replays
        junk = mmar.fused(d["X"], d["W"], d["bias"], d["residual"], P, np.float32(0.3), 99)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(f32_bits(host(out)), ref_bits), rep
        del junk
    # a second graph of the producer MatMul (no workspace either)
    H = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Href = mmar.gelu_linear(d["X"], d["W"], d["bias"])
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        mmar.gelu_linear(d["X"], d["W"], d["bias"], out=H)
    for rep in range(3):
        H.zero_()
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(H.view(torch.int16), Href.view(torch.int16)), rep
