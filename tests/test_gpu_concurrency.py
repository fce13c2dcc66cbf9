"""Two host threads, each on its own stream with its own workspace, running the two-stream
schedule at once: the library's side stream and events are shared per device, so the
calls must not see each other's event records (every output bit-identical to the
single-threaded run)."""
import threading

import numpy as np
import pytest

from workload import make_random_inputs
from helpers import dev, f32_bits, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import chunked_matmul_reduce_amd as mmar  # noqa: E402


def test_streams_schedule_two_threads_own_workspaces():
    M, K, N, P = 1024, 1536, 768, 4
    chunk, ring = (128, N), 2
    cases = []
    for seed in (21, 22):
        inp = make_random_inputs(M, K, N, seed=seed)
        d = {k: dev(inp[k], torch) for k in ("X", "W", "bias", "residual")}
        ref = mmar.fused_ex(d["X"], d["W"], d["bias"], d["residual"], P, 0.1, seed, "persistent")
        torch.cuda.synchronize()
        cases.append((d, seed, f32_bits(host(ref))))
    nbytes = mmar.workspace_bytes("streams", M, N, K, P, chunk=chunk, ring=ring)
    reps = 20
    results = [[None] * reps for _ in cases]
    errors = []

    def worker(i):
        try:
            d, seed, _ = cases[i]
            s = torch.cuda.Stream()
            ws = torch.empty((nbytes // 4,), dtype=torch.float32, device="cuda")
            outs = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(reps)]
            with torch.cuda.stream(s):
                for r in range(reps):
                    mmar.fused_ex(d["X"], d["W"], d["bias"], d["residual"], P, 0.1, seed, "streams",
                                  chunk=chunk, ring=ring, workspace=ws, out=outs[r], stream=s)
            s.synchronize()
            for r in range(reps):
                results[i][r] = f32_bits(host(outs[r]))
        except Exception as e:  # reported by the main thread
            errors.append(e)

    print("two threads x", reps, "calls of the streams schedule", flush=True)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i, (_, _, ref) in enumerate(cases):
        for r in range(reps):
            assert np.array_equal(results[i][r], ref), (i, r)
