"""The no-allocation entry point (mmar_fused_noalloc, static per-device workspace) against
mmar_fused_ex with the same plan: bit-identical outputs on two calls in a row, the second
on a smaller input, for each plan kind that uses the workspace; the oracle bounds the
first call's output; over-capacity plans and the streams schedule are refused."""
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

# (schedule, tile, w_mode, chunk rows or 0, first shape (M, K, N, P), second (smaller) shape)
CASES = [
    ("sequential", "auto", "direct", 128, (1024, 1536, 768, 4), (256, 512, 384, 2)),
    ("persistent", "256x192", "pretranspose", 0, (1024, 2048, 1536, 8), (512, 1024, 384, 4)),
    ("persistent", "256x128", "pretranspose", 0, (768, 1024, 640, 4), (256, 256, 256, 1)),
    ("balanced", "256x128", "direct", 0, (2080, 512, 8192, 4), (2080, 512, 4096, 4)),
    # the split schedule needs workspace only for the pre-transposed weight; its first
    # shape has a tail (288 tiles on 256 CUs), its second none
    ("split", "256x128", "pretranspose", 0, (2080, 512, 4096, 4), (1056, 256, 1024, 2)),
]


def _dev(inp):
    return {k: dev(inp[k], torch) for k in ("X", "W", "bias", "residual")}


@pytest.mark.parametrize("sched,tile,wm,crows,shape1,shape2", CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}" for c in CASES])
def test_noalloc_matches_fused_ex_two_calls(sched, tile, wm, crows, shape1, shape2):
    cap = mmar.noalloc_workspace_capacity()
    assert cap == 64 << 20
    for i, (M, K, N, P) in enumerate((shape1, shape2)):
        print("noalloc", sched, tile, wm, (M, K, N, P), flush=True)
        chunk = (crows, N) if crows else (0, 0)
        need = mmar.workspace_bytes(sched, M, N, K, P, chunk=chunk, w_mode=wm, tile=tile)
        assert 0 < need <= cap, need
        inp = make_random_inputs(M, K, N, seed=100 * i + M + N + P)
        d = _dev(inp)
        seed = 7 + i
        ref = mmar.fused_ex(d["X"], d["W"], d["bias"], d["residual"], P, 0.1, seed, sched,
                            chunk=chunk, w_mode=wm, tile=tile)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        mmar.fused_noalloc(d["X"], d["W"], d["bias"], d["residual"], P, 0.1, seed, sched,
                           chunk=chunk, w_mode=wm, tile=tile, out=out)
        torch.cuda.synchronize()
        got = host(out)
        assert np.array_equal(f32_bits(got), f32_bits(host(ref))), (sched, (M, K, N, P))
        if i == 0:
            inp.update(M=M, K=K, N=N, P=P, p_drop=np.float32(0.1), seed=seed)
            ora, _ = oracle.run_inputs(inp)
            assert_within_tol(got, ora, "noalloc vs oracle")


def test_noalloc_refuses_what_it_cannot_run():
    M, K, N, P = 8192, 12288, 3072, 16
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((N,), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    # the pre-transposed weight alone is 72 MiB, over the 64 MiB capacity
    with pytest.raises(mmar.MmarError) as e:
        mmar.fused_noalloc(X, W, b, r, P, 0.1, 1, "persistent", w_mode="pretranspose", out=out)
    assert e.value.code == mmar.ENOMEM and "static workspace" in str(e.value)
    with pytest.raises(mmar.MmarError) as e:
        mmar.fused_noalloc(X, W, b, r, P, 0.1, 1, "streams", chunk=(256, N), ring=2, out=out)
    assert e.value.code == mmar.EINVAL
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)      # nothing was launched
