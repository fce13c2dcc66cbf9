"""GPU parity of the producer MatMul (H = GeLU(X . W1 + b1), or H = X . W + b with no
activation for an attention block's QKV projection, bf16) and of the MLP built from it
and the block, through the C ABI, against the oracle.

Bar for the bf16 H: every element equals the fp64 value rounded to bf16, except near a
rounding midpoint (within the fp32 error bound), where either neighbour is accepted.
"""
import numpy as np
import pytest

import oracle
from oracle import producer
from workload import WORKLOADS, make_inputs, make_producer_inputs, make_qkv_inputs, make_random_inputs
from helpers import assert_within_tol, dev, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import chunked_matmul_reduce_amd as mmar  # noqa: E402


def _h_bits(H):
    return host(H.view(torch.int16)).view(np.uint16)


SHAPES = [(64, 256, 256), (288, 480, 160), (1056, 2048, 544), (32, 4096, 4096), (256, 96, 128)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_producer_against_oracle(M, K, N):
    print("producer", M, K, N, flush=True)
    inp = make_random_inputs(M, K, N, seed=M * 3 + N)
    X, W, b = (dev(inp[k], torch) for k in ("X", "W", "bias"))
    H = mmar.gelu_linear(X, W, b)
    torch.cuda.synchronize()
    h, _, bound = producer.producer(inp["X"], inp["W"], inp["bias"])
    ties = producer.check_bf16_output(_h_bits(H), h, bound)
    # the bound is generous, so many elements count as near ties; the rest must match
    # exactly, and a wrong column, bias or GeLU would miss the bound almost everywhere
    print("near-tie fraction", ties / (M * N), flush=True)
    assert ties < 0.7 * M * N


def _check_producer_all_rows(hb, X, W, b, activation="gelu_tanh", block=2048):
    """Every row of a bf16 producer output against the oracle, a block of rows at a time
    (bounded host memory)."""
    ties = 0
    for r0 in range(0, hb.shape[0], block):
        rows = np.arange(r0, min(hb.shape[0], r0 + block))
        h, _, bound = producer.producer(X, W, b, rows=rows, activation=activation)
        ties += producer.check_bf16_output(hb[rows], h, bound)
    return ties


def test_producer_full_size_all_rows():
    """The GPT-2 MLP block's first layer: [8192, 3072] x [3072, 12288], every element."""
    w = WORKLOADS["gpt2_mlp"]
    pin = make_producer_inputs(w)
    X0, W1, b1 = (dev(pin[k], torch) for k in ("X0", "W1", "b1"))
    H = mmar.gelu_linear(X0, W1, b1)
    torch.cuda.synchronize()
    print("producer full size: oracle over all rows", flush=True)
    _check_producer_all_rows(_h_bits(H), pin["X0"], pin["W1"], pin["b1"])


def test_mlp_tiny_against_oracle_and_bits_of_parts():
    """mlp = gelu_linear then fused: out equals the block's oracle on the GPU's H, and
    H equals the producer oracle (near-tie rule)."""
    M, D, F, P = 64, 256, 512, 4                 # hidden D, MLP width F = K of the block
    rng = np.random.default_rng(11)
    a = make_random_inputs(M, D, F, seed=21)     # X0 [M, D], W1 [D, F], b1 [F]
    c = make_random_inputs(M, F, D, seed=22)     # W2 [F, D], b2 [D], residual [M, D]
    X0, W1, b1 = (dev(a[k], torch) for k in ("X", "W", "bias"))
    W2, b2, R = (dev(c[k], torch) for k in ("W", "bias", "residual"))
    p, seed = np.float32(0.1), int(rng.integers(1 << 40))
    out, H = mmar.mlp(X0, W1, b1, W2, b2, R, P, p, seed)
    torch.cuda.synchronize()
    hb = _h_bits(H)
    h, _, bound = producer.producer(a["X"], a["W"], a["bias"])
    producer.check_bf16_output(hb, h, bound)
    ora, keep = oracle.run(hb, c["W"], c["bias"], c["residual"], P, p, seed)
    assert_within_tol(host(out), ora)
    out2 = mmar.fused(H, W2, b2, R, P, p, seed)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), host(out2).view(np.uint32))


@pytest.mark.parametrize("chunk", [0, 32, 64, 128])
def test_mlp_chunked_tiny_bits_and_oracle(chunk):
    """mmar_mlp (producer and block in one call; with row chunks, the block of chunk c on a
    second stream beside the producer of chunk c + 1) gives mlp()'s bits for H and out,
    and both match the oracles."""
    M, D, F, P = 256, 256, 512, 4
    a = make_random_inputs(M, D, F, seed=31)
    c = make_random_inputs(M, F, D, seed=32)
    X0, W1, b1 = (dev(a[k], torch) for k in ("X", "W", "bias"))
    W2, b2, R = (dev(c[k], torch) for k in ("W", "bias", "residual"))
    p, seed = np.float32(0.1), 12345
    out_ref, H_ref = mmar.mlp(X0, W1, b1, W2, b2, R, P, p, seed)
    out, H = mmar.mlp_chunked(X0, W1, b1, W2, b2, R, P, p, seed, chunk_m=chunk)
    torch.cuda.synchronize()
    assert np.array_equal(_h_bits(H), _h_bits(H_ref))
    assert np.array_equal(host(out).view(np.uint32), host(out_ref).view(np.uint32))
    hb = _h_bits(H)
    h, _, bound = producer.producer(a["X"], a["W"], a["bias"])
    producer.check_bf16_output(hb, h, bound)
    ora, _ = oracle.run(hb, c["W"], c["bias"], c["residual"], P, p, seed)
    assert_within_tol(host(out), ora)


def test_mlp_chunked_full_size_gpt2():
    """The GPT-2 8.3B MLP (first layer [8192, 3072] x [3072, 12288] + GeLU, then the block,
    P = 16): the chunked pipeline at several row chunks gives the bits of the two calls in
    turn; H against the producer oracle and out against the block oracle on every element."""
    w = WORKLOADS["gpt2_mlp"]
    pin = make_producer_inputs(w)
    inp = make_inputs(w)
    X0, W1, b1 = (dev(pin[k], torch) for k in ("X0", "W1", "b1"))
    W2, b2, R = (dev(inp[k], torch) for k in ("W", "bias", "residual"))
    p, seed = inp["p_drop"], w.seed
    out_ref, H_ref = mmar.mlp(X0, W1, b1, W2, b2, R, w.P, p, seed)
    torch.cuda.synchronize()
    ref_out, ref_h = host(out_ref).view(np.uint32).copy(), _h_bits(H_ref).copy()
    for chunk in (0, 1024, 2048):
        print("mlp chunked", chunk, flush=True)
        out, H = mmar.mlp_chunked(X0, W1, b1, W2, b2, R, w.P, p, seed, chunk_m=chunk,
                                  out=out_ref, hidden=H_ref)
        torch.cuda.synchronize()
        assert np.array_equal(_h_bits(H), ref_h), chunk
        assert np.array_equal(host(out).view(np.uint32), ref_out), chunk
    del X0, W1, b1, W2, b2, R
    torch.cuda.empty_cache()
    print("mlp full size: producer oracle over all rows", flush=True)
    _check_producer_all_rows(ref_h, pin["X0"], pin["W1"], pin["b1"])
    print("mlp full size: block oracle over all rows", flush=True)
    ora, _ = oracle.run(ref_h, inp["W"], inp["bias"], inp["residual"], w.P, p, seed)
    assert_within_tol(ref_out.view(np.float32), ora)


def test_mlp_chunked_rejects_bad_arguments():
    X = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros((256, 512), dtype=torch.bfloat16, device="cuda")
    b1 = torch.zeros((512,), dtype=torch.bfloat16, device="cuda")
    W2 = torch.zeros((512, 256), dtype=torch.bfloat16, device="cuda")
    b2 = torch.zeros((256,), dtype=torch.bfloat16, device="cuda")
    R = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mmar.MmarError):
        mmar.mlp_chunked(X, W1, b1, W2, b2, R, 4, 0.1, 1, chunk_m=48)   # not a multiple of 32
    with pytest.raises(mmar.MmarError):
        mmar.mlp_chunked(X, W1, b1, W2, b2, R, 3, 0.1, 1)                # P does not divide K
    H = torch.empty((64, 512), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((64, 256), dtype=torch.float32, device="cuda")
    rc = mmar.lib.mmar_mlp(X.data_ptr(), W1.data_ptr(), b1.data_ptr(), W2.data_ptr(), b2.data_ptr(),
                           R.data_ptr(), X.data_ptr(), out.data_ptr(), 64, 256, 512, 256, 4, 0.1, 1,
                           0, None)
    assert rc == mmar.EINVAL                                           # H overlaps X0


def test_producer_rejects_bad_arguments():
    X = torch.zeros((64, 250), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((250, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((64,), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mmar.MmarError):
        mmar.gelu_linear(X, W, b)                 # K not a multiple of 32
    X = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    H = torch.empty((64, 64), dtype=torch.bfloat16, device="cuda")
    assert mmar.lib.mmar_gelu_linear(X.data_ptr(), W.data_ptr(), b.data_ptr(), X.data_ptr(),
                                     64, 64, 256, None) == mmar.EINVAL   # H overlaps X
    mmar.gelu_linear(X, W, b, out=H)
    torch.cuda.synchronize()
    assert np.all(_h_bits(H) == 0)                # gelu(0) = 0


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_linear_without_activation_against_oracle(M, K, N):
    print("linear none", M, K, N, flush=True)
    inp = make_random_inputs(M, K, N, seed=M * 5 + N)
    X, W, b = (dev(inp[k], torch) for k in ("X", "W", "bias"))
    H = mmar.linear(X, W, b, "none")
    torch.cuda.synchronize()
    h, _, bound = producer.producer(inp["X"], inp["W"], inp["bias"], activation="none")
    ties = producer.check_bf16_output(_h_bits(H), h, bound)
    print("near-tie fraction", ties / (M * N), flush=True)
    assert ties < 0.7 * M * N
    # the GeLU mode of the same entry point gives gelu_linear's bits
    Hg = mmar.linear(X, W, b, "gelu_tanh")
    Hg2 = mmar.gelu_linear(X, W, b)
    torch.cuda.synchronize()
    assert np.array_equal(_h_bits(Hg), _h_bits(Hg2))


def test_linear_qkv_full_size_all_rows():
    """The GPT-2 attention block's QKV projection: [8192, 3072] x [3072, 9216], bias, no
    activation; every element."""
    w = WORKLOADS["gpt2_attn"]
    pin = make_qkv_inputs(w)
    X0, Wq, bq = (dev(pin[k], torch) for k in ("X0", "Wqkv", "bqkv"))
    H = mmar.linear(X0, Wq, bq, "none")
    torch.cuda.synchronize()
    print("qkv full size: oracle over all rows", flush=True)
    _check_producer_all_rows(_h_bits(H), pin["X0"], pin["Wqkv"], pin["bqkv"], activation="none")


def test_linear_rejects_an_unknown_activation():
    X = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.ones((64,), dtype=torch.bfloat16, device="cuda")
    H = torch.full((64, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mmar.linear(X, W, b, "relu")
    assert mmar.lib.mmar_linear(X.data_ptr(), W.data_ptr(), b.data_ptr(), H.data_ptr(),
                                64, 64, 256, 5, None) == mmar.EINVAL
    torch.cuda.synchronize()
    assert np.all(host(H.float()) == 7.0)        # nothing was launched
    mmar.linear(X, W, b, "none", out=H)
    torch.cuda.synchronize()
    assert np.all(host(H.float()) == 1.0)        # 0 + bias


# The producer's two tile widths: 256 x 128, and 256 x 256 (one slice needs no running
# total, so a tile twice as wide fits the registers).  Shapes with ragged row and column
# tiles, K shorter than the copies' lead (3 steps of 32), and several tiles.
WIDE_SHAPES = [(64, 256, 256), (288, 480, 544), (1056, 2048, 544), (32, 4096, 4096),
               (256, 64, 512), (544, 1024, 2592)]


@pytest.mark.parametrize("act", ["gelu_tanh", "none"])
@pytest.mark.parametrize("M,K,N", WIDE_SHAPES)
def test_wide_tile_matches_narrow_bits_and_oracle(M, K, N, act, monkeypatch):
    print("producer tiles", M, K, N, act, flush=True)
    inp = make_random_inputs(M, K, N, seed=M * 7 + N + K)
    X, W, b = (dev(inp[k], torch) for k in ("X", "W", "bias"))
    monkeypatch.setenv("MMAR_LINEAR_TILE", "256")
    Hw = mmar.linear(X, W, b, act)
    monkeypatch.setenv("MMAR_LINEAR_TILE", "128")
    Hn = mmar.linear(X, W, b, act)
    torch.cuda.synchronize()
    assert np.array_equal(_h_bits(Hw), _h_bits(Hn))
    h, _, bound = producer.producer(inp["X"], inp["W"], inp["bias"], activation=act)
    ties = producer.check_bf16_output(_h_bits(Hw), h, bound)
    assert ties < 0.7 * M * N


def test_wide_tile_full_size_gelu_layer_bits(monkeypatch):
    """The GPT-2 MLP block's first layer on both tile widths: identical bits."""
    w = WORKLOADS["gpt2_mlp"]
    pin = make_producer_inputs(w)
    X0, W1, b1 = (dev(pin[k], torch) for k in ("X0", "W1", "b1"))
    monkeypatch.setenv("MMAR_LINEAR_TILE", "256")
    Hw = mmar.gelu_linear(X0, W1, b1)
    monkeypatch.setenv("MMAR_LINEAR_TILE", "128")
    Hn = mmar.gelu_linear(X0, W1, b1)
    torch.cuda.synchronize()
    assert torch.equal(Hw.view(torch.int16), Hn.view(torch.int16))


@pytest.mark.parametrize("name", ["bert_mlp", "gpt3_mlp"])
def test_wide_tile_full_size_other_mlp_layers(name, monkeypatch):
    """The first MLP layers of the BERT- and GPT-3-shaped blocks ([8192, 2560] x [2560,
    10240] and [2048, 12288] x [12288, 49152]), which the tile choice runs on 256 x 256
    tiles: bits equal to the 256 x 128 tile on every element, and sampled rows against the
    oracle.  Inputs drawn on the device with the workloads' distributions (bf16)."""
    w = WORKLOADS[name]
    M, K, N = w.M, w.N, w.K            # the producer maps [M, N] to [M, K] of the block
    print("wide producer", name, M, K, N, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 300)
    X0 = torch.randn((M, K), generator=g, device="cuda").mul_(w.sigma_x).to(torch.bfloat16)
    W1 = torch.randn((K, N), generator=g, device="cuda").mul_(w.sigma_w).to(torch.bfloat16)
    b1 = torch.randn((N,), generator=g, device="cuda").mul_(w.sigma_bias).to(torch.bfloat16)
    monkeypatch.delenv("MMAR_LINEAR_TILE", raising=False)
    Ha = mmar.gelu_linear(X0, W1, b1)            # the library's own choice
    monkeypatch.setenv("MMAR_LINEAR_TILE", "256")
    Hw = mmar.gelu_linear(X0, W1, b1)
    monkeypatch.setenv("MMAR_LINEAR_TILE", "128")
    Hn = mmar.gelu_linear(X0, W1, b1)
    torch.cuda.synchronize()
    assert torch.equal(Hw.view(torch.int16), Hn.view(torch.int16))
    assert torch.equal(Ha.view(torch.int16), Hn.view(torch.int16))
    rows = np.array([0, 1, 255, 256, M // 2, M - 1])
    xb = host(X0[torch.as_tensor(rows, device="cuda")].view(torch.int16)).view(np.uint16)
    wb = host(W1.view(torch.int16)).view(np.uint16)
    bb = host(b1.view(torch.int16)).view(np.uint16)
    h, _, bound = producer.producer(xb, wb, bb)
    producer.check_bf16_output(_h_bits(Hw)[rows], h, bound)


@pytest.mark.parametrize("M,K,N", [(8192, 3072, 9216), (8192, 3072, 3072), (2080, 512, 1312)])
def test_column_split_between_tile_widths(M, K, N, monkeypatch):
    """Shapes whose columns the library splits between 256 x 256 and 256 x 128 tiles (the
    GPT-2 QKV projection; an attention-shaped layer) or not (a ragged one): the bits of
    the library's choice equal those of either tile width alone."""
    print("column split", M, K, N, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(M + K + N)
    X = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    W = torch.randn((K, N), generator=g, device="cuda").mul_(0.02).to(torch.bfloat16)
    b = torch.randn((N,), generator=g, device="cuda").mul_(0.02).to(torch.bfloat16)
    outs = {}
    for tile in ("auto", "256", "128"):
        if tile == "auto":
            monkeypatch.delenv("MMAR_LINEAR_TILE", raising=False)
        else:
            monkeypatch.setenv("MMAR_LINEAR_TILE", tile)
        for act in ("none", "gelu_tanh"):
            outs[(tile, act)] = mmar.linear(X, W, b, act)
    torch.cuda.synchronize()
    for act in ("none", "gelu_tanh"):
        ref = outs[("128", act)].view(torch.int16)
        assert torch.equal(outs[("auto", act)].view(torch.int16), ref), act
        assert torch.equal(outs[("256", act)].view(torch.int16), ref), act
