"""Seeded synthetic inputs for the fused MatMul -> slice-reduce -> epilogue block.

This module draws the input tensors and nothing else: it holds none of the block's
arithmetic (no products, sums, dropout or Philox).  Both the CPU oracle (through the
tests) and the GPU path (through the tests and ``bench.py``) take their inputs from
here, so the two sides see identical bf16 bit patterns.

Workloads.  The pages measure the tensor-parallel MatMul followed by the AllReduce that
consumes it, on GPT-2 8.3B attention and MLP blocks, BERT 3.9B and a GPT-3 175B
segment (CoCoNet record, "Key takeaways", second to fourth bullets).  They print no
shapes, so the shapes below are those models' row-parallel projections at block level:

* ``tiny``      M=64,   K=256   (P=4,  K/P=64),   N=256    -- small oracle case
* ``gpt2_attn`` M=8192, K=3072  (P=16, K/P=192),  N=3072   -- GPT-2 8.3B attention out-proj
* ``gpt2_mlp``  M=8192, K=12288 (P=16, K/P=768),  N=3072   -- GPT-2 8.3B MLP down-proj
* ``bert_mlp``  M=8192, K=10240 (P=8,  K/P=1280), N=2560   -- BERT 3.9B MLP down-proj
* ``gpt3_mlp``  M=2048, K=49152 (P=8,  K/P=6144), N=12288  -- GPT-3 175B-shaped MLP down-proj

Recipe (the same for every workload): ``numpy.random.default_rng(seed)`` (PCG64) with
seed = the workload's dropout seed; draw X, W, bias, residual in that order as
``standard_normal(dtype=float32) * sigma``; round each to bf16 with round-to-nearest-even.
sigma: X 1, W 0.02 (0.006 for ``gpt3_mlp``), bias 0.02, residual 1.  Dropout p = 0.1
as an fp32 value.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "ORDER", "AdamWorkload", "ADAM_WORKLOADS", "f32_to_bf16_bits",
           "make_adam_inputs", "make_inputs", "make_producer_inputs", "make_random_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    P: int
    seed: int
    p_drop: float = 0.1
    sigma_x: float = 1.0
    sigma_w: float = 0.02
    sigma_bias: float = 0.02
    sigma_res: float = 1.0
    chunk: tuple = (0, 0)          # (0, 0): the library picks the chunk
    desc: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 256, 4, 0, chunk=(32, 64),
                     desc="tiny reference block M=64 K=256 (P=4) N=256"),
    "gpt2_attn": Workload("gpt2_attn", 8192, 3072, 3072, 16, 1,
                          desc="GPT-2 8.3B attention out-proj M=8192 K=3072 (P=16) N=3072"),
    "gpt2_mlp": Workload("gpt2_mlp", 8192, 12288, 3072, 16, 2,
                         desc="GPT-2 8.3B MLP down-proj M=8192 K=12288 (P=16) N=3072"),
    "bert_mlp": Workload("bert_mlp", 8192, 10240, 2560, 8, 3,
                         desc="BERT 3.9B MLP down-proj M=8192 K=10240 (P=8) N=2560"),
    "gpt3_mlp": Workload("gpt3_mlp", 2048, 49152, 12288, 8, 4, sigma_w=0.006,
                         desc="GPT-3 175B-shaped MLP down-proj M=2048 K=49152 (P=8) N=12288"),
}
ORDER = ["tiny", "gpt2_attn", "gpt2_mlp", "bert_mlp", "gpt3_mlp"]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    NaN inputs become the canonical quiet NaN 0x7FC0 (sign kept).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16) | np.uint16(0x7FC0)
    return r


def _draw(rng, shape, sigma):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def make_random_inputs(M, K, N, seed, sigma_x=1.0, sigma_w=0.02, sigma_bias=0.02,
                       sigma_res=1.0):
    """Draw X [M,K], W [K,N], bias [N], residual [M,N] as bf16 bits (uint16)."""
    rng = np.random.default_rng(seed)
    X = _draw(rng, (M, K), sigma_x)
    W = _draw(rng, (K, N), sigma_w)
    bias = _draw(rng, (N,), sigma_bias)
    res = _draw(rng, (M, N), sigma_res)
    return {"X": X, "W": W, "bias": bias, "residual": res}


def make_producer_inputs(w: Workload | str):
    """Inputs of the producer MatMul in front of a block (its MLP's first layer):
    X0 [M, N] (the layer's hidden state), W1 [N, K] and b1 [K], so that
    GeLU(X0 . W1 + b1) is the block's X [M, K].  Same recipe as ``make_inputs`` with
    seed = the workload's seed + 100, drawn in the order X0, W1, b1 (sigma: X0 1, W1 the
    workload's weight sigma, b1 the bias sigma)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed + 100)
    X0 = _draw(rng, (w.M, w.N), w.sigma_x)
    W1 = _draw(rng, (w.N, w.K), w.sigma_w)
    b1 = _draw(rng, (w.K,), w.sigma_bias)
    return {"X0": X0, "W1": W1, "b1": b1, "M": w.M, "N": w.K, "K": w.N}


def make_qkv_inputs(w: Workload | str):
    """Inputs of the QKV projection in front of an attention block's out-projection:
    X0 [M, N] (the hidden state), Wqkv [N, 3K] and bqkv [3K] (Q, K and V of K columns
    each; the attention over them gives the block's X [M, K]).  Same recipe as
    ``make_producer_inputs`` with seed = the workload's seed + 200."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed + 200)
    X0 = _draw(rng, (w.M, w.N), w.sigma_x)
    Wqkv = _draw(rng, (w.N, 3 * w.K), w.sigma_w)
    bqkv = _draw(rng, (3 * w.K,), w.sigma_bias)
    return {"X0": X0, "Wqkv": Wqkv, "bqkv": bqkv, "M": w.M, "N": 3 * w.K, "K": w.N}


@dataclasses.dataclass(frozen=True)
class AdamWorkload:
    """A data-parallel optimizer step: n fp32 parameters, P replicas' gradients."""
    name: str
    n: int
    P: int
    seed: int
    step: int = 10
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    desc: str = ""

    @property
    def bytes(self) -> int:
        """HBM bytes of one fused step: P gradient reads, parameter and both moments read
        and written, the bf16 parameter copy written."""
        return (4 * self.P + 26) * self.n


ADAM_WORKLOADS = {
    # BERT-large (about 335M parameters) with 8 data-parallel replicas
    "bert_large_adam": AdamWorkload("bert_large_adam", 335_141_888, 8, 5,
                                    desc="BERT-large, 335M fp32 parameters, P=8 replicas"),
    # a smaller case the oracle checks element by element
    "adam_16m": AdamWorkload("adam_16m", 16 * 1024 * 1024, 8, 6,
                             desc="16M fp32 parameters, P=8 replicas"),
}


def make_adam_inputs(n: int, P: int, seed: int):
    """Seeded fp32 optimizer state and gradients: PCG64 ``default_rng(seed)``, drawn in the
    order grads [P, n] (sigma 1e-2), param [n] (0.02), m [n] (1e-3), d [n] (1e-3), all
    float32, with v = (2 m)^2 + d^2: a second moment consistent with the first, as along
    an Adam run (|m| / sqrt(v) <= 1/2)."""
    rng = np.random.default_rng(seed)
    f = np.float32
    grads = rng.standard_normal((P, n), dtype=np.float32) * f(1e-2)
    param = rng.standard_normal(n, dtype=np.float32) * f(0.02)
    m = rng.standard_normal(n, dtype=np.float32) * f(1e-3)
    d = rng.standard_normal(n, dtype=np.float32) * f(1e-3)
    v = np.square(f(2) * m) + np.square(d)
    return {"grads": grads, "param": param, "m": m, "v": v}


def make_inputs(w: Workload | str):
    """Inputs of a named workload (see the module docstring for the recipe)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    d = make_random_inputs(w.M, w.K, w.N, w.seed, w.sigma_x, w.sigma_w, w.sigma_bias,
                           w.sigma_res)
    d.update(M=w.M, K=w.K, N=w.N, P=w.P, p_drop=np.float32(w.p_drop), seed=w.seed)
    return d
