"""Python binding of libmmar, the gfx950 fused MatMul -> slice-reduce -> epilogue library.

Argument marshalling only: every step of the block runs in the HIP kernels behind the C
ABI of ``include/mmar.h``.  PyTorch supplies device memory and the current HIP stream.
Importing this package fails if ``libmmar.so`` has not been built
(``python chunked_matmul_reduce_amd/build.py``); there is no fallback.

Block computed (see include/mmar.h for the full contract):
    out = residual + dropout_p(bias + sum_p X[:, K_p] @ W[K_p, :])     (fp32 out)
with bf16 X [M,K], W [K,N], bias [N], residual [M,N]; P equal K-slices; fp32 slice
accumulation from zero; fixed-order fp32 reduction; counter-based Philox4x32-10 mask.
``fused_bf16`` is the same block with its output rounded once more, to bf16.
Around it: ``linear`` / ``gelu_linear`` / ``mlp`` (the producer MatMul + bias and GeLU,
or no activation for an attention block's QKV projection, in front of the block),
``unfused`` (the block one kernel per operation) and ``adam_step`` (the data-parallel
gradient average + Adam step).
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmmar.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "mmar.h")

OK, EINVAL, EALIGN, ENODEV, ENOMEM, EHIP = 0, -1, -2, -3, -4, -5
SCHED_AUTO, SCHED_SEQUENTIAL, SCHED_STREAMS, SCHED_PERSISTENT, SCHED_BALANCED, SCHED_SPLIT = (
    0, 1, 2, 3, 4, 5)
SCHEDULES = {"auto": 0, "sequential": 1, "streams": 2, "persistent": 3, "balanced": 4, "split": 5}
W_AUTO, W_DIRECT, W_PRETRANSPOSE = -1, 0, 1
W_MODES = {"auto": -1, "direct": 0, "pretranspose": 1}
TILE_AUTO, TILE_256x128, TILE_256x192 = -1, 0, 1
TILES = {"auto": -1, "256x128": 0, "256x192": 1}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "mmar_fused": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _U64, _I32, _I32, _P]),
    "mmar_fused_nt": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _U64, _I32, _I32, _P]),
    "mmar_fused_bf16": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _U64, _P]),
    "mmar_workspace_bytes": (_SZ, [_I32, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32]),
    "mmar_fused_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _U64, _I32, _I32,
                                     _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "mmar_transpose_weight": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "mmar_sequential": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _U64, _I32, _I32, _P]),
    "mmar_unfused": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _U64, _P]),
    "mmar_gelu_linear": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "mmar_linear": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P]),
    "mmar_adam_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I32, _I64, _F, _F, _F, _F, _F, _P]),
    "mmar_gemm_only": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P]),
    "mmar_gemm_partials": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I32, _P]),
    "mmar_reduce_epilogue_only": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I32, _F, _U64, _P]),
    "mmar_autotune": (ctypes.c_int, [_I64, _I64, _I64, _I32, ctypes.c_uint32]),
    "mmar_set_plan": (ctypes.c_int, [_I64, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "mmar_get_plan": (ctypes.c_int, [_I64, _I64, _I64, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                                     ctypes.POINTER(_I32), ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                                     ctypes.POINTER(_I32)]),
    "mmar_fused_strided": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _I64, _I64, _I64,
                                          _I32, _F, _U64, _U64, _P]),
    "mmar_fused_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _U64, _I32,
                                          _I32, _I32, _I32, _I32, _I32, _P]),
    "mmar_noalloc_workspace_capacity": (_SZ, []),
    "mmar_mlp": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _F, _U64,
                                _I32, _P]),
    "mmar_last_error": (ctypes.c_char_p, []),
    "mmar_version": (ctypes.c_char_p, []),
    "mmar_release": (ctypes.c_int, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python chunked_matmul_reduce_amd/build.py` (hipcc, gfx950)")
    # PyTorch ships its own HIP runtime (same soname as ROCm's).  Load it first so that
    # libmmar binds to the runtime torch uses: two HIP runtimes in one process do not
    # share the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class MmarError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"mmar error {code}: {msg}")
        self.code = code


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/mmar.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mmar_\w+)\s*\(", text)))


def last_error() -> str:
    return lib.mmar_last_error().decode()


def version() -> str:
    return lib.mmar_version().decode()


def release() -> None:
    _check(lib.mmar_release())


def _check(rc):
    if rc != OK:
        raise MmarError(rc, last_error())


# ---------------------------------------------------------------- tensor helpers
def _torch():
    import torch
    return torch


def _bits(t, name, shape):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16 (or 16-bit bf16 bit patterns), got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _f32(t, name, shape):
    torch = _torch()
    if t.device.type != "cuda" or t.dtype != torch.float32:
        raise TypeError(f"{name} must be a float32 GPU tensor")
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with shape {tuple(shape)}")
    return t.data_ptr()


def _stream(device, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _out(out, shape, like):
    torch = _torch()
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=like.device)
    _f32(out, "out", shape)
    return out


def _shapes(X, W, P):
    if X.dim() != 2 or W.dim() != 2:
        raise ValueError("X must be [M, K] and W [K, N]")
    M, K = X.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError(f"X is [M={M}, K={K}] but W is [{K2}, {N}]")
    return int(M), int(N), int(K)


# ---------------------------------------------------------------- entry points
def fused(X, W, bias, residual, P, p_drop, seed, chunk=(0, 0), out=None, stream=None):
    """mmar_fused: the block with the library's plan for this shape; returns fp32 out."""
    torch = _torch()
    M, N, K = _shapes(X, W, P)
    out = _out(out, (M, N), X)
    with torch.cuda.device(X.device):
        rc = lib.mmar_fused(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)), _bits(bias, "bias", (N,)),
                            _bits(residual, "residual", (M, N)), out.data_ptr(), M, N, K, int(P),
                            float(p_drop), int(seed) & (2 ** 64 - 1), int(chunk[0]), int(chunk[1]),
                            _stream(X.device, stream))
    _check(rc)
    return out


def fused_bf16(X, W, bias, residual, P, p_drop, seed, out=None, stream=None):
    """mmar_fused_bf16: the block with its fp32 result rounded once to bf16; returns bf16
    out [M, N]."""
    torch = _torch()
    M, N, K = _shapes(X, W, P)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    op = _bits(out, "out", (M, N))
    with torch.cuda.device(X.device):
        rc = lib.mmar_fused_bf16(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)),
                                 _bits(bias, "bias", (N,)), _bits(residual, "residual", (M, N)),
                                 op, M, N, K, int(P), float(p_drop), int(seed) & (2 ** 64 - 1),
                                 _stream(X.device, stream))
    _check(rc)
    return out


def fused_ex(X, W, bias, residual, P, p_drop, seed, schedule, chunk=(0, 0), ring=0,
             w_mode="auto", tile="auto", workspace=None, out=None, stream=None):
    """mmar_fused_ex: every choice explicit; ``workspace`` is an optional GPU tensor."""
    torch = _torch()
    if isinstance(schedule, str):
        schedule = SCHEDULES[schedule]
    if isinstance(w_mode, str):
        w_mode = W_MODES[w_mode]
    if isinstance(tile, str):
        tile = TILES[tile]
    M, N, K = _shapes(X, W, P)
    out = _out(out, (M, N), X)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(X.device):
        rc = lib.mmar_fused_ex(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)), _bits(bias, "bias", (N,)),
                               _bits(residual, "residual", (M, N)), out.data_ptr(), M, N, K, int(P),
                               float(p_drop), int(seed) & (2 ** 64 - 1), int(schedule), int(chunk[0]),
                               int(chunk[1]), int(ring), int(w_mode), int(tile), ws_ptr, ws_bytes,
                               _stream(X.device, stream))
    _check(rc)
    return out


def fused_noalloc(X, W, bias, residual, P, p_drop, seed, schedule, chunk=(0, 0), ring=0,
                  w_mode="auto", tile="auto", out=None, stream=None):
    """mmar_fused_noalloc: fused_ex with the library's static per-device workspace
    (``noalloc_workspace_capacity()`` bytes), for callers that cannot allocate; ``out`` must
    be given by such callers (None allocates it here, for convenience in tests)."""
    torch = _torch()
    if isinstance(schedule, str):
        schedule = SCHEDULES[schedule]
    if isinstance(w_mode, str):
        w_mode = W_MODES[w_mode]
    if isinstance(tile, str):
        tile = TILES[tile]
    M, N, K = _shapes(X, W, P)
    out = _out(out, (M, N), X)
    with torch.cuda.device(X.device):
        rc = lib.mmar_fused_noalloc(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)),
                                    _bits(bias, "bias", (N,)), _bits(residual, "residual", (M, N)),
                                    out.data_ptr(), M, N, K, int(P), float(p_drop),
                                    int(seed) & (2 ** 64 - 1), int(schedule), int(chunk[0]),
                                    int(chunk[1]), int(ring), int(w_mode), int(tile),
                                    _stream(X.device, stream))
    _check(rc)
    return out


def noalloc_workspace_capacity() -> int:
    return int(lib.mmar_noalloc_workspace_capacity())


def _rows(t, name, shape, dtypes, align):
    """Data pointer and leading dimension of a 2-D tensor whose rows are contiguous."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows (stride 1 along its last dimension)")
    ld = int(t.stride(0)) if shape[0] > 1 else int(shape[1])
    if ld % align:
        raise ValueError(f"{name}'s leading dimension {ld} is not a multiple of {align}")
    return t.data_ptr(), ld


def fused_strided(X, W, bias, residual, P, p_drop, seed, philox_offset=0, out=None,
                  stream=None):
    """mmar_fused_strided: the block over row-strided views (each 2-D tensor with
    contiguous rows and any row stride: a column block of a wider buffer, say) and with
    the dropout mask's Philox counter words 2-3 set to ``philox_offset``.  ``out`` may be a
    row-strided float32 view; a new dense one is allocated when it is None."""
    torch = _torch()
    M, N, K = _shapes(X, W, P)
    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    xp, ldx = _rows(X, "X", (M, K), b16, 8)
    wp, ldw = _rows(W, "W", (K, N), b16, 8)
    rp, ldr = _rows(residual, "residual", (M, N), b16, 4)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    op, ldo = _rows(out, "out", (M, N), (torch.float32,), 4)
    with torch.cuda.device(X.device):
        rc = lib.mmar_fused_strided(xp, ldx, wp, ldw, _bits(bias, "bias", (N,)), rp, ldr, op, ldo,
                                    M, N, K, int(P), float(p_drop), int(seed) & (2 ** 64 - 1),
                                    int(philox_offset) & (2 ** 64 - 1), _stream(X.device, stream))
    _check(rc)
    return out


def fused_nt(X, Wt, bias, residual, P, p_drop, seed, chunk=(0, 0), out=None, stream=None):
    """mmar_fused_nt: the block with the weight given transposed, Wt = W^T [N, K]."""
    torch = _torch()
    if X.dim() != 2 or Wt.dim() != 2 or Wt.shape[1] != X.shape[1]:
        raise ValueError("X must be [M, K] and Wt [N, K]")
    M, K = (int(v) for v in X.shape)
    N = int(Wt.shape[0])
    out = _out(out, (M, N), X)
    with torch.cuda.device(X.device):
        rc = lib.mmar_fused_nt(_bits(X, "X", (M, K)), _bits(Wt, "Wt", (N, K)), _bits(bias, "bias", (N,)),
                               _bits(residual, "residual", (M, N)), out.data_ptr(), M, N, K, int(P),
                               float(p_drop), int(seed) & (2 ** 64 - 1), int(chunk[0]), int(chunk[1]),
                               _stream(X.device, stream))
    _check(rc)
    return out


def transpose_weight(W, out=None, stream=None):
    """mmar_transpose_weight: W [K, N] -> W^T [N, K] (bf16)."""
    torch = _torch()
    K, N = (int(v) for v in W.shape)
    if out is None:
        out = torch.empty((N, K), dtype=W.dtype, device=W.device)
    with torch.cuda.device(W.device):
        rc = lib.mmar_transpose_weight(_bits(W, "W", (K, N)), _bits(out, "Wt", (N, K)), K, N,
                                       _stream(W.device, stream))
    _check(rc)
    return out


def sequential(X, W, bias, residual, P, p_drop, seed, chunk=(0, 0), out=None, stream=None):
    """mmar_sequential: GEMM of the partials then reduce+epilogue, no overlap."""
    torch = _torch()
    M, N, K = _shapes(X, W, P)
    out = _out(out, (M, N), X)
    with torch.cuda.device(X.device):
        rc = lib.mmar_sequential(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)),
                                 _bits(bias, "bias", (N,)), _bits(residual, "residual", (M, N)),
                                 out.data_ptr(), M, N, K, int(P), float(p_drop),
                                 int(seed) & (2 ** 64 - 1), int(chunk[0]), int(chunk[1]),
                                 _stream(X.device, stream))
    _check(rc)
    return out


def unfused(X, W, bias, residual, P, p_drop, seed, out=None, mask=None, stream=None):
    """mmar_unfused: the block one kernel per operation (partials GEMM, reduction, bias add,
    dropout, residual add).  `mask`: a uint8 [M, N] GPU tensor that receives the keep mask
    (1 = kept), or None.  Returns out."""
    torch = _torch()
    M, N, K = _shapes(X, W, P)
    out = _out(out, (M, N), X)
    mp = None
    if mask is not None:
        if mask.device.type != "cuda" or mask.dtype != torch.uint8 or tuple(mask.shape) != (M, N) \
                or not mask.is_contiguous():
            raise ValueError(f"mask must be a contiguous uint8 GPU tensor of shape {(M, N)}")
        mp = mask.data_ptr()
    with torch.cuda.device(X.device):
        rc = lib.mmar_unfused(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)), _bits(bias, "bias", (N,)),
                              _bits(residual, "residual", (M, N)), out.data_ptr(), mp, M, N, K,
                              int(P), float(p_drop), int(seed) & (2 ** 64 - 1),
                              _stream(X.device, stream))
    _check(rc)
    return out


def gelu_linear(X, W, bias, out=None, stream=None):
    """mmar_gelu_linear: H = GeLU(X . W + bias) as bf16 [M, N] (the producer MatMul)."""
    torch = _torch()
    M, N, K = _shapes(X, W, 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    hp = _bits(out, "out", (M, N))
    with torch.cuda.device(X.device):
        rc = lib.mmar_gelu_linear(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)),
                                  _bits(bias, "bias", (N,)), hp, M, N, K, _stream(X.device, stream))
    _check(rc)
    return out


ACTIVATIONS = {"none": 0, "gelu_tanh": 1}   # MMAR_ACT_NONE, MMAR_ACT_GELU_TANH


def linear(X, W, bias, activation="none", out=None, stream=None):
    """mmar_linear: H = act(X . W + bias) as bf16 [M, N], act "none" (the QKV projection in
    front of an attention block) or "gelu_tanh" (as gelu_linear)."""
    torch = _torch()
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
    M, N, K = _shapes(X, W, 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    hp = _bits(out, "out", (M, N))
    with torch.cuda.device(X.device):
        rc = lib.mmar_linear(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)), _bits(bias, "bias", (N,)),
                             hp, M, N, K, ACTIVATIONS[activation], _stream(X.device, stream))
    _check(rc)
    return out


def mlp(X, W1, b1, W2, b2, residual, P, p_drop, seed, out=None, hidden=None, stream=None):
    """The MLP around the block: H = GeLU(X . W1 + b1) (mmar_gelu_linear), then
    out = residual + dropout(b2 + sum_p H[:, K_p] . W2[K_p, :]) (mmar_fused).  Returns
    (out, H)."""
    H = gelu_linear(X, W1, b1, out=hidden, stream=stream)
    return fused(H, W2, b2, residual, P, p_drop, seed, out=out, stream=stream), H


def mlp_chunked(X, W1, b1, W2, b2, residual, P, p_drop, seed, chunk_m=0, out=None, hidden=None,
                stream=None):
    """mmar_mlp: the same MLP in one call; chunk_m > 0 hands H to the block row chunk by row
    chunk (producer of chunk c+1 beside the block of chunk c, two streams).  Returns
    (out, H)."""
    torch = _torch()
    if X.dim() != 2 or W1.dim() != 2 or W2.dim() != 2:
        raise ValueError("X must be [M, D], W1 [D, K], W2 [K, N]")
    M, D = (int(v) for v in X.shape)
    K = int(W1.shape[1])
    N = int(W2.shape[1])
    if hidden is None:
        hidden = torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
    out = _out(out, (M, N), X)
    with torch.cuda.device(X.device):
        rc = lib.mmar_mlp(_bits(X, "X", (M, D)), _bits(W1, "W1", (D, K)), _bits(b1, "b1", (K,)),
                          _bits(W2, "W2", (K, N)), _bits(b2, "b2", (N,)),
                          _bits(residual, "residual", (M, N)), _bits(hidden, "hidden", (M, K)),
                          out.data_ptr(), M, D, K, N, int(P), float(p_drop),
                          int(seed) & (2 ** 64 - 1), int(chunk_m), _stream(X.device, stream))
    _check(rc)
    return out, hidden


def adam_step(grads, param, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
              param_bf16=None, stream=None):
    """mmar_adam_step: average the P replicas' gradients grads [P, n] (fp32, fixed order),
    Adam-update param, m, v (fp32 [n], in place) and, if given, write the bf16 copy of the
    new parameters to param_bf16."""
    torch = _torch()
    if grads.dim() != 2:
        raise ValueError("grads must be [P, n]")
    P, n = (int(x) for x in grads.shape)
    ptrs = [_f32(grads, "grads", (P, n))] + [_f32(t, nm, (n,)) for t, nm in
                                              ((param, "param"), (m, "m"), (v, "v"))]
    bp = None
    if param_bf16 is not None:
        bp = _bits(param_bf16, "param_bf16", (n,))
    with torch.cuda.device(grads.device):
        rc = lib.mmar_adam_step(*ptrs, bp, n, P, int(step), float(lr), float(beta1), float(beta2),
                                float(eps), float(weight_decay), _stream(grads.device, stream))
    _check(rc)


def gemm_only(X, W, P, chunk=(0, 0), out=None, stream=None):
    """mmar_gemm_only: the reduced fp32 sum T of the P slice partials (no epilogue)."""
    torch = _torch()
    M, N, K = _shapes(X, W, P)
    out = _out(out, (M, N), X)
    with torch.cuda.device(X.device):
        rc = lib.mmar_gemm_only(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)), out.data_ptr(), M, N, K,
                                int(P), int(chunk[0]), int(chunk[1]), _stream(X.device, stream))
    _check(rc)
    return out


def gemm_partials(X, W, P, out=None, stream=None):
    """mmar_gemm_partials: the P fp32 slice partials, [P, M, N]."""
    torch = _torch()
    M, N, K = _shapes(X, W, P)
    out = _out(out, (int(P), M, N), X)
    with torch.cuda.device(X.device):
        rc = lib.mmar_gemm_partials(_bits(X, "X", (M, K)), _bits(W, "W", (K, N)), out.data_ptr(),
                                    M, N, K, int(P), _stream(X.device, stream))
    _check(rc)
    return out


def reduce_epilogue_only(partials, bias, residual, p_drop, seed, out=None, stream=None):
    """mmar_reduce_epilogue_only over partials [P, M, N] (fp32)."""
    torch = _torch()
    if partials.dim() != 3:
        raise ValueError("partials must be [P, M, N]")
    P, M, N = (int(v) for v in partials.shape)
    out = _out(out, (M, N), partials)
    with torch.cuda.device(partials.device):
        rc = lib.mmar_reduce_epilogue_only(_f32(partials, "partials", (P, M, N)),
                                           _bits(bias, "bias", (N,)),
                                           _bits(residual, "residual", (M, N)), out.data_ptr(), M, N, P,
                                           float(p_drop), int(seed) & (2 ** 64 - 1),
                                           _stream(partials.device, stream))
    _check(rc)
    return out


def workspace_bytes(schedule, M, N, K, P, chunk=(0, 0), ring=0, w_mode="auto", tile="auto") -> int:
    if isinstance(schedule, str):
        schedule = SCHEDULES[schedule]
    if isinstance(w_mode, str):
        w_mode = W_MODES[w_mode]
    if isinstance(tile, str):
        tile = TILES[tile]
    n = lib.mmar_workspace_bytes(int(schedule), int(M), int(N), int(K), int(P), int(chunk[0]),
                                 int(chunk[1]), int(ring), int(w_mode), int(tile))
    if n == 0 and last_error():
        raise MmarError(EINVAL, last_error())
    return int(n)


def autotune(M, N, K, P, flags=0) -> None:
    _check(lib.mmar_autotune(int(M), int(N), int(K), int(P), int(flags)))


def set_plan(M, N, K, P, schedule, chunk=(0, 0), ring=0, w_mode="auto", tile="auto") -> None:
    if isinstance(schedule, str):
        schedule = SCHEDULES[schedule]
    if isinstance(w_mode, str):
        w_mode = W_MODES[w_mode]
    if isinstance(tile, str):
        tile = TILES[tile]
    _check(lib.mmar_set_plan(int(M), int(N), int(K), int(P), int(schedule), int(chunk[0]),
                             int(chunk[1]), int(ring), int(w_mode), int(tile)))


def get_plan(M, N, K, P):
    s, cm, cn, r, wm, t = _I32(), _I32(), _I32(), _I32(), _I32(), _I32()
    _check(lib.mmar_get_plan(int(M), int(N), int(K), int(P), ctypes.byref(s), ctypes.byref(cm),
                             ctypes.byref(cn), ctypes.byref(r), ctypes.byref(wm), ctypes.byref(t)))
    return {"schedule": s.value, "chunk": (cm.value, cn.value), "ring": r.value, "w_mode": wm.value,
            "tile": t.value}
