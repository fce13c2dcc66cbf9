"""Host-side checks of the C ABI: the library loads, exports what include/mmar.h
declares, and rejects bad arguments before touching any device."""
import ctypes

import pytest

import chunked_matmul_reduce_amd as mmar

FAKE = 1 << 20          # 16-byte aligned stand-in pointer; never reaches a device


def _fused(**kw):
    a = dict(X=FAKE, W=FAKE * 2, bias=FAKE * 3, res=FAKE * 4, out=FAKE * 64, M=64, N=256, K=256, P=4,
             p=0.1, seed=0, cm=0, cn=0)
    a.update(kw)
    return mmar.lib.mmar_fused(a["X"], a["W"], a["bias"], a["res"], a["out"], a["M"], a["N"], a["K"],
                               a["P"], a["p"], a["seed"], a["cm"], a["cn"], None)


def test_every_declared_function_is_exported():
    names = mmar.header_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(mmar.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mmar._SIGNATURES)


def test_version():
    assert mmar.version().startswith("mmar ") and "gfx950" in mmar.version()


@pytest.mark.parametrize("kw,msg", [
    (dict(X=None), "X is NULL"), (dict(out=None), "out is NULL"),
    (dict(M=0), "positive"), (dict(P=3), "P must divide K"), (dict(K=96, P=2), "multiple of 32"),
    (dict(M=48), "multiples of 32"), (dict(N=40), "multiples of 32"), (dict(P=0), "P must be"),
    (dict(p=-0.1), "p_drop"), (dict(p=1.01), "p_drop"), (dict(p=float("nan")), "p_drop"),
    (dict(p=float("inf")), "p_drop"), (dict(cm=48), "chunk_m"), (dict(cn=100), "chunk_n"),
    (dict(cm=-32), "chunk"), (dict(out=FAKE * 2), "overlaps"),
    (dict(M=1 << 20, K=1 << 12), "2^31"),
])
def test_invalid_arguments_rejected_before_device(kw, msg):
    assert _fused(**kw) == mmar.EINVAL
    assert msg in mmar.last_error()


def test_misaligned_pointer():
    assert _fused(W=FAKE + 8) == mmar.EALIGN
    assert "W" in mmar.last_error()


def test_other_entry_points_validate():
    L = mmar.lib
    assert L.mmar_gemm_only(FAKE, FAKE * 2, FAKE * 8, 64, 256, 250, 4, 0, 0, None) == mmar.EINVAL
    assert L.mmar_gemm_partials(None, FAKE, FAKE, 64, 64, 64, 2, None) == mmar.EINVAL
    assert L.mmar_reduce_epilogue_only(FAKE, FAKE, FAKE, FAKE, 64, 64, 2, 2.0, 0, None) == mmar.EINVAL
    assert L.mmar_reduce_epilogue_only(FAKE, FAKE, FAKE, FAKE, 60, 64, 2, 0.1, 0, None) == mmar.EINVAL
    assert L.mmar_fused_ex(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, 64, 256, 256, 4, 0.1, 0, 7,
                           0, 0, 0, -1, -1, None, 0, None) == mmar.EINVAL
    assert L.mmar_fused_ex(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, 64, 256, 256, 4, 0.1, 0, 2,
                           0, 0, 9, -1, -1, None, 0, None) == mmar.EINVAL
    assert L.mmar_fused_ex(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, 64, 256, 256, 4, 0.1, 0, 2,
                           0, 0, 0, 5, -1, None, 0, None) == mmar.EINVAL
    assert "weight mode" in mmar.last_error()
    assert L.mmar_fused_ex(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, 64, 256, 256, 4, 0.1, 0, 3,
                           0, 0, 0, -1, 2, None, 0, None) == mmar.EINVAL
    assert "tile" in mmar.last_error()
    assert L.mmar_fused_nt(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, 64, 256, 250, 4, 0.1, 0, 0,
                           0, None) == mmar.EINVAL
    assert L.mmar_transpose_weight(FAKE, FAKE, 64, 64, None) == mmar.EINVAL   # overlap
    assert L.mmar_transpose_weight(FAKE, FAKE * 64, 60, 64, None) == mmar.EINVAL
    U = L.mmar_unfused
    assert U(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, None, 64, 256, 250, 4, 0.1, 0, None) == \
        mmar.EINVAL   # P does not divide K
    assert U(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, FAKE * 128 + 4, 64, 256, 256, 4, 0.1, 0,
             None) == mmar.EALIGN   # mask misaligned
    assert U(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, FAKE * 64 + 4096, 64, 256, 256, 4, 0.1, 0,
             None) == mmar.EINVAL   # mask overlaps out
    assert "overlaps" in mmar.last_error()
    assert U(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, None, 64, 256, 256, 4, 1.5, 0, None) == \
        mmar.EINVAL   # p outside [0, 1]
    A = L.mmar_adam_step
    assert A(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 1022, 2, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0,
             None) == mmar.EINVAL   # n not a multiple of 4
    assert A(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 1024, 2, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0,
             None) == mmar.EINVAL   # step 0
    assert A(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 1024, 2, 1, 1e-3, 0.9, 1.0, 1e-8, 0.0,
             None) == mmar.EINVAL   # beta2 = 1
    assert A(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 1024, 2, 1, 1e-3, 0.9, 0.999, 0.0, 0.0,
             None) == mmar.EINVAL   # eps = 0
    assert A(FAKE, FAKE * 2, FAKE * 2 + 1024, FAKE * 4, None, 1024, 2, 1, 1e-3, 0.9, 0.999, 1e-8,
             0.0, None) == mmar.EINVAL   # m overlaps param
    assert A(FAKE, FAKE * 2 + 4, FAKE * 3, FAKE * 4, None, 1024, 2, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0,
             None) == mmar.EALIGN
    assert L.mmar_gelu_linear(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 64, 64, 250, None) == mmar.EINVAL
    assert L.mmar_gelu_linear(FAKE, FAKE * 2, FAKE * 3, FAKE, 64, 64, 256, None) == mmar.EINVAL
    FB = L.mmar_fused_bf16
    assert FB(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 4, 64, 256, 256, 4, 0.1, 1, None) == mmar.EINVAL
    assert FB(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, 64, 256, 250, 4, 0.1, 1, None) == mmar.EINVAL
    assert FB(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64, 64, 256, 256, 4, -0.5, 1, None) == mmar.EINVAL
    assert FB(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 64 + 4, 64, 256, 256, 4, 0.1, 1, None) == mmar.EALIGN
    assert L.mmar_linear(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 64, 64, 256, 2, None) == mmar.EINVAL
    assert L.mmar_linear(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 64, 64, 256, -1, None) == mmar.EINVAL
    assert L.mmar_linear(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 64, 64, 250, 0, None) == mmar.EINVAL
    assert L.mmar_linear(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 64, 64, 256, 7, None) == mmar.EINVAL
    assert b"activation" in L.mmar_last_error()
    assert L.mmar_set_plan(64, 256, 256, 4, 9, 0, 0, 0, -1, -1) == mmar.EINVAL
    assert L.mmar_set_plan(64, 256, 256, 4, 3, 0, 0, 0, -1, 7) == mmar.EINVAL
    assert L.mmar_autotune(64, 256, 250, 4, 0) == mmar.EINVAL


def test_balanced_schedule_workspace_and_chunk():
    """The balanced schedule's tail partials: P x M x (tail columns) x 4 bytes, or
    P x (tail rows) x N x 4; none when the tile count is already a multiple of 256."""
    assert mmar.workspace_bytes("balanced", 8192, 2560, 10240, 8) == 8 * 8192 * 512 * 4
    assert mmar.workspace_bytes("auto", 8192, 2560, 10240, 8) == 0     # default: persistent
    assert mmar.workspace_bytes("balanced", 8192, 3072, 12288, 16) == 0
    assert mmar.workspace_bytes("balanced", 2080, 4096, 512, 4) == 4 * 32 * 4096 * 4
    assert mmar.workspace_bytes("balanced", 8192, 1088, 512, 4) == 4 * 8192 * 64 * 4
    assert mmar.workspace_bytes("balanced", 64, 256, 256, 4) == 0          # one tile
    with pytest.raises(mmar.MmarError):
        mmar.workspace_bytes("balanced", 8192, 2560, 10240, 8, chunk=(4096, 0))
    L = mmar.lib
    assert L.mmar_set_plan(8192, 2560, 10240, 8, 4, 4096, 0, 0, -1, -1) == mmar.EINVAL
    assert L.mmar_workspace_bytes(6, 8192, 2560, 10240, 8, 0, 0, 0, -1, -1) == 0
    assert b"schedule" in L.mmar_last_error()
    # with 256 x 192 tiles: 32 x 14 = 448 tiles; the head is 8192 x 1536 (256 tiles), the
    # tail 8192 x 1024
    assert mmar.workspace_bytes("balanced", 8192, 2560, 10240, 8, tile="256x192") == 8 * 8192 * 1024 * 4
    # 8192 x 3072 on 256 x 192 tiles is 512 tiles: two full rounds, no tail
    assert mmar.workspace_bytes("balanced", 8192, 3072, 12288, 16, tile="256x192") == 0
    assert L.mmar_workspace_bytes(4, 8192, 2560, 10240, 8, 0, 0, 0, -1, 3) == 0


def test_split_schedule_needs_no_workspace():
    """The split schedule's tail runs the fused kernel again on 128 x 128 tiles: no
    partials, so no workspace (only a pre-transposed weight takes any); whole-output
    chunk only."""
    assert mmar.workspace_bytes("split", 8192, 2560, 10240, 8) == 0
    assert mmar.workspace_bytes("split", 8192, 2560, 10240, 8, tile="256x192") == 0
    assert mmar.workspace_bytes("split", 8192, 2560, 10240, 8, w_mode="pretranspose") == \
        10240 * 2560 * 2
    with pytest.raises(mmar.MmarError):
        mmar.workspace_bytes("split", 8192, 2560, 10240, 8, chunk=(0, 1280))
    assert mmar.lib.mmar_set_plan(8192, 2560, 10240, 8, mmar.SCHED_SPLIT, 4096, 0, 0, -1, -1) == \
        mmar.EINVAL


def test_workspace_bytes():
    wt = 12288 * 3072 * 2   # pre-transposed weight of the 8192-row block
    assert mmar.workspace_bytes("persistent", 8192, 3072, 12288, 16) == 0
    assert mmar.workspace_bytes("persistent", 8192, 3072, 12288, 16, w_mode="pretranspose") == wt
    assert mmar.workspace_bytes("sequential", 8192, 3072, 12288, 16) == 4 * 16 * 8192 * 3072
    assert mmar.workspace_bytes("sequential", 8192, 3072, 12288, 16, w_mode="pretranspose") == \
        4 * 16 * 8192 * 3072 + wt
    assert mmar.workspace_bytes("sequential", 64, 256, 256, 4, chunk=(32, 64)) == 4 * 4 * 32 * 64
    assert mmar.workspace_bytes("streams", 1024, 512, 256, 4, chunk=(256, 512), ring=3) == \
        3 * 4 * 4 * 256 * 512
    assert mmar.workspace_bytes("streams", 1024, 512, 256, 4, chunk=(256, 512), ring=3,
                                w_mode="pretranspose") == 3 * 4 * 4 * 256 * 512 + 256 * 512 * 2
    with pytest.raises(mmar.MmarError):
        mmar.workspace_bytes("streams", 1024, 512, 250, 4)


def test_no_device_reports_enodev():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the no-device path is for CPU-only hosts")
    assert _fused() == mmar.ENODEV
    assert mmar.lib.mmar_autotune(64, 256, 256, 4, 0) == mmar.ENODEV
    assert mmar.lib.mmar_release() == mmar.OK


def _strided(**kw):
    a = dict(X=FAKE, ldx=256, W=FAKE * 2, ldw=256, bias=FAKE * 3, res=FAKE * 4, ldr=256,
             out=FAKE * 64, ldo=256, M=64, N=256, K=256, P=4, p=0.1, seed=0, off=0)
    a.update(kw)
    return mmar.lib.mmar_fused_strided(a["X"], a["ldx"], a["W"], a["ldw"], a["bias"], a["res"],
                                       a["ldr"], a["out"], a["ldo"], a["M"], a["N"], a["K"],
                                       a["P"], a["p"], a["seed"], a["off"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(ldx=224), mmar.EINVAL, "leading dimension"), (dict(ldw=200), mmar.EINVAL, "leading"),
    (dict(ldr=128), mmar.EINVAL, "leading"), (dict(ldo=252), mmar.EINVAL, "leading"),
    (dict(ldx=260), mmar.EALIGN, "ldx and ldw"), (dict(ldw=268), mmar.EALIGN, "ldx and ldw"),
    (dict(ldr=258), mmar.EALIGN, "ldr and ldo"), (dict(ldo=262), mmar.EALIGN, "ldr and ldo"),
    (dict(ldx=1 << 26), mmar.EINVAL, "2^31"), (dict(X=None), mmar.EINVAL, "X is NULL"),
    (dict(out=FAKE * 2), mmar.EINVAL, "overlaps"), (dict(P=3), mmar.EINVAL, "P must divide K"),
    (dict(p=1.5), mmar.EINVAL, "p_drop"), (dict(res=FAKE * 4 + 4), mmar.EALIGN, "residual"),
    (dict(W=FAKE * 2 + 8), mmar.EALIGN, "W is not 16-byte"),
    # out's extent with a long row stride reaches the residual at FAKE * 4 + ...
    (dict(out=FAKE * 3 + 1024, ldo=8192), mmar.EINVAL, "overlaps"),
])
def test_strided_entry_validates_before_device(kw, code, msg):
    assert _strided(**kw) == code
    assert msg in mmar.last_error()


def test_strided_entry_without_device():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the no-device path is for CPU-only hosts")
    assert _strided(ldx=264, ldw=320, ldr=260, ldo=300, off=2 ** 64 - 1) == mmar.ENODEV
