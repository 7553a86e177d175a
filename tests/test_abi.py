"""C-ABI boundary on the host: the library loads, exports every function that
include/te_mi355x.h declares, and rejects invalid arguments with the right
status before any HIP call (no compute, no GPU needed)."""

import ctypes
import os

import pytest

from fp8_precision_transformer_amd import binding as B

needs_lib = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")

FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: validation fails first
FAKE_MIS = ctypes.c_void_p(0x10008)    # 8-byte aligned only


@needs_lib
def test_exports_every_header_function():
    L = B.lib()
    names = B.header_functions()
    assert set(names) >= {"te_amax_cast", "te_cast_transpose", "te_scale_update", "te_fp8_gemm",
                          "te_mxfp8_quantize", "te_get_last_error"}
    for n in names:
        assert hasattr(L, n), n
    assert b"gfx950" in L.te_version()


def _gemm(**kw):
    args = dict(a=FAKE, a_dtype=B.TE_E4M3, a_scale=FAKE, b=FAKE, b_dtype=B.TE_E4M3, b_scale=FAKE,
                gran=B.TE_GRAN_TENSOR, m=64, n=64, k=64, bias=None, bias_dtype=B.TE_F32, d=FAKE,
                d_dtype=B.TE_BF16, stream=None)
    args.update(kw)
    return B.lib().te_fp8_gemm(*args.values())


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(n=15), B.TE_ERR_SHAPE),
    (dict(k=24), B.TE_ERR_SHAPE),
    (dict(m=-1), B.TE_ERR_SHAPE),
    (dict(a_dtype=B.TE_F32), B.TE_ERR_DTYPE),
    (dict(a_dtype=B.TE_BF16), B.TE_ERR_DTYPE),
    (dict(d_dtype=B.TE_E4M3), B.TE_ERR_DTYPE),
    (dict(gran=9), B.TE_ERR_ARG),
    (dict(gran=B.TE_GRAN_MX_BLOCK32, k=48), B.TE_ERR_SHAPE),
    (dict(a_dtype=B.TE_BF16, b_dtype=B.TE_BF16, gran=B.TE_GRAN_MX_BLOCK32), B.TE_ERR_UNSUPPORTED),
    (dict(a=None), B.TE_ERR_NULL),
    (dict(a_scale=None), B.TE_ERR_NULL),
    (dict(d=FAKE_MIS), B.TE_ERR_ALIGN),
    (dict(k=0), B.TE_ERR_SHAPE),
    (dict(bias=FAKE, bias_dtype=B.TE_E5M2), B.TE_ERR_DTYPE),
])
def test_gemm_validation(kw, status):
    assert _gemm(**kw) == status
    assert len(B.lib().te_get_last_error()) > 0


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(gran=B.TE_GRAN_MX_BLOCK32_PANEL, k=96), B.TE_ERR_SHAPE),           # panel scales: k % 128
    (dict(gran=B.TE_GRAN_MX_BLOCK32_PANEL, a_dtype=B.TE_E2M1, b_dtype=B.TE_E2M1, k=128), B.TE_ERR_SHAPE),
    (dict(gran=B.TE_GRAN_MX_BLOCK32_PANEL, a_scale=FAKE_MIS), B.TE_ERR_ALIGN),
    (dict(gran=3), B.TE_ERR_ARG),
])
def test_gemm_panel_validation(kw, status):
    kw.setdefault("k", 128)
    assert _gemm(**kw) == status


def _mx_panel(fp4=False, **kw):
    args = dict(x=FAKE, x_dtype=B.TE_BF16, rows=256, cols=256, elem_dtype=B.TE_E4M3, out_row=FAKE,
                scale_row=FAKE, out_col=None, scale_col=None, stream=None)
    args.update(kw)
    if fp4:
        args.pop("elem_dtype")
        return B.lib().te_mxfp4_quantize_panel(*args.values())
    return B.lib().te_mxfp8_quantize_panel(*args.values())


@needs_lib
@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(x_dtype=B.TE_F32), B.TE_ERR_UNSUPPORTED),        # the panel path takes bf16 only
    (dict(rows=192), B.TE_ERR_UNSUPPORTED),                # whole 128 x 128 tiles only
    (dict(cols=160), B.TE_ERR_UNSUPPORTED),
    (dict(rows=-1), B.TE_ERR_SHAPE),
    (dict(out_row=None, scale_row=None), B.TE_ERR_NULL),    # both pairs NULL
    (dict(scale_row=None), B.TE_ERR_NULL),                  # a pair half NULL
    (dict(scale_row=FAKE_MIS), B.TE_ERR_ALIGN),
])
def test_mx_quantize_panel_validation(fp4, kw, status):
    assert _mx_panel(fp4, **kw) == status
    assert len(B.lib().te_get_last_error()) > 0


@needs_lib
def test_mx_scale_panel_bytes():
    L = B.lib()
    assert B.te_mx_scale_panel_bytes(256, 128) == 256 * 4
    assert B.te_mx_scale_panel_bytes(257, 128) == 512 * 4      # whole 256-row panels
    assert B.te_mx_scale_panel_bytes(15872, 4096) == 15872 * 128
    assert B.te_mx_scale_panel_bytes(0, 128) == 0
    assert B.te_mx_scale_panel_bytes(100, 96) == -1 and B.te_mx_scale_panel_bytes(-1, 128) == -1
    assert L.te_mx_scale_panel_bytes(300, 512) == 512 * 512 // 32


@needs_lib
def test_gemm_empty_is_ok_without_launch():
    assert _gemm(m=0) == B.TE_OK
    assert _gemm(n=0, a=None, b=None, d=None) == B.TE_OK


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), B.TE_ERR_SHAPE),
    (dict(x_dtype=B.TE_E4M3), B.TE_ERR_DTYPE),
    (dict(out_dtype=B.TE_BF16), B.TE_ERR_DTYPE),
    (dict(mode=5), B.TE_ERR_ARG),
    (dict(margin=-1), B.TE_ERR_ARG),
    (dict(scale=None), B.TE_ERR_NULL),
    (dict(amax=None), B.TE_ERR_NULL),
    (dict(x=FAKE_MIS), B.TE_ERR_ALIGN),
    (dict(out=FAKE_MIS), B.TE_ERR_ALIGN),
    (dict(workspace=None), B.TE_ERR_NULL),
    (dict(workspace=None, mode=B.TE_SCALE_CURRENT), B.TE_ERR_NULL),
    (dict(workspace=FAKE_MIS), B.TE_ERR_ALIGN),
])
def test_amax_cast_validation(kw, status):
    args = dict(x=FAKE, x_dtype=B.TE_BF16, rows=4, cols=4, out_dtype=B.TE_E4M3, mode=B.TE_SCALE_DELAYED,
                margin=0, scale=FAKE, scale_inv=FAKE, amax=FAKE, out=FAKE, workspace=FAKE, stream=None)
    args.update(kw)
    assert B.lib().te_amax_cast(*args.values()) == status


@needs_lib
def test_cast_transpose_needs_an_output():
    assert B.lib().te_cast_transpose(FAKE, B.TE_BF16, 4, 4, B.TE_E4M3, 0, 0, FAKE, FAKE, FAKE,
                                     None, None, FAKE, None) == B.TE_ERR_NULL
    # the amax workspace is required for every mode that reduces an amax
    for mode in (B.TE_SCALE_DELAYED, B.TE_SCALE_CURRENT):
        assert B.lib().te_cast_transpose(FAKE, B.TE_BF16, 4, 4, B.TE_E4M3, mode, 0, FAKE, FAKE, FAKE,
                                         FAKE, None, None, None) == B.TE_ERR_NULL


@needs_lib
def test_workspace_sizes():
    """The amax workspace is the 32 group lines and the top line of the grid-wide
    reduction (33 x 256 bytes); the dbias workspace is that plus one fp32 partial sum per
    128-row tile and column."""
    assert B.te_amax_workspace_bytes() == 33 * 256
    assert B.te_cast_transpose_dbias_workspace_bytes(128, 16) == 33 * 256 + 16 * 4
    assert B.te_cast_transpose_dbias_workspace_bytes(129, 16) == 33 * 256 + 2 * 16 * 4
    assert B.te_cast_transpose_dbias_workspace_bytes(0, 16) == 33 * 256
    assert B.te_cast_transpose_dbias_workspace_bytes(-1, 16) == -1


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), B.TE_ERR_SHAPE),
    (dict(hist_len=0), B.TE_ERR_SHAPE),
    (dict(fp8_dtype=B.TE_F32), B.TE_ERR_DTYPE),
    (dict(algo=3), B.TE_ERR_ARG),
    (dict(hist=None), B.TE_ERR_NULL),
])
def test_scale_update_validation(kw, status):
    args = dict(hist=FAKE, scale=FAKE, scale_inv=FAKE, n=4, hist_len=16, fp8_dtype=B.TE_E4M3,
                algo=B.TE_AMAX_MAX, margin=0, stream=None)
    args.update(kw)
    assert B.lib().te_scale_update(*args.values()) == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(cols=48), B.TE_ERR_SHAPE),
    (dict(out_row=None, scale_row=None, rows=48), B.TE_ERR_SHAPE),
    (dict(scale_row=None), B.TE_ERR_NULL),
    (dict(out_row=None, scale_row=None, out_col=None, scale_col=None), B.TE_ERR_NULL),
    (dict(elem_dtype=B.TE_E8M0), B.TE_ERR_DTYPE),
])
def test_mxfp8_validation(kw, status):
    args = dict(x=FAKE, x_dtype=B.TE_BF16, rows=64, cols=64, elem_dtype=B.TE_E4M3, out_row=FAKE,
                scale_row=FAKE, out_col=FAKE, scale_col=FAKE, stream=None)
    args.update(kw)
    assert B.lib().te_mxfp8_quantize(*args.values()) == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(cols=48), B.TE_ERR_SHAPE),
    (dict(scale_row=None), B.TE_ERR_NULL),
    (dict(dbias=None), B.TE_ERR_NULL),
    (dict(workspace=None), B.TE_ERR_ARG),
    (dict(workspace_bytes=64 * 4 - 4), B.TE_ERR_ARG),
    (dict(elem_dtype=B.TE_E8M0), B.TE_ERR_DTYPE),
])
def test_mxfp8_dbias_validation(kw, status):
    """te_mxfp8_quantize_dbias checks te_mxfp8_quantize's rules, then the bias gradient
    and its workspace (one fp32 partial per 128-row tile and column), on the host."""
    args = dict(x=FAKE, x_dtype=B.TE_BF16, rows=64, cols=64, elem_dtype=B.TE_E4M3, out_row=FAKE,
                scale_row=FAKE, out_col=FAKE, scale_col=FAKE, dbias=FAKE, workspace=FAKE, workspace_bytes=64 * 4,
                stream=None)
    args.update(kw)
    assert B.lib().te_mxfp8_quantize_dbias(*args.values()) == status


@needs_lib
def test_mxfp8_dbias_workspace_bytes():
    assert B.te_mxfp8_quantize_dbias_workspace_bytes(128, 16) == 16 * 4
    assert B.te_mxfp8_quantize_dbias_workspace_bytes(129, 16) == 2 * 16 * 4
    assert B.te_mxfp8_quantize_dbias_workspace_bytes(0, 16) == 0
    assert B.te_mxfp8_quantize_dbias_workspace_bytes(-1, 16) == -1


@needs_lib
def test_noalloc_dbias_rejects_shapes_above_its_scratch_before_any_launch():
    """Validation on the host: a shape whose partial sums exceed the static scratch is
    TE_ERR_SHAPE before any device call."""
    assert B.te_cast_transpose_dbias_noalloc_max_bytes() == 16 << 20
    st = B.lib().te_cast_transpose_dbias_noalloc(FAKE, B.TE_BF16, 40000, 16384, B.TE_E5M2, B.TE_SCALE_CURRENT, 0,
                                                 FAKE, FAKE, FAKE, None, FAKE, FAKE, None)
    assert st == B.TE_ERR_SHAPE and b"static maximum" in B.lib().te_get_last_error()
    st = B.lib().te_cast_transpose_dbias_noalloc(FAKE, B.TE_BF16, 64, 64, B.TE_E5M2, B.TE_SCALE_CURRENT, 0,
                                                 FAKE, FAKE, FAKE, None, FAKE, None, None)
    assert st == B.TE_ERR_NULL  # dbias required
