"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/fp8w8a8.h declares, and rejects bad arguments before any launch.

Fake device addresses below are never dereferenced: every call here returns from
the argument checks, which run on the host before the device is touched.
"""

import ctypes
import os
import re

import pytest

from fp8_w8a8_quantized_token_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp8w8a8.h")

ALIGNED = 0x10000          # a 64 KiB-aligned fake address
MIS16 = 0x10008            # 8-byte but not 16-byte aligned
MIS4 = 0x10002             # 2-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(fp8\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_header_declares_expected_api():
    names = declared_functions()
    for must in ("fp8_quant_rows", "fp8_quant_weights_per_channel", "fp8_linear_create", "fp8_linear_run",
                 "fp8_linear_destroy", "fp8_linear", "fp8w8a8_status_string", "fp8_linear_workspace_bytes"):
        assert must in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    codes = [_lib.OK, _lib.ERR_INVALID_ARG, _lib.ERR_BAD_SHAPE, _lib.ERR_MISALIGNED, _lib.ERR_BAD_DEVICE,
             _lib.ERR_WORKSPACE_TOO_SMALL, _lib.ERR_HIP, _lib.ERR_CAPTURE, _lib.ERR_TOO_LARGE]
    texts = [lib.fp8w8a8_status_string(c).decode() for c in codes]
    assert len(set(texts)) == len(codes)
    assert lib.fp8w8a8_status_string(12345).decode() == "unknown status"


def q(lib, x, rows, cols, qo, s):
    return lib.fp8_quant_rows(x, rows, cols, qo, s, None)


def test_quant_rows_validation(lib):
    A = ALIGNED
    assert q(lib, None, 4, 16, A, A) == _lib.ERR_INVALID_ARG
    assert q(lib, A, 4, 16, None, A) == _lib.ERR_INVALID_ARG
    assert q(lib, A, 4, 16, A, None) == _lib.ERR_INVALID_ARG
    assert q(lib, A, -1, 16, A, A) == _lib.ERR_BAD_SHAPE
    assert q(lib, A, _lib.MAX_ROWS, 16, A, A) == _lib.ERR_BAD_SHAPE
    for cols in (0, 8, 24, 17, _lib.MAX_DIM + 16):
        assert q(lib, A, 4, cols, A, A) == _lib.ERR_BAD_SHAPE, cols
    assert q(lib, MIS16, 4, 16, A, A) == _lib.ERR_MISALIGNED
    assert q(lib, A, 4, 16, MIS16, A) == _lib.ERR_MISALIGNED
    assert q(lib, A, 4, 16, A, MIS4) == _lib.ERR_MISALIGNED
    assert q(lib, A, 0, 16, A, A) == _lib.OK  # empty activation: a no-op, nothing launched


def test_quant_weights_validation(lib):
    A = ALIGNED
    f = lib.fp8_quant_weights_per_channel
    assert f(A, 0, 16, A, A, None) == _lib.ERR_BAD_SHAPE  # an empty weight is invalid input
    assert f(A, 16, 0, A, A, None) == _lib.ERR_BAD_SHAPE
    assert f(None, 16, 16, A, A, None) == _lib.ERR_INVALID_ARG


def create(lib, n, k, w=ALIGNED, ws=ALIGNED, bias=None, out=True):
    plan = ctypes.c_void_p()
    st = lib.fp8_linear_create(0, n, k, w, ws, bias, ctypes.byref(plan) if out else None)
    return st, plan


def test_create_validation(lib):
    assert create(lib, 16, 16, out=False)[0] == _lib.ERR_INVALID_ARG
    assert create(lib, 16, 16, w=None)[0] == _lib.ERR_INVALID_ARG
    assert create(lib, 16, 16, ws=None)[0] == _lib.ERR_INVALID_ARG
    for n, k in ((0, 16), (16, 0), (8, 16), (16, 8), (24, 32), (32, 40), (_lib.MAX_DIM + 16, 16)):
        assert create(lib, n, k)[0] == _lib.ERR_BAD_SHAPE, (n, k)
    assert create(lib, 16, 16, w=MIS16)[0] == _lib.ERR_MISALIGNED
    assert create(lib, 16, 16, ws=MIS16)[0] == _lib.ERR_MISALIGNED
    assert create(lib, 16, 16, bias=MIS16)[0] == _lib.ERR_MISALIGNED
    st, plan = create(lib, 16, 16)
    assert plan.value is None or st == _lib.OK
    if st != _lib.OK:  # no usable gfx950 device here: the device check, not a crash
        assert st in (_lib.ERR_HIP, _lib.ERR_BAD_DEVICE)
    else:
        lib.fp8_linear_destroy(plan)


def test_run_and_helpers_validation(lib):
    A = ALIGNED
    assert lib.fp8_linear_run(None, 4, A, _lib.A_BF16, None, A, A, 1 << 20, None) == _lib.ERR_INVALID_ARG
    assert lib.fp8_linear_workspace_bytes(None, 128) == 0
    lib.fp8_linear_destroy(None)  # NULL is ignored
    cid, tm, tn, wg = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    assert lib.fp8_linear_plan_config(None, 4, ctypes.byref(cid), ctypes.byref(tm), ctypes.byref(tn),
                                      ctypes.byref(wg)) == _lib.ERR_INVALID_ARG
    n = lib.fp8_gemm_config_count()
    assert n >= 1
    args = (4, 16, 16, A, A, A, A, None, A, None)
    assert lib.fp8_gemm_run_config(-1, *args) == _lib.ERR_INVALID_ARG
    assert lib.fp8_gemm_run_config(n, *args) == _lib.ERR_INVALID_ARG
    assert lib.fp8_gemm_run_config(0, 4, 16, 24, A, A, A, A, None, A, None) == _lib.ERR_BAD_SHAPE
    assert lib.fp8_gemm_run_config(0, 4, 16, 16, MIS16, A, A, A, None, A, None) == _lib.ERR_MISALIGNED
    assert lib.fp8_gemm_run_config(0, 0, 16, 16, A, A, A, A, None, A, None) == _lib.OK  # m == 0 no-op
    # one-shot entry: shape checks before any device work
    assert lib.fp8_linear(A, _lib.A_BF16, None, 4, 24, 16, A, A, None, A, A, 1 << 20, None) == _lib.ERR_BAD_SHAPE


def test_quant_gemm_validation(lib):
    A = ALIGNED
    need = lib.fp8_quant_gemm_workspace_bytes(300, 400)
    # codes and scales each rounded up to 256 bytes, then 1024 launch flags of 8 bytes
    assert need == 120064 + 1280 + 8192
    assert lib.fp8_quant_gemm_workspace_bytes(0, 400) == 0
    ok = (300, 272, 400, A, A, A, A, A, A, need, None)
    bad = lambda **kw: lib.fp8_quant_gemm(*[kw.get(f, v) for f, v in zip(
        ("m", "n", "k", "a", "w", "ws", "b", "out", "work", "bytes", "stream"), ok)])
    assert bad(a=None) == _lib.ERR_INVALID_ARG
    assert bad(out=None) == _lib.ERR_INVALID_ARG
    assert bad(work=None) == _lib.ERR_INVALID_ARG
    assert bad(w=None) == _lib.ERR_INVALID_ARG
    assert bad(k=24) == _lib.ERR_BAD_SHAPE
    assert bad(n=8) == _lib.ERR_BAD_SHAPE
    assert bad(m=-1) == _lib.ERR_BAD_SHAPE
    assert bad(a=MIS16) == _lib.ERR_MISALIGNED
    assert bad(work=A + 128) == _lib.ERR_MISALIGNED
    assert bad(bytes=need - 1) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert bad(m=0, bytes=0) == _lib.OK  # m == 0 is a no-op


def test_binding_refuses_cpu_tensors():
    import torch
    from fp8_w8a8_quantized_token_amd import quant_rows
    with pytest.raises(ValueError, match="GPU tensor"):
        quant_rows(torch.zeros((4, 16), dtype=torch.bfloat16))


def test_act_producers_validation(lib):
    A = ALIGNED
    tb = lib.fp8_act_table_build
    for bad in (0, 4, -1):
        assert tb(bad, A, None) == _lib.ERR_INVALID_ARG, bad
    assert tb(_lib.ACT_SILU, None, None) == _lib.ERR_INVALID_ARG
    assert tb(_lib.ACT_GELU_ERF, MIS16, None) == _lib.ERR_MISALIGNED

    ar = lib.fp8_act_rows
    assert ar(None, 4, 16, A, A, None) == _lib.ERR_INVALID_ARG
    assert ar(A, 4, 16, None, A, None) == _lib.ERR_INVALID_ARG
    assert ar(A, 4, 16, A, None, None) == _lib.ERR_INVALID_ARG
    for cols in (0, 8, 24, _lib.MAX_DIM + 16):
        assert ar(A, 4, cols, A, A, None) == _lib.ERR_BAD_SHAPE, cols
    assert ar(A, -1, 16, A, A, None) == _lib.ERR_BAD_SHAPE
    assert ar(MIS16, 4, 16, A, A, None) == _lib.ERR_MISALIGNED
    assert ar(A, 4, 16, MIS16, A, None) == _lib.ERR_MISALIGNED
    assert ar(A, 4, 16, A, MIS16, None) == _lib.ERR_MISALIGNED
    assert ar(A, 0, 16, A, A, None) == _lib.OK

    aq = lib.fp8_act_quant_rows
    assert aq(A, 4, 16, None, A, A, None) == _lib.ERR_INVALID_ARG
    assert aq(None, 4, 16, A, A, A, None) == _lib.ERR_INVALID_ARG
    assert aq(A, 4, 16, A, A, None, None) == _lib.ERR_INVALID_ARG
    assert aq(A, 4, 24, A, A, A, None) == _lib.ERR_BAD_SHAPE
    assert aq(A, 4, 16, MIS16, A, A, None) == _lib.ERR_MISALIGNED
    assert aq(A, 4, 16, A, A, MIS4, None) == _lib.ERR_MISALIGNED
    assert aq(A, 0, 16, A, A, A, None) == _lib.OK


def test_act_binding_rejects_unknown_kind():
    from fp8_w8a8_quantized_token_amd import act_table
    with pytest.raises(ValueError, match="unknown activation"):
        act_table("relu", device="cpu")


def test_w8a16_validation(lib):
    A = ALIGNED
    plan = ctypes.c_void_p()
    assert lib.fp8_w8a16_create(0, 16, 16, 0, A, A, None, None) == _lib.ERR_INVALID_ARG
    assert lib.fp8_w8a16_create(0, 16, 16, 0, None, A, None, ctypes.byref(plan)) == _lib.ERR_INVALID_ARG
    assert lib.fp8_w8a16_create(0, 16, 16, 7, A, A, None, ctypes.byref(plan)) == _lib.ERR_INVALID_ARG
    for n, k in ((0, 16), (16, 0), (24, 32), (16, 40)):
        assert lib.fp8_w8a16_create(0, n, k, 1, A, A, None, ctypes.byref(plan)) == _lib.ERR_BAD_SHAPE, (n, k)
    assert lib.fp8_w8a16_create(0, 16, 16, 0, MIS16, A, None, ctypes.byref(plan)) == _lib.ERR_MISALIGNED
    assert lib.fp8_w8a16_run(None, 4, A, A, None) == _lib.ERR_INVALID_ARG
    lib.fp8_w8a16_destroy(None)
    n = lib.fp8_w8a16_config_count()
    assert n >= 1
    args = (0, 4, 16, 16, A, A, A, None, A, None)
    assert lib.fp8_w8a16_run_config(-1, *args) == _lib.ERR_INVALID_ARG
    assert lib.fp8_w8a16_run_config(n, *args) == _lib.ERR_INVALID_ARG
    assert lib.fp8_w8a16_run_config(0, 3, 4, 16, 16, A, A, A, None, A, None) == _lib.ERR_INVALID_ARG
    assert lib.fp8_w8a16_run_config(0, 0, 4, 16, 24, A, A, A, None, A, None) == _lib.ERR_BAD_SHAPE
    assert lib.fp8_w8a16_run_config(0, 1, 4, 16, 16, MIS16, A, A, None, A, None) == _lib.ERR_MISALIGNED
    assert lib.fp8_w8a16_run_config(0, 0, 0, 16, 16, A, A, A, None, A, None) == _lib.OK


def test_tensor_quant_validation(lib):
    A = ALIGNED
    ws = lib.fp8_quant_tensor_workspace_bytes()
    assert ws >= 16
    f = lib.fp8_quant_tensor
    assert f(None, 16, 0, A, A, A, ws, None) == _lib.ERR_INVALID_ARG
    assert f(A, 16, 2, A, A, A, ws, None) == _lib.ERR_INVALID_ARG
    assert f(A, 16, 0, A, None, A, ws, None) == _lib.ERR_INVALID_ARG
    assert f(A, 16, 0, A, A, None, ws, None) == _lib.ERR_INVALID_ARG
    for numel in (8, 24, -16):
        assert f(A, numel, 0, A, A, A, ws, None) == _lib.ERR_BAD_SHAPE, numel
    assert f(MIS16, 16, 1, A, A, A, ws, None) == _lib.ERR_MISALIGNED
    assert f(A, 16, 1, A, MIS4 + 1, A, ws, None) == _lib.ERR_MISALIGNED
    assert f(A, 16, 1, A, A, A, ws - 4, None) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert f(A, 0, 1, A, A, A, ws, None) == _lib.OK
    d = lib.fp8_dequant_tensor
    assert d(A, 16, 5, A, A, None) == _lib.ERR_INVALID_ARG
    assert d(A, 16, 0, None, A, None) == _lib.ERR_INVALID_ARG
    assert d(A, 20, 0, A, A, None) == _lib.ERR_BAD_SHAPE
    assert d(A, 16, 0, A, MIS16, None) == _lib.ERR_MISALIGNED
    assert d(A, 0, 0, A, A, None) == _lib.OK


def test_noalloc_run_validation(lib):
    # checks that need no plan and no device: every call below returns before any HIP call
    A = ALIGNED
    assert _lib.NOALLOC_SCRATCH_BYTES == 80 << 20
    assert lib.fp8_linear_run_noalloc(None, 4, A, _lib.A_BF16, None, A, None) == _lib.ERR_INVALID_ARG
    assert lib.fp8_linear_run_noalloc(None, 4, A, _lib.A_E4M3, A, A, None) == _lib.ERR_INVALID_ARG


def test_run_group_validation(lib):
    """The group entry point rejects NULL arrays, NULL elements and a group size outside
    1..FP8W8A8_MAX_GROUP before it reads any plan."""
    A = ALIGNED
    assert re.search(r"#define FP8W8A8_MAX_GROUP (\d+)", open(HEADER).read()).group(1) == str(_lib.MAX_GROUP)
    g = lib.fp8_linear_run_group
    nulls = (ctypes.c_void_p * 2)(None, None)
    outs = (ctypes.c_void_p * 2)(A, A)
    arr = lambda x: ctypes.cast(x, ctypes.c_void_p)  # noqa: E731
    assert g(None, 1, 4, A, _lib.A_BF16, None, arr(outs), A, 1 << 20, None) == _lib.ERR_INVALID_ARG
    assert g(arr(nulls), 2, 4, A, _lib.A_BF16, None, None, A, 1 << 20, None) == _lib.ERR_INVALID_ARG
    assert g(arr(nulls), 2, 4, None, _lib.A_BF16, None, arr(outs), A, 1 << 20, None) == _lib.ERR_INVALID_ARG
    assert g(arr(nulls), 2, 4, A, _lib.A_BF16, None, arr(outs), A, 1 << 20, None) == _lib.ERR_INVALID_ARG
    five = (ctypes.c_void_p * 5)(A, A, A, A, A)
    for n in (0, -1, _lib.MAX_GROUP + 1):
        assert g(arr(five), n, 4, A, _lib.A_BF16, None, arr(five), A, 1 << 20, None) == _lib.ERR_INVALID_ARG, n


def test_group_config_validation(lib):
    """The group-configuration query rejects NULL arrays, elements and outputs and a group
    size outside 1..FP8W8A8_MAX_GROUP before it reads any plan."""
    q = lib.fp8_linear_group_config
    cid = ctypes.c_int(123)
    nulls = (ctypes.c_void_p * 2)(None, None)
    arr = lambda x: ctypes.cast(x, ctypes.c_void_p)  # noqa: E731
    assert q(None, 1, 4, ctypes.byref(cid)) == _lib.ERR_INVALID_ARG
    assert q(arr(nulls), 2, 4, ctypes.byref(cid)) == _lib.ERR_INVALID_ARG
    five = (ctypes.c_void_p * 5)(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED)
    assert q(arr(five), 1, 4, None) == _lib.ERR_INVALID_ARG
    for n in (0, -1, _lib.MAX_GROUP + 1):
        assert q(arr(five), n, 4, ctypes.byref(cid)) == _lib.ERR_INVALID_ARG, n
    assert cid.value == 123  # nothing written on an error


def test_group_binding_rejects_bad_groups():
    from fp8_w8a8_quantized_token_amd import linear_group

    with pytest.raises(ValueError):
        linear_group([], None)
    with pytest.raises(ValueError):
        linear_group([object()] * (_lib.MAX_GROUP + 1), None)


def test_quant_tensor_form_validation(lib):
    A = ALIGNED
    f = lib.fp8_quant_tensor_form
    for form in (-1, 4, 99):
        assert f(form, A, 16, 0, A, A, A, 4096, None) == _lib.ERR_INVALID_ARG, form
    for form in _lib.TENSOR_FORMS.values():
        assert f(form, A, 20, 0, A, A, A, 4096, None) == _lib.ERR_BAD_SHAPE, form
        assert f(form, A, 0, 0, A, A, A, 4096, None) == _lib.OK, form  # empty: a no-op
    assert re.search(r"#define FP8W8A8_TENSOR_FORM_ONE_PASS_NO_WAIT (\d+)", open(HEADER).read()).group(1) == "3"
