"""The C-ABI library loads and exports every entry point of include/qsg.h,
and its host-side argument validation rejects bad calls before any launch
(these calls never reach the GPU)."""

import ctypes
import os
import re

import pytest

from helpers import ROOT, build_library, lib_is_stale

HEADER = os.path.join(ROOT, "include", "qsg.h")


@pytest.fixture(scope="module")
def lib():
    if lib_is_stale():
        build_library()
    import quantize_scaled_gemm_amd as q

    return q.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsg_\w+)\s*\(", text)))


def test_header_declares_the_binding_entry_points():
    import quantize_scaled_gemm_amd as q

    assert declared_functions() == sorted(q.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_version_and_status_strings(lib):
    assert lib.qsg_version() == 100
    assert lib.qsg_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4, -5):
        assert lib.qsg_status_string(code) not in (b"ok", b"unknown status")
    assert lib.qsg_status_string(-99) == b"unknown status"


def test_validation_rejects_before_launch(lib):
    import quantize_scaled_gemm_amd as q

    R = q.Recipe
    # bad dtype / null input / negative shapes
    assert lib.qsg_amax(None, 7, 4, 4, 4, None, None) == -1
    assert lib.qsg_amax(None, 1, 4, 4, 4, 16, None) == -1
    assert lib.qsg_amax(16, 1, -1, 4, 4, 16, None) == -1
    assert b"negative" in lib.qsg_last_error()
    # ld < cols
    assert lib.qsg_cast_transpose(16, 1, 4, 8, 4, 0, 16, 32, None, None, None) == -1
    # misaligned fp32 input
    assert lib.qsg_cast_transpose(18, 0, 4, 8, 8, 0, 16, 32, None, None, None) == -3
    # both outputs null
    assert lib.qsg_cast_transpose(16, 1, 4, 8, 8, 0, 16, None, None, None, None) == -1
    # bad format, margin outside [0, 64]
    assert lib.qsg_compute_scale(16, 5, 0, 16, 16, None) == -1
    assert lib.qsg_compute_scale(16, 0, 65, 16, 16, None) == -1
    # history length, algorithm
    assert lib.qsg_amax_update(16, 0, 0, 16, 0, 0, 0, 16, 16, None) == -1
    assert lib.qsg_amax_update(16, 4, 0, 16, 1, 0, 0, 16, 16, None) == -4
    # recipe shape rules
    rec = R(q.MXFP8, q.E4M3, 0, q.MX_CEIL)
    assert lib.qsg_quantize(16, 1, 64, 48, 48, ctypes.byref(rec), 32, 48, None, None, None) == -2
    rec = R(q.BLOCK_128X128, q.E4M3, 0, 0)
    assert lib.qsg_quantize(16, 1, 128, 192, 192, ctypes.byref(rec), 32, 48, None, None, None) == -2
    rec = R(q.DELAYED, q.E4M3, 0, 0)
    assert lib.qsg_quantize(16, 1, 128, 128, 128, ctypes.byref(rec), 32, 48, None, None, None) == -4
    # GEMM scale-kind pairs and shape rules
    g = lib.qsg_scaled_gemm
    assert g(16, 0, q.MXFP8, 16, 16, 0, q.TENSORWISE, 16, 4, 4, 64, 64, 64, 16, 1, 4, None) == -4
    assert g(16, 0, q.MXFP8, 16, 16, 0, q.MXFP8, 16, 4, 4, 48, 64, 64, 16, 1, 4, None) == -2
    assert g(16, 0, q.BLOCK_1X128, 16, 16, 0, q.BLOCK_128X128, 16, 4, 4, 64, 64, 64, 16, 1, 4, None) == -2
    assert g(16, 0, 9, 16, 16, 0, 0, 16, 4, 4, 64, 64, 64, 16, 1, 4, None) == -1
    assert g(16, 0, 0, 16, 16, 0, 0, 16, 4, 4, 64, 32, 64, 16, 1, 4, None) == -1  # lda < K
    # empty GEMM: nothing to do, no launch
    assert g(None, 0, 0, None, None, 0, 0, None, 0, 4, 64, 64, 64, None, 1, 4, None) == 0
