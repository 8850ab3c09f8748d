"""The C-ABI library loads and exports what include/nvfp4ns.h declares;
host-side validation answers without touching a GPU (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4ns.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(?:ns_status|size_t)\s+(\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm", "ns_workspace_bytes",
                 "ns_orthogonalize", "ns_orthogonalize_grouped"):
        assert want in names


def test_library_exports_every_declared_symbol():
    ns = pytest.importorskip("newton_schulz_amd")
    lib = ctypes.CDLL(ns.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in ns.EXPORTED, name


def test_workspace_sizes_and_validation_on_host():
    ns = pytest.importorskip("newton_schulz_amd")
    lib = ns._lib
    assert lib.ns_workspace_bytes(3072, 8192) == lib.ns_workspace_bytes(8192, 3072)
    wb = lib.ns_workspace_bytes(3072, 8192)
    # X, A, B in fp32 and four packed NVFP4 tensors (215 MB)
    assert 215e6 < wb < 320e6 and wb % 256 == 0
    assert lib.ns_workspace_bytes(3072, 8190) == 0
    assert lib.nvfp4_quantize_workspace_bytes(16, 16) >= 4
    coeffs = (ctypes.c_float * 3)(3.4445, -4.775, 2.0315)
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    other = ctypes.c_void_p(0x100000000)
    # null input
    assert lib.ns_orthogonalize(None, 0, 32, 32, coeffs, 1, 1.0, other, 0, fake, wb, None) == ns.NS_ERR_ARG
    # shape not a multiple of 16
    assert lib.ns_orthogonalize(fake, 0, 30, 32, coeffs, 1, 1.0, other, 0, fake, wb, None) == ns.NS_ERR_SHAPE
    # k <= 0, clip <= 0, clip NaN
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 0, 1.0, other, 0, fake, wb, None) == ns.NS_ERR_ARG
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 1, 0.0, other, 0, fake, wb, None) == ns.NS_ERR_ARG
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 1, float("nan"), other, 0, fake, wb, None) == ns.NS_ERR_ARG
    # out overlapping G
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 1, 1.0, fake, 0, fake, wb, None) == ns.NS_ERR_ARG
    # workspace too small
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 1, 1.0, other, 0, fake, 16, None) == ns.NS_ERR_WORKSPACE
    # quantizer: bad axis, bad shape, no workspace
    assert lib.nvfp4_quantize(fake, 0, 16, 16, 7, fake, fake, fake, fake, 256, None) == ns.NS_ERR_ARG
    assert lib.nvfp4_quantize(fake, 0, 16, 24, 0, fake, fake, fake, fake, 256, None) == ns.NS_ERR_SHAPE
    assert lib.nvfp4_quantize(fake, 0, 16, 16, 0, fake, fake, fake, None, 256, None) == ns.NS_ERR_WORKSPACE
    # symmetric GEMM with different operands
    assert lib.nvfp4_gemm(fake, fake, fake, other, fake, fake, 32, 32, 32, 1, 1.0, 0.0,
                          None, fake, None, None, 0, None) == ns.NS_ERR_ARG
    # beta != 0 without an addend
    assert lib.nvfp4_gemm(fake, fake, fake, fake, fake, fake, 32, 32, 32, 0, 1.0, 2.0,
                          None, fake, None, None, 0, None) == ns.NS_ERR_ARG
    # the 3072^2 x 8192 Gram product has 300 tiles for 8 XCDs of 32 CUs: the
    # tiles left over after one per CU are split along K, which needs a
    # workspace, and a too-small one is refused
    wsg = lib.nvfp4_gemm_workspace_bytes(3072, 3072, 8192, 1)
    assert wsg > 0
    assert lib.nvfp4_gemm(fake, fake, fake, fake, fake, fake, 3072, 3072, 8192, 1, 1.0, 0.0,
                          None, other, None, fake, wsg - 1, None) == ns.NS_ERR_WORKSPACE
    # 3072 x 8192 x 3072 has 1536 tiles, six per CU: nothing is split
    assert lib.nvfp4_gemm_workspace_bytes(3072, 8192, 3072, 0) == 0
