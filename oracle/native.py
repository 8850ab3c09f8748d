"""ctypes loader of the C++ oracle (oracle/cpp/nvfp4_oracle.cpp) -- TEST
INFRASTRUCTURE ONLY, like the rest of this package.

The C++ oracle is a second, independently written CPU implementation of the
NVFP4 quantizer (§2 "NVFP4 format") and of the NVFP4 Newton–Schulz iteration
(§3.4) of Full-Stack FP4 (arXiv 2607.04422), with OpenMP over the host's
cores; bench.py times it as the host baseline.  It is pinned by the same
fixtures and properties as the numpy oracle and cross-checked against it
(tests/test_oracle_native.py).  If the library is missing it is built with
g++ on first use.
"""
import ctypes
import os

import numpy as np

from .nvfp4 import NVFP4Tensor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "cpp", "libnvfp4_oracle.so")
_lib = None

_i64, _vp, _d, _i, _f = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int, ctypes.c_float


def lib():
    global _lib
    if _lib is None:
        src = os.path.join(HERE, "cpp", "nvfp4_oracle.cpp")
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(src):
            import importlib.util
            spec = importlib.util.spec_from_file_location("_orc_build", os.path.join(HERE, "cpp", "build.py"))
            mod = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(mod)
            mod.build()
        L = ctypes.CDLL(LIB)
        L.orc_threads.restype = _i
        L.orc_quantize_rows.argtypes = [_vp, _i, _i64, _i64, _d, _vp, _vp, _vp]
        L.orc_dequantize_rows.argtypes = [_vp, _vp, _f, _i64, _i64, _vp]
        L.orc_gemm_nt.argtypes = [_vp, _vp, _i64, _i64, _i64, _i, _vp]
        L.orc_ns_nvfp4.argtypes = [_vp, _i64, _i64, _vp, _i, _d, _vp]
        L.orc_ns_nvfp4_step.argtypes = [_vp, _i64, _i64, _d, _d, _d, _vp]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads():
    """OpenMP threads the oracle uses (all host cores unless OMP_NUM_THREADS)."""
    return int(lib().orc_threads())


def quantize_rows(t, amax=None):
    """Q_1x16(t) for a float32 or float64 matrix (amax: the tensor maximum to
    use, else the matrix's own)."""
    t = np.ascontiguousarray(t)
    if t.dtype not in (np.float32, np.float64):
        t = t.astype(np.float64)
    rows, cols = t.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    sg = np.empty(1, np.float32)
    lib().orc_quantize_rows(_p(t), 1 if t.dtype == np.float32 else 0, rows, cols,
                            float("nan") if amax is None else float(amax), _p(codes), _p(scales), _p(sg))
    return NVFP4Tensor(codes, scales, np.float32(sg[0]), rows, cols)


def dequantize_rows(q):
    out = np.empty((q.rows, q.cols), np.float64)
    lib().orc_dequantize_rows(_p(np.ascontiguousarray(q.codes)), _p(np.ascontiguousarray(q.scales)),
                              float(q.global_scale), q.rows, q.cols, _p(out))
    return out


def gemm_nt(P, Q, symmetric=False):
    P = np.ascontiguousarray(P, np.float64)
    Q = P if symmetric else np.ascontiguousarray(Q, np.float64)
    M, K = P.shape
    N = Q.shape[0]
    C = np.empty((M, N), np.float64)
    lib().orc_gemm_nt(_p(P), _p(Q), M, N, K, 1 if symmetric else 0, _p(C))
    return C


def ns_nvfp4(G, coeffs, clip=np.inf):
    G = np.ascontiguousarray(G, np.float64)
    m, n = G.shape
    c = np.ascontiguousarray(np.asarray(coeffs, np.float64).reshape(-1))
    out = np.empty((m, n), np.float64)
    lib().orc_ns_nvfp4(_p(G), m, n, _p(c), len(c) // 3, float(clip), _p(out))
    return out


def ns_nvfp4_step(X, a, b, c):
    X = np.ascontiguousarray(X, np.float64)
    m, n = X.shape
    out = np.empty((m, n), np.float64)
    lib().orc_ns_nvfp4_step(_p(X), m, n, float(a), float(b), float(c), _p(out))
    return out
