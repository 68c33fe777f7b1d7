"""TEST INFRASTRUCTURE ONLY -- the CPU oracle for C = alpha*A.B + beta*C0.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package.  The GPU product path (``tile_scheduled_dense_amd``)
never imports it, and the two share no code.

The arithmetic lives in ``oracle_gemm.c`` (plain C, binary64, k increasing),
built with gcc into ``liboracle_gemm.so`` beside it.  This module only marshals
numpy arrays into that library.  See the C file's header for the passages of
the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_gemm.c")
LIB = os.path.join(HERE, "liboracle_gemm.so")

F32, BF16, F16 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "bf16": BF16, "f16": F16}


def compile_library(src: str, out: str, verbose: bool = False) -> str:
    """gcc, binary64, no fast-math and no FP contraction."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-std=c11", "-Wall", "-o", f"{out}.{os.getpid()}.tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(f"{out}.{os.getpid()}.tmp", out)   # per-process name: parallel test workers may build at once
    return out


def build(verbose: bool = False) -> str:
    return compile_library(SRC, LIB, verbose)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _code(dtype):
    return DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)


def _f32_or_none(x):
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype != np.float32:
        raise TypeError("the bias is float32 storage")
    return x


def _check_storage(x, code):
    want = np.float32 if code == F32 else np.uint16
    if x is not None and (x.dtype != want or not x.flags.c_contiguous):
        raise TypeError(f"oracle expects contiguous {want.__name__} storage, got {x.dtype}")


class OracleLibrary:
    """ctypes view of one built copy of oracle_gemm.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.oracle_gemm.argtypes = [i64, i64, i64, i64, ctypes.c_int,
                                    vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                    dbl, dbl, vp, i64, i64, vp]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm_points.argtypes = [i64, i64, i64, i64, ctypes.c_int,
                                           vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                           dbl, dbl, i64, vp, vp, vp, vp, vp]
        lib.oracle_gemm_points.restype = ctypes.c_int
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = dbl
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_f16.restype = dbl
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        lib.oracle_tail.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, ctypes.c_int, ctypes.c_int,
                                    vp, i64, i64, dbl]
        lib.oracle_tail.restype = ctypes.c_int
        lib.oracle_tail_points.argtypes = [i64, vp, vp, vp, vp, vp, i64, ctypes.c_int, ctypes.c_int,
                                           vp, i64, i64, dbl]
        lib.oracle_tail_points.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def gemm(self, M, N, K, dtype, A, lda, B, ldb, C0=None, ldc=None, alpha=1.0, beta=0.0,
             batch=1, strideA=0, strideB=0, strideC=0, with_absden=False, bias=None, bias_stride=0,
             bias_mode=0, activation=0):
        """Full result as float64 (batch, M, N); with_absden adds sum_k |a||b|.

        A, B: flat numpy storage (uint16 bit patterns for bf16/f16, float32 for
        f32) indexed A[b*strideA + i*lda + k], B[b*strideB + k*ldb + j].  C0:
        float32 flat, C0[b*strideC + i*ldc + j], not read when beta == 0.
        """
        code = _code(dtype)
        _check_storage(A, code)
        _check_storage(B, code)
        ldc = max(N, 1) if ldc is None else ldc
        if beta != 0.0 and (C0 is None or C0.dtype != np.float32):
            raise TypeError("beta != 0 needs a float32 C0")
        out = np.empty((batch, M, N), dtype=np.float64)
        den = np.empty((batch, M, N), dtype=np.float64) if with_absden else None
        tail = bias_mode != 0 or activation != 0
        # with a fused tail the contraction runs with beta = 0 and the tail adds beta * C0
        rc = self.lib.oracle_gemm(batch, M, N, K, code, _ptr(A), lda, strideA, _ptr(B), ldb, strideB,
                                  _ptr(C0) if beta != 0.0 and not tail else None, ldc, strideC,
                                  float(alpha), 0.0 if tail else float(beta), _ptr(out), max(N, 1), M * N,
                                  _ptr(den))
        if rc != 0:
            raise ValueError(f"oracle_gemm rejected its arguments (rc={rc})")
        if tail:
            bias = _f32_or_none(bias)
            rc = self.lib.oracle_tail(batch, M, N, _ptr(out), max(N, 1), M * N, _ptr(bias), int(bias_stride),
                                      int(bias_mode), int(activation), _ptr(C0) if beta != 0.0 else None, ldc,
                                      strideC, float(beta))
            if rc != 0:
                raise ValueError(f"oracle_tail rejected its arguments (rc={rc})")
        return (out, den) if with_absden else out

    def gemm_points(self, M, N, K, dtype, A, lda, B, ldb, pts, C0=None, ldc=None, alpha=1.0,
                    beta=0.0, batch=1, strideA=0, strideB=0, strideC=0, bias=None, bias_stride=0,
                    bias_mode=0, activation=0):
        """Values and sum_k |a||b| at sampled outputs pts = int64 (P, 3) of (b, i, j)."""
        code = _code(dtype)
        _check_storage(A, code)
        _check_storage(B, code)
        ldc = max(N, 1) if ldc is None else ldc
        pts = np.ascontiguousarray(pts, dtype=np.int64).reshape(-1, 3)
        pb, pi, pj = (np.ascontiguousarray(pts[:, c]) for c in range(3))
        out = np.empty(len(pts), dtype=np.float64)
        den = np.empty(len(pts), dtype=np.float64)
        tail = bias_mode != 0 or activation != 0
        rc = self.lib.oracle_gemm_points(batch, M, N, K, code, _ptr(A), lda, strideA, _ptr(B), ldb,
                                         strideB, _ptr(C0) if beta != 0.0 and not tail else None, ldc, strideC,
                                         float(alpha), 0.0 if tail else float(beta), len(pts), _ptr(pb),
                                         _ptr(pi), _ptr(pj), _ptr(out), _ptr(den))
        if rc != 0:
            raise ValueError(f"oracle_gemm_points rejected its arguments (rc={rc})")
        if tail:
            bias = _f32_or_none(bias)
            rc = self.lib.oracle_tail_points(len(pts), _ptr(pb), _ptr(pi), _ptr(pj), _ptr(out), _ptr(bias),
                                             int(bias_stride), int(bias_mode), int(activation),
                                             _ptr(C0) if beta != 0.0 else None, ldc, strideC, float(beta))
            if rc != 0:
                raise ValueError(f"oracle_tail_points rejected its arguments (rc={rc})")
        return out, den

    def decode(self, bits, dtype):
        fn = self.lib.oracle_decode_bf16 if dtype == "bf16" else self.lib.oracle_decode_f16
        return np.array([fn(int(b)) for b in np.asarray(bits).ravel()], dtype=np.float64)

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))


_default = None


def _lib() -> OracleLibrary:
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = OracleLibrary(LIB)
    return _default


def load() -> OracleLibrary:
    """The oracle library, compiled first if missing or older than its source.  Call it before
    the process opens the GPU: compiling starts gcc, and a process that has the GPU open starts
    no other program."""
    return _lib()


def gemm(*a, **kw):
    return _lib().gemm(*a, **kw)


def gemm_points(*a, **kw):
    return _lib().gemm_points(*a, **kw)


def decode(bits, dtype):
    return _lib().decode(bits, dtype)


def max_threads() -> int:
    return _lib().max_threads()


def set_threads(n: int) -> None:
    _lib().set_threads(n)
