"""ctypes marshalling for oracle.c (test infrastructure only; no arithmetic here).

Arrays cross the boundary as raw bit patterns: bf16 and fp16 values travel as
uint16 arrays, packed int4 weights as uint8 arrays, int8 weights as int8 and
their fp32 scales as float32 arrays; results come back as fp64.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force=True):
    """Compile oracle.c with gcc.  -O2 without -ffast-math: fp64 sums keep their
    written order (no reassociation, no contraction into fused multiply-adds)."""
    if not force and os.path.exists(LIB_PATH) and \
            os.path.getmtime(LIB_PATH) >= os.path.getmtime(SRC_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC",
                           "-shared", SRC_PATH, "-o", tmp, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        build()
    _lib = open_lib(LIB_PATH)
    return _lib


def use(lib):
    """Make ``lib`` (from open_lib) the library every call goes through; returns
    the previous one.  Lets a test run the pins against a deliberately broken
    build of oracle.c."""
    global _lib
    prev, _lib = _lib, lib
    return prev


def open_lib(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_f16_value.argtypes = [ctypes.c_uint16]
    lib.orc_f16_value.restype = ctypes.c_double
    lib.orc_f16_from_f64.argtypes = [ctypes.c_double]
    lib.orc_f16_from_f64.restype = ctypes.c_uint16
    lib.orc_gemm_dense.argtypes = [P, P, I64, I64, I64, P, P]
    lib.orc_gemm_dense.restype = None
    lib.orc_gemm_f64w.argtypes = [P, P, I64, I64, I64, P, P]
    lib.orc_gemm_f64w.restype = None
    lib.orc_dequant_q4g64.argtypes = [P, P, I64, I64, P]
    lib.orc_dequant_q4g64.restype = None
    lib.orc_gemm_q4g64.argtypes = [P, P, P, I64, I64, I64, P, P]
    lib.orc_gemm_q4g64.restype = None
    lib.orc_quantize_q4g64.argtypes = [P, I64, I64, P, P]
    lib.orc_quantize_q4g64.restype = None
    lib.orc_quantize_i8.argtypes = [P, I64, I64, P, P]
    lib.orc_quantize_i8.restype = None
    lib.orc_dequant_i8.argtypes = [P, P, I64, I64, P]
    lib.orc_dequant_i8.restype = None
    lib.orc_gemm_i8.argtypes = [P, P, P, I64, I64, I64, P, P]
    lib.orc_gemm_i8.restype = None
    lib.orc_swiglu.argtypes = [P, P, I64, P]
    lib.orc_swiglu.restype = None
    lib.orc_residual_add.argtypes = [P, P, I64, P]
    lib.orc_residual_add.restype = None
    lib.orc_bf16_from_f64.argtypes = [ctypes.c_double]
    lib.orc_bf16_from_f64.restype = ctypes.c_uint16
    lib.orc_rmsnorm.argtypes = [P, P, I64, I64, ctypes.c_double, P]
    lib.orc_rmsnorm.restype = None
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s array, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def bf16_value(bits):
    """Exact values of bf16 bit patterns (any shape) as fp64."""
    lib = load()
    b = _c(bits, np.uint16)
    return np.array([lib.orc_bf16_value(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)


def f16_value(bits):
    """Exact values of fp16 bit patterns (any shape) as fp64."""
    lib = load()
    b = _c(bits, np.uint16)
    return np.array([lib.orc_f16_value(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)


def f16_from_f64(values):
    """Nearest fp16 bit patterns (ties to even) for fp64 values."""
    lib = load()
    v = np.asarray(values, dtype=np.float64)
    return np.array([lib.orc_f16_from_f64(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def bf16_from_f64(values):
    """Nearest bfloat16 bit patterns to fp64 values (ties to even)."""
    lib = load()
    v = np.asarray(values, dtype=np.float64)
    return np.array([lib.orc_bf16_from_f64(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def gemm_dense(W, X):
    """W: uint16 [N, K] bf16 bits; X: uint16 [M, K] bf16 bits.
    Returns (Y, B), fp64 [M, N]: the product and sum_k |W x|."""
    lib = load()
    W = _c(W, np.uint16)
    X = _c(X, np.uint16)
    N, K = W.shape
    M, K2 = X.shape
    if K2 != K:
        raise ValueError("K mismatch")
    Y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    lib.orc_gemm_dense(_ptr(W), _ptr(X), M, N, K, _ptr(Y), _ptr(B))
    return Y, B


def gemm_f64w(Wd, X):
    """Product with fp64 weights Wd [N, K] and bf16 X [M, K]; returns (Y, B)."""
    lib = load()
    Wd = _c(Wd, np.float64)
    X = _c(X, np.uint16)
    N, K = Wd.shape
    M = X.shape[0]
    Y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    lib.orc_gemm_f64w(_ptr(Wd), _ptr(X), M, N, K, _ptr(Y), _ptr(B))
    return Y, B


def dequant_q4g64(Wq, S):
    """Wq: uint8 [N, K/2]; S: uint16 [N, K/64] fp16 bits.  Returns fp64 [N, K]."""
    lib = load()
    Wq = _c(Wq, np.uint8)
    S = _c(S, np.uint16)
    N, K2 = Wq.shape
    K = 2 * K2
    if S.shape != (N, K // 64):
        raise ValueError("scale shape mismatch")
    Wd = np.empty((N, K), dtype=np.float64)
    lib.orc_dequant_q4g64(_ptr(Wq), _ptr(S), N, K, _ptr(Wd))
    return Wd


def gemm_q4g64(Wq, S, X):
    """int4-g64 product: Wq uint8 [N, K/2], S uint16 [N, K/64], X uint16 [M, K]."""
    lib = load()
    Wq = _c(Wq, np.uint8)
    S = _c(S, np.uint16)
    X = _c(X, np.uint16)
    N, K2 = Wq.shape
    K = 2 * K2
    M = X.shape[0]
    if X.shape[1] != K or S.shape != (N, K // 64):
        raise ValueError("shape mismatch")
    Y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    lib.orc_gemm_q4g64(_ptr(Wq), _ptr(S), _ptr(X), M, N, K, _ptr(Y), _ptr(B))
    return Y, B


def quantize_q4g64(W):
    """W: uint16 [N, K] bf16 bits, K % 64 == 0.  Returns (Wq uint8 [N, K/2],
    S uint16 [N, K/64])."""
    lib = load()
    W = _c(W, np.uint16)
    N, K = W.shape
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    Wq = np.empty((N, K // 2), dtype=np.uint8)
    S = np.empty((N, K // 64), dtype=np.uint16)
    lib.orc_quantize_q4g64(_ptr(W), N, K, _ptr(Wq), _ptr(S))
    return Wq, S


def quantize_i8(W):
    """W: uint16 [N, K] bf16 bits.  Returns (Wq int8 [N, K], S float32 [N])."""
    lib = load()
    W = _c(W, np.uint16)
    N, K = W.shape
    Wq = np.empty((N, K), dtype=np.int8)
    S = np.empty((N,), dtype=np.float32)
    lib.orc_quantize_i8(_ptr(W), N, K, _ptr(Wq), _ptr(S))
    return Wq, S


def dequant_i8(Wq, S):
    """Wq int8 [N, K], S float32 [N].  Returns fp64 [N, K] = q * s."""
    lib = load()
    Wq = _c(Wq, np.int8)
    S = _c(S, np.float32)
    N, K = Wq.shape
    if S.shape != (N,):
        raise ValueError("scale shape mismatch")
    Wd = np.empty((N, K), dtype=np.float64)
    lib.orc_dequant_i8(_ptr(Wq), _ptr(S), N, K, _ptr(Wd))
    return Wd


def gemm_i8(Wq, S, X):
    """INT8 product: Wq int8 [N, K], S float32 [N], X uint16 [M, K] bf16 bits.
    Returns (Y, B), fp64 [M, N]."""
    lib = load()
    Wq = _c(Wq, np.int8)
    S = _c(S, np.float32)
    X = _c(X, np.uint16)
    N, K = Wq.shape
    M = X.shape[0]
    if X.shape[1] != K or S.shape != (N,):
        raise ValueError("shape mismatch")
    Y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    lib.orc_gemm_i8(_ptr(Wq), _ptr(S), _ptr(X), M, N, K, _ptr(Y), _ptr(B))
    return Y, B


def swiglu(G, U):
    """silu(G) * U elementwise in fp64 (any shape, same shapes)."""
    lib = load()
    G = _c(np.asarray(G, dtype=np.float64), np.float64)
    U = _c(np.asarray(U, dtype=np.float64), np.float64)
    if G.shape != U.shape:
        raise ValueError("shape mismatch")
    H = np.empty(G.shape, dtype=np.float64)
    lib.orc_swiglu(_ptr(G), _ptr(U), G.size, _ptr(H))
    return H


def residual_add(P, R):
    """P (fp64) + R (fp32 residual), elementwise, same shapes."""
    lib = load()
    P = _c(np.asarray(P, dtype=np.float64), np.float64)
    R = _c(R, np.float32)
    if P.shape != R.shape:
        raise ValueError("shape mismatch")
    Y = np.empty(P.shape, dtype=np.float64)
    lib.orc_residual_add(_ptr(P), _ptr(R), P.size, _ptr(Y))
    return Y


def rmsnorm(X, g, eps):
    """RMSNorm of each row of X (bf16 bits [M][K]) with gain g (bf16 bits [K]):
    bf16 bits [M][K] of x g / sqrt(mean x^2 + eps)."""
    lib = load()
    X = _c(X, np.uint16)
    g = _c(g, np.uint16)
    if X.ndim != 2 or g.shape != (X.shape[1],) or X.shape[1] < 1:
        raise ValueError("shape mismatch")
    M, K = X.shape
    H = np.empty((M, K), dtype=np.uint16)
    lib.orc_rmsnorm(_ptr(X), _ptr(g), M, K, float(eps), _ptr(H))
    return H
