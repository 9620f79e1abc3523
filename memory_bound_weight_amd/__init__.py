"""Decode-step linear layers on MI355X (gfx950): Python binding of liblin.so.

The functions here carry the names of the C entry points in include/lin.h and
only marshal arguments: they check dtype, device, contiguity and shape, pass
raw device pointers and torch's current HIP stream, and raise on a non-zero
status.  Every step of every product runs in the library's HIP kernels.  The
library must have been built (``__graft_entry__.build()`` or
``python memory_bound_weight_amd/build.py``); importing fails loudly otherwise.
"""
import ctypes
import json
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblin.so")

LIN_OK = 0
LIN_ERR_NULL = -1
LIN_ERR_SHAPE = -2
LIN_ERR_ALIGN = -3
LIN_ERR_UNSUPPORTED = -4
LIN_ERR_HIP = -5
LIN_ERR_ARG = -6
LIN_ERR_SCRATCH = -7
LIN_STATIC_SCRATCH_BYTES = 16 << 20

LIN_KIND_GEMV_BF16 = 0
LIN_KIND_GEMV_Q4G64 = 1
LIN_KIND_SKINNY_BF16 = 2
LIN_KIND_SKINNY_Q4G64 = 3
LIN_KIND_GEMV_I8 = 4
LIN_KIND_GEMV_BF16_NORM = 5
LIN_KIND_GEMV_Q4G64_NORM = 6
LIN_KIND_GEMV_I8_NORM = 7

LIN_EPI_NONE = 0
LIN_EPI_ADD = 1
LIN_EPI_SWIGLU = 2

LIN_ALGO_VALU = 1
LIN_ALGO_MFMA = 2

LIN_GEMV_MAX_M = 8
LIN_SKINNY_MAX_M = 256

# Every symbol include/lin.h declares.
EXPORTS = ("lin_gemv_bf16", "lin_gemv_q4g64", "lin_gemv_bf16_ep", "lin_gemv_q4g64_ep",
           "lin_gemv_bf16_norm", "lin_gemv_q4g64_norm", "lin_gemv_i8", "lin_gemv_i8_ep",
           "lin_gemv_i8_norm", "lin_gemm_skinny_bf16",
           "lin_gemm_skinny_bf16_noalloc", "lin_gemm_skinny_q4g64", "lin_quantize_i8",
           "lin_q4g64_tiled_size", "lin_q4g64_tile", "lin_autotune",
           "lin_autotune_set", "lin_num_candidates", "lin_candidate", "lin_get_config", "lin_set_config",
           "lin_quantize_q4g64", "lin_stream_read", "lin_status_string", "lin_version")


class LinConfig(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("rows", ctypes.c_int32), ("unroll", ctypes.c_int32),
                ("split", ctypes.c_int32), ("stage_x", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("reserved", ctypes.c_int32), ("us", ctypes.c_float)]

    def as_dict(self):
        return dict(algo=self.algo, rows=self.rows, unroll=self.unroll, split=self.split,
                    stage_x=self.stage_x, tile_m=self.tile_m, waves=self.waves, us=self.us)

    @classmethod
    def from_dict(cls, d):
        c = cls()
        for k in ("algo", "rows", "unroll", "split", "stage_x", "tile_m"):
            setattr(c, k, int(d[k]))
        c.waves = int(d.get("waves", 0))
        return c


class LinError(RuntimeError):
    def __init__(self, status, where):
        super().__init__("%s failed: %s (%d)" % (where, status_string(status), status))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblin.so is not built (%s); run __graft_entry__.build() or "
                          "python memory_bound_weight_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "lin_gemv_bf16": [P, P, P, I64, I64, I64, P],
        "lin_gemv_q4g64": [P, P, P, P, I64, I64, I64, P],
        "lin_gemv_i8": [P, P, P, P, I64, I64, I64, P],
        "lin_gemv_bf16_ep": [P, P, P, I64, I64, I64, I, P, P],
        "lin_gemv_q4g64_ep": [P, P, P, P, I64, I64, I64, I, P, P],
        "lin_gemv_bf16_norm": [P, P, P, ctypes.c_float, P, I64, I64, I64, I, P, P],
        "lin_gemv_q4g64_norm": [P, P, P, P, ctypes.c_float, P, I64, I64, I64, I, P, P],
        "lin_gemv_i8_ep": [P, P, P, P, I64, I64, I64, I, P, P],
        "lin_gemv_i8_norm": [P, P, P, P, ctypes.c_float, P, I64, I64, I64, I, P, P],
        "lin_quantize_i8": [P, P, P, I64, I64, P],
        "lin_gemm_skinny_bf16": [P, P, P, I64, I64, I64, P],
        "lin_gemm_skinny_bf16_noalloc": [P, P, P, I64, I64, I64, ctypes.POINTER(LinConfig), P],
        "lin_gemm_skinny_q4g64": [P, P, P, P, I64, I64, I64, P],
        "lin_q4g64_tiled_size": [I64, I64, ctypes.POINTER(I64), ctypes.POINTER(I64)],
        "lin_q4g64_tile": [P, P, P, P, I64, I64, P],
        "lin_autotune": [I, P, P, P, P, I64, I64, I64, P, ctypes.POINTER(LinConfig)],
        "lin_autotune_set": [I, ctypes.POINTER(P), ctypes.POINTER(P), I, P, P, I64, I64, I64, P,
                             ctypes.POINTER(LinConfig)],
        "lin_num_candidates": [I, I64, I64, I64],
        "lin_candidate": [I, I64, I64, I64, I, ctypes.POINTER(LinConfig)],
        "lin_get_config": [I, I64, I64, I64, ctypes.POINTER(LinConfig)],
        "lin_set_config": [I, I64, I64, I64, ctypes.POINTER(LinConfig)],
        "lin_quantize_q4g64": [P, P, P, I64, I64, P],
        "lin_stream_read": [P, I64, P],
        "lin_status_string": [I],
        "lin_version": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_char_p if name == "lin_status_string" else ctypes.c_int
    return lib


_lib = _load()


def status_string(status):
    return _lib.lin_status_string(int(status)).decode()


def lin_version():
    return _lib.lin_version()


def _check(st, where):
    if st != LIN_OK:
        raise LinError(st, where)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, dtype, name, dims):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if t.dim() != dims:
        raise ValueError("%s must have %d dimensions" % (name, dims))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _as2d(x):
    return x.unsqueeze(0) if x.dim() == 1 else x


def _out(y, M, N, dev):
    if y is None:
        return torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(y, torch.float32, "y", 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must have shape (%d, %d)" % (M, N))
    return y


def lin_gemv_bf16(W, x, y=None):
    """y[m][n] = sum_k W[n][k] x[m][k]; W bf16 [N, K], x bf16 [M, K] or [K]."""
    x = _as2d(x)
    _need(W, torch.bfloat16, "W", 2)
    _need(x, torch.bfloat16, "x", 2)
    N, K = W.shape
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must have K = %d columns" % K)
    y = _out(y, M, N, W.device)
    _check(_lib.lin_gemv_bf16(W.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, K, _stream(W)),
           "lin_gemv_bf16")
    return y


def lin_gemv_q4g64(Wq, S, x, y=None):
    """Same product with int4-g64 weights: Wq uint8 [N, K/2], S fp16 [N, K/64]."""
    x = _as2d(x)
    _need(Wq, torch.uint8, "Wq", 2)
    _need(S, torch.float16, "S", 2)
    _need(x, torch.bfloat16, "x", 2)
    N, K2 = Wq.shape
    K = 2 * K2
    M = x.shape[0]
    if x.shape[1] != K or tuple(S.shape) != (N, K // 64):
        raise ValueError("shape mismatch: Wq [N, K/2], S [N, K/64], x [M, K]")
    y = _out(y, M, N, Wq.device)
    _check(_lib.lin_gemv_q4g64(Wq.data_ptr(), S.data_ptr(), x.data_ptr(), y.data_ptr(),
                               M, N, K, _stream(Wq)), "lin_gemv_q4g64")
    return y


def _epi_out(epilogue, NW, r, y, dev, M=1):
    if epilogue not in (LIN_EPI_NONE, LIN_EPI_ADD, LIN_EPI_SWIGLU):
        raise ValueError("unknown epilogue %r" % (epilogue,))
    N = NW // 2 if epilogue == LIN_EPI_SWIGLU else NW
    if epilogue == LIN_EPI_SWIGLU and NW % 2:
        raise ValueError("the gated product needs an even number of weight rows")
    if epilogue == LIN_EPI_ADD:
        _need(r, torch.float32, "r", 2)
        if tuple(r.shape) != (M, N):
            raise ValueError("r must have shape (%d, %d)" % (M, N))
    return N, _out(y, M, N, dev)


def lin_gemv_bf16_ep(W, x, epilogue, r=None, y=None):
    """bf16 product of up to 8 tokens with a fused epilogue: LIN_EPI_ADD (y = W x + r,
    r [M, N] may be y) or LIN_EPI_SWIGLU (W has 2N rows: y = silu(W[:N] x) * W[N:] x)."""
    x = _as2d(x)
    _need(W, torch.bfloat16, "W", 2)
    _need(x, torch.bfloat16, "x", 2)
    NW, K = W.shape
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must have K = %d columns" % K)
    N, y = _epi_out(epilogue, NW, r, y, W.device, M)
    _check(_lib.lin_gemv_bf16_ep(W.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, K, int(epilogue),
                                 r.data_ptr() if r is not None else None, _stream(W)),
           "lin_gemv_bf16_ep")
    return y


def lin_gemv_q4g64_ep(Wq, S, x, epilogue, r=None, y=None):
    """Batch-1 int4-g64 product with a fused epilogue (see lin_gemv_bf16_ep)."""
    x = _as2d(x)
    _need(Wq, torch.uint8, "Wq", 2)
    _need(S, torch.float16, "S", 2)
    _need(x, torch.bfloat16, "x", 2)
    NW, K2 = Wq.shape
    K = 2 * K2
    M = x.shape[0]
    if x.shape[1] != K or tuple(S.shape) != (NW, K // 64):
        raise ValueError("shape mismatch: Wq [N, K/2], S [N, K/64], x [M, K]")
    N, y = _epi_out(epilogue, NW, r, y, Wq.device, M)
    _check(_lib.lin_gemv_q4g64_ep(Wq.data_ptr(), S.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, K,
                                  int(epilogue), r.data_ptr() if r is not None else None,
                                  _stream(Wq)), "lin_gemv_q4g64_ep")
    return y


def _norm_gain(g, K):
    _need(g, torch.bfloat16, "g", 1)
    if tuple(g.shape) != (K,):
        raise ValueError("g must have shape (%d,)" % K)


def lin_gemv_bf16_norm(W, x, g, eps, epilogue=LIN_EPI_NONE, r=None, y=None):
    """Batch-1 bf16 product of the RMSNorm of x: h = bf16(x g / sqrt(mean x^2 + eps)),
    y = W h, with an optional fused epilogue (see lin_gemv_bf16_ep).  x is not modified."""
    x = _as2d(x)
    _need(W, torch.bfloat16, "W", 2)
    _need(x, torch.bfloat16, "x", 2)
    NW, K = W.shape
    if x.shape != (1, K):
        raise ValueError("x must be one token of K = %d" % K)
    _norm_gain(g, K)
    N, y = _epi_out(epilogue, NW, r, y, W.device)
    _check(_lib.lin_gemv_bf16_norm(W.data_ptr(), x.data_ptr(), g.data_ptr(), float(eps),
                                   y.data_ptr(), 1, N, K, int(epilogue),
                                   r.data_ptr() if r is not None else None, _stream(W)),
           "lin_gemv_bf16_norm")
    return y


def lin_gemv_q4g64_norm(Wq, S, x, g, eps, epilogue=LIN_EPI_NONE, r=None, y=None):
    """Batch-1 int4-g64 product of the RMSNorm of x (see lin_gemv_bf16_norm)."""
    x = _as2d(x)
    _need(Wq, torch.uint8, "Wq", 2)
    _need(S, torch.float16, "S", 2)
    _need(x, torch.bfloat16, "x", 2)
    NW, K2 = Wq.shape
    K = 2 * K2
    if x.shape != (1, K) or tuple(S.shape) != (NW, K // 64):
        raise ValueError("shape mismatch: Wq [N, K/2], S [N, K/64], x [1, K]")
    _norm_gain(g, K)
    N, y = _epi_out(epilogue, NW, r, y, Wq.device)
    _check(_lib.lin_gemv_q4g64_norm(Wq.data_ptr(), S.data_ptr(), x.data_ptr(), g.data_ptr(),
                                    float(eps), y.data_ptr(), 1, N, K, int(epilogue),
                                    r.data_ptr() if r is not None else None, _stream(Wq)),
           "lin_gemv_q4g64_norm")
    return y


def lin_gemv_i8(Wq, S, x, y=None):
    """Same product with INT8 weights Wq int8 [N, K] and one fp32 scale per row S [N]."""
    x = _as2d(x)
    _need(Wq, torch.int8, "Wq", 2)
    _need(S, torch.float32, "S", 1)
    _need(x, torch.bfloat16, "x", 2)
    N, K = Wq.shape
    M = x.shape[0]
    if x.shape[1] != K or tuple(S.shape) != (N,):
        raise ValueError("shape mismatch: Wq [N, K], S [N], x [M, K]")
    y = _out(y, M, N, Wq.device)
    _check(_lib.lin_gemv_i8(Wq.data_ptr(), S.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, K,
                            _stream(Wq)), "lin_gemv_i8")
    return y


def _i8_args(Wq, S, x, one_token=True):
    x = _as2d(x)
    _need(Wq, torch.int8, "Wq", 2)
    _need(S, torch.float32, "S", 1)
    _need(x, torch.bfloat16, "x", 2)
    NW, K = Wq.shape
    if x.shape[1] != K or (one_token and x.shape[0] != 1) or tuple(S.shape) != (NW,):
        raise ValueError("shape mismatch: Wq [N, K], S [N], x [%s, K]" % ("1" if one_token else "M"))
    return x, NW, K


def lin_gemv_i8_ep(Wq, S, x, epilogue, r=None, y=None):
    """Batch-1 INT8 product with a fused epilogue (see lin_gemv_bf16_ep); with the
    gated epilogue, each row's scale is applied before the gate."""
    x, NW, K = _i8_args(Wq, S, x, one_token=False)
    M = x.shape[0]
    N, y = _epi_out(epilogue, NW, r, y, Wq.device, M)
    _check(_lib.lin_gemv_i8_ep(Wq.data_ptr(), S.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, K,
                               int(epilogue), r.data_ptr() if r is not None else None, _stream(Wq)),
           "lin_gemv_i8_ep")
    return y


def lin_gemv_i8_norm(Wq, S, x, g, eps, epilogue=LIN_EPI_NONE, r=None, y=None):
    """Batch-1 INT8 product of the RMSNorm of x (see lin_gemv_bf16_norm)."""
    x, NW, K = _i8_args(Wq, S, x)
    _norm_gain(g, K)
    N, y = _epi_out(epilogue, NW, r, y, Wq.device)
    _check(_lib.lin_gemv_i8_norm(Wq.data_ptr(), S.data_ptr(), x.data_ptr(), g.data_ptr(), float(eps),
                                 y.data_ptr(), 1, N, K, int(epilogue),
                                 r.data_ptr() if r is not None else None, _stream(Wq)),
           "lin_gemv_i8_norm")
    return y


def lin_quantize_i8(W, Wq=None, S=None):
    """INT8 weights from bf16 W [N, K]: returns (Wq int8 [N, K], S fp32 [N])."""
    _need(W, torch.bfloat16, "W", 2)
    N, K = W.shape
    if Wq is None:
        Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if S is None:
        S = torch.empty((N,), dtype=torch.float32, device=W.device)
    _need(Wq, torch.int8, "Wq", 2)
    _need(S, torch.float32, "S", 1)
    _check(_lib.lin_quantize_i8(W.data_ptr(), Wq.data_ptr(), S.data_ptr(), N, K, _stream(W)),
           "lin_quantize_i8")
    return Wq, S


def lin_gemm_skinny_bf16(W, X, Y=None):
    """Y = X . W^T for M <= 256 tokens; W bf16 [N, K], X bf16 [M, K]."""
    X = _as2d(X)
    _need(W, torch.bfloat16, "W", 2)
    _need(X, torch.bfloat16, "X", 2)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X must have K = %d columns" % K)
    Y = _out(Y, M, N, W.device)
    _check(_lib.lin_gemm_skinny_bf16(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K,
                                     _stream(W)), "lin_gemm_skinny_bf16")
    return Y


def lin_gemm_skinny_bf16_noalloc(W, X, Y, cfg=None):
    """lin_gemm_skinny_bf16 without any device allocation: split-K
    configurations use the library's static scratch array.  Y must be given
    (nothing is allocated here either); cfg: a candidate dict, or None for the
    configuration lin_get_config reports."""
    X = _as2d(X)
    _need(W, torch.bfloat16, "W", 2)
    _need(X, torch.bfloat16, "X", 2)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X must have K = %d columns" % K)
    _need(Y, torch.float32, "Y", 2)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be [%d, %d]" % (M, N))
    c = ctypes.byref(LinConfig.from_dict(cfg)) if cfg is not None else None
    _check(_lib.lin_gemm_skinny_bf16_noalloc(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K,
                                             c, _stream(W)), "lin_gemm_skinny_bf16_noalloc")
    return Y


class Q4Tiled:
    """int4-g64 weights of an N x K matrix in the matrix-core tiled layout of
    lin_q4g64_tile: Wt and St are flat uint8 device tensors."""
    __slots__ = ("Wt", "St", "N", "K")

    def __init__(self, Wt, St, N, K):
        self.Wt, self.St, self.N, self.K = Wt, St, int(N), int(K)

    @property
    def shape(self):
        return (self.N, self.K)

    @property
    def dtype(self):
        return "q4g64_tiled"

    @property
    def device(self):
        return self.Wt.device


def lin_q4g64_tiled_size(N, K):
    """(Wt bytes, St bytes) of the tiled layout of an N x K matrix."""
    wt, st = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.lin_q4g64_tiled_size(N, K, ctypes.byref(wt), ctypes.byref(st)),
           "lin_q4g64_tiled_size")
    return wt.value, st.value


def lin_q4g64_tile(Wq, S):
    """Rearrange int4-g64 weights (Wq uint8 [N, K/2], S fp16 [N, K/64]) into the
    tiled layout lin_gemm_skinny_q4g64 reads; returns a Q4Tiled."""
    _need(Wq, torch.uint8, "Wq", 2)
    _need(S, torch.float16, "S", 2)
    N, K = Wq.shape[0], 2 * Wq.shape[1]
    if tuple(S.shape) != (N, K // 64):
        raise ValueError("shape mismatch: Wq [N, K/2], S [N, K/64]")
    wb, sb = lin_q4g64_tiled_size(N, K)
    Wt = torch.empty(max(wb, 16), dtype=torch.uint8, device=Wq.device)
    St = torch.empty(max(sb, 16), dtype=torch.uint8, device=Wq.device)
    _check(_lib.lin_q4g64_tile(Wq.data_ptr(), S.data_ptr(), Wt.data_ptr(), St.data_ptr(), N, K,
                               _stream(Wq)), "lin_q4g64_tile")
    return Q4Tiled(Wt, St, N, K)


def lin_gemm_skinny_q4g64(W, X, Y=None):
    """Y = X . W^T for M <= 256 tokens with int4-g64 weights W (a Q4Tiled from
    lin_q4g64_tile), X bf16 [M, K]."""
    X = _as2d(X)
    if not isinstance(W, Q4Tiled):
        raise TypeError("W must be a Q4Tiled (lin_q4g64_tile)")
    _need(X, torch.bfloat16, "X", 2)
    N, K = W.N, W.K
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X must have K = %d columns" % K)
    Y = _out(Y, M, N, X.device)
    _check(_lib.lin_gemm_skinny_q4g64(W.Wt.data_ptr(), W.St.data_ptr(), X.data_ptr(),
                                      Y.data_ptr(), M, N, K, _stream(X)),
           "lin_gemm_skinny_q4g64")
    return Y


def lin_quantize_q4g64(W, Wq=None, S=None):
    """int4-g64 weights from bf16 W [N, K]: returns (Wq uint8 [N, K/2], S fp16 [N, K/64])."""
    _need(W, torch.bfloat16, "W", 2)
    N, K = W.shape
    if Wq is None:
        Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    if S is None:
        S = torch.empty((N, K // 64), dtype=torch.float16, device=W.device)
    _need(Wq, torch.uint8, "Wq", 2)
    _need(S, torch.float16, "S", 2)
    _check(_lib.lin_quantize_q4g64(W.data_ptr(), Wq.data_ptr(), S.data_ptr(), N, K, _stream(W)),
           "lin_quantize_q4g64")
    return Wq, S


def lin_stream_read(buf):
    """Read every byte of a contiguous device tensor once (the bandwidth ceiling
    a product is compared with); returns nothing."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("lin_stream_read: buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.lin_stream_read(buf.data_ptr(), nbytes, _stream(buf)), "lin_stream_read")


def _shape_args(kind, W, S, x):
    x = _as2d(x)
    if kind == LIN_KIND_SKINNY_Q4G64:
        if not isinstance(W, Q4Tiled):
            raise TypeError("LIN_KIND_SKINNY_Q4G64 takes Q4Tiled weights")
        return x, x.shape[0], W.N, W.K
    if kind in (LIN_KIND_GEMV_Q4G64, LIN_KIND_GEMV_Q4G64_NORM):
        return x, x.shape[0], W.shape[0], 2 * W.shape[1]
    return x, x.shape[0], W.shape[0], W.shape[1]


def lin_autotune(kind, W, x, y, S=None):
    """Time every candidate for this shape on these buffers (cold caches), keep
    the fastest for later calls; returns it as a dict with 'us'."""
    x, M, N, K = _shape_args(kind, W, S, x)
    if isinstance(W, Q4Tiled):
        W, S = W.Wt, W.St
    cfg = LinConfig()
    _check(_lib.lin_autotune(int(kind), W.data_ptr(), S.data_ptr() if S is not None else None,
                             x.data_ptr(), y.data_ptr(), M, N, K, _stream(W), ctypes.byref(cfg)),
           "lin_autotune")
    return cfg.as_dict()


def lin_autotune_set(kind, Ws, x, y, Ss=None):
    """Time every candidate as a graph of back-to-back calls cycling over the
    same-shaped weights Ws (and scales Ss for int4), keep the fastest for later
    calls; returns it as a dict with 'us' (mean per call)."""
    Ws = list(Ws)
    if not Ws:
        raise ValueError("lin_autotune_set needs at least one weight matrix")
    x, M, N, K = _shape_args(kind, Ws[0], Ss[0] if Ss else None, x)
    for W in Ws:
        if tuple(W.shape) != tuple(Ws[0].shape) or W.dtype != Ws[0].dtype:
            raise ValueError("lin_autotune_set: every matrix must have the same shape and dtype")
    if isinstance(Ws[0], Q4Tiled):
        Ss = [W.St for W in Ws]
        Ws = [W.Wt for W in Ws]
    wp = (ctypes.c_void_p * len(Ws))(*[W.data_ptr() for W in Ws])
    sp = None
    if Ss is not None:
        Ss = list(Ss)
        if len(Ss) != len(Ws):
            raise ValueError("lin_autotune_set: one scale tensor per weight matrix")
        sp = (ctypes.c_void_p * len(Ss))(*[S.data_ptr() for S in Ss])
    cfg = LinConfig()
    _check(_lib.lin_autotune_set(int(kind), wp, sp, len(Ws), x.data_ptr(), y.data_ptr(), M, N, K,
                                 _stream(Ws[0]), ctypes.byref(cfg)),
           "lin_autotune_set")
    return cfg.as_dict()


def lin_num_candidates(kind, M, N, K):
    n = _lib.lin_num_candidates(int(kind), M, N, K)
    if n < 0:
        raise LinError(n, "lin_num_candidates")
    return n


def lin_candidate(kind, M, N, K, index):
    cfg = LinConfig()
    _check(_lib.lin_candidate(int(kind), M, N, K, int(index), ctypes.byref(cfg)), "lin_candidate")
    return cfg.as_dict()


def lin_candidates(kind, M, N, K):
    return [lin_candidate(kind, M, N, K, i) for i in range(lin_num_candidates(kind, M, N, K))]


def lin_get_config(kind, M, N, K):
    cfg = LinConfig()
    _check(_lib.lin_get_config(int(kind), M, N, K, ctypes.byref(cfg)), "lin_get_config")
    return cfg.as_dict()


def lin_set_config(kind, M, N, K, cfg):
    """Pin cfg (a dict from lin_candidate) for this shape; None removes the entry."""
    p = ctypes.byref(LinConfig.from_dict(cfg)) if cfg is not None else None
    _check(_lib.lin_set_config(int(kind), M, N, K, p), "lin_set_config")


# ---------------------------------------------------------------- tuning table files

TUNING_DIR = os.path.join(_HERE, "tuning")


def device_arch(index=0):
    """The gfx architecture name of a GPU (e.g. "gfx950"), without feature flags."""
    return torch.cuda.get_device_properties(index).gcnArchName.split(":")[0]


def save_tuning(path, entries):
    """Persist tuned configurations: entries = {(kind, M, N, K): cfg dict}.  The
    table records the architecture and compute-unit count it was tuned on."""
    rows = [dict(kind=k[0], M=k[1], N=k[2], K=k[3], cfg={f: v.get(f, 0) for f in
            ("algo", "rows", "unroll", "split", "stage_x", "tile_m", "waves", "us")})
            for k, v in sorted(entries.items())]
    props = torch.cuda.get_device_properties(0)
    with open(path, "w") as f:
        json.dump({"device": props.name, "arch": device_arch(0),
                   "compute_units": props.multi_processor_count,
                   "version": lin_version(), "entries": rows}, f, indent=1)


def load_tuning(path):
    """Pin every configuration of a tuning file that this library still offers;
    returns the keys applied and the keys that no longer match a candidate.  A
    table tuned on another architecture or compute-unit count applies nothing
    (every key is returned as stale)."""
    with open(path) as f:
        data = json.load(f)
    keys = [(e["kind"], e["M"], e["N"], e["K"]) for e in data["entries"]]
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    if data.get("arch") != device_arch(torch.cuda.current_device()) or \
            data.get("compute_units") != props.multi_processor_count:
        return [], keys
    ok, stale = [], []
    for e, key in zip(data["entries"], keys):
        try:
            lin_set_config(*key, e["cfg"])
            ok.append(key)
        except LinError:
            stale.append(key)
    return ok, stale
