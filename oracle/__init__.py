"""Python handle on the plain-C CPU oracle (``oracle/oracle.c``) for the BitLinear forward.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's CPU
baseline may import this module; the GPU library and its Python binding never do.  It shares
no code with the GPU path.  Arrays are numpy, C-contiguous; the wrappers only marshal them
to the C functions, every step of the arithmetic is in ``oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile ``source`` into a shared library at ``output`` with gcc; returns the path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """Binds the oracle's C functions from one compiled library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(output=path)
        self.path = path
        lib = ctypes.CDLL(path)
        self._lib = lib
        lib.oracle_gamma.argtypes = [_P, _I64, _P]
        lib.oracle_gamma.restype = ctypes.c_float
        lib.oracle_ternary_codes.argtypes = [_P, _I64, ctypes.c_float, _P]
        lib.oracle_ternary_codes.restype = None
        lib.oracle_pack.argtypes = [_P, _I64, _I64, _P]
        lib.oracle_pack.restype = ctypes.c_int
        lib.oracle_unpack.argtypes = [_P, _I64, _I64, _P]
        lib.oracle_unpack.restype = ctypes.c_int
        lib.oracle_quantize_weights.argtypes = [_P, _I64, _I64, _P, _P, _P]
        lib.oracle_quantize_weights.restype = ctypes.c_int
        lib.oracle_quantize_acts_f32.argtypes = [_P, _I64, _I64, _P, ctypes.c_float, _P, _P]
        lib.oracle_quantize_acts_f32.restype = None
        lib.oracle_quantize_acts_bf16.argtypes = [_P, _I64, _I64, _P, ctypes.c_float, _P, _P, _P]
        lib.oracle_quantize_acts_bf16.restype = None
        lib.oracle_matmul.argtypes = [_P, _P, _I64, _I64, _I64, _P]
        lib.oracle_matmul.restype = ctypes.c_int
        lib.oracle_epilogue.argtypes = [_P, _P, ctypes.c_float, _I64, _I64, _P]
        lib.oracle_epilogue.restype = None
        lib.oracle_ffn_act1.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float]
        lib.oracle_ffn_act1.restype = ctypes.c_float
        lib.oracle_ffn_act.argtypes = [ctypes.c_int, _P, _P, _I64, _P]
        lib.oracle_ffn_act.restype = None
        lib.oracle_ffn_act1_f64.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float]
        lib.oracle_ffn_act1_f64.restype = ctypes.c_double
        lib.oracle_ffn_act_f64.argtypes = [ctypes.c_int, _P, _P, _I64, _P]
        lib.oracle_ffn_act_f64.restype = None
        lib.oracle_epilogue_residual.argtypes = [_P, _P, ctypes.c_float, _P, _I64, _I64, _P]
        lib.oracle_epilogue_residual.restype = None
        lib.oracle_forward_entries.argtypes = [_P, _P, _P, ctypes.c_float, _I64, _P, _P, _I64,
                                               _P, _P, _P]
        lib.oracle_forward_entries.restype = ctypes.c_int
        lib.oracle_forward_wonly.argtypes = [_P, _P, ctypes.c_float, _I64, _I64, _I64, _P]
        lib.oracle_forward_wonly.restype = None
        lib.oracle_grad_input.argtypes = [_P, _P, ctypes.c_float, _I64, _I64, _I64, _P]
        lib.oracle_grad_input.restype = None
        lib.oracle_ste_scale.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_double]
        lib.oracle_ste_scale.restype = ctypes.c_double
        lib.oracle_grad_weight.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int,
                                           ctypes.c_double, _I64, _I64, _I64, _P]
        lib.oracle_grad_weight.restype = None
        lib.oracle_b3_row_bytes.argtypes = [_I64]
        lib.oracle_b3_row_bytes.restype = _I64
        lib.oracle_pack_b3.argtypes = [_P, _I64, _I64, _P]
        lib.oracle_pack_b3.restype = ctypes.c_int
        lib.oracle_unpack_b3.argtypes = [_P, _I64, _I64, _P]
        lib.oracle_unpack_b3.restype = ctypes.c_int

    # O1
    def gamma(self, W: np.ndarray) -> Tuple[np.float32, float]:
        W = _c(W, np.float32)
        g64 = ctypes.c_double(0.0)
        g = self._lib.oracle_gamma(_ptr(W), W.size, ctypes.byref(g64))
        return np.float32(g), g64.value

    # O2
    def ternary_codes(self, W: np.ndarray, gamma) -> np.ndarray:
        W = _c(W, np.float32)
        codes = np.empty(W.shape, dtype=np.int8)
        self._lib.oracle_ternary_codes(_ptr(W), W.size, float(np.float32(gamma)), _ptr(codes))
        return codes

    # O3
    def pack(self, codes: np.ndarray) -> np.ndarray:
        codes = _c(codes, np.int8)
        N, K = codes.shape
        packed = np.empty((N, K // 16), dtype=np.uint32)
        rc = self._lib.oracle_pack(_ptr(codes), N, K, _ptr(packed))
        if rc:
            raise ValueError(f"oracle_pack failed: {rc}")
        return packed

    def unpack(self, packed: np.ndarray, K: int) -> np.ndarray:
        packed = _c(packed, np.uint32)
        N = packed.shape[0]
        codes = np.empty((N, K), dtype=np.int8)
        rc = self._lib.oracle_unpack(_ptr(packed), N, K, _ptr(codes))
        if rc:
            raise ValueError(f"oracle_unpack failed: {rc}")
        return codes

    # O1 + O2 + O3
    def quantize_weights(self, W: np.ndarray):
        W = _c(W, np.float32)
        N, K = W.shape
        codes = np.empty((N, K), dtype=np.int8)
        packed = np.empty((N, K // 16), dtype=np.uint32)
        gamma = ctypes.c_float(0.0)
        rc = self._lib.oracle_quantize_weights(_ptr(W), N, K, _ptr(codes), _ptr(packed),
                                               ctypes.byref(gamma))
        if rc:
            raise ValueError(f"oracle_quantize_weights failed: {rc}")
        return packed, np.float32(gamma.value), codes

    # O4
    def quantize_acts(self, X: np.ndarray, g: Optional[np.ndarray] = None, eps: float = 1e-6,
                      bf16: bool = False):
        """X: fp32 [M, K], or raw bf16 bits (uint16) [M, K] with ``bf16=True``."""
        if bf16:
            X = _c(X, np.uint16)
        else:
            X = _c(X, np.float32)
        M, K = X.shape
        gg = None if g is None else _c(g, np.float32)
        Xq = np.empty((M, K), dtype=np.int8)
        sx = np.empty(M, dtype=np.float32)
        if bf16:
            row = np.empty(K, dtype=np.float32)
            self._lib.oracle_quantize_acts_bf16(_ptr(X), M, K, _ptr(gg), float(eps), _ptr(row),
                                                _ptr(Xq), _ptr(sx))
        else:
            self._lib.oracle_quantize_acts_f32(_ptr(X), M, K, _ptr(gg), float(eps), _ptr(Xq),
                                               _ptr(sx))
        return Xq, sx

    # O5
    def matmul(self, Xq: np.ndarray, codes: np.ndarray) -> np.ndarray:
        Xq = _c(Xq, np.int8)
        codes = _c(codes, np.int8)
        M, K = Xq.shape
        N = codes.shape[0]
        assert codes.shape[1] == K
        acc = np.empty((M, N), dtype=np.int32)
        rc = self._lib.oracle_matmul(_ptr(Xq), _ptr(codes), M, N, K, _ptr(acc))
        if rc:
            raise ValueError(f"oracle_matmul failed: {rc}")
        return acc

    # O6
    def epilogue(self, acc: np.ndarray, sx: np.ndarray, gamma) -> np.ndarray:
        acc = _c(acc, np.int32)
        sx = _c(sx, np.float32)
        M, N = acc.shape
        Y = np.empty((M, N), dtype=np.float32)
        self._lib.oracle_epilogue(_ptr(acc), _ptr(sx), float(np.float32(gamma)), M, N, _ptr(Y))
        return Y

    # O5 + O6 on packed weights
    def forward(self, Xq: np.ndarray, sx: np.ndarray, packed: np.ndarray, gamma):
        K = Xq.shape[1]
        codes = self.unpack(packed, K)
        acc = self.matmul(Xq, codes)
        return acc, self.epilogue(acc, sx, gamma)

    def forward_entries(self, Xq, sx, packed, gamma, m_idx, n_idx):
        Xq = _c(Xq, np.int8)
        sx = _c(sx, np.float32)
        packed = _c(packed, np.uint32)
        m_idx = _c(m_idx, np.int64)
        n_idx = _c(n_idx, np.int64)
        K = Xq.shape[1]
        count = m_idx.size
        row = np.empty(K, dtype=np.int8)
        acc = np.empty(count, dtype=np.int32)
        Y = np.empty(count, dtype=np.float32)
        rc = self._lib.oracle_forward_entries(_ptr(Xq), _ptr(sx), _ptr(packed),
                                              float(np.float32(gamma)), K, _ptr(m_idx),
                                              _ptr(n_idx), count, _ptr(row), _ptr(acc), _ptr(Y))
        if rc:
            raise ValueError(f"oracle_forward_entries failed: {rc}")
        return acc, Y

    # O7 (layer chain): FFN activation, kinds as in oracle.c
    SWIGLU, RELU2_GLU, RELU2 = 1, 2, 3

    def ffn_act(self, kind: int, X: np.ndarray, X2: Optional[np.ndarray] = None) -> np.ndarray:
        X = _c(X, np.float32)
        X2 = None if X2 is None else _c(X2, np.float32)
        if X2 is not None:
            assert X2.shape == X.shape
        H = np.empty_like(X)
        self._lib.oracle_ffn_act(int(kind), _ptr(X), _ptr(X2), X.size, _ptr(H))
        return H

    def ffn_act_f64(self, kind: int, X: np.ndarray, X2: Optional[np.ndarray] = None) -> np.ndarray:
        """The activation's fp64 value before its one rounding to fp32 (ffn_act rounds it)."""
        X = _c(X, np.float32)
        X2 = None if X2 is None else _c(X2, np.float32)
        if X2 is not None:
            assert X2.shape == X.shape
        H64 = np.empty(X.shape, dtype=np.float64)
        self._lib.oracle_ffn_act_f64(int(kind), _ptr(X), _ptr(X2), X.size, _ptr(H64))
        return H64

    def ffn_act1(self, kind: int, x: float, x2: float = 0.0) -> np.float32:
        return np.float32(self._lib.oracle_ffn_act1(int(kind), float(np.float32(x)),
                                                    float(np.float32(x2))))

    # O8 (layer chain): residual epilogue
    def epilogue_residual(self, acc: np.ndarray, sx: np.ndarray, gamma, R: np.ndarray) -> np.ndarray:
        acc = _c(acc, np.int32)
        sx = _c(sx, np.float32)
        R = _c(R, np.float32)
        M, N = acc.shape
        assert R.shape == (M, N)
        Y = np.empty((M, N), dtype=np.float32)
        self._lib.oracle_epilogue_residual(_ptr(acc), _ptr(sx), float(np.float32(gamma)), _ptr(R),
                                           M, N, _ptr(Y))
        return Y


    # O9: weight-only ternary forward (full-precision activations)
    def forward_wonly(self, X: np.ndarray, codes: np.ndarray, gamma) -> np.ndarray:
        """X fp32 [M, K] (bf16 inputs widened by the caller), codes int8 [N, K]."""
        X = _c(X, np.float32)
        codes = _c(codes, np.int8)
        M, K = X.shape
        N = codes.shape[0]
        assert codes.shape[1] == K
        Y = np.empty((M, N), dtype=np.float32)
        self._lib.oracle_forward_wonly(_ptr(X), _ptr(codes), float(np.float32(gamma)), M, N, K, _ptr(Y))
        return Y

    # O10: input gradient
    def grad_input(self, dY: np.ndarray, codes: np.ndarray, gamma) -> np.ndarray:
        """dY fp32 [M, N], codes int8 [N, K] -> dX fp32 [M, K]."""
        dY = _c(dY, np.float32)
        codes = _c(codes, np.int8)
        M, N = dY.shape
        K = codes.shape[1]
        assert codes.shape[0] == N
        dX = np.empty((M, K), dtype=np.float32)
        self._lib.oracle_grad_input(_ptr(dY), _ptr(codes), float(np.float32(gamma)), M, N, K, _ptr(dX))
        return dX

    # O11: STE gradient scale
    STE_PASS, STE_HARD, STE_SOFT = 0, 1, 2

    def ste_scale(self, kind: int, w, gamma, beta: float = 2.0) -> float:
        return self._lib.oracle_ste_scale(int(kind), float(np.float32(w)), float(np.float32(gamma)),
                                          float(beta))

    # O12: weight gradient
    def grad_weight(self, dY: np.ndarray, kind: int = 0, W: Optional[np.ndarray] = None, gamma=0.0,
                    beta: float = 2.0, Xq: Optional[np.ndarray] = None,
                    sx: Optional[np.ndarray] = None, Xf: Optional[np.ndarray] = None) -> np.ndarray:
        """dY fp32 [M, N]; activations as (Xq int8 [M, K], sx fp32 [M]) or Xf fp32 [M, K];
        W fp32 [N, K] for the hard and soft kinds -> dW fp32 [N, K]."""
        dY = _c(dY, np.float32)
        M, N = dY.shape
        if Xq is not None:
            Xq = _c(Xq, np.int8)
            sx = _c(sx, np.float32)
            K = Xq.shape[1]
        else:
            Xf = _c(Xf, np.float32)
            K = Xf.shape[1]
        if kind != 0:
            W = _c(W, np.float32)
            assert W.shape == (N, K)
        dW = np.empty((N, K), dtype=np.float32)
        self._lib.oracle_grad_weight(_ptr(dY), _ptr(Xq), _ptr(sx), _ptr(Xf), _ptr(W if kind else None),
                                     float(np.float32(gamma)), int(kind), float(beta), M, N, K, _ptr(dW))
        return dW


    # O13: base-3 packing
    def b3_row_bytes(self, K: int) -> int:
        return int(self._lib.oracle_b3_row_bytes(int(K)))

    def pack_b3(self, codes: np.ndarray) -> np.ndarray:
        codes = _c(codes, np.int8)
        N, K = codes.shape
        out = np.empty((N, self.b3_row_bytes(K)), dtype=np.uint8)
        rc = self._lib.oracle_pack_b3(_ptr(codes), N, K, _ptr(out))
        if rc:
            raise ValueError(f"oracle_pack_b3 failed: {rc}")
        return out

    def unpack_b3(self, packed: np.ndarray, K: int) -> np.ndarray:
        packed = _c(packed, np.uint8)
        N = packed.shape[0]
        assert packed.shape[1] == self.b3_row_bytes(K)
        codes = np.empty((N, K), dtype=np.int8)
        rc = self._lib.oracle_unpack_b3(_ptr(packed), N, K, _ptr(codes))
        if rc:
            raise ValueError(f"oracle_unpack_b3 failed: {rc}")
        return codes


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use if no library is present)."""
    global _default
    if _default is None:
        _default = Oracle(LIBRARY)
    return _default
