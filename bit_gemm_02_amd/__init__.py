"""Python binding of libbitlinear: the BitNet b1.58 BitLinear forward on MI355X (gfx950).

Argument marshalling only.  Each function checks the tensors it is given, allocates missing
outputs with torch (device memory is torch's), and calls the C entry point of the same name
(``bitlinear_<name>`` in ``include/bitlinear.h``) on the current torch stream.  Every step of
the computation runs in the library's HIP kernels; there is no fallback: if the library is
missing or a call is rejected, an exception is raised.

Steps (see the header for the passages each follows):
  quantize_weights  gamma = mean|W| and 2-bit packed ternary codes
  pack_codes        pack pre-ternarized int8 codes
  quantize_acts     per-token absmax int8 activations (optionally with the SubLN RMSNorm)
  forward           exact int32 ternary x int8 product and the gamma * s_x epilogue
  linear_grouped    steps 3 to 5 in one launch for decode-sized token counts
  quantize_acts_ex_grouped / forward_ex_grouped
                    the layer chain's FFN activation before quantization, and products that
                    add a residual in their epilogue (see layer.py)
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libbitlinear.so")

BL_F32, BL_BF16 = 0, 1
MAX_GROUP = 16
MAX_K = 262144
DECODE_MAX_M = 16
LINEAR_FUSED_MAX_M = 4
ACT_NONE, ACT_SWIGLU, ACT_RELU2_GLU, ACT_RELU2 = 0, 1, 2, 3
LINEAR_FUSED_MAX_BYTES = 49152


class BitLinearError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


class _WeightProblem(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("W_packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class _ActProblem(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("X_q", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("x_dtype", ctypes.c_int),
                ("eps", ctypes.c_float)]


class _ForwardProblem(ctypes.Structure):
    _fields_ = [("X_q", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("W_packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("acc", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class _LinearProblem(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("W_packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("X_q", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("x_dtype", ctypes.c_int), ("eps", ctypes.c_float)]


class _ActExProblem(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("X2", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("X_q", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("x_dtype", ctypes.c_int),
                ("act", ctypes.c_int), ("eps", ctypes.c_float)]


class _ForwardExProblem(ctypes.Structure):
    _fields_ = [("X_q", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("W_packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("acc", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class _LinearExProblem(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("W_packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("W2_packed", ctypes.c_void_p), ("gamma2", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("X_q", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("x_dtype", ctypes.c_int), ("act", ctypes.c_int), ("eps", ctypes.c_float)]


class _WonlyProblem(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("W_packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("x_dtype", ctypes.c_int)]


class _GradInputProblem(ctypes.Structure):
    _fields_ = [("dY", ctypes.c_void_p), ("Wt_packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("dX", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("dy_dtype", ctypes.c_int)]


class _GradWeightProblem(ctypes.Structure):
    _fields_ = [("dY", ctypes.c_void_p), ("X_q", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("W", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("dW", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("ste", ctypes.c_int), ("beta", ctypes.c_float)]


STE_PASS, STE_HARD, STE_SOFT = 0, 1, 2

_lib = None


def library_path() -> str:
    return LIBRARY


def lib() -> ctypes.CDLL:
    """Load libbitlinear.so (built by ``bit_gemm_02_amd.build``); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(f"{LIBRARY} is missing: build it with `python -m bit_gemm_02_amd.build`")
    L = ctypes.CDLL(LIBRARY)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.bitlinear_status_string.argtypes = [ctypes.c_int]
    L.bitlinear_status_string.restype = ctypes.c_char_p
    L.bitlinear_abi_version.argtypes = []
    L.bitlinear_abi_version.restype = ctypes.c_int
    L.bitlinear_quantize_weights_workspace.argtypes = [I64, I64]
    L.bitlinear_quantize_weights_workspace.restype = SZ
    L.bitlinear_workspace_bytes.argtypes = [I64, I64]
    L.bitlinear_workspace_bytes.restype = SZ
    L.bitlinear_quantize_weights.argtypes = [P, I64, I64, P, P, P, SZ, P]
    L.bitlinear_quantize_weights.restype = ctypes.c_int
    L.bitlinear_quantize_weights_grouped_workspace.argtypes = [ctypes.c_int]
    L.bitlinear_quantize_weights_grouped_workspace.restype = SZ
    L.bitlinear_quantize_weights_one_read_workspace.argtypes = [P, ctypes.c_int]
    L.bitlinear_quantize_weights_one_read_workspace.restype = SZ
    L.bitlinear_quantize_weights_grouped.argtypes = [P, ctypes.c_int, P, SZ, P]
    L.bitlinear_quantize_weights_grouped.restype = ctypes.c_int
    L.bitlinear_quantize_weights_grouped_noalloc.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_quantize_weights_grouped_noalloc.restype = ctypes.c_int
    L.bitlinear_pack_codes.argtypes = [P, I64, I64, P, P]
    L.bitlinear_pack_codes.restype = ctypes.c_int
    L.bitlinear_quantize_acts.argtypes = [P, ctypes.c_int, I64, I64, P, ctypes.c_float, P, P, P]
    L.bitlinear_quantize_acts.restype = ctypes.c_int
    L.bitlinear_quantize_acts_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_quantize_acts_grouped.restype = ctypes.c_int
    L.bitlinear_forward.argtypes = [P, P, P, P, I64, I64, I64, P, P, P]
    L.bitlinear_forward.restype = ctypes.c_int
    L.bitlinear_forward_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_forward_grouped.restype = ctypes.c_int
    L.bitlinear_linear_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_linear_grouped.restype = ctypes.c_int
    L.bitlinear_quantize_acts_ex_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_quantize_acts_ex_grouped.restype = ctypes.c_int
    L.bitlinear_forward_ex_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_forward_ex_grouped.restype = ctypes.c_int
    L.bitlinear_forward_mixed.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P]
    L.bitlinear_forward_mixed.restype = ctypes.c_int
    L.bitlinear_quantize_step.argtypes = [P, ctypes.c_int, P, ctypes.c_size_t, P, ctypes.c_int, P]
    L.bitlinear_quantize_step.restype = ctypes.c_int
    L.bitlinear_linear_ex_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_linear_ex_grouped.restype = ctypes.c_int
    for fn in ("bitlinear_forward_wonly_grouped", "bitlinear_grad_input_grouped",
               "bitlinear_grad_weight_grouped"):
        getattr(L, fn).argtypes = [P, ctypes.c_int, P]
        getattr(L, fn).restype = ctypes.c_int
    L.bitlinear_transpose_packed.argtypes = [P, I64, I64, P, P]
    L.bitlinear_transpose_packed.restype = ctypes.c_int
    L.bitlinear_b3_row_bytes.argtypes = [I64]
    L.bitlinear_b3_row_bytes.restype = I64
    L.bitlinear_pack_b3.argtypes = [P, I64, I64, P, P]
    L.bitlinear_pack_b3.restype = ctypes.c_int
    L.bitlinear_linear_b3_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_linear_b3_grouped.restype = ctypes.c_int
    L.bitlinear_tiles_bytes.argtypes = [I64, I64]
    L.bitlinear_tiles_bytes.restype = I64
    L.bitlinear_pack_tiles.argtypes = [P, I64, I64, P, P]
    L.bitlinear_pack_tiles.restype = ctypes.c_int
    L.bitlinear_linear_tiles_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_linear_tiles_grouped.restype = ctypes.c_int
    L.bitlinear_pack_quad_rows.argtypes = [P, I64, I64, P, P]
    L.bitlinear_pack_quad_rows.restype = ctypes.c_int
    L.bitlinear_quantize_step_quad_rows.argtypes = [P, ctypes.c_int, P, ctypes.c_size_t, P, ctypes.c_int, P]
    L.bitlinear_quantize_step_quad_rows.restype = ctypes.c_int
    L.bitlinear_forward_quad_rows_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_forward_quad_rows_grouped.restype = ctypes.c_int
    L.bitlinear_forward_ex_quad_rows_grouped.argtypes = [P, ctypes.c_int, P]
    L.bitlinear_forward_ex_quad_rows_grouped.restype = ctypes.c_int
    L.bitlinear_calib_stream.argtypes = [P, I64, P, P]
    L.bitlinear_calib_stream.restype = ctypes.c_int
    L.bitlinear_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    L.bitlinear_calib_mfma.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().bitlinear_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise BitLinearError(fn, status)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def quantize_weights_workspace_bytes(count: int = 1) -> int:
    return int(lib().bitlinear_quantize_weights_grouped_workspace(count))


def quantize_weights_one_read_workspace_bytes(problems, count: int) -> int:
    """Workspace bytes with which the grouped and step calls read each fp32 master once
    (problems: a ctypes array of _WeightProblem)."""
    return int(lib().bitlinear_quantize_weights_one_read_workspace(ctypes.addressof(problems), count))


def _weight_workspace(arr, count: int, one_read: bool, device) -> torch.Tensor:
    nbytes = quantize_weights_workspace_bytes(max(count, 1))
    if one_read and count:
        nbytes = max(nbytes, quantize_weights_one_read_workspace_bytes(arr, count))
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def quantize_weights(W: torch.Tensor, W_packed: Optional[torch.Tensor] = None,
                     gamma: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None,
                     stream=None, one_read: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """W fp32 [N, K] -> (W_packed int32 [N, K/16] holding uint32 words, gamma fp32 [1]).
    one_read: allocate the workspace with which a tensor of 64 MB or more is read once."""
    _dev(W, "W", torch.float32)
    N, K = W.shape
    if W_packed is None:
        W_packed = torch.empty((N, K // 16), dtype=torch.int32, device=W.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    if workspace is None:
        arr = (_WeightProblem * 1)()
        arr[0] = _WeightProblem(_ptr(W), _ptr(W_packed), _ptr(gamma), N, K)
        workspace = _weight_workspace(arr, 1, one_read, W.device)
    _check("bitlinear_quantize_weights",
           lib().bitlinear_quantize_weights(_ptr(W), N, K, _ptr(W_packed), _ptr(gamma),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream)))
    return W_packed, gamma


def quantize_weights_grouped(Ws: Sequence[torch.Tensor],
                             outputs: Optional[Sequence[Tuple[torch.Tensor, torch.Tensor]]] = None,
                             workspace: Optional[torch.Tensor] = None,
                             stream=None, one_read: bool = True) -> List[Tuple[torch.Tensor, torch.Tensor]]:
    """Several independent weight tensors in one grouped call (two kernel launches; three that
    read W once for large sets when the workspace allows: one_read, the default, allocates it)."""
    count = len(Ws)
    arr = (_WeightProblem * max(count, 1))()
    outs = []
    for i, W in enumerate(Ws):
        _dev(W, f"W[{i}]", torch.float32)
        N, K = W.shape
        if outputs is not None:
            P, g = outputs[i]
        else:
            P = torch.empty((N, K // 16), dtype=torch.int32, device=W.device)
            g = torch.empty(1, dtype=torch.float32, device=W.device)
        outs.append((P, g))
        arr[i] = _WeightProblem(_ptr(W), _ptr(P), _ptr(g), N, K)
    if workspace is None:
        workspace = _weight_workspace(arr, count, one_read, Ws[0].device)
    _check("bitlinear_quantize_weights_grouped",
           lib().bitlinear_quantize_weights_grouped(ctypes.addressof(arr), count, _ptr(workspace),
                                                    workspace.numel() * workspace.element_size(),
                                                    _stream(stream)))
    return outs


def quantize_weights_grouped_noalloc(Ws: Sequence[torch.Tensor],
                                     outputs: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                                     stream=None) -> None:
    """The grouped weight quantization into caller-provided outputs with no workspace (the
    library's fixed scratch holds the partial sums; calls overlapping on one GPU race)."""
    count = len(Ws)
    arr = (_WeightProblem * max(count, 1))()
    for i, W in enumerate(Ws):
        _dev(W, f"W[{i}]", torch.float32)
        N, K = W.shape
        P, g = outputs[i]
        arr[i] = _WeightProblem(_ptr(W), _ptr(P), _ptr(g), N, K)
    _check("bitlinear_quantize_weights_grouped_noalloc",
           lib().bitlinear_quantize_weights_grouped_noalloc(ctypes.addressof(arr), count,
                                                            _stream(stream)))


def pack_codes(codes: torch.Tensor, W_packed: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Ternary int8 codes [N, K] in {-1, 0, +1} -> packed words [N, K/16] (int32 storage)."""
    _dev(codes, "codes", torch.int8)
    N, K = codes.shape
    if W_packed is None:
        W_packed = torch.empty((N, K // 16), dtype=torch.int32, device=codes.device)
    _check("bitlinear_pack_codes",
           lib().bitlinear_pack_codes(_ptr(codes), N, K, _ptr(W_packed), _stream(stream)))
    return W_packed


def _x_dtype(X: torch.Tensor) -> int:
    if X.dtype == torch.float32:
        return BL_F32
    if X.dtype == torch.bfloat16:
        return BL_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {X.dtype}")


def quantize_acts(X: torch.Tensor, norm_weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                  X_q: Optional[torch.Tensor] = None, x_scale: Optional[torch.Tensor] = None,
                  stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """X fp32/bf16 [M, K] -> (X_q int8 [M, K], x_scale fp32 [M]); optional fused RMSNorm."""
    _dev(X, "X")
    dt = _x_dtype(X)
    M, K = X.shape
    if norm_weight is not None:
        _dev(norm_weight, "norm_weight", torch.float32)
    if X_q is None:
        X_q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    _check("bitlinear_quantize_acts",
           lib().bitlinear_quantize_acts(_ptr(X), dt, M, K, _ptr(norm_weight), float(eps),
                                         _ptr(X_q), _ptr(x_scale), _stream(stream)))
    return X_q, x_scale


def quantize_acts_grouped(Xs: Sequence[torch.Tensor],
                          norm_weights: Optional[Sequence[Optional[torch.Tensor]]] = None,
                          eps: float = 1e-6, outputs=None, stream=None):
    """Several activation matrices in one launch; returns [(X_q, x_scale), ...]."""
    count = len(Xs)
    arr = (_ActProblem * max(count, 1))()
    outs = []
    for i, X in enumerate(Xs):
        _dev(X, f"X[{i}]")
        M, K = X.shape
        g = None if norm_weights is None else norm_weights[i]
        if outputs is not None:
            Xq, sx = outputs[i]
        else:
            Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
            sx = torch.empty(M, dtype=torch.float32, device=X.device)
        outs.append((Xq, sx))
        arr[i] = _ActProblem(_ptr(X), _ptr(g), _ptr(Xq), _ptr(sx), M, K, _x_dtype(X), float(eps))
    _check("bitlinear_quantize_acts_grouped",
           lib().bitlinear_quantize_acts_grouped(ctypes.addressof(arr), count, _stream(stream)))
    return outs


def quantize_step(Ws: Sequence[torch.Tensor], Xs: Sequence[torch.Tensor],
                  norm_weights: Optional[Sequence[Optional[torch.Tensor]]] = None,
                  eps: float = 1e-6, w_outputs=None, x_outputs=None, workspace=None, stream=None,
                  quad_rows: bool = False, one_read: bool = True):
    """Weight quantization of Ws and activation quantization of Xs in one call (the gamma pass
    and the activation codes share a launch when they can); returns ([(W_packed, gamma)],
    [(X_q, x_scale)]), bit for bit those of the two grouped calls.  quad_rows: the packed
    words in the quad-row layout (bitlinear_quantize_step_quad_rows).  one_read: allocate the
    workspace with which large sets read each master once (same results)."""
    nw, na = len(Ws), len(Xs)
    wa = (_WeightProblem * max(nw, 1))()
    wouts = []
    for i, W in enumerate(Ws):
        _dev(W, f"W[{i}]", torch.float32)
        N, K = W.shape
        if w_outputs is not None:
            P, g = w_outputs[i]
        else:
            P = torch.empty((N, K // 16), dtype=torch.int32, device=W.device)
            g = torch.empty(1, dtype=torch.float32, device=W.device)
        wouts.append((P, g))
        wa[i] = _WeightProblem(_ptr(W), _ptr(P), _ptr(g), N, K)
    xa = (_ActProblem * max(na, 1))()
    xouts = []
    for i, X in enumerate(Xs):
        _dev(X, f"X[{i}]")
        M, K = X.shape
        g = None if norm_weights is None else norm_weights[i]
        if x_outputs is not None:
            Xq, sx = x_outputs[i]
        else:
            Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
            sx = torch.empty(M, dtype=torch.float32, device=X.device)
        xouts.append((Xq, sx))
        xa[i] = _ActProblem(_ptr(X), _ptr(g), _ptr(Xq), _ptr(sx), M, K, _x_dtype(X), float(eps))
    if workspace is None and nw:
        workspace = _weight_workspace(wa, nw, one_read, Ws[0].device)
    fn = "bitlinear_quantize_step_quad_rows" if quad_rows else "bitlinear_quantize_step"
    _check(fn, getattr(lib(), fn)(ctypes.addressof(wa), nw, _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  ctypes.addressof(xa), na, _stream(stream)))
    return wouts, xouts


def forward(X_q: torch.Tensor, x_scale: torch.Tensor, W_packed: torch.Tensor,
            gamma: torch.Tensor, Y: Optional[torch.Tensor] = None,
            acc: Optional[torch.Tensor] = None, return_acc: bool = False, stream=None):
    """Y = (X_q . c^T) * gamma * x_scale[:, None] in fp32; optionally the int32 accumulators."""
    _dev(X_q, "X_q", torch.int8)
    M, K = X_q.shape
    N = W_packed.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X_q.device)
    if return_acc and acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=X_q.device)
    _check("bitlinear_forward",
           lib().bitlinear_forward(_ptr(X_q), _ptr(x_scale), _ptr(W_packed), _ptr(gamma), M, N, K,
                                   _ptr(Y), _ptr(acc), _stream(stream)))
    return (Y, acc) if return_acc else Y


def forward_grouped(problems: Sequence[dict], stream=None, quad_rows: bool = False) -> None:
    """Problems as dicts with keys X_q, x_scale, W_packed, gamma, Y and optional acc; all
    outputs preallocated.  Decode-sized problems (M <= 16) share one launch, the rest another.
    quad_rows: W_packed in the quad-row layout (bitlinear_forward_quad_rows_grouped)."""
    count = len(problems)
    arr = (_ForwardProblem * max(count, 1))()
    for i, p in enumerate(problems):
        M, K = p["X_q"].shape
        N = p["W_packed"].shape[0]
        arr[i] = _ForwardProblem(_ptr(p["X_q"]), _ptr(p["x_scale"]), _ptr(p["W_packed"]),
                                 _ptr(p["gamma"]), _ptr(p["Y"]), _ptr(p.get("acc")), M, N, K)
    fn = "bitlinear_forward_quad_rows_grouped" if quad_rows else "bitlinear_forward_grouped"
    _check(fn, getattr(lib(), fn)(ctypes.addressof(arr), count, _stream(stream)))


def linear_fused(M: int, K: int) -> bool:
    """Whether a layer call of M tokens and K inputs takes the one-launch decode form."""
    return M <= LINEAR_FUSED_MAX_M and M * K <= LINEAR_FUSED_MAX_BYTES


def linear_table(problems: Sequence[dict]):
    """ctypes array for bitlinear_linear_grouped: dicts with keys X (fp32/bf16 [M, K]),
    W_packed, gamma, Y (preallocated fp32 [M, N]) and optional norm_weight, eps, X_q, x_scale
    (code/scale outputs; required when the call is not decode-sized)."""
    arr = (_LinearProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        X = _dev(p["X"], f"X[{i}]")
        M, K = X.shape
        N = p["W_packed"].shape[0]
        arr[i] = _LinearProblem(_ptr(X), _ptr(p.get("norm_weight")), _ptr(p["W_packed"]),
                                _ptr(p["gamma"]), _ptr(p["Y"]), _ptr(p.get("X_q")),
                                _ptr(p.get("x_scale")), M, N, K, _x_dtype(X),
                                float(p.get("eps", 1e-6)))
    return arr


def linear_grouped(problems: Sequence[dict], stream=None) -> None:
    """Layer calls (dicts as for linear_table); decode-sized calls share one fused launch."""
    arr = linear_table(problems)
    _check("bitlinear_linear_grouped",
           lib().bitlinear_linear_grouped(ctypes.addressof(arr), len(problems), _stream(stream)))


def linear(X: torch.Tensor, W_packed: torch.Tensor, gamma: torch.Tensor,
           norm_weight: Optional[torch.Tensor] = None, eps: float = 1e-6, stream=None):
    """Y = BitLinear(X): steps 3 to 5 (one fused launch when decode-sized, else two)."""
    _dev(X, "X")
    M, K = X.shape
    N = W_packed.shape[0]
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    p = dict(X=X, W_packed=W_packed, gamma=gamma, Y=Y, norm_weight=norm_weight, eps=eps)
    if not linear_fused(M, K):
        p["X_q"] = torch.empty((M, K), dtype=torch.int8, device=X.device)
        p["x_scale"] = torch.empty(M, dtype=torch.float32, device=X.device)
    linear_grouped([p], stream=stream)
    return Y


def act_ex_table(problems: Sequence[dict]):
    """ctypes array for bitlinear_quantize_acts_ex_grouped: dicts with X, X_q, x_scale and
    optional X2, norm_weight, act (ACT_*), eps."""
    arr = (_ActExProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        X = _dev(p["X"], f"X[{i}]")
        M, K = X.shape
        X2 = p.get("X2")
        if X2 is not None:
            _dev(X2, f"X2[{i}]", torch.float32)
            if tuple(X2.shape) != (M, K):
                raise ValueError(f"X2[{i}] must have the shape of X")
        arr[i] = _ActExProblem(_ptr(X), _ptr(X2), _ptr(p.get("norm_weight")), _ptr(p["X_q"]),
                               _ptr(p["x_scale"]), M, K, _x_dtype(X), int(p.get("act", ACT_NONE)),
                               float(p.get("eps", 1e-6)))
    return arr


def quantize_acts_ex_grouped(problems: Sequence[dict], stream=None) -> None:
    """Activation quantization with an optional FFN activation in front (see act_ex_table);
    outputs preallocated."""
    arr = act_ex_table(problems)
    _check("bitlinear_quantize_acts_ex_grouped",
           lib().bitlinear_quantize_acts_ex_grouped(ctypes.addressof(arr), len(problems),
                                                    _stream(stream)))


def forward_ex_table(problems: Sequence[dict]):
    """ctypes array for bitlinear_forward_ex_grouped: dicts as for forward_grouped plus an
    optional fp32 residual [M, N]."""
    arr = (_ForwardExProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        M, K = p["X_q"].shape
        N = p["W_packed"].shape[0]
        R = p.get("residual")
        if R is not None:
            _dev(R, f"residual[{i}]", torch.float32)
            if tuple(R.shape) != (M, N):
                raise ValueError(f"residual[{i}] must be [M, N]")
        arr[i] = _ForwardExProblem(_ptr(p["X_q"]), _ptr(p["x_scale"]), _ptr(p["W_packed"]),
                                   _ptr(p["gamma"]), _ptr(p["Y"]), _ptr(p.get("acc")), _ptr(R),
                                   M, N, K)
    return arr


def forward_ex_grouped(problems: Sequence[dict], stream=None, quad_rows: bool = False) -> None:
    """Products with an optional residual added in the epilogue; outputs preallocated.
    quad_rows: W_packed in the quad-row layout (bitlinear_forward_ex_quad_rows_grouped)."""
    arr = forward_ex_table(problems)
    fn = "bitlinear_forward_ex_quad_rows_grouped" if quad_rows else "bitlinear_forward_ex_grouped"
    _check(fn, getattr(lib(), fn)(ctypes.addressof(arr), len(problems), _stream(stream)))


def forward_mixed(prefill: Sequence[dict], decode: Sequence[dict], stream=None) -> None:
    """A mixed batch: prefill products (dicts as for forward_ex_table) and decode layer calls
    (dicts as for linear_table), in one launch when both sets allow it; results equal
    forward_ex_grouped(prefill) followed by linear_grouped(decode)."""
    pre = forward_ex_table(prefill)
    dec = linear_table(decode)
    _check("bitlinear_forward_mixed",
           lib().bitlinear_forward_mixed(ctypes.addressof(pre), len(prefill), ctypes.addressof(dec),
                                         len(decode), _stream(stream)))


def linear_ex_table(problems: Sequence[dict]):
    """ctypes array for bitlinear_linear_ex_grouped: dicts as for linear_grouped plus the
    optional W2_packed / gamma2 (the up projection of a gated pair), act (ACT_*) and an fp32
    residual [M, N]."""
    arr = (_LinearExProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        X = _dev(p["X"], f"X[{i}]")
        M, K = X.shape
        N = p["W_packed"].shape[0]
        W2 = p.get("W2_packed")
        if W2 is not None and tuple(W2.shape) != tuple(p["W_packed"].shape):
            raise ValueError(f"W2_packed[{i}] must have the shape of W_packed")
        R = p.get("residual")
        if R is not None:
            _dev(R, f"residual[{i}]", torch.float32)
            if tuple(R.shape) != (M, N):
                raise ValueError(f"residual[{i}] must be [M, N]")
        arr[i] = _LinearExProblem(_ptr(X), _ptr(p.get("norm_weight")), _ptr(p["W_packed"]),
                                  _ptr(p["gamma"]), _ptr(W2), _ptr(p.get("gamma2")), _ptr(p["Y"]),
                                  _ptr(R), _ptr(p.get("X_q")), _ptr(p.get("x_scale")), M, N, K,
                                  _x_dtype(X), int(p.get("act", ACT_NONE)), float(p.get("eps", 1e-6)))
    return arr


def linear_ex_grouped(problems: Sequence[dict], stream=None) -> None:
    """Decode-sized layer calls with the output stages in the epilogue (gated-pair
    activation, ReLU^2, residual); outputs preallocated.  Every call must fit the fused form
    (linear_fused(M, K))."""
    arr = linear_ex_table(problems)
    _check("bitlinear_linear_ex_grouped",
           lib().bitlinear_linear_ex_grouped(ctypes.addressof(arr), len(problems), _stream(stream)))


# ------------------------------------------------------------- training side

def forward_wonly_grouped(problems: Sequence[dict], stream=None) -> None:
    """Weight-only ternary forward Y = gamma * X C^T: dicts with X (fp32/bf16 [M, K]),
    W_packed, gamma, Y (preallocated fp32 [M, N])."""
    arr = (_WonlyProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        X = _dev(p["X"], f"X[{i}]")
        M, K = X.shape
        N = p["W_packed"].shape[0]
        arr[i] = _WonlyProblem(_ptr(X), _ptr(p["W_packed"]), _ptr(p["gamma"]), _ptr(p["Y"]), M, N, K,
                               _x_dtype(X))
    _check("bitlinear_forward_wonly_grouped",
           lib().bitlinear_forward_wonly_grouped(ctypes.addressof(arr), len(problems), _stream(stream)))


def forward_wonly(X: torch.Tensor, W_packed: torch.Tensor, gamma: torch.Tensor, stream=None):
    Y = torch.empty((X.shape[0], W_packed.shape[0]), dtype=torch.float32, device=X.device)
    forward_wonly_grouped([dict(X=X, W_packed=W_packed, gamma=gamma, Y=Y)], stream)
    return Y


def transpose_packed(W_packed: torch.Tensor, K: Optional[int] = None,
                     Wt_packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Packed codes [N, K/16] -> the transposed codes packed [K, N/16] (N % 16 == 0)."""
    _dev(W_packed, "W_packed", torch.int32)
    N = W_packed.shape[0]
    K = W_packed.shape[1] * 16 if K is None else K
    if Wt_packed is None:
        Wt_packed = torch.empty((K, N // 16), dtype=torch.int32, device=W_packed.device)
    _check("bitlinear_transpose_packed",
           lib().bitlinear_transpose_packed(_ptr(W_packed), N, K, _ptr(Wt_packed), _stream(stream)))
    return Wt_packed


def grad_input_grouped(problems: Sequence[dict], stream=None) -> None:
    """Input gradient dX = gamma * dY C: dicts with dY (fp32/bf16 [M, N]), Wt_packed
    (transpose_packed of the forward's codes, [K, N/16]), gamma, dX (preallocated [M, K])."""
    arr = (_GradInputProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        dY = _dev(p["dY"], f"dY[{i}]")
        M, N = dY.shape
        K = p["Wt_packed"].shape[0]
        if p["Wt_packed"].shape[1] * 16 != N:
            raise ValueError(f"Wt_packed[{i}] must be [K, N/16]")
        arr[i] = _GradInputProblem(_ptr(dY), _ptr(p["Wt_packed"]), _ptr(p["gamma"]), _ptr(p["dX"]),
                                   M, N, K, _x_dtype(dY))
    _check("bitlinear_grad_input_grouped",
           lib().bitlinear_grad_input_grouped(ctypes.addressof(arr), len(problems), _stream(stream)))


def grad_input(dY: torch.Tensor, Wt_packed: torch.Tensor, gamma: torch.Tensor, stream=None):
    dX = torch.empty((dY.shape[0], Wt_packed.shape[0]), dtype=torch.float32, device=dY.device)
    grad_input_grouped([dict(dY=dY, Wt_packed=Wt_packed, gamma=gamma, dX=dX)], stream)
    return dX


def grad_weight_grouped(problems: Sequence[dict], stream=None) -> None:
    """Weight gradient through the STE: dicts with dY (fp32 [M, N]), X_q (int8 [M, K]),
    x_scale ([M]), gamma, dW (preallocated fp32 [N, K]) and optional W (fp32 masters [N, K],
    needed by STE_HARD / STE_SOFT), ste (STE_*), beta (default 2)."""
    arr = (_GradWeightProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        dY = _dev(p["dY"], f"dY[{i}]", torch.float32)
        Xq = _dev(p["X_q"], f"X_q[{i}]", torch.int8)
        M, N = dY.shape
        K = Xq.shape[1]
        if Xq.shape[0] != M or tuple(p["dW"].shape) != (N, K):
            raise ValueError(f"problem {i}: dY [M, N], X_q [M, K], dW [N, K]")
        arr[i] = _GradWeightProblem(_ptr(dY), _ptr(Xq), _ptr(p["x_scale"]), _ptr(p.get("W")),
                                    _ptr(p["gamma"]), _ptr(p["dW"]), M, N, K, int(p.get("ste", STE_PASS)),
                                    float(p.get("beta", 2.0)))
    _check("bitlinear_grad_weight_grouped",
           lib().bitlinear_grad_weight_grouped(ctypes.addressof(arr), len(problems), _stream(stream)))


def grad_weight(dY: torch.Tensor, X_q: torch.Tensor, x_scale: torch.Tensor, gamma: torch.Tensor,
                W: Optional[torch.Tensor] = None, ste: int = STE_PASS, beta: float = 2.0, stream=None):
    dW = torch.empty((dY.shape[1], X_q.shape[1]), dtype=torch.float32, device=dY.device)
    grad_weight_grouped([dict(dY=dY, X_q=X_q, x_scale=x_scale, gamma=gamma, dW=dW, W=W, ste=ste,
                              beta=beta)], stream)
    return dW


# ------------------------------------------------------------- base-3 weights

def b3_row_bytes(K: int) -> int:
    """Bytes per row of the base-3 layout (five codes per byte, 80 weights per 16 bytes)."""
    return int(lib().bitlinear_b3_row_bytes(int(K)))


def pack_b3(W_packed: torch.Tensor, K: Optional[int] = None, W_b3: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    """Two-bit packed codes [N, K/16] -> base-3 bytes (uint8 [N, b3_row_bytes(K)])."""
    _dev(W_packed, "W_packed", torch.int32)
    N = W_packed.shape[0]
    K = W_packed.shape[1] * 16 if K is None else K
    if W_b3 is None:
        W_b3 = torch.empty((N, b3_row_bytes(K)), dtype=torch.uint8, device=W_packed.device)
    _check("bitlinear_pack_b3", lib().bitlinear_pack_b3(_ptr(W_packed), N, K, _ptr(W_b3), _stream(stream)))
    return W_b3


def linear_b3_table(problems: Sequence[dict]):
    """ctypes array for bitlinear_linear_b3_grouped: dicts as for linear_grouped, with
    W_b3 (uint8 [N, b3_row_bytes(K)]) in place of W_packed."""
    arr = (_LinearProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        X = _dev(p["X"], f"X[{i}]")
        M, K = X.shape
        Wb = _dev(p["W_b3"], f"W_b3[{i}]", torch.uint8)
        N = Wb.shape[0]
        if Wb.shape[1] != b3_row_bytes(K):
            raise ValueError(f"W_b3[{i}] must be [N, b3_row_bytes(K)]")
        arr[i] = _LinearProblem(_ptr(X), _ptr(p.get("norm_weight")), _ptr(Wb), _ptr(p["gamma"]),
                                _ptr(p["Y"]), _ptr(p.get("X_q")), _ptr(p.get("x_scale")), M, N, K,
                                _x_dtype(X), float(p.get("eps", 1e-6)))
    return arr


def linear_b3_grouped(problems: Sequence[dict], stream=None) -> None:
    """The fused decode layer call on base-3 weights (every call decode-sized)."""
    arr = linear_b3_table(problems)
    _check("bitlinear_linear_b3_grouped",
           lib().bitlinear_linear_b3_grouped(ctypes.addressof(arr), len(problems), _stream(stream)))


# ------------------------------------------------------------- decode tiles

def tiles_bytes(N: int, K: int) -> int:
    """Bytes of the decode tile layout of an N x K weight matrix."""
    return int(lib().bitlinear_tiles_bytes(int(N), int(K)))


def pack_tiles(W_packed: torch.Tensor, K: Optional[int] = None, W_tiles: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Two-bit packed codes [N, K/16] -> decode tiles (flat int32 [tiles_bytes(N, K) / 4])."""
    _dev(W_packed, "W_packed", torch.int32)
    N = W_packed.shape[0]
    K = W_packed.shape[1] * 16 if K is None else K
    if W_tiles is None:
        W_tiles = torch.empty(tiles_bytes(N, K) // 4, dtype=torch.int32, device=W_packed.device)
    _check("bitlinear_pack_tiles", lib().bitlinear_pack_tiles(_ptr(W_packed), N, K, _ptr(W_tiles),
                                                              _stream(stream)))
    return W_tiles


def linear_tiles_table(problems: Sequence[dict]):
    """ctypes array for bitlinear_linear_tiles_grouped: dicts as for linear_grouped, with
    W_tiles (flat int32, at least tiles_bytes(N, K) / 4 elements) in place of W_packed; N is
    Y's column count."""
    arr = (_LinearProblem * max(len(problems), 1))()
    for i, p in enumerate(problems):
        X = _dev(p["X"], f"X[{i}]")
        M, K = X.shape
        Y = _dev(p["Y"], f"Y[{i}]", torch.float32)
        N = Y.shape[1]
        Wt = _dev(p["W_tiles"], f"W_tiles[{i}]", torch.int32)
        if Wt.numel() * 4 < tiles_bytes(N, K):
            raise ValueError(f"W_tiles[{i}] must hold tiles_bytes(N, K) bytes")
        arr[i] = _LinearProblem(_ptr(X), _ptr(p.get("norm_weight")), _ptr(Wt), _ptr(p["gamma"]),
                                _ptr(Y), _ptr(p.get("X_q")), _ptr(p.get("x_scale")), M, N, K,
                                _x_dtype(X), float(p.get("eps", 1e-6)))
    return arr


def linear_tiles_grouped(problems: Sequence[dict], stream=None) -> None:
    """The fused one-token layer call on decode tiles."""
    arr = linear_tiles_table(problems)
    _check("bitlinear_linear_tiles_grouped",
           lib().bitlinear_linear_tiles_grouped(ctypes.addressof(arr), len(problems), _stream(stream)))


# ---------------------------------------------------------------- quad rows

def pack_quad_rows(W_packed: torch.Tensor, W_quad: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Two-bit packed codes [N, K/16] -> the quad-row layout (a new [N, K/16] int32 tensor
    unless W_quad is given; N % 4 == 0, K % 128 == 0)."""
    _dev(W_packed, "W_packed", torch.int32)
    N, words = W_packed.shape
    if W_quad is None:
        W_quad = torch.empty_like(W_packed)
    _check("bitlinear_pack_quad_rows", lib().bitlinear_pack_quad_rows(_ptr(W_packed), N, words * 16,
                                                                        _ptr(W_quad), _stream(stream)))
    return W_quad


# ----------------------------------------------------------------- measurement helpers

CALIB_INT8, CALIB_BF16 = 0, 1
CALIB_OPS = {CALIB_INT8: 32768, CALIB_BF16: 16384}   # operations per matrix-unit instruction


def calib_stream(buf: torch.Tensor, xor_out: torch.Tensor, stream=None) -> None:
    """XOR of buf's 32-bit words into xor_out (int32 [1], zeroed by the caller): one read of
    buf, the HBM read-stream calibration."""
    buf = _dev(buf, "buf")
    _check("bitlinear_calib_stream",
           lib().bitlinear_calib_stream(_ptr(buf), buf.numel() * buf.element_size(), _ptr(xor_out),
                                        _stream(stream)))


def calib_mfma(kind: int, iters: int, blocks: int, out: torch.Tensor, stream=None) -> int:
    """Matrix-unit loop (kind CALIB_INT8 or CALIB_BF16) into out (int32 [256 * blocks]);
    returns the number of operations it performs."""
    _check("bitlinear_calib_mfma",
           lib().bitlinear_calib_mfma(int(kind), int(iters), int(blocks), _ptr(out), _stream(stream)))
    return blocks * 4 * 8 * iters * CALIB_OPS[kind]
