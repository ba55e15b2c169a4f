"""Python binding of libdbf, the MI355X DBF linear-forward library.

Double Binary Factorization stores a weight matrix as
W = diag(a) A diag(mid) B diag(b) with +/-1 factors A (n x k), B (k x m) and
fp16 scale vectors ("Addition is almost all you need: Compressing large
language models with double binary factorization", gist.science technical
summary, §2.1).  The library evaluates Y = X W^T on the GPU without forming W.

This module only marshals arguments to the C ABI declared in include/dbf.h:
every step of the forward runs in the library's HIP kernels.  PyTorch is
used for device memory and the current stream, nothing else.  If the shared
library has not been built the first call raises a RuntimeError; there is no
fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

__all__ = [
    "DBF_OK", "DBF_ERR_INVALID_ARG", "DBF_ERR_SHAPE", "DBF_ERR_OOM", "DBF_ERR_HIP", "DBF_ERR_UNSUPPORTED",
    "DBF_PATH_AUTO", "DBF_PATH_DECODE", "DBF_PATH_PREFILL", "DBF_PATH_DECODE_TABLE", "DBF_PATH_DECODE_EXACT",
    "EXPORTED_SYMBOLS",
    "DbfError", "lib", "library_path",
    "dbf_pack", "dbf_linear_forward", "dbf_linear_forward_ex", "dbf_free", "dbf_get_info",
    "dbf_status_string", "dbf_pack_signs", "dbf_layout_signs", "dbf_layout_words", "dbf_layout_signs_dec",
    "dbf_layout_words_dec",
    "dbf_timing_enable", "dbf_timing_read", "Layer", "dbf_linear_forward_group", "forward_group",
    "dbf_pack_ex", "dbf_linear_backward_data", "dbf_linear_backward", "DBF_PACK_BACKWARD", "dbf_bqq_pack",
    "dbf_factorize", "factorize", "dbf_linear_forward_noalloc", "dbf_bqq_pack_grouped",
]

DBF_OK = 0
DBF_ERR_INVALID_ARG = 1
DBF_ERR_SHAPE = 2
DBF_ERR_OOM = 3
DBF_ERR_HIP = 4
DBF_ERR_UNSUPPORTED = 5

DBF_PATH_AUTO = 0
DBF_PATH_DECODE = 1
DBF_PATH_PREFILL = 2
DBF_PATH_DECODE_TABLE = 3
DBF_PATH_DECODE_EXACT = 4

DBF_PACK_BACKWARD = 1

DECODE_MAX_BATCH = 16

EXPORTED_SYMBOLS = (
    "dbf_pack", "dbf_pack_ex", "dbf_linear_forward", "dbf_linear_forward_ex", "dbf_linear_forward_group",
    "dbf_linear_backward_data", "dbf_linear_backward", "dbf_free", "dbf_get_info", "dbf_status_string",
    "dbf_pack_signs", "dbf_layout_signs", "dbf_layout_words", "dbf_layout_signs_dec", "dbf_layout_words_dec",
    "dbf_timing_enable", "dbf_timing_read", "dbf_bqq_pack", "dbf_factorize", "dbf_linear_forward_noalloc",
    "dbf_bqq_pack_grouped",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdbf.so")
_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return _LIB_PATH


class DbfError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dbf_status_string(status)} (status {status})")


class _Info(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int32), ("m", ctypes.c_int32), ("k", ctypes.c_int32),
        ("n_pad", ctypes.c_int32), ("m_pad", ctypes.c_int32), ("k_pad", ctypes.c_int32),
        ("max_batch", ctypes.c_int32), ("device", ctypes.c_int32),
        ("packed_bytes", ctypes.c_size_t), ("scale_bytes", ctypes.c_size_t),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


def lib() -> ctypes.CDLL:
    """Load libdbf.so (once).  Raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m dbf_linear_fwd_amd.build` "
            "(the DBF forward has no non-HIP implementation)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.dbf_pack.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, i32, ctypes.POINTER(vp)]
    L.dbf_pack.restype = ctypes.c_int
    L.dbf_linear_forward.argtypes = [vp, vp, vp, i32, vp]
    L.dbf_linear_forward.restype = ctypes.c_int
    L.dbf_linear_forward_ex.argtypes = [vp, vp, vp, i32, i32, vp]
    L.dbf_linear_forward_ex.restype = ctypes.c_int
    L.dbf_linear_forward_noalloc.argtypes = [vp, vp, vp, i32, vp]
    L.dbf_linear_forward_noalloc.restype = ctypes.c_int
    L.dbf_pack_ex.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, i32, i32, ctypes.POINTER(vp)]
    L.dbf_pack_ex.restype = ctypes.c_int
    L.dbf_bqq_pack.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, ctypes.c_uint16, i32, ctypes.POINTER(vp)]
    L.dbf_bqq_pack.restype = ctypes.c_int
    L.dbf_bqq_pack_grouped.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, ctypes.POINTER(vp)]
    L.dbf_bqq_pack_grouped.restype = ctypes.c_int
    L.dbf_factorize.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32,
                                vp, vp, vp, vp, vp, vp, vp]
    L.dbf_factorize.restype = ctypes.c_int
    L.dbf_linear_backward_data.argtypes = [vp, vp, vp, i32, vp]
    L.dbf_linear_backward_data.restype = ctypes.c_int
    L.dbf_linear_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp]
    L.dbf_linear_backward.restype = ctypes.c_int
    L.dbf_linear_forward_group.argtypes = [ctypes.POINTER(vp), i32, vp, ctypes.POINTER(vp), i32, vp]
    L.dbf_linear_forward_group.restype = ctypes.c_int
    L.dbf_free.argtypes = [vp]
    L.dbf_free.restype = None
    L.dbf_get_info.argtypes = [vp, ctypes.POINTER(_Info)]
    L.dbf_get_info.restype = ctypes.c_int
    L.dbf_status_string.argtypes = [ctypes.c_int]
    L.dbf_status_string.restype = ctypes.c_char_p
    L.dbf_pack_signs.argtypes = [vp, i32, i32, vp, i32]
    L.dbf_pack_signs.restype = ctypes.c_int
    L.dbf_layout_signs.argtypes = [vp, i32, i32, vp]
    L.dbf_layout_signs.restype = ctypes.c_int
    L.dbf_layout_words.argtypes = [i32, i32]
    L.dbf_layout_words.restype = sz
    L.dbf_layout_signs_dec.argtypes = [vp, i32, i32, i32, i32, i32, vp]
    L.dbf_layout_signs_dec.restype = ctypes.c_int
    L.dbf_layout_words_dec.argtypes = [i32, i32]
    L.dbf_layout_words_dec.restype = sz
    L.dbf_timing_enable.argtypes = [vp, i32]
    L.dbf_timing_enable.restype = ctypes.c_int
    L.dbf_timing_read.argtypes = [vp, ctypes.POINTER(_KernelTime), i32, ctypes.POINTER(i32)]
    L.dbf_timing_read.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != DBF_OK:
        raise DbfError(status, where)


def _ptr(arr: np.ndarray) -> int:
    return arr.ctypes.data


def dbf_status_string(status: int) -> str:
    return lib().dbf_status_string(int(status)).decode()


def _as_signs(S) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(S), dtype=np.int8)


def _as_half_bits(v) -> np.ndarray:
    v = np.asarray(v)
    if v.dtype == np.uint16:
        return np.ascontiguousarray(v)
    return np.ascontiguousarray(v.astype(np.float16)).view(np.uint16)


def dbf_pack(n: int, m: int, k: int, A_signs, B_signs, a, mid, b, max_batch: int, flags: int = 0) -> int:
    """Build a layer handle (see dbf_pack / dbf_pack_ex in include/dbf.h).  Returns the handle as an int."""
    A = _as_signs(A_signs)
    B = _as_signs(B_signs)
    if A.size != n * k or B.size != k * m:
        raise ValueError("A must hold n*k and B k*m entries")
    a16, mid16, b16 = _as_half_bits(a), _as_half_bits(mid), _as_half_bits(b)
    if a16.size != n or mid16.size != k or b16.size != m:
        raise ValueError("a, mid, b must have lengths n, k, m")
    h = ctypes.c_void_p()
    if flags:
        st = lib().dbf_pack_ex(n, m, k, _ptr(A), _ptr(B), _ptr(a16), _ptr(mid16), _ptr(b16), max_batch, flags,
                               ctypes.byref(h))
    else:
        st = lib().dbf_pack(n, m, k, _ptr(A), _ptr(B), _ptr(a16), _ptr(mid16), _ptr(b16), max_batch,
                            ctypes.byref(h))
    _check(st, "dbf_pack")
    return h.value


def dbf_bqq_pack(n: int, m: int, d: int, p: int, Y, Z, r, s, t, u, max_batch: int) -> int:
    """Handle of a BQQ-form layer (see dbf_bqq_pack in include/dbf.h): Y (p, n, d) and
    Z (p, d, m) of 0/1, fp16 scalars r, s, t (p each) and u."""
    Y8 = np.ascontiguousarray(np.asarray(Y), dtype=np.uint8)
    Z8 = np.ascontiguousarray(np.asarray(Z), dtype=np.uint8)
    if Y8.size != p * n * d or Z8.size != p * d * m:
        raise ValueError("Y must hold p*n*d and Z p*d*m entries")
    r16, s16, t16 = _as_half_bits(r), _as_half_bits(s), _as_half_bits(t)
    if r16.size != p or s16.size != p or t16.size != p:
        raise ValueError("r, s, t must have p entries")
    u16 = int(_as_half_bits(np.asarray([u]))[0])
    h = ctypes.c_void_p()
    _check(lib().dbf_bqq_pack(n, m, d, p, _ptr(Y8), _ptr(Z8), _ptr(r16), _ptr(s16), _ptr(t16), u16, max_batch,
                              ctypes.byref(h)), "dbf_bqq_pack")
    return h.value


def dbf_bqq_pack_grouped(n: int, m: int, d: int, p: int, group: int, Y, Z, r, s, t, u, max_batch: int) -> int:
    """Handle of a BQQ-form layer with group-wise scalars (see dbf_bqq_pack_grouped in
    include/dbf.h): Y (p, n, d) and Z (p, d, m) of 0/1, fp16 r, s, t (p, ngroups) and u
    (ngroups,), ngroups = ceil(m / group)."""
    Y8 = np.ascontiguousarray(np.asarray(Y), dtype=np.uint8)
    Z8 = np.ascontiguousarray(np.asarray(Z), dtype=np.uint8)
    if Y8.size != p * n * d or Z8.size != p * d * m:
        raise ValueError("Y must hold p*n*d and Z p*d*m entries")
    if group < 1:
        raise ValueError("group must be positive")
    ng = -(-m // group)
    r16, s16, t16, u16 = _as_half_bits(r), _as_half_bits(s), _as_half_bits(t), _as_half_bits(u)
    if r16.size != p * ng or s16.size != p * ng or t16.size != p * ng or u16.size != ng:
        raise ValueError(f"r, s, t must have p * ngroups = {p * ng} entries and u ngroups = {ng}")
    h = ctypes.c_void_p()
    _check(lib().dbf_bqq_pack_grouped(n, m, d, p, group, _ptr(Y8), _ptr(Z8), _ptr(r16), _ptr(s16), _ptr(t16),
                                      _ptr(u16), max_batch, ctypes.byref(h)), "dbf_bqq_pack_grouped")
    return h.value


def dbf_factorize(W_ptr: int, n: int, m: int, k: int, U0_ptr: int, V0_ptr: int, dout_ptr: int, din_ptr: int,
                  rho_rel: float, outer: int, inner: int, power_iters: int, A_ptr: int, B_ptr: int, a_ptr: int,
                  mid_ptr: int, b_ptr: int, err_ptr: int, stream: int = 0) -> None:
    _check(lib().dbf_factorize(W_ptr, n, m, k, U0_ptr, V0_ptr, dout_ptr or None, din_ptr or None, rho_rel, outer,
                               inner, power_iters, A_ptr, B_ptr, a_ptr, mid_ptr, b_ptr, err_ptr or None, stream),
           "dbf_factorize")


def factorize(W, k: int, U0, V0, rho_rel: float = 1.0, outer: int = 2, inner: int = 4, power_iters: int = 8,
              d_out=None, d_in=None):
    """DBF factors of W (CUDA float32 tensor, n x m) from the starting factors
    U0 (n x k) and V0 (k x m): returns (A, B, a, mid, b, err) as CUDA tensors
    (int8 +/-1, int8 +/-1, float16 x 3, float32 [outer])."""
    import torch

    def dev32(t, shape, what):
        if t is None:
            return None
        if t.dtype != torch.float32 or not t.is_cuda or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{what} must be a contiguous CUDA float32 tensor of shape {shape}")
        return t
    n, m = W.shape
    dev32(W, (n, m), "W")
    dev32(U0, (n, k), "U0")
    dev32(V0, (k, m), "V0")
    dev32(d_out, (n,), "d_out")
    dev32(d_in, (m,), "d_in")
    dev = W.device
    A = torch.empty((n, k), dtype=torch.int8, device=dev)
    B = torch.empty((k, m), dtype=torch.int8, device=dev)
    a = torch.empty(n, dtype=torch.float16, device=dev)
    mid = torch.empty(k, dtype=torch.float16, device=dev)
    b = torch.empty(m, dtype=torch.float16, device=dev)
    err = torch.empty(outer, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    dbf_factorize(W.data_ptr(), n, m, k, U0.data_ptr(), V0.data_ptr(), d_out.data_ptr() if d_out is not None else 0,
                  d_in.data_ptr() if d_in is not None else 0, rho_rel, outer, inner, power_iters, A.data_ptr(),
                  B.data_ptr(), a.data_ptr(), mid.data_ptr(), b.data_ptr(), err.data_ptr(), stream)
    return A, B, a, mid, b, err


def dbf_linear_forward(h: int, x_ptr: int, y_ptr: int, batch: int, stream: int = 0) -> None:
    _check(lib().dbf_linear_forward(h, x_ptr, y_ptr, batch, stream), "dbf_linear_forward")


def dbf_linear_forward_ex(h: int, x_ptr: int, y_ptr: int, batch: int, path: int, stream: int = 0) -> None:
    _check(lib().dbf_linear_forward_ex(h, x_ptr, y_ptr, batch, path, stream), "dbf_linear_forward_ex")


def dbf_linear_forward_noalloc(h: int, x_ptr: int, y_ptr: int, batch: int, stream: int = 0) -> None:
    """dbf_linear_forward with the kernels' scratch in the library's static device array."""
    _check(lib().dbf_linear_forward_noalloc(h, x_ptr, y_ptr, batch, stream), "dbf_linear_forward_noalloc")


def dbf_linear_forward_group(hs, x_ptr: int, y_ptrs, batch: int, stream: int = 0) -> None:
    """Forwards of several layers that share the input x (device pointers)."""
    hs = list(hs)
    y_ptrs = list(y_ptrs)
    if len(hs) != len(y_ptrs):
        raise ValueError("one output per handle")
    harr = (ctypes.c_void_p * max(len(hs), 1))(*hs)
    yarr = (ctypes.c_void_p * max(len(y_ptrs), 1))(*y_ptrs)
    _check(lib().dbf_linear_forward_group(harr, len(hs), x_ptr, yarr, batch, stream), "dbf_linear_forward_group")


def forward_group(layers, x, outs=None):
    """ys[i] = layers[i](x) for Layer objects sharing the input width; one
    pair of launches for all of them at decode batch sizes."""
    import torch
    if x.dtype != torch.float16 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D float16 CUDA tensor")
    if outs is None:
        outs = [torch.empty((x.shape[0], L.n), dtype=torch.float16, device=x.device) for L in layers]
    if len(outs) != len(layers):
        raise ValueError("one output per layer")
    for L, y in zip(layers, outs):
        if (y.dtype != torch.float16 or not y.is_cuda or tuple(y.shape) != (x.shape[0], L.n) or not y.is_contiguous()
                or y.device != x.device):
            raise ValueError("outs[i] must be a contiguous float16 tensor of shape (batch, n_i) on x's device")
    stream = torch.cuda.current_stream(x.device).cuda_stream
    dbf_linear_forward_group([L.handle for L in layers], x.data_ptr(), [y.data_ptr() for y in outs], x.shape[0],
                             stream)
    return outs


def dbf_linear_backward_data(h: int, dy_ptr: int, dx_ptr: int, batch: int, stream: int = 0) -> None:
    _check(lib().dbf_linear_backward_data(h, dy_ptr, dx_ptr, batch, stream), "dbf_linear_backward_data")


def dbf_linear_backward(h: int, x_ptr: int, dy_ptr: int, dx_ptr: int, da_ptr: int, dmid_ptr: int, db_ptr: int,
                        batch: int, stream: int = 0) -> None:
    _check(lib().dbf_linear_backward(h, x_ptr, dy_ptr, dx_ptr, da_ptr, dmid_ptr, db_ptr, batch, stream),
           "dbf_linear_backward")


def dbf_free(h: Optional[int]) -> None:
    lib().dbf_free(h)


def dbf_get_info(h: int) -> Dict[str, int]:
    info = _Info()
    _check(lib().dbf_get_info(h, ctypes.byref(info)), "dbf_get_info")
    return {name: getattr(info, name) for name, _ in _Info._fields_}


def dbf_pack_signs(S, words_per_row: Optional[int] = None) -> np.ndarray:
    """Pack a +/-1 matrix along its columns (host only)."""
    S = _as_signs(S)
    if S.ndim != 2:
        raise ValueError("S must be 2-D")
    rows, cols = S.shape
    wpr = (cols + 31) // 32 if words_per_row is None else int(words_per_row)
    out = np.zeros((rows, max(wpr, 1)), dtype=np.uint32)
    _check(lib().dbf_pack_signs(_ptr(S), rows, cols, _ptr(out), wpr), "dbf_pack_signs")
    return out


def dbf_layout_words(rows: int, words: int) -> int:
    return int(lib().dbf_layout_words(rows, words))


def dbf_layout_signs(packed: np.ndarray) -> np.ndarray:
    """Device tiling of packed signs (host only)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    rows, words = packed.shape
    out = np.zeros(max(dbf_layout_words(rows, words), 1), dtype=np.uint32)
    _check(lib().dbf_layout_signs(_ptr(packed), rows, words, _ptr(out)), "dbf_layout_signs")
    return out


def dbf_layout_words_dec(rows_pad: int, cols_pad: int) -> int:
    return int(lib().dbf_layout_words_dec(rows_pad, cols_pad))


def dbf_layout_signs_dec(packed: np.ndarray, cols: int, rows_pad: int, cols_pad: int) -> np.ndarray:
    """The batch-1 decode kernels' copy of packed signs (host only)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    rows, words = packed.shape
    out = np.zeros(max(dbf_layout_words_dec(rows_pad, cols_pad), 1), dtype=np.uint32)
    _check(lib().dbf_layout_signs_dec(_ptr(packed), rows, cols, words, rows_pad, cols_pad, _ptr(out)),
           "dbf_layout_signs_dec")
    return out


def dbf_timing_enable(h: int, enable: bool = True) -> None:
    _check(lib().dbf_timing_enable(h, 1 if enable else 0), "dbf_timing_enable")


def dbf_timing_read(h: int) -> Dict[str, Dict[str, float]]:
    """Per kernel name: launches and summed event time (ms) since the last read."""
    cap = 32
    buf = (_KernelTime * cap)()
    cnt = ctypes.c_int32()
    _check(lib().dbf_timing_read(h, buf, cap, ctypes.byref(cnt)), "dbf_timing_read")
    return {buf[i].name.decode(): {"launches": int(buf[i].launches), "total_ms": float(buf[i].total_ms)}
            for i in range(min(cnt.value, cap))}


class Layer:
    """A DBF linear layer on the current GPU: ``y = layer(x)``.

    A (n x k) and B (k x m) are +/-1 arrays; a, mid, b are fp16 vectors.
    ``x`` is a contiguous fp16 CUDA (HIP) tensor of shape (batch, m) with
    batch <= max_batch; the result is a new fp16 tensor of shape (batch, n)
    computed on the current stream.
    """

    def __init__(self, A, B, a, mid, b, max_batch: int = 2048, backward: bool = False):
        A = np.asarray(A)
        B = np.asarray(B)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
            raise ValueError("A must be n x k and B k x m")
        self.n, self.k = A.shape
        self.m = B.shape[1]
        self.max_batch = int(max_batch)
        self.handle = dbf_pack(self.n, self.m, self.k, A, B, a, mid, b, self.max_batch,
                               DBF_PACK_BACKWARD if backward else 0)

    @classmethod
    def bqq(cls, Y, Z, r, s, t, u, max_batch: int = 2048) -> "Layer":
        """A layer with the BQQ-form weight sum_i (r_i Y_i Z_i + s_i Y_i 1 + t_i 1 Z_i) + u 1:
        Y (p, n, d) and Z (p, d, m) of 0/1; forward only."""
        Y = np.asarray(Y)
        Z = np.asarray(Z)
        if Y.ndim != 3 or Z.ndim != 3 or Y.shape[0] != Z.shape[0] or Y.shape[2] != Z.shape[1]:
            raise ValueError("Y must be (p, n, d) and Z (p, d, m)")
        self = cls.__new__(cls)
        p, self.n, d = Y.shape
        self.m = Z.shape[2]
        self.k = p * d
        self.max_batch = int(max_batch)
        self.handle = dbf_bqq_pack(self.n, self.m, d, p, Y, Z, r, s, t, u, self.max_batch)
        return self

    @classmethod
    def bqq_grouped(cls, Y, Z, r, s, t, u, group: int, max_batch: int = 2048) -> "Layer":
        """A BQQ-form layer whose scalars r, s, t (p, ngroups) and u (ngroups,) change from one
        group of `group` input columns to the next; forward only."""
        Y = np.asarray(Y)
        Z = np.asarray(Z)
        if Y.ndim != 3 or Z.ndim != 3 or Y.shape[0] != Z.shape[0] or Y.shape[2] != Z.shape[1]:
            raise ValueError("Y must be (p, n, d) and Z (p, d, m)")
        self = cls.__new__(cls)
        p, self.n, d = Y.shape
        self.m = Z.shape[2]
        self.k = p * d
        self.max_batch = int(max_batch)
        self.handle = dbf_bqq_pack_grouped(self.n, self.m, d, p, int(group), Y, Z, r, s, t, u, self.max_batch)
        return self

    def info(self) -> Dict[str, int]:
        return dbf_get_info(self.handle)

    def forward(self, x, out=None, path: int = DBF_PATH_AUTO):
        import torch
        if x.dtype != torch.float16 or not x.is_cuda or x.dim() != 2 or x.shape[1] != self.m:
            raise ValueError(f"x must be a CUDA float16 tensor of shape (batch, {self.m})")
        dev = getattr(self, "_device", None)
        if dev is None:
            dev = self._device = self.info()["device"]
        if x.device.index is not None and x.device.index != dev:
            raise ValueError("x must be on the layer's device")
        if not x.is_contiguous():
            raise ValueError("x must be contiguous")
        batch = x.shape[0]
        if out is None:
            out = torch.empty((batch, self.n), dtype=torch.float16, device=x.device)
        elif (out.shape != (batch, self.n) or out.dtype != torch.float16 or not out.is_contiguous()
              or not out.is_cuda or out.device != x.device):
            raise ValueError("out must be a contiguous float16 tensor of shape (batch, n) on x's device")
        stream = torch.cuda.current_stream(x.device).cuda_stream
        dbf_linear_forward_ex(self.handle, x.data_ptr(), out.data_ptr(), batch, path, stream)
        return out

    __call__ = forward

    @staticmethod
    def _check_act(t, width, what):
        import torch
        if t.dtype != torch.float16 or not t.is_cuda or t.dim() != 2 or t.shape[1] != width or not t.is_contiguous():
            raise ValueError(f"{what} must be a contiguous CUDA float16 tensor of shape (batch, {width})")

    def backward_data(self, dy, out=None):
        """dX = dY W for dY of shape (batch, n); needs backward=True."""
        import torch
        self._check_act(dy, self.n, "dy")
        if out is None:
            out = torch.empty((dy.shape[0], self.m), dtype=torch.float16, device=dy.device)
        self._check_act(out, self.m, "out")
        if out.shape[0] != dy.shape[0] or out.device != dy.device:
            raise ValueError("out must have dy's batch and device")
        stream = torch.cuda.current_stream(dy.device).cuda_stream
        dbf_linear_backward_data(self.handle, dy.data_ptr(), out.data_ptr(), dy.shape[0], stream)
        return out

    def backward(self, x, dy):
        """(dX fp16, da, dmid, db fp32) at input x for upstream gradient dy; needs backward=True."""
        import torch
        self._check_act(x, self.m, "x")
        self._check_act(dy, self.n, "dy")
        if x.shape[0] != dy.shape[0] or x.device != dy.device:
            raise ValueError("x and dy must have the same batch and device")
        dev = x.device
        dx = torch.empty((x.shape[0], self.m), dtype=torch.float16, device=dev)
        da = torch.empty(self.n, dtype=torch.float32, device=dev)
        dmid = torch.empty(self.k, dtype=torch.float32, device=dev)
        db = torch.empty(self.m, dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        dbf_linear_backward(self.handle, x.data_ptr(), dy.data_ptr(), dx.data_ptr(), da.data_ptr(), dmid.data_ptr(),
                            db.data_ptr(), x.shape[0], stream)
        return dx, da, dmid, db

    def close(self) -> None:
        if getattr(self, "handle", None):
            dbf_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
