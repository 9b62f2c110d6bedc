"""Python binding of the gfx950 fused GEMM-epilogue / back-to-back GEMM library.

Thin ctypes marshalling over the C ABI in ``include/cf.h`` (``libcf.so`` built
from ``csrc/`` by ``build_lib.py``). The functions keep the C names; they take
torch tensors only to read device pointers, strides and the current HIP
stream. Every computation runs in the library's kernels: there is no fallback.
Importing the package builds ``libcf.so`` first when it is missing or was
built from other sources (hipcc, gfx950), and fails loudly when it cannot.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from . import build_lib as _build_lib

LIB_PATH = _build_lib.LIB

try:
    _build_lib.ensure_built()
except Exception as exc:   # no hipcc, or a compile error: no library, no package
    raise ImportError(f"cannot build {LIB_PATH}: {exc}") from exc

_lib = ctypes.CDLL(LIB_PATH)

# ----------------------------------------------------------------------------- C types
CF_OK, CF_ERR_INVALID_ARGUMENT, CF_ERR_UNSUPPORTED, CF_ERR_WORKSPACE, CF_ERR_NO_DEVICE, \
    CF_ERR_HIP, CF_ERR_DEVICE_TIMEOUT = range(7)
CF_F32, CF_BF16 = 0, 1
ACT = {"none": 0, "relu": 1}
ROW_OP = {"none": 0, "softmax": 1, "layernorm": 2, "rmsnorm": 3, "argmax": 4, "topk": 5}
MASK = {"none": 0, "causal": 1}
AXIS = {"row": 0, "column": 1}


class cf_epilogue(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("alpha", ctypes.c_float),
        ("bias", ctypes.c_void_p),
        ("residual", ctypes.c_void_p),
        ("ld_residual", ctypes.c_int64),
        ("residual_dtype", ctypes.c_int),
        ("vec_dtype", ctypes.c_int),
        ("act", ctypes.c_int),
        ("row_op", ctypes.c_int),
        ("gamma", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("x_out", ctypes.c_void_p),
        ("ld_x_out", ctypes.c_int64),
        ("x_out_dtype", ctypes.c_int),
        ("mask", ctypes.c_int),
        ("row_stats", ctypes.c_void_p),
        ("row_index", ctypes.c_void_p),
        ("row_op2", ctypes.c_int),
        ("gamma2", ctypes.c_void_p),
        ("beta2", ctypes.c_void_p),
        ("eps2", ctypes.c_float),
        ("topk", ctypes.c_int32),
        ("axis", ctypes.c_int),
    ]


_i64, _vp, _int, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_EPI_P = ctypes.POINTER(cf_epilogue)

_lib.cf_epilogue_init.argtypes = [_EPI_P]
_lib.cf_epilogue_init.restype = None
_lib.cf_gemm_epilogue_workspace_size.argtypes = [_i64, _i64, _i64, _EPI_P]
_lib.cf_gemm_epilogue_workspace_size.restype = _sz
_lib.cf_workspace_init.argtypes = [_vp, _sz, _vp]
_lib.cf_workspace_init.restype = _int
_lib.cf_workspace_status.argtypes = [_vp, _vp]
_lib.cf_workspace_status.restype = _int
_lib.cf_gemm_epilogue.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _int, _vp, _i64, _int,
                                  _EPI_P, _vp, _sz, _vp]
_lib.cf_gemm_epilogue.restype = _int
_lib.cf_gemm_epilogue_noalloc.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _int, _vp, _i64, _int,
                                          _EPI_P, _vp]
_lib.cf_gemm_epilogue_noalloc.restype = _int
_lib.cf_b2bgemm.argtypes = [_i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _int,
                            _vp, _i64, _i64, _vp, _i64, _i64, _int, _int, _EPI_P, _vp]
_lib.cf_b2bgemm.restype = _int
_lib.cf_status_string.argtypes = [_int]
_lib.cf_status_string.restype = ctypes.c_char_p
_lib.cf_last_hip_error.argtypes = []
_lib.cf_last_hip_error.restype = _int
_lib.cf_version.argtypes = []
_lib.cf_version.restype = ctypes.c_char_p
_lib.cf_set_exchange_timeout_us.argtypes = [ctypes.c_uint64]
_lib.cf_set_exchange_timeout_us.restype = ctypes.c_uint64
_lib.cf_set_exchange_leader_tiles.argtypes = [_int]
_lib.cf_set_exchange_leader_tiles.restype = _int
_lib.cf_set_b2b_pingpong.argtypes = [_int]
_lib.cf_set_b2b_pingpong.restype = _int

EXPORTED = ["cf_epilogue_init", "cf_gemm_epilogue_workspace_size", "cf_workspace_init",
            "cf_workspace_status", "cf_gemm_epilogue", "cf_gemm_epilogue_noalloc", "cf_b2bgemm", "cf_status_string",
            "cf_last_hip_error", "cf_version", "cf_set_exchange_timeout_us", "cf_set_exchange_leader_tiles",
            "cf_set_b2b_pingpong"]


class CfError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.cf_status_string(status).decode()
        if status == CF_ERR_HIP:
            msg += f" (hipError {_lib.cf_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _check(status: int, where: str):
    if status != CF_OK:
        raise CfError(status, where)


# ----------------------------------------------------------------------------- helpers
_DTYPE_CODES = None


def _dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.float32: CF_F32, torch.bfloat16: CF_BF16}
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def _ld(t) -> int:
    """Leading dimension (row stride in elements) of a row-major 2-D (or batched) tensor."""
    st = t.stride()
    if len(st) < 2:
        raise ValueError("expected a matrix")
    if st[-1] != 1:
        raise ValueError("the last dimension must be contiguous")
    return st[-2]


_RAW_STREAM = None


def _stream(stream) -> Optional[int]:
    """The HIP stream handle: `stream` itself (a torch stream or a handle), or
    torch's current stream on the current device. The raw-handle query skips
    building a stream object on every launch."""
    global _RAW_STREAM
    if stream is not None:
        return getattr(stream, "cuda_stream", stream)
    import torch
    if _RAW_STREAM is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _RAW_STREAM = (lambda: raw(torch.cuda.current_device())) if raw is not None else \
            (lambda: torch.cuda.current_stream().cuda_stream)
    return _RAW_STREAM()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_epilogue(*, alpha: float = 1.0, bias=None, residual=None, act: str = "none",
                  row_op: str = "none", gamma=None, beta=None, eps: float = 0.0, x_out=None,
                  mask: str = "none", row_stats=None, row_index=None, row_op2: str = "none", gamma2=None,
                  beta2=None, eps2: float = 0.0, topk: int = 0, axis: str = "row") -> cf_epilogue:
    """cf_epilogue descriptor from tensors (bias/gamma/beta share one dtype).
    ``x_out``: optional [M, N] tensor that receives x before the row operation.
    ``mask``: "causal" for the softmax of cf_b2bgemm.
    ``row_stats``: optional contiguous fp32 tensor for the row operation's per-row
    statistics (log-sum-exp; LayerNorm mean and 1/sigma; RMSNorm 1/rms; the
    row maximum for argmax). ``row_index``: contiguous int32 [M] tensor that
    receives each row's argmax column (row_op "argmax"). ``row_op2`` (with
    ``gamma2``, ``beta2``, ``eps2``): a second row stage applied to the first
    one's output (cf_gemm_epilogue only). ``topk``: k (1..8) for row_op "topk",
    whose ``row_index`` (int32 [M, k]) and ``row_stats`` (fp32 [M, k]) receive
    each row's k largest columns and values. ``axis``: "column" makes the row
    operation (softmax, layernorm, rmsnorm) reduce over the rows of each
    column instead (row_stats then holds per-column statistics)."""
    e = cf_epilogue()
    _lib.cf_epilogue_init(ctypes.byref(e))
    e.axis = AXIS[axis]
    e.alpha = float(alpha)
    e.act = ACT[act]
    e.row_op = ROW_OP[row_op]
    e.eps = float(eps)
    e.mask = MASK[mask]
    e.row_op2 = ROW_OP[row_op2]
    e.topk = int(topk)
    e.eps2 = float(eps2)
    if row_stats is not None:
        import torch
        if row_stats.dtype != torch.float32 or not row_stats.is_contiguous():
            raise TypeError("row_stats must be a contiguous float32 tensor")
        e.row_stats = row_stats.data_ptr()
    if row_index is not None:
        import torch
        if row_index.dtype != torch.int32 or not row_index.is_contiguous():
            raise TypeError("row_index must be a contiguous int32 tensor")
        e.row_index = row_index.data_ptr()
    vecs = [v for v in (bias, gamma, beta, gamma2, beta2) if v is not None]
    if vecs:
        codes = {_dtype_code(v) for v in vecs}
        if len(codes) != 1:
            raise TypeError("bias, gamma, beta, gamma2 and beta2 must share one dtype")
        e.vec_dtype = codes.pop()
        for v in vecs:
            if not v.is_contiguous():
                raise ValueError("bias/gamma/beta must be contiguous")
    e.bias, e.gamma, e.beta = _ptr(bias), _ptr(gamma), _ptr(beta)
    e.gamma2, e.beta2 = _ptr(gamma2), _ptr(beta2)
    if residual is not None:
        e.residual = residual.data_ptr()
        e.ld_residual = _ld(residual)
        e.residual_dtype = _dtype_code(residual)
    if x_out is not None:
        e.x_out = x_out.data_ptr()
        e.ld_x_out = _ld(x_out)
        e.x_out_dtype = _dtype_code(x_out)
    return e


# ----------------------------------------------------------------------------- C entry points
def cf_version() -> str:
    return _lib.cf_version().decode()


def cf_status_string(status: int) -> str:
    return _lib.cf_status_string(status).decode()


def cf_set_exchange_timeout_us(us: int) -> int:
    return int(_lib.cf_set_exchange_timeout_us(int(us)))


def cf_set_exchange_leader_tiles(min_tiles: int) -> int:
    """Strips of at least ``min_tiles`` column tiles exchange leader-follower
    (0: never); returns the previous setting."""
    return int(_lib.cf_set_exchange_leader_tiles(int(min_tiles)))


def cf_set_b2b_pingpong(on: int) -> int:
    """Selects (1) or deselects (0) the ping-pong schedule of cf_b2bgemm's
    softmax; a negative value only reads it. Returns the previous value."""
    return int(_lib.cf_set_b2b_pingpong(int(on)))


def cf_gemm_epilogue_workspace_size(M: int, N: int, K: int, epi: Optional[cf_epilogue] = None) -> int:
    return int(_lib.cf_gemm_epilogue_workspace_size(M, N, K, ctypes.byref(epi) if epi else None))


def cf_workspace_init(ws, stream=None) -> None:
    _check(_lib.cf_workspace_init(ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
           "cf_workspace_init")


def cf_workspace_status(ws, stream=None) -> int:
    """CF_OK, or CF_ERR_DEVICE_TIMEOUT if a strip exchange timed out (synchronises the stream)."""
    return int(_lib.cf_workspace_status(ws.data_ptr(), _stream(stream)))


def cf_gemm_epilogue(A, B, C, *, b_is_nk: bool = False, epi: Optional[cf_epilogue] = None,
                     workspace=None, stream=None, **epi_kwargs) -> None:
    """C = epilogue(A . B) in one kernel. A [M, K]; B [K, N] (or [N, K] with
    b_is_nk); C [M, N] (or None with row_op "argmax"). The epilogue is ``epi`` or built from keyword
    arguments (alpha, bias, residual, act, row_op, gamma, beta, eps, x_out)."""
    if epi is None:
        epi = make_epilogue(**epi_kwargs)
    elif epi_kwargs:
        raise TypeError("pass either epi or epilogue keywords")
    M, K = A.shape
    N = B.shape[0] if b_is_nk else B.shape[1]
    if C is not None and C.shape != (M, N):
        raise ValueError(f"C must be [{M}, {N}]")
    ri = epi_kwargs.get("row_index")
    kk = int(epi_kwargs.get("topk", 0) or 1)
    if ri is not None and ri.numel() < M * kk:
        raise ValueError("row_index is too small for M rows")
    x_out = epi_kwargs.get("x_out")
    if x_out is not None and tuple(x_out.shape) != (M, N):
        raise ValueError(f"x_out must be [{M}, {N}]")
    st = epi_kwargs.get("row_stats")
    per = N if epi_kwargs.get("axis") == "column" else M
    if st is not None and st.numel() < per * (2 if epi_kwargs.get("row_op") == "layernorm" else kk):
        raise ValueError("row_stats is too small for the rows (columns) it covers")
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                           workspace.numel() * workspace.element_size())
    c_ptr, ldc, c_dt = (None, 0, CF_BF16) if C is None else (C.data_ptr(), _ld(C), _dtype_code(C))
    _check(_lib.cf_gemm_epilogue(M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), int(b_is_nk),
                                 _dtype_code(A), c_ptr, ldc, c_dt, ctypes.byref(epi),
                                 ws_ptr, ws_bytes, _stream(stream)), "cf_gemm_epilogue")


def cf_gemm_epilogue_noalloc(A, B, C, *, b_is_nk: bool = False, epi: Optional[cf_epilogue] = None,
                             stream=None) -> None:
    """cf_gemm_epilogue without a workspace argument: the library's static
    per-GPU scratch (16 MiB) serves the strip exchange, so nothing is
    allocated. Calls that overlap on one GPU race."""
    if epi is None:
        epi = make_epilogue()
    M, K = A.shape
    N = B.shape[0] if b_is_nk else B.shape[1]
    if C is not None and C.shape != (M, N):
        raise ValueError(f"C must be [{M}, {N}]")
    c_ptr, ldc, c_dt = (None, 0, CF_BF16) if C is None else (C.data_ptr(), _ld(C), _dtype_code(C))
    _check(_lib.cf_gemm_epilogue_noalloc(M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), int(b_is_nk),
                                         _dtype_code(A), c_ptr, ldc, c_dt, ctypes.byref(epi), _stream(stream)),
           "cf_gemm_epilogue_noalloc")


def cf_b2bgemm(A, B0, B1, O, *, b0_is_lk: bool = False, epi: Optional[cf_epilogue] = None,
               stream=None, **epi_kwargs) -> None:
    """O = F(alpha * A . B0 + bias) . B1 in one kernel per batch. A [batch, M, K]
    (or [M, K]); B0 [batch, K, L] or [batch, L, K] with b0_is_lk (a 2-D B0/B1 is
    shared by all batches); B1 [batch, L, N]; O [batch, M, N]."""
    if epi is None:
        epi = make_epilogue(**epi_kwargs)
    elif epi_kwargs:
        raise TypeError("pass either epi or epilogue keywords")

    def bstride(t):
        st = t.stride()
        return st[0] if len(st) == 3 else 0

    ash = A.shape
    batch = ash[0] if len(ash) == 3 else 1
    M, K = ash[-2], ash[-1]
    L = B0.shape[-2] if b0_is_lk else B0.shape[-1]
    N = B1.shape[-1]
    sa, sb0, sb1, so = bstride(A), bstride(B0), bstride(B1), bstride(O)
    st = epi_kwargs.get("row_stats")
    if st is not None and st.numel() < batch * M:
        raise ValueError("row_stats is too small for batch * M rows")
    _check(_lib.cf_b2bgemm(batch, M, K, L, N, A.data_ptr(), _ld(A), sa, B0.data_ptr(), _ld(B0), sb0,
                           int(b0_is_lk), B1.data_ptr(), _ld(B1), sb1, O.data_ptr(), _ld(O), so,
                           _dtype_code(A), _dtype_code(O), ctypes.byref(epi), _stream(stream)),
           "cf_b2bgemm")


class Workspace:
    """A cleared device workspace that grows on demand (device memory from torch)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, stream=None):
        import torch
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 4096), dtype=torch.uint8, device=self.device)
            cf_workspace_init(self.buf, stream)
        return self.buf
