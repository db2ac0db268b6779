"""ctypes binding of libpg (include/pg.h): argument marshalling only.

Every function takes device tensors (PyTorch-ROCm owns the memory and the
stream), checks dtypes/shapes/contiguity, passes raw pointers and the current
HIP stream to the C entry point of the same name, and raises ``PGError`` on a
non-zero status.  All arithmetic happens in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpg.so")

PG_OK, PG_EINVAL, PG_EUNSUPPORTED, PG_ELAUNCH, PG_EWORKSPACE, PG_ETIMEOUT = 0, -1, -2, -3, -4, -5

_lib = None


class PGError(RuntimeError):
    def __init__(self, name: str, code: int):
        super().__init__(f"{name} failed: {code} ({strerror(code)})")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded libpg.  Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libpg.so is not built ({LIB_PATH}); run `python -m prefill_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


_P = ctypes.c_void_p
_i32 = ctypes.c_int32
_f = ctypes.c_float
_sz = ctypes.c_size_t


class PgQ8(ctypes.Structure):
    """struct pg_q8 of pg.h."""
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


def _declare(L):
    L.pg_strerror.argtypes = [ctypes.c_int]
    L.pg_strerror.restype = ctypes.c_char_p
    L.pg_version.restype = ctypes.c_char_p
    L.gemv_q8.argtypes = [_P, _P, _P, _i32, _i32, _P, _P, _i32, _P]
    L.gemv_f16.argtypes = [_P, _i32, _i32, _P, _P, _i32, _P]
    L.prefill_gemm_q8.argtypes = [_P, _P, _P, _i32, _i32, _P, _i32, _P, _i32, _P, _sz, _P]
    L.decode_frame_q8_status.argtypes = [_P, _sz, _P]
    L.pg_stream_read.argtypes = [_P, _sz, _i32, _P, _P]
    L.prefill_gemm_q8_noalloc.argtypes = [_P, _P, _P, _i32, _i32, _P, _i32, _P, _i32, _P]
    L.prefill_gemm_q8_workspace_bytes.argtypes = [_i32, _i32, _i32]
    L.prefill_gemm_q8_workspace_bytes.restype = _sz
    L.add_rmsnorm.argtypes = [_P, _P, _i32, _P, _f, _i32, _i32, _P, _P]
    L.moe_grouped.argtypes = [_P, _i32, _i32, _P, _i32, _i32, _i32, _P, _P, _P, _i32, _P, _P, _P,
                              _P, _P, _f, _P, _P, _P, _P, _P, _P, _P, _sz, _P]
    L.moe_grouped_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
    L.moe_grouped_workspace_bytes.restype = _sz
    L.gemv_q8_addnorm.argtypes = [_P, _P, _P, _i32, _i32, _P, _P, _P, _f, _P, _P, _P, _i32, _P]
    L.prefill_gemm_q8_addnorm.argtypes = [_P, _P, _P, _i32, _i32, _P, _P, _i32, _P, _f, _i32, _P, _P, _P,
                                          _i32, _P, _sz, _P]
    L.gemv_q8_residual.argtypes = [_P, _P, _P, _i32, _i32, _P, _P, _i32, _P, _P, _i32, _P, _P, _P, _P]
    L.gemv_q8_normed.argtypes = [_P, _P, _P, _i32, _i32, _P, _P, _f, _P, _i32, _P]
    L.gemv_q8_norm_parts.argtypes = [_i32]
    L.gemv_q8_norm_parts.restype = _i32
    L.prefill_frame_q8_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
    L.prefill_frame_q8_workspace_bytes.restype = _sz
    L.prefill_frame_q8.argtypes = [ctypes.POINTER(PgQ8)] * 4 + [_P, _P, _f, _P, _P, _i32, _P, _P, _P, _P, _P, _sz, _P]
    L.prefill_frame_q8_meta.argtypes = [ctypes.POINTER(PgQ8)] * 4 + [_P, _P, _f, _P, _P, _i32, _P, _P, _P, _P, _P, _P,
                                                                     _sz, _P]
    L.decode_frame_q8_workspace_bytes.argtypes = [_i32, _i32]
    L.decode_frame_q8_workspace_bytes.restype = _sz
    L.decode_frame_q8_workspace_init.argtypes = [_P, _sz, _P]
    _q8p = ctypes.POINTER(PgQ8)
    L.decode_frame_q8.argtypes = [_q8p, _q8p, _q8p, _q8p, _P, _P, _f, _P, _P, _P, _P, _P, _P, _P, _sz, _P]
    L.gemv_q82.argtypes = [_P, _P, _P, _i32, _i32, _P, _P, _i32, _P]
    L.prefill_gemm_q82.argtypes = [_P, _P, _P, _i32, _i32, _P, _i32, _P, _i32, _P, _sz, _P]
    L.gemv_q4tp.argtypes = [_P, _P, _P, _i32, _i32, _P, _P, _i32, _P]
    L.prefill_gemm_q4tp.argtypes = [_P, _P, _P, _i32, _i32, _P, _i32, _P, _i32, _P, _sz, _P]
    L.argmax_rows.argtypes = [_P, _i32, _i32, _P, _P]
    L.expert_bank_q82.argtypes = [_P, _P, _P, _i32, _i32, _i32, _P, ctypes.c_int64, _i32, _P, _P, _i32, _P,
                                  ctypes.c_int64, _i32, _P]
    L.expert_bank_q4tp.argtypes = [_P, _P, _P, _i32, _i32, _i32, _P, ctypes.c_int64, _i32, _P, _P, _i32, _P,
                                   ctypes.c_int64, _i32, _P]
    L.attn_kv_append.argtypes = [_P, _P, _i32, _i32, _i32, _P, _P, _i32, _P]
    L.attn_prefill.argtypes = [_P, _P, _P, _i32, _i32, _i32, _i32, _i32, _f, _P, _P, _sz, _P]
    L.attn_prefill_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
    L.attn_prefill_workspace_bytes.restype = _sz
    L.moe_route_sigmoid.argtypes = [_P, _P, _i32, _i32, _i32, _i32, _f, _P, _P, _P]
    L.moe_grouped_sigmoid.argtypes = [_P, _i32, _i32, _P, _i32, _i32, _P, _i32, _f, _P, _P, _P, _i32, _P, _P, _P,
                                      _P, _P, _P, _f, _P, _P, _P, _P, _P, _P, _P, _sz, _P]
    for name in ("gemv_q8", "gemv_f16", "gemv_q82", "prefill_gemm_q82", "prefill_gemm_q4tp", "gemv_q4tp", "argmax_rows", "moe_route_sigmoid", "moe_grouped_sigmoid", "attn_kv_append", "attn_prefill", "expert_bank_q82", "expert_bank_q4tp", "prefill_gemm_q8", "prefill_gemm_q8_noalloc", "add_rmsnorm", "moe_grouped",
                 "gemv_q8_addnorm", "prefill_gemm_q8_addnorm", "gemv_q8_residual", "gemv_q8_normed",
                 "decode_frame_q8_workspace_init", "decode_frame_q8_status", "pg_stream_read", "decode_frame_q8", "prefill_frame_q8", "prefill_frame_q8_meta"):
        getattr(L, name).restype = ctypes.c_int


def strerror(code: int) -> str:
    return lib().pg_strerror(code).decode()


def version() -> str:
    return lib().pg_version().decode()


def _check(name: str, rc: int):
    if rc != PG_OK:
        raise PGError(name, rc)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


@dataclass
class Q8Weight:
    """A q8-block matrix on the device: q int8 [.., rows, cols], scale/bias f32 [.., rows, cols/32]."""

    q: torch.Tensor
    scale: torch.Tensor
    bias: torch.Tensor

    @property
    def rows(self) -> int:
        return self.q.shape[-2]

    @property
    def cols(self) -> int:
        return self.q.shape[-1]

    @staticmethod
    def from_host(q, scale, bias, device="cuda") -> "Q8Weight":
        return Q8Weight(torch.as_tensor(q).to(device), torch.as_tensor(scale).to(device),
                        torch.as_tensor(bias).to(device))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.q, self.scale, self.bias))

    def validate(self, name="W"):
        _dev(self.q, torch.int8, name + ".q")
        _dev(self.scale, torch.float32, name + ".scale")
        _dev(self.bias, torch.float32, name + ".bias")
        if self.scale.shape != self.q.shape[:-1] + (self.q.shape[-1] // 32,) or self.bias.shape != self.scale.shape:
            raise ValueError(f"{name}: scale/bias must be [.., rows, cols/32]")


@dataclass
class Q82Weight:
    """A q8_2f matrix on the device: q int8 [rows, cols], row scales rs float16 [rows],
    column field cf float16 [cols]."""

    q: torch.Tensor
    rs: torch.Tensor
    cf: torch.Tensor

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def cols(self) -> int:
        return self.q.shape[1]

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.q, self.rs, self.cf))

    def validate(self, name="W"):
        _dev(self.q, torch.int8, name + ".q")
        _dev(self.rs, torch.float16, name + ".rs")
        _dev(self.cf, torch.float16, name + ".cf")
        if self.q.dim() != 2 or self.rs.shape != (self.rows,) or self.cf.shape != (self.cols,):
            raise ValueError(f"{name}: q [rows, cols], rs [rows], cf [cols]")


def gemv_q82(W: Q82Weight, x: torch.Tensor, y: torch.Tensor | None = None, act: int = 0, stream=None):
    """y = act(rs * (q (cf * x))) for one position on a q8_2f matrix."""
    W.validate()
    _dev(x, torch.float32, "x")
    if x.numel() != W.cols:
        raise ValueError("x length must equal W.cols")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, "y")
    _check("gemv_q82", lib().gemv_q82(_ptr(W.q), _ptr(W.rs), _ptr(W.cf), W.rows, W.cols, _ptr(x), _ptr(y),
                                      act, _stream(stream)))
    return y


@dataclass
class Q4TPWeight:
    """A q4tp matrix on the device: nib uint8 [rows, cols/2], params int32 [rows] (binary16
    base low, step high; int32 holds the bits), codes uint8 [rows, ceil(5 cols/32 / 8)]."""

    nib: torch.Tensor
    params: torch.Tensor
    codes: torch.Tensor

    @property
    def rows(self) -> int:
        return self.nib.shape[0]

    @property
    def cols(self) -> int:
        return 2 * self.nib.shape[1]

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.nib, self.params, self.codes))

    def validate(self, name="W"):
        _dev(self.nib, torch.uint8, name + ".nib")
        _dev(self.params, torch.int32, name + ".params")
        _dev(self.codes, torch.uint8, name + ".codes")
        if (self.nib.dim() != 2 or self.params.shape != (self.rows,)
                or self.codes.shape != (self.rows, (5 * (self.cols // 32) + 7) // 8)):
            raise ValueError(f"{name}: nib [rows, cols/2], params [rows], codes [rows, ceil(5 cols/32 / 8)]")


def gemv_q4tp(W: Q4TPWeight, x: torch.Tensor, y: torch.Tensor | None = None, act: int = 0, stream=None):
    """y = act(W x) for one position on a q4tp matrix."""
    W.validate()
    _dev(x, torch.float32, "x")
    if x.numel() != W.cols:
        raise ValueError("x length must equal W.cols")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, "y")
    _check("gemv_q4tp", lib().gemv_q4tp(_ptr(W.nib), _ptr(W.params), _ptr(W.codes), W.rows, W.cols, _ptr(x),
                                        _ptr(y), act, _stream(stream)))
    return y


def argmax_rows(logits: torch.Tensor, ids: torch.Tensor | None = None, stream=None):
    """ids[b] = smallest index of row b's largest logit above -3.0e38 (0 if none); int32 out."""
    _dev(logits, torch.float32, "logits")
    L2 = logits.view(1, -1) if logits.dim() == 1 else logits
    if L2.dim() != 2:
        raise ValueError("logits must be [n][vocab] or [vocab]")
    n, vocab = L2.shape
    if ids is None:
        ids = torch.empty(n, dtype=torch.int32, device=logits.device)
    _dev(ids, torch.int32, "ids")
    _check("argmax_rows", lib().argmax_rows(_ptr(L2), n, vocab, _ptr(ids), _stream(stream)))
    return ids


def gemv_q8(W: Q8Weight, x: torch.Tensor, y: torch.Tensor | None = None, act: int = 0, stream=None):
    """y = act(W x) for one position; W is q8-block [rows][cols], x f32 [cols]."""
    W.validate()
    _dev(x, torch.float32, "x")
    if x.numel() != W.cols:
        raise ValueError("x length must equal W.cols")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, "y")
    _check("gemv_q8", lib().gemv_q8(_ptr(W.q), _ptr(W.scale), _ptr(W.bias), W.rows, W.cols,
                                    _ptr(x), _ptr(y), act, _stream(stream)))
    return y


def _rows_view(delta: torch.Tensor | None, cols: int, name: str):
    """Row stride of a device f32 tensor whose rows are contiguous (a view such as qkv[:, :hidden])."""
    if delta is None:
        return cols
    if delta.dtype != torch.float32 or not delta.is_cuda or delta.stride(-1) != 1:
        raise ValueError(f"{name} must be a device f32 tensor with contiguous rows")
    if delta.shape[-1] != cols:
        raise ValueError(f"{name} rows must have {cols} columns")
    return delta.stride(0) if delta.dim() > 1 else cols


def gemv_q8_addnorm(W: Q8Weight, h: torch.Tensor, delta: torch.Tensor | None, w: torch.Tensor, eps: float,
                    y: torch.Tensor | None = None, act: int = 0, h_out: torch.Tensor | None = None,
                    x_out: torch.Tensor | None = None, stream=None):
    """y = act(W . (rmsnorm(h + delta) * w)) at one position; h_out/x_out receive h + delta and the
    normed vector when given.  ``delta`` may be a view with contiguous data (e.g. qkv[:hidden])."""
    W.validate()
    _dev(h, torch.float32, "h")
    _dev(w, torch.float32, "w")
    if h.numel() != W.cols or w.numel() != W.cols:
        raise ValueError("h and w must have W.cols elements")
    if delta is not None:
        if delta.dtype != torch.float32 or not delta.is_cuda or not delta.is_contiguous():
            raise ValueError("delta must be a contiguous device f32 tensor")
        if delta.numel() != W.cols:
            raise ValueError("delta must have W.cols elements")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=h.device)
    _dev(y, torch.float32, "y")
    for t, nm in ((h_out, "h_out"), (x_out, "x_out")):
        if t is not None:
            _dev(t, torch.float32, nm)
            if t.numel() != W.cols:
                raise ValueError(f"{nm} must have W.cols elements")
    _check("gemv_q8_addnorm", lib().gemv_q8_addnorm(
        _ptr(W.q), _ptr(W.scale), _ptr(W.bias), W.rows, W.cols, _ptr(h), _ptr(delta), _ptr(w), eps,
        _ptr(h_out), _ptr(x_out), _ptr(y), act, _stream(stream)))
    return y


def norm_parts(hidden: int) -> int:
    """Length of the sum-of-squares parts gemv_q8_residual writes for ``hidden`` rows."""
    return lib().gemv_q8_norm_parts(hidden)


def gemv_q8_residual(W: Q8Weight, x: torch.Tensor, h: torch.Tensor, w: torch.Tensor, xw: torch.Tensor,
                     parts: torch.Tensor, y: torch.Tensor | None = None, act: int = 0,
                     h_out: torch.Tensor | None = None, stream=None):
    """y = act(W x); for the first len(h) rows h_out = h + y (h_out may be h), xw = w * h_out and
    parts = sums of h_out^2 over groups of 8 rows (the input of gemv_q8_normed)."""
    W.validate()
    for t, nm in ((x, "x"), (h, "h"), (w, "w"), (xw, "xw"), (parts, "parts")):
        _dev(t, torch.float32, nm)
    hidden = h.numel()
    if x.numel() != W.cols or w.numel() != hidden or xw.numel() != hidden or hidden > W.rows:
        raise ValueError("x must have W.cols elements; w and xw len(h) <= W.rows")
    if parts.numel() != norm_parts(hidden):
        raise ValueError(f"parts must have {norm_parts(hidden)} elements")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, "y")
    if h_out is not None:
        _dev(h_out, torch.float32, "h_out")
        if h_out.numel() != hidden:
            raise ValueError("h_out must have len(h) elements")
    _check("gemv_q8_residual", lib().gemv_q8_residual(
        _ptr(W.q), _ptr(W.scale), _ptr(W.bias), W.rows, W.cols, _ptr(x), _ptr(y), act, _ptr(h), _ptr(w), hidden,
        _ptr(h_out), _ptr(xw), _ptr(parts), _stream(stream)))
    return y


def gemv_q8_normed(W: Q8Weight, xw: torch.Tensor, parts: torch.Tensor, eps: float, y: torch.Tensor | None = None,
                   act: int = 0, stream=None):
    """y = act(W xw / sqrt(sum(parts) / W.cols + eps)): the product on the RMS-normed residual that
    gemv_q8_residual prepared."""
    W.validate()
    _dev(xw, torch.float32, "xw")
    _dev(parts, torch.float32, "parts")
    if xw.numel() != W.cols or parts.numel() != norm_parts(W.cols):
        raise ValueError("xw must have W.cols elements and parts norm_parts(W.cols)")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=xw.device)
    _dev(y, torch.float32, "y")
    _check("gemv_q8_normed", lib().gemv_q8_normed(
        _ptr(W.q), _ptr(W.scale), _ptr(W.bias), W.rows, W.cols, _ptr(xw), _ptr(parts), eps, _ptr(y), act,
        _stream(stream)))
    return y


def gemv_f16(W: torch.Tensor, x: torch.Tensor, y: torch.Tensor | None = None, act: int = 0, stream=None):
    """y = act(W x) with W float16 [rows][cols], x f32 [cols], f32 accumulation."""
    _dev(W, torch.float16, "W")
    _dev(x, torch.float32, "x")
    rows, cols = W.shape
    if y is None:
        y = torch.empty(rows, dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, "y")
    _check("gemv_f16", lib().gemv_f16(_ptr(W), rows, cols, _ptr(x), _ptr(y), act, _stream(stream)))
    return y


def prefill_gemm_q8_workspace_bytes(rows: int, cols: int, n: int) -> int:
    return lib().prefill_gemm_q8_workspace_bytes(rows, cols, n)


def prefill_gemm_q8_noalloc(W: Q8Weight, X: torch.Tensor, Y: torch.Tensor, act: int = 0, stream=None):
    """prefill_gemm_q8 with the library's fixed per-device scratch array instead of a
    workspace: Y [n][rows] (given, not allocated) = act(X [n][cols] . W^T).  Calls that
    overlap in time on one device share that array and race."""
    W.validate()
    _dev(X, torch.float32, "X")
    _dev(Y, torch.float32, "Y")
    n = X.shape[0]
    if X.dim() != 2 or X.shape[1] != W.cols or tuple(Y.shape) != (n, W.rows):
        raise ValueError("X must be [n][W.cols] and Y [n][W.rows]")
    _check("prefill_gemm_q8_noalloc", lib().prefill_gemm_q8_noalloc(
        _ptr(W.q), _ptr(W.scale), _ptr(W.bias), W.rows, W.cols, _ptr(X), n, _ptr(Y), act, _stream(stream)))
    return Y


def prefill_gemm_q8(W: Q8Weight, X: torch.Tensor, Y: torch.Tensor | None = None, act: int = 0,
                    workspace: torch.Tensor | None = None, stream=None):
    """Y [n][rows] = act(X [n][cols] . W^T) for one pass of n <= 64 positions."""
    W.validate()
    _dev(X, torch.float32, "X")
    n = X.shape[0]
    if X.dim() != 2 or X.shape[1] != W.cols:
        raise ValueError("X must be [n][W.cols]")
    if Y is None:
        Y = torch.empty(n, W.rows, dtype=torch.float32, device=X.device)
    _dev(Y, torch.float32, "Y")
    need = prefill_gemm_q8_workspace_bytes(W.rows, W.cols, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    _check("prefill_gemm_q8", lib().prefill_gemm_q8(
        _ptr(W.q), _ptr(W.scale), _ptr(W.bias), W.rows, W.cols, _ptr(X), n, _ptr(Y), act,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return Y


def prefill_gemm_q4tp(W: Q4TPWeight, X: torch.Tensor, Y: torch.Tensor | None = None, act: int = 0,
                      workspace: torch.Tensor | None = None, stream=None):
    """Y [n][rows] = act(X [n][cols] . W^T) for one pass of n <= 64 positions on a q4tp
    matrix (w = 2^(base + code step) (nib - 8)); the workspace is sized as for prefill_gemm_q8."""
    W.validate()
    _dev(X, torch.float32, "X")
    n = X.shape[0]
    if X.dim() != 2 or X.shape[1] != W.cols:
        raise ValueError("X must be [n][W.cols]")
    if Y is None:
        Y = torch.empty(n, W.rows, dtype=torch.float32, device=X.device)
    _dev(Y, torch.float32, "Y")
    need = prefill_gemm_q8_workspace_bytes(W.rows, W.cols, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    _check("prefill_gemm_q4tp", lib().prefill_gemm_q4tp(
        _ptr(W.nib), _ptr(W.params), _ptr(W.codes), W.rows, W.cols, _ptr(X), n, _ptr(Y), act,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return Y


def prefill_gemm_q82(W: Q82Weight, X: torch.Tensor, Y: torch.Tensor | None = None, act: int = 0,
                     workspace: torch.Tensor | None = None, stream=None):
    """Y [n][rows] = act(rs * ((cf * X) [n][cols] . q^T)) for one pass of n <= 64 positions
    on a q8_2f matrix; the workspace is sized as for prefill_gemm_q8."""
    W.validate()
    _dev(X, torch.float32, "X")
    n = X.shape[0]
    if X.dim() != 2 or X.shape[1] != W.cols:
        raise ValueError("X must be [n][W.cols]")
    if Y is None:
        Y = torch.empty(n, W.rows, dtype=torch.float32, device=X.device)
    _dev(Y, torch.float32, "Y")
    need = prefill_gemm_q8_workspace_bytes(W.rows, W.cols, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    _check("prefill_gemm_q82", lib().prefill_gemm_q82(
        _ptr(W.q), _ptr(W.rs), _ptr(W.cf), W.rows, W.cols, _ptr(X), n, _ptr(Y), act,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return Y


def prefill_gemm_q8_addnorm(W: Q8Weight, H: torch.Tensor, delta: torch.Tensor | None, w: torch.Tensor,
                            eps: float, Y: torch.Tensor | None = None, act: int = 0,
                            H_out: torch.Tensor | None = None, X_out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None):
    """Y [n][rows] = act((rmsnorm(H + delta) * w) . W^T) for one pass of n <= 64 positions;
    H_out (may be H itself) and X_out receive H + delta and the normed rows when given."""
    W.validate()
    _dev(H, torch.float32, "H")
    _dev(w, torch.float32, "w")
    if H.dim() != 2 or H.shape[1] != W.cols or w.numel() != W.cols:
        raise ValueError("H must be [n][W.cols] and w [W.cols]")
    n = H.shape[0]
    stride = _rows_view(delta, W.cols, "delta")
    if delta is not None and (delta.dim() != 2 or delta.shape[0] != n):
        raise ValueError("delta must be [n][W.cols] (rows may be strided)")
    if Y is None:
        Y = torch.empty(n, W.rows, dtype=torch.float32, device=H.device)
    _dev(Y, torch.float32, "Y")
    for t, nm in ((H_out, "H_out"), (X_out, "X_out")):
        if t is not None:
            _dev(t, torch.float32, nm)
            if t.shape != H.shape:
                raise ValueError(f"{nm} must be [n][W.cols]")
    need = prefill_gemm_q8_workspace_bytes(W.rows, W.cols, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=H.device)
    _check("prefill_gemm_q8_addnorm", lib().prefill_gemm_q8_addnorm(
        _ptr(W.q), _ptr(W.scale), _ptr(W.bias), W.rows, W.cols, _ptr(H), _ptr(delta), stride, _ptr(w), eps, n,
        _ptr(H_out), _ptr(X_out), _ptr(Y), act, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return Y


def add_rmsnorm(h: torch.Tensor, delta: torch.Tensor | None, w: torch.Tensor, eps: float,
                out: torch.Tensor | None = None, delta_stride: int | None = None, stream=None):
    """h += delta (in place, rows ``delta_stride`` apart); returns out = rmsnorm(h) * w.

    ``delta`` may be a strided view whose rows are contiguous (e.g. qkv[:, :hidden])."""
    _dev(h, torch.float32, "h")
    _dev(w, torch.float32, "w")
    h2 = h.view(-1, h.shape[-1])
    n, hidden = h2.shape
    stride = hidden
    if delta is not None:
        if delta.dtype != torch.float32 or not delta.is_cuda or delta.stride(-1) != 1:
            raise ValueError("delta must be a device f32 tensor with contiguous rows")
        stride = delta_stride if delta_stride is not None else (delta.stride(0) if delta.dim() > 1 else hidden)
    if out is None:
        out = torch.empty_like(h)
    _dev(out, torch.float32, "out")
    _check("add_rmsnorm", lib().add_rmsnorm(_ptr(h), _ptr(delta), stride, _ptr(w), eps, hidden, n,
                                            _ptr(out), _stream(stream)))
    return out


def moe_grouped_workspace_bytes(n: int, H: int, I: int, E: int, top_k: int) -> int:
    return lib().moe_grouped_workspace_bytes(n, H, I, E, top_k)


def moe_grouped(X: torch.Tensor, Wr: torch.Tensor, up: Q8Weight, down: Q8Weight, h: torch.Tensor,
                w_norm: torch.Tensor, eps: float, top_k: int, renorm: int = 0,
                workspace: torch.Tensor | None = None, outputs: dict | None = None, stream=None,
                router_bias: torch.Tensor | None = None, scale: float = 1.0,
                shared: torch.Tensor | None = None) -> dict:
    """One routed-MoE pass; updates ``h`` in place and returns the outputs
    {out, logits, sel, route_w, counts, lists} (pre-allocated ones may be passed in ``outputs``).
    With ``router_bias`` [E] the sigmoid + bias router routes (weights scaled by ``scale``,
    renormalised when ``renorm``) and ``shared`` [n][H] (optional) is added with the slots."""
    _dev(X, torch.float32, "X")
    _dev(Wr, torch.float32, "Wr")
    _dev(h, torch.float32, "h")
    _dev(w_norm, torch.float32, "w_norm")
    up.validate("up")
    down.validate("down")
    n, H = X.shape
    E = Wr.shape[0]
    I = up.q.shape[-2]
    if up.q.shape != (E, I, H) or down.q.shape != (E, H, I):
        raise ValueError("expert banks must be up [E][I][H], down [E][H][I]")
    dev = X.device
    o = dict(outputs or {})
    o.setdefault("out", torch.empty(n, H, dtype=torch.float32, device=dev))
    o.setdefault("logits", torch.empty(n, E, dtype=torch.float32, device=dev))
    o.setdefault("sel", torch.empty(n, top_k, dtype=torch.int32, device=dev))
    o.setdefault("route_w", torch.empty(n, top_k, dtype=torch.float32, device=dev))
    o.setdefault("counts", torch.empty(E, dtype=torch.int32, device=dev))
    o.setdefault("lists", torch.empty(E, n, dtype=torch.int32, device=dev))
    need = moe_grouped_workspace_bytes(n, H, I, E, top_k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if router_bias is None:
        if shared is not None:
            raise ValueError("shared needs the sigmoid router (router_bias)")
        _check("moe_grouped", lib().moe_grouped(
            _ptr(X), n, H, _ptr(Wr), E, top_k, renorm, _ptr(up.q), _ptr(up.scale), _ptr(up.bias), I,
            _ptr(down.q), _ptr(down.scale), _ptr(down.bias), _ptr(h), _ptr(w_norm), eps, _ptr(o["out"]),
            _ptr(o["logits"]), _ptr(o["sel"]), _ptr(o["route_w"]), _ptr(o["counts"]), _ptr(o["lists"]),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
        return o
    _dev(router_bias, torch.float32, "router_bias")
    if router_bias.shape != (E,):
        raise ValueError("router_bias must be [E]")
    if shared is not None:
        _dev(shared, torch.float32, "shared")
        if shared.shape != (n, H):
            raise ValueError("shared must be [n][H]")
    _check("moe_grouped_sigmoid", lib().moe_grouped_sigmoid(
        _ptr(X), n, H, _ptr(Wr), E, top_k, _ptr(router_bias), renorm, scale, _ptr(up.q), _ptr(up.scale),
        _ptr(up.bias), I, _ptr(down.q), _ptr(down.scale), _ptr(down.bias),
        None if shared is None else _ptr(shared), _ptr(h), _ptr(w_norm), eps, _ptr(o["out"]),
        _ptr(o["logits"]), _ptr(o["sel"]), _ptr(o["route_w"]), _ptr(o["counts"]), _ptr(o["lists"]),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


def expert_bank_q82(q: torch.Tensor, rs: torch.Tensor, cf: torch.Tensor, x: torch.Tensor, counts: torch.Tensor,
                    lists: torch.Tensor, src_div: int = 1, act: int = 0, out: torch.Tensor | None = None,
                    n_out: int | None = None, stream=None):
    """Grouped q8_2f expert product: q int8 [E][rows][cols], rs f16 [E][rows], cf f16 [E][cols],
    x f32 [*][cols], counts int32 [E], lists int32 [E][cap]; out f32 [n_out][rows] (rows of
    entries listed by an expert are written)."""
    _dev(q, torch.int8, "q")
    _dev(rs, torch.float16, "rs")
    _dev(cf, torch.float16, "cf")
    _dev(x, torch.float32, "x")
    _dev(counts, torch.int32, "counts")
    _dev(lists, torch.int32, "lists")
    E, rows, cols = q.shape
    if rs.shape != (E, rows) or cf.shape != (E, cols) or x.shape[-1] != cols or lists.shape[0] != E:
        raise ValueError("q [E][rows][cols], rs [E][rows], cf [E][cols], x [*][cols], lists [E][cap]")
    if out is None:
        out = torch.zeros(n_out if n_out is not None else lists.shape[1], rows, dtype=torch.float32, device=q.device)
    _dev(out, torch.float32, "out")
    _check("expert_bank_q82", lib().expert_bank_q82(_ptr(q), _ptr(rs), _ptr(cf), E, rows, cols, _ptr(x), cols,
                                                    src_div, _ptr(counts), _ptr(lists), lists.shape[1], _ptr(out),
                                                    rows, act, _stream(stream)))
    return out


def expert_bank_q4tp(nib: torch.Tensor, params: torch.Tensor, codes: torch.Tensor, x: torch.Tensor,
                     counts: torch.Tensor, lists: torch.Tensor, src_div: int = 1, act: int = 0,
                     out: torch.Tensor | None = None, n_out: int | None = None, stream=None):
    """Grouped q4tp expert product: nib uint8 [E][rows][cols/2], params int32 [E][rows] (binary16
    base low, step high), codes uint8 [E][rows][ceil(5 cols/32 / 8)], x f32 [*][cols], counts
    int32 [E], lists int32 [E][cap]; out f32 [n_out][rows] (rows of listed entries are written)."""
    _dev(nib, torch.uint8, "nib")
    _dev(params, torch.int32, "params")
    _dev(codes, torch.uint8, "codes")
    _dev(x, torch.float32, "x")
    _dev(counts, torch.int32, "counts")
    _dev(lists, torch.int32, "lists")
    E, rows, half = nib.shape
    cols = 2 * half
    if (params.shape != (E, rows) or codes.shape != (E, rows, (5 * (cols // 32) + 7) // 8) or x.shape[-1] != cols
            or lists.shape[0] != E):
        raise ValueError("nib [E][rows][cols/2], params [E][rows], codes [E][rows][ceil(5 cols/32 / 8)], "
                         "x [*][cols], lists [E][cap]")
    if out is None:
        out = torch.zeros(n_out if n_out is not None else lists.shape[1], rows, dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    _check("expert_bank_q4tp", lib().expert_bank_q4tp(_ptr(nib), _ptr(params), _ptr(codes), E, rows, cols, _ptr(x),
                                                      cols, src_div, _ptr(counts), _ptr(lists), lists.shape[1],
                                                      _ptr(out), rows, act, _stream(stream)))
    return out


def attn_kv_append(k: torch.Tensor, v: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, pos0: int, stream=None):
    """Write the pass's rows k, v [n][nkv][hd] into the caches [cap][nkv][hd] at pos0."""
    for t, nm in ((k, "k"), (v, "v"), (kc, "kc"), (vc, "vc")):
        _dev(t, torch.float32, nm)
    n = k.shape[0]
    width = k[0].numel()
    if v.shape != k.shape or kc.shape != vc.shape or kc[0].numel() != width:
        raise ValueError("k, v [n][...] and caches [cap][...] of the same row width")
    _check("attn_kv_append", lib().attn_kv_append(_ptr(k), _ptr(v), n, width, pos0, _ptr(kc), _ptr(vc),
                                                  kc.shape[0], _stream(stream)))


def attn_prefill(q: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, pos0: int, scale: float,
                 o: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Causal GQA over a pass: q [n][nh][hd], caches [>= pos0 + n][nkv][hd] -> o [n][nh][hd]."""
    for t, nm in ((q, "q"), (kc, "kc"), (vc, "vc")):
        _dev(t, torch.float32, nm)
    n, nh, hd = q.shape
    nkv = kc.shape[1]
    if kc.shape[2] != hd or vc.shape != kc.shape or kc.shape[0] < pos0 + n:
        raise ValueError("caches must be [>= pos0 + n][nkv][hd]")
    if o is None:
        o = torch.empty(n, nh, hd, dtype=torch.float32, device=q.device)
    _dev(o, torch.float32, "o")
    need = lib().attn_prefill_workspace_bytes(n, pos0, nh, nkv, hd)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _check("attn_prefill", lib().attn_prefill(_ptr(q), _ptr(kc), _ptr(vc), n, pos0, nh, nkv, hd, scale, _ptr(o),
                                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                                              _stream(stream)))
    return o


def moe_route_sigmoid(logits: torch.Tensor, router_bias: torch.Tensor, top_k: int, renorm: int = 1,
                      scale: float = 1.0, stream=None):
    """(sel int32 [n][k], route_w f32 [n][k]) of the sigmoid + bias router."""
    _dev(logits, torch.float32, "logits")
    _dev(router_bias, torch.float32, "router_bias")
    n, E = logits.shape
    sel = torch.empty(n, top_k, dtype=torch.int32, device=logits.device)
    rw = torch.empty(n, top_k, dtype=torch.float32, device=logits.device)
    _check("moe_route_sigmoid", lib().moe_route_sigmoid(_ptr(logits), _ptr(router_bias), n, E, top_k, renorm,
                                                        scale, _ptr(sel), _ptr(rw), _stream(stream)))
    return sel, rw


def decode_frame_q8_workspace_bytes(hidden: int, inter: int) -> int:
    return lib().decode_frame_q8_workspace_bytes(hidden, inter)


def decode_frame_q8_workspace(hidden: int, inter: int, device="cuda", stream=None) -> torch.Tensor:
    """A cleared workspace for decode_frame_q8 at these sizes (hidden, up rows)."""
    ws = torch.empty(decode_frame_q8_workspace_bytes(hidden, inter), dtype=torch.uint8, device=device)
    _check("decode_frame_q8_workspace_init",
           lib().decode_frame_q8_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))
    return ws


def decode_frame_timeouts(workspace: torch.Tensor) -> int:
    """Waits that gave up in launches on this workspace (the counter at byte 8)."""
    return int(workspace[8:12].view(torch.int32).item())


def stream_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of ``src`` once (the HBM read-ceiling measurement; see pg_stream_read)."""
    _check("pg_stream_read", lib().pg_stream_read(_ptr(src), src.numel() * src.element_size(), workgroups,
                                                  _ptr(sink), _stream(stream)))


def decode_frame_q8_status(workspace: torch.Tensor, stream=None) -> None:
    """Wait for the stream; raise PGError (PG_ETIMEOUT) if a barrier wait of a launch on
    this workspace gave up since its init (the outputs are then not trustworthy)."""
    _check("decode_frame_q8_status", lib().decode_frame_q8_status(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def _q8struct(W: Q8Weight, name: str) -> PgQ8:
    W.validate(name)
    return PgQ8(W.q.data_ptr(), W.scale.data_ptr(), W.bias.data_ptr(), W.rows, W.cols)


def decode_frame_q8(qkv: Q8Weight, up: Q8Weight, down: Q8Weight, head: Q8Weight, w1: torch.Tensor,
                    w2: torch.Tensor, eps: float, x0: torch.Tensor, h: torch.Tensor, out: dict,
                    workspace: torch.Tensor, stream=None) -> dict:
    """The q8 decode layer frame at one position in one launch: h is updated in place and
    out = {qkv, u, d, logits} (f32 device vectors) receives the four products."""
    Ws = [_q8struct(W, nm) for W, nm in ((qkv, "qkv"), (up, "up"), (down, "down"), (head, "head"))]
    for t, nm in ((w1, "w1"), (w2, "w2"), (x0, "x0"), (h, "h")):
        _dev(t, torch.float32, nm)
    H = qkv.cols
    for k, n in (("qkv", qkv.rows), ("u", up.rows), ("d", H), ("logits", head.rows)):
        _dev(out[k], torch.float32, k)
        if out[k].numel() != n:
            raise ValueError(f"out[{k!r}] must have {n} elements")
    if any(t.numel() != H for t in (w1, w2, x0, h)):
        raise ValueError("w1, w2, x0 and h must have qkv.cols elements")
    _dev(workspace, torch.uint8, "workspace")
    _check("decode_frame_q8", lib().decode_frame_q8(
        *[ctypes.byref(W) for W in Ws], _ptr(w1), _ptr(w2), eps, _ptr(x0), _ptr(h), _ptr(out["qkv"]),
        _ptr(out["u"]), _ptr(out["d"]), _ptr(out["logits"]), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def prefill_frame_q8_workspace_bytes(hidden: int, qkv_rows: int, inter: int, vocab: int, n: int) -> int:
    return lib().prefill_frame_q8_workspace_bytes(hidden, qkv_rows, inter, vocab, n)


def prefill_frame_q8(qkv: Q8Weight, up: Q8Weight, down: Q8Weight, head: Q8Weight, w1: torch.Tensor,
                     w2: torch.Tensor, eps: float, X0: torch.Tensor, H: torch.Tensor, out: dict,
                     workspace: torch.Tensor, stream=None) -> dict:
    """The q8 layer frame over one prefill pass of n <= 64 positions: H [n][hidden] is
    updated in place and out = {qkv, u, d, logits} ([n][...] f32) receives the products."""
    Ws = [_q8struct(W, nm) for W, nm in ((qkv, "qkv"), (up, "up"), (down, "down"), (head, "head"))]
    for t, nm in ((w1, "w1"), (w2, "w2"), (X0, "X0"), (H, "H")):
        _dev(t, torch.float32, nm)
    n, hidden = X0.shape
    if H.shape != X0.shape or hidden != qkv.cols or w1.numel() != hidden or w2.numel() != hidden:
        raise ValueError("X0 and H must be [n][qkv.cols]; w1, w2 [qkv.cols]")
    for k, cols in (("qkv", qkv.rows), ("u", up.rows), ("d", hidden), ("logits", head.rows)):
        _dev(out[k], torch.float32, k)
        if tuple(out[k].shape) != (n, cols):
            raise ValueError(f"out[{k!r}] must be [{n}][{cols}]")
    _dev(workspace, torch.uint8, "workspace")
    _check("prefill_frame_q8", lib().prefill_frame_q8(
        *[ctypes.byref(W) for W in Ws], _ptr(w1), _ptr(w2), eps, _ptr(X0), _ptr(H), n, _ptr(out["qkv"]),
        _ptr(out["u"]), _ptr(out["d"]), _ptr(out["logits"]), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def prefill_frame_q8_meta(qkv: Q8Weight, up: Q8Weight, down: Q8Weight, head: Q8Weight, w1: torch.Tensor,
                          w2: torch.Tensor, eps: float, X0: torch.Tensor, H: torch.Tensor, meta: torch.Tensor,
                          out: dict, workspace: torch.Tensor, stream=None) -> dict:
    """prefill_frame_q8 with the pass size on the device: meta = int32 tensor [n, pos0] on the
    GPU, read at launch; the pass works on rows pos0 .. pos0 + n - 1 of the prompt's buffers
    X0, H [rows][hidden] and out = {qkv, u, d, logits} ([rows][...])."""
    Ws = [_q8struct(W, nm) for W, nm in ((qkv, "qkv"), (up, "up"), (down, "down"), (head, "head"))]
    for t, nm in ((w1, "w1"), (w2, "w2"), (X0, "X0"), (H, "H")):
        _dev(t, torch.float32, nm)
    _dev(meta, torch.int32, "meta")
    if meta.numel() != 2:
        raise ValueError("meta must hold [n, pos0]")
    rows, hidden = X0.shape
    if H.shape != X0.shape or hidden != qkv.cols or w1.numel() != hidden or w2.numel() != hidden:
        raise ValueError("X0 and H must be [rows][qkv.cols]; w1, w2 [qkv.cols]")
    for k, cols in (("qkv", qkv.rows), ("u", up.rows), ("d", hidden), ("logits", head.rows)):
        _dev(out[k], torch.float32, k)
        if tuple(out[k].shape) != (rows, cols):
            raise ValueError(f"out[{k!r}] must be [{rows}][{cols}]")
    _dev(workspace, torch.uint8, "workspace")
    _check("prefill_frame_q8_meta", lib().prefill_frame_q8_meta(
        *[ctypes.byref(W) for W in Ws], _ptr(w1), _ptr(w2), eps, _ptr(X0), _ptr(H), rows, _ptr(meta),
        _ptr(out["qkv"]), _ptr(out["u"]), _ptr(out["d"]), _ptr(out["logits"]), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out
