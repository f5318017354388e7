"""Activation-sparse linear layers on AMD Instinct MI355X (gfx950).

Python binding of ``libsparse_act.so`` (ctypes).  It only marshals
arguments: every step runs in the library's HIP kernels, on the caller's
current torch stream.  torch supplies device memory and streams; the C ABI is
declared in ``include/sparse_act.h``, and each wrapper below has the name of
the C function it calls.

Layouts: weights are ``WT[d_in][d_out]`` fp16 (W column-major); activations
are fp16 ``[rows][d]``; bitmasks are int32 tensors holding the uint32 words
``[rows][ceil(d/32)]`` (bit ``j`` of word ``w`` is entry ``32*w + j``).

There is no CPU fallback: if the library is missing, or a tensor is not on a
GPU, these functions raise.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "SparseActError", "lib", "workspace",
    "act_sparsify_threshold", "act_sparsify_topk", "act_topk_cutoff", "sparse_gemv_topk",
    "act_sparsify_nm", "act_sparsify_nm_shared",
    "act_sparsify_scored", "sparse_gemv_corrected", "sparse_gemv_scored", "sparse_gemv_scored_nm",
    "act_calibrate_threshold", "sparse_gemv", "sparse_gemv_threshold",
    "sparse_gemv_threshold_noalloc", "rana_adapter_gemv",
    "masked_gemv",
    "dense_gemv", "masked_swiglu_down", "weight_col_norms", "nm_act_spmm", "nm_shared_spmm",
    "dense_gemm",
    "set_gemv_tuning", "set_gemm_tuning", "gemm_plan", "gemv_tiling_info", "workspace_bytes",
    "workspace_zero_bytes", "scratch", "MAX_BATCH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse_act.so")
MAX_BATCH = 8

_vp, _i64, _i32, _f32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_double, ctypes.c_size_t)

_SIGNATURES = {
    "sa_status_string": (ctypes.c_char_p, [_i32]),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_version": (_i32, []),
    "act_sparsify_threshold": (_i32, [_vp, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _i64, _vp]),
    "act_sparsify_topk": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp]),
    "act_topk_cutoff": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "sparse_gemv_topk": (_i32, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _sz, _vp]),
    "act_sparsify_nm": (_i32, [_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp]),
    "act_sparsify_nm_shared": (_i32, [_vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
    "act_calibrate_threshold": (_i32, [_vp, _i64, _f64, _vp, _vp]),
    "sa_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "sparse_gemv_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "sa_workspace_zero_bytes": (_sz, [_i64, _i64, _i64]),
    "sparse_gemv": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _sz, _vp]),
    "sparse_gemv_threshold": (_i32, [_vp, _i64, _i64, _vp, _i64, _f32, _vp, _vp, _sz, _vp]),
    "sparse_gemv_threshold_noalloc": (_i32, [_vp, _i64, _i64, _vp, _i64, _f32, _vp, _vp]),
    "act_sparsify_scored": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _f64, _vp, _vp, _vp,
                                   _vp, _i64, _vp, _vp]),
    "sparse_gemv_scored": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _f64, _i32, _vp, _vp, _vp, _sz,
                                  _vp]),
    "sparse_gemv_scored_nm": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                                     _vp, _sz, _vp]),
    "sparse_gemv_corrected": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp,
                                     _vp, _sz, _vp]),
    "rana_adapter_gemv": (_i32, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _f32, _vp, _vp, _vp,
                                 _sz, _vp]),
    "masked_gemv": (_i32, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "dense_gemv": (_i32, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "masked_swiglu_down": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _f64, _i32, _vp, _vp, _vp,
                                  _vp, _sz, _vp]),
    "weight_col_norms": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "nm_act_spmm": (_i32, [_vp, _vp, _i64, _i64, _i32, _i32, _vp, _i64, _vp, _vp, _sz, _vp]),
    "sa_nm_spmm_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "nm_shared_spmm": (_i32, [_vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _i64, _vp, _vp, _sz,
                              _vp]),
    "sa_nm_shared_spmm_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32, _i32]),
    "sa_read_stream": (_i32, [_vp, _sz, _vp, _vp]),
    "sa_read_stream_grid": (_i32, [_vp, _sz, _vp, _i32, _vp]),
    "dense_gemm": (_i32, [_vp, _i64, _i64, _vp, _i64, _vp, _vp]),
    "sa_set_gemv_tuning": (_i32, [_i32, _i32, _i32]),
    "sa_set_gemm_tuning": (_i32, [_i32, _i32, _i32]),
    "sa_gemv_tiling_info": (_i32, [_i32, _vp, _vp, _vp]),
    "sa_gemv_plan": (_i32, [_i32, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "sa_gemm_plan": (_i32, [_i32, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "sa_set_gemv_test_hooks": (_i32, [_i32]),
}

_lib = None
_lock = threading.Lock()


class SparseActError(RuntimeError):
    """A C entry point returned a non-zero status."""

    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {detail or 'error'} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library, with argument types declared."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(
                        f"{LIB_PATH} is not built; run `python -m sparse_input_gemv_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    f = getattr(L, name)
                    f.restype = res
                    f.argtypes = args
                _lib = L
    return _lib


def _check(status: int, fn: str) -> None:
    if status != 0:
        detail = lib().sa_last_error().decode(errors="replace")
        raise SparseActError(fn, status, detail)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a torch tensor on a GPU")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_ws: dict = {}       # device index -> the GEMV workspace in use
_scratch: dict = {}  # device index -> the matmuls' scratch in use
# Superseded buffers stay allocated until the process ends: a HIP graph
# captured before a buffer grew still holds the old buffer's address, and
# its replays must find memory that is theirs (and, for a GEMV workspace,
# still zero where the library keeps it zero).
_retired: list = []


def workspace_bytes(d_out: int, d_in: int, batch: int = 1) -> int:
    return int(lib().sparse_gemv_workspace_bytes(d_out, d_in, batch))


def workspace_zero_bytes(d_out: int, d_in: int, batch: int = 1) -> int:
    return int(lib().sa_workspace_zero_bytes(d_out, d_in, batch))


def _grow(table: dict, device, nbytes: int, zero: bool, what: str) -> torch.Tensor:
    key = torch.device(device).index or 0
    buf = table.get(key)
    if buf is None or buf.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(
                f"the {what} must grow to {nbytes} bytes while a HIP graph is being captured; "
                "make one eager call of the largest shape before capturing")
        size = max(nbytes, 1 << 20, 0 if buf is None else 2 * buf.numel())
        new = (torch.zeros if zero else torch.empty)(size, dtype=torch.uint8, device=device)
        if buf is not None:
            _retired.append(buf)
        table[key] = buf = new
    return buf


def workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """Per-device GEMV workspace, grown on demand (at least doubling) and reused.

    Allocated zero-filled: its leading region (hand-off counters and slots)
    must start at zero, and the library returns it to zero after every call.
    Only the GEMV family uses it.  Calls on one device share it, so they must
    be ordered on one stream.  Growth is refused during graph capture.
    """
    return _grow(_ws, device, nbytes, True, "GEMV workspace")


def scratch(device: torch.device, nbytes: int) -> torch.Tensor:
    """Per-device scratch of the matmuls (contents undefined), grown on
    demand; separate from the GEMV workspace, whose zero region it must not
    touch."""
    return _grow(_scratch, device, nbytes, False, "matmul scratch")


def _rows(x: torch.Tensor):
    return (1, x.shape[0]) if x.dim() == 1 else (x.shape[0], x.shape[1])


# ---- sparsifiers ------------------------------------------------------------

def act_sparsify_threshold(x: torch.Tensor, t: float, with_mask: bool = True, cap: int | None = None):
    """Returns ``(mask, idx, val, nnz)``; see the C declaration."""
    _dev(x, "x", torch.float16)
    rows, d = _rows(x)
    cap = d if cap is None else cap
    dev = x.device
    shape = (rows,) if x.dim() == 2 else ()
    mask = torch.empty(shape + ((d + 31) // 32,), dtype=torch.int32, device=dev) if with_mask else None
    idx = torch.empty(shape + (cap,), dtype=torch.int32, device=dev)
    val = torch.empty(shape + (cap,), dtype=torch.float16, device=dev)
    nnz = torch.empty((rows,), dtype=torch.int32, device=dev)
    _check(lib().act_sparsify_threshold(_ptr(x), rows, d, float(t), _ptr(mask), _ptr(idx), _ptr(val),
                                        _ptr(nnz), cap, _stream(x)), "act_sparsify_threshold")
    return mask, idx, val, nnz


def act_sparsify_scored(x: torch.Tensor, t: float = 0.0, n: int = 0, m: int = 0,
                        mu: torch.Tensor | None = None, colnorm: torch.Tensor | None = None,
                        with_mask: bool = True):
    """Weight-aware selection of the shifted activation ``x - mu``: a
    threshold on ``|x'| * colnorm`` (``m == 0``) or ``n`` of every ``m``.
    Returns ``(mask, idx, val, nnz, alpha)``; see the C declaration."""
    _dev(x, "x", torch.float16)
    rows, d = _rows(x)
    if mu is not None:
        _dev(mu, "mu", torch.float16)
        if mu.numel() != d:
            raise ValueError(f"mu holds {mu.numel()} values, {d} needed")
    if colnorm is not None:
        _dev(colnorm, "colnorm", torch.float64)
        if colnorm.numel() != d:
            raise ValueError(f"colnorm holds {colnorm.numel()} values, {d} needed")
    cap = d if m == 0 else d // m * n
    dev = x.device
    shape = (rows,) if x.dim() == 2 else ()
    mask = torch.empty(shape + ((d + 31) // 32,), dtype=torch.int32, device=dev) if with_mask else None
    idx = torch.empty(shape + (max(cap, 1),), dtype=torch.int32, device=dev)
    val = torch.empty(shape + (max(cap, 1),), dtype=torch.float16, device=dev)
    nnz = torch.empty((rows,), dtype=torch.int32, device=dev)
    alpha = torch.empty((rows,), dtype=torch.float32, device=dev)
    _check(lib().act_sparsify_scored(_ptr(x), rows, d, _ptr(mu), _ptr(colnorm), int(n), int(m),
                                     float(t), _ptr(mask), _ptr(idx), _ptr(val), _ptr(nnz),
                                     max(cap, 1), _ptr(alpha), _stream(x)), "act_sparsify_scored")
    return mask, idx, val, nnz, alpha


def act_sparsify_topk(x: torch.Tensor, k: int, with_mask: bool = True, cap: int | None = None):
    """Returns ``(mask, idx, val, nnz)`` with exactly ``k`` kept per row."""
    _dev(x, "x", torch.float16)
    rows, d = _rows(x)
    cap = max(k, 1) if cap is None else cap
    dev = x.device
    shape = (rows,) if x.dim() == 2 else ()
    mask = torch.empty(shape + ((d + 31) // 32,), dtype=torch.int32, device=dev) if with_mask else None
    idx = torch.empty(shape + (cap,), dtype=torch.int32, device=dev)
    val = torch.empty(shape + (cap,), dtype=torch.float16, device=dev)
    nnz = torch.empty((rows,), dtype=torch.int32, device=dev)
    _check(lib().act_sparsify_topk(_ptr(x), rows, d, int(k), _ptr(mask), _ptr(idx), _ptr(val),
                                   _ptr(nnz), cap, _stream(x)), "act_sparsify_topk")
    return mask, idx, val, nnz


def act_topk_cutoff(x: torch.Tensor, k: int) -> torch.Tensor:
    """Per row the Top-K cutoff ``(tau, i*)`` as an int32 ``[rows][2]`` tensor."""
    _dev(x, "x", torch.float16)
    rows, d = _rows(x)
    cut = torch.empty((rows, 2), dtype=torch.int32, device=x.device)
    _check(lib().act_topk_cutoff(_ptr(x), rows, d, int(k), _ptr(cut), _stream(x)),
           "act_topk_cutoff")
    return cut


def act_sparsify_nm(x: torch.Tensor, n: int, m: int):
    """Returns ``(mask, val)``: bitmask words and the compressed kept values."""
    _dev(x, "x", torch.float16)
    rows, d = _rows(x)
    shape = (rows,) if x.dim() == 2 else ()
    mask = torch.empty(shape + (d // 32,), dtype=torch.int32, device=x.device)
    val = torch.empty(shape + (d * n // m,), dtype=torch.float16, device=x.device)
    _check(lib().act_sparsify_nm(_ptr(x), rows, d, n, m, _ptr(mask), _ptr(val), _stream(x)),
           "act_sparsify_nm")
    return mask, val


def act_sparsify_nm_shared(x: torch.Tensor, n: int, m: int, tt: int = 32):
    """Returns ``(mask, val)``: one mask row per tile of ``tt`` rows and each
    row's values at its tile's kept positions."""
    _dev(x, "x", torch.float16)
    if x.dim() != 2:
        raise ValueError("x must be [rows][d]")
    rows, d = x.shape
    mask = torch.empty(((rows + tt - 1) // tt, d // 32), dtype=torch.int32, device=x.device)
    val = torch.empty((rows, d * n // m), dtype=torch.float16, device=x.device)
    _check(lib().act_sparsify_nm_shared(_ptr(x), rows, d, n, m, tt, _ptr(mask), _ptr(val),
                                        _stream(x)), "act_sparsify_nm_shared")
    return mask, val


def act_calibrate_threshold(samples: torch.Tensor, s: float) -> torch.Tensor:
    """Threshold (fp32, one-element device tensor) for sparsity ``s``."""
    _dev(samples, "samples", torch.float16)
    out = torch.empty((1,), dtype=torch.float32, device=samples.device)
    _check(lib().act_calibrate_threshold(_ptr(samples), samples.numel(), float(s), _ptr(out),
                                         _stream(samples)), "act_calibrate_threshold")
    return out


# ---- GEMV family ------------------------------------------------------------

def _gemv_out(wt, batch, squeeze, y):
    d_out = wt.shape[1]
    if y is None:
        y = torch.empty((batch, d_out), dtype=torch.float16, device=wt.device)
    else:
        _dev(y, "y", torch.float16)
        if y.numel() < batch * d_out:
            raise ValueError(f"y holds {y.numel()} values, {batch * d_out} needed")
    return y


def _ret(y, squeeze):
    return y[0] if squeeze and y.dim() == 2 else y


def sparse_gemv(wt: torch.Tensor, idx: torch.Tensor, val: torch.Tensor, nnz: torch.Tensor,
                y: torch.Tensor | None = None):
    """``y[b] = W[:, idx[b, :nnz[b]]] @ val[b, :nnz[b]]`` (lists from a sparsifier)."""
    _dev(wt, "wt", torch.float16)
    _dev(idx, "idx", torch.int32)
    _dev(val, "val", torch.float16)
    _dev(nnz, "nnz", torch.int32)
    squeeze = idx.dim() == 1
    batch, cap = _rows(idx)
    d_in, d_out = wt.shape
    y = _gemv_out(wt, batch, squeeze, y)
    nb = workspace_bytes(d_out, d_in, batch)
    ws = workspace(wt.device, nb)
    _check(lib().sparse_gemv(_ptr(wt), d_out, d_in, _ptr(idx), _ptr(val), _ptr(nnz), batch, cap,
                             _ptr(y), _ptr(ws), ws.numel(), _stream(wt)), "sparse_gemv")
    return _ret(y, squeeze)


def sparse_gemv_threshold(wt: torch.Tensor, x: torch.Tensor, t: float,
                          y: torch.Tensor | None = None):
    """Threshold and sparse GEMV in one launch: ``y = W (keep ⊙ x)``."""
    _dev(wt, "wt", torch.float16)
    _dev(x, "x", torch.float16)
    squeeze = x.dim() == 1
    batch, d_in = _rows(x)
    d_out = wt.shape[1]
    y = _gemv_out(wt, batch, squeeze, y)
    ws = workspace(wt.device, workspace_bytes(d_out, d_in, batch))
    _check(lib().sparse_gemv_threshold(_ptr(wt), d_out, d_in, _ptr(x), batch, float(t), _ptr(y),
                                       _ptr(ws), ws.numel(), _stream(wt)), "sparse_gemv_threshold")
    return _ret(y, squeeze)


def sparse_gemv_topk(wt: torch.Tensor, x: torch.Tensor, k: int, y: torch.Tensor | None = None):
    """Per-token Top-K of ``x`` (``k`` kept per row) and the sparse GEMV, no lists."""
    _dev(wt, "wt", torch.float16)
    _dev(x, "x", torch.float16)
    squeeze = x.dim() == 1
    batch, d_in = _rows(x)
    d_out = wt.shape[1]
    y = _gemv_out(wt, batch, squeeze, y)
    ws = workspace(wt.device, workspace_bytes(d_out, d_in, batch))
    _check(lib().sparse_gemv_topk(_ptr(wt), d_out, d_in, _ptr(x), batch, int(k), _ptr(y),
                                  _ptr(ws), ws.numel(), _stream(wt)), "sparse_gemv_topk")
    return _ret(y, squeeze)


def sparse_gemv_threshold_noalloc(wt: torch.Tensor, x: torch.Tensor, t: float,
                                  y: torch.Tensor):
    """``sparse_gemv_threshold`` on the library's fixed per-GPU scratch: the
    call allocates nothing (``y`` is the caller's).  Calls on one GPU share
    that scratch and must be ordered on one stream."""
    _dev(wt, "wt", torch.float16)
    _dev(x, "x", torch.float16)
    squeeze = x.dim() == 1
    batch, d_in = _rows(x)
    d_out = wt.shape[1]
    _gemv_out(wt, batch, squeeze, y)
    _check(lib().sparse_gemv_threshold_noalloc(_ptr(wt), d_out, d_in, _ptr(x), batch, float(t),
                                               _ptr(y), _stream(wt)),
           "sparse_gemv_threshold_noalloc")
    return y


def sparse_gemv_corrected(wt: torch.Tensor, idx: torch.Tensor, val: torch.Tensor,
                          nnz: torch.Tensor, alpha: torch.Tensor | None = None,
                          bias: torch.Tensor | None = None, y: torch.Tensor | None = None):
    """``y[b] = alpha[b] * W[:, idx[b]] @ val[b] + bias`` (either may be None)."""
    _dev(wt, "wt", torch.float16)
    _dev(idx, "idx", torch.int32)
    _dev(val, "val", torch.float16)
    _dev(nnz, "nnz", torch.int32)
    squeeze = idx.dim() == 1
    batch, cap = _rows(idx)
    d_in, d_out = wt.shape
    if alpha is not None:
        _dev(alpha, "alpha", torch.float32)
        if alpha.numel() < batch:
            raise ValueError(f"alpha holds {alpha.numel()} values, {batch} needed")
    if bias is not None:
        _dev(bias, "bias", torch.float16)
        if bias.numel() != d_out:
            raise ValueError(f"bias holds {bias.numel()} values, {d_out} needed")
    y = _gemv_out(wt, batch, squeeze, y)
    ws = workspace(wt.device, workspace_bytes(d_out, d_in, batch))
    _check(lib().sparse_gemv_corrected(_ptr(wt), d_out, d_in, _ptr(idx), _ptr(val), _ptr(nnz),
                                       batch, cap, _ptr(alpha), _ptr(bias), _ptr(y), _ptr(ws),
                                       ws.numel(), _stream(wt)), "sparse_gemv_corrected")
    return _ret(y, squeeze)


def sparse_gemv_scored(wt: torch.Tensor, x: torch.Tensor, t: float,
                       mu: torch.Tensor | None = None, colnorm: torch.Tensor | None = None,
                       var: bool = True, bias: torch.Tensor | None = None,
                       y: torch.Tensor | None = None):
    """One launch: shift, weight-aware threshold, sparse GEMV, variance
    correction and bias, for one row ``x``."""
    _dev(wt, "wt", torch.float16)
    _dev(x, "x", torch.float16)
    d_in, d_out = wt.shape
    if x.numel() != d_in:
        raise ValueError(f"x holds {x.numel()} values, {d_in} needed")
    for name, tt, dt, n in (("mu", mu, torch.float16, d_in), ("colnorm", colnorm, torch.float64, d_in),
                            ("bias", bias, torch.float16, d_out)):
        if tt is not None:
            _dev(tt, name, dt)
            if tt.numel() != n:
                raise ValueError(f"{name} holds {tt.numel()} values, {n} needed")
    y = _gemv_out(wt, 1, True, y)
    ws = workspace(wt.device, workspace_bytes(d_out, d_in, 1))
    _check(lib().sparse_gemv_scored(_ptr(wt), d_out, d_in, _ptr(x), _ptr(mu), _ptr(colnorm),
                                    float(t), int(bool(var)), _ptr(bias), _ptr(y), _ptr(ws),
                                    ws.numel(), _stream(wt)), "sparse_gemv_scored")
    return _ret(y, True)


def sparse_gemv_scored_nm(wt: torch.Tensor, x: torch.Tensor, n: int, m: int,
                          mu: torch.Tensor | None = None, colnorm: torch.Tensor | None = None,
                          var: bool = True, bias: torch.Tensor | None = None,
                          y: torch.Tensor | None = None):
    """One launch: shift, n of every m entries kept by weight-aware score,
    sparse GEMV, variance correction and bias, for one row ``x``."""
    _dev(wt, "wt", torch.float16)
    _dev(x, "x", torch.float16)
    d_in, d_out = wt.shape
    if x.numel() != d_in:
        raise ValueError(f"x holds {x.numel()} values, {d_in} needed")
    for name, tt, dt, cnt in (("mu", mu, torch.float16, d_in),
                              ("colnorm", colnorm, torch.float64, d_in),
                              ("bias", bias, torch.float16, d_out)):
        if tt is not None:
            _dev(tt, name, dt)
            if tt.numel() != cnt:
                raise ValueError(f"{name} holds {tt.numel()} values, {cnt} needed")
    y = _gemv_out(wt, 1, True, y)
    ws = workspace(wt.device, workspace_bytes(d_out, d_in, 1))
    _check(lib().sparse_gemv_scored_nm(_ptr(wt), d_out, d_in, _ptr(x), _ptr(mu), _ptr(colnorm),
                                       int(n), int(m), int(bool(var)), _ptr(bias), _ptr(y),
                                       _ptr(ws), ws.numel(), _stream(wt)), "sparse_gemv_scored_nm")
    return _ret(y, True)


def rana_adapter_gemv(b: torch.Tensor, at: torch.Tensor, x: torch.Tensor, t: float,
                      v: torch.Tensor | None = None, y: torch.Tensor | None = None):
    """RaNA linear-layer rank adapter: ``v = B x``, ``y = A (m ⊙ v)`` with
    ``m_i = v_i**2 >= t``; ``b`` is ``B [r][d_in]`` (row-major), ``at`` is
    ``A^T [r][d_out]``.  Returns ``(v, y)``."""
    _dev(b, "b", torch.float16)
    _dev(at, "at", torch.float16)
    _dev(x, "x", torch.float16)
    squeeze = x.dim() == 1
    batch, d_in = _rows(x)
    r, d_out = b.shape[0], at.shape[1]
    if b.shape[1] != d_in or at.shape[0] != r:
        raise ValueError(f"shapes: b {tuple(b.shape)}, at {tuple(at.shape)}, x rows of {d_in}")
    if v is None:
        v = torch.empty((batch, r), dtype=torch.float16, device=b.device)
    else:
        _dev(v, "v", torch.float16)
        if v.numel() < batch * r:
            raise ValueError(f"v holds {v.numel()} values, {batch * r} needed")
    y = _gemv_out(at, batch, squeeze, y)
    ws = workspace(b.device, workspace_bytes(d_out, r, batch))
    _check(lib().rana_adapter_gemv(_ptr(b), r, d_in, _ptr(at), d_out, _ptr(x), batch, float(t),
                                   _ptr(v), _ptr(y), _ptr(ws), ws.numel(), _stream(b)),
           "rana_adapter_gemv")
    return _ret(v, squeeze), _ret(y, squeeze)


def masked_gemv(wt: torch.Tensor, x: torch.Tensor, mask: torch.Tensor,
                y: torch.Tensor | None = None):
    """``y[b] = W (mask_b ⊙ x_b)`` for bitmask words ``mask``."""
    _dev(wt, "wt", torch.float16)
    _dev(x, "x", torch.float16)
    _dev(mask, "mask", torch.int32)
    squeeze = x.dim() == 1
    batch, d_in = _rows(x)
    d_out = wt.shape[1]
    y = _gemv_out(wt, batch, squeeze, y)
    ws = workspace(wt.device, workspace_bytes(d_out, d_in, batch))
    _check(lib().masked_gemv(_ptr(wt), d_out, d_in, _ptr(x), _ptr(mask), batch, _ptr(y), _ptr(ws),
                             ws.numel(), _stream(wt)), "masked_gemv")
    return _ret(y, squeeze)


def dense_gemv(wt: torch.Tensor, x: torch.Tensor, y: torch.Tensor | None = None):
    """Dense baseline ``y = W x`` on the same kernel skeleton."""
    _dev(wt, "wt", torch.float16)
    _dev(x, "x", torch.float16)
    squeeze = x.dim() == 1
    batch, d_in = _rows(x)
    d_out = wt.shape[1]
    y = _gemv_out(wt, batch, squeeze, y)
    ws = workspace(wt.device, workspace_bytes(d_out, d_in, batch))
    _check(lib().dense_gemv(_ptr(wt), d_out, d_in, _ptr(x), batch, _ptr(y), _ptr(ws), ws.numel(),
                            _stream(wt)), "dense_gemv")
    return _ret(y, squeeze)


def masked_swiglu_down(g: torch.Tensor, u: torch.Tensor, wdt: torch.Tensor, t: float, mode: str,
                       colnorm: torch.Tensor | None = None, y: torch.Tensor | None = None,
                       with_mask: bool = True):
    """CATS (``mode='cats'``) or RaNA (``mode='rana'``) masked down projection.

    Returns ``(y, mask, nnz)``; ``mask``/``nnz`` are None when not requested.
    """
    _dev(g, "g", torch.float16)
    _dev(u, "u", torch.float16)
    _dev(wdt, "wdt", torch.float16)
    m = {"cats": 0, "rana": 1}[mode]
    if colnorm is not None:
        _dev(colnorm, "colnorm", torch.float64)
    d_ff, d_model = wdt.shape
    if y is None:
        y = torch.empty((d_model,), dtype=torch.float16, device=wdt.device)
    mask = torch.empty(((d_ff + 31) // 32,), dtype=torch.int32, device=wdt.device) if with_mask else None
    nnz = torch.empty((1,), dtype=torch.int32, device=wdt.device) if with_mask else None
    ws = workspace(wdt.device, workspace_bytes(d_model, d_ff, 1))
    _check(lib().masked_swiglu_down(_ptr(g), _ptr(u), _ptr(wdt), _ptr(colnorm), d_ff, d_model,
                                    float(t), m, _ptr(y), _ptr(mask), _ptr(nnz), _ptr(ws),
                                    ws.numel(), _stream(wdt)), "masked_swiglu_down")
    return y, mask, nnz


def weight_col_norms(wt: torch.Tensor) -> torch.Tensor:
    """fp64 ``||WT[k, :]||_2`` per input index ``k``."""
    _dev(wt, "wt", torch.float16)
    d_in, d_out = wt.shape
    out = torch.empty((d_in,), dtype=torch.float64, device=wt.device)
    _check(lib().weight_col_norms(_ptr(wt), d_in, d_out, _ptr(out), _stream(wt)),
           "weight_col_norms")
    return out


# ---- batched matmuls ---------------------------------------------------------

WS_TICKET_BYTES = 1 << 20  # SA_WS_TICKET_BYTES
READ_STREAM_SINK_WORDS = 8192  # SA_READ_STREAM_SINK_WORDS


def read_stream(src: torch.Tensor, nbytes: int | None = None, blocks: int | None = None,
                sink: torch.Tensor | None = None) -> torch.Tensor:
    """Bench-only: read ``nbytes`` of ``src`` once (roofline calibration) with
    the default grid, or ``blocks`` x 256 threads; returns the sink, whose xor
    equals the xor of the bytes read."""
    _dev(src, "src", None)
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    words = READ_STREAM_SINK_WORDS if blocks is None else 4 * blocks
    if sink is None or sink.numel() < words:
        sink = torch.empty(words, dtype=torch.int32, device=src.device)
    if blocks is None:
        _check(lib().sa_read_stream(_ptr(src), n, _ptr(sink), _stream(src)), "sa_read_stream")
    else:
        _check(lib().sa_read_stream_grid(_ptr(src), n, _ptr(sink), int(blocks), _stream(src)),
               "sa_read_stream_grid")
    return sink


def nm_act_spmm(xval: torch.Tensor, mask: torch.Tensor, n: int, m: int, wt: torch.Tensor,
                y: torch.Tensor | None = None, use_workspace: bool = True):
    """``Y = (mask ⊙ X) W^T`` from the compressed N:M activations.

    With ``use_workspace`` (the default) patterns other than 2:4 take the
    library's two-pass path through the per-device workspace.
    """
    _dev(xval, "xval", torch.float16)
    _dev(mask, "mask", torch.int32)
    _dev(wt, "wt", torch.float16)
    T = mask.shape[0]
    d_in, d_out = wt.shape
    if y is None:
        y = torch.empty((T, d_out), dtype=torch.float16, device=wt.device)
    ws_ptr, ws_bytes = None, 0
    need = int(lib().sa_nm_spmm_workspace_bytes(T, d_in, n, m))
    if use_workspace and need > 0:
        ws = scratch(wt.device, need)
        ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    _check(lib().nm_act_spmm(_ptr(xval), _ptr(mask), T, d_in, n, m, _ptr(wt), d_out, _ptr(y),
                             ws_ptr, ws_bytes, _stream(wt)), "nm_act_spmm")
    return y


def nm_shared_spmm(xval: torch.Tensor, mask: torch.Tensor, n: int, m: int, tt: int,
                   wt: torch.Tensor, y: torch.Tensor | None = None):
    """``Y[t] = W (mask[t // tt] ⊙ x_t)`` from the tile-shared compressed form
    (the per-device workspace serves the tiles and patterns that need one)."""
    _dev(xval, "xval", torch.float16)
    _dev(mask, "mask", torch.int32)
    _dev(wt, "wt", torch.float16)
    T = xval.shape[0]
    d_in, d_out = wt.shape
    if y is None:
        y = torch.empty((T, d_out), dtype=torch.float16, device=wt.device)
    ws_ptr, ws_bytes = None, 0
    need = int(lib().sa_nm_shared_spmm_workspace_bytes(T, d_in, n, m, tt))
    if need > 0:
        ws = scratch(wt.device, need)
        ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    _check(lib().nm_shared_spmm(_ptr(xval), _ptr(mask), T, d_in, n, m, tt, _ptr(wt), d_out,
                                _ptr(y), ws_ptr, ws_bytes, _stream(wt)), "nm_shared_spmm")
    return y


def dense_gemm(x: torch.Tensor, wt: torch.Tensor, y: torch.Tensor | None = None):
    """Dense baseline ``Y = X W^T`` on MFMA."""
    _dev(x, "x", torch.float16)
    _dev(wt, "wt", torch.float16)
    T, d_in = x.shape
    d_out = wt.shape[1]
    if y is None:
        y = torch.empty((T, d_out), dtype=torch.float16, device=wt.device)
    _check(lib().dense_gemm(_ptr(x), T, d_in, _ptr(wt), d_out, _ptr(y), _stream(wt)), "dense_gemm")
    return y


# ---- tuning -------------------------------------------------------------------

def set_gemv_tuning(tiling: int = -1, target_wgs: int = 0, handoff: int = 0) -> None:
    _check(lib().sa_set_gemv_tuning(tiling, target_wgs, handoff), "sa_set_gemv_tuning")


def set_gemv_test_hooks(flags: int = 0) -> None:
    _check(lib().sa_set_gemv_test_hooks(flags), "sa_set_gemv_test_hooks")


def set_gemm_tuning(tile_rows: int = 0, engine: int = 0, stages: int = 0) -> None:
    _check(lib().sa_set_gemm_tuning(tile_rows, engine, stages), "sa_set_gemm_tuning")


GEMV_OPS = {"threshold": 0, "dense": 1, "masked": 2, "list": 3, "swiglu": 4, "scored": 6,
            "square": 7, "topk": 8}


def gemv_plan(op: str, d_out: int, d_in: int, batch: int = 1, cus: int = 0, resident: int = 0):
    """The decomposition a GEMV entry point would use: a dict with ``kernel``
    ("split-K" or "full-K"), ``tile_o``, ``grid_o``, ``slices`` and ``handoff``
    (0 none, 1 second launch, 2 same launch, 3 same launch in L2).  ``cus`` /
    ``resident`` 0 ask the current device."""
    out = [ctypes.c_int() for _ in range(5)]
    _check(lib().sa_gemv_plan(GEMV_OPS[op], d_out, d_in, batch, cus, resident,
                              *[ctypes.addressof(o) for o in out]), "sa_gemv_plan")
    k, t, g, sl, h = (o.value for o in out)
    return {"kernel": "full-K" if k else "split-K", "tile_o": t, "grid_o": g, "slices": sl,
            "handoff": h}


def gemm_plan(op: str, T: int, d_in: int, d_out: int, n: int = 0, m: int = 0, cus: int = 0):
    """The engine and output tile a matmul call would take: a dict with
    ``engine`` ("staged", "pipelined" or "wide"), ``tile_rows``, ``tile_cols``
    and ``tiles``.  ``op`` is "dense" (dense_gemm) or "nm" (nm_act_spmm with
    pattern n:m); ``cus`` 0 asks the current device."""
    e, r, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    t = ctypes.c_int64()
    _check(lib().sa_gemm_plan({"dense": 0, "nm": 1}[op], T, d_in, d_out, n, m, cus,
                              *[ctypes.addressof(o) for o in (e, r, c, t)]), "sa_gemm_plan")
    return {"engine": {1: "staged", 2: "pipelined", 3: "wide"}[e.value], "tile_rows": r.value,
            "tile_cols": c.value, "tiles": t.value}


def gemv_tiling_info(i: int):
    """``(tile_o, threads, unroll)`` of compiled tiling ``i``, or None past the end."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = lib().sa_gemv_tiling_info(i, ctypes.addressof(a), ctypes.addressof(b), ctypes.addressof(c))
    if st != 0:
        return None
    return a.value, b.value, c.value
