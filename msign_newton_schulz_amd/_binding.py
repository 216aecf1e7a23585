"""ctypes binding of libmsign's C ABI (include/msign.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  Torch provides device memory (inputs, outputs, workspace) and the
stream.  If the library is missing or cannot be loaded, every entry point
raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsign.so")

F32, BF16, F16 = 0, 1, 2
_TORCH_TO_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_STATUS = {0: "ok", 1: "invalid argument", 2: "invalid dtype", 3: "invalid shape",
           4: "workspace", 5: "alias", 6: "HIP error"}
MAX_STEPS = 64
KCLASSES = ("normalize", "xxt", "square", "rect")


class MsignError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"libmsign: {_STATUS.get(status, status)}: {detail}")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, sz, vp, f = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    fp = ctypes.POINTER(ctypes.c_float)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.msign_ns_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.msign_ns_workspace_bytes.restype = sz
    lib.msign_gram_ns_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.msign_gram_ns_workspace_bytes.restype = sz
    lib.syrk_xxt_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.syrk_xxt_workspace_bytes.restype = sz
    lib.msign_ns.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, fp, f, vp, sz, vp]
    lib.msign_ns.restype = ctypes.c_int
    lib.msign_ns_ex.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, fp, f, ctypes.c_uint32, vp, sz, vp]
    lib.msign_ns_ex.restype = ctypes.c_int
    lib.msign_gram_ns.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, fp, f, ip, i32, vp, sz, vp]
    lib.msign_gram_ns.restype = ctypes.c_int
    lib.syrk_xxt.argtypes = [vp, vp, i64, i64, i64, i32, f, vp, f, f, vp, sz, vp]
    lib.syrk_xxt.restype = ctypes.c_int
    lib.msign_status_string.argtypes = [ctypes.c_int]
    lib.msign_status_string.restype = ctypes.c_char_p
    lib.msign_last_error.argtypes = []
    lib.msign_last_error.restype = ctypes.c_char_p
    lib.msign_version.argtypes = []
    lib.msign_version.restype = ctypes.c_char_p
    lib.msign_kernel_timing_enable.argtypes = [i32]
    lib.msign_kernel_timing_enable.restype = ctypes.c_int
    lib.msign_kernel_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.msign_kernel_timing_read.restype = ctypes.c_int
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def version() -> str:
    return _load().msign_version().decode()


def _check(st: int):
    if st != 0:
        raise MsignError(st, _load().msign_last_error().decode())


def _dt(dtype) -> int:
    if dtype in _TORCH_TO_DT:
        return _TORCH_TO_DT[dtype]
    if isinstance(dtype, str):
        return {"f32": F32, "fp32": F32, "bf16": BF16, "f16": F16, "fp16": F16}[dtype]
    raise TypeError(f"unsupported dtype {dtype}")


def _coeff_array(coeffs, steps: int):
    if coeffs is None:
        return None
    flat = []
    rows = list(coeffs)
    if len(rows) == 3 and all(isinstance(v, (int, float)) for v in rows):
        rows = [rows] * steps
    if len(rows) != steps:
        raise ValueError(f"coefficient table needs {steps} rows, got {len(rows)}")
    for r in rows:
        r = [float(v) for v in r]
        if len(r) != 3:
            raise ValueError("each coefficient row needs (a, b, c)")
        flat.extend(r)
    return (ctypes.c_float * len(flat))(*flat)


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _batch_dims(x: torch.Tensor):
    if x.dim() < 2:
        raise ValueError("msign needs at least 2 dims")
    rows, cols = int(x.shape[-2]), int(x.shape[-1])
    batch = int(math.prod(x.shape[:-2])) if x.dim() > 2 else 1
    return batch, rows, cols


def _check_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on a GPU device")


def ns_workspace_bytes(batch: int, rows: int, cols: int, compute_dtype=torch.bfloat16) -> int:
    return int(_load().msign_ns_workspace_bytes(batch, rows, cols, _dt(compute_dtype)))


def gram_ns_workspace_bytes(batch: int, rows: int, cols: int, compute_dtype=torch.float16) -> int:
    return int(_load().msign_gram_ns_workspace_bytes(batch, rows, cols, _dt(compute_dtype)))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == (1 << 64) - 1:
        raise MsignError(3, "invalid sizes for the workspace query")
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


IMPROVED_INIT = 1  # MSIGN_NS_IMPROVED_INIT


def msign_ns(x: torch.Tensor, steps: int = 5, coeffs=None, eps: float = 1e-20,
             compute_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None,
             improved_init: bool = False) -> torch.Tensor:
    """Standard quintic Newton-Schulz msign over the last two dims (C ABI
    `msign_ns`, or `msign_ns_ex` with MSIGN_NS_IMPROVED_INIT when
    `improved_init`).  `coeffs`: None (Keller constants), one (a, b, c) triple
    or a table of `steps` rows.  Returns a tensor shaped and typed like `x`."""
    _check_cuda(x, out, workspace)
    lib = _load()
    x = x.contiguous()
    batch, rows, cols = _batch_dims(x)
    io, cdt = _dt(x.dtype), _dt(compute_dtype)
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("out must be contiguous with the shape and dtype of x")
    nbytes = lib.msign_ns_workspace_bytes(batch, rows, cols, cdt)
    ws = _workspace(nbytes, x.device, workspace)
    carr = _coeff_array(coeffs, steps)
    with torch.cuda.device(x.device):
        st = lib.msign_ns_ex(x.data_ptr(), y.data_ptr(), batch, rows, cols, io, cdt, steps,
                             carr, float(eps), IMPROVED_INIT if improved_init else 0,
                             ws.data_ptr(), ws.numel(), _stream_handle(x.device))
    _check(st)
    return y


def msign_gram_ns(x: torch.Tensor, steps: int = 5, coeffs=None, eps: float = 1e-20,
                  compute_dtype=torch.float16, restart_after: Sequence[int] = (2,),
                  out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gram Newton-Schulz msign over the last two dims (C ABI `msign_gram_ns`);
    `restart_after=()` is the naive form, `(2,)` the stabilised one."""
    _check_cuda(x, out, workspace)
    lib = _load()
    x = x.contiguous()
    batch, rows, cols = _batch_dims(x)
    io, cdt = _dt(x.dtype), _dt(compute_dtype)
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("out must be contiguous with the shape and dtype of x")
    nbytes = lib.msign_gram_ns_workspace_bytes(batch, rows, cols, cdt)
    ws = _workspace(nbytes, x.device, workspace)
    carr = _coeff_array(coeffs, steps)
    rs = [int(r) for r in restart_after]
    rarr = (ctypes.c_int32 * len(rs))(*rs) if rs else None
    with torch.cuda.device(x.device):
        st = lib.msign_gram_ns(x.data_ptr(), y.data_ptr(), batch, rows, cols, io, cdt, steps,
                               carr, float(eps), rarr, len(rs), ws.data_ptr(), ws.numel(),
                               _stream_handle(x.device))
    _check(st)
    return y


def syrk_xxt(x: torch.Tensor, alpha: float = 1.0, d: Optional[torch.Tensor] = None,
             beta: float = 0.0, gamma: float = 0.0,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = alpha X X^T + beta D + gamma I over the last two dims (C ABI
    `syrk_xxt`); C is exactly symmetric."""
    _check_cuda(x, d, out)
    lib = _load()
    x = x.contiguous()
    batch, n, k = _batch_dims(x)
    dt = _dt(x.dtype)
    shape = tuple(x.shape[:-1]) + (n,)
    c = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    if tuple(c.shape) != shape or c.dtype != x.dtype or not c.is_contiguous():
        raise ValueError("out must be contiguous [..., n, n] with the dtype of x")
    if d is not None:
        d = d.contiguous()
        if tuple(d.shape) != shape or d.dtype != x.dtype:
            raise ValueError("d must be [..., n, n] with the dtype of x")
    nbytes = lib.syrk_xxt_workspace_bytes(batch, n, k, dt)
    ws = None
    if nbytes == (1 << 64) - 1:
        raise MsignError(3, "invalid sizes")
    if nbytes > 0:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        st = lib.syrk_xxt(x.data_ptr(), c.data_ptr(), batch, n, k, dt, float(alpha),
                          d.data_ptr() if d is not None else None, float(beta), float(gamma),
                          ws.data_ptr() if ws is not None else None, nbytes,
                          _stream_handle(x.device))
    _check(st)
    return c


def kernel_timing(enable: bool, classes=None):
    """Turn per-kernel-class HIP event timing on or off (measurement only).
    `classes` limits it to some of KCLASSES (default: all)."""
    mask = 0
    if enable:
        names = KCLASSES if classes is None else classes
        for c in names:
            mask |= 1 << KCLASSES.index(c)
    _check(_load().msign_kernel_timing_enable(mask))


def read_kernel_timing():
    """{class: (total_ms, launches)} accumulated since timing was enabled."""
    tot = (ctypes.c_double * 4)()
    cnt = (ctypes.c_int64 * 4)()
    _check(_load().msign_kernel_timing_read(tot, cnt))
    return {KCLASSES[i]: (tot[i], cnt[i]) for i in range(4)}
