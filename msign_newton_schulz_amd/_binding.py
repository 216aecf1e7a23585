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
KCLASSES = ("normalize", "xxt", "square", "rect", "small")


class MsignError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"libmsign: {_STATUS.get(status, status)}: {detail}")


MAX_GROUPS = 4  # MSIGN_MAX_GROUPS


class _Group(ctypes.Structure):
    """msign_group_t"""
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("batch", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class _MuonGroup(ctypes.Structure):
    """muon_group_t"""
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("batch", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


MUON_NS, MUON_GRAM = 0, 1

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
    lib.msign_ns_noalloc.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, fp, f, vp]
    lib.msign_ns_noalloc.restype = ctypes.c_int
    lib.msign_gram_ns.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, fp, f, ip, i32, vp, sz, vp]
    lib.msign_gram_ns.restype = ctypes.c_int
    lib.syrk_xxt.argtypes = [vp, vp, i64, i64, i64, i32, f, vp, f, f, vp, sz, vp]
    lib.syrk_xxt.restype = ctypes.c_int
    lib.syrk_xxt_ex.argtypes = [vp, vp, i64, i64, i64, i32, f, vp, f, f, ctypes.c_uint32, vp, sz, vp]
    lib.syrk_xxt_ex.restype = ctypes.c_int
    gp = ctypes.POINTER(_Group)
    lib.msign_ns_grouped_workspace_bytes.argtypes = [gp, i32, i32]
    lib.msign_ns_grouped_workspace_bytes.restype = sz
    lib.msign_gram_ns_grouped_workspace_bytes.argtypes = [gp, i32, i32]
    lib.msign_gram_ns_grouped_workspace_bytes.restype = sz
    lib.msign_ns_grouped.argtypes = [gp, i32, i32, i32, i32, fp, f, ctypes.c_uint32, vp, sz, vp]
    lib.msign_ns_grouped.restype = ctypes.c_int
    lib.msign_gram_ns_grouped.argtypes = [gp, i32, i32, i32, i32, fp, f, ip, i32, vp, sz, vp]
    lib.msign_gram_ns_grouped.restype = ctypes.c_int
    mp = ctypes.POINTER(_MuonGroup)
    lib.muon_step_workspace_bytes.argtypes = [mp, i32, i32, i32]
    lib.muon_step_workspace_bytes.restype = sz
    lib.muon_step.argtypes = [mp, i32, i32, f, f, i32, i32, i32, fp, f, ctypes.c_uint32, ip, i32, vp, sz, vp]
    lib.muon_step.restype = ctypes.c_int
    lib.msign_mfma_probe.argtypes = [i32, i32, vp, vp]
    lib.msign_mfma_probe.restype = ctypes.c_int
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
DENSE_PRODUCTS = 2  # MSIGN_NS_DENSE_PRODUCTS
SYRK_FULL_TILES = 1  # MSIGN_SYRK_FULL_TILES


def msign_ns(x: torch.Tensor, steps: int = 5, coeffs=None, eps: float = 1e-20,
             compute_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None,
             improved_init: bool = False, dense_products: bool = False) -> torch.Tensor:
    """Standard quintic Newton-Schulz msign over the last two dims (C ABI
    `msign_ns_ex`, with MSIGN_NS_IMPROVED_INIT when `improved_init` and the
    full-tile comparator MSIGN_NS_DENSE_PRODUCTS when `dense_products`).
    `coeffs`: None (Keller constants), one (a, b, c) triple or a table of
    `steps` rows.  Returns a tensor shaped and typed like `x`."""
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
                             carr, float(eps),
                             (IMPROVED_INIT if improved_init else 0) | (DENSE_PRODUCTS if dense_products else 0),
                             ws.data_ptr(), ws.numel(), _stream_handle(x.device))
    _check(st)
    return y


NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024  # MSIGN_NOALLOC_SCRATCH_BYTES


def msign_ns_noalloc(x: torch.Tensor, out: torch.Tensor, steps: int = 5, coeffs=None,
                     eps: float = 1e-20, compute_dtype=torch.bfloat16) -> torch.Tensor:
    """msign_ns through the allocation-free entry point (C ABI
    `msign_ns_noalloc`): the library's fixed per-device scratch replaces the
    workspace, so nothing is allocated; `out` must be given.  Calls that may
    overlap in time on one device race on that scratch."""
    _check_cuda(x, out)
    lib = _load()
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (a copy would allocate)")
    batch, rows, cols = _batch_dims(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous with the shape and dtype of x")
    carr = _coeff_array(coeffs, steps)
    with torch.cuda.device(x.device):
        st = lib.msign_ns_noalloc(x.data_ptr(), out.data_ptr(), batch, rows, cols, _dt(x.dtype),
                                  _dt(compute_dtype), steps, carr, float(eps), _stream_handle(x.device))
    _check(st)
    return out


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


def _groups(xs, outs):
    """Contiguous inputs, outputs and the msign_group_t array of a grouped call."""
    xs = [x.contiguous() for x in xs]
    if not 1 <= len(xs) <= MAX_GROUPS:
        raise ValueError(f"a grouped call takes 1..{MAX_GROUPS} tensors, got {len(xs)}")
    _check_cuda(*xs)
    if len({x.dtype for x in xs}) != 1 or len({x.device for x in xs}) != 1:
        raise ValueError("grouped tensors must share dtype and device")
    if outs is None:
        outs = [torch.empty_like(x) for x in xs]
    outs = list(outs)
    if len(outs) != len(xs):
        raise ValueError("outs needs one tensor per input")
    arr = (_Group * len(xs))()
    for i, (x, y) in enumerate(zip(xs, outs)):
        _check_cuda(y)
        if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
            raise ValueError("each out must be contiguous with the shape and dtype of its input")
        batch, rows, cols = _batch_dims(x)
        arr[i] = _Group(x.data_ptr(), y.data_ptr(), batch, rows, cols)
    return xs, outs, arr


def msign_ns_grouped(xs: Sequence[torch.Tensor], steps: int = 5, coeffs=None, eps: float = 1e-20,
                     compute_dtype=torch.bfloat16, outs: Optional[Sequence[torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None,
                     improved_init: bool = False) -> list:
    """msign_ns over up to MAX_GROUPS tensors of different shapes in one call
    (C ABI `msign_ns_grouped`): each product of the iteration is one launch
    over all of them.  Returns one output per input."""
    lib = _load()
    xs, outs, arr = _groups(xs, outs)
    io, cdt = _dt(xs[0].dtype), _dt(compute_dtype)
    nbytes = lib.msign_ns_grouped_workspace_bytes(arr, len(xs), cdt)
    ws = _workspace(nbytes, xs[0].device, workspace)
    _check_cuda(ws)
    carr = _coeff_array(coeffs, steps)
    with torch.cuda.device(xs[0].device):
        st = lib.msign_ns_grouped(arr, len(xs), io, cdt, steps, carr, float(eps),
                                  IMPROVED_INIT if improved_init else 0, ws.data_ptr(), ws.numel(),
                                  _stream_handle(xs[0].device))
    _check(st)
    return outs


def msign_gram_ns_grouped(xs: Sequence[torch.Tensor], steps: int = 5, coeffs=None, eps: float = 1e-20,
                          compute_dtype=torch.float16, restart_after: Sequence[int] = (2,),
                          outs: Optional[Sequence[torch.Tensor]] = None,
                          workspace: Optional[torch.Tensor] = None) -> list:
    """msign_gram_ns over up to MAX_GROUPS tensors of different shapes in one
    call (C ABI `msign_gram_ns_grouped`).  Returns one output per input."""
    lib = _load()
    xs, outs, arr = _groups(xs, outs)
    io, cdt = _dt(xs[0].dtype), _dt(compute_dtype)
    nbytes = lib.msign_gram_ns_grouped_workspace_bytes(arr, len(xs), cdt)
    ws = _workspace(nbytes, xs[0].device, workspace)
    _check_cuda(ws)
    carr = _coeff_array(coeffs, steps)
    rs = [int(r) for r in restart_after]
    rarr = (ctypes.c_int32 * len(rs))(*rs) if rs else None
    with torch.cuda.device(xs[0].device):
        st = lib.msign_gram_ns_grouped(arr, len(xs), io, cdt, steps, carr, float(eps), rarr, len(rs),
                                       ws.data_ptr(), ws.numel(), _stream_handle(xs[0].device))
    _check(st)
    return outs


def muon_step(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
              moms: Sequence[torch.Tensor], *, lr: float, mu: float, method: str = "ns",
              steps: int = 5, coeffs=None, eps: float = 1e-20, compute_dtype=None,
              restart_after: Sequence[int] = (2,), improved_init: bool = False,
              workspace: Optional[torch.Tensor] = None) -> None:
    """One Muon step in place over up to MAX_GROUPS parameter tensors (C ABI
    `muon_step`): for every matrix over the last two dims, m <- mu m + g and
    w <- w - lr msign(m), msign by standard NS (`method="ns"`, bf16 products
    by default) or Gram NS (`"gram"`, fp16 products, restart after step 2 by
    default).  Parameters and gradients share one dtype; momenta are fp32."""
    lib = _load()
    params, grads, moms = list(params), list(grads), list(moms)
    if not (len(params) == len(grads) == len(moms)) or not 1 <= len(params) <= MAX_GROUPS:
        raise ValueError(f"muon_step takes 1..{MAX_GROUPS} (param, grad, momentum) triples")
    if method not in ("ns", "gram"):
        raise ValueError("method must be 'ns' or 'gram'")
    _check_cuda(*params, *grads, *moms, workspace)
    io = _dt(params[0].dtype)
    arr = (_MuonGroup * len(params))()
    for i, (w, g, m) in enumerate(zip(params, grads, moms)):
        if g.shape != w.shape or m.shape != w.shape:
            raise ValueError("each gradient and momentum must have its parameter's shape")
        if w.dtype != params[0].dtype or g.dtype != w.dtype or m.dtype != torch.float32:
            raise ValueError("parameters and gradients share one dtype; momenta are float32")
        if not (w.is_contiguous() and g.is_contiguous() and m.is_contiguous()):
            raise ValueError("parameters, gradients and momenta must be contiguous")
        batch, rows, cols = _batch_dims(w)
        arr[i] = _MuonGroup(w.data_ptr(), g.data_ptr(), m.data_ptr(), batch, rows, cols)
    meth = MUON_NS if method == "ns" else MUON_GRAM
    if compute_dtype is None:
        compute_dtype = torch.bfloat16 if method == "ns" else torch.float16
    cdt = _dt(compute_dtype)
    nbytes = lib.muon_step_workspace_bytes(arr, len(params), meth, cdt)
    ws = _workspace(nbytes, params[0].device, workspace)
    carr = _coeff_array(coeffs, steps)
    rs = [int(r) for r in restart_after] if method == "gram" else []
    rarr = (ctypes.c_int32 * len(rs))(*rs) if rs else None
    flags = IMPROVED_INIT if improved_init else 0
    with torch.cuda.device(params[0].device):
        st = lib.muon_step(arr, len(params), io, float(mu), float(lr), meth, cdt, steps, carr, float(eps),
                           flags, rarr, len(rs), ws.data_ptr(), ws.numel(), _stream_handle(params[0].device))
    _check(st)


PROBE_BLOCKS, PROBE_THREADS = 512, 256
PROBE_FLOPS_PER_ITER = 512.0 * 4 * 8 * 16 * 16 * 32 * 2  # MSIGN_PROBE_FLOPS_PER_ITER


def mfma_probe(iters: int, dtype=torch.bfloat16, device="cuda", out: Optional[torch.Tensor] = None) -> float:
    """Queue one MFMA-only launch (C ABI `msign_mfma_probe`, measurement
    only) on the current stream; returns its flop count."""
    lib = _load()
    if out is None:
        out = torch.empty(PROBE_BLOCKS * PROBE_THREADS, dtype=torch.float32, device=device)
    _check_cuda(out)
    with torch.cuda.device(out.device):
        st = lib.msign_mfma_probe(_dt(dtype), int(iters), out.data_ptr(), _stream_handle(out.device))
    _check(st)
    return PROBE_FLOPS_PER_ITER * iters


def syrk_xxt(x: torch.Tensor, alpha: float = 1.0, d: Optional[torch.Tensor] = None,
             beta: float = 0.0, gamma: float = 0.0,
             out: Optional[torch.Tensor] = None, full_tiles: bool = False) -> torch.Tensor:
    """C = alpha X X^T + beta D + gamma I over the last two dims (C ABI
    `syrk_xxt`; `syrk_xxt_ex` with MSIGN_SYRK_FULL_TILES when `full_tiles`,
    the plain-product comparator).  C is exactly symmetric unless
    `full_tiles`."""
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
        st = lib.syrk_xxt_ex(x.data_ptr(), c.data_ptr(), batch, n, k, dt, float(alpha),
                             d.data_ptr() if d is not None else None, float(beta), float(gamma),
                             SYRK_FULL_TILES if full_tiles else 0,
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
    k = len(KCLASSES)
    tot = (ctypes.c_double * k)()
    cnt = (ctypes.c_int64 * k)()
    _check(_load().msign_kernel_timing_read(tot, cnt))
    return {KCLASSES[i]: (tot[i], cnt[i]) for i in range(k)}
