"""CPU checks of the C ABI: the library loads, exports every declared symbol
and rejects bad arguments before touching the GPU.  No compute call is made
(nothing here launches a kernel)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msign.h")

mod = pytest.importorskip("msign_newton_schulz_amd._binding")


def _lib():
    if not os.path.exists(mod.LIB_PATH):
        pytest.skip("libmsign.so not built")
    try:
        return mod.library()
    except OSError as e:  # pragma: no cover - missing HIP runtime
        if "undefined symbol" in str(e):
            raise  # a broken build, not a missing runtime
        pytest.skip(f"cannot load libmsign.so here: {e}")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s+\*?([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("msign_ns", "msign_ns_ex", "msign_gram_ns", "syrk_xxt", "msign_ns_workspace_bytes",
                 "msign_gram_ns_workspace_bytes", "syrk_xxt_workspace_bytes",
                 "msign_status_string", "msign_last_error", "msign_version",
                 "msign_kernel_timing_enable", "msign_kernel_timing_read"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = _lib()
    assert b"gfx950" in lib.msign_version()
    for st in range(7):
        assert lib.msign_status_string(st)
    assert lib.msign_status_string(99) == b"unknown status"


def test_workspace_queries():
    lib = _lib()
    big = (1 << 64) - 1
    assert lib.msign_ns_workspace_bytes(0, 10, 10, 1) == 0
    assert lib.msign_ns_workspace_bytes(1, -1, 10, 1) == big
    assert lib.msign_ns_workspace_bytes(1, 10, 10, 7) == big
    # 128 x 256 bf16: fp32 master + one bf16 copy, ping-pong; A, B;
    # norm partials; plus scratch for K-split tiles
    nm, nn = 128 * 256, 128 * 128
    assert lib.msign_ns_workspace_bytes(1, 128, 256, 1) >= 2 * (4 * nm + 2 * nm) + 2 * 2 * nn + 256
    assert lib.msign_ns_workspace_bytes(4, 128, 256, 1) >= 4 * (2 * (4 * nm + 2 * nm) + 2 * 2 * nn)
    # tall and wide share a plan
    assert lib.msign_ns_workspace_bytes(3, 300, 70, 2) == lib.msign_ns_workspace_bytes(3, 70, 300, 2)
    assert lib.msign_gram_ns_workspace_bytes(1, 128, 256, 2) >= 2 * 2 * nm + 5 * 2 * nn + 256
    # short K: no split scratch; ragged k: a zero-padded copy of x
    assert lib.syrk_xxt_workspace_bytes(2, 17, 64, 1) == 0
    assert lib.syrk_xxt_workspace_bytes(2, 17, 33, 1) == 2 * 64 * 64 * 2


FAKE = ctypes.c_void_p(0x10000)
FAKE2 = ctypes.c_void_p(0x20000000)


def _ns(lib, **kw):
    args = dict(x=FAKE, y=FAKE, batch=1, rows=8, cols=16, io=1, cdt=1, steps=5, coeffs=None,
                eps=1e-20, ws=FAKE2, wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.msign_ns(args["x"], args["y"], args["batch"], args["rows"], args["cols"], args["io"],
                        args["cdt"], args["steps"], args["coeffs"], args["eps"], args["ws"],
                        args["wsb"], args["stream"])


def test_ns_argument_errors_before_launch():
    lib = _lib()
    assert _ns(lib, io=5) == 2
    assert _ns(lib, cdt=-1) == 2
    assert _ns(lib, rows=-1) == 3
    assert _ns(lib, batch=70000) == 3
    assert _ns(lib, cols=(1 << 20) + 1) == 3
    assert _ns(lib, steps=0) == 1
    assert _ns(lib, steps=65) == 1
    assert _ns(lib, eps=-1.0) == 1
    assert _ns(lib, eps=float("inf")) == 1
    bad = (ctypes.c_float * 15)(*([1.0] * 14 + [float("nan")]))
    assert _ns(lib, coeffs=bad) == 1
    assert _ns(lib, x=None) == 1
    assert _ns(lib, x=ctypes.c_void_p(0x10001)) == 1
    assert _ns(lib, ws=None) == 4
    assert _ns(lib, wsb=16) == 4
    assert _ns(lib, ws=ctypes.c_void_p(0x20000010)) == 4
    # y overlapping the workspace, and y partially overlapping x
    assert _ns(lib, y=ctypes.c_void_p(0x20000000 + 64)) == 5
    assert _ns(lib, y=ctypes.c_void_p(0x10000 + 2)) == 5
    assert b"overlap" in lib.msign_last_error()
    # empty problems succeed without touching anything
    assert _ns(lib, batch=0, x=None, y=None, ws=None, wsb=0) == 0
    assert _ns(lib, rows=0, x=None, y=None, ws=None, wsb=0) == 0


def test_ns_ex_rejects_unknown_flags():
    lib = _lib()
    args = (FAKE, FAKE, 1, 8, 16, 1, 1, 5, None, 1e-20)
    assert lib.msign_ns_ex(*args, 2, FAKE2, 1 << 30, None) == 1
    assert lib.msign_ns_ex(*args, 0x80000000, FAKE2, 1 << 30, None) == 1
    # a valid flag still goes through the other checks (too small a workspace)
    assert lib.msign_ns_ex(*args, 1, FAKE2, 16, None) == 4


def _gram(lib, restarts, n_restarts, steps=5, **kw):
    arr = (ctypes.c_int32 * len(restarts))(*restarts) if restarts is not None else None
    return lib.msign_gram_ns(FAKE, FAKE, 1, 8, 16, 1, 2, steps, None, 1e-20, arr, n_restarts,
                             kw.get("ws", FAKE2), kw.get("wsb", 1 << 30), None)


def test_gram_restart_list_validation():
    lib = _lib()
    assert _gram(lib, [5], 1) == 1        # must be < steps
    assert _gram(lib, [0], 1) == 1        # must be >= 1
    assert _gram(lib, [3, 2], 2) == 1     # strictly increasing
    assert _gram(lib, [2, 2], 2) == 1
    assert _gram(lib, None, 1) == 1       # null with a count
    assert _gram(lib, [2], 0) == 1        # pointer without a count
    assert _gram(lib, [2], -1) == 1
    assert _gram(lib, [2], 1, wsb=8) == 4


def test_syrk_argument_errors():
    lib = _lib()
    f = lib.syrk_xxt
    assert f(FAKE, FAKE2, 1, 8, 16, 9, 1.0, None, 0.0, 0.0, None, 0, None) == 2
    assert f(FAKE, FAKE2, -1, 8, 16, 1, 1.0, None, 0.0, 0.0, None, 0, None) == 3
    assert f(FAKE, FAKE2, 1, 8, 16, 1, float("nan"), None, 0.0, 0.0, None, 0, None) == 1
    assert f(FAKE, None, 1, 8, 16, 1, 1.0, None, 0.0, 0.0, None, 0, None) == 1
    assert f(FAKE, FAKE, 1, 8, 16, 1, 1.0, None, 0.0, 0.0, None, 0, None) == 5
    # ragged k needs a workspace
    assert f(FAKE, FAKE2, 1, 8, 15, 1, 1.0, None, 0.0, 0.0, None, 0, None) == 4
    assert f(FAKE, FAKE2, 1, 8, 16, 1, 1.0, None, 0.0, 0.0, None, 0, None) == 4
    assert f(FAKE, FAKE2, 0, 8, 16, 1, 1.0, None, 0.0, 0.0, None, 0, None) == 0


def test_timing_read_rejects_null():
    lib = _lib()
    assert lib.msign_kernel_timing_read(None, None) == 1


def test_timing_mask_validation():
    lib = _lib()
    assert lib.msign_kernel_timing_enable(0x10) == 1
    assert lib.msign_kernel_timing_enable(-1) == 1
    assert lib.msign_kernel_timing_enable(0b1000) == 0   # rect only
    assert lib.msign_kernel_timing_enable(0) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    _lib()
    with pytest.raises(ValueError):
        mod.msign_ns(torch.zeros(4, 8))
    with pytest.raises(ValueError):
        mod.syrk_xxt(torch.zeros(4, 8))
