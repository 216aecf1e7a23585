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
    assert lib.msign_ns_ex(*args, 4, FAKE2, 1 << 30, None) == 1
    assert lib.msign_ns_ex(*args, 0x80000000, FAKE2, 1 << 30, None) == 1
    # the dense-products comparator does not combine with the improved init
    assert lib.msign_ns_ex(*args, 3, FAKE2, 1 << 30, None) == 1
    # a valid flag still goes through the other checks (too small a workspace)
    assert lib.msign_ns_ex(*args, 1, FAKE2, 16, None) == 4
    assert lib.msign_ns_ex(*args, 2, FAKE2, 16, None) == 4
    # syrk_xxt_ex: one flag (full tiles); others rejected before any launch
    assert lib.syrk_xxt_ex(FAKE, FAKE2, 1, 8, 64, 1, 1.0, None, 0.0, 0.0, 2, None, 0, None) == 1


def test_noalloc_rejects_before_touching_the_device():
    """msign_ns_noalloc: sizes beyond its fixed scratch, bad dtypes and empty
    problems are settled on the host (no device lookup, no launch)."""
    lib = _lib()
    assert lib.msign_ns_workspace_bytes(1, 1024, 4096, 1) <= mod.NOALLOC_SCRATCH_BYTES
    assert lib.msign_ns_workspace_bytes(1, 2048, 4096, 1) > mod.NOALLOC_SCRATCH_BYTES
    assert lib.msign_ns_noalloc(FAKE, FAKE, 1, 2048, 4096, 1, 1, 5, None, 1e-20, None) == 4
    assert b"scratch" in lib.msign_last_error()
    assert lib.msign_ns_noalloc(FAKE, FAKE, 1, 8, 16, 1, 9, 5, None, 1e-20, None) == 2
    assert lib.msign_ns_noalloc(FAKE, FAKE, 1, 8, 16, 1, 1, 0, None, 1e-20, None) == 1
    assert lib.msign_ns_noalloc(None, None, 0, 8, 16, 1, 1, 5, None, 1e-20, None) == 0


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
    assert lib.msign_kernel_timing_enable(0x20) == 1   # 5 classes: bits 0..4
    assert lib.msign_kernel_timing_enable(0x10) == 0   # the small-matrix kernel only
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


def _garr(*groups):
    arr = (mod._Group * len(groups))()
    for i, g in enumerate(groups):
        arr[i] = mod._Group(*g)
    return arr


def test_grouped_argument_errors():
    lib = _lib()
    ok = (0x10000, 0x10000, 1, 8, 16)
    other = (0x30000, 0x30000, 2, 40, 24)

    def ns(arr, n, ws=FAKE2, wsb=1 << 30):
        return lib.msign_ns_grouped(arr, n, 1, 1, 5, None, 1e-20, 0, ws, wsb, None)

    assert ns(_garr(ok), 0) == 1
    assert ns(_garr(ok, ok, ok, ok, ok), 5) == 1
    assert ns(None, 1) == 1
    # a bad group is named in the message
    assert ns(_garr(ok, (0x40000, 0x40000, -1, 8, 16)), 2) == 3
    assert b"group 1" in lib.msign_last_error()
    # one group's output over another group's input
    assert ns(_garr(ok, (0x50000, 0x10000 + 64, 1, 8, 16)), 2) == 5
    assert b"another" in lib.msign_last_error()
    # inputs may overlap each other (read only): only the workspace is short
    assert ns(_garr((0x10000, 0x60000, 1, 8, 16), (0x10000, 0x70000, 1, 8, 16)), 2, wsb=16) == 4
    assert ns(_garr(ok, other), 2, wsb=16) == 4
    # all groups empty: a no-op
    assert ns(_garr((0, 0, 0, 8, 16), (0, 0, 3, 0, 16)), 2, ws=None, wsb=0) == 0
    g = lib.msign_gram_ns_grouped
    arr = (ctypes.c_int32 * 1)(5)
    assert g(_garr(ok, other), 2, 1, 2, 5, None, 1e-20, arr, 1, FAKE2, 1 << 30, None) == 1


def test_grouped_workspace_queries():
    lib = _lib()
    big = (1 << 64) - 1
    one = (0, 0, 3, 128, 256)
    tall = (0, 0, 2, 300, 70)
    empty = (0, 0, 0, 64, 64)
    for q, single in ((lib.msign_ns_grouped_workspace_bytes, lib.msign_ns_workspace_bytes),
                      (lib.msign_gram_ns_grouped_workspace_bytes, lib.msign_gram_ns_workspace_bytes)):
        # one group is the single-problem call
        assert q(_garr(one), 1, 1) == single(3, 128, 256, 1)
        # empty groups are skipped
        assert q(_garr(one, empty), 2, 1) == q(_garr(one), 1, 1)
        assert q(_garr(empty), 1, 1) == 0
        # the groups' own buffers are all there
        both = q(_garr(one, tall), 2, 1)
        assert both > max(single(3, 128, 256, 1), single(2, 300, 70, 1))
        assert q(_garr(one), 0, 1) == big
        assert q(_garr(one), 1, 9) == big
        assert q(_garr((0, 0, -1, 8, 8)), 1, 1) == big
        assert q(None, 1, 1) == big


def _marr(*groups):
    arr = (mod._MuonGroup * len(groups))()
    for i, g in enumerate(groups):
        arr[i] = mod._MuonGroup(*g)
    return arr


def test_muon_step_argument_errors():
    lib = _lib()
    ok = (0x100000, 0x200000, 0x300000, 1, 8, 16)

    def step(arr, n=1, mu=0.9, lr=0.01, method=0, flags=0, restarts=None, nr=0, ws=FAKE2, wsb=1 << 30, io=1):
        return lib.muon_step(arr, n, io, mu, lr, method, 1, 5, None, 1e-20, flags, restarts, nr, ws, wsb, None)

    assert step(_marr(ok), n=0) == 1
    assert step(None) == 1
    assert step(_marr(ok), method=2) == 1
    assert step(_marr(ok), mu=float("nan")) == 1
    assert step(_marr(ok), lr=float("inf")) == 1
    assert step(_marr(ok), io=7) == 2
    assert step(_marr(ok), flags=4) == 1
    assert step(_marr(ok), method=1, flags=1) == 1          # flags are for NS only
    bad = (ctypes.c_int32 * 1)(9)
    assert step(_marr(ok), method=1, restarts=bad, nr=1) == 1
    assert step(_marr((0x100000, 0x200000, None, 1, 8, 16))) == 1
    assert step(_marr((0x100001, 0x200000, 0x300000, 1, 8, 16))) == 1   # misaligned w
    assert step(_marr((0x100000, 0x200000, 0x300000, -1, 8, 16))) == 3
    assert step(_marr(ok), wsb=16) == 4
    assert step(_marr(ok), ws=ctypes.c_void_p(0x20000010)) == 4
    # m over w, w over another group's gradient, g inside the workspace
    assert step(_marr((0x100000, 0x200000, 0x100000 + 64, 1, 8, 16))) == 5
    assert step(_marr(ok, (0x400000, 0x100000, 0x500000, 1, 8, 16)), n=2) == 5
    assert step(_marr((0x100000, 0x20000000 + 256, 0x300000, 1, 8, 16))) == 5
    # gradients may be shared between groups (read only); steps are checked
    # before anything is launched
    assert lib.muon_step(_marr(ok), 1, 1, 0.9, 0.01, 0, 1, 0, None, 1e-20, 0, None, 0, FAKE2, 1 << 30,
                         None) == 1
    # every group empty: a no-op
    assert step(_marr((0, 0, 0, 0, 8, 16)), ws=None, wsb=0) == 0


def test_muon_step_workspace_query():
    lib = _lib()
    big = (1 << 64) - 1
    # the step is fused into the msign call: its workspace is the msign call's
    for b, r, c in ((3, 128, 256), (2, 300, 70)):
        arr = _marr((0, 0, 0, b, r, c))
        assert lib.muon_step_workspace_bytes(arr, 1, 0, 1) == lib.msign_ns_workspace_bytes(b, r, c, 1)
        assert lib.muon_step_workspace_bytes(arr, 1, 1, 2) == lib.msign_gram_ns_workspace_bytes(b, r, c, 2)
    assert lib.muon_step_workspace_bytes(_marr((0, 0, 0, 0, 8, 8)), 1, 0, 1) == 0
    assert lib.muon_step_workspace_bytes(_marr((0, 0, 0, 1, 8, 8)), 1, 5, 1) == big
    assert lib.muon_step_workspace_bytes(_marr((0, 0, 0, 1, 8, 8)), 0, 0, 1) == big


def test_mfma_probe_argument_errors():
    lib = _lib()
    assert lib.msign_mfma_probe(0, 10, FAKE2, None) == 2      # fp32 has no 16x16x32 form
    assert lib.msign_mfma_probe(1, 0, FAKE2, None) == 1
    assert lib.msign_mfma_probe(1, 10, None, None) == 1
    assert lib.msign_mfma_probe(1, 10, ctypes.c_void_p(0x20000001), None) == 1
