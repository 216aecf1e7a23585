"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Sizes here finish in seconds on the oracle yet span several 128x128 tiles
and ragged tails.  Tolerances: max relative Frobenius error 2e-2 for bf16 and
fp16 products and 1e-4 for fp32 products (against the oracle's NS output);
exact bitwise checks for symmetry, batching and determinism.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from gpu_util import TORCH_DT, announce, f64, require_gpu

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-4}


def _input(rows, cols, io, seed, batch=1, noise=1.0, spike=0):
    return S.small_case(rows, cols, io, seed, batch=batch, noise_std=noise, spike_rank=spike)


# --------------------------------------------------------------- syrk_xxt --

SYRK_SHAPES = [(1, 8), (16, 64), (17, 33), (100, 300), (129, 257), (256, 512), (300, 64)]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n,k", SYRK_SHAPES)
def test_syrk_matches_exact_product(dt, n, k):
    M = require_gpu()
    announce(f"syrk n={n} k={k} dt={dt}")
    x = _input(n, k, dt, 500 + n + k, batch=2)
    c = M.syrk_xxt(x.cuda())
    torch.cuda.synchronize()
    cc = f64(c)
    xx = f64(x)
    ref = xx @ np.swapaxes(xx, -1, -2)
    absx = np.abs(xx)
    scale = absx @ np.swapaxes(absx, -1, -2)
    u = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -23}[dt]
    bound = scale * (u + 2 * k * 2.0 ** -24) + 1e-30
    assert np.all(np.abs(cc - ref) <= bound), float(np.max(np.abs(cc - ref) / bound))
    ct = c.transpose(-1, -2).contiguous()
    assert torch.equal(c, ct), "C must be bitwise symmetric"


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_syrk_fused_epilogue(dt):
    M = require_gpu()
    announce(f"syrk epilogue dt={dt}")
    n, k = 200, 136
    x = _input(n, k, dt, 42)
    d0 = _input(n, n, dt, 43)
    d = ((d0 + d0.transpose(-1, -2)) * 0.5).to(TORCH_DT[dt])  # symmetric
    alpha, beta, gamma = 0.75, -1.5, 2.25
    c = M.syrk_xxt(x.cuda(), alpha=alpha, d=d.cuda(), beta=beta, gamma=gamma)
    torch.cuda.synchronize()
    xx, dd = f64(x)[0], f64(d)[0]
    ref = alpha * xx @ xx.T + beta * dd + gamma * np.eye(n)
    scale = abs(alpha) * np.abs(xx) @ np.abs(xx).T + abs(beta) * np.abs(dd) + abs(gamma)
    u = {"bf16": 2.0 ** -8, "f32": 2.0 ** -22}[dt]
    assert np.all(np.abs(f64(c)[0] - ref) <= scale * (u + 2 * k * 2.0 ** -24))
    assert torch.equal(c, c.transpose(-1, -2).contiguous())


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_syrk_fused_epilogue_big_tiles(dt):
    """C = alpha X X^T + beta D + gamma I on 256 x 256 tiles (5800 x 5800:
    276 triangle tiles, the last row and column ragged), so the staged
    epilogue of the off-diagonal tiles adds D loaded ahead of its stores, in
    each D dtype; element-wise within the product's error bound, bitwise
    symmetric."""
    M = require_gpu()
    announce(f"syrk epilogue 256-tiles dt={dt}")
    n, k = 5800, 320
    x = _input(n, k, dt, 4242)
    d0 = _input(n, n, dt, 4243)
    d = ((d0.float() + d0.float().transpose(-1, -2)) * 0.5).to(TORCH_DT[dt])  # symmetric
    del d0
    alpha, beta, gamma = 0.75, -1.5, 2.25
    c = M.syrk_xxt(x.cuda(), alpha=alpha, d=d.cuda(), beta=beta, gamma=gamma)
    torch.cuda.synchronize()
    xx, dd = f64(x)[0], f64(d)[0]
    ref = alpha * (xx @ xx.T) + beta * dd + gamma * np.eye(n)
    ax = np.abs(xx)
    scale = abs(alpha) * (ax @ ax.T) + abs(beta) * np.abs(dd) + abs(gamma)
    u = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -22}[dt]
    err = np.abs(f64(c)[0] - ref) / (scale * (u + 2 * k * 2.0 ** -24))
    assert float(err.max()) <= 1.0, float(err.max())
    assert torch.equal(c, c.transpose(-1, -2).contiguous()), "C must be bitwise symmetric"


@pytest.mark.parametrize("n,k,batch", [(100, 300, 2), (1536, 1024, 2), (2048, 2048, 4)])
def test_syrk_full_tiles_comparator(n, k, batch):
    """The full-tile comparator (every tile of X X^T, the three tile tiers)
    within the product's error bound, and equal to the triangle kernel's
    result up to the same bound."""
    M = require_gpu()
    announce(f"syrk full tiles n={n} k={k} batch={batch}")
    x = _input(n, k, "bf16", 600 + n, batch=batch)
    xc = x.cuda()
    c = M.syrk_xxt(xc, full_tiles=True)
    t = M.syrk_xxt(xc)
    torch.cuda.synchronize()
    for i in sorted({0, batch - 1}):
        xx = f64(x[i])
        ref = xx @ xx.T
        scale = np.abs(xx) @ np.abs(xx).T
        bound = scale * (2.0 ** -8 + 2 * k * 2.0 ** -24)
        assert np.all(np.abs(f64(c[i]) - ref) <= bound)
        assert np.all(np.abs(f64(c[i]) - f64(t[i])) <= 2 * bound)


def test_syrk_deterministic_and_batched_matches_single():
    M = require_gpu()
    announce("syrk determinism")
    x = _input(384, 1000, "bf16", 7, batch=3).cuda()
    c1 = M.syrk_xxt(x)
    c2 = M.syrk_xxt(x)
    c_single = M.syrk_xxt(x[1:2].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    # the K split of the last round of tiles depends on the launch (batch
    # size), so fp32 sums may round differently: both sit within the
    # product's error bound of the exact value, hence within twice it of
    # each other
    xx = f64(x[1])
    scale = np.abs(xx) @ np.abs(xx).T
    bound = scale * (2.0 ** -8 + 2 * 1000 * 2.0 ** -24)
    assert np.all(np.abs(f64(c1[1]) - f64(c_single[0])) <= 2 * bound)


def test_syrk_empty_k_gives_beta_d_plus_gamma():
    M = require_gpu()
    announce("syrk k=0")
    x = torch.empty((1, 5, 0), dtype=torch.float32, device="cuda")
    d = torch.eye(5, device="cuda").reshape(1, 5, 5) * 3
    c = M.syrk_xxt(x, d=d, beta=2.0, gamma=1.0)
    torch.cuda.synchronize()
    assert torch.equal(c.cpu(), torch.eye(5).reshape(1, 5, 5) * 7)


# ------------------------------------------------------------------ msign_ns --

NS_CASES = [
    # rows, cols, io, compute, batch
    (128, 256, "f32", "f32", 1),    # the small fp32 workload
    (128, 256, "f32", "bf16", 1),
    (200, 70, "bf16", "bf16", 2),   # tall, ragged
    (70, 200, "bf16", "bf16", 2),   # wide, ragged
    (129, 129, "bf16", "f16", 1),   # square, ragged tail
    (1, 37, "bf16", "bf16", 1),     # a vector (n <= 64: fp32 products)
    (1, 37, "bf16", "f16", 1),
    (37, 1, "f16", "f16", 1),
    (37, 1, "bf16", "bf16", 2),
    (64, 300, "bf16", "bf16", 2),   # n = 64, the largest fp32-product size
    (65, 300, "bf16", "bf16", 1),   # n = 65, the smallest bf16-product size
    (96, 160, "f16", "bf16", 3),
    (300, 520, "f32", "f32", 1),
    (100, 130, "f32", "f32", 2),    # fp32 products, ragged both ways
    (256, 128, "f32", "f32", 1),    # fp32 products, tall
]


@pytest.mark.parametrize("rows,cols,io,cdt,batch", NS_CASES)
def test_ns_matches_oracle(rows, cols, io, cdt, batch):
    M = require_gpu()
    announce(f"msign_ns {batch}x{rows}x{cols} io={io} compute={cdt}")
    x = _input(rows, cols, io, 1000 + rows * 7 + cols, batch=batch)
    y = M.msign_ns(x.cuda(), compute_dtype=TORCH_DT[cdt])
    torch.cuda.synchronize()
    assert y.shape == x.shape and y.dtype == x.dtype
    err = O.max_rel_fro_error(f64(y), O.ns(f64(x)))
    assert err <= TOL[cdt], err


def test_ns_tiny_n_runs_fp32_products():
    """n <= 64 runs its products in fp32 whatever compute_dtype: a bf16 call
    gives the bits of the fp32 call, in a grouped call too (its own sub-call
    next to the bf16 group), and reaches the fp32 tolerance before the
    output's own bf16 rounding."""
    M = require_gpu()
    announce("msign_ns n <= 64 fp32 products")
    x = _input(48, 200, "f32", 4711, batch=2)
    big = _input(96, 200, "f32", 4712, batch=1)
    y_bf = M.msign_ns(x.cuda(), compute_dtype=torch.bfloat16)
    y_32 = M.msign_ns(x.cuda(), compute_dtype=torch.float32)
    y_grp, y_big = M.msign_ns_grouped([x.cuda(), big.cuda()], compute_dtype=torch.bfloat16)
    y_big1 = M.msign_ns(big.cuda(), compute_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y_bf, y_32)
    assert torch.equal(y_grp, y_32)
    assert torch.equal(y_big, y_big1)
    assert O.max_rel_fro_error(f64(y_bf), O.ns(f64(x))) <= 1e-4


@pytest.mark.parametrize("rows,cols,batch,cdt", [
    (160, 352, 2, "bf16"),     # 64 x 64 tiles
    (1536, 1536, 2, "bf16"),   # 128 x 128 tiles
    (2048, 2048, 4, "bf16"),   # 256 x 256 tiles
    (200, 96, 1, "f32"),       # tall, fp32 products
])
def test_ns_dense_products_comparator(rows, cols, batch, cdt):
    """NS with X X^T and c A A + b A on every tile (the measurement
    comparator of the triangle products) matches the oracle like the
    symmetric path does."""
    M = require_gpu()
    announce(f"msign_ns dense products {batch}x{rows}x{cols} compute={cdt}")
    x = _input(rows, cols, "f32" if cdt == "f32" else "bf16", 700 + rows, batch=batch)
    y = M.msign_ns(x.cuda(), compute_dtype=TORCH_DT[cdt], dense_products=True)
    torch.cuda.synchronize()
    for i in sorted({0, batch - 1}):
        err = O.max_rel_fro_error(f64(y[i]), O.ns(f64(x[i])))
        assert err <= TOL[cdt], (i, err)


# 64 < n <= 128 and m <= 256 (padded) with 16-bit products: the whole
# iteration in one launch, one workgroup per matrix (timing class "small").
SMALL_CASES = [
    # rows, cols, io, compute, batch, table
    (128, 256, "f32", "bf16", 1, None),     # the 128 x 256 workload in bf16 products
    (128, 256, "bf16", "bf16", 3, None),
    (256, 128, "bf16", "bf16", 2, None),    # tall
    (100, 130, "f16", "f16", 2, None),      # ragged both ways
    (65, 250, "f32", "f16", 1, None),       # smallest n of the kernel
    (120, 192, "bf16", "bf16", 1, "T6"),    # per-step table, T = 6
    (96, 160, "bf16", "bf16", 2, "cubic"),  # c = 0 steps
    (110, 200, "bf16", "bf16", 1, "T1"),
]


@pytest.mark.parametrize("rows,cols,io,cdt,batch,table", SMALL_CASES)
def test_ns_small_matrix_kernel(rows, cols, io, cdt, batch, table):
    M = require_gpu()
    announce(f"msign_ns small kernel {batch}x{rows}x{cols} io={io} compute={cdt} table={table}")
    x = _input(rows, cols, io, 1500 + rows + cols, batch=batch, spike=2)
    coeffs, steps = None, 5
    if table == "T6":
        coeffs = (np.array([[3955, -8306, 5008], [3735, -6681, 3463], [3799, -6499, 3211],
                            [4019, -6385, 2906], [2677, -3029, 1162], [2172, -1833, 682]]) / 1024.0)
        steps = 6
    elif table == "cubic":
        coeffs, steps = np.array([[1.5, -0.5, 0.0]] * 8), 8
    elif table == "T1":
        steps = 1
    M.kernel_timing(True)
    y = M.msign_ns(x.cuda(), steps=steps, coeffs=None if coeffs is None else coeffs.tolist(),
                   compute_dtype=TORCH_DT[cdt])
    y2 = M.msign_ns(x.cuda(), steps=steps, coeffs=None if coeffs is None else coeffs.tolist(),
                    compute_dtype=TORCH_DT[cdt])
    torch.cuda.synchronize()
    counts = M.read_kernel_timing()
    M.kernel_timing(False)
    assert counts["small"][1] == 2 and counts["rect"][1] == 0, counts
    assert torch.equal(y, y2)
    ref = O.ns(f64(x), coeffs=coeffs, steps=steps)
    err = O.max_rel_fro_error(f64(y), ref)
    assert err <= TOL[cdt], err


# Wide inputs already in the compute dtype with cols a multiple of 64: the
# first products read the input itself, the normalisation applied as
# per-matrix factors in their epilogues.  Ragged n exercises the row bounds
# of those reads (K-major rows past n, D rows past n).
DIRECT_CASES = [
    # rows, cols, dtype, batch
    (100, 256, "bf16", 3),
    (300, 640, "f16", 1),
    (2000, 4096, "bf16", 1),    # 256 x 256 tiles, ragged last tile row
    (64, 128, "f32", 2),
    (96, 192, "f32", 1),
]


@pytest.mark.parametrize("rows,cols,dt,batch", DIRECT_CASES)
def test_ns_direct_first_step(rows, cols, dt, batch):
    M = require_gpu()
    announce(f"msign_ns direct first step {batch}x{rows}x{cols} {dt}")
    x = _input(rows, cols, dt, 800 + rows, batch=batch, spike=2)
    y = M.msign_ns(x.cuda(), compute_dtype=TORCH_DT[dt])
    torch.cuda.synchronize()
    for i in sorted({0, batch - 1}):
        err = O.max_rel_fro_error(f64(y[i]), O.ns(f64(x[i])))
        assert err <= TOL[dt], (i, err)


@pytest.mark.parametrize("rows,cols,restarts", [(96, 448, (2,)), (130, 256, ()), (200, 1024, (1, 3))])
def test_gram_direct_first_step(rows, cols, restarts):
    M = require_gpu()
    announce(f"msign_gram_ns direct first step {rows}x{cols} f16 restarts={restarts}")
    x = _input(rows, cols, "f16", 900 + rows, batch=2, spike=2)
    y = M.msign_gram_ns(x.cuda(), compute_dtype=torch.float16, restart_after=restarts)
    torch.cuda.synchronize()
    err = O.max_rel_fro_error(f64(y), O.ns(f64(x)))
    assert err <= 2e-2, err


def test_ns_small_fp32_workload_against_exact_and_oracle():
    """The 128x256 fp32 workload: fp32 products match oracle NS to 1e-4, and
    the oracle itself sits within the pages' bound of the exact U V^T."""
    M = require_gpu()
    gr = S.WORKLOADS["c1_128x256_f32"].groups[0]
    announce("msign_ns 128x256 f32 workload")
    x = S.group_batch(gr)
    y = f64(M.msign_ns(x.cuda(), compute_dtype=torch.float32))
    xs = f64(x)
    assert O.max_rel_fro_error(y, O.ns(xs)) <= 1e-4
    s = np.linalg.svd(xs[0], compute_uv=False)
    bound = float(np.max(np.abs(O.phi(s / np.linalg.norm(s)) - 1)))
    assert O.max_rel_fro_error(y, O.exact_msign(xs)) <= bound + 1e-4


@pytest.mark.parametrize("cdt,tol", [("f32", 1e-4), ("bf16", 2e-2)])
def test_ns_cubic_steps_skip_the_square(cdt, tol):
    """c_t = 0 steps (nil9.net's third-order tables) take the path without
    A A: parity with the oracle, and the A^2 class is launched once per
    quintic step only."""
    M = require_gpu()
    announce(f"msign_ns cubic and mixed tables compute={cdt}")
    # fp32 compute is checked with fp32 input and output (a bf16 output alone
    # carries ~2^-9 relative rounding)
    x = _input(192, 448, "f32" if cdt == "f32" else "bf16", 91, batch=2)
    cubic = [[1.5, -0.5, 0.0]] * 8
    mixed = [[3.4445, -4.7750, 2.0315]] * 3 + [[1.99, -0.99, 0.0]] * 2 + [[1.5, -0.5, 0.0]]
    for table in (cubic, mixed):
        M.kernel_timing(True)
        y = M.msign_ns(x.cuda(), steps=len(table), coeffs=table, compute_dtype=TORCH_DT[cdt])
        torch.cuda.synchronize()
        counts = M.read_kernel_timing()
        M.kernel_timing(False)
        err = O.max_rel_fro_error(f64(y), O.ns(f64(x), coeffs=np.array(table), steps=len(table)))
        assert err <= tol, err
        quintic = sum(1 for r in table if r[2] != 0.0)
        assert counts["square"][1] == quintic
        assert counts["rect"][1] == len(table)


@pytest.mark.parametrize("rows,cols,batch,cdt,tol", [
    (160, 352, 2, "f32", 1e-4),     # 64x64 tiles
    (352, 96, 3, "f32", 1e-4),      # tall input
    (1024, 4096, 1, "bf16", 2e-2),  # 1024x4096 spiked-workload shape
    (2048, 2048, 8, "bf16", 2e-2),  # 256x256 tiles with a K-split last round
])
def test_ns_improved_init(rows, cols, batch, cdt, tol):
    """The improved initial normalisation ("msign算子的Newton-Schulz迭代（上）"
    §改良初值) against the oracle's version of it; sampled matrices of the
    8-matrix batch."""
    M = require_gpu()
    announce(f"msign_ns improved init {batch}x{rows}x{cols} compute={cdt}")
    x = _input(rows, cols, "f32" if cdt == "f32" else "bf16", 300 + rows, batch=batch)
    y = M.msign_ns(x.cuda(), compute_dtype=TORCH_DT[cdt], improved_init=True)
    y_plain = M.msign_ns(x.cuda(), compute_dtype=TORCH_DT[cdt])
    y_again = M.msign_ns(x.cuda(), compute_dtype=TORCH_DT[cdt], improved_init=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y_again)
    for i in sorted({0, batch - 1}):
        ref = O.ns_improved_init(f64(x[i]))
        err = O.max_rel_fro_error(f64(y[i]), ref)
        assert err <= tol
        # the extra division changes the result (s < 1 strictly for rank > 1):
        # the plain iteration is much further from this reference
        assert O.max_rel_fro_error(f64(y_plain[i]), ref) > 2 * max(err, tol / 10)


@pytest.mark.parametrize("where", ["first", "every"])
@pytest.mark.parametrize("method,io,cdt,tol", [("ns", "bf16", "bf16", 2e-2), ("ns", "f32", "f32", 1e-4),
                                               ("gram", "bf16", "f16", 2e-2)])
def test_safety_factor_as_scaled_coefficients(where, method, io, cdt, tol):
    """The safety factor of "Gram Newton-Schulz" §3.3 (formula lost in the
    text) in either plain reading is a per-step table with rows
    (a / s, b / s^3, c / s^5): the first row (X_0 divided by s) or every row.
    The library takes it as any other table; checked against the oracle."""
    M = require_gpu()
    announce(f"safety factor {where} {method} {cdt}")
    s = 1.05
    a, b, c = O.KELLER_ABC
    scaled = [a / s, b / s ** 3, c / s ** 5]
    table = [scaled] + [[a, b, c]] * 4 if where == "first" else [scaled] * 5
    x = _input(192, 640, io, 808, batch=2, noise=0.02, spike=4)
    if method == "ns":
        y = M.msign_ns(x.cuda(), steps=5, coeffs=table, compute_dtype=TORCH_DT[cdt])
    else:
        y = M.msign_gram_ns(x.cuda(), steps=5, coeffs=table, compute_dtype=TORCH_DT[cdt], restart_after=(2,))
    torch.cuda.synchronize()
    ref = O.ns(f64(x), coeffs=np.array(table), steps=5)
    err = O.max_rel_fro_error(f64(y), ref)
    assert err <= tol, err
    # the result follows the table: the plain iteration is much further away
    assert O.max_rel_fro_error(f64(y), O.ns(f64(x))) > 2 * err


def test_ns_improved_init_with_cubic_first_step():
    M = require_gpu()
    announce("msign_ns improved init, cubic table")
    x = _input(128, 320, "f32", 404, batch=2)
    table = [[1.5, -0.5, 0.0]] * 6
    y = M.msign_ns(x.cuda(), steps=6, coeffs=table, compute_dtype=torch.float32, improved_init=True)
    torch.cuda.synchronize()
    ref = O.ns_improved_init(f64(x), coeffs=np.array(table), steps=6)
    assert O.max_rel_fro_error(f64(y), ref) <= 1e-4


@pytest.mark.parametrize("cdt", ["bf16", "f16"])
def test_ns_spiked_alpha4_workload(cdt):
    """1024x4096 bf16, N(0, 0.02^2) + rank-8 spike (full size)."""
    M = require_gpu()
    gr = S.WORKLOADS["c2_1024x4096_bf16"].groups[0]
    announce(f"msign_ns 1024x4096 spiked compute={cdt}")
    x = S.group_batch(gr)
    y = M.msign_ns(x.cuda(), compute_dtype=TORCH_DT[cdt])
    torch.cuda.synchronize()
    err = O.max_rel_fro_error(f64(y), O.ns(f64(x)))
    assert err <= 2e-2, err


def test_ns_per_step_coefficients_and_steps():
    M = require_gpu()
    announce("msign_ns per-step table T=6")
    table = np.array([[3955, -8306, 5008], [3735, -6681, 3463], [3799, -6499, 3211],
                      [4019, -6385, 2906], [2677, -3029, 1162], [2172, -1833, 682]]) / 1024.0
    x = _input(160, 352, "f32", 77)
    y = M.msign_ns(x.cuda(), steps=6, coeffs=table.tolist(), compute_dtype=torch.float32)
    torch.cuda.synchronize()
    assert O.max_rel_fro_error(f64(y), O.ns(f64(x), coeffs=table, steps=6)) <= 1e-4
    y1 = M.msign_ns(x.cuda(), steps=1, compute_dtype=torch.float32)
    torch.cuda.synchronize()
    assert O.max_rel_fro_error(f64(y1), O.ns(f64(x), steps=1)) <= 1e-4


def test_ns_bitwise_invariants():
    M = require_gpu()
    announce("msign_ns invariants")
    x = _input(192, 320, "bf16", 5, batch=4).cuda()
    y = M.msign_ns(x)
    y_again = M.msign_ns(x)
    y_one = M.msign_ns(x[2:3].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y, y_again), "run to run"
    # K = 320 is too short for any launch of this problem to be split along
    # K, so the batch size changes nothing a matrix sees: the same bits
    assert torch.equal(y[2:3], y_one), "batched vs single"
    z = M.msign_ns(torch.zeros_like(x))
    torch.cuda.synchronize()
    assert torch.count_nonzero(z).item() == 0
    # in place
    xc = x.clone()
    M.msign_ns(xc, out=xc)
    torch.cuda.synchronize()
    assert torch.equal(xc, y)


def test_ns_batched_vs_single_with_different_k_splits():
    """2 x 2048^2 against the first matrix alone: the launches split their
    last round of tiles along K 3 ways for the pair and 7 ways for one
    matrix, so some fp32 sums are added in another order.  That flips some
    bf16 roundings of A, B and X, and the iteration carries those like any
    other rounding: the two results are two equally valid roundings of the
    same iteration.  Both must meet the oracle tolerance, and their
    difference must be no larger than two independent draws of their own
    rounding error give (1.5 sqrt(e1^2 + e2^2); much of it is shared, since
    most tiles are computed the same way in both)."""
    M = require_gpu()
    announce("msign_ns 2x2048^2 batched vs single (different K splits)")
    x = _input(2048, 2048, "bf16", 1234, batch=2, spike=4).cuda()
    y = M.msign_ns(x)
    y1 = M.msign_ns(x[0:1].contiguous())
    torch.cuda.synchronize()
    ref = O.ns(f64(x[0:1].cpu()))
    e_b = O.max_rel_fro_error(f64(y[0:1]), ref)
    e_s = O.max_rel_fro_error(f64(y1), ref)
    drift = O.max_rel_fro_error(f64(y[0:1]), f64(y1))
    print(f"[parity] 2048^2 batched vs single: drift {drift:.3e}, errors {e_b:.3e} / {e_s:.3e}", flush=True)
    assert e_b <= 2e-2 and e_s <= 2e-2, (e_b, e_s)
    assert drift <= 1.5 * math.sqrt(e_b ** 2 + e_s ** 2), (drift, e_b, e_s)


def test_ns_transpose_and_scale():
    M = require_gpu()
    announce("msign_ns transpose/scale")
    x = _input(96, 224, "f32", 9)
    y = f64(M.msign_ns(x.cuda(), compute_dtype=torch.float32))
    yt = f64(M.msign_ns(x.transpose(-1, -2).contiguous().cuda(), compute_dtype=torch.float32))
    ys = f64(M.msign_ns((x * 1024).cuda(), compute_dtype=torch.float32))
    assert np.max(np.abs(yt - np.swapaxes(y, -1, -2))) <= 1e-5
    assert np.max(np.abs(ys - y)) <= 1e-5


def test_ns_nan_propagates():
    M = require_gpu()
    announce("msign_ns NaN input")
    x = _input(64, 128, "bf16", 3)
    x[0, 5, 7] = float("nan")
    y = M.msign_ns(x.cuda())
    torch.cuda.synchronize()
    assert torch.isnan(y).any().item()


def test_ns_empty_batch():
    M = require_gpu()
    x = torch.empty((0, 64, 128), dtype=torch.bfloat16, device="cuda")
    assert M.msign_ns(x).shape == x.shape


# ------------------------------------------------------------- msign_gram_ns --

GRAM_CASES = [
    # rows, cols, io, compute, restarts, batch
    (128, 256, "f32", "f32", (2,), 1),
    (128, 256, "f32", "f32", (), 1),
    (128, 256, "f32", "f32", (1, 2, 3, 4), 1),
    (96, 400, "bf16", "f16", (2,), 2),
    (400, 96, "bf16", "f16", (2,), 2),     # tall
    (130, 260, "f16", "f16", (), 1),
    (130, 260, "bf16", "bf16", (2,), 1),
    (1, 40, "f16", "f16", (2,), 1),
    (1, 40, "bf16", "bf16", (2,), 1),    # n <= 64: fp32 products
    (40, 1, "bf16", "bf16", (), 2),
]


@pytest.mark.parametrize("rows,cols,io,cdt,restarts,batch", GRAM_CASES)
def test_gram_matches_oracle_ns(rows, cols, io, cdt, restarts, batch):
    M = require_gpu()
    announce(f"msign_gram_ns {batch}x{rows}x{cols} io={io} compute={cdt} restarts={restarts}")
    x = _input(rows, cols, io, 2000 + rows + cols, batch=batch)
    y = M.msign_gram_ns(x.cuda(), compute_dtype=TORCH_DT[cdt], restart_after=restarts)
    torch.cuda.synchronize()
    xs = f64(x)
    err = O.max_rel_fro_error(f64(y), O.ns(xs))
    assert err <= TOL[cdt], err
    # the oracle's own Gram form agrees with its NS (the pages' equivalence)
    assert O.max_rel_fro_error(O.gram_ns(xs, restart_after=restarts), O.ns(xs)) <= 1e-10


def test_gram_spiked_alpha4_workload_fp16():
    M = require_gpu()
    gr = S.WORKLOADS["c2_1024x4096_bf16"].groups[0]
    announce("msign_gram_ns 1024x4096 spiked fp16 restart {2}")
    x = S.group_batch(gr)
    y = M.msign_gram_ns(x.cuda(), compute_dtype=torch.float16, restart_after=(2,))
    torch.cuda.synchronize()
    err = O.max_rel_fro_error(f64(y), O.ns(f64(x)))
    assert err <= 2e-2, err


def test_gram_bitwise_invariants():
    M = require_gpu()
    announce("msign_gram_ns invariants")
    x = _input(160, 480, "f16", 11, batch=3).cuda()
    y = M.msign_gram_ns(x)
    y2 = M.msign_gram_ns(x)
    y1 = M.msign_gram_ns(x[1:2].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(y[1:2], y1)
    z = M.msign_gram_ns(torch.zeros_like(x))
    torch.cuda.synchronize()
    assert torch.count_nonzero(z).item() == 0
