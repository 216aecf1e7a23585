"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (a single batched call, or one grouped call over the shape
groups of a workload).  The fp64 oracle
runs on sampled matrices of each batch (first and last), one at a time.
BLAS threads are capped at 16 (one GPU's share of the host)."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from gpu_util import announce, block_error_ratio, f64, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _blas_threads():
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        yield
        return
    with threadpool_limits(limits=16):
        yield


def _run_group(M, gr, method, cdt):
    x = S.group_batch(gr, device="cuda")
    if method == "ns":
        y = M.msign_ns(x, compute_dtype=cdt)
    else:
        y = M.msign_gram_ns(x, compute_dtype=cdt, restart_after=(2,))
    torch.cuda.synchronize()
    return x, y


# Tile-local bound next to the whole-matrix contract: no 256 x 256 tile may
# carry more than BLOCK_FACTOR times its even share of the contract's error.
BLOCK_FACTOR = 3.0


def _check_one(y, ref, tol, label):
    err = O.max_rel_fro_error(y[None], ref[None])
    blk = block_error_ratio(y, ref)
    print(f"[parity] {label}: rel fro {err:.3e}, worst 256-tile {blk:.3e}", flush=True)
    assert err <= tol, (label, err)
    assert blk <= BLOCK_FACTOR * tol, (label, blk)


def _check_samples(x, y, tol, label):
    for i in sorted({0, x.shape[0] - 1}):
        announce(f"{label}: oracle on matrix {i}")
        _check_one(f64(y[i]), O.ns_single(f64(x[i])), tol, f"{label} matrix {i}")


@pytest.mark.timeout(900)
def test_square_8192_ns_bf16():
    M = require_gpu()
    gr = S.WORKLOADS["c3_8192x8192_bf16"].groups[0]
    announce("msign_ns 8192x8192 bf16")
    x, y = _run_group(M, gr, "ns", torch.bfloat16)
    y2 = M.msign_ns(x, compute_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "bit-stable run to run"
    _check_samples(x, y, 2e-2, "8192^2 ns")


@pytest.mark.timeout(900)
def test_square_8192_ns_improved_init_bf16():
    """The benchmark's improved-initial-normalisation case at full size,
    against the oracle's version of it."""
    M = require_gpu()
    gr = S.WORKLOADS["c3_8192x8192_bf16"].groups[0]
    announce("msign_ns improved init 8192x8192 bf16")
    x = S.group_batch(gr, device="cuda")
    y = M.msign_ns(x, compute_dtype=torch.bfloat16, improved_init=True)
    torch.cuda.synchronize()
    announce("8192^2 improved init: oracle on matrix 0")
    _check_one(f64(y[0]), O.ns_improved_init_single(f64(x[0])), 2e-2, "8192^2 improved init")


@pytest.mark.timeout(600)
def test_square_8192_syrk_unit():
    M = require_gpu()
    gr = S.WORKLOADS["c3_8192x8192_bf16"].groups[0]
    announce("syrk_xxt 8192x8192 bf16")
    x = S.group_batch(gr, device="cuda")
    c = M.syrk_xxt(x)
    torch.cuda.synchronize()
    assert torch.equal(c, c.transpose(-1, -2).contiguous())
    # rows sampled across the tile grid (first, tile edges, last)
    rows = np.array([0, 1, 255, 256, 4095, 4096, 8191])
    xx = f64(x[0])
    ref = xx[rows] @ xx.T
    got = f64(c[0][torch.as_tensor(rows, device="cuda")])
    scale = np.abs(xx[rows]) @ np.abs(xx).T
    assert np.all(np.abs(got - ref) <= scale * (2.0 ** -8 + 2 * 8192 * 2.0 ** -24))


def _run_grouped(M, workload, method, cdt):
    xs = [S.group_batch(gr, device="cuda") for gr in S.WORKLOADS[workload].groups]
    if method == "ns":
        ys = M.msign_ns_grouped(xs, compute_dtype=cdt)
    else:
        ys = M.msign_gram_ns_grouped(xs, compute_dtype=cdt, restart_after=(2,))
    torch.cuda.synchronize()
    return xs, ys


@pytest.mark.timeout(900)
def test_transformer_block_ns_bf16():
    M = require_gpu()
    announce("msign_ns_grouped block: 16x4096x4096 + 16x14336x4096")
    xs, ys = _run_grouped(M, "c4_block_bf16", "ns", torch.bfloat16)
    for gi, (x, y) in enumerate(zip(xs, ys)):
        _check_samples(x, y, 2e-2, f"block group {gi}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("method,cdt", [("gram", torch.float16), ("ns", torch.bfloat16)])
def test_moe_experts(method, cdt):
    M = require_gpu()
    announce(f"{method} grouped moe: 64x2048x7168 + 8x1024x8192")
    xs, ys = _run_grouped(M, "c5_moe_f16", method, cdt)
    for gi, (x, y) in enumerate(zip(xs, ys)):
        _check_samples(x, y, 2e-2, f"moe {method} group {gi}")


@pytest.mark.timeout(900)
def test_transformer_block_muon_step():
    """One Muon step over the block's two shape groups (the workload as
    gradients, bf16 parameters, fp32 momentum holding a previous step's
    value), checked on sampled matrices against the oracle's muon_step."""
    M = require_gpu()
    announce("muon_step block: 16x4096x4096 + 16x14336x4096")
    gs = [S.group_batch(gr, device="cuda") for gr in S.WORKLOADS["c4_block_bf16"].groups]
    gen = torch.Generator(device="cuda").manual_seed(5)
    ws = [(0.02 * torch.randn(g.shape, generator=gen, device="cuda")).to(torch.bfloat16) for g in gs]
    ms = [0.5 * g.float() for g in gs]
    w0 = [w.clone() for w in ws]
    m0 = [m.clone() for m in ms]
    mu, lr = 0.95, 0.02
    M.muon_step(ws, gs, ms, lr=lr, mu=mu, method="ns", compute_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for gi in range(len(gs)):
        for i in sorted({0, gs[gi].shape[0] - 1}):
            announce(f"muon block group {gi}: oracle on matrix {i}")
            w_ref, m_ref = O.muon_step(f64(w0[gi][i]), f64(gs[gi][i]), f64(m0[gi][i]), mu, lr,
                                       msign=O.ns_single)
            assert np.linalg.norm(f64(ms[gi][i]) - m_ref) <= 1e-6 * np.linalg.norm(m_ref)
            d_ref = f64(w0[gi][i]) - w_ref
            d_gpu = f64(w0[gi][i]) - f64(ws[gi][i])
            bound = 2e-2 * np.linalg.norm(d_ref) + 2.0 ** -9 * np.linalg.norm(w_ref)
            assert np.linalg.norm(d_gpu - d_ref) <= bound, (gi, i)
            # tile-local: the update of no tile may be off by more than its
            # share (W's own bf16 rounding included in the allowance)
            blk = block_error_ratio(d_gpu, d_ref)
            print(f"[parity] muon group {gi} matrix {i}: worst 256-tile {blk:.3e}", flush=True)
            assert blk <= BLOCK_FACTOR * bound / np.linalg.norm(d_ref), (gi, i, blk)


@pytest.mark.timeout(900)
def test_big_tiles_with_ragged_edges():
    """6000 x 6500: 256 x 256 tiles whose last row and column of tiles stick
    out of the matrix (the epilogue's bounds-checked path next to the staged
    one), checked against the oracle; tall input as well."""
    M = require_gpu()
    x = S.small_case(6000, 6500, "bf16", 4242, batch=1, noise_std=1.0, spike_rank=0)
    for label, xi in (("wide", x), ("tall", x.transpose(-1, -2).contiguous())):
        announce(f"msign_ns 6000x6500 {label}")
        y = M.msign_ns(xi.cuda(), compute_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        _check_one(f64(y)[0], O.ns_single(f64(xi)[0]), 2e-2, f"6000x6500 {label}")
