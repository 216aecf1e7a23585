"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (each shape group as one batched call).  The fp64 oracle
runs on sampled matrices of each batch (first and last), one at a time.
BLAS threads are capped at 16 (one GPU's share of the host)."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from gpu_util import announce, f64, require_gpu

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


def _check_samples(x, y, tol, label):
    for i in sorted({0, x.shape[0] - 1}):
        announce(f"{label}: oracle on matrix {i}")
        ref = O.ns_single(f64(x[i]))
        err = O.max_rel_fro_error(f64(y[i])[None], ref[None])
        assert err <= tol, (label, i, err)


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


@pytest.mark.timeout(900)
def test_transformer_block_ns_bf16():
    M = require_gpu()
    for gi, gr in enumerate(S.WORKLOADS["c4_block_bf16"].groups):
        announce(f"msign_ns block group {gi}: {gr.batch}x{gr.rows}x{gr.cols}")
        x, y = _run_group(M, gr, "ns", torch.bfloat16)
        _check_samples(x, y, 2e-2, f"block group {gi}")
        del x, y
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("method,cdt", [("gram", torch.float16), ("ns", torch.bfloat16)])
def test_moe_experts(method, cdt):
    M = require_gpu()
    for gi, gr in enumerate(S.WORKLOADS["c5_moe_f16"].groups):
        announce(f"{method} moe group {gi}: {gr.batch}x{gr.rows}x{gr.cols}")
        x, y = _run_group(M, gr, method, cdt)
        _check_samples(x, y, 2e-2, f"moe {method} group {gi}")
        del x, y
        torch.cuda.empty_cache()


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
        err = O.max_rel_fro_error(f64(y), O.ns(f64(xi)))
        assert err <= 2e-2, (label, err)
