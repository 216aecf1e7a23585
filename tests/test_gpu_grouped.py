"""Grouped calls on the GPU: msign over several shape groups at once, each
product of the iteration one launch over the tiles of every group.

Each group must match the fp64 oracle to the same tolerance as a call on
its own (2e-2 for bf16/fp16 products, 1e-4 for fp32), and agree closely with
that call (the K split of a launch's last round depends on all its groups,
so the last bits may differ).  Cases mix wide, tall and ragged shapes, batch
sizes, an empty group, and sizes where grouping changes the tile size that
a group alone would get.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from gpu_util import TORCH_DT, announce, block_error_ratio, f64, require_gpu

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-4}


def _inputs(shapes, io, seed):
    return [S.small_case(r, c, io, seed + 17 * i, batch=b, noise_std=1.0, spike_rank=2)
            for i, (b, r, c) in enumerate(shapes)]


def _check_groups(ys, xs, ref_fn, tol, sample=None):
    for y, x in zip(ys, xs):
        assert y.shape == x.shape and y.dtype == x.dtype
        if x.numel() == 0:
            continue
        idx = range(x.shape[0]) if sample is None else sorted({0, x.shape[0] - 1})
        for i in idx:
            ref = ref_fn(f64(x[i]))
            err = O.max_rel_fro_error(f64(y[i]), ref)
            assert err <= tol, (tuple(x.shape), i, err)
            # tile-local: no 256 x 256 tile above 3x its share of the bound
            blk = block_error_ratio(f64(y[i]), ref)
            assert blk <= 3 * tol, (tuple(x.shape), i, blk)


NS_GROUPS = [
    # groups (batch, rows, cols), io, compute
    ([(2, 128, 256), (1, 300, 70), (3, 64, 100)], "bf16", "bf16"),
    ([(1, 96, 400), (2, 400, 96)], "f16", "f16"),
    ([(1, 128, 256), (2, 160, 352), (1, 352, 96), (1, 1, 37)], "f32", "f32"),
    ([(2, 200, 70), (0, 64, 64), (1, 70, 200)], "bf16", "bf16"),  # an empty group
]


@pytest.mark.parametrize("shapes,io,cdt", NS_GROUPS)
def test_ns_grouped_matches_oracle_and_single_calls(shapes, io, cdt):
    M = require_gpu()
    announce(f"msign_ns_grouped {shapes} io={io} compute={cdt}")
    xs = _inputs(shapes, io, 4000)
    ys = M.msign_ns_grouped([x.cuda() for x in xs], compute_dtype=TORCH_DT[cdt])
    ys_again = M.msign_ns_grouped([x.cuda() for x in xs], compute_dtype=TORCH_DT[cdt])
    singles = [M.msign_ns(x.cuda(), compute_dtype=TORCH_DT[cdt]) for x in xs]
    torch.cuda.synchronize()
    _check_groups(ys, xs, O.ns, TOL[cdt])
    for y, y2, s in zip(ys, ys_again, singles):
        assert torch.equal(y, y2), "grouped calls must be bit-stable"
        if y.numel():
            assert O.max_rel_fro_error(f64(y), f64(s)) <= TOL[cdt] / 2


GRAM_GROUPS = [
    ([(2, 96, 400), (1, 400, 96), (1, 130, 260)], "bf16", "f16", (2,)),
    ([(1, 128, 256), (2, 64, 300)], "f32", "f32", (2,)),
    ([(1, 130, 260), (2, 70, 140)], "f16", "f16", ()),
]


@pytest.mark.parametrize("shapes,io,cdt,restarts", GRAM_GROUPS)
def test_gram_grouped_matches_oracle(shapes, io, cdt, restarts):
    M = require_gpu()
    announce(f"msign_gram_ns_grouped {shapes} io={io} compute={cdt} restarts={restarts}")
    xs = _inputs(shapes, io, 5000)
    ys = M.msign_gram_ns_grouped([x.cuda() for x in xs], compute_dtype=TORCH_DT[cdt],
                                 restart_after=restarts)
    singles = [M.msign_gram_ns(x.cuda(), compute_dtype=TORCH_DT[cdt], restart_after=restarts)
               for x in xs]
    torch.cuda.synchronize()
    _check_groups(ys, xs, O.ns, TOL[cdt])
    for y, s in zip(ys, singles):
        assert O.max_rel_fro_error(f64(y), f64(s)) <= TOL[cdt] / 2


def test_ns_grouped_improved_init():
    M = require_gpu()
    shapes = [(2, 160, 352), (1, 352, 96)]
    announce(f"msign_ns_grouped improved init {shapes}")
    xs = _inputs(shapes, "f32", 6000)
    ys = M.msign_ns_grouped([x.cuda() for x in xs], compute_dtype=torch.float32, improved_init=True)
    torch.cuda.synchronize()
    _check_groups(ys, xs, O.ns_improved_init, 1e-4)


def test_grouping_changes_tiles_not_results():
    """4 x 1024^2 alone runs on 128 x 128 tiles (40 big tiles); grouped with
    8 x 2048 x 4096 the launches use 256 x 256 tiles and the split of the
    last round falls in the square group.  Sampled matrices of both groups
    against the oracle."""
    M = require_gpu()
    shapes = [(4, 1024, 1024), (8, 2048, 4096)]
    announce(f"msign_ns_grouped tiers {shapes}")
    xs = _inputs(shapes, "bf16", 7000)
    ys = M.msign_ns_grouped([x.cuda() for x in xs], compute_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check_groups(ys, xs, O.ns, 2e-2, sample=True)


def test_gram_grouped_moe_shapes_sampled():
    """The MoE-expert shape groups at reduced batch: 4 x 2048 x 7168 and
    2 x 1024 x 8192, fp16 Gram with restart after step 2."""
    M = require_gpu()
    shapes = [(4, 2048, 7168), (2, 1024, 8192)]
    announce(f"msign_gram_ns_grouped {shapes}")
    xs = _inputs(shapes, "f16", 8000)
    ys = M.msign_gram_ns_grouped([x.cuda() for x in xs], compute_dtype=torch.float16, restart_after=(2,))
    torch.cuda.synchronize()
    _check_groups(ys, xs, O.ns, 2e-2, sample=True)


def test_grouped_rejects_mixed_dtypes():
    M = require_gpu()
    a = torch.zeros(2, 8, 16, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(2, 8, 16, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        M.msign_ns_grouped([a, b])
    with pytest.raises(ValueError):
        M.msign_ns_grouped([a] * 5)


@pytest.mark.parametrize("trial", range(6))
def test_grouped_random_shapes(trial):
    """Seeded random groupings: 2-4 groups, batches 1-3, ragged sizes from
    1 to 700 on either side (wide, tall, vectors), NS and Gram alternately.
    Gram trials draw aspect ratios >= 2 (the method's regime; it squares
    the condition number)."""
    M = require_gpu()
    rng = np.random.default_rng(9000 + trial)
    ng = int(rng.integers(2, 5))
    gram = trial % 2 == 1
    shapes = []
    for _ in range(ng):
        b = int(rng.integers(1, 4))
        if gram:
            n = int(rng.integers(1, 300))
            m = 2 * n + int(rng.integers(0, 300))
            shapes.append((b, n, m) if rng.integers(0, 2) else (b, m, n))
        else:
            shapes.append((b, int(rng.integers(1, 701)), int(rng.integers(1, 701))))
    announce(f"grouped random trial {trial}: {'gram' if gram else 'ns'} {shapes}")
    xs = _inputs(shapes, "f32", 9100 + 10 * trial)
    if gram:
        ys = M.msign_gram_ns_grouped([x.cuda() for x in xs], compute_dtype=torch.float32)
    else:
        ys = M.msign_ns_grouped([x.cuda() for x in xs], compute_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_groups(ys, xs, O.ns, 1e-4)
