"""Muon steps on the GPU (C ABI `muon_step`) against the fp64 oracle's
`muon_step`: m <- mu m + g, w <- w - lr msign(m), over several parameter
groups of different shapes at once.

Each step of a run is compared with the oracle started from the GPU's own
state before that step, so differences do not accumulate.  Bounds: the
momentum is an fp32 elementwise update (relative error 1e-6); the parameter
change w_old - w_new must match lr msign(m) to the msign tolerance (2e-2 for
bf16/fp16 products, 1e-4 for fp32), plus the one rounding of w to its dtype.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from gpu_util import TORCH_DT, announce, f64, require_gpu

pytestmark = pytest.mark.gpu

UNIT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -9, "f16": 2.0 ** -12}


def _state(shapes, pdt, seed):
    ws, ms = [], []
    for i, (b, r, c) in enumerate(shapes):
        rng = np.random.default_rng(seed + i)
        ws.append(torch.from_numpy(rng.standard_normal((b, r, c)) * 0.02).to(TORCH_DT[pdt]).cuda())
        ms.append(torch.zeros(b, r, c, dtype=torch.float32, device="cuda"))
    return ws, ms


def _grads(shapes, pdt, seed):
    return [S.small_case(r, c, pdt, seed + 31 * i, batch=b, noise_std=1.0, spike_rank=2).cuda()
            for i, (b, r, c) in enumerate(shapes)]


def _run(shapes, pdt, method, cdt, tol, nsteps=3, mu=0.95, lr=0.02, **kw):
    M = require_gpu()
    ws, ms = _state(shapes, pdt, 900)
    msign = (lambda x: O.gram_ns(x, restart_after=kw.get("restart_after", (2,)))) if method == "gram" else (
        O.ns_improved_init if kw.get("improved_init") else O.ns)
    for k in range(nsteps):
        gs = _grads(shapes, pdt, 1000 + 10 * k)
        w0 = [f64(w) for w in ws]
        m0 = [f64(m) for m in ms]
        M.muon_step(ws, gs, ms, lr=lr, mu=mu, method=method, compute_dtype=TORCH_DT[cdt], **kw)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            if ws[i].numel() == 0:
                continue
            w_ref, m_ref = O.muon_step(w0[i], f64(gs[i]), m0[i], mu, lr, msign=msign)
            m_err = np.linalg.norm(f64(ms[i]) - m_ref) / np.linalg.norm(m_ref)
            assert m_err <= 1e-6, (k, i, m_err)
            d_ref = w0[i] - w_ref                     # lr msign(m)
            d_gpu = w0[i] - f64(ws[i])
            bound = tol * np.linalg.norm(d_ref) + UNIT[pdt] * np.linalg.norm(w_ref)
            assert np.linalg.norm(d_gpu - d_ref) <= bound, (k, i, np.linalg.norm(d_gpu - d_ref), bound)


def test_muon_ns_fp32_groups():
    announce("muon_step ns f32 [(2,96,160),(1,200,72)]")
    _run([(2, 96, 160), (1, 200, 72)], "f32", "ns", "f32", 1e-4)


def test_muon_ns_bf16_groups():
    announce("muon_step ns bf16 [(2,128,256),(1,300,70),(0,64,64),(3,64,100)]")
    _run([(2, 128, 256), (1, 300, 70), (0, 64, 64), (3, 64, 100)], "bf16", "ns", "bf16", 2e-2)


def test_muon_gram_fp16_groups():
    announce("muon_step gram f16 [(2,96,400),(1,400,96)]")
    _run([(2, 96, 400), (1, 400, 96)], "f16", "gram", "f16", 2e-2, restart_after=(2,))


def test_muon_ns_improved_init():
    announce("muon_step ns improved init f32 [(1,160,352)]")
    _run([(1, 160, 352)], "f32", "ns", "f32", 1e-4, nsteps=2, improved_init=True)


def test_muon_zero_lr_keeps_parameters_and_updates_momentum():
    M = require_gpu()
    announce("muon_step lr=0")
    shapes = [(1, 64, 128)]
    ws, ms = _state(shapes, "bf16", 950)
    w_before = ws[0].clone()
    gs = _grads(shapes, "bf16", 960)
    M.muon_step(ws, gs, ms, lr=0.0, mu=0.5)
    M.muon_step(ws, gs, ms, lr=0.0, mu=0.5)
    torch.cuda.synchronize()
    assert torch.equal(ws[0], w_before)
    assert torch.allclose(ms[0], 1.5 * gs[0].float(), rtol=1e-6, atol=0)
