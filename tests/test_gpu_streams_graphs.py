"""Calls on several streams at once, and calls captured in HIP graphs.

The library only queues kernel launches on the caller's stream (no
allocation, copy, memset or host synchronisation), so:
- concurrent calls on different streams, each with its own output and
  workspace, give exactly the bits of the same calls made one after another;
- a call captured into a graph replays to exactly the eager result.  Each
  graph is replayed several times with eager work and synchronisations in
  between, and every replay is checked.
"""

import pytest
import torch

import synthetic as S
from gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu


def _x(rows, cols, seed, batch=2, dt="bf16"):
    return S.small_case(rows, cols, dt, seed, batch=batch, noise_std=1.0, spike_rank=2).cuda()


def test_concurrent_streams_match_sequential_calls():
    M = require_gpu()
    announce("msign on two streams at once")
    x1 = _x(512, 1024, 11, batch=4)
    x2 = _x(768, 384, 12, batch=3, dt="f16")
    x3, x4 = _x(200, 72, 13), _x(96, 400, 14)
    ref1 = M.msign_ns(x1)
    ref2 = M.msign_gram_ns(x2, compute_dtype=torch.float16)
    ref3, ref4 = M.msign_ns_grouped([x3, x4])
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            y1 = M.msign_ns(x1)
            y3, y4 = M.msign_ns_grouped([x3, x4])
        with torch.cuda.stream(s2):
            y2 = M.msign_gram_ns(x2, compute_dtype=torch.float16)
        torch.cuda.synchronize()
        assert torch.equal(y1, ref1) and torch.equal(y2, ref2)
        assert torch.equal(y3, ref3) and torch.equal(y4, ref4)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_replays_match_eager():
    M = require_gpu()
    announce("msign_ns and msign_ns_grouped captured in graphs")
    x = _x(384, 640, 21)
    xa, xb = _x(256, 512, 22), _x(300, 70, 23, batch=3)
    y = torch.empty_like(x)
    ya, yb = torch.empty_like(xa), torch.empty_like(xb)
    ws = torch.empty(M.ns_workspace_bytes(2, 384, 640, torch.bfloat16), dtype=torch.uint8, device="cuda")
    lib = M.library()
    import msign_newton_schulz_amd._binding as B
    arr = (B._Group * 2)(B._Group(xa.data_ptr(), ya.data_ptr(), 2, 256, 512),
                         B._Group(xb.data_ptr(), yb.data_ptr(), 3, 300, 70))
    wsg = torch.empty(lib.msign_ns_grouped_workspace_bytes(arr, 2, B.BF16), dtype=torch.uint8, device="cuda")
    g1 = _capture(lambda: M.msign_ns(x, out=y, workspace=ws))
    g2 = _capture(lambda: M.msign_ns_grouped([xa, xb], outs=[ya, yb], workspace=wsg))
    for k in range(4):
        # new inputs written eagerly between replays
        x.copy_(_x(384, 640, 100 + k))
        xa.copy_(_x(256, 512, 200 + k))
        xb.copy_(_x(300, 70, 300 + k, batch=3))
        torch.cuda.synchronize()
        g1.replay()
        g2.replay()
        torch.cuda.synchronize()
        ref = M.msign_ns(x)
        refa, refb = M.msign_ns_grouped([xa, xb])
        torch.cuda.synchronize()
        assert torch.equal(y, ref), k
        assert torch.equal(ya, refa) and torch.equal(yb, refb), k


def test_graph_replays_of_gram_ns_match_eager():
    M = require_gpu()
    announce("msign_gram_ns captured in a graph")
    x = _x(256, 1024, 31, dt="f16")
    y = torch.empty_like(x)
    ws = torch.empty(M.gram_ns_workspace_bytes(2, 256, 1024, torch.float16), dtype=torch.uint8, device="cuda")
    g = _capture(lambda: M.msign_gram_ns(x, compute_dtype=torch.float16, out=y, workspace=ws))
    for k in range(4):
        x.copy_(_x(256, 1024, 400 + k, dt="f16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = M.msign_gram_ns(x, compute_dtype=torch.float16)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), k


def test_graph_replays_of_a_muon_step_match_eager_steps():
    M = require_gpu()
    announce("muon_step captured in a graph, replayed 3 times")
    shapes = [(2, 128, 320), (1, 320, 128)]
    gs = [_x(r, c, 40 + i, batch=b) for i, (b, r, c) in enumerate(shapes)]
    gen = torch.Generator(device="cuda").manual_seed(3)
    w0 = [(0.02 * torch.randn(g.shape, generator=gen, device="cuda")).to(torch.bfloat16) for g in gs]
    ws_e, ms_e = [w.clone() for w in w0], [torch.zeros(g.shape, device="cuda") for g in gs]
    ws_g, ms_g = [w.clone() for w in w0], [torch.zeros(g.shape, device="cuda") for g in gs]
    import msign_newton_schulz_amd._binding as B
    arr = (B._MuonGroup * 2)(*[B._MuonGroup(w.data_ptr(), g.data_ptr(), m.data_ptr(), *g.shape)
                               for w, g, m in zip(ws_g, gs, ms_g)])
    nb = M.library().muon_step_workspace_bytes(arr, 2, B.MUON_NS, B.BF16)
    wsp = torch.empty(nb, dtype=torch.uint8, device="cuda")
    step = lambda: M.muon_step(ws_g, gs, ms_g, lr=0.02, mu=0.9, workspace=wsp)
    # capture after the warm-up step: reset the state to the start first
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for w, w_init, m in zip(ws_g, w0, ms_g):
        w.copy_(w_init)
        m.zero_()
    torch.cuda.synchronize()
    for k in range(3):
        g.replay()
        torch.cuda.synchronize()
        M.muon_step(ws_e, gs, ms_e, lr=0.02, mu=0.9)
        torch.cuda.synchronize()
        for a, b in zip(ws_g + ms_g, ws_e + ms_e):
            assert torch.equal(a, b), k
