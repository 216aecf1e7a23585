"""The allocation-free entry point msign_ns_noalloc, through the C ABI: its
results against msign_ns's (the entry point it is a variant of; same
kernels and launch plan, so the same bits) on two calls in a row, the
second smaller, plus the size limit of its scratch.  Collected last: a
failure here hides no other test."""

import pytest
import torch

import synthetic as S
from gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu


def _pair(M, x, cdt):
    ref = M.msign_ns(x, compute_dtype=cdt)
    out = torch.empty_like(x)
    got = M.msign_ns_noalloc(x, out, compute_dtype=cdt)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_matches_msign_ns_twice_second_smaller():
    M = require_gpu()
    big = S.small_case(512, 1024, "bf16", 31, batch=2, noise_std=1.0, spike_rank=4).cuda()
    small = S.small_case(200, 130, "bf16", 32, batch=1, noise_std=1.0, spike_rank=2).cuda()
    announce("msign_ns_noalloc 2x512x1024 bf16, then 1x200x130")
    got, ref = _pair(M, big, torch.bfloat16)
    assert torch.equal(got, ref)
    # the second call reuses the scratch the first one left behind
    got, ref = _pair(M, small, torch.bfloat16)
    assert torch.equal(got, ref)
    announce("msign_ns_noalloc fp32 products 1x96x300 f32")
    x = S.small_case(96, 300, "f32", 33, batch=1, noise_std=1.0, spike_rank=0).cuda()
    got, ref = _pair(M, x, torch.float32)
    assert torch.equal(got, ref)


def test_noalloc_largest_fitting_size_and_rejection():
    M = require_gpu()
    lib = M.library()
    need = lib.msign_ns_workspace_bytes(1, 1024, 4096, 1)
    assert need <= M.NOALLOC_SCRATCH_BYTES
    x = S.small_case(1024, 4096, "bf16", 34, batch=1, noise_std=0.02, spike_rank=8).cuda()
    announce("msign_ns_noalloc 1x1024x4096 bf16 (fits the scratch)")
    got, ref = _pair(M, x, torch.bfloat16)
    assert torch.equal(got, ref)
    # too large for the scratch: an error before anything is launched
    assert lib.msign_ns_workspace_bytes(1, 2048, 4096, 1) > M.NOALLOC_SCRATCH_BYTES
    x2 = torch.zeros(1, 2048, 4096, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(x2, 7.0)
    with pytest.raises(M.MsignError, match="scratch"):
        M.msign_ns_noalloc(x2, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
