"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import msign_newton_schulz_amd as M
    M.library()  # raises if the HIP library is missing: no fallback exists
    return M


def announce(msg: str):
    """Name the case before it touches the GPU, so a fault still names it."""
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def f64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def block_error_ratio(y, ref, block: int = 256) -> float:
    """Largest error of one block x block tile of a matrix, relative to that
    tile's share of the whole reference: max over tiles b of
        ||Y_b - O_b||_F / (||O||_F sqrt(|b| / |O|)).
    An error spread evenly over the matrix gives about the matrix's relative
    Frobenius error on every tile; a wrong tile stands out (a wholly wrong
    64 x 64 tile inside a 256 x 256 one reads about 0.25), where a whole-matrix
    norm at 8192^2 would hide it under 1 %."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape and y.ndim == 2
    total = float(np.linalg.norm(ref))
    if total == 0.0:
        return float(np.linalg.norm(y))
    area = ref.size
    worst = 0.0
    for i in range(0, ref.shape[0], block):
        for j in range(0, ref.shape[1], block):
            e = y[i:i + block, j:j + block] - ref[i:i + block, j:j + block]
            share = total * (e.size / area) ** 0.5
            worst = max(worst, float(np.linalg.norm(e)) / share)
    return worst
