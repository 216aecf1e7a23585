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
