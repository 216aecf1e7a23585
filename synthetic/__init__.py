"""Seeded synthetic inputs for msign workloads.

This module only draws random matrices of the workloads' shapes and value
distributions; it holds none of the msign arithmetic.  Both the CPU oracle
checks and the HIP-path tests and benchmark take their inputs from here.

Recipe (one matrix):  entries drawn as float32 standard normals from
numpy.random.default_rng(SeedSequence([seed, group, index])), scaled by
`noise_std`, plus a spike  sum_{k=1..rank} (1/k) u_k v_k^T  with u_k, v_k
iid N(0, 1) vectors drawn from the same generator, then rounded once to the
workload's I/O dtype (round-to-nearest-even, by torch on the CPU).  The exact
rounded values are what both the GPU path and the oracle receive.

The page workloads (Muon on Kimi K2 and Llama-430M training, an unspecified
8192-dim operator test) are not available; these shapes stand in for them:
square hidden-size matrices, MLP-shaped alpha = 3.5-4 matrices and
fine-grained-MoE alpha = 8 matrices.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Group:
    batch: int
    rows: int
    cols: int
    io_dtype: str          # "f32" | "bf16" | "f16"
    noise_std: float
    spike_rank: int
    seed: int
    group: int


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    groups: Tuple[Group, ...]
    compute: str           # compute dtype of the standard NS path


WORKLOADS: Dict[str, Workload] = {
    "c1_128x256_f32": Workload(
        "c1_128x256_f32",
        "single 128x256 fp32 matrix, iid N(0,1)",
        (Group(1, 128, 256, "f32", 1.0, 0, 1001, 0),), "f32"),
    "c2_1024x4096_bf16": Workload(
        "c2_1024x4096_bf16",
        "single 1024x4096 bf16 matrix (alpha=4), N(0,0.02^2) + rank-8 spike s_k=1/k",
        (Group(1, 1024, 4096, "bf16", 0.02, 8, 1002, 0),), "bf16"),
    "c3_8192x8192_bf16": Workload(
        "c3_8192x8192_bf16",
        "single square 8192x8192 bf16 matrix, iid N(0,1)",
        (Group(1, 8192, 8192, "bf16", 1.0, 0, 1003, 0),), "bf16"),
    "c4_block_bf16": Workload(
        "c4_block_bf16",
        "transformer block: 16 x 4096x4096 + 16 x 14336x4096 bf16, N(0,1e-6) + rank-16 spike",
        (Group(16, 4096, 4096, "bf16", 1e-3, 16, 1004, 0),
         Group(16, 14336, 4096, "bf16", 1e-3, 16, 1004, 1)), "bf16"),
    "c5_moe_f16": Workload(
        "c5_moe_f16",
        "MoE experts: 64 x 2048x7168 + 8 x 1024x8192 fp16, N(0,1) + rank-8 spike",
        (Group(64, 2048, 7168, "f16", 1.0, 8, 1005, 0),
         Group(8, 1024, 8192, "f16", 1.0, 8, 1005, 1)), "bf16"),
}


def rng_for(seed: int, group: int, index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, group, index]))


def draw(rows: int, cols: int, noise_std: float = 1.0, spike_rank: int = 0,
         seed: int = 0, group: int = 0, index: int = 0) -> np.ndarray:
    """One float32 matrix of the recipe in the module docstring."""
    g = rng_for(seed, group, index)
    m = g.standard_normal((rows, cols), dtype=np.float32)
    if noise_std != 1.0:
        m *= np.float32(noise_std)
    if spike_rank > 0:
        u = g.standard_normal((rows, spike_rank), dtype=np.float32)
        v = g.standard_normal((spike_rank, cols), dtype=np.float32)
        s = (1.0 / np.arange(1, spike_rank + 1, dtype=np.float32)).astype(np.float32)
        m += (u * s) @ v
    return m


def torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def to_io(m: np.ndarray, io_dtype: str):
    """Round a float array once to the I/O dtype; returns a CPU torch tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(m)).to(torch_dtype(io_dtype))


def group_matrix(gr: Group, index: int):
    """Matrix `index` of a group, rounded to the group's I/O dtype (CPU tensor)."""
    return to_io(draw(gr.rows, gr.cols, gr.noise_std, gr.spike_rank, gr.seed, gr.group, index),
                 gr.io_dtype)


def group_batch(gr: Group, batch: Optional[int] = None, device=None):
    """The whole group (or its first `batch` matrices) as one [B, rows, cols]
    tensor in the I/O dtype, built matrix by matrix (on `device` if given)."""
    import torch
    b = gr.batch if batch is None else batch
    out = torch.empty((b, gr.rows, gr.cols), dtype=torch_dtype(gr.io_dtype),
                      device=device if device is not None else "cpu")
    for i in range(b):
        out[i].copy_(group_matrix(gr, i))
    return out


def small_case(rows: int, cols: int, io_dtype: str, seed: int, batch: int = 1,
               noise_std: float = 1.0, spike_rank: int = 0):
    """A [batch, rows, cols] test input of the same recipe (CPU tensor)."""
    import torch
    mats = [to_io(draw(rows, cols, noise_std, spike_rank, seed, 0, i), io_dtype)
            for i in range(batch)]
    if batch == 0:
        return torch.empty((0, rows, cols), dtype=torch_dtype(io_dtype))
    return torch.stack(mats)


def as_f64(t) -> np.ndarray:
    """Exact float64 values of a (CPU or device) torch tensor."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def workload_names() -> List[str]:
    return list(WORKLOADS)
