"""msign by Newton-Schulz iteration on MI355X (gfx950).

Python face of libmsign (C ABI in include/msign.h).  The binding only
marshals arguments; all computation runs in the HIP library, which must be
built (`python -m msign_newton_schulz_amd.build`) before use.
"""

from ._binding import (F32, BF16, F16, LIB_PATH, MAX_GROUPS, MsignError,  # noqa: F401
                       gram_ns_workspace_bytes, kernel_timing, library, mfma_probe, msign_gram_ns,
                       msign_gram_ns_grouped, msign_ns, msign_ns_grouped, msign_ns_noalloc, muon_step,
                       ns_workspace_bytes, NOALLOC_SCRATCH_BYTES,
                       read_kernel_timing, syrk_xxt, version)

__all__ = ["msign_ns", "msign_ns_noalloc", "NOALLOC_SCRATCH_BYTES", "msign_gram_ns", "msign_ns_grouped", "msign_gram_ns_grouped", "muon_step", "syrk_xxt", "MsignError", "library", "version",
           "ns_workspace_bytes", "gram_ns_workspace_bytes", "kernel_timing", "read_kernel_timing",
           "mfma_probe", "LIB_PATH", "MAX_GROUPS", "F32", "BF16", "F16"]
