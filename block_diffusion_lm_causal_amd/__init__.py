"""Block-causal / staircase attention for block-diffusion LMs on MI355X (gfx950).

The compute lives in libbca.so (hand-written HIP kernels behind the C ABI of
include/bca.h); ``bca`` is its Python binding.  ``workloads`` draws the seeded
synthetic inputs.  The library is loaded on first use, never at import.
"""
from . import bca, workloads  # noqa: F401
from .bca import (BcaError, decode, decode_workspace, fwd, staircase_bwd,  # noqa: F401
                  staircase_bwd_workspace, staircase_fwd)

__all__ = ["BcaError", "bca", "decode", "decode_workspace", "fwd", "staircase_bwd",
           "staircase_bwd_workspace", "staircase_fwd", "workloads"]
