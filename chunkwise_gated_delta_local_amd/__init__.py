"""Chunked gated delta-rule forward for AMD MI355X (gfx950).

The compute path is a C-ABI shared library (``libgdr.so``, built from
``csrc/``) of hand-written HIP kernels; this package only marshals torch
tensors into it. Importing the package does not load the library; the first
call does, and fails loudly if the library is missing.
"""
from .api import Forward, chunk_fwd, chunk_fwd_debug, recurrent_fwd, workspace_size, validate  # noqa: F401
