"""MI355X (gfx950) sparse-attention backward over top-k-gathered KV rows.

The computation runs in the HIP library built from csrc/ (C ABI in
include/sparse_attn.h); `binding` marshals torch tensors into it and
`workloads` creates seeded synthetic inputs.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "binding", "build"]
