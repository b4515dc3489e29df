"""MI355X-native parent-conditioned draft-tree construction and verification.

The work runs in libdtree.so (HIP kernels for gfx950, C ABI in include/dtree.h).
``binding`` marshals torch tensors to that ABI; ``runner`` wraps a whole round for callers
that hold an ``inputs.Instance``; ``inputs`` draws the seeded synthetic workloads.
"""
from .binding import (DT_BF16, DT_F32, DT_GREEDY, DT_SAMPLE, DtError, alloc_tree,  # noqa: F401
                      alloc_verify, alloc_workspace, dt_build_workspace_bytes, make_params,
                      tree_build, tree_verify_greedy, tree_verify_sample)
