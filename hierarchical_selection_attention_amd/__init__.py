"""Lighthouse attention layer on MI355X (gfx950): HIP kernels behind a C ABI.

Import fails loudly when liblighthouse.so has not been built
(`python hierarchical_selection_attention_amd/build.py`); there is no
fallback implementation.
"""
from ._lib import *  # noqa: F401,F403
from ._lib import (EXPORTS, LIB_PATH, LighthouseError, alloc_workspace, backward, block_backward,  # noqa: F401
                   forward_static,
                   block_forward, block_workspace, dense_backward, dense_forward, dtype_code, forward, peak_probe,
                   read_selection, workspace_tensor)
