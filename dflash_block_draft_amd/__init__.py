"""MI355X-native DFlash/DSpark draft MLA attention.

The compute lives in a HIP library for gfx950 (``libdflash_mla.so``, built from
``csrc/``) behind a small C ABI declared in ``include/dflash_mla.h``.  This
package is its thin Python binding: it marshals torch device tensors and the
current HIP stream into that ABI and nothing else.  The binding is loaded on
first use; if the library is missing, every entry point raises.
"""
from .mla import (  # noqa: F401
    latent_expand, mla_attn, mask_occupancy, attn_workspace_bytes, tile_map_view,
    TILE_M, TILE_N, DflashError,
)
