"""MI355X-native paged MLA decode: a C-ABI HIP library for gfx950 and its Python binding."""
from .api import (  # noqa: F401
    debug_copy_rows,
    get_mla_metadata,
    mla_decode_with_kvcache,
    mla_decode_with_kvcache_no_alloc,
    plan_dims,
    validate_inputs,
    workspace_bytes,
)

from ._lib import NO_ALLOC_SCRATCH_BYTES  # noqa: F401

__all__ = ["get_mla_metadata", "mla_decode_with_kvcache", "mla_decode_with_kvcache_no_alloc",
           "debug_copy_rows", "validate_inputs", "plan_dims", "workspace_bytes", "NO_ALLOC_SCRATCH_BYTES"]
