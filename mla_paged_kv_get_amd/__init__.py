"""MI355X-native paged MLA decode: a C-ABI HIP library for gfx950 and its Python binding."""
from .api import (  # noqa: F401
    debug_copy_rows,
    get_mla_metadata,
    mla_decode_with_kvcache,
    plan_dims,
    validate_inputs,
    workspace_bytes,
)

__all__ = ["get_mla_metadata", "mla_decode_with_kvcache", "debug_copy_rows", "validate_inputs",
           "plan_dims", "workspace_bytes"]
