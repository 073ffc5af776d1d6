"""ctypes view of ``libmla_paged_kv.so`` (the C ABI in include/mla_paged_kv.h).

torch is imported first so that its HIP runtime is the one the library binds
to (both carry the soname libamdhip64.so.7; the dynamic loader reuses the copy
already mapped).  Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the library: one HIP runtime per process)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_paged_kv.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4
MLA_ERR_SCRATCH_LIMIT = 5
NO_ALLOC_SCRATCH_BYTES = 128 << 20     # MLA_NO_ALLOC_SCRATCH_BYTES

EXPORTS = (
    "mla_status_string", "mla_plan_dims", "mla_plan_dims_fp8", "mla_plan_num_workers", "mla_get_metadata",
    "mla_get_metadata_fp8",
    "mla_workspace_bytes",
    "mla_decode_with_kvcache", "mla_decode_with_kvcache_no_alloc", "mla_decode_with_kvcache_phase",
    "mla_decode_with_kvcache_fp8",
    "mla_decode_with_kvcache_fp8_phase", "mla_decode_with_kvcache_dual", "mla_debug_copy_rows",
    "mla_validate_inputs",
)

_c_int = ctypes.c_int
_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_ip = ctypes.POINTER(ctypes.c_int)

_SIGS = {
    "mla_status_string": (ctypes.c_char_p, [_c_int]),
    "mla_plan_dims": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _ip, _ip, _ip]),
    "mla_plan_dims_fp8": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _ip, _ip, _ip]),
    "mla_plan_num_workers": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "mla_get_metadata": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "mla_get_metadata_fp8": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "mla_workspace_bytes": (ctypes.c_size_t, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "mla_decode_with_kvcache": (_c_int, [
        _vp, _vp, _c_i64, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _c_int, _c_int, ctypes.c_float, _vp, _c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "mla_decode_with_kvcache_no_alloc": (_c_int, [
        _vp, _vp, _c_i64, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _c_int, _c_int, ctypes.c_float, _vp, _c_int, _vp, _vp, _vp]),
    "mla_decode_with_kvcache_phase": (_c_int, [
        _vp, _vp, _c_i64, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _c_int, _c_int, ctypes.c_float, _vp, _c_int, _vp, _vp, _vp, ctypes.c_size_t,
        _c_int, _vp]),
    "mla_decode_with_kvcache_fp8": (_c_int, [
        _vp, _vp, _c_i64, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _c_int, _c_int, ctypes.c_float, _vp, _c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "mla_decode_with_kvcache_fp8_phase": (_c_int, [
        _vp, _vp, _c_i64, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _c_int, _c_int, ctypes.c_float, _vp, _c_int, _vp, _vp, _vp, ctypes.c_size_t,
        _c_int, _vp]),
    "mla_decode_with_kvcache_dual": (_c_int, [
        _vp, _vp, _c_i64, _vp, _c_int, _vp, _vp, _c_int,
        _vp, _c_i64, _vp, _c_int, _vp, _vp, _c_int,
        _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _c_int, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _c_int, _vp]),
    "mla_debug_copy_rows": (_c_int, [
        _vp, _vp, _c_i64, _c_int, _vp, _c_int, _vp, _vp, _c_int,
        _vp, _c_i64, _vp, _c_int, _vp, _vp, _c_int,
        _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp, _c_i64, _vp]),
    "mla_validate_inputs": (_c_int, [_vp, _c_int, _vp, _c_int, _c_int, _vp, _c_int, _c_i64, _vp, _vp]),
}

_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = lib().mla_status_string(status).decode()
        super().__init__(f"{where}: {text} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with `python -m mla_paged_kv_get_amd.build`")
        l = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_LOCAL)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(status: int, where: str) -> None:
    if status != MLA_OK:
        if status in (MLA_ERR_INVALID_ARGUMENT, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE_TOO_SMALL,
                      MLA_ERR_SCRATCH_LIMIT):
            raise ValueError(str(MLAError(status, where)))
        raise MLAError(status, where)
