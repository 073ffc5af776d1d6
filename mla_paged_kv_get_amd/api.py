"""Python binding of the paged MLA decode library (argument marshalling only).

The two calls follow "What is FlashMLA" (topnet.top), installation-and-use
section, steps 2 and 3: a metadata call once per decode step, then a decode
call per layer that returns ``(o, lse)``.  torch provides device memory and the
current HIP stream; every step of the computation runs in the HIP library.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

FP8_ROW_BYTES = 656   # packed FP8 cache row: 512 E4M3 codes, 4 float32 scales, 64 bf16 values

D_QK = 576
D_V = 512
PAGE = 64


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _as_bits(t: torch.Tensor, name: str) -> torch.Tensor:
    _need(t.dtype in (torch.bfloat16, torch.int16, torch.uint16), f"{name} must hold bf16 values")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    return t


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    _need(t.dtype == torch.int32 and t.is_contiguous(), f"{name} must be a contiguous int32 tensor")
    return t


def plan_dims(batch: int, s_q: int, num_q_rows: int, h_kv: int, topk: int = 0,
              num_workers: int = 0, fp8: bool = False):
    W, words, items = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    fn = "mla_plan_dims_fp8" if fp8 else "mla_plan_dims"
    _lib.check(getattr(_lib.lib(), fn)(batch, s_q, num_q_rows, h_kv, topk, num_workers,
                                       ctypes.byref(W), ctypes.byref(words), ctypes.byref(items)), fn)
    return W.value, words.value, items.value


def workspace_bytes(batch, s_q, num_q_rows, h_kv, topk, dv, num_workers) -> int:
    return int(_lib.lib().mla_workspace_bytes(batch, s_q, num_q_rows, h_kv, topk, dv, num_workers))


def get_mla_metadata(cache_seqlens: torch.Tensor, num_q_rows: int, h_kv: int, *, s_q: int = 1,
                     topk: int | None = None, num_workers: int | None = None, topk2: int = 0,
                     fp8: bool = False):
    """Split-KV plan: returns ``(tile_scheduler_metadata, num_splits)`` (int32, device).

    ``num_q_rows`` is s_q * h_q / h_kv as in the pages' call.  In sparse mode
    (``topk`` given) every query token is an item of ``topk`` keys and ``s_q``
    must be passed; with an auxiliary cache (dual-cache decode) ``topk2`` is
    the length of its index lists.  ``fp8`` plans for the decode over a packed
    FP8 cache (its row tiling sets the default worker count and the per-run
    overhead); any plan is valid for either decode.
    """
    _i32(cache_seqlens, "cache_seqlens")
    _need(cache_seqlens.is_cuda, "cache_seqlens must be on the GPU")
    batch = cache_seqlens.numel()
    tk = int(topk or 0)
    _need(not (fp8 and topk2), "the FP8 decode has no auxiliary cache (topk2)")
    W, words, items = plan_dims(batch, s_q, num_q_rows, h_kv, tk, int(num_workers or 0), fp8=fp8)
    dev = cache_seqlens.device
    plan = torch.empty(words, dtype=torch.int32, device=dev)
    num_splits = torch.empty(items + 1, dtype=torch.int32, device=dev)
    if fp8:
        _lib.check(_lib.lib().mla_get_metadata_fp8(_ptr(cache_seqlens), batch, s_q, num_q_rows, h_kv, tk,
                                                   W, _ptr(plan), _ptr(num_splits), _stream(dev)),
                   "mla_get_metadata_fp8")
    else:
        _lib.check(_lib.lib().mla_get_metadata(_ptr(cache_seqlens), batch, s_q, num_q_rows, h_kv, tk,
                                               int(topk2), W, _ptr(plan), _ptr(num_splits), _stream(dev)),
                   "mla_get_metadata")
    return plan, num_splits


def _decode_shape(q, kvcache, block_table, cache_seqlens, tile_scheduler_metadata, num_splits, indices):
    """Checks the decode's tensors; returns their sizes and the plan's worker count."""
    _as_bits(q, "q")
    fp8 = kvcache.dtype == torch.uint8
    if fp8:
        _need(kvcache.is_cuda and kvcache.is_contiguous(), "kvcache must be a contiguous CUDA tensor")
        _need(kvcache.dim() == 4 and kvcache.shape[3] == FP8_ROW_BYTES,
              "a packed FP8 kvcache is [pages, 64, h_kv, 656] uint8")
    else:
        _as_bits(kvcache, "kvcache")
    _i32(block_table, "block_table")
    _i32(cache_seqlens, "cache_seqlens")
    _i32(tile_scheduler_metadata, "tile_scheduler_metadata")
    _i32(num_splits, "num_splits")
    _need(q.dim() == 4 and kvcache.dim() == 4, "q is [b, s_q, h_q, d], kvcache is [pages, 64, h_kv, d]")
    B, s_q, h_q, d = q.shape
    num_pages, page, h_kv, d2 = kvcache.shape
    if fp8:
        d2 = 576
    _need(d == d2, "q and kvcache disagree on d_qk")
    _need(block_table.dim() == 2 and block_table.shape[0] == B, "block_table is [b, max_blocks]")
    _need(cache_seqlens.numel() == B, "cache_seqlens is [b]")
    topk = 0
    if indices is not None:
        _i32(indices, "indices")
        _need(indices.dim() == 3 and tuple(indices.shape[:2]) == (B, s_q), "indices is [b, s_q, topk]")
        topk = indices.shape[2]
        _need(topk > 0, "indices needs topk > 0")
    num_q_rows = s_q * h_q // max(h_kv, 1)
    W = int(_lib.lib().mla_plan_num_workers(tile_scheduler_metadata.numel(), B, s_q, num_q_rows,
                                             h_kv, topk))
    _need(W >= 1, "tile_scheduler_metadata does not match this call's shape")
    return fp8, B, s_q, h_q, d, num_pages, page, h_kv, topk, num_q_rows, W


def mla_decode_with_kvcache(q: torch.Tensor, kvcache: torch.Tensor, block_table: torch.Tensor,
                            cache_seqlens: torch.Tensor, dv: int, tile_scheduler_metadata: torch.Tensor,
                            num_splits: torch.Tensor, causal: bool = False,
                            softmax_scale: float | None = None, indices: torch.Tensor | None = None,
                            out: tuple | None = None, workspace: torch.Tensor | None = None,
                            phases: int = 3, aux: tuple | None = None):
    """Paged MLA decode; returns ``(o [b, s_q, h_q, dv] bf16, lse [b, s_q, h_q] fp32)``.

    ``kvcache`` is bf16 ``[pages, 64, h_kv, 576]``, or uint8 ``[pages, 64, h_kv,
    656]`` for packed FP8 rows (512 E4M3 latent codes, 4 float32 block scales,
    64 bf16 RoPE values).  ``phases`` (1 = split kernel, 2 = merge kernel, 3 =
    both) lets a caller launch the two kernels separately with the same
    arguments and buffers; ``phases=4`` is the single-launch decode, whose
    kernel merges split items itself, counting finished runs in counters that
    the plan carries (zeroed by get_mla_metadata, left zero by every completed
    call: single-launch calls that share a plan must not overlap).  ``aux = (kvcache2, block_table2, cache_seqlens2,
    indices2)`` adds an auxiliary bf16 cache (sparse mode): each query token
    attends to the union of its keys in both caches; the plan then comes from
    ``get_mla_metadata(..., topk=topk, topk2=indices2.shape[2])``.
    """
    fp8, B, s_q, h_q, d, num_pages, page, h_kv, topk, num_q_rows, W = _decode_shape(
        q, kvcache, block_table, cache_seqlens, tile_scheduler_metadata, num_splits, indices)
    scale = d ** -0.5 if softmax_scale is None else float(softmax_scale)
    dev = q.device
    if out is None:
        o = torch.empty((B, s_q, h_q, dv), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    else:
        o, lse = out
    need = workspace_bytes(B, s_q, num_q_rows, h_kv, topk, dv, W) if dv > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if aux is not None:
        kv2, bt2, sl2, idx2 = aux
        _need(indices is not None and not fp8, "an auxiliary cache needs sparse mode and bf16 caches")
        _as_bits(kv2, "kvcache2")
        _i32(bt2, "block_table2")
        _i32(sl2, "cache_seqlens2")
        _i32(idx2, "indices2")
        _need(kv2.dim() == 4 and kv2.shape[1] == page and kv2.shape[2] == h_kv and kv2.shape[3] == d,
              "kvcache2 is [pages2, 64, h_kv, d_qk]")
        _need(bt2.dim() == 2 and bt2.shape[0] == B and sl2.numel() == B, "block_table2 / cache_seqlens2 per sequence")
        _need(idx2.dim() == 3 and tuple(idx2.shape[:2]) == (B, s_q), "indices2 is [b, s_q, topk2]")
        _lib.check(_lib.lib().mla_decode_with_kvcache_dual(
            _ptr(q), _ptr(kvcache), num_pages, _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
            _ptr(indices), topk, _ptr(kv2), kv2.shape[0], _ptr(bt2), bt2.shape[1], _ptr(sl2),
            _ptr(idx2) if idx2.shape[2] > 0 else None, idx2.shape[2], page, B, s_q, h_q, h_kv, d, dv,
            _ptr(tile_scheduler_metadata), _ptr(num_splits), W, ctypes.c_float(scale), _ptr(o), _ptr(lse),
            _ptr(workspace), workspace.numel() * workspace.element_size(), int(phases), _stream(dev)),
            "mla_decode_with_kvcache_dual")
        return o, lse
    entry = _lib.lib().mla_decode_with_kvcache_fp8_phase if fp8 else _lib.lib().mla_decode_with_kvcache_phase
    _lib.check(entry(
        _ptr(q), _ptr(kvcache), num_pages, page, _ptr(block_table), block_table.shape[1],
        _ptr(cache_seqlens), B, s_q, h_q, h_kv, d, dv, _ptr(tile_scheduler_metadata),
        _ptr(num_splits), W, int(bool(causal)), ctypes.c_float(scale), _ptr(indices), topk,
        _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        int(phases), _stream(dev)), "mla_decode_with_kvcache")
    return o, lse


def mla_decode_with_kvcache_no_alloc(q: torch.Tensor, kvcache: torch.Tensor, block_table: torch.Tensor,
                                     cache_seqlens: torch.Tensor, dv: int,
                                     tile_scheduler_metadata: torch.Tensor, num_splits: torch.Tensor,
                                     out: tuple, causal: bool = False,
                                     softmax_scale: float | None = None,
                                     indices: torch.Tensor | None = None):
    """The decode without a workspace, writing into ``out = (o, lse)``.

    Neither this function nor the library allocates device memory: the split
    partials go to the library's fixed per-GPU scratch of
    ``NO_ALLOC_SCRATCH_BYTES``; a call that needs more raises ``ValueError``
    (fewer workers in the plan need less).  bf16 caches only.  No-alloc calls
    that overlap on one GPU share that scratch and race.
    """
    _need(kvcache.dtype != torch.uint8, "the no-alloc decode takes bf16 caches")
    fp8, B, s_q, h_q, d, num_pages, page, h_kv, topk, num_q_rows, W = _decode_shape(
        q, kvcache, block_table, cache_seqlens, tile_scheduler_metadata, num_splits, indices)
    o, lse = out
    scale = d ** -0.5 if softmax_scale is None else float(softmax_scale)
    _lib.check(_lib.lib().mla_decode_with_kvcache_no_alloc(
        _ptr(q), _ptr(kvcache), num_pages, page, _ptr(block_table), block_table.shape[1],
        _ptr(cache_seqlens), B, s_q, h_q, h_kv, d, dv, _ptr(tile_scheduler_metadata),
        _ptr(num_splits), W, int(bool(causal)), ctypes.c_float(scale), _ptr(indices), topk,
        _ptr(o), _ptr(lse), _stream(q.device)), "mla_decode_with_kvcache_no_alloc")
    return o, lse


def debug_copy_rows(q: torch.Tensor, kvcache: torch.Tensor, block_table: torch.Tensor,
                    cache_seqlens: torch.Tensor, tile_scheduler_metadata: torch.Tensor,
                    num_splits: torch.Tensor, causal: bool = False, indices: torch.Tensor | None = None,
                    aux: tuple | None = None) -> torch.Tensor:
    """Indexing probe: run the split decode kernel and return, for every cache
    row its tile copies read, the byte offset of that row from ``kvcache``
    (int64 ``[planes, items, tiles, 64]``, -1 where no copy read; packed FP8
    caches add a second plane: the row whose scales were read)."""
    fp8 = kvcache.dtype == torch.uint8
    B, s_q, h_q, d = q.shape
    num_pages, _, h_kv, _ = kvcache.shape
    topk = 0 if indices is None else indices.shape[2]
    topk2 = 0 if aux is None else aux[3].shape[2]
    num_q_rows = s_q * h_q // h_kv
    W = int(_lib.lib().mla_plan_num_workers(tile_scheduler_metadata.numel(), B, s_q, num_q_rows, h_kv, topk))
    _need(W >= 1, "tile_scheduler_metadata does not match this call's shape")
    items = B * h_kv * (s_q if topk else 1)
    tiles = (-(-topk // 64) + -(-topk2 // 64)) if topk else block_table.shape[1]
    planes = 2 if fp8 else 1
    out = torch.full((planes, items, tiles, 64), -1, dtype=torch.int64, device=q.device)
    o = torch.empty((B, s_q, h_q, D_V), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q.device)
    need = workspace_bytes(B, s_q, num_q_rows, h_kv, topk, D_V, W)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    kv2 = bt2 = sl2 = idx2 = None
    if aux is not None:
        kv2, bt2, sl2, idx2 = aux
    _lib.check(_lib.lib().mla_debug_copy_rows(
        _ptr(q), _ptr(kvcache), num_pages, 1 if fp8 else 0, _ptr(block_table), block_table.shape[1],
        _ptr(cache_seqlens), _ptr(indices), topk, _ptr(kv2), kv2.shape[0] if kv2 is not None else 0,
        _ptr(bt2), bt2.shape[1] if bt2 is not None else 0, _ptr(sl2),
        _ptr(idx2) if topk2 > 0 else None, topk2, B, s_q, h_q, h_kv, 576 if fp8 else d, int(bool(causal)),
        _ptr(tile_scheduler_metadata), _ptr(num_splits), W, _ptr(o), _ptr(lse), _ptr(ws),
        ws.numel(), _ptr(out), out.numel(), _stream(q.device)), "mla_debug_copy_rows")
    return out


def validate_inputs(block_table: torch.Tensor, cache_seqlens: torch.Tensor, num_pages: int,
                    indices: torch.Tensor | None = None, s_q: int = 1) -> int:
    """Number of out-of-range block-table entries / lengths (synchronises)."""
    _i32(block_table, "block_table")
    _i32(cache_seqlens, "cache_seqlens")
    B, mb = block_table.shape
    topk = 0
    if indices is not None:
        _i32(indices, "indices")
        s_q, topk = indices.shape[1], indices.shape[2]
    err = torch.empty(1, dtype=torch.int32, device=block_table.device)
    _lib.check(_lib.lib().mla_validate_inputs(_ptr(block_table), mb, _ptr(cache_seqlens), B, s_q,
                                              _ptr(indices), topk, num_pages, _ptr(err),
                                              _stream(block_table.device)),
               "mla_validate_inputs")
    return int(err.item())
