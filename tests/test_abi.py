"""The C-ABI library on the CPU: it loads, exports what the header declares,
and rejects bad arguments before enqueuing anything (no GPU needed)."""
import ctypes
import os
import re

import pytest
import torch

from mla_paged_kv_get_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(mla_\w+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol():
    l = _lib.lib()
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(l, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_one_hip_runtime_mapped():
    _lib.lib()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) <= 1, paths


def test_status_strings():
    l = _lib.lib()
    for s in range(6):
        assert l.mla_status_string(s)
    assert l.mla_status_string(99) == b"unknown status"


def _dims(*a):
    W, w, it = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = _lib.lib().mla_plan_dims(*a, ctypes.byref(W), ctypes.byref(w), ctypes.byref(it))
    return st, W.value, w.value, it.value


def test_plan_dims():
    # words = 8 (W + 1) plan rows + one arrival counter per item and 64- (or 16-) row tile
    assert _dims(64, 1, 16, 1, 0, 256) == (0, 256, 8 * 257 + 64, 64)
    assert _dims(16, 8, 8 * 128, 1, 2048, 100) == (0, 100, 8 * 101 + 128 * 2, 128)  # sparse: items = b * s_q
    assert _dims(32, 2, 256, 1, 0, 128) == (0, 128, 8 * 129 + 32 * 4, 32)
    assert _dims(4, 1, 16, 2, 0, 8) == (0, 8, 8 * 9 + 8, 8)                     # h_kv = 2: items = b * h_kv
    assert _dims(4, 2, 2 * 16, 4, 64, 8) == (0, 8, 8 * 9 + 32, 32)             # sparse: items = b * s_q * h_kv
    assert _dims(4, 3, 16, 1, 64, 8)[0] == _lib.MLA_ERR_INVALID_ARGUMENT        # rows not a multiple of s_q
    assert _dims(-1, 1, 16, 1, 0, 8)[0] == _lib.MLA_ERR_INVALID_ARGUMENT
    assert _dims(4, 1, 16, 1, 0, -3)[0] == _lib.MLA_ERR_INVALID_ARGUMENT


def test_plan_dims_fp8_and_metadata_fp8_checks():
    # the FP8 plan has the same words (the arrival counters cover the finest
    # row tiling of either format) and rejects the same arguments
    l = _lib.lib()
    for args in [(64, 1, 16, 1, 0, 256), (16, 8, 8 * 128, 1, 2048, 128), (32, 2, 256, 1, 0, 64)]:
        W, w, it = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        st = l.mla_plan_dims_fp8(*args, ctypes.byref(W), ctypes.byref(w), ctypes.byref(it))
        assert (st, W.value, w.value, it.value) == _dims(*args)
    W, w, it = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert l.mla_plan_dims_fp8(4, 3, 16, 1, 64, 8, ctypes.byref(W), ctypes.byref(w),
                               ctypes.byref(it)) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_get_metadata_fp8(DUMMY, 4, 1, 16, 1, 0, 8, None, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_get_metadata_fp8(DUMMY, 4, 1, 16, 1, 0, 0, DUMMY, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_get_metadata_fp8(None, 4, 1, 16, 1, 0, 8, DUMMY, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_get_metadata_fp8(DUMMY, (1 << 20) + 1, 1, 16, 1, 0, 8, DUMMY, DUMMY,
                                  None) == _lib.MLA_ERR_UNSUPPORTED


def test_workspace_bytes():
    l = _lib.lib()
    # (items + W) partial slots of rows x (512 bf16 outputs + one fp32 LSE)
    row = 512 * 2 + 4
    assert l.mla_workspace_bytes(64, 1, 16, 1, 0, 512, 256) == (64 + 256) * 16 * row
    assert l.mla_workspace_bytes(16, 8, 1024, 1, 2048, 512, 256) == (128 + 256) * 128 * row
    assert l.mla_workspace_bytes(64, 1, 16, 1, 0, 512, 0) == 0
    assert l.mla_workspace_bytes(8, 1, 32, 4, 0, 512, 64) == (32 + 64) * 32 * row   # h_kv = 4
    # items of more than 64 rows: slots of whole 32-row blocks
    assert l.mla_workspace_bytes(2, 1, 100, 1, 0, 512, 8) == (2 + 8) * 128 * row
    assert l.mla_workspace_bytes(2, 1, 64, 1, 0, 512, 8) == (2 + 8) * 64 * row


DUMMY = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails its host checks


def _decode(**kw):
    a = dict(q=DUMMY, kv=DUMMY, num_pages=10, page=64, bt=DUMMY, mb=4, sl=DUMMY, batch=2, s_q=1,
             h_q=16, h_kv=1, d=576, dv=512, plan=DUMMY, ns=DUMMY, W=8, causal=0, scale=0.05,
             idx=None, topk=0, o=DUMMY, lse=DUMMY, ws=DUMMY, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return _lib.lib().mla_decode_with_kvcache(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(d=448), _lib.MLA_ERR_UNSUPPORTED),
    (dict(d=512, ws_bytes=100), _lib.MLA_ERR_WORKSPACE_TOO_SMALL),           # d_qk = 512 is accepted
    (dict(dv=256), _lib.MLA_ERR_UNSUPPORTED),
    (dict(page=32), _lib.MLA_ERR_UNSUPPORTED),
    (dict(h_kv=2, h_q=16, ws_bytes=100), _lib.MLA_ERR_WORKSPACE_TOO_SMALL),    # h_kv = 2 is accepted
    (dict(h_q=15, h_kv=2), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(q=None), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(o=None), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(causal=2), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(idx=DUMMY, topk=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(idx=None, topk=16), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(idx=DUMMY, topk=16, causal=1), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(W=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=100), _lib.MLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(s_q=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(mb=0), _lib.MLA_ERR_INVALID_ARGUMENT),
])
def test_decode_rejects(kw, code):
    assert _decode(**kw) == code


def test_decode_empty_batch_is_noop():
    assert _decode(batch=0) == _lib.MLA_OK


def test_decode_empty_batch_takes_null_arrays():
    # zero-length per-sequence arrays may be null; the shared ones may not
    empty = dict(batch=0, q=None, bt=None, sl=None, o=None, lse=None)
    assert _decode(**empty) == _lib.MLA_OK
    assert _decode(**empty, idx=None, topk=16) == _lib.MLA_OK
    assert _decode(**empty, kv=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert _decode(**empty, plan=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert _decode(**empty, idx=None, topk=16, causal=1) == _lib.MLA_ERR_INVALID_ARGUMENT


def _no_alloc(**kw):
    a = dict(q=DUMMY, kv=DUMMY, num_pages=10, page=64, bt=DUMMY, mb=4, sl=DUMMY, batch=2, s_q=1,
             h_q=16, h_kv=1, d=576, dv=512, plan=DUMMY, ns=DUMMY, W=8, causal=0, scale=0.05,
             idx=None, topk=0, o=DUMMY, lse=DUMMY, stream=None)
    a.update(kw)
    return _lib.lib().mla_decode_with_kvcache_no_alloc(*a.values())


def test_no_alloc_scratch_size_matches_header():
    txt = open(os.path.join(ROOT, "include", "mla_paged_kv.h")).read()
    m = re.search(r"#define MLA_NO_ALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NO_ALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,code", [
    (dict(d=448), _lib.MLA_ERR_UNSUPPORTED),
    (dict(page=32), _lib.MLA_ERR_UNSUPPORTED),
    (dict(q=None), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(causal=2), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(idx=DUMMY, topk=16, causal=1), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(W=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    # partials of (items + W) x 128 rows x 1028 bytes: 4096 + 8 slots need 0.54 GB
    (dict(batch=4096, h_q=128), _lib.MLA_ERR_SCRATCH_LIMIT),
    (dict(W=1 << 14, h_q=128), _lib.MLA_ERR_SCRATCH_LIMIT),
])
def test_no_alloc_rejects_before_any_hip_call(kw, code):
    assert _no_alloc(**kw) == code


def test_no_alloc_limit_is_the_workspace_size():
    l = _lib.lib()
    W = 1
    while l.mla_workspace_bytes(2, 1, 128, 1, 0, 512, W + 1) <= _lib.NO_ALLOC_SCRATCH_BYTES:
        W += 1
    assert _no_alloc(W=W + 1, h_q=128) == _lib.MLA_ERR_SCRATCH_LIMIT
    if torch.cuda.device_count() == 0:
        # the largest worker count whose partials fit passes the host checks;
        # the first HIP call then fails (no GPU: nothing is launched)
        assert _no_alloc(W=W, h_q=128) == _lib.MLA_ERR_HIP


def test_no_alloc_empty_batch_is_noop():
    assert _no_alloc(batch=0, q=None, bt=None, sl=None, o=None, lse=None) == _lib.MLA_OK


def test_phase_argument_checked():
    l = _lib.lib()
    args = [DUMMY, DUMMY, 10, 64, DUMMY, 4, DUMMY, 2, 1, 16, 1, 576, 512, DUMMY, DUMMY, 8, 0,
            ctypes.c_float(0.05), None, 0, DUMMY, DUMMY, DUMMY, 1 << 40]
    assert l.mla_decode_with_kvcache_phase(*args, 0, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_decode_with_kvcache_phase(*args, 5, None) == _lib.MLA_ERR_INVALID_ARGUMENT


def test_fp8_entries_reject():
    l = _lib.lib()
    args = [DUMMY, DUMMY, 10, 64, DUMMY, 4, DUMMY, 2, 1, 16, 1, 576, 512, DUMMY, DUMMY, 8, 0,
            ctypes.c_float(0.05), None, 0, DUMMY, DUMMY, DUMMY, 1 << 40]
    assert l.mla_decode_with_kvcache_fp8_phase(*args, 0, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    bad_d = list(args)
    bad_d[11] = 656                      # d_qk counts values, not bytes
    assert l.mla_decode_with_kvcache_fp8(*bad_d, None) == _lib.MLA_ERR_UNSUPPORTED
    bad_scale = list(args)
    bad_scale[17] = ctypes.c_float(-1.0)
    assert l.mla_decode_with_kvcache_fp8(*bad_scale, None) == _lib.MLA_ERR_INVALID_ARGUMENT


def _dual(**kw):
    a = dict(q=DUMMY, kv=DUMMY, num_pages=10, bt=DUMMY, mb=4, sl=DUMMY, idx=DUMMY, topk=64,
             kv2=DUMMY, num_pages2=10, bt2=DUMMY, mb2=4, sl2=DUMMY, idx2=DUMMY, topk2=32,
             page=64, batch=2, s_q=1, h_q=16, h_kv=1, d=512, dv=512, plan=DUMMY, ns=DUMMY, W=8,
             scale=ctypes.c_float(0.05), o=DUMMY, lse=DUMMY, ws=DUMMY, ws_bytes=1 << 40, phases=3,
             stream=None)
    a.update(kw)
    return _lib.lib().mla_decode_with_kvcache_dual(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(idx=None), _lib.MLA_ERR_INVALID_ARGUMENT),           # the main list is required
    (dict(topk=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(idx2=None), _lib.MLA_ERR_INVALID_ARGUMENT),          # topk2 > 0 needs its list
    (dict(kv2=None), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(num_pages2=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(mb2=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(d=448), _lib.MLA_ERR_UNSUPPORTED),
    (dict(phases=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=100), _lib.MLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(idx2=None, topk2=0, ws_bytes=100), _lib.MLA_ERR_WORKSPACE_TOO_SMALL),   # no auxiliary keys: accepted
])
def test_dual_rejects(kw, code):
    assert _dual(**kw) == code


def test_metadata_rejects():
    l = _lib.lib()
    # (cache_seqlens, batch, s_q, num_q_rows, h_kv, topk, topk2, W, plan, num_splits, stream)
    assert l.mla_get_metadata(DUMMY, 4, 1, 16, 1, 0, 0, 8, None, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_get_metadata(DUMMY, 4, 1, 16, 1, 0, 0, 0, DUMMY, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_get_metadata(DUMMY, 4, 1, 16, 0, 0, 0, 8, DUMMY, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_get_metadata(None, 4, 1, 16, 1, 0, 0, 8, DUMMY, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    # topk2 (the auxiliary lists of the dual-cache decode) needs topk and is >= 0
    assert l.mla_get_metadata(DUMMY, 4, 1, 16, 1, 0, 32, 8, DUMMY, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_get_metadata(DUMMY, 4, 1, 16, 1, 64, -1, 8, DUMMY, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    # the tiles of an item (both lists) must be countable in an int
    assert l.mla_get_metadata(DUMMY, 4, 1, 16, 1, 2 ** 31 - 1, 2 ** 31 - 1, 8, DUMMY, DUMMY,
                              None) == _lib.MLA_ERR_UNSUPPORTED


def test_metadata_item_cap():
    # one call plans at most MLA_PLAN_MAX_ITEMS = 2^20 items (dense: batch * h_kv;
    # sparse: batch * s_q * h_kv), and past MLA_PLAN_LDS_ITEMS = 16384 items with
    # at most 4096 workers; the rest is rejected before anything is enqueued
    l = _lib.lib()
    cap, lds = 1 << 20, 16384
    assert l.mla_get_metadata(DUMMY, cap + 1, 1, 16, 1, 0, 0, 8, DUMMY, DUMMY, None) == _lib.MLA_ERR_UNSUPPORTED
    assert l.mla_get_metadata(DUMMY, cap // 2 + 1, 1, 32, 2, 0, 0, 8, DUMMY, DUMMY, None) == _lib.MLA_ERR_UNSUPPORTED
    assert l.mla_get_metadata(DUMMY, 1, cap + 1, (cap + 1) * 16, 1, 64, 0, 8, DUMMY, DUMMY,
                              None) == _lib.MLA_ERR_UNSUPPORTED
    assert l.mla_get_metadata(DUMMY, 2, cap // 2 + 1, (cap // 2 + 1) * 16, 1, 64, 32, 8, DUMMY, DUMMY,
                              None) == _lib.MLA_ERR_UNSUPPORTED
    assert l.mla_get_metadata(DUMMY, lds + 1, 1, 16, 1, 0, 0, 4097, DUMMY, DUMMY, None) == _lib.MLA_ERR_UNSUPPORTED
    assert l.mla_get_metadata(DUMMY, 1, lds + 1, (lds + 1) * 16, 1, 64, 0, 4097, DUMMY, DUMMY,
                              None) == _lib.MLA_ERR_UNSUPPORTED
    hdr = open(os.path.join(ROOT, "include", "mla_paged_kv.h")).read()
    assert re.search(r"#define MLA_PLAN_MAX_ITEMS\s+1048576\b", hdr)
    assert re.search(r"#define MLA_PLAN_LDS_ITEMS\s+16384\b", hdr)


def test_debug_and_validate_reject():
    l = _lib.lib()
    probe = dict(q=DUMMY, kv=DUMMY, num_pages=10, fmt=0, bt=DUMMY, mb=4, sl=DUMMY, idx=None, topk=0,
                 kv2=None, num_pages2=0, bt2=None, mb2=0, sl2=None, idx2=None, topk2=0, batch=2, s_q=1,
                 h_q=16, h_kv=1, d=576, causal=0, plan=DUMMY, ns=DUMMY, W=8, o=DUMMY, lse=DUMMY,
                 ws=DUMMY, ws_bytes=1 << 40, out=DUMMY, out_elems=2 * 4 * 64, stream=None)

    def copy_rows(**kw):
        a = dict(probe)
        a.update(kw)
        return l.mla_debug_copy_rows(*a.values())
    assert copy_rows(out=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert copy_rows(out_elems=2 * 4 * 64 - 1) == _lib.MLA_ERR_INVALID_ARGUMENT       # [items, max_blocks, 64]
    assert copy_rows(fmt=1, out_elems=2 * 4 * 64) == _lib.MLA_ERR_INVALID_ARGUMENT    # FP8: two planes
    assert copy_rows(fmt=2) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert copy_rows(kv2=DUMMY) == _lib.MLA_ERR_INVALID_ARGUMENT                      # dual cache is sparse
    assert copy_rows(d=448) == _lib.MLA_ERR_UNSUPPORTED
    assert l.mla_validate_inputs(DUMMY, 4, DUMMY, 2, 1, None, 0, 10, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert l.mla_validate_inputs(DUMMY, 4, DUMMY, 2, 1, None, 0, 0, DUMMY, None) == _lib.MLA_ERR_INVALID_ARGUMENT


def test_product_path_does_not_use_the_oracle():
    import mla_paged_kv_get_amd
    pkg = os.path.dirname(mla_paged_kv_get_amd.__file__)
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b|\boracle\.|mla_oracle", txt, re.M), fn


def test_plan_num_workers_inverts_plan_dims():
    l = _lib.lib()
    for shape in [(64, 1, 16, 1, 0), (16, 8, 1024, 1, 2048), (32, 2, 256, 1, 0), (3, 1, 40, 1, 0)]:
        for W in (1, 7, 256):
            st, Wd, words, _ = _dims(*shape, W)
            assert st == 0 and Wd == W
            assert l.mla_plan_num_workers(words, *shape) == W
    assert l.mla_plan_num_workers(5, 64, 1, 16, 1, 0) == -1
    assert l.mla_plan_num_workers(8 * 10 + 64 + 3, 64, 1, 16, 1, 0) == -1  # not whole rows
    assert l.mla_plan_num_workers(8 + 64, 64, 1, 16, 1, 0) == -1           # header only
