"""The no-alloc decode (mla_decode_with_kvcache_no_alloc) against the decode
that takes a workspace.

Both run the same split and merge kernels with the same plan, so the outputs
must agree bit for bit.  Each test makes two calls in a row, the second on a
smaller input than the first, so the second runs over the scratch contents the
first left behind.  A call whose partials exceed the fixed scratch must fail
before launching anything and leave later calls working.
"""
import numpy as np
import pytest
import torch

from mla_paged_kv_get_amd import _lib
from mla_paged_kv_get_amd import workloads as wl
from tests.helpers import Dev, compare

pytestmark = pytest.mark.gpu


def _m():
    import mla_paged_kv_get_amd as m
    return m


def _plan(d, num_workers=None):
    w = d.w
    h_kv = w.kv.shape[2]
    return _m().get_mla_metadata(d.sl, w.s_q * w.h_q // h_kv, h_kv, s_q=w.s_q, topk=w.topk,
                                 num_workers=num_workers)


def _no_alloc(d, plan, ns):
    w = d.w
    o = torch.full((w.B, w.s_q, w.h_q, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.s_q, w.h_q), float("nan"), dtype=torch.float32, device="cuda")
    _m().mla_decode_with_kvcache_no_alloc(d.q, d.kv, d.bt, d.sl, 512, plan, ns, out=(o, lse),
                                          causal=w.causal, indices=d.idx)
    return o, lse


def _check_same(w, num_workers=None):
    print(f"no-alloc vs workspace decode: {w.name} B={w.B} s_q={w.s_q} h_q={w.h_q}", flush=True)
    d = Dev(w)
    plan, ns = _plan(d, num_workers)
    m = _m()
    need = m.workspace_bytes(w.B, w.s_q, w.s_q * w.h_q // w.kv.shape[2], w.kv.shape[2], w.topk or 0,
                             512, int(plan[0].item()))
    assert need <= _lib.NO_ALLOC_SCRATCH_BYTES
    o, lse = _no_alloc(d, plan, ns)
    ref_o, ref_lse = m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, plan, ns, causal=w.causal,
                                               indices=d.idx)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), f"{w.name}: O differs"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), f"{w.name}: LSE differs"
    return d, o, lse


def test_dense_large_then_small():
    _check_same(wl.NAMED["near_ridge"]())            # 128 heads, partials of 96 MiB
    _check_same(wl.NAMED["memory_bound"]())          # 16 heads, 10 MiB


def test_causal_mtp_then_ragged_small():
    _check_same(wl.NAMED["mtp_causal"](), num_workers=128)
    L = np.array([1, 63, 64, 65, 200, 0, 4097, 129])
    w = wl.build("no-alloc-ragged", 81, L, B=len(L), s_q=2, h_q=16, num_pages=300, causal=True,
                 poison=True)
    d, o, lse = _check_same(w, num_workers=37)
    compare(w, o, lse, label=w.name)                  # and the oracle, at its tolerance


def test_sparse_large_then_small():
    _check_same(wl.NAMED["sparse_topk"]())
    w = wl.build("no-alloc-sparse", 82, np.array([300, 90, 0]), B=3, s_q=2, h_q=128, num_pages=20,
                 poison=True, topk=None)
    rng = np.random.default_rng(83)
    idx = np.full((3, 2, 150), -1, dtype=np.int32)
    idx[0, 0, :100] = rng.choice(300, 100, replace=False)
    idx[0, 1, :150] = rng.choice(300, 150, replace=False)
    idx[1, 0, 20:40] = np.arange(20)
    w.indices = idx
    d, o, lse = _check_same(w, num_workers=5)
    compare(w, o, lse, label=w.name)


def test_over_the_limit_is_refused_and_later_calls_work():
    w = wl.NAMED["near_ridge"]()
    d = Dev(w)
    plan, ns = _plan(d, num_workers=1024)            # (128 + 1024) x 128 rows x 513 floats > 128 MiB
    with pytest.raises(ValueError, match="no-alloc"):
        _no_alloc(d, plan, ns)
    _check_same(wl.NAMED["tiny"]())
