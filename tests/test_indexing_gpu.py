"""Bit-exact indexing of the decode kernels, read from the kernels themselves.

mla_debug_copy_rows runs the split decode kernel and has it record, from the
registers its tile copies use, the byte offset of every cache row it reads.
The expected offsets come from the page-table definition ("What is FlashMLA",
topnet.top: 64-token pages reached through block_table, section "FlashMLA의
주요 특성" and the installation-and-use section, step 3) via
oracle.physical_rows: row (page * 64 + slot) of latent head g sits at byte
((page * 64 + slot) * h_kv + g) * row_bytes.

Keys that are not in the key set (slots past L in a sequence's last page,
index-list padding) are never read from outside the sequence: the kernels
read a valid row of the same sequence instead and mask the score.  Which row
that is is this library's convention, stated in the decode kernel and checked
here exactly: past L, the last valid slot of the same page; padding, the
sequence's token 0 (the pool's row 0 for a sequence with no row in that
cache).  Tiles no run reads are never written (-1).
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc
from mla_paged_kv_get_amd import workloads as wl
from tests.helpers import Dev

pytestmark = pytest.mark.gpu


def _m():
    import mla_paged_kv_get_amd as m
    return m


def _row_bytes(w):
    return w.kv.shape[3] * w.kv.itemsize


def expected_dense(w):
    h_kv = w.kv.shape[2]
    rb = _row_bytes(w)
    mb = w.block_table.shape[1]
    exp = np.full((w.B * h_kv, mb, 64), -1, dtype=np.int64)
    for b in range(w.B):
        L = int(w.cache_seqlens[b])
        for t in range(-(-L // 64)):
            nvalid = min(64, L - 64 * t)
            pos = 64 * t + np.minimum(np.arange(64), nvalid - 1)     # past L: the last valid slot
            rows = orc.physical_rows(w.block_table, b, pos)
            for g in range(h_kv):
                exp[b * h_kv + g, t] = (rows * h_kv + g) * rb
    return exp


def _list_rows(bt, b, idx, L, h_kv, g, rb):
    """Offsets of the rows a tile of index-list entries reads (padding: token 0)."""
    ok = (idx >= 0) & (idx < L)
    pos = np.where(ok, idx, 0)
    if L > 0:
        rows = orc.physical_rows(bt, b, pos)
    else:
        rows = np.zeros(idx.shape, dtype=np.int64)      # no row of the sequence: pool row 0
    return (rows * h_kv + g) * rb


def expected_sparse(w, kv_delta=0):
    h_kv = w.kv.shape[2]
    rb = _row_bytes(w)
    topk = w.indices.shape[2]
    nb1 = -(-topk // 64)
    topk2 = 0 if w.aux is None else w.aux[3].shape[2]
    nb = nb1 + -(-topk2 // 64)
    exp = np.full((w.B * w.s_q * h_kv, nb, 64), -1, dtype=np.int64)
    for b in range(w.B):
        L = int(w.cache_seqlens[b])
        for s in range(w.s_q):
            idx = np.full(nb1 * 64, -1, dtype=np.int64)
            idx[:topk] = w.indices[b, s]
            for g in range(h_kv):
                item = (b * w.s_q + s) * h_kv + g
                exp[item, :nb1] = _list_rows(w.block_table, b, idx, L, h_kv, g, rb).reshape(nb1, 64)
                if topk2:
                    kv2, bt2, sl2, idx2 = w.aux
                    i2 = np.full((nb - nb1) * 64, -1, dtype=np.int64)
                    i2[:topk2] = idx2[b, s]
                    exp[item, nb1:] = (kv_delta + _list_rows(bt2, b, i2, int(sl2[b]), h_kv, g, rb)).reshape(nb - nb1, 64)
    return exp


def probe(w, num_workers=None):
    m = _m()
    d = Dev(w)
    h_kv = w.kv.shape[2]
    topk2 = 0 if w.aux is None else w.aux[3].shape[2]
    plan, ns = m.get_mla_metadata(d.sl, w.s_q * w.h_q // h_kv, h_kv, s_q=w.s_q, topk=w.topk,
                                  num_workers=num_workers, topk2=topk2)
    out = m.debug_copy_rows(d.q, d.kv, d.bt, d.sl, plan, ns, causal=w.causal, indices=d.idx, aux=d.aux)
    torch.cuda.synchronize()
    delta = 0
    if d.aux is not None:
        delta = d.aux[0].data_ptr() - d.kv.data_ptr()
    return out.cpu().numpy(), delta


def check(w, num_workers=None):
    got, delta = probe(w, num_workers)
    exp = expected_sparse(w, delta) if w.indices is not None else expected_dense(w)
    assert (got[0] == exp).all(), f"{w.name}: {(got[0] != exp).sum()} row offsets differ"
    if w.kv.dtype == np.uint8:      # packed FP8: the rows whose scales are read
        assert (got[1] == exp).all(), f"{w.name}: scale rows differ"


@pytest.mark.parametrize("name", ["tiny", "memory_bound", "near_ridge", "mtp_causal", "grouped_heads",
                                  "memory_bound_fp8"])
def test_copy_rows_dense_workloads(name):
    check(wl.NAMED[name]())


@pytest.mark.parametrize("name", ["sparse_topk", "sparse_topk_fp8", "dual_cache"])
def test_copy_rows_sparse_workloads(name):
    w = wl.NAMED[name]()
    w.indices[0, 0, :5] = [-1, 65536, 70000, -7, 3]      # padding entries among the keys
    check(w)


@pytest.mark.parametrize("W", [1, 3, 37])
def test_copy_rows_split_runs(W):
    # runs crossing item boundaries and items split over several workers
    L = np.array([1, 63, 64, 65, 200, 0, 4097, 129])
    for h_q, h_kv, s_q, causal in [(16, 1, 1, False), (128, 1, 2, True), (64, 8, 1, False),
                                   (256, 2, 1, False)]:
        w = wl.build("copy-rows", 70, L, B=len(L), s_q=s_q, h_q=h_q, h_kv=h_kv, num_pages=300,
                     causal=causal, poison=True)
        check(w, num_workers=W)
    w = wl.build("copy-rows-sparse", 71, np.array([300, 90, 0]), B=3, s_q=2, h_q=128, num_pages=20,
                 poison=True, topk=None)
    rng = np.random.default_rng(72)
    idx = np.full((3, 2, 150), -1, dtype=np.int32)
    idx[0, 0, :100] = rng.choice(300, 100, replace=False)
    idx[0, 1, :150] = rng.choice(300, 150, replace=False)
    idx[1, 0, 20:40] = np.arange(20)
    w.indices = idx
    check(w, num_workers=W)
