"""GPU parity of 512-value rows (d_qk = 512) and of the dual-cache sparse
decode (main + auxiliary cache, one softmax over both key sets) against the
CPU oracle, through the C ABI.  Same bar: max|dO| <= 2e-2, max|dLSE| <= 1e-3.
"""
import numpy as np
import pytest
import torch

from mla_paged_kv_get_amd import workloads as wl
from tests.helpers import Dev, compare, run_gpu

pytestmark = pytest.mark.gpu

EDGE_L = [1, 2, 63, 64, 65, 127, 128, 129, 0, 200, 4097]


@pytest.mark.parametrize("h_q", [16, 128])
def test_d512_edge_lengths(h_q):
    w = wl.build("edge-512", 80, np.array(EDGE_L), B=len(EDGE_L), s_q=1, h_q=h_q, num_pages=200,
                 poison=True, d_qk=512)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"d512 edge h_q={h_q}")


@pytest.mark.parametrize("h_q,s_q,h_kv", [(16, 2, 1), (128, 2, 1), (64, 2, 2)])
def test_d512_causal(h_q, s_q, h_kv):
    L = [1, 3, 64, 65, 130, 0, 700]
    w = wl.build("causal-512", 81, np.array(L), B=len(L), s_q=s_q, h_q=h_q, h_kv=h_kv, num_pages=40,
                 causal=True, poison=True, d_qk=512)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"d512 causal h_q={h_q}")
    o2, lse2, _ = run_gpu(Dev(w), num_workers=7)
    compare(w, o2, lse2, label=f"d512 causal W=7 h_q={h_q}")


def _dual(seed, h_q, d_qk, topk, topk2, lengths, lengths2, s_q=2):
    lengths = np.array(lengths)
    w = wl.build("dual", seed, lengths, B=len(lengths), s_q=s_q, h_q=h_q,
                 num_pages=int(((lengths + 63) // 64).sum()) + 4, poison=True, d_qk=d_qk)
    rng = np.random.default_rng(seed + 1)
    idx = np.full((len(lengths), s_q, topk), -1, dtype=np.int32)
    for b, L in enumerate(lengths):
        for s in range(s_q):
            n = min(topk, int(L))
            idx[b, s, :n] = rng.choice(int(L), n, replace=False)
    idx[0, 0, 5:9] = -1
    idx[-1, -1, :] = -1                    # a token with no main key
    w.indices = idx
    return wl.add_aux_cache(w, rng, np.array(lengths2), topk2, 2 * len(lengths) + 4, poison=True)


@pytest.mark.parametrize("h_q,d_qk", [(16, 576), (16, 512), (128, 512), (64, 576)])
def test_dual_small(h_q, d_qk):
    w = _dual(82, h_q, d_qk, 100, 70, [300, 90, 129, 5], [100, 0, 65, 130])
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"dual h_q={h_q} d={d_qk}")
    o2, lse2, _ = run_gpu(Dev(w), num_workers=5)
    compare(w, o2, lse2, label=f"dual W=5 h_q={h_q} d={d_qk}")


def test_dual_no_auxiliary_keys():
    # topk2 = 0: the dual call equals the single-cache sparse call
    w = _dual(83, 16, 512, 128, 0, [300, 90], [50, 10])
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="dual topk2=0")
    d = Dev(w)
    d.aux = None
    o1, l1, _ = run_gpu(d)
    assert torch.equal(o.view(torch.int16), o1.view(torch.int16)) and torch.equal(lse, l1)


def test_dual_cache_workload_full():
    # the whole dual-cache workload (b=16, s_q=2, h_q=128, 512-value rows)
    w = wl.dual_cache()
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="dual-cache d512")
