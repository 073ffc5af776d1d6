"""GPU parity of the packed FP8 cache path (512 E4M3 latent codes with four
float32 block scales and 64 bf16 RoPE values per row) against the CPU oracle,
through the C ABI.  Same bar as the bf16 path: max|dO| <= 2e-2 against the
oracle's float64 O, max|dLSE| <= 1e-3.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc
from mla_paged_kv_get_amd import workloads as wl
from tests.helpers import Dev, compare, run_gpu

pytestmark = pytest.mark.gpu

EDGE_L = [1, 2, 63, 64, 65, 127, 128, 129, 0, 200, 4097]


@pytest.mark.parametrize("poison", [False, True])
def test_fp8_tiny(poison):
    w = wl.build("tiny-fp8", 70, np.array([37, 130]), B=2, s_q=1, h_q=16, num_pages=8, poison=poison,
                 kv_format="fp8")
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"fp8 tiny poison={poison}")


def test_fp8_memory_bound_full():
    w = wl.memory_bound_fp8(poison=True)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="fp8 memory-bound")


@pytest.mark.parametrize("h_q", [16, 64, 128])
def test_fp8_edge_lengths(h_q):
    w = wl.build("edge-fp8", 71, np.array(EDGE_L), B=len(EDGE_L), s_q=1, h_q=h_q, num_pages=200,
                 poison=True, kv_format="fp8")
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"fp8 edge h_q={h_q}")


@pytest.mark.parametrize("h_q,s_q,h_kv", [(16, 2, 1), (128, 2, 1), (32, 2, 2), (256, 1, 4)])
def test_fp8_causal_and_grouped(h_q, s_q, h_kv):
    L = [1, 2, 3, 64, 65, 130, 0, 700]
    w = wl.build("causal-fp8", 72, np.array(L), B=len(L), s_q=s_q, h_q=h_q, h_kv=h_kv, num_pages=40,
                 causal=True, poison=True, kv_format="fp8")
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"fp8 causal h_q={h_q} s_q={s_q} h_kv={h_kv}")
    o2, lse2, _ = run_gpu(Dev(w), num_workers=5)
    compare(w, o2, lse2, label=f"fp8 causal W=5 h_q={h_q}")


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_sparse_pads(h_q):
    w = wl.build("sparse-fp8", 73, np.array([300, 90, 0]), B=3, s_q=2, h_q=h_q, num_pages=20,
                 poison=True, topk=None, kv_format="fp8")
    rng = np.random.default_rng(74)
    idx = np.full((3, 2, 150), -1, dtype=np.int32)
    idx[0, 0, :100] = rng.choice(300, 100, replace=False)
    idx[0, 1, :150] = rng.choice(300, 150, replace=False)
    idx[0, 1, 7] = 300
    idx[1, 0, 20:40] = np.arange(20)
    w.indices = idx
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"fp8 sparse h_q={h_q}")
    lg = lse.cpu().numpy()
    assert np.isneginf(lg[1, 1]).all() and np.isneginf(lg[2]).all()


def test_fp8_sparse_topk_full():
    # the whole packed-FP8 sparse top-k workload (b=16, s_q=8, h_q=128, k=2048)
    w = wl.sparse_topk_fp8()
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="fp8 sparse-topk")


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_single_key_gives_v(h_q):
    # one key: P = 1 and LSE = its score; O is its dequantized V row (the kernel
    # rounds the scale, as a probability factor, and O to bf16: two roundings)
    w = wl.build("single-fp8", 75, np.array([1, 1]), B=2, s_q=1, h_q=h_q, num_pages=4, kv_format="fp8")
    o, lse, _ = run_gpu(Dev(w))
    og = o.float().cpu().numpy().astype(np.float64)
    for b in range(2):
        v0 = orc.fp8_rows_to_f64(w.kv[w.block_table[b, 0], 0, 0])[:512]
        np.testing.assert_allclose(og[b, 0], np.broadcast_to(v0, og[b, 0].shape), rtol=2 ** -7, atol=0)
    compare(w, o, lse, label=f"fp8 single key h_q={h_q}")


def test_fp8_split_count_invariance():
    w = wl.build("splits-fp8", 76, np.array([4096, 1, 2000, 777, 64, 65]), B=6, s_q=2, h_q=16,
                 num_pages=200, causal=True, poison=True, kv_format="fp8")
    for W in (1, 33, 700):
        o, lse, _ = run_gpu(Dev(w), num_workers=W)
        compare(w, o, lse, label=f"fp8 W={W}")


@pytest.mark.parametrize("topk", [None, 32])
def test_fp8_many_short_items(topk):
    # Items of one or two tiles back to back (16-row tiles): the query rows of
    # each come in with its first tile, through two alternating LDS slots.
    rng = np.random.default_rng(78)
    L = rng.integers(0, 130, size=150)
    if topk is not None:
        L = np.maximum(L, topk)
    w = wl.build("many-fp8", 78, L, B=len(L), s_q=1, h_q=16, num_pages=400, poison=True,
                 topk=topk, rng=rng, kv_format="fp8")
    for W in (1, 2, 37):
        o, lse, _ = run_gpu(Dev(w), num_workers=W)
        compare(w, o, lse, label=f"fp8 many items topk={topk} W={W}")


def test_fp8_plan_bit_exact_and_bf16_plan_also_valid():
    # the FP8 plan: the oracle's schedule with the 64-row variant's overhead (4)
    # and, by default, one workgroup per CU for both row tiles of every worker;
    # the FP8 decode of the full sparse top-k workload on it, and on the bf16
    # call's plan (any plan is valid for either decode), against the oracle
    import mla_paged_kv_get_amd as m
    w = wl.sparse_topk_fp8()
    d = Dev(w)
    rows = w.s_q * w.h_q
    plan8, ns8 = m.get_mla_metadata(d.sl, rows, 1, s_q=w.s_q, topk=w.topk, fp8=True)
    plan16, _ = m.get_mla_metadata(d.sl, rows, 1, s_q=w.s_q, topk=w.topk)
    torch.cuda.synchronize()
    p = plan8.cpu().numpy()
    W8, W16 = int(p[0]), int(plan16[0].item())
    assert int(p[1]) == 4 and W8 * 2 == W16                 # 64-row tiles: two per worker
    ref_p, ref_ns = orc.plan([64 * (-(-w.topk // 64))] * (w.B * w.s_q), W8, 4)
    assert (p[:ref_p.size] == ref_p).all()
    assert (ns8.cpu().numpy() == ref_ns).all()
    o8, lse8, _ = run_gpu(d, plan=(plan8, ns8))
    compare(w, o8, lse8, label="fp8 sparse top-k, FP8 plan")
    plan16, ns16 = m.get_mla_metadata(d.sl, rows, 1, s_q=w.s_q, topk=w.topk)
    o16, lse16, _ = run_gpu(d, plan=(plan16, ns16))
    compare(w, o16, lse16, label="fp8 sparse top-k, bf16 plan")
