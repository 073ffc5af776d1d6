"""GPU parity of the HIP path against the CPU oracle (through the C ABI).

Floating point: max|dO| <= 2e-2 against the oracle's float64 O and
max|dLSE| <= 1e-3.  Integer work (plan, num_splits, row addressing) is
compared bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc
from mla_paged_kv_get_amd import workloads as wl
from tests.helpers import Dev, compare, run_gpu, i32_dev, bits_to_dev

pytestmark = pytest.mark.gpu


def _m():
    import mla_paged_kv_get_amd as m
    return m


# ---------------------------------------------------------------------------
# Scheduler and addressing: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("W", [1, 3, 64, 256, 1000, None])
def test_plan_bit_exact(W):
    m = _m()
    rng = np.random.default_rng(123)
    cases = [
        ([37, 130], 16, 1, None),
        (list(wl.memory_bound().cache_seqlens) if W in (256, None) else list(rng.integers(1, 4097, 64)), 16, 1, None),
        (list(rng.integers(0, 300, 50)) + [0, 0, 5000], 128, 2, None),
        ([65536] * 4, 128, 8, 2048),
    ]
    if W in (256, None):
        # many items per scheduler thread, empty ones among them
        cases.append((list(rng.integers(0, 1500, 3000)), 16, 1, None))
    for lengths, h_q, s_q, topk in cases:
        sl = i32_dev(np.array(lengths))
        plan, ns = m.get_mla_metadata(sl, s_q * h_q, 1, s_q=s_q, topk=topk, num_workers=W)
        torch.cuda.synchronize()
        p = plan.cpu().numpy()
        Wg, c = int(p[0]), int(p[1])
        if W is not None:
            assert Wg == W
        items = [topk] * (len(lengths) * s_q) if topk else lengths
        ref_p, ref_ns = orc.plan(items, Wg, c)
        assert (p[:ref_p.size] == ref_p).all(), f"plan differs for W={Wg} lengths={lengths[:5]}"
        assert (p[ref_p.size:] == 0).all()          # the single-launch arrival counters
        assert (ns.cpu().numpy() == ref_ns).all()


@pytest.mark.parametrize("lengths,W", [
    ([512000] * 140, 4096),     # W' T >= 2^32, items marking their workers
    ([64000] * 66, 70000),      # W' T >= 2^32, workers searching the item starts
    ([6400] * 64, 5000),        # W' T < 2^32, workers searching the item starts
    ([100000] * 3, 256),        # items reaching over 32 workers each
])
def test_plan_bit_exact_division_paths(lengths, W):
    # the scheduler's quotients by T and W' go by multiplication or in double
    # precision, and its rows come from item marks or from a search
    m = _m()
    sl = i32_dev(np.array(lengths))
    plan, ns = m.get_mla_metadata(sl, 16, 1, num_workers=W)
    torch.cuda.synchronize()
    p = plan.cpu().numpy()
    c = int(p[1])
    ref_p, ref_ns = orc.plan(lengths, W, c)
    assert (p[:ref_p.size] == ref_p).all()
    assert (ns.cpu().numpy() == ref_ns).all()


@pytest.mark.parametrize("items,W", [(256, 256), (257, 256), (256, 257), (1, 256), (255, 1),
                                     (16384, 64), (16385, 64), (16385, 2048)])
def test_plan_bit_exact_path_boundaries(items, W):
    # the edges between the scheduler's paths: one item and one worker per
    # thread (up to 256 of each), items in LDS (up to 16384), no per-item LDS state
    m = _m()
    rng = np.random.default_rng(items + W)
    lengths = [int(x) for x in rng.integers(0, 900, items)]
    sl = i32_dev(np.array(lengths))
    plan, ns = m.get_mla_metadata(sl, 16, 1, num_workers=W)
    torch.cuda.synchronize()
    p = plan.cpu().numpy()
    ref_p, ref_ns = orc.plan(lengths, W, int(p[1]))
    assert (p[:ref_p.size] == ref_p).all(), f"{(p[:ref_p.size] != ref_p).sum()} plan words differ"
    assert (ns.cpu().numpy() == ref_ns).all()


@pytest.mark.parametrize("case", ["dense", "dense-grouped", "sparse", "sparse-dual", "axis-past-2-31"])
def test_plan_bit_exact_past_lds_items(case):
    # more than 16384 items: the scheduler that keeps no per-item state in LDS
    m = _m()
    rng = np.random.default_rng(91)
    topk, topk2, s_q, h_q, h_kv, W = None, 0, 1, 16, 1, 256
    if case == "dense":
        lengths = [int(x) for x in rng.integers(0, 700, 17000)]
    elif case == "dense-grouped":                       # 9000 sequences x 2 latent heads
        lengths, h_q, h_kv, W = [int(x) for x in rng.integers(1, 3000, 9000)], 32, 2, 64
    elif case == "sparse":                              # one sequence, 16500 query tokens
        lengths, topk, s_q, W = [20000], 100, 16500, 37
    elif case == "sparse-dual":
        lengths, topk, topk2, s_q, W = [5000, 9000], 64, 32, 8300, 200
    else:
        lengths, W = [int(x) for x in rng.integers(2**30, 2**31 - 1, 16400)], 64
    sl = i32_dev(np.array(lengths))
    plan, ns = m.get_mla_metadata(sl, s_q * h_q // h_kv, h_kv, s_q=s_q, topk=topk, num_workers=W,
                                  topk2=topk2)
    torch.cuda.synchronize()
    p = plan.cpu().numpy()
    if topk:
        tiles = -(-topk // 64) + -(-topk2 // 64)
        items = [64 * tiles] * (len(lengths) * s_q * h_kv)
    else:
        items = [L for L in lengths for _ in range(h_kv)]
    assert len(items) > 16384
    ref_p, ref_ns = orc.plan(items, W, int(p[1]))
    assert (p[:ref_p.size] == ref_p).all(), f"{case}: {(p[:ref_p.size] != ref_p).sum()} plan words differ"
    assert (p[ref_p.size:] == 0).all()          # the single-launch arrival counters
    assert (ns.cpu().numpy() == ref_ns).all()


@pytest.mark.parametrize("case", ["dense-random", "dense-halves", "sparse", "search"])
def test_plan_bit_exact_axis_past_2_31(case):
    # total cost past 2^31 (lengths near 2^31): the scheduler's 64-bit axis
    m = _m()
    rng = np.random.default_rng(77)
    topk, s_q, h_q, W = None, 1, 16, 256
    if case == "dense-random":
        lengths = [int(x) for x in rng.integers(2**30, 2**31 - 1, 120)] + [0, 5, 2**31 - 1]
    elif case == "dense-halves":
        lengths, W = [64 * (2**25 - 1)] * 70, 140       # two workers per item, exactly
    elif case == "sparse":
        lengths, topk, s_q, h_q, W = [1000] * 100, 2**30, 2, 128, 1000
    else:
        lengths, W = [int(x) for x in rng.integers(2**29, 2**31 - 1, 300)], 5000   # no marking
    sl = i32_dev(np.array(lengths))
    plan, ns = m.get_mla_metadata(sl, s_q * h_q, 1, s_q=s_q, topk=topk, num_workers=W)
    torch.cuda.synchronize()
    p = plan.cpu().numpy()
    items = [topk] * (len(lengths) * s_q) if topk else lengths
    ref_p, ref_ns = orc.plan(items, W, int(p[1]))
    T = (int(ref_p[6]) & 0xFFFFFFFF) + (int(ref_p[7]) << 32)
    assert T >= 2**31
    assert (p[:ref_p.size] == ref_p).all(), f"{case}: {(p[:ref_p.size] != ref_p).sum()} plan words differ"
    assert (ns.cpu().numpy() == ref_ns).all()


@pytest.mark.parametrize("h_q", [16, 128])
def test_all_sequences_empty(h_q):
    # every item has no key: no worker gets a block, every row is o = 0, lse = -inf
    w = wl.build("all-empty", 38, np.zeros(5, dtype=np.int64), B=5, s_q=2, h_q=h_q, num_pages=4,
                 causal=True, poison=True)
    for phases in (3, 4):
        m = _m()
        d = Dev(w)
        plan, ns = m.get_mla_metadata(d.sl, 2 * h_q, 1, s_q=2)
        o, lse = m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, plan, ns, causal=True, phases=phases)
        torch.cuda.synchronize()
        assert (o.float().cpu().numpy() == 0).all()
        assert np.isneginf(lse.cpu().numpy()).all()
        assert (ns.cpu().numpy() == 0).all()


def test_empty_batch():
    # no sequence: every worker row is empty, no split, and the decode writes nothing
    m = _m()
    sl = i32_dev(np.zeros(0, dtype=np.int32))
    plan, ns = m.get_mla_metadata(sl, 16, 1)
    torch.cuda.synchronize()
    p = plan.cpu().numpy()
    ref_p, ref_ns = orc.plan([], int(p[0]), int(p[1]))
    assert (p[:ref_p.size] == ref_p).all()
    assert (ns.cpu().numpy() == ref_ns).all()
    q = torch.zeros((0, 1, 16, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 1, 576), dtype=torch.bfloat16, device="cuda")
    bt = i32_dev(np.zeros((0, 1), dtype=np.int32))
    o, lse = m.mla_decode_with_kvcache(q, kv, bt, sl, 512, plan, ns)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (0, 1, 16, 512) and tuple(lse.shape) == (0, 1, 16)


def test_plan_bit_exact_dual_cache_lists():
    # sparse items of the dual-cache decode have ceil(topk / 64) + ceil(topk2 / 64) tiles
    m = _m()
    sl = i32_dev(np.array([5000, 300, 64]))
    for topk, topk2, W in [(2048, 512, 64), (100, 1, 7), (64, 0, 5), (65, 700, 256)]:
        plan, ns = m.get_mla_metadata(sl, 2 * 128, 1, s_q=2, topk=topk, topk2=topk2, num_workers=W)
        torch.cuda.synchronize()
        p = plan.cpu().numpy()
        tiles = -(-topk // 64) + -(-topk2 // 64)
        ref_p, ref_ns = orc.plan([64 * tiles] * 6, W, int(p[1]))
        assert (p[:ref_p.size] == ref_p).all(), (topk, topk2, W)
        assert (ns.cpu().numpy() == ref_ns).all()


# ---------------------------------------------------------------------------
# Decode parity on the named workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("poison", [False, True])
def test_tiny(poison):
    w = wl.tiny(poison=poison)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"tiny poison={poison}")


@pytest.mark.parametrize("poison", [False, True])
def test_memory_bound_full(poison):
    w = wl.memory_bound(poison=poison)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"memory-bound poison={poison}")


def test_near_ridge_full():
    w = wl.near_ridge()
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="near-ridge")


@pytest.mark.parametrize("W", [200, 700])
def test_near_ridge_full_split(W):
    # most sequences split over several workers: the merge of partials at full size
    w = wl.near_ridge()
    o, lse, plan = run_gpu(Dev(w), num_workers=W)
    ns = plan[1].cpu().numpy()
    assert (np.diff(ns) > 1).mean() > 0.5
    compare(w, o, lse, label=f"near-ridge W={W}")


def test_mtp_causal_full():
    w = wl.mtp_causal()
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="mtp-causal")


def test_sparse_topk_full():
    w = wl.sparse_topk()
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="sparse-topk")


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
EDGE_L = [1, 2, 63, 64, 65, 127, 128, 129, 0, 200, 4097]


@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
def test_edge_lengths(h_q):
    w = wl.build("edge", 31, np.array(EDGE_L), B=len(EDGE_L), s_q=1, h_q=h_q, num_pages=200, poison=True)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"edge h_q={h_q}")


@pytest.mark.parametrize("h_q,s_q", [(16, 2), (8, 2), (128, 2), (64, 4)])
def test_causal_edges(h_q, s_q):
    L = [1, 2, 3, 64, 65, 130, 0]
    w = wl.build("causal-edge", 32, np.array(L), B=len(L), s_q=s_q, h_q=h_q, num_pages=40,
                 causal=True, poison=True)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"causal h_q={h_q} s_q={s_q}")


@pytest.mark.parametrize("h_q,s_q,causal", [(100, 1, False), (40, 3, True)])
def test_wide_rows_not_multiple_of_32(h_q, s_q, causal):
    # 100 and 120 rows per item: the 128-row variant's partials are 32-row blocks,
    # the last one part padding; whole items and several split counts
    L = [1, 65, 300, 2049, 0]
    w = wl.build("rows-odd", 50 + s_q, np.array(L), B=len(L), s_q=s_q, h_q=h_q, num_pages=60,
                 causal=causal, poison=True)
    for W in (None, 3, 7):
        o, lse, _ = run_gpu(Dev(w), num_workers=W)
        compare(w, o, lse, label=f"h_q={h_q} s_q={s_q} W={W}")


def test_noncausal_multi_token():
    w = wl.build("mtp-noncausal", 33, np.array([100, 7, 300]), B=3, s_q=2, h_q=64, num_pages=20)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="s_q=2 non-causal")


def test_sparse_pads_and_empty():
    w = wl.build("sparse-pad", 34, np.array([300, 90, 0]), B=3, s_q=2, h_q=128, num_pages=20,
                 poison=True, topk=None)
    rng = np.random.default_rng(4)
    idx = np.full((3, 2, 150), -1, dtype=np.int32)
    idx[0, 0, :100] = rng.choice(300, 100, replace=False)
    idx[0, 1, :150] = rng.choice(300, 150, replace=False)
    idx[0, 1, 7] = 300          # out of range -> padding
    idx[1, 0, 20:40] = np.arange(20)
    # idx[1, 1] all padding; sequence 2 is empty
    w.indices = idx
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="sparse pads")
    lg = lse.cpu().numpy()
    assert np.isneginf(lg[1, 1]).all() and np.isneginf(lg[2]).all()
    assert (o[1, 1].float().cpu().numpy() == 0).all()


# ---------------------------------------------------------------------------
# Several latent heads (h_kv > 1): query head h reads latent head h // (h_q / h_kv)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("h_kv,h_q,s_q,causal", [
    (2, 16, 1, False),      # 8 rows per item: 16-row tiles
    (4, 64, 2, True),       # 32 rows per item: 64-row tiles, causal
    (2, 256, 1, False),     # 128 rows per item: one 128-row tile
    (2, 256, 2, True),      # 256 rows per item: two 128-row tiles, causal
    (8, 64, 4, True),       # 32 rows per item from four tokens of 8 heads
])
def test_grouped_latent_heads(h_kv, h_q, s_q, causal):
    L = [1, 64, 65, 300, 0, 2049]
    w = wl.build("grouped", 40 + h_kv, np.array(L), B=len(L), s_q=s_q, h_q=h_q, h_kv=h_kv,
                 num_pages=60, causal=causal, poison=True)
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"h_kv={h_kv} h_q={h_q} s_q={s_q} causal={causal}")
    o2, lse2, _ = run_gpu(Dev(w), num_workers=3)
    compare(w, o2, lse2, label=f"h_kv={h_kv} W=3")


def test_sparse_prefill_sampled():
    # 4096 query tokens of one sequence, each with 2048 of the keys it may see:
    # every output finite, 64 tokens spread over the sequence (both ends, and
    # the tokens whose item boundaries fall at worker ends of the plan) against
    # the oracle
    w = wl.sparse_prefill()
    o, lse, plan = run_gpu(Dev(w))
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rows = plan[0].cpu().numpy()[8:].reshape(-1, 8)[: int(plan[0][0].item())]
    ends = sorted({int(x) for x in rows[:, 0] if x >= 0} | {int(x) for x in rows[:, 2] if x >= 0})
    toks = sorted(set(np.linspace(0, 4095, 40).astype(int)) | set(ends[:: max(1, len(ends) // 24)]))
    compare(w, o, lse, items=[(0, int(t)) for t in toks], label="sparse-prefill")


def test_sparse_prefill_past_lds_items():
    # 16500 query tokens of 16 rows (16500 items: the plan without per-item LDS
    # state; over 64 items per worker): every output finite, tokens on both
    # sides of item 16384 and spread over the rest against the oracle, and the
    # single-launch decode bit for bit equal to the two launches
    T, ctx, k = 16500, 100, 64
    w = wl.build("prefill-16k", 62, np.array([ctx + T]), B=1, s_q=T, h_q=16,
                 num_pages=(ctx + T) // 64 + 4, topk=None)
    rng = np.random.default_rng(63)
    idx = np.full((1, T, k), -1, dtype=np.int32)
    for t in range(T):
        n = min(k, ctx + t + 1)
        idx[0, t, :n] = rng.choice(ctx + t + 1, n, replace=False)
    w.indices = idx
    d = Dev(w)
    o, lse, plan = run_gpu(d)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    toks = sorted({0, 1, 16383, 16384, 16385, T - 1} | set(int(x) for x in np.linspace(0, T - 1, 14)))
    compare(w, o, lse, items=[(0, t) for t in toks], label="prefill T=16500")
    m = _m()
    ws = torch.empty(m.workspace_bytes(1, T, T * 16, 1, k, 512, int(plan[0][0].item())), dtype=torch.uint8,
                     device="cuda")
    o1 = torch.empty_like(o)
    lse1 = torch.empty_like(lse)
    m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, plan[0], plan[1], causal=w.causal, indices=d.idx,
                              out=(o1, lse1), workspace=ws, phases=4)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o.view(torch.int16)) and torch.equal(lse1, lse)


@pytest.mark.parametrize("h_q", [16, 128])
def test_sparse_prefill_small_full(h_q):
    # every query token checked: T = 200 new tokens after 100 of context, causal
    # index lists with padding where a token sees fewer keys than top-k
    T, ctx, k = 200, 100, 160
    w = wl.build("prefill-small", 60, np.array([ctx + T]), B=1, s_q=T, h_q=h_q, num_pages=12,
                 poison=True, topk=None)
    rng = np.random.default_rng(61)
    idx = np.full((1, T, k), -1, dtype=np.int32)
    for t in range(T):
        n = min(k, ctx + t + 1)
        idx[0, t, :n] = rng.choice(ctx + t + 1, n, replace=False)
    w.indices = idx
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"prefill T={T} h_q={h_q}")


def test_grouped_heads_workload_full():
    w = wl.grouped_heads()
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label="grouped-heads b32 h128 hkv8")


@pytest.mark.parametrize("h_kv,h_q", [(2, 32), (4, 256), (2, 256)])   # 16, 64 and 128 rows per item
def test_grouped_latent_heads_sparse(h_kv, h_q):
    w = wl.build("grouped-sparse", 50 + h_kv, np.array([700, 129, 2000]), B=3, s_q=2, h_q=h_q,
                 h_kv=h_kv, num_pages=60, poison=True, topk=128)
    w.indices[1, 0, 5:9] = -1
    o, lse, _ = run_gpu(Dev(w))
    compare(w, o, lse, label=f"sparse h_kv={h_kv} h_q={h_q}")


def test_grouped_plan_bit_exact():
    m = _m()
    lengths = [37, 130, 0, 5000, 64]
    for h_kv, s_q, topk in [(2, 1, None), (4, 2, None), (2, 2, 256)]:
        plan, ns = m.get_mla_metadata(i32_dev(np.array(lengths)), s_q * 16, h_kv, s_q=s_q, topk=topk,
                                      num_workers=7)
        torch.cuda.synchronize()
        p = plan.cpu().numpy()
        items = [topk] * (len(lengths) * s_q * h_kv) if topk else list(np.repeat(lengths, h_kv))
        ref_p, ref_ns = orc.plan(items, int(p[0]), int(p[1]))
        assert (p[:ref_p.size] == ref_p).all() and (ns.cpu().numpy() == ref_ns).all(), (h_kv, s_q, topk)
        assert (p[ref_p.size:] == 0).all()


def test_softmax_scale():
    w = wl.tiny()
    o, lse, _ = run_gpu(Dev(w), softmax_scale=0.11)
    compare(w, o, lse, softmax_scale=0.11, label="scale 0.11")


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("W", [1, 5, 33, 700])
def test_split_count_invariance(W):
    w = wl.build("splits", 35, np.array([4096, 1, 2000, 777, 64, 65]), B=6, s_q=2, h_q=16,
                 num_pages=200, causal=True, poison=True)
    o, lse, plan = run_gpu(Dev(w), num_workers=W)
    compare(w, o, lse, label=f"W={W}")


def test_split_count_invariance_wide_rows():
    w = wl.build("splits-wide", 36, np.array([3000, 129, 64]), B=3, s_q=1, h_q=128, num_pages=80)
    for W in (1, 4, 90):
        o, lse, _ = run_gpu(Dev(w), num_workers=W)
        compare(w, o, lse, label=f"h128 W={W}")


@pytest.mark.parametrize("h_q,topk", [(16, None), (128, None), (16, 32)])
def test_many_items_per_worker(h_q, topk):
    # Over 64 items per worker: the lengths and split slots of items past the
    # first 64 are read one by one instead of from the per-lane tables.
    rng = np.random.default_rng(77)
    L = rng.integers(0, 130, size=150)           # empty, one-page and two-page sequences
    if topk is not None:
        L = np.maximum(L, topk)
    w = wl.build("many-items", 77, L, B=len(L), s_q=1, h_q=h_q, num_pages=400, poison=True,
                 topk=topk, rng=rng)
    for W in (1, 2):
        o, lse, plan = run_gpu(Dev(w), num_workers=W)
        rows = plan[0].cpu().numpy()[8:8 * (W + 1)].reshape(W, 8)   # one row of 8 words per worker
        assert (rows[:, 2] - rows[:, 0]).max() >= 64
        compare(w, o, lse, label=f"h_q={h_q} topk={topk} W={W}")


def test_page_permutation_bit_exact():
    w = wl.memory_bound()
    d = Dev(w)
    o1, l1, plan = run_gpu(d)
    perm = np.random.default_rng(8).permutation(w.kv.shape[0])
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    d.kv = bits_to_dev(kv2)
    d.bt = i32_dev(perm[w.block_table].astype(np.int32))
    o2, l2, _ = run_gpu(d, plan=plan)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_single_key_gives_v_exactly():
    w = wl.build("single", 37, np.array([1, 1, 1]), B=3, s_q=1, h_q=128, num_pages=6)
    o, lse, _ = run_gpu(Dev(w))
    og = o.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(3):
        v0 = w.kv[w.block_table[b, 0], 0, 0, :512]
        assert (og[b, 0] == v0[None, :]).all()
    compare(w, o, lse, label="single key")


def test_deterministic():
    w = wl.mtp_causal()
    d = Dev(w)
    o1, l1, plan = run_gpu(d)
    o2, l2, _ = run_gpu(d, plan=plan)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_plan_reused_across_layers():
    # one plan, several "layers" (different q and cache, same lengths)
    m = _m()
    base = wl.build("layers", 38, np.array([500, 33, 1200]), B=3, s_q=1, h_q=16, num_pages=40)
    d = Dev(base)
    plan = m.get_mla_metadata(d.sl, 16, 1)
    for layer in range(3):
        w = wl.build("layers", 100 + layer, np.array([500, 33, 1200]), B=3, s_q=1, h_q=16, num_pages=40)
        dl = Dev(w)
        dl.sl = d.sl
        o, lse, _ = run_gpu(dl, plan=plan)
        compare(w, o, lse, label=f"layer {layer}")


def test_validate_inputs():
    m = _m()
    w = wl.memory_bound()
    bt, sl = i32_dev(w.block_table), i32_dev(w.cache_seqlens)
    assert m.validate_inputs(bt, sl, w.kv.shape[0]) == 0
    bad = w.block_table.copy()
    bad[3, 0] = w.kv.shape[0] + 5
    assert m.validate_inputs(i32_dev(bad), sl, w.kv.shape[0]) >= 1
    ws = wl.sparse_topk(B=2)
    assert m.validate_inputs(i32_dev(ws.block_table), i32_dev(ws.cache_seqlens), ws.kv.shape[0],
                             indices=i32_dev(ws.indices)) == 0


def test_phase_split_equals_one_call():
    m = _m()
    w = wl.build("phases", 39, np.array([4096, 1, 2000, 777, 64, 65, 0]), B=7, s_q=2, h_q=16,
                 num_pages=200, causal=True, poison=True)
    d = Dev(w)
    plan, ns = m.get_mla_metadata(d.sl, 32, 1, num_workers=37)
    o3, l3 = m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, plan, ns, causal=True)
    o1 = torch.empty_like(o3)
    l1 = torch.empty_like(l3)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, plan, ns, causal=True, out=(o1, l1),
                              workspace=ws, phases=1)
    m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, plan, ns, causal=True, out=(o1, l1),
                              workspace=ws, phases=2)
    torch.cuda.synchronize()
    assert torch.equal(o3.view(torch.int16), o1.view(torch.int16)) and torch.equal(l3, l1)
    compare(w, o3, l3, label="phases")


def test_graph_capture_replays_match_eager():
    """The whole step (plan, split decode, merge) captured in a HIP graph: every
    replay, with eager work and synchronizations in between, gives the eager
    result bit for bit (the path records no memset and allocates nothing inside
    the library), and that result matches the oracle."""
    m = _m()
    w = wl.build("graph", 41, np.array([1500, 64, 1, 3000, 700]), B=5, s_q=1, h_q=16,
                 num_pages=200, causal=False, poison=True)
    d = Dev(w)
    plan0, _ = m.get_mla_metadata(d.sl, 16, 1, num_workers=23)
    W = int(plan0[0].item())
    o = torch.empty((w.B, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, 1, 16), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(m.workspace_bytes(w.B, 1, 16, 1, 0, 512, W), 16), dtype=torch.uint8, device="cuda")

    def step():
        p, n = m.get_mla_metadata(d.sl, 16, 1, num_workers=23)
        m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, p, n, out=(o, lse), workspace=ws, phases=1)
        m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, p, n, out=(o, lse), workspace=ws, phases=2)

    step()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    compare(w, o_ref, l_ref, label="graph eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        o.fill_(0)
        lse.fill_(0)
        if rep == 2:
            step()                               # eager work between replays
        torch.cuda.synchronize()
        o.fill_(0)
        lse.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"replay {rep}: O differs"
        assert torch.equal(lse, l_ref), f"replay {rep}: LSE differs"
