"""The single-launch decode (phases = 4: the decode kernel merges the
partials of split items itself and writes the items without keys) against the
two-launch decode (bit for bit) and the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from mla_paged_kv_get_amd import workloads as wl
from tests.helpers import Dev, compare

pytestmark = pytest.mark.gpu


def _m():
    import mla_paged_kv_get_amd as m
    return m


def _run(d, plan, phases, ws):
    m = _m()
    w = d.w
    o = torch.empty((w.B, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.s_q, w.h_q), dtype=torch.float32, device="cuda")
    m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, plan[0], plan[1], causal=w.causal, indices=d.idx,
                              out=(o, lse), workspace=ws, phases=phases, aux=d.aux)
    torch.cuda.synchronize()
    return o, lse


def _plan(d, W=None):
    m = _m()
    w = d.w
    h_kv = w.kv.shape[2]
    topk2 = w.aux[3].shape[2] if w.aux is not None else 0
    return m.get_mla_metadata(d.sl, w.s_q * w.h_q // h_kv, h_kv, s_q=w.s_q, topk=w.topk, num_workers=W,
                              topk2=topk2)


def _cases():
    rng = np.random.default_rng(90)
    sp = wl.build("sparse-pad", 91, np.array([300, 90, 0]), B=3, s_q=2, h_q=128, num_pages=20,
                  poison=True, topk=None)
    idx = np.full((3, 2, 150), -1, dtype=np.int32)
    idx[0, 0, :100] = rng.choice(300, 100, replace=False)
    idx[0, 1, :150] = rng.choice(300, 150, replace=False)
    idx[1, 0, 20:40] = np.arange(20)
    sp.indices = idx
    return [
        ("memory-bound", lambda: wl.memory_bound(poison=True), None),
        ("mtp-causal", wl.mtp_causal, None),
        ("splits", lambda: wl.build("splits", 92, np.array([4096, 1, 2000, 777, 64, 65, 0]), B=7, s_q=2,
                                    h_q=16, num_pages=200, causal=True, poison=True), 37),
        ("sparse-pad-empty", lambda: sp, 7),
        ("fp8", lambda: wl.build("fp8", 93, np.array([3000, 0, 129, 700]), B=4, s_q=1, h_q=16, num_pages=80,
                                 poison=True, kv_format="fp8"), 21),
        ("grouped-d512", lambda: wl.build("g512", 94, np.array([2000, 65, 0, 999]), B=4, s_q=1, h_q=64,
                                          h_kv=2, num_pages=60, poison=True, d_qk=512), 19),
        ("wide-splits", lambda: wl.build("wsplits", 97, np.array([4096, 1, 2000, 777, 64, 65, 0]), B=7,
                                         s_q=1, h_q=128, num_pages=200, poison=True), 37),
        # 120 rows per item: the two-launch merge reads 32-row blocks of which the
        # last is part padding, the single launch row-major partials
        ("wide-odd-rows", lambda: wl.build("wodd", 98, np.array([3000, 1, 777, 65, 0]), B=5, s_q=3,
                                           h_q=40, num_pages=100, causal=True, poison=True), 23),
    ]


@pytest.mark.parametrize("case", range(8))
def test_single_launch_equals_two_launches(case):
    name, make, W = _cases()[case]
    w = make()
    d = Dev(w)
    plan = _plan(d, W)
    m = _m()
    h_kv = w.kv.shape[2]
    Wn = int(plan[0][0].item())
    need = m.workspace_bytes(w.B, w.s_q, w.s_q * w.h_q // h_kv, h_kv, w.topk or 0, 512, Wn)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o3, l3 = _run(d, plan, 3, ws)
    for rep in range(2):        # the arrival counters come back to zero after every call
        o4, l4 = _run(d, plan, 4, ws)
        assert torch.equal(o3.view(torch.int16), o4.view(torch.int16)), f"{name}: O differs (call {rep})"
        assert torch.equal(l3, l4), f"{name}: LSE differs (call {rep})"
    items = None if w.B * w.s_q <= 64 else [(0, 0), (w.B - 1, w.s_q - 1), (w.B // 2, 0)]
    compare(w, o4, l4, items=items, label=f"single launch {name}")


def test_single_launch_plan_counters_left_zero():
    # the plan's arrival counters are zero after the plan and after every single-launch call,
    # and one workspace serves calls of two shapes in a row
    ws = torch.empty(1 << 26, dtype=torch.uint8, device="cuda")
    for seed, lengths in ((95, [4096, 1, 300, 0, 77]), (96, [65, 2000])):
        w = wl.build("reuse", seed, np.array(lengths), B=len(lengths), s_q=1, h_q=16, num_pages=120, poison=True)
        d = Dev(w)
        plan = _plan(d, 9)
        torch.cuda.synchronize()
        words = 8 * (int(plan[0][0].item()) + 1)
        assert int(plan[0][words:].abs().sum()) == 0
        for _ in range(2):
            o4, l4 = _run(d, plan, 4, ws)
            assert int(plan[0][words:].abs().sum()) == 0
            compare(w, o4, l4, label=f"reuse {lengths}")
