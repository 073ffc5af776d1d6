"""Shared helpers of the test suite: device copies of workloads and comparisons."""
from __future__ import annotations

import numpy as np
import torch

from oracle import mla_oracle as orc

O_TOL = 2e-2      # max |O_gpu - O_oracle| (bf16 output, inputs ~ N(0, 1))
LSE_TOL = 1e-3    # max |LSE_gpu - LSE_oracle|


def bits_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def kv_to_dev(a: np.ndarray) -> torch.Tensor:
    """bf16 cache (uint16 bit patterns) or packed FP8 cache (uint8 rows) to the GPU."""
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return bits_to_dev(a)


def i32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class Dev:
    """Device copies of a workload's inputs."""

    def __init__(self, w):
        self.w = w
        self.q = bits_to_dev(w.q)
        self.kv = kv_to_dev(w.kv)
        self.bt = i32_dev(w.block_table)
        self.sl = i32_dev(w.cache_seqlens)
        self.idx = i32_dev(w.indices) if w.indices is not None else None
        self.aux = None
        if w.aux is not None:
            kv2, bt2, sl2, idx2 = w.aux
            self.aux = (kv_to_dev(kv2), i32_dev(bt2), i32_dev(sl2), i32_dev(idx2))


def run_gpu(d: Dev, num_workers=None, plan=None, softmax_scale=None):
    import mla_paged_kv_get_amd as m
    w = d.w
    if plan is None:
        h_kv = w.kv.shape[2]
        topk2 = w.aux[3].shape[2] if d.aux is not None else 0
        plan = m.get_mla_metadata(d.sl, w.s_q * w.h_q // h_kv, h_kv, s_q=w.s_q, topk=w.topk,
                                  num_workers=num_workers, topk2=topk2, fp8=w.kv.dtype == np.uint8)
    o, lse = m.mla_decode_with_kvcache(d.q, d.kv, d.bt, d.sl, 512, plan[0], plan[1], causal=w.causal,
                                       softmax_scale=softmax_scale, indices=d.idx, aux=d.aux)
    torch.cuda.synchronize()
    return o, lse, plan


def o_to_f64(o: torch.Tensor) -> np.ndarray:
    return o.float().cpu().numpy().astype(np.float64)


def compare(w, o, lse, items=None, softmax_scale=None, label=""):
    """Compare GPU outputs with the oracle on the given (b, s) items (all by default)."""
    O_ref, L_ref = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, causal=w.causal,
                              softmax_scale=softmax_scale, indices=w.indices, items=items, aux=w.aux)
    og = o_to_f64(o)
    lg = lse.cpu().numpy().astype(np.float64)
    todo = items if items is not None else [(b, s) for b in range(w.B) for s in range(w.s_q)]
    worst_o = 0.0
    worst_l = 0.0
    for b, s in todo:
        assert np.isfinite(og[b, s]).all(), f"{label}: non-finite O at item {(b, s)}"
        do = np.abs(og[b, s] - O_ref[b, s]).max()
        ref_l = L_ref[b, s]
        same_inf = np.isneginf(ref_l) & np.isneginf(lg[b, s])
        with np.errstate(invalid="ignore"):          # -inf - -inf where both are empty
            dl = np.where(same_inf, 0.0, np.abs(lg[b, s] - ref_l))
        assert not np.isnan(dl).any(), f"{label}: LSE NaN at {(b, s)}"
        worst_o = max(worst_o, float(do))
        worst_l = max(worst_l, float(dl.max()))
    assert worst_o <= O_TOL, f"{label}: max|dO| = {worst_o:.3e} > {O_TOL}"
    assert worst_l <= LSE_TOL, f"{label}: max|dLSE| = {worst_l:.3e} > {LSE_TOL}"
    return worst_o, worst_l
