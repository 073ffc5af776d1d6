"""Pins for the CPU oracle (runs without a GPU).

Each test checks the oracle against something other than itself: a library
routine (torch's scaled_dot_product_attention and bfloat16 casts), a closed
form, a brute-force loop on tiny inputs, an invariant of the definition, or a
hand-worked fixture under tests/golden/.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mla_oracle as orc
from mla_paged_kv_get_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _contiguous_cache(w, b, g=0):
    """Sequence b's K rows of latent head g in logical order, built page by page
    (independent of the oracle's row arithmetic): concatenate whole pages in
    block-table order."""
    L = int(w.cache_seqlens[b])
    n = -(-L // 64)
    pages = [torch.from_numpy(w.kv[int(w.block_table[b, j])].astype(np.int32)) for j in range(n)]
    rows = torch.cat(pages, dim=0)[:L, g, :]               # [L, 576] int32 holding bf16 bits
    return rows.to(torch.int16).view(torch.bfloat16).to(torch.float64)


def _q(w, b, s):
    return torch.from_numpy(w.q[b, s].astype(np.int32)).to(torch.int16).view(torch.bfloat16).double()


def small(seed, lengths, s_q=1, h_q=16, causal=False, num_pages=None, poison=False, topk=None, h_kv=1):
    lengths = np.asarray(lengths)
    need = int(((lengths + 63) // 64).sum())
    return wl.build("t", seed, lengths, B=len(lengths), s_q=s_q, h_q=h_q,
                    num_pages=num_pages or need + 3, causal=causal, poison=poison, topk=topk, h_kv=h_kv)


# ----------------------------------------------------------------------------
# bf16 conversions
# ----------------------------------------------------------------------------
def test_bf16_upcast_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16).double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_generator_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e38], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert (ours == ref).all()


# ----------------------------------------------------------------------------
# Packed FP8 rows
# ----------------------------------------------------------------------------
def test_e4m3_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok]) and np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_closed_forms():
    # OCP E4M3: bias 7, 3 mantissa bits, e = 0 subnormal, S.1111.111 NaN, max 448
    v = orc.e4m3_to_f64(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0xB8, 0x00, 0x80, 0x7F, 0xFF, 0x3C],
                                 dtype=np.uint8))
    assert list(v[:8]) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 * 2.0 ** -9, -1.0, 0.0, -0.0]
    assert np.isnan(v[8]) and np.isnan(v[9]) and v[10] == 1.5


def _fp8_row(latent_codes, scales, rope_bits):
    r = np.empty(656, dtype=np.uint8)
    r[:512] = latent_codes
    r[512:528] = np.asarray(scales, dtype="<f4").view(np.uint8)
    r[528:] = np.asarray(rope_bits, dtype="<u2").view(np.uint8)
    return r


def test_fp8_row_layout():
    codes = np.full(512, 0x38, dtype=np.uint8)          # 1.0
    codes[130] = 0x40                                    # 2.0 in block 1
    codes[511] = 0xC4                                    # -3.0 in block 3
    rope = np.full(64, 0x3FC0, dtype=np.uint16)          # 1.5
    rope[63] = 0xC000                                    # -2.0
    v = orc.fp8_rows_to_f64(_fp8_row(codes, [0.5, 2.0, 4.0, -0.25], rope))
    assert v.shape == (576,)
    assert (v[:128] == 0.5).all() and v[128] == 2.0 and v[130] == 4.0 and (v[256:384] == 4.0).all()
    assert v[384] == -0.25 and v[511] == 0.75
    assert (v[512:575] == 1.5).all() and v[575] == -2.0


def test_fp8_decode_equals_bf16_decode_on_exact_values():
    # power-of-two scales: every dequantized value is a bf16, so the bf16 cache built from them
    # (through torch's float8 and bfloat16 conversions) must give the very same float64 result
    w = small(21, [70, 129], h_q=16, h_kv=2, causal=True, s_q=2)
    rng = np.random.default_rng(5)
    kv8 = wl.packed_fp8_rows(rng, w.kv.shape[:3])
    sc = np.exp2(rng.integers(-8, 3, size=w.kv.shape[:3] + (4,))).astype("<f4")
    kv8[..., 512:528] = sc.view(np.uint8)
    lat = torch.from_numpy(kv8[..., :512].copy()).view(torch.float8_e4m3fn).to(torch.float32)
    lat = lat * torch.from_numpy(np.repeat(sc, 128, axis=-1))
    bf = np.empty(w.kv.shape, dtype=np.uint16)
    bf[..., :512] = lat.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bf[..., 512:] = kv8[..., 528:].copy().view("<u2")
    O8, L8 = orc.decode(w.q, kv8, w.block_table, w.cache_seqlens, 512, causal=True)
    Ob, Lb = orc.decode(w.q, bf, w.block_table, w.cache_seqlens, 512, causal=True)
    assert np.array_equal(O8, Ob) and np.array_equal(L8, Lb)


def test_fp8_decode_matches_sdpa():
    w = wl.build("t8", 22, np.array([100, 1, 200]), B=3, s_q=1, h_q=16, num_pages=10, kv_format="fp8")
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    for b in range(3):
        L = int(w.cache_seqlens[b])
        pages = [w.kv[int(w.block_table[b, j]), :, 0, :] for j in range(-(-L // 64))]
        rows = np.concatenate(pages, axis=0)[:L]                       # [L, 656]
        lat = torch.from_numpy(rows[:, :512].copy()).view(torch.float8_e4m3fn).to(torch.float64)
        sc = torch.from_numpy(rows[:, 512:528].copy().view("<f4").astype(np.float64))
        rope = torch.from_numpy(rows[:, 528:].copy().view("<u2").astype(np.int32)).to(torch.int16)
        K = torch.cat([lat * sc.repeat_interleave(128, dim=1), rope.view(torch.bfloat16).double()], dim=1)
        q = _q(w, b, 0)
        ref = F.scaled_dot_product_attention(q[None, :, None, :], K[None, None].expand(1, 16, -1, -1),
                                             K[None, None, :, :512].expand(1, 16, -1, -1), scale=576 ** -0.5)
        np.testing.assert_allclose(O[b, 0], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_fp8_poison_rows_never_read():
    w = wl.build("t8p", 23, np.array([65, 3]), B=2, s_q=1, h_q=16, num_pages=6, kv_format="fp8", poison=True)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    assert np.isfinite(O).all() and np.isfinite(LSE).all()


# ----------------------------------------------------------------------------
# Decode vs. a library routine (torch SDPA in float64 on the CPU)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("lengths,h_q", [([37, 130], 16), ([1, 64, 65, 200], 8), ([129], 32)])
def test_decode_matches_torch_sdpa(lengths, h_q):
    w = small(11, lengths, h_q=h_q)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    scale = 576 ** -0.5
    for b in range(w.B):
        K = _contiguous_cache(w, b)
        q = _q(w, b, 0)                                       # [h, 576]
        ref = F.scaled_dot_product_attention(q[None, :, None, :], K[None, None].expand(1, h_q, -1, -1),
                                             K[None, None, :, :512].expand(1, h_q, -1, -1), scale=scale)
        np.testing.assert_allclose(O[b, 0], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("h_kv,h_q", [(2, 16), (4, 8), (8, 8)])
def test_grouped_latent_heads_match_sdpa(h_kv, h_q):
    # query head h reads latent head h // (h_q / h_kv) (contiguous groups)
    w = small(12, [70, 1, 129], h_q=h_q, h_kv=h_kv, s_q=2)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    group = h_q // h_kv
    scale = 576 ** -0.5
    for b in range(w.B):
        Ks = torch.stack([_contiguous_cache(w, b, h // group) for h in range(h_q)])   # [h_q, L, 576]
        for s in range(2):
            q = _q(w, b, s)
            ref = F.scaled_dot_product_attention(q[None, :, None, :], Ks[None], Ks[None, :, :, :512], scale=scale)
            np.testing.assert_allclose(O[b, s], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)
            lse = torch.logsumexp(scale * torch.einsum("hd,hnd->hn", q, Ks), dim=1).numpy()
            np.testing.assert_allclose(LSE[b, s], lse, rtol=0, atol=1e-12)


def test_grouped_heads_equal_separate_single_head_caches():
    # h_kv latent heads == h_kv independent single-head problems on the split cache
    w = small(13, [200, 65], h_q=16, h_kv=4, causal=True, s_q=2)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, causal=True)
    for g in range(4):
        Og, Lg = orc.decode(np.ascontiguousarray(w.q[:, :, 4 * g:4 * g + 4]),
                            np.ascontiguousarray(w.kv[:, :, g:g + 1]), w.block_table, w.cache_seqlens,
                            512, causal=True)
        assert np.array_equal(O[:, :, 4 * g:4 * g + 4], Og) and np.array_equal(LSE[:, :, 4 * g:4 * g + 4], Lg)


def test_d512_rows_match_sdpa():
    # 512-value rows: K = V = the whole row, default scale 512^-0.5
    w = wl.build("t512", 24, np.array([70, 1, 129]), B=3, s_q=2, h_q=16, num_pages=8, d_qk=512,
                 causal=True)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, causal=True)
    for b in range(3):
        K = _contiguous_cache(w, b)                              # [L, 512]
        L = K.shape[0]
        for s in range(2):
            n = L - 2 + s + 1
            q = _q(w, b, s)
            ref = F.scaled_dot_product_attention(q[None, :, None, :], K[None, None, :n].expand(1, 16, -1, -1),
                                                 K[None, None, :n].expand(1, 16, -1, -1), scale=512 ** -0.5)
            np.testing.assert_allclose(O[b, s], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def _dual_small(seed, d_qk=576, topk2=40, lengths2=(100, 0, 65)):
    lengths = np.array([300, 90, 129])
    w = wl.build("dual", seed, lengths, B=3, s_q=2, h_q=16, num_pages=12, poison=True, topk=64, d_qk=d_qk)
    w.indices[1, 0, 10:20] = -1
    rng = np.random.default_rng(seed + 1)
    return wl.add_aux_cache(w, rng, np.array(lengths2), topk2, 6, poison=True)


@pytest.mark.parametrize("d_qk", [576, 512])
def test_dual_equals_one_cache_holding_both(d_qk):
    # the union over two caches == one sparse call over a single cache that holds the
    # auxiliary pages after the main ones, each sequence's auxiliary blocks appended to
    # its block table and its auxiliary positions shifted past its main blocks
    w = _dual_small(25, d_qk)
    kv2, bt2, sl2, idx2 = w.aux
    pool1 = w.kv.shape[0]
    kv = np.concatenate([w.kv, kv2], axis=0)
    nb1 = -(-w.cache_seqlens.astype(np.int64) // 64)
    mb = int((nb1 + bt2.shape[1]).max())
    bt = np.zeros((w.B, mb), dtype=np.int32)
    lens = np.zeros(w.B, dtype=np.int32)
    idx = np.full((w.B, w.s_q, w.indices.shape[2] + idx2.shape[2]), -1, dtype=np.int32)
    for b in range(w.B):
        n1 = int(nb1[b])
        bt[b, :n1] = w.block_table[b, :n1]
        bt[b, n1:n1 + bt2.shape[1]] = bt2[b] + pool1
        lens[b] = n1 * 64 + int(sl2[b])
        for s in range(w.s_q):
            m1 = w.indices[b, s]
            m1 = np.where((m1 >= 0) & (m1 < w.cache_seqlens[b]), m1, -1)
            m2 = idx2[b, s]
            m2 = np.where((m2 >= 0) & (m2 < sl2[b]), m2 + n1 * 64, -1)
            idx[b, s] = np.concatenate([m1, m2])
    O2, L2 = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, indices=w.indices, aux=w.aux)
    O1, L1 = orc.decode(w.q, kv, bt, lens, 512, indices=idx)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_dual_matches_sdpa_on_gathered_keys():
    w = _dual_small(26, 512, topk2=30)
    kv2, bt2, sl2, idx2 = w.aux
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, indices=w.indices, aux=w.aux)
    for b, s in [(0, 0), (1, 1), (2, 0)]:
        rows = []
        for cache, table, L, ix in ((w.kv, w.block_table, w.cache_seqlens[b], w.indices[b, s]),
                                    (kv2, bt2, sl2[b], idx2[b, s])):
            for j in ix[(ix >= 0) & (ix < L)]:
                rows.append(cache[int(table[b, j // 64]), j % 64, 0].astype(np.int32))
        K = torch.from_numpy(np.stack(rows)).to(torch.int16).view(torch.bfloat16).double()
        q = _q(w, b, s)
        ref = F.scaled_dot_product_attention(q[None, :, None, :], K[None, None].expand(1, 16, -1, -1),
                                             K[None, None].expand(1, 16, -1, -1), scale=512 ** -0.5)
        np.testing.assert_allclose(O[b, s], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[b, s], torch.logsumexp(512 ** -0.5 * (K @ q.T), dim=0).numpy(),
                                   rtol=0, atol=1e-12)


def test_causal_matches_sdpa_with_explicit_mask():
    # bottom-right alignment: token s of s_q sees keys 0 .. L - s_q + s
    w = small(12, [70, 5, 130], s_q=3, h_q=8, causal=True)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, causal=True)
    scale = 576 ** -0.5
    for b in range(w.B):
        K = _contiguous_cache(w, b)
        L = K.shape[0]
        for s in range(3):
            mask = torch.arange(L) <= (L - 3 + s)
            q = _q(w, b, s)
            ref = F.scaled_dot_product_attention(q[None, :, None, :], K[None, None].expand(1, 8, -1, -1),
                                                 K[None, None, :, :512].expand(1, 8, -1, -1),
                                                 attn_mask=mask[None, None, None, :], scale=scale)
            np.testing.assert_allclose(O[b, s], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# Brute force in pure Python (tiny): no max-subtraction, math.fsum, explicit gather
# ----------------------------------------------------------------------------
def _brute(qrow, K, dv, scale):
    scores = [scale * math.fsum(a * b for a, b in zip(qrow, krow)) for krow in K]
    e = [math.exp(x) for x in scores]
    den = math.fsum(e)
    o = [math.fsum(e[j] * K[j][c] for j in range(len(K))) / den for c in range(dv)]
    return o, math.log(den)


def test_decode_brute_force_tiny():
    w = small(13, [3, 66], h_q=4)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    for b in range(w.B):
        K = _contiguous_cache(w, b).tolist()
        for h in range(4):
            qrow = _q(w, b, 0)[h].tolist()
            o, lse = _brute(qrow, K, 512, 1 / 24)
            np.testing.assert_allclose(O[b, 0, h], o, rtol=0, atol=1e-12)
            assert abs(LSE[b, 0, h] - lse) < 1e-12


def test_softmax_scale_is_used():
    w = small(14, [40], h_q=2)
    O1, L1 = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, softmax_scale=0.1)
    K = _contiguous_cache(w, 0).tolist()
    o, lse = _brute(_q(w, 0, 0)[1].tolist(), K, 512, 0.1)
    np.testing.assert_allclose(O1[0, 0, 1], o, rtol=0, atol=1e-12)
    assert abs(L1[0, 0, 1] - lse) < 1e-12


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------
def test_single_key_gives_that_rows_v():
    w = small(15, [1, 1], h_q=16)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    for b in range(2):
        row = orc.bf16_to_f64(w.kv[w.block_table[b, 0], 0, 0])
        assert (O[b, 0] == row[None, :512]).all()              # V = first 512 values
        q = orc.bf16_to_f64(w.q[b, 0])
        np.testing.assert_allclose(LSE[b, 0], (q @ row) / 24.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L", [2, 63, 64, 65, 129, 300])
def test_equal_scores_give_mean_of_v(L):
    # q has zero latent part and every row has the same RoPE part, so every
    # score equals the same value S0 while V (the latent part) differs.
    w = small(16, [L], h_q=4)
    w.q[..., :512] = 0
    rope = w.kv[w.block_table[0, 0], 0, 0, 512:].copy()
    w.kv[..., 512:] = rope
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    V = np.stack([orc.bf16_to_f64(w.kv[w.block_table[0, j // 64], j % 64, 0, :512]) for j in range(L)])
    s0 = (orc.bf16_to_f64(w.q[0, 0, :, 512:]) @ orc.bf16_to_f64(rope)) / 24.0
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(V.mean(0), (4, 512)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE[0, 0], s0 + math.log(L), rtol=0, atol=1e-12)


def test_empty_key_set():
    w = small(17, [0, 5], s_q=2, h_q=4, causal=True, num_pages=4)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, causal=True)
    assert (O[0] == 0).all() and np.isneginf(LSE[0]).all()
    assert np.isfinite(LSE[1]).all()
    w1 = small(18, [1], s_q=2, h_q=4, causal=True)
    O1, L1 = orc.decode(w1.q, w1.kv, w1.block_table, w1.cache_seqlens, 512, causal=True)
    assert (O1[0, 0] == 0).all() and np.isneginf(L1[0, 0]).all()   # token 0 sees L - 2 + 0 + 1 = 0 keys
    assert np.isfinite(L1[0, 1]).all()


# ----------------------------------------------------------------------------
# Invariants of the definition
# ----------------------------------------------------------------------------
def test_page_permutation_invariance():
    w = small(19, [37, 130, 64], h_q=8, num_pages=12)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    rng = np.random.default_rng(7)
    perm = rng.permutation(w.kv.shape[0])            # new physical page of old page p = perm[p]
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    bt2 = perm[w.block_table]
    O2, LSE2 = orc.decode(w.q, kv2, bt2, w.cache_seqlens, 512)
    assert (O == O2).all() and (LSE == LSE2).all()


def test_poison_rows_never_read():
    clean = small(20, [37, 130, 1], h_q=8, num_pages=10)
    dirty = small(20, [37, 130, 1], h_q=8, num_pages=10, poison=True)
    assert (dirty.kv == wl.BF16_NAN).any()
    O, LSE = orc.decode(clean.q, clean.kv, clean.block_table, clean.cache_seqlens, 512)
    O2, LSE2 = orc.decode(dirty.q, dirty.kv, dirty.block_table, dirty.cache_seqlens, 512)
    assert (O == O2).all() and (LSE == LSE2).all()


def test_causal_row_equals_shorter_noncausal():
    w = small(21, [100], s_q=4, h_q=4, causal=True)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, causal=True)
    for s in range(4):
        Ls = np.array([100 - 4 + s + 1], dtype=np.int32)
        o1, l1 = orc.decode(w.q[:, s:s + 1], w.kv, w.block_table, Ls, 512)
        assert np.allclose(O[0, s], o1[0, 0], rtol=0, atol=1e-13)
        assert np.allclose(LSE[0, s], l1[0, 0], rtol=0, atol=1e-13)


def test_sparse_reductions():
    w = small(22, [90, 200], s_q=2, h_q=4)
    Od, Ld = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    # all positions, shuffled, plus -1 pads and out-of-range entries -> dense result
    rng = np.random.default_rng(3)
    idx = np.full((2, 2, 210), -1, dtype=np.int32)
    for b, L in enumerate([90, 200]):
        for s in range(2):
            idx[b, s, :L] = rng.permutation(L)
            idx[b, s, L:L + 3] = [L, L + 7, -5]
    Os, Ls = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, indices=idx)
    np.testing.assert_allclose(Os, Od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Ls, Ld, rtol=0, atol=1e-13)
    # causal prefix as index list == causal decode
    wc = small(22, [90, 200], s_q=2, h_q=4, causal=True)
    Oc, Lc = orc.decode(wc.q, wc.kv, wc.block_table, wc.cache_seqlens, 512, causal=True)
    idx2 = np.full((2, 2, 200), -1, dtype=np.int32)
    for b, L in enumerate([90, 200]):
        for s in range(2):
            n = L - 2 + s + 1
            idx2[b, s, :n] = np.arange(n)[::-1]
    Os2, Ls2 = orc.decode(wc.q, wc.kv, wc.block_table, wc.cache_seqlens, 512, indices=idx2)
    np.testing.assert_allclose(Os2, Oc, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Ls2, Lc, rtol=0, atol=1e-13)


def test_sparse_subset_matches_sdpa():
    w = small(23, [300], s_q=2, h_q=4, topk=50)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, indices=w.indices)
    K = _contiguous_cache(w, 0)
    for s in range(2):
        sel = torch.from_numpy(w.indices[0, s].astype(np.int64))
        Ks = K[sel]
        ref = F.scaled_dot_product_attention(_q(w, 0, s)[None, :, None, :], Ks[None, None].expand(1, 4, -1, -1),
                                             Ks[None, None, :, :512].expand(1, 4, -1, -1), scale=1 / 24)
        np.testing.assert_allclose(O[0, s], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_merge_of_disjoint_splits():
    w = small(24, [250], h_q=8)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512)
    rng = np.random.default_rng(5)
    order = rng.permutation(250)
    cuts = [0, 17, 18, 120, 250]
    po, pl = [], []
    for a, c in zip(cuts[:-1], cuts[1:]):
        idx = np.full((1, 1, 250), -1, dtype=np.int32)
        idx[0, 0, :c - a] = order[a:c]
        o, l = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, indices=idx)
        po.append(o[0, 0])
        pl.append(l[0, 0])
    # an empty split (LSE = -inf) must carry no weight
    po.append(np.zeros_like(po[0]))
    pl.append(np.full_like(pl[0], -np.inf))
    Om, Lm = orc.merge_splits(np.stack(po), np.stack(pl))
    np.testing.assert_allclose(Om, O[0, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lm, LSE[0, 0], rtol=0, atol=1e-13)
    Oe, Le = orc.merge_splits(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert (Oe == 0).all() and np.isneginf(Le).all()


def test_physical_rows_closed_form():
    bt = np.array([[5, 2, 7], [1, 0, 3]])
    assert list(orc.physical_rows(bt, 0, [0, 63, 64, 130])) == [320, 383, 128, 450]
    assert list(orc.physical_rows(bt, 1, [5, 127, 128])) == [69, 63, 192]


# ----------------------------------------------------------------------------
# Scheduler: hand-worked fixtures and invariants
# ----------------------------------------------------------------------------
def _read_plan_examples():
    ex, cur = [], None
    for line in open(os.path.join(GOLDEN, "plan_examples.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "example":
            cur = {"rows": []}
            ex.append(cur)
        elif key == "row":
            cur["rows"].append([int(v) for v in vals])
        else:
            cur[key] = [int(v) for v in vals]
    return ex


def test_plan_hand_worked_examples():
    exs = _read_plan_examples()
    assert len(exs) == 5
    for e in exs:
        p, ns = orc.plan(e["lengths"], e["workers"][0], e["overhead"][0])
        rows = p.reshape(-1, 8)
        assert list(rows[0]) == e["header"]
        assert [list(r) for r in rows[1:]] == e["rows"]
        assert list(ns) == e["num_splits"]


def _check_plan_invariants(lengths, W, c):
    p, ns = orc.plan(lengths, W, c)
    rows = p.reshape(-1, 8)
    nblk = [-(-L // 64) for L in lengths]
    T, We = (int(rows[0, 6]) & 0xFFFFFFFF) + (int(rows[0, 7]) << 32), rows[0, 2]
    P = -(-T // We) if We else 0          # the longest worker interval
    runs = orc.plan_runs(p, lengths)
    cover = [np.zeros(n, dtype=int) for n in nblk]
    per_item = {i: [] for i in range(len(lengths))}
    for w, wr in enumerate(runs):
        cost = 0
        for (i, lo, hi, k) in wr:
            assert 0 <= lo < hi <= nblk[i]
            cover[i][lo:hi] += 1
            per_item[i].append((w, lo, hi, k))
            cost += hi - lo
        cost += c * len(wr)
        assert cost <= P + 2 * c                 # every worker stays near its share
    for i in range(len(lengths)):
        assert (cover[i] == 1).all()             # every block exactly once
        segs = per_item[i]
        assert [k for (_, _, _, k) in segs] == list(range(len(segs)))
        for a, b in zip(segs, segs[1:]):
            assert a[2] == b[1] and a[0] < b[0]  # contiguous, in worker order
        assert ns[i + 1] - ns[i] == len(segs)
    assert ns[0] == 0 and ns[-1] == sum(len(v) for v in per_item.values())
    assert ns[-1] <= len(lengths) + W


def _t(rows):
    return (int(rows[0, 6]) & 0xFFFFFFFF) + (int(rows[0, 7]) << 32)


def test_plan_axis_past_2_31_closed_form():
    # n = 2^25 - 1 blocks per item (lengths just under 2^31), 70 items: the
    # total cost passes 2^31 and is stored as two 32-bit words
    n = 2**25 - 1
    # one worker per item: worker w owns exactly item w's units
    p, ns = orc.plan([64 * n] * 70, 70, 4)
    rows = p.reshape(-1, 8).astype(np.int64)
    assert _t(rows) == 70 * (n + 4) and list(rows[0, :6]) == [70, 4, 70, 70, orc.PLAN_VERSION, 64]
    for w in range(70):
        assert list(rows[1 + w]) == [w, 0, w, n, 0, 0, 0, 0]
    assert list(ns) == list(range(71))
    # overhead 1 and two workers per item: each item's 2^25 units split in halves,
    # its first unit being the overhead
    p, ns = orc.plan([64 * n] * 70, 140, 1)
    rows = p.reshape(-1, 8).astype(np.int64)
    assert _t(rows) == 70 * 2**25
    for i in range(70):
        assert list(rows[1 + 2 * i]) == [i, 0, i, 2**24 - 1, 0, 0, 0, 0]
        assert list(rows[2 + 2 * i]) == [i, 2**24 - 1, i, n, 1, 0, 0, 0]
    assert list(ns) == list(range(0, 141, 2))


def test_plan_invariants_random():
    rng = np.random.default_rng(9)
    for _ in range(150):
        B = int(rng.integers(1, 40))
        lengths = [int(x) for x in rng.integers(0, 3000, size=B)]
        if rng.random() < 0.3:
            lengths[int(rng.integers(0, B))] = 0
        W = int(rng.integers(1, 70))
        c = int(rng.integers(1, 7))
        _check_plan_invariants(lengths, W, c)


def test_plan_invariants_exhaustive_pairs():
    for L0 in range(0, 200, 7):
        for L1 in range(0, 200, 11):
            for W in (1, 2, 3, 5, 8):
                for c in (2, 3):
                    _check_plan_invariants([L0, L1], W, c)


def test_decode_by_plan_equals_decode():
    w = small(25, [37, 130, 0, 300, 64], s_q=2, h_q=4, causal=True)
    O, LSE = orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, causal=True)
    for W in (1, 3, 7, 16):
        p, _ = orc.plan(w.cache_seqlens, W, 2)
        O2, L2 = orc.decode_by_plan(w.q, w.kv, w.block_table, w.cache_seqlens, 512, p, causal=True)
        np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L2, LSE, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# Work accounting
# ----------------------------------------------------------------------------
def test_work_closed_forms():
    b, f = orc.work([4096] * 128, 1, 128, False)
    assert b == 128 * 4096 * 1152 and f == 128 * 128 * 4096 * 2 * 1088
    b, f = orc.work([100, 7], 2, 4, True)
    assert b == 107 * 1152 and f == 4 * (99 + 100 + 6 + 7) * 2176
    idx = np.array([[[0, 5, -1, 99]]])
    b, f = orc.work([50], 1, 8, False, indices=idx)
    assert b == 2 * 1152 and f == 8 * 2 * 2176
    b, f = orc.work([100, 7], 1, 32, False, h_kv=4)     # each key read once per latent head
    assert b == 107 * 4 * 1152 and f == 32 * 107 * 2176
    b, f = orc.work([100, 7], 1, 16, False, row_bytes=656)   # packed FP8 rows
    assert b == 107 * 656 and f == 16 * 107 * 2176
    # dual cache: 2 main keys (0, 5) and 1 auxiliary key (3 < 4) for the one token
    b, f = orc.work([50], 1, 8, False, d_qk=512, indices=idx,
                    aux=(np.array([4]), np.array([[[3, 4, -1]]])))
    assert b == 3 * 1024 and f == 8 * 3 * 2 * 1024


def test_bench_work_accounting_matches_oracle():
    """bench.py's byte and FLOP counts agree with orc.work on every kind of
    workload it times (dense, causal, sparse, grouped heads, packed FP8, dual
    cache with 512-value rows)."""
    import bench
    cases = [
        wl.build("w-dense", 90, np.array([300, 1, 0, 129]), B=4, s_q=1, h_q=16, num_pages=20),
        wl.build("w-causal", 91, np.array([300, 1, 0, 129]), B=4, s_q=3, h_q=32, num_pages=20, causal=True),
        wl.build("w-grouped", 92, np.array([77, 640]), B=2, s_q=2, h_q=64, h_kv=4, num_pages=20),
        wl.build("w-sparse", 93, np.array([300, 200]), B=2, s_q=2, h_q=128, num_pages=20, topk=100),
        wl.build("w-fp8", 94, np.array([300, 5]), B=2, s_q=1, h_q=16, num_pages=20, kv_format="fp8"),
        wl.build("w-fp8-sparse", 95, np.array([300, 90]), B=2, s_q=2, h_q=128, num_pages=20, topk=64,
                 kv_format="fp8"),
    ]
    cases[3].indices[1, 0, :7] = -1        # padding entries
    rng = np.random.default_rng(96)
    dual = wl.build("w-dual", 96, np.array([300, 200]), B=2, s_q=2, h_q=128, num_pages=20, topk=64,
                    rng=rng, d_qk=512)
    cases.append(wl.add_aux_cache(dual, rng, np.array([100, 0]), 80, 8))
    for w in cases:
        h_kv = w.kv.shape[2]
        row_bytes = w.kv.shape[3] * w.kv.itemsize
        aux = (w.aux[2], w.aux[3]) if w.aux is not None else None
        ref = orc.work(w.cache_seqlens, w.s_q, w.h_q, w.causal, d_qk=w.q.shape[3], topk=w.topk,
                       indices=w.indices, h_kv=h_kv, row_bytes=row_bytes, aux=aux)
        assert bench.algorithmic_work(w) == ref, w.name


def test_named_workload_recipes():
    w = wl.tiny()
    assert list(w.cache_seqlens) == [37, 130] and w.kv.shape == (8, 64, 1, 576)
    used = set(w.block_table[0, :1]) | set(w.block_table[1, :3])
    assert len(used) == 4
    w = wl.memory_bound()
    assert w.cache_seqlens.min() >= 1 and w.cache_seqlens.max() <= 4096 and w.kv.shape[0] == 6000
    assert w.block_table.shape == (64, 64)
    w = wl.grouped_heads()
    assert w.kv.shape[2] == 8 and w.h_q == 128 and w.block_table.shape == (32, 64)
    w = wl.sparse_prefill(T=64)
    assert w.indices.shape == (1, 64, 2048) and int(w.cache_seqlens[0]) == 4096 + 64
    for t in range(64):     # causally valid, unique
        row = w.indices[0, t]
        assert row.min() >= 0 and row.max() <= 4096 + t and len(np.unique(row)) == 2048
