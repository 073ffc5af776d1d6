"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers and lays them out (sequence lengths,
page permutations, block tables, bf16 bit patterns of N(0, 1) values, sparse
top-k index lists).  It holds none of the decode arithmetic; the tests and the
benchmark feed the same arrays to the HIP library and to the CPU reference.

Recipe (NumPy PCG64, seed = workload number): draw the lengths, then the page
permutation, then q, then the cache, then (sparse only) the indices.  Normal
values are drawn as float32 and rounded to bf16, ties to even.  Pages are
handed out consecutively from the permutation, sequence by sequence.  Rows that
no sequence references (unassigned pages, slots past a sequence's length in its
last page) and the block-table padding page may be filled with NaN ("poison")
so that any read of them shows up in the outputs.

Packed FP8 caches (656 bytes per row: 512 OCP E4M3 codes, 4 float32 scales,
64 bf16 RoPE values) are drawn in the same order: the latent values as float32
N(0, 1), each block of 128 given the scale max|x| / 448 and cast to E4M3 by
torch's float8_e4m3fn conversion (round to nearest even), then the RoPE values
as bf16 N(0, 1).  Poisoned FP8 rows hold the NaN code 0x7F, NaN scales and
NaN RoPE values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE = 64
D_QK = 576
D_V = 512
BF16_NAN = 0x7FC0
FP8_ROW_BYTES = 656
E4M3_NAN = 0x7F


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def packed_fp8_rows(rng: np.random.Generator, shape, chunk: int = 1 << 22) -> np.ndarray:
    """Packed FP8 rows [*shape, 656] (uint8) of N(0, 1) latent values and bf16 RoPE values."""
    import torch
    n = int(np.prod(shape))
    out = np.empty((n, FP8_ROW_BYTES), dtype=np.uint8)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        x = rng.standard_normal((m, 4, 128), dtype=np.float32)
        scale = (np.abs(x).max(axis=2) / np.float32(448.0)).astype(np.float32)     # [m, 4]
        scale[scale == 0] = 1.0
        codes = torch.from_numpy(x / scale[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out[i:i + m, :512] = codes.reshape(m, 512)
        out[i:i + m, 512:528] = scale.astype("<f4").view(np.uint8).reshape(m, 16)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        rope = f32_to_bf16_bits(rng.standard_normal((m, 64), dtype=np.float32))
        out[i:i + m, 528:656] = rope.astype("<u2").view(np.uint8).reshape(m, 128)
    return out.reshape(*shape, FP8_ROW_BYTES)


def poison_fp8_rows(rows: np.ndarray) -> None:
    """Fill packed FP8 rows (last axis 656) with NaN codes, scales and RoPE values, in place."""
    rows[..., :512] = E4M3_NAN
    rows[..., 512:528] = np.full(4, np.nan, dtype="<f4").view(np.uint8)
    rows[..., 528:656] = np.full(64, BF16_NAN, dtype="<u2").view(np.uint8)


def normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0, 1) values drawn as float32 and rounded to bf16 bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        out[i:i + m] = f32_to_bf16_bits(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(shape)


@dataclass
class Workload:
    """One decode call's inputs (host arrays)."""
    name: str
    q: np.ndarray              # uint16 [B, s_q, h_q, d_qk]  (d_qk = 576 or 512)
    kv: np.ndarray             # uint16 [num_pages, 64, h_kv, d_qk] (or uint8 [.., 656] packed FP8)
    block_table: np.ndarray    # int32 [B, max_blocks]
    cache_seqlens: np.ndarray  # int32 [B]
    causal: bool = False
    indices: np.ndarray | None = None   # int32 [B, s_q, topk]
    dv: int = D_V
    softmax_scale: float | None = None
    meta: dict = field(default_factory=dict)
    # dual-cache sparse decode: (kv2, block_table2, cache_seqlens2, indices2)
    aux: tuple | None = None

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def s_q(self):
        return self.q.shape[1]

    @property
    def h_q(self):
        return self.q.shape[2]

    @property
    def topk(self):
        return None if self.indices is None else self.indices.shape[2]


def build(name: str, seed: int, lengths: np.ndarray | None, *, B: int, s_q: int, h_q: int,
          num_pages: int, causal: bool = False, max_blocks: int | None = None,
          poison: bool = False, h_kv: int = 1, topk: int | None = None,
          rng: np.random.Generator | None = None, pad_page: int | None = None,
          dv: int = D_V, kv_format: str = "bf16", d_qk: int = D_QK) -> Workload:
    """Assemble a workload.  ``lengths`` may be drawn by the caller from ``rng``
    (the same generator is then used for the rest, keeping the draw order)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = np.asarray(lengths, dtype=np.int64)
    nblk = (lengths + PAGE - 1) // PAGE
    mb = int(max(1, nblk.max())) if max_blocks is None else int(max_blocks)
    need = int(nblk.sum())
    padded = bool((nblk < mb).any())
    spare = 1 if (pad_page is None and padded) else 0
    pool = max(num_pages, need + spare)
    perm = rng.permutation(pool)
    bt = np.empty((B, mb), dtype=np.int32)
    if pad_page is not None:
        pad = int(pad_page)
    else:
        pad = int(perm[need]) if need < pool else 0
    bt[:] = pad
    off = 0
    for b in range(B):
        n = int(nblk[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    q = normal_bf16(rng, (B, s_q, h_q, d_qk))
    if kv_format == "fp8":
        kv = packed_fp8_rows(rng, (pool, PAGE, h_kv))
    elif kv_format == "bf16":
        kv = normal_bf16(rng, (pool, PAGE, h_kv, d_qk))
    else:
        raise ValueError(f"unknown kv_format {kv_format!r}")
    indices = None
    if topk is not None:
        indices = np.empty((B, s_q, topk), dtype=np.int32)
        for b in range(B):
            for s in range(s_q):
                hi = int(lengths[b]) - s_q + s + 1
                indices[b, s] = rng.choice(hi, size=topk, replace=False)
    if poison:
        referenced = np.zeros((pool, PAGE), dtype=bool)
        for b in range(B):
            L = int(lengths[b])
            for j in range(int(nblk[b])):
                n_valid = min(PAGE, L - j * PAGE)
                referenced[bt[b, j], :n_valid] = True
        if kv_format == "fp8":
            bad = kv[~referenced]           # a copy: [rows, h_kv, 656]
            poison_fp8_rows(bad)
            kv[~referenced] = bad
        else:
            kv[~referenced] = BF16_NAN
    return Workload(name=name, q=q, kv=kv, block_table=bt,
                    cache_seqlens=lengths.astype(np.int32), causal=causal,
                    indices=indices, dv=dv,
                    meta=dict(seed=seed, pool_pages=pool, pad_page=pad, poison=poison))


# ---------------------------------------------------------------------------
# The five named workloads (sizes of the headline decode scenarios)
# ---------------------------------------------------------------------------
def tiny(poison: bool = False) -> Workload:
    """b=2, s_q=1, h_q=16, lengths {37, 130}; 4 of 8 physical pages, shuffled."""
    rng = np.random.default_rng(1)
    lengths = np.array([37, 130])
    return build("tiny b2 h16 L{37,130}", 1, lengths, B=2, s_q=1, h_q=16, num_pages=8,
                 poison=poison, rng=rng)


def memory_bound(poison: bool = False) -> Workload:
    """b=64, s_q=1, h_q=16, lengths uniform in [1, 4096], 6000-page pool."""
    rng = np.random.default_rng(2)
    lengths = rng.integers(1, 4097, size=64)
    return build("memory-bound b64 h16 L~U[1,4096]", 2, lengths, B=64, s_q=1, h_q=16,
                 num_pages=6000, max_blocks=64, poison=poison, rng=rng)


def near_ridge(poison: bool = False) -> Workload:
    """b=128, s_q=1, h_q=128, every length 4096, 8192-page pool."""
    rng = np.random.default_rng(3)
    lengths = np.full(128, 4096)
    return build("near-ridge b128 h128 L4096", 3, lengths, B=128, s_q=1, h_q=128,
                 num_pages=8192, max_blocks=64, poison=poison, rng=rng)


def mtp_causal(poison: bool = False) -> Workload:
    """b=32, s_q=2 causal, h_q=128, lengths log-uniform in [256, 16384], 8192-page pool."""
    rng = np.random.default_rng(4)
    lengths = np.floor(np.exp(rng.uniform(np.log(256), np.log(16384), size=32))).astype(np.int64)
    return build("mtp-causal b32 sq2 h128 L~logU[256,16384]", 4, lengths, B=32, s_q=2,
                 h_q=128, num_pages=8192, causal=True, max_blocks=256, poison=poison, rng=rng)


def sparse_topk(poison: bool = False, B: int = 16) -> Workload:
    """b=16, s_q=8, h_q=128, length 65536, top-k 2048 unique unsorted indices per query token."""
    rng = np.random.default_rng(5)
    lengths = np.full(B, 65536)
    return build(f"sparse-topk b{B} sq8 h128 L65536 k2048", 5, lengths, B=B, s_q=8, h_q=128,
                 num_pages=B * 1024, max_blocks=1024, topk=2048, poison=poison, rng=rng)


def sparse_prefill(poison: bool = False, T: int = 4096) -> Workload:
    """Sparse prefill: one sequence of 4096 context tokens followed by T = 4096
    new query tokens (s_q = T), h_q=128, top-k 2048 unique unsorted indices per
    query token drawn from the keys it may see (positions 0 .. 4096 + t)."""
    rng = np.random.default_rng(7)
    lengths = np.array([4096 + T])
    return build(f"sparse-prefill b1 T{T} h128 L{4096 + T} k2048", 7, lengths, B=1, s_q=T, h_q=128,
                 num_pages=(4096 + T) // PAGE + 8, topk=2048, poison=poison, rng=rng)


def add_aux_cache(w: Workload, rng: np.random.Generator, lengths2, topk2: int, num_pages2: int,
                  poison: bool = False) -> Workload:
    """Give a sparse workload an auxiliary cache (dual-cache decode), drawn after
    everything else: its page permutation, its rows, then per query token topk2
    unique unsorted positions below its sequence's auxiliary length (-1 past it)."""
    lengths2 = np.asarray(lengths2, dtype=np.int64)
    B, s_q, h_kv, d = w.B, w.s_q, w.kv.shape[2], w.kv.shape[3]
    nblk = (lengths2 + PAGE - 1) // PAGE
    mb = int(max(1, nblk.max()))
    need = int(nblk.sum())
    pool = max(num_pages2, need + 1)
    perm = rng.permutation(pool)
    bt = np.full((B, mb), int(perm[need]), dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(nblk[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    kv2 = normal_bf16(rng, (pool, PAGE, h_kv, d))
    idx2 = np.full((B, s_q, topk2), -1, dtype=np.int32)
    for b in range(B):
        for s in range(s_q):
            n = min(topk2, int(lengths2[b]))
            if n:
                idx2[b, s, :n] = rng.choice(int(lengths2[b]), size=n, replace=False)
    if poison:
        referenced = np.zeros((pool, PAGE), dtype=bool)
        for b in range(B):
            for j in range(int(nblk[b])):
                referenced[bt[b, j], :min(PAGE, int(lengths2[b]) - j * PAGE)] = True
        kv2[~referenced] = BF16_NAN
    w.aux = (kv2, bt, lengths2.astype(np.int32), idx2)
    return w


def dual_cache(poison: bool = False, B: int = 16) -> Workload:
    """Dual-cache sparse decode over 512-value rows: b=16, s_q=2, h_q=128;
    main cache length 32768 with top-k 2048, auxiliary cache of 1024 tokens
    of which each query token takes 512."""
    rng = np.random.default_rng(10)
    lengths = np.full(B, 32768)
    w = build(f"dual-cache d512 b{B} sq2 h128 L32768 k2048 + L1024 k512", 10, lengths, B=B, s_q=2,
              h_q=128, num_pages=B * 512, max_blocks=512, topk=2048, poison=poison, rng=rng, d_qk=512)
    return add_aux_cache(w, rng, np.full(B, 1024), 512, B * 16 + 1, poison=poison)


def grouped_heads(poison: bool = False) -> Workload:
    """b=32, s_q=1, h_q=128 over h_kv=8 latent heads (16 query heads each),
    lengths uniform in [1, 4096], 1200-page pool."""
    rng = np.random.default_rng(6)
    lengths = rng.integers(1, 4097, size=32)
    return build("grouped-heads b32 h128 hkv8 L~U[1,4096]", 6, lengths, B=32, s_q=1, h_q=128, h_kv=8,
                 num_pages=1200, max_blocks=64, poison=poison, rng=rng)


def memory_bound_fp8(poison: bool = False) -> Workload:
    """The memory-bound decode shape over a packed FP8 cache (656-byte rows)."""
    rng = np.random.default_rng(8)
    lengths = rng.integers(1, 4097, size=64)
    return build("memory-bound fp8 b64 h16 L~U[1,4096]", 8, lengths, B=64, s_q=1, h_q=16,
                 num_pages=6000, max_blocks=64, poison=poison, rng=rng, kv_format="fp8")


def sparse_topk_fp8(poison: bool = False, B: int = 16) -> Workload:
    """The sparse top-k shape over a packed FP8 cache."""
    rng = np.random.default_rng(9)
    lengths = np.full(B, 65536)
    return build(f"sparse-topk fp8 b{B} sq8 h128 L65536 k2048", 9, lengths, B=B, s_q=8, h_q=128,
                 num_pages=B * 1024, max_blocks=1024, topk=2048, poison=poison, rng=rng,
                 kv_format="fp8")


NAMED = {
    "tiny": tiny,
    "memory_bound": memory_bound,
    "near_ridge": near_ridge,
    "mtp_causal": mtp_causal,
    "sparse_topk": sparse_topk,
    "grouped_heads": grouped_heads,
    "sparse_prefill": sparse_prefill,
    "memory_bound_fp8": memory_bound_fp8,
    "sparse_topk_fp8": sparse_topk_fp8,
    "dual_cache": dual_cache,
}
