"""CPU oracle for paged MLA decode — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never calls it, and this module imports nothing from the
product package.

Everything here is the plain definition of what the decode computes, written in
float64 with NumPy (one library matmul per query token is the only "fast" step):

* Page addressing.  "What is FlashMLA" (topnet.top), section "FlashMLA의 주요
  특성" (paged KV cache with 64-token blocks) and section "FlashMLA 설치 및
  사용", step 3 (the decode call takes ``block_table`` and ``cache_seqlens``):
  logical token j of sequence b lives in physical page ``block_table[b, j // 64]``
  at slot ``j % 64``.
* Latent attention.  "Novita AI, H100 및 H200에서 FlashMLA 평가", section
  "MLA란 무엇인가요?" (one compressed latent K/V per token, with a decoupled RoPE
  part, shared by all heads): each cached row holds 576 values; K is the whole
  row, V is its first ``dv`` (=512) values.
* Outputs ``(o, lse)`` of the decode call (topnet.top, step 3).  O is the
  softmax-weighted mean of V; LSE is the natural log of the sum of exponentials
  of the scaled scores.
* ``causal`` (topnet.top, step 3) is read as bottom-right alignment: the s_q
  query tokens are the last s_q tokens already in the cache, so query token s
  sees keys 0 .. L - s_q + s.
* Top-k sparse attention ("FlashInfer, SM120 GPU를 위한 희소 MLA 커널",
  section "왜 이게 좋은가?", item 2: attend only the top-k selected tokens):
  query token (b, s) attends to the logical positions ``indices[b, s, :topk]``;
  an entry outside ``[0, L_b)`` (e.g. -1) is padding and is skipped.
* Empty key set: O = 0, LSE = -inf.
* Rows of 512 values ("FlashInfer, SM120 GPU를 위한 희소 MLA 커널", 들어가며:
  models with d_qk = 512 beside d_qk = 576): K is the whole row and V, with
  dv = 512, the whole row too.
* Dual cache (the same page, section "코드 분석", item 1: a main and an
  auxiliary cache used together): in sparse mode a query token attends to the
  union of its keys in the main cache (``indices`` through ``block_table``)
  and in the auxiliary cache (``indices2`` through ``block_table2``, valid
  below ``cache_seqlens2``), with one softmax over both sets.
* FP8 cache ("FlashInfer, SM120 GPU를 위한 희소 MLA 커널", section "코드 분석",
  item 5: a packed KV cache whose scale format is a parameter; "Blackwell을
  위한 새로운 MLA 백엔드: TOKENSPEED_MLA 분석": FP8 KV caches).  The pages fix
  no layout; the one read here packs each cached row into 656 bytes: the 512
  latent values as OCP E4M3 codes, one float32 scale per block of 128 latent
  values (4 scales), then the 64 RoPE values in bf16.  A latent value is its
  code's value times its block's scale; K and V are then as above.
* ``plan`` — the split-KV tile scheduler (``get_mla_metadata`` of topnet.top,
  step 2, returns ``tile_scheduler_metadata`` and ``num_splits``).  The pages do
  not say how work is split; :func:`plan` states the scheduler this library
  uses, item by item and worker by worker.
* ``merge_splits`` — log-sum-exp merge of partial results over disjoint key
  subsets (the ``num_splits`` / scratch-buffer step of the same pages).

Pins: every function here is checked in ``tests/test_oracle.py`` against
closed forms, library special cases, brute force and invariants.
"""
from __future__ import annotations

import numpy as np

PAGE = 64          # tokens per KV page (topnet.top, "FlashMLA의 주요 특성")
D_QK = 576         # latent (512) + decoupled RoPE (64) values per cached row
D_V = 512          # V = first 512 values of the row
FP8_ROW_BYTES = 656    # packed FP8 row: 512 E4M3 codes, 4 float32 scales, 64 bf16 RoPE values
FP8_BLOCK = 128        # latent values per scale


# --------------------------------------------------------------------------
# bf16 bit patterns -> float64 (exact: every bf16 is a float32 is a float64)
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Exact upcast of raw bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes) -> np.ndarray:
    """Value of OCP 8-bit floating-point E4M3 codes (exact in float64).

    Bit 7 is the sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the
    mantissa m.  e = 0 encodes the subnormals m/8 * 2^-6; the code with e = 15
    and m = 7 is NaN; there are no infinities (the largest value is 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) == 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp8_rows_to_f64(rows) -> np.ndarray:
    """Packed FP8 rows [..., 656] (uint8) -> their 576 values in float64.

    Bytes 0..511: E4M3 codes of the latent values; bytes 512..527: four
    little-endian float32 scales, scale j for latent values 128 j .. 128 j + 127;
    bytes 528..655: the 64 RoPE values as little-endian bf16.
    """
    r = np.array(rows, dtype=np.uint8, copy=True)
    lat = e4m3_to_f64(r[..., :512])
    scales = np.ascontiguousarray(r[..., 512:528]).view("<f4").astype(np.float64)
    lat = lat * np.repeat(scales, FP8_BLOCK, axis=-1)
    rope = bf16_to_f64(np.ascontiguousarray(r[..., 528:656]).view("<u2"))
    return np.concatenate([lat, rope], axis=-1)


# --------------------------------------------------------------------------
# Page addressing
# --------------------------------------------------------------------------
def physical_rows(block_table: np.ndarray, b: int, positions) -> np.ndarray:
    """Physical cache row of each logical token position of sequence ``b``.

    Row id = ``block_table[b, j // 64] * 64 + j % 64`` (int64).  The byte
    offset of the row in the cache is ``row * h_kv * 576 * 2``.
    """
    pos = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(block_table, dtype=np.int64)[b, pos // PAGE]
    return pages * PAGE + pos % PAGE


def key_positions(b: int, s: int, seqlen: int, s_q: int, causal: bool,
                  indices: np.ndarray | None, topk: int | None) -> np.ndarray:
    """Logical key positions attended to by query token ``s`` of sequence ``b``."""
    if indices is None:
        end = seqlen - s_q + s + 1 if causal else seqlen
        return np.arange(max(end, 0), dtype=np.int64)
    k = indices.shape[-1] if topk is None else topk
    idx = np.asarray(indices[b, s, :k], dtype=np.int64)
    return idx[(idx >= 0) & (idx < seqlen)]


# --------------------------------------------------------------------------
# Decode (the plain definition)
# --------------------------------------------------------------------------
def decode(q_bits: np.ndarray, kv_bits: np.ndarray, block_table: np.ndarray,
           cache_seqlens: np.ndarray, dv: int = D_V, causal: bool = False,
           softmax_scale: float | None = None, indices: np.ndarray | None = None,
           topk: int | None = None, items=None, aux=None):
    """float64 MLA decode.

    q_bits   uint16 [B, s_q, h_q, d]           (bf16 bit patterns)
    kv_bits  uint16 [num_pages, 64, h_kv, d]   (bf16 bit patterns), or
             uint8  [num_pages, 64, h_kv, 656] (packed FP8 rows, see fp8_rows_to_f64)
    block_table int [B, max_blocks]; cache_seqlens int [B]
    indices  optional int [B, s_q, topk] logical positions (sparse mode)
    items    optional iterable of (b, s) pairs to compute (others stay NaN)
    aux      optional auxiliary cache (kv2_bits, block_table2, cache_seqlens2,
             indices2) of the dual-cache sparse decode; its keys join each
             query token's key set

    Returns (O float64 [B, s_q, h_q, dv], LSE float64 [B, s_q, h_q]).
    """
    B, s_q, h_q, d = q_bits.shape
    h_kv = kv_bits.shape[2]
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    if indices is not None and causal:
        raise ValueError("causal and indices are exclusive")
    scale = d ** -0.5 if softmax_scale is None else float(softmax_scale)
    fp8 = kv_bits.dtype == np.uint8
    if fp8 and kv_bits.shape[-1] != FP8_ROW_BYTES:
        raise ValueError("packed FP8 rows have 656 bytes")
    rows = kv_bits.reshape(-1, h_kv, kv_bits.shape[-1])
    row_values = fp8_rows_to_f64 if fp8 else bf16_to_f64
    group = h_q // h_kv
    out = np.full((B, s_q, h_q, dv), np.nan)
    lse = np.full((B, s_q, h_q), np.nan)
    todo = items if items is not None else [(b, s) for b in range(B) for s in range(s_q)]
    if aux is not None:
        if indices is None:
            raise ValueError("the auxiliary cache needs sparse mode")
        kv2, bt2, sl2, idx2 = aux
        rows2 = kv2.reshape(-1, h_kv, kv2.shape[-1])
    for b, s in todo:
        L = int(cache_seqlens[b])
        pos = key_positions(b, s, L, s_q, causal, indices, topk)
        rid = physical_rows(block_table, b, pos)
        rid2 = np.zeros(0, dtype=np.int64)
        if aux is not None:
            pos2 = key_positions(b, s, int(sl2[b]), s_q, False, idx2, None)
            rid2 = physical_rows(bt2, b, pos2)
        if rid.size + rid2.size == 0:
            out[b, s] = 0.0
            lse[b, s] = -np.inf
            continue
        for g in range(h_kv):
            K = row_values(rows[rid, g, :])                  # [n, d]
            if aux is not None:
                K = np.concatenate([K, row_values(rows2[rid2, g, :])], axis=0)
            V = K[:, :dv]                                    # [n, dv]
            Q = bf16_to_f64(q_bits[b, s, g * group:(g + 1) * group, :])  # [group, d]
            S = scale * (Q @ K.T)                            # [group, n]
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            l = P.sum(axis=1, keepdims=True)
            out[b, s, g * group:(g + 1) * group] = (P @ V) / l
            lse[b, s, g * group:(g + 1) * group] = (m + np.log(l))[:, 0]
    return out, lse


# --------------------------------------------------------------------------
# Split merge (log-sum-exp combine of partial results)
# --------------------------------------------------------------------------
def merge_splits(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge partial attention results over disjoint key subsets.

    o_parts [n, ..., dv] (each normalised by its own subset), lse_parts [n, ...].
    Returns (O, LSE) equal to attention over the union of the subsets.
    Parts with LSE = -inf (empty subsets) carry no weight; if every part is
    empty the result is O = 0, LSE = -inf.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lse_parts - safe)                              # [n, ...]
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(tot > 0, safe + np.log(tot), -np.inf)
        o = np.where(tot[..., None] > 0,
                     (w[..., None] * o_parts).sum(axis=0) / np.where(tot > 0, tot, 1.0)[..., None],
                     0.0)
    return o, lse


# --------------------------------------------------------------------------
# Split-KV scheduler ("tile_scheduler_metadata" / "num_splits")
# --------------------------------------------------------------------------
PLAN_WORDS = 8        # int32 words per plan row
PLAN_VERSION = 3


def plan(lengths, num_workers: int, overhead: int):
    """Split-KV schedule over ``num_workers`` workers (reading of the pages).

    Each item (a sequence; in sparse mode a query token) of length ``len``
    has n = ceil(len / 64) blocks and costs ``overhead + n`` units, the
    overhead standing for loading its queries (a lead of ceil(overhead / 2)
    units before its blocks) and writing its result (a tail of
    floor(overhead / 2) units after them).  Items are laid end to end on a
    cost axis of total T.  The first W' = min(W, T) workers share the axis
    evenly: worker w owns the units [floor(w T / W'), floor((w + 1) T / W')),
    at least one unit each; the others get nothing.  Block b of item i
    occupies the unit C_i + lead + b, C_i being the item's start.  A worker
    processes, for every item, the blocks whose units fall inside its
    interval (a contiguous run, possibly empty); the non-empty runs of one
    item, in worker order, are the item's splits, numbered 0, 1, ...  (Every
    run loads its queries and writes its result, a split one included; with
    the overhead at both ends of an item, the workers that start or end
    inside an item are charged alike.)

    Returns (plan int32 [(W + 1) * 8], num_splits int32 [num_items + 1]):
      plan row 0  = [W, overhead, W', num_items, version, 64, T mod 2^32,
                     T div 2^32] (T as two 32-bit words: the axis may pass 2^31)
      plan row 1+w = [first item, its first block, last item, end block of the
                      last item, split number of the first item's run, 0, 0, 0]
                    or [-1, 0, -1, 0, 0, 0, 0, 0] for a worker with no blocks.
      num_splits  = exclusive prefix sum of the per-item split counts.
    """
    lengths = [int(x) for x in lengths]
    W = int(num_workers)
    c = int(overhead)
    if W < 1 or c < 1:
        raise ValueError("need num_workers >= 1 and overhead >= 1")
    lead = (c + 1) // 2          # the tail, c - lead units, follows the blocks
    nblk = [-(-L // PAGE) if L > 0 else 0 for L in lengths]
    start = []
    acc = 0
    for n in nblk:
        start.append(acc)
        acc += c + n
    T = acc
    We = min(W, T)
    rows = np.zeros((W + 1, PLAN_WORDS), dtype=np.int64)
    t_lo = T & 0xFFFFFFFF
    rows[0] = [W, c, We, len(lengths), PLAN_VERSION, PAGE, t_lo - (t_lo >> 31 << 32), T >> 32]
    counts = [0] * len(lengths)
    for w in range(W):
        if w < We:
            lo, hi = (w * T) // We, ((w + 1) * T) // We
        else:
            lo = hi = T
        runs = []
        for i, n in enumerate(nblk):
            if n == 0:
                continue
            first = start[i] + lead               # unit of block 0
            b_lo = min(max(lo - first, 0), n)
            b_hi = min(max(hi - first, 0), n)
            if b_lo < b_hi:
                runs.append((i, b_lo, b_hi, counts[i]))
                counts[i] += 1
        if runs:
            rows[1 + w] = [runs[0][0], runs[0][1], runs[-1][0], runs[-1][2], runs[0][3], 0, 0, 0]
        else:
            rows[1 + w] = [-1, 0, -1, 0, 0, 0, 0, 0]
    num_splits = np.zeros(len(lengths) + 1, dtype=np.int64)
    num_splits[1:] = np.cumsum(counts)
    return rows.reshape(-1).astype(np.int32), num_splits.astype(np.int32)


def plan_runs(plan_words: np.ndarray, lengths):
    """Expand a plan into its runs: list over workers of [(item, blk_lo, blk_hi, split)]."""
    rows = np.asarray(plan_words, dtype=np.int64).reshape(-1, PLAN_WORDS)
    W = int(rows[0, 0])
    nblk = [-(-int(L) // PAGE) if int(L) > 0 else 0 for L in lengths]
    out = []
    for w in range(W):
        i0, b0, i1, b1, k0 = (int(x) for x in rows[1 + w, :5])
        runs = []
        if i0 >= 0:
            for i in range(i0, i1 + 1):
                lo = b0 if i == i0 else 0
                hi = b1 if i == i1 else nblk[i]
                if lo < hi:
                    runs.append((i, lo, hi, k0 if i == i0 else 0))
        out.append(runs)
    return out


def decode_by_plan(q_bits, kv_bits, block_table, cache_seqlens, dv, plan_words,
                   causal=False, softmax_scale=None):
    """Dense decode evaluated split by split as the plan prescribes, then merged.

    Used to show that any plan reproduces :func:`decode` (split invariance).
    """
    B, s_q, h_q, d = q_bits.shape
    lengths = [int(x) for x in cache_seqlens]
    runs = plan_runs(plan_words, lengths)
    parts = {b: [] for b in range(B)}
    for wr in runs:
        for (i, lo, hi, k) in wr:
            parts[i].append((k, lo, hi))
    O = np.zeros((B, s_q, h_q, dv))
    LSE = np.full((B, s_q, h_q), -np.inf)
    for b in range(B):
        if not parts[b]:
            continue
        po, pl = [], []
        for (k, lo, hi) in sorted(parts[b]):
            # restrict the key set to positions in [lo*64, hi*64) via a sparse index list
            L = lengths[b]
            sub = []
            for s in range(s_q):
                end = L - s_q + s + 1 if causal else L
                pos = np.arange(lo * PAGE, min(hi * PAGE, max(end, 0)), dtype=np.int64)
                sub.append(pos)
            width = max(1, max(len(p) for p in sub))
            idx = np.full((B, s_q, width), -1, dtype=np.int64)
            for s in range(s_q):
                idx[b, s, :len(sub[s])] = sub[s]
            o_k, l_k = decode(q_bits, kv_bits, block_table, cache_seqlens, dv, False,
                              softmax_scale, idx, None, items=[(b, s) for s in range(s_q)])
            po.append(o_k[b])
            pl.append(l_k[b])
        O[b], LSE[b] = merge_splits(np.stack(po), np.stack(pl))
    return O, LSE


# --------------------------------------------------------------------------
# Work accounting used by the benchmark (algorithmic bytes and flops)
# --------------------------------------------------------------------------
def work(cache_seqlens, s_q: int, h_q: int, causal: bool, d_qk: int = D_QK, dv: int = D_V,
         topk: int | None = None, indices=None, h_kv: int = 1, row_bytes: int | None = None,
         aux=None):
    """(KV bytes read once per key, FLOPs) of one decode call.

    KV bytes count each (sequence, key, latent head) row once at its stored
    size: ``row_bytes`` (default 2 bytes per value, i.e. a bf16 row; a packed
    FP8 row is 656 bytes).  FLOPs are 2 * (d_qk + dv) per (query row, key).
    ``aux = (cache_seqlens2, indices2)`` adds the auxiliary cache's keys of a
    dual-cache sparse decode (entries inside [0, cache_seqlens2[b])), whose
    rows have the same size.
    """
    if row_bytes is None:
        row_bytes = d_qk * 2
    if indices is not None:
        idx = np.asarray(indices)
        L = np.asarray(cache_seqlens).reshape(-1, 1, 1)
        keys_per_token = ((idx >= 0) & (idx < L)).sum()
        if aux is not None:
            L2 = np.asarray(aux[0]).reshape(-1, 1, 1)
            idx2 = np.asarray(aux[1])
            keys_per_token = keys_per_token + ((idx2 >= 0) & (idx2 < L2)).sum()
        kv_rows = keys_per_token
        qk = keys_per_token * h_q
    else:
        if aux is not None:
            raise ValueError("an auxiliary cache needs sparse mode")
        kv_rows = 0
        qk = 0
        for L in (int(x) for x in cache_seqlens):
            kv_rows += L
            for s in range(s_q):
                qk += h_q * (max(L - s_q + s + 1, 0) if causal else L)
    return int(kv_rows) * h_kv * int(row_bytes), int(qk) * 2 * (d_qk + dv)


__all__ = ["PAGE", "D_QK", "D_V", "FP8_ROW_BYTES", "FP8_BLOCK", "e4m3_to_f64", "fp8_rows_to_f64", "bf16_to_f64", "physical_rows", "key_positions", "decode",
           "merge_splits", "plan", "plan_runs", "decode_by_plan", "work",
           "PLAN_WORDS", "PLAN_VERSION"]
