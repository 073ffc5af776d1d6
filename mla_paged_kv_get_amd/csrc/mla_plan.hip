// Split-KV tile scheduler ("get_mla_metadata" of "What is FlashMLA",
// topnet.top, installation-and-use section, step 2: it returns the tile
// scheduler metadata and num_splits).  The pages do not say how work is split;
// this kernel implements the rule stated in the C header:
//   n_i = ceil(len_i / 64) blocks, item cost = overhead + n_i (a lead of
//   ceil(overhead / 2) units before the blocks, a tail of floor(overhead / 2)
//   after them), items laid end to end on a cost axis (start C_i, total T);
//   the first W' = min(W, T) workers share the axis evenly, worker w owning
//   units [floor(w T / W'), floor((w + 1) T / W')); block b of item i sits on
//   unit C_i + lead + b.
// One workgroup computes it from closed forms: unit x belongs to worker
// floor(((x + 1) W' - 1) / T), so the workers touching item i's blocks are
// owner(C_i + lead) .. owner(C_{i+1} - tail - 1), every one of them with at
// least one block, and the split count and split numbers follow without a walk.
// A worker's first and last items are the least and greatest items that reach
// it.  With up to kScatterW workers and no item reaching more than
// kScatterSpan of them, each item marks its workers (LDS min / max); otherwise
// each worker searches the item starts.
// The cost axis is 64-bit: the kernel first sums the item costs in 64 bits;
// when the total fits 31 bits (every realistic batch) the axis is kept in
// 32-bit integers, otherwise in 64-bit ones (item starts in LDS as int64, no
// marking).  Block numbers inside an item always fit 32 bits.
// Three paths give the same words: up to 256 items and workers on a narrow
// 32-bit axis, one item and one worker per thread (plan_small); up to
// kPlanMaxItems items, the item starts in LDS (plan_body); beyond, a second
// kernel with no per-item state in LDS (plan_kernel_large).
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanMaxItems = 16384;       // item starts in LDS up to this many items
constexpr int kPlanLargeItems = 1 << 20;   // beyond: plan_kernel_large, up to this many
constexpr int kScatterW = 4096;
constexpr int kScatterSpan = 32;

// floor(n / d) for n < 2^32 from m = floor((2^32 - 1) / d): the high word of
// n m is the quotient or one less, and one comparison settles which.
__device__ __forceinline__ uint32_t udiv(uint32_t n, uint32_t d, uint32_t m) {
  uint32_t q = __umulhi(n, m);
  if (n - q * d >= d) ++q;
  return q;
}

// 64-bit integer division, out of line (a long instruction sequence that only
// the 64-bit schedule needs).
__device__ __attribute__((noinline)) int64_t div_wide(int64_t num, int64_t den) { return num / den; }

// floor(num / den) for 0 <= num < 2^53 (kWide: 2^63) and den >= 1.  Below
// 2^53 the quotient in double precision is within one of the floor, and one
// comparison each way fixes it; above, 64-bit integer division.
template <bool kWide>
__device__ __forceinline__ int64_t floor_div(int64_t num, int64_t den) {
  if constexpr (kWide) {
    if (num >= ((int64_t)1 << 53)) return div_wide(num, den);
  }
  int64_t q = (int64_t)((double)num / (double)den);
  if (q * den > num) --q;
  else if ((q + 1) * den <= num) ++q;
  return q;
}

// Inclusive scan over the 64 lanes of a wave by DPP moves (register to
// register, no LDS round trip): shifts by 1, 2, 4, 8 lanes inside each row of
// 16, then the last lane of row 0 added to row 1 (and of row 2 to row 3), then
// the last lane of row 1 to rows 2 and 3.  Lanes a move does not reach add 0.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
  return v;
}

// Inclusive scan of one int per thread over the workgroup; `total` receives
// the sum over all threads.  One barrier; `wave_sums` must not be written
// again before the next barrier.
__device__ int block_inclusive_scan(int v, int* wave_sums, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_inclusive_sum(v);
  if (lane == 63) wave_sums[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < kPlanWaves; ++j) {
    const int s = wave_sums[j];
    before += j < wave ? s : 0;
    tot += s;
  }
  total = tot;
  return v + before;
}

// Exclusive scan of one int64 per thread over the workgroup, for values below
// 2^38; `total` receives the sum.  The low 23 and the high bits go through two
// 32-bit DPP scans (a wave's sums stay below 2^29 and 2^21), joined after one
// barrier; `wave_lo` / `wave_hi` must not be written again before the next.
__device__ int64_t block_exclusive_scan64(int64_t v, int* wave_lo, int* wave_hi, int64_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lo = wave_inclusive_sum((int)(v & 0x7fffff));
  const int hi = wave_inclusive_sum((int)(v >> 23));
  if (lane == 63) {
    wave_lo[wave] = lo;
    wave_hi[wave] = hi;
  }
  __syncthreads();
  int64_t before = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < kPlanWaves; ++j) {
    const int64_t s = ((int64_t)wave_hi[j] << 23) + wave_lo[j];
    before += j < wave ? s : 0;
    tot += s;
  }
  total = tot;
  return before + ((int64_t)hi << 23) + lo - v;
}

// Blocks of item i: topk keys (sparse) or the length of its sequence i / item_div
// (dense; item_div = number of KV heads, items being (sequence, KV head)).
__device__ __forceinline__ int item_blocks(const int32_t* seqlens, int topk, int item_div, int i) {
  const int len = topk > 0 ? topk : seqlens[i / item_div];
  return len > 0 ? len / kPage + (len % kPage != 0) : 0;   // no overflow near 2^31
}

// The schedule once the total cost T is known.  Ax is the cost-axis integer
// (int when T fits 31 bits, else int64_t); `run` is the start of the thread's
// first item.  `start` receives the item starts (num_items + 1 of them); for
// Ax = int it arrives holding each item's block count, parked there by the
// kernel.  first_s / last_s (kScatterW each) are null when marking is not
// available.
template <typename Ax>
__device__ void plan_body(const int32_t* __restrict__ seqlens, int topk, int num_items,
                          int item_div, int W, int c, int32_t* __restrict__ plan,
                          int32_t* __restrict__ num_splits, Ax* start, int* first_s, int* last_s,
                          Ax run, const Ax T, int* sums_b, int* span_w) {
  const int tid = threadIdx.x;
  const int per = (num_items + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(tid * per, num_items), i1 = min(i0 + per, num_items);
  // an item's overhead: cl units before its blocks, ct after them
  const int cl = (c + 1) / 2, ct = c / 2;
  const bool can_mark = first_s != nullptr && W <= kScatterW;
  if (can_mark) {
    for (int w = tid; w < W; w += kPlanThreads) {
      first_s[w] = num_items;   // none
      last_s[w] = -1;
    }
  }

  // Start of every item on the cost axis.
  for (int i = i0; i < i1; ++i) {
    int n;
    if constexpr (sizeof(Ax) == 4) {
      n = start[i];
    } else {
      n = item_blocks(seqlens, topk, item_div, i);
    }
    start[i] = run;
    run += c + n;
  }
  if (tid == 0) start[num_items] = T;
  __syncthreads();
  const int We = (int)min((Ax)W, T);
  // The divisions below are by T or by W', with numerators under W' T.  When
  // that is below 2^32 they go by multiplication, otherwise by floor_div (for
  // a 32-bit axis W' T < 2^51).
  constexpr bool kWideAx = sizeof(Ax) == 8;
  const bool narrow = T > 0 && (uint64_t)We * (uint64_t)T < (1ull << 32);
  const uint32_t mT = narrow ? 0xffffffffu / (uint32_t)T : 0u;
  const uint32_t mW = narrow ? 0xffffffffu / (uint32_t)We : 0u;
  // Owner of unit x (T >= 1 whenever an item has a block), and the first unit
  // of worker w <= W'.
  auto owner = [&](Ax x) -> int {
    if (T <= 0) return 0;
    const int64_t n = ((int64_t)x + 1) * We - 1;
    return narrow ? (int)udiv((uint32_t)n, (uint32_t)T, mT) : (int)floor_div<kWideAx>(n, T);
  };
  auto unit0 = [&](int w) -> Ax {
    const int64_t n = (int64_t)w * T;
    return narrow ? (Ax)udiv((uint32_t)n, (uint32_t)We, mW) : (Ax)floor_div<kWideAx>(n, We);
  };

  // Split counts (the number of workers each item reaches) and the largest.
  int nsplit = 0;
  int span = 0;
  for (int i = i0; i < i1; ++i) {
    const Ax first = start[i] + cl, end = start[i + 1] - ct;
    if (end > first) {
      const int n = owner(end - 1) - owner(first) + 1;
      nsplit += n;
      span = max(span, n);
    }
  }
  const bool wide = __builtin_amdgcn_ballot_w64(span > kScatterSpan) != 0;
  if ((tid & 63) == 0) span_w[tid >> 6] = wide;   // published by the scan's barrier
  int S;
  const int sincl = block_inclusive_scan(nsplit, sums_b, S);
  bool any_wide = false;
  for (int j = 0; j < kPlanWaves; ++j) any_wide |= span_w[j] != 0;
  const bool scatter = can_mark && !any_wide;
  int srun = sincl - nsplit;
  for (int i = i0; i < i1; ++i) {
    num_splits[i] = srun;
    const Ax first = start[i] + cl, end = start[i + 1] - ct;
    if (end > first) {
      const int wl = owner(first), wh = owner(end - 1);
      srun += wh - wl + 1;
      if (scatter) {
        for (int w = wl; w <= wh; ++w) {
          atomicMin(&first_s[w], i);
          atomicMax(&last_s[w], i);
        }
      }
    }
  }
  if (tid == 0) num_splits[num_items] = S;
  if (scatter) __syncthreads();

  // One row per worker.
  for (int w = tid; w < W; w += kPlanThreads) {
    int32_t* row = plan + kPlanWords * (1 + w);
    Ax lo = T, hi = T;
    if (w < We) {
      lo = unit0(w);
      hi = unit0(w + 1);
    }
    int first_item = -1, first_blk = 0, last_item = -1, last_end = 0, split = 0;
    if (scatter) {
      if (first_s[w] < num_items) {
        first_item = first_s[w];
        last_item = last_s[w];
        const Ax ff = start[first_item] + cl;
        first_blk = (int)(max(lo, ff) - ff);
        split = w - owner(ff);
        last_end = (int)(min(hi, start[last_item + 1] - ct) - start[last_item] - cl);
      }
    } else if (lo < hi) {
      // Last item starting at or before lo.
      int a = 0, b = num_items - 1;
      while (a < b) {
        const int m = (a + b + 1) >> 1;
        if (start[m] <= lo) a = m; else b = m - 1;
      }
      for (int i = a; i < num_items && start[i] < hi; ++i) {
        const Ax bl = max(lo, start[i] + cl), bh = min(hi, start[i + 1] - ct);
        if (bl < bh) {
          first_item = i;
          first_blk = (int)(bl - start[i] - cl);
          split = w - owner(start[i] + cl);
          break;
        }
      }
      if (first_item >= 0) {
        // Last item starting before hi.
        a = first_item;
        b = num_items - 1;
        while (a < b) {
          const int m = (a + b + 1) >> 1;
          if (start[m] < hi) a = m; else b = m - 1;
        }
        for (int i = a; i >= first_item; --i) {
          const Ax bl = max(lo, start[i] + cl), bh = min(hi, start[i + 1] - ct);
          if (bl < bh) {
            last_item = i;
            last_end = (int)(bh - start[i] - cl);
            break;
          }
        }
      }
    }
    row[0] = first_item;
    row[1] = first_item >= 0 ? first_blk : 0;
    row[2] = last_item;
    row[3] = last_end;
    row[4] = first_item >= 0 ? split : 0;
    row[5] = 0;
    row[6] = 0;
    row[7] = 0;
  }
  if (tid == 0) {
    plan[0] = W;
    plan[1] = c;
    plan[2] = We;
    plan[3] = num_items;
    plan[4] = kPlanVersion;
    plan[5] = kPage;
    plan[6] = (int32_t)(uint32_t)((uint64_t)T & 0xffffffffu);   // T, low and high words
    plan[7] = (int32_t)((uint64_t)T >> 32);
  }
}

// The 64-bit schedule, out of line: it only runs when the total cost passes
// 2^31, and the kernel's 32-bit path stays compact.
__device__ __attribute__((noinline)) void plan_body_wide(const int32_t* seqlens, int topk,
                                                         int num_items, int item_div, int W, int c,
                                                         int32_t* plan, int32_t* num_splits,
                                                         int64_t* start, int64_t run, int64_t T,
                                                         int* sums_b, int* span_w) {
  plan_body<int64_t>(seqlens, topk, num_items, item_div, W, c, plan, num_splits, start, nullptr,
                     nullptr, run, T, sums_b, span_w);
}

// The same schedule for at most kPlanThreads items and workers on a 32-bit
// axis with W' T < 2^32 (every decode batch of up to 256 sequences or query
// tokens): thread t holds item t (n blocks, start `run`) and worker t, so no
// thread loops over items or workers and every division goes by
// multiplication.  Item t marks the workers its blocks reach in LDS
// (s_first / s_last), and worker t reads its first and last item from there.
// s_start has kPlanThreads + 1 entries; s_first and s_last kPlanThreads.
__device__ __forceinline__ void plan_small(int num_items, int W, int c, int32_t* __restrict__ plan,
                                           int32_t* __restrict__ num_splits, int n, int run, int T,
                                           int* s_start, int* s_first, int* s_last, int* sums_b) {
  const int tid = threadIdx.x;
  const int cl = (c + 1) / 2, ct = c / 2;   // an item's overhead: cl units before its blocks, ct after them
  const int We = min(W, T);
  const uint32_t mT = T > 0 ? 0xffffffffu / (uint32_t)T : 0u;
  const uint32_t mW = We > 0 ? 0xffffffffu / (uint32_t)We : 0u;
  auto owner = [&](int x) -> int {   // worker owning unit x (T >= 1 when any item has a block)
    return (int)udiv((uint32_t)(x + 1) * (uint32_t)We - 1u, (uint32_t)T, mT);
  };
  const bool has_item = tid < num_items;
  if (has_item) s_start[tid] = run;
  if (tid == 0) s_start[num_items] = T;
  if (tid < W) {
    s_first[tid] = num_items;   // none
    s_last[tid] = -1;
  }
  const int wl = has_item && n > 0 ? owner(run + cl) : 0;
  const int ns = has_item && n > 0 ? owner(run + cl + n - 1) - wl + 1 : 0;
  int S;
  const int sincl = block_inclusive_scan(ns, sums_b, S);   // its barrier publishes the stores above
  if (has_item) num_splits[tid] = sincl - ns;
  if (tid == 0) num_splits[num_items] = S;
  for (int w = wl; w < wl + ns; ++w) {
    atomicMin(&s_first[w], tid);
    atomicMax(&s_last[w], tid);
  }
  __syncthreads();
  if (tid < W) {
    // {first item, its first block, last item, end block in it, split number
    // of the first run}, or no blocks
    int fi = s_first[tid], first_blk = 0, li = -1, last_end = 0, split = 0;
    if (fi < num_items) {
      li = s_last[tid];
      const int lo = (int)udiv((uint32_t)tid * (uint32_t)T, (uint32_t)We, mW);
      const int hi = (int)udiv((uint32_t)(tid + 1) * (uint32_t)T, (uint32_t)We, mW);
      const int ff = s_start[fi] + cl;
      first_blk = max(lo, ff) - ff;
      last_end = min(hi, s_start[li + 1] - ct) - s_start[li] - cl;
      split = tid - owner(ff);
    } else {
      fi = -1;
    }
    int32_t* row = plan + kPlanWords * (1 + tid);
    row[0] = fi;
    row[1] = first_blk;
    row[2] = li;
    row[3] = last_end;
    row[4] = split;
    row[5] = 0;
    row[6] = 0;
    row[7] = 0;
  }
  if (tid == 0) {
    plan[0] = W;
    plan[1] = c;
    plan[2] = We;
    plan[3] = num_items;
    plan[4] = kPlanVersion;
    plan[5] = kPage;
    plan[6] = T;
    plan[7] = 0;
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seqlens,
                                                            int topk, int num_items, int item_div,
                                                            int W, int c,
                                                            int32_t* __restrict__ plan,
                                                            int32_t* __restrict__ num_splits,
                                                            int32_t* __restrict__ counters,
                                                            int num_counters) {
  // Item starts: int [num_items + 1] followed by the marking arrays, or int64
  // [num_items + 1] alone.
  constexpr int kStartInts = (kPlanMaxItems + 1 + 3) & ~3;
  static_assert(kStartInts + 2 * kScatterW <= 2 * (kPlanMaxItems + 1), "marking arrays must fit");
  __shared__ int64_t raw[kPlanMaxItems + 1];
  __shared__ int sums_lo[kPlanWaves], sums_hi[kPlanWaves], sums_b[kPlanWaves], span_w[kPlanWaves];
  const int tid = threadIdx.x;
  const int per = (num_items + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(tid * per, num_items), i1 = min(i0 + per, num_items);

  // arrival counters of the single-launch decode start at zero
  for (int i = tid; i < num_counters; i += kPlanThreads) counters[i] = 0;

  // Block counts, parked in the 32-bit start array, and the 64-bit total
  // (a thread's items cost below 64 (2^25 + 8) < 2^38).
  static_assert(kPlanMaxItems <= 64 * kPlanThreads, "at most 64 items per thread");
  int* start32 = reinterpret_cast<int*>(raw);
  int64_t local = 0;
  for (int i = i0; i < i1; ++i) {
    const int n = item_blocks(seqlens, topk, item_div, i);
    start32[i] = n;
    local += c + n;
  }
  int64_t total;
  const int64_t run = block_exclusive_scan64(local, sums_lo, sums_hi, total);
  if (num_items <= kPlanThreads && W <= kPlanThreads && total <= 0x7fffffff &&
      (uint64_t)min((int64_t)W, total) * (uint64_t)total < (1ull << 32)) {
    // one item per thread: its block count is the one parked by this thread
    plan_small(num_items, W, c, plan, num_splits, i1 > i0 ? start32[i0] : 0, (int)run, (int)total,
               start32, start32 + kStartInts, start32 + kStartInts + kScatterW, sums_b);
  } else if (total <= 0x7fffffff) {
    plan_body<int>(seqlens, topk, num_items, item_div, W, c, plan, num_splits, start32,
                   start32 + kStartInts, start32 + kStartInts + kScatterW, (int)run, (int)total,
                   sums_b, span_w);
  } else {
    plan_body_wide(seqlens, topk, num_items, item_div, W, c, plan, num_splits, raw, run, total,
                   sums_b, span_w);
  }
}

// Batches of more than kPlanMaxItems items (a sparse prefill of that many
// query tokens): the same schedule with no per-item state in LDS.  Each
// thread walks a contiguous range of items three times (block counts come
// from the lengths each time): the cost of its range; the split counts of
// its items, with each item marking the workers its blocks reach (LDS min /
// max of the item index, so W <= kScatterW); then each item writes the row
// words of the workers it is the first or the last item of, and num_splits.
// Worker threads write the rows of workers with no item and the zero words.
// The 64-bit axis throughout; the range costs are scanned by one thread.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel_large(const int32_t* __restrict__ seqlens,
                                                                  int topk, int num_items, int item_div,
                                                                  int W, int c,
                                                                  int32_t* __restrict__ plan,
                                                                  int32_t* __restrict__ num_splits,
                                                                  int32_t* __restrict__ counters,
                                                                  int num_counters) {
  __shared__ int first_s[kScatterW], last_s[kScatterW];
  __shared__ int64_t s_run[kPlanThreads + 1];
  __shared__ int sums_b[kPlanWaves];
  const int tid = threadIdx.x;
  const int per = (num_items + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(tid * per, num_items), i1 = min(i0 + per, num_items);
  const int cl = (c + 1) / 2, ct = c / 2;   // an item's overhead: cl units before its blocks, ct after them

  for (int i = tid; i < num_counters; i += kPlanThreads) counters[i] = 0;
  for (int w = tid; w < W; w += kPlanThreads) {
    first_s[w] = num_items;   // none
    last_s[w] = -1;
  }
  int64_t local = 0;
  for (int i = i0; i < i1; ++i) local += c + item_blocks(seqlens, topk, item_div, i);
  s_run[tid] = local;
  __syncthreads();
  if (tid == 0) {
    int64_t r = 0;
    for (int t = 0; t < kPlanThreads; ++t) {
      const int64_t v = s_run[t];
      s_run[t] = r;
      r += v;
    }
    s_run[kPlanThreads] = r;
  }
  __syncthreads();
  const int64_t run = s_run[tid], T = s_run[kPlanThreads];
  const int64_t We = min((int64_t)W, T);
  auto owner = [&](int64_t x) -> int { return (int)floor_div<true>((x + 1) * We - 1, T); };
  auto unit0 = [&](int w) -> int64_t { return floor_div<true>((int64_t)w * T, We); };

  // split counts, and the marks
  int nsplit = 0;
  int64_t C = run;
  for (int i = i0; i < i1; ++i) {
    const int n = item_blocks(seqlens, topk, item_div, i);
    if (n > 0) {
      const int wl = owner(C + cl), wh = owner(C + cl + n - 1);
      nsplit += wh - wl + 1;
      for (int w = wl; w <= wh; ++w) {
        atomicMin(&first_s[w], i);
        atomicMax(&last_s[w], i);
      }
    }
    C += c + n;
  }
  int S;
  const int sincl = block_inclusive_scan(nsplit, sums_b, S);   // its barrier publishes the marks

  // num_splits, and the row words of the workers whose first or last item it is
  int srun = sincl - nsplit;
  C = run;
  for (int i = i0; i < i1; ++i) {
    num_splits[i] = srun;
    const int n = item_blocks(seqlens, topk, item_div, i);
    if (n > 0) {
      const int64_t first = C + cl, end = C + cl + n;
      const int wl = owner(first), wh = owner(end - 1);
      for (int w = wl; w <= wh; ++w) {
        int32_t* row = plan + kPlanWords * (1 + w);
        if (first_s[w] == i) {
          row[0] = i;
          row[1] = (int)(max(unit0(w), first) - first);
          row[4] = w - wl;
        }
        if (last_s[w] == i) {
          row[2] = i;
          row[3] = (int)(min(unit0(w + 1), end) - first);
        }
      }
      srun += wh - wl + 1;
    }
    C += c + n;
  }
  if (tid == 0) num_splits[num_items] = S;
  for (int w = tid; w < W; w += kPlanThreads) {
    int32_t* row = plan + kPlanWords * (1 + w);
    if (first_s[w] == num_items) {
      row[0] = -1;
      row[1] = 0;
      row[2] = -1;
      row[3] = 0;
      row[4] = 0;
    }
    row[5] = 0;
    row[6] = 0;
    row[7] = 0;
  }
  if (tid == 0) {
    plan[0] = W;
    plan[1] = c;
    plan[2] = (int32_t)We;
    plan[3] = num_items;
    plan[4] = kPlanVersion;
    plan[5] = kPage;
    plan[6] = (int32_t)(uint32_t)((uint64_t)T & 0xffffffffu);   // T, low and high words
    plan[7] = (int32_t)((uint64_t)T >> 32);
  }
}

}  // namespace

int plan_max_items() { return kPlanLargeItems; }
int plan_large_max_workers(int num_items) { return num_items > kPlanMaxItems ? kScatterW : (1 << 20); }

hipError_t launch_plan(const int32_t* seqlens, int topk, int num_items, int item_div, int num_workers,
                       int overhead, int32_t* plan, int32_t* num_splits, int32_t* counters,
                       int num_counters, hipStream_t stream) {
  if (num_items > kPlanMaxItems)
    hipLaunchKernelGGL(plan_kernel_large, dim3(1), dim3(kPlanThreads), 0, stream, seqlens, topk,
                       num_items, item_div, num_workers, overhead, plan, num_splits, counters,
                       num_counters);
  else
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seqlens, topk, num_items,
                       item_div, num_workers, overhead, plan, num_splits, counters, num_counters);
  return hipGetLastError();
}

}  // namespace mla
