// Split-KV tile scheduler ("get_mla_metadata" of "What is FlashMLA",
// topnet.top, installation-and-use section, step 2: it returns the tile
// scheduler metadata and num_splits).  The pages do not say how work is split;
// this kernel implements the rule stated in the C header:
//   n_i = ceil(len_i / 64) blocks, item cost = overhead + n_i, items laid end
//   to end on a cost axis (start C_i, total T); the first W' = min(W, T)
//   workers share the axis evenly, worker w owning units
//   [floor(w T / W'), floor((w + 1) T / W')); block b of item i sits on unit
//   C_i + overhead + b.
// One workgroup computes it from closed forms: unit x belongs to worker
// floor(((x + 1) W' - 1) / T), so the workers touching item i's blocks are
// owner(C_i + overhead) .. owner(C_{i+1} - 1), every one of them with at
// least one block, and the split count and split numbers follow without a walk.
// A worker's first and last items are the least and greatest items that reach
// it.  With up to kScatterW workers and no item reaching more than
// kScatterSpan of them, each item marks its workers (LDS min / max); otherwise
// each worker searches the item starts.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanMaxItems = 16384;
constexpr int kScatterW = 4096;
constexpr int kScatterSpan = 32;

// floor(n / d) for n < 2^32 from m = floor((2^32 - 1) / d): the high word of
// n m is the quotient or one less, and one comparison settles which.
__device__ __forceinline__ uint32_t udiv(uint32_t n, uint32_t d, uint32_t m) {
  uint32_t q = __umulhi(n, m);
  if (n - q * d >= d) ++q;
  return q;
}

// floor(num / den) for 0 <= num < 2^53 and den >= 1: the quotient in double
// precision is within one of the floor, and one comparison each way fixes it.
__device__ __forceinline__ int64_t floor_div(int64_t num, int64_t den) {
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

// Blocks of item i: topk keys (sparse) or the length of its sequence i / item_div
// (dense; item_div = number of KV heads, items being (sequence, KV head)).
__device__ __forceinline__ int item_blocks(const int32_t* seqlens, int topk, int item_div, int i) {
  const int len = topk > 0 ? topk : seqlens[i / item_div];
  return len > 0 ? (len + kPage - 1) / kPage : 0;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seqlens,
                                                            int topk, int num_items, int item_div,
                                                            int W, int c,
                                                            int32_t* __restrict__ plan,
                                                            int32_t* __restrict__ num_splits,
                                                            int32_t* __restrict__ counters,
                                                            int num_counters) {
  __shared__ int start[kPlanMaxItems + 1];
  __shared__ int first_s[kScatterW], last_s[kScatterW];   // least / greatest item reaching worker w
  __shared__ int sums_a[kPlanWaves], sums_b[kPlanWaves], span_w[kPlanWaves];
  const int tid = threadIdx.x;
  const int per = (num_items + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(tid * per, num_items), i1 = min(i0 + per, num_items);

  // arrival counters of the single-launch decode start at zero
  for (int i = tid; i < num_counters; i += kPlanThreads) counters[i] = 0;
  if (W <= kScatterW) {
    for (int w = tid; w < W; w += kPlanThreads) {
      first_s[w] = num_items;   // none
      last_s[w] = -1;
    }
  }

  // Start of every item on the cost axis (the blocks are parked in start[]
  // until the scan is done).
  int local = 0;
  for (int i = i0; i < i1; ++i) {
    const int n = item_blocks(seqlens, topk, item_div, i);
    start[i] = n;
    local += c + n;
  }
  int T;
  const int incl = block_inclusive_scan(local, sums_a, T);
  int run = incl - local;
  for (int i = i0; i < i1; ++i) {
    const int n = start[i];
    start[i] = run;
    run += c + n;
  }
  if (tid == 0) start[num_items] = T;
  __syncthreads();
  const int We = min(W, T);
  // The divisions below are by T or by W', with numerators under W' T.  When
  // that is below 2^32 they go by multiplication, otherwise in double precision.
  const bool narrow = T > 0 && (uint64_t)We * (uint64_t)T < (1ull << 32);
  const uint32_t mT = narrow ? 0xffffffffu / (uint32_t)T : 0u;
  const uint32_t mW = narrow ? 0xffffffffu / (uint32_t)We : 0u;
  // Owner of unit x (T >= 1 whenever an item has a block), and the first unit
  // of worker w <= W'.
  auto owner = [&](int x) -> int {
    if (T <= 0) return 0;
    const int64_t n = ((int64_t)x + 1) * We - 1;
    return narrow ? (int)udiv((uint32_t)n, (uint32_t)T, mT) : (int)floor_div(n, T);
  };
  auto unit0 = [&](int w) -> int {
    const int64_t n = (int64_t)w * T;
    return narrow ? (int)udiv((uint32_t)n, (uint32_t)We, mW) : (int)floor_div(n, We);
  };

  // Split counts (the number of workers each item reaches) and the largest.
  local = 0;
  int span = 0;
  for (int i = i0; i < i1; ++i) {
    const int first = start[i] + c, end = start[i + 1];
    if (end > first) {
      const int n = owner(end - 1) - owner(first) + 1;
      local += n;
      span = max(span, n);
    }
  }
  const bool wide = __builtin_amdgcn_ballot_w64(span > kScatterSpan) != 0;
  if ((tid & 63) == 0) span_w[tid >> 6] = wide;   // published by the scan's barrier
  int S;
  const int sincl = block_inclusive_scan(local, sums_b, S);
  bool any_wide = false;
  for (int j = 0; j < kPlanWaves; ++j) any_wide |= span_w[j] != 0;
  const bool scatter = W <= kScatterW && !any_wide;
  run = sincl - local;
  for (int i = i0; i < i1; ++i) {
    num_splits[i] = run;
    const int first = start[i] + c, end = start[i + 1];
    if (end > first) {
      const int wl = owner(first), wh = owner(end - 1);
      run += wh - wl + 1;
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
    int lo = T, hi = T;
    if (w < We) {
      lo = unit0(w);
      hi = unit0(w + 1);
    }
    int first_item = -1, first_blk = 0, last_item = -1, last_end = 0, split = 0;
    if (scatter) {
      if (first_s[w] < num_items) {
        first_item = first_s[w];
        last_item = last_s[w];
        const int ff = start[first_item] + c;
        first_blk = max(lo, ff) - ff;
        split = w - owner(ff);
        last_end = min(hi, start[last_item + 1]) - start[last_item] - c;
      }
    } else if (lo < hi) {
      // Last item starting at or before lo.
      int a = 0, b = num_items - 1;
      while (a < b) {
        const int m = (a + b + 1) >> 1;
        if (start[m] <= lo) a = m; else b = m - 1;
      }
      for (int i = a; i < num_items && start[i] < hi; ++i) {
        const int bl = max(lo, start[i] + c), bh = min(hi, start[i + 1]);
        if (bl < bh) {
          first_item = i;
          first_blk = bl - start[i] - c;
          split = w - owner(start[i] + c);
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
          const int bl = max(lo, start[i] + c), bh = min(hi, start[i + 1]);
          if (bl < bh) {
            last_item = i;
            last_end = bh - start[i] - c;
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
    plan[6] = T;
    plan[7] = 0;
  }
}

}  // namespace

int plan_max_items() { return kPlanMaxItems; }

hipError_t launch_plan(const int32_t* seqlens, int topk, int num_items, int item_div, int num_workers,
                       int overhead, int32_t* plan, int32_t* num_splits, int32_t* counters,
                       int num_counters, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seqlens, topk, num_items,
                     item_div, num_workers, overhead, plan, num_splits, counters, num_counters);
  return hipGetLastError();
}

}  // namespace mla
