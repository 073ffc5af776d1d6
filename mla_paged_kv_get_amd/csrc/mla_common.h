// Shared constants, device helpers and launch descriptors of the gfx950 paged
// MLA decode library.  Kernels live in mla_plan.hip, mla_decode.hip and
// mla_aux.hip; the C ABI in mla_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;                 // tokens per cache page
constexpr int kDqk = 576;                 // values per latent row (512 latent + 64 RoPE)
constexpr int kDv = 512;                  // V = first 512 values of the row
constexpr int kRowBytes = kDqk * 2;       // 1152 B per cached row
constexpr int kChunks = kRowBytes / 16;   // 72 chunks of 16 B per row
constexpr int kTileBytes = kPage * kRowBytes;  // 73728 B per 64-row tile
// Packed FP8 rows: 512 E4M3 latent codes, 4 float32 scales (one per 128
// latent values), 64 bf16 RoPE values.
constexpr int kRowBytes8 = 656;
constexpr int kRaw8Bytes = kPage * kRowBytes8;     // 41984 B per 64-row tile as copied
constexpr int kRaw8ScaleOff = kPage * 640;         // scales of a copied tile: [4 blocks][64 rows] float32
constexpr int kPlanWords = 8;
constexpr int kPlanVersion = 3;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#define MLA_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define MLA_GBL(p) ((const __attribute__((address_space(1))) void*)(p))

// Whether an index-list entry is a key of a sequence of length L.
__device__ __forceinline__ bool sparse_key_valid(int idx, int L) {
  return idx >= 0 && idx < L;
}

// Arguments of the decode kernels (passed by value).
struct DecodeArgs {
  const uint16_t* q;          // [items * M, 576]   (dense: [B, s_q, h_q, 576])
  const uint16_t* kv;         // [num_pages * 64, 576]
  const int32_t* block_table; // [B, max_blocks]
  const int32_t* seqlens;     // [B]
  const int32_t* indices;     // [B * s_q, topk] or null
  const int32_t* plan;        // [(W + 1) * 8]
  const int32_t* num_splits;  // [items + 1]
  uint16_t* o;                // [items * M, 512]
  float* lse;                 // [items * M]
  uint16_t* part_o;           // [slots * part_rows, 512] bf16 partial outputs
  float* part_lse;            // [slots * part_rows] their LSEs
  int part_rows;              // rows per partial slot: M, or M rounded up to 32 (128-row variant)
  int part_blocks;            // partial O in 32-row blocks in accumulator order (128-row, two launches)
  int max_blocks;
  int batch;
  int s_q;
  int h_q;
  int M;                      // query rows per item
  int num_items;
  int num_workers;
  int m_tiles;                // workgroups per worker (row tiles)
  int topk;                   // 0 = dense
  int causal;
  float scale_log2;           // softmax_scale * log2(e)
  int h_kv;                   // latent KV heads (items are (sequence or query token, KV head))
  int G;                      // query heads per KV head, h_q / h_kv
  int kv_format;              // 0: bf16 rows; 1: packed FP8 rows
  int d_qk;                   // values per cached row: 576 (512 latent + 64 RoPE) or 512
  // Sparse mode with a second (auxiliary) cache: item keys are the main
  // list's tiles (nb1 = ceil(topk / 64) of them) followed by the auxiliary
  // list's; kv2 == nullptr when there is none.
  const uint16_t* kv2;
  const int32_t* block_table2;
  const int32_t* seqlens2;
  const int32_t* indices2;
  int max_blocks2;
  int topk2;
  int nb1;                    // tiles of the main list of a sparse item
  int nb_sparse;              // tiles of a sparse item (both lists)
  // Single-launch mode: the decode kernel merges the partials of split items
  // itself (the last run of an item and row tile to finish does it) and
  // writes the items without keys; arrivals[item * m_tiles + row tile] (in
  // the plan, after its rows) counts finished runs and is zero outside a
  // launch.
  int fused;
  int* arrivals;
  // Division of an item index by the items per sequence (topk > 0: h_kv s_q,
  // else h_kv) and by h_kv, by multiplication: mul = floor((2^32 - 1) / div)
  // (set on the host; see div_by).
  unsigned seq_div, seq_mul, head_mul;
  // Indexing probe (null in normal calls): the kernel also writes, for every
  // row it copies, the byte offset from kv of the cache row the copy reads:
  // dbg_rows[(item * dbg_tiles + tile) * 64 + row of the tile]; packed FP8
  // rows add the row whose scales the copy reads at dbg_rows[dbg_plane + same
  // index].  Entries of tiles no run copies are left as they were.
  int64_t* dbg_rows;
  int dbg_tiles;
  int64_t dbg_plane;
};

// floor(n / d) for 0 <= n < 2^31 from m = floor((2^32 - 1) / d): the high
// word of n m is floor(n / d) or one less (its error is below 2 n / 2^32 < 1),
// and one comparison settles which.
__device__ __forceinline__ int div_by(int n, unsigned d, unsigned m) {
  unsigned q = __umulhi((unsigned)n, m);
  if ((unsigned)n - q * d >= d) ++q;
  return (int)q;
}

// Row of q / o / lse ([batch * s_q * h_q] rows) holding query row `row` of
// work item `item`.  Dense: item = b * h_kv + g, row = s * G + j -> token
// (b, s), head g * G + j.  Sparse: item = (b * s_q + s) * h_kv + g, row = j.
__device__ __forceinline__ int64_t q_row(const DecodeArgs& a, int item, int row) {
  const int tok_or_b = div_by(item, (unsigned)a.h_kv, a.head_mul), g = item - tok_or_b * a.h_kv;
  if (a.topk > 0) return (int64_t)tok_or_b * (a.h_kv * a.G) + g * a.G + row;
  const int s = row / a.G, j = row - s * a.G;
  return ((int64_t)tok_or_b * a.s_q + s) * (a.h_kv * a.G) + g * a.G + j;
}
// Sequence (block-table row, length) of work item `item`.
__device__ __forceinline__ int item_seq(const DecodeArgs& a, int item) {
  return div_by(item, a.seq_div, a.seq_mul);
}

// Launchers (defined next to their kernels).
hipError_t launch_plan(const int32_t* seqlens, int topk, int num_items, int item_div, int num_workers,
                       int overhead, int32_t* plan, int32_t* num_splits, int32_t* counters,
                       int num_counters, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int variant, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_validate(const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                           int batch, int s_q, const int32_t* indices, int topk,
                           int64_t num_pages, int32_t* error_count, hipStream_t stream);

// Decode variants: how a workgroup covers an item's query rows.
enum Variant : int {
  kVariantRows16 = 0,    // <= 16 rows: 4 waves split each 64-token tile 4 ways
  kVariantRows64 = 1,    // 17..64 rows (and packed FP8 caches above 16): 64-row
                         // tiles, two wave pairs of 32 rows
  kVariantRows128 = 2,   // > 64 rows, bf16 caches: 128-row tiles, each wave 32
                         // rows over every key and output column
};
constexpr int variant_rows(int v) { return v == kVariantRows16 ? 16 : v == kVariantRows64 ? 64 : 128; }
// Plan cost of a run of an item, in blocks, laid out half before and half
// after its blocks (measured: an item boundary costs about 1.6 tiles of a
// 16-row worker, where 1 unit ahead of the blocks balanced best; items over
// 64 rows balanced best at 3, split 2 + 1, among 2 to 6).  The variant is
// the one the decode of the plan's cache format runs (the metadata calls for
// bf16 and for packed FP8 caches).
constexpr int variant_overhead(int v) { return v == kVariantRows16 ? 1 : v == kVariantRows128 ? 3 : 4; }
// kv_format 0: bf16 rows; 1: packed FP8 rows (no 128-row variant).
inline int pick_variant(int rows_per_item, int kv_format) {
  if (rows_per_item <= 16) return kVariantRows16;
  return (kv_format == 1 || rows_per_item <= 64) ? kVariantRows64 : kVariantRows128;
}
// Arrival counters per item of the single-launch decode: one per row tile of
// the narrowest variant the row count can run with (any cache format).
inline int counter_tiles(int rows_per_item) { return rows_per_item <= 16 ? 1 : (rows_per_item + 63) / 64; }

}  // namespace mla
