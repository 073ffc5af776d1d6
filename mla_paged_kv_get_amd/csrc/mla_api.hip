// C ABI of the paged MLA decode library (declared in include/mla_paged_kv.h).
// Host-side argument checks, worker sizing and kernel launches; the kernels
// are in mla_plan.hip, mla_decode.hip and mla_aux.hip.
#include "mla_paged_kv.h"

#include <math.h>

#include <atomic>
#include <mutex>

#include "mla_common.h"

namespace mla {
int plan_max_items();
int plan_large_max_workers(int num_items);
}

namespace {

using namespace mla;

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];   // 0 = not queried yet

int cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return MLA_ERR_HIP;
    g_cu_count[dev] = n;
  }
  *out = g_cu_count[dev];
  return MLA_OK;
}

struct Shape {
  int items;        // work items
  int rows;         // query rows per item
  int variant;
  int m_tiles;      // workgroups per worker
};

// kv_format selects the decode variant (0: bf16 rows; 1: packed FP8 rows).
// Plans are sized for bf16 rows: an FP8 decode may run more workgroups per
// worker than the plan's W assumed (its row tiles are narrower), which only
// lengthens the grid.
int shape_of(int batch, int s_q, int num_q_rows, int h_kv, int topk, Shape* s, int kv_format = 0) {
  if (batch < 0 || s_q < 1 || num_q_rows < 1 || h_kv < 1) return MLA_ERR_INVALID_ARGUMENT;
  // Items: (sequence, KV head) in dense mode, (query token, KV head) in sparse mode.
  if (topk > 0) {
    if (num_q_rows % s_q) return MLA_ERR_INVALID_ARGUMENT;
    const int64_t items = (int64_t)batch * s_q * h_kv;
    if (items > (1 << 30)) return MLA_ERR_INVALID_ARGUMENT;
    s->items = (int)items;
    s->rows = num_q_rows / s_q;
  } else {
    const int64_t items = (int64_t)batch * h_kv;
    if (items > (1 << 30)) return MLA_ERR_INVALID_ARGUMENT;
    s->items = (int)items;
    s->rows = num_q_rows;
  }
  s->variant = pick_variant(s->rows, kv_format);
  const int vr = variant_rows(s->variant);
  s->m_tiles = (s->rows + vr - 1) / vr;
  return MLA_OK;
}

int workers_for(const Shape& s, int request, int* W) {
  if (request > 0) {
    *W = request;
    return MLA_OK;
  }
  int cus = 0;
  const int st = cu_count(&cus);
  if (st != MLA_OK) return st;
  // One workgroup per CU (each holds two 72 KB tiles of LDS); the row tiles of
  // a worker share the CUs.
  *W = cus / s.m_tiles > 0 ? cus / s.m_tiles : 1;
  return MLA_OK;
}

// Rows per partial slot: the 128-row variant writes its partials in blocks of
// 32 rows, so its slots are rounded up to a whole number of blocks.
int part_rows_of(const Shape& s) {
  return s.variant == kVariantRows128 ? (s.rows + 31) / 32 * 32 : s.rows;
}

size_t workspace_for(const Shape& s, int dv, int W) {
  const size_t slots = (size_t)s.items + (size_t)W;
  // bf16 partial outputs, then their fp32 LSEs
  return slots * (size_t)part_rows_of(s) * ((size_t)dv * sizeof(uint16_t) + sizeof(float));
}

// Arrival counters of the single-launch mode, after the plan's rows: one per
// item and row tile of the narrowest variant (so that a decode of either cache
// format indexes inside them).
int64_t plan_counters(const Shape& s) { return (int64_t)s.items * counter_tiles(s.rows); }

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape (needs d_qk=576, dv=512, page 64)";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the no-alloc decode's fixed buffer holds";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// The plan's sizes and the plan for decodes of one cache format (kv_format 0:
// bf16 rows; 1: packed FP8 rows): the format picks the decode variant, whose
// row tiles set the default worker count and whose overhead is the plan's.
int plan_dims_for(int batch, int s_q, int num_q_rows, int h_kv, int topk, int kv_format,
                  int num_workers_request, int* out_num_workers, int* out_plan_words,
                  int* out_num_items) {
  if (!out_num_workers || !out_plan_words || !out_num_items) return MLA_ERR_INVALID_ARGUMENT;
  if (num_workers_request < 0) return MLA_ERR_INVALID_ARGUMENT;
  Shape s;
  int st = shape_of(batch, s_q, num_q_rows, h_kv, topk, &s, kv_format);
  if (st != MLA_OK) return st;
  if (num_workers_request > (1 << 20)) return MLA_ERR_INVALID_ARGUMENT;
  int W = 0;
  st = workers_for(s, num_workers_request, &W);
  if (st != MLA_OK) return st;
  const int64_t words = (int64_t)kPlanWords * (W + 1) + plan_counters(s);
  if (words > 0x7fffffff) return MLA_ERR_UNSUPPORTED;
  *out_num_workers = W;
  *out_plan_words = (int)words;
  *out_num_items = s.items;
  return MLA_OK;
}

int get_metadata_for(const int32_t* cache_seqlens, int batch, int s_q, int num_q_rows, int h_kv,
                     int topk, int topk2, int kv_format, int num_workers, int32_t* plan,
                     int32_t* num_splits, void* stream) {
  if (!plan || !num_splits) return MLA_ERR_INVALID_ARGUMENT;
  if (topk <= 0 && !cache_seqlens && batch > 0) return MLA_ERR_INVALID_ARGUMENT;
  if (num_workers < 1 || num_workers > (1 << 20)) return MLA_ERR_INVALID_ARGUMENT;
  if (topk2 < 0 || (topk2 > 0 && topk <= 0)) return MLA_ERR_INVALID_ARGUMENT;
  Shape s;
  const int st = shape_of(batch, s_q, num_q_rows, h_kv, topk, &s, kv_format);
  if (st != MLA_OK) return st;
  if (s.items > mla::plan_max_items()) return MLA_ERR_UNSUPPORTED;
  if (num_workers > mla::plan_large_max_workers(s.items)) return MLA_ERR_UNSUPPORTED;
  // Sparse items: the tiles of the main list, then those of the auxiliary list
  // (dual cache), each list in 64-key tiles.
  int64_t tile_keys = 0;
  if (topk > 0) {
    tile_keys = (int64_t)kPage * (((int64_t)topk + kPage - 1) / kPage + ((int64_t)topk2 + kPage - 1) / kPage);
    if (tile_keys > 0x7fffffff) return MLA_ERR_UNSUPPORTED;
  }
  const int overhead = variant_overhead(s.variant);
  const hipError_t e = launch_plan(cache_seqlens, (int)tile_keys, s.items, h_kv, num_workers,
                                   overhead, plan, num_splits,
                                   plan + (int64_t)kPlanWords * (num_workers + 1),
                                   (int)plan_counters(s), reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

int mla_plan_dims(int batch, int s_q, int num_q_rows, int h_kv, int topk, int num_workers_request,
                  int* out_num_workers, int* out_plan_words, int* out_num_items) {
  return plan_dims_for(batch, s_q, num_q_rows, h_kv, topk, 0, num_workers_request, out_num_workers,
                       out_plan_words, out_num_items);
}

int mla_plan_dims_fp8(int batch, int s_q, int num_q_rows, int h_kv, int topk, int num_workers_request,
                      int* out_num_workers, int* out_plan_words, int* out_num_items) {
  return plan_dims_for(batch, s_q, num_q_rows, h_kv, topk, 1, num_workers_request, out_num_workers,
                       out_plan_words, out_num_items);
}

int mla_plan_num_workers(int plan_words, int batch, int s_q, int num_q_rows, int h_kv, int topk) {
  Shape s;
  if (shape_of(batch, s_q, num_q_rows, h_kv, topk, &s) != MLA_OK) return -1;
  const int64_t rows_words = (int64_t)plan_words - plan_counters(s);
  if (rows_words < 2 * kPlanWords || rows_words % kPlanWords) return -1;
  return (int)(rows_words / kPlanWords - 1);
}

int mla_get_metadata(const int32_t* cache_seqlens, int batch, int s_q, int num_q_rows, int h_kv,
                     int topk, int topk2, int num_workers, int32_t* plan, int32_t* num_splits,
                     void* stream) {
  return get_metadata_for(cache_seqlens, batch, s_q, num_q_rows, h_kv, topk, topk2, 0, num_workers,
                          plan, num_splits, stream);
}

int mla_get_metadata_fp8(const int32_t* cache_seqlens, int batch, int s_q, int num_q_rows, int h_kv,
                         int topk, int num_workers, int32_t* plan, int32_t* num_splits, void* stream) {
  return get_metadata_for(cache_seqlens, batch, s_q, num_q_rows, h_kv, topk, 0, 1, num_workers, plan,
                          num_splits, stream);
}

size_t mla_workspace_bytes(int batch, int s_q, int num_q_rows, int h_kv, int topk, int dv,
                           int num_workers) {
  Shape s;
  if (shape_of(batch, s_q, num_q_rows, h_kv, topk, &s) != MLA_OK || dv < 1 || num_workers < 1)
    return 0;
  return workspace_for(s, dv, num_workers);
}

}  // extern "C"

namespace {
// The auxiliary cache of the dual-cache sparse decode.
struct AuxCache {
  const void* kv;
  int64_t num_pages;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seqlens;
  const int32_t* indices;
  int topk;
};

// The decode for both cache formats (kv_format 0: bf16 rows of d_qk values;
// 1: packed FP8 rows of kRowBytes8 bytes holding d_qk values), with an
// optional auxiliary cache (sparse mode only).
int decode_impl(const void* q, const void* kvcache, int64_t num_pages, int page_size,
                const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                int batch, int s_q, int h_q, int h_kv, int d_qk, int dv, const int32_t* plan,
                const int32_t* num_splits, int num_workers, int causal, float softmax_scale,
                const int32_t* indices, int topk, void* o, float* lse, void* workspace,
                size_t workspace_bytes, int kv_format, const AuxCache* aux, int phases,
                void* stream, int64_t* dbg_rows = nullptr, int64_t dbg_elems = 0,
                int (*fixed_scratch)(void**) = nullptr) {
  if (phases < 1 || phases > 4) return MLA_ERR_INVALID_ARGUMENT;
  if (batch < 0 || s_q < 1 || h_q < 1 || h_kv < 1 || max_blocks < 1 || num_pages < 1)
    return MLA_ERR_INVALID_ARGUMENT;
  if (h_q % h_kv) return MLA_ERR_INVALID_ARGUMENT;
  if (page_size != kPage || dv != kDv) return MLA_ERR_UNSUPPORTED;
  if (d_qk != kDqk && !(d_qk == 512 && kv_format == 0)) return MLA_ERR_UNSUPPORTED;
  // The per-sequence arrays (query rows, block tables, lengths, index lists,
  // outputs) may be null when there is no sequence.
  const bool any = batch > 0;
  if (aux) {
    if (topk <= 0 || aux->topk < 0 || aux->num_pages < 1 || aux->max_blocks < 1 || !aux->kv ||
        (any && (!aux->block_table || !aux->seqlens)) || (aux->topk <= 0 && aux->indices) ||
        (any && aux->topk > 0 && !aux->indices))
      return MLA_ERR_INVALID_ARGUMENT;
    if ((int64_t)aux->max_blocks * kPage > (int64_t)0x7fffffff) return MLA_ERR_INVALID_ARGUMENT;
    if (aux->num_pages > ((int64_t)1 << 31) / kPage) return MLA_ERR_UNSUPPORTED;
  }
  if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARGUMENT;
  if ((topk <= 0 && indices) || (any && topk > 0 && !indices)) return MLA_ERR_INVALID_ARGUMENT;
  if (topk > 0 && causal) return MLA_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARGUMENT;
  if (num_workers < 1 || num_workers > (1 << 20)) return MLA_ERR_INVALID_ARGUMENT;
  if (!kvcache || !plan || !num_splits) return MLA_ERR_INVALID_ARGUMENT;
  if (any && (!q || !block_table || !cache_seqlens || !o || !lse)) return MLA_ERR_INVALID_ARGUMENT;
  if ((int64_t)max_blocks * kPage > (int64_t)0x7fffffff) return MLA_ERR_INVALID_ARGUMENT;
  if (num_pages > ((int64_t)1 << 31) / kPage) return MLA_ERR_UNSUPPORTED;
  Shape s;
  const int num_q_rows = s_q * h_q / h_kv;
  int st = shape_of(batch, s_q, num_q_rows, h_kv, topk, &s, kv_format);
  if (st != MLA_OK) return st;
  const size_t need = workspace_for(s, dv, num_workers);
  // fixed_scratch: the no-alloc decode, whose buffer (workspace_bytes long) is
  // only looked up once every argument has been checked and there is work.
  if (workspace_bytes < need) return fixed_scratch ? MLA_ERR_SCRATCH_LIMIT : MLA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace && !fixed_scratch) return MLA_ERR_INVALID_ARGUMENT;
  // Probe: one int64 per (item, tile, row) of every tile an item can have (and
  // a second plane for the scale rows of packed FP8 tiles).
  const int nb_sparse = topk > 0 ? (topk + kPage - 1) / kPage +
                                       (aux && aux->topk > 0 ? (aux->topk + kPage - 1) / kPage : 0)
                                 : 0;
  const int dbg_tiles = topk > 0 ? nb_sparse : max_blocks;
  const int64_t dbg_plane = (int64_t)s.items * dbg_tiles * kPage;
  if (dbg_rows) {
    if (phases == 2 || phases == 4) return MLA_ERR_INVALID_ARGUMENT;
    if (dbg_elems < dbg_plane * (kv_format == 1 ? 2 : 1)) return MLA_ERR_INVALID_ARGUMENT;
  }
  if (batch == 0) return MLA_OK;
  if (fixed_scratch) {
    const int st_ws = fixed_scratch(&workspace);
    if (st_ws != MLA_OK) return st_ws;
  }

  DecodeArgs a;
  a.dbg_rows = dbg_rows;
  a.dbg_tiles = dbg_tiles;
  a.dbg_plane = dbg_plane;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kvcache);
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.indices = indices;
  a.plan = plan;
  a.num_splits = num_splits;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  const size_t slots = (size_t)s.items + (size_t)num_workers;
  a.part_rows = part_rows_of(s);
  a.part_o = static_cast<uint16_t*>(workspace);
  a.part_lse = reinterpret_cast<float*>(a.part_o + slots * (size_t)a.part_rows * kDv);
  // the plan carries the arrival counters (zeroed by mla_get_metadata)
  a.arrivals = const_cast<int32_t*>(plan) + (int64_t)kPlanWords * (num_workers + 1);
  a.fused = phases == 4;
  a.part_blocks = s.variant == kVariantRows128 && !a.fused;
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.s_q = s_q;
  a.h_q = h_q;
  a.M = s.rows;
  a.num_items = s.items;
  a.num_workers = num_workers;
  a.m_tiles = s.m_tiles;
  a.topk = topk > 0 ? topk : 0;
  a.causal = causal;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.h_kv = h_kv;
  a.G = h_q / h_kv;
  a.seq_div = (unsigned)(topk > 0 ? h_kv * s_q : h_kv);
  a.seq_mul = 0xffffffffu / a.seq_div;
  a.head_mul = 0xffffffffu / (unsigned)h_kv;
  a.kv_format = kv_format;
  a.d_qk = d_qk;
  a.nb1 = topk > 0 ? (topk + kPage - 1) / kPage : 0;
  a.nb_sparse = nb_sparse;
  a.kv2 = nullptr;
  a.block_table2 = nullptr;
  a.seqlens2 = nullptr;
  a.indices2 = nullptr;
  a.max_blocks2 = 0;
  a.topk2 = 0;
  if (aux && aux->topk > 0) {
    a.kv2 = static_cast<const uint16_t*>(aux->kv);
    a.block_table2 = aux->block_table;
    a.seqlens2 = aux->seqlens;
    a.indices2 = aux->indices;
    a.max_blocks2 = aux->max_blocks;
    a.topk2 = aux->topk;
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (phases == 4) {
    if (launch_decode(a, s.variant, hs) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
  }
  if (phases & 1) {
    if (launch_decode(a, s.variant, hs) != hipSuccess) return MLA_ERR_HIP;
  }
  if (phases & 2) {
    if (launch_combine(a, hs) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

// The no-alloc decode's scratch: one copy per GPU the library runs on, held
// until the process ends.  Host code never uses this name as an address (on
// the host it is a stand-in); it uses the device address looked up below.
static __device__ __align__(256) unsigned char scratch[MLA_NO_ALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up once per device.
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_with_kvcache_no_alloc(const void* q, const void* kvcache, int64_t num_pages,
                                     int page_size, const int32_t* block_table, int max_blocks,
                                     const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                     int h_kv, int d_qk, int dv, const int32_t* plan,
                                     const int32_t* num_splits, int num_workers, int causal,
                                     float softmax_scale, const int32_t* indices, int topk,
                                     void* o, float* lse, void* stream) {
  return decode_impl(q, kvcache, num_pages, page_size, block_table, max_blocks, cache_seqlens,
                     batch, s_q, h_q, h_kv, d_qk, dv, plan, num_splits, num_workers, causal,
                     softmax_scale, indices, topk, o, lse, nullptr, MLA_NO_ALLOC_SCRATCH_BYTES, 0,
                     nullptr, 3, stream, nullptr, 0, scratch_ptr);
}

int mla_decode_with_kvcache_phase(const void* q, const void* kvcache, int64_t num_pages,
                                  int page_size, const int32_t* block_table, int max_blocks,
                                  const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                  int h_kv, int d_qk, int dv, const int32_t* plan,
                                  const int32_t* num_splits, int num_workers, int causal,
                                  float softmax_scale, const int32_t* indices, int topk, void* o,
                                  float* lse, void* workspace, size_t workspace_bytes, int phases,
                                  void* stream) {
  return decode_impl(q, kvcache, num_pages, page_size, block_table, max_blocks, cache_seqlens,
                     batch, s_q, h_q, h_kv, d_qk, dv, plan, num_splits, num_workers, causal,
                     softmax_scale, indices, topk, o, lse, workspace, workspace_bytes, 0, nullptr,
                     phases, stream);
}

int mla_decode_with_kvcache(const void* q, const void* kvcache, int64_t num_pages, int page_size,
                            const int32_t* block_table, int max_blocks,
                            const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                            int d_qk, int dv, const int32_t* plan, const int32_t* num_splits,
                            int num_workers, int causal, float softmax_scale,
                            const int32_t* indices, int topk, void* o, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, kvcache, num_pages, page_size, block_table, max_blocks, cache_seqlens,
                     batch, s_q, h_q, h_kv, d_qk, dv, plan, num_splits, num_workers, causal,
                     softmax_scale, indices, topk, o, lse, workspace, workspace_bytes, 0, nullptr, 3,
                     stream);
}

int mla_decode_with_kvcache_fp8_phase(const void* q, const void* kvcache, int64_t num_pages,
                                      int page_size, const int32_t* block_table, int max_blocks,
                                      const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                      int h_kv, int d_qk, int dv, const int32_t* plan,
                                      const int32_t* num_splits, int num_workers, int causal,
                                      float softmax_scale, const int32_t* indices, int topk,
                                      void* o, float* lse, void* workspace,
                                      size_t workspace_bytes, int phases, void* stream) {
  return decode_impl(q, kvcache, num_pages, page_size, block_table, max_blocks, cache_seqlens,
                     batch, s_q, h_q, h_kv, d_qk, dv, plan, num_splits, num_workers, causal,
                     softmax_scale, indices, topk, o, lse, workspace, workspace_bytes, 1, nullptr,
                     phases, stream);
}

int mla_decode_with_kvcache_fp8(const void* q, const void* kvcache, int64_t num_pages,
                                int page_size, const int32_t* block_table, int max_blocks,
                                const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                int h_kv, int d_qk, int dv, const int32_t* plan,
                                const int32_t* num_splits, int num_workers, int causal,
                                float softmax_scale, const int32_t* indices, int topk, void* o,
                                float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_impl(q, kvcache, num_pages, page_size, block_table, max_blocks, cache_seqlens,
                     batch, s_q, h_q, h_kv, d_qk, dv, plan, num_splits, num_workers, causal,
                     softmax_scale, indices, topk, o, lse, workspace, workspace_bytes, 1, nullptr, 3,
                     stream);
}

int mla_decode_with_kvcache_dual(const void* q, const void* kvcache, int64_t num_pages,
                                 const int32_t* block_table, int max_blocks,
                                 const int32_t* cache_seqlens, const int32_t* indices, int topk,
                                 const void* kvcache2, int64_t num_pages2,
                                 const int32_t* block_table2, int max_blocks2,
                                 const int32_t* cache_seqlens2, const int32_t* indices2, int topk2,
                                 int page_size, int batch, int s_q, int h_q, int h_kv, int d_qk,
                                 int dv, const int32_t* plan, const int32_t* num_splits,
                                 int num_workers, float softmax_scale, void* o, float* lse,
                                 void* workspace, size_t workspace_bytes, int phases,
                                 void* stream) {
  if (!indices || topk <= 0) return MLA_ERR_INVALID_ARGUMENT;
  const AuxCache aux{kvcache2, num_pages2, block_table2, max_blocks2, cache_seqlens2, indices2, topk2};
  return decode_impl(q, kvcache, num_pages, page_size, block_table, max_blocks, cache_seqlens,
                     batch, s_q, h_q, h_kv, d_qk, dv, plan, num_splits, num_workers, 0,
                     softmax_scale, indices, topk, o, lse, workspace, workspace_bytes, 0, &aux,
                     phases, stream);
}

int mla_debug_copy_rows(const void* q, const void* kvcache, int64_t num_pages, int kv_format,
                        const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                        const int32_t* indices, int topk, const void* kvcache2, int64_t num_pages2,
                        const int32_t* block_table2, int max_blocks2,
                        const int32_t* cache_seqlens2, const int32_t* indices2, int topk2,
                        int batch, int s_q, int h_q, int h_kv, int d_qk, int causal,
                        const int32_t* plan, const int32_t* num_splits, int num_workers, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, int64_t* rows_out,
                        int64_t rows_out_elems, void* stream) {
  if (!rows_out || (kv_format != 0 && kv_format != 1)) return MLA_ERR_INVALID_ARGUMENT;
  if (kvcache2 && (kv_format != 0 || topk <= 0)) return MLA_ERR_INVALID_ARGUMENT;
  const AuxCache aux{kvcache2, num_pages2, block_table2, max_blocks2, cache_seqlens2, indices2, topk2};
  return decode_impl(q, kvcache, num_pages, kPage, block_table, max_blocks, cache_seqlens, batch, s_q,
                     h_q, h_kv, d_qk, kDv, plan, num_splits, num_workers, causal,
                     1.f / sqrtf((float)d_qk), indices, topk, o, lse, workspace, workspace_bytes,
                     kv_format, kvcache2 ? &aux : nullptr, 1, stream, rows_out, rows_out_elems);
}

int mla_validate_inputs(const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                        int batch, int s_q, const int32_t* indices, int topk, int64_t num_pages,
                        int32_t* error_count, void* stream) {
  if (!block_table || !cache_seqlens || !error_count || max_blocks < 1 || batch < 0 || s_q < 1 ||
      num_pages < 1)
    return MLA_ERR_INVALID_ARGUMENT;
  if ((indices != nullptr) != (topk > 0)) return MLA_ERR_INVALID_ARGUMENT;
  const hipError_t e = launch_validate(block_table, max_blocks, cache_seqlens, batch, s_q, indices,
                                       topk, num_pages, error_count,
                                       reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
