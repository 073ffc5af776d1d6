/*
 * mla_paged_kv.h — C ABI of the MI355X (gfx950) paged MLA decode library.
 *
 * Multi-head latent attention decode over a paged, compressed-latent KV
 * cache.  Every cached token is one latent row of 576 bf16 values shared by
 * all query heads (512 latent values followed by 64 decoupled-RoPE values;
 * "Novita AI, H100 및 H200에서 FlashMLA 평가", section "MLA란 무엇인가요?").
 * K is the whole row, V is its first dv = 512 values.  Rows live in pages of
 * 64 tokens reached through a per-sequence block table, and sequences have
 * their own lengths ("What is FlashMLA", topnet.top, section "FlashMLA의 주요
 * 특성" and the installation-and-use section, steps 2 and 3).
 *
 * The library follows the two-call shape of those steps: a metadata call that
 * plans the split-KV work once per decode step (reusable by every layer while
 * the lengths do not change), and a decode call per layer returning (o, lse).
 *
 * Conventions shared by every entry point
 *  - Pointers marked "device" are device (HBM) addresses on the current HIP
 *    device; the others are host addresses.  The caller owns every buffer.  The
 *    library allocates no memory and keeps no pointer after a call returns,
 *    except that enqueued kernels use the buffers until they finish on `stream`.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work; errors inside kernels surface at the caller's next synchronisation.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns a nonzero status and enqueues nothing.  No C++ exception
 *    crosses this boundary.
 *  - Tensors are dense and row-major (C order).
 *
 * Shapes (bf16 values are passed as raw 16-bit patterns):
 *   q            [batch, s_q, h_q, d_qk]        bf16, device
 *   kvcache      [num_pages, 64, h_kv, d_qk]    bf16, device
 *   block_table  [batch, max_blocks]            int32, device; entry j of row b
 *                is the physical page of logical tokens 64*j .. 64*j + 63
 *   cache_seqlens[batch]                        int32, device; L_b >= 0
 *   indices      [batch, s_q, topk]             int32, device (sparse mode only)
 *   o            [batch, s_q, h_q, dv]          bf16, device (output)
 *   lse          [batch, s_q, h_q]              fp32, device (output)
 * Supported: d_qk = 576 or 512 (bf16 caches; packed FP8 caches hold 576
 * values), dv = 512, page size 64, any h_kv dividing h_q.  With
 * h_kv > 1 latent heads (grouped latent attention), query head h uses KV head
 * h / (h_q / h_kv); row (page * 64 + slot) of head g sits at element offset
 * ((page * 64 + slot) * h_kv + g) * d_qk of kvcache.
 */
#ifndef MLA_PAGED_KV_H_
#define MLA_PAGED_KV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARGUMENT 1   /* null pointer, bad size, inconsistent shapes */
#define MLA_ERR_UNSUPPORTED 2        /* a shape this build does not implement */
#define MLA_ERR_WORKSPACE_TOO_SMALL 3
#define MLA_ERR_HIP 4                /* a HIP runtime call or kernel launch failed */
#define MLA_ERR_SCRATCH_LIMIT 5      /* beyond the no-alloc decode's fixed scratch */

#define MLA_PAGE_SIZE 64
#define MLA_D_QK 576
#define MLA_D_V 512
#define MLA_PLAN_WORDS 8             /* int32 words per plan row */
#define MLA_PLAN_MAX_ITEMS 1048576   /* items one metadata call can plan */
#define MLA_PLAN_LDS_ITEMS 16384     /* beyond this many items, at most 4096 workers */
#define MLA_NO_ALLOC_SCRATCH_BYTES ((size_t)128 << 20)   /* per GPU, see below */

/* Human-readable text of a status code (static storage, never NULL). */
const char* mla_status_string(int status);

/*
 * mla_plan_dims — host only; sizes the metadata call's outputs.
 *
 * The work of one decode call is a list of items.  Dense mode (topk <= 0):
 * one item per (sequence, KV head), item = b * h_kv + g, of length
 * cache_seqlens[b], with num_q_rows = s_q * h_q / h_kv query rows sharing it
 * (the pages' second argument of the metadata call).  Sparse mode (topk > 0):
 * one item per (query token, KV head), item = (b * s_q + s) * h_kv + g, whose
 * keys are the topk entries of indices[b, s, :], with num_q_rows / s_q rows
 * each.
 *
 *   num_workers_request  0 = let the library choose (CU count and the decode
 *                        variant picked for this row count); > 0 forces it
 *   out_num_workers      workers W of the plan (host)
 *   out_plan_words       int32 words of the plan buffer (host): 8 * (W + 1)
 *                        words of plan rows, then items * T int32 arrival
 *                        counters of the single-launch decode, T = 1 when an
 *                        item has at most 16 rows, else ceil(rows / 64) (the
 *                        plan does not know the cache format, so it covers the
 *                        finest row tiling any decode of this shape uses)
 *   out_num_items        items of the call; num_splits holds items + 1 words (host)
 * Needs the current HIP device only when num_workers_request == 0.  The
 * metadata call plans at most MLA_PLAN_MAX_ITEMS items, and with more than
 * MLA_PLAN_LDS_ITEMS items at most 4096 workers; beyond, it returns
 * MLA_ERR_UNSUPPORTED.
 */
int mla_plan_dims(int batch, int s_q, int num_q_rows, int h_kv, int topk,
                  int num_workers_request, int* out_num_workers,
                  int* out_plan_words, int* out_num_items);

/*
 * mla_plan_dims_fp8 — mla_plan_dims for decodes over a packed FP8 cache
 * (mla_decode_with_kvcache_fp8).  The pages' metadata call takes no cache
 * format; this library's decode picks its row tiling by the format (packed
 * FP8 items of more than 16 rows run in 64-row tiles, bf16 items of more than
 * 64 rows in 128-row tiles), and the default worker count follows the tiling:
 * one workgroup per CU for every worker's row tiles.  Same arguments, outputs
 * and status codes.
 */
int mla_plan_dims_fp8(int batch, int s_q, int num_q_rows, int h_kv, int topk,
                      int num_workers_request, int* out_num_workers,
                      int* out_plan_words, int* out_num_items);

/*
 * mla_plan_num_workers — host only; the W of a plan of `plan_words` words made
 * for this call shape (inverse of mla_plan_dims), or -1 if the size does not
 * fit the shape.
 */
int mla_plan_num_workers(int plan_words, int batch, int s_q, int num_q_rows, int h_kv,
                         int topk);

/*
 * mla_get_metadata — split-KV tile scheduler ("get_mla_metadata" of the
 * pages, topnet.top installation-and-use section, step 2).
 *
 * Splits every item's 64-token blocks into contiguous runs spread over W
 * workers so that each worker gets about the same number of blocks plus a
 * fixed per-run overhead, and counts each item's runs (splits).  Integer only
 * and deterministic.
 *
 *   cache_seqlens  [batch] int32, device (read in sparse mode as well: index
 *                  entries outside [0, L_b) are padding)
 * Rule: item i has n_i blocks (dense: ceil(cache_seqlens[i / h_kv] / 64);
 * sparse: ceil(topk / 64) + ceil(topk2 / 64), topk2 being the length of the
 * auxiliary index lists of the dual-cache decode, 0 otherwise) and costs
 * overhead + n_i units (overhead = 1 block for items of at most 16 query
 * rows, 4 for 17 to 64 rows, 3 for more: the bf16 decode's row tiling;
 * mla_get_metadata_fp8 plans for the FP8 decode's), the overhead split
 * into a lead of ceil(overhead / 2) units before the item's blocks and a tail
 * of floor(overhead / 2) units after them; items are laid end to end on a cost
 * axis (total T); the first W' = min(W, T) workers share it evenly, worker w
 * owning the units [floor(w T / W'), floor((w + 1) T / W')); block b of item i
 * sits on unit (start of item i) + lead + b, and a worker gets the blocks on
 * its units.
 *
 *   topk, topk2    index-list lengths of the sparse modes (0 for dense; topk2
 *                  only with topk > 0)
 *   plan           [out_plan_words] int32, device (output).  Row 0 = {W, per-run
 *                  overhead in blocks, W', items, version 3, 64, total cost T
 *                  mod 2^32, T div 2^32} (the cost axis is 64-bit); row
 *                  1 + w = {first item, its first block, last item, end block
 *                  (exclusive) in the last item, split number of the run in
 *                  the first item, 0, 0, 0}, or
 *                  {-1, 0, -1, 0, 0, 0, 0, 0} for a worker with no blocks.
 *                  The rows are followed by the arrival counters of the
 *                  single-launch decode, which this call sets to zero.
 *   num_splits     [items + 1] int32, device (output): exclusive prefix sum
 *                  of the per-item split counts.
 * The plan stays valid for every decode call with the same lengths, batch,
 * s_q, topk, topk2 and W; items of length 0 get no split.  The decode calls
 * only read it, except the single-launch decode (phases = 4), which counts
 * finished runs in the plan's arrival counters and leaves them zero when it
 * completes: single-launch calls that share one plan must not overlap (two
 * streams), while two-launch calls may.  More than MLA_PLAN_MAX_ITEMS items,
 * or more than MLA_PLAN_LDS_ITEMS items with W > 4096: MLA_ERR_UNSUPPORTED
 * (batches past MLA_PLAN_LDS_ITEMS items, such as a sparse prefill of that
 * many query tokens, are planned by a kernel that keeps no per-item state
 * in LDS).  Any lengths up to 2^31 - 1 are planned exactly (the
 * total cost may pass 2^31; block numbers inside an item stay below 2^25).
 */
int mla_get_metadata(const int32_t* cache_seqlens, int batch, int s_q,
                     int num_q_rows, int h_kv, int topk, int topk2, int num_workers,
                     int32_t* plan, int32_t* num_splits, void* stream);

/*
 * mla_get_metadata_fp8 — mla_get_metadata for decodes over a packed FP8 cache
 * (no auxiliary lists: topk2 = 0).  The same rule with the overhead of the
 * FP8 decode's row tiling (1 block for items of at most 16 rows, else 4);
 * with W from mla_plan_dims_fp8 every row tile of every worker has a CU at
 * once.  Any plan, of either call, is valid for either decode; this one
 * balances the FP8 decode.
 */
int mla_get_metadata_fp8(const int32_t* cache_seqlens, int batch, int s_q,
                         int num_q_rows, int h_kv, int topk, int num_workers,
                         int32_t* plan, int32_t* num_splits, void* stream);

/*
 * mla_workspace_bytes — host only; bytes of the decode scratch buffer: room
 * for (items + W) partial results of R rows, each dv bf16 output values and
 * one fp32 LSE, i.e. (items + W) x R x (2 dv + 4) bytes (split runs write one
 * each; at most items + W - 1 are used).  R = rows per item, rounded up to a
 * multiple of 32 for items of more than 64 rows (their partials are written
 * in 32-row blocks).  The partial outputs are rounded to bf16 once, like the
 * final output; the merge weights them in fp32.
 */
size_t mla_workspace_bytes(int batch, int s_q, int num_q_rows, int h_kv, int topk,
                           int dv, int num_workers);

/*
 * mla_decode_with_kvcache — the decode ("flash_mla_with_kvcache" of the pages,
 * topnet.top installation-and-use section, step 3).
 *
 * For query token s of sequence b and head h, with key set J:
 *   dense, causal = 0:  J = {0 .. L_b - 1}
 *   dense, causal = 1:  J = {0 .. L_b - s_q + s}  (the s_q query tokens are the
 *                       last s_q tokens of the cache)
 *   sparse (indices):   J = {indices[b, s, t] : 0 <= indices[b, s, t] < L_b}
 *   S_j   = softmax_scale * <q[b, s, h, :], K_j>   (K_j = cache row of key j)
 *   o     = sum_j exp(S_j - m) V_j / sum_j exp(S_j - m), rounded to bf16
 *   lse   = m + ln(sum_j exp(S_j - m)) with m = max_j S_j (natural log)
 * An empty J gives o = 0 and lse = -inf.  Cache rows outside J (slots past L_b
 * in a sequence's last page, pages not in the first ceil(L_b / 64) block-table
 * entries) are never read.
 *
 *   num_pages       pages in kvcache (used to check the plan's bounds only on
 *                   the validation call; not read by the kernels)
 *   page_size       must be 64
 *   d_qk, dv        d_qk = 576 (512 latent + 64 RoPE values per row; V = the
 *                   first 512) or 512 (the d_qk = 512 rows named by "FlashInfer,
 *                   SM120 GPU를 위한 희소 MLA 커널", 들어가며; V = the whole row);
 *                   dv = 512
 *   max_blocks      columns of block_table
 *   plan, num_splits, num_workers   from mla_get_metadata with the same
 *                   lengths / batch / s_q / topk and num_q_rows = s_q*h_q/h_kv
 *   causal          0 or 1 (must be 0 in sparse mode)
 *   softmax_scale   > 0 (the Python binding defaults to d_qk^-0.5)
 *   indices, topk   NULL and 0 for dense mode
 *   workspace       device scratch of at least mla_workspace_bytes(...) bytes
 * With batch = 0 the call does nothing and returns MLA_OK; q, block_table,
 * cache_seqlens, indices, o and lse may then be NULL (zero-length arrays).
 */
int mla_decode_with_kvcache(const void* q, const void* kvcache, int64_t num_pages,
                            int page_size, const int32_t* block_table, int max_blocks,
                            const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                            int h_kv, int d_qk, int dv, const int32_t* plan,
                            const int32_t* num_splits, int num_workers, int causal,
                            float softmax_scale, const int32_t* indices, int topk,
                            void* o, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * mla_decode_with_kvcache_no_alloc — mla_decode_with_kvcache for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It takes no workspace: the split
 * partials go to a buffer of MLA_NO_ALLOC_SCRATCH_BYTES (128 MiB) that the
 * library holds in a file-scope device array, one copy on every GPU it runs
 * on, kept until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); the first call that launches work on
 * a device looks up that device's copy (hipGetSymbolAddress), so a caller that
 * captures graphs makes one such call first.  A call whose partials
 * (mla_workspace_bytes of the same arguments) exceed the buffer returns
 * MLA_ERR_SCRATCH_LIMIT and launches nothing; fewer workers in the plan need
 * less.  Nothing in the buffer has to start at zero: every partial the merge
 * reads is written by the split kernel of the same call, so the contents left
 * by an earlier call never reach a result.  All calls on one GPU share its
 * buffer: no-alloc calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  bf16 caches, dense or
 * sparse; every other argument, check and status is that of
 * mla_decode_with_kvcache (two launches).
 */
int mla_decode_with_kvcache_no_alloc(const void* q, const void* kvcache, int64_t num_pages,
                                     int page_size, const int32_t* block_table, int max_blocks,
                                     const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                     int h_kv, int d_qk, int dv, const int32_t* plan,
                                     const int32_t* num_splits, int num_workers, int causal,
                                     float softmax_scale, const int32_t* indices, int topk,
                                     void* o, float* lse, void* stream);

/*
 * mla_decode_with_kvcache_phase — the same decode in two separately launched
 * phases, for callers that time or overlap them: phases = 1 runs the split
 * kernel only (items covered by one worker get their final o / lse, the others
 * get partials in `workspace`); phases = 2 runs the merge of the partials
 * only (it must follow phase 1 on the same stream with the same arguments);
 * phases = 3 runs both and is mla_decode_with_kvcache.  phases = 4 is the
 * single-launch decode (a fixed launch overhead matters: "Blackwell을 위한
 * 새로운 MLA 백엔드: TOKENSPEED_MLA 분석", section "왜 이게 좋은 최적화인가?",
 * item 3): one kernel, in
 * which the last run of each split item to finish merges the item's partials
 * and items without a key are written as well.  Its runs exchange partials
 * through `workspace` at agent scope and count arrivals in the plan's arrival
 * counters (after its rows; zeroed by mla_get_metadata, left zero by every
 * completed call): single-launch calls that share a plan or a workspace must
 * not overlap.  Any other value returns MLA_ERR_INVALID_ARGUMENT.  Same
 * arguments, checks and ownership rules as mla_decode_with_kvcache.
 */
int mla_decode_with_kvcache_phase(const void* q, const void* kvcache, int64_t num_pages,
                                  int page_size, const int32_t* block_table, int max_blocks,
                                  const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                  int h_kv, int d_qk, int dv, const int32_t* plan,
                                  const int32_t* num_splits, int num_workers, int causal,
                                  float softmax_scale, const int32_t* indices, int topk,
                                  void* o, float* lse, void* workspace,
                                  size_t workspace_bytes, int phases, void* stream);

/*
 * mla_decode_with_kvcache_fp8 / mla_decode_with_kvcache_fp8_phase — the same
 * decode over a packed FP8 cache (a packed KV cache with a per-block scale
 * format: "FlashInfer, SM120 GPU를 위한 희소 MLA 커널", section "코드 분석",
 * item 5; FP8 KV caches: "Blackwell을 위한 새로운 MLA 백엔드: TOKENSPEED_MLA
 * 분석").  The pages fix no layout; this library's is:
 *
 *   kvcache  [num_pages, 64, h_kv, 656] bytes, device.  Row bytes 0..511: the
 *            512 latent values as OCP E4M3 codes; bytes 512..527: four
 *            little-endian float32 scales, scale j multiplying latent values
 *            128 j .. 128 j + 127; bytes 528..655: the 64 RoPE values as bf16.
 *
 * K_j is the row's 576 values (latent code x its block's scale, then RoPE),
 * V_j its first 512; d_qk must be 576 (the number of values, not bytes).  In
 * the kernels the codes enter the bf16 matrix products as they are (every
 * E4M3 value is a bf16 value) and the scales never do: Q K^T is accumulated
 * per 128-value block and each block's sum is multiplied by the key's scale
 * in fp32, and in P V each key's probability is multiplied by its scale for
 * the output columns' block before P is rounded to bf16.  Every other
 * argument, check, status and the phases argument are those of
 * mla_decode_with_kvcache(_phase), with the same plan.
 */
int mla_decode_with_kvcache_fp8(const void* q, const void* kvcache, int64_t num_pages,
                                int page_size, const int32_t* block_table, int max_blocks,
                                const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                int h_kv, int d_qk, int dv, const int32_t* plan,
                                const int32_t* num_splits, int num_workers, int causal,
                                float softmax_scale, const int32_t* indices, int topk,
                                void* o, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);
int mla_decode_with_kvcache_fp8_phase(const void* q, const void* kvcache, int64_t num_pages,
                                      int page_size, const int32_t* block_table, int max_blocks,
                                      const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                      int h_kv, int d_qk, int dv, const int32_t* plan,
                                      const int32_t* num_splits, int num_workers, int causal,
                                      float softmax_scale, const int32_t* indices, int topk,
                                      void* o, float* lse, void* workspace,
                                      size_t workspace_bytes, int phases, void* stream);

/*
 * mla_decode_with_kvcache_dual — sparse decode over two caches at once (the
 * dual-cache scenario, a main and an auxiliary cache used together:
 * "FlashInfer, SM120 GPU를 위한 희소 MLA 커널", section "코드 분석", item 1).
 * Query token (b, s) attends to the union of its main-list keys
 * (indices[b, s, :topk] into the main cache, valid below cache_seqlens[b])
 * and its auxiliary-list keys (indices2[b, s, :topk2] into the auxiliary
 * cache, valid below cache_seqlens2[b]), with one softmax over both; entries
 * outside [0, L) of their list are padding.  Both caches are bf16 [pages, 64,
 * h_kv, d_qk] with their own block tables; d_qk is 576 or 512 (the same rows
 * as mla_decode_with_kvcache).  The plan comes from mla_get_metadata with the
 * same topk and topk2: every item has ceil(topk / 64) + ceil(topk2 / 64)
 * tiles of 64 keys, the main list's first.  topk2 may be 0 (indices2 NULL).
 * causal is not an argument (sparse mode); the other arguments, checks and
 * phases are those of mla_decode_with_kvcache_phase.
 */
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
                                 void* stream);

/*
 * mla_debug_copy_rows — indexing probe (test use).  Runs the split decode
 * kernel (phase 1 of the decode: every argument as for the decode entry point
 * of the same cache format; kv_format 0 = bf16 rows, 1 = packed FP8 rows;
 * kvcache2 != NULL selects the dual-cache decode, bf16 and sparse only,
 * with its auxiliary arguments as for mla_decode_with_kvcache_dual, else they
 * are ignored), and has the kernel also write, for every cache row one of its
 * tile copies reads, the byte offset of that row from kvcache, taken from the
 * very registers the copy instructions use.  The tiles and rows of 64-token
 * pages follow "What is FlashMLA" (topnet.top), section "FlashMLA의 주요 특성",
 * and the block table the installation-and-use section, step 3.
 *
 *   rows_out       int64, device: [items, T, 64] with T = max_blocks (dense)
 *                  or ceil(topk / 64) + ceil(topk2 / 64) (sparse); entry
 *                  (i, t, r) is the offset read for row r of tile t of item i
 *                  (auxiliary-cache rows as offsets from kvcache too).  FP8
 *                  adds a second plane [items, T, 64] after the first: the
 *                  row whose float32 scales the copy reads.  Entries of tiles
 *                  no run copies are not written (the caller fills them).
 *   rows_out_elems capacity of rows_out in int64 values; too small:
 *                  MLA_ERR_INVALID_ARGUMENT.
 * The softmax scale is d_qk^-0.5; o, lse and workspace receive what phase 1
 * of the decode writes.
 */
int mla_debug_copy_rows(const void* q, const void* kvcache, int64_t num_pages, int kv_format,
                        const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                        const int32_t* indices, int topk, const void* kvcache2, int64_t num_pages2,
                        const int32_t* block_table2, int max_blocks2,
                        const int32_t* cache_seqlens2, const int32_t* indices2, int topk2,
                        int batch, int s_q, int h_q, int h_kv, int d_qk, int causal,
                        const int32_t* plan, const int32_t* num_splits, int num_workers, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, int64_t* rows_out,
                        int64_t rows_out_elems, void* stream);

/*
 * mla_validate_inputs — opt-in device-side check of the index data the host
 * cannot see: every block-table entry a key can reach lies in [0, num_pages),
 * L_b <= max_blocks * 64 and L_b >= 0.  Writes the number of violations to
 * *error_count (one int32, device; zeroed by this call) on `stream`.
 */
int mla_validate_inputs(const int32_t* block_table, int max_blocks,
                        const int32_t* cache_seqlens, int batch, int s_q,
                        const int32_t* indices, int topk, int64_t num_pages,
                        int32_t* error_count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_KV_H_ */
