// Input validation kernels: every block-table entry a key can reach must name
// a page of the pool ("What is FlashMLA", topnet.top: 64-token pages reached
// through block_table), and every length must fit the block table.
#include "mla_common.h"

namespace mla {
namespace {

__global__ void zero_i32(int32_t* p) { if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = 0; }

__global__ void validate_dense(const int32_t* __restrict__ bt, int max_blocks,
                               const int32_t* __restrict__ seqlens, int batch, int64_t num_pages,
                               int32_t* err) {
  const int64_t n = (int64_t)batch * max_blocks;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(e / max_blocks);
    const int j = (int)(e % max_blocks);
    const int L = seqlens[b];
    int bad = 0;
    if (j == 0 && (L < 0 || (int64_t)L > (int64_t)max_blocks * kPage)) bad = 1;
    if ((int64_t)j * kPage < (int64_t)L) {
      const int p = bt[e];
      if (p < 0 || p >= num_pages) bad = 1;
    }
    if (bad) atomicAdd(err, 1);
  }
}

__global__ void validate_sparse(const int32_t* __restrict__ bt, int max_blocks,
                                const int32_t* __restrict__ seqlens, int batch, int s_q,
                                const int32_t* __restrict__ indices, int topk, int64_t num_pages,
                                int32_t* err) {
  const int64_t n = (int64_t)batch * s_q * topk;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(e / ((int64_t)s_q * topk));
    const int L = seqlens[b];
    int bad = 0;
    if (e % ((int64_t)s_q * topk) == 0 && (L < 0 || (int64_t)L > (int64_t)max_blocks * kPage)) bad = 1;
    const int idx = indices[e];
    if (!bad && sparse_key_valid(idx, L)) {
      const int p = bt[(int64_t)b * max_blocks + (idx >> 6)];
      if (p < 0 || p >= num_pages) bad = 1;
    }
    if (bad) atomicAdd(err, 1);
  }
}

int grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

}  // namespace

hipError_t launch_validate(const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                           int batch, int s_q, const int32_t* indices, int topk,
                           int64_t num_pages, int32_t* error_count, hipStream_t stream) {
  hipLaunchKernelGGL(zero_i32, dim3(1), dim3(64), 0, stream, error_count);
  if (indices == nullptr) {
    const int64_t n = (int64_t)batch * max_blocks;
    hipLaunchKernelGGL(validate_dense, dim3(grid_for(n)), dim3(256), 0, stream, block_table,
                       max_blocks, seqlens, batch, num_pages, error_count);
  } else {
    const int64_t n = (int64_t)batch * s_q * topk;
    hipLaunchKernelGGL(validate_sparse, dim3(grid_for(n)), dim3(256), 0, stream, block_table,
                       max_blocks, seqlens, batch, s_q, indices, topk, num_pages, error_count);
  }
  return hipGetLastError();
}

}  // namespace mla
