// Split decode launches for the 16- and 64-row variants, and the merge of
// split items.  The kernels are in mla_decode_kernel.h; the 128-row variant is
// built in mla_decode_rows128.hip (see the build flags there).
#include "mla_decode_kernel.h"

namespace mla {
hipError_t launch_rows128(const DecodeArgs& a, hipStream_t stream);
namespace {

// Merge of the partial results of items split over several workers, and the
// empty result of items with no key (the unfused path).  One wave per row.
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int item = blockIdx.x;
  const int slot0 = a.num_splits[item];
  const int n = a.num_splits[item + 1] - slot0;
  if (n == 1) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = blockIdx.y * 4 + wave; r < a.M; r += 4 * gridDim.y) {
    if (n == 0) write_empty_row(a, item, r, lane);
    else merge_row<false>(a, item, slot0, n, r, lane);
  }
}

// Merge of items split over several workers whose partial outputs are 32-row
// blocks in accumulator order (the 128-row variant, two launches): one
// workgroup per (item, block, quarter of the 512 columns), its 4096 values of
// each partial read contiguously (16 bytes per thread and partial), each
// value weighted by its row's log-sum-exp weight, and the result written out
// through LDS as 256-byte row segments.  The arithmetic per value is
// merge_row's (the same weights, summed in the same order), so both merges
// give the same bits.
constexpr int kBlockQuarters = 4;

// Weighted sum of the block partials k of one thread's two chunks (values
// 8 c .. 8 c + 7 of chunk c = v[i]; the first four belong to block row ja, the
// last four to jb), partial weights from s_w[k].
__device__ __forceinline__ void add_block_partial(const uint4 (&v)[2], float wa, float wb, float (&acc)[2][8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const unsigned w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    // a bf16 value is the upper half of the float it denotes
    acc[i][0] += wa * __uint_as_float(w4[0] << 16);
    acc[i][1] += wa * __uint_as_float(w4[0] & 0xffff0000u);
    acc[i][2] += wa * __uint_as_float(w4[1] << 16);
    acc[i][3] += wa * __uint_as_float(w4[1] & 0xffff0000u);
    acc[i][4] += wb * __uint_as_float(w4[2] << 16);
    acc[i][5] += wb * __uint_as_float(w4[2] & 0xffff0000u);
    acc[i][6] += wb * __uint_as_float(w4[3] << 16);
    acc[i][7] += wb * __uint_as_float(w4[3] & 0xffff0000u);
  }
}

// Items of at most N <= 8 splits: every read of the block goes out at once
// (the N partials' chunks, the last partial standing in for those past n, and
// thread (j, p)'s LSE of partial p of row j), so the merge waits for memory
// once instead of three times (LSEs for the maxima, LSEs for the weights,
// then the partials).  Same weights and order of sums as the general loop.
template <int N>
__device__ __forceinline__ void merge_block_batch(const DecodeArgs& a, const float* lse0,
                                                  const uint16_t* blk0, int64_t stride, int n,
                                                  int tid, int ja, int jb, float* s_mx,
                                                  float (*s_w)[32], float (&acc)[2][8],
                                                  float& tot) {
  uint4 v[N][2];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int kk = k < n ? k : n - 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) v[k][i] = *reinterpret_cast<const uint4*>(blk0 + kk * stride + 2048 * i);
  }
  const int j = tid >> 3, p = tid & 7;
  const float lk = lse0[(int64_t)(p < n ? p : n - 1) * a.part_rows + j];
  float mx = p < n ? lk : -INFINITY;
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
  if (p == 0) s_mx[j] = mx;
  if (p < n) s_w[p][j] = (mx == -INFINITY || lk == -INFINITY) ? 0.f : expf(lk - mx);
  __syncthreads();
  if (tid < 32)
    for (int k = 0; k < n; ++k) tot += s_w[k][tid];
#pragma unroll
  for (int k = 0; k < N; ++k)
    if (k < n) add_block_partial(v[k], s_w[k][ja], s_w[k][jb], acc);
}

__global__ __launch_bounds__(256) void combine_blocks_kernel(DecodeArgs a) {
  const int item = blockIdx.x;
  const int r0 = 32 * (blockIdx.y / kBlockQuarters);   // first row of the block inside the item
  const int cq = blockIdx.y % kBlockQuarters;           // column quarter: columns 128 cq .. 128 cq + 127
  const int slot0 = a.num_splits[item];
  const int n = a.num_splits[item + 1] - slot0;
  if (n == 1 || r0 >= a.M) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rend = min(r0 + 32, a.M);
  if (n == 0) {
    if (cq == 0)
      for (int r = r0 + wave; r < rend; r += 4) write_empty_row(a, item, r, lane);
    return;
  }
  constexpr int kRowPad = 136;   // bf16 values per staged row segment (272 bytes: rows fall on distinct banks)
  __shared__ float s_mx[32];
  __shared__ float s_inv[32];
  __shared__ float s_w[32][32];   // weights of partials k0 .. k0 + 31 of the block's rows
  __shared__ __attribute__((aligned(16))) uint16_t s_out[32 * kRowPad];
  const float* lse0 = a.part_lse + (int64_t)slot0 * a.part_rows + r0;
  // This thread's two chunks of 8 values: chunk c = 512 cq + tid + 256 i of
  // the block covers values 8 c .. 8 c + 7, the pieces of writing lanes
  // 2 c mod 64 and 2 c mod 64 + 1 (rows (2 c) mod 32 and (2 c + 1) mod 32 of
  // the block) in piece c / 32 = 4 d + q4 (column quarter d / 4).
  float acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  float tot = 0.f;   // threads 0..31: the weight sum of row tid
  const int ja = (2 * tid) & 31, jb = (2 * tid + 1) & 31;   // the same for both chunks
  const uint16_t* blk0 = a.part_o + ((int64_t)slot0 * a.part_rows + r0) * kDv + 8 * (512 * cq + tid);
  const int64_t stride = (int64_t)a.part_rows * kDv;
  if (n <= 2) {
    merge_block_batch<2>(a, lse0, blk0, stride, n, tid, ja, jb, s_mx, s_w, acc, tot);
  } else if (n <= 4) {
    merge_block_batch<4>(a, lse0, blk0, stride, n, tid, ja, jb, s_mx, s_w, acc, tot);
  } else if (n <= 8) {
    merge_block_batch<8>(a, lse0, blk0, stride, n, tid, ja, jb, s_mx, s_w, acc, tot);
  } else {
    // row maxima: 8 threads per row, each over every 8th partial
    {
      const int j = tid >> 3, p = tid & 7;
      float mx = -INFINITY;
      for (int k = p; k < n; k += 8) mx = fmaxf(mx, lse0[(int64_t)k * a.part_rows + j]);
#pragma unroll
      for (int d = 1; d < 8; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
      if (p == 0) s_mx[j] = mx;
    }
    for (int k0 = 0; k0 < n; k0 += 32) {
      const int kn = min(32, n - k0);
      __syncthreads();   // s_mx is written; the previous weights are used
      for (int e = tid; e < 32 * kn; e += 256) {
        const int k = e >> 5, j = e & 31;
        const float lk = lse0[(int64_t)(k0 + k) * a.part_rows + j];
        s_w[k][j] = (s_mx[j] == -INFINITY || lk == -INFINITY) ? 0.f : expf(lk - s_mx[j]);
      }
      __syncthreads();
      if (tid < 32)
        for (int k = 0; k < kn; ++k) tot += s_w[k][tid];
#pragma unroll 4
      for (int k = 0; k < kn; ++k) {
        const uint16_t* src = blk0 + (int64_t)(k0 + k) * stride;
        uint4 v[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) v[i] = *reinterpret_cast<const uint4*>(src + 2048 * i);
        add_block_partial(v, s_w[k][ja], s_w[k][jb], acc);
      }
    }
  }
  if (tid < 32) {
    s_inv[tid] = tot > 0.f ? 1.f / tot : 0.f;
    const int r = r0 + tid;
    if (cq == 0 && r < rend) a.lse[q_row(a, item, r)] = tot > 0.f ? s_mx[tid] + logf(tot) : -INFINITY;
  }
  __syncthreads();
  // normalised values into row order: value e of the piece of writing lane l
  // in piece (d, q4) is column 32 d + 8 q4 + 4 (l / 32) + e of row l mod 32
  // (staged relative to the quarter's first column)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = 512 * cq + tid + 256 * i;
    const int pc = c >> 5;                          // 4 d + q4
    const int la = (2 * c) & 63, lb = la + 1;
    const int cb = 32 * (pc >> 2) + 8 * (pc & 3) - 128 * cq;
    bf16x4 xa, xb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xa[e] = (__bf16)(acc[i][e] * s_inv[ja]);
      xb[e] = (__bf16)(acc[i][4 + e] * s_inv[jb]);
    }
    *reinterpret_cast<bf16x4*>(s_out + ja * kRowPad + cb + 4 * (la >> 5)) = xa;
    *reinterpret_cast<bf16x4*>(s_out + jb * kRowPad + cb + 4 * (lb >> 5)) = xb;
  }
  __syncthreads();
  // row segments out: 16 threads per row, 16 bytes each
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i, j = q >> 4, c16 = q & 15;
    const int r = r0 + j;
    if (r < rend)
      *reinterpret_cast<uint4*>(a.o + q_row(a, item, r) * kDv + 128 * cq + 8 * c16) =
          *reinterpret_cast<const uint4*>(s_out + j * kRowPad + 8 * c16);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int variant, hipStream_t stream) {
  if (variant == kVariantRows128) return launch_rows128(a, stream);
  const bool r16 = variant == kVariantRows16;
  if (a.kv_format == 1)
    return r16 ? launch_variant<kVariantRows16, true, 576>(a, stream)
               : launch_variant<kVariantRows64, true, 576>(a, stream);
  if (a.d_qk == 512)
    return r16 ? launch_variant<kVariantRows16, false, 512>(a, stream)
               : launch_variant<kVariantRows64, false, 512>(a, stream);
  return r16 ? launch_variant<kVariantRows16, false, 576>(a, stream)
             : launch_variant<kVariantRows64, false, 576>(a, stream);
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_items == 0) return hipSuccess;
  if (a.part_blocks) {
    hipLaunchKernelGGL(combine_blocks_kernel, dim3(a.num_items, (a.M + 31) / 32 * kBlockQuarters), dim3(256), 0,
                       stream, a);
  } else {
    const int gy = min((a.M + 3) / 4, 32);
    hipLaunchKernelGGL(combine_kernel, dim3(a.num_items, gy), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
