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
  const int gy = min((a.M + 3) / 4, 32);
  hipLaunchKernelGGL(combine_kernel, dim3(a.num_items, gy), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
