// Split decode launches for the 128-row variant (items of more than 64 query
// rows over bf16 caches).  Each wave holds its 32 rows' output accumulators,
// 32 x 512 fp32 values, in the 256 accumulation registers (AGPRs), and its
// query rows, scores and operands in the 256 vector registers; this file is
// therefore built with the MFMAs in their AGPR-accumulator form (the other
// decode variants are built with VGPR accumulators).
#include "mla_decode_kernel.h"

namespace mla {

hipError_t launch_rows128(const DecodeArgs& a, hipStream_t stream) {
  return a.d_qk == 512 ? launch_variant<kVariantRows128, false, 512>(a, stream)
                       : launch_variant<kVariantRows128, false, 576>(a, stream);
}

}  // namespace mla
