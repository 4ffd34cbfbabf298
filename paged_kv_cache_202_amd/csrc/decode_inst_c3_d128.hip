// Partition-kernel instantiations for caches of 3-bit codes (two per byte,
// per-row float32 scales) with head dim 128; bf16 queries.
#include "decode_kernel.h"

namespace pkv {
namespace decode {

template <>
Launcher pick_rows<kCodes3, 128>(int G, int RP, int W) {
  constexpr int DT = kCodes3, D = 128;
#define PKV_CASE(g, rp)                                                  \
  if (G == g && RP == rp)                                                \
    return W == 8   ? &launch_decode<DT, D, g, rp, 8>                   \
           : W == 4 ? &launch_decode<DT, D, g, rp, 4>                   \
           : W == 1 ? &launch_decode<DT, D, g, rp, 1>                   \
                    : nullptr;
  // at most 4 rows per wavefront: 16 fp32 accumulators per row and lane
  PKV_CASE(1, 1) PKV_CASE(1, 2) PKV_CASE(1, 4)
  PKV_CASE(2, 2) PKV_CASE(2, 4)
  PKV_CASE(4, 4)
  PKV_CASE(8, 4)
#undef PKV_CASE
  return nullptr;
}

}  // namespace decode
}  // namespace pkv
