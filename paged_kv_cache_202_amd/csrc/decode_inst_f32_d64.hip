// Partition-kernel instantiations for f32 caches with head dim 64.
#include "decode_kernel.h"

namespace pkv {
namespace decode {

template <>
Launcher pick_rows<PKV_F32, 64>(int G, int RP, int W) {
  constexpr int DT = PKV_F32, D = 64;
#define PKV_CASE(g, rp)                                                  \
  if (G == g && RP == rp)                                                \
    return W == 8   ? &launch_decode<DT, D, g, rp, 8>                   \
           : W == 4 ? &launch_decode<DT, D, g, rp, 4>                   \
           : W == 1 ? &launch_decode<DT, D, g, rp, 1>                   \
                    : &launch_decode<DT, D, g, rp, 0>;
  PKV_CASE(1, 1) PKV_CASE(1, 2) PKV_CASE(1, 4) PKV_CASE(1, 8)
  PKV_CASE(2, 2) PKV_CASE(2, 4) PKV_CASE(2, 8)
  PKV_CASE(4, 4) PKV_CASE(4, 8)
  PKV_CASE(8, 8)
#undef PKV_CASE
  return nullptr;
}

}  // namespace decode
}  // namespace pkv
