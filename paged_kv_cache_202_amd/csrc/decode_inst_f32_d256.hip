// Partition-kernel instantiations for f32 caches with head dim 256.
#include "decode_kernel.h"

namespace pkv {
namespace decode {

template <>
Launcher pick_rows<PKV_F32, 256>(int G, int RP, int NS, int W) {
  constexpr int DT = PKV_F32, D = 256;
#define PKV_CASE(g, rp, ns)                                              \
  if (G == g && RP == rp && NS == ns)                                    \
    return W == 8   ? &launch_decode<DT, D, g, rp, ns, 8>               \
           : W == 4 ? &launch_decode<DT, D, g, rp, ns, 4>               \
                    : &launch_decode<DT, D, g, rp, ns, 0>;
  PKV_CASE(1, 1, 1) PKV_CASE(1, 2, 1) PKV_CASE(1, 4, 1) PKV_CASE(1, 4, 2)
  PKV_CASE(2, 2, 1) PKV_CASE(2, 4, 1) PKV_CASE(2, 4, 2)
  PKV_CASE(4, 4, 1) PKV_CASE(4, 4, 2)
  PKV_CASE(8, 4, 2)
#undef PKV_CASE
  return nullptr;
}

}  // namespace decode
}  // namespace pkv
