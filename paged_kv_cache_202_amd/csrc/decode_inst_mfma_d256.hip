// Instantiations of the MFMA decode kernel over caches of 8-bit and 3-bit codes
// with head dim 256: 4, 8 or 16 query rows per wavefront, 1, 4 or 8
// wavefronts per workgroup.
#include "decode_mfma.h"

namespace pkv {
namespace decode {

template <>
Launcher pick_mfma<256>(int DT, int RW, int W) {
#define PKV_CASE(dt, rw)                                  \
  if (DT == dt && RW == rw)                               \
    return W == 8   ? &launch_mfma<dt, 256, rw, 8>        \
           : W == 4 ? &launch_mfma<dt, 256, rw, 4>        \
           : W == 1 ? &launch_mfma<dt, 256, rw, 1>        \
                    : nullptr;
  PKV_CASE(PKV_I8, 4) PKV_CASE(PKV_I8, 8) PKV_CASE(PKV_I8, 16)
  PKV_CASE(kCodes3, 4) PKV_CASE(kCodes3, 8) PKV_CASE(kCodes3, 16)
#undef PKV_CASE
  return nullptr;
}

template <>
Launcher pick_mfma_stream<256>(int, int) {
  return nullptr;  // the stream mode covers head dims up to 128
}

}  // namespace decode
}  // namespace pkv
