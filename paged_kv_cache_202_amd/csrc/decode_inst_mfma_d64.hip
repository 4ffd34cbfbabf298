// Instantiations of the MFMA decode kernel over bf16 caches and caches of 8-bit codes
// with head dim 64: 4, 8 or 16 query rows per wavefront, 1, 4 or 8
// wavefronts per workgroup.
#include "decode_mfma.h"

namespace pkv {
namespace decode {

template <>
Launcher pick_mfma<64>(int DT, int RW, int W) {
#define PKV_CASE(dt, rw)                                  \
  if (DT == dt && RW == rw)                               \
    return W == 8   ? &launch_mfma<dt, 64, rw, 8>        \
           : W == 4 ? &launch_mfma<dt, 64, rw, 4>        \
           : W == 1 ? &launch_mfma<dt, 64, rw, 1>        \
                    : nullptr;
  PKV_CASE(PKV_BF16, 4) PKV_CASE(PKV_BF16, 8) PKV_CASE(PKV_BF16, 16)
  PKV_CASE(PKV_I8, 4) PKV_CASE(PKV_I8, 8) PKV_CASE(PKV_I8, 16)
#undef PKV_CASE
  return nullptr;
}

template <>
Launcher pick_mfma_stream<64>(int DT, int RW) {
  if (DT == PKV_BF16)
    return RW == 4    ? &launch_mfma_stream<PKV_BF16, 64, 4>
           : RW == 8  ? &launch_mfma_stream<PKV_BF16, 64, 8>
           : RW == 16 ? &launch_mfma_stream<PKV_BF16, 64, 16>
                      : nullptr;
  if (DT == PKV_I8)
    return RW == 4    ? &launch_mfma_stream<PKV_I8, 64, 4>
           : RW == 8  ? &launch_mfma_stream<PKV_I8, 64, 8>
           : RW == 16 ? &launch_mfma_stream<PKV_I8, 64, 16>
                      : nullptr;
  return nullptr;
}

}  // namespace decode
}  // namespace pkv
