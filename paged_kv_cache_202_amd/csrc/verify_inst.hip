// MFMA multi-query (verify) kernel instantiations: bf16 caches, head dims
// 64, 128 and 256, four wavefronts per workgroup.
#include "verify_mfma.h"

namespace pkv {
namespace decode {

template <int D>
static void launch_verify(const DecodeArgs &a, const StreamArgs &, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((verify_mfma_kernel<D, kVerifyWaves>), grid, dim3(kVerifyWaves * 64), 0, s,
                     a);
}

Launcher pick_verify(int D) {
  if (D == 64) return &launch_verify<64>;
  if (D == 128) return &launch_verify<128>;
  if (D == 256) return &launch_verify<256>;
  return nullptr;
}

}  // namespace decode
}  // namespace pkv
