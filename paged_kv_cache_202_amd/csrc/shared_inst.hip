// Instantiations of the shared-prefix kernel (bf16 caches).
#include "shared_prefix.h"

namespace pkv {
namespace decode {

template <int D, int W, int RT>
void launch_prefix(const DecodeArgs &a, const ShareArgs &s, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((prefix_mfma_kernel<D, W, RT>), grid, dim3(W * 64), 0, st, a, s);
}

template <int D>
PrefixLauncher pick_for_dim(int W, int RT) {
  if (RT == 2) {
    // two row tiles hold twice the accumulators: built where they fit in registers
    if constexpr (D <= 128) return W == 8 ? &launch_prefix<D, 8, 2> : nullptr;
    return nullptr;
  }
  if (RT != 1) return nullptr;
  return W == 8 ? &launch_prefix<D, 8, 1>
       : W == 4 ? &launch_prefix<D, 4, 1>
       : W == 2 ? &launch_prefix<D, 2, 1>
       : W == 1 ? &launch_prefix<D, 1, 1>
                : nullptr;
}

PrefixLauncher pick_prefix(int D, int W, int RT) {
  return D == 64    ? pick_for_dim<64>(W, RT)
         : D == 128 ? pick_for_dim<128>(W, RT)
         : D == 256 ? pick_for_dim<256>(W, RT)
                    : nullptr;
}

}  // namespace decode
}  // namespace pkv
