// Instantiations of the MFMA row-tile kernels (bf16 caches): the shared-prefix
// kernel and the chunked-prefill kernel.
#include "group_decode.h"
#include "shared_prefix.h"

namespace pkv {
namespace decode {

template <int D, int W, int RT, bool CHUNK>
void launch_rows(const DecodeArgs &a, const ShareArgs &s, dim3 grid, hipStream_t st) {
  if constexpr (CHUNK)
    hipLaunchKernelGGL((chunk_mfma_kernel<D, W, RT>), grid, dim3(W * 64), 0, st, a, s);
  else
    hipLaunchKernelGGL((prefix_mfma_kernel<D, W, RT>), grid, dim3(W * 64), 0, st, a, s);
}

template <int D, bool CHUNK>
PrefixLauncher pick_for_dim(int W, int RT) {
  if (RT == 2) {
    // two row tiles hold twice the accumulators: built where they fit in registers
    if constexpr (D <= 128) return W == 8 ? &launch_rows<D, 8, 2, CHUNK> : nullptr;
    return nullptr;
  }
  if (RT != 1) return nullptr;
  return W == 8 ? &launch_rows<D, 8, 1, CHUNK>
       : W == 4 ? &launch_rows<D, 4, 1, CHUNK>
       : W == 2 ? &launch_rows<D, 2, 1, CHUNK>
       : W == 1 ? &launch_rows<D, 1, 1, CHUNK>
                : nullptr;
}

template <bool CHUNK>
PrefixLauncher pick_rows_kernel(int D, int W, int RT) {
  return D == 64    ? pick_for_dim<64, CHUNK>(W, RT)
         : D == 128 ? pick_for_dim<128, CHUNK>(W, RT)
         : D == 256 ? pick_for_dim<256, CHUNK>(W, RT)
                    : nullptr;
}

PrefixLauncher pick_prefix(int D, int W, int RT, bool chunk) {
  return chunk ? pick_rows_kernel<true>(D, W, RT) : pick_rows_kernel<false>(D, W, RT);
}

template <int D, int RT>
void launch_group(const DecodeArgs &a, const ShareArgs &s, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((group_mfma_kernel<D, RT>), grid, dim3(512), 0, st, a, s);
}

GroupLauncher pick_group(int D, int RT) {
  if (D == 64) return RT == 2 ? &launch_group<64, 2> : RT == 1 ? &launch_group<64, 1> : nullptr;
  if (D == 128) return RT == 2 ? &launch_group<128, 2> : RT == 1 ? &launch_group<128, 1> : nullptr;
  return nullptr;
}

}  // namespace decode
}  // namespace pkv
