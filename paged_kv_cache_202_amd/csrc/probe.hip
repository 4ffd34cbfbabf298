// Measurement aid, not part of the attention path: the rate at which a
// gfx950 workgroup of eight wavefronts streams scattered 4 KiB chunks of
// HBM, read the way the decode kernels read K/V (16-byte loads per lane,
// 1 KiB per instruction; in LDS mode the same non-temporal direct-to-LDS
// gathers into per-wavefront rings of 4, 8 or 16 KiB, read back by each
// lane). With chunks in
// table order it measures a sequential stream; with a random order, the
// access pattern of a paged cache whose blocks were handed out from a
// shuffled free list. Each workgroup XORs every word it read into one
// value, so that the reads are used and the caller can check them.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_kernel.h"
#include "pagedkv.h"
#include "status.h"

namespace {

using pkv::decode::gather_lds16;
using pkv::decode::kKvNonTemporal;
using pkv::decode::u32x4_t;
using pkv::decode::wait_vmcnt;
using pkv::fail;

constexpr int kProbeWaves = 8;

// Wavefront w of workgroup x reads chunks k = x W + w + j (W grid.x): chunk
// k at byte order[k] * LOADS KiB, LOADS 16-byte loads a lane. Register modes
// (0, 1) load a chunk and fold it in, and rely on resident wavefronts for
// loads in flight (no LDS: up to four workgroups a CU); LDS mode (2) keeps
// RING bytes a wavefront in flight in a ring of RING / (LOADS KiB) chunks.
template <int MODE, int LOADS, int RING>
__global__ void __launch_bounds__(kProbeWaves * 64)
read_probe_kernel(const char *__restrict__ buf, const int32_t *__restrict__ order, int32_t n,
                  uint32_t n_buf_chunks, uint32_t *__restrict__ sink) {
  constexpr int kChunk = LOADS * 1024;
  constexpr int kSlots = RING / kChunk;
  static_assert(kSlots >= 1, "a ring holds at least one chunk");
  __shared__ u32x4_t ring[MODE == 2 ? kProbeWaves * RING / 16 : 1];
  __shared__ uint32_t red[kProbeWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stride = gridDim.x * kProbeWaves;
  const int first = blockIdx.x * kProbeWaves + wave;
  // a chunk index past the buffer reads its last chunk instead
  auto chunk_ptr = [&](int k) {
    return buf + (size_t)min((uint32_t)order[k], n_buf_chunks - 1) * kChunk + lane * 16;
  };
  uint32_t x = 0;
  if constexpr (MODE == 2) {
    PKV_LDS char *mine = (PKV_LDS char *)&ring[0] + wave * RING;
    auto stage = [&](int k, int slot) {
      const char *src = chunk_ptr(k);
      PKV_LDS char *dst = mine + slot * kChunk;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) gather_lds16<kKvNonTemporal>(src + i * 1024, dst + i * 1024);
    };
    const int mine_n = first < n ? (n - first + stride - 1) / stride : 0;
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
      if (j < mine_n) stage(first + j * stride, j);
    for (int j = 0; j < mine_n; ++j) {
      const int ahead = min(mine_n - 1 - j, kSlots - 1);  // chunks staged after j
      pkv::decode::static_for<kSlots>([&](auto ac) {
        constexpr int A = decltype(ac)::value;
        if (ahead == A) wait_vmcnt<A * LOADS>();
      });
      const PKV_LDS char *p = mine + (j % kSlots) * kChunk + lane * 16;
      u32x4_t v[LOADS];
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v[i]) : "v"(p + i * 1024)
                     : "memory");
      if (j + kSlots < mine_n) stage(first + (j + kSlots) * stride, j % kSlots);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
  } else {
    for (int k = first; k < n; k += stride) {
      const u32x4_t *src = (const u32x4_t *)chunk_ptr(k);
      u32x4_t v[LOADS];
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        v[i] = MODE == 1 ? __builtin_nontemporal_load(src + i * 64) : src[i * 64];
#pragma unroll
      for (int i = 0; i < LOADS; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
  }
  // the workgroup's XOR: lanes, then wavefronts
  for (int d = 32; d >= 1; d >>= 1) x ^= __shfl_xor(x, d, 64);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kProbeWaves; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

template <int MODE, int RING>
void launch_probe(int loads, dim3 grid, hipStream_t st, const char *b, const int32_t *order,
                  int32_t n, uint32_t nb, uint32_t *sink) {
  const dim3 block(kProbeWaves * 64);
  // chunks larger than the ring are refused by the caller
  if (loads == 1)
    hipLaunchKernelGGL((read_probe_kernel<MODE, 1, RING>), grid, block, 0, st, b, order, n, nb,
                       sink);
  else if (loads == 2)
    hipLaunchKernelGGL((read_probe_kernel<MODE, 2, RING>), grid, block, 0, st, b, order, n, nb,
                       sink);
  else if (loads == 4)
    hipLaunchKernelGGL((read_probe_kernel<MODE, 4, RING>), grid, block, 0, st, b, order, n, nb,
                       sink);
  else if constexpr (RING >= 8192)
    hipLaunchKernelGGL((read_probe_kernel<MODE, 8, RING>), grid, block, 0, st, b, order, n, nb,
                       sink);
}

}  // namespace

extern "C" int paged_kv_read_probe(const void *buf, size_t buf_bytes, const int32_t *order,
                                   int32_t n_chunks, int32_t chunk_bytes, int mode,
                                   int32_t ring_bytes, int32_t n_wg, uint32_t *sink,
                                   void *stream) {
  if (!buf || !order || !sink) return fail(PKV_EINVAL, "NULL pointer");
  if (n_chunks <= 0 || n_wg <= 0 || n_wg > 65535)
    return fail(PKV_EINVAL, "n_chunks and n_wg must be positive (n_wg <= 65535)");
  if (chunk_bytes != 1024 && chunk_bytes != 2048 && chunk_bytes != 4096 && chunk_bytes != 8192)
    return fail(PKV_EINVAL, "chunk_bytes must be 1, 2, 4 or 8 KiB, not %d", chunk_bytes);
  if ((uintptr_t)buf % 16) return fail(PKV_EINVAL, "buf must be 16-byte aligned");
  const size_t n_buf = buf_bytes / (size_t)chunk_bytes;
  if (n_buf == 0) return fail(PKV_EINVAL, "buffer smaller than one chunk");
  if (n_buf > (size_t)INT32_MAX)
    return fail(PKV_EINVAL, "buffer has more chunks than an int32 index reaches");
  if (mode < 0 || mode > 2) return fail(PKV_EINVAL, "mode must be 0, 1 or 2, not %d", mode);
  if (mode == 2 && ring_bytes != 4096 && ring_bytes != 8192 && ring_bytes != 16384)
    return fail(PKV_EINVAL, "ring_bytes must be 4, 8 or 16 KiB, not %d", ring_bytes);
  if (mode == 2 && ring_bytes < chunk_bytes)
    return fail(PKV_EINVAL, "a ring of %d bytes cannot hold a %d-byte chunk", ring_bytes,
                chunk_bytes);
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(n_wg);
  const char *b = (const char *)buf;
  const int loads = chunk_bytes / 1024;
  const uint32_t nb = (uint32_t)n_buf;
  if (mode == 0) launch_probe<0, 16384>(loads, grid, st, b, order, n_chunks, nb, sink);
  else if (mode == 1) launch_probe<1, 16384>(loads, grid, st, b, order, n_chunks, nb, sink);
  else if (ring_bytes == 4096) launch_probe<2, 4096>(loads, grid, st, b, order, n_chunks, nb, sink);
  else if (ring_bytes == 8192) launch_probe<2, 8192>(loads, grid, st, b, order, n_chunks, nb, sink);
  else launch_probe<2, 16384>(loads, grid, st, b, order, n_chunks, nb, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "read probe launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
