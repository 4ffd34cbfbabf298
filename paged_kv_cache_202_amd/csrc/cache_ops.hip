// Device cache maintenance for gfx950: the slot-mapped cache write and the
// copy-on-write block copy.
//
// Cache write: "NeuralOps v1.3.4: Serving Primitives & KV Cache Optimization"
// (Highlights: slot mapping; Architectural Breakdown 1: block table). The
// copy: course page "Module 10. KV Caches and Efficient Inference", notebook
// section 5 "Page pool: prefix sharing and copy-on-write" (a writer into a
// shared partial block first gets a private copy).
//
// Both are pure byte movement, bound by HBM bandwidth. Every (token, KV head)
// row of D elements is contiguous in the source and in the destination pool
// ([num_blocks, Hkv, block_size, D]), and a whole block is contiguous too, so
// each thread moves 16-byte vectors and consecutive lanes touch consecutive
// addresses on both sides.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace {

// One thread per 16-byte vector of the new rows; grid-stride.
__global__ void __launch_bounds__(256)
cache_write_kernel(const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new,
                   uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache,
                   const int32_t *__restrict__ slots, int64_t total_vec, int32_t vec_per_row,
                   int32_t Hkv, int32_t bs, int64_t num_slots) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_vec; i += stride) {
    const int64_t row = i / vec_per_row;  // t * Hkv + h
    const int32_t v = (int32_t)(i - row * vec_per_row);
    const int64_t t = row / Hkv;
    const int32_t h = (int32_t)(row - t * Hkv);
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    const int64_t blk = s / bs, off = s - blk * bs;
    const int64_t dst = ((blk * Hkv + h) * bs + off) * vec_per_row + v;
    k_cache[dst] = k_new[i];
    v_cache[dst] = v_new[i];
  }
}

// blockIdx.y = pair index, blockIdx.z = pool (0: k_cache, 1: v_cache);
// threads stride over the block's 16-byte vectors.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache,
                   const pkv_cow_t *__restrict__ pairs, int64_t vec_per_block,
                   int32_t num_blocks) {
  const pkv_cow_t pr = pairs[blockIdx.y];
  if (pr.src < 0 || pr.src >= num_blocks || pr.dst < 0 || pr.dst >= num_blocks) return;
  uint4 *pool = blockIdx.z ? v_cache : k_cache;
  const uint4 *src = pool + (int64_t)pr.src * vec_per_block;
  uint4 *dst = pool + (int64_t)pr.dst * vec_per_block;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < vec_per_block;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// Per-row integer codes of the course page's teaching quantizer (project
// demo, Demo 2: symmetric codes, one scale per row), BITS = 8 or 3: for each
// new (token, KV head) row x of D values, limit = 2^(BITS-1) - 1, scale =
// max |x| / limit (1 for a row of zeros), code = clip(round-half-even(x /
// scale), -limit, limit), in float64 as the page computes; the scale is
// stored as float32 in the scale row [blk, h, K = 0 / V = 1, :] beside the
// other's. 8-bit codes are stored as int8; 3-bit codes two per byte as the
// 4-bit float e2m1 (sign, 2 exponent bits, 1 mantissa bit), which holds
// every code in [-3, 3] exactly, even dim in the low nibble. One wavefront
// per row: each lane holds D / 64 consecutive elements.
// e2m1 bits of an integer code in [-3, 3]: 0, 1, 2, 3 are 0x0, 0x2, 0x4,
// 0x5 (1 = 2^0, 2 = 2^1, 3 = 1.5 x 2^1); bit 3 is the sign (0 stays +0).
__device__ __forceinline__ uint32_t e2m1_code(int c) {
  const int m = c < 0 ? -c : c;
  return (c < 0 ? 8u : 0u) | (m == 3 ? 5u : 2u * (uint32_t)m);
}

template <int D, int BITS, typename T>
__global__ void __launch_bounds__(256)
cache_write_q_kernel(const T *__restrict__ k_new, const T *__restrict__ v_new,
                     int8_t *__restrict__ k_codes, int8_t *__restrict__ v_codes,
                     float *__restrict__ scales, const int32_t *__restrict__ slots, int64_t rows, int32_t Hkv, int32_t bs,
                     int64_t num_slots) {
  constexpr int EPL = D / 64;
  constexpr double kLimit = (1 << (BITS - 1)) - 1;
  static_assert(BITS == 8 || (BITS == 3 && EPL % 2 == 0), "8-bit, or 3-bit with whole bytes");
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * Hkv + h
  if (row >= rows) return;
  const int64_t t = row / Hkv;
  const int32_t h = (int32_t)(row - t * Hkv);
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;
  const int64_t blk = s / bs, off = s - blk * bs;
  const int64_t dst = (blk * Hkv + h) * bs + off;  // row of the code pools
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const T *src = (which ? v_new : k_new) + row * D + lane * EPL;
    double x[EPL];
    double mx = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if constexpr (sizeof(T) == 2) {  // bf16 bits: the float32 with these upper bits
        x[e] = (double)__uint_as_float((uint32_t)((const uint16_t *)src)[e] << 16);
      } else {
        x[e] = (double)src[e];
      }
      mx = fmax(mx, fabs(x[e]));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmax(mx, __shfl_xor(mx, m, 64));
    double scale = mx / kLimit;
    if (scale == 0.0) scale = 1.0;
    int c[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) c[e] = (int)fmin(fmax(rint(x[e] / scale), -kLimit), kLimit);
    if constexpr (BITS == 8) {
      int8_t *codes = (which ? v_codes : k_codes) + dst * D + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) codes[e] = (int8_t)c[e];
    } else {
      uint8_t *codes = (uint8_t *)(which ? v_codes : k_codes) + dst * (D / 2) + lane * (EPL / 2);
#pragma unroll
      for (int e = 0; e < EPL; e += 2)
        codes[e / 2] = (uint8_t)(e2m1_code(c[e]) | (e2m1_code(c[e + 1]) << 4));
    }
    if (lane == 0) scales[((blk * Hkv + h) * 2 + which) * bs + off] = (float)scale;
  }
}

int elem_bytes(int dtype) {
  return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : dtype == PKV_I8 ? 1 : 0;
}

}  // namespace

using pkv::fail;

#ifdef PKV_DEBUG_SLOTS
// Debug builds only: refuse a slot mapping that names one slot twice (see
// paged_kv_check_slots). The mapping is copied to the host and the stream
// waited for, which a production write must not do.
static int debug_check_slots(const int32_t *slot_mapping, int32_t T, int64_t num_slots,
                             hipStream_t stream) {
  std::vector<int32_t> host(T);
  hipError_t e = hipMemcpyAsync(host.data(), slot_mapping, sizeof(int32_t) * (size_t)T,
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(PKV_EHIP, "slot check copy: %s", hipGetErrorString(e));
  return paged_kv_check_slots(host.data(), T, num_slots, nullptr);
}
#define PKV_CHECK_SLOTS(slots, T, n, stream) \
  do {                                                                          \
    if (int rc_ = debug_check_slots(slots, T, n, (hipStream_t)(stream))) return rc_; \
  } while (0)
#else
#define PKV_CHECK_SLOTS(slots, T, n, stream) \
  do {                                       \
  } while (0)
#endif

extern "C" int paged_cache_write(const void *k_new, const void *v_new, void *k_cache,
                                 void *v_cache, const int32_t *slot_mapping, int32_t T,
                                 int32_t num_blocks, int32_t Hkv, int32_t D,
                                 int32_t block_size, int dtype, void *stream) {
  const int es = elem_bytes(dtype);
  if (!es) return fail(PKV_EINVAL, "unsupported dtype %d", dtype);
  if (T < 0 || num_blocks <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "sizes must be positive (T >= 0)");
  if ((D * es) % 16)
    return fail(PKV_EINVAL, "a row of D=%d elements must be a multiple of 16 bytes", D);
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_EINVAL, "NULL pointer");
  for (const void *p : {k_new, v_new, (const void *)k_cache, (const void *)v_cache})
    if ((uintptr_t)p % 16) return fail(PKV_EINVAL, "K/V pointers must be 16-byte aligned");
  PKV_CHECK_SLOTS(slot_mapping, T, (int64_t)num_blocks * block_size, stream);
  const int32_t vpr = D * es / 16;
  const int64_t total = (int64_t)T * Hkv * vpr;
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(cache_write_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const uint4 *)k_new, (const uint4 *)v_new, (uint4 *)k_cache,
                     (uint4 *)v_cache, slot_mapping, total, vpr, Hkv, block_size,
                     (int64_t)num_blocks * block_size);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "cache write launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int paged_kv_copy_blocks(void *k_cache, void *v_cache, const pkv_cow_t *pairs,
                                    int32_t n, int32_t num_blocks, int32_t Hkv, int32_t D,
                                    int32_t block_size, int dtype, void *stream) {
  const int es = elem_bytes(dtype);
  if (!es) return fail(PKV_EINVAL, "unsupported dtype %d", dtype);
  if (n < 0 || num_blocks <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "sizes must be positive (n >= 0)");
  if (n > 65535) return fail(PKV_EINVAL, "at most 65535 pairs per call");
  const int64_t block_bytes = (int64_t)Hkv * block_size * D * es;
  if (block_bytes % 16) return fail(PKV_EINVAL, "block bytes must be a multiple of 16");
  if (n == 0) return PKV_OK;
  if (!k_cache || !pairs) return fail(PKV_EINVAL, "NULL pointer");
  if ((uintptr_t)k_cache % 16 || (uintptr_t)v_cache % 16)
    return fail(PKV_EINVAL, "K/V pools must be 16-byte aligned");
  const int64_t vpb = block_bytes / 16;
  int gx = (int)((vpb + 255) / 256);
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, n, v_cache ? 2 : 1), dim3(256), 0,
                     (hipStream_t)stream,
                     (uint4 *)k_cache, (uint4 *)v_cache, pairs, vpb, num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "block copy launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

template <int BITS>
static int cache_write_q(const void *k_new, const void *v_new, int8_t *k_codes, int8_t *v_codes,
                         float *scales, const int32_t *slot_mapping, int32_t T,
                         int32_t num_blocks, int32_t Hkv, int32_t D, int32_t block_size,
                         int dtype, void *stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16)
    return fail(PKV_EINVAL, "new rows must be f32 or bf16 (dtype %d)", dtype);
  if (T < 0 || num_blocks <= 0 || Hkv <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "sizes must be positive (T >= 0)");
  if (D != 128 && D != 256 && (BITS == 3 || D != 64))
    return fail(PKV_EINVAL, "head dim %d unsupported for %d-bit codes", D, BITS);
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !k_codes || !v_codes || !scales || !slot_mapping)
    return fail(PKV_EINVAL, "NULL pointer");
  const int64_t rows = (int64_t)T * Hkv;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  PKV_CHECK_SLOTS(slot_mapping, T, num_slots, stream);
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  hipStream_t s = (hipStream_t)stream;
#define PKV_Q(d)                                                                            \
  if (D == d) {                                                                             \
    if constexpr (BITS == 8 || d >= 128) {                                                  \
      if (dtype == PKV_BF16)                                                                \
        hipLaunchKernelGGL((cache_write_q_kernel<d, BITS, uint16_t>), grid, block, 0, s,     \
                           (const uint16_t *)k_new, (const uint16_t *)v_new, k_codes,        \
                           v_codes, scales, slot_mapping, rows, Hkv, block_size, num_slots); \
      else                                                                                  \
        hipLaunchKernelGGL((cache_write_q_kernel<d, BITS, float>), grid, block, 0, s,        \
                           (const float *)k_new, (const float *)v_new, k_codes, v_codes,     \
                           scales, slot_mapping, rows, Hkv, block_size, num_slots);          \
    }                                                                                       \
  }
  PKV_Q(64) PKV_Q(128) PKV_Q(256)
#undef PKV_Q
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "cache write launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int paged_cache_write_q8(const void *k_new, const void *v_new, int8_t *k_codes,
                                    int8_t *v_codes, float *scales,
                                    const int32_t *slot_mapping, int32_t T, int32_t num_blocks,
                                    int32_t Hkv, int32_t D, int32_t block_size, int dtype,
                                    void *stream) {
  return cache_write_q<8>(k_new, v_new, k_codes, v_codes, scales, slot_mapping, T, num_blocks,
                          Hkv, D, block_size, dtype, stream);
}

extern "C" int paged_cache_write_q3(const void *k_new, const void *v_new, uint8_t *k_codes,
                                    uint8_t *v_codes, float *scales,
                                    const int32_t *slot_mapping, int32_t T, int32_t num_blocks,
                                    int32_t Hkv, int32_t D, int32_t block_size, int dtype,
                                    void *stream) {
  return cache_write_q<3>(k_new, v_new, (int8_t *)k_codes, (int8_t *)v_codes, scales,
                          slot_mapping, T, num_blocks, Hkv, D, block_size, dtype, stream);
}
