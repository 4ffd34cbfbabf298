// Shared-prefix attention on MFMA for gfx950 (MI355X): the prefix phase of
// paged attention for groups of sequences whose block tables begin with the
// same physical blocks. Sharing blocks within and across requests is the
// point of PagedAttention (vLLM abstract on the papers page "external
// vector cache"); forking a prefix by reference counts is the page pool of
// the course page "Module 10. KV Caches and Efficient Inference", notebook
// section 5. The arithmetic is the decode kernels' -- each query row's
// max-subtracted softmax over the keys it sees (that page's project demo,
// Demo 2), computed online -- restricted to the shared tokens; the private
// rest of every context is handled by the ordinary kernels from the
// group's prefix length on, and a log-sum-exp merge joins the two.
//
// Design (for CDNA4):
//   * the query rows of all members of a group are stacked: a 16-row MFMA
//     tile holds 16 / RPM members' rows (RPM = G x query tokens, padded to a
//     power of two). One workgroup = W wavefronts = W row tiles of the same
//     (group, KV head, prefix partition), RT = 1 or 2 tiles per wavefront
//     sharing each K/V read; every prefix tile is gathered once
//     into the workgroup's LDS ring by direct-to-LDS loads and read by all W
//     wavefronts, so each shared K/V byte leaves L2 once per W row tiles
//     instead of once per member;
//   * the gathers place bytes so that the reads are conflict-free: K in the
//     order its MFMA A operand is read (lane l's c-th 16 bytes at
//     (c * 64 + l) * 16), V in token rows whose 16-byte chunks are
//     XOR-swizzled by token, read back with the transposing LDS read as the
//     A operand of the transposed product O^T += V^T P^T;
//   * per tile: S^T = K Q^T with v_mfma_f32_16x16x32_bf16, online softmax
//     with a lazily raised maximum, P rounded to bf16, O^T += V^T P^T with
//     v_mfma_f32_16x16x16_bf16 -- the verify kernel's arithmetic. Computing
//     O transposed leaves each row's outputs in the lane that holds its
//     softmax statistics, so rescaling needs no cross-lane moves;
//   * a ring of 4 or 8 tile slots and one workgroup barrier per tile: a slot
//     is refilled right after the barrier that follows the last reads of it,
//     so all but one slot are in flight;
//   * each wavefront writes its rows' unnormalised partials (m, l, acc) for
//     its prefix partition; the merge kernel joins them with the suffix's.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "decode_kernel.h"
#include "verify_mfma.h"

namespace pkv {
namespace decode {

// Sharing groups as the prefix kernel sees them (all device arrays).
struct ShareArgs {
  const int32_t *group_start;   // [n_groups + 1] offsets into members
  const int32_t *members;       // sequence indices, grouped
  const int32_t *group_tokens;  // [n_groups] shared prefix tokens (multiple of 16)
  int32_t n_groups;
  int32_t n_members;    // length of members (= group_start[n_groups])
  int32_t chunks;       // workgroups (of W row tiles) per group along grid.z
  int32_t rpm;          // query rows per member, padded to a power of two
  int32_t prefix_part;  // tokens per prefix partition (multiple of 16)
};

template <int D, int W = 1>
struct PrefixGeo {
  static constexpr int NC = D / 32;                // A-operand chunks per lane (16 B each)
  static constexpr int NCB = D / 16;               // column blocks of P V
  static constexpr int kHalf = kTile * D * 2;      // bytes of a K (or V) tile
  static constexpr int kTileBytes = 2 * kHalf;     // K then V
  static constexpr int kLoads = kTileBytes / 1024; // 1 KiB gathers per tile
  static constexpr int kRowChunks = D / 8;         // 16-byte chunks per V token row
  // tiles in the ring: 128 KiB for workgroups of eight wavefronts (their
  // registers allow one workgroup per CU, so the LDS would idle otherwise),
  // 64 KiB else, at most 16 tiles
  static constexpr int kRingBytes = W >= 8 ? 131072 : 65536;
  static constexpr int kSlots =
      kRingBytes / kTileBytes > 16 ? 16 : kRingBytes / kTileBytes;
  static_assert(kSlots >= 4 && (kSlots & (kSlots - 1)) == 0, "ring of 4, 8 or 16 slots");
};

// XOR swizzle of the 16-byte chunks of V token row t. A transposing read of
// a 16-lane group names 32 bytes (a chunk pair) of each of four consecutive
// tokens; XOR-ing with 2 t moves the four tokens' pairs to four different
// 32-byte bank ranges (and eight consecutive tokens to all sixteen chunks of
// a row), where XOR-ing with t would leave tokens t and t ^ 1 on one range.
template <int D>
__device__ __forceinline__ int v_swizzle(int t) {
  return (2 * t) & (PrefixGeo<D>::kRowChunks - 1);
}

// One tile's MFMA operands from an LDS slot, with one wait for all of them.
// K: this lane's NC 16-byte A-operand chunks at kp + c * 1024 (the gathers
// put them there). V: the A operand of O^T += V^T P^T for each 16-dim column
// block, read with the gfx950 transposing LDS read (ds_read_b64_tr_b16):
// within each group of 16 lanes, lane s names 8 bytes holding elements
// 4 s' .. 4 s' + 3 of a 64-element window and lane i receives window elements
// i, i + 16, i + 32, i + 48. So if lane s of group lg names dims
// cb * 16 + 4 (s % 4) .. + 3 of token 4 lg + s / 4, lane i receives
// V[4 lg + u][cb * 16 + i], u = 0..3. va[cb] is this lane's address for
// column block cb.
template <int D>
__device__ __forceinline__ void read_kv(u32x4_t (&k)[D / 32], uint2 (&v)[D / 16],
                                        const PKV_LDS char *kp,
                                        const PKV_LDS char *const (&va)[D / 16]);

template <>
__device__ __forceinline__ void read_kv<64>(u32x4_t (&k)[2], uint2 (&v)[4],
                                           const PKV_LDS char *kp,
                                           const PKV_LDS char *const (&va)[4]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %7\n\t"
      "ds_read_b64_tr_b16 %3, %8\n\t"
      "ds_read_b64_tr_b16 %4, %9\n\t"
      "ds_read_b64_tr_b16 %5, %10\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(kp), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])
      : "memory");
}

template <>
__device__ __forceinline__ void read_kv<128>(u32x4_t (&k)[4], uint2 (&v)[8],
                                           const PKV_LDS char *kp,
                                           const PKV_LDS char *const (&va)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %12 offset:2048\n\t"
      "ds_read_b128 %3, %12 offset:3072\n\t"
      "ds_read_b64_tr_b16 %4, %13\n\t"
      "ds_read_b64_tr_b16 %5, %14\n\t"
      "ds_read_b64_tr_b16 %6, %15\n\t"
      "ds_read_b64_tr_b16 %7, %16\n\t"
      "ds_read_b64_tr_b16 %8, %17\n\t"
      "ds_read_b64_tr_b16 %9, %18\n\t"
      "ds_read_b64_tr_b16 %10, %19\n\t"
      "ds_read_b64_tr_b16 %11, %20\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(kp), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
      : "memory");
}

template <>
__device__ __forceinline__ void read_kv<256>(u32x4_t (&k)[8], uint2 (&v)[16],
                                           const PKV_LDS char *kp,
                                           const PKV_LDS char *const (&va)[16]) {
  asm volatile(
      "ds_read_b128 %0, %24\n\t"
      "ds_read_b128 %1, %24 offset:1024\n\t"
      "ds_read_b128 %2, %24 offset:2048\n\t"
      "ds_read_b128 %3, %24 offset:3072\n\t"
      "ds_read_b128 %4, %24 offset:4096\n\t"
      "ds_read_b128 %5, %24 offset:5120\n\t"
      "ds_read_b128 %6, %24 offset:6144\n\t"
      "ds_read_b128 %7, %24 offset:7168\n\t"
      "ds_read_b64_tr_b16 %8, %25\n\t"
      "ds_read_b64_tr_b16 %9, %26\n\t"
      "ds_read_b64_tr_b16 %10, %27\n\t"
      "ds_read_b64_tr_b16 %11, %28\n\t"
      "ds_read_b64_tr_b16 %12, %29\n\t"
      "ds_read_b64_tr_b16 %13, %30\n\t"
      "ds_read_b64_tr_b16 %14, %31\n\t"
      "ds_read_b64_tr_b16 %15, %32\n\t"
      "ds_read_b64_tr_b16 %16, %33\n\t"
      "ds_read_b64_tr_b16 %17, %34\n\t"
      "ds_read_b64_tr_b16 %18, %35\n\t"
      "ds_read_b64_tr_b16 %19, %36\n\t"
      "ds_read_b64_tr_b16 %20, %37\n\t"
      "ds_read_b64_tr_b16 %21, %38\n\t"
      "ds_read_b64_tr_b16 %22, %39\n\t"
      "ds_read_b64_tr_b16 %23, %40\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
      : "v"(kp), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]), "v"(va[8]), "v"(va[9]), "v"(va[10]), "v"(va[11]), "v"(va[12]), "v"(va[13]), "v"(va[14]), "v"(va[15])
      : "memory");
}

// The same for the two adjacent slots of a trip of two tiles (the second
// slot's operands at the same addresses plus one tile).
template <int D>
__device__ __forceinline__ void read_kv2(u32x4_t (&k)[2][D / 32], uint2 (&v)[2][D / 16],
                                         const PKV_LDS char *kp,
                                         const PKV_LDS char *const (&va)[D / 16]);

template <>
__device__ __forceinline__ void read_kv2<64>(u32x4_t (&k)[2][2], uint2 (&v)[2][4],
                                            const PKV_LDS char *kp,
                                            const PKV_LDS char *const (&va)[4]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %12 offset:4096\n\t"
      "ds_read_b128 %3, %12 offset:5120\n\t"
      "ds_read_b64_tr_b16 %4, %13\n\t"
      "ds_read_b64_tr_b16 %5, %14\n\t"
      "ds_read_b64_tr_b16 %6, %15\n\t"
      "ds_read_b64_tr_b16 %7, %16\n\t"
      "ds_read_b64_tr_b16 %8, %13 offset:4096\n\t"
      "ds_read_b64_tr_b16 %9, %14 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %15 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %16 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[1][0]), "=&v"(k[1][1]), "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3])
      : "v"(kp), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])
      : "memory");
}

template <>
__device__ __forceinline__ void read_kv2<128>(u32x4_t (&k)[2][4], uint2 (&v)[2][8],
                                            const PKV_LDS char *kp,
                                            const PKV_LDS char *const (&va)[8]) {
  asm volatile(
      "ds_read_b128 %0, %24\n\t"
      "ds_read_b128 %1, %24 offset:1024\n\t"
      "ds_read_b128 %2, %24 offset:2048\n\t"
      "ds_read_b128 %3, %24 offset:3072\n\t"
      "ds_read_b128 %4, %24 offset:8192\n\t"
      "ds_read_b128 %5, %24 offset:9216\n\t"
      "ds_read_b128 %6, %24 offset:10240\n\t"
      "ds_read_b128 %7, %24 offset:11264\n\t"
      "ds_read_b64_tr_b16 %8, %25\n\t"
      "ds_read_b64_tr_b16 %9, %26\n\t"
      "ds_read_b64_tr_b16 %10, %27\n\t"
      "ds_read_b64_tr_b16 %11, %28\n\t"
      "ds_read_b64_tr_b16 %12, %29\n\t"
      "ds_read_b64_tr_b16 %13, %30\n\t"
      "ds_read_b64_tr_b16 %14, %31\n\t"
      "ds_read_b64_tr_b16 %15, %32\n\t"
      "ds_read_b64_tr_b16 %16, %25 offset:8192\n\t"
      "ds_read_b64_tr_b16 %17, %26 offset:8192\n\t"
      "ds_read_b64_tr_b16 %18, %27 offset:8192\n\t"
      "ds_read_b64_tr_b16 %19, %28 offset:8192\n\t"
      "ds_read_b64_tr_b16 %20, %29 offset:8192\n\t"
      "ds_read_b64_tr_b16 %21, %30 offset:8192\n\t"
      "ds_read_b64_tr_b16 %22, %31 offset:8192\n\t"
      "ds_read_b64_tr_b16 %23, %32 offset:8192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[0][2]), "=&v"(k[0][3]), "=&v"(k[1][0]), "=&v"(k[1][1]), "=&v"(k[1][2]), "=&v"(k[1][3]), "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[0][4]), "=&v"(v[0][5]), "=&v"(v[0][6]), "=&v"(v[0][7]), "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3]), "=&v"(v[1][4]), "=&v"(v[1][5]), "=&v"(v[1][6]), "=&v"(v[1][7])
      : "v"(kp), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
      : "memory");
}

// The K half and the V half of a trip of two D = 128 tiles, each read on
// its own (same addresses as read_kv2<128>), so that a wavefront's V reads
// come after its score products and softmax: the wavefronts of a SIMD then
// do not all read LDS at once after the trip's barrier and then all wait on
// the matrix core (chunked prefill 4 x 512 rows at 8K: 384.7 -> 368.9 us;
// reading each tile's K right before its products instead: 384.1 us).
// K of a tile pair at kp + OFF (tiles 8 KiB apart), with one wait.
template <int OFF>
__device__ __forceinline__ void read_k2_128(u32x4_t (&k)[2][4], const PKV_LDS char *kp) {
  static_assert(OFF >= 0 && OFF + 11264 < 65536, "LDS immediate offsets are 16 bits");
  asm volatile(
      "ds_read_b128 %0, %8 offset:%9\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %8 offset:%14\n\t"
      "ds_read_b128 %6, %8 offset:%15\n\t"
      "ds_read_b128 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[0][2]), "=&v"(k[0][3]), "=&v"(k[1][0]),
        "=&v"(k[1][1]), "=&v"(k[1][2]), "=&v"(k[1][3])
      : "v"(kp), "i"(OFF), "i"(OFF + 1024), "i"(OFF + 2048), "i"(OFF + 3072), "i"(OFF + 8192),
        "i"(OFF + 9216), "i"(OFF + 10240), "i"(OFF + 11264)
      : "memory");
}

// V of a tile pair, transposed: column block cb at va[cb] + OFF and + OFF +
// 8 KiB, with one wait.
template <int OFF>
__device__ __forceinline__ void read_v2_128(uint2 (&v)[2][8], const PKV_LDS char *const (&va)[8]) {
  static_assert(OFF >= 0 && OFF + 8192 < 65536, "LDS immediate offsets are 16 bits");
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %2, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %4, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %6, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%25\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:%25\n\t"
      "ds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
      "ds_read_b64_tr_b16 %12, %20 offset:%25\n\t"
      "ds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[0][4]),
        "=&v"(v[0][5]), "=&v"(v[0][6]), "=&v"(v[0][7]), "=&v"(v[1][0]), "=&v"(v[1][1]),
        "=&v"(v[1][2]), "=&v"(v[1][3]), "=&v"(v[1][4]), "=&v"(v[1][5]), "=&v"(v[1][6]),
        "=&v"(v[1][7])
      : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]),
        "v"(va[7]), "i"(OFF), "i"(OFF + 8192)
      : "memory");
}

// The largest of three floats (the compiler forms v_max3_f32; inline
// assembly here would hide from its hazard checks that the operands come
// straight from the matrix cores).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// K halves and V halves on their own for the other head dims, so that a
// trip's K can be read for its score products while the V of the trip
// before is still to come: D = 64 (two tiles a trip, 4 KiB apart) and
// D = 256 (one tile a trip).
__device__ __forceinline__ void read_k2_64(u32x4_t (&k)[2][2], const PKV_LDS char *kp) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:4096\n\t"
      "ds_read_b128 %3, %4 offset:5120\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[1][0]), "=&v"(k[1][1])
      : "v"(kp)
      : "memory");
}

__device__ __forceinline__ void read_v2_64(uint2 (&v)[2][4], const PKV_LDS char *const (&va)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:4096\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:4096\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[1][0]),
        "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3])
      : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])
      : "memory");
}

__device__ __forceinline__ void read_k_256(u32x4_t (&k)[8], const PKV_LDS char *kp) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
        "=&v"(k[6]), "=&v"(k[7])
      : "v"(kp)
      : "memory");
}

__device__ __forceinline__ void read_v_256(uint2 (&v)[16], const PKV_LDS char *const (&va)[16]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %18\n\t"
      "ds_read_b64_tr_b16 %3, %19\n\t"
      "ds_read_b64_tr_b16 %4, %20\n\t"
      "ds_read_b64_tr_b16 %5, %21\n\t"
      "ds_read_b64_tr_b16 %6, %22\n\t"
      "ds_read_b64_tr_b16 %7, %23\n\t"
      "ds_read_b64_tr_b16 %8, %24\n\t"
      "ds_read_b64_tr_b16 %9, %25\n\t"
      "ds_read_b64_tr_b16 %10, %26\n\t"
      "ds_read_b64_tr_b16 %11, %27\n\t"
      "ds_read_b64_tr_b16 %12, %28\n\t"
      "ds_read_b64_tr_b16 %13, %29\n\t"
      "ds_read_b64_tr_b16 %14, %30\n\t"
      "ds_read_b64_tr_b16 %15, %31\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]),
        "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
      : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]),
        "v"(va[7]), "v"(va[8]), "v"(va[9]), "v"(va[10]), "v"(va[11]), "v"(va[12]),
        "v"(va[13]), "v"(va[14]), "v"(va[15])
      : "memory");
}

// Where the query rows of a workgroup come from.
enum class RowSource {
  kSharedGroups,  // stacked rows of a sharing group's members over their common prefix
  kChunk,         // one sequence's query chunk (G x nq rows) over its own context, causal
};

template <int D, int W, int RT, RowSource SRC>
__device__ __forceinline__ void mfma_rows_body(const DecodeArgs &a, const ShareArgs &s) {
  using Gp = PrefixGeo<D, W>;
  constexpr int NC = Gp::NC, NCB = Gp::NCB, kSlots = Gp::kSlots;
  // 16-token tiles per trip: at D = 128 four (a longer run of products
  // between softmax steps), two at D = 64, one at D = 256
  constexpr int TT = D == 128 ? 4 : D == 64 ? 2 : 1;
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  __shared__ u32x4_t sm_ring[kSlots * Gp::kTileBytes / 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int p = blockIdx.x, h = blockIdx.y;
  const int nq = a.nq, G = a.Hq / a.Hkv;
  const int max_ctx = a.max_blocks * a.bs;
  const int tile0 = (blockIdx.z % s.chunks) * W * RT;  // first row tile of this workgroup
  const float nan = __builtin_nanf("");

  // Per workgroup: the partition's tokens [t_begin, t_end) and the table row
  // that addresses them. Per lane and row tile r: the sequence of row ln
  // (-1: none), its flat row index (b, query, head) and the keys it sees.
  int t_begin, t_end, bad;
  const int32_t *trow;
  int b_row[RT], lim_r[RT];
  size_t qrow[RT];
  if constexpr (SRC == RowSource::kSharedGroups) {
    const int grp = blockIdx.z / s.chunks;
    if (grp >= s.n_groups) return;
    // group bounds are clamped to the members array, so that inconsistent
    // arrays cannot send reads out of it
    const int ms = max(0, min(s.n_members, load_const(s.group_start + grp)));
    const int me = max(ms, min(s.n_members, load_const(s.group_start + grp + 1)));
    const int prefix_req = load_const(s.group_tokens + grp);
    // a prefix that is not whole tiles or runs past the table poisons the group
    const int prefix = max(0, min(prefix_req, max_ctx)) & ~(kTile - 1);
    t_begin = p * s.prefix_part;
    const int mpt = kVerifyRows / s.rpm;  // members per row tile
    // workgroup-uniform exits: no tokens in this partition, no rows in this chunk
    if (t_begin >= prefix || ms + tile0 * mpt >= me) return;
    t_end = min(prefix, t_begin + s.prefix_part);
    // the leader's table row holds the shared blocks
    const int leader_raw = load_const(s.members + ms);
    const int leader = leader_raw >= 0 && leader_raw < a.B ? leader_raw : 0;
    trow = a.tables + (size_t)leader * a.max_blocks;
    bad = leader != leader_raw || prefix != prefix_req;
    const int rr = ln % s.rpm;  // row within the member
    const int qi = rr / G;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int mem_idx = ms + (tile0 + wave * RT + r) * mpt + ln / s.rpm;
      const int b_raw = mem_idx < me && qi < nq ? s.members[mem_idx] : -1;
      b_row[r] = b_raw >= 0 && b_raw < a.B ? b_raw : -1;
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int b = max(b_row[r], 0);
      const int L = a.lens[b];
      // a member whose length is out of range is left to the merge kernel (NaN)
      const bool live = b_row[r] >= 0 && L >= nq && L <= max_ctx;
      lim_r[r] = live ? L - nq + qi + 1 : 0;
      qrow[r] = ((size_t)b * nq + min(qi, nq - 1)) * a.Hq + h * G + rr % G;
    }
  } else {
    // rows r = query * G + head of one sequence; query i sees the first
    // L - nq + i + 1 keys
    const int b = blockIdx.z / s.chunks;
    if (b >= a.B) return;
    const int L = load_const(a.lens + b);
    // a length out of range is left to the merge kernel (NaN)
    if (L < nq || L > max_ctx) return;
    const int rows = G * nq;
    if (tile0 * kVerifyRows >= rows) return;
    const int r_last = min(rows, (tile0 + W * RT) * kVerifyRows) - 1;
    const int lim_max = L - nq + r_last / G + 1;  // keys seen by the workgroup's last row
    t_begin = p * s.prefix_part;
    if (t_begin >= lim_max) return;  // causal: no row here sees this partition
    t_end = min(lim_max, t_begin + s.prefix_part);
    trow = a.tables + (size_t)b * a.max_blocks;
    bad = 0;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int R = (tile0 + wave * RT + r) * kVerifyRows + ln;
      const int qi = min(R, rows - 1) / G, g = min(R, rows - 1) % G;
      b_row[r] = R < rows ? b : -1;
      lim_r[r] = R < rows ? L - nq + qi + 1 : 0;
      qrow[r] = ((size_t)b * nq + qi) * a.Hq + h * G + g;
    }
  }
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;

  // ---- set-up loads, issued side by side: the table window, the query rows --
  // lane i holds the block id of tile 64 w + i of the current window w
  // (clamped to the partition's last tile)
  auto table_window = [&](int w) {
    return trow[(t_begin + min(64 * w + lane, n_tiles - 1) * kTile) / a.bs];
  };
  int tblv = table_window(0);
  uint4 qb[RT][NC];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const uint16_t *qp = (const uint16_t *)a.q + qrow[r] * D + lg * (D / 4);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 v = *reinterpret_cast<const uint4 *>(qp + c * 8);
      qb[r][c] = lim_r[r] > 0 ? v : make_uint4(0, 0, 0, 0);
    }
  }
  // all of it is waited for here, once, before the first gather
  settle_v(tblv);
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int c = 0; c < NC; ++c) settle_v(qb[r][c]);
    settle_v(lim_r[r]);
  }

  const char *kbase = (const char *)a.kc;
  const char *vbase = (const char *)a.vc;
  PKV_LDS char *ring = (PKV_LDS char *)&sm_ring[0];
  // bad (workgroup-uniform): a tile came from a bad table entry, or the
  // group's description was unusable; the rows' partials become NaN
  // global byte offsets, inside a tile, of the 16 bytes lane l moves in
  // gather j: K in A-operand read order, V in swizzled token rows
  const int k_src = ln * (D * 2) + lg * (D / 2);  // + 16 j
  auto v_src = [&](int j) {
    const int pos = j * 1024 + lane * 16;  // destination byte in the V half
    const int t = pos / (D * 2), cp = (pos % (D * 2)) / 16;
    return t * (D * 2) + (cp ^ v_swizzle<D>(t)) * 16;
  };
  // bytes of one block (all KV heads) and this KV head's offset inside it
  const size_t blk_bytes = (size_t)a.Hkv * a.bs * (D * 2);
  const size_t head_off = (size_t)h * a.bs * (D * 2);
  const bool bs16 = a.bs == kTile;  // a block is one tile: no offset inside it
  auto stage = [&](int slot, int k, int blk) {
    const int t0 = t_begin + k * kTile;
    if (blk < 0 || blk >= a.num_blocks) {
      bad = 1;
      blk = 0;
    }
    const size_t tile = (size_t)(uint32_t)blk * blk_bytes + head_off +
                        (bs16 ? 0 : (size_t)(t0 % a.bs) * (D * 2));
    PKV_LDS char *dst = ring + slot * Gp::kTileBytes;
#pragma unroll
    for (int i = 0; i < (Gp::kLoads + W - 1) / W; ++i) {
      const int j = wave + i * W;  // this wavefront's gathers of the tile
      if (j < Gp::kLoads / 2)
        gather_lds16<0>(kbase + tile + k_src + j * 16, dst + j * 1024);
      else if (j < Gp::kLoads)
        gather_lds16<0>(vbase + tile + v_src(j - Gp::kLoads / 2), dst + j * 1024);
    }
  };
  constexpr int kPerWave = (Gp::kLoads + W - 1) / W;  // gathers per wavefront per tile

  // this lane's transposing-read addresses, relative to the V half of a
  // slot: dims cb * 16 + 4 (ln % 4) .. + 3 of token 4 lg + ln / 4, whose
  // 16-byte chunk sits at position chunk ^ swizzle(token)
  int v_addr[NCB];
  {
    const int t = 4 * lg + (ln >> 2);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = 2 * cb + ((ln >> 1) & 1);
      v_addr[cb] = Gp::kHalf + t * (D * 2) + ((c ^ v_swizzle<D>(t)) << 4) + (ln & 1) * 8;
    }
  }

  // O^T accumulators: o[r][cb][e] = O[row ln][dim cb * 16 + 4 lg + e], so
  // a row's statistics and its outputs live in the same lane
  f32x4_t o[RT][NCB];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[r][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_row[RT], l_part[RT];  // running max (log2 units) and weight-sum share of row ln
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m_row[r] = kNegInf;
    l_part[r] = 0.f;
  }
  float scale_log2 = a.scale_log2;  // waited for here, not inside the loop
  settle_s(scale_log2);
  if (scale_log2 < 0.f) {
    // q.k x scale = (-q).k x (-scale): negating bf16 queries is exact, and a
    // positive scale lets the largest raw score stand for the largest scaled one
    scale_log2 = -scale_log2;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        qb[r][c].x ^= 0x80008000u;
        qb[r][c].y ^= 0x80008000u;
        qb[r][c].z ^= 0x80008000u;
        qb[r][c].w ^= 0x80008000u;
      }
  }

  // keys of this partition visible to row ln of tile r
  int lim_p[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) lim_p[r] = min(lim_r[r], t_end);

  // TT tiles per trip share one barrier, one LDS wait and one softmax step;
  // every trip stages all TT tiles (past the end: the last tile again), so
  // that each wavefront's count of gathers in flight stays exact
  constexpr int kTrips = kSlots / TT;  // trips the ring holds
  const int n_trips = (n_tiles + TT - 1) / TT;
  auto stage_trip = [&](int j) {
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      const int kn = TT * j + u;
      if ((kn & 63) == 0 && kn > 0) {  // next window of block ids (drains the ring once)
        tblv = table_window(kn >> 6);
        settle_v(tblv);
      }
      stage(kn % kSlots, min(kn, n_tiles - 1), __builtin_amdgcn_readlane(tblv, kn & 63));
    }
  };
  // this lane's LDS read addresses inside slot 0: its K chunks, and the V
  // chunk of each column block (a trip adds its slot's offset)
  const PKV_LDS char *k_rd = ring + lane * 16;
  const PKV_LDS char *v_rd[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
    v_rd[cb] = ring + v_addr[cb] - (D == 128 ? Gp::kHalf : 0);  // D = 128: kHalf in the offset

  // Trips go in windows of kWin with one barrier each: within a window the
  // wavefronts drift apart, so that while some read LDS others run the
  // matrix cores or the softmax, instead of all doing the same in step.
  constexpr int kWin = kTrips >= 8 ? 2 : 1;
  // prologue: trips 0 .. kTrips - kWin - 1 in flight
#pragma unroll
  for (int j = 0; j < kTrips - kWin; ++j)
    if (j < n_trips) stage_trip(j);
  for (int j = 0; j < n_trips; ++j) {
    if (j % kWin == 0) {
      // this wavefront's gathers of trips j .. j + kWin - 1 have landed (the
      // later ones, up to kTrips - 2 kWin trips, may not) ...
      const int ahead = max(0, min(n_trips - j - kWin, kTrips - 2 * kWin));
      static_for<kTrips - 2 * kWin + 1>([&](auto ac) {
        constexpr int A = decltype(ac)::value;
        if (ahead == A) wait_vmcnt<A * TT * kPerWave>();
      });
      // ... and so have everyone's; everyone is done reading the window
      // before, whose slots take the trips kTrips - kWin ahead
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int u = 0; u < kWin; ++u)
        if (j + kTrips - kWin + u < n_trips) stage_trip(j + kTrips - kWin + u);
    }
    const int so = ((TT * j) % kSlots) * Gp::kTileBytes;  // the trip's slot
    const int t0 = t_begin + TT * j * kTile;

    // the K half of the trip's tiles; V is read after the softmax
    u32x4_t kr[TT][NC];
    if constexpr (D == 128) {
      // tile pairs, 16 KiB apart in the ring
      static_for<TT / 2>([&](auto pc) {
        constexpr int pp = decltype(pc)::value;
        read_k2_128<pp * 16384>(*reinterpret_cast<u32x4_t(*)[2][NC]>(&kr[2 * pp][0]), k_rd + so);
      });
    } else if constexpr (D == 64)
      read_k2_64(kr, k_rd + so);
    else
      read_k_256(kr[0], k_rd + so);

    // S^T = K Q^T per tile and row tile: sv[u][r][e] = q.k of row ln with
    // token t0 + 16 u + 4 lg + e (unscaled; the scale enters the exponent)
    f32x4_t sv[TT][RT];
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int r = 0; r < RT; ++r) sv[u][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int u = 0; u < TT; ++u)
#pragma unroll
        for (int r = 0; r < RT; ++r)
          sv[u][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, kr[u][c]), __builtin_bit_cast(bf16x8_t, qb[r][c]),
              sv[u][r], 0, 0, 0);

    uint2 pa[TT][RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (!__all(t0 + TT * kTile <= lim_p[r])) {
        // tokens a row does not see (causal, or past the partition) score
        // -inf: token t0 + 16 u + 4 lg + e, compared as 16 u + e against the
        // lane's bound (constants in the compares)
        const int d = lim_p[r] - t0 - 4 * lg;
#pragma unroll
        for (int u = 0; u < TT; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * u + e >= d) sv[u][r][e] = kNegInf;
      }
      // the lazy maximum: raised only when a score passes it by kLazyLog2;
      // scale_log2 > 0 (a negative scale was moved into the query), so the
      // largest raw score gives the largest scaled one
      float rmax;
      if constexpr (TT == 4) {
        const float a0 = max3f(sv[0][r][0], sv[0][r][1], sv[0][r][2]);
        const float a1 = max3f(sv[0][r][3], sv[1][r][0], sv[1][r][1]);
        const float a2 = max3f(sv[1][r][2], sv[1][r][3], sv[2][r][0]);
        const float a3 = max3f(sv[2][r][1], sv[2][r][2], sv[2][r][3]);
        const float a4 = max3f(sv[3][r][0], sv[3][r][1], sv[3][r][2]);
        rmax = max3f(max3f(a0, a1, a2), max3f(a3, a4, sv[3][r][3]), a0);
      } else {
        rmax = kNegInf;
#pragma unroll
        for (int u = 0; u < TT; ++u)
          rmax = fmaxf(rmax, fmaxf(fmaxf(sv[u][r][0], sv[u][r][1]), fmaxf(sv[u][r][2], sv[u][r][3])));
      }
      const float tmax = rmax * scale_log2;
      if (__any(tmax > m_row[r] + kLazyLog2)) {
        // row ln's scores are spread over the four lane groups
        float gmax = fmaxf(tmax, exact_xor<16>(tmax));
        gmax = fmaxf(gmax, exact_xor<32>(gmax));
        const float mn = fmaxf(m_row[r], gmax);
        const float alpha = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_row[r] - mn);
        m_row[r] = mn;
        l_part[r] *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[r][cb] *= alpha;
      }
      // weights exp2(s * scale_log2 - m): a masked score (-inf) gives 0, and
      // the maximum is floored so that a row with no visible key yet (maximum
      // -inf) gives 0 too, not NaN
      const float neg_m = -fmaxf(m_row[r], -3.0e38f);
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        float pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pw[e] = __builtin_amdgcn_exp2f(fmaf(sv[u][r][e], scale_log2, neg_m));
          l_part[r] += pw[e];
        }
        pa[u][r] = make_uint2(pack_bf16(pw[0], pw[1]), pack_bf16(pw[2], pw[3]));
      }
    }

    // the V half, read transposed
    uint2 vb[TT][NCB];
    {
      const PKV_LDS char *va[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) va[cb] = v_rd[cb] + so;
      if constexpr (D == 128) {
        // the V half sits kHalf into each slot: part of the immediate offset
        static_for<TT / 2>([&](auto pc) {
          constexpr int pp = decltype(pc)::value;
          read_v2_128<Gp::kHalf + pp * 16384>(*reinterpret_cast<uint2(*)[2][NCB]>(&vb[2 * pp][0]),
                                              va);
        });
      } else if constexpr (D == 64)
        read_v2_64(vb, va);
      else
        read_v_256(vb[0], va);
    }
    if (t0 + TT * kTile > t_end) {
      // the last trip: V of tokens past the partition (stale slots past a
      // context's end, or the repeated last tile) is zeroed, since a zero
      // weight times a non-finite value would still poison the product
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const int tk = t0 + u * kTile + 4 * lg;
        const unsigned xm = (tk < t_end ? 0xffffu : 0u) | (tk + 1 < t_end ? 0xffff0000u : 0u);
        const unsigned ym = (tk + 2 < t_end ? 0xffffu : 0u) | (tk + 3 < t_end ? 0xffff0000u : 0u);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          vb[u][cb].x &= xm;
          vb[u][cb].y &= ym;
        }
      }
    }

    // O^T += V^T P^T: A operand V[token][dim cb * 16 + ln], B operand
    // P[row ln][token]; lane group lg supplies tokens 4 lg .. 4 lg + 3 of each
    // tile of the trip (the same token order on both sides), and the V read
    // serves all row tiles
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        if constexpr (TT >= 2) {
          // two tiles' tokens per product (k = 32)
#pragma unroll
          for (int u = 0; u < TT; u += 2) {
            const u32x4_t va2 = {vb[u][cb].x, vb[u][cb].y, vb[u + 1][cb].x, vb[u + 1][cb].y};
            const u32x4_t pb2 = {pa[u][r].x, pa[u][r].y, pa[u + 1][r].x, pa[u + 1][r].y};
            o[r][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, va2), __builtin_bit_cast(bf16x8_t, pb2), o[r][cb],
                0, 0, 0);
          }
        } else {
          o[r][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(i16x4_t, vb[0][cb]), __builtin_bit_cast(i16x4_t, pa[0][r]),
              o[r][cb], 0, 0, 0);
        }
      }
  }

  // ---- this wavefront's partials for prefix partition p: row ln of each tile
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float l_row = l_part[r];
    l_row += exact_xor<16>(l_row);
    l_row += exact_xor<32>(l_row);
    if (b_row[r] < 0) continue;
    const size_t pi = qrow[r] * a.num_parts + p;
    float *acc = a.part_acc + pi * D + 4 * lg;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      *reinterpret_cast<float4 *>(acc + cb * 16) =
          make_float4(o[r][cb][0], o[r][cb][1], o[r][cb][2], o[r][cb][3]);
    if (lg == 0) {
      a.part_m[pi] = bad ? nan : m_row[r];
      a.part_l[pi] = l_row;
    }
  }
}

template <int D, int W, int RT>
__global__ void __launch_bounds__(W * 64, W >= 4 ? 2 : 1)
prefix_mfma_kernel(const DecodeArgs a, const ShareArgs s) {
  mfma_rows_body<D, W, RT, RowSource::kSharedGroups>(a, s);
}

// Chunked prefill: grid (KV partitions, Hkv, B x chunks); s carries only
// chunks and prefix_part (the partition length).
template <int D, int W, int RT>
__global__ void __launch_bounds__(W * 64, W >= 4 ? 2 : 1)
chunk_mfma_kernel(const DecodeArgs a, const ShareArgs s) {
  mfma_rows_body<D, W, RT, RowSource::kChunk>(a, s);
}

using PrefixLauncher = void (*)(const DecodeArgs &, const ShareArgs &, dim3, hipStream_t);

// Launcher of the prefix kernel (chunk = false) or the chunk kernel for a
// head dim, W wavefronts per workgroup (1, 2, 4 or 8) and RT row tiles per
// wavefront (1 or 2); nullptr if none. Defined in shared_inst.hip.
PrefixLauncher pick_prefix(int D, int W, int RT, bool chunk = false);

}  // namespace decode
}  // namespace pkv
