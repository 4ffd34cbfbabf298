#pragma once
// Paged attention decode on the matrix cores (gfx950), over bf16 caches and
// over caches of 8-bit or 3-bit per-row codes. Same contract and partials as
// the partition kernel of decode_kernel.h, instantiated in
// decode_inst_mfma_d<D>.hip.
//
// What it computes: attention of each sequence's query rows over its paged
// K/V (vLLM abstract on the papers page "external vector cache"; causal
// visibility of several query tokens: course page "Module 10. KV Caches and
// Efficient Inference", notebook section 2); for code caches every K and V
// element is code * its row's scale -- the reconstruction of that page's
// project demo (Demo 2) quantizer.
//
// Design (for CDNA4; the pages give no kernel): per 16-token tile the VALU
// form spends about 310 (bf16) to 400 (3-bit codes) vector instructions per
// wavefront (widening, dot products, a reduce-scatter, weight broadcasts,
// 128 FMAs), and at 16 lanes per SIMD that costs about as long as the
// tile's HBM traffic. Here both products run on MFMA and the VALU only
// widens codes and runs the softmax:
//   * S^T = K Q^T with v_mfma_f32_16x16x32 (bf16, or f16 for 8-bit codes):
//     A = a token's row (lane l: token l % 16, a quarter of the row; 8-bit
//     codes widened to fp16 in registers), B = the query rows (row l % 16,
//     the same quarter). The output leaves lane l the scores of row l % 16
//     for tokens 4 (l / 16) .. + 3. 3-bit codes are stored as fp4 (e2m1)
//     and enter v_mfma_scale_f32_16x16x128_f8f6f4 as they are read (A, no
//     widening at all); the query is its B operand as two fp8 (e4m3) pieces
//     hi + lo, exact for bf16 queries (mfma_fp4_fp8 gives the k order).
//   * those four weights (times their tokens' V scales for codes) are the
//     B operand of O^T += V^T P^T as they stand. Its A operand (4 tokens x
//     1 dim per lane) comes from the gfx950 transposing LDS reads: for
//     bf16, ds_read_b64_tr_b16 (in each 16-lane group lane i receives
//     element i % 4 of the 4 named by lanes i / 4 + 4 u, u = 0..3); for
//     codes, ds_read_b64_tr_b8 (lane i receives byte i % 8 of the 8 named
//     by lanes i / 8 + 2 u, u = 0..7), so one read gives a lane 4 tokens of
//     two 16-dim column blocks.
//   * bf16 weights are split into bf16 pairs hi + lo and contracted in one
//     16x16x32 product whose k runs over (tokens, hi) then (tokens, lo) with
//     V repeated: 16 significant bits per weight, so results move by no
//     more than fp32 rounding across partitionings. In a context's last
//     tile, V slots past its end (stale bits, maybe NaN) are zeroed.
//   * 8-bit codes widen exactly: (code ^ 0x80) in the low byte of fp16
//     0x64xx is 1152 + code; the offsets are removed once per score
//     (1152 x sum q) and once per output (1152 x the sum of the fp16
//     weights used).
//   * 3-bit codes, two e2m1 nibbles per byte (dim 2 i in the low nibble of
//     byte i): the same tile scheme on rows of D / 2 bytes. V comes from the
//     4-bit transposing read ds_read_b64_tr_b4, arranged so that each byte
//     of the result holds two consecutive tokens of one dim: one
//     v_cvt_scalef32_pk_f16_fp4 per byte gives the A operand as exact fp16,
//     with no rearranging (read_nib_codes).
//   * up to 16 query rows (G x query tokens) per wavefront at no extra MFMA
//     work; the staging, ring, lazy softmax and partials are the partition
//     kernel's. K rows are stored in the LDS ring with their 16-byte chunks
//     permuted per token (chunk c of token t at c ^ (t mod chunks per row))
//     so the per-token reads of the A operand spread over the LDS banks.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "decode_kernel.h"
#include "verify_mfma.h"

namespace pkv {
namespace decode {

typedef _Float16 h16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h16x8_t __attribute__((ext_vector_type(8)));
typedef float c32x4_t __attribute__((ext_vector_type(4)));

// Byte geometry of a tile whose token rows are RB bytes (D for 8-bit codes,
// D / 2 for 3-bit ones).
template <int RB>
struct CodeGeo {
  static constexpr int CPT = RB / 16;   // 16-byte chunks per token row
  static constexpr int TPL = 64 / CPT;  // tokens per 1 KiB load row
  static constexpr int NL = kTile / TPL;  // load rows per half tile
  static constexpr int KCH = CPT / 4;   // K chunks a lane reads (a quarter row)
  static constexpr int NV = RB / 32;    // transposing V reads per tile
  static_assert(CPT >= 4 && CPT <= 16 && NL >= 1, "rows of 64, 128 or 256 bytes");
};

// This lane's byte offset inside a tile's K rows for the gather of load
// row i: lane l fetches chunk (l % CPT) ^ (t % CPT) of token t = i * TPL +
// l / CPT, so that LDS position p of token t holds chunk p ^ (t % CPT).
template <int RB>
__device__ __forceinline__ int code_k_lane_offset(int lane, int i) {
  using Gc = CodeGeo<RB>;
  const int tl = lane / Gc::CPT, t = i * Gc::TPL + tl;
  return i * 1024 + tl * RB + 16 * ((lane % Gc::CPT) ^ (t % Gc::CPT));
}

// This lane's byte offset inside a tile's bf16 V rows for the gather of
// load row i: lane l fetches chunk (l % CPT) ^ (2 t % CPT) of token t =
// i * TPL + l / CPT, so that LDS position p of token t holds chunk
// p ^ (2 t % CPT). The four tokens one transposing read names (rows a
// multiple of the bank width apart) then fall on different banks.
template <int RB>
__device__ __forceinline__ int bf16_v_lane_offset(int lane, int i) {
  using Gc = CodeGeo<RB>;
  const int tl = lane / Gc::CPT, t = i * Gc::TPL + tl;
  return i * 1024 + tl * RB + 16 * ((lane % Gc::CPT) ^ ((2 * t) % Gc::CPT));
}

// One tile's operands from an LDS slot, with one wait for all of them.
// K: this lane's KCH chunks (token l % 16, chunks KCH (l / 16) .. + KCH - 1,
// at LDS offsets ka[c]); V: NV transposing reads at va + 32 j; scales: the
// K and V scales of tokens 4 (l / 16) .. + 3. RB: bytes per token row.
template <int RB>
__device__ __forceinline__ void read_codes(u32x4_t (&k)[CodeGeo<RB>::KCH],
                                           uint2 (&v)[CodeGeo<RB>::NV], float4 &ks,
                                           float4 &vs, const PKV_LDS char *const (&ka)[CodeGeo<RB>::KCH],
                                           const PKV_LDS char *va, const PKV_LDS char *sa);

template <>
__device__ __forceinline__ void read_codes<64>(u32x4_t (&k)[1], uint2 (&v)[2], float4 &ks,
                                               float4 &vs, const PKV_LDS char *const (&ka)[1],
                                               const PKV_LDS char *va, const PKV_LDS char *sa) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b64_tr_b8 %1, %6\n\t"
      "ds_read_b64_tr_b8 %2, %6 offset:32\n\t"
      "ds_read_b128 %3, %7\n\t"
      "ds_read_b128 %4, %7 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(ks), "=&v"(vs)
      : "v"(ka[0]), "v"(va), "v"(sa)
      : "memory");
}

template <>
__device__ __forceinline__ void read_codes<128>(u32x4_t (&k)[2], uint2 (&v)[4], float4 &ks,
                                                float4 &vs, const PKV_LDS char *const (&ka)[2],
                                                const PKV_LDS char *va, const PKV_LDS char *sa) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b64_tr_b8 %2, %10\n\t"
      "ds_read_b64_tr_b8 %3, %10 offset:32\n\t"
      "ds_read_b64_tr_b8 %4, %10 offset:64\n\t"
      "ds_read_b64_tr_b8 %5, %10 offset:96\n\t"
      "ds_read_b128 %6, %11\n\t"
      "ds_read_b128 %7, %11 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]),
        "=&v"(ks), "=&v"(vs)
      : "v"(ka[0]), "v"(ka[1]), "v"(va), "v"(sa)
      : "memory");
}

template <>
__device__ __forceinline__ void read_codes<256>(u32x4_t (&k)[4], uint2 (&v)[8], float4 &ks,
                                                float4 &vs, const PKV_LDS char *const (&ka)[4],
                                                const PKV_LDS char *va, const PKV_LDS char *sa) {
  asm volatile(
      "ds_read_b128 %0, %14\n\t"
      "ds_read_b128 %1, %15\n\t"
      "ds_read_b128 %2, %16\n\t"
      "ds_read_b128 %3, %17\n\t"
      "ds_read_b64_tr_b8 %4, %18\n\t"
      "ds_read_b64_tr_b8 %5, %18 offset:32\n\t"
      "ds_read_b64_tr_b8 %6, %18 offset:64\n\t"
      "ds_read_b64_tr_b8 %7, %18 offset:96\n\t"
      "ds_read_b64_tr_b8 %8, %18 offset:128\n\t"
      "ds_read_b64_tr_b8 %9, %18 offset:160\n\t"
      "ds_read_b64_tr_b8 %10, %18 offset:192\n\t"
      "ds_read_b64_tr_b8 %11, %18 offset:224\n\t"
      "ds_read_b128 %12, %19\n\t"
      "ds_read_b128 %13, %19 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]),
        "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(ks), "=&v"(vs)
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va), "v"(sa)
      : "memory");
}

// 3-bit tiles (rows of RB = D / 2 bytes of e2m1 nibbles): as read_codes, but
// V by 4-bit transposing reads, ds_read_b64_tr_b4. In each 16-lane group
// lane i receives nibble i of the 8-byte word each lane u of the group
// names, at nibble position u (measured on gfx950 with an in-bounds read of
// tagged words). Lane u names token 4 (l / 16) + u % 4 and the 16-dim block
// u / 4 of each 64-dim run (read h: run h, at va + 32 h), so byte 2 b of the
// result holds that lane's dim of block b for tokens 0 and 1 of its four,
// byte 2 b + 1 for tokens 2 and 3.
template <int RB>
__device__ __forceinline__ void read_nib_codes(u32x4_t (&k)[CodeGeo<RB>::KCH],
                                               uint2 (&v)[CodeGeo<RB>::NV], float4 &ks,
                                               float4 &vs,
                                               const PKV_LDS char *const (&ka)[CodeGeo<RB>::KCH],
                                               const PKV_LDS char *va, const PKV_LDS char *sa);

template <>
__device__ __forceinline__ void read_nib_codes<64>(u32x4_t (&k)[1], uint2 (&v)[2], float4 &ks,
                                                   float4 &vs, const PKV_LDS char *const (&ka)[1],
                                                   const PKV_LDS char *va,
                                                   const PKV_LDS char *sa) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b64_tr_b4 %1, %6\n\t"
      "ds_read_b64_tr_b4 %2, %6 offset:32\n\t"
      "ds_read_b128 %3, %7\n\t"
      "ds_read_b128 %4, %7 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(ks), "=&v"(vs)
      : "v"(ka[0]), "v"(va), "v"(sa)
      : "memory");
}

template <>
__device__ __forceinline__ void read_nib_codes<128>(u32x4_t (&k)[2], uint2 (&v)[4], float4 &ks,
                                                    float4 &vs, const PKV_LDS char *const (&ka)[2],
                                                    const PKV_LDS char *va,
                                                    const PKV_LDS char *sa) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b64_tr_b4 %2, %10\n\t"
      "ds_read_b64_tr_b4 %3, %10 offset:32\n\t"
      "ds_read_b64_tr_b4 %4, %10 offset:64\n\t"
      "ds_read_b64_tr_b4 %5, %10 offset:96\n\t"
      "ds_read_b128 %6, %11\n\t"
      "ds_read_b128 %7, %11 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]),
        "=&v"(ks), "=&v"(vs)
      : "v"(ka[0]), "v"(ka[1]), "v"(va), "v"(sa)
      : "memory");
}

// bf16 tiles: KCH K chunks (as for codes) and D / 16 transposing 16-bit V
// reads, column block cb at va[cb] (ds_read_b64_tr_b16: in each 16-lane
// group lane i receives element i % 4 of the 4 named by lanes i / 4 + 4 u,
// u = 0..3).
template <int RB>
__device__ __forceinline__ void read_bf16(u32x4_t (&k)[CodeGeo<RB>::KCH],
                                          uint2 (&v)[RB / 32],
                                          const PKV_LDS char *const (&ka)[CodeGeo<RB>::KCH],
                                          const PKV_LDS char *const (&va)[RB / 32]);

template <>
__device__ __forceinline__ void read_bf16<128>(u32x4_t (&k)[2], uint2 (&v)[4],
                                               const PKV_LDS char *const (&ka)[2],
                                               const PKV_LDS char *const (&va)[4]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b64_tr_b16 %2, %8\n\t"
      "ds_read_b64_tr_b16 %3, %9\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(ka[0]), "v"(ka[1]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])
      : "memory");
}

template <>
__device__ __forceinline__ void read_bf16<256>(u32x4_t (&k)[4], uint2 (&v)[8],
                                               const PKV_LDS char *const (&ka)[4],
                                               const PKV_LDS char *const (&va)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\t"
      "ds_read_b64_tr_b16 %5, %17\n\t"
      "ds_read_b64_tr_b16 %6, %18\n\t"
      "ds_read_b64_tr_b16 %7, %19\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %21\n\t"
      "ds_read_b64_tr_b16 %10, %22\n\t"
      "ds_read_b64_tr_b16 %11, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]),
        "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
        "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
      : "memory");
}

// Four int8 codes (one word) as four fp16 values 1152 + code.
__device__ __forceinline__ uint2 codes_f16x4(uint32_t w) {
  return make_uint2(codes_f16_lo(w), codes_f16_hi(w));
}
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// S^T += K Q^T over 128 dims with 3-bit codes: A = 32 fp4 (e2m1) codes per
// lane as stored (u32x4), B = 32 fp8 (e4m3) query values per lane, block
// scales 1 (E8M0 127); row (A) and column (B) = lane % 16. The products'
// k index as measured on gfx950: lane group g of A holds k = 32 g + i in
// its nibble i (even i in the low nibble of a byte); lane group g of B holds
// k = 16 g + j in its byte j < 16 and k = 64 + 16 g + (j - 16) in byte
// j >= 16.
__device__ __forceinline__ c32x4_t mfma_fp4_fp8(u32x4_t a, const uint32_t (&b)[8], c32x4_t c) {
  const i32x8_t av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8_t bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3],
                      (int)b[4], (int)b[5], (int)b[6], (int)b[7]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 0, 0, 127, 0, 127);
}

// a * b, except that the result is 0 whenever a or b is 0, even against an
// infinite or NaN other factor (the rule of v_mul_legacy_f32); otherwise the
// ordinary rounded product. The compiler's hazard checks do not look into
// inline assembly, and `a` is a v_exp_f32 result here: a vector read of a
// transcendental's result needs one wait state, hence the s_nop.
__device__ __forceinline__ float mul_zero_wins(float a, float b) {
  float r;
  asm("s_nop 0\n\tv_mul_legacy_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Four fp32 values as the low (word_hi false) or high half of fp8 (e4m3,
// round to nearest even) bytes 0..3 of a word.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}

// K/V rows in flight per wavefront: 4 KiB, at least one tile (two 3-bit
// tiles at D = 128, one 8-bit or bf16 tile). Random 16-token tiles of a
// paged cache came back faster with fewer of them outstanding: per call on
// the 8K batch, 3-bit codes 55.1 us at 16 KiB, 53.4 at 8, 51.1 at 4, 60 at
// 2; 8-bit codes 93.0 / 90.1 / 89.3; the 128K split-K call 339.5 us at
// 16 KiB, 326.8 at 4; bf16 the same at one tile as at two.
constexpr int kMfmaRingBudget = 4096;

template <int DT, int D, int RW, int kWaves, bool kStream>
__global__ void __launch_bounds__(kWaves * 64)
decode_mfma_kernel(const DecodeArgs a, const StreamArgs sa) {
  constexpr bool kNib = DT == kCodes3;
  constexpr bool kBf = DT == PKV_BF16;  // bf16 K/V: no codes, no scales
  constexpr int RB = kBf ? 2 * D : kNib ? D / 2 : D;  // bytes per token row
  using Gc = CodeGeo<RB>;
  constexpr int NL = Gc::NL, KCH = Gc::KCH, NV = Gc::NV;
  constexpr int NC = D / 32;   // q.k MFMAs per tile (32 dims each)
  constexpr int NCB = D / 16;  // 16-dim output column blocks
  constexpr float kOffset = DT == PKV_I8 ? 1152.f : 0.f;  // fp16 form = offset + code
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  constexpr int kStride = kWaves * kTile;  // tokens between a wavefront's tiles
  using Ring = TileRing<NL, !kBf, kMfmaRingBudget>;
  constexpr int kSlots = Ring::kSlots;
  static_assert(DT == PKV_BF16 || DT == PKV_I8 || DT == kCodes3, "bf16, 8-bit or 3-bit codes");
  static_assert(!kBf || NV == NCB, "one transposing read per bf16 column block");
  static_assert(RW == 4 || RW == 8 || RW == 16, "rows per wavefront");
  static_assert(!kStream || kWaves == 8, "stream mode: eight wavefronts per workgroup");

  struct Merge {
    float acc[kWaves][RW][D];
    float m[kWaves][RW];
    float l[kWaves][RW];
    int bad[kWaves];
  };
  __shared__ union {
    u32x4_t ring[kWaves * Ring::kBytes / 16];
    Merge mg;
  } sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lg = lane >> 4;  // MFMA column (query row) and lane group
  // Independent wavefronts (parts_per_wg > 0): wavefront w of workgroup x
  // streams the run of parts_per_wg consecutive partitions from
  // p = (x W + w) ppw on as one softmax state and writes it itself as the
  // partial of partition p; the reduce reads only the runs' first slots. No
  // store is issued while tiles are in flight (stores count in vmcnt too,
  // and would make the ring's counted waits drain it). Else the
  // workgroup's wavefronts interleave the tiles of partition p = x and
  // merge in LDS.
  //
  // Stream mode (kStream): the stream decomposition of the VALU stream
  // kernel on the matrix cores. The (sequence, KV head) units are laid end
  // to end as one stream of slots: unit u = b Hkv + g holds c = sa.seg_cost
  // slots without work (what starting a segment costs, in tile times)
  // followed by its ceil(L_b / 16) tiles; wavefront w of the N =
  // sa.n_waves takes slots [w T / N, (w + 1) T / N): equal costs whatever
  // the lengths (with c = 0 a wavefront over many short units would start
  // many segments and finish last). Its range is cut into segments at unit
  // boundaries; each segment runs as an independent run (q set-up, ring,
  // softmax state) and leaves its unnormalised partials under id w + u, RW
  // rows each, for reduce_stream_kernel. A segment's partial is stored only
  // once its last tile has been consumed, so no store overlaps gathers in
  // flight.
  const bool indep = kStream || a.parts_per_wg > 0;
  const int nq = a.nq, G = a.Hq / a.Hkv;
  const int max_ctx = a.max_blocks * a.bs;

  int64_t spos = 0, send = 0;  // stream: this wavefront's slot range
  // the unit at hand: sequence, KV head, slots per unit of the sequence
  // (c + its tiles), the sequence's length, the unit's first slot
  int cur_b = 0, cur_g = 0, cur_span = 0, cur_L = 0;
  int64_t cur_us = 0;
  int64_t stream_w = 0;
  const int seg_cost = kStream ? sa.seg_cost : 0;
  auto unit_span = [&](int len) {
    const int nt = seq_tiles(len, nq, max_ctx);
    return nt > 0 ? nt + seg_cost : 0;
  };
  if constexpr (kStream) {
    // slots per unit of each sequence, prefix over sequences, in LDS (the
    // ring's space, before any tile is staged); workgroup 0 also leaves it
    // for the reduce
    int *tp = reinterpret_cast<int *>(&sm.ring[0]);  // [B + 1]
    int *scan = tp + a.B + 1;                        // [kWaves * 64]
    constexpr int kThreads = kWaves * 64;
    const int B = a.B, tid = threadIdx.x;
    const int per = (B + kThreads - 1) / kThreads;
    const int lo = min(B, tid * per), hi = min(B, lo + per);
    int own = 0;
    for (int bb = lo; bb < hi; ++bb) own += unit_span(load_const(a.lens + bb));
    scan[tid] = own;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    int run_tot = scan[tid] - own;
    for (int bb = lo; bb < hi; ++bb) {
      tp[bb] = run_tot;
      run_tot += unit_span(load_const(a.lens + bb));
    }
    if (tid == kThreads - 1) tp[B] = scan[kThreads - 1];
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = tid; i <= B; i += kThreads) sa.tile_pre[i] = tp[i];
    const int HU = a.Hkv;
    const int64_t T = (int64_t)__builtin_amdgcn_readfirstlane(tp[B]) * HU;
    const int64_t N = sa.n_waves;
    stream_w = (int64_t)blockIdx.x * kWaves + wave;
    spos = stream_w * T / N;
    send = (stream_w + 1) * T / N;
    if (spos < send) {  // the unit holding slot spos: HU tp[lo] <= spos < HU tp[lo + 1]
      int l0 = 0, h0 = B;
      while (h0 - l0 > 1) {
        const int mid = (l0 + h0) >> 1;
        if ((int64_t)__builtin_amdgcn_readfirstlane(tp[mid]) * HU <= spos) l0 = mid; else h0 = mid;
      }
      const int pre = __builtin_amdgcn_readfirstlane(tp[l0]);
      cur_b = l0;
      cur_span = __builtin_amdgcn_readfirstlane(tp[l0 + 1]) - pre;
      const int64_t local = spos - (int64_t)pre * HU;
      cur_g = (int)(local / cur_span);
      cur_us = (int64_t)pre * HU + (int64_t)cur_g * cur_span;
      cur_L = load_const(a.lens + l0);
    }
    __syncthreads();  // the prefix is read: the ring's space is free again
  }

  // stream mode: the next unit of the stream (past this sequence's units,
  // the next sequence with tiles); false past the last one
  auto next_unit = [&]() {
    cur_us += cur_span;
    if (++cur_g < a.Hkv) return true;
    cur_g = 0;
    do {
      if (++cur_b >= a.B) return false;
      cur_L = load_const(a.lens + cur_b);
      cur_span = unit_span(cur_L);
    } while (cur_span == 0);
    return true;
  };

  for (;;) {  // one pass, or one pass per segment in stream mode
    int seg_tiles = 0;  // stream: tiles of this segment
    int ppw, p, b, g, row0, L, t_begin, t_end;
    if constexpr (kStream) {
      // this range's part of the unit's tiles (none if it holds only the
      // unit's cost slots)
      int64_t lo_s, hi_s;
      for (;;) {
        if (spos >= send || cur_us >= send) return;
        lo_s = max(spos, cur_us + seg_cost);
        hi_s = min(send, cur_us + cur_span);
        if (hi_s > lo_s) break;
        if (cur_us + cur_span >= send || !next_unit()) return;
      }
      seg_tiles = (int)(hi_s - lo_s);
      const int k0 = (int)(lo_s - cur_us - seg_cost);
      ppw = 1;
      p = 0;
      b = cur_b;
      g = cur_g;
      row0 = 0;
      L = cur_L;
      t_begin = k0 * kTile;
      t_end = min(L, (k0 + seg_tiles) * kTile);
    } else {
      ppw = indep ? a.parts_per_wg : 1;
      p = indep ? ((int)blockIdx.x * kWaves + wave) * ppw : (int)blockIdx.x;
      b = blockIdx.z;
      g = blockIdx.y % a.Hkv;
      row0 = (blockIdx.y / a.Hkv) * RW;
      L = load_const(a.lens + b);

      if (L < nq || L > max_ctx) {  // a row would see no key, or the table is too short
        if (a.num_parts == 1 && p == 0) {
          const float nan = __builtin_nanf("");
          for (int idx = threadIdx.x; idx < RW * D; idx += kWaves * 64) {
            const int r = row0 + idx / D, d = idx % D, qi = r / G;
            if (qi >= nq) continue;
            const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (r % G);
            a.out[row * D + d] = nan;
            if (d == 0 && a.lse) a.lse[row] = nan;
          }
        }
        return;  // with partitions, the reduce kernel writes the NaN rows
      }
      t_begin = p * a.part_tokens;
      if (t_begin >= L) return;  // past this sequence's end: the reduce reads nothing here
      t_end = min(L, t_begin + ppw * a.part_tokens);
    }

    // this wavefront's tiles of [t_begin, t_end), and lane i's block id of
    // its tile i, loaded ahead of the query so that the two loads' latencies
    // overlap instead of adding up
    const int wstart = indep ? t_begin : t_begin + wave * kTile;  // this wavefront's first tile
    const int wstride = indep ? kTile : kStride;                   // and the step between its tiles
    const int n_tiles = wstart < t_end ? (t_end - wstart + wstride - 1) / wstride : 0;
    auto tile_t0 = [&](int k) { return wstart + k * wstride; };
    const int32_t *trow = a.tables + (size_t)b * a.max_blocks;
    auto table_window = [&](int w) {
      return trow[tile_t0(min(64 * w + lane, n_tiles - 1)) / a.bs];
    };
    const int tblv0 = n_tiles > 0 ? table_window(0) : 0;

    // ---- this lane's query row ln as the B operand of the q.k MFMAs: the
    //      lane's quarter of the dims (lg * D / 4 ..), 8 per MFMA; bf16 as is
    //      for bf16 K, else fp16 in the order the K codes widen, scaled by 2^-e
    //      so that the row's largest entry is in [2^7, 2^8) (fp16 keeps 11
    //      bits) ---------------------------------------------------------------
    const int rr = row0 + ln, qi = rr / G;
    const bool row_live = ln < RW && qi < nq;
    uint32_t qb[NC][4];
    uint32_t qp[KCH][2][8];  // 3-bit codes: the query as fp8 pieces hi + lo
    float qcorr, qfac;
    int lim;  // keys visible to row ln
    if constexpr (kNib) {
      // B operand of the fp4 x fp8 products: for product c (the lane's K
      // chunk c), byte j of this lane's 32 is dim 32 (KCH (2 (j / 16) +
      // lg / 2) + c) + 16 (lg % 2) + j % 16 -- the dim that the fp4 code it
      // meets belongs to. Each dim scaled by 2^-e (the row's largest entry
      // in [2^7, 2^8)) and split into e4m3 pieces hi = rne(x), lo = rne(x -
      // hi): a bf16 value has 8 significant bits and e4m3 4, so hi + lo is
      // x exactly unless x sits more than 10 binades below the row maximum
      // (then within 2^-10 absolute, 2^-18 of the maximum).
      float x[KCH][2][16];
      if (row_live) {
        const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (rr % G);
        const uint16_t *qrow = (const uint16_t *)a.q + row * D;
#pragma unroll
        for (int c = 0; c < KCH; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint4 *src = reinterpret_cast<const uint4 *>(
                qrow + 32 * (KCH * (2 * h + lg / 2) + c) + 16 * (lg % 2));
            const uint4 t[2] = {src[0], src[1]};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const uint32_t wv[4] = {t[u].x, t[u].y, t[u].z, t[u].w};
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                x[c][h][8 * u + 2 * v] = bf16_lo(wv[v]);
                x[c][h][8 * u + 2 * v + 1] = bf16_hi(wv[v]);
              }
            }
          }
      } else {
#pragma unroll
        for (int c = 0; c < KCH; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 16; ++t) x[c][h][t] = 0.f;
      }
      // a negative scale moves into the query (negation is exact), so that
      // the factor qfac below is positive
      if (a.scale_log2 < 0.f) {
#pragma unroll
        for (int c = 0; c < KCH; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 16; ++t) x[c][h][t] = -x[c][h][t];
      }
      float mx = 0.f;
#pragma unroll
      for (int c = 0; c < KCH; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < 16; ++t) mx = fmaxf(mx, fabsf(x[c][h][t]));
      mx = fmaxf(mx, exact_xor<16>(mx));
      mx = fmaxf(mx, exact_xor<32>(mx));
      int ex = 0;
      frexpf(mx, &ex);
      const int e = mx == 0.f ? 0 : ex - 8;
#pragma unroll
      for (int c = 0; c < KCH; ++c)
#pragma unroll
        for (int m = 0; m < 8; ++m) {  // word m: bytes 4 m .. 4 m + 3
          const float *xs = &x[c][m / 4][4 * (m % 4)];
          const float v0 = ldexpf(xs[0], -e), v1 = ldexpf(xs[1], -e);
          const float v2 = ldexpf(xs[2], -e), v3 = ldexpf(xs[3], -e);
          const uint32_t hw = fp8x4(v0, v1, v2, v3);
          const f32x2_t d01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hw, false);
          const f32x2_t d23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hw, true);
          qp[c][0][m] = hw;
          qp[c][1][m] = fp8x4(v0 - d01.x, v1 - d01.y, v2 - d23.x, v3 - d23.y);
        }
      qcorr = 0.f;
      // at least 1e-30: a masked raw score (-inf) times it stays -inf, and
      // with scale 0 every visible weight is still exp2(0) = 1
      qfac = fmaxf(ldexpf(1.f, e) * fabsf(a.scale_log2), 1e-30f);
      lim = row_live ? L - nq + qi + 1 : 0;
    } else {
      uint32_t w[D / 8];  // bf16 pairs: dims 2 j, 2 j + 1 of the quarter
      if (row_live) {
        const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (rr % G);
        const uint4 *src =
            reinterpret_cast<const uint4 *>((const uint16_t *)a.q + row * D + lg * (D / 4));
#pragma unroll
        for (int j = 0; j < D / 32; ++j) {
          const uint4 t = src[j];
          w[4 * j] = t.x; w[4 * j + 1] = t.y; w[4 * j + 2] = t.z; w[4 * j + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < D / 8; ++j) w[j] = 0u;
      }
      auto qdim = [&](int d) { return d % 2 ? bf16_hi(w[d / 2]) : bf16_lo(w[d / 2]); };
      // a negative scale moves into the query (negation is exact), so that
      // the factor qfac below is positive
      const bool neg = a.scale_log2 < 0.f;
      if constexpr (kBf) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j) qb[c][j] = w[4 * c + j] ^ (neg ? 0x80008000u : 0u);
      }
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < D / 8; ++j)
        mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
      mx = fmaxf(mx, exact_xor<16>(mx));
      mx = fmaxf(mx, exact_xor<32>(mx));
      int ex = 0;
      frexpf(mx, &ex);
      const int e = kBf || mx == 0.f ? 0 : ex - 8;
      float sum = 0.f;
#pragma unroll
      for (int c = 0; c < NC && !kBf; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // MFMA c, k = 2 j, 2 j + 1: dims 8 c + (2 j, 2 j + 1)
          const int d0 = 8 * c + 2 * j, d1 = d0 + 1;
          const float sg = neg ? -1.f : 1.f;
          const _Float16 lo = (_Float16)(sg * ldexpf(qdim(d0), -e));
          const _Float16 hi = (_Float16)(sg * ldexpf(qdim(d1), -e));
          sum += (float)lo + (float)hi;
          qb[c][j] = __builtin_bit_cast(uint32_t, f16x2_t{lo, hi});
        }
      sum += exact_xor<16>(sum);
      sum += exact_xor<32>(sum);
      qcorr = kOffset * sum;
      qfac = fmaxf(ldexpf(1.f, e) * fabsf(a.scale_log2), 1e-30f);  // as above
      lim = row_live ? L - nq + qi + 1 : 0;
    }

    const char *kbase = (const char *)a.kc;
    const char *vbase = (const char *)a.vc;
    int koff[NL], voff[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      koff[i] = code_k_lane_offset<RB>(lane, i);
      voff[i] = kBf ? bf16_v_lane_offset<RB>(lane, i) : i * 1024 + lane * 16;
    }
    // scales: lanes 0-15 the K rows' of the tile's 16 tokens, lanes 16-31 the
    // V rows' (lanes 32-63 repeat them), one contiguous run per (block, head)
    const int32_t soff = (lane & 16 ? a.bs : 0) + (lane & 15);
    int bad = 0;
    // gather the tile at logical token t0 (from block blk) into a ring slot,
    // in TileRing::stage's order: the scales (codes), the K rows (chunks
    // permuted per token), the V rows
    auto stage_tile = [&](Ring &ring, int slot, int t0, int blk) {
      if (blk < 0 || blk >= a.num_blocks) {  // bad table entry: read block 0, poison later
        bad = 1;
        blk = 0;
      }
      const size_t rowi = ((size_t)blk * a.Hkv + g) * a.bs + (size_t)(t0 % a.bs);
      PKV_LDS char *dst = ring.base + slot * Ring::kTileBytes;
      if constexpr (!kBf) {
        const size_t srow = ((size_t)blk * a.Hkv + g) * 2 * a.bs + (size_t)(t0 % a.bs);
        gather_lds4<kKvNonTemporal>((const char *)(a.scales + srow + soff),
                                    dst + Ring::kCodeBytes);
      }
      const char *kp = kbase + rowi * RB, *vp = vbase + rowi * RB;
#pragma unroll
      for (int i = 0; i < NL; ++i) gather_lds16<kKvNonTemporal>(kp + koff[i], dst + i * 1024);
#pragma unroll
      for (int i = 0; i < NL; ++i)
        gather_lds16<kKvNonTemporal>(vp + voff[i], dst + (NL + i) * 1024);
    };


    // O^T accumulators, offsets included: o[cb][e] = O^T[m = 4 lg + e][row ln]
    // of column block cb (8-bit: dim 16 cb + m; 3-bit: see the merge below)
    c32x4_t o[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = c32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_row = kNegInf, l_part = 0.f, w_part = 0.f;
    // the raw score (before the factor qfac > 0) past which the running
    // maximum is raised: (m_row + kLazyLog2) / qfac
    const float rqfac = 1.f / qfac;
    float thr = kNegInf;

    // The partial of partition pp, or in stream mode of segment id pp,
    // straight from the registers (independent wavefronts).
    auto flush = [&](int64_t pp) {
      float lt = l_part, wt = w_part;
      lt += exact_xor<16>(lt);
      lt += exact_xor<32>(lt);
      wt += exact_xor<16>(wt);
      wt += exact_xor<32>(wt);
      const float off = -kOffset * wt;
      if (row_live) {
        const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (rr % G);
        const size_t pi = kStream ? (size_t)pp * RW + ln : row * a.num_parts + a.part_base + pp;
        float *dst = a.part_acc + pi * D;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          *reinterpret_cast<float4 *>(dst + 16 * cb + 4 * lg) =
              make_float4(o[cb][0] + off, o[cb][1] + off, o[cb][2] + off, o[cb][3] + off);
        if (lg == 0) {
          a.part_m[pi] = bad ? __builtin_nanf("") : m_row;
          a.part_l[pi] = lt;
        }
      }
    };

    if (n_tiles > 0) {
      int tblv = tblv0;
      settle_v(tblv);
      auto table_at = [&](int k) { return __builtin_amdgcn_readlane(tblv, k & 63); };
      Ring ring;
      PKV_LDS char *ring_base = (PKV_LDS char *)&sm.ring[0] + wave * Ring::kBytes;
      ring.init(ring_base, lane);
      // read-back addresses inside slot 0 (a slot adds slot * kTileBytes)
      const PKV_LDS char *ka[KCH];
      {
        const int t = ln, tl = t % Gc::TPL;
        const PKV_LDS char *row = ring_base + (t / Gc::TPL) * 1024 + tl * RB;
#pragma unroll
        for (int c = 0; c < KCH; ++c) ka[c] = row + 16 * ((KCH * lg + c) ^ (t % Gc::CPT));
      }
      // V, codes: lane s of group lg names token 4 lg + (s / 2) % 4, bytes
      // 16 ((s / 2) / 4) + 8 (s % 2) .. + 7 of each 32-byte column pair; bf16:
      // token 4 lg + s / 4, dims 4 (s % 4) .. + 3 of each 16-dim column block
      // cb (bytes 32 cb + 8 (s % 4), whose 16-byte chunk c sits at position
      // c ^ (2 t % CPT)), one address per column block
      const PKV_LDS char *va;
      const PKV_LDS char *vab[Gc::NV];
      {
        // 3-bit: lane s names token 4 lg + s % 4, the 8-byte word s / 4 of
        // each 32-byte run (read_nib_codes)
        const int u = kBf ? ln >> 2 : kNib ? ln : ln >> 1, t = 4 * lg + (u & 3);
        const int col = kBf ? 8 * (ln & 3) : kNib ? 8 * (ln >> 2) : 16 * (u >> 2) + 8 * (ln & 1);
        const PKV_LDS char *row =
            ring_base + NL * 1024 + (t / Gc::TPL) * 1024 + (t % Gc::TPL) * RB;
        va = row + col;
#pragma unroll
        for (int cb = 0; cb < Gc::NV; ++cb) {
          const int c = 2 * cb + ((ln >> 1) & 1);
          vab[cb] = row + 16 * (c ^ ((2 * t) % Gc::CPT)) + 8 * (ln & 1);
        }
      }
      const PKV_LDS char *sa = ring_base + Ring::kCodeBytes + 16 * lg;
#pragma unroll
      for (int k = 0; k < kSlots; ++k)
        if (k < n_tiles) stage_tile(ring, k, tile_t0(k), table_at(k));
      const uint32_t ones = __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)1.f, (_Float16)1.f});

      for (int k = 0; k < n_tiles; ++k) {
        const int slot = k & (kSlots - 1);
        const int ahead = min(n_tiles - 1 - k, kSlots - 1);
        wait_ahead<kSlots, Ring::kLoads>(k + kSlots <= n_tiles, ahead);
        u32x4_t kr[KCH];
        uint2 vt[NV];
        float4 ksc = make_float4(1.f, 1.f, 1.f, 1.f), vsc = ksc;
        {
          const int so = slot * Ring::kTileBytes;
          const PKV_LDS char *kas[KCH];
#pragma unroll
          for (int c = 0; c < KCH; ++c) kas[c] = ka[c] + so;
          if constexpr (kBf) {
            const PKV_LDS char *vas[Gc::NV];
#pragma unroll
            for (int cb = 0; cb < Gc::NV; ++cb) vas[cb] = vab[cb] + so;
            read_bf16<RB>(kr, vt, kas, vas);
          } else
            if constexpr (kNib)
              read_nib_codes<RB>(kr, vt, ksc, vsc, kas, va + so, sa + so);
            else
              read_codes<RB>(kr, vt, ksc, vsc, kas, va + so, sa + so);
        }
        if (k + kSlots < n_tiles) {  // the slot is free again: refill it
          const int kn = k + kSlots;
          if ((kn & 63) == 0) {  // next window of block ids (drains the ring once)
            tblv = table_window(kn >> 6);
            settle_v(tblv);
          }
          stage_tile(ring, slot, tile_t0(kn), table_at(kn));
        }

        // S^T = K Q^T: s[e] = row ln . token 4 lg + e (codes with offsets)
        c32x4_t s = c32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (kNib) {  // the fp4 codes as stored, the query's fp8 pieces
#pragma unroll
          for (int c = 0; c < KCH; ++c) {
            s = mfma_fp4_fp8(kr[c], qp[c][0], s);
            s = mfma_fp4_fp8(kr[c], qp[c][1], s);
          }
        }
#pragma unroll
        for (int c = 0; c < NC && !kNib; ++c) {
          if constexpr (kBf) {
            const u32x4_t bv = {qb[c][0], qb[c][1], qb[c][2], qb[c][3]};
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[c]),
                                                        __builtin_bit_cast(bf16x8_t, bv), s, 0, 0,
                                                        0);
            continue;
          }
          u32x4_t av;
          {  // two words: 8 dims in order
            const u32x4_t kw = kr[c / 2];
            const uint2 lo = codes_f16x4(kw[2 * (c % 2)]), hi = codes_f16x4(kw[2 * (c % 2) + 1]);
            av = u32x4_t{lo.x, lo.y, hi.x, hi.y};
          }
          const u32x4_t bv = {qb[c][0], qb[c][1], qb[c][2], qb[c][3]};
          s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8_t, av),
                                                     __builtin_bit_cast(h16x8_t, bv), s, 0, 0, 0);
        }
        const int t0 = tile_t0(k);
        const float kss[4] = {ksc.x, ksc.y, ksc.z, ksc.w};
        const float vss[4] = {vsc.x, vsc.y, vsc.z, vsc.w};
        // raw scores rs = score / qfac: the maximum test against thr, the
        // scaling inside the exponent's fma
        float rs[4];
        bool need = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = t0 + 4 * lg + e < lim;
          const float sq = kOffset != 0.f ? s[e] - qcorr : s[e];
          rs[e] = vis ? (kBf ? s[e] : sq * kss[e]) : kNegInf;
          need |= rs[e] > thr;
        }
        if (__any(need)) {  // raise the running maximum of row ln
          float tmax = fmaxf(fmaxf(rs[0], rs[1]), fmaxf(rs[2], rs[3]));
          tmax = fmaxf(tmax, exact_xor<16>(tmax));
          tmax = fmaxf(tmax, exact_xor<32>(tmax)) * qfac;
          const float mn = fmaxf(m_row, tmax);
          const float alpha = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_row - mn);
          m_row = mn;
          thr = (mn + kLazyLog2) * rqfac;
          l_part *= alpha;
          w_part *= alpha;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
        }
        // exp2(-inf) = 0 for masked scores; the maximum is floored so that a
        // row with no visible key yet gives 0, not NaN
        const float m_sub = fmaxf(m_row, -3.0e38f);
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pw = __builtin_amdgcn_exp2f(fmaf(rs[e], qfac, -m_sub));  // 0 when masked
          l_part += pw;
          // the V scale of a masked token may be stale (even NaN): its zero
          // weight wins the product
          pv[e] = kBf ? pw : mul_zero_wins(pw, vss[e]);
        }
        if constexpr (kBf) {
          // O^T += V^T P^T with bf16 weights; in a context's last tile the
          // slots past it may hold stale bits (even NaN), zeroed so that a
          // zero weight times NaN cannot reach the accumulators
          if (t0 + kTile > L) {  // wavefront-uniform
            const int tv = t0 + 4 * lg;
            const uint32_t m01 = (tv < L ? 0xffffu : 0u) | (tv + 1 < L ? 0xffff0000u : 0u);
            const uint32_t m23 = (tv + 2 < L ? 0xffffu : 0u) | (tv + 3 < L ? 0xffff0000u : 0u);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
              vt[j].x &= m01;
              vt[j].y &= m23;
            }
          }
          // each weight as a bf16 pair hi + lo (16 significant bits): one
          // 16x16x32 product over k = (tokens, hi) then (tokens, lo), V
          // repeated along k, so the weights lose no more than fp32 rounding
          // would across partitionings
          const uint32_t h01 = pack_bf16(pv[0], pv[1]), h23 = pack_bf16(pv[2], pv[3]);
          const uint32_t l01 = pack_bf16(pv[0] - bf16_lo(h01), pv[1] - bf16_hi(h01));
          const uint32_t l23 = pack_bf16(pv[2] - bf16_lo(h23), pv[3] - bf16_hi(h23));
          const u32x4_t pb2 = {h01, h23, l01, l23};
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const u32x4_t va2 = {vt[cb].x, vt[cb].y, vt[cb].x, vt[cb].y};
            o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va2),
                                                            __builtin_bit_cast(bf16x8_t, pb2),
                                                            o[cb], 0, 0, 0);
          }
          continue;
        }
        const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[0], pv[1]));
        const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[2], pv[3]));
        // the fp16 weights' sum: what the V offsets add, removed at the end
        if constexpr (DT == PKV_I8) w_part = dot2_f16(p01, ones, dot2_f16(p23, ones, w_part));
        const h16x4_t pb = __builtin_bit_cast(h16x4_t, make_uint2(p01, p23));

        // O^T += V^T P^T: A = V[tokens 4 lg .. + 3][one dim per lane]
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          if constexpr (kNib) {  // read j: 16-dim blocks 4 j .. 4 j + 3
            const uint32_t xy[2] = {vt[j].x, vt[j].y};
            static_for<4>([&](auto bc) {
              // bytes 2 bb and 2 bb + 1 of the read: tokens (0, 1) and (2, 3)
              // of this lane's four, its dim of block 4 j + bb, exact fp16
              constexpr int bb = decltype(bc)::value;
              const uint32_t w = xy[bb >> 1];
              const f16x2_t c01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.f, 2 * (bb & 1));
              const f16x2_t c23 =
                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.f, 2 * (bb & 1) + 1);
              const h16x4_t av = {c01.x, c01.y, c23.x, c23.y};
              o[4 * j + bb] =
                  __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb, o[4 * j + bb], 0, 0, 0);
            });
          } else {  // dims 32 j + ln and 32 j + 16 + ln
            o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                __builtin_bit_cast(h16x4_t, codes_f16x4(vt[j].x)), pb, o[2 * j], 0, 0, 0);
            o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                __builtin_bit_cast(h16x4_t, codes_f16x4(vt[j].y)), pb, o[2 * j + 1], 0, 0, 0);
          }
        }
      }
    }

    if constexpr (kStream) {
      flush(stream_w + (int64_t)b * a.Hkv + g);
      // the range ends in this unit, or goes on with the next one
      if (cur_us + cur_span >= send || !next_unit()) return;
      continue;
    }
    if (indep) {
      flush(p);
      return;
    }

    // ---- wavefront totals: row ln's weight sums over the four lane groups,
    //      the V offsets removed, then the merge of the wavefronts in LDS -----
    l_part += exact_xor<16>(l_part);
    l_part += exact_xor<32>(l_part);
    w_part += exact_xor<16>(w_part);
    w_part += exact_xor<32>(w_part);
    const float off = -kOffset * w_part;
    __syncthreads();  // the partials overwrite the other wavefronts' rings
    if (ln < RW) {
      float *dst = sm.mg.acc[wave][ln];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        *reinterpret_cast<float4 *>(dst + 16 * cb + 4 * lg) =
            make_float4(o[cb][0] + off, o[cb][1] + off, o[cb][2] + off, o[cb][3] + off);
      if (lg == 0) {
        sm.mg.m[wave][ln] = m_row;
        sm.mg.l[wave][ln] = l_part;
      }
    }
    bad = __builtin_amdgcn_readfirstlane(bad);
    if (lane == 0) sm.mg.bad[wave] = bad;
    __syncthreads();

    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any_bad |= sm.mg.bad[w];
    const float nan = __builtin_nanf("");
    for (int idx = threadIdx.x; idx < RW * D; idx += kWaves * 64) {
      const int r = idx / D, d = idx % D, rrow = row0 + r, qr = rrow / G;
      if (qr >= nq) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.mg.m[w][r]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.mg.m[w][r];
        const float f = mw == kNegInf ? 0.f : exp2f(mw - M);
        num = fmaf(f, sm.mg.acc[w][r][d], num);
        den = fmaf(f, sm.mg.l[w][r], den);
      }
      const size_t row = ((size_t)b * nq + qr) * a.Hq + g * G + (rrow % G);
      if (a.num_parts == 1) {
        a.out[row * D + d] = any_bad || den == 0.f ? nan : num / den;
        if (d == 0 && a.lse) a.lse[row] = any_bad || den == 0.f ? nan : (M + log2f(den)) * kLn2;
      } else {
        const size_t pi = row * a.num_parts + a.part_base + p;
        a.part_acc[pi * D + d] = num;
        if (d == 0) {
          a.part_m[pi] = any_bad ? nan : M;
          a.part_l[pi] = den;
        }
      }
    }
    return;
  }  // the pass
}

template <int DT, int D, int RW, int W>
void launch_mfma(const DecodeArgs &a, const StreamArgs &sa, dim3 grid, hipStream_t s) {
  constexpr int RB = DT == PKV_BF16 ? 2 * D : DT == kCodes3 ? D / 2 : D;
  static_assert(W * TileRing<CodeGeo<RB>::NL, DT != PKV_BF16, kMfmaRingBudget>::kBytes <= 163840,
                "LDS of the rings");
  hipLaunchKernelGGL((decode_mfma_kernel<DT, D, RW, W, false>), grid, dim3(W * 64), 0, s, a,
                     sa);
}

// Most sequences of a stream-mode launch: its slot prefix [B + 1] and the
// scan's 512 entries live in the ring's LDS before the first tile.
constexpr int kMfmaStreamSeqs = 4096;
// Slots without work at the head of each unit in stream mode: what a
// segment's start costs (query load, block-id window, ring fill: a few
// dependent memory latencies) in the time of one 16-token tile of a
// wavefront. Measured on the variable-length batch of 256: bf16 283.3 us
// at 2, 281.7 at 3, 283.8 at 4; over 8-bit codes 157 us at 2 to 6 alike
// (166 at 0).
constexpr int kMfmaStreamSegCost = 3;

// Stream mode over bf16 caches or caches of codes (eight independent
// wavefronts per workgroup, grid.x = sa.n_waves / 8), then the merge of its
// segments.
template <int DT, int D, int RW>
void launch_mfma_stream(const DecodeArgs &a, const StreamArgs &sa, dim3 grid, hipStream_t s) {
  constexpr int RB = DT == PKV_BF16 ? 2 * D : DT == kCodes3 ? D / 2 : D;
  static_assert(8 * TileRing<CodeGeo<RB>::NL, DT != PKV_BF16, kMfmaRingBudget>::kBytes >=
                    (kMfmaStreamSeqs + 1 + 512) * 4,
                "the slot prefix fits the rings' LDS");
  hipLaunchKernelGGL((decode_mfma_kernel<DT, D, RW, 8, true>), grid, dim3(8 * 64), 0, s, a,
                     sa);
  hipLaunchKernelGGL((reduce_stream_kernel<D, RW>), dim3(a.Hkv, a.B), dim3(RW * D / 4), 0, s,
                     a, sa);
}

// Launcher of the MFMA decode kernel for DT = PKV_BF16 (D 64 or 128),
// PKV_I8 or kCodes3, head dim D, RW query rows per wavefront (4, 8 or 16)
// and W wavefronts per workgroup (1, 4 or 8); nullptr if none. Defined in
// decode_inst_mfma_d<D>.hip.
template <int D>
Launcher pick_mfma(int DT, int RW, int W);

// Launcher of the stream mode over DT = PKV_BF16 or PKV_I8 (head dim D 64
// or 128) or kCodes3 (D 128), RW query rows per wavefront (4, 8 or 16),
// which also launches the merge; nullptr if none. Defined in
// decode_inst_mfma_d<D>.hip.
template <int D>
Launcher pick_mfma_stream(int DT, int RW);

}  // namespace decode
}  // namespace pkv
