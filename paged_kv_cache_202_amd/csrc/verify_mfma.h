// Multi-query paged attention on MFMA for gfx950 (MI355X): the verify step
// of speculative decoding, where each sequence checks nq draft tokens at
// once and every KV head serves a 16-row query tile (G query heads x nq
// tokens). Causal rule: query i of nq sees the first L - nq + i + 1 tokens
// (course page "Module 10. KV Caches and Efficient Inference", notebook
// section 2: query j of a suffix sees prefix + j + 1 keys). The attention is
// the max-subtracted softmax of that page's project demo (Demo 2), computed
// online; "NeuralOps v1.3.4", Speculative Decoding Pipeline, names the
// single-pass parallel verification this serves.
//
// Design (for CDNA4):
//   * one workgroup of kWaves wavefronts per (partition, KV head, sequence);
//     wavefronts take interleaved 16-token tiles, merged in LDS at the end;
//   * per tile, S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (D/32 of them):
//     the K tile is the A operand, read straight from HBM (16 bytes a lane,
//     a lane holding D/4 contiguous dims of one token); Q^T is the B operand,
//     kept in registers with the same dim assignment. The accumulator layout
//     puts, in lane l, the scores of query row l % 16 for tokens
//     4 (l / 16) + 0..3 -- exactly the A-operand layout the P V product needs;
//   * online softmax on those accumulators (row max across the 4 lane groups
//     by permlane swaps, lazily raised as in the decode kernel), P rounded to
//     bf16;
//   * O += P V with v_mfma_f32_16x16x16_bf16 (D/16 column blocks). V is the
//     B operand (token-major in k), so each tile of V goes through a
//     bank-padded LDS tile and is read back transposed;
//   * fp32 accumulation throughout; the next tile's loads are in flight while
//     the current one is consumed.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "decode_kernel.h"

namespace pkv {
namespace decode {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

constexpr int kVerifyWaves = 4;
constexpr int kVerifyRows = 16;  // query rows per KV head in one MFMA tile

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2v_t t = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, t);
}

template <int D>
struct VerifyGeo {
  static constexpr int NC = D / 32;       // 16-byte loads per lane per K (or V) tile
  static constexpr int NCB = D / 16;      // column blocks of the P V product
  static constexpr int ROWW = D / 2 + 2;  // LDS words per V row: 4 rows apart = 8 banks apart
  static_assert(D % 32 == 0, "head dim must be a multiple of 32");
};

template <int D, int kWaves>
__global__ void __launch_bounds__(kWaves * 64)
verify_mfma_kernel(const DecodeArgs a) {
  using Gv = VerifyGeo<D>;
  constexpr int NC = Gv::NC, NCB = Gv::NCB, ROWW = Gv::ROWW;
  constexpr int kStride = kWaves * kTile;
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  constexpr int kVWords = kTile * ROWW;  // one wavefront's V tile
  constexpr int kSmWords = kWaves * kVerifyRows * D > kWaves * kVWords
                               ? kWaves * kVerifyRows * D
                               : kWaves * kVWords;
  // V tiles during the loop; wavefront accumulators for the merge after it
  __shared__ uint32_t sm_raw[kSmWords];
  __shared__ float sm_m[kWaves][kVerifyRows];
  __shared__ float sm_l[kWaves][kVerifyRows];
  __shared__ int sm_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nq = a.nq, G = a.Hq / a.Hkv, R = G * nq;
  const int L = load_const(a.lens + b);
  const int max_ctx = a.max_blocks * a.bs;
  const float nan = __builtin_nanf("");

  if (L < nq || L > max_ctx) {  // a row would see no key, or the table is too short
    if (a.num_parts == 1 && p == 0) {
      for (int idx = threadIdx.x; idx < R * D; idx += kWaves * 64) {
        const int r = idx / D, d = idx % D, qi = r / G;
        const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (r % G);
        a.out[row * D + d] = nan;
        if (d == 0 && a.lse) a.lse[row] = nan;
      }
    }
    return;
  }
  // earlier tokens belong to the prefix phase (clamped: bad values cannot
  // send reads outside the table)
  const int start = a.starts ? min(max(load_const(a.starts + b), 0), L) : 0;
  const int t_begin = start + p * a.part_tokens;
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + a.part_tokens);

  // ---- Q^T as the B operand: row ln, dims lg * D/4 + c * 8 .. +8 ----------
  uint4 qb[NC];
  {
    const int qi = ln / G;
    const size_t row = ((size_t)b * nq + (ln < R ? qi : 0)) * a.Hq + g * G + (ln % G);
    const uint16_t *qp = (const uint16_t *)a.q + row * D + lg * (D / 4);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qb[c] = ln < R ? *reinterpret_cast<const uint4 *>(qp + c * 8) : make_uint4(0, 0, 0, 0);
  }
  // visible keys of this lane's softmax row (row ln); 0 for padding rows
  const int lim = ln < R ? L - nq + ln / G + 1 : 0;
  const int min_lim = L - nq + 1;

  f32x4_t o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_row = kNegInf;  // running max of row ln (log2 units)
  float l_part = 0.f;     // this lane's share of row ln's weight sum
  int bad = 0;

  uint32_t *vt = sm_raw + wave * kVWords;
  const int32_t *trow = a.tables + (size_t)b * a.max_blocks;
  const char *kbase = (const char *)a.kc;
  const char *vbase = (const char *)a.vc;
  const size_t lane_off = (size_t)ln * (D * 2) + (size_t)lg * (D / 2);
  auto tile_offset = [&](int t0, int blk) -> size_t {
    if (blk < 0 || blk >= a.num_blocks) {
      bad = 1;
      blk = 0;
    }
    return (((size_t)blk * a.Hkv + g) * a.bs + (size_t)(t0 % a.bs)) * (D * 2) + lane_off;
  };
  // Plain (temporal) loads: in the verify step sequences usually share a
  // prefix, and its blocks are then re-read by every sharer; kept in L2 they
  // are served from there (measured: 113 -> 81 us for 64 sharers of a
  // 2048-token prefix), where non-temporal loads would bypass it.
  auto load = [&](uint4 (&kr)[NC], uint4 (&vr)[NC], size_t off) {
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = *reinterpret_cast<const uint4 *>(kbase + off + c * 16);
#pragma unroll
    for (int c = 0; c < NC; ++c) vr[c] = *reinterpret_cast<const uint4 *>(vbase + off + c * 16);
  };

  auto process = [&](const uint4 (&kr)[NC], const uint4 (&vr)[NC], int t0) {
    // S^T = K Q^T: s[e] = score of row ln with token t0 + 4 lg + e
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[c]),
                                                  __builtin_bit_cast(bf16x8_t, qb[c]), s, 0, 0,
                                                  0);
    float sc[4];
    bool need = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool vis = t0 + 4 * lg + e < lim;
      sc[e] = vis ? s[e] * a.scale_log2 : kNegInf;
      need |= sc[e] > m_row + kLazyLog2;
    }
    if (__any(need)) {
      float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      tmax = fmaxf(tmax, exact_xor<16>(tmax));
      tmax = fmaxf(tmax, exact_xor<32>(tmax));
      const float mn = fmaxf(m_row, tmax);
      const float alpha = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_row - mn);
      m_row = mn;
      l_part *= alpha;
      // O holds rows 4 lg + e: their factors live in lanes 4 lg + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float al = __shfl(alpha, 4 * lg + e, 64);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[cb][e] *= al;
      }
    }
    float pw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pw[e] = sc[e] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sc[e] - m_row);
      l_part += pw[e];
    }
    const uint2 pa = make_uint2(pack_bf16(pw[0], pw[1]), pack_bf16(pw[2], pw[3]));

    // V tile -> LDS (row = token ln; past-the-context rows are zeroed so
    // that stale bits cannot reach the product), then read back transposed
    const bool zero = t0 + kTile > min_lim && t0 + ln >= L;
    uint2 *vrow = reinterpret_cast<uint2 *>(vt + ln * ROWW + lg * (D / 8));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 w = zero ? make_uint4(0, 0, 0, 0) : vr[c];
      vrow[2 * c] = make_uint2(w.x, w.y);
      vrow[2 * c + 1] = make_uint2(w.z, w.w);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint16_t *vt16 = reinterpret_cast<const uint16_t *>(vt);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      // B operand: V[token 4 lg + u][dim cb * 16 + ln], u = 0..3
      const int col = cb * 16 + ln;
      const uint32_t u0 = vt16[(4 * lg + 0) * (2 * ROWW) + col];
      const uint32_t u1 = vt16[(4 * lg + 1) * (2 * ROWW) + col];
      const uint32_t u2 = vt16[(4 * lg + 2) * (2 * ROWW) + col];
      const uint32_t u3 = vt16[(4 * lg + 3) * (2 * ROWW) + col];
      const uint2 vb = make_uint2(u0 | (u1 << 16), u2 | (u3 << 16));
      o[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, pa),
                                                       __builtin_bit_cast(i16x4_t, vb), o[cb],
                                                       0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // software pipeline, as in the decode kernel
  const int n_tiles = t_begin + wave * kTile < t_end
                          ? (t_end - (t_begin + wave * kTile) + kStride - 1) / kStride
                          : 0;
  auto tile_t0 = [&](int k) { return t_begin + wave * kTile + k * kStride; };
  auto table_at = [&](int k) {
    return load_const(trow + tile_t0(k < n_tiles ? k : n_tiles - 1) / a.bs);
  };
  if (n_tiles > 0) {
    uint4 ka[NC], va[NC], kb[NC], vb[NC];
    load(ka, va, tile_offset(tile_t0(0), table_at(0)));
    int blk1 = table_at(1), blk2 = table_at(2);
    int k = 0;
    for (; k + 2 < n_tiles; k += 2) {
      const int nb1 = table_at(k + 3), nb2 = table_at(k + 4);
      load(kb, vb, tile_offset(tile_t0(k + 1), blk1));
      process(ka, va, tile_t0(k));
      load(ka, va, tile_offset(tile_t0(k + 2), blk2));
      process(kb, vb, tile_t0(k + 1));
      blk1 = nb1;
      blk2 = nb2;
    }
    if (k + 1 < n_tiles) {
      load(kb, vb, tile_offset(tile_t0(k + 1), blk1));
      process(ka, va, tile_t0(k));
      process(kb, vb, tile_t0(k + 1));
    } else {
      process(ka, va, tile_t0(k));
    }
  }

  // ---- wavefront totals: row sums across the 4 lane groups -----------------
  float l_row = l_part;
  l_row += exact_xor<16>(l_row);
  l_row += exact_xor<32>(l_row);
  __syncthreads();  // every wavefront is done with its V tile region
  float *sm_o = reinterpret_cast<float *>(sm_raw) + wave * kVerifyRows * D;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm_o[(4 * lg + e) * D + cb * 16 + ln] = o[cb][e];
  if (lg == 0) {
    sm_m[wave][ln] = m_row;
    sm_l[wave][ln] = l_row;
  }
  if (lane == 0) sm_bad[wave] = bad;  // wavefront-uniform (scalar table reads)
  __syncthreads();

  // ---- merge the wavefronts; write output or partials ----------------------
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any_bad |= sm_bad[w];
  const float *smo = reinterpret_cast<const float *>(sm_raw);
  for (int idx = threadIdx.x; idx < R * D; idx += kWaves * 64) {
    const int r = idx / D, d = idx % D, qi = r / G;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][r];
      const float f = mw == kNegInf ? 0.f : exp2f(mw - M);
      num = fmaf(f, smo[(w * kVerifyRows + r) * D + d], num);
      den = fmaf(f, sm_l[w][r], den);
    }
    const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (r % G);
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
}

// Launcher for a head dim (nullptr if none); defined in verify_inst.hip.
Launcher pick_verify(int D);

}  // namespace decode
}  // namespace pkv
