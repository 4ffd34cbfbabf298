#pragma once
// Paged attention decode for gfx950 (MI355X): the partition kernel (a
// template, instantiated in decode_inst_*.hip) and its helpers.
//
// Method: PagedAttention (vLLM abstract on the papers page "external vector
// cache") -- attention of each sequence's new query token(s) over a KV cache
// held in fixed-size physical blocks reached through a per-sequence block
// table. Causal visibility for several query tokens per sequence follows the
// course page "Module 10. KV Caches and Efficient Inference", notebook
// section 2 (query j of a suffix sees prefix + j + 1 keys); the attention
// itself is the max-subtracted softmax of that page's project demo (Demo 2),
// computed here online in one pass.
//
// Work decomposition (designed for CDNA4, not taken from the pages):
//   * grid = (context partitions, KV heads, sequences); one workgroup of
//     WAVES wavefronts per (partition, KV head, sequence). All G = Hq / Hkv
//     query heads of a KV head (times the query tokens) are handled by the
//     same wavefront, so every K/V byte loaded from HBM feeds all of them.
//   * a wavefront consumes one 16-token tile per step. The tile of one KV
//     head is a contiguous 16 * D-element run of one block, read with one
//     16-byte load per lane per 1 KiB, fully coalesced; lanes own a slice of
//     D for a few tokens, so the loads feed the arithmetic directly from
//     registers with no LDS staging.
//   * q.k partial sums are reduced across the lanes that share a token with
//     a reduce-scatter (each step halves the values a lane carries), so
//     every lane ends with whole scores; exponentials are taken once per
//     score; the weights are then broadcast back for the V accumulation.
//   * online softmax with a lazy maximum: the running maximum is only raised
//     (and the accumulators rescaled) when a score exceeds it by more than
//     kLazyLog2, which keeps the common step free of cross-lane max
//     reductions while bounding weights by 2^kLazyLog2 (exact in float32).
//   * fp32 accumulation; bf16 q.k uses the packed bf16 dot instruction
//     (exact products, fp32 sums).
//   * a workgroup merges its wavefronts in LDS. With one partition it writes
//     the normalised output; otherwise it writes unnormalised partials
//     (m, l, acc) and the reduce kernel merges them:
//     M = max m_p, out = sum 2^(m_p-M) acc_p / sum 2^(m_p-M) l_p.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>
#include <type_traits>

#include "pagedkv.h"

namespace pkv {
namespace decode {


constexpr int kTile = 16;          // tokens per wavefront step
constexpr float kLazyLog2 = 8.0f;  // tolerated growth of a score over the running max
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- cross-lane exchange ---------------------------------------------------
// Partner of a lane across bit M of its lane id. Within a 16-lane row the
// partners come from DPP (quad_perm, row_half_mirror, row_mirror: lane ^ 1,
// ^3, ^7, ^15); across rows from permlane16/32 swaps (lane ^ 16, ^ 32). Each
// partner differs from the lane in bit M and agrees on every higher bit,
// which is all a butterfly (reduce or reduce-scatter) over bits M, M/2, ...
// needs.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Compile-time loop: f(integral_constant<int, I>) for I = 0 .. N-1.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

template <int M>
__device__ __forceinline__ float xor_partner(float x) {
  if constexpr (M == 1) {
    return dpp_mov<0xB1>(x);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return dpp_mov<0x1B>(x);  // quad_perm [3,2,1,0]
  } else if constexpr (M == 4) {
    return dpp_mov<0x141>(x);  // row_half_mirror
  } else if constexpr (M == 8) {
    return dpp_mov<0x140>(x);  // row_mirror
  } else if constexpr (M == 16) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const bool even_row = ((threadIdx.x >> 4) & 1) == 0;
    return __uint_as_float(even_row ? r[1] : r[0]);
  } else {
    static_assert(M == 32, "lane bit out of range");
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const bool low_half = (threadIdx.x & 32) == 0;
    return __uint_as_float(low_half ? r[1] : r[0]);
  }
}

// The lane exactly lane ^ M (M >= 8): unlike xor_partner, lower lane bits are
// preserved, as needed when lanes below M hold different data.
template <int M>
__device__ __forceinline__ float exact_xor(float x) {
  if constexpr (M == 8) {
    return dpp_mov<0x128>(x);  // row_ror:8 within a 16-lane row is lane ^ 8
  } else {
    static_assert(M == 16 || M == 32, "exact_xor covers lane bits 3..5");
    return xor_partner<M>(x);  // the permlane swaps are exact
  }
}

template <int M>
__device__ __forceinline__ float wave_max_from(float x) {
  if constexpr (M >= 1) {
    x = fmaxf(x, xor_partner<M>(x));
    return wave_max_from<M / 2>(x);
  } else {
    return x;
  }
}
template <int M>
__device__ __forceinline__ float wave_sum_from(float x) {
  if constexpr (M >= 1) {
    x += xor_partner<M>(x);
    return wave_sum_from<M / 2>(x);
  } else {
    return x;
  }
}
__device__ __forceinline__ float wave_max(float x) { return wave_max_from<32>(x); }
__device__ __forceinline__ float wave_sum(float x) { return wave_sum_from<32>(x); }

// Value of lane `src` (0..LPT-1) of this lane's token group, for a
// compile-time source lane.
template <int LPT, int SRC>
__device__ __forceinline__ float group_bcast(float x, int lane) {
  if constexpr (LPT == 16) {
    return dpp_mov<0x150 + SRC>(x);  // row_newbcast
  } else if constexpr (LPT == 8) {
    const float lo = dpp_mov<0x150 + SRC>(x), hi = dpp_mov<0x150 + 8 + SRC>(x);
    return (lane & 8) ? hi : lo;
  } else {
    return __shfl(x, (lane & ~(LPT - 1)) + SRC, 64);
  }
}

// Geometry of one (dtype, head dim) pair as seen by a wavefront.
template <int DT, int D>
struct Geo {
  static constexpr int ES = DT == PKV_F32 ? 4 : 2;  // bytes per element
  static constexpr int TB = D * ES;                  // bytes per token row
  static constexpr int LPT = TB / 16;                // lanes sharing one token
  static constexpr int TPL = 64 / LPT;               // tokens per 1 KiB load
  static constexpr int NL = kTile / TPL;             // loads per lane per tile
  static constexpr int EPL = 16 / ES;                // elements per lane per load
  static_assert(LPT >= 1 && LPT <= 64 && 64 % LPT == 0, "unsupported head size");
  static_assert(NL >= 1, "a tile must cover whole loads");
};

struct DecodeArgs {
  float *out;
  float *lse;
  float *part_m;
  float *part_l;
  float *part_acc;
  const void *q;
  const void *kc;
  const void *vc;
  const int32_t *tables;
  const int32_t *lens;
  int32_t B, max_blocks, nq, Hq, Hkv, bs, num_blocks, part_tokens, num_parts;
  float scale_log2;
};

// One step of the reduce-scatter over lane bit M with `cnt` live values:
// the lane keeps the lower half of the values when its bit M is clear, the
// upper half when set, adding the partner's copy of the half it keeps.
template <int M, int V, int CNT>
__device__ __forceinline__ void rs_step(float (&x)[V], int jl) {
  if constexpr (CNT > 1) {
    constexpr int H = CNT / 2;
    const bool upper = (jl & M) != 0;
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const float lo = x[k], hi = x[k + H];
      x[k] = (upper ? hi : lo) + xor_partner<M>(upper ? lo : hi);
    }
  } else {
    x[0] += xor_partner<M>(x[0]);
  }
}

// Reduce-scatter of V per-lane partial sums across the LPT lanes of a token
// group (lane bits below LPT). After it, a lane holds C = max(1, V / LPT)
// complete sums: values own .. own + C - 1, own = jl * V / LPT.
template <int LPT, int V, int M = LPT / 2, int CNT = V>
__device__ __forceinline__ void reduce_scatter(float (&x)[V], int jl) {
  if constexpr (M >= 1) {
    rs_step<M, V, CNT>(x, jl);
    reduce_scatter<LPT, V, M / 2, (CNT > 1 ? CNT / 2 : 1)>(x, jl);
  }
}

template <int M, int LPT, int RP, int EPL>
__device__ __forceinline__ void sum_over_groups(float (&acc)[RP][EPL]) {
  if constexpr (M < 64) {
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[r][e] += exact_xor<M>(acc[r][e]);
    sum_over_groups<M * 2, LPT, RP, EPL>(acc);
  }
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// K/V rows are read once per step: non-temporal loads keep them from
// displacing reusable lines (tables, queries) and measured faster on MI355X.
__device__ __forceinline__ uint4 stream_load(const char *p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <int NL>
__device__ __forceinline__ void load_tile(uint4 (&kr)[NL], uint4 (&vr)[NL], const char *kp,
                                          const char *vp) {
#pragma unroll
  for (int i = 0; i < NL; ++i) kr[i] = stream_load(kp + i * 1024);
#pragma unroll
  for (int i = 0; i < NL; ++i) vr[i] = stream_load(vp + i * 1024);
}

// ---------------------------------------------------------------------------
// One wavefront's attention state for RP query rows of one KV head:
// queries, running max / sum and fp32 accumulators, and the per-tile math.
// ---------------------------------------------------------------------------
template <int DT, int D, int G, int RP>
struct DecodeWave {
  using Gm = Geo<DT, D>;
  static constexpr int LPT = Gm::LPT, TPL = Gm::TPL, NL = Gm::NL, EPL = Gm::EPL;
  static constexpr int V = RP * NL;                   // partial sums per lane per tile
  static constexpr int C = V >= LPT ? V / LPT : 1;    // whole scores per lane
  static constexpr int DUP = V >= LPT ? 1 : LPT / V;  // lanes holding the same score
  static constexpr float kNegInf = -std::numeric_limits<float>::infinity();

  int lane, grp, jl, d0;
  uint32_t qw[RP][4];  // bf16 query slices, two per word
  float qf[RP][4];     // fp32 query slices
  int own_row[C], own_tok[C], own_lim[C];
  float acc[RP][EPL];
  float m_run[RP];
  float m_own[C], l_own[C];
  int L, min_lim;
  int bad;

  __device__ __forceinline__ void init(int lane_) {
    lane = lane_;
    grp = lane / LPT;
    jl = lane % LPT;
    d0 = jl * EPL;
    const int own = jl * V / LPT;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int v = own + c;
      own_row[c] = v / NL;
      own_tok[c] = (v % NL) * TPL + grp;  // token offset inside the tile
    }
  }

  // Start a (sequence b, KV head g) item of context length L_: load the
  // query rows r = qi * G + gj (head g * G + gj) and reset the statistics.
  __device__ __forceinline__ void begin(const DecodeArgs &a, int b, int g, int L_) {
    const int nq = a.nq;
    L = L_;
    min_lim = L - nq + 1;
    bad = 0;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int qi = r / G;
      const size_t row = ((size_t)b * nq + (qi < nq ? qi : 0)) * a.Hq + g * G + (r % G);
      if constexpr (DT == PKV_BF16) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (qi < nq) w = *reinterpret_cast<const uint4 *>((const uint16_t *)a.q + row * D + d0);
        qw[r][0] = w.x; qw[r][1] = w.y; qw[r][2] = w.z; qw[r][3] = w.w;
      } else {
        float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
        if (qi < nq) w = *reinterpret_cast<const float4 *>((const float *)a.q + row * D + d0);
        qf[r][0] = w.x; qf[r][1] = w.y; qf[r][2] = w.z; qf[r][3] = w.w;
      }
      m_run[r] = kNegInf;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int qi = own_row[c] / G;
      own_lim[c] = qi < nq ? L - nq + qi + 1 : 0;  // visible keys of that row
      m_own[c] = kNegInf;
      l_own[c] = 0.f;
    }
  }

  // Consume one 16-token tile starting at logical token t0 whose K/V rows
  // are in kr / vr.
  __device__ __forceinline__ void process(const uint4 (&kr)[NL], const uint4 (&vr)[NL], int t0,
                                          float scale_log2) {
    // partial q.k over this lane's EPL dims: x[r * NL + i]
    float x[V];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float s = 0.f;
        if constexpr (DT == PKV_BF16) {
          s = dot2_bf16(qw[r][0], kr[i].x, s);
          s = dot2_bf16(qw[r][1], kr[i].y, s);
          s = dot2_bf16(qw[r][2], kr[i].z, s);
          s = dot2_bf16(qw[r][3], kr[i].w, s);
        } else {
          s = fmaf(qf[r][0], __uint_as_float(kr[i].x), s);
          s = fmaf(qf[r][1], __uint_as_float(kr[i].y), s);
          s = fmaf(qf[r][2], __uint_as_float(kr[i].z), s);
          s = fmaf(qf[r][3], __uint_as_float(kr[i].w), s);
        }
        x[r * NL + i] = s;
      }
    }
    reduce_scatter<LPT, V>(x, jl);

    float sc[C];
    bool need = false;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool vis = t0 + own_tok[c] < own_lim[c];
      sc[c] = vis ? x[c] * scale_log2 : kNegInf;
      need |= sc[c] > m_own[c] + kLazyLog2;
    }
    if (__any(need)) {
      float alpha[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        float xm = kNegInf;
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (own_row[c] == r) xm = fmaxf(xm, sc[c]);
        const float mt = wave_max(xm);
        const float mn = fmaxf(m_run[r], mt);
        alpha[r] = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run[r] - mn);
        m_run[r] = mn;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[r][e] *= alpha[r];
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float mo = m_own[c], al = 1.f;
#pragma unroll
        for (int r = 0; r < RP; ++r)
          if (own_row[c] == r) {
            mo = m_run[r];
            al = alpha[r];
          }
        m_own[c] = mo;
        l_own[c] *= al;
      }
    }
    float pw[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      pw[c] = sc[c] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sc[c] - m_own[c]);
      l_own[c] += pw[c];
    }
    // every lane of the group needs all V weights of its tokens: each is
    // broadcast from its owner lane right before its FMAs
    // in a tail tile, slots past the context may hold stale bits (even NaN):
    // their V is zeroed so that 0 * NaN cannot reach acc
    const bool tail = t0 + kTile > min_lim;
    static_for<NL>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      float vv[EPL];
      if constexpr (DT == PKV_BF16) {
        vv[0] = bf16_lo(vr[i].x); vv[1] = bf16_hi(vr[i].x);
        vv[2] = bf16_lo(vr[i].y); vv[3] = bf16_hi(vr[i].y);
        vv[4] = bf16_lo(vr[i].z); vv[5] = bf16_hi(vr[i].z);
        vv[6] = bf16_lo(vr[i].w); vv[7] = bf16_hi(vr[i].w);
      } else {
        vv[0] = __uint_as_float(vr[i].x); vv[1] = __uint_as_float(vr[i].y);
        vv[2] = __uint_as_float(vr[i].z); vv[3] = __uint_as_float(vr[i].w);
      }
      if (tail && t0 + i * TPL + grp >= L) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vv[e] = 0.f;
      }
      static_for<RP>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        constexpr int v = r * NL + i;
        constexpr int src = V >= LPT ? v / C : v * DUP;
        const float w = group_bcast<LPT, src>(pw[v % C], lane);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[r][e] = fmaf(w, vv[e], acc[r][e]);
      });
    });
  }

  // Sum acc over the token groups (every lane then holds the totals of its
  // dims) and return each row's sum of weights.
  __device__ __forceinline__ void totals(float (&l_row)[RP]) {
    sum_over_groups<LPT, LPT, RP, EPL>(acc);
    const bool counted = (jl % DUP) == 0;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float xs = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (own_row[c] == r && counted) xs += l_own[c];
      l_row[r] = wave_sum(xs);
    }
  }
};

// Byte offset of the 16-token tile at logical token t0 of KV head g in
// block blk, for this lane.
template <int TB>
__device__ __forceinline__ size_t tile_bytes_offset(const DecodeArgs &a, int g, int t0, int blk,
                                                    int lane) {
  return ((size_t)blk * a.Hkv + g) * ((size_t)a.bs * TB) + (size_t)(t0 % a.bs) * TB +
         (size_t)lane * 16;
}

// ---------------------------------------------------------------------------
// Workgroup-split kernel: one workgroup of kWaves wavefronts per (partition,
// KV head, sequence); the wavefronts take interleaved tiles and are merged
// in LDS. Used when there are enough (sequence, KV head) pairs to fill the
// chip with one partition each.
// ---------------------------------------------------------------------------
template <int DT, int D, int G, int RP, int kWaves>
__global__ void __launch_bounds__(kWaves * 64)
decode_partition_kernel(const DecodeArgs a) {
  using W = DecodeWave<DT, D, G, RP>;
  using Gm = Geo<DT, D>;
  constexpr int NL = Gm::NL, EPL = Gm::EPL;
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  constexpr int kStride = kWaves * kTile;  // tokens between a wavefront's tiles

  __shared__ float sm_acc[kWaves][RP][D];
  __shared__ float sm_m[kWaves][RP];
  __shared__ float sm_l[kWaves][RP];
  __shared__ int sm_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nq = a.nq;
  const int L = a.lens[b];
  const int max_ctx = a.max_blocks * a.bs;

  if (L < nq || L > max_ctx) {  // a row would see no key, or the table is too short
    if (a.num_parts == 1 && p == 0) {
      const float nan = __builtin_nanf("");
      for (int idx = threadIdx.x; idx < RP * D; idx += kWaves * 64) {
        const int r = idx / D, d = idx % D, qi = r / G;
        if (qi >= nq) continue;
        const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (r % G);
        a.out[row * D + d] = nan;
        if (d == 0 && a.lse) a.lse[row] = nan;
      }
    }
    return;  // with partitions, the reduce kernel writes the NaN rows
  }
  const int t_begin = p * a.part_tokens;
  if (t_begin >= L) return;  // past this sequence's end: the reduce reads nothing here
  const int t_end = min(L, t_begin + a.part_tokens);

  W st;
  st.init(lane);
  st.begin(a, b, g, L);

  const int32_t *trow = a.tables + (size_t)b * a.max_blocks;
  const char *kbase = (const char *)a.kc;
  const char *vbase = (const char *)a.vc;
  auto tile_offset = [&](int t0, int blk) -> size_t {
    if (blk < 0 || blk >= a.num_blocks) {  // bad table entry: read block 0, poison later
      st.bad = 1;
      blk = 0;
    }
    return tile_bytes_offset<Gm::TB>(a, g, t0, blk, lane);
  };

  // Software pipeline: the next tile's K/V loads are in flight while the
  // current tile is consumed. The steady-state loop issues its loads
  // unconditionally (two tiles per trip, alternating register sets) so the
  // compiler's wait counts leave the prefetched loads outstanding; the last
  // one or two tiles are peeled. Block ids are read one trip ahead.
  const int n_tiles = t_begin + wave * kTile < t_end
                          ? (t_end - (t_begin + wave * kTile) + kStride - 1) / kStride
                          : 0;
  auto tile_t0 = [&](int k) { return t_begin + wave * kTile + k * kStride; };
  auto table_at = [&](int k) { return trow[tile_t0(k < n_tiles ? k : n_tiles - 1) / a.bs]; };
  if (n_tiles > 0) {
    uint4 ka[NL], va[NL], kb[NL], vb[NL];
    {
      const size_t off = tile_offset(tile_t0(0), table_at(0));
      load_tile<NL>(ka, va, kbase + off, vbase + off);
    }
    int blk1 = table_at(1), blk2 = table_at(2);
    int k = 0;
    for (; k + 2 < n_tiles; k += 2) {
      const int nb1 = table_at(k + 3), nb2 = table_at(k + 4);
      {
        const size_t off = tile_offset(tile_t0(k + 1), blk1);
        load_tile<NL>(kb, vb, kbase + off, vbase + off);
      }
      st.process(ka, va, tile_t0(k), a.scale_log2);
      {
        const size_t off = tile_offset(tile_t0(k + 2), blk2);
        load_tile<NL>(ka, va, kbase + off, vbase + off);
      }
      st.process(kb, vb, tile_t0(k + 1), a.scale_log2);
      blk1 = nb1;
      blk2 = nb2;
    }
    if (k + 1 < n_tiles) {
      const size_t off = tile_offset(tile_t0(k + 1), blk1);
      load_tile<NL>(kb, vb, kbase + off, vbase + off);
      st.process(ka, va, tile_t0(k), a.scale_log2);
      st.process(kb, vb, tile_t0(k + 1), a.scale_log2);
    } else {
      st.process(ka, va, tile_t0(k), a.scale_log2);
    }
  }

  // ---- wavefront totals, then merge the wavefronts in LDS ------------------
  float l_row[RP];
  st.totals(l_row);
  if (lane < W::LPT) {
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][r][st.d0 + e] = st.acc[r][e];
  }
  if (lane == 0) {  // bad is wavefront-uniform: it comes from scalar table reads
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      sm_m[wave][r] = st.m_run[r];
      sm_l[wave][r] = l_row[r];
    }
    sm_bad[wave] = st.bad;
  }
  __syncthreads();

  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any_bad |= sm_bad[w];
  const float nan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < RP * D; idx += kWaves * 64) {
    const int r = idx / D, d = idx % D, qi = r / G;
    if (qi >= nq) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][r];
      const float f = mw == kNegInf ? 0.f : exp2f(mw - M);
      num = fmaf(f, sm_acc[w][r][d], num);
      den = fmaf(f, sm_l[w][r], den);
    }
    const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (r % G);
    if (a.num_parts == 1) {
      a.out[row * D + d] = any_bad || den == 0.f ? nan : num / den;
      if (d == 0 && a.lse) a.lse[row] = any_bad || den == 0.f ? nan : (M + log2f(den)) * kLn2;
    } else {
      const size_t pi = row * a.num_parts + p;
      a.part_acc[pi * D + d] = num;
      if (d == 0) {
        a.part_m[pi] = any_bad ? nan : M;
        a.part_l[pi] = den;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Work-item kernel for split contexts: persistent wavefronts, each taking
// (sequence, KV head, partition) items in round robin from a dense list
// (partitions past a sequence's end are not items). A wavefront streams the
// tiles of its items back to back -- the software pipeline runs across item
// boundaries -- and writes unnormalised partials per item; the reduce kernel
// merges them. No LDS merge, no barriers after the item list is built.
// ---------------------------------------------------------------------------
constexpr int kItemWaves = 4;  // wavefronts per workgroup (independent)

template <int DT, int D, int G, int RP>
__global__ void __launch_bounds__(kItemWaves * 64)
decode_items_kernel(const DecodeArgs a) {
  using W = DecodeWave<DT, D, G, RP>;
  using Gm = Geo<DT, D>;
  constexpr int NL = Gm::NL, EPL = Gm::EPL;
  constexpr int kThreads = kItemWaves * 64;
  extern __shared__ int sm_pre[];  // [B + 1]: partitions before sequence b
  __shared__ int sm_scan[kThreads];

  const int B = a.B, P = a.part_tokens, nq = a.nq, Hkv = a.Hkv;
  const int max_ctx = a.max_blocks * a.bs;

  // ---- dense item list: prefix sums of partitions per sequence ------------
  {
    const int per = (B + kThreads - 1) / kThreads;
    const int lo = min(B, (int)threadIdx.x * per), hi = min(B, lo + per);
    int sum = 0;
    for (int b = lo; b < hi; ++b) {
      const int L = a.lens[b];
      sum += (L >= nq && L <= max_ctx) ? (L + P - 1) / P : 0;
    }
    sm_scan[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan
      const int v = threadIdx.x >= off ? sm_scan[threadIdx.x - off] : 0;
      __syncthreads();
      sm_scan[threadIdx.x] += v;
      __syncthreads();
    }
    int run = sm_scan[threadIdx.x] - sum;  // exclusive prefix of this chunk
    for (int b = lo; b < hi; ++b) {
      sm_pre[b] = run;
      const int L = a.lens[b];
      run += (L >= nq && L <= max_ctx) ? (L + P - 1) / P : 0;
    }
    if (threadIdx.x == kThreads - 1) sm_pre[B] = sm_scan[kThreads - 1];
    __syncthreads();
  }
  const int total = __builtin_amdgcn_readfirstlane(sm_pre[B]) * Hkv;

  const int lane = threadIdx.x & 63;
  const int n_waves = gridDim.x * kItemWaves;
  const int first = __builtin_amdgcn_readfirstlane(blockIdx.x * kItemWaves + (threadIdx.x >> 6));
  if (first >= total) return;

  // item id -> (b, g, token range); ids of one sequence are contiguous
  struct Cursor {
    int id, b, g, t, t_end;
  };
  auto locate = [&](Cursor &c) {
    int lo = 0, hi = B;  // sm_pre[lo] * Hkv <= id < sm_pre[hi] * Hkv
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(sm_pre[mid]) * Hkv <= c.id) lo = mid; else hi = mid;
    }
    const int p0 = __builtin_amdgcn_readfirstlane(sm_pre[lo]);
    const int np = __builtin_amdgcn_readfirstlane(sm_pre[lo + 1]) - p0;
    const int local = c.id - p0 * Hkv;
    c.b = lo;
    c.g = local / np;
    const int p = local - c.g * np;
    c.t = p * P;
    c.t_end = min(a.lens[lo], c.t + P);
  };
  auto advance = [&](Cursor &c) {  // next tile of this wavefront's stream
    if (c.id >= total) return;
    c.t += kTile;
    if (c.t >= c.t_end) {
      c.id += n_waves;
      if (c.id < total) locate(c);
    }
  };
  auto table_entry = [&](const Cursor &c) {
    return a.tables[(size_t)c.b * a.max_blocks + c.t / a.bs];
  };

  W st;
  st.init(lane);
  const char *kbase = (const char *)a.kc;
  const char *vbase = (const char *)a.vc;
  // Offset of a tile; a bad table entry reads block 0 and flags the tile so
  // that its item's partials are poisoned when the tile is consumed.
  auto offset = [&](const Cursor &c, int blk, int &tile_bad) -> size_t {
    tile_bad = blk < 0 || blk >= a.num_blocks;
    return tile_bytes_offset<Gm::TB>(a, c.g, c.t, tile_bad ? 0 : blk, lane);
  };

  // Tiles in this wavefront's stream (all tiles of its items, in order).
  int n_tiles = 0;
  for (Cursor c{first, 0, 0, 0, 0}; c.id < total; c.id += n_waves) {
    locate(c);
    n_tiles += (c.t_end - c.t + kTile - 1) / kTile;
  }

  // Cursors: cur = tile being consumed, iss = next tile to load, pre = the
  // one after (its block id is read a step ahead). The steady-state loop
  // has the same shape as the workgroup-split kernel's: two tiles per trip,
  // alternating register sets, loads issued unconditionally, the last one or
  // two tiles peeled.
  Cursor cur{first, 0, 0, 0, 0};
  locate(cur);
  st.begin(a, cur.b, cur.g, a.lens[cur.b]);
  Cursor iss = cur;
  advance(iss);
  Cursor pre = iss;
  advance(pre);
  int bad_a = 0, bad_b = 0;
  const size_t off0 = offset(cur, table_entry(cur), bad_a);
  int blk_iss = iss.id < total ? table_entry(iss) : 0;
  int blk_pre = pre.id < total ? table_entry(pre) : 0;

  // Load the tile at `iss`, then move the cursors on.
  auto issue = [&](uint4 (&kr)[NL], uint4 (&vr)[NL], int &tile_bad) {
    const size_t off = offset(iss, blk_iss, tile_bad);
    load_tile<NL>(kr, vr, kbase + off, vbase + off);
    iss = pre;
    blk_iss = blk_pre;
    advance(pre);
    blk_pre = pre.id < total ? table_entry(pre) : 0;
  };
  // Consume the tile in kr / vr at cursor `cur`; at an item's last tile,
  // write the item's partials and start the next item.
  auto consume = [&](const uint4 (&kr)[NL], const uint4 (&vr)[NL], int tile_bad) {
    st.bad |= tile_bad;
    st.process(kr, vr, cur.t, a.scale_log2);
    if (cur.t + kTile < cur.t_end) {
      cur.t += kTile;
      return;
    }
    float l_row[RP];
    st.totals(l_row);
    const int p = cur.t / P;
    const float nan = __builtin_nanf("");
    if (lane < W::LPT) {
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const int qi = r / G;
        if (qi >= nq) continue;
        const size_t row = ((size_t)cur.b * nq + qi) * a.Hq + cur.g * G + (r % G);
        float *dst = a.part_acc + (row * a.num_parts + p) * D + st.d0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[e] = st.acc[r][e];
        if (lane == 0) {
          a.part_m[row * a.num_parts + p] = st.bad ? nan : st.m_run[r];
          a.part_l[row * a.num_parts + p] = l_row[r];
        }
      }
    }
    advance(cur);
    if (cur.id < total) st.begin(a, cur.b, cur.g, a.lens[cur.b]);
  };

  uint4 ka[NL], va[NL], kb[NL], vb[NL];
  load_tile<NL>(ka, va, kbase + off0, vbase + off0);
  int k = 0;
  for (; k + 2 < n_tiles; k += 2) {
    issue(kb, vb, bad_b);
    consume(ka, va, bad_a);
    issue(ka, va, bad_a);
    consume(kb, vb, bad_b);
  }
  if (k + 1 < n_tiles) {
    issue(kb, vb, bad_b);
    consume(ka, va, bad_a);
    consume(kb, vb, bad_b);
  } else {
    consume(ka, va, bad_a);
  }
}

using Launcher = void (*)(const DecodeArgs &, dim3, hipStream_t);

template <int DT, int D, int G, int RP, int W>
void launch_decode(const DecodeArgs &a, dim3 grid, hipStream_t s) {
  if constexpr (W == 0) {  // work-item kernel; grid.x persistent workgroups
    hipLaunchKernelGGL((decode_items_kernel<DT, D, G, RP>), grid, dim3(kItemWaves * 64),
                       (a.B + 1) * sizeof(int), s, a);
  } else {
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, RP, W>), grid, dim3(W * 64), 0, s, a);
  }
}

// Launcher for (dtype, D) and rows per wavefront RP = G * (query tokens
// rounded up to a power of two): W = 4 or 8 wavefronts per workgroup of the
// workgroup-split kernel, or W = 0 for the work-item kernel; nullptr if no
// such kernel is built. Defined in decode_inst_<dtype>_d<D>.hip.
template <int DT, int D>
Launcher pick_rows(int G, int RP, int W);

// Largest RP with a kernel.
constexpr int kMaxRows = 8;

}  // namespace decode
}  // namespace pkv
