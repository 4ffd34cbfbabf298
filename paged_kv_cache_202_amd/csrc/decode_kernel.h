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
  // Query rows of a KV head are r = qi * G + gj (query token qi, head gj of
  // the group); a wavefront holds RP of them and `slices` wavefronts share
  // a KV head's rows: slice s holds rows s * RP .. s * RP + RP - 1.
  int32_t slices;
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

// Read-only metadata (block tables, context lengths) read at a
// wavefront-uniform address: through the constant address space the load is
// a scalar load, even in loops that also store to global memory, so it never
// waits on the vector-memory counter that tracks the K/V stream.
template <class T>
__device__ __forceinline__ T load_const(const T *p) {
  return *(const __attribute__((address_space(4))) T *)(p);
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

  // Start a (sequence b, KV head g) item of context length L_ for rows
  // row0 .. row0 + RP - 1: load those query rows and reset the statistics.
  __device__ __forceinline__ void begin(const DecodeArgs &a, int b, int g, int L_, int row0) {
    const int nq = a.nq;
    L = L_;
    min_lim = L - nq + 1;
    bad = 0;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int rr = row0 + r;
      const int qi = rr / G;
      const size_t row = ((size_t)b * nq + (qi < nq ? qi : 0)) * a.Hq + g * G + (rr % G);
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
      const int qi = (row0 + own_row[c]) / G;
      own_lim[c] = qi < nq ? L - nq + qi + 1 : 0;  // visible keys of that row
      m_own[c] = kNegInf;
      l_own[c] = 0.f;
    }
  }

  // Fresh statistics for a new partition of the same (b, g): queries kept.
  __device__ __forceinline__ void restart() {
    bad = 0;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      m_run[r] = kNegInf;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
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

// NS row sets of RP rows each in one wavefront (RW = NS * RP rows): every
// loaded K/V tile feeds all of them, so a KV head's rows need not be split
// over wavefronts that would each stream the same bytes.
template <int DT, int D, int G, int RP, int NS>
struct DecodeWaveSet {
  using One = DecodeWave<DT, D, G, RP>;
  static constexpr int LPT = One::LPT, EPL = One::EPL, RW = RP * NS;
  One w[NS];
  int bad;  // a tile of the current item came from a bad table entry
  int d0;

  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int j = 0; j < NS; ++j) w[j].init(lane);
    d0 = w[0].d0;
  }
  __device__ __forceinline__ void begin(const DecodeArgs &a, int b, int g, int L, int row0) {
    bad = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) w[j].begin(a, b, g, L, row0 + j * RP);
  }
  __device__ __forceinline__ void restart() {
    bad = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) w[j].restart();
  }
  __device__ __forceinline__ void process(const uint4 (&kr)[One::NL], const uint4 (&vr)[One::NL],
                                          int t0, float scale_log2) {
#pragma unroll
    for (int j = 0; j < NS; ++j) w[j].process(kr, vr, t0, scale_log2);
  }
  __device__ __forceinline__ void totals(float (&l_row)[RW]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float l[RP];
      w[j].totals(l);
#pragma unroll
      for (int r = 0; r < RP; ++r) l_row[j * RP + r] = l[r];
    }
  }
  __device__ __forceinline__ float acc(int r, int e) const { return w[r / RP].acc[r % RP][e]; }
  __device__ __forceinline__ float m(int r) const { return w[r / RP].m_run[r % RP]; }
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
template <int DT, int D, int G, int RP, int NS, int kWaves>
__global__ void __launch_bounds__(kWaves * 64)
decode_partition_kernel(const DecodeArgs a) {
  using W = DecodeWaveSet<DT, D, G, RP, NS>;
  constexpr int RW = W::RW;  // query rows of this wavefront
  using Gm = Geo<DT, D>;
  constexpr int NL = Gm::NL, EPL = Gm::EPL;
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  constexpr int kStride = kWaves * kTile;  // tokens between a wavefront's tiles

  __shared__ float sm_acc[kWaves][RW][D];
  __shared__ float sm_m[kWaves][RW];
  __shared__ float sm_l[kWaves][RW];
  __shared__ int sm_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // blockIdx.y = slice * Hkv + KV head: the slices of one KV head are Hkv
  // workgroups apart, so they run on the same XCD and share its L2
  const int p = blockIdx.x, b = blockIdx.z;
  const int g = blockIdx.y % a.Hkv, row0 = (blockIdx.y / a.Hkv) * RW;
  const int nq = a.nq;
  const int L = load_const(a.lens + b);
  const int max_ctx = a.max_blocks * a.bs;

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
  const int t_begin = p * a.part_tokens;
  if (t_begin >= L) return;  // past this sequence's end: the reduce reads nothing here
  const int t_end = min(L, t_begin + a.part_tokens);

  W st;
  st.init(lane);
  st.begin(a, b, g, L, row0);

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
  auto table_at = [&](int k) {
    return load_const(trow + tile_t0(k < n_tiles ? k : n_tiles - 1) / a.bs);
  };
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
  float l_row[RW];
  st.totals(l_row);
  if (lane < W::LPT) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][r][st.d0 + e] = st.acc(r, e);
  }
  if (lane == 0) {  // bad is wavefront-uniform: it comes from scalar table reads
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      sm_m[wave][r] = st.m(r);
      sm_l[wave][r] = l_row[r];
    }
    sm_bad[wave] = st.bad;
  }
  __syncthreads();

  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any_bad |= sm_bad[w];
  const float nan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < RW * D; idx += kWaves * 64) {
    const int r = idx / D, d = idx % D, rr = row0 + r, qi = rr / G;
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
    const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + (rr % G);
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
// Stream kernel (stream-K decomposition) for mixed lengths and split
// contexts. All (sequence, KV head) units are laid end to end as one stream
// of 16-token tiles -- unit u = b * Hkv + g holds ceil(L_b / 16) tiles -- and
// persistent wavefront w takes tiles [w T / N, (w + 1) T / N) of it: every
// wavefront gets the same number of tiles, whatever the lengths. A
// wavefront's range is cut into segments at unit boundaries, at multiples of
// the requested partition size, and at its own ends; each segment leaves
// unnormalised partials (m, l, acc) under the id w + (global index of its
// partition), unique because both terms only grow along the stream. The
// reduce kernel finds a row's segments from the same arithmetic. No atomics,
// no LDS merge, no barriers after the prefix sums are built.
// ---------------------------------------------------------------------------
constexpr int kStreamWaves = 4;  // wavefronts per workgroup (independent)

// Stream geometry shared by the stream kernel and its reduce kernel.
struct StreamArgs {
  int32_t *tile_pre;  // [B + 1] tiles per unit, prefix over sequences
  int32_t *part_pre;  // [B + 1] partitions per unit, prefix over sequences
  int32_t n_waves;    // N
};

__device__ __forceinline__ int seq_tiles(int L, int nq, int max_ctx) {
  return (L >= nq && L <= max_ctx) ? (L + kTile - 1) / kTile : 0;
}
__device__ __forceinline__ int seq_parts(int L, int nq, int max_ctx, int P) {
  return (L >= nq && L <= max_ctx) ? (P > 0 ? (L + P - 1) / P : 1) : 0;
}
// Wavefront whose range holds stream tile `pos`: the largest w with
// floor(w T / N) <= pos.
__device__ __forceinline__ int64_t stream_wave(int64_t pos, int64_t T, int64_t N) {
  return ((pos + 1) * N + T - 1) / T - 1;
}

template <int DT, int D, int G, int RP, int NS>
__global__ void __launch_bounds__(kStreamWaves * 64)
decode_stream_kernel(const DecodeArgs a, const StreamArgs sa) {
  using W = DecodeWaveSet<DT, D, G, RP, NS>;
  constexpr int RW = W::RW;  // query rows of this wavefront
  using Gm = Geo<DT, D>;
  constexpr int NL = Gm::NL, EPL = Gm::EPL;
  constexpr int kThreads = kStreamWaves * 64;
  extern __shared__ int sm_dyn[];  // tile prefix [B + 1], then partition prefix [B + 1]
  __shared__ int sm_scan[2][kThreads];

  // Units: each sequence contributes HU = Hkv * slices of them, unit vg of
  // a sequence being KV head vg / slices, row slice vg % slices.
  const int B = a.B, P = a.part_tokens, nq = a.nq, S = a.slices, HU = a.Hkv * a.slices;
  const int max_ctx = a.max_blocks * a.bs;
  int *sm_tp = sm_dyn;
  int *sm_pp = sm_dyn + B + 1;

  // ---- prefix sums over sequences (every workgroup; workgroup 0 also
  //      leaves them in the workspace for the reduce kernel) ---------------
  {
    const int per = (B + kThreads - 1) / kThreads;
    const int lo = min(B, (int)threadIdx.x * per), hi = min(B, lo + per);
    int st_ = 0, sp_ = 0;
    for (int b = lo; b < hi; ++b) {
      const int L = load_const(a.lens + b);
      st_ += seq_tiles(L, nq, max_ctx);
      sp_ += seq_parts(L, nq, max_ctx, P);
    }
    sm_scan[0][threadIdx.x] = st_;
    sm_scan[1][threadIdx.x] = sp_;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scans
      const int v0 = threadIdx.x >= off ? sm_scan[0][threadIdx.x - off] : 0;
      const int v1 = threadIdx.x >= off ? sm_scan[1][threadIdx.x - off] : 0;
      __syncthreads();
      sm_scan[0][threadIdx.x] += v0;
      sm_scan[1][threadIdx.x] += v1;
      __syncthreads();
    }
    int rt = sm_scan[0][threadIdx.x] - st_, rp = sm_scan[1][threadIdx.x] - sp_;
    for (int b = lo; b < hi; ++b) {
      sm_tp[b] = rt;
      sm_pp[b] = rp;
      const int L = load_const(a.lens + b);
      rt += seq_tiles(L, nq, max_ctx);
      rp += seq_parts(L, nq, max_ctx, P);
    }
    if (threadIdx.x == kThreads - 1) {
      sm_tp[B] = sm_scan[0][kThreads - 1];
      sm_pp[B] = sm_scan[1][kThreads - 1];
    }
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i <= B; i += kThreads) {
        sa.tile_pre[i] = sm_tp[i];
        sa.part_pre[i] = sm_pp[i];
      }
  }

  const int64_t T = (int64_t)__builtin_amdgcn_readfirstlane(sm_tp[B]) * HU;
  const int64_t N = sa.n_waves;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kStreamWaves + (threadIdx.x >> 6));
  const int64_t pos0 = (int64_t)w * T / N, pos1 = (int64_t)(w + 1) * T / N;
  const int n_tiles = (int)(pos1 - pos0);
  if (n_tiles <= 0) return;
  const int lane = threadIdx.x & 63;
  const int ptiles = P > 0 ? P / kTile : 0;  // tiles per partition (0: unbounded)

  // A cursor is a tile of the stream: sequence b, unit g of the sequence
  // (KV head g / S, row slice g % S), tile k of the unit, plus the unit's
  // tile count and the sequence's length.
  struct Cursor {
    int b, g, k, nt, L;
  };
  auto locate = [&](int64_t pos) {
    int lo = 0, hi = B;  // HU * sm_tp[lo] <= pos < HU * sm_tp[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)__builtin_amdgcn_readfirstlane(sm_tp[mid]) * HU <= pos) lo = mid; else hi = mid;
    }
    Cursor c;
    c.b = lo;
    c.nt = __builtin_amdgcn_readfirstlane(sm_tp[lo + 1]) - __builtin_amdgcn_readfirstlane(sm_tp[lo]);
    const int local = (int)(pos - (int64_t)__builtin_amdgcn_readfirstlane(sm_tp[lo]) * HU);
    c.g = local / c.nt;
    c.k = local - c.g * c.nt;
    c.L = load_const(a.lens + lo);
    return c;
  };
  auto step = [&](Cursor &c) {  // the next tile of the stream
    if (++c.k < c.nt) return;
    c.k = 0;
    if (++c.g < HU) return;
    c.g = 0;
    do {  // next sequence that has tiles
      ++c.b;
      c.L = c.b < B ? load_const(a.lens + c.b) : 0;
      c.nt = c.b < B ? seq_tiles(c.L, nq, max_ctx) : 1;
    } while (c.nt == 0);
  };
  auto table_entry = [&](const Cursor &c) {
    return load_const(a.tables + (size_t)c.b * a.max_blocks + (c.k * kTile) / a.bs);
  };

  W st;
  st.init(lane);
  const char *kbase = (const char *)a.kc;
  const char *vbase = (const char *)a.vc;
  auto offset = [&](const Cursor &c, int blk, int &tile_bad) -> size_t {
    tile_bad = blk < 0 || blk >= a.num_blocks;
    return tile_bytes_offset<Gm::TB>(a, c.g / S, c.k * kTile, tile_bad ? 0 : blk, lane);
  };

  Cursor cur = locate(pos0);
  st.begin(a, cur.b, cur.g / S, cur.L, (cur.g % S) * RW);
  int left = n_tiles;  // tiles of this wavefront not yet consumed
  Cursor iss = cur;
  if (n_tiles > 1) step(iss);
  Cursor pre = iss;
  if (n_tiles > 2) step(pre);
  int issued = 1;  // tiles whose loads have been issued
  int bad_a = 0, bad_b = 0;
  const size_t off0 = offset(cur, table_entry(cur), bad_a);
  int blk_iss = n_tiles > 1 ? table_entry(iss) : 0;
  int blk_pre = n_tiles > 2 ? table_entry(pre) : 0;

  auto issue = [&](uint4 (&kr)[NL], uint4 (&vr)[NL], int &tile_bad) {
    const size_t off = offset(iss, blk_iss, tile_bad);
    load_tile<NL>(kr, vr, kbase + off, vbase + off);
    ++issued;
    iss = pre;
    blk_iss = blk_pre;
    if (issued + 1 < n_tiles) {
      step(pre);
      blk_pre = table_entry(pre);
    }
  };
  // Consume the tile at `cur`; close the segment when the tile ends the
  // unit, a partition, or this wavefront's range.
  auto consume = [&](const uint4 (&kr)[NL], const uint4 (&vr)[NL], int tile_bad) {
    st.bad |= tile_bad;
    st.process(kr, vr, cur.k * kTile, a.scale_log2);
    --left;
    const bool unit_end = cur.k + 1 == cur.nt;
    const bool part_end = ptiles > 0 && (cur.k + 1) % ptiles == 0;
    if (!(unit_end || part_end || left == 0)) {
      ++cur.k;
      return;
    }
    float l_row[RW];
    st.totals(l_row);
    const int p = ptiles > 0 ? cur.k / ptiles : 0;
    const int64_t gp = (int64_t)__builtin_amdgcn_readfirstlane(sm_pp[cur.b]) * HU +
                       (int64_t)cur.g * (sm_pp[cur.b + 1] - sm_pp[cur.b]) + p;
    const int64_t sid = w + gp;
    const float nan = __builtin_nanf("");
    if (lane < W::LPT) {
      float *dst = a.part_acc + (size_t)sid * RW * D + st.d0;
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[r * D + e] = st.acc(r, e);
      if (lane == 0)
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          a.part_m[(size_t)sid * RW + r] = st.bad ? nan : st.m(r);
          a.part_l[(size_t)sid * RW + r] = l_row[r];
        }
    }
    if (left == 0) return;
    const int b0 = cur.b, g0 = cur.g;
    step(cur);
    if (cur.b != b0 || cur.g != g0)
      st.begin(a, cur.b, cur.g / S, cur.L, (cur.g % S) * RW);
    else  // a new partition of the same unit: same queries, fresh statistics
      st.restart();
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

// Merge of the stream kernel's segments: one workgroup per (query row,
// sequence), thread d owns output element d.
template <int D, int RW, int G>
__global__ void __launch_bounds__(D)
reduce_stream_kernel(const DecodeArgs a, const StreamArgs sa) {
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  const int rowq = blockIdx.x;  // qi * Hq + h
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int nq = a.nq, P = a.part_tokens, HU = a.Hkv * a.slices;
  const int qi = rowq / a.Hq, h = rowq % a.Hq;
  const int rr = qi * G + (h % G);             // row within the KV head
  const int vg = (h / G) * a.slices + rr / RW;  // its unit within the sequence
  const int r = rr % RW;                        // its row within the unit
  const size_t row = (size_t)b * nq * a.Hq + rowq;
  const float nan = __builtin_nanf("");
  const int L = load_const(a.lens + b);
  if (L < nq || L > a.max_blocks * a.bs) {
    a.out[row * D + d] = nan;
    if (d == 0 && a.lse) a.lse[row] = nan;
    return;
  }
  const int64_t T = (int64_t)sa.tile_pre[a.B] * HU;
  const int64_t N = sa.n_waves;
  const int nt = sa.tile_pre[b + 1] - sa.tile_pre[b];
  const int np = sa.part_pre[b + 1] - sa.part_pre[b];
  const int64_t u0 = (int64_t)sa.tile_pre[b] * HU + (int64_t)vg * nt;  // first tile of the unit
  const int64_t gp0 = (int64_t)sa.part_pre[b] * HU + (int64_t)vg * np;
  const int ptiles = P > 0 ? P / kTile : nt;
  // pass 1: maximum
  float M = kNegInf;
  bool bad = false;
  // the wavefronts holding a partition's tiles, in order: from the one that
  // holds its first tile, hop to the one holding the tile after each range
  // (wavefronts with empty ranges hold no segment)
  for (int p = 0; p < np; ++p) {
    const int64_t first = u0 + (int64_t)p * ptiles;
    const int64_t last = u0 + min(nt, (p + 1) * ptiles) - 1;
    for (int64_t pos = first; pos <= last;) {
      const int64_t ww = stream_wave(pos, T, N);
      pos = (ww + 1) * T / N;
      const float m = a.part_m[(size_t)(ww + gp0 + p) * RW + r];
      bad |= m != m;
      M = fmaxf(M, m);
    }
  }
  float num = 0.f, den = 0.f;
  for (int p = 0; p < np; ++p) {
    const int64_t first = u0 + (int64_t)p * ptiles;
    const int64_t last = u0 + min(nt, (p + 1) * ptiles) - 1;
    for (int64_t pos = first; pos <= last;) {
      const int64_t ww = stream_wave(pos, T, N);
      pos = (ww + 1) * T / N;
      const size_t sid = (size_t)(ww + gp0 + p);
      const float m = a.part_m[sid * RW + r];
      const float f = m == kNegInf ? 0.f : exp2f(m - M);
      num = fmaf(f, a.part_acc[(sid * RW + r) * D + d], num);
      den = fmaf(f, a.part_l[sid * RW + r], den);
    }
  }
  a.out[row * D + d] = bad || den == 0.f ? nan : num / den;
  if (d == 0 && a.lse) a.lse[row] = bad || den == 0.f ? nan : (M + log2f(den)) * kLn2;
}

using Launcher = void (*)(const DecodeArgs &, const StreamArgs &, dim3, hipStream_t);

template <int DT, int D, int G, int RP, int NS, int W>
void launch_decode(const DecodeArgs &a, const StreamArgs &sa, dim3 grid, hipStream_t s) {
  if constexpr (W == 0) {  // stream kernel + its reduce; grid.x persistent workgroups
    hipLaunchKernelGGL((decode_stream_kernel<DT, D, G, RP, NS>), grid, dim3(kStreamWaves * 64),
                       2 * (a.B + 1) * sizeof(int), s, a, sa);
    hipLaunchKernelGGL((reduce_stream_kernel<D, RP * NS, G>), dim3(a.nq * a.Hq, a.B), dim3(D),
                       0, s, a, sa);
  } else {
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, RP, NS, W>), grid, dim3(W * 64), 0, s,
                       a);
  }
}

// Launcher for (dtype, D) and rows per wavefront RP = G * (query tokens
// rounded up to a power of two): W = 4 or 8 wavefronts per workgroup of the
// workgroup-split kernel, or W = 0 for the stream kernel (which also
// launches its reduce); nullptr if no such kernel is built. Defined in
// decode_inst_<dtype>_d<D>.hip.
template <int DT, int D>
Launcher pick_rows(int G, int RP, int NS, int W);

// Most query rows per KV head on the VALU kernels (as up to 4 slices of 4).
constexpr int kMaxRows = 16;

}  // namespace decode
}  // namespace pkv
