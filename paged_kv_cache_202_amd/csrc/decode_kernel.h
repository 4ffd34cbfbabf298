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
//     head is a contiguous 16 * D-element run of one block, gathered with
//     one 16-byte direct-to-LDS load per lane per 1 KiB (fully coalesced)
//     into a per-wavefront ring of LDS slots: tiles in flight hold no
//     registers, so two (16 KiB) stay in flight per wavefront even with
//     eight query rows. Each lane reads back the 16 bytes it gathered --
//     its slice of D for a few tokens -- just before the tile is used.
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
// The same with a zero accumulator, in the three-operand form that takes
// the zero as an inline constant (the two-operand form the compiler picks
// for chains would first need a register cleared).
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// q.k of two fp16 pairs into an fp32 sum (v_dot2_f32_f16: exact products).
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                c, false);
}

// Two int8 codes (bytes 0 and 1, or 2 and 3, of w) as the fp16 pair
// (1152 + c0, 1152 + c1): with u = c + 128 in 0..255, the fp16 whose bits
// are 0x6400 | u is exactly 1024 + u, so the conversion is byte moves only.
// (v_perm_b32 picks each result byte from the 8 bytes {S0, S1}, S1 being
// bytes 0..3: S0 = 0x64646464 supplies the high bytes.)
__device__ __forceinline__ uint32_t codes_f16_lo(uint32_t w) {
  return __builtin_amdgcn_perm(0x64646464u, w ^ 0x80808080u, 0x04010400u);
}
__device__ __forceinline__ uint32_t codes_f16_hi(uint32_t w) {
  return __builtin_amdgcn_perm(0x64646464u, w ^ 0x80808080u, 0x04030402u);
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
  // every lane reads a valid source lane for the patterns used here, so the
  // previous value of the destination is never kept and needs no set-up
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
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

// The lane exactly lane ^ M (M >= 4): unlike xor_partner, lower lane bits are
// preserved, as needed when lanes below M hold different data.
template <int M>
__device__ __forceinline__ float exact_xor(float x) {
  if constexpr (M == 4) {  // (final sums only) a bit-mode swizzle: xor mask 4
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101f));
  } else if constexpr (M == 8) {
    return dpp_mov<0x128>(x);  // row_ror:8 within a 16-lane row is lane ^ 8
  } else {
    static_assert(M == 16 || M == 32, "exact_xor covers lane bits 2..5");
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

// Element type of caches of 3-bit codes, two per byte (low nibble first),
// each stored as code + 8; an internal type of the decode kernels.
constexpr int kCodes3 = 3;

// Geometry of one (dtype, head dim) pair as seen by a wavefront.
template <int DT, int D>
struct Geo {
  static constexpr int ES = DT == PKV_F32 ? 4 : 2;  // bytes per element (fp32, bf16)
  static constexpr int TB = D * ES;                   // bytes per token row
  static constexpr int LB = 16;                       // bytes of a row a lane holds
  static constexpr int LPT = TB / LB;                // lanes sharing one token
  static constexpr int TPL = 64 / LPT;               // tokens per load row
  static constexpr int NL = kTile / TPL;             // loads per lane per tile
  static constexpr int EPL = 16 / ES;  // elements per lane per load
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
  // Shared-prefix launches only (else nullptr / 0): starts[b] tokens of
  // sequence b are covered by its group's prefix phase, which writes
  // partition slots [0, part_base) in prefix_part-token pieces; the
  // ordinary kernels cover [starts[b], L) from slot part_base on.
  const int32_t *starts;
  int32_t part_base;
  int32_t prefix_part;
  // Caches of codes only (the matrix-core code kernel; else nullptr): the
  // float32 scale of each (block, KV head, slot) row, K and V side by side,
  // [num_blocks, Hkv, 2 (K, V), bs].
  const float *scales;
  // MFMA decode kernel only: > 0 makes its wavefronts independent, each
  // streaming a run of this many consecutive partitions through its ring and
  // writing the run's partials into its first partition's slot (the reduce
  // reads those slots only); 0: the wavefronts of a workgroup share one
  // partition and merge in LDS.
  int32_t parts_per_wg;
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

#define PKV_LDS __attribute__((address_space(3)))

// Cache policy of the K/V gathers: non-temporal. Every K/V byte is read once
// per call, so the rows should not displace reusable lines (tables, queries).
constexpr int kKvNonTemporal = 2;


// N (2, 4 or 8) 16-byte LDS reads at p, p + 1 KiB, ..., and a wait for
// them, in one statement so that no use of a result can be scheduled before
// the wait.
template <int N>
__device__ __forceinline__ void lds_rows(u32x4_t *t, const PKV_LDS char *p) {
  if constexpr (N == 2) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1])
        : "v"(p)
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
        : "v"(p)
        : "memory");
  } else {
    static_assert(N == 8, "2, 4 or 8 rows per read");
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
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]),
          "=&v"(t[6]), "=&v"(t[7])
        : "v"(p)
        : "memory");
  }
}

// One 1 KiB direct-to-LDS gather: lane i's 16 bytes from src (per lane)
// land at dst + 16 i (dst wavefront-uniform). AUX is the cache policy.
template <int AUX>
__device__ __forceinline__ void gather_lds16(const char *src, PKV_LDS char *dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, AUX);
}
// The same with 4 bytes per lane (256 bytes).
template <int AUX>
__device__ __forceinline__ void gather_lds4(const char *src, PKV_LDS char *dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, AUX);
}

// A value a loop reads, waited for here and kept in a register from here
// on: if its load were first used inside the loop, the compiler's wait for
// it would sit in every trip and also wait for the gathers in flight.
// (Device functions: AMDGPU register constraints cannot appear in a kernel
// body, which the host compiler also checks.)
__device__ __forceinline__ void settle_s(float &x) { asm volatile("" : "+s"(x)); }
__device__ __forceinline__ void settle_v(int &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle_v(uint4 &x) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}

// Wait until at most VM vector-memory operations of this wavefront are
// pending.
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt is six bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(VM) : "memory");
}

// Wait until at most ahead * L vector-memory operations are pending, for a
// wavefront-uniform ahead in [0, S) of a ring of S slots. `steady` must be
// ahead == S - 1 (a full ring ahead), given as its own condition: tested
// first, the common case costs one compare and branch; tested as a value of
// ahead, the compiler folds it into a search over all S cases.
template <int S, int L>
__device__ __forceinline__ void wait_ahead(bool steady, int ahead) {
  if (steady) {
    wait_vmcnt<(S - 1) * L>();
    return;
  }
  static_for<S - 1>([&](auto ac) {
    constexpr int A = decltype(ac)::value;
    if (ahead == A) wait_vmcnt<A * L>();
  });
}

// ---------------------------------------------------------------------------
// Per-wavefront ring of LDS slots that K/V tiles are gathered into with
// direct-to-LDS loads (global_load_lds_dwordx4: lane i's 16 bytes land at
// slot + 16 i). A tile in flight holds no VGPRs; it is read back into
// registers, one 16-byte row piece per lane, just before it is consumed.
// Slot layout: K rows 0 .. NL-1 (1 KiB each, one per load), then V rows.
// The wavefront waits for its own loads only (vmcnt), so the ring needs no
// barrier; the compiler cannot track which LDS bytes a pending DMA writes,
// so the read-back and its waits are written out here.
// ---------------------------------------------------------------------------
template <int NL, bool SC = false, int kRowBudget = 16384>
struct TileRing {
  static constexpr int kCodeBytes = 2 * NL * 1024;
  // with per-row scales (code caches), after the K and V rows: the tile's 16
  // K scales, its 16 V scales, and 128 bytes the other lanes of their
  // 4-byte gather fill with copies (every lane takes part: a gather under a
  // lane mask could be split by the compiler into several instructions,
  // which would break the counting of loads in flight)
  static constexpr int kTileBytes = kCodeBytes + (SC ? 256 : 0);
  // at least one tile, else as many as fit the budget of rows (16 KiB: two
  // tiles of a D = 128 bf16 head, four of a D = 64 one)
  static constexpr int kSlots = kCodeBytes >= kRowBudget ? 1 : kRowBudget / kCodeBytes;
  static constexpr int kBytes = kSlots * kTileBytes;  // per wavefront
  static constexpr int kLoads = 2 * NL + (SC ? 1 : 0);  // DMA instructions per tile
  static_assert((kSlots & (kSlots - 1)) == 0, "slot count must be a power of two");

  PKV_LDS char *base;  // this wavefront's ring (wavefront-uniform)
  const PKV_LDS char *mine;  // base + 16 * lane

  __device__ __forceinline__ void init(PKV_LDS char *ring, int lane) {
    base = ring;
    mine = ring + lane * 16;
  }

  // Gather one tile into `slot`: kp / vp already include this lane's 16 B.
  // With scales, sp is this lane's 4 bytes of them: lane l takes K scale
  // l % 16 (l % 32 < 16) or V scale l % 16 (otherwise); issued first, so
  // that waiting for the K rows also covers both scales.
  __device__ __forceinline__ void stage(int slot, const char *kp, const char *vp,
                                        const char *sp = nullptr) {
    PKV_LDS char *dst = base + slot * kTileBytes;
    if constexpr (SC) gather_lds4<kKvNonTemporal>(sp, dst + kCodeBytes);
#pragma unroll
    for (int i = 0; i < NL; ++i) gather_lds16<kKvNonTemporal>(kp + i * 1024, dst + i * 1024);
#pragma unroll
    for (int i = 0; i < NL; ++i)
      gather_lds16<kKvNonTemporal>(vp + i * 1024, dst + (NL + i) * 1024);
  }

  // Read back the K half (HALF = 0) or the V half (HALF = 1) of the tile in
  // `slot` once its gathers have landed. `ahead` (wavefront-uniform, below
  // kSlots) whole tiles were staged after it and stay in flight:
  // vector-memory loads complete in issue order, so the wait leaves exactly
  // those (and, for K, this tile's V rows) pending. Other loads or stores
  // issued later only make the wait stricter. Only the wait depends on
  // `ahead`, so the reads themselves are not duplicated per case.
  template <int HALF>
  __device__ __forceinline__ void fetch(int slot, int ahead, uint4 (&r)[NL]) const {
    static_for<kSlots>([&](auto ac) {
      constexpr int A = decltype(ac)::value;
      if (ahead == A) wait_vmcnt<A * kLoads + (HALF == 0 ? NL : 0)>();
    });
    const PKV_LDS char *p = mine + slot * kTileBytes + HALF * NL * 1024;
    u32x4_t t[NL];
    if constexpr (NL == 1) {
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(t[0]) : "v"(p) : "memory");
    } else if constexpr (NL <= 8) {
      lds_rows<NL>(t, p);
    } else {
#pragma unroll
      for (int c = 0; c < NL / 8; ++c) lds_rows<8>(t + 8 * c, p + c * 8192);
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) r[i] = make_uint4(t[i].x, t[i].y, t[i].z, t[i].w);
  }
};

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
  using Row = uint4;  // what one load gives a lane: 16 bytes

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

  // Consume one 16-token tile starting at logical token t0: its K rows are
  // in kr, and get_v(vr) supplies its V rows once the weights are known (so
  // the V half of a gather may still be landing during the q.k work).
  template <class GetV>
  __device__ __forceinline__ void process(const Row (&kr)[NL], GetV &&get_v, int t0,
                                          float scale_log2) {
    // partial q.k over this lane's EPL dims: x[r * NL + i]
    float x[V];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float s = 0.f;
        if constexpr (DT == PKV_BF16) {
          s = dot2_bf16_first(qw[r][0], kr[i].x);
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
    // their V is zeroed (before widening) so that 0 * NaN cannot reach acc
    Row vr[NL];
    get_v(vr);
    if (t0 + kTile > min_lim) {  // wavefront-uniform: only a context's last tile
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (t0 + i * TPL + grp >= L) vr[i] = make_uint4(0u, 0u, 0u, 0u);
    }
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
  constexpr int RW = RP;  // query rows of this wavefront
  using Gm = Geo<DT, D>;
  constexpr int NL = Gm::NL, EPL = Gm::EPL;
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  constexpr int kStride = kWaves * kTile;  // tokens between a wavefront's tiles
  using Ring = TileRing<NL>;
  constexpr int kSlots = Ring::kSlots;

  // the tile rings while streaming; the wavefronts' partials once done
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
  auto &sm_acc = sm.mg.acc;
  auto &sm_m = sm.mg.m;
  auto &sm_l = sm.mg.l;
  auto &sm_bad = sm.mg.bad;

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
  // earlier tokens belong to the prefix phase (clamped: bad values cannot
  // send reads outside the table)
  const int start = a.starts ? min(max(load_const(a.starts + b), 0), L) : 0;
  const int t_begin = start + p * a.part_tokens;
  if (t_begin >= L) return;  // past this sequence's end: the reduce reads nothing here
  const int t_end = min(L, t_begin + a.part_tokens);

  W st;
  st.init(lane);
  st.begin(a, b, g, L, row0);

  const int32_t *trow = a.tables + (size_t)b * a.max_blocks;
  const char *kbase = (const char *)a.kc;
  const char *vbase = (const char *)a.vc;
  // gather the tile at logical token t0 (from block blk) into a ring slot
  auto stage_tile = [&](auto &ring, int slot, int t0, int blk) {
    if (blk < 0 || blk >= a.num_blocks) {  // bad table entry: read block 0, poison later
      st.bad = 1;
      blk = 0;
    }
    const size_t off = tile_bytes_offset<Gm::TB>(a, g, t0, blk, lane);
    ring.stage(slot, kbase + off, vbase + off);
  };

  // Pipeline: up to kSlots tiles are gathered into the wavefront's LDS ring
  // ahead of the one being consumed; a slot is refilled as soon as its tile
  // has been read back.
  const int n_tiles = t_begin + wave * kTile < t_end
                          ? (t_end - (t_begin + wave * kTile) + kStride - 1) / kStride
                          : 0;
  auto tile_t0 = [&](int k) { return t_begin + wave * kTile + k * kStride; };
  // Block ids: lane i holds that of this wavefront's tile 64 w + i of the
  // current window w (one vector load per 64 tiles, read out with
  // v_readlane; no scalar load inside the loop).
  auto table_window = [&](int w) {
    return trow[tile_t0(min(64 * w + lane, n_tiles - 1)) / a.bs];
  };
  if (n_tiles > 0) {
    int tblv = table_window(0);
    settle_v(tblv);
    auto table_at = [&](int k) { return __builtin_amdgcn_readlane(tblv, k & 63); };
    Ring ring;
    ring.init((PKV_LDS char *)&sm.ring[0] + wave * Ring::kBytes, lane);
#pragma unroll
    for (int k = 0; k < kSlots; ++k)
      if (k < n_tiles) stage_tile(ring, k, tile_t0(k), table_at(k));
    // the scale is waited for here, not at its first use inside the loop,
    // where the wait would also catch each step's block-id read
    float scale_log2 = a.scale_log2;
    settle_s(scale_log2);
    for (int k = 0; k < n_tiles; ++k) {
      const int slot = k & (kSlots - 1);
      const int ahead = min(n_tiles - 1 - k, kSlots - 1);
      typename W::Row kr[NL];
      ring.template fetch<0>(slot, ahead, kr);
      st.process(
          kr,
          [&](typename W::Row (&vr)[NL]) {
            ring.template fetch<1>(slot, ahead, vr);
            if (k + kSlots < n_tiles) {  // the slot is free again: refill it
              const int kn = k + kSlots;
              if ((kn & 63) == 0) {  // next window of block ids (drains the ring once)
                tblv = table_window(kn >> 6);
                settle_v(tblv);
              }
              stage_tile(ring, slot, tile_t0(kn), table_at(kn));
            }
          },
          tile_t0(k), scale_log2);
    }
  }

  // ---- wavefront totals, then merge the wavefronts in LDS ------------------
  float l_row[RW];
  st.totals(l_row);
  __syncthreads();  // the partials overwrite the other wavefronts' rings
  if (lane < W::LPT) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][r][st.d0 + e] = st.acc[r][e];
  }
  if (lane == 0) {  // bad is wavefront-uniform: it comes from scalar table reads
#pragma unroll
    for (int r = 0; r < RW; ++r) {
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
      const size_t pi = row * a.num_parts + a.part_base + p;
      a.part_acc[pi * D + d] = num;
      if (d == 0) {
        a.part_m[pi] = any_bad ? nan : M;
        a.part_l[pi] = den;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stream kernel (stream-K decomposition) for batches of mixed lengths. All
// (sequence, KV head slice) units are laid end to end as one stream of
// 16-token tiles -- unit u = b * HU + g holds ceil(L_b / 16) tiles -- and
// persistent wavefront w takes tiles [w T / N, (w + 1) T / N) of it: every
// wavefront gets the same number of tiles, whatever the lengths. A
// wavefront's range is cut into segments at unit boundaries and at its own
// ends; each segment leaves unnormalised partials (m, l, acc) under the id
// w + u, unique because both terms only grow along the stream. The
// wavefronts holding a unit's tiles are consecutive, so the reduce kernel
// finds a unit's segments from its first and last tile alone. No atomics,
// no LDS merge, no barriers after the prefix sums are built.
// ---------------------------------------------------------------------------
constexpr int kStreamWaves = 4;  // wavefronts per workgroup (independent)

// Stream geometry shared by the stream kernel and its reduce kernel.
struct StreamArgs {
  int32_t *tile_pre;  // [B + 1] slots per unit, prefix over sequences
  int32_t n_waves;    // N
  // slots without work at the head of each unit with tiles (0 here: a
  // unit's slots are its tiles; the matrix-core stream mode charges each
  // unit the cost of starting a segment)
  int32_t seg_cost;
};

__device__ __forceinline__ int seq_tiles(int L, int nq, int max_ctx) {
  return (L >= nq && L <= max_ctx) ? (L + kTile - 1) / kTile : 0;
}
// Wavefront whose range holds stream tile `pos`: the largest w with
// floor(w T / N) <= pos.
__device__ __forceinline__ int64_t stream_wave(int64_t pos, int64_t T, int64_t N) {
  return ((pos + 1) * N + T - 1) / T - 1;
}

template <int DT, int D, int G, int RP>
__global__ void __launch_bounds__(kStreamWaves * 64)
decode_stream_kernel(const DecodeArgs a, const StreamArgs sa) {
  using W = DecodeWave<DT, D, G, RP>;
  constexpr int RW = RP;  // query rows of this wavefront
  using Gm = Geo<DT, D>;
  constexpr int NL = Gm::NL, EPL = Gm::EPL;
  constexpr int kThreads = kStreamWaves * 64;
  using Ring = TileRing<NL>;
  constexpr int kSlots = Ring::kSlots;
  extern __shared__ int sm_tp[];  // tile prefix [B + 1]
  __shared__ int sm_scan[kThreads];
  __shared__ u32x4_t sm_ring[kStreamWaves * Ring::kBytes / 16];

  // Units: each sequence contributes HU = Hkv * slices of them, unit vg of
  // a sequence being KV head vg / slices, row slice vg % slices.
  const int B = a.B, nq = a.nq, S = a.slices, HU = a.Hkv * a.slices;
  const int max_ctx = a.max_blocks * a.bs;

  // ---- prefix sum of tiles over sequences (every workgroup; workgroup 0
  //      also leaves it in the workspace for the reduce kernel) ------------
  {
    const int per = (B + kThreads - 1) / kThreads;
    const int lo = min(B, (int)threadIdx.x * per), hi = min(B, lo + per);
    int st_ = 0;
    for (int b = lo; b < hi; ++b) st_ += seq_tiles(load_const(a.lens + b), nq, max_ctx);
    sm_scan[threadIdx.x] = st_;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan
      const int v = threadIdx.x >= off ? sm_scan[threadIdx.x - off] : 0;
      __syncthreads();
      sm_scan[threadIdx.x] += v;
      __syncthreads();
    }
    int rt = sm_scan[threadIdx.x] - st_;
    for (int b = lo; b < hi; ++b) {
      sm_tp[b] = rt;
      rt += seq_tiles(load_const(a.lens + b), nq, max_ctx);
    }
    if (threadIdx.x == kThreads - 1) sm_tp[B] = sm_scan[kThreads - 1];
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i <= B; i += kThreads) sa.tile_pre[i] = sm_tp[i];
  }

  const int64_t T = (int64_t)__builtin_amdgcn_readfirstlane(sm_tp[B]) * HU;
  const int64_t N = sa.n_waves;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kStreamWaves + (threadIdx.x >> 6));
  const int64_t pos0 = (int64_t)w * T / N, pos1 = (int64_t)(w + 1) * T / N;
  const int n_tiles = (int)(pos1 - pos0);
  if (n_tiles <= 0) return;
  const int lane = threadIdx.x & 63;

  // A cursor is a tile of the stream: sequence b, unit g of the sequence
  // (KV head g / S, row slice g % S), tile k of the unit, plus the unit's
  // tile count and the sequence's length (kept in registers: once gathers
  // are in flight, no LDS reads but the ring's).
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

  Ring ring;
  ring.init((PKV_LDS char *)&sm_ring[0] + (threadIdx.x >> 6) * Ring::kBytes, lane);

  Cursor cur = locate(pos0);  // the tile to consume next
  st.begin(a, cur.b, cur.g / S, cur.L, (cur.g % S) * RW);
  Cursor iss = cur;    // the tile to gather next
  int blk_iss = table_entry(iss);
  int issued = 0;     // tiles whose gathers have been issued
  int bad_slots = 0;  // bit s: the tile in slot s came from a bad table entry

  auto issue = [&](int slot) {
    int tile_bad;
    const size_t off = offset(iss, blk_iss, tile_bad);
    ring.stage(slot, kbase + off, vbase + off);
    bad_slots = (bad_slots & ~(1 << slot)) | (tile_bad << slot);
    if (++issued < n_tiles) {  // block id of the next gather, read ahead
      step(iss);
      blk_iss = table_entry(iss);
    }
  };
  float scale_log2 = a.scale_log2;  // waited for here (see the other kernel)
  settle_s(scale_log2);

#pragma unroll
  for (int s = 0; s < kSlots; ++s)
    if (s < n_tiles) issue(s);
  // Segments: runs of tiles of one unit that end at the unit's end or at
  // this wavefront's end. The per-tile loop stays free of the segment
  // bookkeeping; gathers run ahead across segments.
  int i = 0;  // tiles consumed
  for (;;) {
    const int n_seg = min(cur.nt - cur.k, n_tiles - i);
    const int k0 = cur.k;
    for (int j = 0; j < n_seg; ++j, ++i) {
      const int slot = i & (kSlots - 1);
      const int ahead = min(n_tiles - 1 - i, kSlots - 1);
      uint4 kr[NL];
      ring.template fetch<0>(slot, ahead, kr);
      st.bad |= (bad_slots >> slot) & 1;
      st.process(
          kr,
          [&](uint4 (&vr)[NL]) {
            ring.template fetch<1>(slot, ahead, vr);
            if (issued < n_tiles) issue(slot);  // the slot is free again
          },
          (k0 + j) * kTile, scale_log2);
    }
    cur.k = k0 + n_seg - 1;  // the segment's last tile

    // close the segment: unnormalised partials under its id
    float l_row[RW];
    st.totals(l_row);
    const int64_t sid = w + (int64_t)cur.b * HU + cur.g;
    const float nan = __builtin_nanf("");
    if (lane < W::LPT) {
      float *dst = a.part_acc + (size_t)sid * RW * D + st.d0;
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[r * D + e] = st.acc[r][e];
      if (lane == 0)
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          a.part_m[(size_t)sid * RW + r] = st.bad ? nan : st.m_run[r];
          a.part_l[(size_t)sid * RW + r] = l_row[r];
        }
    }
    if (i == n_tiles) break;
    const int b0 = cur.b, g0 = cur.g;
    step(cur);
    if (cur.b != b0 || cur.g != g0)
      st.begin(a, cur.b, cur.g / S, cur.L, (cur.g % S) * RW);
    else  // a new partition of the same unit: same queries, fresh statistics
      st.restart();
  }
}

// Merge of the stream kernels' segments (this file's VALU kernel and the
// matrix-core kernel's stream mode): one workgroup per (unit, sequence) --
// grid (Hkv * slices, B) -- holding the unit's RW rows, D / 4 threads per
// row and four output elements per thread; two passes over the unit's
// segments w + u, w = w0 .. w1 (their maximum, then the weighted sums), so
// that the loads of each pass are independent.
template <int D, int RW>
__global__ void __launch_bounds__(RW * D / 4)
reduce_stream_kernel(const DecodeArgs a, const StreamArgs sa) {
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  constexpr int TPR = D / 4;  // threads per row
  const int vg = blockIdx.x, b = blockIdx.y;  // unit within the sequence, sequence
  const int r = threadIdx.x / TPR, d4 = (threadIdx.x % TPR) * 4;
  const int nq = a.nq, S = a.slices, HU = a.Hkv * S, G = a.Hq / a.Hkv;
  const int g = vg / S, rr = (vg % S) * RW + r;  // KV head, row within it
  if (rr >= G * nq) return;                      // a padding row of the unit
  const int qi = rr / G;
  const size_t row = ((size_t)b * nq + qi) * a.Hq + g * G + rr % G;
  const float nan = __builtin_nanf("");
  float4 *dst = reinterpret_cast<float4 *>(a.out + row * D + d4);
  // the sequence's metadata in one round of independent loads
  const int L = load_const(a.lens + b);
  const int pre_b = load_const(sa.tile_pre + b), pre_b1 = load_const(sa.tile_pre + b + 1);
  const int pre_all = load_const(sa.tile_pre + a.B);
  if (L < nq || L > a.max_blocks * a.bs) {
    *dst = make_float4(nan, nan, nan, nan);
    if (d4 == 0 && a.lse) a.lse[row] = nan;
    return;
  }
  const int64_t T = (int64_t)pre_all * HU;
  const int64_t N = sa.n_waves;
  const int span = pre_b1 - pre_b, nt = span - sa.seg_cost;  // slots, tiles per unit
  const int64_t first = (int64_t)pre_b * HU + (int64_t)vg * span + sa.seg_cost;  // first tile
  const int64_t w0 = stream_wave(first, T, N), w1 = stream_wave(first + nt - 1, T, N);
  const int64_t u = (int64_t)b * HU + vg;
  // with fewer tiles than wavefronts, some wavefronts hold none (and wrote
  // nothing under their id)
  auto held = [&](int64_t w) { return T >= N || w * T / N != (w + 1) * T / N; };
  float M = kNegInf;
  bool bad = false;
#pragma unroll 4
  for (int64_t w = w0; w <= w1; ++w) {
    const float m = held(w) ? a.part_m[(size_t)(w + u) * RW + r] : kNegInf;
    bad |= m != m;
    M = fmaxf(M, m);
  }
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (M != kNegInf) {
#pragma unroll 4
    for (int64_t w = w0; w <= w1; ++w) {
      if (!held(w)) continue;
      const size_t si = (size_t)(w + u) * RW + r;
      const float m = a.part_m[si];
      // no visible key in the segment: weight 0 (m = -inf)
      const float f = m == kNegInf ? 0.f : exp2f(m - M);
      const float4 v = *reinterpret_cast<const float4 *>(a.part_acc + si * D + d4);
      num.x = fmaf(f, v.x, num.x);
      num.y = fmaf(f, v.y, num.y);
      num.z = fmaf(f, v.z, num.z);
      num.w = fmaf(f, v.w, num.w);
      den = fmaf(f, a.part_l[si], den);
    }
  }
  const bool dead = bad || den == 0.f;
  *dst = dead ? make_float4(nan, nan, nan, nan)
              : make_float4(num.x / den, num.y / den, num.z / den, num.w / den);
  if (d4 == 0 && a.lse) a.lse[row] = dead ? nan : (M + log2f(den)) * kLn2;
}

using Launcher = void (*)(const DecodeArgs &, const StreamArgs &, dim3, hipStream_t);

// Bytes of LDS one workgroup may allocate on gfx950.
constexpr int kLdsLimit = 163840;

// LDS of the stream kernel for B sequences: the tile rings and the scan
// array, plus the per-sequence tile prefix.
template <int DT, int D>
constexpr int64_t stream_lds_bytes(int64_t B) {
  return (int64_t)kStreamWaves * TileRing<Geo<DT, D>::NL>::kBytes +
         kStreamWaves * 64 * (int64_t)sizeof(int) + (B + 1) * (int64_t)sizeof(int);
}

template <int DT, int D, int G, int RP, int W>
void launch_decode(const DecodeArgs &a, const StreamArgs &sa, dim3 grid, hipStream_t s) {
  // eight wavefronts' tile rings must fit the workgroup's LDS
  constexpr int kRing = TileRing<Geo<DT, D>::NL>::kBytes;
  if constexpr (W == 8 && 8 * kRing > kLdsLimit) {
    launch_decode<DT, D, G, RP, 4>(a, sa, grid, s);
  } else if constexpr (W == 0) {  // stream kernel + its reduce; grid.x persistent workgroups
    hipLaunchKernelGGL((decode_stream_kernel<DT, D, G, RP>), grid, dim3(kStreamWaves * 64),
                       (a.B + 1) * sizeof(int), s, a, sa);
    hipLaunchKernelGGL((reduce_stream_kernel<D, RP>), dim3(a.Hkv * a.slices, a.B),
                       dim3(RP * D / 4), 0, s, a, sa);
  } else {
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, RP, W>), grid, dim3(W * 64), 0, s,
                       a);
  }
}

// Launcher for (dtype, D) and rows per wavefront RP = G * (query tokens
// rounded up to a power of two): W = 4 or 8 wavefronts per workgroup of the
// workgroup-split kernel (W = 1: one wavefront per partition), or W = 0 for
// the stream kernel (which also launches its reduce); nullptr if no such
// kernel is built. Defined in decode_inst_<dtype>_d<D>.hip.
template <int DT, int D>
Launcher pick_rows(int G, int RP, int W);

// Most query rows per KV head on the VALU kernels (as up to 4 slices of 4).
constexpr int kMaxRows = 16;

}  // namespace decode
}  // namespace pkv
