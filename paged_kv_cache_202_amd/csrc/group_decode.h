// Shared-prefix attention in one pass on the matrix cores (gfx950): each
// workgroup takes the stacked query rows of a few members of a sharing
// group, for one KV head, and runs them over the group's shared prefix and
// over each member's own rest, so the prefix's partial results never leave
// the chip.
//
// What it computes is paged attention (vLLM abstract on the papers page
// "external vector cache": a KV cache of fixed-size blocks, shared within
// and across requests) for sequences forked from a common parent (the page
// pool's share_prefix: course page "Module 10. KV Caches and Efficient
// Inference", notebook section 5): each query row's max-subtracted softmax
// over the keys it sees (that page's project demo, Demo 2), query token i of
// nq seeing the first L - nq + i + 1 keys (notebook section 2).
//
// Design (for CDNA4; the pages give no kernel):
//   * rows: one 16-row MFMA tile holds 16 / rpm members' rows (rpm = G x nq
//     padded to a power of two); a workgroup holds RT such tiles and all of
//     its eight wavefronts hold all of them;
//   * tiles: one list per workgroup that interleaves, evenly, the shared
//     prefix's tiles (every row sees them) with each member's own tiles past
//     the prefix (only that member's rows see them). The wavefronts take
//     every eighth entry, so each has prefix tiles (mostly L2 hits: the
//     workgroups of one KV head land on one XCD, grid.x being the KV head)
//     and members' tiles (HBM) in flight together, and all finish together;
//   * per wavefront a ring of LDS slots filled by direct-to-LDS gathers: K
//     rows with their 16-byte chunks permuted per token (the A-operand reads
//     of a token's quarter row spread over the banks), V rows XOR-swizzled
//     by 2 t (the four tokens a transposing read names sit in four bank
//     ranges);
//   * per tile and active row tile: S^T = K Q^T on v_mfma_f32_16x16x32_bf16,
//     the lazy-maximum softmax of the other row-tile kernels, P rounded to
//     bf16, O^T += V^T P^T on v_mfma_f32_16x16x16_bf16 with V read by
//     ds_read_b64_tr_b16;
//   * at the end the eight wavefronts' (m, l, acc) merge in LDS -- each
//     row's weights once, then every thread four output dims -- and the
//     workgroup writes its rows' normalised outputs and lse: no partials,
//     no reduce launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "decode_kernel.h"
#include "shared_prefix.h"
#include "verify_mfma.h"

namespace pkv {
namespace decode {

template <int D>
struct GroupGeo {
  static constexpr int RB = 2 * D;              // bytes of a bf16 token row
  static constexpr int CPT = RB / 16;           // 16-byte chunks per token row
  static constexpr int TPL = 64 / CPT;          // tokens per 1 KiB gather
  static constexpr int NL = kTile / TPL;        // gathers per half tile
  static constexpr int KCH = CPT / 4;           // K chunks a lane reads (a quarter row)
  static constexpr int NC = D / 32;             // q.k MFMAs per tile
  static constexpr int NCB = D / 16;            // 16-dim output column blocks
  static constexpr int kHalf = kTile * RB;      // bytes of K (or V) of a tile
  static constexpr int kTileBytes = 2 * kHalf;
  static constexpr int kSlots = kTileBytes >= 8192 ? 2 : 4;  // 16 KiB a wavefront
  static_assert(KCH == NC, "one 16-byte K chunk per q.k MFMA");
};

// One tile's operands from the LDS slot OFF bytes past the ring with one
// wait: K chunks at ka[c] + OFF, V by transposing reads at va[cb] + OFF (the
// slot is a constant of the unrolled loop, so the offset is an immediate).
template <int D, int OFF>
__device__ __forceinline__ void read_group_tile(u32x4_t (&k)[D / 32], uint2 (&v)[D / 16],
                                                const PKV_LDS char *const (&ka)[D / 32],
                                                const PKV_LDS char *const (&va)[D / 16]) {
  static_assert(OFF >= 0 && OFF + 4096 < 65536, "LDS immediate offsets are 16 bits");
  if constexpr (D == 64) {
    asm volatile(
        "ds_read_b128 %0, %6 offset:%12\n\t"
        "ds_read_b128 %1, %7 offset:%12\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %11 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(ka[0]), "v"(ka[1]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "i"(OFF)
        : "memory");
  } else {
    static_assert(D == 128, "head dims 64 and 128");
    asm volatile(
        "ds_read_b128 %0, %12 offset:%24\n\t"
        "ds_read_b128 %1, %13 offset:%24\n\t"
        "ds_read_b128 %2, %14 offset:%24\n\t"
        "ds_read_b128 %3, %15 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %10, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %11, %23 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]),
          "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
          "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]), "i"(OFF)
        : "memory");
  }
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Most members a workgroup holds (RT = 2 row tiles of 16 one-row members).
constexpr int kGroupMaxMembers = 32;

// grid (Hkv, n_groups x s.chunks), eight wavefronts; s.rpm rows per member,
// RT * 16 / s.rpm members per workgroup.
template <int D, int RT>
__global__ void __launch_bounds__(512, 2) group_mfma_kernel(const DecodeArgs a, const ShareArgs s) {
  using Gg = GroupGeo<D>;
  constexpr int W = 8;
  constexpr int NL = Gg::NL, KCH = Gg::KCH, NC = Gg::NC, NCB = Gg::NCB, CPT = Gg::CPT;
  constexpr int TPL = Gg::TPL, RB = Gg::RB, kSlots = Gg::kSlots;
  constexpr int ROWS = RT * 16;
  // two row tiles: O^T += V^T P^T for both at once on v_mfma_f32_32x32x16_bf16
  // (32 dims x 32 rows a product: four per tile at D = 128, not sixteen
  // 16x16x16 products)
  constexpr bool kWide = RT == 2;
  constexpr int NB32 = D / 32;  // 32-dim blocks
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  // rows padded by four floats: the 16 rows one wavefront writes at once
  // then start in 16 different bank groups instead of one
  constexpr int kAccPitch = D + 4;
  struct Merge {
    float acc[W][ROWS][kAccPitch];
    float m[W][ROWS];
    float l[W][ROWS];
  };
  __shared__ union {
    u32x4_t ring[W * kSlots * Gg::kTileBytes / 16];
    Merge mg;
  } sm;
  // the workgroup's members: sequence, length, first of its own tiles,
  // and where each member's own tiles start in the tile list
  __shared__ int mem_b[kGroupMaxMembers], mem_len[kGroupMaxMembers];
  __shared__ int mem_cum[kGroupMaxMembers + 1];
  __shared__ int wg_bad;
  // per row at the merge: each wavefront's factor, the sum of weights, the maximum
  __shared__ float sm_f[W][ROWS], sm_den[ROWS], sm_max[ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x;
  const int grp = blockIdx.y / s.chunks, chunk = blockIdx.y % s.chunks;
  const int nq = a.nq, G = a.Hq / a.Hkv;
  const int max_ctx = a.max_blocks * a.bs;
  const int rpm = s.rpm, mpt = kVerifyRows / rpm, mpw = RT * mpt;
  if (grp >= s.n_groups) return;
  // group bounds clamped to the members array, so that inconsistent arrays
  // cannot send reads out of it
  const int ms = max(0, min(s.n_members, load_const(s.group_start + grp)));
  const int me = max(ms, min(s.n_members, load_const(s.group_start + grp + 1)));
  const int m0 = ms + chunk * mpw;
  if (m0 >= me) return;  // workgroup-uniform
  const int nmem = min(mpw, me - m0);
  const int prefix_req = load_const(s.group_tokens + grp);
  // a prefix that is not whole tiles or runs past the table poisons the group
  const int prefix = max(0, min(prefix_req, max_ctx)) & ~(kTile - 1);
  const int np_tiles = prefix / kTile;
  const int leader_raw = load_const(s.members + ms);
  const int leader = leader_raw >= 0 && leader_raw < a.B ? leader_raw : 0;
  const int32_t *lrow = a.tables + (size_t)leader * a.max_blocks;

  // ---- members: lanes of wavefront 0 fill the small tables --------------
  if (threadIdx.x < 64) {
    int b = -1, L = 0, own = 0;
    if (lane < nmem) {
      const int braw = s.members[m0 + lane];
      b = braw >= 0 && braw < a.B ? braw : -1;
      L = b >= 0 ? a.lens[b] : 0;
      // tiles past the prefix (none for a length out of range: its rows are NaN)
      if (b >= 0 && L >= nq && L <= max_ctx && L >= prefix) own = (L + kTile - 1) / kTile - np_tiles;
      mem_b[lane] = b;
      mem_len[lane] = L;
    }
    // exclusive prefix of the members' own tile counts
    int incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane <= nmem && lane <= kGroupMaxMembers) mem_cum[lane] = incl - own;
    if (lane == 0) wg_bad = leader != leader_raw || prefix != prefix_req;
  }
  __syncthreads();
  const int n_list = np_tiles + mem_cum[nmem];  // tiles in the workgroup's list

  // ---- this lane's rows: member, sequence, query row, visible keys -------
  int mw[RT], lim[RT];
  uint4 qb[RT][NC];
  bool live[RT];
  size_t orow[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    mw[r] = r * mpt + ln / rpm;
    const int rr = ln % rpm, qi = rr / G;
    const int b = mw[r] < nmem ? mem_b[mw[r]] : -1;
    const int L = mw[r] < nmem ? mem_len[mw[r]] : 0;
    live[r] = b >= 0 && qi < nq && L >= nq && L <= max_ctx;
    lim[r] = live[r] ? L - nq + qi + 1 : 0;
    const int bb = max(b, 0);
    orow[r] = ((size_t)bb * nq + min(qi, nq - 1)) * a.Hq + g * G + rr % G;
    const uint16_t *qp = (const uint16_t *)a.q + orow[r] * D + lg * (D / 4);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 v = *reinterpret_cast<const uint4 *>(qp + c * 8);
      qb[r][c] = live[r] ? v : make_uint4(0, 0, 0, 0);
    }
  }
  float scale_log2 = a.scale_log2;
  settle_s(scale_log2);
  if (scale_log2 < 0.f) {
    // q.k x scale = (-q).k x (-scale): negating bf16 queries is exact
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

  // ---- this wavefront's share of the list: entries wave + 8 j. The list
  //      interleaves the prefix's tiles and the members' own tiles evenly
  //      (entry i is an own tile when floor((i + 1) ns / n) > floor(i ns / n)),
  //      so that every wavefront has reads from L2 and from HBM in flight
  //      throughout --------------------------------------------------------
  const int n_mine = wave < n_list ? (n_list - wave + W - 1) / W : 0;
  const int n_own = n_list - np_tiles;
  auto list_index = [&](int j) { return wave + W * j; };
  // tile of list entry i: member (-1: the prefix) and tile index in its context
  auto locate = [&](int i, int &m, int &k) {
    const int own_before = (int)((int64_t)i * n_own / n_list);
    if ((int)((int64_t)(i + 1) * n_own / n_list) == own_before) {
      m = -1;
      k = i - own_before;
      return;
    }
    const int r = own_before;
    int lo = 0, hi = nmem;  // the member with mem_cum[m] <= r < mem_cum[m + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (mem_cum[mid] <= r) lo = mid; else hi = mid;
    }
    m = lo;
    k = np_tiles + r - mem_cum[lo];
  };
  // lane x holds this wavefront's tile 64 w + x: its block, and its member
  // and tile index packed as (m + 1) << 26 | k
  auto window = [&](int w, int &code) {
    const int j = min(64 * w + lane, max(n_mine - 1, 0));
    int m, k;
    locate(list_index(j), m, k);
    code = ((m + 1) << 26) | k;
    const int32_t *row = m < 0 ? lrow : a.tables + (size_t)max(mem_b[m], 0) * a.max_blocks;
    return row[k * kTile / a.bs];
  };

  // ---- ring, gather offsets, read-back addresses --------------------------
  PKV_LDS char *ring = (PKV_LDS char *)&sm.ring[0] + wave * kSlots * Gg::kTileBytes;
  const char *kbase = (const char *)a.kc;
  const char *vbase = (const char *)a.vc;
  uint32_t koff[NL], voff[NL];  // unsigned: a uniform base plus a 32-bit lane offset
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    // the 1 KiB gather i: lane l fills LDS bytes 16 l of token t = i TPL + l / CPT;
    // K position p holds chunk p ^ (t % CPT), V position p chunk p ^ (2 t % CPT)
    const int t = i * TPL + lane / CPT, p = lane % CPT;
    koff[i] = t * RB + 16 * (p ^ (t % CPT));
    voff[i] = t * RB + 16 * (p ^ ((2 * t) % CPT));
  }
  const PKV_LDS char *ka[KCH];
  {
    const int t = ln;
    const PKV_LDS char *row = ring + (t / TPL) * 1024 + (t % TPL) * RB;
#pragma unroll
    for (int c = 0; c < KCH; ++c) ka[c] = row + 16 * ((KCH * lg + c) ^ (t % CPT));
  }
  const PKV_LDS char *va[NCB];
  if constexpr (kWide) {
    // the 32x32x16 A operand V^T of 32-dim block b: lane l holds dim
    // 32 b + l % 32 of tokens 8 (l / 32) .. + 7, from two transposing reads
    // (half h of the tokens: read 2 b + h); in them lane s of 16-lane group
    // G names dims 4 (s % 4) .. + 3 of dims 32 b + 16 (G % 2) .. of token
    // 8 (G / 2) + 4 h + s / 4
#pragma unroll
    for (int b = 0; b < NB32; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 8 * (lg >> 1) + 4 * h + (ln >> 2);
        const PKV_LDS char *row = ring + Gg::kHalf + (t / TPL) * 1024 + (t % TPL) * RB;
        const int c = 2 * (2 * b + (lg & 1)) + ((ln >> 1) & 1);
        va[2 * b + h] = row + 16 * (c ^ ((2 * t) % CPT)) + 8 * (ln & 1);
      }
  } else {
    // lane s of group lg names dims 4 (s % 4) .. + 3 of column block cb of
    // token 4 lg + s / 4: byte 32 cb + 8 (s % 4) of its row, chunk-swizzled
    const int t = 4 * lg + (ln >> 2);
    const PKV_LDS char *row = ring + Gg::kHalf + (t / TPL) * 1024 + (t % TPL) * RB;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = 2 * cb + ((ln >> 1) & 1);
      va[cb] = row + 16 * (c ^ ((2 * t) % CPT)) + 8 * (ln & 1);
    }
  }
  const size_t blk_bytes = (size_t)a.Hkv * a.bs * RB;
  const size_t head_off = (size_t)g * a.bs * RB;
  int bad = 0;
  auto stage = [&](int slot, int k, int blk) {
    if (blk < 0 || blk >= a.num_blocks) {  // bad table entry: read block 0, poison later
      bad = 1;
      blk = 0;
    }
    const size_t tile = (size_t)(uint32_t)blk * blk_bytes + head_off +
                        (size_t)((k * kTile) % a.bs) * RB;
    const char *kt = kbase + tile, *vt = vbase + tile;
    PKV_LDS char *dst = ring + slot * Gg::kTileBytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) gather_lds16<kKvNonTemporal>(kt + koff[i], dst + i * 1024);
#pragma unroll
    for (int i = 0; i < NL; ++i) gather_lds16<kKvNonTemporal>(vt + voff[i], dst + (NL + i) * 1024);
  };

  // O^T: per row tile and 16-dim column block (16x16 layout: lane holds row
  // ln, dims 4 lg .. + 3), or, two row tiles, per 32-dim block (32x32
  // layout: lane l holds row tile (l / 16) % 2, row l % 16, and in register
  // i dim 8 (i / 4) + 4 (l / 32) + i % 4 of the block)
  f32x4_t o[RT][NCB];
  f32x16_t ow[NB32];
  if constexpr (kWide) {
#pragma unroll
    for (int b = 0; b < NB32; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) ow[b][i] = 0.f;
  } else {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) o[r][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float m_row[RT], l_part[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m_row[r] = kNegInf;
    l_part[r] = 0.f;
  }

  // per row tile: the fewest keys any of its live rows sees (a tile wholly
  // below it needs no mask for that row tile)
  int lim_min[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int v = live[r] ? lim[r] : 0x7fffffff;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) v = min(v, __shfl_xor(v, d, 64));
    lim_min[r] = __builtin_amdgcn_readfirstlane(v);
  }

  if (n_mine > 0) {
    int codev;
    int tblv = window(0, codev);
    settle_v(tblv);  // with the queries: waited for once, before the first gather
    settle_v(codev);
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) settle_v(qb[r][c]);
    auto stage_j = [&](int j) {
      const int code = __builtin_amdgcn_readlane(codev, j & 63);
      stage(j % kSlots, code & ((1 << 26) - 1), __builtin_amdgcn_readlane(tblv, j & 63));
    };
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
      if (j < n_mine) stage_j(j);
    // one tile: every row tile runs it, rows that do not see it masked to
    // -inf (weight 0), so that every tile takes the same straight path
    auto tile = [&](int j, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      const int ahead = min(n_mine - 1 - j, kSlots - 1);
      static_for<kSlots>([&](auto ac) {
        constexpr int A = decltype(ac)::value;
        if (ahead == A) wait_vmcnt<A * 2 * NL>();
      });
      u32x4_t kr[KCH];
      uint2 vt[NCB];
      read_group_tile<D, SLOT * Gg::kTileBytes>(kr, vt, ka, va);
      const int code = __builtin_amdgcn_readlane(codev, j & 63);
      const int mcur = (code >> 26) - 1, kcur = code & ((1 << 26) - 1);
      const int t0 = kcur * kTile;
      if (mcur >= 0 && t0 + kTile > mem_len[mcur]) {
        // the member's last tile: slots past its length may hold stale bits
        // (even NaN), zeroed so that a zero weight cannot meet them
        const int Lm = mem_len[mcur];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          // the tokens this lane's V elements come from
          const int tv = kWide ? t0 + 8 * (lg >> 1) + 4 * (cb & 1) : t0 + 4 * lg;
          vt[cb].x &= (tv < Lm ? 0xffffu : 0u) | (tv + 1 < Lm ? 0xffff0000u : 0u);
          vt[cb].y &= (tv + 2 < Lm ? 0xffffu : 0u) | (tv + 3 < Lm ? 0xffff0000u : 0u);
        }
      }
      // S^T = K Q^T per row tile (one row tile: in two chains of half the
      // dims each, so that the products do not wait on one another)
      f32x4_t sv[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        constexpr int NCH = RT == 1 ? 2 : 1;
        f32x4_t acc[NCH];
#pragma unroll
        for (int h = 0; h < NCH; ++h) acc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[c % NCH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, kr[c]), __builtin_bit_cast(bf16x8_t, qb[r][c]),
              acc[c % NCH], 0, 0, 0);
        sv[r] = acc[0];
        if constexpr (NCH == 2) sv[r] += acc[1];
      }
      uint2 pb[RT];     // each row tile's weights, bf16
      float alpha[RT];  // each row tile's rescale of this lane's row
      bool rescale = false;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        // wavefront-uniform: the prefix's tile (or the member's own tile, its
        // row tile holding that member only) wholly below every row's limit
        const bool whole = (mcur < 0 || (mpt == 1 && mcur == r)) && t0 + kTile <= lim_min[r];
        if (!whole) {
          // keys a row does not see (another member's, causal) score -inf
          const bool mine = mcur < 0 || mw[r] == mcur;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!mine || t0 + 4 * lg + e >= lim[r]) sv[r][e] = kNegInf;
        }
        const float tmax =
            fmaxf(fmaxf(sv[r][0], sv[r][1]), fmaxf(sv[r][2], sv[r][3])) * scale_log2;
        alpha[r] = 1.f;
        if (__any(tmax > m_row[r] + kLazyLog2)) {
          // row ln's scores are spread over the four lane groups
          float gmax = fmaxf(tmax, exact_xor<16>(tmax));
          gmax = fmaxf(gmax, exact_xor<32>(gmax));
          const float mn = fmaxf(m_row[r], gmax);
          alpha[r] = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_row[r] - mn);
          m_row[r] = mn;
          l_part[r] *= alpha[r];
          rescale = true;
          if constexpr (!kWide) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) o[r][cb] *= alpha[r];
          }
        }
        // a masked score gives exp2(-inf) = 0; the floored maximum keeps a
        // row with no visible key yet at 0, not NaN
        const float neg_m = -fmaxf(m_row[r], -3.0e38f);
        float pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pw[e] = __builtin_amdgcn_exp2f(fmaf(sv[r][e], scale_log2, neg_m));
          l_part[r] += pw[e];
        }
        pb[r] = make_uint2(pack_bf16(pw[0], pw[1]), pack_bf16(pw[2], pw[3]));
        if constexpr (!kWide) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            o[r][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(i16x4_t, vt[cb]), __builtin_bit_cast(i16x4_t, pb[r]),
                o[r][cb], 0, 0, 0);
        }
      }
      if constexpr (kWide) {
        if (rescale) {
          // lane l's accumulator rows belong to row tile (l / 16) % 2
          const float al = (lane & 16) ? alpha[1] : alpha[0];
#pragma unroll
          for (int b = 0; b < NB32; ++b) ow[b] *= al;
        }
        // P^T of both row tiles as the B operand: lane l takes row tile
        // (l / 16) % 2's row l % 16, tokens 8 (l / 32) .. + 7. Row tile 0's
        // weights sit in every lane (tokens 4 lg ..), so the swap of 16-lane
        // rows gives, per dword, the low tokens (first result) and the high
        // tokens (second result)
        const auto sx = __builtin_amdgcn_permlane16_swap(pb[0].x, pb[1].x, false, false);
        const auto sy = __builtin_amdgcn_permlane16_swap(pb[0].y, pb[1].y, false, false);
        const uint4 pp = make_uint4(sx[0], sy[0], sx[1], sy[1]);
#pragma unroll
        for (int b = 0; b < NB32; ++b) {
          const uint4 va4 = make_uint4(vt[2 * b].x, vt[2 * b].y, vt[2 * b + 1].x, vt[2 * b + 1].y);
          ow[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va4),
                                                         __builtin_bit_cast(bf16x8_t, pp),
                                                         ow[b], 0, 0, 0);
        }
      }
      // the slot is free again: refill it, after this tile's products are
      // issued, so that the gathers' issue overlaps the matrix core's work
      if (j + kSlots < n_mine) {
        const int jn = j + kSlots;
        if ((jn & 63) == 0) {  // next window of tiles (drains the ring once)
          tblv = window(jn >> 6, codev);
          settle_v(tblv);
          settle_v(codev);
        }
        stage_j(jn);
      }
    };
    // unrolled by the ring depth: tile j sits in slot j % kSlots
    for (int j0 = 0; j0 < n_mine; j0 += kSlots)
      static_for<kSlots>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        if (j0 + S < n_mine) tile(j0 + S, sc);
      });
  }

  // ---- merge the wavefronts in LDS, then write each live row -------------
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    l_part[r] += exact_xor<16>(l_part[r]);
    l_part[r] += exact_xor<32>(l_part[r]);
  }
  bad = __builtin_amdgcn_readfirstlane(bad);
  __syncthreads();  // the partials overwrite the rings
  if constexpr (kWide) {
    float *dst = sm.mg.acc[wave][lane & 31] + 4 * (lane >> 5);
#pragma unroll
    for (int b = 0; b < NB32; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(dst + 32 * b + 8 * q) = make_float4(
            ow[b][4 * q], ow[b][4 * q + 1], ow[b][4 * q + 2], ow[b][4 * q + 3]);
  } else {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float *dst = sm.mg.acc[wave][r * 16 + ln];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        *reinterpret_cast<float4 *>(dst + 16 * cb + 4 * lg) =
            make_float4(o[r][cb][0], o[r][cb][1], o[r][cb][2], o[r][cb][3]);
    }
  }
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    if (lg == 0) {
      sm.mg.m[wave][r * 16 + ln] = m_row[r];
      sm.mg.l[wave][r * 16 + ln] = l_part[r];
    }
  }
  if (bad && lane == 0) wg_bad = 1;
  __syncthreads();
  // per row: the largest maximum, each wavefront's factor and the sum of
  // weights, once (one thread a row), then the outputs four dims a thread
  const float nan = __builtin_nanf("");
  const int any_bad = wg_bad;
  if (threadIdx.x < ROWS) {
    const int row = threadIdx.x;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm.mg.m[w][row]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mwv = sm.mg.m[w][row];
      const float f = mwv == kNegInf ? 0.f : exp2f(mwv - M);
      sm_f[w][row] = f;
      den = fmaf(f, sm.mg.l[w][row], den);
    }
    sm_den[row] = den;
    sm_max[row] = M;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < ROWS * D / 4; idx += W * 64) {
    const int row = idx / (D / 4), d4 = 4 * (idx % (D / 4));
    const int r = row / 16, l16 = row % 16;
    const int mwr = r * mpt + l16 / rpm, rr = l16 % rpm, qi = rr / G;
    if (mwr >= nmem || qi >= nq) continue;
    const int b = mem_b[mwr];
    if (b < 0) continue;
    const int L = mem_len[mwr];
    const float den = sm_den[row];
    const bool ok = L >= nq && L <= max_ctx && L >= prefix && !any_bad && den > 0.f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = sm_f[w][row];
      const float4 v = *reinterpret_cast<const float4 *>(&sm.mg.acc[w][row][d4]);
      num.x = fmaf(f, v.x, num.x);
      num.y = fmaf(f, v.y, num.y);
      num.z = fmaf(f, v.z, num.z);
      num.w = fmaf(f, v.w, num.w);
    }
    const size_t orow_i = ((size_t)b * nq + qi) * a.Hq + g * G + rr % G;
    const float inv = 1.f / den;
    *reinterpret_cast<float4 *>(a.out + orow_i * D + d4) =
        ok ? make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv)
           : make_float4(nan, nan, nan, nan);
    if (d4 == 0 && a.lse) a.lse[orow_i] = ok ? (sm_max[row] + log2f(den)) * kLn2 : nan;
  }
}

using GroupLauncher = void (*)(const DecodeArgs &, const ShareArgs &, dim3, hipStream_t);

// Launcher of the one-pass shared-prefix kernel for head dim D (64 or 128)
// and RT row tiles per workgroup (1 or 2); nullptr if none. Defined in
// shared_inst.hip.
GroupLauncher pick_group(int D, int RT);

}  // namespace decode
}  // namespace pkv
