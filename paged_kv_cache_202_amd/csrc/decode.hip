// Paged attention decode for gfx950 (MI355X): the partition kernel and the
// log-sum-exp reduce kernel.
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

#include "pagedkv.h"
#include "status.h"

namespace {

constexpr int kTile = 16;          // tokens per wavefront step
constexpr int kWaves = 4;          // wavefronts per workgroup
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
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
  int32_t max_blocks, nq, Hq, Hkv, bs, num_blocks, part_tokens, num_parts;
  float scale_log2;
};

// Reduce-scatter of V per-lane partial sums across the LPT lanes of a token
// group (lane bits below LPT). After it, a lane holds C = max(1, V / LPT)
// complete sums: values own .. own + C - 1, own = jl * V / LPT.
template <int LPT, int V>
__device__ __forceinline__ void reduce_scatter(float (&x)[V], int jl) {
  int cnt = V;
#pragma unroll
  for (int m = LPT / 2; m >= 1; m >>= 1) {
    if (cnt > 1) {
      const int half = cnt / 2;
      const bool upper = (jl & m) != 0;
#pragma unroll
      for (int k = 0; k < V / 2; ++k) {
        if (k < half) {
          const float lo = x[k], hi = x[k + half];
          const float send = upper ? lo : hi;
          const float keep = upper ? hi : lo;
          x[k] = keep + __shfl_xor(send, m, 64);
        }
      }
      cnt = half;
    } else {
      x[0] += __shfl_xor(x[0], m, 64);
    }
  }
}

template <int DT, int D, int G, int RP>
__global__ void __launch_bounds__(kWaves * 64)
decode_partition_kernel(const DecodeArgs a) {
  using Gm = Geo<DT, D>;
  constexpr int LPT = Gm::LPT, TPL = Gm::TPL, NL = Gm::NL, EPL = Gm::EPL;
  constexpr int V = RP * NL;                    // partial sums per lane per tile
  constexpr int C = V >= LPT ? V / LPT : 1;     // whole scores per lane
  constexpr int DUP = V >= LPT ? 1 : LPT / V;   // lanes holding the same score
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();

  __shared__ float sm_acc[kWaves][RP][D];
  __shared__ float sm_m[kWaves][RP];
  __shared__ float sm_l[kWaves][RP];
  __shared__ int sm_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane / LPT, jl = lane % LPT;
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

  // ---- query rows: r = qi * G + gj, head g * G + gj ----------------------
  const int d0 = jl * EPL;
  uint32_t qw[RP][EPL / 2 > 0 ? EPL / 2 : 1];  // bf16 pairs
  float qf[RP][EPL];                           // fp32
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
  }

  // ---- scores this lane owns after the reduce-scatter --------------------
  const int own = jl * V / LPT;
  int own_row[C], own_tok[C], own_lim[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int v = own + c;
    own_row[c] = v / NL;
    own_tok[c] = (v % NL) * TPL + grp;       // token offset inside the tile
    const int qi = own_row[c] / G;
    own_lim[c] = qi < nq ? L - nq + qi + 1 : 0;  // visible keys of that row
  }

  float acc[RP][EPL];
  float m_run[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    m_run[r] = kNegInf;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
  }
  float m_own[C], l_own[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    m_own[c] = kNegInf;
    l_own[c] = 0.f;
  }

  const int32_t *trow = a.tables + (size_t)b * a.max_blocks;
  int bad = 0;
  const int min_lim = L - nq + 1;

  for (int t0 = t_begin + wave * kTile; t0 < t_end; t0 += kWaves * kTile) {
    int blk = trow[t0 / a.bs];
    if (blk < 0 || blk >= a.num_blocks) {
      bad = 1;
      blk = 0;
    }
    const size_t base = (((size_t)blk * a.Hkv + g) * a.bs + (t0 % a.bs)) * (size_t)Gm::TB +
                        (size_t)lane * 16;
    const char *kp = (const char *)a.kc + base;
    const char *vp = (const char *)a.vc + base;
    uint4 kr[NL], vr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) kr[i] = *reinterpret_cast<const uint4 *>(kp + i * 1024);
#pragma unroll
    for (int i = 0; i < NL; ++i) vr[i] = *reinterpret_cast<const uint4 *>(vp + i * 1024);

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
      sc[c] = vis ? x[c] * a.scale_log2 : kNegInf;
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
        alpha[r] = mn == kNegInf ? 1.f : exp2f(m_run[r] - mn);
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
      pw[c] = sc[c] == kNegInf ? 0.f : exp2f(sc[c] - m_own[c]);
      l_own[c] += pw[c];
    }
    // every lane of the group needs all V weights of its tokens
    float pa[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int src = grp * LPT + (V >= LPT ? v / C : v * DUP);
      pa[v] = __shfl(pw[v % C], src, 64);
    }
    // in a tail tile, slots past the context may hold stale bits (even NaN):
    // their V is zeroed so that 0 * NaN cannot reach acc
    const bool tail = t0 + kTile > min_lim;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
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
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const float w = pa[r * NL + i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[r][e] = fmaf(w, vv[e], acc[r][e]);
      }
    }
  }

  // ---- wavefront totals ---------------------------------------------------
#pragma unroll
  for (int m = LPT; m < 64; m <<= 1)
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[r][e] += __shfl_xor(acc[r][e], m, 64);
  const bool counted = (jl % DUP) == 0;
  float l_row[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float xs = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (own_row[c] == r && counted) xs += l_own[c];
    l_row[r] = wave_sum(xs);
  }
  if (lane < LPT) {
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][r][d0 + e] = acc[r][e];
  }
  if (lane == 0) {  // bad is wavefront-uniform: it comes from scalar table reads
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      sm_m[wave][r] = m_run[r];
      sm_l[wave][r] = l_row[r];
    }
    sm_bad[wave] = bad;
  }
  __syncthreads();

  // ---- merge the wavefronts; write output or partials ----------------------
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

// One workgroup per (query row, sequence); thread d owns output element d.
template <int D>
__global__ void __launch_bounds__(D)
reduce_partitions_kernel(const DecodeArgs a) {
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  const int rowq = blockIdx.x;  // qi * Hq + h
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = a.lens[b];
  const int qi = rowq / a.Hq;
  const size_t row = (size_t)b * a.nq * a.Hq + rowq;
  const float nan = __builtin_nanf("");
  if (L < a.nq || L > a.max_blocks * a.bs) {
    a.out[row * D + d] = nan;
    if (d == 0 && a.lse) a.lse[row] = nan;
    return;
  }
  (void)qi;
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  const float *pm = a.part_m + row * a.num_parts;
  const float *pl = a.part_l + row * a.num_parts;
  const float *pacc = a.part_acc + row * a.num_parts * D;
  float M = kNegInf;
  bool bad = false;
  for (int p = 0; p < np; ++p) {
    const float m = pm[p];
    bad |= m != m;
    M = fmaxf(M, m);
  }
  float num = 0.f, den = 0.f;
  for (int p = 0; p < np; ++p) {
    const float m = pm[p];
    const float f = m == kNegInf ? 0.f : exp2f(m - M);
    num = fmaf(f, pacc[(size_t)p * D + d], num);
    den = fmaf(f, pl[p], den);
  }
  a.out[row * D + d] = bad || den == 0.f ? nan : num / den;
  if (d == 0 && a.lse) a.lse[row] = bad || den == 0.f ? nan : (M + log2f(den)) * kLn2;
}

int elem_bytes(int dtype) { return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : 0; }

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Partition size in tokens and count for a launch.
void choose_partitions(int32_t B, int32_t Hkv, int64_t max_ctx, int32_t req, int32_t *P,
                       int32_t *NP) {
  if (req > 0) {
    *P = req;
  } else {
    const int64_t units = (int64_t)B * Hkv;
    const int64_t target_wgs = 1024;  // 4 wavefronts each: 16 per CU on 256 CUs
    int64_t np = (target_wgs + units - 1) / units;
    const int64_t min_tokens = 256;
    const int64_t cap = (max_ctx + min_tokens - 1) / min_tokens;
    if (np > cap) np = cap;
    if (np < 1) np = 1;
    int64_t per = (max_ctx + np - 1) / np;
    const int64_t align = (int64_t)kTile * kWaves;
    per = (per + align - 1) / align * align;
    *P = (int32_t)per;
  }
  *NP = (int32_t)((max_ctx + *P - 1) / *P);
  if (*NP < 1) *NP = 1;
}

using Launcher = void (*)(const DecodeArgs &, dim3, hipStream_t);

template <int DT, int D, int G, int RP>
void launch_decode(const DecodeArgs &a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, RP>), grid, dim3(kWaves * 64), 0, s, a);
}

// Rows per wavefront RP = G * (query tokens rounded up to a power of two).
constexpr int kMaxRows = 8;

template <int DT, int D>
Launcher pick_rows(int G, int RP) {
#define PKV_CASE(g, rp) \
  if (G == g && RP == rp) return &launch_decode<DT, D, g, rp>;
  PKV_CASE(1, 1) PKV_CASE(1, 2) PKV_CASE(1, 4) PKV_CASE(1, 8)
  PKV_CASE(2, 2) PKV_CASE(2, 4) PKV_CASE(2, 8)
  PKV_CASE(4, 4) PKV_CASE(4, 8)
  PKV_CASE(8, 8)
#undef PKV_CASE
  return nullptr;
}

Launcher pick_launcher(int dtype, int D, int G, int RP) {
  if (dtype == PKV_F32) {
    if (D == 64) return pick_rows<PKV_F32, 64>(G, RP);
    if (D == 128) return pick_rows<PKV_F32, 128>(G, RP);
    if (D == 256) return pick_rows<PKV_F32, 256>(G, RP);
  } else if (dtype == PKV_BF16) {
    if (D == 64) return pick_rows<PKV_BF16, 64>(G, RP);
    if (D == 128) return pick_rows<PKV_BF16, 128>(G, RP);
    if (D == 256) return pick_rows<PKV_BF16, 256>(G, RP);
  }
  return nullptr;
}

template <int D>
void launch_reduce(const DecodeArgs &a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((reduce_partitions_kernel<D>), grid, dim3(D), 0, s, a);
}

Launcher pick_reduce(int D) {
  if (D == 64) return &launch_reduce<64>;
  if (D == 128) return &launch_reduce<128>;
  if (D == 256) return &launch_reduce<256>;
  return nullptr;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bytes of partials for a partitioned launch: acc [rows, NP, D], m, l [rows, NP].
size_t partial_bytes(int64_t rows, int32_t NP, int32_t D) {
  return align_up((size_t)rows * NP * D * 4, 256) + 2 * align_up((size_t)rows * NP * 4, 256);
}

}  // namespace

using pkv::fail;

static int check_sizes(int32_t B, int32_t nq, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t max_blocks, int32_t bs, int32_t part) {
  if (B <= 0 || nq <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_blocks <= 0 || bs <= 0)
    return fail(PKV_EINVAL, "sizes must be positive");
  if (Hq % Hkv) return fail(PKV_EINVAL, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (D != 64 && D != 128 && D != 256) return fail(PKV_EINVAL, "head dim %d unsupported", D);
  if (bs % kTile) return fail(PKV_EINVAL, "block_size %d is not a multiple of 16", bs);
  if ((int64_t)max_blocks * bs > INT32_MAX) return fail(PKV_EINVAL, "table too wide");
  if (part < 0 || part % kTile) return fail(PKV_EINVAL, "partition_tokens must be 0 or k*16");
  if (B > 65535 || Hkv > 65535) return fail(PKV_EINVAL, "B and Hkv must be <= 65535");
  const int G = Hq / Hkv;
  if (G * next_pow2(nq) > kMaxRows)
    return fail(PKV_EINVAL, "G * nq = %d * %d exceeds %d rows per wavefront", G, nq, kMaxRows);
  return PKV_OK;
}

extern "C" int paged_attention_workspace_size(int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                                              int32_t D, int32_t max_blocks, int32_t bs,
                                              int32_t part, size_t *bytes) {
  if (!bytes) return fail(PKV_EINVAL, "bytes is NULL");
  if (int rc = check_sizes(B, nq, Hq, Hkv, D, max_blocks, bs, part)) return rc;
  int32_t P, NP;
  choose_partitions(B, Hkv, (int64_t)max_blocks * bs, part, &P, &NP);
  *bytes = NP == 1 ? 0 : partial_bytes((int64_t)B * nq * Hq, NP, D);
  return PKV_OK;
}

extern "C" int paged_attention_decode(float *out, const void *q, const void *k_cache,
                                      const void *v_cache, const int32_t *block_tables,
                                      int32_t max_blocks, const int32_t *context_lens, int32_t B,
                                      int32_t nq, int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t bs, int32_t num_blocks, float scale, int dtype,
                                      int32_t part, void *workspace, size_t workspace_bytes,
                                      float *lse_out, void *stream) {
  const int es = elem_bytes(dtype);
  if (!es) return fail(PKV_EINVAL, "unsupported dtype %d", dtype);
  if (int rc = check_sizes(B, nq, Hq, Hkv, D, max_blocks, bs, part)) return rc;
  if (num_blocks <= 0) return fail(PKV_EINVAL, "num_blocks must be positive");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "NULL pointer");
  for (const void *p : {(const void *)out, q, k_cache, v_cache})
    if ((uintptr_t)p % 16) return fail(PKV_EINVAL, "out, q, K and V must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale must be finite");
  int32_t P, NP;
  choose_partitions(B, Hkv, (int64_t)max_blocks * bs, part, &P, &NP);
  const int G = Hq / Hkv;
  const int RP = G * next_pow2(nq);
  Launcher launch = pick_launcher(dtype, D, G, RP);
  if (!launch) return fail(PKV_EINVAL, "no kernel for G=%d, nq=%d", G, nq);
  DecodeArgs a{};
  a.out = out;
  a.lse = lse_out;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.max_blocks = max_blocks;
  a.nq = nq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.bs = bs;
  a.num_blocks = num_blocks;
  a.part_tokens = P;
  a.num_parts = NP;
  a.scale_log2 = scale * kLog2e;
  if (NP > 1) {
    const int64_t rows = (int64_t)B * nq * Hq;
    const size_t need = partial_bytes(rows, NP, D);
    if (!workspace || workspace_bytes < need)
      return fail(PKV_EINVAL, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if ((uintptr_t)workspace % 256) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
    char *w = (char *)workspace;
    a.part_acc = (float *)w;
    w += align_up((size_t)rows * NP * D * 4, 256);
    a.part_m = (float *)w;
    w += align_up((size_t)rows * NP * 4, 256);
    a.part_l = (float *)w;
  }
  hipStream_t s = (hipStream_t)stream;
  launch(a, dim3(NP, Hkv, B), s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "decode launch: %s", hipGetErrorString(e));
  if (NP > 1) {
    pick_reduce(D)(a, dim3(nq * Hq, B), s);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_EHIP, "reduce launch: %s", hipGetErrorString(e));
  }
  return PKV_OK;
}
