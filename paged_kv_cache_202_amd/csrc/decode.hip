// Paged attention decode for gfx950 (MI355X): launch planning, the
// log-sum-exp reduce kernel, and the C-ABI entry points.
//
// The partition kernel and the method it implements are described in
// decode_kernel.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "decode_kernel.h"
#include "verify_mfma.h"
#include "shared_prefix.h"
#include "group_decode.h"
#include "decode_mfma.h"
#include "pagedkv.h"
#include "status.h"

namespace pkv {
namespace decode {
namespace {

// Split-K merge: workgroups of 256 threads, D / 4 threads per group owning
// four output elements each. With many partitions per row (GPR = 1024 / D
// groups per row), the groups of a workgroup take every GPR-th partition of
// one row with a running maximum and are merged in LDS; with few (GPR = 1),
// each group merges one row alone. M = max m_p,
// out = sum 2^(m_p-M) acc_p / sum 2^(m_p-M) l_p.
constexpr int kReduceThreads = 256;

template <int D, int GPR>
__global__ void __launch_bounds__(kReduceThreads)
reduce_partitions_kernel(const DecodeArgs a) {
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  constexpr int TPG = D / 4;                // threads per group
  constexpr int NG = kReduceThreads / TPG;  // groups per workgroup
  constexpr int RPW = NG / GPR;             // rows per workgroup
  __shared__ float sm_m[NG], sm_den[NG];
  __shared__ float4 sm_num[NG][TPG];
  const int grp = threadIdx.x / TPG, t = threadIdx.x % TPG;
  const int sub = grp % GPR;                          // this group's share of its row
  const int rowq = blockIdx.x * RPW + grp / GPR;      // qi * Hq + h
  const int b = blockIdx.y;
  const bool row_ok = rowq < a.nq * a.Hq;             // workgroup-uniform when GPR > 1
  const int L = load_const(a.lens + b);
  const size_t row = (size_t)b * a.nq * a.Hq + (row_ok ? rowq : 0);
  const float nan = __builtin_nanf("");
  float *o = a.out + row * D + 4 * t;
  if (L < a.nq || L > a.max_blocks * a.bs) {
    if (row_ok && sub == 0) {
      o[0] = nan;
      o[1] = nan;
      o[2] = nan;
      o[3] = nan;
      if (t == 0 && a.lse) a.lse[row] = nan;
    }
    return;
  }
  // slots written for this row: partitions [0, ceil(lim / P)) for a row that
  // sees lim keys (a partition past them may have been skipped altogether);
  // with a shared prefix, prefix pieces [0, ceil(start / PP)) and then the
  // suffix's partitions from slot part_base on
  const int start = a.starts ? min(max(load_const(a.starts + b), 0), L) : 0;
  const int np_pre = a.starts ? (start + a.prefix_part - 1) / a.prefix_part : 0;
  const int lim = L - a.nq + (row_ok ? rowq : 0) / a.Hq + 1;  // keys this row sees
  const int np_suf = (max(lim - start, 0) + a.part_tokens - 1) / a.part_tokens;
  const int np = row_ok ? min(a.num_parts, a.part_base + np_suf) : 0;
  const float *pm = a.part_m + row * a.num_parts;
  const float *pl = a.part_l + row * a.num_parts;
  const float4 *pacc = reinterpret_cast<const float4 *>(a.part_acc + row * a.num_parts * D);
  float M = kNegInf, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  bool bad = false;
  // the MFMA kernel's independent wavefronts leave one partial per run of
  // parts_per_wg partitions, in the run's first slot
  const int run = a.parts_per_wg > 1 ? a.parts_per_wg : 1;
#pragma unroll 4
  for (int p = sub * run; p < np; p += GPR * run) {
    if (p >= np_pre && p < a.part_base) continue;  // prefix pieces past this row's prefix
    const float m = pm[p];
    bad |= m != m;
    if (m == kNegInf) continue;  // no visible key in the partition (or an empty slot)
    const float l = pl[p];
    const float4 v = pacc[(size_t)p * TPG + t];
    if (m > M) {
      const float c = exp2f(M - m);  // 0 while M is still -inf
      num.x *= c; num.y *= c; num.z *= c; num.w *= c;
      den *= c;
      M = m;
    }
    const float f = exp2f(m - M);
    num.x = fmaf(f, v.x, num.x);
    num.y = fmaf(f, v.y, num.y);
    num.z = fmaf(f, v.z, num.z);
    num.w = fmaf(f, v.w, num.w);
    den = fmaf(f, l, den);
  }
  if constexpr (GPR > 1) {
    // a group's bad flag is the same in all its threads: fold it into M
    if (t == 0) {
      sm_m[grp] = bad ? nan : M;
      sm_den[grp] = den;
    }
    sm_num[grp][t] = num;
    __syncthreads();
    if (sub != 0) return;
    float Mt = kNegInf;
    bool any_bad = false;
#pragma unroll
    for (int g = 0; g < GPR; ++g) {
      any_bad |= sm_m[grp + g] != sm_m[grp + g];
      Mt = fmaxf(Mt, sm_m[grp + g]);
    }
    float dt = 0.f;
    float4 nt = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int g = 0; g < GPR; ++g) {
      const float mg = sm_m[grp + g];
      const float f = mg == kNegInf || mg != mg ? 0.f : exp2f(mg - Mt);
      const float4 v = sm_num[grp + g][t];
      nt.x = fmaf(f, v.x, nt.x);
      nt.y = fmaf(f, v.y, nt.y);
      nt.z = fmaf(f, v.z, nt.z);
      nt.w = fmaf(f, v.w, nt.w);
      dt = fmaf(f, sm_den[grp + g], dt);
    }
    M = Mt;
    den = dt;
    num = nt;
    bad = any_bad;
  }
  if (!row_ok) return;
  const bool nan_out = bad || den == 0.f;
  o[0] = nan_out ? nan : num.x / den;
  o[1] = nan_out ? nan : num.y / den;
  o[2] = nan_out ? nan : num.z / den;
  o[3] = nan_out ? nan : num.w / den;
  if (t == 0 && a.lse) a.lse[row] = nan_out ? nan : (M + log2f(den)) * kLn2;
}

int elem_bytes(int dtype) { return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : 0; }

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Launch plan. The chip holds about kResidentWaves decode wavefronts at once
// (256 CUs x 4 SIMDs x 2 wavefronts of up to 256 VGPRs).
//  * Workgroup-split (waves = 1, 4 or 8): one workgroup per (partition, KV
//    head, sequence); its wavefronts take interleaved tiles of the
//    partition and merge in LDS. With one partition it needs no workspace
//    and no reduce launch. Short partitions (under 128 tiles) get one
//    wavefront, long ones four or eight. Used for a requested partition
//    size, and by default: one partition per context when the (sequence,
//    KV head) pairs fill a round of wavefronts, else as many equal
//    partitions as fill one.
//  * Stream (waves = 0): kResidentWaves persistent wavefronts share the
//    stream of all tiles equally; a reduce launch merges their segments.
//    Used for balanced scheduling of mixed lengths (partition_tokens = -1).
constexpr int64_t kResidentWaves = 2048;

// Whether the stream kernel's LDS (tile rings plus two per-sequence
// prefixes) fits one workgroup for B sequences.
bool stream_fits(int dtype, int32_t D, int64_t B) {
  int64_t bytes = 0;
#define PKV_LDS_CASE(dt, d) \
  if (dtype == dt && D == d) bytes = stream_lds_bytes<dt, d>(B);
  PKV_LDS_CASE(PKV_F32, 64) PKV_LDS_CASE(PKV_F32, 128) PKV_LDS_CASE(PKV_F32, 256)
  PKV_LDS_CASE(PKV_BF16, 64) PKV_LDS_CASE(PKV_BF16, 128) PKV_LDS_CASE(PKV_BF16, 256)
#undef PKV_LDS_CASE
  return bytes > 0 && bytes <= kLdsLimit;
}

struct Plan {
  int waves;            // 1, 4 or 8: workgroup-split kernel; 0: stream kernel
  int32_t part_tokens;  // stream: 0 = no partition cuts
  int32_t num_parts;    // workgroup-split: partitions per context
  int32_t grid_x;
};

// Whether the stream kernels' per-sequence prefix of slots (32-bit) holds
// B sequences of up to max_ctx tokens, each charged `cost` extra slots.
bool stream_prefix_fits(int64_t B, int64_t max_ctx, int64_t cost) {
  return B * ((max_ctx + kTile - 1) / kTile + cost) <= INT32_MAX;
}

Plan plan_launch(int64_t B, int64_t Hkv, int64_t max_ctx, int32_t req, bool stream_ok) {
  Plan pl{};
  const int64_t units = B * Hkv;
  if (req == -1 && stream_ok && stream_prefix_fits(B, max_ctx, 0)) {
    pl.waves = 0;
    pl.part_tokens = 0;
    pl.num_parts = 1;
    pl.grid_x = (int32_t)(kResidentWaves / kStreamWaves);
    return pl;
  }
  const int64_t whole = (max_ctx + kTile - 1) / kTile * kTile;  // one partition
  int64_t P = req > 0 ? req : whole;
  if (req == 0 && units * 8 < kResidentWaves && max_ctx >= 1024) {
    // too few pairs: split every context into enough partitions of eight
    // wavefronts to fill a round
    const int64_t np = (kResidentWaves + units * 8 - 1) / (units * 8);
    P = ((max_ctx + np - 1) / np + kTile - 1) / kTile * kTile;
  }
  pl.part_tokens = (int32_t)P;
  pl.num_parts = (int32_t)((max_ctx + P - 1) / P);
  if (pl.num_parts < 1) pl.num_parts = 1;
  const int64_t tiles_per_part = (P + kTile - 1) / kTile;
  pl.grid_x = pl.num_parts;
  if (tiles_per_part < 128)
    pl.waves = 1;
  else if (tiles_per_part >= 256 && units * pl.num_parts * 8 <= 2 * kResidentWaves)
    pl.waves = 8;
  else
    pl.waves = 4;
  return pl;
}

template <int D>
void launch_reduce(const DecodeArgs &a, const StreamArgs &, dim3 grid, hipStream_t s) {
  // grid.x = query rows per sequence; up to 16 slots per row: one group per
  // row, looping over them
  constexpr int NG = kReduceThreads / (D / 4);
  if (a.num_parts <= 16) {
    grid.x = (grid.x + NG - 1) / NG;
    hipLaunchKernelGGL((reduce_partitions_kernel<D, 1>), grid, dim3(kReduceThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((reduce_partitions_kernel<D, NG>), grid, dim3(kReduceThreads), 0, s, a);
  }
}

Launcher pick_reduce(int D) {
  if (D == 64) return &launch_reduce<64>;
  if (D == 128) return &launch_reduce<128>;
  if (D == 256) return &launch_reduce<256>;
  return nullptr;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bytes of partials for a partitioned workgroup-split launch:
// acc [rows, NP, D], m, l [rows, NP].
size_t partial_bytes(int64_t rows, int32_t NP, int32_t D) {
  return align_up((size_t)rows * NP * D * 4, 256) + 2 * align_up((size_t)rows * NP * 4, 256);
}

// Stream launch workspace: the per-sequence tile prefix, then segment
// partials acc [S, RP, D], m, l [S, RP] with S = N + units segment ids
// (segment id w + u: wavefront w < N, unit u < units).
size_t stream_segments(int64_t units) { return kResidentWaves + units; }
size_t stream_bytes(int64_t B, int64_t units, int32_t RP, int32_t D) {
  const size_t S = stream_segments(units);
  return align_up((size_t)(B + 1) * 4, 256) + align_up(S * RP * D * 4, 256) +
         2 * align_up(S * RP * 4, 256);
}

Launcher pick_mfma_stream_decode(int dtype, int D, int RW) {
  if (D == 64) return pick_mfma_stream<64>(dtype, RW);
  if (D == 128) return pick_mfma_stream<128>(dtype, RW);
  return nullptr;
}

// Rows per wavefront of the matrix-core kernels for `rows` query rows of a
// KV head.
int32_t mfma_rows(int32_t rows) { return rows <= 4 ? 4 : rows <= 8 ? 8 : 16; }

Launcher pick_mfma_decode(int dtype, int D, int RW, int W) {
  if (D == 64) return pick_mfma<64>(dtype, RW, W);
  if (D == 128) return pick_mfma<128>(dtype, RW, W);
  if (D == 256) return pick_mfma<256>(dtype, RW, W);
  return nullptr;
}

Launcher pick_launcher(int dtype, int D, int G, int RP, int W) {
  if (dtype == PKV_F32) {
    if (D == 64) return pick_rows<PKV_F32, 64>(G, RP, W);
    if (D == 128) return pick_rows<PKV_F32, 128>(G, RP, W);
    if (D == 256) return pick_rows<PKV_F32, 256>(G, RP, W);
  } else if (dtype == PKV_BF16) {
    if (D == 64) return pick_rows<PKV_BF16, 64>(G, RP, W);
    if (D == 128) return pick_rows<PKV_BF16, 128>(G, RP, W);
    if (D == 256) return pick_rows<PKV_BF16, 256>(G, RP, W);
  }
  return nullptr;
}

}  // namespace
}  // namespace decode
}  // namespace pkv

using pkv::fail;
using namespace pkv::decode;

static int check_sizes(int32_t B, int32_t nq, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t max_blocks, int32_t bs, int32_t part) {
  if (B <= 0 || nq <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_blocks <= 0 || bs <= 0)
    return fail(PKV_EINVAL, "sizes must be positive");
  if (Hq % Hkv) return fail(PKV_EINVAL, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (D != 64 && D != 128 && D != 256) return fail(PKV_EINVAL, "head dim %d unsupported", D);
  if (bs % kTile) return fail(PKV_EINVAL, "block_size %d is not a multiple of 16", bs);
  if ((int64_t)max_blocks * bs > INT32_MAX) return fail(PKV_EINVAL, "table too wide");
  if (part < -1 || (part > 0 && part % kTile))
    return fail(PKV_EINVAL, "partition_tokens must be -1, 0 or a positive multiple of 16");
  if (B > 65535 || Hkv > 65535) return fail(PKV_EINVAL, "B and Hkv must be <= 65535");
  return PKV_OK;
}

// The kernel family for a launch: the MFMA tile for bf16 multi-query rows
// (up to 16 rows per KV head), else the VALU kernels (up to kMaxRows rows).
static bool use_mfma(int dtype, int32_t nq, int32_t G) {
  return dtype == PKV_BF16 && nq > 1 && G * nq <= kVerifyRows;
}

// Chunked prefill: more than one 16-row tile of query rows per KV head, on
// the MFMA row-tile kernel (bf16).
static bool use_chunk(int dtype, int32_t nq, int32_t G) {
  return dtype == PKV_BF16 && G * nq > kVerifyRows;
}

static int check_rows(int dtype, int32_t nq, int32_t G) {
  if (use_mfma(dtype, nq, G) || use_chunk(dtype, nq, G)) return PKV_OK;
  if (G * next_pow2(nq) > kMaxRows)
    return fail(PKV_EINVAL,
                "G * nq = %d * %d rows per KV head: more than %d need bf16 caches", G, nq,
                kMaxRows);
  return PKV_OK;
}

// Launch shape of the chunk kernel: W wavefronts x RT row tiles per
// workgroup, `chunks` workgroups per (sequence, KV head) along grid.z, and
// the context cut into np partitions of pp tokens (all multiples of 16).
struct ChunkPlan {
  int32_t W, RT, chunks, np, pp;
};

static int chunk_plan(int32_t B, int32_t nq, int32_t G, int32_t Hkv, int32_t D, int64_t max_ctx,
                      int32_t part, ChunkPlan *cp) {
  const int32_t tiles = (G * nq + kVerifyRows - 1) / kVerifyRows;  // row tiles per KV head
  cp->RT = tiles >= 16 && D <= 128 ? 2 : 1;
  const int32_t per_wave = (tiles + cp->RT - 1) / cp->RT;
  cp->W = per_wave >= 8 ? 8 : next_pow2(per_wave);
  cp->chunks = (tiles + cp->W * cp->RT - 1) / (cp->W * cp->RT);
  if ((int64_t)B * cp->chunks > 65535)
    return fail(PKV_EINVAL, "B * row chunks = %d * %d exceed one launch", B, cp->chunks);
  if (part > 0) {
    cp->pp = part;
  } else {
    // enough partitions that the workgroups fill a round of wavefronts
    const int64_t per_part = (int64_t)B * Hkv * cp->chunks * cp->W;
    int64_t np = (kResidentWaves + per_part - 1) / per_part;
    const int64_t most = (max_ctx + 2 * kTile - 1) / (2 * kTile);  // at least 32 tokens each
    if (np > most) np = most;
    if (np < 1) np = 1;
    cp->pp = (int32_t)(((max_ctx + np - 1) / np + kTile - 1) / kTile * kTile);
  }
  cp->np = (int32_t)((max_ctx + cp->pp - 1) / cp->pp);
  return PKV_OK;
}

// Workspace a launch needs, for either kernel family (the larger of the two
// possibilities, so the size does not depend on the dtype).
// How the VALU kernels hold the G * nq query rows of a KV head (rounded up
// to a power of two): up to RP = 8 rows per wavefront, all fed by every
// tile the wavefront loads, and S wavefront slices when more rows remain (a
// slice streams the KV head's bytes again, so it is the last resort).
static void row_split(int32_t G, int32_t nq, int32_t *RP, int32_t *S) {
  const int32_t all = G * next_pow2(nq);
  *RP = all < 8 ? all : 8;
  *S = all / *RP;
}

static size_t workspace_need(int32_t B, int32_t nq, int32_t Hq, int32_t Hkv, int32_t D,
                             int64_t max_ctx, int32_t part) {
  if (use_chunk(PKV_BF16, nq, Hq / Hkv)) {
    ChunkPlan cp;
    if (chunk_plan(B, nq, Hq / Hkv, Hkv, D, max_ctx, part, &cp)) return 0;
    return partial_bytes((int64_t)B * nq * Hq, cp.np, D);
  }
  int32_t RP, S;
  row_split(Hq / Hkv, nq, &RP, &S);
  const int64_t units = (int64_t)B * Hkv * S;
  const int32_t RW = RP;
  size_t need = 0;
  for (bool stream_ok : {true, false}) {
    const Plan pl = plan_launch(B, Hkv, max_ctx, part, stream_ok);
    size_t n = 0;
    if (pl.waves == 0) {
      n = stream_bytes(B, units, RW, D);
      if (nq == 1 && D <= 128)  // the matrix-core kernel's stream mode (bf16)
        n = std::max(n, stream_bytes(B, (int64_t)B * Hkv, mfma_rows(Hq / Hkv), D));
    } else if (pl.num_parts > 1)
      n = partial_bytes((int64_t)B * nq * Hq, pl.num_parts, D);
    if (n > need) need = n;
  }
  return need;
}

extern "C" int paged_attention_workspace_size(int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                                              int32_t D, int32_t max_blocks, int32_t bs,
                                              int32_t part, size_t *bytes) {
  if (!bytes) return fail(PKV_EINVAL, "bytes is NULL");
  if (int rc = check_sizes(B, nq, Hq, Hkv, D, max_blocks, bs, part)) return rc;
  if (use_chunk(PKV_BF16, nq, Hq / Hkv)) {
    ChunkPlan cp;
    if (int rc = chunk_plan(B, nq, Hq / Hkv, Hkv, D, (int64_t)max_blocks * bs, part, &cp))
      return rc;
  }
  *bytes = workspace_need(B, nq, Hq, Hkv, D, (int64_t)max_blocks * bs, part);
  return PKV_OK;
}

// Chunked prefill (bf16, more than 16 query rows per KV head): the chunk
// kernel writes (m, l, acc) per row and context partition; the partition
// reduce merges them (a single partition too: it also normalises).
static int chunk_attention(float *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, int32_t max_blocks,
                           const int32_t *context_lens, int32_t B, int32_t nq, int32_t Hq,
                           int32_t Hkv, int32_t D, int32_t bs, int32_t num_blocks, float scale,
                           int32_t part, void *workspace, size_t workspace_bytes, float *lse_out,
                           hipStream_t s) {
  const int32_t G = Hq / Hkv;
  ChunkPlan cp;
  if (int rc = chunk_plan(B, nq, G, Hkv, D, (int64_t)max_blocks * bs, part, &cp)) return rc;
  PrefixLauncher chunk = pick_prefix(D, cp.W, cp.RT, true);
  if (!chunk) return fail(PKV_EINVAL, "no chunk kernel for D=%d", D);
  const int64_t rows = (int64_t)B * nq * Hq;
  const size_t need = partial_bytes(rows, cp.np, D);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_EINVAL, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if ((uintptr_t)workspace % 256) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
  DecodeArgs a{};
  a.out = out;
  a.lse = lse_out;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.B = B;
  a.max_blocks = max_blocks;
  a.nq = nq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.bs = bs;
  a.num_blocks = num_blocks;
  a.part_tokens = cp.pp;
  a.num_parts = cp.np;
  a.slices = 1;
  a.scale_log2 = scale * kLog2e;
  char *w = (char *)workspace;
  a.part_acc = (float *)w;
  w += align_up((size_t)rows * cp.np * D * 4, 256);
  a.part_m = (float *)w;
  w += align_up((size_t)rows * cp.np * 4, 256);
  a.part_l = (float *)w;
  ShareArgs sh{};
  sh.chunks = cp.chunks;
  sh.prefix_part = cp.pp;
  chunk(a, sh, dim3(cp.np, Hkv, B * cp.chunks), s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "chunk launch: %s", hipGetErrorString(e));
  StreamArgs sa{};
  pick_reduce(D)(a, sa, dim3(nq * Hq, B), s);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "reduce launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

// The attention call for fp32 and bf16 caches (scales = nullptr) and for
// caches of codes (dtype PKV_I8 or kCodes3, bf16 queries, per-row scales
// [num_blocks, Hkv, 2, bs]).
static int decode_impl(float *out, const void *q, const void *k_cache, const void *v_cache,
                       const float *scales, const int32_t *block_tables,
                       int32_t max_blocks, const int32_t *context_lens, int32_t B, int32_t nq,
                       int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t num_blocks,
                       float scale, int dtype, int32_t part, void *workspace,
                       size_t workspace_bytes, float *lse_out, void *stream) {
  if (int rc = check_sizes(B, nq, Hq, Hkv, D, max_blocks, bs, part)) return rc;
  if (num_blocks <= 0) return fail(PKV_EINVAL, "num_blocks must be positive");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "NULL pointer");
  for (const void *p : {(const void *)out, q, k_cache, v_cache})
    if ((uintptr_t)p % 16) return fail(PKV_EINVAL, "out, q, K and V must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale must be finite");
  const int G = Hq / Hkv;
  if (int rc = check_rows(dtype, nq, G)) return rc;
  if (use_chunk(dtype, nq, G))
    return chunk_attention(out, q, k_cache, v_cache, block_tables, max_blocks, context_lens, B,
                           nq, Hq, Hkv, D, bs, num_blocks, scale, part, workspace,
                           workspace_bytes, lse_out, (hipStream_t)stream);
  const bool mfma = use_mfma(dtype, nq, G);
  // the matrix-core kernel's stream mode: one query token, D <= 128, bf16
  // caches or caches of codes, batches whose slot prefix fits its LDS and
  // 32 bits
  const bool mstream_ok =
      !mfma && nq == 1 && D <= 128 &&
      (dtype == PKV_BF16 || dtype == PKV_I8 || dtype == kCodes3) && B <= kMfmaStreamSeqs &&
      stream_prefix_fits(B, (int64_t)max_blocks * bs, kMfmaStreamSegCost);
  const Plan pl = plan_launch(B, Hkv, (int64_t)max_blocks * bs, part,
                              !mfma && (mstream_ok || stream_fits(dtype, D, B)));
  const int32_t P = pl.part_tokens, NP = pl.num_parts;
  int32_t RP, S;
  row_split(G, nq, &RP, &S);
  if (mfma) S = 1;
  // the balanced plan on the stream mode where it serves the call (else on
  // the VALU stream kernel: fp32, D = 256, more sequences)
  const bool mstream = pl.waves == 0 && mstream_ok;
  // matrix-core kernel: every row of a KV head in one wavefront (code caches;
  // bf16 decode with one query token and D <= 128)
  const bool codes = dtype == PKV_I8 || dtype == kCodes3 || mstream ||
                     (dtype == PKV_BF16 && nq == 1 && D <= 128 && pl.waves != 0 && !mfma);
  if (codes) {
    RP = mfma_rows(G * nq);
    S = 1;
  }
  const int32_t RW = RP;
  const bool streamed = pl.waves == 0 && !mfma;
  // Short partitions on the MFMA kernel: rather than a one-wavefront
  // workgroup per partition, workgroups of 8 independent wavefronts, each
  // streaming ppw consecutive partitions (as many as leave about one round
  // of wavefronts) and writing their partials.
  int32_t ppw = 0, W = pl.waves;
  dim3 grid = streamed ? dim3(pl.grid_x) : dim3(NP, Hkv * S, B);
  if (mstream) {
    W = 8;
    grid = dim3((uint32_t)(kResidentWaves / 8));
  } else if (codes && pl.waves == 1 && NP > 1) {
    ppw = (int32_t)std::min<int64_t>(
        NP, std::max<int64_t>(1, (int64_t)B * Hkv * NP / kResidentWaves));
    const int32_t runs = (NP + ppw - 1) / ppw;
    W = 8;
    grid.x = (runs + W - 1) / W;
  }
  Launcher launch = mfma      ? pick_verify(D)
                    : mstream ? pick_mfma_stream_decode(dtype, D, RP)
                    : codes   ? pick_mfma_decode(dtype, D, RP, W)
                            : pick_launcher(dtype, D, G, RP, pl.waves);
  if (!launch) return fail(PKV_EINVAL, "no kernel for G=%d, nq=%d", G, nq);
  DecodeArgs a{};
  a.out = out;
  a.lse = lse_out;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.B = B;
  a.max_blocks = max_blocks;
  a.nq = nq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.bs = bs;
  a.num_blocks = num_blocks;
  a.part_tokens = P;
  a.num_parts = NP;
  a.slices = S;
  a.scale_log2 = scale * kLog2e;
  a.scales = scales;
  a.parts_per_wg = ppw;
  StreamArgs sa{};
  size_t need = 0;
  if (streamed)
    need = stream_bytes(B, (int64_t)B * Hkv * S, RW, D);
  else if (NP > 1)
    need = partial_bytes((int64_t)B * nq * Hq, NP, D);
  if (need) {
    if (!workspace || workspace_bytes < need)
      return fail(PKV_EINVAL, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if ((uintptr_t)workspace % 256) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
    char *w = (char *)workspace;
    if (streamed) {
      const size_t nseg = stream_segments((int64_t)B * Hkv * S);
      sa.tile_pre = (int32_t *)w;
      w += align_up((size_t)(B + 1) * 4, 256);
      sa.n_waves = mstream ? (int32_t)(grid.x * 8) : (int32_t)(pl.grid_x * kStreamWaves);
      sa.seg_cost = mstream ? kMfmaStreamSegCost : 0;
      a.part_acc = (float *)w;
      w += align_up(nseg * RW * D * 4, 256);
      a.part_m = (float *)w;
      w += align_up(nseg * RW * 4, 256);
      a.part_l = (float *)w;
    } else {
      const int64_t rows = (int64_t)B * nq * Hq;
      a.part_acc = (float *)w;
      w += align_up((size_t)rows * NP * D * 4, 256);
      a.part_m = (float *)w;
      w += align_up((size_t)rows * NP * 4, 256);
      a.part_l = (float *)w;
    }
  }
  hipStream_t s = (hipStream_t)stream;
  launch(a, sa, grid, s);  // the stream launcher also launches its reduce
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "decode launch: %s", hipGetErrorString(e));
  if (!streamed && NP > 1) {
    pick_reduce(D)(a, sa, dim3(nq * Hq, B), s);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_EHIP, "reduce launch: %s", hipGetErrorString(e));
  }
  return PKV_OK;
}

extern "C" int paged_attention_decode(float *out, const void *q, const void *k_cache,
                                      const void *v_cache, const int32_t *block_tables,
                                      int32_t max_blocks, const int32_t *context_lens, int32_t B,
                                      int32_t nq, int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t bs, int32_t num_blocks, float scale, int dtype,
                                      int32_t part, void *workspace, size_t workspace_bytes,
                                      float *lse_out, void *stream) {
  if (!elem_bytes(dtype))
    return fail(PKV_EINVAL, "unsupported dtype %d (int8 codes: paged_attention_decode_q8)",
                dtype);
  return decode_impl(out, q, k_cache, v_cache, nullptr, block_tables, max_blocks,
                     context_lens, B, nq, Hq, Hkv, D, bs, num_blocks, scale, dtype, part,
                     workspace, workspace_bytes, lse_out, stream);
}

// ---------------------------------------------------------------------------
// paged_attention_decode for callers that cannot allocate: the partials live
// in a file-scope device array instead of a caller workspace. Each GPU the
// library runs on holds its own copy until the process ends; its address on
// a device is asked for once, with that device current, and kept.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void *scratch_ptr[kMaxDevices];

// The scratch array's device address on the calling thread's current device.
static int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_EINVAL, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PKV_EHIP, "address of the scratch array: %s", hipGetErrorString(e));
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return PKV_OK;
}

extern "C" int paged_attention_decode_noalloc(float *out, const void *q, const void *k_cache,
                                              const void *v_cache, const int32_t *block_tables,
                                              int32_t max_blocks, const int32_t *context_lens,
                                              int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                                              int32_t D, int32_t bs, int32_t num_blocks,
                                              float scale, int dtype, int32_t part,
                                              float *lse_out, void *stream) {
  if (!elem_bytes(dtype))
    return fail(PKV_EINVAL, "unsupported dtype %d", dtype);
  size_t need = 0;
  if (int rc = paged_attention_workspace_size(B, nq, Hq, Hkv, D, max_blocks, bs, part, &need))
    return rc;
  if (need > kScratchBytes)
    return fail(PKV_EINVAL,
                "this call needs %zu bytes of partials; the no-allocation entry point holds "
                "%zu (pass a workspace to paged_attention_decode instead)",
                need, kScratchBytes);
  void *ws = nullptr;
  if (need)
    if (int rc = scratch_address(&ws)) return rc;
  return decode_impl(out, q, k_cache, v_cache, nullptr, block_tables, max_blocks,
                     context_lens, B, nq, Hq, Hkv, D, bs, num_blocks, scale, dtype, part, ws,
                     need ? kScratchBytes : 0, lse_out, stream);
}

extern "C" int paged_attention_decode_q3(float *out, const void *q, const uint8_t *k_codes,
                                         const uint8_t *v_codes, const float *scales,
                                         const int32_t *block_tables,
                                         int32_t max_blocks, const int32_t *context_lens,
                                         int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                                         int32_t D, int32_t bs, int32_t num_blocks, float scale,
                                         int32_t part, void *workspace, size_t workspace_bytes,
                                         float *lse_out, void *stream) {
  if (!scales) return fail(PKV_EINVAL, "NULL pointer");
  if ((uintptr_t)scales % 16) return fail(PKV_EINVAL, "the scale array must be 16-byte aligned");
  if (D != 128 && D != 256) return fail(PKV_EINVAL, "head dim %d unsupported for 3-bit codes", D);
  return decode_impl(out, q, k_codes, v_codes, scales, block_tables, max_blocks,
                     context_lens, B, nq, Hq, Hkv, D, bs, num_blocks, scale, kCodes3, part,
                     workspace, workspace_bytes, lse_out, stream);
}

extern "C" int paged_attention_decode_q8(float *out, const void *q, const int8_t *k_codes,
                                         const int8_t *v_codes, const float *scales,
                                         const int32_t *block_tables,
                                         int32_t max_blocks, const int32_t *context_lens,
                                         int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                                         int32_t D, int32_t bs, int32_t num_blocks, float scale,
                                         int32_t part, void *workspace, size_t workspace_bytes,
                                         float *lse_out, void *stream) {
  if (!scales) return fail(PKV_EINVAL, "NULL pointer");
  if ((uintptr_t)scales % 16) return fail(PKV_EINVAL, "the scale array must be 16-byte aligned");
  return decode_impl(out, q, k_codes, v_codes, scales, block_tables, max_blocks,
                     context_lens, B, nq, Hq, Hkv, D, bs, num_blocks, scale, PKV_I8, part,
                     workspace, workspace_bytes, lse_out, stream);
}

// ---------------------------------------------------------------------------
// Shared prefixes: the prefix kernel over each group's stacked query rows,
// then the ordinary kernels from seq_prefix[b] on, then the merge.
// ---------------------------------------------------------------------------
namespace {

struct SharePlan {
  int32_t W;       // wavefronts per prefix workgroup
  int32_t RT;      // row tiles per wavefront
  int32_t chunks;  // prefix workgroups per group along grid.z
  int32_t rpm;     // rows per member, padded to a power of two
  int32_t npp;     // prefix partitions (slots 0 .. npp - 1)
  int32_t pp;      // tokens per prefix partition
};

int share_plan(int32_t G, int32_t nq, int32_t Hkv, int32_t D, int32_t n_groups,
               int32_t max_members, int32_t max_prefix, SharePlan *sp) {
  sp->rpm = next_pow2(G * nq);
  if (sp->rpm > kVerifyRows)
    return fail(PKV_EINVAL, "G * nq = %d * %d rows per member exceed one 16-row tile", G, nq);
  if (n_groups <= 0 || max_members < 1 || max_prefix < kTile || max_prefix % kTile)
    return fail(PKV_EINVAL, "group sizes: n_groups %d, max_members %d, max_prefix %d", n_groups,
                max_members, max_prefix);
  const int32_t mpt = kVerifyRows / sp->rpm;                 // members per row tile
  const int32_t tiles = (max_members + mpt - 1) / mpt;       // row tiles of the largest group
  sp->W = tiles >= 8 ? 8 : next_pow2(tiles);
  // two row tiles per wavefront share each K/V read where both accumulators
  // fit in registers
  sp->RT = tiles >= 16 && D <= 128 ? 2 : 1;
  sp->chunks = (tiles + sp->W * sp->RT - 1) / (sp->W * sp->RT);
  // enough prefix partitions that the prefix workgroups fill a round
  const int64_t per_part = (int64_t)n_groups * Hkv * sp->chunks * sp->W;
  int64_t npp = (kResidentWaves + per_part - 1) / per_part;
  if (npp > max_prefix / kTile) npp = max_prefix / kTile;
  if (npp < 1) npp = 1;
  sp->pp = (int32_t)(((max_prefix + npp - 1) / npp + kTile - 1) / kTile * kTile);
  sp->npp = (max_prefix + sp->pp - 1) / sp->pp;
  if ((int64_t)n_groups * sp->chunks > 65535)
    return fail(PKV_EINVAL, "too many groups for one launch");
  return PKV_OK;
}

}  // namespace

// Tokens past the longest shared prefix up to which the one-pass kernel
// serves a batch: its workgroups stream their members' own tokens alone, so
// long private rests go to the partitioned kernels instead.
constexpr int64_t kOnePassRest = 4096;

static size_t shared_workspace_need(int32_t B, int32_t nq, int32_t Hq, int32_t Hkv, int32_t D,
                                    int64_t max_ctx, int32_t part, const SharePlan &sp) {
  const Plan pl = plan_launch(B, Hkv, max_ctx, part, false);
  return partial_bytes((int64_t)B * nq * Hq, sp.npp + pl.num_parts, D);
}

extern "C" int paged_attention_shared_workspace_size(int32_t B, int32_t nq, int32_t Hq,
                                                     int32_t Hkv, int32_t D, int32_t max_blocks,
                                                     int32_t bs, int32_t part, int32_t n_groups,
                                                     int32_t max_members, int32_t max_prefix,
                                                     size_t *bytes) {
  if (!bytes) return fail(PKV_EINVAL, "bytes is NULL");
  if (int rc = check_sizes(B, nq, Hq, Hkv, D, max_blocks, bs, part)) return rc;
  const int64_t max_ctx = (int64_t)max_blocks * bs;
  size_t need = workspace_need(B, nq, Hq, Hkv, D, max_ctx, part);
  if (n_groups > 0) {
    SharePlan sp;
    if (int rc = share_plan(Hq / Hkv, nq, Hkv, D, n_groups, max_members, max_prefix, &sp)) return rc;
    const size_t n = shared_workspace_need(B, nq, Hq, Hkv, D, max_ctx, part, sp);
    if (n > need) need = n;
  }
  *bytes = need;
  return PKV_OK;
}

extern "C" int paged_attention_decode_shared(
    float *out, const void *q, const void *k_cache, const void *v_cache,
    const int32_t *block_tables, int32_t max_blocks, const int32_t *context_lens, int32_t B,
    int32_t nq, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t num_blocks, float scale,
    int dtype, int32_t part, const int32_t *seq_prefix, const int32_t *group_start,
    const int32_t *members, const int32_t *group_tokens, int32_t n_groups, int32_t n_members,
    int32_t max_members, int32_t max_prefix, void *workspace, size_t workspace_bytes,
    float *lse_out, void *stream) {
  if (n_groups == 0)
    return paged_attention_decode(out, q, k_cache, v_cache, block_tables, max_blocks,
                                  context_lens, B, nq, Hq, Hkv, D, bs, num_blocks, scale, dtype,
                                  part, workspace, workspace_bytes, lse_out, stream);
  if (dtype != PKV_BF16) return fail(PKV_EINVAL, "shared prefixes need a bf16 cache");
  if (int rc = check_sizes(B, nq, Hq, Hkv, D, max_blocks, bs, part)) return rc;
  if (num_blocks <= 0) return fail(PKV_EINVAL, "num_blocks must be positive");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !seq_prefix ||
      !group_start || !members || !group_tokens)
    return fail(PKV_EINVAL, "NULL pointer");
  for (const void *p : {(const void *)out, q, k_cache, v_cache})
    if ((uintptr_t)p % 16) return fail(PKV_EINVAL, "out, q, K and V must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale must be finite");
  if (n_groups < 0 || n_members < 2 * n_groups || n_members > B || max_members > B ||
      max_prefix > max_blocks * bs)
    return fail(PKV_EINVAL, "group sizes out of range");
  const int G = Hq / Hkv;
  if (int rc = check_rows(dtype, nq, G)) return rc;
  SharePlan sp;
  if (int rc = share_plan(G, nq, Hkv, D, n_groups, max_members, max_prefix, &sp)) return rc;
  const int64_t max_ctx = (int64_t)max_blocks * bs;

  // Every sequence in a group, and little past the prefixes: one pass per
  // (KV head, a few members) over the shared prefix and each member's own
  // tokens, merged on chip -- no prefix partials, no reduce launch.
  if (D <= 128 && n_members == B && max_ctx <= (int64_t)max_prefix + kOnePassRest) {
    const int32_t mpt = kVerifyRows / sp.rpm;
    const int64_t wg2 = (int64_t)Hkv * n_groups * ((max_members + 2 * mpt - 1) / (2 * mpt));
    const int32_t RT = wg2 >= kResidentWaves / 8 ? 2 : 1;
    const int32_t chunks = (max_members + RT * mpt - 1) / (RT * mpt);
    GroupLauncher one = pick_group(D, RT);
    if (!one) return fail(PKV_EINVAL, "no one-pass kernel for D=%d", D);
    if ((int64_t)n_groups * chunks > 65535) return fail(PKV_EINVAL, "too many groups for one launch");
    DecodeArgs a{};
    a.out = out;
    a.lse = lse_out;
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tables = block_tables;
    a.lens = context_lens;
    a.B = B;
    a.max_blocks = max_blocks;
    a.nq = nq;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.bs = bs;
    a.num_blocks = num_blocks;
    a.scale_log2 = scale * kLog2e;
    ShareArgs sh{};
    sh.group_start = group_start;
    sh.members = members;
    sh.group_tokens = group_tokens;
    sh.n_groups = n_groups;
    sh.n_members = n_members;
    sh.chunks = chunks;
    sh.rpm = sp.rpm;
    one(a, sh, dim3(Hkv, n_groups * chunks), (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_EHIP, "one-pass launch: %s", hipGetErrorString(e));
    return PKV_OK;
  }

  // the rest of every context: the ordinary kernels, never the stream
  const bool mfma = use_mfma(dtype, nq, G);
  const Plan pl = plan_launch(B, Hkv, max_ctx, part, false);
  int32_t RP, S;
  row_split(G, nq, &RP, &S);
  if (mfma) S = 1;
  Launcher launch = mfma ? pick_verify(D) : pick_launcher(dtype, D, G, RP, pl.waves);
  PrefixLauncher prefix = pick_prefix(D, sp.W, sp.RT);
  if (!launch || !prefix) return fail(PKV_EINVAL, "no kernel for G=%d, nq=%d", G, nq);

  const int32_t slots = sp.npp + pl.num_parts;
  const size_t need = partial_bytes((int64_t)B * nq * Hq, slots, D);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_EINVAL, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if ((uintptr_t)workspace % 256) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");

  DecodeArgs a{};
  a.out = out;
  a.lse = lse_out;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.B = B;
  a.max_blocks = max_blocks;
  a.nq = nq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.bs = bs;
  a.num_blocks = num_blocks;
  a.part_tokens = pl.part_tokens;
  a.num_parts = slots;
  a.slices = S;
  a.scale_log2 = scale * kLog2e;
  a.starts = seq_prefix;
  a.part_base = sp.npp;
  a.prefix_part = sp.pp;
  const int64_t rows = (int64_t)B * nq * Hq;
  char *w = (char *)workspace;
  a.part_acc = (float *)w;
  w += align_up((size_t)rows * slots * D * 4, 256);
  a.part_m = (float *)w;
  w += align_up((size_t)rows * slots * 4, 256);
  a.part_l = (float *)w;

  ShareArgs sh{};
  sh.group_start = group_start;
  sh.members = members;
  sh.group_tokens = group_tokens;
  sh.n_groups = n_groups;
  sh.n_members = n_members;
  sh.chunks = sp.chunks;
  sh.rpm = sp.rpm;
  sh.prefix_part = sp.pp;

  hipStream_t s = (hipStream_t)stream;
  StreamArgs sa{};
  prefix(a, sh, dim3(sp.npp, Hkv, n_groups * sp.chunks), s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "prefix launch: %s", hipGetErrorString(e));
  launch(a, sa, dim3(pl.num_parts, Hkv * S, B), s);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "decode launch: %s", hipGetErrorString(e));
  pick_reduce(D)(a, sa, dim3(nq * Hq, B), s);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "reduce launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
