// Paged attention decode for gfx950 (MI355X): launch planning, the
// log-sum-exp reduce kernel, and the C-ABI entry points.
//
// The partition kernel and the method it implements are described in
// decode_kernel.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "decode_kernel.h"
#include "verify_mfma.h"
#include "pagedkv.h"
#include "status.h"

namespace pkv {
namespace decode {
namespace {

// One workgroup per (query row, sequence); thread d owns output element d.
template <int D>
__global__ void __launch_bounds__(D)
reduce_partitions_kernel(const DecodeArgs a) {
  constexpr float kNegInf = -std::numeric_limits<float>::infinity();
  const int rowq = blockIdx.x;  // qi * Hq + h
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = load_const(a.lens + b);
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

// Launch plan. The chip holds about kResidentWaves decode wavefronts at once
// (256 CUs x 4 SIMDs x 2 wavefronts at ~190-230 VGPRs each).
//  * Workgroup-split (waves = 4 or 8): one workgroup per (partition, KV
//    head, sequence). With one partition it needs no workspace and no
//    reduce launch: the choice when the (sequence, KV head) pairs alone
//    fill a round of long-running wavefronts and lengths are alike.
//  * Stream (waves = 0): kResidentWaves persistent wavefronts share the
//    stream of all tiles equally, cut at requested partition boundaries;
//    a reduce launch merges the segments. The choice for a requested
//    partition size, for balanced scheduling of mixed lengths
//    (partition_tokens = -1), and when the pairs are too few.
constexpr int64_t kResidentWaves = 2048;
constexpr int64_t kMaxStreamSeqs = 8000;  // LDS holds two per-sequence prefixes

struct Plan {
  int waves;          // 4 or 8: workgroup-split kernel; 0: stream kernel
  int32_t part_tokens;  // stream: 0 = no partition cuts
  int32_t num_parts;    // workgroup-split: partitions per context
  int32_t grid_x;
};

Plan plan_launch(int64_t B, int64_t Hkv, int64_t max_ctx, int32_t req, bool stream_ok) {
  Plan pl{};
  const int64_t units = B * Hkv;
  const int64_t whole = (max_ctx + kTile - 1) / kTile * kTile;  // one partition
  bool stream;
  int64_t P;
  if (req == -1) {
    stream = true;
    P = 0;
  } else if (req > 0) {
    P = req;
    stream = (max_ctx + P - 1) / P > 1;
  } else {  // stream only long contexts of too few pairs
    stream = units * 8 < kResidentWaves && max_ctx >= 1024;
    P = stream ? 0 : whole;
  }
  if (stream && stream_ok && B <= kMaxStreamSeqs) {
    pl.waves = 0;
    pl.part_tokens = (int32_t)P;
    pl.num_parts = P > 0 ? (int32_t)((max_ctx + P - 1) / P) : 1;
    pl.grid_x = (int32_t)(kResidentWaves / kStreamWaves);
    return pl;
  }
  if (P <= 0) P = whole;
  pl.part_tokens = (int32_t)P;
  pl.num_parts = (int32_t)((max_ctx + P - 1) / P);
  if (pl.num_parts < 1) pl.num_parts = 1;
  const int64_t tiles_per_part = (P + kTile - 1) / kTile;
  pl.waves = (tiles_per_part >= 64 && units * pl.num_parts * 8 <= 2 * kResidentWaves) ? 8 : 4;
  pl.grid_x = pl.num_parts;
  return pl;
}

template <int D>
void launch_reduce(const DecodeArgs &a, const StreamArgs &, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((reduce_partitions_kernel<D>), grid, dim3(D), 0, s, a);
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

// Stream launch workspace: the two per-sequence prefixes, then segment
// partials acc [S, RP, D], m, l [S, RP] with S = N + units * NP segment ids.
size_t stream_segments(int64_t units, int32_t NP) { return kResidentWaves + units * NP; }
size_t stream_bytes(int64_t B, int64_t units, int32_t NP, int32_t RP, int32_t D) {
  const size_t S = stream_segments(units, NP);
  return 2 * align_up((size_t)(B + 1) * 4, 256) + align_up(S * RP * D * 4, 256) +
         2 * align_up(S * RP * 4, 256);
}

Launcher pick_launcher(int dtype, int D, int G, int RP, int NS, int W) {
  if (dtype == PKV_F32) {
    if (D == 64) return pick_rows<PKV_F32, 64>(G, RP, NS, W);
    if (D == 128) return pick_rows<PKV_F32, 128>(G, RP, NS, W);
    if (D == 256) return pick_rows<PKV_F32, 256>(G, RP, NS, W);
  } else if (dtype == PKV_BF16) {
    if (D == 64) return pick_rows<PKV_BF16, 64>(G, RP, NS, W);
    if (D == 128) return pick_rows<PKV_BF16, 128>(G, RP, NS, W);
    if (D == 256) return pick_rows<PKV_BF16, 256>(G, RP, NS, W);
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

static int check_rows(int dtype, int32_t nq, int32_t G) {
  if (use_mfma(dtype, nq, G)) return PKV_OK;
  if (G * next_pow2(nq) > kMaxRows)
    return fail(PKV_EINVAL, "G * nq = %d * %d exceeds the supported rows per KV head", G, nq);
  return PKV_OK;
}

// Workspace a launch needs, for either kernel family (the larger of the two
// possibilities, so the size does not depend on the dtype).
// How the VALU kernels hold the G * nq query rows of a KV head (rounded up
// to a power of two): sets of RP <= 4 rows, NS <= 2 sets per wavefront
// sharing every loaded tile, and S wavefront slices when more rows remain
// (a slice streams the KV head's bytes again, so it is the last resort).
static void row_split(int32_t G, int32_t nq, int32_t *RP, int32_t *NS, int32_t *S) {
  const int32_t all = G * next_pow2(nq);
  *RP = all < 4 ? all : 4;
  *NS = all / *RP < 2 ? all / *RP : 2;
  *S = all / (*RP * *NS);
}

static size_t workspace_need(int32_t B, int32_t nq, int32_t Hq, int32_t Hkv, int32_t D,
                             int64_t max_ctx, int32_t part) {
  int32_t RP, NS, S;
  row_split(Hq / Hkv, nq, &RP, &NS, &S);
  const int64_t units = (int64_t)B * Hkv * S;
  const int32_t RW = RP * NS;
  size_t need = 0;
  for (bool stream_ok : {true, false}) {
    const Plan pl = plan_launch(B, Hkv, max_ctx, part, stream_ok);
    size_t n = 0;
    if (pl.waves == 0)
      n = stream_bytes(B, units, pl.num_parts, RW, D);
    else if (pl.num_parts > 1)
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
  *bytes = workspace_need(B, nq, Hq, Hkv, D, (int64_t)max_blocks * bs, part);
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
  const int G = Hq / Hkv;
  if (int rc = check_rows(dtype, nq, G)) return rc;
  const bool mfma = use_mfma(dtype, nq, G);
  const Plan pl = plan_launch(B, Hkv, (int64_t)max_blocks * bs, part, !mfma);
  const int32_t P = pl.part_tokens, NP = pl.num_parts;
  int32_t RP, NS, S;
  row_split(G, nq, &RP, &NS, &S);
  if (mfma) S = 1;
  const int32_t RW = RP * NS;
  Launcher launch = mfma ? pick_verify(D) : pick_launcher(dtype, D, G, RP, NS, pl.waves);
  if (!launch) return fail(PKV_EINVAL, "no kernel for G=%d, nq=%d", G, nq);
  const bool streamed = pl.waves == 0 && !mfma;
  const dim3 grid = streamed ? dim3(pl.grid_x) : dim3(NP, Hkv * S, B);
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
  StreamArgs sa{};
  size_t need = 0;
  if (streamed)
    need = stream_bytes(B, (int64_t)B * Hkv * S, NP, RW, D);
  else if (NP > 1)
    need = partial_bytes((int64_t)B * nq * Hq, NP, D);
  if (need) {
    if (!workspace || workspace_bytes < need)
      return fail(PKV_EINVAL, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if ((uintptr_t)workspace % 256) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
    char *w = (char *)workspace;
    if (streamed) {
      const size_t nseg = stream_segments((int64_t)B * Hkv * S, NP);
      sa.tile_pre = (int32_t *)w;
      w += align_up((size_t)(B + 1) * 4, 256);
      sa.part_pre = (int32_t *)w;
      w += align_up((size_t)(B + 1) * 4, 256);
      sa.n_waves = (int32_t)(pl.grid_x * kStreamWaves);
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
