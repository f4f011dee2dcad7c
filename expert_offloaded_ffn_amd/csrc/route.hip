// moe_route: router logits, selection keys, group-limited top-k, gates and the
// expert histogram.
//
// The pages leave the router arithmetic open ("The Billion-Token Bottleneck",
// section "The Geometry of the Problem": a router decides which few experts
// handle each token). This file implements the reading stated in moe.h.
//
// Kernels:
//  route_logits_mfma  bf16 logits on MFMA 16x16x32, split over K across the waves
//                     of a block (operands read straight from global in the MFMA
//                     fragment layout; the router weights stay L2-resident).
//  route_logits_wide  bf16 logits of large batches over many experts: 64 x 128 tiles
//                     over all of K, both operands through a direct-to-LDS ring.
//  route_logits_f32   fp32 logits, one thread per (token, expert) dot product.
//  route_select       one wavefront per token: keys, group limit, k rounds of a
//                     64-lane arg-max over packed (key, ~index) words, gates, and
//                     a per-block LDS histogram flushed with one atomic per bin.
//  route_logit_slices logits of up to 64 tokens split over K across many workgroups
//                     (moe_route_permute).
//  route_select_slices a wavefront per token: the sum of its slices, then its selection.
//  route_finish_small the slices' sum, then selection and grouping of those tokens in
//                     one workgroup (moe_route_permute).
#include <type_traits>

#include "group_small.h"
#include "lds_dma.h"
#include "moe_internal.h"
#include "route_small.h"

namespace moeffn {
namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxGroups = 64;

// -------------------------------------------------------------- logits ---
// A block owns MT m-tiles of 16 tokens x 64 expert columns (4 n-tiles of 16); its WK
// waves split K, each accumulating MT x 4 MFMA tiles over its K range; the partials are
// summed through LDS in wave order (deterministic) by the first wave. Column c < E reads
// w_router row c; c == E (when w_sg is given) reads w_sg. Small batches, and any batch
// whose experts fit one 64-column group, use MT = 1 and WK = 16; large batches over many
// experts MT = 4, WK = 4.
// Output: raw logits into scores[t, c] for c < E, and into shared_logit[t].
template <int MT, int WK>
__global__ __launch_bounds__(64 * WK) void route_logits_mfma(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w_router,
    const bf16_t* __restrict__ w_sg, float* __restrict__ scores, float* __restrict__ shared_logit,
    int32_t* __restrict__ counts, int T, int d, int E) {
  __shared__ f32x4_t red[WK - 1][MT][4][64];
  if (counts != nullptr && blockIdx.x == 0 && blockIdx.y == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = 0;
  }
  const int ncols = E + (w_sg != nullptr ? 1 : 0);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16 * MT;
  const int c0 = blockIdx.y * 64;
  const int ntile = min(4, (ncols - c0 + 15) / 16);
  const int KT = d / 32;
  const int k0 = (KT * wave) / WK, k1 = (KT * (wave + 1)) / WK;

  const int koff = 8 * (lane >> 4);
  const bf16_t* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) arow[m] = x + (size_t)min(t0 + m * 16 + (lane & 15), T - 1) * d + koff;
  const bf16_t* brow[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int c = min(c0 + n * 16 + (lane & 15), ncols - 1);
    brow[n] = (c < E ? w_router + (size_t)c * d : w_sg) + koff;
  }
  f32x4_t acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // operands of k-step kt + 1 are loaded while the MFMAs of k-step kt run (two register
  // sets, alternating), so each wave keeps two steps of loads in flight
  bf16x8_t b0[4], a0[MT], b1[4], a1[MT];
  auto load = [&](int kt, bf16x8_t* b, bf16x8_t* a) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
      if (n < ntile) b[n] = *reinterpret_cast<const bf16x8_t*>(brow[n] + kt * 32);
#pragma unroll
    for (int m = 0; m < MT; ++m) a[m] = *reinterpret_cast<const bf16x8_t*>(arow[m] + kt * 32);
  };
  auto mma = [&](const bf16x8_t* b, const bf16x8_t* a) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (n < ntile) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
  };
  if (k0 < k1) load(k0, b0, a0);
  for (int kt = k0; kt < k1; kt += 2) {
    if (kt + 1 < k1) load(kt + 1, b1, a1);
    mma(b0, a0);
    if (kt + 1 < k1) {
      if (kt + 2 < k1) load(kt + 2, b0, a0);
      mma(b1, a1);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) red[wave - 1][m][n][lane] = acc[m][n];
  }
  __syncthreads();
  if (wave != 0) return;
  // D layout: lane l holds rows 4*(l/16)+i, column l%16.
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if (n >= ntile) continue;
      f32x4_t v = acc[m][n];
      for (int w = 0; w < WK - 1; ++w) v += red[w][m][n][lane];
      const int c = c0 + n * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + m * 16 + 4 * (lane >> 4) + i;
        if (t < T && c < ncols) {
          if (c < E) scores[(size_t)t * E + c] = v[i];
          else shared_logit[t] = v[i];
        }
      }
    }
}

// More than 256 tokens over more than 64 columns: a block owns 64 tokens x 128 columns over all
// of K, so x is read once per 128 columns and the router weights once per 64 tokens. Both
// operands stream through an LDS ring of kRlStages stages of 64 K-values (direct-to-LDS loads:
// 64 token rows, 8 KiB, and 128 weight rows, 16 KiB, a stage; row r's 16-byte chunk c sits at
// 128 r + 16 (c ^ f(r)), so the 16 rows of a fragment read cover every bank once), issued
// kRlStages - 1 stages ahead of the MFMAs. Wave w owns columns 32w..32w+31 of the block's 64
// tokens: 4 x 2 tiles of 16x16x32 bf16 MFMAs accumulated in k order. Output as
// route_logits_mfma.
constexpr int kRlStages = 6, kRlA = 0, kRlB = 8192, kRlStage = 24576;

__device__ __forceinline__ int rl_swz(int r) { return ((r >> 1) + 4 * (r & 1)) & 7; }

__global__ __launch_bounds__(256) void route_logits_wide(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ w_router,
                                                         const bf16_t* __restrict__ w_sg, float* __restrict__ scores,
                                                         float* __restrict__ shared_logit, int32_t* __restrict__ counts,
                                                         int T, int d, int E) {
  __shared__ __attribute__((aligned(1024))) char ring[kRlStages * kRlStage];
  if (counts != nullptr && blockIdx.x == 0 && blockIdx.y == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = 0;
  }
  const int ncols = E + (w_sg != nullptr ? 1 : 0);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 128;
  const int KS = d / 64;
  // this lane's sources: token rows 16w + 8i + l/8 (i < 2) and weight rows 32w + 8i + l/8
  // (i < 4) of the tile, chunk (l % 8) ^ f(row), which lands at position l % 8 of its row;
  // rows past the last token or column read a clamped copy, never stored
  const bf16_t* asrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * w + 8 * i + (lane >> 3);
    asrc[i] = x + (size_t)min(t0 + r, T - 1) * d + 8 * ((lane & 7) ^ rl_swz(r));
  }
  const bf16_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * w + 8 * i + (lane >> 3);
    const int c = min(c0 + r, ncols - 1);
    bsrc[i] = (c < E ? w_router + (size_t)c * d : w_sg) + 8 * ((lane & 7) ^ rl_swz(r));
  }
  auto issue = [&](int s) {
    char* buf = ring + (s % kRlStages) * kRlStage;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_asm(asrc[i] + s * 64, buf + kRlA + (2 * w + i) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_asm(bsrc[i] + s * 64, buf + kRlB + (4 * w + i) * 1024);
  };
  // fragment offsets within a stage for k-step ks of 2: A row 16 m + l % 16, B row
  // 32 w + 16 n + l % 16, chunk 4 ks + l / 16
  const int fr = rl_swz(lane & 15), g4 = lane >> 4;
  f32x4_t acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int s = 0; s < min(kRlStages - 1, KS); ++s) issue(s);
  for (int s = 0; s < KS; ++s) {
    // stage s has landed for this wave when at most the 6 loads of each later stage already
    // issued are outstanding; the barrier then makes it so for every wave, and every wave is
    // done with stage s - 1's buffer, which the loads issued below overwrite
    switch (min(kRlStages - 2, KS - 1 - s)) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<6>(); break;
      case 2: wait_vmcnt<12>(); break;
      case 3: wait_vmcnt<18>(); break;
      default: wait_vmcnt<24>(); break;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_no_fence();
    if (s + kRlStages - 1 < KS) issue(s + kRlStages - 1);
    const char* buf = ring + (s % kRlStages) * kRlStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 16 * ((4 * ks + g4) ^ fr);
      bf16x8_t a[4], b[2];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        a[m] = *reinterpret_cast<const bf16x8_t*>(buf + kRlA + 128 * (16 * m + (lane & 15)) + ch);
#pragma unroll
      for (int n = 0; n < 2; ++n)
        b[n] = *reinterpret_cast<const bf16x8_t*>(buf + kRlB + 128 * (32 * w + 16 * n + (lane & 15)) + ch);
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
    }
  }
  // D layout: lane l holds rows 4 (l / 16) + i, column l % 16
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int c = c0 + 32 * w + 16 * n + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * m + 4 * g4 + i;
        if (t < T && c < ncols) {
          if (c < E) scores[(size_t)t * E + c] = acc[m][n][i];
          else shared_logit[t] = acc[m][n][i];
        }
      }
    }
}

template <typename T_>
__device__ __forceinline__ float load_as_f32(const T_* p, size_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_f32<bf16_t>(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }

template <typename T_>
__global__ __launch_bounds__(256) void route_logits_valu(
    const T_* __restrict__ x, const T_* __restrict__ w_router, const T_* __restrict__ w_sg,
    float* __restrict__ scores, float* __restrict__ shared_logit, int32_t* __restrict__ counts,
    int T, int d, int E) {
  if (counts != nullptr && blockIdx.x == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = 0;
  }
  const int ncols = E + (w_sg != nullptr ? 1 : 0);
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T * ncols) return;
  const int t = (int)(gid / ncols), c = (int)(gid % ncols);
  const T_* wrow = c < E ? w_router + (size_t)c * d : w_sg;
  float s = 0.f;
  for (int i = 0; i < d; ++i) s = fmaf(load_as_f32(x, (size_t)t * d + i), load_as_f32(wrow, (size_t)i), s);
  if (c < E) scores[(size_t)t * E + c] = s;
  else shared_logit[t] = s;
}

// -------------------------------------------------------------- select ---

constexpr int kSelWaves = 4;     // waves per block

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_select(
    float* __restrict__ scores, const float* __restrict__ logit_bias, const float* __restrict__ select_bias,
    float* __restrict__ shared_gate, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    int32_t* __restrict__ counts, int T, int E, int k, int score_fn, int renormalize, float route_scale,
    int n_groups, int topk_groups, int group_topn, int tok_per_wave) {
  __shared__ int hist[kMaxE];
  __shared__ float wkeys[kSelWaves][kMaxE];
  const int wave = threadIdx.x >> 6;
  if (counts != nullptr)
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int it = 0; it < tok_per_wave; ++it) {
    const int t = (blockIdx.x * kSelWaves + wave) * tok_per_wave + it;
    if (t >= T) break;
    select_token<PER_LANE>(t, scores + (size_t)t * E, scores, logit_bias, select_bias, shared_gate, topk_idx, topk_gate,
                           counts != nullptr ? hist : nullptr, wkeys[wave], E, k, score_fn, renormalize,
                           route_scale, n_groups, topk_groups, group_topn);
  }
  if (counts != nullptr) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      if (hist[e]) atomicAdd(&counts[e], hist[e]);
  }
}

template <int PL>
void launch_select(int tpw, hipStream_t s, float* scores, const float* lb, const float* sb, float* sg,
                   int32_t* idx, float* gate, int32_t* counts, const moe_route_cfg& c) {
  dim3 grid((c.T + kSelWaves * tpw - 1) / (kSelWaves * tpw));
  hipLaunchKernelGGL(route_select<PL>, grid, dim3(256), 0, s, scores, lb, sb, sg, idx, gate, counts, c.T,
                     c.n_experts, c.top_k, c.score_fn, c.renormalize, c.route_scale, c.n_groups,
                     c.topk_groups, c.group_topn, tpw);
}

// -------------------------------------------------------- small batches ---
// The logits of up to 64 tokens split over K (route_slice_wave in route_small.h). Up to 16
// tokens, one workgroup then adds each logit's slices in slice order, selects and groups
// (route_finish_small: select_token, group_small); for more tokens the slices would be as
// many bytes as the router weights, too many for one workgroup to read back, so a wavefront
// per token sums and selects (route_select_slices) and the one-workgroup grouping follows.
// (one workgroup reading back the slices of 17..64 tokens measured slower than the two
// launches: 0.244 vs 0.231 ms per Qwen-shaped step at 64 tokens)
constexpr int kFuseMaxT = 16;
constexpr int kFuseMaxE = 256;

// grid (slices, column groups of 64, m-tiles of 16), 4 waves: wave w takes n-tile w of the
// group. Output: part[slice][t][c] fp32 for t < T, c < E (+1 with the shared gate column).
__global__ __launch_bounds__(256) void route_logit_slices(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ w_router,
                                                          const bf16_t* __restrict__ w_sg, float* __restrict__ part,
                                                          int32_t* __restrict__ counts, int T, int d, int E) {
  const int wave = threadIdx.x >> 6;
  if (counts != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)   // route_select_slices adds to them
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = 0;
  const int ncols = E + (w_sg != nullptr ? 1 : 0);
  const int c0 = blockIdx.y * 64 + wave * 16;
  if (c0 >= ncols) return;   // the whole wave: its n-tile lies past the last column
  route_slice_wave<false>(x, w_router, w_sg, part, T, d, E, ncols, blockIdx.x, c0, blockIdx.z * 16);
}

template <int PER_LANE, int KMAX>
__global__ __launch_bounds__(1024) void route_finish_small(
    const float* __restrict__ part, int nsl, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, float* __restrict__ shared_gate, float* __restrict__ scores,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src, int32_t* __restrict__ perm_dst, int T, int E,
    int ncols, int k, int score_fn, int renormalize, float route_scale, int n_groups, int topk_groups,
    int group_topn) {
  __shared__ float lg[kFuseMaxT * (kFuseMaxE + 1)];   // the summed logits, [t][ncols]
  __shared__ float wkeys[16][kFuseMaxE];
  __shared__ int32_t off[kFuseMaxE];
  __shared__ int32_t wave_sum[16];
  __shared__ int32_t idx_lds[kFuseMaxT * 32];   // the selection, read back by the grouping
  const int wave = threadIdx.x >> 6;
  route_sum_slices<false>(part, nsl, T * ncols, 0, T * ncols, lg, scores, shared_gate, E, ncols);
  __syncthreads();
  for (int t = wave; t < T; t += 16)
    select_token<PER_LANE>(t, lg + t * ncols, scores, logit_bias, select_bias, shared_gate, topk_idx, topk_gate, nullptr,
                           wkeys[wave], E, k, score_fn, renormalize, route_scale, n_groups, topk_groups, group_topn,
                           idx_lds);
  __syncthreads();
  group_small<KMAX>(idx_lds, counts, offsets, perm_src, perm_dst, T, k, E, off, wave_sum);
}

// 17..64 tokens: one wavefront per token sums the token's slices (slice order, 8 slice loads
// in flight per column) into an LDS row, then selects on it like route_select (the
// expert histogram included); moe_permute's one-workgroup grouping follows.
constexpr int kSliceMaxT = 64;

template <int PER_LANE>
__global__ __launch_bounds__(64 * kSelWaves) void route_select_slices(
    const float* __restrict__ part, int nsl, int ncols, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, float* __restrict__ shared_gate, float* __restrict__ scores,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, int32_t* __restrict__ counts, int T, int E, int k,
    int score_fn, int renormalize, float route_scale, int n_groups, int topk_groups, int group_topn) {
  __shared__ int hist[kFuseMaxE];
  __shared__ float wkeys[kSelWaves][kFuseMaxE];
  __shared__ float lg[kSelWaves][kFuseMaxE + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (counts != nullptr)
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kSelWaves + wave;
  if (t < T) {
    for (int c = lane; c < ncols; c += 64) {
      float v = 0.f;
      for (int s0 = 0; s0 < nsl; s0 += 8) {
        float buf[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (s0 + q < nsl) buf[q] = part[((size_t)(s0 + q) * T + t) * ncols + c];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (s0 + q < nsl) v = (s0 + q == 0) ? buf[q] : v + buf[q];
      }
      lg[wave][c] = v;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (shared_gate != nullptr && lane == 0) shared_gate[t] = lg[wave][E];   // the raw logit; sigmoid below
    select_token<PER_LANE>(t, lg[wave], scores, logit_bias, select_bias, shared_gate, topk_idx, topk_gate,
                           counts != nullptr ? hist : nullptr, wkeys[wave], E, k, score_fn, renormalize,
                           route_scale, n_groups, topk_groups, group_topn);
  }
  if (counts != nullptr) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      if (hist[e]) atomicAdd(&counts[e], hist[e]);
  }
}

// Configuration checks shared by moe_route and moe_route_permute.
moe_status check_route_cfg(const moe_route_cfg& c, const char* who) {
  MOE_REQUIRE(c.T >= 0, MOE_EINVAL, "%s: T=%d < 0", who, c.T);
  MOE_REQUIRE(c.d_model >= 1 && c.d_model % 8 == 0, MOE_EINVAL, "%s: d_model=%d must be a positive multiple of 8", who,
              c.d_model);
  MOE_REQUIRE(c.n_experts >= 1 && c.n_experts <= kMaxE, MOE_EINVAL, "%s: n_experts=%d outside [1, %d]", who,
              c.n_experts, kMaxE);
  MOE_REQUIRE(c.top_k >= 1 && c.top_k <= c.n_experts && c.top_k <= kMaxK, MOE_EINVAL,
              "%s: top_k=%d outside [1, min(E, %d)]", who, c.top_k, kMaxK);
  MOE_REQUIRE(c.score_fn == MOE_SOFTMAX || c.score_fn == MOE_SIGMOID, MOE_EINVAL, "%s: bad score_fn %d", who,
              c.score_fn);
  MOE_REQUIRE(c.act_dtype == MOE_F32 || c.act_dtype == MOE_BF16, MOE_EUNSUPPORTED, "%s: act_dtype %d unsupported", who,
              c.act_dtype);
  const int G = c.n_groups < 1 ? 1 : c.n_groups;
  if (G > 1) {
    MOE_REQUIRE(G <= kMaxGroups && c.n_experts % G == 0, MOE_EINVAL, "%s: n_groups=%d must divide E=%d (max %d)", who,
                G, c.n_experts, kMaxGroups);
    MOE_REQUIRE(c.topk_groups >= 1 && c.topk_groups <= G, MOE_EINVAL, "%s: topk_groups=%d outside [1, n_groups]", who,
                c.topk_groups);
    MOE_REQUIRE(c.group_topn >= 1 && c.group_topn <= c.n_experts / G && c.group_topn <= 8, MOE_EINVAL,
                "%s: group_topn=%d outside [1, min(E/n_groups, 8)]", who, c.group_topn);
    MOE_REQUIRE(c.top_k <= c.topk_groups * (c.n_experts / G), MOE_EINVAL, "%s: top_k exceeds the experts of the kept groups",
                who);
  }
  return MOE_OK;
}

}  // namespace

moe_status check_route_config(const moe_route_cfg& c, const char* who) { return check_route_cfg(c, who); }

}  // namespace moeffn

using namespace moeffn;

extern "C" moe_status moe_route(const moe_route_cfg* cfg, const void* x, const void* w_router,
                                const float* logit_bias, const float* select_bias,
                                const void* w_shared_gate, float* shared_gate, float* scores,
                                int32_t* topk_idx, float* topk_gate, int32_t* counts, void* stream) {
  clear_error();
  MOE_REQUIRE(cfg != nullptr, MOE_EINVAL, "moe_route: cfg is NULL");
  const moe_route_cfg c = *cfg;
  if (moe_status st = check_route_cfg(c, "moe_route")) return st;
  MOE_REQUIRE(!(select_bias && c.score_fn == MOE_SOFTMAX), MOE_EINVAL, "moe_route: select_bias needs sigmoid scoring");
  const int G = c.n_groups < 1 ? 1 : c.n_groups;
  if (c.T == 0) return MOE_OK;   // nothing to write: empty outputs may have null pointers
  MOE_REQUIRE((w_shared_gate == nullptr) == (shared_gate == nullptr), MOE_EINVAL,
              "moe_route: w_shared_gate and shared_gate go together");
  MOE_REQUIRE(x && w_router && scores && topk_idx && topk_gate, MOE_EINVAL, "moe_route: NULL tensor argument");
  MOE_REQUIRE(aligned(x, 16) && aligned(w_router, 16) && (!w_shared_gate || aligned(w_shared_gate, 16)), MOE_EINVAL,
              "moe_route: x, w_router, w_shared_gate must be 16-byte aligned");

  moe_route_cfg cc = c;
  cc.n_groups = G;
  hipStream_t s = as_stream(stream);
  const int ncols = c.n_experts + (w_shared_gate ? 1 : 0);
  if (c.act_dtype == MOE_BF16 && c.d_model % 32 == 0) {
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w_router);
    const bf16_t* sgb = static_cast<const bf16_t*>(w_shared_gate);
    // 16-token blocks fill the chip when one 64-column group covers every expert; with
    // more columns, 64-token blocks re-read x fewer times
    if (c.T <= 256 || ncols <= 64) {
      dim3 grid((c.T + 15) / 16, (ncols + 63) / 64);
      hipLaunchKernelGGL((route_logits_mfma<1, 16>), grid, dim3(1024), 0, s, xb, wb, sgb, scores, shared_gate, counts,
                         c.T, c.d_model, c.n_experts);
    } else if (c.d_model % 64 == 0) {
      dim3 grid((c.T + 63) / 64, (ncols + 127) / 128);
      hipLaunchKernelGGL(route_logits_wide, grid, dim3(256), 0, s, xb, wb, sgb, scores, shared_gate, counts, c.T,
                         c.d_model, c.n_experts);
    } else {
      dim3 grid((c.T + 63) / 64, (ncols + 63) / 64);
      hipLaunchKernelGGL((route_logits_mfma<4, 4>), grid, dim3(256), 0, s, xb, wb, sgb, scores, shared_gate, counts,
                         c.T, c.d_model, c.n_experts);
    }
  } else {
    const long long n = (long long)c.T * ncols;
    dim3 grid((unsigned)((n + 255) / 256));
    if (c.act_dtype == MOE_BF16)
      hipLaunchKernelGGL(route_logits_valu<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(w_router), static_cast<const bf16_t*>(w_shared_gate), scores,
                         shared_gate, counts, c.T, c.d_model, c.n_experts);
    else
      hipLaunchKernelGGL(route_logits_valu<float>, grid, dim3(256), 0, s, static_cast<const float*>(x),
                         static_cast<const float*>(w_router), static_cast<const float*>(w_shared_gate), scores,
                         shared_gate, counts, c.T, c.d_model, c.n_experts);
  }
  if (moe_status st = check_launch("moe_route logits")) return st;
  const int per_lane = (c.n_experts + 63) / 64;
  // Tokens per wavefront. A large batch over at most 64 experts takes 2 (fewer, fuller
  // workgroups for a short selection); over more experts, whose selection is a long chain of
  // dependent wave reductions, 1, so more wavefronts per SIMD hide it (DeepSeek-V3 shape,
  // 8192 tokens: 62 vs 90 us with 4 per wavefront; Mixtral shape: 12.0 vs 13.1 us with 2).
  const int tpw = c.T >= 2048 && per_lane <= 1 ? 2 : 1;
  if (per_lane <= 1) launch_select<1>(tpw, s, scores, logit_bias, select_bias, shared_gate, topk_idx, topk_gate, counts, cc);
  else if (per_lane <= 2) launch_select<2>(tpw, s, scores, logit_bias, select_bias, shared_gate, topk_idx, topk_gate, counts, cc);
  else if (per_lane <= 4) launch_select<4>(tpw, s, scores, logit_bias, select_bias, shared_gate, topk_idx, topk_gate, counts, cc);
  else launch_select<16>(tpw, s, scores, logit_bias, select_bias, shared_gate, topk_idx, topk_gate, counts, cc);
  return check_launch("moe_route select");
}

extern "C" size_t moe_route_permute_workspace_size(int32_t T, int32_t k, int32_t E, int32_t d_model) {
  if (T < 0 || E < 1 || d_model < 1) return 0;
  const size_t grouping = moe_permute_workspace_size(T, k, E);
  // the logit slices exist only on the sliced path (bf16 is checked at the call)
  const bool sliced = T >= 1 && T <= kSliceMaxT && E <= kFuseMaxE && d_model % 32 == 0;
  const size_t slices = sliced ? align_up((size_t)route_slices(d_model) * T * (E + 1) * sizeof(float), 256) : 0;
  return grouping > slices ? grouping : slices;
}

extern "C" moe_status moe_route_permute(const moe_route_cfg* cfg, const void* x, const void* w_router,
                                        const float* logit_bias, const float* select_bias,
                                        const void* w_shared_gate, float* shared_gate, float* scores,
                                        int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets,
                                        int32_t* perm_src, int32_t* perm_dst, void* ws, size_t ws_bytes,
                                        void* stream) {
  clear_error();
  MOE_REQUIRE(cfg != nullptr, MOE_EINVAL, "moe_route_permute: cfg is NULL");
  const moe_route_cfg c = *cfg;
  if (moe_status st = check_route_cfg(c, "moe_route_permute")) return st;
  const size_t need = moe_route_permute_workspace_size(c.T, c.top_k, c.n_experts, c.d_model);
  MOE_REQUIRE(ws_bytes >= need, MOE_ECAPACITY, "moe_route_permute: workspace %zu < %zu bytes", ws_bytes, need);
  const bool sliced = c.T >= 1 && c.T <= kSliceMaxT && c.n_experts <= kFuseMaxE && c.act_dtype == MOE_BF16 &&
                      c.d_model % 32 == 0;
  if (!sliced) {
    if (moe_status st = moe_route(cfg, x, w_router, logit_bias, select_bias, w_shared_gate, shared_gate, scores,
                                  topk_idx, topk_gate, counts, stream))
      return st;
    return moe_permute(c.T, c.top_k, c.n_experts, topk_idx, offsets, perm_src, perm_dst, 0, nullptr, 0, nullptr, 0,
                       nullptr, 0, ws, ws_bytes, stream);
  }
  MOE_REQUIRE(!(select_bias && c.score_fn == MOE_SOFTMAX), MOE_EINVAL,
              "moe_route_permute: select_bias needs sigmoid scoring");
  MOE_REQUIRE((w_shared_gate == nullptr) == (shared_gate == nullptr), MOE_EINVAL,
              "moe_route_permute: w_shared_gate and shared_gate go together");
  MOE_REQUIRE(x && w_router && scores && topk_idx && topk_gate && offsets && perm_src && perm_dst && ws, MOE_EINVAL,
              "moe_route_permute: NULL tensor argument");
  MOE_REQUIRE(aligned(x, 16) && aligned(w_router, 16) && (!w_shared_gate || aligned(w_shared_gate, 16)) &&
                  aligned(ws, 16),
              MOE_EINVAL, "moe_route_permute: x, w_router, w_shared_gate and ws must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  const int G = c.n_groups < 1 ? 1 : c.n_groups;
  const int ncols = c.n_experts + (w_shared_gate ? 1 : 0);
  const int nsl = route_slices(c.d_model);
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(route_logit_slices, dim3(nsl, (ncols + 63) / 64, (c.T + 15) / 16), dim3(256), 0, s,
                     static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router),
                     static_cast<const bf16_t*>(w_shared_gate), part, counts, c.T, c.d_model, c.n_experts);
  if (c.T > kFuseMaxT) {
    auto sel = [&](auto pl) {
      constexpr int PL = decltype(pl)::value;
      hipLaunchKernelGGL((route_select_slices<PL>), dim3((c.T + kSelWaves - 1) / kSelWaves), dim3(64 * kSelWaves), 0,
                         s, part, nsl, ncols, logit_bias, select_bias, shared_gate, scores, topk_idx, topk_gate, counts,
                         c.T, c.n_experts, c.top_k, c.score_fn, c.renormalize, c.route_scale, G, c.topk_groups,
                         c.group_topn);
    };
    if (c.n_experts <= 64) sel(std::integral_constant<int, 1>{});
    else if (c.n_experts <= 128) sel(std::integral_constant<int, 2>{});
    else sel(std::integral_constant<int, 4>{});
    if (moe_status st = check_launch("moe_route_permute select")) return st;
    // at most 64 tokens: the one-workgroup grouping, which leaves the partials in ws alone
    return moe_permute(c.T, c.top_k, c.n_experts, topk_idx, offsets, perm_src, perm_dst, 0, nullptr, 0, nullptr, 0,
                       nullptr, 0, ws, ws_bytes, stream);
  }
  auto go = [&](auto pl, auto km) {
    constexpr int PL = decltype(pl)::value, KM = decltype(km)::value;
    hipLaunchKernelGGL((route_finish_small<PL, KM>), dim3(1), dim3(1024), 0, s, part, nsl, logit_bias, select_bias,
                       shared_gate, scores, topk_idx, topk_gate, counts, offsets, perm_src, perm_dst, c.T,
                       c.n_experts, ncols, c.top_k, c.score_fn, c.renormalize, c.route_scale, G, c.topk_groups,
                       c.group_topn);
  };
  auto by_k = [&](auto pl) {
    if (c.top_k <= 2) go(pl, std::integral_constant<int, 2>{});
    else if (c.top_k <= 4) go(pl, std::integral_constant<int, 4>{});
    else if (c.top_k <= 8) go(pl, std::integral_constant<int, 8>{});
    else go(pl, std::integral_constant<int, 32>{});
  };
  if (c.n_experts <= 64) by_k(std::integral_constant<int, 1>{});
  else if (c.n_experts <= 128) by_k(std::integral_constant<int, 2>{});
  else by_k(std::integral_constant<int, 4>{});
  return check_launch("moe_route_permute");
}
