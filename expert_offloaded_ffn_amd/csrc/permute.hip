// moe_permute: stable expert-major grouping of the (token, slot) pairs, and the
// optional row gather / per-row e4m3 quantisation of the expert inputs.
//
// The grouping lets each selected expert run once over all of its rows ("NovaLLM:
// Running Massive MoE Models Fully In-Memory", section 3: only the experts that
// were hit run). The order inside an expert is by ascending token, which makes
// the permutation unique and the whole path deterministic.
//
// Three passes of a counting sort over blocks of 64 tokens (a block's experts are split over
// the kPermWaves wavefronts of its workgroup, each walking its share: e = w, w + kPermWaves, ...):
//  block_counts  for every expert e, a 64-lane ballot of "this token picked e";
//                popcount = the block's count for e.
//  scan          one 1024-thread block: chunked sums over the blocks of each
//                expert, shuffle scans over the chunks and over the experts give
//                offsets and base[b][e] = offsets[e] + sum_{b'<b} cnt[b'][e].
//  scatter       the same ballots; a pair's row is base[b][e] plus the number
//                of lower lanes (= earlier tokens) in the ballot.
// A batch of at most 64 tokens runs all three passes in one workgroup (permute_small).
#include <type_traits>

#include "group_small.h"
#include "moe_internal.h"

namespace moeffn {
namespace {

constexpr int kMaxE = 1024;
// Wavefronts per 64-token block in the count and scatter passes: the walk over the experts is
// a chain of dependent ballots, so splitting it shortens each chain (DeepSeek-V3 shape: 8192
// tokens, 256 experts).
constexpr int kPermWaves = 4;

// KMAX is a compile-time bound on k, so each lane's expert list stays in registers.
template <int KMAX>
__global__ __launch_bounds__(64 * kPermWaves) void permute_block_counts(const int32_t* __restrict__ idx,
                                                                        int32_t* __restrict__ cnt, int T, int k,
                                                                        int E) {
  const int b = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = b * 64 + lane;
  int mine[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) mine[j] = (t < T && j < k) ? idx[(size_t)t * k + j] : -1;
  for (int e = w; e < E; e += kPermWaves) {
    bool has = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) has |= (mine[j] == e);
    const uint64_t m = __ballot(has);
    if (lane == 0) cnt[(size_t)b * E + e] = __popcll(m);
  }
}

// One block of 1024 threads. Each expert's blocks are split into C chunks (C a power of
// two, at most 64, with C * E <= 1024); thread (e, c) = (tid / C, tid % C) sums the
// counts of chunk c, the C chunk sums of an expert (adjacent lanes of one wavefront) are
// scanned with shuffles, the expert totals are scanned across the block into offsets,
// and every thread then writes base[b][e] for the blocks of its chunk.
__global__ __launch_bounds__(1024) void permute_scan(const int32_t* __restrict__ cnt, int32_t* __restrict__ base,
                                                     int32_t* __restrict__ offsets, int nb, int E) {
  __shared__ int32_t off[kMaxE];
  __shared__ int32_t wave_sum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int C = 64;
  while (C > 1 && C * E > 1024) C >>= 1;
  const int e = tid / C, c = tid % C;
  const bool on = e < E;
  const int per = (nb + C - 1) / C;
  const int b0 = min(nb, c * per), b1 = min(nb, b0 + per);
  // (the counts are loaded 8 at a time, so a thread's chunk costs a few memory round trips,
  // not one per block)
  int sum = 0;
  if (on)
    for (int b = b0; b < b1; b += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = b + u < b1 ? cnt[(size_t)(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
  int inc = sum;   // inclusive scan over the chunks of expert e
  for (int o = 1; o < C; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (c >= o) inc += v;
  }
  if (on && c == C - 1) off[e] = inc;   // expert total
  __syncthreads();
  // exclusive scan of the E totals: within each wavefront, then across wavefronts
  const int t = tid < E ? off[tid] : 0;
  int ti = t;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(ti, o, 64);
    if (lane >= o) ti += v;
  }
  if (lane == 63) wave_sum[wave] = ti;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_sum[w];
  const int excl = before + ti - t;
  __syncthreads();   // every thread has read off[] before it is overwritten
  if (tid < E) {
    off[tid] = excl;
    offsets[tid] = excl;
  }
  if (tid == E - 1) offsets[E] = excl + t;
  __syncthreads();
  if (on) {
    int running = off[e] + inc - sum;
    for (int b = b0; b < b1; b += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = b + u < b1 ? cnt[(size_t)(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b + u < b1) {
          base[(size_t)(b + u) * E + e] = running;
          running += v[u];
        }
    }
  }
}

// T <= 64 (a single block of tokens): the three passes in one workgroup of 16 wavefronts.
// One block of at most 64 tokens: the whole counting sort in one workgroup.
template <int KMAX>
__global__ __launch_bounds__(1024) void permute_small(const int32_t* __restrict__ idx, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm_src, int32_t* __restrict__ perm_dst,
                                                      int T, int k, int E) {
  __shared__ int32_t off[kMaxE];
  __shared__ int32_t wave_sum[16];
  group_small<KMAX>(idx, nullptr, offsets, perm_src, perm_dst, T, k, E, off, wave_sum);
}

template <int KMAX>
__global__ __launch_bounds__(64 * kPermWaves) void permute_scatter(const int32_t* __restrict__ idx,
                                                                   const int32_t* __restrict__ cnt,
                                                                   const int32_t* __restrict__ base,
                                                                   int32_t* __restrict__ perm_src,
                                                                   int32_t* __restrict__ perm_dst, int T, int k, int E) {
  const int b = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = b * 64 + lane;
  int mine[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) mine[j] = (t < T && j < k) ? idx[(size_t)t * k + j] : -1;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = w; e < E; e += kPermWaves) {
    if (cnt[(size_t)b * E + e] == 0) continue;  // uniform across the wave
    int jj = -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) jj = (mine[j] == e) ? j : jj;
    const uint64_t m = __ballot(jj >= 0);
    if (jj >= 0) {
      const int r = base[(size_t)b * E + e] + __popcll(m & below);
      const int p = t * k + jj;
      perm_src[r] = p;
      perm_dst[p] = r;
    }
  }
}

// ------------------------------------------------------------- gather ---
// One wavefront per output row, 16 bytes per lane per step.
__global__ __launch_bounds__(256) void gather_rows_copy(const uint8_t* __restrict__ x, uint8_t* __restrict__ out,
                                                        const int32_t* __restrict__ perm_src, int rows, int k,
                                                        int row_bytes) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int src = perm_src ? perm_src[r] / k : r;
  const uint4* s = reinterpret_cast<const uint4*>(x + (size_t)src * row_bytes);
  uint4* o = reinterpret_cast<uint4*>(out + (size_t)r * row_bytes);
  for (int i = lane; i < row_bytes / 16; i += 64) o[i] = s[i];
}

// One wavefront per row; 16 lanes x 8 values cover a 128-column block.
template <typename TIn>
__global__ __launch_bounds__(256) void gather_rows_quant_e4m3(const TIn* __restrict__ x, uint8_t* __restrict__ out,
                                                              float* __restrict__ out_scale,
                                                              const int32_t* __restrict__ perm_src, int rows, int k,
                                                              int d) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int src = perm_src ? perm_src[r] / k : r;
  const TIn* xs = x + (size_t)src * d;
  for (int c0 = 0; c0 < d; c0 += 512) {   // 4 blocks of 128 per step
    const int col = c0 + lane * 8;
    float v[8];
    if (col < d) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (sizeof(TIn) == 2) v[i] = bf16_to_f32(xs[col + i]);
        else v[i] = xs[col + i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = max_row16(amax);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    if (col < d) {
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(v[i] / scale, -448.0f), 448.0f);
      const uint32_t lo = f32x4_to_e4m3x4(q[0], q[1], q[2], q[3]);
      const uint32_t hi = f32x4_to_e4m3x4(q[4], q[5], q[6], q[7]);
      *reinterpret_cast<uint2*>(out + (size_t)r * d + col) = make_uint2(lo, hi);
      if ((lane & 15) == 0) out_scale[(size_t)r * (d / 128) + col / 128] = scale;
    }
  }
}

// OCP MXFP8 conversion, one wavefront per row; 4 lanes x 8 values cover a 32-value block:
// shared exponent X = floor(log2 max|v|) - 8 (clamped to [-127, 127], -127 for a zero block),
// codes e4m3_rne(clamp(v * 2^-X, +-448)) (the scaling is exact), E8M0 byte X + 127.
template <typename TIn>
__global__ __launch_bounds__(256) void gather_rows_quant_mxfp8(const TIn* __restrict__ x, uint8_t* __restrict__ out,
                                                               uint8_t* __restrict__ out_exp,
                                                               const int32_t* __restrict__ perm_src, int rows, int k,
                                                               int d) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int src = perm_src ? perm_src[r] / k : r;
  const TIn* xs = x + (size_t)src * d;
  for (int c0 = 0; c0 < d; c0 += 512) {   // 16 blocks of 32 per step
    const int col = c0 + lane * 8;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (col < d) {
        if constexpr (sizeof(TIn) == 2) v[i] = bf16_to_f32(xs[col + i]);
        else v[i] = xs[col + i];
      } else {
        v[i] = 0.f;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = max_quad(amax);
    const int X = min(max(amax > 0.f ? ilogbf(amax) - 8 : -127, -127), 127);
    if (col < d) {
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(ldexpf(v[i], -X), -448.0f), 448.0f);
      const uint32_t lo = f32x4_to_e4m3x4(q[0], q[1], q[2], q[3]);
      const uint32_t hi = f32x4_to_e4m3x4(q[4], q[5], q[6], q[7]);
      *reinterpret_cast<uint2*>(out + (size_t)r * d + col) = make_uint2(lo, hi);
      if ((lane & 3) == 0) out_exp[(size_t)r * (d / 32) + col / 32] = static_cast<uint8_t>(X + 127);
    }
  }
}

}  // namespace
}  // namespace moeffn

using namespace moeffn;

extern "C" size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  const size_t nb = (size_t)(T + 63) / 64;
  return align_up(nb * E * sizeof(int32_t), 256) * 2;
}

extern "C" moe_status moe_permute(int32_t T, int32_t k, int32_t E, const int32_t* topk_idx, int32_t* offsets,
                                  int32_t* perm_src, int32_t* perm_dst, int32_t d, const void* x, int32_t x_dtype,
                                  void* x_out, int32_t out_dtype, float* x_out_scale, int32_t gather, void* ws,
                                  size_t ws_bytes, void* stream) {
  clear_error();
  MOE_REQUIRE(T >= 0, MOE_EINVAL, "moe_permute: T=%d < 0", T);
  MOE_REQUIRE(E >= 1 && E <= kMaxE, MOE_EINVAL, "moe_permute: E=%d outside [1, %d]", E, kMaxE);
  MOE_REQUIRE(k >= 1 && k <= E && k <= 32, MOE_EINVAL, "moe_permute: k=%d outside [1, min(E, 32)]", k);
  MOE_REQUIRE((long long)T * k < (1ll << 31), MOE_EINVAL, "moe_permute: T*k overflows int32");
  MOE_REQUIRE(offsets != nullptr, MOE_EINVAL, "moe_permute: offsets is NULL");
  const size_t need = moe_permute_workspace_size(T, k, E);
  MOE_REQUIRE(ws_bytes >= need, MOE_ECAPACITY, "moe_permute: workspace %zu < %zu bytes", ws_bytes, need);
  if (x_out != nullptr) {
    MOE_REQUIRE(x != nullptr && d > 0, MOE_EINVAL, "moe_permute: x_out needs x and d > 0");
    MOE_REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_EUNSUPPORTED, "moe_permute: x_dtype %d unsupported", x_dtype);
    MOE_REQUIRE(out_dtype == x_dtype || out_dtype == MOE_FP8_E4M3 || out_dtype == MOE_MXFP8, MOE_EUNSUPPORTED,
                "moe_permute: conversion %d -> %d unsupported", x_dtype, out_dtype);
    MOE_REQUIRE(aligned(x, 16) && aligned(x_out, 16), MOE_EINVAL, "moe_permute: x and x_out must be 16-byte aligned");
    const int esz = x_dtype == MOE_F32 ? 4 : 2;
    MOE_REQUIRE((d * esz) % 16 == 0, MOE_EINVAL, "moe_permute: row bytes must be a multiple of 16");
    if (out_dtype == MOE_FP8_E4M3) {
      MOE_REQUIRE(d % 128 == 0 && x_out_scale != nullptr, MOE_EINVAL,
                  "moe_permute: e4m3 output needs d %% 128 == 0 and x_out_scale");
    }
    if (out_dtype == MOE_MXFP8) {
      MOE_REQUIRE(d % 32 == 0 && x_out_scale != nullptr, MOE_EINVAL,
                  "moe_permute: MXFP8 output needs d %% 32 == 0 and x_out_scale (the E8M0 bytes)");
    }
  }
  hipStream_t s = as_stream(stream);
  if (T == 0) {
    // offsets stay well defined for an empty batch
    hipLaunchKernelGGL(permute_scan, dim3(1), dim3(1024), 0, s, (const int32_t*)nullptr, (int32_t*)nullptr, offsets,
                       0, E);
    return check_launch("moe_permute scan");
  }
  MOE_REQUIRE(topk_idx && perm_src && perm_dst && ws, MOE_EINVAL, "moe_permute: NULL argument");
  const int nb = (T + 63) / 64;
  int32_t* cnt = static_cast<int32_t*>(ws);
  int32_t* base = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + need / 2);
  auto sort = [&](auto kmax) {
    constexpr int KM = decltype(kmax)::value;
    if (nb == 1) {   // one block of tokens: one launch instead of three
      hipLaunchKernelGGL(permute_small<KM>, dim3(1), dim3(1024), 0, s, topk_idx, offsets, perm_src, perm_dst, T, k, E);
      return;
    }
    hipLaunchKernelGGL(permute_block_counts<KM>, dim3(nb), dim3(64 * kPermWaves), 0, s, topk_idx, cnt, T, k, E);
    hipLaunchKernelGGL(permute_scan, dim3(1), dim3(1024), 0, s, cnt, base, offsets, nb, E);
    hipLaunchKernelGGL(permute_scatter<KM>, dim3(nb), dim3(64 * kPermWaves), 0, s, topk_idx, cnt, base, perm_src,
                       perm_dst, T, k, E);
  };
  if (k <= 2) sort(std::integral_constant<int, 2>{});
  else if (k <= 4) sort(std::integral_constant<int, 4>{});
  else if (k <= 8) sort(std::integral_constant<int, 8>{});
  else sort(std::integral_constant<int, 32>{});
  if (moe_status st = check_launch("moe_permute sort")) return st;
  if (x_out == nullptr) return MOE_OK;
  const int rows = gather ? T * k : T;
  const int32_t* src = gather ? perm_src : nullptr;
  dim3 grid((rows + 3) / 4);
  if (out_dtype == x_dtype) {
    const int esz = x_dtype == MOE_F32 ? 4 : 2;
    hipLaunchKernelGGL(gather_rows_copy, grid, dim3(256), 0, s, static_cast<const uint8_t*>(x),
                       static_cast<uint8_t*>(x_out), src, rows, k, d * esz);
  } else if (out_dtype == MOE_MXFP8) {
    uint8_t* ex = reinterpret_cast<uint8_t*>(x_out_scale);
    if (x_dtype == MOE_BF16)
      hipLaunchKernelGGL(gather_rows_quant_mxfp8<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(x),
                         static_cast<uint8_t*>(x_out), ex, src, rows, k, d);
    else
      hipLaunchKernelGGL(gather_rows_quant_mxfp8<float>, grid, dim3(256), 0, s, static_cast<const float*>(x),
                         static_cast<uint8_t*>(x_out), ex, src, rows, k, d);
  } else if (x_dtype == MOE_BF16) {
    hipLaunchKernelGGL(gather_rows_quant_e4m3<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(x),
                       static_cast<uint8_t*>(x_out), x_out_scale, src, rows, k, d);
  } else {
    hipLaunchKernelGGL(gather_rows_quant_e4m3<float>, grid, dim3(256), 0, s, static_cast<const float*>(x),
                       static_cast<uint8_t*>(x_out), x_out_scale, src, rows, k, d);
  }
  return check_launch("moe_permute gather");
}
