// The bf16 decode kernels of the grouped FFN: weight streaming for batches with at most
// 64 rows per expert.
#pragma once

#include "ffn_common.h"

namespace moeffn {
namespace {

// -------------------------------------------------------- decode path ---
// Few rows per expert (decode batches): the layer is bound by streaming each active
// expert's weights once from HBM. A workgroup owns one active expert and one group of
// 32 weight rows (GATEUP: 16 gate + 16 up rows -> 16 hidden columns; DOWN: 32 output
// columns); its 8 waves split K. Weight tiles go straight from global memory into MFMA
// B fragments (the bundle's 1 KiB tile layout is the fragment layout, so every wave load
// is 1 KiB contiguous); A rows (at most 64 per pass, in m-blocks of 16) come from L2.
// The split-K partials are summed through LDS in wave order (deterministic).

// The i-th expert (ascending id) that has rows and a slot, or -1 when there are not that
// many: one ballot per 64 experts; the result is uniform across the wavefront, and every
// wavefront of a block computes the same answer.
__device__ __forceinline__ int nth_active_expert(const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ slot_of_expert, int E, int i) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int seen = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const bool on = e < E && offsets[e + 1] > offsets[e] && slot_of_expert[e] >= 0;
    const uint64_t m = __ballot(on);
    const int c = __popcll(m);
    if (i < seen + c) {
      const uint64_t hit = __ballot(on && __popcll(m & below) == i - seen);
      return e0 + __ffsll((unsigned long long)hit) - 1;
    }
    seen += c;
  }
  return -1;
}

struct DecodeArgs {
  const bf16_t* a;
  const int32_t* a_row_src;
  int a_row_div;
  const int32_t* offsets;
  const int32_t* slot_of_expert;
  int E;
  const char* pool;
  int64_t slot_stride;
  int64_t b_off;
  int N, K;
  void* out;
  int out_dtype;
};

#ifndef MOEFFN_DEC_CHUNK
#define MOEFFN_DEC_CHUNK 4
#endif
#ifndef MOEFFN_DEC_WAVES
#define MOEFFN_DEC_WAVES 8
#endif
#ifndef MOEFFN_DEC_MINBLOCKS
#define MOEFFN_DEC_MINBLOCKS 1
#endif
constexpr int kDecChunk = MOEFFN_DEC_CHUNK;   // k-tiles whose loads are issued together
constexpr int kDecWaves = MOEFFN_DEC_WAVES;   // waves per workgroup (split-K)

// Blocks [0, nb0) work on problem p0, the rest on p1 (two independent grouped FFNs, e.g.
// the routed experts and the shared expert, in one launch).
template <int MODE>
__global__ __launch_bounds__(64 * kDecWaves, MOEFFN_DEC_MINBLOCKS) void ffn_decode_bf16(DecodeArgs p0, DecodeArgs p1,
                                                                                       int nb0) {
  __shared__ f32x4_t red[kDecWaves - 1][4][2][64];   // partials of waves 1..: [wave][m-block][n-tile][lane]
  const bool second = (int)blockIdx.x >= nb0;
  const DecodeArgs p = second ? p1 : p0;
  const int bid = second ? (int)blockIdx.x - nb0 : (int)blockIdx.x;
  const int G = p.N / 32;
  const int i = bid / G, g = bid % G;
  const int e = nth_active_expert(p.offsets, p.slot_of_expert, p.E, i);
  if (e < 0) return;
  const int row0 = p.offsets[e];
  const int n_e = p.offsets[e + 1] - row0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int KT = p.K / 32;
  const int kt0 = (KT * w) / kDecWaves, kt1 = (KT * (w + 1)) / kDecWaves;
  const char* B = p.pool + (int64_t)p.slot_of_expert[e] * p.slot_stride + p.b_off;
  const char* b0 = B + ((int64_t)(2 * g) * KT) * 1024 + 16 * lane;      // n-tile 2g
  const char* b1 = B + ((int64_t)(2 * g + 1) * KT) * 1024 + 16 * lane;  // n-tile 2g+1

  for (int mc = 0; mc < n_e; mc += 64) {
    const int mbn = min(4, (n_e - mc + 15) / 16);
    const bf16_t* arow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      int r = mc + m * 16 + (lane & 15);
      r = r < n_e ? r : n_e - 1;
      const int src = p.a_row_src ? p.a_row_src[row0 + r] / p.a_row_div : row0 + r;
      arow[m] = p.a + (size_t)src * p.K + 8 * (lane >> 4);
    }
    f32x4_t acc[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m][0] = acc[m][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kt0; k0 < kt1; k0 += kDecChunk) {
      const int nk = min(kDecChunk, kt1 - k0);
      bf16x8_t fb[kDecChunk][2];
#pragma unroll
      for (int c = 0; c < kDecChunk; ++c) {
        if (c < nk) {
          fb[c][0] = *reinterpret_cast<const bf16x8_t*>(b0 + (int64_t)(k0 + c) * 1024);
          fb[c][1] = *reinterpret_cast<const bf16x8_t*>(b1 + (int64_t)(k0 + c) * 1024);
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < mbn) {
#pragma unroll
          for (int c = 0; c < kDecChunk; ++c) {
            if (c < nk) {
              const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(arow[m] + (k0 + c) * 32);
              acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[c][0], acc[m][0], 0, 0, 0);
              acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[c][1], acc[m][1], 0, 0, 0);
            }
          }
        }
      }
    }
    if (w > 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (m < mbn) {
          red[w - 1][m][0][lane] = acc[m][0];
          red[w - 1][m][1][lane] = acc[m][1];
        }
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m >= mbn) continue;
        for (int ww = 0; ww < kDecWaves - 1; ++ww) {
          acc[m][0] += red[ww][m][0][lane];
          acc[m][1] += red[ww][m][1][lane];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = mc + m * 16 + 4 * (lane >> 4) + q;
          if (r >= n_e) continue;
          if constexpr (MODE == MODE_GATEUP) {
            const int F = p.N / 2;
            static_cast<bf16_t*>(p.out)[(size_t)(row0 + r) * F + g * 16 + (lane & 15)] =
                f32_to_bf16(silu_fast(acc[m][0][q]) * acc[m][1][q]);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const size_t o = (size_t)(row0 + r) * p.N + (2 * g + j) * 16 + (lane & 15);
              if (p.out_dtype == MOE_BF16) static_cast<bf16_t*>(p.out)[o] = f32_to_bf16(acc[m][j][q]);
              else static_cast<float*>(p.out)[o] = acc[m][j][q];
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace moeffn
