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
// columns); its 8 waves split K. A long down projection over at most 64 rows (a shared
// expert's) is also split over K across workgroups, whose fp32 partials the last one to
// arrive adds in a fixed order. Weight tiles go straight from global memory into MFMA
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
  int rows;          // the problem's rows (indexing of the split partials)
  int splits;        // DOWN: workgroups sharing one (expert, group)'s K range; 1 otherwise
  float* part;       // DOWN with splits > 1: fp32 partials [splits][rows][N]
  int32_t* arrived;  // DOWN with splits > 1: per (active expert, group) arrival counts
  int32_t* clear;    // GATEUP: the arrival counts of the down launch that follows, cleared here
  int clear_n;
  int32_t* clear2;   // GATEUP: the combine's per-group arrival counts of that launch, cleared here
  int clear2_n;
  int rchunks;       // workgroups per (expert, group), each taking 16 rows (1: one takes all rows)
  int64_t s_off;     // MXFP4: byte offset of the matrix's E8M0 scales inside a bundle
};

// Eight FP4 E2M1 codes (two per byte, element 2j in the low nibble of byte j) times the
// E8M0 scale 2^(e-127) as bf16, exactly (an E2M1 value times a power of two is a bf16 value),
// with the gfx950 scaled conversion (two codes per instruction).
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t codes, uint32_t e) {
  const float scale = e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);   // 2^(e-127)
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The combine folded into a decode down launch: once every (expert, 32-column group) unit of
// both problems has stored its outputs for group g, the last workgroup to finish one adds,
// for every token, the gate-weighted rows of its k experts and the gated shared-expert row
// over those 32 columns, exactly as moe_combine does (fp32, j ascending, shared term last,
// one rounding). The expert outputs are fp32 values (already rounded to the problem's y
// dtype) in the workspace, written and read with device-scope accesses.
struct DecodeCombine {
  int T, k, d;
  const int32_t* perm_dst;   // [T*k] -> row of y_routed
  const float* gate;         // [T*k]
  const float* shared_gate;  // [T] or NULL (= 1 when y_shared is given)
  const float* y_routed;     // [T*k, d]
  const float* y_shared;     // [T, d] or NULL
  void* out;                 // [T, d] out_dtype
  int out_dtype;
  int32_t* arrived;          // [d / 32], zero when the launch starts
  int nprob;                 // problems in the launch (units of both count)
};

// Number of experts that have rows and a slot (the units of one 32-column group); offsets
// NULL is one group (see decode_block).
__device__ __forceinline__ int count_active_experts(const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ slot_of_expert, int E) {
  const int lane = threadIdx.x & 63;
  if (offsets == nullptr) return slot_of_expert[0] >= 0 ? 1 : 0;
  int n = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    n += __popcll(__ballot(e < E && offsets[e + 1] > offsets[e] && slot_of_expert[e] >= 0));
  }
  return n;
}

// The part of the combine a thread can load before its group is complete: the rows and
// gates of the first 8 experts of its (token, 4 columns) item (T <= 64, so one item per
// thread of a 512-thread workgroup) and the shared gate.
struct CombinePre {
  int rr[8];
  float gg[8];
  float sg;
};

__device__ __forceinline__ void decode_combine_preload(const DecodeCombine& cb, CombinePre& pre) {
  const int it = threadIdx.x;
  if (it >= cb.T * 8) return;
  const int t = it >> 3, k = cb.k;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (u < k) {
      pre.rr[u] = cb.perm_dst[(size_t)t * k + u];
      pre.gg[u] = cb.gate[(size_t)t * k + u];
    }
  pre.sg = cb.y_shared ? (cb.shared_gate ? cb.shared_gate[t] : 1.0f) : 0.0f;
}

// Columns 32 g .. 32 g + 31 of out for every token, from the expert outputs (see
// DecodeCombine); one (token, 4 columns) item per thread, the loads of up to 8 expert rows
// issued before the first add.
__device__ __forceinline__ void decode_combine_group(const DecodeCombine& cb, int g, const CombinePre& pre) {
  const int k = cb.k, d = cb.d;
  const int it = threadIdx.x;
  if (it >= cb.T * 8) return;
  const int t = it >> 3, c = 32 * g + 4 * (it & 7);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += 8) {
    int rr[8];
    float gg[8], v[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < k) {
        rr[u] = j0 == 0 ? pre.rr[u] : cb.perm_dst[(size_t)t * k + j0 + u];
        gg[u] = j0 == 0 ? pre.gg[u] : cb.gate[(size_t)t * k + j0 + u];
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < k)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[u][q] = __hip_atomic_load(cb.y_routed + (size_t)rr[u] * d + c + q, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < k)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(gg[u], v[u][q], acc[q]);
  }
  if (cb.y_shared) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      acc[q] = fmaf(pre.sg, __hip_atomic_load(cb.y_shared + (size_t)t * d + c + q, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT), acc[q]);
  }
  if (cb.out_dtype == MOE_BF16) {
    const uint32_t w0 = f32x2_to_bf16x2(acc[0], acc[1]);
    const uint32_t w1 = f32x2_to_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<uint2*>(static_cast<bf16_t*>(cb.out) + (size_t)t * d + c) = make_uint2(w0, w1);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(cb.out) + (size_t)t * d + c) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

// An output value of the down projection: stored as y_dtype, or (folded combine) as the
// fp32 value of that rounding with a device-scope store, so the combining workgroup, on any
// XCD, reads it without a cache-wide write-back.
template <bool COMB>
__device__ __forceinline__ void store_y(const DecodeArgs& p, size_t o, float v) {
  if constexpr (COMB) {
    const float r = p.out_dtype == MOE_BF16 ? bf16_to_f32(f32_to_bf16(v)) : v;
    __hip_atomic_store(static_cast<float*>(p.out) + o, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    if (p.out_dtype == MOE_BF16) static_cast<bf16_t*>(p.out)[o] = f32_to_bf16(v);
    else static_cast<float*>(p.out)[o] = v;
  }
}

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
constexpr int kDecMaxSplits = 8;              // workgroups per (expert, group) of a split down GEMM
#ifndef MOEFFN_DEC_MX_CHUNKS
#define MOEFFN_DEC_MX_CHUNKS 2
#endif
constexpr int kDecMxChunks = MOEFFN_DEC_MX_CHUNKS;   // MXFP4 chunks of 4 k-steps loaded at once
// Waves per SIMD the one-m-block MXFP4 kernels are built for (the second launch bound):
// 6 keeps three workgroups per CU with the chunks above in flight.
#ifndef MOEFFN_DEC_MX_WAVES_PER_SIMD
#define MOEFFN_DEC_MX_WAVES_PER_SIMD 6
#endif
constexpr int kDecMxWavesPerSimd = MOEFFN_DEC_MX_WAVES_PER_SIMD;

// One decode workgroup's LDS.
template <int MB>
struct DecodeLds {
  f32x4_t red[kDecWaves - 1][MB][2][64];   // partials of waves 1..: [wave][m-block][n-tile][lane]
  int s_last;                              // split K: this workgroup arrived last
  int s_glast;                             // COMB: last unit of its column group
};

// Workgroup bid of a decode launch of problem p (p0 and p1 are the launch's problems, which
// the folded combine counts units of). SPLIT launches carry a down projection split over K;
// the others compile without that code.
// MB is the number of 16-row m-blocks a pass covers: 1 for decode batches (a quarter of the
// accumulators and of the reduction LDS of 4, so more workgroups and more loads in flight fit
// on a CU; an expert with more rows takes several passes, a one-expert problem several
// workgroups, see rchunks), 4 for larger ones.
// YF32 (DOWN only) stores the outputs as the fp32 values of their y-dtype rounding with
// device-scope stores, for a combine that reads them in the same launch or the next one;
// COMB (needs YF32) folds that combine into the launch (DecodeCombine). WF is the weight
// format: 0 bf16 tiles, 1 MXFP4 chunks (codes and scales of 4 k-steps per load, decoded to
// bf16 in registers; the waves split K in whole chunks).
template <int MODE, bool SPLIT, int MB, bool YF32, bool COMB, int WF>
__device__ __forceinline__ void decode_block(const DecodeArgs& p, int bid, const DecodeArgs& p0,
                                             const DecodeArgs& p1, const DecodeCombine& cb, DecodeLds<MB>& L) {
  static_assert(!COMB || MODE == MODE_DOWN, "the combine follows the down projection");
  static_assert(!COMB || YF32, "the folded combine reads fp32 outputs");
  static_assert(!YF32 || MODE == MODE_DOWN, "only the down projection has outputs to combine");
  auto& red = L.red;
  if constexpr (MODE == MODE_GATEUP) {
    if (bid == 0 && p.clear != nullptr)
      for (int j = threadIdx.x; j < p.clear_n; j += blockDim.x) p.clear[j] = 0;
    if (bid == 0 && p.clear2 != nullptr)
      for (int j = threadIdx.x; j < p.clear2_n; j += blockDim.x) p.clear2[j] = 0;
  }
  // The block's coordinates are uniform; integer division runs on the vector unit, so they
  // are moved back to scalar registers, which keeps the expert's offsets and slot on scalar loads.
  const int G = p.N / 32;
  const int S = (SPLIT && MODE == MODE_DOWN) ? p.splits : 1;
  const int R = p.rchunks;
  int unit, s = 0, c = 0;   // (active expert, group), K split, 16-row chunk
  if (R > 1) {
    // the R chunks of units 8q .. 8q + 7 are blocks 8Rq .. 8Rq + 8R - 1, chunk c of unit
    // 8q + x at 8Rq + 8c + x: the blocks that read one weight group run on one XCD
    // (block b on XCD b % 8) at about the same time, so the chunks after the first find it in L2
    const int q = bid / (8 * R), rem = bid - q * 8 * R;
    c = rem >> 3;
    unit = q * 8 + (rem & 7);
  } else {
    unit = bid / S;
    s = bid - unit * S;
  }
  unit = __builtin_amdgcn_readfirstlane(unit);
  c = __builtin_amdgcn_readfirstlane(c);
  const int i = __builtin_amdgcn_readfirstlane(unit / G);
  const int g = unit - i * G;
  // offsets == NULL: one group over rows [0, rows) (a shared expert's problem, whose [0, T]
  // offsets the caller need not hold)
  const bool one = p.offsets == nullptr;
  const int e = __builtin_amdgcn_readfirstlane(one ? ((i == 0 && p.slot_of_expert[0] >= 0) ? 0 : -1)
                                                    : nth_active_expert(p.offsets, p.slot_of_expert, p.E, i));
  if (e < 0) return;
  const int row0 = one ? 0 : p.offsets[e];
  const int n_e = one ? p.rows : p.offsets[e + 1] - row0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int KT = p.K / 32;
  const int ks0 = (KT * s) / S, ks = (KT * (s + 1)) / S - ks0;   // this split's k-steps
  int kt0 = ks0 + (ks * w) / kDecWaves, kt1 = ks0 + (ks * (w + 1)) / kDecWaves;
  const char* bundle = p.pool + (int64_t)p.slot_of_expert[e] * p.slot_stride;
  const char* B = bundle + p.b_off;
  const char* b0 = B + ((int64_t)(2 * g) * KT) * 1024 + 16 * lane;      // n-tile 2g
  const char* b1 = B + ((int64_t)(2 * g + 1) * KT) * 1024 + 16 * lane;  // n-tile 2g+1
  const char* sc0 = nullptr;
  const char* sc1 = nullptr;
  if constexpr (WF == 1) {
    // MXFP4 (no K split): chunks of 4 k-steps, 1 KiB of codes and 64 bytes of scales each
    const int KC = KT / 4;
    kt0 = 4 * ((KC * w) / kDecWaves);
    kt1 = 4 * ((KC * (w + 1)) / kDecWaves);
    b0 = B + ((int64_t)(2 * g) * KC) * 1024 + 16 * lane;
    b1 = B + ((int64_t)(2 * g + 1) * KC) * 1024 + 16 * lane;
    const char* Sg = bundle + p.s_off;
    sc0 = Sg + ((int64_t)(2 * g) * KC) * 64 + 4 * (lane & 15);
    sc1 = Sg + ((int64_t)(2 * g + 1) * KC) * 64 + 4 * (lane & 15);
  }

  const int mc_end = R > 1 ? min(n_e, 16 * c + 16) : n_e;
  for (int mc = 16 * c; mc < mc_end; mc += 16 * MB) {
    const int mbn = min(MB, (n_e - mc + 15) / 16);
    const bf16_t* arow[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      int r = mc + m * 16 + (lane & 15);
      r = r < n_e ? r : n_e - 1;
      const int src = p.a_row_src ? p.a_row_src[row0 + r] / p.a_row_div : row0 + r;
      arow[m] = p.a + (size_t)src * p.K + 8 * (lane >> 4);
    }
    f32x4_t acc[MB][2];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m][0] = acc[m][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (WF == 1) {
      // MXFP4: a chunk of 4 k-steps is 16 bytes of codes and 4 of scales per lane and n-tile,
      // a third of a bf16 chunk's bytes, so up to kDecMxChunks chunks are loaded at once (one
      // round trip for the wave's K range at these sizes) and each k-step is decoded to bf16
      // fragments just before its MFMAs
      constexpr int NC = MB == 1 ? kDecMxChunks : 1;   // (a four-m-block pass has no registers to spare)
      for (int k0 = kt0; k0 < kt1; k0 += 4 * NC) {
        uint4 w0[NC], w1[NC];
        uint32_t e0[NC], e1[NC];
#pragma unroll
        for (int u = 0; u < NC; ++u) {
          if (k0 + 4 * u < kt1) {
            const int64_t ch = k0 / 4 + u;
            w0[u] = *reinterpret_cast<const uint4*>(b0 + ch * 1024);
            w1[u] = *reinterpret_cast<const uint4*>(b1 + ch * 1024);
            e0[u] = *reinterpret_cast<const uint32_t*>(sc0 + ch * 64);
            e1[u] = *reinterpret_cast<const uint32_t*>(sc1 + ch * 64);
          }
        }
#pragma unroll
        for (int u = 0; u < NC; ++u) {
          if (k0 + 4 * u < kt1) {
            const uint32_t c0w[4] = {w0[u].x, w0[u].y, w0[u].z, w0[u].w};
            const uint32_t c1w[4] = {w1[u].x, w1[u].y, w1[u].z, w1[u].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const bf16x8_t f0 = fp4x8_to_bf16(c0w[c], (e0[u] >> (8 * c)) & 255u);
              const bf16x8_t f1 = fp4x8_to_bf16(c1w[c], (e1[u] >> (8 * c)) & 255u);
#pragma unroll
              for (int m = 0; m < MB; ++m) {
                if (m < mbn) {
                  const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(arow[m] + (int64_t)(k0 + 4 * u + c) * 32);
                  acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f0, acc[m][0], 0, 0, 0);
                  acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f1, acc[m][1], 0, 0, 0);
                }
              }
            }
          }
        }
      }
    }
    for (int k0 = kt0; WF == 0 && k0 < kt1; k0 += kDecChunk) {
      const int nk = min(kDecChunk, kt1 - k0);
      // the chunk's tiles as constant offsets from one pointer per n-tile, so the loads issue
      // back to back with immediate offsets
      bf16x8_t fb[kDecChunk][2];
      {
        const char* q0 = b0 + (int64_t)k0 * 1024;
        const char* q1 = b1 + (int64_t)k0 * 1024;
#pragma unroll
        for (int c = 0; c < kDecChunk; ++c) {
          if (c < nk) {
            fb[c][0] = *reinterpret_cast<const bf16x8_t*>(q0 + c * 1024);
            fb[c][1] = *reinterpret_cast<const bf16x8_t*>(q1 + c * 1024);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < mbn) {
          const bf16_t* qa = arow[m] + (int64_t)k0 * 32;
#pragma unroll
          for (int c = 0; c < kDecChunk; ++c) {
            if (c < nk) {
              const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(qa + c * 32);
              acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[c][0], acc[m][0], 0, 0, 0);
              acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[c][1], acc[m][1], 0, 0, 0);
            }
          }
        }
      }
    }
    if (w > 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
        if (m < mbn) {
          red[w - 1][m][0][lane] = acc[m][0];
          red[w - 1][m][1][lane] = acc[m][1];
        }
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
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
          } else if (S == 1) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
              store_y<YF32>(p, (size_t)(row0 + r) * p.N + (2 * g + j) * 16 + (lane & 15), acc[m][j][q]);
          } else if constexpr (SPLIT) {
            // device-scope stores (written through to the coherent level, not left in this
            // XCD's L2), so no cache-wide write-back is needed to publish them
#pragma unroll
            for (int j = 0; j < 2; ++j)
              __hip_atomic_store(&p.part[((size_t)s * p.rows + row0 + r) * p.N + (2 * g + j) * 16 + (lane & 15)],
                                 acc[m][j][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    if (SPLIT && MODE == MODE_DOWN && S > 1) {
      // K split over S workgroups (at most 4 rows, so one pass of mc): the last to arrive
      // adds the S partials in split order, so the sum does not depend on arrival order.
      // The partial's stores have completed (stores count in vmcnt) before this split is
      // counted. A full release fence would also write back the whole L2 of this XCD, and the
      // matching acquire would invalidate it, evicting the rows the other groups re-read.
      if (w == 0) {
        wait_vmcnt<0>();
        int last = 0;
        if (lane == 0) last = atomicAdd(&p.arrived[unit], 1) == S - 1;
        if (lane == 0) L.s_last = last;
      }
      __syncthreads();
      if (L.s_last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // no load moves above the count
        // the group's n_e x 32 outputs over the whole workgroup (one pass), the S loads
        // issued before the first add; device-scope loads never
        // see a stale line of this XCD's L2
#pragma unroll 1
        for (int x = threadIdx.x; x < n_e * 32; x += 64 * kDecWaves) {
          const size_t o = (size_t)(row0 + (x >> 5)) * p.N + 32 * g + (x & 31);
          float v[kDecMaxSplits];
#pragma unroll
          for (int t = 0; t < kDecMaxSplits; ++t)
            if (t < S)
              v[t] = __hip_atomic_load(&p.part[(size_t)t * p.rows * p.N + o], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
          float acc_v = v[0];
#pragma unroll
          for (int t = 1; t < kDecMaxSplits; ++t)
            if (t < S) acc_v += v[t];
          store_y<YF32>(p, o, acc_v);
        }
      }
    }
    __syncthreads();
  }
  if constexpr (COMB) {
    // This workgroup finished a unit (expert e, group g) when it ran the whole K range or
    // was the last of its K splits. Its stores have completed before the unit is counted;
    // the workgroup that counts the group's last unit combines the group's columns.
    bool done = true;
    if constexpr (SPLIT) done = S == 1 || L.s_last;
    if (done) {
      CombinePre pre;
      decode_combine_preload(cb, pre);   // overlaps the wait for this workgroup's stores
      wait_vmcnt<0>();
      __syncthreads();
      if (w == 0) {
        const int units = count_active_experts(p0.offsets, p0.slot_of_expert, p0.E) * p0.rchunks +
                          (cb.nprob > 1 ? count_active_experts(p1.offsets, p1.slot_of_expert, p1.E) * p1.rchunks : 0);
        if (lane == 0) L.s_glast = atomicAdd(&cb.arrived[g], 1) == units - 1;
      }
      __syncthreads();
      if (L.s_glast) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // no load moves above the count
        decode_combine_group(cb, g, pre);
      }
    }
  }
}

// Blocks [0, nb0) work on problem p0, the rest on p1 (two independent grouped FFNs, e.g.
// the routed experts and the shared expert, in one launch), both in projection MODE.
template <int MODE, bool SPLIT, int MB, bool COMB = false, int WF = 0>
__global__ __launch_bounds__(64 * kDecWaves, WF == 1 && MB == 1 ? kDecMxWavesPerSimd : MOEFFN_DEC_MINBLOCKS) void ffn_decode_bf16(
    DecodeArgs p0, DecodeArgs p1, int nb0, DecodeCombine cb) {
  __shared__ DecodeLds<MB> L;
  const bool second = (int)blockIdx.x >= nb0;
  decode_block<MODE, SPLIT, MB, COMB, COMB, WF>(second ? p1 : p0, second ? (int)blockIdx.x - nb0 : (int)blockIdx.x,
                                                p0, p1, cb, L);
}

// Two problems in different projections in one launch: blocks [0, nb0) run the down
// projection of dn (split over K when SPLIT; fp32 outputs for a later folded combine when
// YF32), the rest the gate/up projection of gu. Both one m-block per pass.
template <bool SPLIT, bool YF32, int WF>
__global__ __launch_bounds__(64 * kDecWaves, WF == 1 ? kDecMxWavesPerSimd : MOEFFN_DEC_MINBLOCKS) void ffn_decode_down_gateup(DecodeArgs dn,
                                                                                             DecodeArgs gu,
                                                                                             int nb0) {
  __shared__ DecodeLds<1> L;
  const DecodeCombine no_cb{};
  if ((int)blockIdx.x < nb0)
    decode_block<MODE_DOWN, SPLIT, 1, YF32, false, WF>(dn, (int)blockIdx.x, dn, dn, no_cb, L);
  else
    decode_block<MODE_GATEUP, false, 1, false, false, WF>(gu, (int)blockIdx.x - nb0, gu, gu, no_cb, L);
}

}  // namespace
}  // namespace moeffn
