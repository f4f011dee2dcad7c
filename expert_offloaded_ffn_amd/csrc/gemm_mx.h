// The MXFP4 prefill GEMM of the grouped FFN: FP4 E2M1 expert weights with one E8M0 scale per
// 32 inputs (the bundle's MXFP4 matrices) against MXFP8 activations (E4M3 elements with one
// E8M0 scale per 32) on CDNA4's block-scaled MFMA, v_mfma_scale_f32_16x16x128_f8f6f4 with an
// E4M3 A operand and an E2M1 B operand. The hardware applies both scales per 32-element block,
// so a tile accumulates straight through K in fp32 with no promotion on the VALU.
//
// Operand layouts of the instruction (checked on the chip): an E2M1 operand holds in lane l the
// 32 consecutive K values 32 (l / 16) .. + 31 of row l % 16, two per byte, low nibble first; an
// E4M3 operand holds K 16 (l / 16) .. + 15 in its first 16 bytes and 64 + 16 (l / 16) .. + 15
// in the next 16; lane l's scale byte is that of row l % 16 and the 32-value block l / 16.
//
// The bundle's MXFP4 chunk (16 rows x 128 inputs, 1 KiB) keeps, for the decode kernels, lane
// l's 16 bytes as four 4-byte pieces of 8 values at K = 32 c + 8 (l / 16): the B fragment of
// lane l is the piece l / 16 of lanes (l % 16) + 16 p, p = 0..3, so four 4-byte LDS reads
// (bank-conflict free) assemble it without changing the bundle.
//
// Tile, waves and tile order as in the fp8 GEMM (256 x 256 on 8 waves of 128 x 64; gate waves
// hand G to the up waves of the same hidden columns in the epilogue); a 3-stage LDS ring of
// 50 KiB stages. Gate/up writes H as MXFP8 (codes [rows, F], exponents [rows, F/32]).
#pragma once

#include "gemm_fp8.h"

namespace moeffn {
namespace {

// LDS ring stage (128 inputs): A codes 256 rows x 128 B (row r's 16-byte chunk c at 128 r +
// 16 (c ^ f(r))), A exponents 256 rows x 4 B, B codes 16 n-blocks x 1 KiB (the bundle's
// chunks), B exponents 16 n-blocks x 64 B (the bundle's, byte 4 r + c: row r, block c).
constexpr int kXA = 0, kXAS = 32768, kXB = 33792, kXBS = 50176, kXStage = 51200, kXStages = 3;

struct MxProb {
  const uint8_t* a;            // E4M3 codes, rows of K bytes
  const uint8_t* a_exp;        // E8M0 exponents, rows of K/32 bytes (same row indexing as a)
  const int32_t* a_row_src;    // NULL: GEMM row r reads row r of a
  int a_row_div;
  const int32_t* offsets;      // [E+1]
  const int32_t* slot_of_expert;
  const char* pool;
  int64_t slot_stride;
  int64_t b_off, bs_off;       // codes and exponents of B ([N, K]) in a bundle
  int E, N, K;
  void* out;                   // GATEUP: H codes [rows, N/2]; DOWN: y [rows, N] (bf16 or f32)
  uint8_t* out_exp;            // GATEUP: H exponents [rows, N/64]
  int out_dtype;
};

struct MxArgs {
  MxProb p[2];
  int E0, n_exp;
  const int32_t* tile_prefix;
  int32_t* counters;
};

// E8M0 shared exponent of an MX block of E4M3 values with largest magnitude a (>= 0): X =
// floor(log2 a) - 8, clamped to [-127, 127], -127 for a == 0; returns the E8M0 byte X + 127.
__device__ __forceinline__ int mx_exp_e4m3(float a) {
  const int X = a > 0.f ? ilogbf(a) - 8 : -127;
  return min(max(X, -127), 127) + 127;
}

template <int MODE>
__device__ __forceinline__ void mx_tile(const MxProb& p, char* ring, int e, int row0, int row_end, int n0) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int KC = p.K / 128, KE = p.K / 32;
  const int valid = min(kQBM, row_end - row0);
  const char* bundle = uniform_ptr(p.pool + (int64_t)p.slot_of_expert[e] * p.slot_stride);

  // DMA per stage: wave w loads A rows 32w..32w+31 (4 x 8 rows, as the fp8 GEMM), B n-blocks
  // 2w, 2w+1 (1 KiB each); waves 0-3 the A exponents of rows 64w..64w+63 (4 bytes each), waves
  // 4-7 the B exponents of n-blocks 4(w-4)..4(w-4)+3 (64 bytes each).
  uint32_t a_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = 32 * w + 8 * t + (lane >> 3);
    const int rr = min(r, valid - 1);
    const int src = p.a_row_src ? p.a_row_src[row0 + rr] / p.a_row_div : row0 + rr;
    a_off[t] = (uint32_t)src * (uint32_t)p.K + 16u * (uint32_t)((lane & 7) ^ fp8_swz(r & 15));
  }
  uint32_t x_off;   // this wave's exponent load (A rows for w < 4, B n-blocks for w >= 4)
  if (w < 4) {
    const int rr = min(64 * w + lane, valid - 1);
    const int src = p.a_row_src ? p.a_row_src[row0 + rr] / p.a_row_div : row0 + rr;
    x_off = (uint32_t)src * (uint32_t)KE;
  } else {
    const int nb = n0 / 16 + 4 * (w - 4) + (lane >> 4);
    x_off = (uint32_t)(nb * KC) * 64u + 4u * (lane & 15);
  }
  const uint32_t b_off = (uint32_t)((n0 / 16 + 2 * w) * KC) * 1024u + 16u * lane;
  const uint32_t b_step = (uint32_t)KC * 1024u;
  const char* a_base = uniform_ptr(reinterpret_cast<const char*>(p.a));
  const char* ae_base = uniform_ptr(reinterpret_cast<const char*>(p.a_exp));
  const char* b_base = uniform_ptr(bundle + p.b_off);
  const char* be_base = uniform_ptr(bundle + p.bs_off);
  const int a_rows_w = valid - 32 * w;
  auto issue = [&](int s) {
    char* buf = ring + (s % kXStages) * kXStage;
    const char* ab = a_base + (size_t)s * 128;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (8 * t < a_rows_w) dma16_sb(ab, a_off[t], buf + kXA + (4 * w + t) * 1024);
    const char* bb = b_base + (size_t)s * 1024;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_sb(bb, b_off + i * b_step, buf + kXB + (2 * w + i) * 1024);
    if (w < 4) dma4_sb(ae_base + (size_t)s * 4, x_off, buf + kXAS + 256 * w);
    else dma4_sb(be_base + (size_t)s * 64, x_off, buf + kXBS + 256 * (w - 4));
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A fragment of m-block i: row 16 i + l % 16 of the wave row, chunks g and 4 + g (g = l / 16)
  const int g4 = lane >> 4, fr = fp8_swz(lane & 15);
  const int a_frag0 = kXA + 128 * (128 * wm + (lane & 15)) + 16 * (g4 ^ fr);
  const int a_frag1 = kXA + 128 * (128 * wm + (lane & 15)) + 16 * ((4 + g4) ^ fr);
  const int a_xfrag = kXAS + 4 * (128 * wm + (lane & 15)) + g4;
  auto nblk = [&](int j) { return MODE == MODE_GATEUP ? (wn >> 1) * 8 + 2 * j + (wn & 1) : wn * 4 + j; };
  const int nmb = min(8, (valid - 128 * wm + 15) >> 4);

  // loads this wave issues per stage: its A instructions (rows past the tile's last row are
  // not loaded), two B code loads and one exponent load
  const int n_ld = min(4, max(0, (a_rows_w + 7) >> 3)) + 3;
  // The k loop for NMB computed m-blocks per wave (the wave's m-blocks with rows, rounded up to
  // an even count; the extra one of an odd count computes on rows past the tile's last and is
  // never stored).
  auto kloop = [&](auto nmb_c) {
    constexpr int NMB = decltype(nmb_c)::value;
    issue(0);
    if (KC > 1) issue(1);
    for (int s = 0; s < KC; ++s) {
      // stage s has landed for every wave (each wave waits until only its loads of stage
      // s + 1 are outstanding), and every wave is done with stage s - 1's buffer, which the
      // loads of stage s + 2 issued below overwrite
      if (s + 1 < KC) {
        switch (n_ld) {
          case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
          case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
          case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
          case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
          default: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        }
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_no_fence();
      if (s + 2 < KC) issue(s + 2);
      if constexpr (NMB > 0) {
        const char* buf = ring + (s % kXStages) * kXStage;
        i32x8_t fb[4];
        int sb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const char* blk = buf + kXB + nblk(j) * 1024 + 4 * g4;
          const int* q = reinterpret_cast<const int*>(blk + 16 * (lane & 15));
          fb[j] = i32x8_t{q[0], q[64], q[128], q[192], 0, 0, 0, 0};   // pieces of lanes (l%16) + 16 p
          sb[j] = *reinterpret_cast<const uint8_t*>(buf + kXBS + nblk(j) * 64 + 4 * (lane & 15) + g4);
        }
        auto frag_a = [&](int i) {
          const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(buf + a_frag0 + 2048 * i);
          const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(buf + a_frag1 + 2048 * i);
          return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        auto scale_a = [&](int i) { return (int)*reinterpret_cast<const uint8_t*>(buf + a_xfrag + 64 * i); };
        // Software pipeline over the m-blocks: m-block i + 1's fragment and scale are read
        // from LDS before m-block i's four MFMAs issue, so the reads overlap the matrix core;
        // scheduling-group barriers pin that order.
        i32x8_t fa = frag_a(0);
        int sa = scale_a(0);
#pragma unroll
        for (int i = 0; i < NMB; ++i) {
          i32x8_t fa_n;
          int sa_n = 0;
          if (i < NMB - 1) {
            fa_n = frag_a(i + 1);
            sa_n = scale_a(i + 1);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)   // formats: A E4M3 (0), B E2M1 (4)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[j], acc[i][j], 0, 4, 0, sa, 0, sb[j]);
          if (i < NMB - 1) {
            fa = fa_n;
            sa = sa_n;
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // the next m-block's LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // this m-block's MFMAs
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // nmb is uniform (from the tile's row range and the wave row), so this is a scalar branch
  const int nmb_even = nmb <= 0 ? 0 : (nmb + 1) & ~1;
  if (nmb_even == 0) kloop(std::integral_constant<int, 0>{});
  else if (nmb_even == 2) kloop(std::integral_constant<int, 2>{});
  else if (nmb_even == 4) kloop(std::integral_constant<int, 4>{});
  else if (nmb_even == 6) kloop(std::integral_constant<int, 6>{});
  else kloop(std::integral_constant<int, 8>{});
  __syncthreads();   // every wave is done with the ring (its space is reused below)

  if constexpr (MODE == MODE_GATEUP) {
    // The gate wave (wn even) and the up wave (wn odd) of a hidden half hold G and U of the
    // same 128 x 64 block. The up wave finishes m-blocks [0, h), the gate wave [h, nmb): each
    // hands the other its values of the other's m-blocks through the pair's 32 KiB of LDS
    // ([i][j][lane] f32x4: G of m-blocks < h, U of the rest), so all eight waves share the
    // epilogue.
    const int h = (nmb + 1) >> 1;
    const bool up = (wn & 1) != 0;
    f32x4_t* X = reinterpret_cast<f32x4_t*>(ring + (wm * 2 + (wn >> 1)) * 32768);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (up ? (i >= h && i < nmb) : (i < h)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) X[(i * 4 + j) * 64 + lane] = acc[i][j];
      }
    }
    __syncthreads();
    // H = silu(G) * U; its MX blocks of 32 hidden columns are the n-block pairs (0, 1) and
    // (2, 3) of this wave, so a row's block maximum is a 16-lane reduction. The codes are
    // staged ([rows from m-block i0][64 B]) over the part of the pair region this wave reads
    // (from m-block i0 on, 4 KiB each), which the other wave does not touch: m-block i's codes
    // end below m-block i + 1's values, and a wave's LDS accesses complete in order.
    const int i0 = up ? 0 : h, i1 = up ? h : nmb;
    uint8_t* codes = reinterpret_cast<uint8_t*>(ring + (wm * 2 + (wn >> 1)) * 32768 + i0 * 4096);
    const int F = p.N / 2;
    const int hcol0 = n0 / 2 + 64 * (wn >> 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i >= i0 && i < i1) {
        float hv[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t o = X[(i * 4 + j) * 64 + lane];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = up ? o[q] : acc[i][j][q];
            const float u = up ? acc[i][j][q] : o[q];
            hv[j][q] = silu_fast(g) * u;
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lr = 16 * (i - i0) + 4 * (lane >> 4) + q;   // row among this wave's
          const int tr = 128 * wm + 16 * i + 4 * (lane >> 4) + q;   // row within the tile
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float m = fmaxf(fabsf(hv[2 * b][q]), fabsf(hv[2 * b + 1][q]));
            m = max_row16(m);
            const int ex = mx_exp_e4m3(m);
            const float inv = ldexpf(1.0f, 127 - ex);   // 2^-X, exact
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const float y = fminf(fmaxf(hv[2 * b + jj][q] * inv, -448.0f), 448.0f);
              codes[lr * 64 + 16 * (2 * b + jj) + (lane & 15)] = static_cast<uint8_t>(f32_to_e4m3_rne(y));
            }
            if ((lane & 15) == 0 && tr < valid)
              p.out_exp[(size_t)(row0 + tr) * (F / 32) + hcol0 / 32 + b] = static_cast<uint8_t>(ex);
          }
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own writes, read back below
    uint8_t* Hq = static_cast<uint8_t*>(p.out);
    const int nrows = 16 * (i1 - i0);   // at most 64
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * 64 + lane;   // 256 chunks of 16 B: row idx/4, chunk idx%4
      const int lr = idx >> 2, ch = idx & 3;
      const int tr = 128 * wm + 16 * i0 + lr;
      if (lr < nrows && tr < valid) {
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(codes + lr * 64 + 16 * ch);
        *reinterpret_cast<i32x4_t*>(Hq + (size_t)(row0 + tr) * F + hcol0 + 16 * ch) = v;
      }
    }
  } else if (p.out_dtype == MOE_BF16) {
    bf16_t* yl = reinterpret_cast<bf16_t*>(ring + w * 16384);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nmb) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            yl[(16 * i + 4 * (lane >> 4) + q) * 64 + 16 * j + (lane & 15)] = f32_to_bf16(acc[i][j][q]);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bf16_t* Y = static_cast<bf16_t*>(p.out);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int idx = it * 64 + lane;
      const int lr = idx >> 3, ch = idx & 7;
      const int tr = 128 * wm + lr;
      if (tr < valid) {
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(yl + lr * 64 + 8 * ch);
        *reinterpret_cast<i32x4_t*>(Y + (size_t)(row0 + tr) * p.N + n0 + 64 * wn + 8 * ch) = v;
      }
    }
  } else {
    float* Y = static_cast<float*>(p.out);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nmb) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int tr = 128 * wm + 16 * i + 4 * (lane >> 4) + q;
            if (tr < valid) Y[(size_t)(row0 + tr) * p.N + n0 + 64 * wn + 16 * j + (lane & 15)] = acc[i][j][q];
          }
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void ffn_gemm_mx(MxArgs a) {
  __shared__ __attribute__((aligned(1024))) char ring[kXStages * kXStage];
  __shared__ int s_tile;
  const int NT0 = a.p[0].N / kQBN, NT1 = a.p[1].N / kQBN;
  const int total = a.tile_prefix[a.n_exp];
  int range = 0;
  for (;;) {
    if (threadIdx.x == 0) s_tile = take_tile(a.counters, total, range);
    __syncthreads();
    const int L = __builtin_amdgcn_readfirstlane(s_tile);
    if (L < 0) return;
    int g, mt, nt;
    grouped_tile_coords(a.tile_prefix, a.n_exp, a.E0, NT0, NT1, L, g, mt, nt);
    const bool second = g >= a.E0;
    const MxProb& p = second ? a.p[1] : a.p[0];
    const int e = __builtin_amdgcn_readfirstlane(second ? g - a.E0 : g);
    const int row0 = __builtin_amdgcn_readfirstlane(p.offsets[e] + mt * kQBM);
    const int row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
    mx_tile<MODE>(p, ring, e, row0, row_end, __builtin_amdgcn_readfirstlane(nt * kQBN));
    __syncthreads();
  }
}

}  // namespace
}  // namespace moeffn
