// The fp8 (e4m3 with fp32 block scales) prefill GEMM of the grouped FFN.
#pragma once

#include "ffn_common.h"

namespace moeffn {
namespace {

// ----------------------------------------------------------- fp8 path ---
// e4m3 operands with fp32 block scales (per row per 128 columns for activations, per
// 128x128 block for weights). The scales are arbitrary fp32 values, which the MFMA's
// power-of-two (E8M0) scale operands cannot carry, so every 16x16x128 MFMA covers exactly
// one 128-column scale block and its partial product is promoted on the VALU:
// acc += P * (s_row * s_weight). The accumulators therefore live in VGPRs, which bounds
// a wave's tile: block tile 128 x 256 on 8 waves of 64 x 64 (two per SIMD), one
// 128-column scale block per stage, a 3-deep LDS ring fed by direct-to-LDS loads two
// stages ahead.
// LDS stage: A 128 rows x 128 B (8 blocks of 16 rows, row r's 16-byte chunk c at slot
// 8r + (c ^ f(r)), f(r) = ((r >> 1) + 4 (r & 1)) & 7, so a row is one 128-byte DMA
// segment and fragment reads are bank-conflict-free), B 16 tiles of 2 KiB (the bundle
// layout), the 128 row scales of the stage's block.

constexpr int kF8BM = 128, kF8BN = 256, kF8Stages = 3;
constexpr int kF8MaxKB = 128;   // K up to 16384 (weight scales of a tile are staged in LDS)
constexpr int kF8A = 0, kF8B = 16384, kF8S = 49152, kF8StageBytes = 50176;

struct Fp8Args {
  const uint8_t* a;
  const float* a_scale;        // [*, K/128]
  const int32_t* a_row_src;
  int a_row_div;
  const int32_t* offsets;
  const int32_t* slot_of_expert;
  const int32_t* tile_prefix;
  int32_t* counters;           // [8] per-XCD tile counters (zeroed by ffn_tile_map)
  const char* pool;
  int64_t slot_stride;
  int64_t b_off;
  int64_t s_off0, s_off1;      // GATEUP: gate and up scale grids [F/128][K/128]; DOWN: down grid [d/128][F/128]
  int N, K;
  void* out;                   // GATEUP: Hq [rows, N/2] e4m3; DOWN: y [rows, N]
  float* out_scale;            // GATEUP: Hs [rows, N/256]
  int out_dtype;
  int E;
};

// 4 bytes per lane from global into LDS at lds_base + 4 * lane, as inline assembly (see
// dma16_asm). lds_base must be wave-uniform.
__device__ __forceinline__ void dma4_asm(const void* g, const void* lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory");
}

// One 128 x 256 tile on 8 waves (2 wave rows of 64 x 4 wave columns of 64, two waves per
// SIMD, so one wave's block-scale promotion and LDS reads run while the other's MFMAs do).
// The weight block scales the tile needs (two per 128-column stage) are staged in LDS
// first (s_wscale), so the main loop issues no global loads of its own besides the ring.
template <int MODE>
__device__ __forceinline__ void gemm_fp8_tile(const Fp8Args& p, char (*smem)[kF8StageBytes],
                                              float (*amax_x)[kF8BM], float (*s_wscale)[kF8MaxKB], int e, int row0,
                                              int row_end, int n0) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 2, wn = w & 3;   // wave row (4 m-blocks) x wave column (4 n-blocks)
  const int KB = p.K / 128;
  const char* bundle = p.pool + (int64_t)p.slot_of_expert[e] * p.slot_stride;
  const char* B = bundle + p.b_off;
  // GATEUP: [0] gate and [1] up scales of the tile's 128 hidden rows; DOWN: the scales of
  // the tile's two 128-column blocks (wave column wn uses [wn / 2])
  for (int i = threadIdx.x; i < 2 * KB; i += blockDim.x) {
    const int which = i / KB, s = i - which * KB;
    const float* grid;
    int blk;
    if constexpr (MODE == MODE_GATEUP) {
      grid = reinterpret_cast<const float*>(bundle + (which ? p.s_off1 : p.s_off0));
      blk = n0 / 256;
    } else {
      grid = reinterpret_cast<const float*>(bundle + p.s_off0);
      blk = n0 / 128 + which;
    }
    s_wscale[which][s] = grid[blk * KB + s];
  }
  __syncthreads();
  auto f = [](int r) { return ((r >> 1) + 4 * (r & 1)) & 7; };
  auto src_row = [&](int r) {
    r = r < row_end ? r : row_end - 1;
    return p.a_row_src ? p.a_row_src[r] / p.a_row_div : r;
  };

  // Per stage each wave issues 7 DMA instructions: A rows 16w .. 16w+15 (two of 8 rows;
  // lane j loads chunk (j%8) ^ f(r) of row r = 16w + 8t + j/8), B n-blocks 2w and 2w+1
  // (two 1 KiB halves each) and one of the row-scale quarters (rows 64 (w & 1) + lane into
  // slot w & 3; waves 4-7 repeat 0-3 with the same bytes, so every wave has the same count).
  const uint8_t* aptr[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tr = 16 * w + 8 * t + (lane >> 3);   // row within the 128-row tile
    aptr[t] = p.a + (size_t)src_row(row0 + tr) * p.K + 16 * ((lane & 7) ^ f(tr & 15));
  }
  const float* sptr = p.a_scale + (size_t)src_row(row0 + 64 * (w & 1) + lane) * KB;
  const char* bptr = B + ((int64_t)(n0 / 16 + w * 2) * KB) * 2048 + 16 * lane;

  auto issue = [&](int s) {
    char* base = smem[s % kF8Stages];
#pragma unroll
    for (int t = 0; t < 2; ++t) dma16_asm(aptr[t] + s * 128, base + kF8A + (2 * w + t) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        dma16_asm(bptr + ((int64_t)i * KB + s) * 2048 + h * 1024, base + kF8B + (w * 2 + i) * 2048 + h * 1024);
    dma4_asm(sptr + s, base + kF8S + (w & 3) * 256);
  };
  auto wait_dma = [&](bool more) {
    if (more) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment read offsets: A (row l%16, chunks 2(l/16) and 2(l/16)+1), B (two halves)
  const int ar = lane & 15, ac = 2 * (lane >> 4);
  const int a_off0 = 16 * (8 * ar + ((ac + 0) ^ f(ar)));
  const int a_off1 = 16 * (8 * ar + ((ac + 1) ^ f(ar)));

  const int e8m0_one = 127;   // MFMA block scale 2^0: the fp32 block scales are applied in software
  // A wave row whose 64 rows all lie past the expert's last row (the short last m-tile of an
  // expert whose rows just pass a multiple of 128) only moves data: it issues its share of
  // the DMA and joins the barriers, but reads no fragments and issues no MFMAs; its
  // accumulators stay zero and the epilogue stores no row of it.
  const bool idle = row0 + wm * 64 >= row_end;
  issue(0);
  if (KB > 1) issue(1);
  for (int s = 0; s < KB; ++s) {
    wait_dma(s + 1 < KB);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_no_fence();
    if (s + 2 < KB) issue(s + 2);
    if (idle) continue;
    const char* base = smem[s % kF8Stages];
    i32x8_t fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* blk = base + kF8A + (wm * 4 + i) * 2048;
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(blk + a_off0);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(blk + a_off1);
      fa[i] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // Software-pipelined block-scale promotion. The 16 MFMAs of the stage (n-block jj,
    // m-block i: k = 4 jj + i) write a ring of 6 partial tiles; partial k is promoted
    // (acc += part * row scale * weight scale) after MFMA k + 4 has been issued, so the
    // VALU work of one tile runs while the matrix core computes the next ones, and every
    // partial has had four MFMA issue slots to complete (the hazard recognizer does not
    // see into the inline-asm MFMAs; the drain waits explicitly). GATEUP walks the gate
    // n-blocks (even j) before the up n-blocks (odd j), so one set of combined scales is
    // live at a time.
    const f32x4_t* sa_p = reinterpret_cast<const f32x4_t*>(base + kF8S + 4 * (wm * 64 + 4 * (lane >> 4)));
    f32x4_t sc[4];
    auto make_sc = [&](int which) {
      const float sw = s_wscale[which][s];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = sa_p[4 * i] * sw;
    };
    make_sc(MODE == MODE_GATEUP ? 0 : wn >> 1);
    auto jof = [](int jj) { return MODE == MODE_GATEUP ? ((jj & 1) << 1) | (jj >> 1) : jj; };
    auto load_b = [&](int jj) {
      const char* blk = base + kF8B + (wn * 4 + jof(jj)) * 2048 + 16 * lane;
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(blk);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(blk + 1024);
      return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    i32x8_t fbuf[2];
    fbuf[0] = load_b(0);
    f32x4_t part[6];
#pragma unroll
    for (int k = 0; k < 20; ++k) {
      if (k < 16) {
        const int jj = k >> 2, i = k & 3;
        if (i == 0 && jj + 1 < 4) fbuf[(jj + 1) & 1] = load_b(jj + 1);
        // ("memory" keeps the compiler from sinking the next n-block's LDS reads to their use)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
                     : "=v"(part[k % 6])
                     : "v"(fa[i]), "v"(fbuf[jj & 1]), "v"(e8m0_one)
                     : "memory");
      }
      if (k == 16) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      if (k >= 4) {
        const int kk = k - 4, i = kk & 3, jj = kk >> 2;
        if (MODE == MODE_GATEUP && kk == 8) make_sc(1);   // the up n-blocks start here
        acc[i][jof(jj)] += part[kk % 6] * sc[i];
      }
    }
  }

  const int rbase = row0 + wm * 64 + 4 * (lane >> 4);
  if constexpr (MODE == MODE_GATEUP) {
    // H = silu(G) * U over this tile's 128 hidden columns (32 per wave column), then per-row
    // e4m3 quantisation with one scale per row for the 128 columns (amax over the 4 waves)
    const int F = p.N / 2;
    float h[4][2][4];  // [m-block][pair][row q]
    float am[4][4];    // [m-block][row q]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float m = 0.f;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const float v = silu_f32(acc[i][2 * pp][q]) * acc[i][2 * pp + 1][q];
          h[i][pp][q] = v;
          m = fmaxf(m, fabsf(v));
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        am[i][q] = m;
      }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) amax_x[wn][wm * 64 + i * 16 + 4 * (lane >> 4) + q] = am[i][q];
    }
    __syncthreads();
    uint8_t* Hq = static_cast<uint8_t*>(p.out);
    const int hcol0 = n0 / 2 + wn * 32 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = wm * 64 + i * 16 + 4 * (lane >> 4) + q;
        const int r = row0 + lr;
        const float a = fmaxf(fmaxf(amax_x[0][lr], amax_x[1][lr]), fmaxf(amax_x[2][lr], amax_x[3][lr]));
        const float scale = a > 0.f ? a / 448.0f : 1.0f;
        if (r < row_end) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const float y = fminf(fmaxf(h[i][pp][q] / scale, -448.0f), 448.0f);
            Hq[(size_t)r * F + hcol0 + pp * 16] = static_cast<uint8_t>(f32_to_e4m3_rne(y));
          }
          if (wn == 0 && (lane & 15) == 0) p.out_scale[(size_t)r * (F / 128) + n0 / kF8BN] = scale;
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rbase + i * 16 + q;
          if (r < row_end) {
            if (p.out_dtype == MOE_BF16) static_cast<bf16_t*>(p.out)[(size_t)r * p.N + col] = f32_to_bf16(acc[i][j][q]);
            else static_cast<float*>(p.out)[(size_t)r * p.N + col] = acc[i][j][q];
          }
        }
      }
  }
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void ffn_gemm_fp8(Fp8Args p) {
  __shared__ __attribute__((aligned(1024))) char smem[kF8Stages][kF8StageBytes];
  __shared__ float amax_x[4][kF8BM];
  __shared__ float s_wscale[2][kF8MaxKB];
  __shared__ int s_tile;
  const int NT = p.N / kF8BN;
  const int total = p.tile_prefix[p.E] * NT;
  int range = 0;   // thread 0: XCD ranges this block has used up
  for (;;) {
    if (threadIdx.x == 0) s_tile = take_tile(p.counters, total, range);
    __syncthreads();
    const int L = s_tile;
    if (L < 0) return;
    int e, mt, mte, nt;
    tile_coords(p.tile_prefix, p.E, NT, L, e, mt, mte, nt);
    const int row0 = p.offsets[e] + mt * kF8BM;
    gemm_fp8_tile<MODE>(p, smem, amax_x, s_wscale, e, row0, p.offsets[e + 1], nt * kF8BN);
    // every wave is done with the ring, the scale and amax arrays, and has read s_tile
    __syncthreads();
  }
}

}  // namespace
}  // namespace moeffn
