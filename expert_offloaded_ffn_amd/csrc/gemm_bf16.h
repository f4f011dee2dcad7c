// The bf16 prefill GEMM of the grouped FFN (gate/up + SwiGLU, and down).
//
// ffn_gemm_bf16 is a persistent tile engine on MFMA 16x16x32 bf16: 256 x 256 block tiles
// (an expert's last m-tile up to 320 rows), 8 waves of 128 x 64, two per SIMD in two
// groups that take turns, so one wave's LDS reads hide under the other's MFMAs. A and B
// move from global memory straight into LDS (global_load_lds_dwordx4, no staging
// registers) in the 1 KiB fragment-tile layout, so every wave load and every fragment read
// is 1 KiB contiguous. A 4-deep ring of 32-column stages keeps loads three stages ahead, with
// one barrier per stage. Tiles are taken from per-XCD queues, so the m-tiles that share a
// weight tile run on one XCD's L2. Mode GATEUP writes H = silu(G) * U (bf16), mode DOWN
// writes Y.
#pragma once

#include "ffn_common.h"

namespace moeffn {
namespace {

#ifndef MOEFFN_GEMM_STAGES
#define MOEFFN_GEMM_STAGES 4
#endif
// An expert's last m-tile holds up to kBM + kTallRows rows, so a group of n rows takes
// ceil((n - kTallRows) / kBM) tiles instead of ceil(n / kBM): a few rows past a multiple
// of kBM ride along in the last tile rather than costing a whole pass over the weights.
#ifndef MOEFFN_TALL_ROWS
#define MOEFFN_TALL_ROWS 64
#endif
constexpr int kTallRows = MOEFFN_TALL_ROWS;
#ifndef MOEFFN_ACC
#define MOEFFN_ACC(x) "+v"(x)
#endif
constexpr int kGemmWaves = 8;                 // 2 wave rows x 4 wave columns of 64
constexpr int kStages = MOEFFN_GEMM_STAGES;   // LDS ring depth (BK = 32 per stage)
constexpr int kStageA = (kBM + kTallRows) * 64;   // A: up to 320 rows x 32 bf16
constexpr int kStageBytes = kStageA + kBN * 64;   // + B: 256 rows x 32 bf16 (36 KiB)

// One 256-column tile of B against a (256 or, on an expert's last m-tile, up to 320)-row
// tile of A. TALL selects 10 instead of 8 m-blocks of 16 rows per wave.
template <int MODE, bool TALL, typename Claim>
__device__ __forceinline__ void gemm_bf16_tile(const GemmArgs& p, char (*smem)[kStageBytes], int e, int row0,
                                               int row_end, int n0, Claim&& claim) {
  constexpr int MB = TALL ? 10 : 8;   // m-blocks per wave
  // the wave index is uniform across the wave: keep it (and what derives from it) scalar
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KS = p.K / 32;  // stages of 32 columns
  const char* B = p.pool + (int64_t)p.slot_of_expert[e] * p.slot_stride + p.b_off;

  // Per stage this wave loads A blocks 2w, 2w+1 (and 16 + w on a tall tile, waves 0-3)
  // and B blocks 2w, 2w+1. An A block is 16 rows x 32 columns; lane l fetches 16 bytes of
  // row r = l/4, so each quad of lanes reads one row's 64 contiguous bytes. Chunk c of
  // row r is stored at slot 4r + (c ^ g(r)) with g(r) = (r3 << 1) | r2 (bits of r): the
  // MFMA fragment reads (row l%16, chunk l/16) then touch distinct 16-byte slots modulo 32
  // within every 32 consecutive lanes, and so also within every 16, whichever of the two
  // lane groups the LDS serves a 16-byte read in.
  const bool extra_a = TALL && w < 4;
  const int dma_per_stage = 4 + (extra_a ? 1 : 0);
  auto swz = [](int r) { return (((r >> 3) & 1) << 1) | ((r >> 2) & 1); };
  const int a_chunk = (lane & 3) ^ swz(lane >> 2);
  auto a_src = [&](int blk) {
    int r = row0 + blk * 16 + (lane >> 2);
    r = r < row_end ? r : row_end - 1;
    const int src = p.a_row_src ? p.a_row_src[r] / p.a_row_div : r;
    return p.a + (size_t)src * p.K + 8 * a_chunk;
  };
  // running source pointers, advanced one stage per issue (stages are issued in order);
  // the DMA instructions take them as their address operands directly
  const bf16_t* arow0 = a_src(2 * w);
  const bf16_t* arow1 = a_src(2 * w + 1);
  const bf16_t* arow2 = extra_a ? a_src(16 + w) : arow0;
  const char* bptr0 = B + ((int64_t)(n0 / 16 + 2 * w) * KS) * 1024 + 16 * lane;
  const char* bptr1 = bptr0 + (int64_t)KS * 1024;
  auto issue = [&](int s) {
    char* base = smem[s % kStages];
    dma16_asm(arow0, base + (2 * w) * 1024);
    dma16_asm(arow1, base + (2 * w + 1) * 1024);
    if (extra_a) dma16_asm(arow2, base + (16 + w) * 1024);
    dma16_asm(bptr0, base + kStageA + (2 * w) * 1024);
    dma16_asm(bptr1, base + kStageA + (2 * w + 1) * 1024);
    arow0 += 32;
    arow1 += 32;
    arow2 += 32;
    bptr0 += 1024;
    bptr1 += 1024;
  };
  // wave row wm (MB m-blocks) x wave column wn (4 n-blocks). Waves w and w + 4 share a
  // SIMD; they form the two groups that take turns (see the main loop).
  const int g = w >> 2;
  const int wm = g, wn = w & 3;
  const int a_slot = 16 * (4 * (lane & 15) + ((lane >> 4) ^ swz(lane & 15)));  // row l%16, chunk l/16
  bf16x8_t fa[MB], fb[4];
  auto read = [&](int s) {
    const char* base = smem[s % kStages];
#pragma unroll
    for (int i = 0; i < MB; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(base + (wm * MB + i) * 1024 + a_slot);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[j] = *reinterpret_cast<const bf16x8_t*>(base + kStageA + (wn * 4 + j) * 1024 + 16 * lane);
  };

  f32x4_t acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The MFMAs are written as inline assembly with the accumulators pinned to AGPRs: with
  // the builtin, the register allocator rotates the loop-carried accumulator tiles between
  // registers at the loop back-edge, and the copies (plus their hazard NOPs) cost about a
  // third of the MFMA issue rate.
  auto mma = [&]() {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : MOEFFN_ACC(acc[i][j]) : "v"(fa[i]), "v"(fb[j]));
  };

  // Main loop, one barrier per stage. Between barrier s and barrier s + 1, group 0 runs
  // the MFMAs of stage s and then reads the fragments of stage s + 1, while group 1 reads
  // stage s and then runs its MFMAs; group 0 raises its wave priority for its MFMA burst,
  // so on every SIMD the two bursts follow each other and each group's LDS reads overlap
  // the other group's MFMAs. Stages s and s + 1 are read between barriers s and s + 1, so
  // the DMA of stage s + 3 (issued then) goes into the buffer of stage s - 1, which both
  // groups finished reading before barrier s. Before barrier s + 1 every wave waits for
  // its own part of stage s + 2 to land, and the barrier makes it visible to all.
  static_assert(kStages == 4, "the schedule below keeps stages s - 1 .. s + 2 in the ring");
  constexpr int kDmaG0 = TALL ? 5 : 4;   // DMA instructions per stage of a group-0 wave
  for (int s = 0; s < 3 && s < KS; ++s) issue(s);
  wait_vmcnt_le(dma_per_stage * min(KS - 1, 2));   // stage 0 has landed
  barrier_no_fence();
  if (g == 0) {
    read(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if (KS > 1) wait_vmcnt_le(dma_per_stage * (min(KS - 1, 2) - 1));   // stage 1 has landed
  barrier_no_fence();
  // (one code path for both groups, so a single set of fragment registers is live)
  for (int s = 0; s < KS; ++s) {
    if (g == 0) {
      __builtin_amdgcn_s_setprio(1);
      mma();
      __builtin_amdgcn_s_setprio(0);
    }
    if (s + 3 < KS) issue(s + 3);
    if (s + 1 - g < KS) read(s + 1 - g);   // group 0 reads stage s + 1, group 1 stage s
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (g == 1) mma();
    if (s + 3 < KS) {
      if (g == 0) wait_vmcnt<kDmaG0>();
      else wait_vmcnt<4>();
    } else if (s + 2 < KS) {
      wait_vmcnt<0>();
    }
    if (s + 1 < KS) barrier_no_fence();
  }
  // the next tile is claimed now, so the atomic's round trip overlaps the epilogue
  claim();
  // the last MFMAs must retire before their accumulators are read: the hazard recognizer
  // does not see inside the inline assembly, so the wait states are placed by hand. The
  // CDNA3/CDNA4 ISA asks for at most 19 between an XDL MFMA (16 passes at most) writing a
  // VGPR and a VALU or memory instruction reading it; these four s_nop 7 give 32.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // epilogue: lane holds rows 4*(lane/16)+q, column lane%16 of each 16x16 tile
  const int rbase = row0 + wm * MB * 16 + 4 * (lane >> 4);
  if constexpr (MODE == MODE_GATEUP) {
    const int F = p.N / 2;
    bf16_t* H = static_cast<bf16_t*>(p.out);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int hcol = n0 / 2 + wn * 32 + pp * 16 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rbase + i * 16 + q;
          if (r < row_end) {
            const float g = acc[i][2 * pp][q], u = acc[i][2 * pp + 1][q];
            H[(size_t)r * F + hcol] = f32_to_bf16_int(silu_fast(g) * u);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rbase + i * 16 + q;
          if (r < row_end) {
            if (p.out_dtype == MOE_BF16) static_cast<bf16_t*>(p.out)[(size_t)r * p.N + col] = f32_to_bf16_int(acc[i][j][q]);
            else static_cast<float*>(p.out)[(size_t)r * p.N + col] = acc[i][j][q];
          }
        }
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(64 * kGemmWaves, 1) void ffn_gemm_bf16(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages][kStageBytes];
  __shared__ int32_t s_prefix[kMaxE + 1];   // the m-tile prefix, searched once per tile
  __shared__ int s_tile;
  const int NT = p.N / kBN;
  for (int i = threadIdx.x; i <= p.E; i += blockDim.x) s_prefix[i] = p.tile_prefix[i];
  const int total = p.tile_prefix[p.E] * NT;
  int range = 0;   // thread 0: how many XCD ranges this block has used up
  // thread 0 claims a block's next tile: the first here, each later one right after the k loop
  // of the tile before it (its atomic then overlaps that tile's epilogue)
  auto claim = [&]() {
    if (threadIdx.x == 0) s_tile = take_tile(p.counters, total, range);
  };
  claim();
  __syncthreads();
  for (;;) {
    const int L = __builtin_amdgcn_readfirstlane(s_tile);
    if (L < 0) return;
    int e, mt, mte, nt;
    tile_coords(s_prefix, p.E, NT, L, e, mt, mte, nt);
    // (read from LDS, so the compiler cannot see they are uniform: keep them scalar)
    e = __builtin_amdgcn_readfirstlane(e);
    mt = __builtin_amdgcn_readfirstlane(mt);
    mte = __builtin_amdgcn_readfirstlane(mte);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int row0 = p.offsets[e] + mt * kBM;
    const int row_end = mt + 1 < mte ? row0 + kBM : p.offsets[e + 1];
    // every wave reads s_tile before the tile's first barrier, and thread 0 overwrites it only
    // after the k loop
    if (kTallRows > 0 && row_end - row0 > kBM)
      gemm_bf16_tile<MODE, (kTallRows > 0)>(p, smem, e, row0, row_end, nt * kBN, claim);
    else
      gemm_bf16_tile<MODE, false>(p, smem, e, row0, row_end, nt * kBN, claim);
    // every wave is done with the LDS ring, and s_tile holds the next tile
    __syncthreads();
  }
}

}  // namespace
}  // namespace moeffn
