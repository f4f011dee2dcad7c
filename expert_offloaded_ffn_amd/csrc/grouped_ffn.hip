// moe_grouped_ffn: every selected expert's SwiGLU FFN over the rows grouped to it.
//
// "The Billion-Token Bottleneck" (section "The Geometry of the Problem") makes
// each expert a feed-forward network; "NovaLLM: Running Massive MoE Models
// Fully In-Memory" (section 3) runs only the experts that were hit. The expert
// weights are read through the slot table (pool + slot * stride), which is how
// the same kernels serve a fully resident layer and the expert slot pool.
//
// Kernels:
//  ffn_tile_map       per-expert m-tile counts -> prefix (device side; no host sync)
//  ffn_gemm_bf16      prefill tile engine on MFMA 16x16x32 bf16: 256x256 block
//                     tiles, 8 waves of 128x64 (two per SIMD, so one wave's LDS
//                     reads hide under the other's MFMAs). A and B move from global memory
//                     straight into LDS (global_load_lds_dwordx4, no staging
//                     registers) in the 1 KiB fragment-tile layout, so every wave
//                     load and every fragment read is 1 KiB contiguous. A 4-deep ring
//                     of 32-column stages keeps loads three stages ahead; one
//                     barrier per stage. Tiles are mapped XCD-aware so
//                     the m-tiles that share a weight tile run on one XCD's L2.
//                     Mode GATEUP writes H = silu(G) * U (bf16), mode DOWN writes Y.
//  ffn_f32_*          fp32 VALU path (one thread per output element) for fp32
//                     weights.
#include <algorithm>

#include "moe_internal.h"

namespace moeffn {
namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kMaxE = 1024;

// Bundle geometry (must match moe_pack_expert).
struct BundleGeom {
  int64_t gu_off, dn_off, sg_off, su_off, sd_off, bytes;
};

__host__ __device__ inline BundleGeom bundle_geom(int d, int F, int dt) {
  BundleGeom g{};
  auto al = [](int64_t v) { return (v + 255) / 256 * 256; };
  if (dt == MOE_BF16) {
    g.gu_off = 0;
    g.dn_off = al((int64_t)2 * F * d * 2);
    g.bytes = g.dn_off + al((int64_t)d * F * 2);
  } else if (dt == MOE_FP8_E4M3) {
    g.gu_off = 0;
    g.dn_off = al((int64_t)2 * F * d);
    g.sg_off = g.dn_off + al((int64_t)d * F);
    g.su_off = g.sg_off + al((int64_t)(F / 128) * (d / 128) * 4);
    g.sd_off = g.su_off + al((int64_t)(F / 128) * (d / 128) * 4);
    g.bytes = g.sd_off + al((int64_t)(d / 128) * (F / 128) * 4);
  } else {
    g.gu_off = 0;                               // W_gate^T [F, d] then W_up^T [F, d]
    g.dn_off = al((int64_t)2 * F * d * 4);      // W_down^T [d, F]
    g.bytes = g.dn_off + al((int64_t)d * F * 4);
  }
  return g;
}

// ----------------------------------------------------------- tile map ---
// tile_prefix[e] = m-tiles of active experts before e; tile_prefix[E] = total.
__global__ __launch_bounds__(1024) void ffn_tile_map(const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ slot_of_expert,
                                                     int32_t* __restrict__ tile_prefix, int E, int bm, int tall,
                                                     int32_t* __restrict__ counters, int n_counters) {
  __shared__ int32_t v[kMaxE];
  const int e = threadIdx.x;
  if (e < n_counters) counters[e] = 0;
  if (e < E) {
    const int n = offsets[e + 1] - offsets[e];
    // m-tiles of bm rows; the last one may hold up to bm + tall rows
    const int m = n <= bm + tall ? 1 : (n - tall + bm - 1) / bm;
    v[e] = (n > 0 && slot_of_expert[e] >= 0) ? m : 0;
  }
  __syncthreads();
  if (e == 0) {
    int acc = 0;
    for (int i = 0; i < E; ++i) {
      tile_prefix[i] = acc;
      acc += v[i];
    }
    tile_prefix[E] = acc;
  }
}

struct GemmArgs {
  const bf16_t* a;             // [*, K] row-major
  const int32_t* a_row_src;    // NULL: GEMM row r reads a row r
  int a_row_div;
  const int32_t* offsets;      // [E+1]
  const int32_t* slot_of_expert;
  const int32_t* tile_prefix;  // [E+1]
  int32_t* counters;           // [8] tiles taken from each XCD's range (zeroed by ffn_tile_map)
  const char* pool;
  int64_t slot_stride;
  int64_t b_off;               // byte offset of B inside a bundle
  int N, K;                    // B is [N, K] in 1 KiB fragment tiles
  void* out;                   // GATEUP: H [rows, N/2] bf16; DOWN: Y [rows, N]
  int out_dtype;
  int E;
};

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

// Tile L of a launch -> (expert e, m-tile mt of mte, n-tile nt). Tiles run expert by
// expert; within an expert the m-tiles of one n-tile are adjacent, so the tiles that
// share a weight tile are taken close together in time by the same XCD.
__device__ __forceinline__ void tile_coords(const int32_t* tile_prefix, int E, int NT, int L, int& e, int& mt,
                                            int& mte, int& nt) {
  const int q = L / NT;
  int lo = 0, hi = E - 1;  // last e with tile_prefix[e] <= q
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_prefix[mid] <= q) lo = mid;
    else hi = mid - 1;
  }
  e = lo;
  const int base = tile_prefix[e];
  mte = tile_prefix[e + 1] - base;
  const int local = L - base * NT;
  nt = local / mte;
  mt = local % mte;
}

// Persistent blocks (one per CU) take tiles from per-XCD queues. Workgroups are dealt
// round-robin over the 8 XCDs, so block b runs on XCD b % 8. The tiles are cut into 8
// contiguous ranges, one per XCD (tiles that share a weight tile stay in one XCD's L2);
// block b takes the next tile of its own
// XCD's range with an atomic counter and, once that range is used up, of the other ranges
// in turn. Work moves to whichever CU is free, so tiles of unequal cost (an expert's
// taller last m-tile) and XCDs with more of them do not leave CUs idle. Returns -1 when
// every range is used up; each counter is visited at most once more per block after it
// runs out, so every block reaches that exit.
__device__ __forceinline__ int take_tile(int32_t* counters, int total, int& range) {
  const int per = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  while (range < 8) {
    const int x = (xcd + range) & 7;
    const int lo = x * per;
    const int n = min(per, total - lo);
    if (n > 0) {
      const int i = atomicAdd(counters + x, 1);
      if (i < n) return lo + i;
    }
    ++range;
  }
  return -1;
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4, with the LDS base in M0), issued as inline assembly: the
// compiler then does not track the LDS write, so it adds no "vmcnt(0)" before later LDS
// reads; callers order them with explicit vmcnt waits and barriers. Each asm block sets M0
// itself; M0 is reserved by the compiler (so it is not listed as clobbered) and the
// compiled kernels here make no other use of it. lds_base must be wave-uniform.
__device__ __forceinline__ void dma16_asm(const void* g, const void* lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}

// Workgroup barrier without the release fence __syncthreads() carries: that fence
// makes the compiler wait for every outstanding global load, including the LDS DMA
// of later stages. Callers wait for what they need (vmcnt/lgkmcnt) first.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most n of this wave's vector-memory instructions (here: LDS DMA) are
// outstanding; n is rounded down to an available immediate, which only waits longer.
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if (n >= 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (n >= 20) asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
  else if (n >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n >= 15) asm volatile("s_waitcnt vmcnt(15)" ::: "memory");
  else if (n >= 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if (n >= 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

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
template <int MODE, bool TALL>
__device__ __forceinline__ void gemm_bf16_tile(const GemmArgs& p, char (*smem)[kStageBytes], int e, int row0,
                                               int row_end, int n0) {
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
  // the last MFMAs must retire before their accumulators are read (the hazard
  // recognizer does not see inside the inline assembly)
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
            H[(size_t)r * F + hcol] = f32_to_bf16(silu_fast(g) * u);
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
            if (p.out_dtype == MOE_BF16) static_cast<bf16_t*>(p.out)[(size_t)r * p.N + col] = f32_to_bf16(acc[i][j][q]);
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
  __shared__ int s_tile;
  const int NT = p.N / kBN;
  const int total = p.tile_prefix[p.E] * NT;
  int range = 0;   // thread 0: how many XCD ranges this block has used up
  for (;;) {
    if (threadIdx.x == 0) s_tile = take_tile(p.counters, total, range);
    __syncthreads();
    const int L = s_tile;
    if (L < 0) return;
    int e, mt, mte, nt;
    tile_coords(p.tile_prefix, p.E, NT, L, e, mt, mte, nt);
    const int row0 = p.offsets[e] + mt * kBM;
    const int row_end = mt + 1 < mte ? row0 + kBM : p.offsets[e + 1];
    if (kTallRows > 0 && row_end - row0 > kBM)
      gemm_bf16_tile<MODE, (kTallRows > 0)>(p, smem, e, row0, row_end, nt * kBN);
    else
      gemm_bf16_tile<MODE, false>(p, smem, e, row0, row_end, nt * kBN);
    // every wave is done with the LDS ring and has read s_tile before they are reused
    __syncthreads();
  }
}

// -------------------------------------------------------- decode path ---
// Few rows per expert (decode batches): the layer is bound by streaming each active
// expert's weights once from HBM. A workgroup owns one active expert and one group of
// 32 weight rows (GATEUP: 16 gate + 16 up rows -> 16 hidden columns; DOWN: 32 output
// columns); its 4 waves split K. Weight tiles go straight from global memory into MFMA
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

template <int MODE>
__global__ __launch_bounds__(64 * kDecWaves, MOEFFN_DEC_MINBLOCKS) void ffn_decode_bf16(DecodeArgs p) {
  __shared__ f32x4_t red[kDecWaves - 1][4][2][64];   // partials of waves 1..: [wave][m-block][n-tile][lane]
  const int G = p.N / 32;
  const int i = blockIdx.x / G, g = blockIdx.x % G;
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

// ----------------------------------------------------------- fp8 path ---
// e4m3 operands with fp32 block scales (per row per 128 columns for activations, per
// 128x128 block for weights). The scales are arbitrary fp32 values, which the MFMA's
// power-of-two (E8M0) scale operands cannot carry, so every 16x16x128 MFMA covers exactly
// one 128-column scale block and its partial product is promoted on the VALU:
// acc += P * (s_row * s_weight). The accumulators therefore live in VGPRs, which bounds
// a wave's tile to 64 x 128: block tile 128 x 256, 4 waves (2 x 2), one 128-column scale
// block per stage, a 3-deep LDS ring fed by direct-to-LDS loads two stages ahead.
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
  issue(0);
  if (KB > 1) issue(1);
  for (int s = 0; s < KB; ++s) {
    wait_dma(s + 1 < KB);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_no_fence();
    if (s + 2 < KB) issue(s + 2);
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

// ---------------------------------------------------------- fp32 path ---
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E - 1;  // last e with offsets[e] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn_f32_gateup(const float* __restrict__ a, const int32_t* __restrict__ a_row_src,
                                                      int a_row_div, const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ slot_of_expert,
                                                      const char* __restrict__ pool, int64_t stride,
                                                      float* __restrict__ H, int rows, int d, int F, int E) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)rows * F) return;
  const int r = (int)(gid / F), f = (int)(gid % F);
  const int e = expert_of_row(offsets, E, r);
  const int slot = slot_of_expert[e];
  if (slot < 0) return;
  const float* wg = reinterpret_cast<const float*>(pool + (int64_t)slot * stride) + (size_t)f * d;
  const float* wu = wg + (size_t)F * d;
  const int src = a_row_src ? a_row_src[r] / a_row_div : r;
  const float* x = a + (size_t)src * d;
  float g = 0.f, u = 0.f;
  for (int i = 0; i < d; ++i) {
    g = fmaf(x[i], wg[i], g);
    u = fmaf(x[i], wu[i], u);
  }
  H[(size_t)r * F + f] = silu_f32(g) * u;
}

__global__ __launch_bounds__(256) void ffn_f32_down(const float* __restrict__ H, const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ slot_of_expert,
                                                    const char* __restrict__ pool, int64_t stride, int64_t dn_off,
                                                    void* __restrict__ y, int y_dtype, int rows, int d, int F, int E) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)rows * d) return;
  const int r = (int)(gid / d), c = (int)(gid % d);
  const int e = expert_of_row(offsets, E, r);
  const int slot = slot_of_expert[e];
  if (slot < 0) return;
  const float* wd = reinterpret_cast<const float*>(pool + (int64_t)slot * stride + dn_off) + (size_t)c * F;
  const float* h = H + (size_t)r * F;
  float s = 0.f;
  for (int i = 0; i < F; ++i) s = fmaf(h[i], wd[i], s);
  if (y_dtype == MOE_BF16) static_cast<bf16_t*>(y)[(size_t)r * d + c] = f32_to_bf16(s);
  else static_cast<float*>(y)[(size_t)r * d + c] = s;
}

// Compute units of the current device (cached per device).
long long cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Workspace: H [rows, F] (fp32, bf16 or e4m3) [+ e4m3 H scales [rows, F/128]], then the
// tile prefix and the per-XCD work counters of the persistent GEMMs.
size_t ws_layout(const moe_expert_table* t, int rows, int act_dtype, size_t* h_off, size_t* map_off,
                 size_t* hs_off = nullptr) {
  const size_t hsz = act_dtype == MOE_F32 ? 4 : act_dtype == MOE_FP8_E4M3 ? 1 : 2;
  *h_off = 0;
  size_t end = align_up((size_t)rows * t->d_ff * hsz, 256);
  if (hs_off) *hs_off = end;
  if (act_dtype == MOE_FP8_E4M3) end += align_up((size_t)rows * (t->d_ff / 128) * 4, 256);
  *map_off = end;   // tile prefix [E+1], then the work counters [16]
  return *map_off + align_up((size_t)(t->n_experts + 2) * 4, 256) + 256;
}

}  // namespace
}  // namespace moeffn

using namespace moeffn;

extern "C" size_t moe_bundle_bytes(int32_t d_model, int32_t d_ff, int32_t w_dtype) {
  if (d_model < 1 || d_ff < 1) return 0;
  if (w_dtype == MOE_BF16 && (d_model % 32 || d_ff % 32)) return 0;
  if (w_dtype == MOE_FP8_E4M3 && (d_model % 128 || d_ff % 128)) return 0;
  if (w_dtype == MOE_F32 && d_model % 4) return 0;
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16 && w_dtype != MOE_FP8_E4M3) return 0;
  return (size_t)bundle_geom(d_model, d_ff, w_dtype).bytes;
}

extern "C" size_t moe_grouped_ffn_workspace_size(const moe_expert_table* table, int32_t rows, int32_t act_dtype) {
  if (!table || rows < 0) return 0;
  size_t h, m;
  return ws_layout(table, rows, act_dtype, &h, &m);
}

extern "C" moe_status moe_grouped_ffn(const moe_expert_table* table, int32_t rows, const int32_t* offsets,
                                      const void* a, const float* a_scale, int32_t act_dtype,
                                      const int32_t* a_row_src, int32_t a_row_div, void* y, int32_t y_dtype,
                                      void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  MOE_REQUIRE(table != nullptr, MOE_EINVAL, "moe_grouped_ffn: table is NULL");
  const moe_expert_table t = *table;
  MOE_REQUIRE(rows >= 0, MOE_EINVAL, "moe_grouped_ffn: rows=%d < 0", rows);
  MOE_REQUIRE(t.n_experts >= 1 && t.n_experts <= kMaxE, MOE_EINVAL, "moe_grouped_ffn: n_experts=%d outside [1, %d]",
              t.n_experts, kMaxE);
  const size_t bb = moe_bundle_bytes(t.d_model, t.d_ff, t.w_dtype);
  MOE_REQUIRE(bb > 0, MOE_EINVAL, "moe_grouped_ffn: unsupported sizes d=%d F=%d for w_dtype %d", t.d_model, t.d_ff,
              t.w_dtype);
  MOE_REQUIRE(t.slot_stride >= (int64_t)bb && t.slot_stride % 256 == 0, MOE_EINVAL,
              "moe_grouped_ffn: slot_stride %lld must be >= bundle bytes %zu and a multiple of 256",
              (long long)t.slot_stride, bb);
  MOE_REQUIRE(y_dtype == MOE_F32 || y_dtype == MOE_BF16, MOE_EUNSUPPORTED, "moe_grouped_ffn: y_dtype %d", y_dtype);
  if (a_row_src) MOE_REQUIRE(a_row_div >= 1, MOE_EINVAL, "moe_grouped_ffn: a_row_div must be >= 1");
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(t.pool && t.slot_of_expert && offsets && a && y && ws, MOE_EINVAL, "moe_grouped_ffn: NULL argument");
  MOE_REQUIRE(aligned(t.pool, 256) && aligned(a, 16) && aligned(y, 16) && aligned(ws, 256), MOE_EINVAL,
              "moe_grouped_ffn: pool needs 256-B, a and y 16-B, ws 256-B alignment");
  size_t h_off, map_off;
  const size_t need = ws_layout(&t, rows, act_dtype, &h_off, &map_off);
  MOE_REQUIRE(ws_bytes >= need, MOE_ECAPACITY, "moe_grouped_ffn: workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t s = as_stream(stream);
  const BundleGeom g = bundle_geom(t.d_model, t.d_ff, t.w_dtype);
  char* wsb = static_cast<char*>(ws);
  const int E = t.n_experts, d = t.d_model, F = t.d_ff;

  if (t.w_dtype == MOE_F32) {
    MOE_REQUIRE(act_dtype == MOE_F32, MOE_EUNSUPPORTED, "moe_grouped_ffn: fp32 weights need fp32 activations");
    float* H = reinterpret_cast<float*>(wsb + h_off);
    const long long n1 = (long long)rows * F, n2 = (long long)rows * d;
    hipLaunchKernelGGL(ffn_f32_gateup, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, static_cast<const float*>(a),
                       a_row_src, a_row_div, offsets, t.slot_of_expert, static_cast<const char*>(t.pool),
                       t.slot_stride, H, rows, d, F, E);
    hipLaunchKernelGGL(ffn_f32_down, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, H, offsets,
                       t.slot_of_expert, static_cast<const char*>(t.pool), t.slot_stride, g.dn_off, y, y_dtype, rows,
                       d, F, E);
    return check_launch("moe_grouped_ffn f32");
  }
  if (t.w_dtype == MOE_BF16) {
    MOE_REQUIRE(act_dtype == MOE_BF16, MOE_EUNSUPPORTED, "moe_grouped_ffn: bf16 weights need bf16 activations");
    MOE_REQUIRE((2 * F) % kBN == 0 && d % kBN == 0, MOE_EUNSUPPORTED,
                "moe_grouped_ffn: bf16 prefill tiles need d and 2F multiples of %d", kBN);
    int32_t* tile_prefix = reinterpret_cast<int32_t*>(wsb + map_off);
    bf16_t* H = reinterpret_cast<bf16_t*>(wsb + h_off);
    // Rows per expert are bounded by the number of distinct source rows: at most
    // rows / a_row_div tokens (each picks an expert once) or all rows.
    const int max_rows_e = a_row_src ? (rows + a_row_div - 1) / a_row_div : rows;
    if (max_rows_e <= 64 && (2 * F) % 32 == 0 && d % 32 == 0) {
      const int max_active = E < rows ? E : rows;
      DecodeArgs q{};
      q.a = static_cast<const bf16_t*>(a);
      q.a_row_src = a_row_src;
      q.a_row_div = a_row_div;
      q.offsets = offsets;
      q.slot_of_expert = t.slot_of_expert;
      q.E = E;
      q.pool = static_cast<const char*>(t.pool);
      q.slot_stride = t.slot_stride;
      q.b_off = g.gu_off;
      q.N = 2 * F;
      q.K = d;
      q.out = H;
      q.out_dtype = MOE_BF16;
      prof_mark(s, MOE_PROF_DEC_GATEUP, false);
      hipLaunchKernelGGL(ffn_decode_bf16<MODE_GATEUP>, dim3(max_active * (q.N / 32)), dim3(64 * kDecWaves), 0, s, q);
      prof_mark(s, MOE_PROF_DEC_GATEUP, true);
      q.a = H;
      q.a_row_src = nullptr;
      q.a_row_div = 1;
      q.b_off = g.dn_off;
      q.N = d;
      q.K = F;
      q.out = y;
      q.out_dtype = y_dtype;
      prof_mark(s, MOE_PROF_DEC_DOWN, false);
      hipLaunchKernelGGL(ffn_decode_bf16<MODE_DOWN>, dim3(max_active * (q.N / 32)), dim3(64 * kDecWaves), 0, s, q);
      prof_mark(s, MOE_PROF_DEC_DOWN, true);
      return check_launch("moe_grouped_ffn bf16 decode");
    }
    int32_t* counters = reinterpret_cast<int32_t*>(wsb + map_off + align_up((size_t)(E + 2) * 4, 256));
    hipLaunchKernelGGL(ffn_tile_map, dim3(1), dim3(((E + 63) / 64) * 64), 0, s, offsets, t.slot_of_expert,
                       tile_prefix, E, kBM, kTallRows, counters, 16);
    const int max_mt = (rows + kBM - 1) / kBM + (E < rows ? E : rows);
    const long long n_cu = cu_count();
    GemmArgs p{};
    p.a_row_src = a_row_src;
    p.a_row_div = a_row_div;
    p.offsets = offsets;
    p.slot_of_expert = t.slot_of_expert;
    p.tile_prefix = tile_prefix;
    p.counters = counters;
    p.pool = static_cast<const char*>(t.pool);
    p.slot_stride = t.slot_stride;
    p.E = E;
    // gate/up + SwiGLU: B = W_gu [2F, d]
    p.a = static_cast<const bf16_t*>(a);
    p.b_off = g.gu_off;
    p.N = 2 * F;
    p.K = d;
    p.out = H;
    p.out_dtype = MOE_BF16;
    // persistent: at most one block per CU, a multiple of 8 (one per XCD in turn)
    long long nblk = std::min((long long)max_mt * (p.N / kBN), n_cu);
    prof_mark(s, MOE_PROF_GATEUP, false);
    hipLaunchKernelGGL(ffn_gemm_bf16<MODE_GATEUP>, dim3((unsigned)((nblk + 7) / 8 * 8)), dim3(64 * kGemmWaves), 0, s, p);
    prof_mark(s, MOE_PROF_GATEUP, true);
    // down: B = W_dn [d, F], A = H (already in row order)
    p.a = H;
    p.a_row_src = nullptr;
    p.a_row_div = 1;
    p.b_off = g.dn_off;
    p.N = d;
    p.K = F;
    p.out = y;
    p.out_dtype = y_dtype;
    p.counters = counters + 8;
    nblk = std::min((long long)max_mt * (p.N / kBN), n_cu);
    prof_mark(s, MOE_PROF_DOWN, false);
    hipLaunchKernelGGL(ffn_gemm_bf16<MODE_DOWN>, dim3((unsigned)((nblk + 7) / 8 * 8)), dim3(64 * kGemmWaves), 0, s, p);
    prof_mark(s, MOE_PROF_DOWN, true);
    return check_launch("moe_grouped_ffn bf16");
  }
  // fp8 weights: e4m3 activations with per-row per-128 scales
  MOE_REQUIRE(act_dtype == MOE_FP8_E4M3 && a_scale != nullptr, MOE_EUNSUPPORTED,
              "moe_grouped_ffn: fp8 weights need e4m3 activations and their scales");
  MOE_REQUIRE((2 * F) % kF8BN == 0 && d % kF8BN == 0 && d % 128 == 0 && F % 128 == 0, MOE_EUNSUPPORTED,
              "moe_grouped_ffn: fp8 tiles need d and 2F multiples of %d and F a multiple of 128", kF8BN);
  MOE_REQUIRE(aligned(a_scale, 4), MOE_EINVAL, "moe_grouped_ffn: a_scale must be 4-byte aligned");
  MOE_REQUIRE(d / 128 <= kF8MaxKB && F / 128 <= kF8MaxKB, MOE_EUNSUPPORTED,
              "moe_grouped_ffn: fp8 tiles need d and F at most %d", 128 * kF8MaxKB);
  {
    size_t hs_off;
    ws_layout(&t, rows, act_dtype, &h_off, &map_off, &hs_off);
    int32_t* tile_prefix = reinterpret_cast<int32_t*>(wsb + map_off);
    uint8_t* Hq = reinterpret_cast<uint8_t*>(wsb + h_off);
    float* Hs = reinterpret_cast<float*>(wsb + hs_off);
    int32_t* counters = reinterpret_cast<int32_t*>(wsb + map_off + align_up((size_t)(E + 2) * 4, 256));
    hipLaunchKernelGGL(ffn_tile_map, dim3(1), dim3(((E + 63) / 64) * 64), 0, s, offsets, t.slot_of_expert,
                       tile_prefix, E, kF8BM, 0, counters, 16);
    const int max_mt = (rows + kF8BM - 1) / kF8BM + (E < rows ? E : rows);
    const long long n_cu = cu_count();
    Fp8Args p{};
    p.a = static_cast<const uint8_t*>(a);
    p.a_scale = a_scale;
    p.a_row_src = a_row_src;
    p.a_row_div = a_row_div;
    p.offsets = offsets;
    p.slot_of_expert = t.slot_of_expert;
    p.tile_prefix = tile_prefix;
    p.counters = counters;
    p.pool = static_cast<const char*>(t.pool);
    p.slot_stride = t.slot_stride;
    p.E = E;
    p.b_off = g.gu_off;
    p.s_off0 = g.sg_off;
    p.s_off1 = g.su_off;
    p.N = 2 * F;
    p.K = d;
    p.out = Hq;
    p.out_scale = Hs;
    long long nblk = std::min((long long)max_mt * (p.N / kF8BN), n_cu);
    prof_mark(s, MOE_PROF_GATEUP, false);
    hipLaunchKernelGGL(ffn_gemm_fp8<MODE_GATEUP>, dim3((unsigned)((nblk + 7) / 8 * 8)), dim3(512), 0, s, p);
    prof_mark(s, MOE_PROF_GATEUP, true);
    p.a = Hq;
    p.a_scale = Hs;
    p.a_row_src = nullptr;
    p.a_row_div = 1;
    p.b_off = g.dn_off;
    p.s_off0 = g.sd_off;
    p.s_off1 = 0;
    p.N = d;
    p.K = F;
    p.out = y;
    p.out_scale = nullptr;
    p.out_dtype = y_dtype;
    p.counters = counters + 8;
    nblk = std::min((long long)max_mt * (p.N / kF8BN), n_cu);
    prof_mark(s, MOE_PROF_DOWN, false);
    hipLaunchKernelGGL(ffn_gemm_fp8<MODE_DOWN>, dim3((unsigned)((nblk + 7) / 8 * 8)), dim3(512), 0, s, p);
    prof_mark(s, MOE_PROF_DOWN, true);
  }
  return check_launch("moe_grouped_ffn fp8");
}
