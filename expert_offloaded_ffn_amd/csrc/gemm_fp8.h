// The fp8 (e4m3 with fp32 block scales) prefill GEMM of the grouped FFN.
//
// Operands: activations as e4m3 codes with one fp32 scale per row per 128 columns, weights as
// e4m3 codes with one fp32 scale per 128 x 128 block (the DeepSeek-V3-shaped workload's
// format). The scales are arbitrary fp32 values, which the MFMA's power-of-two (E8M0) scale
// operands cannot carry, so every 16x16x128 MFMA covers exactly one 128-column scale block and
// its partial product is promoted on the VALU: acc += P * (s_row * s_weight). That is one FMA
// per output element per 128 columns, so the accumulators live in VGPRs.
//
// Tile 256 x 256 on 8 waves (2 wave rows of 128 rows x 4 wave columns of 64 columns, two waves
// per SIMD): per 128-column stage a block moves 64 KB into LDS for 8.4 M MACs, and a wave
// reads 24 KB of fragments for 1 M MACs. An expert's m-tiles of one n-tile are adjacent in
// the tile order and taken by one XCD, so they share the weight tile in its L2.
//
// In the gate/up GEMM the weight rows alternate between gate and up every 16 (the bundle
// layout), so a 256-column tile holds 128 hidden columns of each. Wave columns 0 and 2 take the
// gate n-blocks of the two halves, 1 and 3 the up n-blocks of the same hidden columns: a wave's
// 64 columns then share one weight block scale per stage. The epilogue hands the gate values to
// the up waves through LDS, which form H = silu(G) * U, quantise it per row per 128 hidden
// columns (one scale per tile row: the tile covers exactly one such block) and store it.
//
// One launch runs one or two problems (the routed experts and a shared expert: the shared
// expert is a group of its own in the same tile list, so it neither competes with the routed
// GEMM from a second stream nor re-reads its activations once per n-tile from its own launch).
#pragma once

#include <type_traits>

#include "ffn_common.h"

namespace moeffn {
namespace {

constexpr int kQBM = 256, kQBN = 256;
constexpr int kQMaxKB = 128;     // K up to 16384 (the tile's weight block scales are staged in LDS)
// LDS ring stage of a tile of more than 128 rows (two stages): A 256 rows x 128 B (row r's
// 16-byte chunk c at 128 r + 16 (c ^ f(r))), B 16 n-blocks of 2 KiB in the bundle's fragment
// order, the 256 row scales of the stage.
constexpr int kQA = 0, kQB = 32768, kQS = 65536, kQStage = 66560;
// A tile of at most 128 rows computes on its first wave row only, so a stage's MFMAs are short
// against the round trip of its loads: three stages of A 128 rows, B and 128 row scales keep
// the loads of two stages in flight while one is computed.
constexpr int kQsA = 0, kQsB = 16384, kQsS = 49152, kQsStage = 49664, kQsStages = 3;
constexpr int kQRing = 2 * kQStage > kQsStages * kQsStage ? 2 * kQStage : kQsStages * kQsStage;

// One grouped-FFN problem of a launch.
struct Fp8Prob {
  const uint8_t* a;            // e4m3 codes, rows of K bytes
  const float* a_scale_t;      // [K/128][a_scale_ld]: block kb's scale of GEMM row r at kb*ld + r
  int a_scale_ld;              // >= rows + 256 (a tile may read past the last row)
  const int32_t* a_row_src;    // NULL: GEMM row r reads row r of a
  int a_row_div;
  const int32_t* offsets;      // [E+1]
  const int32_t* slot_of_expert;
  const char* pool;
  int64_t slot_stride;
  int64_t b_off;               // byte offset of B (the [N, K] fragment tiles) in a bundle
  int64_t s_off0, s_off1;      // GATEUP: gate and up scale grids [F/128][K/128]; DOWN: [d/128][F/128]
  int E, N, K;
  void* out;                   // GATEUP: Hq [rows, N/2] e4m3; DOWN: y [rows, N] (bf16 or f32)
  float* out_scale_t;          // GATEUP: Hs [N/256][out_scale_ld] (kb-major for the down GEMM)
  int out_scale_ld;
  int out_dtype;
};

struct Fp8Args {
  Fp8Prob p[2];
  int E0;                      // experts of problem 0; global expert g >= E0 is problem 1's g - E0
  int n_exp;                   // E0 (+ E1)
  const int32_t* tile_prefix;  // [n_exp + 1]: tiles (m-tiles x n-tiles) before global expert g
  int32_t* counters;           // [8] per-XCD tile counters (zeroed by fp8_tile_map)
};

// Tile prefixes of the gate/up and the down GEMM of a launch of one or two grouped problems
// (global expert g < E0 is problem 0's expert g, else problem 1's g - E0): per expert its
// m-tiles of 256 rows times the problem's n-tiles of 256 columns, and zeroed tile counters.
struct TileMapArgs {
  const int32_t* offsets[2];
  const int32_t* slot_of_expert[2];
  int E0, n_exp;
  int nt_gu[2], nt_dn[2];
};

__global__ __launch_bounds__(1024) void grouped_tile_map(TileMapArgs m, int32_t* prefix_gu, int32_t* prefix_dn,
                                                         int32_t* counters, int n_counters) {
  __shared__ int32_t wsum[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < n_counters) counters[tid] = 0;
  // thread tid owns the experts [c0, c1): their tiles, summed, then an exclusive scan of the
  // per-thread sums over the workgroup (shuffles within a wavefront, then the wavefront sums)
  const int per = (m.n_exp + 1023) / 1024;   // at most 3 (n_exp <= 2 * kMaxE + 2)
  const int c0 = min(m.n_exp, tid * per), c1 = min(m.n_exp, c0 + per);
  int ta[3], tb[3];
  int sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    ta[i] = tb[i] = 0;
    const int g = c0 + i;
    if (g < c1) {
      const int q = g < m.E0 ? 0 : 1;
      const int e = g - (q ? m.E0 : 0);
      const int n = m.offsets[q][e + 1] - m.offsets[q][e];
      const int mt = (n > 0 && m.slot_of_expert[q][e] >= 0) ? (n + kQBM - 1) / kQBM : 0;
      ta[i] = mt * m.nt_gu[q];
      tb[i] = mt * m.nt_dn[q];
    }
    sa += ta[i];
    sb += tb[i];
  }
  int ia = sa, ib = sb;   // inclusive scans within the wavefront
  for (int o = 1; o < 64; o <<= 1) {
    const int va = __shfl_up(ia, o, 64), vb = __shfl_up(ib, o, 64);
    if (lane >= o) {
      ia += va;
      ib += vb;
    }
  }
  if (lane == 63) {
    wsum[0][wave] = ia;
    wsum[1][wave] = ib;
  }
  __syncthreads();
  int a = ia - sa, b = ib - sb;   // exclusive
  for (int w = 0; w < wave; ++w) {
    a += wsum[0][w];
    b += wsum[1][w];
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int g = c0 + i;
    if (g < c1) {
      prefix_gu[g] = a;
      prefix_dn[g] = b;
      a += ta[i];
      b += tb[i];
    }
  }
  if (tid == 1023) {   // the last thread's running sums are the totals
    prefix_gu[m.n_exp] = a;
    prefix_dn[m.n_exp] = b;
  }
}

// Scales of the activation rows in the order and layout the GEMM reads them:
// out[kb * ld + r] = a_scale[src(r) * KB + kb] for GEMM rows r < rows (src(r) = a_row_src[r] /
// div, or r), and 1 for r in [rows, ld), which a last tile may read.
__global__ __launch_bounds__(256) void fp8_scales_kb_major(const float* __restrict__ a_scale,
                                                           const int32_t* __restrict__ a_row_src, int div, int rows,
                                                           int KB, int ld, float* __restrict__ out) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)KB * ld) return;
  const int kb = (int)(i / ld), r = (int)(i % ld);
  float v = 1.0f;
  if (r < rows) v = a_scale[(size_t)(a_row_src ? a_row_src[r] / div : r) * KB + kb];
  out[i] = v;
}

// Direct-to-LDS loads with a scalar base and a 32-bit per-lane offset (global_load_lds with
// saddr), as inline assembly for the reason given at dma16_asm; each sets M0 itself, which the
// build checks. lds_base and g_base must be wave-uniform.
__device__ __forceinline__ void dma16_sb(const void* g_base, uint32_t off, const void* lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(g_base), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4_sb(const void* g_base, uint32_t off, const void* lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(g_base), "s"(lds)
               : "memory");
}

__device__ __forceinline__ int fp8_swz(int r) { return ((r >> 1) + 4 * (r & 1)) & 7; }

// A pointer the compiler cannot prove wave-uniform (it was loaded through a vector load) made
// uniform, so it can be a scalar base of the direct-to-LDS loads.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// One 256 x 256 tile: rows [row0, row_end) of expert e (at most 256 of them), columns n0..n0+255.
template <int MODE, typename Claim>
__device__ __forceinline__ void fp8_tile(const Fp8Prob& p, char* ring, float (*s_wscale)[kQMaxKB],
                                         float (*amax_x)[kQBM], int e, int row0, int row_end, int n0,
                                         Claim&& claim) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int KB = p.K / 128;
  const int valid = min(kQBM, row_end - row0);
  const char* bundle = uniform_ptr(p.pool + (int64_t)p.slot_of_expert[e] * p.slot_stride);
  // the tile's weight block scales: GATEUP [0] gate, [1] up of hidden block n0/256; DOWN the
  // scales of column blocks n0/128 and n0/128 + 1 (wave column wn uses [wn >> 1])
  for (int i = threadIdx.x; i < 2 * KB; i += blockDim.x) {
    const int which = i / KB, s = i - which * KB;
    float v;
    if constexpr (MODE == MODE_GATEUP)
      v = reinterpret_cast<const float*>(bundle + (which ? p.s_off1 : p.s_off0))[(n0 / 256) * KB + s];
    else
      v = reinterpret_cast<const float*>(bundle + p.s_off0)[(n0 / 128 + which) * KB + s];
    s_wscale[which][s] = v;
  }

  // DMA: per stage wave w loads tile rows RW w .. RW w + RW - 1 of A (RW = 32, or 16 in a tile
  // of at most 128 rows: instructions of 8 rows; lane j takes row RW w + 8t + j/8, chunk
  // (j%8) ^ f(row), which lands at position j%8), B n-blocks 2w and 2w+1 (two 1 KiB halves
  // each) and, for w < 4 (w < 2), the row scales of rows 64w..64w+63.
  const bool small = valid <= 128;
  const int rpw = small ? 16 : 32, n_ta = small ? 2 : 4;
  uint32_t a_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a_off[t] = 0;
    if (t < n_ta) {
      const int r = rpw * w + 8 * t + (lane >> 3);
      const int rr = min(r, valid - 1);
      const int src = p.a_row_src ? p.a_row_src[row0 + rr] / p.a_row_div : row0 + rr;
      a_off[t] = (uint32_t)src * (uint32_t)p.K + 16u * (uint32_t)((lane & 7) ^ fp8_swz(r & 15));
    }
  }
  const uint32_t b_off = (uint32_t)((n0 / 16 + 2 * w) * KB) * 2048u + 16u * lane;
  const uint32_t b_step = (uint32_t)KB * 2048u;
  const char* a_base = uniform_ptr(reinterpret_cast<const char*>(p.a));
  const char* b_base = uniform_ptr(bundle + p.b_off);
  const char* s_base = uniform_ptr(reinterpret_cast<const char*>(p.a_scale_t + row0));
  // bytes between the row scales of consecutive stages, in a register: the loads' asm blocks
  // clobber memory, so a field of p read inside the loop is reloaded from the kernel
  // arguments every stage
  const size_t s_step = (size_t)p.a_scale_ld * 4;
  const int a_rows_w = valid - rpw * w;   // rows of this wave's A share that exist
  // loads this wave issues per stage of a small tile: its A instructions (rows past the tile's
  // last row are not loaded), four B loads and, for w < 2, one row-scale load
  const int n_ld_small = min(2, max(0, (a_rows_w + 7) >> 3)) + 4 + (w < 2 ? 1 : 0);

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment offsets: A row 16 i + l%16 of the wave row, chunks 2(l/16) and 2(l/16)+1
  const int fr = fp8_swz(lane & 15), ac = 2 * (lane >> 4);
  const int a_frag0 = 128 * (128 * wm + (lane & 15)) + 16 * (ac ^ fr);
  const int a_frag1 = 128 * (128 * wm + (lane & 15)) + 16 * ((ac + 1) ^ fr);
  const int s_frag = 4 * (128 * wm + 4 * (lane >> 4));
  // the wave's n-blocks: GATEUP gate (wn even) or up (wn odd) n-blocks of hidden half wn >> 1;
  // DOWN four consecutive ones
  auto nblk = [&](int j) { return MODE == MODE_GATEUP ? (wn >> 1) * 8 + 2 * j + (wn & 1) : wn * 4 + j; };
  const int nmb = min(8, (valid - 128 * wm + 15) >> 4);   // m-blocks of the wave with rows (<= 0: none)
  const int wsel = MODE == MODE_GATEUP ? (wn & 1) : (wn >> 1);
  const f32x4_t zero{0.f, 0.f, 0.f, 0.f};

  // The k loop for NMB computed m-blocks per wave (0, 2, 4, 6 or 8: the wave's m-blocks with
  // rows, rounded up to an even count) on the two-stage ring (SMALL false) or the three-stage
  // ring of a tile of at most 128 rows. The extra m-block of an odd count computes on rows past
  // the tile's last (clamped copies of it, or stale LDS where no load was issued); those rows
  // are never stored.
  auto kloop = [&](auto small_c, auto nmb_c) {
    constexpr bool SMALL = decltype(small_c)::value;
    constexpr int NMB = decltype(nmb_c)::value;
    constexpr int A0 = SMALL ? kQsA : kQA, B0 = SMALL ? kQsB : kQB, S0 = SMALL ? kQsS : kQS;
    constexpr int STAGE = SMALL ? kQsStage : kQStage, NS = SMALL ? kQsStages : 2, TA = SMALL ? 2 : 4;
    auto issue = [&](int s) {
      char* buf = ring + (s % NS) * STAGE;
      const char* ab = a_base + (size_t)s * 128;
#pragma unroll
      for (int t = 0; t < TA; ++t)
        if (8 * t < a_rows_w) dma16_sb(ab, a_off[t], buf + A0 + (TA * w + t) * 1024);
      const char* bb = b_base + (size_t)s * 2048;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          dma16_sb(bb, b_off + i * b_step + h * 1024, buf + B0 + (2 * w + i) * 2048 + h * 1024);
      if (w < (SMALL ? 2 : 4)) dma4_sb(s_base + (size_t)s * s_step, 4u * (64 * w + lane), buf + S0 + 256 * w);
    };
    issue(0);
    if (NS > 2 && KB > 1) issue(1);
    for (int s = 0; s < KB; ++s) {
      // stage s has landed for every wave (on the three-stage ring each wave waits until only
      // its loads of stage s + 1 are outstanding), and every wave is done with stage s - 1's
      // buffer, which the loads issued below overwrite (at s = 0 the weight scales above are
      // written)
      if constexpr (NS == 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        if (s + 1 < KB) {
          switch (n_ld_small) {
            case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
            case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
            case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
          }
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_no_fence();
      // the three-stage ring issues stage s + 2 here; the two-stage ring issues stage s + 1
      // after the first m-block's MFMAs (below), so every wave starts its MFMAs right after
      // the barrier instead of queueing its loads first (gate/up 2.907 -> 2.874 ms)
      if constexpr (NS > 2) {
        if (s + NS - 1 < KB) issue(s + NS - 1);
      }
      if constexpr (NMB > 0) {
        const char* buf = ring + (s % NS) * STAGE;
        const float sw = s_wscale[wsel][s];
        i32x8_t fb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const char* blk = buf + B0 + nblk(j) * 2048 + 16 * lane;
          const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(blk);
          const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(blk + 1024);
          fb[j] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        auto frag_a = [&](int i) {
          const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(buf + A0 + a_frag0 + 2048 * i);
          const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(buf + A0 + a_frag1 + 2048 * i);
          return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        auto row_scales = [&](int i) { return *reinterpret_cast<const f32x4_t*>(buf + S0 + s_frag + 64 * i) * sw; };
        // operand formats 0 (e4m3), block scales 2^0: the fp32 scales are applied on the VALU
        auto mfma = [&](const i32x8_t& fa, int j) {
          return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[j], zero, 0, 0, 0, 127, 0, 127);
        };
        // Software pipeline over the wave's NMB m-blocks. Per m-block i: read m-block i + 1's
        // fragment and row scales from LDS, then issue i's four MFMAs, each followed by four of
        // the FMAs that promote m-block i - 1's partial products (issued a whole block earlier,
        // so they are ready), then form i + 1's combined scales. Scheduling-group barriers pin
        // that order (the compiler would otherwise promote each result right after its MFMA
        // and wait for it), and a scheduling barrier per m-block keeps it from hoisting every
        // block's reads, which would not fit the registers.
        i32x8_t fa = frag_a(0);
        f32x4_t sc = row_scales(0);
        f32x4_t part[2][4], psc[2];
#pragma unroll
        for (int i = 0; i < NMB; ++i) {
          i32x8_t fa_n;
          f32x4_t sa_n;
          if (i < NMB - 1) {
            fa_n = frag_a(i + 1);
            sa_n = *reinterpret_cast<const f32x4_t*>(buf + S0 + s_frag + 64 * (i + 1));
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) part[i & 1][j] = mfma(fa, j);
          psc[i & 1] = sc;
          if (i > 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i - 1][j] += part[(i - 1) & 1][j] * psc[(i - 1) & 1];
          }
          if (i < NMB - 1) {
            fa = fa_n;
            sc = sa_n * sw;
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // the next m-block's LDS reads
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU (promotions)
          }
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);     // the next combined scales
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (NS == 2) {
            // every wave of a tile of more than 128 rows has at least two m-blocks
            if (i == 0 && s + 1 < KB) issue(s + 1);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[NMB - 1][j] += part[(NMB - 1) & 1][j] * psc[(NMB - 1) & 1];
      }
    }
  };
  // nmb is uniform (from the tile's row range and the wave row), so these are scalar branches.
  // A tile of more than 128 rows gives its first wave row 8 m-blocks, its second 1 to 8; one of
  // at most 128 rows gives its first wave row 1 to 8 and its second none.
  using Big = std::false_type;
  using Small = std::true_type;
  const int nmb_even = nmb <= 0 ? 0 : (nmb + 1) & ~1;
  if (small) {
    if (nmb_even == 0) kloop(Small{}, std::integral_constant<int, 0>{});
    else if (nmb_even == 2) kloop(Small{}, std::integral_constant<int, 2>{});
    else if (nmb_even == 4) kloop(Small{}, std::integral_constant<int, 4>{});
    else if (nmb_even == 6) kloop(Small{}, std::integral_constant<int, 6>{});
    else kloop(Small{}, std::integral_constant<int, 8>{});
  } else {
    if (nmb_even == 2) kloop(Big{}, std::integral_constant<int, 2>{});
    else if (nmb_even == 4) kloop(Big{}, std::integral_constant<int, 4>{});
    else if (nmb_even == 6) kloop(Big{}, std::integral_constant<int, 6>{});
    else kloop(Big{}, std::integral_constant<int, 8>{});
  }
  // the next tile is claimed now, so the atomic's round trip overlaps the epilogue
  claim();
  // every wave is done with the ring (its space is reused below)
  __syncthreads();

  // output rows of lane l: 128 wm + 16 i + 4 (l / 16) + q; columns 16 j + l % 16 of the wave's 64
  if constexpr (MODE == MODE_GATEUP) {
    // The gate wave (wn even) and the up wave (wn odd) of a hidden half hold G and U of the
    // same 128 x 64 block. The up wave finishes m-blocks [0, h), the gate wave [h, nmb): each
    // hands the other its values of the other's m-blocks through the pair's 32 KiB of LDS
    // ([i][j][lane] f32x4: G of m-blocks < h, U of the rest), so all eight waves (all four
    // SIMDs) share the epilogue instead of the four up waves alone.
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
    // H = silu(G) U for this wave's m-blocks, and its rows' maxima over its 64 hidden columns
    const int i0 = up ? 0 : h, i1 = up ? h : nmb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i >= i0 && i < i1) {
        float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t o = X[(i * 4 + j) * 64 + lane];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = up ? o[q] : acc[i][j][q];
            const float u = up ? acc[i][j][q] : o[q];
            const float hv = silu_fast(g) * u;
            acc[i][j][q] = hv;
            am[q] = fmaxf(am[q], fabsf(hv));
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) am[q] = fmaxf(am[q], __shfl_xor(am[q], off, 64));
        }
        if ((lane & 15) == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) amax_x[wn >> 1][128 * wm + 16 * i + 4 * (lane >> 4) + q] = am[q];
        }
      }
    }
    __syncthreads();
    // per row: one scale for the tile's 128 hidden columns; this wave's codes staged in LDS
    // (4 KiB per wave, [64 rows][64 B], rows from m-block i0) for 16-byte stores
    uint8_t* codes = reinterpret_cast<uint8_t*>(ring + w * 4096);
    const int F = p.N / 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i >= i0 && i < i1) {
        // lane l computes the scale of row 4 (l / 16) + l % 4 of the m-block (one divide and
        // one reciprocal where every lane took four of each); DPP quad broadcasts hand row q's
        // to the lanes that hold it. One reciprocal per row instead of a full-precision divide
        // per value: the quotient may move by an ulp, which changes a code only next to a
        // rounding tie.
        const int trq = 128 * wm + 16 * i + 4 * (lane >> 4) + (lane & 3);
        const float aq = fmaxf(amax_x[0][trq], amax_x[1][trq]);
        const float scq = aq > 0.f ? aq / 448.0f : 1.0f;
        const float invq = 1.0f / scq;
        // the hidden half 0 pair writes the rows' scales (each row by the one wave that
        // finishes it)
        if ((wn >> 1) == 0 && (lane & 15) < 4 && trq < valid)
          p.out_scale_t[(size_t)(n0 / 256) * p.out_scale_ld + row0 + trq] = scq;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lr = 16 * (i - i0) + 4 * (lane >> 4) + q;   // row among this wave's
          const float inv = quad_bcast(invq, q);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float y = fminf(fmaxf(acc[i][j][q] * inv, -448.0f), 448.0f);
            codes[lr * 64 + 16 * j + (lane & 15)] = static_cast<uint8_t>(f32_to_e4m3_rne(y));
          }
        }
      }
    }
    // this wave's LDS writes are done before its lanes read each other's bytes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint8_t* Hq = static_cast<uint8_t*>(p.out);
    const int hcol0 = n0 / 2 + 64 * (wn >> 1);
    const int nrows = 16 * (i1 - i0);   // at most 64
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * 64 + lane;               // 256 chunks of 16 B: row idx/4, chunk idx%4
      const int lr = idx >> 2, ch = idx & 3;
      const int tr = 128 * wm + 16 * i0 + lr;
      if (lr < nrows && tr < valid) {
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(codes + lr * 64 + 16 * ch);
        *reinterpret_cast<i32x4_t*>(Hq + (size_t)(row0 + tr) * F + hcol0 + 16 * ch) = v;
      }
    }
  } else if (p.out_dtype == MOE_BF16) {
    // y staged through LDS per wave ([128 rows][64 cols] bf16, 16 KiB) for 16-byte stores
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
      const int idx = it * 64 + lane;               // 1024 chunks of 16 B: row idx/8, chunk idx%8
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

// Tile L -> (global expert g, m-tile mt, n-tile nt) from a tile prefix over n_exp experts
// (problem 0's first, with NT0 n-tiles each, then problem 1's with NT1). Tiles run expert by
// expert; within an expert the m-tiles of one n-tile are adjacent, so the tiles that share a
// weight tile are taken close together in time by the same XCD.
__device__ __forceinline__ void grouped_tile_coords(const int32_t* pre, int n_exp, int E0, int NT0, int NT1, int L,
                                                    int& g, int& mt, int& nt) {
  int lo = 0, hi = n_exp - 1;   // last g with pre[g] <= L
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= L) lo = mid;
    else hi = mid - 1;
  }
  g = lo;
  const int NT = g < E0 ? NT0 : NT1;
  const int mte = (pre[g + 1] - pre[g]) / NT;
  const int local = L - pre[g];
  nt = local / mte;
  mt = local - nt * mte;
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void ffn_gemm_fp8(Fp8Args a) {
  __shared__ __attribute__((aligned(1024))) char ring[kQRing];
  __shared__ float s_wscale[2][kQMaxKB];
  __shared__ float amax_x[2][kQBM];
  __shared__ int32_t s_prefix[2 * kMaxE + 2];   // the tile prefix, searched once per tile
  __shared__ int s_tile;
  const int NT0 = a.p[0].N / kQBN, NT1 = a.p[1].N / kQBN;
  for (int i = threadIdx.x; i <= a.n_exp; i += blockDim.x) s_prefix[i] = a.tile_prefix[i];
  const int total = a.tile_prefix[a.n_exp];
  int range = 0;   // thread 0: XCD ranges this block has used up
  // thread 0 claims a block's next tile: the first here, each later one right after the k loop
  // of the tile before it (its atomic then overlaps that tile's epilogue)
  auto claim = [&]() {
    if (threadIdx.x == 0) s_tile = take_tile(a.counters, total, range);
  };
  claim();
  __syncthreads();
  for (;;) {
    const int L = __builtin_amdgcn_readfirstlane(s_tile);
    if (L < 0) return;
    int g, mt, nt;
    grouped_tile_coords(s_prefix, a.n_exp, a.E0, NT0, NT1, L, g, mt, nt);
    // (read from LDS, so the compiler cannot see they are uniform: keep them scalar)
    g = __builtin_amdgcn_readfirstlane(g);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const bool second = g >= a.E0;
    const Fp8Prob& p = second ? a.p[1] : a.p[0];
    const int e = __builtin_amdgcn_readfirstlane(second ? g - a.E0 : g);
    const int row0 = __builtin_amdgcn_readfirstlane(p.offsets[e] + mt * kQBM);
    const int row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
    // every wave reads s_tile before the k loop's first barrier, and thread 0 overwrites it
    // only after the k loop
    fp8_tile<MODE>(p, ring, s_wscale, amax_x, e, row0, row_end, __builtin_amdgcn_readfirstlane(nt * kQBN), claim);
    // every wave is done with the ring, the scale and amax arrays, and s_tile holds the next tile
    __syncthreads();
  }
}

}  // namespace
}  // namespace moeffn
