// Pieces shared by the grouped FFN kernels: the bundle geometry written by moe_pack_expert, the
// device-side tile map, the persistent-GEMM argument block and tile queues, and the
// wait helper of the direct-to-LDS rings (the loads themselves are in lds_dma.h).
#pragma once

#include <algorithm>

#include "lds_dma.h"
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
  } else if (dt == MOE_MXFP4) {
    // codes (two per byte) then E8M0 scales (one per 32 inputs of a row), per matrix
    g.gu_off = 0;
    g.sg_off = al((int64_t)2 * F * d / 2);
    g.dn_off = g.sg_off + al((int64_t)2 * F * (d / 32));
    g.sd_off = g.dn_off + al((int64_t)d * F / 2);
    g.bytes = g.sd_off + al((int64_t)d * (F / 32));
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


}  // namespace
}  // namespace moeffn
