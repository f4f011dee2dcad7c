// Stable expert-major grouping of at most 64 tokens inside one workgroup of NW wavefronts.
//
// The grouping lets each selected expert run once over all of its rows ("NovaLLM:
// Running Massive MoE Models Fully In-Memory", section 3: only the experts that were
// hit run); rows of one expert are ordered by ascending token. Every wavefront holds
// all tokens (lane = token) and takes experts w, w + NW, ...: a ballot per expert gives
// its count, a workgroup-wide scan over the experts gives the offsets, and a second
// ballot per expert ranks each (token, slot) pair among the expert's tokens.
//
// Used by moe_permute for one block of tokens and by the fused small-batch routing
// kernel (1024 threads, NW = 16), and by the fused decode step (512 threads, NW = 8); all
// need T <= 64 and E <= 64 * NW.
#pragma once

#include "moe_internal.h"

namespace moeffn {

// idx [T, k] (device or LDS, written before the call and visible to the workgroup); counts
// may be NULL. off is LDS scratch of E ints, wave_sum LDS scratch of NW ints.
template <int KMAX, int NW = 16>
__device__ __forceinline__ void group_small(const int32_t* __restrict__ idx, int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
                                            int32_t* __restrict__ perm_dst, int T, int k, int E, int32_t* off,
                                            int32_t* wave_sum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mine[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) mine[j] = (lane < T && j < k) ? idx[(size_t)lane * k + j] : -1;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = wave; e < E; e += NW) {
    bool has = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) has |= (mine[j] == e);
    const uint64_t m = __ballot(has);
    if (lane == 0) {
      off[e] = __popcll(m);
      if (counts) counts[e] = __popcll(m);
    }
  }
  __syncthreads();
  // exclusive scan of the counts over the experts (thread e holds expert e)
  const int c = tid < E ? off[tid] : 0;
  int inc = c;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  if (lane == 63) wave_sum[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_sum[w];
  const int excl = before + inc - c;
  __syncthreads();   // every count has been read before it is overwritten
  if (tid < E) {
    off[tid] = excl;
    offsets[tid] = excl;
  }
  if (tid == E - 1) offsets[E] = excl + c;
  __syncthreads();
  for (int e = wave; e < E; e += NW) {
    int slot = -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (mine[j] == e) slot = j;
    const uint64_t m = __ballot(slot >= 0);
    if (slot >= 0) {
      const int pos = off[e] + __popcll(m & below);
      perm_src[pos] = lane * k + slot;
      perm_dst[lane * k + slot] = pos;
    }
  }
}

}  // namespace moeffn
