// The first launch of a fused decode step (moe_decode_step): the router logits split over K
// beside the shared expert's gate/up projection, which needs no routing, so the shared
// expert's weights stream while the routing runs instead of after it ("NovaLLM: Running
// Massive MoE Models Fully In-Memory", section 3, Optimization #3: fewer launches and less
// idle time per decode step).
//
// Workgroups [0, nb_route) route. The slice items of m-tile mt (16 tokens) are spread over
// bpm workgroups, one wave per (n-tile, slice) item; each stores its partial logits at device
// scope, waits for the stores, and counts itself on the m-tile's arrival counter. The last to
// arrive adds the m-tile's slices in slice order and selects its tokens (select_token, one
// wavefront per token), exactly as the two-launch routing does. With more than one m-tile,
// each selecting workgroup publishes its tokens' expert lists at device scope and counts
// itself once more; the last groups every token (group_small). Each last arriver sets its
// counter back to zero, so the counters are zero again when the launch ends.
// The remaining workgroups run the shared expert's gate/up units (decode_block).
#pragma once

#include "decode_bf16.h"
#include "group_small.h"
#include "route_small.h"

namespace moeffn {
namespace {

constexpr int kStepMaxT = 64;    // tokens of a decode step
constexpr int kStepMaxE = 256;   // routed experts (the selection keeps 4 keys per lane)
constexpr int kStepMaxK = 32;

struct StepRoute {
  const bf16_t* x;
  const bf16_t* w_router;
  const bf16_t* w_sg;          // NULL without a shared gate
  const float* logit_bias;
  const float* select_bias;
  float* part;                 // [nsl][T][ncols] partial logits
  int32_t* idx_stage;          // [T * k] the selection, for the grouping workgroup (n_mt > 1)
  int32_t* arrive;             // [n_mt + 1] zero when the launch starts, zero again when it ends
  float* shared_gate;
  float* scores;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_src;
  int32_t* perm_dst;
  int T, d, E, ncols, nsl, n_nt, n_mt, bpm, k;
  int score_fn, renormalize;
  float route_scale;
  int n_groups, topk_groups, group_topn;
};

struct StepRouteLds {
  float lg[16 * (kStepMaxE + 1)];        // one m-tile's summed logits, [t][ncols]
  float wkeys[kDecWaves][kStepMaxE];
  int32_t off[kStepMaxE];
  int32_t wave_sum[kDecWaves];
  int32_t idx[kStepMaxT * kStepMaxK];    // the selection at [t * k + j]
  int s_last;
};

template <int PL, int KM>
__device__ __forceinline__ void step_route_block(const StepRoute& r, int b, StepRouteLds& L) {
  const int wave = threadIdx.x >> 6;
  const int mt = b / r.bpm, local = b - mt * r.bpm;
  const int item = local * kDecWaves + wave;
  if (item < r.n_nt * r.nsl) {
    const int nt = item / r.nsl, sl = item - nt * r.nsl;
    route_slice_wave<true>(r.x, r.w_router, r.w_sg, r.part, r.T, r.d, r.E, r.ncols, sl, 16 * nt, 16 * mt);
  }
  // every wave's partials have reached the coherent level before the workgroup is counted
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    L.s_last = atomicAdd(&r.arrive[mt], 1) == r.bpm - 1;
    if (L.s_last) __hip_atomic_store(&r.arrive[mt], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!L.s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // no load moves above the count
  const int t0 = 16 * mt, nt = min(16, r.T - t0);
  route_sum_slices<true>(r.part, r.nsl, r.T * r.ncols, t0 * r.ncols, (t0 + nt) * r.ncols, L.lg, r.scores,
                         r.shared_gate, r.E, r.ncols);
  __syncthreads();
  for (int t = wave; t < nt; t += kDecWaves)
    select_token<PL>(t0 + t, L.lg + t * r.ncols, r.scores, r.logit_bias, r.select_bias, r.shared_gate, r.topk_idx,
                     r.topk_gate, nullptr, L.wkeys[wave], r.E, r.k, r.score_fn, r.renormalize, r.route_scale,
                     r.n_groups, r.topk_groups, r.group_topn, L.idx);
  __syncthreads();
  if (r.n_mt > 1) {
    // publish this m-tile's selection, then the last m-tile to get here groups every token
    for (int i = threadIdx.x; i < nt * r.k; i += blockDim.x)
      __hip_atomic_store(&r.idx_stage[t0 * r.k + i], L.idx[t0 * r.k + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0) {
      L.s_last = atomicAdd(&r.arrive[r.n_mt], 1) == r.n_mt - 1;
      if (L.s_last) __hip_atomic_store(&r.arrive[r.n_mt], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!L.s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    for (int i = threadIdx.x; i < r.T * r.k; i += blockDim.x)
      L.idx[i] = __hip_atomic_load(&r.idx_stage[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  group_small<KM, kDecWaves>(L.idx, r.counts, r.offsets, r.perm_src, r.perm_dst, r.T, r.k, r.E, L.off, L.wave_sum);
}

// Workgroups [0, nb_route) route (those past the last m-tile's do nothing: nb_route is
// rounded up to a multiple of 8 so the shared expert's units keep their XCD placement), the
// rest run the shared expert's gate/up units (gu), when there is a shared expert.
template <int PL, int KM, int WF>
__global__ __launch_bounds__(64 * kDecWaves, WF == 1 ? kDecMxWavesPerSimd : MOEFFN_DEC_MINBLOCKS) void decode_step_front(StepRoute r, int nb_route,
                                                                                        DecodeArgs gu) {
  __shared__ union {
    StepRouteLds route;
    DecodeLds<1> ffn;
  } L;
  const int b = (int)blockIdx.x;
  if (b >= nb_route) {
    const DecodeCombine no_cb{};
    decode_block<MODE_GATEUP, false, 1, false, false, WF>(gu, b - nb_route, gu, gu, no_cb, L.ffn);
    return;
  }
  if (b < r.n_mt * r.bpm) step_route_block<PL, KM>(r, b, L.route);
}

}  // namespace
}  // namespace moeffn
