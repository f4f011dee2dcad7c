// Routing pieces shared by the routing kernels (route.hip) and the fused decode step
// (decode_step.h): the orderable (key, index) encoding and wave-wide reductions, the
// selection of one token by one wavefront, and the logits of a small batch split over K
// into slices that many workgroups compute at once.
//
// The pages leave the router arithmetic open ("The Billion-Token Bottleneck", section
// "The Geometry of the Problem": a router decides which few experts handle each token);
// the reading implemented is the one moe.h states for moe_route.
#pragma once

#include "moe_internal.h"

namespace moeffn {

// The routing configuration checks of moe_route (MOE_OK or the error, recorded for who);
// defined in route.hip.
moe_status check_route_config(const moe_route_cfg& c, const char* who);

namespace {

// -------------------------------------------------------------- select ---
// Orderable encoding: larger (key, then lower index) -> larger word; 0 = none.
__device__ __forceinline__ uint64_t pack_key(float key, int idx) {
  if (key == 0.0f) key = 0.0f;  // -0 and +0 tie
  uint32_t u = __float_as_uint(key);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int unpack_idx(uint64_t w) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(w & 0xFFFFFFFFu));
}

// The 64-bit value of the lane that the DPP control CTRL names (a permutation inside each row
// of 16 lanes; every lane of the wavefront active).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Largest value over the wavefront, in every lane (called with every lane active). Inside each
// row of 16 lanes four DPP steps (swap neighbours, swap pairs, mirror halves of 8, mirror the
// row) leave the row's largest value in all its lanes; the four rows' values are then read
// into scalar registers. (Register moves between lanes, where a butterfly of shuffles would
// take an LDS permute per 32-bit half and step.)
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v = o > v ? o : v;
  o = dpp_u64<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v = o > v ? o : v;
  o = dpp_u64<0x141>(v);   // row_half_mirror
  v = o > v ? o : v;
  o = dpp_u64<0x140>(v);   // row_mirror
  v = o > v ? o : v;
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
    const uint64_t x = ((uint64_t)hi << 32) | lo;
    m = x > m ? x : m;
  }
  return m;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Selection for token t by one wavefront: keys, the group limit, k rounds of a wave-wide
// arg-max, the gates, and the sigmoid of the shared gate's logit. Reads the token's raw
// logits from src_row (scores' row t, or a copy in LDS) and writes its keys to scores; wk is
// LDS scratch of E floats owned by this wavefront; hist (LDS, may be NULL) counts the
// selected experts; idx_copy (LDS, may be NULL) receives the selection at [t * k + j].
template <int PER_LANE>
__device__ __forceinline__ void select_token(
    int t, const float* src_row, float* __restrict__ scores, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias,
    float* __restrict__ shared_gate, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, int* hist,
    float* wk, int E, int k, int score_fn, int renormalize, float route_scale, int n_groups, int topk_groups,
    int group_topn, int32_t* idx_copy = nullptr) {
  const int lane = threadIdx.x & 63;
  const int gsz = n_groups > 0 ? E / n_groups : E;
  float logit[PER_LANE], key[PER_LANE];
  bool live[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    live[i] = e < E;
    float l = 0.f;
    if (live[i]) {
      l = src_row[e];
      if (logit_bias) l += logit_bias[e];
    }
    logit[i] = l;
    float kv = l;
    if (score_fn == MOE_SIGMOID) {
      const float s = 1.0f / (1.0f + expf(-l));
      logit[i] = s;  // for sigmoid routing keep s for the gates
      kv = s;
      if (select_bias && live[i]) kv = s + select_bias[e];
    }
    key[i] = kv;
    if (live[i]) scores[(size_t)t * E + e] = kv;
  }

  // group limit: lanes g < n_groups score their group from the keys in LDS
  if (n_groups > 1 && topk_groups < n_groups) {
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (live[i]) wk[lane + 64 * i] = key[i];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint64_t gword = 0;
    if (lane < n_groups) {
      // the group's group_topn largest keys, summed largest first in fp32
      float top[8];
      const int nt = min(group_topn, 8);
      for (int i = 0; i < nt; ++i) top[i] = -INFINITY;
      for (int m = 0; m < gsz; ++m) {
        float v = wk[lane * gsz + m];
        for (int i = 0; i < nt; ++i) {
          if (v > top[i]) { float tmp = top[i]; top[i] = v; v = tmp; }
        }
      }
      float sum = top[0];
      for (int i = 1; i < nt; ++i) sum = sum + top[i];
      gword = pack_key(sum, lane);
    }
    uint64_t keep_mask = 0;
    for (int r = 0; r < topk_groups; ++r) {
      const uint64_t best = wave_max_u64(gword);
      const int g = unpack_idx(best);
      keep_mask |= 1ull << g;
      if (lane == g) gword = 0;
    }
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      if (live[i] && !((keep_mask >> (e / gsz)) & 1ull)) live[i] = false;
    }
    __builtin_amdgcn_wave_barrier();
  }

  // top-k: k rounds of a wave-wide arg-max
  int sel_idx = 0;
  float sel_val = 0.f;  // logit (softmax) or s (sigmoid) of the lane-th winner
  for (int r = 0; r < k; ++r) {
    uint64_t mine = 0;
    int mine_i = -1;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      if (live[i]) {
        const uint64_t w = pack_key(key[i], lane + 64 * i);
        if (w > mine) { mine = w; mine_i = i; }
      }
    }
    const uint64_t best = wave_max_u64(mine);
    const int e = unpack_idx(best);
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      if (lane + 64 * i == e) { live[i] = false; v = logit[i]; }
    }
    // broadcast the winner's value from its owner lane
    const int owner = e & 63;
    v = __shfl(v, owner, 64);
    if (lane == r) { sel_idx = e; sel_val = v; }
    (void)mine_i;
  }

  // gates (lanes r < k hold winner r)
  float g = 0.f;
  if (score_fn == MOE_SOFTMAX) {
    const float m = __shfl(sel_val, 0, 64);  // the best key is the largest selected logit
    if (renormalize) {
      const float z = lane < k ? expf(sel_val - m) : 0.f;
      const float denom = wave_sum_f32(z);
      g = z / denom;
    } else {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i)
        if (lane + 64 * i < E) part += expf(logit[i] - m);
      const float denom = wave_sum_f32(part);
      g = lane < k ? expf(sel_val - m) / denom : 0.f;
    }
  } else {
    const float s = lane < k ? sel_val : 0.f;
    if (renormalize) g = s / wave_sum_f32(s);
    else g = s;
  }
  g *= route_scale;
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = sel_idx;
    if (idx_copy) idx_copy[t * k + lane] = sel_idx;   // (LDS) for a grouping in the same workgroup
    topk_gate[(size_t)t * k + lane] = g;
    if (hist) atomicAdd(&hist[sel_idx], 1);
  }
  if (shared_gate && lane == 0) {
    const float l = shared_gate[t];
    shared_gate[t] = 1.0f / (1.0f + expf(-l));
  }
}

// ------------------------------------------------- logits split over K ---
// A decode step routes at most 64 tokens. One workgroup could hold all of their logits, but
// a single CU pulls the router weights from HBM slowly, so the logits are split over K into
// slices of kSliceSteps k-steps of 32: one wave per (slice, n-tile of 16 columns, m-tile of
// 16 tokens), every load of the slice issued at once. A logit is then the sum of its slices
// in slice order, whichever kernel adds them, so every path gives the same bits.
constexpr int kSliceSteps = 4;

inline int route_slices(int d) { return (d / 32 + kSliceSteps - 1) / kSliceSteps; }

// One wave's slice item: columns c0..c0+15 (column c < E reads w_router row c, c == E the
// shared gate's weights), tokens t0..t0+15, k-steps of slice sl. Output part[sl][t][c] fp32
// for t < T, c < ncols; COHERENT stores at device scope (written through to the coherent
// level) for a reader in the same launch on another XCD.
template <bool COHERENT>
__device__ __forceinline__ void route_slice_wave(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w_router,
                                                 const bf16_t* __restrict__ w_sg, float* __restrict__ part, int T,
                                                 int d, int E, int ncols, int sl, int c0, int t0) {
  const int lane = threadIdx.x & 63;
  const int KT = d / 32;
  const int k0 = sl * kSliceSteps, nk = min(KT - k0, kSliceSteps);
  const int koff = 8 * (lane >> 4);
  const int c = min(c0 + (lane & 15), ncols - 1);
  const bf16_t* brow = (c < E ? w_router + (size_t)c * d : w_sg) + koff + k0 * 32;
  const bf16_t* arow = x + (size_t)min(t0 + (lane & 15), T - 1) * d + koff + k0 * 32;
  bf16x8_t b[kSliceSteps], a[kSliceSteps];
#pragma unroll
  for (int j = 0; j < kSliceSteps; ++j) {
    if (j < nk) {
      b[j] = *reinterpret_cast<const bf16x8_t*>(brow + j * 32);
      a[j] = *reinterpret_cast<const bf16x8_t*>(arow + j * 32);
    }
  }
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kSliceSteps; ++j)
    if (j < nk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[j], acc, 0, 0, 0);
  // D layout: lane l holds rows 4*(l/16)+i, column l%16
  const int col = c0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * (lane >> 4) + i;
    if (t < T && col < ncols) {
      float* o = part + ((size_t)sl * T + t) * ncols + col;
      if constexpr (COHERENT) __hip_atomic_store(o, acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *o = acc[i];
    }
  }
}

// Logits j in [j0, j1) of the [T][ncols] array (n = T * ncols) as the sums of their nsl
// slices in slice order, by the whole workgroup: into lg[j - j0], the routed ones into
// scores[t][c] and the shared gate's into shared_gate[t] (its raw logit, which select_token
// turns into the gate). A thread takes up to 2 logits at a time and issues 16 slices of each
// (32 loads; 16 slices cover d = 2048) before the first add. COHERENT loads at device scope
// read partials stored by other workgroups of the same launch.
template <bool COHERENT>
__device__ __forceinline__ void route_sum_slices(const float* __restrict__ part, int nsl, int n, int j0, int j1,
                                                 float* lg, float* __restrict__ scores,
                                                 float* __restrict__ shared_gate, int E, int ncols) {
  constexpr int kE = 2, kS = 16;
  for (int jb = j0 + (int)threadIdx.x; jb < j1; jb += kE * (int)blockDim.x) {
    float v[kE];
    for (int s0 = 0; s0 < nsl; s0 += kS) {
      float buf[kE][kS];
#pragma unroll
      for (int u = 0; u < kE; ++u) {
        const int j = jb + u * (int)blockDim.x;
#pragma unroll
        for (int q = 0; q < kS; ++q)
          if (j < j1 && s0 + q < nsl) {
            const float* src = part + (size_t)(s0 + q) * n + j;
            if constexpr (COHERENT) buf[u][q] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else buf[u][q] = *src;
          }
      }
#pragma unroll
      for (int u = 0; u < kE; ++u)
#pragma unroll
        for (int q = 0; q < kS; ++q)
          if (s0 + q < nsl) v[u] = (s0 + q == 0) ? buf[u][q] : v[u] + buf[u][q];
    }
#pragma unroll
    for (int u = 0; u < kE; ++u) {
      const int j = jb + u * (int)blockDim.x;
      if (j >= j1) continue;
      lg[j - j0] = v[u];
      const int t = j / ncols, c = j - t * ncols;
      if (c < E) scores[(size_t)t * E + c] = v[u];
      else shared_gate[t] = v[u];
    }
  }
}

}  // namespace
}  // namespace moeffn
