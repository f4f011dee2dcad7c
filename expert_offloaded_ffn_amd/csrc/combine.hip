// moe_combine: gate-weighted sum of each token's expert rows back in token
// order, plus the always-resident shared expert ("Running 35B MoE Models on 8GB
// GPUs", section "Gotcha": shared experts sit outside the routed, cached set).
//
// One wavefront per (token, 512-column chunk); each lane owns 8 consecutive columns, reads
// the k expert rows through perm_dst with 16-byte (bf16) or 32-byte (fp32) loads, eight rows'
// loads in flight at once, accumulates in fp32 in slot order j = 0..k-1, adds the shared
// term last and rounds once.
#include <type_traits>

#include "moe_internal.h"

namespace moeffn {
namespace {

// Eight consecutive values of a row: the raw 16 (bf16) or 32 (fp32) bytes, loaded first and
// converted later, so several rows' loads can be in flight at once.
template <typename TY>
struct Raw8;
template <>
struct Raw8<bf16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float v[8]) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void get(float v[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// KMAX bounds k (8 or 32), so the token's rows and gates stay in registers; the rows of a
// column chunk are loaded 8 at a time before the first add (the adds keep slot order).
template <typename TY, typename TO, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const TY* __restrict__ y, const int32_t* __restrict__ perm_dst,
                                                      const float* __restrict__ gate, const TY* __restrict__ shared_y,
                                                      const float* __restrict__ shared_gate, TO* __restrict__ out,
                                                      int T, int k, int d, int span) {
  // one wavefront per (token, span of 512-column chunks)
  const int nchunk = (d + 511) / 512;
  const int groups = (nchunk + span - 1) / span;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = item / groups, gi = item - t * groups;
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int rows[KMAX];
  float g[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      rows[j] = perm_dst[(size_t)t * k + j];
      g[j] = gate[(size_t)t * k + j];
    }
  }
  const float sg = shared_y ? (shared_gate ? shared_gate[t] : 1.0f) : 0.0f;
  const int c_end = min(d, (gi + 1) * span * 512);
  for (int c = gi * span * 512 + lane * 8; c < c_end; c += 512) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j0 = 0; j0 < KMAX; j0 += 8) {
      if (j0 < k) {
        Raw8<TY> raw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (j0 + u < k) raw[u].load(y + (size_t)rows[j0 + u] * d + c);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (j0 + u < k) {
            float v[8];
            raw[u].get(v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j0 + u], v[i], acc[i]);
          }
        }
      }
    }
    if (shared_y) {
      Raw8<TY> raw;
      raw.load(shared_y + (size_t)t * d + c);
      float v[8];
      raw.get(v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(sg, v[i], acc[i]);
    }
    if constexpr (sizeof(TO) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = f32x2_to_bf16x2(acc[2 * i], acc[2 * i + 1]);
      *reinterpret_cast<uint4*>(out + (size_t)t * d + c) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      *reinterpret_cast<float4*>(out + (size_t)t * d + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(out + (size_t)t * d + c + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// 512-column chunks per wavefront for large batches. One: many short wavefronts leave no
// partly filled last round (DeepSeek-V3 shape, 8,192 tokens x 7,168 columns, k = 8: 223 us,
// against 230 / 234 / 243 us for 2 / 4 / 14 chunks, and 263 us with the rows loaded one at a time).
#ifndef MOEFFN_COMBINE_SPAN
#define MOEFFN_COMBINE_SPAN 1
#endif
constexpr int kCombineSpan = MOEFFN_COMBINE_SPAN;

}  // namespace
}  // namespace moeffn

using namespace moeffn;

extern "C" moe_status moe_combine(int32_t T, int32_t k, int32_t d, const void* y, int32_t y_dtype,
                                  const int32_t* perm_dst, const float* topk_gate, const void* shared_y,
                                  const float* shared_gate, void* out, int32_t out_dtype, void* stream) {
  clear_error();
  MOE_REQUIRE(T >= 0 && k >= 1 && k <= 32 && d >= 8 && d % 8 == 0, MOE_EINVAL,
              "moe_combine: need T >= 0, 1 <= k <= 32, d a positive multiple of 8 (T=%d k=%d d=%d)", T, k, d);
  MOE_REQUIRE(y_dtype == MOE_F32 || y_dtype == MOE_BF16, MOE_EUNSUPPORTED, "moe_combine: y_dtype %d", y_dtype);
  MOE_REQUIRE(out_dtype == MOE_F32 || out_dtype == MOE_BF16, MOE_EUNSUPPORTED, "moe_combine: out_dtype %d", out_dtype);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(y && perm_dst && topk_gate && out, MOE_EINVAL, "moe_combine: NULL argument");
  MOE_REQUIRE(aligned(y, 16) && aligned(out, 16) && (!shared_y || aligned(shared_y, 16)), MOE_EINVAL,
              "moe_combine: y, shared_y and out must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  const int nchunk = (d + 511) / 512;
  const int span = T >= 512 ? min(nchunk, kCombineSpan) : 1;
  const long long items = (long long)T * ((nchunk + span - 1) / span);
  dim3 grid((unsigned)((items + 3) / 4)), block(256);
  auto go = [&](auto km) {
    constexpr int KM = decltype(km)::value;
    if (y_dtype == MOE_BF16 && out_dtype == MOE_BF16)
      hipLaunchKernelGGL((combine_kernel<bf16_t, bf16_t, KM>), grid, block, 0, s, (const bf16_t*)y, perm_dst,
                         topk_gate, (const bf16_t*)shared_y, shared_gate, (bf16_t*)out, T, k, d, span);
    else if (y_dtype == MOE_BF16)
      hipLaunchKernelGGL((combine_kernel<bf16_t, float, KM>), grid, block, 0, s, (const bf16_t*)y, perm_dst,
                         topk_gate, (const bf16_t*)shared_y, shared_gate, (float*)out, T, k, d, span);
    else if (out_dtype == MOE_BF16)
      hipLaunchKernelGGL((combine_kernel<float, bf16_t, KM>), grid, block, 0, s, (const float*)y, perm_dst, topk_gate,
                         (const float*)shared_y, shared_gate, (bf16_t*)out, T, k, d, span);
    else
      hipLaunchKernelGGL((combine_kernel<float, float, KM>), grid, block, 0, s, (const float*)y, perm_dst, topk_gate,
                         (const float*)shared_y, shared_gate, (float*)out, T, k, d, span);
  };
  if (k <= 8) go(std::integral_constant<int, 8>{});
  else go(std::integral_constant<int, 32>{});
  return check_launch("moe_combine");
}
