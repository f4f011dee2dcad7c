// moe_grouped_ffn: every selected expert's SwiGLU FFN over the rows grouped to it.
//
// "The Billion-Token Bottleneck" (section "The Geometry of the Problem") makes
// each expert a feed-forward network; "NovaLLM: Running Massive MoE Models
// Fully In-Memory" (section 3) runs only the experts that were hit. The expert
// weights are read through the slot table (pool + slot * stride), which is how
// the same kernels serve a fully resident layer and the expert slot pool.
//
// Kernels (one header per family):
//  ffn_common.h   bundle geometry, ffn_tile_map (per-expert m-tile counts -> prefix on the
//                 device, no host sync), the persistent tile queues, DMA helpers
//  gemm_bf16.h    ffn_gemm_bf16, the bf16 prefill tile engine (gate/up + SwiGLU, down)
//  gemm_fp8.h     ffn_gemm_fp8, the e4m3 prefill engine with fp32 block scales
//  gemm_mx.h      ffn_gemm_mx, MXFP4 weights x MXFP8 activations on the block-scaled MFMA
//  decode_bf16.h  ffn_decode_bf16, weight streaming for at most 64 rows per expert; one
//                 launch can carry two problems (routed experts and the shared expert)
//  decode_step.h  decode_step_front, the routing beside the shared expert's gate/up
//                 (moe_decode_step)
//  this file      ffn_f32_* (fp32 VALU path, one thread per output element) and the host
//                 side: argument checks, workspace layout, launches
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "decode_bf16.h"
#include "decode_step.h"
#include "ffn_common.h"
#include "gemm_bf16.h"
#include "gemm_fp8.h"
#include "gemm_mx.h"
#include "moe_internal.h"

namespace moeffn {
namespace {
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

// K splits of a decode down projection. With at most 4 rows (one or a few tokens: the
// routed experts touched are few, so their short workgroups end early) a down GEMM longer
// than 64 k-steps of 32 spreads each (expert, 32-column group) over workgroups of about 48
// k-steps (a shared expert's F is several routed experts' F), so its few long workgroups do
// not set the launch's length. The choice depends on the problem alone, so a problem gives
// the same bits alone or batched.
int decode_down_splits(const moe_expert_table* t, int rows) {
  if (t->w_dtype != MOE_BF16 || rows > 4) return 1;
  const int kt = t->d_ff / 32;
  return kt > 64 ? std::min(8, (kt + 47) / 48) : 1;
}

// Workspace: H [rows, F] (fp32, bf16 or e4m3), then the tile prefix and the per-XCD work
// counters of the persistent GEMMs, then (for a split decode down projection) the fp32
// partials [splits][rows][d] and the arrival counts. fp8 problems add the e4m3 H scales
// [F/128][rows + 256] and the activation scales [d/128][rows + 256] (both block-major in GEMM
// row order, as the fp8 GEMM reads them), and their map holds the gate/up and the down tile
// prefixes of up to two problems.
constexpr int kFp8MapInts = 2 * (2 * kMaxE + 2) + 16;

size_t ws_layout(const moe_expert_table* t, int rows, int act_dtype, size_t* h_off, size_t* map_off,
                 size_t* hs_off = nullptr, size_t* part_off = nullptr, size_t* arrived_off = nullptr,
                 size_t* as_off = nullptr) {
  const size_t hsz = act_dtype == MOE_F32 ? 4 : (act_dtype == MOE_FP8_E4M3 || act_dtype == MOE_MXFP8) ? 1 : 2;
  *h_off = 0;
  size_t end = align_up((size_t)rows * t->d_ff * hsz, 256);
  if (hs_off) *hs_off = end;
  if (act_dtype == MOE_FP8_E4M3) end += align_up((size_t)(rows + 256) * (t->d_ff / 128) * 4, 256);
  if (act_dtype == MOE_MXFP8) end += align_up((size_t)rows * (t->d_ff / 32), 256);   // H E8M0 bytes
  if (as_off) *as_off = end;
  if (act_dtype == MOE_FP8_E4M3) end += align_up((size_t)(rows + 256) * (t->d_model / 128) * 4, 256);
  *map_off = end;   // tile prefix [E+1], then the work counters [16]
  if (act_dtype == MOE_FP8_E4M3 || act_dtype == MOE_MXFP8) end = *map_off + align_up((size_t)kFp8MapInts * 4, 256);
  else end = *map_off + align_up((size_t)(t->n_experts + 2) * 4, 256) + 256;
  const int S = decode_down_splits(t, rows);
  if (part_off) *part_off = end;
  if (S > 1) end += align_up((size_t)S * rows * t->d_model * 4, 256);
  if (arrived_off) *arrived_off = end;
  if (S > 1) end += align_up((size_t)std::min(t->n_experts, rows) * (t->d_model / 32) * 4, 256);
  return end;
}

}  // namespace
}  // namespace moeffn

using namespace moeffn;

extern "C" size_t moe_bundle_bytes(int32_t d_model, int32_t d_ff, int32_t w_dtype) {
  if (d_model < 1 || d_ff < 1) return 0;
  if (w_dtype == MOE_BF16 && (d_model % 32 || d_ff % 32)) return 0;
  if ((w_dtype == MOE_FP8_E4M3 || w_dtype == MOE_MXFP4) && (d_model % 128 || d_ff % 128)) return 0;
  if (w_dtype == MOE_F32 && d_model % 4) return 0;
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16 && w_dtype != MOE_FP8_E4M3 && w_dtype != MOE_MXFP4) return 0;
  return (size_t)bundle_geom(d_model, d_ff, w_dtype).bytes;
}

extern "C" size_t moe_grouped_ffn_workspace_size(const moe_expert_table* table, int32_t rows, int32_t act_dtype) {
  if (!table || rows < 0) return 0;
  size_t h, m;
  return ws_layout(table, rows, act_dtype, &h, &m);
}

namespace moeffn {
namespace {

// One grouped FFN problem: the arguments of one moe_grouped_ffn call.
struct FfnCall {
  moe_expert_table t;
  int rows;
  const int32_t* offsets;
  const void* a;
  const float* a_scale;
  int act_dtype;
  const int32_t* a_row_src;
  int a_row_div;
  void* y;
  int y_dtype;
  char* ws;
  size_t ws_bytes;
};

// The argument checks of moe_grouped_ffn; an empty problem (rows == 0) needs no pointers.
moe_status check_call(const FfnCall& c, const char* who) {
  const moe_expert_table& t = c.t;
  const int rows = c.rows, act_dtype = c.act_dtype;
  MOE_REQUIRE(rows >= 0, MOE_EINVAL, "%s: rows=%d < 0", who, rows);
  MOE_REQUIRE(t.n_experts >= 1 && t.n_experts <= kMaxE, MOE_EINVAL, "%s: n_experts=%d outside [1, %d]", who,
              t.n_experts, kMaxE);
  const size_t bb = moe_bundle_bytes(t.d_model, t.d_ff, t.w_dtype);
  MOE_REQUIRE(bb > 0, MOE_EINVAL, "%s: unsupported sizes d=%d F=%d for w_dtype %d", who, t.d_model, t.d_ff, t.w_dtype);
  MOE_REQUIRE(t.slot_stride >= (int64_t)bb && t.slot_stride % 256 == 0, MOE_EINVAL,
              "%s: slot_stride %lld must be >= bundle bytes %zu and a multiple of 256", who, (long long)t.slot_stride,
              bb);
  MOE_REQUIRE(c.y_dtype == MOE_F32 || c.y_dtype == MOE_BF16, MOE_EUNSUPPORTED, "%s: y_dtype %d", who, c.y_dtype);
  if (c.a_row_src) MOE_REQUIRE(c.a_row_div >= 1, MOE_EINVAL, "%s: a_row_div must be >= 1", who);
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(t.pool && t.slot_of_expert && c.offsets && c.a && c.y && c.ws, MOE_EINVAL, "%s: NULL argument", who);
  MOE_REQUIRE(aligned(t.pool, 256) && aligned(c.a, 16) && aligned(c.y, 16) && aligned(c.ws, 256), MOE_EINVAL,
              "%s: pool needs 256-B, a and y 16-B, ws 256-B alignment", who);
  size_t h_off, map_off;
  const size_t need = ws_layout(&t, rows, act_dtype, &h_off, &map_off);
  MOE_REQUIRE(c.ws_bytes >= need, MOE_ECAPACITY, "%s: workspace %zu < %zu bytes", who, c.ws_bytes, need);
  const int d = t.d_model, F = t.d_ff;
  if (t.w_dtype == MOE_F32) {
    MOE_REQUIRE(act_dtype == MOE_F32, MOE_EUNSUPPORTED, "%s: fp32 weights need fp32 activations", who);
  } else if (t.w_dtype == MOE_MXFP4 && act_dtype == MOE_MXFP8) {
    // the block-scaled MFMA path (any rows per expert)
    MOE_REQUIRE(c.a_scale != nullptr, MOE_EINVAL, "%s: MXFP8 activations need their E8M0 bytes (a_scale)", who);
    MOE_REQUIRE((2 * F) % kQBN == 0 && d % kQBN == 0, MOE_EUNSUPPORTED,
                "%s: MXFP4 prefill tiles need d and 2F multiples of %d", who, kQBN);
    const long long a_rows = c.a_row_src ? (rows + c.a_row_div - 1) / c.a_row_div : rows;
    MOE_REQUIRE(std::max(a_rows * d, (long long)rows * F) < (1ll << 32) && (long long)F * d < (1ll << 32),
                MOE_EUNSUPPORTED, "%s: MXFP4 activations or weights larger than 4 GiB per matrix", who);
  } else if (t.w_dtype == MOE_MXFP4) {
    MOE_REQUIRE(act_dtype == MOE_BF16, MOE_EUNSUPPORTED, "%s: mxfp4 weights need bf16 or MXFP8 activations", who);
    const int max_rows_e = c.a_row_src ? (rows + c.a_row_div - 1) / c.a_row_div : rows;
    MOE_REQUIRE(max_rows_e <= 64, MOE_EUNSUPPORTED,
                "%s: mxfp4 weights with bf16 activations run on the decode kernels (at most 64 rows per expert, "
                "here up to %d; MXFP8 activations take the prefill path)", who, max_rows_e);
  } else if (t.w_dtype == MOE_BF16) {
    MOE_REQUIRE(act_dtype == MOE_BF16, MOE_EUNSUPPORTED, "%s: bf16 weights need bf16 activations", who);
    MOE_REQUIRE((2 * F) % kBN == 0 && d % kBN == 0, MOE_EUNSUPPORTED,
                "%s: bf16 prefill tiles need d and 2F multiples of %d", who, kBN);
  } else {
    MOE_REQUIRE(act_dtype == MOE_FP8_E4M3 && c.a_scale != nullptr, MOE_EUNSUPPORTED,
                "%s: fp8 weights need e4m3 activations and their scales", who);
    MOE_REQUIRE((2 * F) % kQBN == 0 && d % kQBN == 0 && d % 128 == 0 && F % 128 == 0, MOE_EUNSUPPORTED,
                "%s: fp8 tiles need d and 2F multiples of %d and F a multiple of 128", who, kQBN);
    MOE_REQUIRE(aligned(c.a_scale, 4), MOE_EINVAL, "%s: a_scale must be 4-byte aligned", who);
    MOE_REQUIRE(d / 128 <= kQMaxKB && F / 128 <= kQMaxKB, MOE_EUNSUPPORTED, "%s: fp8 tiles need d and F at most %d",
                who, 128 * kQMaxKB);
    // the fp8 GEMM addresses A rows and weight tiles with 32-bit offsets
    const long long a_rows = c.a_row_src ? (rows + c.a_row_div - 1) / c.a_row_div : rows;
    MOE_REQUIRE(std::max(a_rows * d, (long long)rows * F) < (1ll << 32) && 2ll * F * d < (1ll << 32), MOE_EUNSUPPORTED,
                "%s: fp8 activations or weights larger than 4 GiB per matrix", who);
  }
  return MOE_OK;
}

// bf16 and MXFP4 problems whose experts get at most 64 rows each take the weight-streaming
// decode kernels (MXFP4 only those). Rows per expert are bounded by the number of distinct source rows: at most
// rows / a_row_div tokens (each picks an expert once) or all rows.
bool decode_path(const FfnCall& c) {
  if ((c.t.w_dtype != MOE_BF16 && c.t.w_dtype != MOE_MXFP4) || c.act_dtype == MOE_MXFP8 || c.rows == 0) return false;
  const int max_rows_e = c.a_row_src ? (c.rows + c.a_row_div - 1) / c.a_row_div : c.rows;
  return max_rows_e <= 64;
}

// The decode kernels' arguments and block counts for one problem: gate/up + SwiGLU into
// H (in the problem's workspace), then down into y over S K splits.
// R > 1 gives each (expert, 32-row group) R workgroups of 16 rows each (see ffn_decode_bf16).
void decode_args(const FfnCall& c, int S, int R, DecodeArgs* gu, DecodeArgs* dn, int* nb_gu, int* nb_dn) {
  size_t h_off, map_off, hs_off, part_off, arrived_off;
  ws_layout(&c.t, c.rows, c.act_dtype, &h_off, &map_off, &hs_off, &part_off, &arrived_off);
  const BundleGeom g = bundle_geom(c.t.d_model, c.t.d_ff, c.t.w_dtype);
  bf16_t* H = reinterpret_cast<bf16_t*>(c.ws + h_off);
  const int E = c.t.n_experts, d = c.t.d_model, F = c.t.d_ff;
  const int max_active = E < c.rows ? E : c.rows;
  DecodeArgs q{};
  q.a = static_cast<const bf16_t*>(c.a);
  q.a_row_src = c.a_row_src;
  q.a_row_div = c.a_row_div;
  q.offsets = c.offsets;
  q.slot_of_expert = c.t.slot_of_expert;
  q.E = E;
  q.pool = static_cast<const char*>(c.t.pool);
  q.slot_stride = c.t.slot_stride;
  q.b_off = g.gu_off;
  q.s_off = g.sg_off;   // MXFP4 scales of W_gu (unused for bf16)
  q.N = 2 * F;
  q.K = d;
  q.out = H;
  q.out_dtype = MOE_BF16;
  q.rows = c.rows;
  q.splits = 1;
  q.rchunks = R;
  q.clear = S > 1 ? reinterpret_cast<int32_t*>(c.ws + arrived_off) : nullptr;
  q.clear_n = S > 1 ? max_active * (d / 32) : 0;
  *gu = q;
  // R > 1: the units padded to a multiple of 8, each with R workgroups
  auto blocks = [&](int units) { return R > 1 ? (units + 7) / 8 * 8 * R : units; };
  *nb_gu = blocks(max_active * (q.N / 32));
  q.a = H;
  q.a_row_src = nullptr;
  q.a_row_div = 1;
  q.b_off = g.dn_off;
  q.s_off = g.sd_off;
  q.N = d;
  q.K = F;
  q.out = c.y;
  q.out_dtype = c.y_dtype;
  q.splits = S;
  q.part = S > 1 ? reinterpret_cast<float*>(c.ws + part_off) : nullptr;
  q.arrived = S > 1 ? reinterpret_cast<int32_t*>(c.ws + arrived_off) : nullptr;
  q.clear = nullptr;
  q.clear_n = 0;
  *dn = q;
  *nb_dn = blocks(max_active * (q.N / 32) * S);
}

#ifndef MOEFFN_DEC_MB1_MAX_ROWS
#define MOEFFN_DEC_MB1_MAX_ROWS 64
#endif

// One or two decode problems in one gate/up launch and one down launch; the blocks of the
// first problem come first in dispatch order. With cb, the down launch also combines (the
// problems' y are then the fp32 buffers cb reads, and cb->arrived is cleared by the gate/up
// launch).
moe_status launch_decode(const FfnCall* calls, int n, hipStream_t s, const DecodeCombine* cb = nullptr) {
  DecodeArgs gu[2], dn[2];
  int ngu[2] = {0, 0}, ndn[2] = {0, 0};
  // One 16-row m-block per pass (71 VGPRs, so more workgroups fit on a CU) while no expert of
  // a routed problem can hold more than MOEFFN_DEC_MB1_MAX_ROWS rows; a one-expert problem (a
  // shared expert) with more than 16 rows then takes one workgroup per 16 rows. Else 4 m-blocks
  // per pass (112 VGPRs; a 2-block pass at the 6-wave cap spills and measured slower).
  int max_rows_e = 0;
  bool split = false;
  for (int i = 0; i < n; ++i) {
    const FfnCall& c = calls[i];
    if (c.t.n_experts > 1) max_rows_e = std::max(max_rows_e, c.a_row_src ? (c.rows + c.a_row_div - 1) / c.a_row_div : c.rows);
    split |= decode_down_splits(&c.t, c.rows) > 1;
  }
  const bool mb1 = split || max_rows_e <= MOEFFN_DEC_MB1_MAX_ROWS;
  for (int i = 0; i < n; ++i) {
    const FfnCall& c = calls[i];
    const int R = (mb1 && c.t.n_experts == 1 && c.rows > 16) ? (c.rows + 15) / 16 : 1;
    decode_args(c, decode_down_splits(&c.t, c.rows), R, &gu[i], &dn[i], &ngu[i], &ndn[i]);
  }
  if (cb != nullptr) {
    gu[0].clear2 = cb->arrived;
    gu[0].clear2_n = cb->d / 32;
  }
  const DecodeCombine no_cb{};
  if (n == 1) {
    gu[1] = gu[0];
    dn[1] = dn[0];
  }
  const dim3 block(64 * kDecWaves);
  auto go = [&](auto sp, auto mb, auto wf) {
    constexpr bool SP = decltype(sp)::value;
    constexpr int MB = decltype(mb)::value;
    constexpr int WF = decltype(wf)::value;
    prof_mark(s, MOE_PROF_DEC_GATEUP, false);
    hipLaunchKernelGGL((ffn_decode_bf16<MODE_GATEUP, SP, MB, false, WF>), dim3(ngu[0] + ngu[1]), block, 0, s,
                       gu[0], gu[1], ngu[0], no_cb);
    prof_mark(s, MOE_PROF_DEC_GATEUP, true);
    prof_mark(s, MOE_PROF_DEC_DOWN, false);
    if (cb != nullptr)
      hipLaunchKernelGGL((ffn_decode_bf16<MODE_DOWN, SP, MB, true, WF>), dim3(ndn[0] + ndn[1]), block, 0, s, dn[0],
                         dn[1], ndn[0], *cb);
    else
      hipLaunchKernelGGL((ffn_decode_bf16<MODE_DOWN, SP, MB, false, WF>), dim3(ndn[0] + ndn[1]), block, 0, s,
                         dn[0], dn[1], ndn[0], no_cb);
    prof_mark(s, MOE_PROF_DEC_DOWN, true);
  };
  using T1 = std::true_type;
  using F0 = std::false_type;
  using M1 = std::integral_constant<int, 1>;
  using M4 = std::integral_constant<int, 4>;
  using BF = std::integral_constant<int, 0>;
  using FP4 = std::integral_constant<int, 1>;
  if (calls[0].t.w_dtype == MOE_MXFP4) {   // (the callers launch only same-format problems together)
    if (mb1) go(F0{}, M1{}, FP4{});
    else go(F0{}, M4{}, FP4{});
  } else if (split) {   // at most 4 rows
    go(T1{}, M1{}, BF{});
  } else if (mb1) {
    go(F0{}, M1{}, BF{});
  } else {
    go(F0{}, M4{}, BF{});
  }
  return check_launch("moe_grouped_ffn bf16 decode");
}

// One or two checked fp8 problems (the routed experts, then a shared expert) in one gate/up
// launch and one down launch: the activation scales are laid out block-major in GEMM row
// order, one tile map covers both problems (in the first problem's workspace), and the
// persistent GEMMs take the tiles of both from the same queues.
moe_status run_fp8(const FfnCall* c, int n, hipStream_t s) {
  Fp8Args gu{}, dn{};
  int32_t *prefix_gu = nullptr, *prefix_dn = nullptr, *counters = nullptr;
  long long bound_gu = 0, bound_dn = 0;
  for (int i = 0; i < n; ++i) {
    const FfnCall& q = c[i];
    const moe_expert_table& t = q.t;
    size_t h_off, map_off, hs_off, as_off;
    ws_layout(&t, q.rows, q.act_dtype, &h_off, &map_off, &hs_off, nullptr, nullptr, &as_off);
    const BundleGeom g = bundle_geom(t.d_model, t.d_ff, t.w_dtype);
    const int d = t.d_model, F = t.d_ff, ld = q.rows + 256;
    float* As = reinterpret_cast<float*>(q.ws + as_off);
    float* Hs = reinterpret_cast<float*>(q.ws + hs_off);
    uint8_t* Hq = reinterpret_cast<uint8_t*>(q.ws + h_off);
    if (i == 0) {
      prefix_gu = reinterpret_cast<int32_t*>(q.ws + map_off);
      prefix_dn = prefix_gu + 2 * kMaxE + 2;
      counters = prefix_dn + 2 * kMaxE + 2;
    }
    const long long n_as = (long long)(d / 128) * ld;
    hipLaunchKernelGGL(fp8_scales_kb_major, dim3((unsigned)((n_as + 255) / 256)), dim3(256), 0, s, q.a_scale,
                       q.a_row_src, q.a_row_div, q.rows, d / 128, ld, As);
    Fp8Prob& a = gu.p[i];
    a.a = static_cast<const uint8_t*>(q.a);
    a.a_scale_t = As;
    a.a_scale_ld = ld;
    a.a_row_src = q.a_row_src;
    a.a_row_div = q.a_row_div;
    a.offsets = q.offsets;
    a.slot_of_expert = t.slot_of_expert;
    a.pool = static_cast<const char*>(t.pool);
    a.slot_stride = t.slot_stride;
    a.b_off = g.gu_off;
    a.s_off0 = g.sg_off;
    a.s_off1 = g.su_off;
    a.E = t.n_experts;
    a.N = 2 * F;
    a.K = d;
    a.out = Hq;
    a.out_scale_t = Hs;
    a.out_scale_ld = ld;
    a.out_dtype = MOE_FP8_E4M3;
    Fp8Prob& b = dn.p[i];
    b = a;
    b.a = Hq;
    b.a_scale_t = Hs;
    b.a_row_src = nullptr;
    b.a_row_div = 1;
    b.b_off = g.dn_off;
    b.s_off0 = g.sd_off;
    b.s_off1 = 0;
    b.N = d;
    b.K = F;
    b.out = q.y;
    b.out_scale_t = nullptr;
    b.out_scale_ld = 0;
    b.out_dtype = q.y_dtype;
    // at most rows / 256 + min(E, rows) m-tiles
    const long long mt = q.rows / kQBM + std::min<long long>(t.n_experts, q.rows);
    bound_gu += mt * (2 * F / kQBN);
    bound_dn += mt * (d / kQBN);
  }
  gu.E0 = dn.E0 = c[0].t.n_experts;
  gu.n_exp = dn.n_exp = c[0].t.n_experts + (n > 1 ? c[1].t.n_experts : 0);
  if (n == 1) gu.p[1] = gu.p[0], dn.p[1] = dn.p[0];
  TileMapArgs m{};
  for (int i = 0; i < 2; ++i) {
    m.offsets[i] = gu.p[i].offsets;
    m.slot_of_expert[i] = gu.p[i].slot_of_expert;
    m.nt_gu[i] = gu.p[i].N / kQBN;
    m.nt_dn[i] = dn.p[i].N / kQBN;
  }
  m.E0 = gu.E0;
  m.n_exp = gu.n_exp;
  hipLaunchKernelGGL(grouped_tile_map, dim3(1), dim3(1024), 0, s, m, prefix_gu, prefix_dn, counters, 16);
  gu.tile_prefix = prefix_gu;
  gu.counters = counters;
  dn.tile_prefix = prefix_dn;
  dn.counters = counters + 8;
  const long long n_cu = cu_count();
  // persistent: at most one block per CU, a multiple of 8 (one per XCD in turn)
  long long nblk = std::min(bound_gu, n_cu);
  prof_mark(s, MOE_PROF_GATEUP, false);
  hipLaunchKernelGGL(ffn_gemm_fp8<MODE_GATEUP>, dim3((unsigned)((nblk + 7) / 8 * 8)), dim3(512), 0, s, gu);
  prof_mark(s, MOE_PROF_GATEUP, true);
  nblk = std::min(bound_dn, n_cu);
  prof_mark(s, MOE_PROF_DOWN, false);
  hipLaunchKernelGGL(ffn_gemm_fp8<MODE_DOWN>, dim3((unsigned)((nblk + 7) / 8 * 8)), dim3(512), 0, s, dn);
  prof_mark(s, MOE_PROF_DOWN, true);
  return check_launch("moe_grouped_ffn fp8");
}

// One or two checked MXFP4 problems with MXFP8 activations in one gate/up launch and one down
// launch of the block-scaled MFMA GEMM (tile map in the first problem's workspace).
moe_status run_mx(const FfnCall* c, int n, hipStream_t s) {
  MxArgs gu{}, dn{};
  int32_t *prefix_gu = nullptr, *prefix_dn = nullptr, *counters = nullptr;
  long long bound_gu = 0, bound_dn = 0;
  for (int i = 0; i < n; ++i) {
    const FfnCall& q = c[i];
    const moe_expert_table& t = q.t;
    size_t h_off, map_off, hs_off;
    ws_layout(&t, q.rows, q.act_dtype, &h_off, &map_off, &hs_off);
    const BundleGeom g = bundle_geom(t.d_model, t.d_ff, t.w_dtype);
    const int d = t.d_model, F = t.d_ff;
    uint8_t* Hq = reinterpret_cast<uint8_t*>(q.ws + h_off);
    uint8_t* He = reinterpret_cast<uint8_t*>(q.ws + hs_off);
    if (i == 0) {
      prefix_gu = reinterpret_cast<int32_t*>(q.ws + map_off);
      prefix_dn = prefix_gu + 2 * kMaxE + 2;
      counters = prefix_dn + 2 * kMaxE + 2;
    }
    MxProb& a = gu.p[i];
    a.a = static_cast<const uint8_t*>(q.a);
    a.a_exp = reinterpret_cast<const uint8_t*>(q.a_scale);
    a.a_row_src = q.a_row_src;
    a.a_row_div = q.a_row_div;
    a.offsets = q.offsets;
    a.slot_of_expert = t.slot_of_expert;
    a.pool = static_cast<const char*>(t.pool);
    a.slot_stride = t.slot_stride;
    a.b_off = g.gu_off;
    a.bs_off = g.sg_off;
    a.E = t.n_experts;
    a.N = 2 * F;
    a.K = d;
    a.out = Hq;
    a.out_exp = He;
    a.out_dtype = MOE_MXFP8;
    MxProb& b = dn.p[i];
    b = a;
    b.a = Hq;
    b.a_exp = He;
    b.a_row_src = nullptr;
    b.a_row_div = 1;
    b.b_off = g.dn_off;
    b.bs_off = g.sd_off;
    b.N = d;
    b.K = F;
    b.out = q.y;
    b.out_exp = nullptr;
    b.out_dtype = q.y_dtype;
    const long long mt = q.rows / kQBM + std::min<long long>(t.n_experts, q.rows);
    bound_gu += mt * (2 * F / kQBN);
    bound_dn += mt * (d / kQBN);
  }
  gu.E0 = dn.E0 = c[0].t.n_experts;
  gu.n_exp = dn.n_exp = c[0].t.n_experts + (n > 1 ? c[1].t.n_experts : 0);
  if (n == 1) gu.p[1] = gu.p[0], dn.p[1] = dn.p[0];
  TileMapArgs m{};
  for (int i = 0; i < 2; ++i) {
    m.offsets[i] = gu.p[i].offsets;
    m.slot_of_expert[i] = gu.p[i].slot_of_expert;
    m.nt_gu[i] = gu.p[i].N / kQBN;
    m.nt_dn[i] = dn.p[i].N / kQBN;
  }
  m.E0 = gu.E0;
  m.n_exp = gu.n_exp;
  hipLaunchKernelGGL(grouped_tile_map, dim3(1), dim3(1024), 0, s, m, prefix_gu, prefix_dn, counters, 16);
  gu.tile_prefix = prefix_gu;
  gu.counters = counters;
  dn.tile_prefix = prefix_dn;
  dn.counters = counters + 8;
  const long long n_cu = cu_count();
  long long nblk = std::min(bound_gu, n_cu);
  prof_mark(s, MOE_PROF_GATEUP, false);
  hipLaunchKernelGGL(ffn_gemm_mx<MODE_GATEUP>, dim3((unsigned)((nblk + 7) / 8 * 8)), dim3(512), 0, s, gu);
  prof_mark(s, MOE_PROF_GATEUP, true);
  nblk = std::min(bound_dn, n_cu);
  prof_mark(s, MOE_PROF_DOWN, false);
  hipLaunchKernelGGL(ffn_gemm_mx<MODE_DOWN>, dim3((unsigned)((nblk + 7) / 8 * 8)), dim3(512), 0, s, dn);
  prof_mark(s, MOE_PROF_DOWN, true);
  return check_launch("moe_grouped_ffn mxfp4");
}

// Runs one checked problem on stream s.
moe_status run_call(const FfnCall& c, hipStream_t s) {
  if (c.rows == 0) return MOE_OK;
  const moe_expert_table& t = c.t;
  const int rows = c.rows, act_dtype = c.act_dtype, y_dtype = c.y_dtype, a_row_div = c.a_row_div;
  const int32_t* offsets = c.offsets;
  const int32_t* a_row_src = c.a_row_src;
  const void* a = c.a;
  const float* a_scale = c.a_scale;
  void* y = c.y;
  size_t h_off, map_off;
  ws_layout(&t, rows, act_dtype, &h_off, &map_off);
  const BundleGeom g = bundle_geom(t.d_model, t.d_ff, t.w_dtype);
  char* wsb = c.ws;
  const int E = t.n_experts, d = t.d_model, F = t.d_ff;

  if (t.w_dtype == MOE_F32) {
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
  if (t.w_dtype == MOE_MXFP4 && act_dtype == MOE_MXFP8) return run_mx(&c, 1, s);
  if (t.w_dtype == MOE_MXFP4) return launch_decode(&c, 1, s);   // (check_call admits decode problems only)
  if (t.w_dtype == MOE_BF16) {
    int32_t* tile_prefix = reinterpret_cast<int32_t*>(wsb + map_off);
    bf16_t* H = reinterpret_cast<bf16_t*>(wsb + h_off);
    if (decode_path(c)) return launch_decode(&c, 1, s);
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
  return run_fp8(&c, 1, s);
}



}  // namespace
}  // namespace moeffn

using namespace moeffn;

extern "C" moe_status moe_grouped_ffn(const moe_expert_table* table, int32_t rows, const int32_t* offsets,
                                      const void* a, const float* a_scale, int32_t act_dtype,
                                      const int32_t* a_row_src, int32_t a_row_div, void* y, int32_t y_dtype,
                                      void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  MOE_REQUIRE(table != nullptr, MOE_EINVAL, "moe_grouped_ffn: table is NULL");
  const FfnCall c{*table, rows, offsets, a, a_scale, act_dtype, a_row_src, a_row_div, y, y_dtype,
                  static_cast<char*>(ws), ws_bytes};
  if (moe_status st = check_call(c, "moe_grouped_ffn")) return st;
  return run_call(c, as_stream(stream));
}

extern "C" size_t moe_grouped_ffn_batch_workspace_size(const moe_ffn_problem* problems, int32_t n) {
  if (!problems || n < 1 || n > 2) return 0;
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (!problems[i].table || problems[i].rows < 0) return 0;
    size_t h, m;
    total += align_up(ws_layout(problems[i].table, problems[i].rows, problems[i].act_dtype, &h, &m), 256);
  }
  return total;
}

extern "C" moe_status moe_grouped_ffn_batch(const moe_ffn_problem* problems, int32_t n, void* ws, size_t ws_bytes,
                                            void* stream) {
  clear_error();
  MOE_REQUIRE(problems != nullptr && n >= 1 && n <= 2, MOE_EINVAL, "moe_grouped_ffn_batch: n=%d outside [1, 2]", n);
  FfnCall c[2];
  size_t off = 0;
  bool any_rows = false;
  for (int i = 0; i < n; ++i) {
    const moe_ffn_problem& q = problems[i];
    MOE_REQUIRE(q.table != nullptr, MOE_EINVAL, "moe_grouped_ffn_batch: problem %d has no table", i);
    MOE_REQUIRE(q.rows >= 0, MOE_EINVAL, "moe_grouped_ffn_batch: problem %d rows=%d < 0", i, q.rows);
    size_t h, m;
    const size_t need = ws_layout(q.table, q.rows, q.act_dtype, &h, &m);
    c[i] = FfnCall{*q.table, q.rows, q.offsets, q.a, q.a_scale, q.act_dtype, q.a_row_src, q.a_row_div, q.y,
                   q.y_dtype, ws ? static_cast<char*>(ws) + off : nullptr, need};
    off += align_up(need, 256);
    any_rows |= q.rows > 0;
  }
  if (any_rows) {
    MOE_REQUIRE(ws != nullptr, MOE_EINVAL, "moe_grouped_ffn_batch: NULL workspace");
    MOE_REQUIRE(ws_bytes >= off, MOE_ECAPACITY, "moe_grouped_ffn_batch: workspace %zu < %zu bytes", ws_bytes, off);
  }
  for (int i = 0; i < n; ++i)
    if (moe_status st = check_call(c[i], "moe_grouped_ffn_batch")) return st;
  hipStream_t s = as_stream(stream);
  if (n == 2 && decode_path(c[0]) && decode_path(c[1]) && c[0].t.w_dtype == c[1].t.w_dtype)
    return launch_decode(c, 2, s);
  if (n == 2 && c[0].t.w_dtype == MOE_FP8_E4M3 && c[1].t.w_dtype == MOE_FP8_E4M3 && c[0].rows > 0 && c[1].rows > 0 &&
      c[0].t.d_model == c[1].t.d_model)
    return run_fp8(c, 2, s);   // both problems in one launch per GEMM
  if (n == 2 && c[0].t.w_dtype == MOE_MXFP4 && c[1].t.w_dtype == MOE_MXFP4 && c[0].act_dtype == MOE_MXFP8 &&
      c[1].act_dtype == MOE_MXFP8 && c[0].rows > 0 && c[1].rows > 0 && c[0].t.d_model == c[1].t.d_model)
    return run_mx(c, 2, s);
  for (int i = 0; i < n; ++i)
    if (moe_status st = run_call(c[i], s)) return st;
  return MOE_OK;
}

// The fused decode FFN + combine: the problems as in moe_grouped_ffn_batch (shared first),
// the expert outputs in fp32 buffers after the batch workspace, then the combine's group
// arrival counts.
namespace moeffn {
namespace {
struct FusedLayout {
  size_t batch, y_routed, y_shared, arrived, total;
};
FusedLayout fused_layout(const moe_ffn_problem* routed, const moe_ffn_problem* shared) {
  FusedLayout L{};
  size_t h, m;
  if (shared) L.batch += align_up(ws_layout(shared->table, shared->rows, shared->act_dtype, &h, &m), 256);
  L.batch += align_up(ws_layout(routed->table, routed->rows, routed->act_dtype, &h, &m), 256);
  const size_t d = routed->table->d_model;
  L.y_routed = L.batch;
  L.y_shared = L.y_routed + align_up((size_t)routed->rows * d * 4, 256);
  L.arrived = L.y_shared + (shared ? align_up((size_t)shared->rows * d * 4, 256) : 0);
  L.total = L.arrived + align_up(d / 32 * 4, 256);
  return L;
}
}  // namespace
}  // namespace moeffn

extern "C" size_t moe_grouped_ffn_combine_workspace_size(const moe_ffn_problem* routed,
                                                          const moe_ffn_problem* shared) {
  if (!routed || !routed->table || routed->rows < 0) return 0;
  if (shared && (!shared->table || shared->rows < 0 || shared->table->d_model != routed->table->d_model)) return 0;
  return fused_layout(routed, shared).total;
}

extern "C" moe_status moe_grouped_ffn_combine(const moe_ffn_problem* routed, const moe_ffn_problem* shared,
                                              const moe_combine_args* comb, void* ws, size_t ws_bytes,
                                              void* stream) {
  clear_error();
  MOE_REQUIRE(routed != nullptr && routed->table != nullptr && comb != nullptr, MOE_EINVAL,
              "moe_grouped_ffn_combine: routed problem, its table and comb must not be NULL");
  MOE_REQUIRE(!shared || shared->table != nullptr, MOE_EINVAL, "moe_grouped_ffn_combine: shared problem has no table");
  const int T = comb->T, k = comb->k, d = routed->table->d_model;
  MOE_REQUIRE(T >= 0 && k >= 1 && k <= 32, MOE_EINVAL, "moe_grouped_ffn_combine: need T >= 0 and 1 <= k <= 32 (T=%d k=%d)",
              T, k);
  MOE_REQUIRE(T <= 64, MOE_EUNSUPPORTED, "moe_grouped_ffn_combine: T=%d > 64 (decode batches only)", T);
  MOE_REQUIRE(routed->rows == T * k, MOE_EINVAL, "moe_grouped_ffn_combine: routed rows %d != T*k = %d", routed->rows,
              T * k);
  if (shared) {
    MOE_REQUIRE(shared->rows == T, MOE_EINVAL, "moe_grouped_ffn_combine: shared rows %d != T = %d", shared->rows, T);
    MOE_REQUIRE(shared->table->d_model == d, MOE_EINVAL, "moe_grouped_ffn_combine: shared d_model %d != %d",
                shared->table->d_model, d);
  }
  MOE_REQUIRE(comb->out_dtype == MOE_F32 || comb->out_dtype == MOE_BF16, MOE_EUNSUPPORTED,
              "moe_grouped_ffn_combine: out_dtype %d", comb->out_dtype);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(comb->perm_dst && comb->topk_gate && comb->out && ws, MOE_EINVAL,
              "moe_grouped_ffn_combine: NULL perm_dst, topk_gate, out or workspace");
  MOE_REQUIRE(aligned(comb->out, 16) && aligned(ws, 256), MOE_EINVAL,
              "moe_grouped_ffn_combine: out needs 16-B and ws 256-B alignment");
  const FusedLayout L = fused_layout(routed, shared);
  MOE_REQUIRE(ws_bytes >= L.total, MOE_ECAPACITY, "moe_grouped_ffn_combine: workspace %zu < %zu bytes", ws_bytes,
              L.total);
  char* w = static_cast<char*>(ws);
  float* y_routed = reinterpret_cast<float*>(w + L.y_routed);
  float* y_shared = shared ? reinterpret_cast<float*>(w + L.y_shared) : nullptr;
  FfnCall c[2];
  int n = 0;
  size_t off = 0;
  size_t h, m;
  for (const moe_ffn_problem* q : {shared, routed}) {
    if (!q) continue;
    const size_t need = ws_layout(q->table, q->rows, q->act_dtype, &h, &m);
    c[n] = FfnCall{*q->table, q->rows, q->offsets, q->a, q->a_scale, q->act_dtype, q->a_row_src, q->a_row_div,
                   q == routed ? (void*)y_routed : (void*)y_shared, q->y_dtype, w + off, need};
    off += align_up(need, 256);
    if (moe_status st = check_call(c[n], "moe_grouped_ffn_combine")) return st;
    MOE_REQUIRE(decode_path(c[n]), MOE_EUNSUPPORTED,
                "moe_grouped_ffn_combine: the %s problem is not a decode problem (bf16 weights, at most 64 rows per "
                "expert)", q == routed ? "routed" : "shared");
    ++n;
  }
  MOE_REQUIRE(n == 1 || c[0].t.w_dtype == c[1].t.w_dtype, MOE_EUNSUPPORTED,
              "moe_grouped_ffn_combine: the shared and routed experts must have the same weight format");
  DecodeCombine cb{};
  cb.T = T;
  cb.k = k;
  cb.d = d;
  cb.perm_dst = comb->perm_dst;
  cb.gate = comb->topk_gate;
  cb.shared_gate = shared ? comb->shared_gate : nullptr;
  cb.y_routed = y_routed;
  cb.y_shared = y_shared;
  cb.out = comb->out;
  cb.out_dtype = comb->out_dtype;
  cb.arrived = reinterpret_cast<int32_t*>(w + L.arrived);
  cb.nprob = n;
  return launch_decode(c, n, as_stream(stream), &cb);
}

// ---------------------------------------------------------------- decode step --
// A resident layer's whole decode step in three launches (four past kStepFoldMaxT tokens):
//  1. decode_step_front: routing (logits split over K, then selection and grouping by the
//     last workgroups to finish) beside the shared expert's gate/up units;
//  2. the shared expert's down units beside the routed experts' gate/up units
//     (ffn_decode_down_gateup), or the routed gate/up alone without a shared expert;
//  3. the routed experts' down units, with the combine folded in up to kStepFoldMaxT tokens,
//     else followed by moe_combine.
// Every piece runs the same arithmetic as moe_route_permute, moe_grouped_ffn_batch and
// moe_combine (or moe_grouped_ffn_combine), so the results are bit-identical to those calls.
namespace moeffn {
namespace {

// Largest step whose combine runs inside the routed down launch. Each workgroup that
// finishes a unit then waits for its stores and an arrival count before it exits; that pays
// off only while the down launch is about one round of workgroups (1-4 tokens: MI355X,
// Qwen1.5-MoE shape, 0.056 vs 0.058 ms per step at one token, 0.1185 vs 0.1175 ms at eight).
#ifndef MOEFFN_STEP_FOLD_MAX_T
#define MOEFFN_STEP_FOLD_MAX_T 4
#endif
constexpr int kStepFoldMaxT = MOEFFN_STEP_FOLD_MAX_T;

struct StepLayout {
  size_t part, idx, ws_shared, ws_routed, y_routed, y_shared, comb_arrived, total;
};

// Workspace: the routing's arrival counters in bytes [0, 256), the partial logits, the
// published selection, the shared and the routed problem's moe_grouped_ffn workspaces, the
// expert outputs (fp32 room), the combine's arrival counts.
StepLayout step_layout(const moe_route_cfg& c, const moe_expert_table* routed, const moe_expert_table* shared) {
  StepLayout L{};
  const int T = c.T, k = c.top_k, d = c.d_model;
  size_t h, m;
  L.part = 256;
  L.idx = L.part + align_up((size_t)route_slices(d) * T * (c.n_experts + 1) * 4, 256);
  L.ws_shared = L.idx + align_up((size_t)T * k * 4, 256);
  L.ws_routed = L.ws_shared + (shared ? align_up(ws_layout(shared, T, MOE_BF16, &h, &m), 256) : 0);
  L.y_routed = L.ws_routed + align_up(ws_layout(routed, T * k, MOE_BF16, &h, &m), 256);
  L.y_shared = L.y_routed + align_up((size_t)T * k * d * 4, 256);
  L.comb_arrived = L.y_shared + (shared ? align_up((size_t)T * d * 4, 256) : 0);
  L.total = L.comb_arrived + align_up((size_t)(d / 32) * 4, 256);
  return L;
}

}  // namespace
}  // namespace moeffn

extern "C" size_t moe_decode_step_workspace_size(const moe_route_cfg* cfg, const moe_expert_table* routed,
                                                 const moe_expert_table* shared) {
  if (!cfg || !routed || cfg->T < 1 || cfg->T > kStepMaxT || cfg->top_k < 1 || cfg->n_experts < 1 ||
      cfg->d_model < 32 || cfg->d_model % 32)
    return 0;
  if (shared && shared->d_model != routed->d_model) return 0;
  return step_layout(*cfg, routed, shared).total;
}

extern "C" moe_status moe_decode_step(const moe_route_cfg* cfg, const void* x, const void* w_router,
                                      const float* logit_bias, const float* select_bias, const void* w_shared_gate,
                                      const moe_expert_table* routed, const moe_expert_table* shared,
                                      const moe_decode_out* o, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  MOE_REQUIRE(cfg != nullptr && routed != nullptr && o != nullptr, MOE_EINVAL,
              "moe_decode_step: cfg, the routed table and the outputs must not be NULL");
  const moe_route_cfg& c = *cfg;
  if (moe_status st = check_route_config(c, "moe_decode_step")) return st;
  const int T = c.T, k = c.top_k, E = c.n_experts, d = c.d_model;
  MOE_REQUIRE(T >= 1 && T <= kStepMaxT, MOE_EUNSUPPORTED, "moe_decode_step: T=%d outside [1, %d] (decode steps only)",
              T, kStepMaxT);
  MOE_REQUIRE(c.act_dtype == MOE_BF16 && d % 32 == 0 && E <= kStepMaxE, MOE_EUNSUPPORTED,
              "moe_decode_step: needs bf16 activations, d_model a multiple of 32 and at most %d experts", kStepMaxE);
  MOE_REQUIRE(routed->n_experts == E && routed->d_model == d, MOE_EINVAL,
              "moe_decode_step: the routed table has E=%d d=%d, the routing E=%d d=%d", routed->n_experts,
              routed->d_model, E, d);
  MOE_REQUIRE(routed->w_dtype == MOE_BF16 || routed->w_dtype == MOE_MXFP4, MOE_EUNSUPPORTED,
              "moe_decode_step: weights must be bf16 or MXFP4 (w_dtype %d)", routed->w_dtype);
  if (shared) {
    MOE_REQUIRE(shared->n_experts == 1 && shared->d_model == d && shared->w_dtype == routed->w_dtype, MOE_EINVAL,
                "moe_decode_step: the shared table must hold one expert of the routed experts' d_model and format");
  }
  MOE_REQUIRE(!(select_bias && c.score_fn == MOE_SOFTMAX), MOE_EINVAL, "moe_decode_step: select_bias needs sigmoid scoring");
  MOE_REQUIRE((w_shared_gate == nullptr) == (o->shared_gate == nullptr), MOE_EINVAL,
              "moe_decode_step: w_shared_gate and shared_gate go together");
  MOE_REQUIRE(x && w_router && o->scores && o->topk_idx && o->topk_gate && o->offsets && o->perm_src && o->perm_dst &&
                  o->out && ws,
              MOE_EINVAL, "moe_decode_step: NULL tensor argument");
  MOE_REQUIRE(aligned(x, 16) && aligned(w_router, 16) && (!w_shared_gate || aligned(w_shared_gate, 16)) &&
                  aligned(o->out, 16) && aligned(ws, 256),
              MOE_EINVAL, "moe_decode_step: x, w_router, w_shared_gate and out need 16-B, ws 256-B alignment");
  MOE_REQUIRE(o->out_dtype == MOE_F32 || o->out_dtype == MOE_BF16, MOE_EUNSUPPORTED, "moe_decode_step: out_dtype %d",
              o->out_dtype);
  const StepLayout L = step_layout(c, routed, shared);
  MOE_REQUIRE(ws_bytes >= L.total, MOE_ECAPACITY, "moe_decode_step: workspace %zu < %zu bytes", ws_bytes, L.total);
  char* w = static_cast<char*>(ws);
  const bool fold = T <= kStepFoldMaxT;
  size_t h, m;
  // the two problems, checked as moe_grouped_ffn calls (the shared one is given the routed
  // offsets only to pass the pointer check: its decode arguments drop them, see below)
  FfnCall rc{*routed, T * k, o->offsets, x, nullptr, MOE_BF16, o->perm_src, k, w + L.y_routed, MOE_BF16,
             w + L.ws_routed, ws_layout(routed, T * k, MOE_BF16, &h, &m)};
  if (moe_status st = check_call(rc, "moe_decode_step (routed)")) return st;
  MOE_REQUIRE(decode_path(rc), MOE_EUNSUPPORTED, "moe_decode_step: the routed problem is not a decode problem");
  DecodeArgs gu_r, dn_r, gu_s{}, dn_s{};
  int ngu_r = 0, ndn_r = 0, ngu_s = 0, ndn_s = 0;
  decode_args(rc, decode_down_splits(routed, T * k), 1, &gu_r, &dn_r, &ngu_r, &ndn_r);
  const int S_r = decode_down_splits(routed, T * k);
  int S_s = 1;
  if (shared) {
    FfnCall sc{*shared, T, o->offsets, x, nullptr, MOE_BF16, nullptr, 1, w + L.y_shared, MOE_BF16, w + L.ws_shared,
               ws_layout(shared, T, MOE_BF16, &h, &m)};
    if (moe_status st = check_call(sc, "moe_decode_step (shared)")) return st;
    S_s = decode_down_splits(shared, T);
    decode_args(sc, S_s, T > 16 ? (T + 15) / 16 : 1, &gu_s, &dn_s, &ngu_s, &ndn_s);
    gu_s.offsets = dn_s.offsets = nullptr;   // one group over rows [0, T)
  }
  DecodeCombine cb{};
  if (fold) {
    cb.T = T;
    cb.k = k;
    cb.d = d;
    cb.perm_dst = o->perm_dst;
    cb.gate = o->topk_gate;
    cb.shared_gate = shared ? o->shared_gate : nullptr;
    cb.y_routed = reinterpret_cast<const float*>(w + L.y_routed);
    cb.y_shared = shared ? reinterpret_cast<const float*>(w + L.y_shared) : nullptr;
    cb.out = o->out;
    cb.out_dtype = o->out_dtype;
    cb.arrived = reinterpret_cast<int32_t*>(w + L.comb_arrived);
    cb.nprob = 1;
    gu_r.clear2 = cb.arrived;
    gu_r.clear2_n = d / 32;
  }
  // routing: m-tiles of 16 tokens, each with its (n-tile, slice) items over bpm workgroups
  StepRoute r{};
  r.x = static_cast<const bf16_t*>(x);
  r.w_router = static_cast<const bf16_t*>(w_router);
  r.w_sg = static_cast<const bf16_t*>(w_shared_gate);
  r.logit_bias = logit_bias;
  r.select_bias = select_bias;
  r.part = reinterpret_cast<float*>(w + L.part);
  r.idx_stage = reinterpret_cast<int32_t*>(w + L.idx);
  r.arrive = reinterpret_cast<int32_t*>(w);
  r.shared_gate = o->shared_gate;
  r.scores = o->scores;
  r.topk_idx = o->topk_idx;
  r.topk_gate = o->topk_gate;
  r.counts = o->counts;
  r.offsets = o->offsets;
  r.perm_src = o->perm_src;
  r.perm_dst = o->perm_dst;
  r.T = T;
  r.d = d;
  r.E = E;
  r.ncols = E + (w_shared_gate ? 1 : 0);
  r.nsl = route_slices(d);
  r.n_nt = (r.ncols + 15) / 16;
  r.n_mt = (T + 15) / 16;
  r.bpm = (r.n_nt * r.nsl + kDecWaves - 1) / kDecWaves;
  r.k = k;
  r.score_fn = c.score_fn;
  r.renormalize = c.renormalize;
  r.route_scale = c.route_scale;
  r.n_groups = c.n_groups < 1 ? 1 : c.n_groups;
  r.topk_groups = c.topk_groups;
  r.group_topn = c.group_topn;
  const int nb_route = (r.n_mt * r.bpm + 7) / 8 * 8;
  hipStream_t s = as_stream(stream);
  const dim3 block(64 * kDecWaves);
  const DecodeCombine no_cb{};
  auto go = [&](auto pl, auto km, auto wf) {
    constexpr int PL = decltype(pl)::value, KM = decltype(km)::value, WF = decltype(wf)::value;
    hipLaunchKernelGGL((decode_step_front<PL, KM, WF>), dim3(nb_route + ngu_s), block, 0, s, r, nb_route, gu_s);
    prof_mark(s, MOE_PROF_DEC_GATEUP, false);
    if (shared) {
      auto k2 = [&](auto sp, auto yf) {
        constexpr bool SP = decltype(sp)::value, YF = decltype(yf)::value;
        hipLaunchKernelGGL((ffn_decode_down_gateup<SP, YF, WF>), dim3(ndn_s + ngu_r), block, 0, s, dn_s, gu_r, ndn_s);
      };
      if (S_s > 1) {
        if (fold) k2(std::true_type{}, std::true_type{});
        else k2(std::true_type{}, std::false_type{});
      } else {
        if (fold) k2(std::false_type{}, std::true_type{});
        else k2(std::false_type{}, std::false_type{});
      }
    } else {
      hipLaunchKernelGGL((ffn_decode_bf16<MODE_GATEUP, false, 1, false, WF>), dim3(ngu_r), block, 0, s, gu_r, gu_r,
                         ngu_r, no_cb);
    }
    prof_mark(s, MOE_PROF_DEC_GATEUP, true);
    prof_mark(s, MOE_PROF_DEC_DOWN, false);
    auto k3 = [&](auto sp) {
      constexpr bool SP = decltype(sp)::value;
      if (fold)
        hipLaunchKernelGGL((ffn_decode_bf16<MODE_DOWN, SP, 1, true, WF>), dim3(ndn_r), block, 0, s, dn_r, dn_r, ndn_r,
                           cb);
      else
        hipLaunchKernelGGL((ffn_decode_bf16<MODE_DOWN, SP, 1, false, WF>), dim3(ndn_r), block, 0, s, dn_r, dn_r,
                           ndn_r, no_cb);
    };
    if (S_r > 1) k3(std::true_type{});
    else k3(std::false_type{});
    prof_mark(s, MOE_PROF_DEC_DOWN, true);
  };
  auto by_wf = [&](auto pl, auto km) {
    if (routed->w_dtype == MOE_MXFP4) go(pl, km, std::integral_constant<int, 1>{});
    else go(pl, km, std::integral_constant<int, 0>{});
  };
  auto by_k = [&](auto pl) {
    if (k <= 8) by_wf(pl, std::integral_constant<int, 8>{});
    else by_wf(pl, std::integral_constant<int, 32>{});
  };
  if (E <= 64) by_k(std::integral_constant<int, 1>{});
  else if (E <= 128) by_k(std::integral_constant<int, 2>{});
  else by_k(std::integral_constant<int, 4>{});
  if (moe_status st = check_launch("moe_decode_step")) return st;
  if (fold) return MOE_OK;
  return moe_combine(T, k, d, w + L.y_routed, MOE_BF16, o->perm_dst, o->topk_gate, shared ? w + L.y_shared : nullptr,
                     shared ? o->shared_gate : nullptr, o->out, o->out_dtype, stream);
}

// ------------------------------------------------------- no-allocation variant --
// moe_grouped_ffn_combine for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the workspace is a
// file-scope device array of MOE_NOALLOC_SCRATCH_BYTES, one copy per GPU the library runs on,
// held until the process ends. In host code `scratch` names a host-side stand-in, not device
// memory; its device address on each GPU comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is passed to the kernels. The kernels of a
// call clear the arrival counts they use (the gate/up launch zeroes them for the down launch),
// so nothing has to start at zero between calls; calls that overlap on one GPU share the array
// and race.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moeffn {
namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

moe_status scratch_address(void** out) {
  int dev = -1;
  MOE_HIP(hipGetDevice(&dev));
  MOE_REQUIRE(dev >= 0 && dev < 64, MOE_EUNSUPPORTED, "moe_grouped_ffn_combine_noalloc: device %d outside [0, 64)",
              dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    MOE_REQUIRE(p != nullptr && aligned(p, 256), MOE_EHIP,
                "moe_grouped_ffn_combine_noalloc: no 256-B aligned device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace
}  // namespace moeffn

extern "C" moe_status moe_grouped_ffn_combine_noalloc(const moe_ffn_problem* routed, const moe_ffn_problem* shared,
                                                      const moe_combine_args* comb, void* stream) {
  clear_error();
  MOE_REQUIRE(routed != nullptr && routed->table != nullptr && comb != nullptr, MOE_EINVAL,
              "moe_grouped_ffn_combine_noalloc: routed problem, its table and comb must not be NULL");
  const size_t need = moe_grouped_ffn_combine_workspace_size(routed, shared);
  MOE_REQUIRE(need > 0, MOE_EINVAL, "moe_grouped_ffn_combine_noalloc: invalid problems (no workspace size)");
  MOE_REQUIRE(need <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_ECAPACITY,
              "moe_grouped_ffn_combine_noalloc: the step needs %zu bytes of scratch, more than the %zu this entry "
              "point holds per device (use moe_grouped_ffn_combine with a workspace)",
              need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (moe_status st = scratch_address(&ws)) return st;
  return moe_grouped_ffn_combine(routed, shared, comb, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
