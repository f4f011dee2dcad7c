// Internal helpers shared by the library's translation units: status/error
// reporting, argument checks, element conversions and MFMA vector types.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "moe.h"  // include/ is on the include path

namespace moeffn {

// ---------------------------------------------------------------- errors --
void set_error(const char* fmt, ...);
void clear_error();

#define MOE_REQUIRE(cond, code, ...)            \
  do {                                          \
    if (!(cond)) {                              \
      ::moeffn::set_error(__VA_ARGS__);         \
      return (code);                            \
    }                                           \
  } while (0)

#define MOE_HIP(call)                                                              \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      ::moeffn::set_error("%s failed: %s", #call, hipGetErrorString(e_));          \
      return MOE_EHIP;                                                             \
    }                                                                              \
  } while (0)

// Any error left by earlier asynchronous work (or a failed launch) becomes MOE_EHIP.
moe_status check_launch(const char* what);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Timing marks around heavy kernels (no-op unless moe_profile_enable(1)).
void prof_mark(hipStream_t s, int kind, bool end);

// ----------------------------------------------------------- conversions --
typedef unsigned short bf16_t;  // bf16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN, its payload is not kept). The gfx950
// conversion instruction the compiler emits for the cast gave, on the MI355X, the same bits
// as the rounding written out in integer arithmetic (add 0x7FFF plus the kept lsb, drop 16
// bits) on every finite input tried: each exponent with tie, below-tie and above-tie low
// halves, subnormals, the largest values and 16 M random values.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  const __bf16 h = static_cast<__bf16>(f);
  bf16_t b;
  __builtin_memcpy(&b, &h, sizeof(b));
  return b;
}
// The same rounding in integer arithmetic (add 0x7FFF plus the kept lsb, drop 16 bits), for
// the bf16 GEMM: with the conversion instruction there, its down projection compiled to a main
// loop that ran 2.3% slower (Mixtral shape, same box), though the loop has no conversion.
__device__ __forceinline__ bf16_t f32_to_bf16_int(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}
// Two values -> two bf16 in one 32-bit word (a in the low half), one packed conversion.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 h2_t;
  const h2_t h = __builtin_convertvector(f2_t{a, b}, h2_t);
  uint32_t w;
  __builtin_memcpy(&w, &h, sizeof(w));
  return w;
}

// fp32 -> OCP e4m3 code (bias 7, max 448), round to nearest even; |v| <= 448 (callers
// clamp). Subnormals (below 2^-6) are multiples of 2^-9; normals keep 3 mantissa bits. The
// gfx950 packed conversion does exactly this: on the MI355X it gave the same byte as the
// rounding written out in integer arithmetic for every code, every midpoint between codes
// and its neighbours, both zeros, the subnormal edges and 16 M random values in range.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float v) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false)) & 0xFFu;
}
// Four clamped values -> their e4m3 codes in bytes 0..3 (two packed conversions).
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// MFMA operand/accumulator vectors.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

// silu(g) = g * sigmoid(g). Precise: IEEE division (fp32 paths). Fast: hardware exp and
// reciprocal (about 1 ulp each), used where the result is rounded to bf16 or e4m3 anyway.
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Largest v over each row of 16 lanes, in every lane of the row; called with every lane active.
// Four DPP moves inside the row (swap neighbours, swap pairs, mirror each half of 8, mirror the
// row) take the place of a butterfly of LDS permutes. The maximum is exact, so the result is the
// same whatever the order.
__device__ __forceinline__ float max_row16(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}
// The same over each group of 4 lanes (two quad swaps).
__device__ __forceinline__ float max_quad(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

// Lane q's v of each group of 4 lanes, in all four (q a compile-time constant after unrolling;
// every lane active).
__device__ __forceinline__ float quad_bcast(float v, int q) {
  switch (q) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x00, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x55, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xFF, 0xF, 0xF, false));
  }
}

}  // namespace moeffn
