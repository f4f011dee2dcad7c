// Direct-to-LDS loads and the waits around them, shared by the grouped FFN kernels and the
// router logits of large batches.
#pragma once

#include "moe_internal.h"

namespace moeffn {
namespace {

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4, with the LDS base in M0), issued as inline assembly: the
// compiler then does not track the LDS write, so it adds no "vmcnt(0)" before later LDS
// reads; callers order them with explicit vmcnt waits and barriers. Each asm block sets M0
// itself. The compiler reserves M0 and does not honour it as a clobber, so it is not listed;
// instead the build disassembles the compiled kernels and fails unless every instruction
// naming M0 is one of these sequences (build.py check_m0). lds_base must be wave-uniform.
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

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace
}  // namespace moeffn
