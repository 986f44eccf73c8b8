// Internal helpers shared by the gfx950 kernels of the fused MoE forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: gfx950
// v_cvt_pk_bf16_f32, the same rounding as f32_to_bf16 on finite inputs.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// silu(g) * u with silu(g) = g / (1 + e^-g); the quotient uses the hardware reciprocal
// (about 1 ulp), far below the bf16 rounding the result gets.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// gpt-oss's clamped SwiGLU ("swigluoai"): the gate is clamped above at 7 and the up value to
// [-7, 7]; act = g * sigmoid(1.702 g) * (u + 1).
__device__ __forceinline__ float swigluoai_mul(float g, float u) {
  g = fminf(g, 7.0f);
  u = fminf(fmaxf(u, -7.0f), 7.0f);
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-1.702f * g)) * (u + 1.0f);
}

// The activation of the gate/up pair: act 0 = silu, 1 = swigluoai (MOE_ACT_*).
__device__ __forceinline__ float act_mul(float g, float u, int act) {
  return act == 1 ? swigluoai_mul(g, u) : silu_mul(g, u);
}

// 16-byte global -> LDS load (gfx950 global_load_lds_dwordx4): lane l's 16 bytes at
// base + voff land at LDS byte address lds_addr + 16 l; base and lds_addr are wave-uniform.
// Written as inline asm on purpose: the compiler has to assume that such a load may touch
// both LDS and global memory, and once one is in flight it degrades every later LDS wait to
// lgkmcnt(0), which serialises the fragment reads of the next K slice with the MFMAs of the
// current one. The compiler does not see the load, so the caller waits for it explicitly
// (s_waitcnt vmcnt) before any wave reads the data. M0 carries the LDS address (an operand
// of the asm, so the compiler writes it); one wait state separates that write from the
// load. Device pass only (the host pass needs the kernel's launch stub alone).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
#endif
}

// dma16 with the non-temporal hint (nt): data read once, streamed past the caches' reuse.
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds_addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
#endif
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  using lds_ptr = const __attribute__((address_space(3))) uint8_t*;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(p)));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }  // vmcnt(n)
constexpr int wait_vm_lgkm0(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }  // + lgkmcnt(0)
constexpr int kWaitVm0 = wait_vm(0);
constexpr int kWaitVmLgkm0 = wait_vm_lgkm0(0);

// Workgroup barrier without the release fence of __syncthreads (which would also wait for
// every outstanding global->LDS load); callers wait explicitly for what must have landed.
// The memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_barrier" ::: "memory");
#endif
}

// Plain 16-byte global load.
__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte global load with the non-temporal hint.
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}

inline int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

}  // namespace moe

namespace moe {

template <class T>
struct as_is {
  using type = T;
};

// Kernel launch that reports its own status: hipLaunchKernel returns the launch's error code
// directly, so an error left pending by earlier, unrelated work is neither taken for this
// launch's nor cleared. The arguments convert to the kernel's parameter types.
template <typename... P>
inline int launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                  typename as_is<P>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, s) ==
                 hipSuccess
             ? MOE_OK
             : MOE_EHIP;
}

}  // namespace moe
