// Shared device-side types and helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dit {

typedef uint16_t bf16_t;                                             // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));           // MFMA bf16 operand
typedef float f32x16 __attribute__((ext_vector_type(16)));           // 32x32 MFMA accumulator
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));          // 16-byte move
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));          // 8-byte move

// SiLU x·sigmoid(x) = x / (1 + e^-x), with the hardware reciprocal (within
// 1 ulp) instead of the IEEE division sequence: the result is rounded to bf16
// next, which this error changes only when it straddles a rounding boundary.
// Saturates to -0 for very negative x (e^-x = inf, reciprocal 0).
__device__ __forceinline__ float silu_f(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// float -> bf16, round to nearest even (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));           // 16-byte fp32 move
// Two floats -> packed bf16 pair (a in the low half), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Conversions for the activation element type act_t (kernels.h).
#ifdef DIT_F32
__device__ __forceinline__ float act2f(act_t v) { return v; }
__device__ __forceinline__ act_t f2act(float f) { return f; }
#else
__device__ __forceinline__ float act2f(act_t v) { return bf2f(v); }
__device__ __forceinline__ act_t f2act(float f) { return f2bf(f); }
#endif
// Store 4 / 8 consecutive activations from floats (16-byte aligned for 8).
__device__ __forceinline__ void store_act4(act_t* p, float a, float b, float c, float d) {
#ifdef DIT_F32
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
#else
  u32x2 w;
  w.x = pack2bf(a, b);
  w.y = pack2bf(c, d);
  *reinterpret_cast<u32x2*>(p) = w;
#endif
}
__device__ __forceinline__ void load_act2(const act_t* p, float& a, float& b) {
#ifdef DIT_F32
  const float2 v = *reinterpret_cast<const float2*>(p);
  a = v.x; b = v.y;
#else
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
  a = bf2f((bf16_t)(v & 0xffff)); b = bf2f((bf16_t)(v >> 16));
#endif
}
// 8 consecutive activations <-> floats (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void load_act8(const act_t* p, float (&f)[8]) {
#ifdef DIT_F32
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
#else
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
#endif
}
__device__ __forceinline__ void store_act8(act_t* p, const float (&f)[8]) {
#ifdef DIT_F32
  reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
#else
  u32x4 v;
  v.x = pack2bf(f[0], f[1]); v.y = pack2bf(f[2], f[3]);
  v.z = pack2bf(f[4], f[5]); v.w = pack2bf(f[6], f[7]);
  *reinterpret_cast<u32x4*>(p) = v;
#endif
}
__device__ __forceinline__ void store_act2(act_t* p, float a, float b) {
#ifdef DIT_F32
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
#else
  *reinterpret_cast<uint32_t*>(p) = pack2bf(a, b);
#endif
}

// v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] · B[16x32].
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32];
// accumulator register r of lane l holds C[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; a counter at its maximum is not waited on).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kWaitLgkm0 = 0xF | 0xC000 | 0x70;

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its outstanding global loads (a full __syncthreads
// fence would drain every in-flight prefetch).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS destination pointer of a buffer_load ... lds (address space 3).
#define LDSP(p) ((__attribute__((address_space(3))) void*)(p))

// Compute units of the current device (cached per device; 0 if unknown).
inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

// One kernel launch; the events, when given, are taken by the kernel's own
// dispatch packet (start as it starts, stop as it ends), so timing puts no
// extra packet between kernels.
template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                     Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0u, s, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// The events of a launch with nothing to run (empty input), so that a
// timed launch always records both.
inline void mark_empty(const LaunchEvents& ev, hipStream_t s) {
  if (ev.start) (void)hipEventRecord(ev.start, s);
  if (ev.stop) (void)hipEventRecord(ev.stop, s);
}

// A pointer the caller knows to be the same in every lane, moved to scalar
// registers (so a buffer resource built from it needs no per-lane loop).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource over [p, p + bytes): loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-causal visibility in row-limit form: key j is visible to a query
// whose largest visible key is `lim` (and j must be a real key, j < S).
__device__ __forceinline__ bool key_visible(int j, int lim, int S) { return j <= lim && j < S; }

// Classification of a key tile [kv0, kv0+BKV) for a group of queries whose
// limits lie in [lim_min, lim_max]: 0 = nothing visible (skip),
// 1 = everything visible (no per-element test), 2 = test per element.
template <int BKV>
__device__ __forceinline__ int tile_class(int kv0, int lim_min, int lim_max, int S) {
  if (kv0 > lim_max) return 0;
  if (kv0 + BKV - 1 <= lim_min && kv0 + BKV <= S) return 1;
  return 2;
}

}  // namespace dit
