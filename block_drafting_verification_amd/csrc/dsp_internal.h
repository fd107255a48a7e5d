// Internal helpers shared by the HIP translation units of libdsp (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "dsp.h"

namespace dsp {

// ---------------------------------------------------------------- host side
int32_t fail(int32_t code, const char* fmt, ...);   // records dsp_last_error, returns code
void clear_error();
int32_t hip_check(hipError_t e, const char* what);  // DSP_OK or DSP_ERR_HIP

// Kernel timing (off unless dsp_prof_enable selects the kernel id): prof_events hands out
// a start/stop event pair when the id is selected, prof_commit files the pair for
// dsp_prof_query once the launch carrying them is enqueued.
bool prof_events(int kernel, hipEvent_t* start, hipEvent_t* stop);
// Current value of a DSP_OPT_* option.
int64_t option(int32_t opt);
void prof_commit(int kernel, hipEvent_t start, hipEvent_t stop);

// Launch `kernel` on stream s. When its id is being timed, the events ride on the
// dispatch packet itself (hipExtLaunchKernelGGL), so they bracket the kernel's own
// execution rather than the host's launch gap.
template <typename... KArgs, typename... Args>
inline void launch(int kid, void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                   Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (prof_events(kid, &e0, &e1)) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0u, (KArgs)args...);
    prof_commit(kid, e0, e1);
  } else {
    kernel<<<grid, block, shmem, s>>>((KArgs)args...);
  }
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Simple bump allocator over a caller-provided workspace.
struct WsCarver {
  uintptr_t base;
  size_t off = 0;
  explicit WsCarver(void* p) : base((uintptr_t)p) {}
  template <typename T> T* take(size_t count) {
    off = align_up(off, 256);
    T* p = (T*)(base + off);
    off += count * sizeof(T);
    return p;
  }
  size_t used() const { return align_up(off, 256); }
};

// ---------------------------------------------------------------- device side
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_val(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Monotone map float -> uint32 (larger float => larger integer); -0 is folded onto +0.
__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}
// Arg-max key: larger value first, then the lower index.
__device__ __forceinline__ uint64_t amax_key(float f, uint32_t idx) {
  return ((uint64_t)ord_f32(f) << 32) | (uint64_t)(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t amax_index(uint64_t k) { return 0xffffffffu - (uint32_t)k; }
__device__ __forceinline__ float amax_value(uint64_t k) { return unord_f32((uint32_t)(k >> 32)); }

// Philox4x64-10 (Salmon et al., SC'11): 64x64->128 multiply S-box, 10 rounds,
// Weyl key schedule.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t h0 = __umul64hi(M0, c[0]), l0 = M0 * c[0];
    const uint64_t h1 = __umul64hi(M1, c[2]), l1 = M1 * c[2];
    const uint64_t n0 = h1 ^ c[1] ^ k0, n2 = h0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = l1; c[2] = n2; c[3] = l0;
  }
}
__device__ __forceinline__ double unit_double(uint64_t w) {
  return (double)(w >> 11) * 0x1.0p-53;
}

// Lane exchange at xor distance TS (1..32) inside a wavefront, with fixed patterns:
// DPP quad permutes for 1 and 2, ds_swizzle xor masks for 4, 8 and 16 (no LDS memory
// access), ds_bpermute only for 32.
template <int TS>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  if (TS == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  if (TS == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  if (TS == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x101F);  // and 31, xor 4
  if (TS == 8) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x201F);
  if (TS == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 63) ^ 32) << 2), (int)x);
}

// Wave (64 lanes) reductions; deterministic butterfly order.
template <typename T> __device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { T w = __shfl_xor(v, o, 64); v = w > v ? w : v; }
  return v;
}
template <typename T> __device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { T w = __shfl_xor(v, o, 64); v = w < v ? w : v; }
  return v;
}
template <typename T> __device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block reductions for blockDim.x = 64 * NW; every thread gets the result.
template <int NW, typename T> __device__ __forceinline__ T block_max(T v, T* sm) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = sm[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = sm[i] > r ? sm[i] : r;
  return r;
}
template <int NW, typename T> __device__ __forceinline__ T block_min(T v, T* sm) {
  v = wave_min(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = sm[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = sm[i] < r ? sm[i] : r;
  return r;
}
template <int NW, typename T> __device__ __forceinline__ T block_sum(T v, T* sm) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = sm[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += sm[i];
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2d = 0.69314718055994530942;
constexpr double kLog2ed = 1.4426950408889634074;

}  // namespace dsp
