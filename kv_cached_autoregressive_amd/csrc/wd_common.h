// Device-side helpers shared by the decoder-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wd_kernels.h"

namespace wd {

// Storage types.  Half and bfloat16 are kept as raw 16-bit patterns and
// converted explicitly, so the rounding is visible: float -> f16 uses the
// hardware round-to-nearest-even convert, float -> bf16 rounds to nearest even
// in integer arithmetic (NaN kept quiet).
struct bf16_t { uint16_t x; };
typedef _Float16 f16_t;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_bits_to_f(uint32_t lo16) { return __uint_as_float(lo16 << 16); }

__device__ __forceinline__ uint16_t f_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(f16_t v) { return (float)v; }
__device__ __forceinline__ float to_f(bf16_t v) { return bf16_bits_to_f(v.x); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ f16_t from_f<f16_t>(float v) { return (f16_t)v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { bf16_t r; r.x = f_to_bf16_bits(v); return r; }

// 8 consecutive elements -> 8 floats.  p must be 16-byte aligned for 16-bit
// types and 32-byte aligned for float.
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void unpack_h8(const uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t lo = (uint16_t)(w[i] & 0xffffu), hi = (uint16_t)(w[i] >> 16);
    f[2 * i] = (float)__builtin_bit_cast(f16_t, lo);
    f[2 * i + 1] = (float)__builtin_bit_cast(f16_t, hi);
  }
}
__device__ __forceinline__ void unpack_b8(const uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const f16_t* p, float (&f)[8]) {
  unpack_h8(*reinterpret_cast<const uint4*>(p), f);
}
__device__ __forceinline__ void load8(const bf16_t* p, float (&f)[8]) {
  unpack_b8(*reinterpret_cast<const uint4*>(p), f);
}

// Raw 16-byte (or 32-byte for float) fetch and later unpack, so that several
// loads can be issued before their data is consumed.
template <typename T> struct Raw8 { uint4 v; };
template <> struct Raw8<float> { float4 a, b; };
__device__ __forceinline__ Raw8<float> fetch8(const float* p) {
  Raw8<float> r; r.a = reinterpret_cast<const float4*>(p)[0]; r.b = reinterpret_cast<const float4*>(p)[1]; return r;
}
__device__ __forceinline__ Raw8<f16_t> fetch8(const f16_t* p) { Raw8<f16_t> r; r.v = *reinterpret_cast<const uint4*>(p); return r; }
__device__ __forceinline__ Raw8<bf16_t> fetch8(const bf16_t* p) { Raw8<bf16_t> r; r.v = *reinterpret_cast<const uint4*>(p); return r; }
__device__ __forceinline__ void unpack8(const Raw8<float>& r, float (&f)[8]) {
  f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w; f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
}
__device__ __forceinline__ void unpack8(const Raw8<f16_t>& r, float (&f)[8]) { unpack_h8(r.v, f); }
__device__ __forceinline__ void unpack8(const Raw8<bf16_t>& r, float (&f)[8]) { unpack_b8(r.v, f); }

// fp32 -> (hi, lo) 16-bit pair with hi + lo ~= v to ~16 significant bits
template <typename T>
__device__ __forceinline__ void split_hi_lo(float v, T& hi, T& lo) {
  hi = from_f<T>(v);
  lo = from_f<T>(v - to_f(hi));
}
template <typename T>
__device__ __forceinline__ void store_split(void* hi_base, void* lo_base, int64_t off, float v) {
  T h, l;
  split_hi_lo<T>(v, h, l);
  reinterpret_cast<T*>(hi_base)[off] = h;
  reinterpret_cast<T*>(lo_base)[off] = l;
}

// Butterfly sum / max over the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, WAVE));
  return v;
}

// Block-wide sum for blockDim.x == NT (multiple of 64); `red` holds NT/64 floats.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) t += red[i];
  return t;
}
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) t = fmaxf(t, red[i]);
  return t;
}

__device__ __forceinline__ void raise_err(unsigned* err, unsigned bits) {
  if (err) atomicOr(err, bits);
}

// Totally ordered 64-bit key of (value, index): larger value wins, then lower
// index.  -0.0 is folded into +0.0 so equal values tie on the index.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - (uint32_t)idx);
}

// Sum over k < G of p[k * stride], added in order k = 0..G-1.  Every load is issued
// before the first add (G <= GMAX; indices past G-1 reload the last slab and are not
// added), so the G loads overlap instead of paying one memory round trip each.  Partial
// slabs are read once: nontemporal loads keep them out of the L2 (3.4% on the large-v3
// step, within noise at 8-16 rows).
template <int GMAX>
__device__ __forceinline__ float sum_parts(const float* __restrict__ p, int64_t stride, int G) {
  float v[GMAX];
#pragma unroll
  for (int k = 0; k < GMAX; ++k) v[k] = __builtin_nontemporal_load(p + (int64_t)min(k, G - 1) * stride);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < GMAX; ++k) s += k < G ? v[k] : 0.f;
  return s;
}

// A raw buffer resource over `bytes` bytes at `base` (32-bit byte offsets; a load past the
// end returns zeros instead of touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// One 16-byte load per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds):
// lane i's bytes land at lds_wave + 16 i, so `lds_wave` is the wave's (uniform) 1 KB slot.
// The load counts in vmcnt like any vector load and writes no VGPR.  (The buffer form, not
// global_load_lds: with the latter in a loop, hipcc waits for every outstanding LDS read
// before the first use of any of them; with this one it counts them.)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t off, void* lds_wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave, 16, off, 0, 0, 0);
}
// s_waitcnt with vmcnt = N (N < 16) and the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

}  // namespace wd
