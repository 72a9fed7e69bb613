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

// DPP lane moves within a 16-lane row (all rows and banks enabled; every source lane exists)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i of 8 <- lane 7 - i
constexpr int DPP_ROR8 = 0x128;        // lane i of 16 <- lane (i + 8) mod 16

// Sum over SEGS (8 or 16) consecutive lanes (one cache row of the decode attention, one DPP
// row); every lane of the group gets the same bits (each step adds a value and its partner's
// in either order).
template <int SEGS>
__device__ __forceinline__ float seg_sum(float d) {
  static_assert(SEGS == 8 || SEGS == 16, "lanes per row");
  d += dpp_mov<DPP_XOR1>(d);
  d += dpp_mov<DPP_XOR2>(d);
  d += dpp_mov<DPP_HALF_MIRROR>(d);   // quads hold equal values: the mirror brings the other quad's
  if constexpr (SEGS == 16) d += dpp_mov<DPP_ROR8>(d);
  return d;
}

// The values of lanes i and i ^ OFF (OFF = 8, 16, 32): own and partner for OFF = 8 (a DPP
// rotation), the lower and upper lane of the pair for 16 and 32 (the gfx950 permlane swaps
// hand both to both lanes).  Callers combine the two symmetrically, so either order serves.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float& u, float& w) {
  if constexpr (OFF == 8) {
    u = x;
    w = dpp_mov<DPP_ROR8>(x);
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    const int r0 = r[0], r1 = r[1];   // (bit-casting r[1] in place reads r[0] with this hipcc)
    u = __int_as_float(r0);
    w = __int_as_float(r1);
  } else {
    static_assert(OFF == 32, "pair distance");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    const int r0 = r[0], r1 = r[1];   // (bit-casting r[1] in place reads r[0] with this hipcc)
    u = __int_as_float(r0);
    w = __int_as_float(r1);
  }
}

// Sum / max over the 64 lanes of a wave without LDS round trips: DPP steps within each
// 16-lane row, then the two permlane swaps; every lane gets the same bits.
__device__ __forceinline__ float wave_sum(float v) {
  v = seg_sum<16>(v);
  float u, w;
  lane_pair<16>(v, u, w);
  v = u + w;
  lane_pair<32>(v, u, w);
  return u + w;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<DPP_XOR1>(v));
  v = fmaxf(v, dpp_mov<DPP_XOR2>(v));
  v = fmaxf(v, dpp_mov<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_mov<DPP_ROR8>(v));
  float u, w;
  lane_pair<16>(v, u, w);
  v = fmaxf(u, w);
  lane_pair<32>(v, u, w);
  return fmaxf(u, w);
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
