// Cross K/V projection, once per audio window: C = X W^T + [0 | b_v] with X the
// encoder states [n_enc*frames, d] and W the fused [Wk; Wv] [2d, d], rounded to
// the cache dtype and scattered into the head-major caches
// [n_enc][H][max_frames][hd] (K for n < d, V for n >= d).
//
// This is the one dense contraction of the decoder (wavo decoder.rs
// `record_cross`: one GEMM with the fused bias per layer), so it runs on the
// matrix cores: v_mfma_f32_16x16x32 (f16 or bf16 inputs, fp32 accumulate).
// Block tile 128x128, four waves of 64x64, K step 32.  Fragments are loaded
// straight from global memory in the MFMA operand layout (lane l holds 8
// consecutive k of row l%16, k offset 8*(l/16)), one step ahead of use.
// The fp32 mode uses a plain LDS-tiled VALU kernel.
#include <algorithm>

#include "wd_common.h"
#include "wd_kernels.h"

namespace wd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, const f32x4_t& c, bf16_t*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, const f32x4_t& c, f16_t*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

struct XkvOut {
  const float* bias; int M, N, d, frames, max_frames, H, hd;
  void* Kc; void* Vc;
};

template <typename CT>
__device__ __forceinline__ void xkv_store(const XkvOut& o, int m, int n, float v) {
  if (m >= o.M || n >= o.N) return;
  v += o.bias[n];
  const int e = m / o.frames, f = m - e * o.frames;
  const bool isv = n >= o.d;
  const int c_all = isv ? n - o.d : n;
  const int h = c_all / o.hd, c = c_all - h * o.hd;
  CT* base = reinterpret_cast<CT*>(isv ? o.Vc : o.Kc);
  base[(((int64_t)e * o.H + h) * o.max_frames + f) * o.hd + c] = from_f<CT>(v);
}

template <typename T, typename CT>
__global__ __launch_bounds__(256) void k_xkv_mfma(const T* __restrict__ X, const T* __restrict__ W, int K, XkvOut o) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m0 = blockIdx.x * 128 + (wv & 1) * 64;
  const int n0 = blockIdx.y * 128 + (wv >> 1) * 64;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const T* ap[4];
  const T* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ap[i] = X + (int64_t)min(m0 + i * 16 + lr, o.M - 1) * K + lk;
    bp[i] = W + (int64_t)min(n0 + i * 16 + lr, o.N - 1) * K + lk;
  }
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = *reinterpret_cast<const uint4*>(ap[i]);
    b[i] = *reinterpret_cast<const uint4*>(bp[i]);
  }
  for (int k0 = 0; k0 < K; k0 += 32) {
    uint4 an[4], bn[4];
    const int kn = (k0 + 32 < K) ? k0 + 32 : k0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      an[i] = *reinterpret_cast<const uint4*>(ap[i] + kn);
      bn[i] = *reinterpret_cast<const uint4*>(bp[i] + kn);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j], (T*)nullptr);
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = an[i]; b[i] = bn[i]; }
  }
  // D fragment: lane holds rows 4*(lane/16)+e of column lane%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        xkv_store<CT>(o, m0 + i * 16 + (lane >> 4) * 4 + e, n0 + j * 16 + lr, acc[i][j][e]);
}

// fp32: 64x64 block tile, 4x4 per thread, K tiles of 16 through LDS.
template <typename CT>
__global__ __launch_bounds__(256) void k_xkv_f32(const float* __restrict__ X, const float* __restrict__ W, int K, XkvOut o) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = t; i < 64 * 16; i += 256) {
      const int r = i >> 4, k = i & 15;
      const int m = min(m0 + r, o.M - 1), n = min(n0 + r, o.N - 1);
      const bool kin = k0 + k < K;
      As[k][r] = kin ? X[(int64_t)m * K + k0 + k] : 0.f;
      Bs[k][r] = kin ? W[(int64_t)n * K + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = As[k][ty * 4 + i]; bv[i] = Bs[k][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) xkv_store<CT>(o, m0 + ty * 4 + i, n0 + tx * 4 + j, acc[i][j]);
}

template <typename T>
static hipError_t run_mfma(const void* X, const void* W, int K, const XkvOut& o, int cache_dtype, hipStream_t s) {
  dim3 grid((o.M + 127) / 128, (o.N + 127) / 128);
  switch (cache_dtype) {
    case DT_F32: k_xkv_mfma<T, float><<<grid, 256, 0, s>>>((const T*)X, (const T*)W, K, o); break;
    case DT_F16: k_xkv_mfma<T, f16_t><<<grid, 256, 0, s>>>((const T*)X, (const T*)W, K, o); break;
    case DT_BF16: k_xkv_mfma<T, bf16_t><<<grid, 256, 0, s>>>((const T*)X, (const T*)W, K, o); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cross_kv_gemm(const void* X, const void* W, const float* bias, int w_dtype, int M, int d,
                                int frames, int max_frames, int H, int hd, void* Kc, void* Vc,
                                int cache_dtype, hipStream_t s) {
  if (M <= 0 || d <= 0 || frames <= 0 || frames > max_frames || M % frames || H * hd != d || !bias)
    return hipErrorInvalidValue;
  XkvOut o{bias, M, 2 * d, d, frames, max_frames, H, hd, Kc, Vc};
  if (w_dtype == DT_F32) {
    dim3 grid((M + 63) / 64, (2 * d + 63) / 64);
    switch (cache_dtype) {
      case DT_F32: k_xkv_f32<float><<<grid, 256, 0, s>>>((const float*)X, (const float*)W, d, o); break;
      case DT_F16: k_xkv_f32<f16_t><<<grid, 256, 0, s>>>((const float*)X, (const float*)W, d, o); break;
      case DT_BF16: k_xkv_f32<bf16_t><<<grid, 256, 0, s>>>((const float*)X, (const float*)W, d, o); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (d % 32) return hipErrorInvalidValue;  // whole K steps of 32
  if (w_dtype == DT_F16) return run_mfma<f16_t>(X, W, d, o, cache_dtype, s);
  if (w_dtype == DT_BF16) return run_mfma<bf16_t>(X, W, d, o, cache_dtype, s);
  return hipErrorInvalidValue;
}

}  // namespace wd
