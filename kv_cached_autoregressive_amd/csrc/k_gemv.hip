// Skinny GEMM for the decoder step: out[b, n] = sum_k W[n, k] * y[b, k] for the
// B rows of one step, W streamed once from HBM in its storage dtype, y in fp32.
//
// Shape of the work: each wave owns R consecutive weight rows and walks K in
// 16-byte slices per lane (8 elements), so one wave-wide load covers 1 KB (16-bit
// weights) of contiguous row memory.  The activations of BG rows are staged per
// K-chunk in LDS, laid out so that the two float4 reads a lane makes per slice
// are contiguous across lanes (no bank conflicts).  After the K walk the R*BG
// partial sums are reduce-scattered over the wave (about R*BG shuffles instead
// of 6*R*BG for a full butterfly), leaving one output per lane group, which the
// epilogue finishes: bias, residual add, erf-GELU, the Whisper q|k|v split with
// the K/V cache append, or the tied-head logits with per-block argmax keys.
//
// Batches above BG run as extra grid rows (blockIdx.y), re-reading W.
#include <algorithm>

#include "wd_common.h"
#include "wd_kernels.h"

namespace wd {

template <int NV>
struct Log2 { static constexpr int v = (NV <= 1) ? 0 : 1 + Log2<NV / 2>::v; };
template <>
struct Log2<1> { static constexpr int v = 0; };

// Reduce-scatter of NV (power of two, <= 64) per-lane partial sums over a wave.
// Returns in every lane the full sum of value index (lane >> (6 - log2 NV)).
template <int NV>
__device__ __forceinline__ float reduce_scatter(float (&v)[NV], int lane) {
  constexpr int L2 = Log2<NV>::v;
#pragma unroll
  for (int st = 0; st < L2; ++st) {
    const int s = 32 >> st;
    const int half = NV >> (st + 1);
    const bool up = (lane & s) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = up ? v[i] : v[i + half];
      const float keep = up ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, s, WAVE);
    }
  }
  float t = v[0];
#pragma unroll
  for (int s = (32 >> L2); s > 0; s >>= 1) t += __shfl_xor(t, s, WAVE);
  return t;
}

__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <typename CT>
__device__ __forceinline__ void store_cache(void* base, int64_t idx, float v) {
  reinterpret_cast<CT*>(base)[idx] = from_f<CT>(v);
}

template <typename WT, int R, int BG>
__global__ __launch_bounds__(256) void k_gemv(GemvParams p) {
  constexpr int KC = (BG <= 8) ? 1024 : 512;  // staged K per chunk (multiple of 512)
  constexpr int NV = R * BG;
  __shared__ float ys[BG * KC];
  __shared__ unsigned long long kmax[BG];
  const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
  const int row0 = (blockIdx.x * 4 + wv) * R;
  const int b0 = blockIdx.y * BG;
  const int N = p.N, K = p.K;
  const WT* __restrict__ W = reinterpret_cast<const WT*>(p.W);

  float acc[R][BG];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < BG; ++b) acc[r][b] = 0.f;

  for (int kc0 = 0; kc0 < K; kc0 += KC) {
    const int kcl = min(KC, K - kc0);
    __syncthreads();
    for (int i = threadIdx.x; i < BG * (KC / 4); i += 256) {
      const int b = i / (KC / 4), k4 = (i - b * (KC / 4)) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (b0 + b < p.B && k4 < kcl) {
        const float* src = p.Y + (int64_t)(b0 + b) * p.ldy + kc0 + k4;
        if (p.ymode == Y_SWIGLU) {
          const float* up = src + K;
          v = make_float4(silu(src[0]) * up[0], silu(src[1]) * up[1], silu(src[2]) * up[2], silu(src[3]) * up[3]);
        } else {
          v = *reinterpret_cast<const float4*>(src);
        }
      }
      const int w = k4 & 511;
      const int dst = b * KC + (k4 & ~511) + ((w >> 2) & 1) * 256 + (w >> 3) * 4;
      *reinterpret_cast<float4*>(&ys[dst]) = v;
    }
    __syncthreads();
    for (int kk = lane * 8; kk < kcl; kk += 512) {
      float w8[R][8];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (row0 + r < N) {
          load8(W + (int64_t)(row0 + r) * K + kc0 + kk, w8[r]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) w8[r][j] = 0.f;
        }
      }
      const int base = (kk & ~511) + lane * 4;
#pragma unroll
      for (int b = 0; b < BG; ++b) {
        const float4 y0 = *reinterpret_cast<const float4*>(&ys[b * KC + base]);
        const float4 y1 = *reinterpret_cast<const float4*>(&ys[b * KC + base + 256]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float a = acc[r][b];
          a = fmaf(w8[r][0], y0.x, a); a = fmaf(w8[r][1], y0.y, a);
          a = fmaf(w8[r][2], y0.z, a); a = fmaf(w8[r][3], y0.w, a);
          a = fmaf(w8[r][4], y1.x, a); a = fmaf(w8[r][5], y1.y, a);
          a = fmaf(w8[r][6], y1.z, a); a = fmaf(w8[r][7], y1.w, a);
          acc[r][b] = a;
        }
      }
    }
  }

  float flat[NV];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < BG; ++b) flat[r * BG + b] = acc[r][b];
  const float v = reduce_scatter<NV>(flat, lane);
  const int idx = lane >> (6 - Log2<NV>::v);
  const bool owner = (lane & ((64 >> Log2<NV>::v) - 1)) == 0;
  const int r = idx / BG, bb = idx - (idx / BG) * BG;
  const int n = row0 + r, b = b0 + bb;
  const bool valid = owner && n < N && b < p.B;

  if (p.epi == EPI_LOGITS) {
    if (threadIdx.x < BG) kmax[threadIdx.x] = 0ull;
    __syncthreads();
    if (valid) {
      if (p.out) p.out[(int64_t)b * p.ldo + n] = v;
      if (v != v) raise_err(p.err, ERR_NAN);
      atomicMax(&kmax[bb], argmax_key(v != v ? -INFINITY : v, n));
    }
    __syncthreads();
    if (threadIdx.x < BG && b0 + (int)threadIdx.x < p.B)
      p.amax[(int64_t)blockIdx.x * p.ldp + b0 + threadIdx.x] = kmax[threadIdx.x];
    return;
  }
  if (!valid) return;
  const float bias = p.bias ? p.bias[n] : 0.f;
  switch (p.epi) {
    case EPI_STORE: p.out[(int64_t)b * p.ldo + n] = (v + bias) * p.scale; break;
    case EPI_RESID: p.out[(int64_t)b * p.ldo + n] += v + bias; break;
    case EPI_GELU: p.out[(int64_t)b * p.ldo + n] = gelu_erf(v + bias); break;
    case EPI_QKV: {
      const int seg = n / p.d, c_all = n - seg * p.d;
      if (seg == 0) {
        p.out[(int64_t)b * p.ldo + c_all] = (v + bias) * p.scale;
      } else {
        const int pos = p.pos[b];
        if (pos < 0 || pos >= p.ctx) break;
        const int h = c_all / p.hd, c = c_all - h * p.hd;
        const int64_t at = (int64_t)b * p.kv_bstride + ((int64_t)h * p.ctx + pos) * p.hd + c;
        void* base = seg == 1 ? p.Kc : p.Vc;
        const float val = seg == 1 ? v : v + bias;  // keys carry no bias
        if (p.cache_dtype == DT_F32) store_cache<float>(base, at, val);
        else if (p.cache_dtype == DT_F16) store_cache<f16_t>(base, at, val);
        else store_cache<bf16_t>(base, at, val);
      }
      break;
    }
    default: break;
  }
}

struct Shape { int R, BG; };
static Shape pick(int B) {
  if (B <= 1) return {4, 1};
  if (B <= 2) return {4, 2};
  if (B <= 4) return {4, 4};
  if (B <= 8) return {4, 8};
  return {2, 16};
}

int gemv_blocks(int N, int B) {
  const Shape sh = pick(B);
  return (N + 4 * sh.R - 1) / (4 * sh.R);
}

template <typename WT>
static hipError_t run(const GemvParams& p, hipStream_t s) {
  const Shape sh = pick(p.B);
  dim3 grid((p.N + 4 * sh.R - 1) / (4 * sh.R), (p.B + sh.BG - 1) / sh.BG);
  if (sh.BG == 1) k_gemv<WT, 4, 1><<<grid, 256, 0, s>>>(p);
  else if (sh.BG == 2) k_gemv<WT, 4, 2><<<grid, 256, 0, s>>>(p);
  else if (sh.BG == 4) k_gemv<WT, 4, 4><<<grid, 256, 0, s>>>(p);
  else if (sh.BG == 8) k_gemv<WT, 4, 8><<<grid, 256, 0, s>>>(p);
  else k_gemv<WT, 2, 16><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvParams& p, hipStream_t s) {
  if (p.N <= 0 || p.K <= 0 || (p.K % 8) || p.B <= 0 || p.B > 64 || !p.W || !p.Y) return hipErrorInvalidValue;
  if (p.ymode == Y_SWIGLU ? p.ldy < 2 * p.K : p.ldy < p.K) return hipErrorInvalidValue;
  if ((p.ldy % 4) || (reinterpret_cast<uintptr_t>(p.Y) % 16)) return hipErrorInvalidValue;
  if (p.epi == EPI_LOGITS) {
    if (!p.amax || p.ldp < p.B) return hipErrorInvalidValue;
    if (p.out && p.ldo < p.N) return hipErrorInvalidValue;
  } else if (!p.out) {
    return hipErrorInvalidValue;
  }
  if (p.epi == EPI_QKV && (p.N != 3 * p.d || !p.pos || !p.Kc || !p.Vc || p.hd <= 0 || p.d != p.H * p.hd))
    return hipErrorInvalidValue;
  switch (p.w_dtype) {
    case DT_F32: return run<float>(p, s);
    case DT_F16: return run<f16_t>(p, s);
    case DT_BF16: return run<bf16_t>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wd
