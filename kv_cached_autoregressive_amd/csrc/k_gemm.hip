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
#include <cstdlib>

#include "wd_common.h"
#include "wd_kernels.h"

namespace wd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t xv4u;

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

// LDS-tiled variant for d % 128 == 0 and hd == 64 (every Whisper shape here).
//  * Block tile 256 (rows of X) x 128 (output columns = two heads of K or of V); four waves
//    as 2 x 2, each 128 x 64 (8 x 4 MFMA tiles of 16 x 16, 128 accumulators per lane).
//  * K tiles of 64: the next tile's global loads (16 B per thread, 128 B per row segment)
//    are in flight while the current one is multiplied out of LDS; rows are padded to
//    72 elements (144 B) so the 16 lanes reading one fragment column hit distinct banks.
//  * Block order: workgroup L runs on XCD L % 8; the 128-column tiles of one 256-row panel
//    of X go to consecutive workgroups of the same XCD, so that panel is fetched into that
//    XCD's L2 once and reused for every column tile.
//  * Epilogue: bias, rounding to the cache type, then each half of the tile (128 rows)
//    goes through LDS and out as whole 128-byte cache rows ([n_enc][H][max_frames][64]).
constexpr int XBM = 256, XBN = 128, XBK = 64, XLD = XBK + 8;

template <typename T, typename CT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_xkv_tiled(const T* __restrict__ X, const T* __restrict__ W, int K, XkvOut o,
                                                   int n_mt, int n_nt) {
  __shared__ __align__(16) T As[XBM * XLD];
  __shared__ __align__(16) T Bs[XBN * XLD];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int L = blockIdx.x, xcd = L % 8, j = L / 8;
  const int mt = xcd + 8 * (j / n_nt), nt = j - (j / n_nt) * n_nt;
  if (mt >= n_mt) return;
  const int m0 = mt * XBM, n0 = nt * XBN;
  const int wm = wv & 1, wn = wv >> 1;
  const int lr = lane & 15, lq = lane >> 4;

  // global -> register staging: thread t moves 16 B of rows t/8 + 32*i, k chunk (t%8)*8
  const int gr = t >> 3, gk = (t & 7) * 8;
  // rows past M (a partial last panel) reload row M-1; their products are never stored
  const T* xa = X + (int64_t)(m0 + gr) * K + gk;
  const T* wb = W + (int64_t)(n0 + gr) * K + gk;
  const T* xend = X + (int64_t)(o.M - 1) * K + gk;
  // W tiles are fetched nontemporally: they stream past the L2, which keeps the X panel
  // that the column tiles of this XCD share
  uint4 ra[8], rb[4];
  auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const T* src = m0 + gr + 32 * i < o.M ? xa + (int64_t)(32 * i) * K : xend;
      ra[i] = *reinterpret_cast<const uint4*>(src + k0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rb[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                  reinterpret_cast<const xv4u*>(wb + (int64_t)(32 * i) * K + k0)));
  };
  auto lstore = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(As + (gr + 32 * i) * XLD + gk) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(Bs + (gr + 32 * i) * XLD + gk) = rb[i];
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = K / XBK;
  gload(0);
  lstore();
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload((kt + 1) * XBK);
#pragma unroll
    for (int ks = 0; ks < XBK / 32; ++ks) {
      uint4 a[8], b[4];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[i] = *reinterpret_cast<const uint4*>(As + (wm * 128 + i * 16 + lr) * XLD + ks * 32 + lq * 8);
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
        b[jn] = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + jn * 16 + lr) * XLD + ks * 32 + lq * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[i][jn] = mfma16x16x32(a[i], b[jn], acc[i][jn], (T*)nullptr);
    }
    __syncthreads();   // every wave is done with this tile
    if (kt + 1 < KT) {
      lstore();
      __syncthreads();
    }
  }

  // epilogue: tile column c (0..127) is output column n0 + c; the tile's 128 columns are two
  // heads of one cache (K if n0 < d, else V)
  const bool isv = n0 >= o.d;
  const int h0 = (isv ? n0 - o.d : n0) / 64;
  CT* base = reinterpret_cast<CT*>(isv ? o.Vc : o.Kc);
  CT* Cs = reinterpret_cast<CT*>(As);   // 128 rows x 136 columns of CT per half (272 B rows)
  constexpr int CLD = XBN + 8;
  float bias[4];
#pragma unroll
  for (int jn = 0; jn < 4; ++jn) bias[jn] = o.bias[n0 + wn * 64 + jn * 16 + lr];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Cs[(i * 16 + lq * 4 + e) * CLD + wn * 64 + jn * 16 + lr] = from_f<CT>(acc[i][jn][e] + bias[jn]);
    }
    __syncthreads();
    // 128 rows x 2 heads x 64 channels: 16-byte chunks, 8 per (row, head)
    constexpr int CH = 16 / sizeof(CT);
    for (int q = t; q < 128 * 2 * (64 / CH); q += 256) {
      const int r = q / (2 * (64 / CH)), rem = q - r * (2 * (64 / CH));
      const int hh = rem / (64 / CH), c = (rem - hh * (64 / CH)) * CH;
      const int m = m0 + half * 128 + r;
      if (m < o.M) {
        const int e = m / o.frames, f = m - e * o.frames;
        CT* dst = base + (((int64_t)e * o.H + h0 + hh) * o.max_frames + f) * 64 + c;
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(Cs + r * CLD + hh * 64 + c);
      }
    }
    __syncthreads();
  }
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

// Tiled kernel unless WD_XKV_TILED=0 (for comparisons) or the shape does not fit it.
static bool xkv_tiled_on() {
  static int mode = -1;
  if (mode < 0) {
    const char* e = getenv("WD_XKV_TILED");
    mode = e ? atoi(e) : 1;
  }
  return mode != 0;
}

template <typename T>
static hipError_t run_mfma(const void* X, const void* W, int K, const XkvOut& o, int cache_dtype, hipStream_t s) {
  if (xkv_tiled_on() && o.hd == 64 && o.d % XBN == 0 && K % XBK == 0 && cache_dtype != DT_F32) {
    const int n_mt = (o.M + XBM - 1) / XBM, n_nt = o.N / XBN;
    dim3 grid(8 * ((n_mt + 7) / 8) * n_nt);
    if (cache_dtype == DT_F16) k_xkv_tiled<T, f16_t><<<grid, 256, 0, s>>>((const T*)X, (const T*)W, K, o, n_mt, n_nt);
    else k_xkv_tiled<T, bf16_t><<<grid, 256, 0, s>>>((const T*)X, (const T*)W, K, o, n_mt, n_nt);
    return hipGetLastError();
  }
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
