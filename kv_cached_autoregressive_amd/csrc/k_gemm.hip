// Cross K/V projection, once per audio window: C = X W^T + [0 | b_v] with X the
// encoder states [n_enc*frames, d] and W the fused [Wk; Wv] [2d, d], rounded to
// the cache dtype and scattered into the head-major caches
// [n_enc][H][max_frames][hd] (K for n < d, V for n >= d).
//
// This is the one dense contraction of the decoder (wavo decoder.rs
// `record_cross`: one GEMM with the fused bias per layer), so it runs on the
// matrix cores: v_mfma_f32_16x16x32 (f16 or bf16 inputs, fp32 accumulate).
// X is repacked into the MFMA fragment order once per window (it feeds every
// layer) and W is stored in that order at load, so every operand load is one
// contiguous 1 KB tile.  The fp32 mode uses a plain LDS-tiled VALU kernel over
// row-major operands.
#include <algorithm>
#include <cstdlib>

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

// Row-major [M, d] -> fragment order (16-byte slices: 8 consecutive k of one row).
template <typename T>
__global__ __launch_bounds__(256) void k_pack_rows(const T* __restrict__ src, T* __restrict__ dst, int64_t M, int d) {
  const int64_t n = M * (d / 8);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / (d / 8);
    const int k = (int)(i - r * (d / 8)) * 8;
    *reinterpret_cast<uint4*>(dst + frag_offset(r, k, d)) = *reinterpret_cast<const uint4*>(src + r * d + k);
  }
}

hipError_t launch_pack_rows(const void* X, int w_dtype, void* Xf, int64_t M, int d, hipStream_t s) {
  if (M <= 0 || d <= 0 || d % 32 || !X || !Xf) return hipErrorInvalidValue;
  const int blocks = (int)std::min<int64_t>((M * (d / 8) + 255) / 256, 65536);
  if (w_dtype == DT_BF16) k_pack_rows<bf16_t><<<blocks, 256, 0, s>>>((const bf16_t*)X, (bf16_t*)Xf, M, d);
  else if (w_dtype == DT_F16) k_pack_rows<f16_t><<<blocks, 256, 0, s>>>((const f16_t*)X, (f16_t*)Xf, M, d);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Block tile 128 rows of X x 128 output columns (128 / hd heads of K or of V); four waves of
// 64 x 64 (4 x 4 MFMA tiles), operands one K step ahead.  Workgroup L runs on XCD L % 8: the
// column tiles of one 128-row panel of X go to consecutive workgroups of one XCD, so that
// panel is read into that XCD's L2 once.  Epilogue: V bias, rounding to the cache type, and
// whole 128-byte cache rows written through LDS.
template <typename T, typename CT>
__global__ __launch_bounds__(256) void k_xkv_frag(const T* __restrict__ Xf, const T* __restrict__ Wf, int K,
                                                  XkvOut o, int n_mt, int n_nt) {
  constexpr int CLD = 128 + 8;
  __shared__ __align__(16) CT Cs[128 * CLD];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int L = blockIdx.x, xcd = L % 8, j = L / 8;
  const int mt = xcd + 8 * (j / n_nt), nt = j - (j / n_nt) * n_nt;
  if (mt >= n_mt) return;
  const int wm = wv & 1, wn = wv >> 1;
  const int rt0 = mt * 8 + wm * 4, ct0 = nt * 8 + wn * 4;
  const int KST = K >> 5, lr = lane & 15, lq = lane >> 4;
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u* __restrict__ A = reinterpret_cast<const v4u*>(Xf);
  const v4u* __restrict__ B = reinterpret_cast<const v4u*>(Wf);
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  v4u a[4], b[4];
  auto load = [&](int st, v4u (&fa)[4], v4u (&fb)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = A[((int64_t)(rt0 + i) * KST + st) * 64 + lane];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) fb[jn] = B[((int64_t)(ct0 + jn) * KST + st) * 64 + lane];
  };
  load(0, a, b);
  for (int st = 0; st < KST; ++st) {
    v4u na[4], nb[4];
    load(min(st + 1, KST - 1), na, nb);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
        acc[i][jn] = mfma16x16x32(__builtin_bit_cast(uint4, a[i]), __builtin_bit_cast(uint4, b[jn]), acc[i][jn], (T*)nullptr);
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = na[i]; b[i] = nb[i]; }
  }
  // tile (i, jn): lane holds rows (rt0+i)*16 + 4*lq + e of column (ct0+jn)*16 + lr
  const int n0 = nt * 128;
  const bool isv = n0 >= o.d;
  const int h0 = (isv ? n0 - o.d : n0) / o.hd;   // first head of the tile (128 / hd heads)
#pragma unroll
  for (int jn = 0; jn < 4; ++jn) {
    const float bias = o.bias[n0 + wn * 64 + jn * 16 + lr];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Cs[(wm * 64 + i * 16 + lq * 4 + e) * CLD + wn * 64 + jn * 16 + lr] = from_f<CT>(acc[i][jn][e] + bias);
  }
  __syncthreads();
  // 128 rows x 128 columns in 16-byte chunks; a head's channels are one contiguous cache row
  constexpr int CH = 16 / sizeof(CT), RC = 128 / CH;
  CT* base = reinterpret_cast<CT*>(isv ? o.Vc : o.Kc);
  for (int q = t; q < 128 * RC; q += 256) {
    const int r = q / RC, c = (q - r * RC) * CH;
    const int hh = c / o.hd, ch = c - hh * o.hd;
    const int m = mt * 128 + r;
    if (m < o.M) {
      const int e = m / o.frames, f = m - e * o.frames;
      CT* dst = base + (((int64_t)e * o.H + h0 + hh) * o.max_frames + f) * o.hd + ch;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(Cs + r * CLD + c);
    }
  }
}

// Block tile 256 rows of X x 128 output columns; eight waves as 4 x 2, each 64 x 64 (4 x 4 MFMA
// tiles).  Per 32-deep K step the block's 16 + 8 operand tiles (1 KB each, fragment order) are
// loaded once into LDS and every wave reads its 4 + 4 tiles from there, so each fragment
// leaves L2 once per block instead of once per wave.  The loads go straight from global
// memory (buffer loads with the LDS destination) into a ring of three LDS slots (no staging
// registers, no LDS stores); each step waits for its own loads by count and meets the other
// waves at a bare barrier (a full __syncthreads would also wait for the loads still in
// flight), and half of a step's MFMAs hide the fragment reads of the next.  Same XCD panel
// order and epilogue as k_xkv_frag, the 256 rows in two halves.  At most 128 VGPRs, so two
// workgroups share a CU.  (256 x 256 blocks of eight 128 x 64 waves, one workgroup per CU,
// measured slower: 22.3 against 21.0 ms per large-v3 window; reading each step's fragments
// after its barrier, loads two steps ahead: 20.6 against 20.1 ms.)
template <typename T, typename CT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_xkv_lds(const T* __restrict__ Xf, const T* __restrict__ Wf, int K,
                                                 XkvOut o, int n_mt, int n_nt, int pg) {
  constexpr int RT = 16, CTL = 8, NTL = RT + CTL;   // tiles per block and K step
  constexpr int CLD = 128 + 8;
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  constexpr int NSLOT = 3;
  __shared__ __align__(16) v4u stage[NSLOT][NTL * 64];        // 3 x 24 KB
  static_assert(sizeof(stage) >= 128 * CLD * sizeof(CT), "epilogue tile fits the staging buffers");
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // workgroup L runs on XCD L % 8; that XCD's j-th workgroup takes, within a group of pg of
  // its row panels, column tile j / pg of panel j % pg: the group's X panels stay in the XCD's
  // L2 while the W column tiles sweep past them, each W tile used pg times in a row
  const int L = blockIdx.x, xcd = L % 8, j = L / 8;
  const int grp = j / (pg * n_nt), w_in = j - grp * pg * n_nt;
  const int nt = w_in / pg, mt = xcd + 8 * (grp * pg + (w_in - nt * pg));
  if (mt >= n_mt) return;
  const int wm = wv & 3, wn = wv >> 2;
  const int KST = K >> 5, lr = lane & 15, lq = lane >> 4;
  const v4u* __restrict__ A = reinterpret_cast<const v4u*>(Xf) + (int64_t)mt * RT * KST * 64;
  const v4u* __restrict__ B = reinterpret_cast<const v4u*>(Wf) + (int64_t)nt * CTL * KST * 64;
  // a K step's 24 tiles go straight to LDS, wave wv loading tiles wv, 8 + wv (X) and 16 + wv
  // (W); the step index is clamped so every thread issues exactly 3 loads per step and the
  // vmcnt arithmetic below stays exact
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(A, RT * KST * 1024), rb = buf_rsrc(B, CTL * KST * 1024);
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int slot = st % NSLOT;
    st = min(st, KST - 1);
    const uint32_t so = (uint32_t)(st * 64 + lane) * 16;
    lds_dma16(ra, (uint32_t)wv * KST * 1024 + so, &stage[slot][wv * 64]);
    lds_dma16(ra, (uint32_t)(8 + wv) * KST * 1024 + so, &stage[slot][(8 + wv) * 64]);
    lds_dma16(rb, (uint32_t)wv * KST * 1024 + so, &stage[slot][(16 + wv) * 64]);
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Three slots, loads three K steps ahead of the MFMAs.  Step st: the reads of row tiles 2, 3
  // and the MFMAs of row tiles 0, 1 (their fragments and the column fragments read during
  // step st - 1); a barrier at which every thread's loads of step st + 1 have landed and every
  // wave has read all of slot st, so that slot takes the loads of st + 3; then the reads of
  // step st + 1's row tiles 0, 1 and column tiles, hidden behind the MFMAs of row tiles 2, 3.
  // Two register sets alternate by step (no copies, which would wait for the reads).
  auto rd_rows = [&](int st, int i0, v4u (&fa)[2]) __attribute__((always_inline)) {
    const v4u* S = stage[st % NSLOT];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = S[(wm * 4 + i0 + i) * 64 + lane];
  };
  auto rd_cols = [&](int st, v4u (&fb)[4]) __attribute__((always_inline)) {
    const v4u* S = stage[st % NSLOT];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) fb[jn] = S[(RT + wn * 4 + jn) * 64 + lane];
  };
  auto mfmas = [&](int i0, const v4u (&fa)[2], const v4u (&fb)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
        acc[i0 + i][jn] = mfma16x16x32(__builtin_bit_cast(uint4, fa[i]), __builtin_bit_cast(uint4, fb[jn]), acc[i0 + i][jn], (T*)nullptr);
  };
  auto step = [&](int st, const v4u (&pa)[2], const v4u (&pb)[4], v4u (&na)[2], v4u (&nb)[4]) __attribute__((always_inline)) {
    v4u qa[2];
    rd_rows(st, 2, qa);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0, pa, pb);
    __builtin_amdgcn_sched_barrier(0);    // (the scheduler would move MFMAs across the barrier)
    wait_vmcnt<3>();                      // this thread's loads of step st + 1 have landed
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of slot st are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(st + 3);
    rd_rows(st + 1, 0, na);               // past the end: a slot's stale tiles, never used
    rd_cols(st + 1, nb);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(2, qa, pb);
    __builtin_amdgcn_sched_barrier(0);
  };
  issue(0);
  issue(1);
  issue(2);
  wait_vmcnt<6>();                    // this thread's loads of step 0 have landed
  __builtin_amdgcn_s_barrier();       // ... and every thread's
  v4u a0[2], b0[4], a1[2], b1[4];
  rd_rows(0, 0, a0);
  rd_cols(0, b0);
  int st = 0;
  for (; st + 1 < KST; st += 2) {
    step(st, a0, b0, a1, b1);
    step(st + 1, a1, b1, a0, b0);
  }
  if (st < KST) step(st, a0, b0, a1, b1);
  wait_vmcnt<0>();                    // the clamped loads past the end land before LDS is reused
  __syncthreads();
  // epilogue through LDS (the staging buffers), 128 rows at a time: waves 0, 1 (rows 0..127)
  // then waves 2, 3 of each column half
  CT* Cs = reinterpret_cast<CT*>(&stage[0][0]);
  const int n0 = nt * 128;
  const bool isv = n0 >= o.d;
  const int h0 = (isv ? n0 - o.d : n0) / o.hd;   // first head of the tile (128 / hd heads)
  constexpr int CH = 16 / sizeof(CT), RC = 128 / CH;
  CT* base = reinterpret_cast<CT*>(isv ? o.Vc : o.Kc);
  for (int half = 0; half < 2; ++half) {
    if ((wm >> 1) == half) {
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        const float bias = o.bias[n0 + wn * 64 + jn * 16 + lr];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Cs[((wm & 1) * 64 + i * 16 + lq * 4 + e) * CLD + wn * 64 + jn * 16 + lr] = from_f<CT>(acc[i][jn][e] + bias);
      }
    }
    __syncthreads();
    for (int q = t; q < 128 * RC; q += 512) {
      const int r = q / RC, c = (q - r * RC) * CH;
      const int hh = c / o.hd, ch = c - hh * o.hd;
      const int m = mt * 256 + half * 128 + r;
      if (m < o.M) {
        const int e = m / o.frames, f = m - e * o.frames;
        CT* dst = base + (((int64_t)e * o.H + h0 + hh) * o.max_frames + f) * o.hd + ch;
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(Cs + r * CLD + c);
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
  // 16-bit: X already in fragment order (launch_pack_rows, rows padded to 256), W in fragment
  // order; 128 / hd heads per 128-column tile
  if ((hd != 64 && hd != 128) || d % 128 || (cache_dtype != DT_F16 && cache_dtype != DT_BF16)) return hipErrorInvalidValue;
  // 256-row blocks with LDS-shared operands once they fill the chip twice over (large-v3: 7500
  // blocks, 902 -> 704 us per layer; whisper-small 1128, 84.6 -> 81.0 us), else 128-row blocks
  // (whisper-base, one encoder set: 48 blocks of 256 rows took 17.4 us against 13.5 us).
  const bool lds = (int64_t)((M + 255) / 256) * (2 * d / 128) >= 512;
  if (lds) {
    constexpr int pg = 4;   // row panels per L2 group
    const int n_mt = (M + 255) / 256, n_nt = 2 * d / 128;
    const int per_xcd = ((n_mt + 7) / 8 + pg - 1) / pg * pg;   // panels per XCD, whole groups
    const dim3 grid(8 * per_xcd * n_nt);
#define WD_XKV(T_)                                                                                          \
  if (cache_dtype == DT_F16) k_xkv_lds<T_, f16_t><<<grid, 512, 0, s>>>((const T_*)X, (const T_*)W, d, o, n_mt, n_nt, pg); \
  else k_xkv_lds<T_, bf16_t><<<grid, 512, 0, s>>>((const T_*)X, (const T_*)W, d, o, n_mt, n_nt, pg);
    if (w_dtype == DT_F16) { WD_XKV(f16_t) }
    else if (w_dtype == DT_BF16) { WD_XKV(bf16_t) }
    else return hipErrorInvalidValue;
#undef WD_XKV
    return hipGetLastError();
  }
  const int n_mt = (M + 127) / 128, n_nt = 2 * d / 128;
  const dim3 grid(8 * ((n_mt + 7) / 8) * n_nt);
#define WD_XKV(T_)                                                                                          \
  if (cache_dtype == DT_F16) k_xkv_frag<T_, f16_t><<<grid, 256, 0, s>>>((const T_*)X, (const T_*)W, d, o, n_mt, n_nt); \
  else k_xkv_frag<T_, bf16_t><<<grid, 256, 0, s>>>((const T_*)X, (const T_*)W, d, o, n_mt, n_nt);
  if (w_dtype == DT_F16) { WD_XKV(f16_t) }
  else if (w_dtype == DT_BF16) { WD_XKV(bf16_t) }
  else return hipErrorInvalidValue;
#undef WD_XKV
  return hipGetLastError();
}

}  // namespace wd
