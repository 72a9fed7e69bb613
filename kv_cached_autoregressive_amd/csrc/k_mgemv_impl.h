// Skinny GEMM on the matrix cores for 16-bit weights: out[b, n] = sum_k W[n,k] y[b,k]
// over the B rows of one decoder step (B padded to 16, 32 or 64).
//
// The weights were repacked at load into MFMA fragment order, so each wave
// fetches one contiguous 1 KB tile (16 rows x 32 k) per 16-byte lane load and
// feeds it straight to v_mfma_f32_16x16x32 as the A operand.  The activations
// arrive from their producer (norm, attention, GELU/SwiGLU epilogue) already in
// the same fragment order and split into hi + lo 16-bit parts; every weight tile
// meets both parts, so the product keeps ~16 bits of each fp32 activation while
// the weights stream at their storage width.
//
// Work split: a wave owns NBW 16-row blocks and a 1/KS slice of K; the KS waves
// of a row tile sit in one workgroup and add their partial tiles through LDS
// (fixed order, so results are reproducible run to run).  Loads run one K step
// ahead of the MFMAs.  Epilogues: bias, scale, residual add, erf-GELU or SwiGLU
// written back in split fragment order for the next GEMM, the Whisper q|k|v split
// with the K/V cache append, and tied-head logits with per-block argmax keys.
//
// This file holds the kernels and shape policy; it is compiled as several translation units
// (k_mgemv*.hip) so the kernel instantiations of each weight dtype build in parallel.  The
// unit that defines WD_MG_MAIN holds the public launchers.
#pragma once
#include <algorithm>
#include <cstdio>
#include <type_traits>
#include <cstdlib>

#include "wd_common.h"
#include "wd_kernels.h"

namespace wd {

typedef __attribute__((ext_vector_type(8))) __bf16 mbf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 mf16x8_t;
typedef __attribute__((ext_vector_type(4))) float mf32x4_t;

__device__ __forceinline__ mf32x4_t mma(const uint4& a, const uint4& b, const mf32x4_t& c, bf16_t*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mbf16x8_t, a), __builtin_bit_cast(mbf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ mf32x4_t mma(const uint4& a, const uint4& b, const mf32x4_t& c, f16_t*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mf16x8_t, a), __builtin_bit_cast(mf16x8_t, b), c, 0, 0, 0);
}

typedef uint32_t mv4u __attribute__((ext_vector_type(4)));   // one 16-byte fragment slice
__device__ __forceinline__ mf32x4_t mma(const mv4u& a, const mv4u& b, const mf32x4_t& c, bf16_t*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mbf16x8_t, a), __builtin_bit_cast(mbf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ mf32x4_t mma(const mv4u& a, const mv4u& b, const mf32x4_t& c, f16_t*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mf16x8_t, a), __builtin_bit_cast(mf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float m_gelu(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float m_silu(float z) { return z / (1.0f + expf(-z)); }

template <typename CT>
__device__ __forceinline__ void put_cache(void* base, int64_t idx, float v) {
  reinterpret_cast<CT*>(base)[idx] = from_f<CT>(v);
}

template <typename T>
__device__ __forceinline__ void epi_one(const MGemvParams& p, int n, int b, float v) {
  const float bias = p.bias ? p.bias[n] : 0.f;
  switch (p.epi) {
    case EPI_STORE: p.out[(int64_t)b * p.ldo + n] = (v + bias) * p.scale; break;
    case EPI_RESID: atomicAdd(&p.out[(int64_t)b * p.ldo + n], v + bias); break;  // sole writer: x + v exactly
    case EPI_GELU_SPLIT: store_split<T>(p.yo_hi, p.yo_lo, frag_offset(b, n, p.N), m_gelu(v + bias)); break;
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
        if (p.cache_dtype == DT_F32) put_cache<float>(base, at, val);
        else if (p.cache_dtype == DT_F16) put_cache<f16_t>(base, at, val);
        else put_cache<bf16_t>(base, at, val);
      }
      break;
    }
    default: break;
  }
}

// Epilogue on the accumulator tiles of one wave.  The activations were the MFMA A
// operand, so tile (nb, bb) holds batch rows bb*16 + 4*(lane/16) + r along the
// registers and output column (tile*NBW + nb)*16 + lane%16 along the lanes: stores
// of one register index cover 16 consecutive outputs of 4 rows.  Only `active`
// waves hold final sums; all threads of the workgroup must call it (the logits
// path synchronises).  kmax: >= NBB*16 u64 of LDS.
template <typename T, int NBW, int NBB, int NW>
__device__ __forceinline__ void mg_epilogue(const MGemvParams& p, mf32x4_t (&acc)[NBW][NBB], bool active, int tile,
                                            int NB, unsigned long long* kmax) {
  const int lane = threadIdx.x & 63;
  const int rsub = (lane >> 4) * 4, col = lane & 15;

  if (p.epi == EPI_LOGITS) {
    __syncthreads();   // the caller's LDS buffer (aliased by kmax) is no longer read
    for (int i = threadIdx.x; i < NBB * 16; i += NW * 64) kmax[i] = 0ull;
    __syncthreads();
    if (active) {
#pragma unroll
      for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int b = bb * 16 + rsub + r;
          unsigned long long best = 0ull;
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            const int n = (tile * NBW + nb) * 16 + col;
            if (n < p.N && b < p.B && tile * NBW + nb < NB) {
              float v = acc[nb][bb][r];
              if (p.out) p.out[(int64_t)b * p.ldo + n] = v;
              if (v != v) { raise_err(p.err, ERR_NAN); v = -INFINITY; }
              const unsigned long long k = argmax_key(v, n);
              best = k > best ? k : best;
            }
          }
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {   // the 16 lanes holding row b
            const unsigned long long t = __shfl_xor(best, o, WAVE);
            best = t > best ? t : best;
          }
          if (col == 0 && b < p.B) atomicMax(&kmax[b], best);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < p.B; i += NW * 64) p.amax[(int64_t)blockIdx.x * p.ldp + i] = kmax[i];
    return;
  }
  if (!active) return;
  if (p.epi == EPI_SWIGLU_SPLIT) {  // row blocks alternate gate, up for the same 16 outputs
    const int half = p.N >> 1;
#pragma unroll
    for (int nb = 0; nb + 1 < NBW; nb += 2)
#pragma unroll
      for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = ((tile * NBW + nb) >> 1) * 16 + col;
          const int b = bb * 16 + rsub + r;
          if (j < half && b < p.B)
            store_split<T>(p.yo_hi, p.yo_lo, frag_offset(b, j, half), m_silu(acc[nb][bb][r]) * acc[nb + 1][bb][r]);
        }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = (tile * NBW + nb) * 16 + col;
        const int b = bb * 16 + rsub + r;
        if (n < p.N && b < p.B && tile * NBW + nb < NB) epi_one<T>(p, n, b, acc[nb][bb][r]);
      }
}

constexpr int mg_waves(int KS) { return KS >= 4 ? KS : 4; }

// Weights are read once per step: nontemporal loads keep them out of the L2's way
// (measured 3% on the Qwen3 step, 1% on the large-v3 step).
__device__ __forceinline__ mv4u wload(const mv4u* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint4 wload(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const mv4u*>(p)));
}

// A wave's steps past its last one (the ring overruns by up to D-1) load the last
// step again and multiply by zeroed weights: no load sits under a branch, so the
// compiler's wait counts keep D-1 steps of loads in flight.
__device__ __forceinline__ uint4 keep_if(const uint4& v, bool live) {
  const uint32_t m = live ? 0xffffffffu : 0u;
  return uint4{v.x & m, v.y & m, v.z & m, v.w & m};
}
__device__ __forceinline__ mv4u keep_if(const mv4u& v, bool live) {
  const uint32_t m = live ? 0xffffffffu : 0u;
  return v & m;
}

template <typename T, int NBW, int NBB, int KS, int D>
__global__ __launch_bounds__(64 * mg_waves(KS)) void k_mgemv(MGemvParams p) {
  constexpr int RT = KS >= 4 ? 1 : 4 / KS;   // row tiles per workgroup (>= 4 waves)
  constexpr int NW = RT * KS;                // waves per workgroup
  constexpr int REDF = KS > 1 ? NW * NBW * NBB * 256 : 0;
  constexpr int LDSF = REDF > NBB * 32 ? REDF : NBB * 32;   // argmax keys reuse the buffer
  __shared__ __align__(16) float red[LDSF];
  unsigned long long* kmax = reinterpret_cast<unsigned long long*>(red);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt = w % RT, ks = w / RT;
  const int tile = blockIdx.x * RT + rt;
  const int NB = (p.N + 15) >> 4;
  const int KST = p.K >> 5;
  const int s0 = (ks * KST) / KS, n = ((ks + 1) * KST) / KS - s0;   // n >= 1 (host: KS <= K/32)
  const uint4* __restrict__ Wv = reinterpret_cast<const uint4*>(p.W);
  const uint4* __restrict__ Yh = reinterpret_cast<const uint4*>(p.Yhi);
  const uint4* __restrict__ Yl = reinterpret_cast<const uint4*>(p.Ylo);

  int64_t wbase[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) wbase[nb] = (int64_t)min(tile * NBW + nb, NB - 1) * KST * 64 + lane;

  mf32x4_t acc[NBW][NBB];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb) acc[nb][bb] = mf32x4_t{0.f, 0.f, 0.f, 0.f};

  // ring of D k-steps of fragments: loads run D-1 steps ahead of the MFMAs
  uint4 wr[D][NBW], hr[D][NBB], lr[D][NBB];
  auto load = [&](int i, uint4 (&wd)[NBW], uint4 (&hd)[NBB], uint4 (&ld)[NBB]) __attribute__((always_inline)) {
    const int st = s0 + min(i, n - 1);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) wd[nb] = wload(Wv + wbase[nb] + (int64_t)st * 64);
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb) {
      const int64_t yi = ((int64_t)bb * KST + st) * 64 + lane;
      hd[bb] = Yh[yi];
      ld[bb] = Yl[yi];
    }
  };
#pragma unroll
  for (int j = 0; j < D - 1; ++j) load(j, wr[j], hr[j], lr[j]);
  for (int i = 0; i < n; i += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      constexpr int dummy = 0;
      (void)dummy;
      load(i + j + D - 1, wr[(j + D - 1) % D], hr[(j + D - 1) % D], lr[(j + D - 1) % D]);
      const bool live = i + j < n;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const uint4 wv = keep_if(wr[j][nb], live);
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb) {
          acc[nb][bb] = mma(hr[j][bb], wv, acc[nb][bb], (T*)nullptr);
          acc[nb][bb] = mma(lr[j][bb], wv, acc[nb][bb], (T*)nullptr);
        }
      }
    }
  }

  if constexpr (KS > 1) {  // add the K-slice partials of the row tile, fixed order
    if (ks > 0) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((w * NBW + nb) * NBB + bb) * 256 + r * 64 + lane] = acc[nb][bb][r];
    }
    __syncthreads();
    if (ks == 0) {
      for (int k2 = 1; k2 < KS; ++k2) {
        const int w2 = rt + k2 * RT;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nb][bb][r] += red[((w2 * NBW + nb) * NBB + bb) * 256 + r * 64 + lane];
      }
    }
  }
  mg_epilogue<T, NBW, NBB, NW>(p, acc, ks == 0, tile, NB, kmax);
}

// Latency-bound variant for the per-layer projections: a wave issues the loads of
// its whole weight slice (NS K steps x NBW tiles, K = KS * NS * 32 exactly) before
// the first MFMA, so the HBM round trip is paid about once per wave instead of
// once per step; the activation tiles (L2-resident) follow through a 3-deep
// register ring.  Straight-line code: every load stays in flight until its use.
template <typename T, int NBW, int NBB, int KS, int NS>
__global__ __launch_bounds__(64 * mg_waves(KS)) void k_mgemv_pf(MGemvParams p) {
  constexpr int RT = KS >= 4 ? 1 : 4 / KS;
  constexpr int NW = RT * KS;
  constexpr int DY = 3;
  constexpr int RED = KS > 1 ? NW * NBW * NBB * 256 : 0;
  constexpr int LDSF = RED > NBB * 32 ? RED : NBB * 32;
  __shared__ __align__(16) float red[LDSF];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt = w % RT, ks = w / RT;
  const int tile = blockIdx.x * RT + rt;
  const int NB = (p.N + 15) >> 4;
  constexpr int KST = KS * NS;
  const int s0 = ks * NS;
  const mv4u* __restrict__ Wv = reinterpret_cast<const mv4u*>(p.W);
  const mv4u* __restrict__ Yh = reinterpret_cast<const mv4u*>(p.Yhi);
  const mv4u* __restrict__ Yl = reinterpret_cast<const mv4u*>(p.Ylo);

  mv4u wr[NS][NBW];
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
      wr[i][nb] = wload(Wv + ((int64_t)min(tile * NBW + nb, NB - 1) * KST + s0 + i) * 64 + lane);

  mv4u hr[DY][NBB], lr[DY][NBB];
  auto loadY = [&](int i, mv4u (&h)[NBB], mv4u (&l)[NBB]) __attribute__((always_inline)) {
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb) {
      const int64_t yi = ((int64_t)bb * KST + s0 + i) * 64 + lane;
      h[bb] = Yh[yi];
      l[bb] = Yl[yi];
    }
  };
#pragma unroll
  for (int d = 0; d < DY - 1 && d < NS; ++d) loadY(d, hr[d], lr[d]);

  mf32x4_t acc[NBW][NBB];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb) acc[nb][bb] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i + DY - 1 < NS) loadY(i + DY - 1, hr[(i + DY - 1) % DY], lr[(i + DY - 1) % DY]);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int bb = 0; bb < NBB; ++bb) {
        acc[nb][bb] = mma(hr[i % DY][bb], wr[i][nb], acc[nb][bb], (T*)nullptr);
        acc[nb][bb] = mma(lr[i % DY][bb], wr[i][nb], acc[nb][bb], (T*)nullptr);
      }
  }

  if constexpr (KS > 1) {
    if (ks > 0) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((w * NBW + nb) * NBB + bb) * 256 + r * 64 + lane] = acc[nb][bb][r];
    }
    __syncthreads();
    if (ks == 0) {
      for (int k2 = 1; k2 < KS; ++k2) {
        const int w2 = rt + k2 * RT;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nb][bb][r] += red[((w2 * NBW + nb) * NBB + bb) * 256 + r * 64 + lane];
      }
    }
  }
  mg_epilogue<T, NBW, NBB, NW>(p, acc, ks == 0, tile, NB, reinterpret_cast<unsigned long long*>(red));
}

// Variant for B > 16: the RT waves of a K group share each K step's activation
// fragments through LDS (loaded once per group, double-buffered, one barrier per
// step), so activation traffic from L2 drops by RT; each wave streams only its own
// weight tiles, DW steps ahead.  KS groups split K inside the workgroup and add
// their partial tiles through LDS in fixed order.
template <typename T, int NBW, int NBB, int KS, int RT>
__global__ __launch_bounds__(64 * KS * RT) void k_mgemv_lds(MGemvParams p) {
  constexpr int NW = KS * RT;
  constexpr int FR = 2 * NBB;                 // activation tiles per K step (hi, lo per 16 rows)
  constexpr int LPT = (FR + RT - 1) / RT;     // tile loads per thread of a group
  constexpr int DY = 4, DW = 4;               // register lead of activation / weight loads
  constexpr int YB = KS * 2 * FR * 64;        // mv4u of the double-buffered staging
  constexpr int RB = (NW * NBW * NBB * 256 + 3) / 4;   // mv4u of the reduction buffer
  constexpr int LB = YB > RB ? YB : RB;
  __shared__ mv4u lds[LB > NBB * 8 ? LB : NBB * 8];   // staging, then reduction, then argmax keys
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt = w % RT, ks = w / RT;
  const int tg = rt * 64 + lane;              // thread index inside the K group
  const int NB = (p.N + 15) >> 4;
  const int KST = p.K >> 5;
  const int s0 = (ks * KST) / KS, n = ((ks + 1) * KST) / KS - s0;   // n >= 1 (host: KS <= K/32)
  const int iters = (KST + KS - 1) / KS;      // uniform trip count over the workgroup
  const mv4u* __restrict__ Wv = reinterpret_cast<const mv4u*>(p.W);
  const mv4u* __restrict__ Yh = reinterpret_cast<const mv4u*>(p.Yhi);
  const mv4u* __restrict__ Yl = reinterpret_cast<const mv4u*>(p.Ylo);
  mv4u* ybuf = lds + (size_t)ks * 2 * FR * 64;

  const int blk0 = blockIdx.x * RT * NBW + rt * NBW;
  int64_t wbase[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) wbase[nb] = (int64_t)min(blk0 + nb, NB - 1) * KST * 64 + lane;

  mf32x4_t acc[NBW][NBB];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb) acc[nb][bb] = mf32x4_t{0.f, 0.f, 0.f, 0.f};

  // Steps past a group's last one reload its last step (and its MFMAs see zeroed
  // weights): no global load sits under a branch, so the wait counts stay exact.
  mv4u yr[DY][LPT], wr[DW][NBW];
  auto loadY = [&](int i, mv4u (&dst)[LPT]) __attribute__((always_inline)) {
    const int st = s0 + min(i, n - 1);
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int flat = tg + j * RT * 64, f = min(flat >> 6, FR - 1);
      const int64_t gi = ((int64_t)(f >> 1) * KST + st) * 64 + (flat & 63);
      const mv4u* src = (f & 1) ? Yl : Yh;
      dst[j] = src[gi];
    }
  };
  auto storeY = [&](int slot, const mv4u (&src)[LPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int flat = tg + j * RT * 64;
      if (FR % RT == 0 || (flat >> 6) < FR) ybuf[(size_t)slot * FR * 64 + flat] = src[j];
    }
  };
  auto loadW = [&](int i, mv4u (&dst)[NBW]) __attribute__((always_inline)) {
    const int st = s0 + min(i, n - 1);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) dst[nb] = wload(Wv + wbase[nb] + (int64_t)st * 64);
  };

#pragma unroll
  for (int d = 0; d < DY; ++d) loadY(d, yr[d]);
#pragma unroll
  for (int d = 0; d < DW - 1; ++d) loadW(d, wr[d]);
  storeY(0, yr[0]);

  // one K step; U is a compile-time constant so every ring index is static
  auto step = [&](int i, auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    __syncthreads();                        // step i's tiles visible; the other slot is free
    storeY((u + 1) & 1, yr[(u + 1) % DY]);
    loadY(i + DY, yr[u % DY]);
    loadW(i + DW - 1, wr[(u + DW - 1) % DW]);
    const bool live = i < n;
    const mv4u* yb = ybuf + (size_t)(u & 1) * FR * 64;
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb) {
      const mv4u h = yb[(2 * bb) * 64 + lane];
      const mv4u l = yb[(2 * bb + 1) * 64 + lane];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const mv4u wv = keep_if(wr[u % DW][nb], live);
        acc[nb][bb] = mma(h, wv, acc[nb][bb], (T*)nullptr);
        acc[nb][bb] = mma(l, wv, acc[nb][bb], (T*)nullptr);
      }
    }
  };
  for (int i0 = 0; i0 < iters; i0 += 4) {   // trip counts uniform over the workgroup
    step(i0, std::integral_constant<int, 0>{});
    step(i0 + 1, std::integral_constant<int, 1>{});
    step(i0 + 2, std::integral_constant<int, 2>{});
    step(i0 + 3, std::integral_constant<int, 3>{});
  }

  float* red = reinterpret_cast<float*>(lds);
  if constexpr (KS > 1) {
    __syncthreads();  // staging no longer read
    if (ks > 0) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((w * NBW + nb) * NBB + bb) * 256 + r * 64 + lane] = acc[nb][bb][r];
    }
    __syncthreads();
    if (ks == 0) {
      for (int k2 = 1; k2 < KS; ++k2) {
        const int w2 = rt + k2 * RT;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nb][bb][r] += red[((w2 * NBW + nb) * NBB + bb) * 256 + r * 64 + lane];
      }
    }
  }
  __syncthreads();  // the buffer is reused for argmax keys
  mg_epilogue<T, NBW, NBB, NW>(p, acc, ks == 0, blk0 / NBW, NB, reinterpret_cast<unsigned long long*>(lds));
}

// Split-K skinny GEMM for any B (16-, 32- or 64-row tiles).  At 32..64 rows the activations
// of a K step (hi + lo, 4-8 KB) outweigh its weight tile, so the kernel is shaped around
// reading them as rarely as possible, and at every B the K split gives enough workgroups:
// a workgroup of NWV waves owns NWV*NBW 16-row tiles (64..128 outputs) and one of G groups of
// at most S K steps.  Every load of the group is issued up front (a step's activation slice,
// then its weight tiles); the activations are staged once in LDS behind one barrier (a
// barrier per step measured slower: its LDS round trips outweigh the overlap), and each
// wave then runs the MFMAs of all its steps back to back.  With G > 1 the K groups write fp32
// partials part[g][b][n] that the consumer adds in order (the next norm for a residual, the
// attention prologue for q and the appended K/V row, else launch_mgemv_finish); with G == 1
// the usual epilogue runs here.
template <typename T, int NBW, int NBB, int S, int KS>
__global__ __launch_bounds__(256 * KS) void k_mgemv_sk(MGemvParams p) {
  // 4 column waves x KS K slices: the KS waves of a column tile take alternate steps of the
  // group (more waves per CU keep more loads in flight) and add up through LDS at the end
  constexpr int NWV = 4, NW = NWV * KS;
  constexpr int YT = NBB * 2;                              // activation tiles of one step
  constexpr int PER = (YT * 64 + 64 * NW - 1) / (64 * NW);  // staging loads per thread per step
  constexpr int STAGE = S * YT * 64;                       // mv4u of the staging buffer
  constexpr int RED = KS > 1 ? (NW - NWV) * NBW * NBB * 64 : 0;   // mv4u of the K-slice partials
  __shared__ mv4u ys[(STAGE > RED ? STAGE : RED) > NBB * 8 ? (STAGE > RED ? STAGE : RED) : NBB * 8];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = w % NWV, ks = w / NWV;
  const int NB = (p.N + 15) >> 4;
  const int KST = p.K >> 5;
  const int G = p.part_G;
  // Workgroups go to the 8 XCDs round-robin by launch index.  With G a multiple of 8, K
  // group g runs on XCD g % 8 for every column group, so each XCD's L2 fetches only its own
  // eighth of the activations; otherwise column groups take G consecutive indices.
  const int L = blockIdx.x;
  int g, cg;
  if (G % 8 == 0) {
    const int gx = G / 8, xcd = L % 8, q = L / 8;
    g = xcd + 8 * (q % gx);
    cg = q / gx;
  } else {
    g = L % G;
    cg = L / G;
  }
  const int s_lo = (g * KST) / G, n = ((g + 1) * KST) / G - s_lo;   // 1 <= n <= S (host)
  const int tile = cg * NWV + cw;                                   // this wave's group of NBW tiles
  const mv4u* __restrict__ Wv = reinterpret_cast<const mv4u*>(p.W);
  const mv4u* __restrict__ Yh = reinterpret_cast<const mv4u*>(p.Yhi);
  const mv4u* __restrict__ Yl = reinterpret_cast<const mv4u*>(p.Ylo);
  int64_t wbase[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) wbase[nb] = (int64_t)min(tile * NBW + nb, NB - 1) * KST * 64 + lane;

  // all loads up front, in step order (steps past n reload step n-1; their MFMAs see zero
  // weights); a wave loads the weight tiles of its own steps only
  constexpr int SW = (S + KS - 1) / KS;                    // steps per K slice
  mv4u yr[S][PER], wr[SW][NBW];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int st = s_lo + min(i, n - 1);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int flat = min((int)threadIdx.x + j * 64 * NW, YT * 64 - 1);
      const int t = flat >> 6;                    // tile: row block t/2, hi or lo by t%2
      const mv4u* src = (t & 1) ? Yl : Yh;
      yr[i][j] = src[((int64_t)(t >> 1) * KST + st) * 64 + (flat & 63)];
    }
    if (i % KS == 0) {
      const int mine = s_lo + min(i + ks, n - 1);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) wr[i / KS][nb] = wload(Wv + wbase[nb] + (int64_t)mine * 64);
    }
  }

  mf32x4_t acc[NBW][NBB];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb) acc[nb][bb] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < S; ++i) {
    mv4u* slot = ys + i * YT * 64;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int flat = threadIdx.x + j * 64 * NW;
      if ((YT * 64) % (64 * NW) == 0 || flat < YT * 64) slot[flat] = yr[i][j];
    }
  }
  __syncthreads();   // every step's activation tiles are in LDS
#pragma unroll
  for (int i0 = 0; i0 < S; i0 += KS) {
    const int mi = i0 + ks;                       // this K slice's step
    const bool live = mi < n && mi < S;
    mv4u wv[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) wv[nb] = keep_if(wr[i0 / KS][nb], live);
    const mv4u* sl = ys + min(mi, S - 1) * YT * 64;
#pragma unroll
    for (int part = 0; part < 2; ++part)          // hi then lo: consecutive MFMAs are independent
#pragma unroll
      for (int bb = 0; bb < NBB; ++bb) {
        const mv4u y = sl[(bb * 2 + part) * 64 + lane];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[nb][bb] = mma(y, wv[nb], acc[nb][bb], (T*)nullptr);
      }
  }
  if constexpr (KS > 1) {   // add the K slices of each column tile, fixed order
    __syncthreads();        // the staging buffer is reused for the slice partials
    float* red = reinterpret_cast<float*>(ys);
    if (ks > 0) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[((((ks - 1) * NWV + cw) * NBW + nb) * NBB + bb) * 256 + r * 64 + lane] = acc[nb][bb][r];
    }
    __syncthreads();
    if (ks == 0) {
      for (int k2 = 1; k2 < KS; ++k2)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[nb][bb][r] += red[((((k2 - 1) * NWV + cw) * NBW + nb) * NBB + bb) * 256 + r * 64 + lane];
    }
  }
  if (G == 1) {
    __syncthreads();   // the staging buffer is reused for argmax keys
    mg_epilogue<T, NBW, NBB, NW>(p, acc, ks == 0, tile, NB, reinterpret_cast<unsigned long long*>(ys));
    return;
  }
  if (ks != 0) return;
  const int rsub = (lane >> 4) * 4, col = lane & 15;
  float* P = p.part + (int64_t)g * p.B * p.N;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int nn = (tile * NBW + nb) * 16 + col, b = bb * 16 + rsub + r;
        if (nn < p.N && b < p.B && tile * NBW + nb < NB) {
          // 32-64 rows: megabytes of partials, read once by the next kernel, go around the L2
          // (2.5% on the large-v3 step); up to 16 rows they stay cached (slower otherwise)
          if constexpr (NBB > 1) __builtin_nontemporal_store(acc[nb][bb][r], &P[(int64_t)b * p.N + nn]);
          else P[(int64_t)b * p.N + nn] = acc[nb][bb][r];
        }
      }
}

// Sum of the G partials of each output (in order), then the launch's epilogue.
template <typename T, int GMAX>
__global__ __launch_bounds__(256) void k_mgemv_finish(MGemvParams p, int G) {
  const bool swiglu = p.epi == EPI_SWIGLU_SPLIT;
  const int cols = swiglu ? p.N >> 1 : p.N;
  const int64_t total = (int64_t)p.B * cols, slab = (int64_t)p.B * p.N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int b = (int)(e / cols), j = (int)(e - (int64_t)b * cols);
    if (swiglu) {   // gate and up of output j sit in consecutive 16-row blocks
      const int ng = (j >> 4) * 32 + (j & 15);
      const float* P = p.part + (int64_t)b * p.N + ng;
      const float vg = sum_parts<GMAX>(P, slab, G), vu = sum_parts<GMAX>(P + 16, slab, G);
      store_split<T>(p.yo_hi, p.yo_lo, frag_offset(b, j, cols), m_silu(vg) * vu);
    } else {
      epi_one<T>(p, j, b, sum_parts<GMAX>(p.part + (int64_t)b * p.N + j, slab, G));
    }
  }
}

struct SkShape { int NBW, NBB, G, NSC; };
// per-dtype entry points, each defined in its own translation unit
hipError_t mrun_bf16(const MGemvParams& p, hipStream_t st);
hipError_t mrun_f16(const MGemvParams& p, hipStream_t st);
// Split-K shape: 4 waves per workgroup, NBW = 2 (128 outputs) for the wide or deep
// projections; S K steps per group so that ~256 workgroups cover the shape (2 <= S <= 8),
// G = ceil(K steps / S), and the LDS chunk is 4 or 8 steps (no padded steps for S <= 4).
static bool sk_pick(int N, int K, int B, int epi, SkShape& s) {
  if (epi == EPI_LOGITS) return false;
  const int NB = (N + 15) / 16, KST = K / 32;
  s.NBB = B <= 16 ? 1 : B <= 32 ? 2 : 4;
  // (SwiGLU's in-kernel epilogue needs gate and up in one wave: NBW = 2)
  s.NBW = (NB >= 256 || KST >= 128 || epi == EPI_SWIGLU_SPLIT) ? 2 : 1;
  // up to 16 rows and at least 8 MB of 16-bit weights: 16-column tiles and K groups of up to
  // 16 steps (half the partial slabs of 8-step groups; measured 14.4 -> 13.3 us on the Qwen3
  // gate|up, 4.7% on its step)
  const bool narrow = s.NBB == 1 && (epi != EPI_SWIGLU_SPLIT || KST > 16) &&
                      (int64_t)KST * ((NB + 3) / 4) >= 8 * 256;
  if (narrow) s.NBW = 1;
  int ncg = (NB + 4 * s.NBW - 1) / (4 * s.NBW);
  int S = (KST * ncg + 255) / 256;
  S = std::max(2, std::min(S, narrow ? 16 : 8));
  int G = (KST + S - 1) / S;
  if (narrow) {
    if (G > 32) return false;
    s.G = G;
    s.NSC = std::max(4, (KST + G - 1) / G);
    if (s.NSC > 8) s.NSC = 16;   // instantiated: 4..8 and 16 (steps past a group's end are padding)
    return true;
  }
  if (ncg * G > 256 && s.NBW == 1) {   // past one workgroup per CU: wider column groups
    s.NBW = 2;
    ncg = (NB + 7) / 8;
    S = std::max(2, std::min((KST * ncg + 255) / 256, 8));
    G = (KST + S - 1) / S;
  }
  // narrow outputs (N <= 2048): every XCD would fetch all the activations, which weigh as
  // much as the partials; with G a multiple of 8 each XCD fetches one K eighth of them
  if (N <= 2048 && KST >= 16) G = 8 * ((KST + 63) / 64);
  if (G > 32) return false;             // the consumers add at most 32 partial slabs
  s.G = G;
  s.NSC = std::max(4, (KST + G - 1) / G);   // the longest group's steps (4..8): at most one padded step
  if (s.NSC > 8) s.NSC = 16;
  return true;
}
#ifdef WD_MG_MAIN
int mgemv_groups(int N, int K, int B, int epi) {
  SkShape s;
  return sk_pick(N, K, B, epi, s) ? s.G : 1;
}
#endif  // WD_MG_MAIN

template <typename T>
static hipError_t skrun(const MGemvParams& p0, const SkShape& s, hipStream_t st) {
  const int NB = (p0.N + 15) / 16;
  const int ncg = (NB + 4 * s.NBW - 1) / (4 * s.NBW);
  if (s.G > 1 && (!p0.part || (int64_t)s.G * p0.B * p0.N > p0.part_cap)) return hipErrorInvalidValue;
  MGemvParams p = p0;
  p.part_G = s.G;
  const dim3 grid(ncg * s.G);
#define WD_SK(NBW_, NBB_, NSC_)                                                  \
  if (s.NBW == NBW_ && s.NBB == NBB_ && s.NSC == NSC_) {                         \
    k_mgemv_sk<T, NBW_, NBB_, NSC_, 1><<<grid, 256, 0, st>>>(p);                 \
    return hipGetLastError();                                                    \
  }
#define WD_SK_S(S_) WD_SK(1, 1, S_) WD_SK(2, 1, S_) WD_SK(1, 2, S_) WD_SK(2, 2, S_) WD_SK(1, 4, S_) WD_SK(2, 4, S_)
  WD_SK_S(4) WD_SK_S(5) WD_SK_S(6) WD_SK_S(7) WD_SK_S(8) WD_SK(1, 1, 16) WD_SK(2, 1, 16)
#undef WD_SK_S
#undef WD_SK
  return hipErrorInvalidValue;
}

#ifdef WD_MG_MAIN
hipError_t launch_mgemv_finish(const MGemvParams& p, int G, hipStream_t s) {
  if (G < 1 || !p.part || p.B <= 0 || p.N <= 0 || (int64_t)G * p.B * p.N > p.part_cap) return hipErrorInvalidValue;
  if (p.epi == EPI_LOGITS) return hipErrorInvalidValue;
  if (G > 32) return hipErrorInvalidValue;
  const int64_t total = (int64_t)p.B * p.N;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
#define WD_FIN(T_)                                                                                \
  if (G <= 4) k_mgemv_finish<T_, 4><<<blocks, 256, 0, s>>>(p, G);                                 \
  else if (G <= 8) k_mgemv_finish<T_, 8><<<blocks, 256, 0, s>>>(p, G);                            \
  else if (G <= 16) k_mgemv_finish<T_, 16><<<blocks, 256, 0, s>>>(p, G);                          \
  else k_mgemv_finish<T_, 32><<<blocks, 256, 0, s>>>(p, G);
  if (p.w_dtype == DT_BF16) { WD_FIN(bf16_t) }
  else if (p.w_dtype == DT_F16) { WD_FIN(f16_t) }
  else return hipErrorInvalidValue;
#undef WD_FIN
  return hipGetLastError();
}
#endif  // WD_MG_MAIN

struct MShape { int NBW, NBB, KS; };
// Shape per projection: enough waves in flight for a weight stream of a few MB, K split
// over the waves of a workgroup so each walks at most ~10 K steps, and several 16-row
// blocks per wave where N is large (fewer activation re-reads per weight byte).
static MShape mpick(int N, int K, int B, int epi) {
  MShape s;
  s.NBB = B <= 16 ? 1 : (B <= 32 ? 2 : 4);
  const int nblocks = (N + 15) / 16, ksteps = K / 32;
  if (nblocks >= 1024) {
    // the tied head: 2 row blocks per wave, twice the workgroups of 4 (whisper-small head 19.1
    // -> 17.1 us, 203 -> 406 workgroups on 256 CUs; Qwen3 head 112.2 -> 111.1 us)
    s.NBW = 2;
    s.KS = (s.NBW == 2 && ksteps >= 32) ? 2 : 1;
  } else if (nblocks >= 128 || epi == EPI_SWIGLU_SPLIT) {
    s.NBW = 2;
    s.KS = ksteps >= 64 ? 8 : 4;
  } else {
    s.NBW = 1;
    s.KS = ksteps >= 96 ? 16 : (ksteps >= 32 ? 8 : 4);
    if (s.NBB == 4 && s.KS > 8) s.KS = 8;   // 16 waves x 64-wide tiles would spill
  }
  if (s.KS > ksteps) { s.NBW = 2; s.KS = 1; }   // every wave needs at least one K step
  return s;
}
static int rows_per_block(const MShape& s) { return s.NBW * (s.KS >= 4 ? 1 : 4 / s.KS); }

struct LShape { int NBW, KS, RT; };
static LShape lpick(int N, int K, int epi);
static int lds_blocks(const LShape& s, int N);
// The LDS-shared variant pays off where many waves re-read the same activation
// tiles: the large-N shapes (the tied head) at B > 16.
static bool use_lds(int N, int NBB) { return NBB > 1 && (N + 15) / 16 >= 1024; }
#ifdef WD_MG_MAIN
int mgemv_blocks_k(int N, int K, int B) {
  const MShape s = mpick(N, K, B, EPI_LOGITS);
  if (use_lds(N, s.NBB)) return lds_blocks(lpick(N, K, EPI_LOGITS), N);
  return ((N + 15) / 16 + rows_per_block(s) - 1) / rows_per_block(s);
}
#endif  // WD_MG_MAIN
#ifdef WD_MG_MAIN
int mgemv_blocks(int N, int B) {
  int most = 1;
  for (int K : {32, 1024, 2048, 4096, 8192})  // the logits launch has K = d; cover any K
    for (int b = 1; b <= B; b += 15) most = std::max(most, mgemv_blocks_k(N, K, std::min(b, B)));
  return std::max(most, mgemv_blocks_k(N, 32, B));
}
#endif  // WD_MG_MAIN

constexpr int DEPTH = 3;

template <typename T, int NBB>
static hipError_t mrun_b(const MGemvParams& p, const MShape& s, hipStream_t st) {
  const int per = rows_per_block(s);
  const int grid = ((p.N + 15) / 16 + per - 1) / per;
  const int threads = 64 * (s.KS >= 4 ? s.KS : 4);
#define WD_MG(NBW_, KS_) \
  if (s.NBW == NBW_ && s.KS == KS_) { k_mgemv<T, NBW_, NBB, KS_, DEPTH><<<grid, threads, 0, st>>>(p); return hipGetLastError(); }
  if constexpr (NBB < 4) { WD_MG(4, 1) }
  WD_MG(2, 1) WD_MG(2, 2) WD_MG(2, 4) WD_MG(2, 8)
  WD_MG(1, 4) WD_MG(1, 8)
  if constexpr (NBB < 4) { WD_MG(1, 16) }
#undef WD_MG
  return hipErrorInvalidValue;
}

// Shapes of the LDS-shared variant (B > 16): NBW rows-blocks per wave, KS K groups,
// RT waves sharing each group's activation tiles.
static LShape lpick(int N, int K, int epi) {
  const int nblocks = (N + 15) / 16;
  LShape s;
  if (nblocks >= 1024) s = {2, 1, 4};
  else if (nblocks >= 128 || epi == EPI_SWIGLU_SPLIT) s = {2, 4, 2};
  else s = {1, 8, 2};
  if (s.KS > K / 32) s = {2, 1, 4};   // every K group needs at least one step
  return s;
}
static int lds_blocks(const LShape& s, int N) { return ((N + 15) / 16 + s.RT * s.NBW - 1) / (s.RT * s.NBW); }

template <typename T, int NBB>
static hipError_t lrun(const MGemvParams& p, const LShape& s, hipStream_t st) {
  const int grid = lds_blocks(s, p.N);
#define WD_ML(NBW_, KS_, RT_) \
  if (s.NBW == NBW_ && s.KS == KS_ && s.RT == RT_) { \
    k_mgemv_lds<T, NBW_, NBB, KS_, RT_><<<grid, 64 * KS_ * RT_, 0, st>>>(p); return hipGetLastError(); }
  WD_ML(1, 4, 2) WD_ML(1, 2, 4) WD_ML(1, 4, 4)
  if constexpr (NBB < 4) { WD_ML(1, 8, 2) }   // 1024 threads x 64-wide tiles would spill
  WD_ML(2, 1, 4) WD_ML(2, 2, 4) WD_ML(2, 4, 2) WD_ML(2, 4, 4) WD_ML(2, 2, 2)
#undef WD_ML
  return hipErrorInvalidValue;
}

// Shape of the prefetch variant: NBW tiles per wave and K = KS waves x NS steps
// exactly, NS <= 12 so a wave's weight slice fits in registers.  Shapes without
// an exact split (or B in 17..32) take the ring kernel.
struct PShape { int NBW, NBB, KS, NS; };
static bool pf_pick(int N, int K, int B, int epi, PShape& s) {
  const int nblocks = (N + 15) / 16, kst = K / 32;
  if (nblocks >= 1024) return false;
  s.NBB = B <= 16 ? 1 : (B <= 32 ? 2 : 4);
  if (s.NBB == 2) return false;
  s.NBW = (nblocks >= 128 || epi == EPI_SWIGLU_SPLIT) ? 2 : 1;
  static const int split[][3] = {{12, 2, 6},  {16, 2, 8},  {24, 4, 6},   {32, 4, 8},    {40, 4, 10},   {48, 8, 6},
                                 {64, 8, 8},  {80, 8, 10}, {96, 16, 6}, {128, 16, 8}, {160, 16, 10}, {192, 16, 12}};
  for (const auto& t : split)
    if (t[0] == kst) {
      s.KS = t[1];
      s.NS = t[2];
      return !(s.KS == 16 && s.NBB * s.NBW >= 2);   // 1024-thread groups: 128 VGPRs
    }
  return false;
}

template <typename T, int NBB>
static hipError_t pfrun(const MGemvParams& p, const PShape& s, hipStream_t st) {
  const int per = s.NBW * (s.KS >= 4 ? 1 : 4 / s.KS);
  const int grid = ((p.N + 15) / 16 + per - 1) / per;
  const int threads = 64 * (s.KS >= 4 ? s.KS : 4);
#define WD_PF(NBW_, KS_, NS_)                                                              \
  if (s.NBW == NBW_ && s.KS == KS_ && s.NS == NS_) {                                       \
    k_mgemv_pf<T, NBW_, NBB, KS_, NS_><<<grid, threads, 0, st>>>(p);                       \
    return hipGetLastError();                                                              \
  }
#define WD_PF_ALL(NBW_) \
  WD_PF(NBW_, 2, 6) WD_PF(NBW_, 2, 8) WD_PF(NBW_, 4, 6) WD_PF(NBW_, 4, 8) WD_PF(NBW_, 4, 10) \
  WD_PF(NBW_, 8, 6) WD_PF(NBW_, 8, 8) WD_PF(NBW_, 8, 10)
  WD_PF_ALL(1) WD_PF_ALL(2)
  if constexpr (NBB == 1) { WD_PF(1, 16, 6) WD_PF(1, 16, 8) WD_PF(1, 16, 10) WD_PF(1, 16, 12) }
#undef WD_PF_ALL
#undef WD_PF
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t mrun(const MGemvParams& p, hipStream_t st) {
  SkShape sk;
  if (sk_pick(p.N, p.K, p.B, p.epi, sk)) return skrun<T>(p, sk, st);
  PShape pf;
  if (p.epi != EPI_LOGITS && pf_pick(p.N, p.K, p.B, p.epi, pf)) {
    if (pf.NBB == 1) return pfrun<T, 1>(p, pf, st);
    return pfrun<T, 4>(p, pf, st);
  }
  const MShape s = mpick(p.N, p.K, p.B, p.epi);
  if (s.NBB == 1) return mrun_b<T, 1>(p, s, st);
  if (use_lds(p.N, s.NBB)) {
    const LShape l = lpick(p.N, p.K, p.epi);
    if (s.NBB == 2) return lrun<T, 2>(p, l, st);
    return lrun<T, 4>(p, l, st);
  }
  if (s.NBB == 2) return mrun_b<T, 2>(p, s, st);
  return mrun_b<T, 4>(p, s, st);
}

#ifdef WD_MG_MAIN
hipError_t launch_mgemv(const MGemvParams& p, hipStream_t s) {
  if (p.N <= 0 || p.K <= 0 || (p.K % 32) || p.B <= 0 || p.B > 64 || !p.W || !p.Yhi || !p.Ylo)
    return hipErrorInvalidValue;
  switch (p.epi) {
    case EPI_STORE: case EPI_RESID: if (!p.out) return hipErrorInvalidValue; break;
    case EPI_GELU_SPLIT: if (!p.yo_hi || !p.yo_lo) return hipErrorInvalidValue; break;
    case EPI_SWIGLU_SPLIT: if (!p.yo_hi || !p.yo_lo || (p.N % 32)) return hipErrorInvalidValue; break;
    case EPI_QKV:
      if (!p.out || p.N != 3 * p.d || !p.pos || !p.Kc || !p.Vc || p.hd <= 0 || p.d != p.H * p.hd)
        return hipErrorInvalidValue;
      break;
    case EPI_LOGITS: if (!p.amax || p.ldp < p.B) return hipErrorInvalidValue; break;
    default: return hipErrorInvalidValue;
  }
  if (p.w_dtype == DT_BF16) return mrun_bf16(p, s);
  if (p.w_dtype == DT_F16) return mrun_f16(p, s);
  return hipErrorInvalidValue;
}
#endif  // WD_MG_MAIN

}  // namespace wd
