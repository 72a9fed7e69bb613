// Batched prompt prefill of the Qwen3-ASR language model (transcribe.cpp qwen3_asr/decoder.h
// `PrefillBuild` / `PrefillBuildBatched`: the whole prompt in one graph, audio embeddings
// spliced in at an offset, causal attention, K/V written for every prompt position).
//
// The prompt is processed in chunks of positions; the rows of a chunk are (stream b,
// position t0 + j) in the order r = b * C + j.  Per layer a chunk runs: RMSNorm (the decode
// step's norm kernel over R rows), the q|k|v projection as a dense MFMA GEMM, the per-head
// q/k norm + RoPE + K/V append (the decode step's kernel with a row -> stream map), causal
// attention over cache rows 0..t of each row's stream, the out projection with the residual
// add, RMSNorm, gate|up with the SwiGLU epilogue, and down with the residual add.
//
// This file: the chunk's embedding rows, the dense GEMM over fragment-layout operands, and
// the causal prefill attention.
#include <algorithm>

#include "wd_common.h"
#include "wd_kernels.h"

namespace wd {

typedef __attribute__((ext_vector_type(8))) __bf16 pbf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 pf16x8_t;
typedef __attribute__((ext_vector_type(4))) float pf32x4_t;
typedef uint32_t pv4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ pf32x4_t pmma(const pv4u& a, const pv4u& b, const pf32x4_t& c, bf16_t*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pbf16x8_t, a), __builtin_bit_cast(pbf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ pf32x4_t pmma(const pv4u& a, const pv4u& b, const pf32x4_t& c, f16_t*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(pf16x8_t, a), __builtin_bit_cast(pf16x8_t, b), c, 0, 0, 0);
}

// ---- chunk embedding rows --------------------------------------------------------------------
// x[b*C + j] = audio row (offset <= t < offset + A) or E[tokens[b*T + t]], t = t0 + j, for
// j < Cn; rows j >= Cn are zero.  pos[b*C + j] = t (or -1 past Cn).  E is in fragment layout.
template <typename WT>
__global__ __launch_bounds__(256) void k_pf_embed(float* __restrict__ x, int32_t* __restrict__ pos,
                                                  const WT* __restrict__ E, const int32_t* __restrict__ tokens,
                                                  int T, const WT* __restrict__ emb, int A, int offset, int t0,
                                                  int C, int Cn, int d, int V, unsigned* err) {
  const int r = blockIdx.x, b = r / C, j = r - b * C, t = t0 + j;
  float* xr = x + (int64_t)r * d;
  if (j >= Cn) {
    for (int i = threadIdx.x; i < d; i += 256) xr[i] = 0.f;
    if (threadIdx.x == 0) pos[r] = -1;
    return;
  }
  if (threadIdx.x == 0) pos[r] = t;
  if (emb && t >= offset && t < offset + A) {
    const WT* er = emb + ((int64_t)b * A + (t - offset)) * d;
    for (int i = threadIdx.x; i < d; i += 256) xr[i] = to_f(er[i]);
    return;
  }
  const int tok = tokens[(int64_t)b * T + t];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0) raise_err(err, ERR_TOKEN);
    for (int i = threadIdx.x; i < d; i += 256) xr[i] = 0.f;
    return;
  }
  for (int i = threadIdx.x; i < d; i += 256) xr[i] = to_f(E[frag_offset(tok, i, d)]);
}

hipError_t launch_pf_embed(float* x, int32_t* pos, const void* E, int w_dtype, const int32_t* tokens, int T,
                           const void* emb, int A, int offset, int t0, int B, int C, int Cn, int d, int V,
                           unsigned* err, hipStream_t s) {
  if (B <= 0 || C <= 0 || Cn <= 0 || Cn > C || !tokens || !x || !pos || d % 32 || (A > 0 && !emb)) return hipErrorInvalidValue;
  if (w_dtype == DT_BF16)
    k_pf_embed<bf16_t><<<B * C, 256, 0, s>>>(x, pos, (const bf16_t*)E, tokens, T, (const bf16_t*)emb, A, offset, t0, C,
                                             Cn, d, V, err);
  else if (w_dtype == DT_F16)
    k_pf_embed<f16_t><<<B * C, 256, 0, s>>>(x, pos, (const f16_t*)E, tokens, T, (const f16_t*)emb, A, offset, t0, C,
                                            Cn, d, V, err);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---- dense GEMM over fragment-layout operands -------------------------------------------------
// C[r][n] = sum_k (Ahi + Alo)[r][k] W[n][k]: A is the split activation [Rp, K] and W the
// repacked weight [N, K], both in fragment order, so every MFMA operand is one contiguous
// 1 KB tile read with 16-byte lane loads; operands run one K step ahead of the MFMAs.
// WC = 4: block 128 x 128 (waves 2 x 2 of 4 x 4 tiles); WC = 2: block 64 x 128 (waves 1 x 4
// of 4 x 2 tiles), twice the blocks for narrow outputs.
template <typename T, int EPI, int WC>
__global__ __launch_bounds__(256) void k_fgemm(FgParams p) {
  constexpr int WR = 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rt0 = WC == 4 ? blockIdx.x * 8 + (w & 1) * 4 : blockIdx.x * 4;   // first 16-row tile of this wave
  const int ct0 = WC == 4 ? blockIdx.y * 8 + (w >> 1) * 4 : blockIdx.y * 8 + w * 2;   // first 16-column tile
  const int KST = p.K >> 5;
  const pv4u* __restrict__ Ah = reinterpret_cast<const pv4u*>(p.Ahi);
  const pv4u* __restrict__ Al = reinterpret_cast<const pv4u*>(p.Alo);
  const pv4u* __restrict__ Wt = reinterpret_cast<const pv4u*>(p.W);
  pf32x4_t acc[WR][WC];
#pragma unroll
  for (int i = 0; i < WR; ++i)
#pragma unroll
    for (int j = 0; j < WC; ++j) acc[i][j] = pf32x4_t{0.f, 0.f, 0.f, 0.f};
  pv4u ah[WR], al[WR], wf[WC];
  auto load = [&](int s, pv4u (&h)[WR], pv4u (&l)[WR], pv4u (&f)[WC]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WR; ++i) {
      h[i] = Ah[((int64_t)(rt0 + i) * KST + s) * 64 + lane];
      l[i] = Al[((int64_t)(rt0 + i) * KST + s) * 64 + lane];
    }
#pragma unroll
    for (int j = 0; j < WC; ++j) f[j] = Wt[((int64_t)(ct0 + j) * KST + s) * 64 + lane];
  };
  load(0, ah, al, wf);
  for (int s = 0; s < KST; ++s) {
    pv4u nh[WR], nl[WR], nf[WC];
    load(min(s + 1, KST - 1), nh, nl, nf);
#pragma unroll
    for (int i = 0; i < WR; ++i)
#pragma unroll
      for (int j = 0; j < WC; ++j) {
        acc[i][j] = pmma(ah[i], wf[j], acc[i][j], (T*)nullptr);
        acc[i][j] = pmma(al[i], wf[j], acc[i][j], (T*)nullptr);
      }
#pragma unroll
    for (int i = 0; i < WR; ++i) { ah[i] = nh[i]; al[i] = nl[i]; }
#pragma unroll
    for (int j = 0; j < WC; ++j) wf[j] = nf[j];
  }
  // tile (i, j): lane holds rows (rt0+i)*16 + 4*(lane/16) + e of column (ct0+j)*16 + lane%16
  const int rsub = (lane >> 4) * 4, col = lane & 15;
  if constexpr (EPI == FG_SWIGLU) {
    // weight row blocks alternate gate, up for the same 16 outputs: tiles (0,1), (2,3)
    const int half = p.N >> 1;
#pragma unroll
    for (int j = 0; j < WC; j += 2)
#pragma unroll
      for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = (rt0 + i) * 16 + rsub + e, jj = ((ct0 + j) >> 1) * 16 + col;
          if (r < p.R) {
            const float g = acc[i][j][e], u = acc[i][j + 1][e];
            store_split<T>(p.Ohi, p.Olo, frag_offset(r, jj, half), g / (1.0f + expf(-g)) * u);
          }
        }
  } else {
#pragma unroll
    for (int i = 0; i < WR; ++i)
#pragma unroll
      for (int j = 0; j < WC; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = (rt0 + i) * 16 + rsub + e, n = (ct0 + j) * 16 + col;
          if (r < p.R) {
            float* o = p.out + (int64_t)r * p.ldo + n;
            if constexpr (EPI == FG_RESID) *o += acc[i][j][e];
            else *o = acc[i][j][e];
          }
        }
  }
}

hipError_t launch_fgemm(const FgParams& p, hipStream_t s) {
  if (p.R <= 0 || p.N <= 0 || p.N % 128 || p.K <= 0 || p.K % 32 || !p.W || !p.Ahi || !p.Alo) return hipErrorInvalidValue;
  if (p.epi == FG_SWIGLU ? (!p.Ohi || !p.Olo || p.N % 256) : (!p.out || p.ldo < p.N)) return hipErrorInvalidValue;
  // 128-row blocks unless they leave CUs idle (then 64-row blocks; A is padded to 128 rows)
  const bool wide = (int64_t)((p.R + 127) / 128) * (p.N / 128) >= 256;
  const dim3 grid(wide ? (p.R + 127) / 128 : (p.R + 63) / 64, p.N / 128);
#define WD_FG(T_)                                                                                        \
  switch (p.epi) {                                                                                       \
    case FG_STORE: if (wide) k_fgemm<T_, FG_STORE, 4><<<grid, 256, 0, s>>>(p);                           \
                   else k_fgemm<T_, FG_STORE, 2><<<grid, 256, 0, s>>>(p); break;                         \
    case FG_RESID: if (wide) k_fgemm<T_, FG_RESID, 4><<<grid, 256, 0, s>>>(p);                           \
                   else k_fgemm<T_, FG_RESID, 2><<<grid, 256, 0, s>>>(p); break;                         \
    case FG_SWIGLU: if (wide) k_fgemm<T_, FG_SWIGLU, 4><<<grid, 256, 0, s>>>(p);                         \
                    else k_fgemm<T_, FG_SWIGLU, 2><<<grid, 256, 0, s>>>(p); break;                       \
    default: return hipErrorInvalidValue;                                                                \
  }
  if (p.w_dtype == DT_BF16) { WD_FG(bf16_t) }
  else if (p.w_dtype == DT_F16) { WD_FG(f16_t) }
  else return hipErrorInvalidValue;
#undef WD_FG
  return hipGetLastError();
}

// ---- causal prefill attention ------------------------------------------------------------------
// One block per (tile of PQ positions, kv head g, stream b): its PQ * G queries (G query heads
// per kv head, GQA) attend over cache rows 0..t of their own position t.  Two threads per
// query, each with half of the head's channels; K and V come through LDS in tiles of PK rows
// (every lane of a wave reads the same key row: broadcast), and each query keeps an online
// softmax state.  q is the scaled, normed and rotated query [R, Hq*hd] fp32; the output o goes
// to the split fragment layout [Rp, Hq*hd] of the out projection.
constexpr int PQ = 64, PK = 32;

template <typename CT, typename OT, int HD>
__global__ __launch_bounds__(256) void k_pf_attn(PfAttnParams p) {
  constexpr int HH = HD / 2;   // channels per thread
  __shared__ __align__(16) CT Ks[PK * HD];   // cache type (fp32 tiles measured slower: twice the LDS bytes)
  __shared__ __align__(16) CT Vs[PK * HD];
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  const int t = threadIdx.x, qi = t >> 1, half = t & 1;
  const int nq = PQ * G;                       // queries of the block (<= 128)
  const int jq = qi / G, hq = g * G + qi % G;  // position within the chunk, query head
  const bool active = qi < nq && tile * PQ + jq < p.Cn;
  const int jrow = min(tile * PQ + jq, p.Cn - 1);
  const int r = b * p.C + jrow;
  const int tpos = p.t0 + jrow;                // absolute position of this query
  // the block's last position bounds the rows it streams
  const int jlast = min(tile * PQ + PQ, p.Cn) - 1;
  const int rows = p.t0 + jlast + 1;
  float q[HH], o[HH];
  const float* qr = p.q + (int64_t)r * p.Hq * HD + hq * HD + half * HH;
#pragma unroll
  for (int c = 0; c < HH; c += 4) {
    const float4 v = *reinterpret_cast<const float4*>(qr + c);
    q[c] = v.x; q[c + 1] = v.y; q[c + 2] = v.z; q[c + 3] = v.w;
  }
#pragma unroll
  for (int c = 0; c < HH; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  const CT* Kb = reinterpret_cast<const CT*>(p.K) + (int64_t)b * p.kv_bstride + (int64_t)g * p.ctx * HD;
  const CT* Vb = reinterpret_cast<const CT*>(p.V) + (int64_t)b * p.kv_bstride + (int64_t)g * p.ctx * HD;
  constexpr int CH = 16 / sizeof(CT);          // elements per 16-byte chunk
  constexpr int NCH = PK * HD / CH;            // chunks per tile
  for (int k0 = 0; k0 < rows; k0 += PK) {
    __syncthreads();   // the previous tile is no longer read
    for (int i = t; i < NCH; i += 256) {
      const int kr = min(k0 + (i * CH) / HD, rows - 1), kc = (i * CH) % HD;
      *reinterpret_cast<uint4*>(Ks + i * CH) = *reinterpret_cast<const uint4*>(Kb + (int64_t)kr * HD + kc);
      *reinterpret_cast<uint4*>(Vs + i * CH) = *reinterpret_cast<const uint4*>(Vb + (int64_t)kr * HD + kc);
    }
    __syncthreads();
    const int kn = min(PK, rows - k0);
    for (int kk = 0; kk < kn; ++kk) {
      const CT* kr = Ks + kk * HD + half * HH;
      float sc = 0.f;
#pragma unroll
      for (int c = 0; c < HH; ++c) sc = fmaf(q[c], to_f(kr[c]), sc);
      sc += __shfl_xor(sc, 1, WAVE);
      if (k0 + kk <= tpos) {   // causal: rows 0..t of this query's position
        if (sc > m) {
          const float f = expf(m - sc);
          l *= f;
#pragma unroll
          for (int c = 0; c < HH; ++c) o[c] *= f;
          m = sc;
        }
        const float e = expf(sc - m);
        l += e;
        const CT* vr = Vs + kk * HD + half * HH;
#pragma unroll
        for (int c = 0; c < HH; ++c) o[c] = fmaf(e, to_f(vr[c]), o[c]);
      }
    }
  }
  if (!active) return;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const int K = p.Hq * HD;
#pragma unroll
  for (int c = 0; c < HH; c += 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = o[c + e] * inv;
    OT h8[8], l8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_hi_lo<OT>(v[e], h8[e], l8[e]);
    const int64_t off = frag_offset(r, hq * HD + half * HH + c, K);   // 8 contiguous elements
    __builtin_memcpy(reinterpret_cast<OT*>(p.o_hi) + off, h8, 16);
    __builtin_memcpy(reinterpret_cast<OT*>(p.o_lo) + off, l8, 16);
  }
}

hipError_t launch_pf_attn(const PfAttnParams& p, hipStream_t s) {
  const int G = p.Hkv > 0 ? p.Hq / p.Hkv : 0;
  if (p.B <= 0 || p.C <= 0 || p.Cn <= 0 || p.Cn > p.C || G <= 0 || p.Hq % p.Hkv || PQ * G > 128 ||
      p.t0 < 0 || p.t0 + p.Cn > p.ctx || !p.q || !p.K || !p.V || !p.o_hi || !p.o_lo)
    return hipErrorInvalidValue;
  const dim3 grid((p.Cn + PQ - 1) / PQ, p.Hkv, p.B);
#define WD_PFA(CT_, HD_)                                                                        \
  if (p.o_dtype == DT_BF16) k_pf_attn<CT_, bf16_t, HD_><<<grid, 256, 0, s>>>(p);               \
  else if (p.o_dtype == DT_F16) k_pf_attn<CT_, f16_t, HD_><<<grid, 256, 0, s>>>(p);            \
  else return hipErrorInvalidValue;
  if (p.hd == 128 && p.cache_dtype == DT_F16) { WD_PFA(f16_t, 128) }
  else if (p.hd == 128 && p.cache_dtype == DT_BF16) { WD_PFA(bf16_t, 128) }
  else if (p.hd == 64 && p.cache_dtype == DT_F16) { WD_PFA(f16_t, 64) }
  else if (p.hd == 64 && p.cache_dtype == DT_BF16) { WD_PFA(bf16_t, 64) }
  else return hipErrorInvalidValue;
#undef WD_PFA
  return hipGetLastError();
}

}  // namespace wd
