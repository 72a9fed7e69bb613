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
// the causal prefill attention (flash attention on the matrix cores).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

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

// (hi, lo) split of one value into the fragment-layout pair; bf16 by the hardware round-to-
// nearest-even convert (the same bits as from_f's integer rounding for every finite value, in
// two instructions instead of about fourteen: the GELU epilogue of the encoder's fc1 writes
// 491 M of them per launch)
template <typename T>
__device__ __forceinline__ void fg_store_split(void* hi_base, void* lo_base, int64_t off, float v) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const __bf16 h = (__bf16)v, l = (__bf16)(v - (float)h);
    reinterpret_cast<uint16_t*>(hi_base)[off] = __builtin_bit_cast(uint16_t, h);
    reinterpret_cast<uint16_t*>(lo_base)[off] = __builtin_bit_cast(uint16_t, l);
  } else {
    store_split<T>(hi_base, lo_base, off, v);
  }
}

// ---- dense GEMM over fragment-layout operands -------------------------------------------------
// C[r][n] = sum_k (Ahi + Alo)[r][k] W[n][k]: A is the split activation [Rp, K] and W the
// repacked weight [N, K], both in fragment order, so every MFMA operand is one contiguous
// 1 KB tile read with 16-byte lane loads; operands run one K step ahead of the MFMAs.
// WC = 4: block 128 x 128 (waves 2 x 2 of 4 x 4 tiles); WC = 2: block 64 x 128 (waves 1 x 4
// of 4 x 2 tiles), twice the blocks for narrow outputs.
// Epilogue of the dense GEMM: wave tiles (i, j) at 16-row tile rt0 + i, 16-column tile ct0 + j.
template <typename T, int EPI, int WR, int WC>
__device__ __forceinline__ void fg_epilogue(const FgParams& p, const pf32x4_t (&acc)[WR][WC], int rt0, int ct0,
                                            int lane) {
  // tile (i, j): lane holds rows (rt0+i)*16 + 4*(lane/16) + e of column (ct0+j)*16 + lane%16
  const int rsub = (lane >> 4) * 4, col = lane & 15;
  if constexpr (EPI == FG_ENC_QKV) {
    const int d = p.N / 3;
#pragma unroll
    for (int j = 0; j < WC; ++j) {
      const int n = (ct0 + j) * 16 + col, sec = n / d, c = n - sec * d;
      const int h = c / p.kv_hd, ch = c - h * p.kv_hd;
      const float bn = sec == 0 ? (p.bias ? p.bias[c] : 0.f) : sec == 2 ? (p.bias2 ? p.bias2[c] : 0.f) : 0.f;
#pragma unroll
      for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = (rt0 + i) * 16 + rsub + e;
          if (r < p.R) {
            const float v = acc[i][j][e] + bn;
            if (sec == 0) {
              p.out[(int64_t)r * d + c] = v * p.scale;
            } else {
              const int b = r / p.kv_P, fr = r - b * p.kv_P;
              const int64_t kv = (((int64_t)b * p.kv_H + h) * p.kv_P + fr) * p.kv_hd + ch;
              reinterpret_cast<T*>(sec == 1 ? p.Kc : p.Vc)[kv] = from_f<T>(v);
            }
          }
        }
    }
  } else if constexpr (EPI == FG_SWIGLU) {
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
            fg_store_split<T>(p.Ohi, p.Olo, frag_offset(r, jj, half), g / (1.0f + expf(-g)) * u);
          }
        }
  } else {
#pragma unroll
    for (int j = 0; j < WC; ++j) {
      const int n = (ct0 + j) * 16 + col;
      const float bn = p.bias ? p.bias[n] : 0.f;
#pragma unroll
      for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = (rt0 + i) * 16 + rsub + e;
          if (r < p.R) {
            const float c = acc[i][j][e] + bn;
            if constexpr (EPI == FG_GELU_SPLIT) {
              fg_store_split<T>(p.Ohi, p.Olo, frag_offset(r, n, p.N), 0.5f * c * (1.0f + erff(c * 0.70710678118654752f)));
            } else {
              float* o = p.out + (int64_t)r * p.ldo + n;
              if constexpr (EPI == FG_RESID) *o += c;
              else if constexpr (EPI == FG_GELU)
                *o = 0.5f * c * (1.0f + erff(c * 0.70710678118654752f)) +
                     (p.pos ? p.pos[(int64_t)(r % p.pos_rows) * p.N + n] : 0.f);
              else *o = c;
            }
          }
        }
    }
  }
}

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
  fg_epilogue<T, EPI, WR, WC>(p, acc, rt0, ct0, lane);
}

// 128 x 128 blocks (waves 2 x 2 of 4 x 4 tiles) with the block's operand tiles of a K step
// (8 Ahi + 8 Alo + 8 W, 1 KB each) staged once in LDS, so each fragment leaves L2 once per
// block instead of once per wave.  The tiles go straight from global memory into two LDS
// slots (buffer loads with the LDS destination, six per thread and step, no staging registers
// and no LDS stores), one K step ahead of the MFMAs; each step waits for its own loads by count
// and meets the other waves at a bare barrier.  Measured against staging the next step through
// registers: Qwen3 prefill 52.9 -> 49.5 ms, large-v3 encoder window 381 -> 361 ms; a ring of
// three slots (72 KB, two workgroups per CU instead of three) sat in between.
// Block order (workgroup L runs on XCD L % 8): with n_mt = 8 q + r row panels, XCD x owns
// panels x, x + 8, ..., x + 8 (q - 1) and takes them in groups of pg, column tile by column
// tile within a group, so a group's A panels stay in the XCD's L2 while each W tile is used pg
// times in a row; the (panel, tile) units of the last r panels are then shared out evenly, so
// every XCD gets the same work at any row count.  (A plain 2-D grid sent every panel to every
// XCD whenever n_mt % 8 != 0: the 3104-row prefill chunk fetched 2.7 GB per gate|up launch
// against 0.8 GB for the 4096-row chunk; plain panel-major runs fixed that but re-read W for
// every panel.)
struct FgOrder { int n_mt, n_nt, pg, per_xcd; };
template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_fgemm_lds(FgParams p, FgOrder od) {
  constexpr int WR = 4, WC = 4, NTL = 24, NSLOT = 2;
  __shared__ __align__(16) pv4u stage[NSLOT][NTL * 64];   // 2 x 24 KB: three workgroups per CU
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int q = od.n_mt >> 3, bulk = q * od.n_nt;
  int mt, nt;
  if (j < bulk) {
    const int gi = j / (od.pg * od.n_nt), within = j - gi * od.pg * od.n_nt;
    const int gsz = min(od.pg, q - gi * od.pg);
    nt = within / gsz;
    mt = xcd + 8 * (gi * od.pg + (within - nt * gsz));
  } else {
    const int r = od.n_mt - 8 * q, tail = r * od.n_nt, per = (tail + 7) >> 3;
    const int tu = xcd * per + (j - bulk);
    if (tu >= tail) return;
    mt = 8 * q + tu / od.n_nt;
    nt = tu - (tu / od.n_nt) * od.n_nt;
  }
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int rt0 = mt * 8 + wm * 4, ct0 = nt * 8 + wn * 4;
  const int KST = p.K >> 5;
  const pv4u* __restrict__ Ah = reinterpret_cast<const pv4u*>(p.Ahi) + (int64_t)mt * 8 * KST * 64;
  const pv4u* __restrict__ Al = reinterpret_cast<const pv4u*>(p.Alo) + (int64_t)mt * 8 * KST * 64;
  const pv4u* __restrict__ Wt = reinterpret_cast<const pv4u*>(p.W) + (int64_t)nt * 8 * KST * 64;
  // wave w loads tiles w and 4 + w of Ahi, of Alo and of W; the step is clamped so that every
  // thread issues exactly 6 loads per step and the vmcnt arithmetic stays exact
  const uint32_t pbytes = (uint32_t)(8 * KST) * 1024;
  const __amdgpu_buffer_rsrc_t rh = buf_rsrc(Ah, pbytes), rl = buf_rsrc(Al, pbytes), rw = buf_rsrc(Wt, pbytes);
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int slot = st % NSLOT;
    st = min(st, KST - 1);
    const uint32_t so = (uint32_t)(st * 64 + lane) * 16, t0 = (uint32_t)w * KST * 1024, t4 = (uint32_t)(4 + w) * KST * 1024;
    lds_dma16(rh, t0 + so, &stage[slot][w * 64]);
    lds_dma16(rh, t4 + so, &stage[slot][(4 + w) * 64]);
    lds_dma16(rl, t0 + so, &stage[slot][(8 + w) * 64]);
    lds_dma16(rl, t4 + so, &stage[slot][(12 + w) * 64]);
    lds_dma16(rw, t0 + so, &stage[slot][(16 + w) * 64]);
    lds_dma16(rw, t4 + so, &stage[slot][(20 + w) * 64]);
  };
  pf32x4_t acc[WR][WC];
#pragma unroll
  for (int i = 0; i < WR; ++i)
#pragma unroll
    for (int j = 0; j < WC; ++j) acc[i][j] = pf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NSLOT - 1; ++k) issue(k);
  for (int st = 0; st < KST; ++st) {
    wait_vmcnt<6 * (NSLOT - 2)>();    // this thread's loads of step st have landed
    __builtin_amdgcn_s_barrier();     // ... and every thread's; every wave is done with step st - 1
    issue(st + NSLOT - 1);            // into the slot of step st - 1
    const pv4u* S = stage[st % NSLOT];
    pv4u ah[WR], al[WR], wf[WC];
#pragma unroll
    for (int j = 0; j < WC; ++j) wf[j] = S[(16 + wn * 4 + j) * 64 + lane];
#pragma unroll
    for (int i = 0; i < WR; ++i) {
      ah[i] = S[(wm * 4 + i) * 64 + lane];
      al[i] = S[(8 + wm * 4 + i) * 64 + lane];
    }
#pragma unroll
    for (int i = 0; i < WR; ++i)
#pragma unroll
      for (int j = 0; j < WC; ++j) {
        acc[i][j] = pmma(ah[i], wf[j], acc[i][j], (T*)nullptr);
        acc[i][j] = pmma(al[i], wf[j], acc[i][j], (T*)nullptr);
      }
  }
  wait_vmcnt<0>();   // the clamped loads past the end land before the workgroup's LDS is released
  fg_epilogue<T, EPI, WR, WC>(p, acc, rt0, ct0, lane);
}

// 256 x 128 blocks of eight 64 x 64 waves (4 x 2), the block's 16 Ahi + 16 Alo + 8 W tiles of
// a K step through two 40 KB LDS slots (buffer loads, five per thread and step), two blocks per
// CU.  Same XCD block order as k_fgemm_lds over 256-row panels; A is padded to 128 rows only,
// so the last panel's buffer resource ends at the padded rows (reads past it return zeros).
template <typename T, int EPI>
__global__ __launch_bounds__(512) void k_fgemm_lds8(FgParams p, FgOrder od) {
  constexpr int WR = 4, WC = 4, NTL = 40, NSLOT = 2;
  __shared__ __align__(16) pv4u stage[NSLOT][NTL * 64];   // 2 x 40 KB
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int q = od.n_mt >> 3, bulk = q * od.n_nt;
  int mt, nt;
  if (j < bulk) {
    const int gi = j / (od.pg * od.n_nt), within = j - gi * od.pg * od.n_nt;
    const int gsz = min(od.pg, q - gi * od.pg);
    nt = within / gsz;
    mt = xcd + 8 * (gi * od.pg + (within - nt * gsz));
  } else {
    const int r = od.n_mt - 8 * q, tail = r * od.n_nt, per = (tail + 7) >> 3;
    const int tu = xcd * per + (j - bulk);
    if (tu >= tail) return;
    mt = 8 * q + tu / od.n_nt;
    nt = tu - (tu / od.n_nt) * od.n_nt;
  }
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 3, wn = w >> 2;
  const int rt0 = mt * 16 + wm * 4, ct0 = nt * 8 + wn * 4;
  const int KST = p.K >> 5;
  const pv4u* __restrict__ Ah = reinterpret_cast<const pv4u*>(p.Ahi) + (int64_t)mt * 16 * KST * 64;
  const pv4u* __restrict__ Al = reinterpret_cast<const pv4u*>(p.Alo) + (int64_t)mt * 16 * KST * 64;
  const pv4u* __restrict__ Wt = reinterpret_cast<const pv4u*>(p.W) + (int64_t)nt * 8 * KST * 64;
  const int rpad = (p.R + 127) & ~127, a_tiles = min(16, (rpad - mt * 256) >> 4);
  const uint32_t abytes = (uint32_t)(a_tiles * KST) * 1024, wbytes = (uint32_t)(8 * KST) * 1024;
  const __amdgpu_buffer_rsrc_t rh = buf_rsrc(Ah, abytes), rl = buf_rsrc(Al, abytes), rw = buf_rsrc(Wt, wbytes);
  auto issue = [&](int st) __attribute__((always_inline)) {
    pv4u* S = stage[st % NSLOT];
    st = min(st, KST - 1);
    const uint32_t so = (uint32_t)(st * 64 + lane) * 16, t0 = (uint32_t)w * KST * 1024, t8 = (uint32_t)(8 + w) * KST * 1024;
    lds_dma16(rh, t0 + so, S + w * 64);
    lds_dma16(rh, t8 + so, S + (8 + w) * 64);
    lds_dma16(rl, t0 + so, S + (16 + w) * 64);
    lds_dma16(rl, t8 + so, S + (24 + w) * 64);
    lds_dma16(rw, t0 + so, S + (32 + w) * 64);
  };
  pf32x4_t acc[WR][WC];
#pragma unroll
  for (int i = 0; i < WR; ++i)
#pragma unroll
    for (int jj = 0; jj < WC; ++jj) acc[i][jj] = pf32x4_t{0.f, 0.f, 0.f, 0.f};
  issue(0);
  for (int st = 0; st < KST; ++st) {
    wait_vmcnt<0>();                  // this thread's loads of step st have landed
    __builtin_amdgcn_s_barrier();     // ... and every thread's; every wave is done with step st - 1
    issue(st + 1);                    // into the slot of step st - 1
    const pv4u* S = stage[st % NSLOT];
    pv4u ah[WR], al[WR], wf[WC];
#pragma unroll
    for (int jj = 0; jj < WC; ++jj) wf[jj] = S[(32 + wn * 4 + jj) * 64 + lane];
#pragma unroll
    for (int i = 0; i < WR; ++i) {
      ah[i] = S[(wm * 4 + i) * 64 + lane];
      al[i] = S[(16 + wm * 4 + i) * 64 + lane];
    }
    __builtin_amdgcn_s_setprio(1);   // MFMA issue first while this wave has operands (encoder window -0.5%)
#pragma unroll
    for (int i = 0; i < WR; ++i)
#pragma unroll
      for (int jj = 0; jj < WC; ++jj) {
        acc[i][jj] = pmma(ah[i], wf[jj], acc[i][jj], (T*)nullptr);
        acc[i][jj] = pmma(al[i], wf[jj], acc[i][jj], (T*)nullptr);
      }
    __builtin_amdgcn_s_setprio(0);
  }
  wait_vmcnt<0>();   // the clamped loads past the end land before the workgroup's LDS is released
  fg_epilogue<T, EPI, WR, WC>(p, acc, rt0, ct0, lane);
}


hipError_t launch_fgemm(const FgParams& p, hipStream_t s) {
  if (p.R <= 0 || p.N <= 0 || p.N % 128 || p.K <= 0 || p.K % 32 || !p.W || !p.Ahi || !p.Alo) return hipErrorInvalidValue;
  if (p.epi == FG_SWIGLU ? (!p.Ohi || !p.Olo || p.N % 256)
      : p.epi == FG_GELU_SPLIT ? (!p.Ohi || !p.Olo)
      : p.epi == FG_ENC_QKV ? (!p.out || !p.Kc || !p.Vc || p.N % 3 || p.kv_P <= 0 || p.kv_H <= 0 || p.kv_hd <= 0 ||
                               p.kv_H * p.kv_hd != p.N / 3 || p.R % p.kv_P)
      : (!p.out || p.ldo < p.N || (p.epi == FG_GELU && p.pos && p.pos_rows <= 0)))
    return hipErrorInvalidValue;
  // 128-row blocks unless they leave CUs idle (then 64-row blocks; A is padded to 128 rows)
  const bool wide = (int64_t)((p.R + 127) / 128) * (p.N / 128) >= 256;
  const dim3 grid(wide ? (p.R + 127) / 128 : (p.R + 63) / 64, p.N / 128);
  // 128-row blocks stage their operands through LDS, in XCD-owned panel groups; a group's A
  // panels (128 rows x K, hi and lo) take about 3 MB of the XCD's 4 MB L2
  FgOrder od;
  od.n_mt = (p.R + 127) / 128;
  od.n_nt = p.N / 128;
  od.pg = std::max(1, std::min(8, (3 << 20) / (128 * p.K * 4)));
  od.per_xcd = (od.n_mt >> 3) * od.n_nt + ((od.n_mt & 7) * od.n_nt + 7) / 8;
  // 256-row blocks once they fill the chip twice over
  // (encoder window 341 -> 328 ms, Qwen3 prefill 46.4 -> 45.9 ms against 128-row blocks only)
  const bool wide8 = (int64_t)((p.R + 255) / 256) * (p.N / 128) >= 512;
  FgOrder od8;
  od8.n_mt = (p.R + 255) / 256;
  od8.n_nt = p.N / 128;
  od8.pg = std::max(1, std::min(8, (3 << 20) / (256 * p.K * 4)));
  od8.per_xcd = (od8.n_mt >> 3) * od8.n_nt + ((od8.n_mt & 7) * od8.n_nt + 7) / 8;
#define WD_FG1(T_, E_)                                                                                   \
  if (wide8) k_fgemm_lds8<T_, E_><<<8 * od8.per_xcd, 512, 0, s>>>(p, od8);                            \
  else if (wide) k_fgemm_lds<T_, E_><<<8 * od.per_xcd, 256, 0, s>>>(p, od);                            \
  else k_fgemm<T_, E_, 2><<<grid, 256, 0, s>>>(p);
#define WD_FG(T_)                                                                                        \
  switch (p.epi) {                                                                                       \
    case FG_STORE: WD_FG1(T_, FG_STORE) break;                                                           \
    case FG_RESID: WD_FG1(T_, FG_RESID) break;                                                           \
    case FG_SWIGLU: WD_FG1(T_, FG_SWIGLU) break;                                                         \
    case FG_GELU: WD_FG1(T_, FG_GELU) break;                                                             \
    case FG_GELU_SPLIT: WD_FG1(T_, FG_GELU_SPLIT) break;                                                 \
    case FG_ENC_QKV: WD_FG1(T_, FG_ENC_QKV) break;                                                       \
    default: return hipErrorInvalidValue;                                                                \
  }
  if (p.w_dtype == DT_BF16) { WD_FG(bf16_t) }
  else if (p.w_dtype == DT_F16) { WD_FG(f16_t) }
  else return hipErrorInvalidValue;
#undef WD_FG
#undef WD_FG1
  return hipGetLastError();
}

// ---- causal prefill attention ------------------------------------------------------------------
// Flash attention on the matrix cores.  A block takes 64 queries of one kv head g and stream b,
// enumerated (position j, query head g*G + i) as q = j*G + i; wave w holds 16 of them.  Cache
// rows stream through LDS in tiles of 32 keys, K and V as stored ([key][hd], rows padded).
// Per tile a wave computes S^T = K Q^T (16 keys x 16 queries per MFMA tile, q split into hi + lo
// in the cache type), so a lane holds 4 keys of one query; the online softmax state of that
// query lives in the lane; P^T (split hi + lo) is the B operand of O^T += V^T P^T as it stands,
// with the A operand (V^T in the same key order) read from the V tile by the transposing LDS
// load (ds_read_b64_tr_b16).  Causal: key k counts for the query at position t when k <= t.  q is the scaled,
// normed and rotated query [R, Hq*hd] fp32; o goes to the split fragment layout [Rp, Hq*hd].
constexpr int PA_KT = 32;    // keys per tile
constexpr int PA_QB = 64;    // queries per block (4 waves x 16)

template <typename CT>
__device__ __forceinline__ uint32_t pa_bits(CT v) {
  if constexpr (sizeof(CT) == 2 && std::is_same<CT, bf16_t>::value) return v.x;
  else return (uint32_t)__builtin_bit_cast(uint16_t, v);
}
// Two floats -> packed hi and lo 16-bit pairs (hi = round(v), lo = round(v - hi)).  bf16 takes
// the hardware round-to-nearest-even convert (v_cvt_pk_bf16_f32, two values per instruction;
// the same bits as the integer rounding of from_f for every finite value): the attention's
// inner loop is bound by its VALU work, and the integer rounding took about 7 instructions a
// value.
template <typename CT>
__device__ __forceinline__ uint32_t pa_pack2(float a, float b, uint32_t& lo) {
  if constexpr (std::is_same<CT, bf16_t>::value) {
    const __bf16 ha = (__bf16)a, hb = (__bf16)b;
    const __bf16 la = (__bf16)(a - (float)ha), lb = (__bf16)(b - (float)hb);
    lo = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
  } else {
    CT ha, la, hb, lb;
    split_hi_lo<CT>(a, ha, la);
    split_hi_lo<CT>(b, hb, lb);
    lo = pa_bits(la) | (pa_bits(lb) << 16);
    return pa_bits(ha) | (pa_bits(hb) << 16);
  }
}
constexpr float PA_LOG2E = 1.4426950408889634f;

// Block order: the (stream, kv head, query block) units are numbered query block fastest and
// cut into 8 equal runs, one per XCD (workgroup L runs on XCD L % 8), so the query blocks that
// stream one (stream, kv head) slab of K and V share one XCD's L2 instead of pulling the slab
// into all eight.
template <typename CT, typename OT, int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 3))) void k_pf_attn(PfAttnParams p, int n_qb,
                                                                                            int per_xcd) {
  constexpr int KLD = HD + 8;                 // K tile row stride (elements): conflict-free 16 B reads
  constexpr int VLD = HD + 8;                 // V tile row stride (elements), rows = keys
  constexpr int NCH = PA_KT * HD / 8;         // 16-byte chunks per tile (K or V)
  constexpr int CPT = NCH / 256;              // chunks per thread
  constexpr int KS = HD / 32;                 // MFMA k-steps over the head dim
  constexpr int HT = HD / 16;                 // output channel tiles
  __shared__ __align__(16) CT Ks[PA_KT * KLD];
  __shared__ __align__(16) CT Vs[PA_KT * VLD];
  const int u = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (u >= n_qb * p.Hkv * p.B) return;
  const int qb = u % n_qb, g = (u / n_qb) % p.Hkv, b = u / (n_qb * p.Hkv);
  const int G = p.Hq / p.Hkv;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int col = lane & 15, grp = lane >> 4;

  // this lane's query (column col of the wave's 16)
  const int qidx = qb * PA_QB + wv * 16 + col;
  const int jq = qidx / G, hq = g * G + (qidx - jq * G);
  const bool active = jq < p.Cn;
  const int jc = min(jq, p.Cn - 1);
  const int tq = p.t0 + jc;
  const int r = b * p.C + jc;
  // key ranges: the block's (staged) and the wave's (computed)
  const int rows_blk = p.full ? p.t0 + p.Cn : p.t0 + min(p.Cn - 1, (qb * PA_QB + PA_QB - 1) / G) + 1;
  const int rows_w = p.full ? rows_blk : p.t0 + min(p.Cn - 1, (qb * PA_QB + wv * 16 + 15) / G) + 1;
  const int tmax = p.full ? rows_blk - 1 : tq;   // the last key this lane's query sees

  // q^T as the B operand: lane (col, grp) holds channels 32 ks + 8 grp .. +8 of its query
  pv4u qh[KS], ql[KS];
  {
    const float* qr = p.q + (int64_t)r * p.Hq * HD + hq * HD + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 u0 = *reinterpret_cast<const float4*>(qr + 32 * ks);
      const float4 u1 = *reinterpret_cast<const float4*>(qr + 32 * ks + 4);
      uint32_t l0, l1, l2, l3;
      // scores in log2 units (q times log2 e), so the softmax exponentials are bare exp2
      qh[ks][0] = pa_pack2<CT>(u0.x * PA_LOG2E, u0.y * PA_LOG2E, l0);
      qh[ks][1] = pa_pack2<CT>(u0.z * PA_LOG2E, u0.w * PA_LOG2E, l1);
      qh[ks][2] = pa_pack2<CT>(u1.x * PA_LOG2E, u1.y * PA_LOG2E, l2);
      qh[ks][3] = pa_pack2<CT>(u1.z * PA_LOG2E, u1.w * PA_LOG2E, l3);
      ql[ks][0] = l0; ql[ks][1] = l1; ql[ks][2] = l2; ql[ks][3] = l3;
    }
  }
  pf32x4_t acc[HT];
#pragma unroll
  for (int h = 0; h < HT; ++h) acc[h] = pf32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  const CT* Kb = reinterpret_cast<const CT*>(p.K) + (int64_t)b * p.kv_bstride + (int64_t)g * p.ctx * HD;
  const CT* Vb = reinterpret_cast<const CT*>(p.V) + (int64_t)b * p.kv_bstride + (int64_t)g * p.ctx * HD;
  uint4 kst[CPT], vst[CPT];
  auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int i = t + 256 * u;
      const int kr = min(k0 + i / (HD / 8), rows_blk - 1), c0 = (i % (HD / 8)) * 8;
      kst[u] = *reinterpret_cast<const uint4*>(Kb + (int64_t)kr * HD + c0);
      vst[u] = *reinterpret_cast<const uint4*>(Vb + (int64_t)kr * HD + c0);
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < rows_blk; k0 += PA_KT) {
    __syncthreads();   // the previous tile is no longer read
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int i = t + 256 * u;
      const int kk = i / (HD / 8), c0 = (i % (HD / 8)) * 8;
      *reinterpret_cast<uint4*>(Ks + kk * KLD + c0) = kst[u];
      *reinterpret_cast<uint4*>(Vs + kk * VLD + c0) = vst[u];
    }
    __syncthreads();
    if (k0 + PA_KT < rows_blk) fetch(k0 + PA_KT);   // next tile in flight during the math
    if (k0 < rows_w) {
      // S^T: two 16-key tiles; lane holds keys k0 + 16 kt + 4 grp + e of its query
      pf32x4_t sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sc[kt] = pf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const pv4u a = *reinterpret_cast<const pv4u*>(Ks + (kt * 16 + col) * KLD + 32 * ks + 8 * grp);
          sc[kt] = pmma(a, qh[ks], sc[kt], (CT*)nullptr);
          sc[kt] = pmma(a, ql[ks], sc[kt], (CT*)nullptr);
        }
      }
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + kt * 16 + 4 * grp + e;
          sv[kt * 4 + e] = key <= tmax ? sc[kt][e] : -INFINITY;
          mx = fmaxf(mx, sv[kt * 4 + e]);
        }
      {   // over the four 16-lane key groups of the query (permlane swaps, no LDS)
        float u, w;
        lane_pair<16>(mx, u, w);
        lane_pair<32>(fmaxf(u, w), u, w);
        mx = fmaxf(u, w);
      }
      const float mn = fmaxf(m, mx);          // finite: key 0 counts for every query
      const float f = __builtin_amdgcn_exp2f(m - mn);   // 2^(m - mn): 0 while m is -inf
      m = mn;
      lsum *= f;
#pragma unroll
      for (int h = 0; h < HT; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[h][e] *= f;
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - mn);
        lsum += pv[i];
      }
      pv4u ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo;
        ph[i] = pa_pack2<CT>(pv[2 * i], pv[2 * i + 1], lo);
        pl[i] = lo;
      }
      // O^T += V^T P^T; A operand: channel row col of tile h, keys 4 grp .. +4 and 16 + 4 grp .. +4,
      // read from the row-major V tile by the gfx950 transposing LDS load: within each 16-lane
      // group, lane r points at key 4 grp + r / 4, channels h*16 + 4 (r % 4) .. +4, and lane i
      // gets channel h*16 + i of the group's 4 keys
#pragma unroll
      for (int h = 0; h < HT; ++h) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        const CT* vr = Vs + (4 * grp + (col >> 2)) * VLD + h * 16 + 4 * (col & 3);
        const v4s t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vr));
        const v4s t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vr + 16 * VLD));
        const uint2 v0 = __builtin_bit_cast(uint2, t0), v1 = __builtin_bit_cast(uint2, t1);
        const pv4u a = pv4u{v0.x, v0.y, v1.x, v1.y};
        acc[h] = pmma(a, ph, acc[h], (CT*)nullptr);
        acc[h] = pmma(a, pl, acc[h], (CT*)nullptr);
      }
    }
  }
  {
    float u, w;
    lane_pair<16>(lsum, u, w);
    lane_pair<32>(u + w, u, w);
    lsum = u + w;
  }
  if (!active) return;
  const float inv = 1.0f / lsum;
  const int K = p.Hq * HD;
#pragma unroll
  for (int h = 0; h < HT; ++h) {
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      uint32_t lo;
      hw[e >> 1] = pa_pack2<OT>(acc[h][e] * inv, acc[h][e + 1] * inv, lo);
      lw[e >> 1] = lo;
    }
    const int64_t off = frag_offset(r, hq * HD + h * 16 + 4 * grp, K);   // 4 contiguous channels
    *reinterpret_cast<uint2*>(reinterpret_cast<OT*>(p.o_hi) + off) = uint2{hw[0], hw[1]};
    *reinterpret_cast<uint2*>(reinterpret_cast<OT*>(p.o_lo) + off) = uint2{lw[0], lw[1]};
  }
}

hipError_t launch_pf_attn(const PfAttnParams& p, hipStream_t s) {
  const int G = p.Hkv > 0 ? p.Hq / p.Hkv : 0;
  if (p.B <= 0 || p.C <= 0 || p.Cn <= 0 || p.Cn > p.C || G <= 0 || p.Hq % p.Hkv ||
      p.t0 < 0 || p.t0 + p.Cn > p.ctx || !p.q || !p.K || !p.V || !p.o_hi || !p.o_lo)
    return hipErrorInvalidValue;
  const int n_qb = (p.Cn * G + PA_QB - 1) / PA_QB;
  const int per_xcd = (n_qb * p.Hkv * p.B + 7) / 8;
  const dim3 grid(8 * per_xcd);
#define WD_PFA(CT_, HD_)                                                                        \
  if (p.o_dtype == DT_BF16) k_pf_attn<CT_, bf16_t, HD_><<<grid, 256, 0, s>>>(p, n_qb, per_xcd);   \
  else if (p.o_dtype == DT_F16) k_pf_attn<CT_, f16_t, HD_><<<grid, 256, 0, s>>>(p, n_qb, per_xcd); \
  else return hipErrorInvalidValue;
  if (p.hd == 128 && p.cache_dtype == DT_F16) { WD_PFA(f16_t, 128) }
  else if (p.hd == 128 && p.cache_dtype == DT_BF16) { WD_PFA(bf16_t, 128) }
  else if (p.hd == 64 && p.cache_dtype == DT_F16) { WD_PFA(f16_t, 64) }
  else if (p.hd == 64 && p.cache_dtype == DT_BF16) { WD_PFA(bf16_t, 64) }
  else return hipErrorInvalidValue;
#undef WD_PFA
  return hipGetLastError();
}

// ---- audio encoder glue ------------------------------------------------------------------------
template <typename S, typename T>
__global__ __launch_bounds__(256) void k_conv_windows(const S* __restrict__ x, int nb, int L, int C, int stride,
                                                      int Lout, int Kp, T* __restrict__ a_hi, T* __restrict__ a_lo) {
  const int64_t n = (int64_t)nb * Lout * Kp;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / Kp;
    const int kk = (int)(i - r * Kp);
    const int b = (int)(r / Lout), o = (int)(r - (int64_t)b * Lout);
    float v = 0.f;
    if (kk < 3 * C) {
      const int c = kk / 3, k = kk - c * 3, t = o * stride + k - 1;
      if (t >= 0 && t < L) v = to_f(x[((int64_t)b * L + t) * C + c]);
    }
    store_split<T>(a_hi, a_lo, frag_offset(r, kk, Kp), v);
  }
}

hipError_t launch_conv_windows(const void* x, int x_dtype, int nb, int L, int C, int stride, int Lout, int Kp,
                               void* a_hi, void* a_lo, int a_dtype, hipStream_t s) {
  if (!x || !a_hi || !a_lo || nb <= 0 || L <= 0 || C <= 0 || Lout <= 0 || Kp % 32 || Kp < 3 * C ||
      (stride != 1 && stride != 2))
    return hipErrorInvalidValue;
  const int blocks = (int)std::min<int64_t>(((int64_t)nb * Lout * Kp + 255) / 256, 65536);
#define WD_CW(S_, T_) k_conv_windows<S_, T_><<<blocks, 256, 0, s>>>((const S_*)x, nb, L, C, stride, Lout, Kp, (T_*)a_hi, (T_*)a_lo)
#define WD_CW_S(T_)                                      \
  if (x_dtype == DT_F32) WD_CW(float, T_);               \
  else if (x_dtype == DT_F16) WD_CW(f16_t, T_);          \
  else if (x_dtype == DT_BF16) WD_CW(bf16_t, T_);        \
  else return hipErrorInvalidValue;
  if (a_dtype == DT_BF16) { WD_CW_S(bf16_t) }
  else if (a_dtype == DT_F16) { WD_CW_S(f16_t) }
  else return hipErrorInvalidValue;
#undef WD_CW_S
#undef WD_CW
  return hipGetLastError();
}

template <typename S, typename T>
__global__ __launch_bounds__(256) void k_pack_pad(const S* __restrict__ src, int64_t rows, int Ks, T* __restrict__ dst,
                                                  int Kp) {
  const int64_t n = rows * Kp;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / Kp;
    const int k = (int)(i - r * Kp);
    dst[frag_offset(r, k, Kp)] = from_f<T>(k < Ks ? to_f(src[r * Ks + k]) : 0.f);
  }
}

hipError_t launch_pack_pad(const void* src, int src_dtype, int64_t rows, int Ks, void* dst, int dst_dtype, int Kp,
                           hipStream_t s) {
  if (!src || !dst || rows <= 0 || Ks <= 0 || Kp < Ks || Kp % 32 || rows % 16) return hipErrorInvalidValue;
  const int blocks = (int)std::min<int64_t>((rows * Kp + 255) / 256, 65536);
#define WD_PP(S_, T_) k_pack_pad<S_, T_><<<blocks, 256, 0, s>>>((const S_*)src, rows, Ks, (T_*)dst, Kp)
#define WD_PP_S(T_)                                      \
  if (src_dtype == DT_F32) WD_PP(float, T_);             \
  else if (src_dtype == DT_F16) WD_PP(f16_t, T_);        \
  else if (src_dtype == DT_BF16) WD_PP(bf16_t, T_);      \
  else return hipErrorInvalidValue;
  if (dst_dtype == DT_BF16) { WD_PP_S(bf16_t) }
  else if (dst_dtype == DT_F16) { WD_PP_S(f16_t) }
  else return hipErrorInvalidValue;
#undef WD_PP_S
#undef WD_PP
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void k_cast(const float* __restrict__ x, T* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) y[i] = from_f<T>(x[i]);
}

hipError_t launch_cast(const float* x, void* y, int y_dtype, int64_t n, hipStream_t s) {
  if (!x || !y || n <= 0) return hipErrorInvalidValue;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 65536);
  if (y_dtype == DT_BF16) k_cast<bf16_t><<<blocks, 256, 0, s>>>(x, (bf16_t*)y, n);
  else if (y_dtype == DT_F16) k_cast<f16_t><<<blocks, 256, 0, s>>>(x, (f16_t*)y, n);
  else if (y_dtype == DT_F32) k_cast<float><<<blocks, 256, 0, s>>>(x, (float*)y, n);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace wd
