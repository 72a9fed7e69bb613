// Small kernels of the decoder step: weight repack, embedding, row norms,
// Qwen3 per-head QK norm + RoPE + cache append, argmax finalisation and the
// beam-reorder cache gather.  All are tiny next to the weight and cache
// streams; they are written for coalesced 16-byte accesses where it matters.
#include <algorithm>
#include <climits>

#include "wd_common.h"
#include "wd_kernels.h"

namespace wd {

typedef float nt4f __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// repack: row copy with dtype conversion and a row remap (fused q|k|v, gate|up blocks)
// ------------------------------------------------------------------------------------------
template <typename S, typename D>
__global__ void k_copy_rows(const S* __restrict__ src, D* __restrict__ dst, int64_t rows,
                            int64_t cols, int64_t row_mul, int64_t row_add) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i - r * cols;
    dst[(r * row_mul + row_add) * cols + c] = from_f<D>(to_f(src[i]));
  }
}

template <typename S>
static hipError_t copy_rows_to(const S* src, void* dst, int dst_dtype, int64_t rows, int64_t cols,
                               int64_t mul, int64_t add, hipStream_t s) {
  const int64_t n = rows * cols;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 65536);
  if (n <= 0) return hipSuccess;
  switch (dst_dtype) {
    case DT_F32: k_copy_rows<<<blocks, 256, 0, s>>>(src, (float*)dst, rows, cols, mul, add); break;
    case DT_F16: k_copy_rows<<<blocks, 256, 0, s>>>(src, (f16_t*)dst, rows, cols, mul, add); break;
    case DT_BF16: k_copy_rows<<<blocks, 256, 0, s>>>(src, (bf16_t*)dst, rows, cols, mul, add); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, int src_dtype, void* dst, int dst_dtype, int64_t rows,
                            int64_t cols, int64_t row_mul, int64_t row_add, hipStream_t s) {
  switch (src_dtype) {
    case DT_F32: return copy_rows_to((const float*)src, dst, dst_dtype, rows, cols, row_mul, row_add, s);
    case DT_F16: return copy_rows_to((const f16_t*)src, dst, dst_dtype, rows, cols, row_mul, row_add, s);
    case DT_BF16: return copy_rows_to((const bf16_t*)src, dst, dst_dtype, rows, cols, row_mul, row_add, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
__global__ void k_fill(T* p, T v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill<<<(int)std::min<int64_t>((n + 255) / 256, 4096), 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill<<<(int)std::min<int64_t>((n + 255) / 256, 4096), 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// per-call inputs copied into the context's own buffers, so that a captured step graph reads
// fixed addresses: tokens (stride tok_stride), positions (or the constant pos_const when
// pos is null), and optionally B rows of `row_bytes` bytes (source stride src_stride bytes)
// ------------------------------------------------------------------------------------------
__global__ void k_stage(const int32_t* __restrict__ tok, int tok_stride, const int32_t* __restrict__ pos,
                        int pos_const, int32_t* __restrict__ tok_out, int32_t* __restrict__ pos_out, int B,
                        const uint4* __restrict__ rows, int64_t src_stride16, uint4* __restrict__ rows_out,
                        int row16) {
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    tok_out[b] = tok[(int64_t)b * tok_stride];
    pos_out[b] = pos ? pos[b] : pos_const;
  }
  if (rows)
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (int64_t)B * row16;
         i += (int64_t)gridDim.x * blockDim.x) {
      const int64_t b = i / row16, c = i - b * row16;
      rows_out[i] = rows[b * src_stride16 + c];
    }
}

hipError_t launch_stage(const int32_t* tok, int tok_stride, const int32_t* pos, int pos_const, int32_t* tok_out,
                        int32_t* pos_out, int B, const void* rows, int64_t src_stride_bytes, void* rows_out,
                        int64_t row_bytes, hipStream_t s) {
  if (!tok || !tok_out || !pos_out || B <= 0 || B > 1024) return hipErrorInvalidValue;
  if (rows && (row_bytes % 16 || src_stride_bytes % 16 || !rows_out)) return hipErrorInvalidValue;
  const int row16 = rows ? (int)(row_bytes / 16) : 0;
  const int blocks = rows ? (int)std::min<int64_t>(((int64_t)B * row16 + 255) / 256, 1024) : 1;
  k_stage<<<blocks, 256, 0, s>>>(tok, tok_stride, pos, pos_const, tok_out, pos_out, B, (const uint4*)rows,
                                 src_stride_bytes / 16, (uint4*)rows_out, row16);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// embedding: token row + learned position row (Whisper) or token row (Qwen3), or an
// embedding override row (prompt audio splice).  Out-of-range ids/positions raise the
// device flag and produce a zero row.
// ------------------------------------------------------------------------------------------
template <typename WT>
__global__ __launch_bounds__(256) void k_embed(float* __restrict__ x, const WT* __restrict__ E,
                                               const WT* __restrict__ P, const int32_t* tok,
                                               int tok_stride, const int32_t* pos,
                                               const WT* __restrict__ ov, int64_t ov_stride, int d,
                                               int V, int ctx, unsigned* err, bool E_frag) {
  const int b = blockIdx.x;
  const int p = pos[b];
  const bool bad_p = p < 0 || p >= ctx;
  int t = 0;
  bool bad_t = false;
  if (!ov) {
    t = tok[(int64_t)b * tok_stride];
    bad_t = t < 0 || t >= V;
  }
  if (threadIdx.x == 0 && (bad_p || bad_t)) raise_err(err, (bad_p ? ERR_POS : 0u) | (bad_t ? ERR_TOKEN : 0u));
  float* xr = x + (int64_t)b * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float v = 0.f;
    if (!bad_p && !bad_t) {
      if (ov) {
        v = to_f(ov[(int64_t)b * ov_stride + i]);
      } else {
        v = to_f(E[E_frag ? frag_offset(t, i, d) : (int64_t)t * d + i]);
        if (P) v += to_f(P[(int64_t)p * d + i]);
      }
    }
    xr[i] = v;
  }
}

hipError_t launch_embed(float* x, const void* E, const void* P, int w_dtype, const int32_t* tok,
                        int tok_stride, const int32_t* pos, const void* ov, int64_t ov_stride,
                        int B, int d, int V, int ctx, unsigned* err, bool E_frag, hipStream_t s) {
  if (B <= 0 || d <= 0 || (!ov && !tok) || !pos || (E_frag && d % 32)) return hipErrorInvalidValue;
  switch (w_dtype) {
    case DT_F32: k_embed<<<B, 256, 0, s>>>(x, (const float*)E, (const float*)P, tok, tok_stride, pos, (const float*)ov, ov_stride, d, V, ctx, err, E_frag); break;
    case DT_F16: k_embed<<<B, 256, 0, s>>>(x, (const f16_t*)E, (const f16_t*)P, tok, tok_stride, pos, (const f16_t*)ov, ov_stride, d, V, ctx, err, E_frag); break;
    case DT_BF16: k_embed<<<B, 256, 0, s>>>(x, (const bf16_t*)E, (const bf16_t*)P, tok, tok_stride, pos, (const bf16_t*)ov, ov_stride, d, V, ctx, err, E_frag); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// row norms, one block per row, the row read once into registers: LayerNorm takes the
// mean, then the variance of the centred values (eps inside the square root); RMSNorm
// the mean square.  Output fp32 row-major, or the split fragment layout for the MFMA GEMM.
// ------------------------------------------------------------------------------------------
constexpr int NORM_MAXE = 16;  // d <= 4096

// One block per row.
template <typename OT, bool SPLIT>
__global__ __launch_bounds__(256) void k_norm(const float* __restrict__ x, float* __restrict__ y,
                                              OT* __restrict__ yh, OT* __restrict__ yl,
                                              const float* __restrict__ g,
                                              const float* __restrict__ bvec, int d, float eps) {
  __shared__ float red[4];
  const int row = blockIdx.x, t = threadIdx.x;
  const float* xr = x + (int64_t)row * d;
  float v[NORM_MAXE], gv[NORM_MAXE], bv[NORM_MAXE];
#pragma unroll
  for (int j = 0; j < NORM_MAXE; ++j) {  // all loads issued before any reduction
    const int i = t + j * 256;
    v[j] = i < d ? xr[i] : 0.f;
    gv[j] = i < d ? g[i] : 0.f;
    bv[j] = (bvec && i < d) ? bvec[i] : 0.f;
  }
  float mean = 0.f;
  if (bvec) {
    float s1 = 0.f;
#pragma unroll
    for (int j = 0; j < NORM_MAXE; ++j) s1 += v[j];
    mean = block_sum<256>(s1, red) / (float)d;
  }
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < NORM_MAXE; ++j) {
    const int i = t + j * 256;
    const float c = i < d ? v[j] - mean : 0.f;
    s2 += c * c;
  }
  const float rs = 1.0f / sqrtf(block_sum<256>(s2, red) / (float)d + eps);
#pragma unroll
  for (int j = 0; j < NORM_MAXE; ++j) {
    const int i = t + j * 256;
    if (i < d) {
      const float o = (v[j] - mean) * rs * gv[j] + bv[j];
      if constexpr (SPLIT) store_split<OT>(yh, yl, frag_offset(row, i, d), o);
      else y[(int64_t)row * d + i] = o;   // (fp32 path: two-pass mean and variance)
    }
  }
}

// Row norm for the MFMA path, one 256-thread block per row, 4 consecutive columns per thread
// and pass (PASS passes of 1024 columns; d % 32 == 0).  With GMAX > 0, first x += pbias +
// sum_g part[g][row][:] (the G <= GMAX partial slabs of a split-K residual projection,
// added in order g = 0..G-1, all loads in flight together) and the new x is written back.
// The row stays in registers: the mean comes from a first block reduction and the variance
// from a second one over the centred values (no cancellation when the mean is large against
// the spread).  The output goes to the split fragment layout (4 consecutive k are
// contiguous there).  With SKIP (d not a multiple of
// 1024) a wave whose 256 columns of pass j all lie past d loads nothing for that pass, and
// every live pass's loads are issued before any is summed; the sums keep the same order.
template <typename OT, int PASS, int GMAX, bool SKIP>
__global__ __launch_bounds__(256) void k_norm4(float* __restrict__ x, OT* __restrict__ yh, OT* __restrict__ yl,
                                               const float* __restrict__ g, const float* __restrict__ bvec, int d,
                                               float eps, const float* __restrict__ part, int G, int B,
                                               const float* __restrict__ pbias) {
  __shared__ float red[2][4];
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  float* xr = x + (int64_t)row * d;
  float4 v[PASS], gv[PASS], bv[PASS];
  if constexpr (SKIP) {
    const int wcol = 4 * __builtin_amdgcn_readfirstlane(t & ~63);   // first column of this wave
    constexpr int GL = GMAX > 0 ? GMAX : 1;
    float4 pb[PASS], q[PASS][GL];
#pragma unroll
    for (int j = 0; j < PASS; ++j) {
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (wcol + 1024 * j < d) {   // uniform over the wave; lanes past d load the last chunk
        const int c = min(4 * t + 1024 * j, d - 4);
        v[j] = *reinterpret_cast<const float4*>(xr + c);
        gv[j] = *reinterpret_cast<const float4*>(g + c);
        bv[j] = bvec ? *reinterpret_cast<const float4*>(bvec + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (GMAX > 0) {
          pb[j] = pbias ? *reinterpret_cast<const float4*>(pbias + c) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int k = 0; k < GMAX; ++k)
            q[j][k] = __builtin_bit_cast(float4, __builtin_nontemporal_load(
                reinterpret_cast<const nt4f*>(part + ((int64_t)min(k, G - 1) * B + row) * d + c)));
        }
      }
    }
    if constexpr (GMAX > 0) {
#pragma unroll
      for (int j = 0; j < PASS; ++j) {
        if (wcol + 1024 * j < d) {   // x, then the bias, then the partials g = 0..G-1
          float4 a = v[j];
          if (pbias) { a.x += pb[j].x; a.y += pb[j].y; a.z += pb[j].z; a.w += pb[j].w; }
#pragma unroll
          for (int k = 0; k < GMAX; ++k)
            if (k < G) { a.x += q[j][k].x; a.y += q[j][k].y; a.z += q[j][k].z; a.w += q[j][k].w; }
          v[j] = a;
        }
      }
    }
  } else {
#pragma unroll
  for (int j = 0; j < PASS; ++j) {   // loads clamped to the last chunk; chunks past d are not used
    const int c = min(4 * t + 1024 * j, d - 4);
    float4 a = *reinterpret_cast<const float4*>(xr + c);
    gv[j] = *reinterpret_cast<const float4*>(g + c);
    bv[j] = bvec ? *reinterpret_cast<const float4*>(bvec + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (GMAX > 0) {
      if (pbias) {
        const float4 pb = *reinterpret_cast<const float4*>(pbias + c);
        a.x += pb.x; a.y += pb.y; a.z += pb.z; a.w += pb.w;
      }
      float4 q[GMAX];
#pragma unroll
      for (int k = 0; k < GMAX; ++k)
        q[k] = __builtin_bit_cast(float4, __builtin_nontemporal_load(   // read once (see sum_parts)
            reinterpret_cast<const nt4f*>(part + ((int64_t)min(k, G - 1) * B + row) * d + c)));
#pragma unroll
      for (int k = 0; k < GMAX; ++k)
        if (k < G) { a.x += q[k].x; a.y += q[k].y; a.z += q[k].z; a.w += q[k].w; }
    }
    v[j] = a;
  }
  }
  float mean = 0.f;   // LayerNorm (bvec given), or RMSNorm without bias (mean 0)
  if (bvec) {
    float s1 = 0.f;
#pragma unroll
    for (int j = 0; j < PASS; ++j)
      if (4 * t + 1024 * j < d) s1 += (v[j].x + v[j].y) + (v[j].z + v[j].w);
    s1 = wave_sum(s1);
    if (lane == 0) red[0][w] = s1;
    __syncthreads();
    mean = ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) / (float)d;
  }
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < PASS; ++j) {
    const int c = 4 * t + 1024 * j;
    if (c < d) {
      if constexpr (GMAX > 0) *reinterpret_cast<float4*>(xr + c) = v[j];
      const float a = v[j].x - mean, b = v[j].y - mean, e = v[j].z - mean, f = v[j].w - mean;
      s2 += (a * a + b * b) + (e * e + f * f);
    }
  }
  s2 = wave_sum(s2);
  if (lane == 0) red[1][w] = s2;
  __syncthreads();
  const float var = ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) / (float)d;
  const float rs = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int j = 0; j < PASS; ++j) {
    const int c = 4 * t + 1024 * j;
    if (c < d) {
      const float o[4] = {(v[j].x - mean) * rs * gv[j].x + bv[j].x, (v[j].y - mean) * rs * gv[j].y + bv[j].y,
                          (v[j].z - mean) * rs * gv[j].z + bv[j].z, (v[j].w - mean) * rs * gv[j].w + bv[j].w};
      OT h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_hi_lo<OT>(o[e], h[e], l[e]);
      const int64_t off = frag_offset(row, c, d);   // c % 4 == 0: 4 contiguous elements
      uint2 hp, lp;
      __builtin_memcpy(&hp, h, 8);
      __builtin_memcpy(&lp, l, 8);
      *reinterpret_cast<uint2*>(reinterpret_cast<OT*>(yh) + off) = hp;
      *reinterpret_cast<uint2*>(reinterpret_cast<OT*>(yl) + off) = lp;
    }
  }
}

// Norm of x + pbias + sum_g part[g][row][:] (the G partial slabs of a split-K residual
// projection, added in order g = 0..G-1); the new x is written back.  1024 threads per row,
// at most PE elements each, so each thread has all of its PE * GMAX partial loads in flight.
// With SKIP (d not a multiple of 1024), a wave whose columns of pass j all lie past d loads
// nothing for that pass (at d = 1280 the second pass has 4 live waves of 16, which the others
// would only reload clamped; large-v3 step 1.1% faster).  Without SKIP the passes stay
// branch-free (the branches cost the Qwen3 step 1.1% at d = 2048, where every wave is live).
template <typename OT, int PE, int GMAX, bool SKIP>
__global__ __launch_bounds__(1024) void k_norm_part(float* __restrict__ x, OT* __restrict__ yh, OT* __restrict__ yl,
                                                    const float* __restrict__ g, const float* __restrict__ bvec,
                                                    int d, float eps, const float* __restrict__ part, int G, int B,
                                                    const float* __restrict__ pbias) {
  __shared__ float red[16];
  const int row = blockIdx.x, t = threadIdx.x;
  float* xr = x + (int64_t)row * d;
  const int64_t pstride = (int64_t)B * d;
  float v[PE];
  if constexpr (SKIP) {
    const int wbase = __builtin_amdgcn_readfirstlane(t & ~63);   // first column of this wave
    // every live pass's loads are issued before any of them is summed (one round trip; two
    // when the 4-pass, 32-slab case would not fit the 128 registers of a 1024-thread block)
    constexpr int JB = PE * GMAX > 96 ? PE / 2 : PE;
#pragma unroll
    for (int j0 = 0; j0 < PE; j0 += JB) {
      float xb[JB], pv[JB][GMAX];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int j = j0 + jj;
        if (wbase + j * 1024 < d) {   // uniform over the wave
          const int i = min(t + j * 1024, d - 1);
          xb[jj] = xr[i] + (pbias ? pbias[i] : 0.f);
          const float* pp = part + (int64_t)row * d + i;
#pragma unroll
          for (int k = 0; k < GMAX; ++k) pv[jj][k] = __builtin_nontemporal_load(pp + (int64_t)min(k, G - 1) * pstride);
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int j = j0 + jj;
        v[j] = 0.f;
        if (wbase + j * 1024 < d) {
          float sp = 0.f;   // g = 0..G-1 in order, then onto x + bias (as sum_parts adds them)
#pragma unroll
          for (int k = 0; k < GMAX; ++k) sp += k < G ? pv[jj][k] : 0.f;
          v[j] = xb[jj] + sp;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < PE; ++j) {
      const int i = min(t + j * 1024, d - 1);
      v[j] = xr[i] + (pbias ? pbias[i] : 0.f) + sum_parts<GMAX>(part + (int64_t)row * d + i, pstride, G);
    }
  }
  float s1 = 0.f;
#pragma unroll
  for (int j = 0; j < PE; ++j)
    if (t + j * 1024 < d) {
      xr[t + j * 1024] = v[j];
      s1 += v[j];
    }
  float mean = 0.f;
  if (bvec) mean = block_sum<1024>(s1, red) / (float)d;
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < PE; ++j) {
    const float c = t + j * 1024 < d ? v[j] - mean : 0.f;
    s2 += c * c;
  }
  const float rs = 1.0f / sqrtf(block_sum<1024>(s2, red) / (float)d + eps);
#pragma unroll
  for (int j = 0; j < PE; ++j) {
    const int i = t + j * 1024;
    if (i < d) store_split<OT>(yh, yl, frag_offset(row, i, d), (v[j] - mean) * rs * g[i] + (bvec ? bvec[i] : 0.f));
  }
}

template <typename OT>
static hipError_t norm_part(float* x, void* yh, void* yl, const float* g, const float* b, int B, int d, float eps,
                            const float* part, int G, const float* pbias, hipStream_t s) {
  if (G > 32 || d > 4096) return hipErrorInvalidValue;
#define WD_NP(PE_, GM_)                                                                                    \
  do {                                                                                                     \
    if (d % 1024) k_norm_part<OT, PE_, GM_, true><<<B, 1024, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, part, G, B, pbias); \
    else k_norm_part<OT, PE_, GM_, false><<<B, 1024, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, part, G, B, pbias); \
  } while (0)
  if (d <= 2048) {
    if (G <= 8) WD_NP(2, 8); else if (G <= 16) WD_NP(2, 16); else if (G <= 24) WD_NP(2, 24); else WD_NP(2, 32);
  } else {
    if (G <= 8) WD_NP(4, 8); else if (G <= 16) WD_NP(4, 16); else if (G <= 24) WD_NP(4, 24); else WD_NP(4, 32);
  }
#undef WD_NP
  return hipGetLastError();
}

template <typename OT>
static hipError_t norm4(float* x, void* yh, void* yl, const float* g, const float* b, int B, int d, float eps,
                        const float* part, int G, const float* pbias, hipStream_t s) {
  if (d > 4096 || (part && (G < 1 || G > 8))) return hipErrorInvalidValue;
  const int pass = (d + 1023) / 1024;
#define WD_N4(P_, GM_)                                                                                  \
  do {                                                                                                   \
    if (d % 1024) k_norm4<OT, P_, GM_, true><<<B, 256, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, part, G, B, pbias); \
    else k_norm4<OT, P_, GM_, false><<<B, 256, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, part, G, B, pbias); \
  } while (0)
#define WD_N4P(P_) \
  if (!part) WD_N4(P_, 0); else WD_N4(P_, 8);
  if (pass == 1) { WD_N4P(1) } else if (pass == 2) { WD_N4P(2) } else { WD_N4P(4) }
#undef WD_N4P
#undef WD_N4
  return hipGetLastError();
}

hipError_t launch_norm(const float* x, float* y, const float* g, const float* b, int B, int d,
                       float eps, hipStream_t s) {
  if (B <= 0 || d <= 0 || d > 256 * NORM_MAXE || !g) return hipErrorInvalidValue;
  k_norm<float, false><<<B, 256, 0, s>>>(x, y, nullptr, nullptr, g, b, d, eps);
  return hipGetLastError();
}

// Row norm for many rows (the encoder's 96,000 and the prefill chunks' 4,096): one wave per
// row, four rows per block, the row's d = 256 E4 values in registers (E4 float4 per lane),
// both reductions wave-wide (no LDS, no barrier); two passes (mean, then the centred sum of
// squares).  One 256-thread block per row left the encoder's norms bound by block turnover:
// 96,000 short blocks, 438 us per launch at 2.2 TB/s.
// 16 rows (waves) per block: one block writes every row of the 16-row fragment tiles it touches,
// so their lines fill in one XCD's L2 (encoder window 329.4 -> 325.1 ms against 4 rows)
constexpr int NORM_ROWS_PB = 16;
template <typename OT, int E4>
__global__ __launch_bounds__(64 * NORM_ROWS_PB) void k_norm_rows(const float* __restrict__ x, OT* __restrict__ yh,
                                                   OT* __restrict__ yl, const float* __restrict__ g,
                                                   const float* __restrict__ bvec, int d, float eps, int B) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NORM_ROWS_PB + (threadIdx.x >> 6);
  if (row >= B) return;   // the whole wave
  const float* xr = x + (int64_t)row * d;
  float4 v[E4], gv[E4], bv[E4];
#pragma unroll
  for (int j = 0; j < E4; ++j) {
    const int c = 4 * (lane + 64 * j);
    v[j] = *reinterpret_cast<const float4*>(xr + c);
    gv[j] = *reinterpret_cast<const float4*>(g + c);
    bv[j] = bvec ? *reinterpret_cast<const float4*>(bvec + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mean = 0.f;   // LayerNorm (bvec given), or RMSNorm without bias
  if (bvec) {
    float s1 = 0.f;
#pragma unroll
    for (int j = 0; j < E4; ++j) s1 += (v[j].x + v[j].y) + (v[j].z + v[j].w);
    mean = wave_sum(s1) / (float)d;
  }
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < E4; ++j) {
    const float a = v[j].x - mean, b = v[j].y - mean, e = v[j].z - mean, f = v[j].w - mean;
    s2 += (a * a + b * b) + (e * e + f * f);
  }
  const float rs = 1.0f / sqrtf(wave_sum(s2) / (float)d + eps);
#pragma unroll
  for (int j = 0; j < E4; ++j) {
    const int c = 4 * (lane + 64 * j);
    const float o[4] = {(v[j].x - mean) * rs * gv[j].x + bv[j].x, (v[j].y - mean) * rs * gv[j].y + bv[j].y,
                        (v[j].z - mean) * rs * gv[j].z + bv[j].z, (v[j].w - mean) * rs * gv[j].w + bv[j].w};
    OT h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_hi_lo<OT>(o[e], h[e], l[e]);
    const int64_t off = frag_offset(row, c, d);   // 4 contiguous elements
    uint2 hp, lp;
    __builtin_memcpy(&hp, h, 8);
    __builtin_memcpy(&lp, l, 8);
    *reinterpret_cast<uint2*>(yh + off) = hp;
    *reinterpret_cast<uint2*>(yl + off) = lp;
  }
}

template <typename OT>
static hipError_t norm_rows(const float* x, void* yh, void* yl, const float* g, const float* b, int B, int d,
                            float eps, hipStream_t s) {
  const dim3 grid((B + NORM_ROWS_PB - 1) / NORM_ROWS_PB);
  switch (d / 256) {
    case 2: k_norm_rows<OT, 2><<<grid, 64 * NORM_ROWS_PB, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, B); break;
    case 3: k_norm_rows<OT, 3><<<grid, 64 * NORM_ROWS_PB, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, B); break;
    case 4: k_norm_rows<OT, 4><<<grid, 64 * NORM_ROWS_PB, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, B); break;
    case 5: k_norm_rows<OT, 5><<<grid, 64 * NORM_ROWS_PB, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, B); break;
    case 6: k_norm_rows<OT, 6><<<grid, 64 * NORM_ROWS_PB, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, B); break;
    case 8: k_norm_rows<OT, 8><<<grid, 64 * NORM_ROWS_PB, 0, s>>>(x, (OT*)yh, (OT*)yl, g, b, d, eps, B); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_norm_split(float* x, void* y_hi, void* y_lo, int act_dtype, const float* g,
                             const float* b, int B, int d, float eps, hipStream_t s,
                             const float* part, int G, const float* pbias) {
  if (B <= 0 || d <= 0 || d > 4096 || (d % 32) || !g || !y_hi || !y_lo) return hipErrorInvalidValue;
  // many rows and no partial slabs to fold (encoder, prefill chunks): a wave per row
  const int e4 = d / 256;
  if (!part && B >= 1024 && d % 256 == 0 && (e4 >= 2 && e4 <= 8 && e4 != 7)) {
    if (act_dtype == DT_BF16) return norm_rows<bf16_t>(x, y_hi, y_lo, g, b, B, d, eps, s);
    if (act_dtype == DT_F16) return norm_rows<f16_t>(x, y_hi, y_lo, g, b, B, d, eps, s);
    return hipErrorInvalidValue;
  }
  // up to 8 partial slabs: 256 threads with 16-byte loads; more: 1024 threads (more loads in flight)
  const bool wide = part && G > 8;
  if (act_dtype == DT_BF16)
    return wide ? norm_part<bf16_t>(x, y_hi, y_lo, g, b, B, d, eps, part, G, pbias, s)
                : norm4<bf16_t>(x, y_hi, y_lo, g, b, B, d, eps, part, G, pbias, s);
  if (act_dtype == DT_F16)
    return wide ? norm_part<f16_t>(x, y_hi, y_lo, g, b, B, d, eps, part, G, pbias, s)
                : norm4<f16_t>(x, y_hi, y_lo, g, b, B, d, eps, part, G, pbias, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------------
// fragment-layout repack: source row r of a [rows, K] matrix lands in fused row
// (r / 16) * blk_mul * 16 + blk_add * 16 + r % 16 of the destination
// ------------------------------------------------------------------------------------------
template <typename S, typename D>
__global__ void k_pack_frag(const S* __restrict__ src, D* __restrict__ dst, int64_t rows, int64_t K,
                            int64_t blk_mul, int64_t blk_add) {
  const int64_t n = rows * K;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / K, k = i - r * K;
    const int64_t fr = (r >> 4) * blk_mul * 16 + blk_add * 16 + (r & 15);
    dst[frag_offset(fr, k, K)] = from_f<D>(to_f(src[i]));
  }
}

template <typename S>
static hipError_t pack_to(const S* src, void* dst, int dst_dtype, int64_t rows, int64_t K, int64_t mul,
                          int64_t add, hipStream_t s) {
  const int64_t n = rows * K;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 65536);
  if (n <= 0) return hipSuccess;
  switch (dst_dtype) {
    case DT_F16: k_pack_frag<<<blocks, 256, 0, s>>>(src, (f16_t*)dst, rows, K, mul, add); break;
    case DT_BF16: k_pack_frag<<<blocks, 256, 0, s>>>(src, (bf16_t*)dst, rows, K, mul, add); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pack_frag(const void* src, int src_dtype, void* dst, int dst_dtype, int64_t rows,
                            int64_t K, int64_t blk_mul, int64_t blk_add, hipStream_t s) {
  if (K % 32 || blk_mul < 1 || blk_add < 0) return hipErrorInvalidValue;
  if (rows % 16 && blk_mul != 1) return hipErrorInvalidValue;
  switch (src_dtype) {
    case DT_F32: return pack_to((const float*)src, dst, dst_dtype, rows, K, blk_mul, blk_add, s);
    case DT_F16: return pack_to((const f16_t*)src, dst, dst_dtype, rows, K, blk_mul, blk_add, s);
    case DT_BF16: return pack_to((const bf16_t*)src, dst, dst_dtype, rows, K, blk_mul, blk_add, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------------------------------
// Qwen3: per-head RMSNorm of q and k over head_dim, NeoX RoPE at the row's position,
// q scaled by 1/sqrt(hd) into q_out, k and v appended to the cache row.  One wave per
// (head slot, row): slots [0,Hq) are q heads, [Hq,Hq+Hkv) k heads, the rest v heads.
// The rotation angle pos * base^(-2i/hd) and its sine/cosine are taken in double.
// ------------------------------------------------------------------------------------------
template <typename CT, int GMAX>
__global__ __launch_bounds__(64) void k_qk_rope_append(const float* __restrict__ qkv, int Hq, int Hkv,
                                                       int hd, const int32_t* pos, int ctx,
                                                       const float* __restrict__ qn,
                                                       const float* __restrict__ kn, float eps,
                                                       const float* __restrict__ rope_cs, float qscale, float* q_out,
                                                       CT* Kc, CT* Vc, int64_t kv_bstride,
                                                       const float* __restrict__ part, int G, int B, int rps) {
  __shared__ float z[256];
  const int slot = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int nslot = Hq + 2 * Hkv;
  const int64_t off = ((int64_t)b * nslot + slot) * hd;
  float v[4];   // this lane's channels lane + 64 j of the head (hd <= 256)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = min(lane + 64 * j, hd - 1);
    v[j] = part ? sum_parts<GMAX>(part + off + c, (int64_t)B * nslot * hd, G) : qkv[off + c];
  }
  const int p = pos[b];
  const bool ok = p >= 0 && p < ctx;
  if (slot >= Hq + Hkv) {  // value head: plain append
    if (!ok) return;
    const int g = slot - Hq - Hkv;
    CT* dst = Vc + (int64_t)(b / rps) * kv_bstride + ((int64_t)g * ctx + p) * hd;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < hd) dst[lane + 64 * j] = from_f<CT>(v[j]);
    return;
  }
  const float* gain = slot < Hq ? qn : kn;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane + 64 * j < hd) ss += v[j] * v[j];
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane + 64 * j < hd) z[lane + 64 * j] = v[j] * rs * gain[lane + 64 * j];
  __syncthreads();
  const int half = hd / 2;
  const float* cs_row = rope_cs + (int64_t)(ok ? p : 0) * half;
  const float* sn_row = cs_row + (int64_t)ctx * half;
  for (int i = lane; i < half; i += 64) {
    const float cs = cs_row[i], sn = sn_row[i];
    const float a = z[i], bb = z[i + half];
    const float r0 = a * cs - bb * sn, r1 = bb * cs + a * sn;
    if (slot < Hq) {
      float* qo = q_out + ((int64_t)b * Hq + slot) * hd;
      qo[i] = r0 * qscale;
      qo[i + half] = r1 * qscale;
    } else if (ok) {
      const int g = slot - Hq;
      CT* dst = Kc + (int64_t)(b / rps) * kv_bstride + ((int64_t)g * ctx + p) * hd;
      dst[i] = from_f<CT>(r0);
      dst[i + half] = from_f<CT>(r1);
    }
  }
}

template <typename CT>
static void qk_rope_run(dim3 grid, hipStream_t s, const float* qkv, int Hq, int Hkv, int hd, const int32_t* pos,
                        int ctx, const float* qn, const float* kn, float eps, const float* rope_cs, float qscale, float* q_out,
                        void* Kc, void* Vc, int64_t kv_bstride, const float* part, int G, int B, int rps) {
  if (!part || G <= 8)
    k_qk_rope_append<CT, 8><<<grid, 64, 0, s>>>(qkv, Hq, Hkv, hd, pos, ctx, qn, kn, eps, rope_cs, qscale, q_out,
                                                (CT*)Kc, (CT*)Vc, kv_bstride, part, G, B, rps);
  else if (G <= 16)
    k_qk_rope_append<CT, 16><<<grid, 64, 0, s>>>(qkv, Hq, Hkv, hd, pos, ctx, qn, kn, eps, rope_cs, qscale, q_out,
                                                 (CT*)Kc, (CT*)Vc, kv_bstride, part, G, B, rps);
  else
    k_qk_rope_append<CT, 32><<<grid, 64, 0, s>>>(qkv, Hq, Hkv, hd, pos, ctx, qn, kn, eps, rope_cs, qscale, q_out,
                                                 (CT*)Kc, (CT*)Vc, kv_bstride, part, G, B, rps);
}

hipError_t launch_qk_rope_append(const float* qkv, int B, int Hq, int Hkv, int hd, const int32_t* pos,
                                 int ctx, const float* qn, const float* kn, float eps, const float* rope_cs,
                                 float qscale, float* q_out, void* Kc, void* Vc, int cache_dtype,
                                 int64_t kv_bstride, hipStream_t s, const float* part, int G, int rps) {
  if (B <= 0 || hd > 256 || (hd % 2) || Hq <= 0 || Hkv <= 0 || rps < 1 || !rope_cs) return hipErrorInvalidValue;
  if (part ? (G < 1 || G > 32) : !qkv) return hipErrorInvalidValue;
  dim3 grid(Hq + 2 * Hkv, B);
  switch (cache_dtype) {
    case DT_F32: qk_rope_run<float>(grid, s, qkv, Hq, Hkv, hd, pos, ctx, qn, kn, eps, rope_cs, qscale, q_out, Kc, Vc, kv_bstride, part, G, B, rps); break;
    case DT_F16: qk_rope_run<f16_t>(grid, s, qkv, Hq, Hkv, hd, pos, ctx, qn, kn, eps, rope_cs, qscale, q_out, Kc, Vc, kv_bstride, part, G, B, rps); break;
    case DT_BF16: qk_rope_run<bf16_t>(grid, s, qkv, Hq, Hkv, hd, pos, ctx, qn, kn, eps, rope_cs, qscale, q_out, Kc, Vc, kv_bstride, part, G, B, rps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_rope_table(float* __restrict__ cs, int ctx, int hd, float base) {
  const int half = hd / 2;
  const int64_t n = (int64_t)ctx * half;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    const int p = (int)(j / half), i = (int)(j - (int64_t)p * half);
    const double th = (double)p * pow((double)base, -2.0 * (double)i / (double)hd);
    cs[j] = (float)cos(th);
    cs[n + j] = (float)sin(th);
  }
}

hipError_t launch_rope_table(float* cs, int ctx, int hd, float base, hipStream_t s) {
  if (!cs || ctx <= 0 || hd <= 0 || hd % 2 || !(base > 0.f)) return hipErrorInvalidValue;
  const int blocks = (int)std::min<int64_t>(((int64_t)ctx * (hd / 2) + 255) / 256, 4096);
  k_rope_table<<<blocks, 256, 0, s>>>(cs, ctx, hd, base);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// argmax: max over the per-block keys of each row; the key order makes the lowest
// index win ties.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_argmax_final(const unsigned long long* __restrict__ amax,
                                                      int nparts, int ldp, int32_t* out) {
  __shared__ unsigned long long red[256];
  const int b = blockIdx.x;
  unsigned long long m = 0;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    const unsigned long long k = amax[(int64_t)i * ldp + b];
    m = k > m ? k : m;
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      const unsigned long long o = red[threadIdx.x + s];
      if (o > red[threadIdx.x]) red[threadIdx.x] = o;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[b] = (int32_t)(0xffffffffu - (uint32_t)(red[0] & 0xffffffffull));
}

hipError_t launch_argmax_final(const unsigned long long* amax, int nparts, int ldp, int B,
                               int32_t* out, hipStream_t s) {
  if (B <= 0 || nparts <= 0 || ldp < B) return hipErrorInvalidValue;
  k_argmax_final<<<B, 256, 0, s>>>(amax, nparts, ldp, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// beam candidates: per row the W largest logits (ties: lower id first; NaN counts as -inf) and
// the row's log-sum-exp, so log_softmax(v) = logit(v) - lse.  Pass 1: TK_P blocks per row, each
// over a contiguous part of the row; every thread keeps its own top W and (max, sum exp), the
// block merges the lists pairwise in LDS and writes one partial list and (max, sum exp).  Pass
// 2: one wave per row merges the TK_P partial lists and sums.  (Register lists are indexed
// with compile-time indices only, so they stay in registers.)
// ------------------------------------------------------------------------------------------
constexpr int TK_MAX = 8, TK_NT = 256, TK_P = 32, TK_EPT = 8;   // TK_EPT: loads per thread per pass

__device__ __forceinline__ bool tk_better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// insert (x, i) into the sorted list (v, id) of length W (<= TK_MAX) if it belongs there
__device__ __forceinline__ void tk_insert(float (&v)[TK_MAX], int (&id)[TK_MAX], int W, float x, int i) {
  float lv = v[0];
  int li = id[0];
#pragma unroll
  for (int k = 1; k < TK_MAX; ++k)
    if (k == W - 1) { lv = v[k]; li = id[k]; }
  if (!tk_better(x, i, lv, li)) return;
  bool placed = false;
#pragma unroll
  for (int k = TK_MAX - 1; k >= 1; --k) {
    if (k < W && !placed) {
      if (tk_better(x, i, v[k - 1], id[k - 1])) { v[k] = v[k - 1]; id[k] = id[k - 1]; }
      else { v[k] = x; id[k] = i; placed = true; }
    }
  }
  if (!placed) { v[0] = x; id[0] = i; }
}

// (max, sum exp) pairs: merge b into a
__device__ __forceinline__ void tk_lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  s = (m == -INFINITY ? 0.f : s * expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mn));
  m = mn;
}

// Order-preserving 64-bit key of (value, id): larger key = larger value, then lower id (-0 is
// taken as +0, as the value comparison takes them equal).
__device__ __forceinline__ unsigned long long tk_key(float v, int id) {
  const uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)(0x7FFFFFFF - id);
}

// The wave's best W entries over its lanes' sorted lists, in order: W rounds of a butterfly
// maximum of the lanes' head keys; the lane whose head won moves on (equal keys are only the
// empty (-inf, INT_MAX) entries, past which every list stays empty).  Round k's entry goes to
// out_v[k] / out_i[k] from lane 0 (out_* may be LDS or global).
__device__ __forceinline__ void tk_wave_merge(const float (&v)[TK_MAX], const int (&id)[TK_MAX], int W,
                                              float* out_v, int* out_i) {
  const int t = threadIdx.x & 63;
  int h = 0;   // this lane's next unconsumed entry
  for (int k = 0; k < W; ++k) {
    float hv = -INFINITY;
    int hi = INT_MAX;
#pragma unroll
    for (int j = 0; j < TK_MAX; ++j)
      if (j == h) { hv = v[j]; hi = id[j]; }
    const unsigned long long mine = tk_key(hv, hi);
    unsigned long long best = mine;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long other = __shfl_xor(best, o, WAVE);
      best = other > best ? other : best;
    }
    if (mine == best) ++h;
    if (t == 0) {
      const uint32_t ob = (uint32_t)(best >> 32);
      out_v[k] = __uint_as_float((ob & 0x80000000u) ? (ob & 0x7FFFFFFFu) : ~ob);
      out_i[k] = 0x7FFFFFFF - (int)(uint32_t)(best & 0xFFFFFFFFu);
    }
  }
}

__global__ __launch_bounds__(TK_NT) void k_topk_part(const float* __restrict__ logits, int V, int64_t ld, int W,
                                                      int chunk, float* __restrict__ pv, int* __restrict__ pi,
                                                      float* __restrict__ pm, float* __restrict__ ps) {
  __shared__ float sv[TK_NT / 64][TK_MAX];
  __shared__ int si[TK_NT / 64][TK_MAX];
  __shared__ float sm[TK_NT / 64], ss[TK_NT / 64];
  const int part = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const float* row = logits + (int64_t)b * ld;
  const int i0 = part * chunk, i1 = min(V, i0 + chunk);
  float v[TK_MAX];
  int id[TK_MAX];
#pragma unroll
  for (int k = 0; k < TK_MAX; ++k) { v[k] = -INFINITY; id[k] = INT_MAX; }
  float m = -INFINITY, sum = 0.f;
  for (int base = i0; base < i1; base += TK_NT * TK_EPT) {
    float xs[TK_EPT];   // every load of the pass in flight before any is used
#pragma unroll
    for (int u = 0; u < TK_EPT; ++u) {
      const int i = base + t + u * TK_NT;
      xs[u] = row[min(i, i1 - 1)];
    }
#pragma unroll
    for (int u = 0; u < TK_EPT; ++u) {
      const int i = base + t + u * TK_NT;
      if (i < i1) {
        float x = xs[u];
        if (x != x) x = -INFINITY;   // NaN
        if (x != -INFINITY) {
          if (x > m) { sum = sum * expf(m - x) + 1.f; m = x; }
          else sum += expf(x - m);
        }
        tk_insert(v, id, W, x, i);
      }
    }
  }
  // each wave's best W into LDS, then wave 0 merges the waves' lists
  tk_wave_merge(v, id, W, sv[t >> 6], si[t >> 6]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tk_lse_merge(m, sum, __shfl_xor(m, o, WAVE), __shfl_xor(sum, o, WAVE));
  if ((t & 63) == 0) { sm[t >> 6] = m; ss[t >> 6] = sum; }
  __syncthreads();
  if (t >= 64) return;
#pragma unroll
  for (int k = 0; k < TK_MAX; ++k) {
    const bool in = t < TK_NT / 64 && k < W;
    v[k] = in ? sv[min(t, TK_NT / 64 - 1)][k] : -INFINITY;
    id[k] = in ? si[min(t, TK_NT / 64 - 1)][k] : INT_MAX;
  }
  const int64_t o = ((int64_t)b * gridDim.x + part);
  tk_wave_merge(v, id, W, pv + o * TK_MAX, pi + o * TK_MAX);
  if (t == 0) {
    float M = sm[0], S = ss[0];
    for (int w = 1; w < TK_NT / 64; ++w) tk_lse_merge(M, S, sm[w], ss[w]);
    pm[o] = M;
    ps[o] = S;
  }
}

__global__ __launch_bounds__(64) void k_topk_final(const float* __restrict__ pv, const int* __restrict__ pi,
                                                    const float* __restrict__ pm, const float* __restrict__ ps,
                                                    int P, int W, float* __restrict__ top_val,
                                                    int32_t* __restrict__ top_id, float* __restrict__ lse) {
  const int b = blockIdx.x, t = threadIdx.x;
  float v[TK_MAX];
  int id[TK_MAX];
#pragma unroll
  for (int k = 0; k < TK_MAX; ++k) { v[k] = -INFINITY; id[k] = INT_MAX; }
  float m = -INFINITY, s = 0.f;
  for (int q = t; q < P; q += 64) {   // lane t: the lists of parts t, t + 64, ...
    const int64_t o = (int64_t)b * P + q;
#pragma unroll
    for (int k = 0; k < TK_MAX; ++k)
      if (k < W) tk_insert(v, id, W, pv[o * TK_MAX + k], pi[o * TK_MAX + k]);
    tk_lse_merge(m, s, pm[o], ps[o]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tk_lse_merge(m, s, __shfl_xor(m, o, WAVE), __shfl_xor(s, o, WAVE));
  tk_wave_merge(v, id, W, top_val + (int64_t)b * W, top_id + (int64_t)b * W);
  if (t == 0) lse[b] = m == -INFINITY ? -INFINITY : m + logf(s);
}

int topk_parts(int V) { return std::max(1, std::min(TK_P, (V + 4 * TK_NT - 1) / (4 * TK_NT))); }

size_t topk_scratch_bytes(int B, int V) {
  const size_t P = topk_parts(V);
  return (size_t)B * P * (TK_MAX * 8 + 8);
}

hipError_t launch_topk_lse(const float* logits, int B, int V, int64_t ld, int W, float* top_val, int32_t* top_id,
                           float* lse, void* scratch, hipStream_t s) {
  if (!logits || !top_val || !top_id || !lse || !scratch || B <= 0 || V <= 0 || ld < V || W < 1 || W > TK_MAX ||
      W > V)
    return hipErrorInvalidValue;
  const int P = topk_parts(V), chunk = (V + P - 1) / P;
  float* pv = reinterpret_cast<float*>(scratch);
  int* pi = reinterpret_cast<int*>(pv + (size_t)B * P * TK_MAX);
  float* pm = reinterpret_cast<float*>(pi + (size_t)B * P * TK_MAX);
  float* ps = pm + (size_t)B * P;
  k_topk_part<<<dim3(P, B), TK_NT, 0, s>>>(logits, V, ld, W, chunk, pv, pi, pm, ps);
  k_topk_final<<<B, 64, 0, s>>>(pv, pi, pm, ps, P, W, top_val, top_id, lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// beam reorder: for every (layer, K|V) block, new row b <- old row idx[b], cache rows
// 0..n_rows-1 of every head, 16 bytes per thread.  Source and destination are the two
// halves of the ping-pong cache, so the gather never reads what it writes.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_reorder(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                 BeamIdx idx, int H, int64_t slab_vec,
                                                 int64_t copy_vec, int64_t block_vec) {
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int64_t blk = (int64_t)blockIdx.z * block_vec;
  const int64_t so = blk + ((int64_t)idx.v[b] * H + h) * slab_vec;
  const int64_t dof = blk + ((int64_t)b * H + h) * slab_vec;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < copy_vec; i += (int64_t)gridDim.x * 256)
    dst[dof + i] = src[so + i];
}

hipError_t launch_reorder(const void* src, void* dst, int elt_bytes, const BeamIdx& idx, int B, int Bmax,
                          int H, int ctx, int hd, int n_rows, int n_blocks, hipStream_t s) {
  if (B <= 0 || B > 64 || B > Bmax || n_rows < 0 || n_rows > ctx || n_blocks <= 0) return hipErrorInvalidValue;
  if (((int64_t)hd * elt_bytes) % 16) return hipErrorInvalidValue;
  for (int b = 0; b < B; ++b)
    if (idx.v[b] < 0 || idx.v[b] >= B) return hipErrorInvalidValue;
  if (n_rows == 0) return hipSuccess;
  const int64_t row_vec = (int64_t)hd * elt_bytes / 16;
  const int64_t slab_vec = (int64_t)ctx * row_vec;
  const int64_t copy_vec = (int64_t)n_rows * row_vec;
  const int64_t block_vec = (int64_t)Bmax * H * slab_vec;
  dim3 grid((unsigned)std::min<int64_t>((copy_vec + 255) / 256, 64), B * H, n_blocks);
  k_reorder<<<grid, 256, 0, s>>>((const uint4*)src, (uint4*)dst, idx, H, slab_vec, copy_vec, block_vec);
  return hipGetLastError();
}

template <bool DEV>
__global__ __launch_bounds__(256) void k_reorder_dev(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     const int32_t* __restrict__ idx, int B, int H, int64_t slab_vec,
                                                     int64_t copy_vec, int64_t block_vec) {
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int from = min(max(idx[b], 0), B - 1);
  const int64_t blk = (int64_t)blockIdx.z * block_vec;
  const int64_t so = blk + ((int64_t)from * H + h) * slab_vec;
  const int64_t dof = blk + ((int64_t)b * H + h) * slab_vec;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < copy_vec; i += (int64_t)gridDim.x * 256)
    dst[dof + i] = src[so + i];
}

hipError_t launch_reorder_dev(const void* src, void* dst, int elt_bytes, const int32_t* idx, int B, int Bmax,
                              int H, int ctx, int hd, int n_rows, int n_blocks, hipStream_t s) {
  if (!idx || B <= 0 || B > Bmax || n_rows < 0 || n_rows > ctx || n_blocks <= 0) return hipErrorInvalidValue;
  if (((int64_t)hd * elt_bytes) % 16) return hipErrorInvalidValue;
  if (n_rows == 0) return hipSuccess;
  const int64_t row_vec = (int64_t)hd * elt_bytes / 16;
  const int64_t slab_vec = (int64_t)ctx * row_vec;
  const int64_t copy_vec = (int64_t)n_rows * row_vec;
  const int64_t block_vec = (int64_t)Bmax * H * slab_vec;
  dim3 grid((unsigned)std::min<int64_t>((copy_vec + 255) / 256, 64), B * H, n_blocks);
  k_reorder_dev<true><<<grid, 256, 0, s>>>((const uint4*)src, (uint4*)dst, idx, B, H, slab_vec, copy_vec, block_vec);
  return hipGetLastError();
}

// Beam selection in one wave: lane i < rows * W holds candidate (i / W, i % W).  Each of the W
// rounds takes the best remaining candidate by a butterfly over the 64 lanes (a total order:
// not NaN before NaN, then higher score, then lower flat index), and the lane holding it drops
// out.  Every score is read before any is written, so `scores` is updated in place.
struct BeamKey { double c; long long flat; int live; };
__device__ __forceinline__ bool beam_better(const BeamKey& a, const BeamKey& b) {
  if (a.live != b.live) return a.live > b.live;
  const bool an = a.c != a.c, bn = b.c != b.c;
  if (an != bn) return bn;
  if (!an && a.c != b.c) return a.c > b.c;
  return a.flat < b.flat;
}
__global__ __launch_bounds__(64) void k_beam_merge(const float* __restrict__ top_val, const int32_t* __restrict__ top_id,
                                                   const float* __restrict__ lse, double* scores,
                                                   int32_t* __restrict__ beam_idx, int32_t* __restrict__ tokens, int W,
                                                   int rows, int V) {
  const int lane = threadIdx.x;
  BeamKey me{-INFINITY, 0x7fffffffffffffffLL, 0};
  if (lane < rows * W) {
    const int b = lane / W;
    me.c = scores[b] + ((double)top_val[lane] - (double)lse[b]);
    me.flat = (long long)b * V + top_id[lane];
    me.live = 1;
  }
  double out_c = 0.0;
  long long out_flat = 0;
  for (int r = 0; r < W; ++r) {
    BeamKey best = me;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      BeamKey other;
      other.c = __shfl_xor(best.c, o, 64);
      other.flat = __shfl_xor(best.flat, o, 64);
      other.live = __shfl_xor(best.live, o, 64);
      if (beam_better(other, best)) best = other;
    }
    if (me.live && me.flat == best.flat) me.live = 0;   // flat indices are distinct
    if (lane == r) {
      out_c = best.c;
      out_flat = best.flat;
    }
  }
  if (lane < W) {
    scores[lane] = out_c;
    beam_idx[lane] = (int32_t)(out_flat / V);
    tokens[lane] = (int32_t)(out_flat % V);
  }
}

hipError_t launch_beam_merge(const float* top_val, const int32_t* top_id, const float* lse, double* scores,
                             int32_t* beam_idx, int32_t* tokens, int W, int rows, int V, hipStream_t s) {
  if (!top_val || !top_id || !lse || !scores || !beam_idx || !tokens || W < 1 || W > 8 || V < 1 ||
      (rows != 1 && rows != W))
    return hipErrorInvalidValue;
  k_beam_merge<<<1, 64, 0, s>>>(top_val, top_id, lse, scores, beam_idx, tokens, W, rows, V);
  return hipGetLastError();
}

}  // namespace wd
