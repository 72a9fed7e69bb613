// Attention of one query token per row over a K/V cache, split over cache rows
// (flash-decoding).  Used for the causal self-attention (rows 0..pos of the
// row's own cache, appended before this launch) and for the cross-attention
// (all frames of the row's encoder set, no mask).
//
// One block = (row split, kv head, kv batch).  Every query that reads that K/V
// slab is served by the same block, so the slab is streamed from HBM once: the
// beams of a beam search sharing one broadcast encoder set, and the query
// heads of a GQA group.
//
// Per block: pass 1 streams K rows (16 B per lane, a wave covers 4 or 8 whole
// rows per load so loads are fully coalesced), dots them with the query slice
// each lane holds in registers and reduces over the lanes of a row; scores go to
// LDS.  Pass 2 takes the max and exp-sums (fp32).  Pass 3 streams V rows with
// the same lane mapping and accumulates p_j * V_j.  With one split the block
// normalises and writes o; otherwise it writes (o, max, sum) partials that a
// combine kernel rescales and adds.
#include <algorithm>

#include "wd_common.h"
#include "wd_kernels.h"

namespace wd {

template <typename CT, int HD, int NQ>
__global__ __launch_bounds__(256) void k_attn(AttnParams p) {
  constexpr int SEGS = HD / 8;          // lanes per cache row
  constexpr int RPP = 256 / SEGS;       // rows per block pass
  constexpr int UNR = 4;                // independent row loads in flight per lane
  extern __shared__ float sc[];         // scores [NQ][split_rows]
  __shared__ float red[4][NQ][HD];
  __shared__ float stat[2][NQ][4];

  const int s = blockIdx.x, g = blockIdx.y, kvb = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int seg = t % SEGS, rr = t / SEGS;
  const int G = p.Hq / p.Hkv;
  const int nq = p.q_per_kvb * G;
  const int bq0 = kvb * p.q_per_kvb;

  int n_rows = p.n_rows_fixed;
  if (p.pos) {
    const int ps = p.pos[bq0];
    n_rows = (ps < 0 || ps >= p.rows_cap) ? 0 : ps + 1;
  }
  const int r_lo = s * p.split_rows;
  const int r_hi = min(r_lo + p.split_rows, n_rows);
  const int SR = p.split_rows;

  auto qrow = [&](int qi) { return bq0 + qi / G; };
  auto qhead = [&](int qi) { return g * G + qi % G; };

  if (r_lo >= r_hi) {  // empty split: neutral partial (or zero output)
    for (int i = t; i < nq * HD; i += 256) {
      const int qi = i / HD, c = i - qi * HD;
      const int bq = qrow(qi), h = qhead(qi);
      if (p.n_splits == 1) {
        p.out[(int64_t)bq * p.out_ld + h * HD + c] = 0.f;
      } else {
        float* pp = p.part + (((int64_t)bq * p.Hq + h) * p.n_splits + s) * (HD + 2);
        pp[c] = 0.f;
        if (c == 0) { pp[HD] = -INFINITY; pp[HD + 1] = 0.f; }
      }
    }
    return;
  }

  const CT* __restrict__ Kp = reinterpret_cast<const CT*>(p.K) + (int64_t)kvb * p.kvb_stride + (int64_t)g * p.rows_cap * HD;
  const CT* __restrict__ Vp = reinterpret_cast<const CT*>(p.V) + (int64_t)kvb * p.kvb_stride + (int64_t)g * p.rows_cap * HD;

  float qv[NQ][8];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    if (qi < nq) {
      load8(p.q + (int64_t)qrow(qi) * p.q_ld + qhead(qi) * HD + seg * 8, qv[qi]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[qi][j] = 0.f;
    }
  }

  // ---- pass 1: scores -------------------------------------------------------------------
  for (int r = r_lo + rr; r - rr < r_hi; r += RPP * UNR) {
    Raw8<CT> raw[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int ru = min(r + u * RPP, r_hi - 1);
      raw[u] = fetch8(Kp + (int64_t)ru * HD + seg * 8);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float kf[8];
      unpack8(raw[u], kf);
      const int ru = r + u * RPP;
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) d = fmaf(qv[qi][j], kf[j], d);
#pragma unroll
        for (int o = 1; o < SEGS; o <<= 1) d += __shfl_xor(d, o, WAVE);
        if (seg == 0 && ru < r_hi && qi < nq) sc[qi * SR + (ru - r_lo)] = d;
      }
    }
  }
  __syncthreads();

  // ---- pass 2: max and exp-sum per query ------------------------------------------------------
  const int nr = r_hi - r_lo;
  float mq[NQ], lq[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    float m = -INFINITY;
    if (qi < nq)
      for (int i = t; i < nr; i += 256) m = fmaxf(m, sc[qi * SR + i]);
    m = wave_max(m);
    if (lane == 0) stat[0][qi][wv] = m;
  }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi)
    mq[qi] = fmaxf(fmaxf(stat[0][qi][0], stat[0][qi][1]), fmaxf(stat[0][qi][2], stat[0][qi][3]));
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    float l = 0.f;
    if (qi < nq)
      for (int i = t; i < nr; i += 256) {
        const float e = expf(sc[qi * SR + i] - mq[qi]);
        sc[qi * SR + i] = e;
        l += e;
      }
    l = wave_sum(l);
    if (lane == 0) stat[1][qi][wv] = l;
  }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) lq[qi] = stat[1][qi][0] + stat[1][qi][1] + stat[1][qi][2] + stat[1][qi][3];

  // ---- pass 3: weighted sum of V rows -------------------------------------------------------------
  float acc[NQ][8];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[qi][j] = 0.f;
  for (int r = r_lo + rr; r - rr < r_hi; r += RPP * UNR) {
    Raw8<CT> raw[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int ru = min(r + u * RPP, r_hi - 1);
      raw[u] = fetch8(Vp + (int64_t)ru * HD + seg * 8);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int ru = r + u * RPP;
      if (ru < r_hi) {
        float vf[8];
        unpack8(raw[u], vf);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
          if (qi < nq) {
            const float w = sc[qi * SR + (ru - r_lo)];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[qi][j] = fmaf(w, vf[j], acc[qi][j]);
          }
        }
      }
    }
  }
  // reduce over the lanes of a wave that hold the same segment, then over waves
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = acc[qi][j];
#pragma unroll
      for (int o = SEGS; o < 64; o <<= 1) a += __shfl_xor(a, o, WAVE);
      acc[qi][j] = a;
    }
  if (lane < SEGS) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wv][qi][seg * 8 + j] = acc[qi][j];
  }
  __syncthreads();
  for (int i = t; i < nq * HD; i += 256) {
    const int qi = i / HD, c = i - qi * HD;
    float o = 0.f;
    float m = 0.f, l = 1.f;
#pragma unroll
    for (int q2 = 0; q2 < NQ; ++q2)
      if (q2 == qi) { m = mq[q2]; l = lq[q2]; }
    o = red[0][qi][c] + red[1][qi][c] + red[2][qi][c] + red[3][qi][c];
    const int bq = qrow(qi), h = qhead(qi);
    if (p.n_splits == 1) {
      p.out[(int64_t)bq * p.out_ld + h * HD + c] = o / l;
    } else {
      float* pp = p.part + (((int64_t)bq * p.Hq + h) * p.n_splits + s) * (HD + 2);
      pp[c] = o;
      if (c == 0) { pp[HD] = m; pp[HD + 1] = l; }
    }
  }
}

template <int HD>
__global__ __launch_bounds__(HD) void k_attn_combine(const float* __restrict__ part, int n_splits,
                                                     float* __restrict__ out, int out_ld, int Hq) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const int b = bh / Hq, h = bh - (bh / Hq) * Hq;
  const float* pp = part + (int64_t)bh * n_splits * (HD + 2);
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, pp[s * (HD + 2) + HD]);
  float L = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float* q = pp + s * (HD + 2);
      const float w = expf(q[HD] - M);
      L += w * q[HD + 1];
      o += w * q[c];
    }
  }
  out[(int64_t)b * out_ld + h * HD + c] = L > 0.f ? o / L : 0.f;
}

template <typename CT, int HD>
static hipError_t run_hd(const AttnParams& p, int nq, hipStream_t s) {
  dim3 grid(p.n_splits, p.Hkv, p.B / p.q_per_kvb);
  // the kernel touches score rows qi < nq only
  const size_t smem = (size_t)p.split_rows * nq * sizeof(float);
  if (nq <= 1) k_attn<CT, HD, 1><<<grid, 256, smem, s>>>(p);
  else if (nq <= 2) k_attn<CT, HD, 2><<<grid, 256, smem, s>>>(p);
  else if (nq <= 4) k_attn<CT, HD, 4><<<grid, 256, smem, s>>>(p);
  else k_attn<CT, HD, 8><<<grid, 256, smem, s>>>(p);
  return hipGetLastError();
}

template <typename CT>
static hipError_t run_ct(const AttnParams& p, int nq, hipStream_t s) {
  if (p.hd == 64) return run_hd<CT, 64>(p, nq, s);
  if (p.hd == 128) return run_hd<CT, 128>(p, nq, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  if (p.B <= 0 || p.Hq <= 0 || p.Hkv <= 0 || p.Hq % p.Hkv || p.q_per_kvb <= 0 || p.B % p.q_per_kvb)
    return hipErrorInvalidValue;
  const int nq = p.q_per_kvb * (p.Hq / p.Hkv);
  if (nq > 8 || p.split_rows <= 0 || p.n_splits <= 0) return hipErrorInvalidValue;
  if ((size_t)p.split_rows * nq * sizeof(float) > 48 * 1024) return hipErrorInvalidValue;
  if (p.pos && p.q_per_kvb != 1) return hipErrorInvalidValue;  // per-row lengths need own slabs
  if (!p.pos && (p.n_rows_fixed < 0 || p.n_rows_fixed > p.rows_cap)) return hipErrorInvalidValue;
  if ((int64_t)p.split_rows * p.n_splits < (p.pos ? p.rows_cap : p.n_rows_fixed)) return hipErrorInvalidValue;
  if (p.n_splits > 1 && !p.part) return hipErrorInvalidValue;
  if (!p.q || !p.K || !p.V || !p.out || (p.q_ld % 4) || (p.out_ld < p.Hq * p.hd)) return hipErrorInvalidValue;
  switch (p.cache_dtype) {
    case DT_F32: return run_ct<float>(p, nq, s);
    case DT_F16: return run_ct<f16_t>(p, nq, s);
    case DT_BF16: return run_ct<bf16_t>(p, nq, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_combine(const AttnParams& p, hipStream_t s) {
  if (p.n_splits <= 1) return hipSuccess;
  if (!p.part || !p.out) return hipErrorInvalidValue;
  if (p.hd == 64) k_attn_combine<64><<<p.B * p.Hq, 64, 0, s>>>(p.part, p.n_splits, p.out, p.out_ld, p.Hq);
  else if (p.hd == 128) k_attn_combine<128><<<p.B * p.Hq, 128, 0, s>>>(p.part, p.n_splits, p.out, p.out_ld, p.Hq);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace wd
