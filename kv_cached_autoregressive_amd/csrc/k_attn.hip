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
// Per block, one pass over its rows: K and V rows stream together (16 B per
// lane; a wave covers 4 or 8 whole rows per load, fully coalesced), the lanes of
// a row reduce the q.k dot product with DPP adds, and each lane keeps an online
// softmax state (running max, running exp-sum and its slice of the weighted V
// sum), rescaled when the max grows.  The lanes' states are merged at the end
// (DPP moves and permlane swaps within a wave, LDS across waves).
//
// Scores are kept in base 2: q is scaled by log2(e) once, so every exponential
// is a bare v_exp_f32 and the softmax weights are unchanged.  With a 16-bit
// cache q is split into (hi, lo) halves of the cache type (q = hi + lo to about
// 16 bits, each half's products exact in fp32), so the 8 channels a lane holds
// take 8 packed dot2 instructions and the K row is never unpacked.  With one split the block
// normalises and writes o; otherwise it writes (o, max, sum) partials that a
// combine kernel rescales and adds.
#include <algorithm>
#include <type_traits>

#include "wd_common.h"
#include "wd_kernels.h"

namespace wd {

// K/V rows are read once per launch: nontemporal loads keep them from displacing the L2
// lines other data lives in (measured: the large-v3 cross-attention went from 87.5 to
// 76.3 us per launch, and the rest of the step sped up too).
typedef uint32_t nt4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ Raw8<float> fetch8_nt(const float* p) {
  Raw8<float> r;
  const nt4u a = __builtin_nontemporal_load(reinterpret_cast<const nt4u*>(p));
  const nt4u b = __builtin_nontemporal_load(reinterpret_cast<const nt4u*>(p) + 1);
  r.a = __builtin_bit_cast(float4, a); r.b = __builtin_bit_cast(float4, b);
  return r;
}
// 8 floats rounded to the cache type, in the register form a fetch produces
template <typename CT>
__device__ __forceinline__ Raw8<CT> pack8(const float* f) {
  Raw8<CT> r;
  if constexpr (sizeof(CT) == 4) {
    r.a = make_float4(f[0], f[1], f[2], f[3]);
    r.b = make_float4(f[4], f[5], f[6], f[7]);
  } else {
    CT h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = from_f<CT>(f[e]);
    __builtin_memcpy(&r.v, h, 16);
  }
  return r;
}
template <typename T>
__device__ __forceinline__ Raw8<T> fetch8_nt(const T* p) {
  Raw8<T> r;
  const nt4u a = __builtin_nontemporal_load(reinterpret_cast<const nt4u*>(p));
  r.v = __builtin_bit_cast(uint4, a);
  return r;
}

constexpr float ATT_LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// q in the form the score takes: fp32 for a float cache, else (hi, lo) pairs of the cache type
template <typename CT> struct QOp { uint32_t h[4], l[4]; };
template <> struct QOp<float> { float v[8]; };
template <typename CT>
__device__ __forceinline__ QOp<CT> make_qop(const float (&f)[8]) {
  QOp<CT> q;
  if constexpr (sizeof(CT) == 4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) q.v[j] = f[j];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t hb[2], lb[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float v = f[2 * i + e];
        if constexpr (std::is_same<CT, bf16_t>::value) {
          const __bf16 h = (__bf16)v, l = (__bf16)(v - (float)h);
          hb[e] = __builtin_bit_cast(uint16_t, h);
          lb[e] = __builtin_bit_cast(uint16_t, l);
        } else {
          const f16_t h = (f16_t)v, l = (f16_t)(v - (float)h);
          hb[e] = __builtin_bit_cast(uint16_t, h);
          lb[e] = __builtin_bit_cast(uint16_t, l);
        }
      }
      q.h[i] = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
      q.l[i] = (uint32_t)lb[0] | ((uint32_t)lb[1] << 16);
    }
  }
  return q;
}
// this lane's part of q.k over its 8 channels
template <typename CT>
__device__ __forceinline__ float qk8(const QOp<CT>& q, const Raw8<CT>& k) {
  if constexpr (sizeof(CT) == 4) {
    float kf[8];
    unpack8(k, kf);
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) d = fmaf(q.v[j], kf[j], d);
    return d;
  } else {
    const uint32_t kw[4] = {k.v.x, k.v.y, k.v.z, k.v.w};
    float dh = 0.f, dl = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (std::is_same<CT, bf16_t>::value) {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        dh = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, q.h[i]), __builtin_bit_cast(b2, kw[i]), dh, false);
        dl = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, q.l[i]), __builtin_bit_cast(b2, kw[i]), dl, false);
      } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        dh = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, q.h[i]), __builtin_bit_cast(h2, kw[i]), dh, false);
        dl = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, q.l[i]), __builtin_bit_cast(h2, kw[i]), dl, false);
      }
    }
    return dh + dl;
  }
}

// o for (row bq, head h, channel c): fp32 row-major, or split fragment layout
__device__ __forceinline__ void write_o(float* out, int out_ld, void* o_hi, void* o_lo, int o_dtype, int Hq,
                                        int HD, int bq, int h, int c, float v) {
  if (o_hi) {
    const int64_t off = frag_offset(bq, (int64_t)h * HD + c, (int64_t)Hq * HD);
    if (o_dtype == DT_BF16) store_split<bf16_t>(o_hi, o_lo, off, v);
    else store_split<f16_t>(o_hi, o_lo, off, v);
  } else {
    out[(int64_t)bq * out_ld + h * HD + c] = v;
  }
}

// One query per block (NQ == 1) is kept to <= 96 VGPRs: 5 waves per SIMD, so the self
// attention's 1280 blocks of 4 waves (64 rows x 20 heads) are resident at once, with no
// second partial round.  The cross attention, 1500 rows per slab, and any launch with fewer
// slabs take NW = 8 waves (more rows in flight per slab).  CROSS only separates the two uses into distinct kernels for profiling (the cross
// attention over the encoder frames has no positions; the self attention reads rows 0..pos).
template <typename CT, int HD, int NQ, bool CROSS, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn(AttnParams p) {
  constexpr int NT = 64 * NW;
  constexpr int SEGS = HD / 8;          // lanes per cache row (16 bytes each)
  constexpr int RPP = NT / SEGS;        // rows per block pass
  // rows per pass per lane (x2 in flight), for K and for V; 8 queries per block keep 3 (2 in
  // 4-wave blocks) so that nothing spills (the 5-beam cross-attention)
  constexpr int UNR = NQ >= 8 && NW == 4 ? 2 : NQ == 1 || NQ >= 8 ? 3 : 4;
  __shared__ float red[NW][NQ][HD + 2];

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
  } else if (p.rows_kvb) {   // ragged KV sets: this set's own length
    n_rows = min(max(p.rows_kvb[kvb], 0), p.n_rows_fixed);
  }
  const int r_lo = s * p.split_rows;
  const int r_hi = min(r_lo + p.split_rows, n_rows);

  auto qrow = [&](int qi) { return bq0 + qi / G; };
  auto qhead = [&](int qi) { return g * G + qi % G; };

  if (r_lo >= r_hi) {  // empty split: neutral partial (or zero output)
    for (int i = t; i < nq * HD; i += NT) {
      const int qi = i / HD, c = i - qi * HD;
      const int bq = qrow(qi), h = qhead(qi);
      if (p.n_splits == 1) {
        write_o(p.out, p.out_ld, p.o_hi, p.o_lo, p.o_dtype, p.Hq, HD, bq, h, c, 0.f);
      } else {
        float* pp = p.part + (((int64_t)bq * p.Hq + h) * p.n_splits + s) * (HD + 2);
        pp[c] = 0.f;
        if (c == 0) { pp[HD] = -INFINITY; pp[HD + 1] = 0.f; }
      }
    }
    return;
  }

  // (no __restrict__: the append below writes a row that the loop then reads)
  const CT* Kp = reinterpret_cast<const CT*>(p.K) + (int64_t)kvb * p.kvb_stride + (int64_t)g * p.rows_cap * HD;
  const CT* Vp = reinterpret_cast<const CT*>(p.V) + (int64_t)kvb * p.kvb_stride + (int64_t)g * p.rows_cap * HD;
  const int64_t qslab = (int64_t)p.B * p.qpart_ld;
  // the in-order sum of a value's qG partial slabs, with 8 loads in flight when qG <= 8 (the
  // usual split) and 16 otherwise: slots past qG reload the last slab, so fewer slots mean
  // fewer wasted loads (early-position large-v3 self-attention 13.3 -> 12.5 us)
  auto psum = [&](const float* src) __attribute__((always_inline)) {
    return p.qG <= 8 ? sum_parts<8>(src, qslab, p.qG) : sum_parts<16>(src, qslab, p.qG);
  };

  // Software pipeline: the K/V rows of the next pass are requested before the current one
  // is reduced, so a wave never waits on an empty queue; UNR is sized so the single-query
  // kernel stays at <= 96 VGPRs (5 waves per SIMD, all blocks resident).  Rows past the
  // split reload its last row (not counted); no load sits under a branch.
  Raw8<CT> kr[UNR], vr[UNR];
  auto fetch = [&](int r0, Raw8<CT> (&kd)[UNR], Raw8<CT> (&vd)[UNR]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int ru = min(r0 + u * RPP, r_hi - 1);
      kd[u] = fetch8_nt(Kp + (int64_t)ru * HD + seg * 8);
      vd[u] = fetch8_nt(Vp + (int64_t)ru * HD + seg * 8);
    }
  };
  // The first pass is requested before the q prologue below, so its latency overlaps the
  // partial sums; a row appended by the prologue is patched into it from LDS.
  fetch(r_lo + rr, kr, vr);
  __shared__ float apv[2 * HD];   // the appended row (k, then v) before rounding to the cache type
  const int ps_app = n_rows - 1;
  const bool appended = p.qpart && p.append && p.pos && ps_app >= r_lo && ps_app < r_hi;

  // q (and the appended row) from split-K partials: each value is summed once per block
  // (one thread per value, its G loads in flight together), q through LDS
  __shared__ float qs[NQ * HD];
  if (p.qpart && p.rope) {
    // Qwen3: raw q heads and the appended k, v summed into LDS, then per-head RMSNorm and
    // the NeoX rotation (cos and sin of the position's angles from the table)
    __shared__ float kvs[2 * HD], cs_[HD / 2], sn_[HD / 2], rsq[NQ + 1];
    const int ps = n_rows - 1;
    const bool own = p.append && ps >= r_lo && ps < r_hi;
    // the rotation of row ps, requested by the block's last HD/2 threads ahead of the sums
    const int ti = t - (NT - HD / 2);
    float rc = 0.f, rsn = 0.f;
    if (ti >= 0) {
      rc = p.rope_cs[(int64_t)ps * (HD / 2) + ti];
      rsn = p.rope_cs[((int64_t)p.rows_cap + ps) * (HD / 2) + ti];
    }
    // q values, then the appended k and v, spread over the threads (one round trip when
    // nq * HD + 2 HD <= NT)
    const int nqv = nq * HD;
    for (int i = t; i < nqv + (own ? 2 * HD : 0); i += NT) {
      if (i < nqv) {
        const int qi = i / HD, c = i - qi * HD;
        qs[i] = psum(p.qpart + (int64_t)qrow(qi) * p.qpart_ld + p.q_off + qhead(qi) * HD + c);
      } else {
        const int j = i - nqv, c = j % HD;
        kvs[j] = psum(p.qpart + (int64_t)bq0 * p.qpart_ld + (j >= HD ? p.v_off : p.k_off) + g * HD + c);
      }
    }
    if (ti >= 0) {
      cs_[ti] = rc;
      sn_[ti] = rsn;
    }
    __syncthreads();
    const int nh = nq + (own ? 1 : 0);   // q heads, then the appended k
    for (int hh = wv; hh < nh; hh += NW) {
      const float* z = hh < nq ? qs + hh * HD : kvs;
      float ss = 0.f;
      for (int c = lane; c < HD; c += 64) ss += z[c] * z[c];
      ss = wave_sum(ss);
      if (lane == 0) rsq[hh] = 1.0f / sqrtf(ss / (float)HD + p.eps);
    }
    __syncthreads();
    CT* Kw = reinterpret_cast<CT*>(const_cast<void*>(p.K)) + (int64_t)kvb * p.kvb_stride + ((int64_t)g * p.rows_cap + ps) * HD;
    CT* Vw = reinterpret_cast<CT*>(const_cast<void*>(p.V)) + (int64_t)kvb * p.kvb_stride + ((int64_t)g * p.rows_cap + ps) * HD;
    for (int j = t; j < nh * (HD / 2); j += NT) {
      const int hh = j / (HD / 2), i = j - hh * (HD / 2);
      float* z = hh < nq ? qs + hh * HD : kvs;
      const float* gain = hh < nq ? p.qn : p.kn;
      const float a = z[i] * rsq[hh] * gain[i], b2 = z[i + HD / 2] * rsq[hh] * gain[i + HD / 2];
      const float r0 = a * cs_[i] - b2 * sn_[i], r1 = b2 * cs_[i] + a * sn_[i];
      if (hh < nq) {
        z[i] = r0 * p.qscale;
        z[i + HD / 2] = r1 * p.qscale;
      } else {
        Kw[i] = from_f<CT>(r0);
        Kw[i + HD / 2] = from_f<CT>(r1);
        apv[i] = r0;
        apv[i + HD / 2] = r1;
      }
    }
    if (own)
      for (int c = t; c < HD; c += NT) {
        Vw[c] = from_f<CT>(kvs[HD + c]);
        apv[HD + c] = kvs[HD + c];
      }
    __syncthreads();   // q in LDS; the appended row visible to the block's loads below
  } else if (p.qpart) {
    // q values, then (when the appended row lives in this block's split) its k and v, spread
    // over the threads; the row is written before any row is read
    const int nqv = nq * HD;
    for (int i = t; i < nqv + (appended ? 2 * HD : 0); i += NT) {
      if (i < nqv) {
        const int qi = i / HD, c = i - qi * HD;
        const int col = qhead(qi) * HD + c;
        const float* src = p.qpart + (int64_t)qrow(qi) * p.qpart_ld + p.q_off + col;
        qs[i] = (psum(src) + (p.qbias ? p.qbias[col] : 0.f)) * p.qscale;
      } else {
        const int j = i - nqv, c = j % HD;
        const bool isv = j >= HD;
        const float* src = p.qpart + (int64_t)bq0 * p.qpart_ld + (isv ? p.v_off : p.k_off) + g * HD + c;
        float v = psum(src);
        if (isv && p.vbias) v += p.vbias[g * HD + c];
        CT* base = reinterpret_cast<CT*>(const_cast<void*>(isv ? p.V : p.K));
        base[(int64_t)kvb * p.kvb_stride + ((int64_t)g * p.rows_cap + ps_app) * HD + c] = from_f<CT>(v);
        apv[j] = v;
      }
    }
    __syncthreads();   // q in LDS; the appended row visible to the block's loads below
  }
  if (appended) {   // the prefetched first pass predates the append: take that row from LDS
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (min(r_lo + rr + u * RPP, r_hi - 1) == ps_app) {
        kr[u] = pack8<CT>(apv + seg * 8);
        vr[u] = pack8<CT>(apv + HD + seg * 8);
      }
  }

  QOp<CT> qv[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    float f[8];
    if (qi < nq) {
      if (p.qpart) {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = qs[qi * HD + seg * 8 + j];
      } else {
        load8(p.q + (int64_t)qrow(qi) * p.q_ld + qhead(qi) * HD + seg * 8, f);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] *= ATT_LOG2E;
    qv[qi] = make_qop<CT>(f);
  }

  // one pass over the rows: each lane keeps, per query, the running max m, the
  // running sum l of exp(score - m) and its slice of sum exp(score - m) * V
  float m[NQ], l[NQ], acc[NQ][8];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    m[qi] = -INFINITY;
    l[qi] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[qi][j] = 0.f;
  }
  // the rows of one pass (kr, vr hold them) into each lane's running state
  auto pass = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const bool live = r + u * RPP < r_hi;
      float vf[8];
      unpack8(vr[u], vf);
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        const float d = seg_sum<SEGS>(qk8<CT>(qv[qi], kr[u]));
        if (live && qi < nq) {
          if (d > m[qi]) {  // new running max: rescale what was accumulated
            const float sc = exp2_fast(m[qi] - d);
            l[qi] *= sc;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[qi][j] *= sc;
            m[qi] = d;
          }
          const float e = exp2_fast(d - m[qi]);
          l[qi] += e;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[qi][j] = fmaf(e, vf[j], acc[qi][j]);
        }
      }
    }
  };
  // every pass but the last requests the next one first; the last requests nothing, so no
  // block waits on loads it will not use (trip count uniform over the block)
  const int npass = (r_hi - r_lo + RPP * UNR - 1) / (RPP * UNR);
  int r = r_lo + rr;
  for (int it = 1; it < npass; ++it, r += RPP * UNR) {
    Raw8<CT> kn[UNR], vn[UNR];
    fetch(r + RPP * UNR, kn, vn);
    pass(r);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      kr[u] = kn[u];
      vr[u] = vn[u];
    }
  }
  pass(r);
  // merge the (m, l, acc) of the lanes holding the same segment: within the wave,
  // then across the NW waves through LDS
  auto merge = [&](auto off) __attribute__((always_inline)) {
    constexpr int OFF = decltype(off)::value;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      float mu, mw, lu, lw;
      lane_pair<OFF>(m[qi], mu, mw);
      lane_pair<OFF>(l[qi], lu, lw);
      const float mn = fmaxf(mu, mw);
      const float fu = mn == -INFINITY ? 0.f : exp2_fast(mu - mn);
      const float fw = mn == -INFINITY ? 0.f : exp2_fast(mw - mn);
      l[qi] = lu * fu + lw * fw;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float au, aw;
        lane_pair<OFF>(acc[qi][j], au, aw);
        acc[qi][j] = au * fu + aw * fw;
      }
      m[qi] = mn;
    }
  };
  if constexpr (SEGS == 8) merge(std::integral_constant<int, 8>());
  merge(std::integral_constant<int, 16>());
  merge(std::integral_constant<int, 32>());
  if (lane < SEGS) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wv][qi][seg * 8 + j] = acc[qi][j];
      if (seg == 0) { red[wv][qi][HD] = m[qi]; red[wv][qi][HD + 1] = l[qi]; }
    }
  }
  __syncthreads();
  for (int i = t; i < nq * HD; i += NT) {
    const int qi = i / HD, c = i - qi * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, red[w2][qi][HD]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const float f = red[w2][qi][HD] == -INFINITY ? 0.f : exp2_fast(red[w2][qi][HD] - M);
      L += f * red[w2][qi][HD + 1];
      o += f * red[w2][qi][c];
    }
    const int bq = qrow(qi), h = qhead(qi);
    if (p.n_splits == 1) {
      write_o(p.out, p.out_ld, p.o_hi, p.o_lo, p.o_dtype, p.Hq, HD, bq, h, c, o / L);
    } else {
      float* pp = p.part + (((int64_t)bq * p.Hq + h) * p.n_splits + s) * (HD + 2);
      pp[c] = o;
      if (c == 0) { pp[HD] = M; pp[HD + 1] = L; }
    }
  }
}

// Every split's (m, l, o[c]) is loaded before any arithmetic (splits past n_splits reload
// the last one and get weight 0), so the loads overlap instead of one round trip per split.
template <int HD, int MAXS>
__global__ __launch_bounds__(HD) void k_attn_combine(const float* __restrict__ part, int n_splits,
                                                     float* __restrict__ out, int out_ld, int Hq,
                                                     void* o_hi, void* o_lo, int o_dtype) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const int b = bh / Hq, h = bh - (bh / Hq) * Hq;
  const float* pp = part + (int64_t)bh * n_splits * (HD + 2);
  float m[MAXS], l[MAXS], ov[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const float* q = pp + min(s, n_splits - 1) * (HD + 2);
    m[s] = q[HD];
    l[s] = q[HD + 1];
    ov[s] = q[c];
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) M = s < n_splits ? fmaxf(M, m[s]) : M;
  float L = 0.f, o = 0.f;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const float w = (s < n_splits && M != -INFINITY) ? exp2_fast(m[s] - M) : 0.f;
    L += w * l[s];
    o += w * ov[s];
  }
  write_o(out, out_ld, o_hi, o_lo, o_dtype, Hq, HD, b, h, c, L > 0.f ? o / L : 0.f);
}

template <typename CT, int HD, bool C, int NW>
static hipError_t run_nw(const AttnParams& p, int nq, hipStream_t s) {
  dim3 grid(p.n_splits, p.Hkv, p.B / p.q_per_kvb);
  if (nq <= 1) k_attn<CT, HD, 1, C, NW><<<grid, 64 * NW, 0, s>>>(p);
  else if (nq <= 2) k_attn<CT, HD, 2, C, NW><<<grid, 64 * NW, 0, s>>>(p);
  else if (nq <= 4) k_attn<CT, HD, 4, C, NW><<<grid, 64 * NW, 0, s>>>(p);
  else k_attn<CT, HD, 8, C, NW><<<grid, 64 * NW, 0, s>>>(p);
  return hipGetLastError();
}

template <typename CT, int HD>
static hipError_t run_hd(const AttnParams& p, int nq, hipStream_t s) {
  if (p.pos) return p.nw == 8 ? run_nw<CT, HD, false, 8>(p, nq, s) : run_nw<CT, HD, false, 4>(p, nq, s);
  return p.nw == 8 ? run_nw<CT, HD, true, 8>(p, nq, s) : run_nw<CT, HD, true, 4>(p, nq, s);
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
  if (nq > 8 || p.split_rows <= 0 || p.n_splits <= 0 || (p.nw != 4 && p.nw != 8)) return hipErrorInvalidValue;
  if (p.pos && p.q_per_kvb != 1) return hipErrorInvalidValue;  // per-row lengths need own slabs
  if (!p.pos && (p.n_rows_fixed < 0 || p.n_rows_fixed > p.rows_cap)) return hipErrorInvalidValue;
  if ((int64_t)p.split_rows * p.n_splits < (p.pos ? p.rows_cap : p.n_rows_fixed)) return hipErrorInvalidValue;
  if (p.n_splits > 1 && !p.part) return hipErrorInvalidValue;
  if ((!p.q && !p.qpart) || !p.K || !p.V || (!p.qpart && (p.q_ld % 4))) return hipErrorInvalidValue;
  if (p.qpart && (p.qG < 1 || p.qG > 16 || p.qpart_ld <= 0)) return hipErrorInvalidValue;
  if (p.append && (!p.qpart || !p.pos || (p.Hq != p.Hkv && !p.rope))) return hipErrorInvalidValue;
  if (p.rope && (!p.qpart || !p.pos || !p.qn || !p.kn || !(p.eps > 0.f) || !p.rope_cs))
    return hipErrorInvalidValue;
  if (p.o_hi ? (!p.o_lo || (p.Hq * p.hd) % 32 || (p.o_dtype != DT_F16 && p.o_dtype != DT_BF16))
             : (!p.out || p.out_ld < p.Hq * p.hd))
    return hipErrorInvalidValue;
  switch (p.cache_dtype) {
    case DT_F32: return run_ct<float>(p, nq, s);
    case DT_F16: return run_ct<f16_t>(p, nq, s);
    case DT_BF16: return run_ct<bf16_t>(p, nq, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_combine(const AttnParams& p, hipStream_t s) {
  if (p.n_splits <= 1) return hipSuccess;
  if (!p.part || (!p.out && !p.o_hi)) return hipErrorInvalidValue;
  if (p.n_splits > 64) return hipErrorInvalidValue;
#define WD_CMB(HD_, MS_) \
  k_attn_combine<HD_, MS_><<<p.B * p.Hq, HD_, 0, s>>>(p.part, p.n_splits, p.out, p.out_ld, p.Hq, p.o_hi, p.o_lo, p.o_dtype)
  if (p.hd == 64) {
    if (p.n_splits <= 8) WD_CMB(64, 8); else if (p.n_splits <= 16) WD_CMB(64, 16);
    else if (p.n_splits <= 32) WD_CMB(64, 32); else WD_CMB(64, 64);
  } else if (p.hd == 128) {
    if (p.n_splits <= 8) WD_CMB(128, 8); else if (p.n_splits <= 16) WD_CMB(128, 16);
    else if (p.n_splits <= 32) WD_CMB(128, 32); else WD_CMB(128, 64);
  } else {
    return hipErrorInvalidValue;
  }
#undef WD_CMB
  return hipGetLastError();
}

}  // namespace wd
