// Host runtime of the decoder step: configuration checks, workspace plan, weight
// repack, and the launch sequence of one step.  Exports the C ABI of wd.h.
//
// Device layout inside the caller's workspace (every region 256-byte aligned):
//   weights    per layer, row-major [out, in] in w_dtype, row blocks fused:
//              Whisper q|k|v [3d, d], cross k|v [2d, d]; Qwen3 q|k|v
//              [(Hq+2Hkv)hd, d], gate|up [2ff, d]; biases and norm vectors fp32
//              (the K blocks of the fused biases are zero)
//   self cache per buffer, per layer: K then V, each [max_batch][Hkv][context][hd]
//              (head-major, one contiguous [context, hd] slab per row and head);
//              two buffers when the rows share one encoder set (beam reorder)
//   cross      per layer: K then V, each [n_enc][H][max_frames][hd]
//   scratch    x, y, q, qkv, o, h (fp32), split partials, argmax keys, error word
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "wd.h"
#include "wd_kernels.h"

namespace {

using wd::DT_BF16;
using wd::DT_F16;
using wd::DT_F32;

thread_local std::string g_load_error;

int dtype_bytes(int dt) { return dt == DT_F32 ? 4 : (dt == DT_F16 || dt == DT_BF16) ? 2 : 0; }

struct LayerOff {
  // Whisper
  size_t wqkv, wo, wcq, wckv, wco, w1, w2;
  size_t bqkv, bo, bcq, bckv, bco, b1, b2, ln1g, ln1b, ln2g, ln2b, ln3g, ln3b;
  // Qwen3
  size_t wgu, wdn, n1g, n2g, qn, kn;
};

struct Plan {
  size_t total = 0;
  bool mfma = false;        // 16-bit weights: fragment layout + MFMA skinny GEMM
  size_t yh = 0, yl = 0, oh = 0, ol = 0, hh = 0, hl = 0;   // split activations [B_pad, K]
  std::vector<LayerOff> L;
  size_t embed = 0, pos = 0, lnfg = 0, lnfb = 0;
  size_t self[2] = {0, 0};
  size_t self_slab = 0;   // bytes of one K (or V) block of one layer
  int n_bufs = 1;
  size_t cross = 0, cross_slab = 0;
  size_t xfrag = 0;          // encoder states in fragment order (cross-K/V GEMM operand, 16-bit)
  size_t frames_dev = 0;     // per encoder set frame counts [n_enc] int32 (ragged windows)
  size_t x = 0, y = 0, q = 0, qkv = 0, o = 0, h = 0, part = 0, amax = 0, err = 0, pos_tmp = 0;
  size_t rope = 0;           // Qwen3: cos [context][hd/2], then sin [context][hd/2]
  size_t topk = 0;           // wd_topk partial lists
  size_t beam = 0;           // wd_beam_step candidates: values [8][8] f32, ids [8][8] i32, lse [8] f32
  size_t gpart = 0; int64_t gpart_cap = 0;   // split-K GEMM partials [G][B][N] fp32
  size_t tok_in = 0, ov_in = 0;              // staged tokens [B] and embedding override rows [B, d]
  int max_splits = 1, amax_parts = 1;
  // batched Qwen3 prefill: chunks of pf_pos_chunk positions for all rows (pf_rows = rows of a chunk)
  int pf_rows = 0, pf_pos_chunk = 0;
  size_t pf_x = 0, pf_pos = 0, pf_ah = 0, pf_al = 0, pf_hh = 0, pf_hl = 0, pf_qkv = 0, pf_q = 0;
};

struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    const size_t at = off;
    off += bytes;
    return at;
  }
};

// Activation rows padded to the MFMA GEMM's row tile (16, 32 or 64 rows): every row a
// tile reads exists (rows past B stay zero).
int row_pad(int max_batch) { return max_batch <= 16 ? 16 : max_batch <= 32 ? 32 : 64; }

bool valid_dt(int dt) { return dt == DT_F32 || dt == DT_F16 || dt == DT_BF16; }

// Returns an empty string when cfg is acceptable, else the reason.
std::string check_config(const wd_config& c) {
  if (c.arch != WD_ARCH_WHISPER && c.arch != WD_ARCH_QWEN3) return "arch must be 0 (whisper) or 1 (qwen3)";
  if (c.d_model <= 0 || c.d_model % 32) return "d_model must be a positive multiple of 32";
  if (c.head_dim != 64 && c.head_dim != 128) return "head_dim must be 64 or 128";
  if (c.n_heads <= 0 || c.n_kv_heads <= 0 || c.n_heads % c.n_kv_heads) return "n_kv_heads must divide n_heads";
  if (c.n_heads / c.n_kv_heads > 8) return "at most 8 query heads per kv head";
  if (c.n_layers <= 0 || c.vocab <= 0 || c.context <= 0) return "n_layers, vocab, context must be positive";
  if (c.d_ff <= 0 || c.d_ff % 8) return "d_ff must be a positive multiple of 8";
  if (c.max_batch < 1 || c.max_batch > WD_MAX_BATCH) return "max_batch must be in [1, 64]";
  if (!valid_dt(c.w_dtype) || !valid_dt(c.cache_dtype)) return "unknown dtype";
  if (!(c.norm_eps > 0.f)) return "norm_eps must be positive";
  if (c.arch == WD_ARCH_WHISPER) {
    if (c.n_kv_heads != c.n_heads || c.n_heads * c.head_dim != c.d_model) return "whisper: heads * head_dim must equal d_model";
    if (c.max_frames <= 0) return "whisper: max_frames must be positive";
    if (c.w_dtype != DT_F32 && c.d_model % 128) return "whisper: 16-bit weights need d_model % 128 == 0 (cross K/V GEMM tiles)";
    if (c.n_enc <= 0 || c.max_batch % c.n_enc) return "whisper: n_enc must divide max_batch";
    if (c.max_batch / c.n_enc > 8) return "whisper: at most 8 rows per encoder set";
  } else {
    if (!(c.rope_base > 0.f)) return "qwen3: rope_base must be positive";
    if (c.n_enc != 0) return "qwen3: n_enc must be 0";
  }
  return "";
}

// Launch shape of an attention over `rows` cache rows of `slabs` K/V slabs (measured on the
// three batched workloads):
//  * >= 512 slabs: one block per slab, of 4 waves for the self-attention (5 resident per CU
//    at <= 96 VGPRs) and of 8 for the cross-attention over all encoder frames (its 1500 rows
//    per slab want more rows in flight: 74.8 against 76.0 us per large-v3 launch);
//  * otherwise blocks of 8 waves and about 256 blocks in total, so a slab is split only
//    below ~170 slabs (each split costs a combine launch, about 4 us): one split at the
//    192 slabs of the whisper-small step, 4 splits of 256 rows at the 64 of the Qwen3 step;
//  * splits of at least 64 rows, at most 64 splits (the combine's limit).
void split_for(int rows, int slabs, int nq, int* split_rows, int* n_splits, int* nw, bool cross = false) {
  const bool wide = slabs < 512;
  const int want = wide ? std::max(1, (256 + slabs / 2) / slabs) : 1;
  int r = (rows + want - 1) / want;
  r = std::max(r, (rows + 63) / 64);   // at most 64 splits (the combine's limit)
  r = std::max(r, 64);
  r = (r + 31) & ~31;
  r = std::min(r, std::max(12288 / std::max(nq, 1), (rows + 63) / 64));
  r = std::max(r, 1);
  *split_rows = r;
  *n_splits = std::max(1, (rows + r - 1) / r);
  *nw = (wide || cross) ? 8 : 4;
}

// Rows per chunk of the batched prefill (streams x positions): they feed dense MFMA GEMMs;
// 4096 rows (512 positions of 8 streams) make 512 output tiles of 128 x 128 at N = 2048.
// Measured on the 900-position, 8-stream prefill: 103 ms at 128 positions per chunk, 72 at
// 256, 62 at 512, 67-68 at 768 and 1024.
constexpr int PF_ROWS = 4096, PF_MAX_POS = 512;
int pf_positions(int max_batch) {
  return std::max(16, std::min(PF_MAX_POS, PF_ROWS / max_batch / 16 * 16));
}

Plan make_plan(const wd_config& c) {
  Plan p;
  Bump b;
  const size_t d = c.d_model, ff = c.d_ff, hd = c.head_dim, hq = c.n_heads, hkv = c.n_kv_heads;
  const size_t wb = dtype_bytes(c.w_dtype), cb = dtype_bytes(c.cache_dtype), f4 = 4;
  const size_t Bm = c.max_batch;
  p.mfma = c.w_dtype != DT_F32;
  // fragment layout pads matrix rows to 16 (only the tied head's vocab rows can be ragged)
  const size_t V = p.mfma ? ((size_t)c.vocab + 15) / 16 * 16 : (size_t)c.vocab;
  p.L.resize(c.n_layers);
  for (auto& l : p.L) {
    std::memset(&l, 0, sizeof(l));
    if (c.arch == WD_ARCH_WHISPER) {
      l.wqkv = b.take(3 * d * d * wb); l.wo = b.take(d * d * wb); l.wcq = b.take(d * d * wb);
      l.wckv = b.take(2 * d * d * wb); l.wco = b.take(d * d * wb);
      l.w1 = b.take(ff * d * wb); l.w2 = b.take(d * ff * wb);
      l.bqkv = b.take(3 * d * f4); l.bo = b.take(d * f4); l.bcq = b.take(d * f4);
      l.bckv = b.take(2 * d * f4); l.bco = b.take(d * f4); l.b1 = b.take(ff * f4); l.b2 = b.take(d * f4);
      l.ln1g = b.take(d * f4); l.ln1b = b.take(d * f4); l.ln2g = b.take(d * f4);
      l.ln2b = b.take(d * f4); l.ln3g = b.take(d * f4); l.ln3b = b.take(d * f4);
    } else {
      l.wqkv = b.take((hq + 2 * hkv) * hd * d * wb); l.wo = b.take(d * hq * hd * wb);
      l.wgu = b.take(2 * ff * d * wb); l.wdn = b.take(d * ff * wb);
      l.n1g = b.take(d * f4); l.n2g = b.take(d * f4); l.qn = b.take(hd * f4); l.kn = b.take(hd * f4);
    }
  }
  p.embed = b.take(V * d * wb);
  if (c.arch == WD_ARCH_WHISPER) {
    p.pos = b.take((size_t)c.context * d * wb);
    p.lnfb = b.take(d * f4);
  }
  p.lnfg = b.take(d * f4);
  p.n_bufs = (c.arch == WD_ARCH_WHISPER && c.n_enc == 1 && c.max_batch > 1) ? 2 : 1;
  p.self_slab = Bm * hkv * (size_t)c.context * hd * cb;
  for (int i = 0; i < p.n_bufs; ++i) p.self[i] = b.take(2 * p.self_slab * c.n_layers);
  if (c.arch == WD_ARCH_WHISPER) {
    p.cross_slab = (size_t)c.n_enc * hq * (size_t)c.max_frames * hd * cb;
    p.cross = b.take(2 * p.cross_slab * c.n_layers);
    if (p.mfma) p.xfrag = b.take(((size_t)c.n_enc * c.max_frames + 255) / 256 * 256 * d * wb);   // X in fragment order
    p.frames_dev = b.take((size_t)c.n_enc * 4);
  }
  const size_t wide = std::max({d, 2 * ff, (hq + 2 * hkv) * hd});
  p.x = b.take(Bm * d * f4);
  p.y = b.take(Bm * wide * f4);
  p.q = b.take(Bm * hq * hd * f4);
  p.qkv = b.take(Bm * (hq + 2 * hkv) * hd * f4);
  p.o = b.take(Bm * hq * hd * f4);
  p.h = b.take(Bm * 2 * ff * f4);
  const int rows_max = std::max(c.context, c.arch == WD_ARCH_WHISPER ? c.max_frames : 0);
  p.max_splits = (rows_max + 63) / 64;
  p.part = b.take(Bm * hq * (size_t)p.max_splits * (hd + 2) * f4);
  if (p.mfma) {
    const size_t Bp = row_pad(c.max_batch);
    const size_t kmax = std::max(d, hq * hd);
    p.yh = b.take(Bp * kmax * wb); p.yl = b.take(Bp * kmax * wb);
    p.oh = b.take(Bp * hq * hd * wb); p.ol = b.take(Bp * hq * hd * wb);
    p.hh = b.take(Bp * ff * wb); p.hl = b.take(Bp * ff * wb);
    int64_t cap = 0;
    auto shape = [&](int N, int K, int epi) {
      const int G = wd::mgemv_groups(N, K, c.max_batch, epi);
      if (G > 1) cap = std::max(cap, (int64_t)G * (int64_t)Bm * N);
    };
    if (c.arch == WD_ARCH_WHISPER) {
      shape(3 * d, d, wd::EPI_QKV); shape(d, d, wd::EPI_RESID); shape(d, d, wd::EPI_STORE);
      shape(ff, d, wd::EPI_GELU_SPLIT); shape(d, ff, wd::EPI_RESID);
    } else {
      shape((hq + 2 * hkv) * hd, d, wd::EPI_STORE); shape(d, hq * hd, wd::EPI_RESID);
      shape(2 * ff, d, wd::EPI_SWIGLU_SPLIT); shape(d, ff, wd::EPI_RESID);
    }
    p.gpart_cap = cap;
    if (cap) p.gpart = b.take((size_t)cap * f4);
  }
  p.amax_parts = std::max(wd::gemv_blocks(c.vocab, c.max_batch), wd::mgemv_blocks(c.vocab, c.max_batch));
  p.amax = b.take((size_t)p.amax_parts * Bm * 8);
  p.topk = b.take(wd::topk_scratch_bytes((int)Bm, c.vocab));   // beam-candidate partial lists
  p.beam = b.take(8 * 8 * 4 * 2 + 8 * 4);
  p.err = b.take(64);
  p.pos_tmp = b.take(Bm * 4);
  p.tok_in = b.take(Bm * 4);
  if (c.arch == WD_ARCH_QWEN3) p.rope = b.take((size_t)c.context * hd * f4);
  if (c.arch == WD_ARCH_QWEN3 && p.mfma) {
    p.pf_pos_chunk = pf_positions((int)Bm);
    const size_t R = ((size_t)Bm * p.pf_pos_chunk + 127) / 128 * 128, nqkv = (hq + 2 * hkv) * hd;
    p.pf_rows = (int)R;
    p.pf_x = b.take(R * d * f4);
    p.pf_pos = b.take(R * 4);
    p.pf_ah = b.take(R * std::max(d, hq * hd) * wb); p.pf_al = b.take(R * std::max(d, hq * hd) * wb);
    p.pf_hh = b.take(R * ff * wb); p.pf_hl = b.take(R * ff * wb);
    p.pf_qkv = b.take(R * nqkv * f4);
    p.pf_q = b.take(R * hq * hd * f4);
  }
  p.ov_in = b.take(Bm * d * wb);
  p.total = (b.off + 255) & ~size_t(255);
  return p;
}

// Audio encoder (optional, Whisper): weights and buffers in a second caller-owned workspace.
struct EncLayer { size_t ln1g, ln1b, wqkv, bq, bv, wo, bo, ln2g, ln2b, w1, b1, w2, b2; };
struct EncPlan {
  int mels = 0, frames = 0, P = 0, layers = 0, dff = 0, max_sets = 0, kp1 = 0;
  size_t conv1w = 0, conv1b = 0, conv2w = 0, conv2b = 0, pos = 0, lnpg = 0, lnpb = 0;
  std::vector<EncLayer> L;
  // buffers: rows of the stem's first convolution (sets x frames) and of the layers (sets x P),
  // both rounded up to the GEMM's 128-row tiles
  size_t x1 = 0, x = 0, ah = 0, al = 0, hh = 0, hl = 0, qkv = 0, q = 0, K = 0, V = 0;
  size_t states = 0;         // encoder states [max_sets, P, d] in w_dtype (wd_listen)
  size_t total = 0;
};

EncPlan make_enc_plan(const wd_config& c, int mels, int frames, int layers, int dff, int max_sets) {
  EncPlan p;
  Bump b;
  const size_t d = c.d_model, wb = dtype_bytes(c.w_dtype), f4 = 4;
  p.mels = mels; p.frames = frames; p.layers = layers; p.dff = dff; p.max_sets = max_sets;
  p.P = (frames - 1) / 2 + 1;
  p.kp1 = (3 * mels + 31) / 32 * 32;
  p.conv1w = b.take(d * p.kp1 * wb); p.conv1b = b.take(d * f4);
  p.conv2w = b.take(d * 3 * d * wb); p.conv2b = b.take(d * f4);
  p.pos = b.take((size_t)p.P * d * f4);
  p.lnpg = b.take(d * f4); p.lnpb = b.take(d * f4);
  for (int l = 0; l < layers; ++l) {
    EncLayer e{};
    e.ln1g = b.take(d * f4); e.ln1b = b.take(d * f4); e.ln2g = b.take(d * f4); e.ln2b = b.take(d * f4);
    e.wqkv = b.take(3 * d * d * wb); e.bq = b.take(d * f4); e.bv = b.take(d * f4);
    e.wo = b.take(d * d * wb); e.bo = b.take(d * f4);
    e.w1 = b.take((size_t)dff * d * wb); e.b1 = b.take((size_t)dff * f4);
    e.w2 = b.take(d * dff * wb); e.b2 = b.take(d * f4);
    p.L.push_back(e);
  }
  const size_t r1 = ((size_t)max_sets * frames + 127) / 128 * 128, r = ((size_t)max_sets * p.P + 127) / 128 * 128;
  const size_t ka = std::max({(size_t)p.kp1 * r1, 3 * d * r, d * r});   // widest split A operand
  p.x1 = b.take(r1 * d * f4);
  p.x = b.take(r * d * f4);
  p.ah = b.take(ka * wb); p.al = b.take(ka * wb);
  p.hh = b.take(r * dff * wb); p.hl = b.take(r * dff * wb);
  p.qkv = b.take(r * d * f4);   // the final norm's fp32 output (q, K and V come from the GEMM's epilogue)
  p.q = b.take(r * d * f4);
  p.K = b.take((size_t)max_sets * p.P * d * wb); p.V = b.take((size_t)max_sets * p.P * d * wb);
  p.states = b.take((size_t)max_sets * p.P * d * wb);
  p.total = (b.off + 255) & ~size_t(255);
  return p;
}

std::string check_enc(const wd_config& c, int mels, int frames, int layers, int dff, int max_sets) {
  if (c.arch != WD_ARCH_WHISPER) return "the audio encoder belongs to a whisper context";
  if (c.w_dtype == DT_F32) return "the audio encoder runs with 16-bit weights";
  if (mels < 1 || frames < 1 || layers < 1 || max_sets < 1) return "n_mels, frames, n_layers, max_sets must be positive";
  if (dff <= 0 || dff % 128) return "the encoder d_ff must be a positive multiple of 128";
  if (c.d_model % 128) return "d_model must be a multiple of 128";
  if ((frames - 1) / 2 + 1 > c.max_frames) return "(frames - 1) / 2 + 1 exceeds max_frames";
  return "";
}

struct ProfPair { hipEvent_t a, b; int n; };

// A captured step: every launch of one wd_step call, replayed with hipGraphLaunch
// while the call's device pointers, row count, current self cache and frame count
// stay the same (the positions and tokens are read from device memory at run time).
struct GraphKey {
  void* logits; void* argmax; int B, cur, frames, kind;   // kind: 0 step, 1 prefill row, 2 prefill row with override
  bool ragged;                                              // per-set frame counts (wd_cross_kv_ragged)
  bool operator==(const GraphKey& o) const {
    return logits == o.logits && argmax == o.argmax && B == o.B && cur == o.cur && frames == o.frames &&
           kind == o.kind && ragged == o.ragged;
  }
};
struct GraphEntry { GraphKey key; hipGraphExec_t exec; };

}  // namespace

struct wd_ctx {
  wd_config cfg{};
  Plan plan;
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  int cur = 0;               // current self-cache buffer
  bool cross_ready = false;
  int frames = 0;            // frames of the current window (the longest set when ragged)
  bool ragged = false;       // per-set frame counts in plan.frames_dev
  std::vector<int32_t> frames_host;   // staging of the last ragged window's counts
  EncPlan* enc = nullptr;    // the audio encoder, once wd_load_encoder ran
  char* enc_ws = nullptr;
  std::string err;
  // captured steps (small cache, least recently used evicted first); off with
  // wd_set_option(WD_OPT_GRAPHS, 0), while profiling, or on the legacy null stream
  bool use_graphs = true;
  std::vector<GraphEntry> graphs;
  // measurement
  int prof_kernel = -1, prof_layer = -1, prof_repeats = 1;
  std::vector<ProfPair> prof;
  size_t prof_used = 0;

  template <typename T = void>
  T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  void* self_k(int l) const { return ws + plan.self[cur] + (size_t)l * 2 * plan.self_slab; }
  void* self_v(int l) const { return ws + plan.self[cur] + (size_t)l * 2 * plan.self_slab + plan.self_slab; }
  void* cross_k(int l) const { return ws + plan.cross + (size_t)l * 2 * plan.cross_slab; }
  void* cross_v(int l) const { return ws + plan.cross + (size_t)l * 2 * plan.cross_slab + plan.cross_slab; }
};

namespace {

wd_status fail(wd_ctx* ctx, wd_status st, const std::string& msg) {
  if (ctx) ctx->err = msg;
  else g_load_error = msg;
  return st;
}

#define HIPCHK(ctx, expr, what)                                                        \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(ctx, WD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e_)); \
  } while (0)

// kernel classes for measurement
enum { PK_CROSS_ATTN = 0, PK_SELF_ATTN = 1, PK_LOGITS = 2, PK_XKV_GEMM = 3, PK_FC1 = 4 };

bool prof_on(wd_ctx* c, int kind, int layer) {
  return c->prof_kernel == kind && (c->prof_layer < 0 || c->prof_layer == layer) &&
         c->prof_used < c->prof.size();
}
void prof_begin(wd_ctx* c, bool on) {
  if (on) (void)hipEventRecord(c->prof[c->prof_used].a, c->stream);
}
void prof_end(wd_ctx* c, bool on) {
  if (on) {
    (void)hipEventRecord(c->prof[c->prof_used].b, c->stream);
    c->prof[c->prof_used].n = c->prof_repeats;
    ++c->prof_used;
  }
}

// Rows of one step share encoder sets in groups of q_per_kvb rows.
int rows_per_set(const wd_config& c, int B) {
  if (c.n_enc == 1) return B;
  return c.max_batch / c.n_enc;
}

// The step's layers and head for 16-bit weights: every projection on the MFMA skinny
// GEMM, activations handed between kernels in the split fragment layout.
wd_status run_layers_mfma(wd_ctx* c, const int32_t* pos, int B, float* logits, int32_t* argmax, bool head) {
  const wd_config& g = c->cfg;
  const Plan& P = c->plan;
  hipStream_t s = c->stream;
  const int d = g.d_model, hd = g.head_dim, hq = g.n_heads, hkv = g.n_kv_heads, ff = g.d_ff;
  const bool whisper = g.arch == WD_ARCH_WHISPER;
  const int adt = g.w_dtype;  // activation split dtype = weight dtype
  float* x = c->at<float>(P.x);
  float* q = c->at<float>(P.q);
  float* qkv = c->at<float>(P.qkv);
  float* part = c->at<float>(P.part);
  unsigned* err = c->at<unsigned>(P.err);
  void *yh = c->at(P.yh), *yl = c->at(P.yl), *oh = c->at(P.oh), *ol = c->at(P.ol);
  void *hh = c->at(P.hh), *hl = c->at(P.hl);
  const int64_t kv_bstride = (int64_t)hkv * g.context * hd;
  const float qscale = 1.0f / sqrtf((float)hd);

  int s_rows, s_splits, s_nw;
  split_for(g.context, B * hkv, hq / hkv, &s_rows, &s_splits, &s_nw);
  const int qpk = whisper ? rows_per_set(g, B) : 1;
  int c_rows = 0, c_splits = 1, c_nw = 4;
  if (whisper) split_for(c->frames, (B / qpk) * hkv, qpk, &c_rows, &c_splits, &c_nw, true);

  float* gpart = P.gpart_cap ? c->at<float>(P.gpart) : nullptr;
  auto proj = [&](const void* W, int N, int K, const void* Yh, const void* Yl, int epi, const float* bias,
                  float* out, int ldo, float scale) {
    wd::MGemvParams m{};
    m.W = W; m.w_dtype = g.w_dtype; m.N = N; m.K = K; m.Yhi = Yh; m.Ylo = Yl; m.B = B; m.epi = epi;
    m.bias = bias; m.out = out; m.ldo = ldo; m.scale = scale; m.err = err;
    m.yo_hi = hh; m.yo_lo = hl;
    m.part = gpart; m.part_cap = P.gpart_cap;
    return m;
  };
  // A split-K residual projection leaves its partials (and bias) to the next norm, which
  // adds them into x; any other split-K epilogue runs in the finish kernel right away.
  const float* pend_bias = nullptr;
  int pend_G = 0;
  // With sums_in_consumer the caller's next kernel reads the partials itself (the attention
  // prologue, the Qwen3 q/k norm + RoPE); *Gout receives G.
  auto gemm = [&](const wd::MGemvParams& m, const char* what, int* Gout = nullptr, int gmax = 16) -> wd_status {
    HIPCHK(c, wd::launch_mgemv(m, s), what);
    const int G = wd::mgemv_groups(m.N, m.K, m.B, m.epi);
    if (Gout) *Gout = G <= gmax ? G : 1;
    if (G > 1) {
      if (m.epi == wd::EPI_RESID) {
        pend_bias = m.bias;
        pend_G = G;
      } else if (!Gout || G > gmax) {
        HIPCHK(c, wd::launch_mgemv_finish(m, G, s), what);
      }
    }
    return WD_OK;
  };
  auto norm = [&](void* oh_, void* ol_, const float* gain, const float* bias, const char* what) -> wd_status {
    HIPCHK(c, wd::launch_norm_split(x, oh_, ol_, adt, gain, bias, B, d, g.norm_eps, s, pend_G ? gpart : nullptr,
                                    pend_G, pend_bias), what);
    pend_G = 0;
    pend_bias = nullptr;
    return WD_OK;
  };
#define WDCHK(expr) do { const wd_status st_ = (expr); if (st_ != WD_OK) return st_; } while (0)

  for (int l = 0; l < g.n_layers; ++l) {
    const LayerOff& L = P.L[l];
    wd::AttnParams ap{};
    ap.cache_dtype = g.cache_dtype; ap.B = B; ap.Hq = hq; ap.Hkv = hkv; ap.hd = hd; ap.part = part;
    ap.o_hi = oh; ap.o_lo = ol; ap.o_dtype = adt;
    if (whisper) {
      WDCHK(norm(yh, yl, c->at<float>(L.ln1g), c->at<float>(L.ln1b), "ln1"));
      wd::MGemvParams m = proj(c->at(L.wqkv), 3 * d, d, yh, yl, wd::EPI_QKV, c->at<float>(L.bqkv), q, d, qscale);
      m.d = d; m.H = hq; m.hd = hd; m.ctx = g.context; m.pos = pos;
      m.Kc = c->self_k(l); m.Vc = c->self_v(l); m.cache_dtype = g.cache_dtype; m.kv_bstride = kv_bstride;
      int G = 1;
      WDCHK(gemm(m, "qkv projection", &G));
      if (G > 1) {   // the self-attention sums q and the appended k, v from the partials
        ap.qpart = gpart; ap.qG = G; ap.qpart_ld = 3 * d; ap.q_off = 0; ap.qbias = m.bias; ap.qscale = qscale;
        ap.append = true; ap.k_off = d; ap.v_off = 2 * d; ap.vbias = m.bias + 2 * d;
      }
    } else {
      WDCHK(norm(yh, yl, c->at<float>(L.n1g), nullptr, "norm1"));
      const int nqkv = (hq + 2 * hkv) * hd;
      int G = 1;
      WDCHK(gemm(proj(c->at(L.wqkv), nqkv, d, yh, yl, wd::EPI_STORE, nullptr, qkv, nqkv, 1.0f), "qkv projection", &G, 32));
      if (G <= 16) {   // the attention prologue takes q/k norm, RoPE and the K/V append
        ap.qpart = G > 1 ? gpart : qkv; ap.qG = G; ap.qpart_ld = nqkv; ap.q_off = 0; ap.qbias = nullptr;
        ap.qscale = qscale; ap.append = true; ap.k_off = hq * hd; ap.v_off = (hq + hkv) * hd; ap.vbias = nullptr;
        ap.rope = true; ap.qn = c->at<float>(L.qn); ap.kn = c->at<float>(L.kn); ap.eps = g.norm_eps;
        ap.rope_cs = c->at<float>(P.rope);
      } else {
        HIPCHK(c, wd::launch_qk_rope_append(qkv, B, hq, hkv, hd, pos, g.context, c->at<float>(L.qn),
                                            c->at<float>(L.kn), g.norm_eps, c->at<float>(P.rope), qscale, q,
                                            c->self_k(l), c->self_v(l), g.cache_dtype, kv_bstride, s, gpart, G),
               "qk norm/rope/append");
      }
    }
    ap.q = q; ap.q_ld = hq * hd; ap.K = c->self_k(l); ap.V = c->self_v(l);
    ap.kvb_stride = kv_bstride; ap.rows_cap = g.context; ap.pos = pos; ap.n_rows_fixed = 0;
    ap.q_per_kvb = 1; ap.split_rows = s_rows; ap.n_splits = s_splits; ap.nw = s_nw; ap.out = nullptr; ap.out_ld = 0;
    {
      const bool on = prof_on(c, PK_SELF_ATTN, l);
      prof_begin(c, on);
      for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
        HIPCHK(c, wd::launch_attention(ap, s), "self attention");
      prof_end(c, on);
    }
    HIPCHK(c, wd::launch_attention_combine(ap, s), "self attention combine");
    WDCHK(gemm(proj(c->at(L.wo), d, hq * hd, oh, ol, wd::EPI_RESID, whisper ? c->at<float>(L.bo) : nullptr, x, d, 1.0f),
               "out projection"));
    if (whisper) {
      WDCHK(norm(yh, yl, c->at<float>(L.ln2g), c->at<float>(L.ln2b), "ln2"));
      int Gq = 1;
      WDCHK(gemm(proj(c->at(L.wcq), d, d, yh, yl, wd::EPI_STORE, c->at<float>(L.bcq), q, d, qscale), "cross q projection",
                 &Gq));
      wd::AttnParams cp = ap;
      cp.append = false; cp.qpart = nullptr;
      if (Gq > 1) {   // the cross-attention sums q from the partials
        cp.qpart = gpart; cp.qG = Gq; cp.qpart_ld = d; cp.q_off = 0; cp.qbias = c->at<float>(L.bcq); cp.qscale = qscale;
      }
      cp.K = c->cross_k(l); cp.V = c->cross_v(l);
      cp.kvb_stride = (int64_t)hq * g.max_frames * hd; cp.rows_cap = g.max_frames;
      cp.pos = nullptr; cp.n_rows_fixed = c->frames; cp.q_per_kvb = qpk;
      cp.rows_kvb = c->ragged ? c->at<int32_t>(P.frames_dev) : nullptr;
      cp.split_rows = c_rows; cp.n_splits = c_splits; cp.nw = c_nw;
      {
        const bool on = prof_on(c, PK_CROSS_ATTN, l);
        prof_begin(c, on);
        for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
          HIPCHK(c, wd::launch_attention(cp, s), "cross attention");
        prof_end(c, on);
      }
      HIPCHK(c, wd::launch_attention_combine(cp, s), "cross attention combine");
      WDCHK(gemm(proj(c->at(L.wco), d, d, oh, ol, wd::EPI_RESID, c->at<float>(L.bco), x, d, 1.0f), "cross out projection"));
      WDCHK(norm(yh, yl, c->at<float>(L.ln3g), c->at<float>(L.ln3b), "ln3"));
      {
        const bool on = prof_on(c, PK_FC1, l);
        prof_begin(c, on);
        for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
          WDCHK(gemm(proj(c->at(L.w1), ff, d, yh, yl, wd::EPI_GELU_SPLIT, c->at<float>(L.b1), nullptr, 0, 1.0f), "fc1"));
        prof_end(c, on);
      }
      WDCHK(gemm(proj(c->at(L.w2), d, ff, hh, hl, wd::EPI_RESID, c->at<float>(L.b2), x, d, 1.0f), "fc2"));
    } else {
      WDCHK(norm(yh, yl, c->at<float>(L.n2g), nullptr, "norm2"));
      {
        const bool on = prof_on(c, PK_FC1, l);
        prof_begin(c, on);
        for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
          WDCHK(gemm(proj(c->at(L.wgu), 2 * ff, d, yh, yl, wd::EPI_SWIGLU_SPLIT, nullptr, nullptr, 0, 1.0f),
                   "gate|up projection"));
        prof_end(c, on);
      }
      WDCHK(gemm(proj(c->at(L.wdn), d, ff, hh, hl, wd::EPI_RESID, nullptr, x, d, 1.0f), "down projection"));
    }
  }
  // without the head (prefill positions before the last) the pending residual still lands in x
  if (!head) {
    if (pend_G) WDCHK(norm(yh, yl, c->at<float>(P.lnfg), whisper ? c->at<float>(P.lnfb) : nullptr, "final residual"));
    return WD_OK;
  }
  WDCHK(norm(yh, yl, c->at<float>(P.lnfg), whisper ? c->at<float>(P.lnfb) : nullptr, "final norm"));
#undef WDCHK
  wd::MGemvParams hm = proj(c->at(P.embed), g.vocab, d, yh, yl, wd::EPI_LOGITS, nullptr, logits, g.vocab, 1.0f);
  hm.amax = c->at<unsigned long long>(P.amax); hm.ldp = g.max_batch;
  {
    const bool on = prof_on(c, PK_LOGITS, -1);
    prof_begin(c, on);
    for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
      HIPCHK(c, wd::launch_mgemv(hm, s), "logits");
    prof_end(c, on);
  }
  HIPCHK(c, wd::launch_argmax_final(hm.amax, wd::mgemv_blocks_k(g.vocab, d, B), g.max_batch, B, argmax, s), "argmax");
  return WD_OK;
}

// One decoder step over rows 0..B-1.  tok: ids (stride tok_stride) or null with ov;
// pos: device positions; ov: embedding override rows (stride ov_stride) or null.
wd_status run_step(wd_ctx* c, const int32_t* tok, int tok_stride, const int32_t* pos, const void* ov,
                   int64_t ov_stride, int B, float* logits, int32_t* argmax, bool head) {
  const wd_config& g = c->cfg;
  const Plan& P = c->plan;
  hipStream_t s = c->stream;
  const int d = g.d_model, hd = g.head_dim, hq = g.n_heads, hkv = g.n_kv_heads, ff = g.d_ff;
  const bool whisper = g.arch == WD_ARCH_WHISPER;
  float* x = c->at<float>(P.x);
  float* y = c->at<float>(P.y);
  float* q = c->at<float>(P.q);
  float* qkv = c->at<float>(P.qkv);
  float* o = c->at<float>(P.o);
  float* h = c->at<float>(P.h);
  float* part = c->at<float>(P.part);
  unsigned* err = c->at<unsigned>(P.err);
  const int64_t kv_bstride = (int64_t)hkv * g.context * hd;
  const float qscale = 1.0f / sqrtf((float)hd);

  HIPCHK(c, wd::launch_embed(x, c->at(P.embed), whisper ? c->at(P.pos) : nullptr, g.w_dtype, tok, tok_stride,
                             pos, ov, ov_stride, B, d, g.vocab, g.context, err, P.mfma, s), "embed");
  if (P.mfma) return run_layers_mfma(c, pos, B, logits, argmax, head);

  // self-attention split policy (positions live on the device, so split by context)
  int s_rows, s_splits, s_nw;
  split_for(g.context, B * hkv, hq / hkv, &s_rows, &s_splits, &s_nw);
  const int qpk = whisper ? rows_per_set(g, B) : 1;
  int c_rows = 0, c_splits = 1, c_nw = 4;
  if (whisper) split_for(c->frames, (B / qpk) * hkv, qpk, &c_rows, &c_splits, &c_nw, true);

  for (int l = 0; l < g.n_layers; ++l) {
    const LayerOff& L = P.L[l];
    wd::GemvParams gp{};
    gp.w_dtype = g.w_dtype;
    gp.B = B;
    gp.err = err;
    gp.scale = 1.0f;
    wd::AttnParams ap{};
    ap.cache_dtype = g.cache_dtype;
    ap.B = B;
    ap.Hq = hq;
    ap.Hkv = hkv;
    ap.hd = hd;
    ap.part = part;

    if (whisper) {
      HIPCHK(c, wd::launch_norm(x, y, c->at<float>(L.ln1g), c->at<float>(L.ln1b), B, d, g.norm_eps, s), "ln1");
      gp.W = c->at(L.wqkv); gp.N = 3 * d; gp.K = d; gp.Y = y; gp.ldy = d; gp.ymode = wd::Y_PLAIN;
      gp.epi = wd::EPI_QKV; gp.bias = c->at<float>(L.bqkv); gp.out = q; gp.ldo = d; gp.scale = qscale;
      gp.d = d; gp.H = hq; gp.hd = hd; gp.ctx = g.context; gp.pos = pos;
      gp.Kc = c->self_k(l); gp.Vc = c->self_v(l); gp.cache_dtype = g.cache_dtype; gp.kv_bstride = kv_bstride;
      HIPCHK(c, wd::launch_gemv(gp, s), "qkv projection");
    } else {
      HIPCHK(c, wd::launch_norm(x, y, c->at<float>(L.n1g), nullptr, B, d, g.norm_eps, s), "norm1");
      const int nqkv = (hq + 2 * hkv) * hd;
      gp.W = c->at(L.wqkv); gp.N = nqkv; gp.K = d; gp.Y = y; gp.ldy = d; gp.ymode = wd::Y_PLAIN;
      gp.epi = wd::EPI_STORE; gp.bias = nullptr; gp.out = qkv; gp.ldo = nqkv;
      HIPCHK(c, wd::launch_gemv(gp, s), "qkv projection");
      HIPCHK(c, wd::launch_qk_rope_append(qkv, B, hq, hkv, hd, pos, g.context, c->at<float>(L.qn),
                                          c->at<float>(L.kn), g.norm_eps, c->at<float>(P.rope), qscale, q,
                                          c->self_k(l), c->self_v(l), g.cache_dtype, kv_bstride, s),
             "qk norm/rope/append");
    }
    // self-attention over rows 0..pos of each row's own cache
    ap.q = q; ap.q_ld = hq * hd; ap.K = c->self_k(l); ap.V = c->self_v(l);
    ap.kvb_stride = kv_bstride; ap.rows_cap = g.context; ap.pos = pos; ap.n_rows_fixed = 0;
    ap.q_per_kvb = 1; ap.split_rows = s_rows; ap.n_splits = s_splits; ap.nw = s_nw; ap.out = o; ap.out_ld = hq * hd;
    {
      const bool on = prof_on(c, PK_SELF_ATTN, l);
      prof_begin(c, on);
      for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
        HIPCHK(c, wd::launch_attention(ap, s), "self attention");
      prof_end(c, on);
    }
    HIPCHK(c, wd::launch_attention_combine(ap, s), "self attention combine");
    // output projection + residual
    gp.W = c->at(L.wo); gp.N = d; gp.K = hq * hd; gp.Y = o; gp.ldy = hq * hd; gp.ymode = wd::Y_PLAIN;
    gp.epi = wd::EPI_RESID; gp.bias = whisper ? c->at<float>(L.bo) : nullptr; gp.out = x; gp.ldo = d;
    HIPCHK(c, wd::launch_gemv(gp, s), "out projection");

    if (whisper) {
      // cross-attention: LN2, cross q, attend over all frames of the row's encoder set
      HIPCHK(c, wd::launch_norm(x, y, c->at<float>(L.ln2g), c->at<float>(L.ln2b), B, d, g.norm_eps, s), "ln2");
      gp.W = c->at(L.wcq); gp.N = d; gp.K = d; gp.Y = y; gp.ldy = d; gp.epi = wd::EPI_STORE;
      gp.bias = c->at<float>(L.bcq); gp.out = q; gp.ldo = d; gp.scale = qscale;
      HIPCHK(c, wd::launch_gemv(gp, s), "cross q projection");
      gp.scale = 1.0f;
      wd::AttnParams cp = ap;
      cp.K = c->cross_k(l); cp.V = c->cross_v(l);
      cp.kvb_stride = (int64_t)hq * g.max_frames * hd; cp.rows_cap = g.max_frames;
      cp.pos = nullptr; cp.n_rows_fixed = c->frames; cp.q_per_kvb = qpk;
      cp.rows_kvb = c->ragged ? c->at<int32_t>(P.frames_dev) : nullptr;
      cp.split_rows = c_rows; cp.n_splits = c_splits; cp.nw = c_nw;
      {
        const bool on = prof_on(c, PK_CROSS_ATTN, l);
        prof_begin(c, on);
        for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
          HIPCHK(c, wd::launch_attention(cp, s), "cross attention");
        prof_end(c, on);
      }
      HIPCHK(c, wd::launch_attention_combine(cp, s), "cross attention combine");
      gp.W = c->at(L.wco); gp.N = d; gp.K = d; gp.Y = o; gp.ldy = d; gp.epi = wd::EPI_RESID;
      gp.bias = c->at<float>(L.bco); gp.out = x; gp.ldo = d;
      HIPCHK(c, wd::launch_gemv(gp, s), "cross out projection");
      // FFN
      HIPCHK(c, wd::launch_norm(x, y, c->at<float>(L.ln3g), c->at<float>(L.ln3b), B, d, g.norm_eps, s), "ln3");
      gp.W = c->at(L.w1); gp.N = ff; gp.K = d; gp.Y = y; gp.ldy = d; gp.epi = wd::EPI_GELU;
      gp.bias = c->at<float>(L.b1); gp.out = h; gp.ldo = ff;
      {
        const bool on = prof_on(c, PK_FC1, l);
        prof_begin(c, on);
        for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
          HIPCHK(c, wd::launch_gemv(gp, s), "fc1");
        prof_end(c, on);
      }
      gp.W = c->at(L.w2); gp.N = d; gp.K = ff; gp.Y = h; gp.ldy = ff; gp.epi = wd::EPI_RESID;
      gp.bias = c->at<float>(L.b2); gp.out = x; gp.ldo = d;
      HIPCHK(c, wd::launch_gemv(gp, s), "fc2");
    } else {
      HIPCHK(c, wd::launch_norm(x, y, c->at<float>(L.n2g), nullptr, B, d, g.norm_eps, s), "norm2");
      gp.W = c->at(L.wgu); gp.N = 2 * ff; gp.K = d; gp.Y = y; gp.ldy = d; gp.epi = wd::EPI_STORE;
      gp.bias = nullptr; gp.out = h; gp.ldo = 2 * ff;
      {
        const bool on = prof_on(c, PK_FC1, l);
        prof_begin(c, on);
        for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
          HIPCHK(c, wd::launch_gemv(gp, s), "gate|up projection");
        prof_end(c, on);
      }
      gp.W = c->at(L.wdn); gp.N = d; gp.K = ff; gp.Y = h; gp.ldy = 2 * ff; gp.ymode = wd::Y_SWIGLU;
      gp.epi = wd::EPI_RESID; gp.out = x; gp.ldo = d;
      HIPCHK(c, wd::launch_gemv(gp, s), "down projection");
    }
  }
  if (!head) return WD_OK;
  // final norm, tied-embedding logits, argmax
  HIPCHK(c, wd::launch_norm(x, y, c->at<float>(P.lnfg), whisper ? c->at<float>(P.lnfb) : nullptr, B, d,
                            g.norm_eps, s), "final norm");
  wd::GemvParams hp{};
  hp.W = c->at(P.embed); hp.w_dtype = g.w_dtype; hp.N = g.vocab; hp.K = d; hp.Y = y; hp.ldy = d; hp.B = B;
  hp.ymode = wd::Y_PLAIN; hp.epi = wd::EPI_LOGITS; hp.out = logits; hp.ldo = g.vocab; hp.scale = 1.0f;
  hp.amax = c->at<unsigned long long>(P.amax); hp.ldp = g.max_batch; hp.err = err;
  {
    const bool on = prof_on(c, PK_LOGITS, -1);
    prof_begin(c, on);
    for (int r_ = 0; r_ < (on ? c->prof_repeats : 1); ++r_)
      HIPCHK(c, wd::launch_gemv(hp, s), "logits");
    prof_end(c, on);
  }
  HIPCHK(c, wd::launch_argmax_final(hp.amax, wd::gemv_blocks(g.vocab, B), g.max_batch, B, argmax, s), "argmax");
  return WD_OK;
}

struct Need {
  std::string name;
  int64_t numel;
  bool matrix;
};

std::vector<Need> required(const wd_config& c) {
  std::vector<Need> n;
  const int64_t d = c.d_model, ff = c.d_ff, hd = c.head_dim, hq = c.n_heads, hkv = c.n_kv_heads;
  n.push_back({"embed", (int64_t)c.vocab * d, true});
  if (c.arch == WD_ARCH_WHISPER) {
    n.push_back({"pos", (int64_t)c.context * d, true});
    n.push_back({"ln_f.g", d, false});
    n.push_back({"ln_f.b", d, false});
    for (int i = 0; i < c.n_layers; ++i) {
      const std::string p = "dec." + std::to_string(i) + ".";
      for (const char* ln : {"ln1", "ln2", "ln3"}) {
        n.push_back({p + ln + ".g", d, false});
        n.push_back({p + ln + ".b", d, false});
      }
      for (const char* a : {"self", "cross"}) {
        for (const char* m : {"q", "k", "v", "o"}) n.push_back({p + a + "." + m + ".w", d * d, true});
        for (const char* m : {"q", "v", "o"}) n.push_back({p + a + "." + m + ".b", d, false});
      }
      n.push_back({p + "fc1.w", ff * d, true});
      n.push_back({p + "fc1.b", ff, false});
      n.push_back({p + "fc2.w", d * ff, true});
      n.push_back({p + "fc2.b", d, false});
    }
  } else {
    n.push_back({"norm_f.g", d, false});
    for (int i = 0; i < c.n_layers; ++i) {
      const std::string p = "dec." + std::to_string(i) + ".";
      n.push_back({p + "norm1.g", d, false});
      n.push_back({p + "norm2.g", d, false});
      n.push_back({p + "q_norm.g", hd, false});
      n.push_back({p + "k_norm.g", hd, false});
      n.push_back({p + "self.q.w", hq * hd * d, true});
      n.push_back({p + "self.k.w", hkv * hd * d, true});
      n.push_back({p + "self.v.w", hkv * hd * d, true});
      n.push_back({p + "self.o.w", d * hq * hd, true});
      n.push_back({p + "mlp.gate.w", ff * d, true});
      n.push_back({p + "mlp.up.w", ff * d, true});
      n.push_back({p + "mlp.down.w", d * ff, true});
    }
  }
  return n;
}

}  // namespace

// ---- device scratch of wd_topk_noalloc ----------------------------------------------------------
// The per-part candidate lists of up to WD_TOPK_NOALLOC_MAX_ROWS rows (at most 32 parts per row,
// each W <= 8 (value, id) pairs and a (max, sum) pair): a file-scope device array, so the entry
// point needs no workspace and allocates nothing.  Each GPU holds its own copy until the
// process ends; its device address is looked up once per device, with that device current.
// The array has external linkage: the runtime resolves a registered device variable by its
// symbol name in the code object, and an internal-linkage (static) one stays a local symbol
// that lookup cannot find.
constexpr size_t kTopkScratchBytes = (size_t)WD_TOPK_NOALLOC_MAX_ROWS * 32 * (8 * 8 + 8);
__device__ __align__(256) unsigned char scratch[kTopkScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The current device's address of `scratch` (the host-side symbol is only a stand-in).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}
}  // namespace

// ---- machine floors (measurement support) -------------------------------------------------------
namespace {
constexpr int kProbeEmptyBlocks = 1280;   // the large-v3 step's attention grids
constexpr int kProbeStreamBlocks = 1280;  // slabs, as the cross-attention's (encoder set, head) blocks
__global__ __launch_bounds__(256) void k_probe_empty() {}
// Block i reads the i-th of gridDim.x equal slabs of a and of b (the cross-attention's K and V
// slab of one block), eight waves, six 16-byte nontemporal lane loads of each array in flight per
// lane; the words' xor reaches memory only in the (practically never taken) case it equals a
// fixed constant, so no load is dropped.
__global__ __launch_bounds__(512) void k_probe_stream(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                      int64_t n16, float* __restrict__ sink) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  constexpr int UNR = 6;
  const int64_t slab = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * slab, hi = min(lo + slab, n16);
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 512 * UNR) {
    u4 va[UNR], vb[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t j = min(i + u * 512, hi - 1);
      va[u] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(a) + j);
      vb[u] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(b) + j);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc ^= va[u].x ^ va[u].y ^ va[u].z ^ va[u].w ^ vb[u].x ^ vb[u].y ^ vb[u].z ^ vb[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = 1.f;
}
constexpr int kProbeHandoffBlocks = 256;
// One hand-off between dependent kernels: block i reads the slab that block (i + shift) % grid
// wrote in the previous launch (shift 0: the same block index, so the same XCD, as blocks reach
// the XCDs round-robin by launch index; shift 1: the next XCD's) and writes its own slab.
__global__ __launch_bounds__(256) void k_probe_handoff(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                       int slab16, int shift) {
  const int from = (blockIdx.x + shift) % gridDim.x;
  for (int i = threadIdx.x; i < slab16; i += 256) {
    uint4 v = src[(int64_t)from * slab16 + i];
    v.x ^= 1u;
    dst[(int64_t)blockIdx.x * slab16 + i] = v;
  }
}
// A cross-workgroup reduction inside one kernel: every block publishes one value, makes it
// visible device-wide with a fence and counts itself in; the block that counts last adds the
// values (nobody waits) and re-arms the counter for the next launch.
__global__ __launch_bounds__(256) void k_probe_fence(float* __restrict__ part, unsigned* __restrict__ ctr) {
  __shared__ bool last;
  if (threadIdx.x == 0) {
    part[blockIdx.x] = (float)blockIdx.x;
    __threadfence();
    last = atomicAdd(ctr, 1u) == gridDim.x - 1;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  __shared__ float red[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < (int)gridDim.x; i += 256) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 256; ++i) s += red[i];
    reinterpret_cast<float*>(ctr)[1] = s;
    ctr[0] = 0u;
  }
}
}  // namespace

extern "C" {

int32_t wd_abi_version(void) { return WD_ABI_VERSION; }

size_t wd_workspace_bytes(const wd_config* cfg) {
  if (!cfg || !check_config(*cfg).empty()) return 0;
  return make_plan(*cfg).total;
}

wd_status wd_load(const wd_config* cfg, const wd_tensor* weights, int32_t n_weights, void* workspace,
                  size_t ws_bytes, void* stream, wd_ctx** out) {
  try {
    if (!cfg || !out) return fail(nullptr, WD_ERR_ARG, "wd_load: cfg and out must not be null");
    *out = nullptr;
    const std::string why = check_config(*cfg);
    if (!why.empty()) return fail(nullptr, WD_ERR_ARG, "wd_load: " + why);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
      return fail(nullptr, WD_ERR_ARG, "wd_load: workspace must be a 256-byte aligned device pointer");
    if (n_weights < 0 || (n_weights > 0 && !weights)) return fail(nullptr, WD_ERR_ARG, "wd_load: bad weight list");
    const Plan plan = make_plan(*cfg);
    if (ws_bytes < plan.total)
      return fail(nullptr, WD_ERR_OOM, "wd_load: workspace of " + std::to_string(ws_bytes) + " bytes, need " +
                                           std::to_string(plan.total));
    // name -> tensor, with shape and dtype checks
    std::map<std::string, const wd_tensor*> byname;
    for (int i = 0; i < n_weights; ++i) {
      const wd_tensor& t = weights[i];
      if (!t.name) return fail(nullptr, WD_ERR_ARG, "wd_load: tensor with null name");
      const std::string nm(t.name);
      if (nm.size() >= 4 && nm.compare(nm.size() - 4, 4, ".k.b") == 0)
        return fail(nullptr, WD_ERR_ARG, "wd_load: '" + nm + "': the key projections carry no bias");
      if (byname.count(nm)) return fail(nullptr, WD_ERR_ARG, "wd_load: duplicate tensor '" + nm + "'");
      byname[nm] = &t;
    }
    const auto need = required(*cfg);
    if (byname.size() != need.size()) {
      for (const auto& kv : byname) {
        bool known = false;
        for (const auto& n : need) known = known || n.name == kv.first;
        if (!known) return fail(nullptr, WD_ERR_ARG, "wd_load: unknown tensor '" + kv.first + "'");
      }
    }
    for (const auto& n : need) {
      auto it = byname.find(n.name);
      if (it == byname.end()) return fail(nullptr, WD_ERR_ARG, "wd_load: missing tensor '" + n.name + "'");
      const wd_tensor& t = *it->second;
      if (!t.data) return fail(nullptr, WD_ERR_ARG, "wd_load: '" + n.name + "' has a null data pointer");
      if (t.numel != n.numel)
        return fail(nullptr, WD_ERR_ARG, "wd_load: '" + n.name + "' has " + std::to_string(t.numel) +
                                             " elements, expected " + std::to_string(n.numel));
      if (!valid_dt(t.dtype)) return fail(nullptr, WD_ERR_ARG, "wd_load: '" + n.name + "' has an unknown dtype");
      if (n.matrix && t.dtype != cfg->w_dtype)
        return fail(nullptr, WD_ERR_ARG, "wd_load: matrix '" + n.name + "' must be in w_dtype");
    }

    wd_ctx* c = new (std::nothrow) wd_ctx();
    if (!c) return fail(nullptr, WD_ERR_INTERNAL, "wd_load: out of host memory");
    c->cfg = *cfg;
    c->plan = plan;
    c->stream = reinterpret_cast<hipStream_t>(stream);
    c->ws = reinterpret_cast<char*>(workspace);
    hipStream_t s = c->stream;
    const int wdt = cfg->w_dtype;
    auto T = [&](const std::string& nm) { return byname[nm]; };
    auto cp = [&](const std::string& nm, size_t dst, int dst_dt, int64_t rows, int64_t cols, int64_t add) {
      const wd_tensor* t = T(nm);
      return wd::launch_copy_rows(t->data, t->dtype, c->ws + dst, dst_dt, rows, cols, 1, add, s);
    };
    auto vcopy = [&](const std::string& nm, size_t dst_byte, int64_t n) {
      const wd_tensor* t = T(nm);
      return wd::launch_copy_rows(t->data, t->dtype, c->ws + dst_byte, DT_F32, 1, n, 1, 0, s);
    };
    auto zero = [&](size_t dst_byte, int64_t nwords) {
      return wd::launch_fill_u32(reinterpret_cast<uint32_t*>(c->ws + dst_byte), 0u, nwords, s);
    };
    const int64_t d = cfg->d_model, ff = cfg->d_ff, hd = cfg->head_dim, hq = cfg->n_heads, hkv = cfg->n_kv_heads;
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    // fragment-layout pack into fused row blocks (16-bit weights) or plain row copy (fp32)
    auto mat = [&](const std::string& nm, size_t dst, int64_t rows, int64_t K, int64_t blk_mul, int64_t blk_add,
                   int64_t row_add) {
      if (!plan.mfma) return cp(nm, dst, wdt, rows, K, row_add);
      const wd_tensor* t = T(nm);
      return wd::launch_pack_frag(t->data, t->dtype, c->ws + dst, wdt, rows, K, blk_mul, blk_add, s);
    };
    if (plan.mfma) chk(zero(plan.embed, ((int64_t)(cfg->vocab + 15) / 16 * 16) * d * dtype_bytes(wdt) / 4));
    chk(mat("embed", plan.embed, cfg->vocab, d, 1, 0, 0));
    if (plan.mfma) {
      const int64_t Bp = row_pad(cfg->max_batch);
      for (size_t off : {plan.yh, plan.yl}) chk(zero(off, Bp * std::max(d, hq * hd) * dtype_bytes(wdt) / 4));
      for (size_t off : {plan.oh, plan.ol}) chk(zero(off, Bp * hq * hd * dtype_bytes(wdt) / 4));
      for (size_t off : {plan.hh, plan.hl}) chk(zero(off, Bp * ff * dtype_bytes(wdt) / 4));
    }
    if (cfg->arch == WD_ARCH_WHISPER) {
      chk(cp("pos", plan.pos, wdt, cfg->context, d, 0));
      chk(vcopy("ln_f.g", plan.lnfg, d));
      chk(vcopy("ln_f.b", plan.lnfb, d));
      for (int i = 0; i < cfg->n_layers && e == hipSuccess; ++i) {
        const std::string p = "dec." + std::to_string(i) + ".";
        const LayerOff& L = plan.L[i];
        chk(mat(p + "self.q.w", L.wqkv, d, d, 1, 0, 0));
        chk(mat(p + "self.k.w", L.wqkv, d, d, 1, d / 16, d));
        chk(mat(p + "self.v.w", L.wqkv, d, d, 1, 2 * d / 16, 2 * d));
        chk(mat(p + "self.o.w", L.wo, d, d, 1, 0, 0));
        chk(mat(p + "cross.q.w", L.wcq, d, d, 1, 0, 0));
        chk(mat(p + "cross.k.w", L.wckv, d, d, 1, 0, 0));       // fused [Wk; Wv] (fragment order for 16-bit)
        chk(mat(p + "cross.v.w", L.wckv, d, d, 1, d / 16, d));
        chk(mat(p + "cross.o.w", L.wco, d, d, 1, 0, 0));
        chk(mat(p + "fc1.w", L.w1, ff, d, 1, 0, 0));
        chk(mat(p + "fc2.w", L.w2, d, ff, 1, 0, 0));
        chk(vcopy(p + "self.q.b", L.bqkv, d));
        chk(zero(L.bqkv + d * 4, d));                 // keys: no bias
        chk(vcopy(p + "self.v.b", L.bqkv + 2 * d * 4, d));
        chk(vcopy(p + "self.o.b", L.bo, d));
        chk(vcopy(p + "cross.q.b", L.bcq, d));
        chk(zero(L.bckv, d));                         // fused cross bias [0 | b_v]
        chk(vcopy(p + "cross.v.b", L.bckv + d * 4, d));
        chk(vcopy(p + "cross.o.b", L.bco, d));
        chk(vcopy(p + "fc1.b", L.b1, ff));
        chk(vcopy(p + "fc2.b", L.b2, d));
        chk(vcopy(p + "ln1.g", L.ln1g, d)); chk(vcopy(p + "ln1.b", L.ln1b, d));
        chk(vcopy(p + "ln2.g", L.ln2g, d)); chk(vcopy(p + "ln2.b", L.ln2b, d));
        chk(vcopy(p + "ln3.g", L.ln3g, d)); chk(vcopy(p + "ln3.b", L.ln3b, d));
      }
    } else {
      chk(vcopy("norm_f.g", plan.lnfg, d));
      chk(wd::launch_rope_table(reinterpret_cast<float*>(c->ws + plan.rope), cfg->context, (int)hd, cfg->rope_base, s));
      for (int i = 0; i < cfg->n_layers && e == hipSuccess; ++i) {
        const std::string p = "dec." + std::to_string(i) + ".";
        const LayerOff& L = plan.L[i];
        chk(mat(p + "self.q.w", L.wqkv, hq * hd, d, 1, 0, 0));
        chk(mat(p + "self.k.w", L.wqkv, hkv * hd, d, 1, hq * hd / 16, hq * hd));
        chk(mat(p + "self.v.w", L.wqkv, hkv * hd, d, 1, (hq + hkv) * hd / 16, (hq + hkv) * hd));
        chk(mat(p + "self.o.w", L.wo, d, hq * hd, 1, 0, 0));
        // gate and up: contiguous halves (fp32 path) or alternating 16-row blocks (MFMA path)
        chk(mat(p + "mlp.gate.w", L.wgu, ff, d, 2, 0, 0));
        chk(mat(p + "mlp.up.w", L.wgu, ff, d, 2, 1, ff));
        chk(mat(p + "mlp.down.w", L.wdn, d, ff, 1, 0, 0));
        chk(vcopy(p + "norm1.g", L.n1g, d));
        chk(vcopy(p + "norm2.g", L.n2g, d));
        chk(vcopy(p + "q_norm.g", L.qn, hd));
        chk(vcopy(p + "k_norm.g", L.kn, hd));
      }
    }
    chk(zero(plan.err, 16));
    if (e != hipSuccess) {
      std::string m = std::string("wd_load: repack launch failed: ") + hipGetErrorString(e);
      delete c;
      return fail(nullptr, WD_ERR_HIP, m);
    }
    *out = c;
    return WD_OK;
  } catch (...) {
    return fail(nullptr, WD_ERR_INTERNAL, "wd_load: internal error");
  }
}

// Every layer's cross K/V from the encoder states [n_enc, frames, d] (one window).
wd_status cross_kv_impl(wd_ctx* ctx, const void* enc, int32_t frames, const char* who) {
  const wd_config& g = ctx->cfg;
  const void* X = enc;
  if (ctx->plan.mfma) {   // X feeds every layer: repack it into fragment order once
    HIPCHK(ctx, wd::launch_pack_rows(enc, g.w_dtype, ctx->at(ctx->plan.xfrag), (int64_t)g.n_enc * frames, g.d_model,
                                     ctx->stream), who);
    X = ctx->at(ctx->plan.xfrag);
  }
  for (int l = 0; l < g.n_layers; ++l) {
    const LayerOff& L = ctx->plan.L[l];
    const bool on = prof_on(ctx, PK_XKV_GEMM, l);
    prof_begin(ctx, on);
    HIPCHK(ctx, wd::launch_cross_kv_gemm(X, ctx->at(L.wckv), ctx->at<float>(L.bckv), g.w_dtype,
                                         g.n_enc * frames, g.d_model, frames, g.max_frames, g.n_heads,
                                         g.head_dim, ctx->cross_k(l), ctx->cross_v(l), g.cache_dtype,
                                         ctx->stream), who);
    prof_end(ctx, on);
  }
  ctx->cross_ready = true;
  ctx->frames = frames;
  return WD_OK;
}

wd_status wd_cross_kv(wd_ctx* ctx, const void* enc, int32_t frames) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    if (g.arch != WD_ARCH_WHISPER) return fail(ctx, WD_ERR_STATE, "wd_cross_kv: no cross-attention in this arch");
    if (!enc) return fail(ctx, WD_ERR_ARG, "wd_cross_kv: enc must not be null");
    if (frames < 1 || frames > g.max_frames) return fail(ctx, WD_ERR_ARG, "wd_cross_kv: frames outside [1, max_frames]");
    const wd_status st = cross_kv_impl(ctx, enc, frames, "cross K/V projection");
    if (st == WD_OK) ctx->ragged = false;
    return st;
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_cross_kv: internal error");
  }
}

wd_status wd_cross_kv_ragged(wd_ctx* ctx, const void* enc, const int32_t* frames) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    if (g.arch != WD_ARCH_WHISPER) return fail(ctx, WD_ERR_STATE, "wd_cross_kv_ragged: no cross-attention in this arch");
    if (!enc || !frames) return fail(ctx, WD_ERR_ARG, "wd_cross_kv_ragged: null pointer");
    int F = 0;
    for (int e = 0; e < g.n_enc; ++e) {
      if (frames[e] < 1 || frames[e] > g.max_frames)
        return fail(ctx, WD_ERR_ARG, "wd_cross_kv_ragged: a set's frames outside [1, max_frames]");
      F = std::max(F, (int)frames[e]);
    }
    ctx->frames_host.assign(frames, frames + g.n_enc);
    HIPCHK(ctx, hipMemcpyAsync(ctx->at(ctx->plan.frames_dev), ctx->frames_host.data(), (size_t)g.n_enc * 4,
                               hipMemcpyHostToDevice, ctx->stream), "wd_cross_kv_ragged: frame counts");
    const wd_status st = cross_kv_impl(ctx, enc, F, "cross K/V projection (ragged)");
    if (st == WD_OK) ctx->ragged = true;
    return st;
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_cross_kv_ragged: internal error");
  }
}

static wd_status check_rows(wd_ctx* ctx, int32_t B, const char* who) {
  const wd_config& g = ctx->cfg;
  if (B < 1 || B > g.max_batch) return fail(ctx, WD_ERR_ARG, std::string(who) + ": B outside [1, max_batch]");
  if (g.arch == WD_ARCH_WHISPER) {
    if (!ctx->cross_ready) return fail(ctx, WD_ERR_STATE, std::string(who) + ": call wd_cross_kv first");
    const int r = rows_per_set(g, B);
    if (B % r) return fail(ctx, WD_ERR_ARG, std::string(who) + ": B must be a multiple of max_batch / n_enc");
  }
  return WD_OK;
}

// One step over the staged inputs (tokens in tok_in, positions in pos_tmp, override rows in
// ov_in when `ov`), replayed from a captured graph when the context allows it.  Graphs are
// keyed by everything a step bakes in: output buffers, B, the current self cache, the frame
// count and the step kind; the per-call inputs are copied into fixed buffers beforehand.
static wd_status staged_step(wd_ctx* ctx, int32_t B, float* logits, int32_t* argmax, bool head, bool ov) {
  const Plan& P = ctx->plan;
  const int32_t* tok = ctx->at<int32_t>(P.tok_in);
  const int32_t* pos = ctx->at<int32_t>(P.pos_tmp);
  const void* ovp = ov ? ctx->at(P.ov_in) : nullptr;
  const int64_t ovs = (int64_t)ctx->cfg.d_model;
  if (!ctx->use_graphs || ctx->prof_kernel >= 0 || ctx->stream == nullptr)
    return run_step(ctx, tok, 1, pos, ovp, ovs, B, logits, argmax, head);
  const GraphKey key{logits, argmax, B, ctx->cur, ctx->frames, head ? 0 : (ov ? 2 : 1), ctx->ragged};
  for (size_t i = 0; i < ctx->graphs.size(); ++i)
    if (ctx->graphs[i].key == key) {   // least recently used order: a hit moves to the back
      const GraphEntry hit = ctx->graphs[i];
      ctx->graphs.erase(ctx->graphs.begin() + (ptrdiff_t)i);
      ctx->graphs.push_back(hit);
      HIPCHK(ctx, hipGraphLaunch(hit.exec, ctx->stream), "step: graph launch");
      return WD_OK;
    }
  HIPCHK(ctx, hipStreamBeginCapture(ctx->stream, hipStreamCaptureModeThreadLocal), "step: begin capture");
  const wd_status r = run_step(ctx, tok, 1, pos, ovp, ovs, B, logits, argmax, head);
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(ctx->stream, &graph);
  if (r != WD_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return r;
  }
  if (ec != hipSuccess) return fail(ctx, WD_ERR_HIP, std::string("step: end capture: ") + hipGetErrorString(ec));
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (ei != hipSuccess) return fail(ctx, WD_ERR_HIP, std::string("step: instantiate: ") + hipGetErrorString(ei));
  if (ctx->graphs.size() >= 8) {
    // the least recently used graph may still be running (launched by an earlier step on
    // this stream): wait for the stream before destroying it
    HIPCHK(ctx, hipStreamSynchronize(ctx->stream), "step: graph cache eviction");
    (void)hipGraphExecDestroy(ctx->graphs.front().exec);
    ctx->graphs.erase(ctx->graphs.begin());
  }
  ctx->graphs.push_back({key, exec});
  HIPCHK(ctx, hipGraphLaunch(exec, ctx->stream), "step: graph launch");
  return WD_OK;
}

wd_status wd_step(wd_ctx* ctx, const int32_t* tokens, const int32_t* positions, int32_t B, float* logits,
                  int32_t* argmax) {
  if (!ctx) return WD_ERR_ARG;
  try {
    if (!tokens || !positions || !argmax) return fail(ctx, WD_ERR_ARG, "wd_step: tokens, positions, argmax must not be null");
    const wd_status st = check_rows(ctx, B, "wd_step");
    if (st != WD_OK) return st;
    const Plan& P = ctx->plan;
    HIPCHK(ctx, wd::launch_stage(tokens, 1, positions, 0, ctx->at<int32_t>(P.tok_in), ctx->at<int32_t>(P.pos_tmp), B,
                                 nullptr, 0, nullptr, 0, ctx->stream), "wd_step: stage inputs");
    return staged_step(ctx, B, logits, argmax, true, false);
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_step: internal error");
  }
}

namespace {

// Final norm, tied-head logits and argmax of the B rows in x (16-bit weights).
wd_status run_head_mfma(wd_ctx* c, int B, float* logits, int32_t* argmax) {
  const wd_config& g = c->cfg;
  const Plan& P = c->plan;
  hipStream_t s = c->stream;
  const bool whisper = g.arch == WD_ARCH_WHISPER;
  HIPCHK(c, wd::launch_norm_split(c->at<float>(P.x), c->at(P.yh), c->at(P.yl), g.w_dtype, c->at<float>(P.lnfg),
                                  whisper ? c->at<float>(P.lnfb) : nullptr, B, g.d_model, g.norm_eps, s),
         "final norm");
  wd::MGemvParams hm{};
  hm.W = c->at(P.embed); hm.w_dtype = g.w_dtype; hm.N = g.vocab; hm.K = g.d_model;
  hm.Yhi = c->at(P.yh); hm.Ylo = c->at(P.yl); hm.B = B; hm.epi = wd::EPI_LOGITS;
  hm.out = logits; hm.ldo = g.vocab; hm.scale = 1.0f; hm.err = c->at<unsigned>(P.err);
  hm.amax = c->at<unsigned long long>(P.amax); hm.ldp = g.max_batch;
  HIPCHK(c, wd::launch_mgemv(hm, s), "logits");
  HIPCHK(c, wd::launch_argmax_final(hm.amax, wd::mgemv_blocks_k(g.vocab, g.d_model, B), g.max_batch, B, argmax, s),
         "argmax");
  return WD_OK;
}

// Batched Qwen3 prefill: the prompt in chunks of up to pf_pos_chunk positions for all B rows, each
// layer as dense GEMMs over the chunk's rows, the per-head q/k norm + RoPE + append of the
// decode step, and a causal prefill attention over the cache; then the head on the last
// position of every row.  Runs eagerly (no graph): a few launches per layer and chunk.
wd_status prefill_batched(wd_ctx* c, const int32_t* tokens, int B, int T, const void* embeds, int A, int offset,
                          float* logits, int32_t* argmax) {
  const wd_config& g = c->cfg;
  const Plan& P = c->plan;
  hipStream_t s = c->stream;
  const int d = g.d_model, hd = g.head_dim, hq = g.n_heads, hkv = g.n_kv_heads, ff = g.d_ff;
  const int nqkv = (hq + 2 * hkv) * hd, CH = P.pf_pos_chunk;
  const int adt = g.w_dtype;
  const float qscale = 1.0f / sqrtf((float)hd);
  const int64_t kv_bstride = (int64_t)hkv * g.context * hd;
  float* x = c->at<float>(P.pf_x);
  int32_t* pos = c->at<int32_t>(P.pf_pos);
  void *ah = c->at(P.pf_ah), *al = c->at(P.pf_al), *hh = c->at(P.pf_hh), *hl = c->at(P.pf_hl);
  unsigned* err = c->at<unsigned>(P.err);
  int R_ = 0;   // rows of the current chunk
  auto gemm = [&](const void* W, int N, int K, const void* Ahi, const void* Alo, int epi, float* out, int ldo,
                  const char* what) -> wd_status {
    wd::FgParams f{};
    f.W = W; f.w_dtype = g.w_dtype; f.N = N; f.K = K; f.Ahi = Ahi; f.Alo = Alo; f.R = R_; f.epi = epi;
    f.out = out; f.ldo = ldo; f.Ohi = hh; f.Olo = hl;
    HIPCHK(c, wd::launch_fgemm(f, s), what);
    return WD_OK;
  };
#define WDCHK(expr) do { const wd_status st_ = (expr); if (st_ != WD_OK) return st_; } while (0)
  for (int t0 = 0; t0 < T; t0 += CH) {
    // a chunk's rows are b * C + j: the last, shorter chunk takes only the rows it has
    const int Cn = std::min(CH, T - t0), C = Cn, R = B * C;
    R_ = R;
    HIPCHK(c, wd::launch_pf_embed(x, pos, c->at(P.embed), g.w_dtype, tokens, T, embeds, A, offset, t0, B, C, Cn, d,
                                  g.vocab, err, s), "prefill: embed");
    for (int l = 0; l < g.n_layers; ++l) {
      const LayerOff& L = P.L[l];
      HIPCHK(c, wd::launch_norm_split(x, ah, al, adt, c->at<float>(L.n1g), nullptr, R, d, g.norm_eps, s), "prefill: norm1");
      WDCHK(gemm(c->at(L.wqkv), nqkv, d, ah, al, wd::FG_STORE, c->at<float>(P.pf_qkv), nqkv, "prefill: qkv"));
      HIPCHK(c, wd::launch_qk_rope_append(c->at<float>(P.pf_qkv), R, hq, hkv, hd, pos, g.context, c->at<float>(L.qn),
                                          c->at<float>(L.kn), g.norm_eps, c->at<float>(P.rope), qscale, c->at<float>(P.pf_q),
                                          c->self_k(l), c->self_v(l), g.cache_dtype, kv_bstride, s, nullptr, 0, C),
             "prefill: qk norm/rope/append");
      wd::PfAttnParams pa{};
      pa.q = c->at<float>(P.pf_q); pa.K = c->self_k(l); pa.V = c->self_v(l); pa.cache_dtype = g.cache_dtype;
      pa.kv_bstride = kv_bstride; pa.ctx = g.context; pa.B = B; pa.C = C; pa.Cn = Cn; pa.t0 = t0;
      pa.Hq = hq; pa.Hkv = hkv; pa.hd = hd; pa.o_hi = ah; pa.o_lo = al; pa.o_dtype = adt;
      HIPCHK(c, wd::launch_pf_attn(pa, s), "prefill: attention");
      WDCHK(gemm(c->at(L.wo), d, hq * hd, ah, al, wd::FG_RESID, x, d, "prefill: out projection"));
      HIPCHK(c, wd::launch_norm_split(x, ah, al, adt, c->at<float>(L.n2g), nullptr, R, d, g.norm_eps, s), "prefill: norm2");
      WDCHK(gemm(c->at(L.wgu), 2 * ff, d, ah, al, wd::FG_SWIGLU, nullptr, 0, "prefill: gate|up"));
      WDCHK(gemm(c->at(L.wdn), d, ff, hh, hl, wd::FG_RESID, x, d, "prefill: down projection"));
    }
    if (t0 + Cn == T) {   // the last position of every row -> the step's x, then the head
      HIPCHK(c, hipMemcpy2DAsync(c->at<float>(P.x), (size_t)d * 4, x + (size_t)(Cn - 1) * d, (size_t)C * d * 4,
                                 (size_t)d * 4, B, hipMemcpyDeviceToDevice, s), "prefill: last rows");
      WDCHK(run_head_mfma(c, B, logits, argmax));
    }
  }
#undef WDCHK
  return WD_OK;
}

// The batched prefill serves 16-bit Qwen3 contexts (the plan has its chunk buffers); any other
// context runs every prompt position as a decode step.
bool prefill_batched_on(const wd_ctx* c) { return c->plan.pf_rows > 0; }

}  // namespace

wd_status wd_prefill(wd_ctx* ctx, const int32_t* tokens, int32_t B, int32_t T, const void* embeds, int32_t A,
                     int32_t offset, float* logits, int32_t* argmax) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    if (!tokens || !argmax) return fail(ctx, WD_ERR_ARG, "wd_prefill: tokens and argmax must not be null");
    if (T < 1 || T > g.context) return fail(ctx, WD_ERR_ARG, "wd_prefill: T outside [1, context]");
    if (A < 0 || offset < 0 || offset + A > T || (A > 0 && !embeds))
      return fail(ctx, WD_ERR_ARG, "wd_prefill: audio rows must lie inside the prompt");
    const wd_status st = check_rows(ctx, B, "wd_prefill");
    if (st != WD_OK) return st;
    const Plan& P = ctx->plan;
    if (prefill_batched_on(ctx)) return prefill_batched(ctx, tokens, B, T, embeds, A, offset, logits, argmax);
    const size_t eb = dtype_bytes(g.w_dtype);
    const int64_t row_bytes = (int64_t)g.d_model * eb;
    for (int t = 0; t < T; ++t) {
      const bool ov = A > 0 && t >= offset && t < offset + A;
      const void* src = ov ? reinterpret_cast<const char*>(embeds) + (size_t)(t - offset) * row_bytes : nullptr;
      HIPCHK(ctx, wd::launch_stage(tokens + t, T, nullptr, t, ctx->at<int32_t>(P.tok_in), ctx->at<int32_t>(P.pos_tmp),
                                   B, src, (int64_t)A * row_bytes, ov ? ctx->at(P.ov_in) : nullptr, row_bytes,
                                   ctx->stream), "wd_prefill: stage inputs");
      const wd_status r = staged_step(ctx, B, t == T - 1 ? logits : nullptr, argmax, t == T - 1, ov);
      if (r != WD_OK) return r;
    }
    return WD_OK;
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_prefill: internal error");
  }
}

wd_status wd_reorder(wd_ctx* ctx, const int32_t* beam_idx, int32_t B, int32_t n_rows) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    if (ctx->plan.n_bufs < 2) return fail(ctx, WD_ERR_STATE, "wd_reorder: needs n_enc == 1 and max_batch > 1");
    if (!beam_idx) return fail(ctx, WD_ERR_ARG, "wd_reorder: beam_idx must not be null");
    if (B < 1 || B > g.max_batch) return fail(ctx, WD_ERR_ARG, "wd_reorder: B outside [1, max_batch]");
    if (n_rows < 0 || n_rows > g.context) return fail(ctx, WD_ERR_ARG, "wd_reorder: n_rows outside [0, context]");
    wd::BeamIdx idx{};
    bool ident = true;
    for (int b = 0; b < B; ++b) {
      if (beam_idx[b] < 0 || beam_idx[b] >= B) return fail(ctx, WD_ERR_ARG, "wd_reorder: beam index outside [0, B)");
      idx.v[b] = beam_idx[b];
      ident = ident && beam_idx[b] == b;
    }
    if (ident || n_rows == 0) return WD_OK;
    const int nxt = 1 - ctx->cur;
    HIPCHK(ctx, wd::launch_reorder(ctx->ws + ctx->plan.self[ctx->cur], ctx->ws + ctx->plan.self[nxt],
                                   dtype_bytes(g.cache_dtype), idx, B, g.max_batch, g.n_kv_heads, g.context,
                                   g.head_dim, n_rows, 2 * g.n_layers, ctx->stream), "beam reorder");
    ctx->cur = nxt;
    return WD_OK;
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_reorder: internal error");
  }
}

size_t wd_encoder_workspace_bytes(const wd_ctx* ctx, int32_t n_mels, int32_t frames, int32_t n_layers,
                                   int32_t d_ff, int32_t max_sets) {
  if (!ctx || !check_enc(ctx->cfg, n_mels, frames, n_layers, d_ff, max_sets).empty()) return 0;
  return make_enc_plan(ctx->cfg, n_mels, frames, n_layers, d_ff, max_sets).total;
}

wd_status wd_load_encoder(wd_ctx* ctx, int32_t n_mels, int32_t frames, int32_t n_layers, int32_t d_ff,
                          int32_t max_sets, const wd_tensor* weights, int32_t n_weights, void* workspace,
                          size_t ws_bytes) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    const std::string why = check_enc(g, n_mels, frames, n_layers, d_ff, max_sets);
    if (!why.empty()) return fail(ctx, WD_ERR_ARG, "wd_load_encoder: " + why);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
      return fail(ctx, WD_ERR_ARG, "wd_load_encoder: workspace must be a 256-byte aligned device pointer");
    if (n_weights < 0 || (n_weights > 0 && !weights)) return fail(ctx, WD_ERR_ARG, "wd_load_encoder: bad weight list");
    EncPlan plan = make_enc_plan(g, n_mels, frames, n_layers, d_ff, max_sets);
    if (ws_bytes < plan.total)
      return fail(ctx, WD_ERR_OOM, "wd_load_encoder: workspace of " + std::to_string(ws_bytes) + " bytes, need " +
                                       std::to_string(plan.total));
    const int64_t d = g.d_model, P = plan.P;
    struct Need { std::string name; int64_t numel; bool matrix; };
    std::vector<Need> need = {{"enc.conv1.w", d * n_mels * 3, true}, {"enc.conv1.b", d, false},
                              {"enc.conv2.w", d * d * 3, true}, {"enc.conv2.b", d, false},
                              {"enc.pos", P * d, false}, {"enc.ln_post.g", d, false}, {"enc.ln_post.b", d, false}};
    for (int l = 0; l < n_layers; ++l) {
      const std::string p = "enc." + std::to_string(l) + ".";
      for (const char* v : {"ln1.g", "ln1.b", "ln2.g", "ln2.b", "attn.q.b", "attn.v.b", "attn.o.b", "fc2.b"})
        need.push_back({p + v, d, false});
      for (const char* m : {"attn.q.w", "attn.k.w", "attn.v.w", "attn.o.w"}) need.push_back({p + m, d * d, true});
      need.push_back({p + "fc1.w", (int64_t)d_ff * d, true});
      need.push_back({p + "fc1.b", d_ff, false});
      need.push_back({p + "fc2.w", d * d_ff, true});
    }
    std::map<std::string, const wd_tensor*> byname;
    for (int i = 0; i < n_weights; ++i) {
      const wd_tensor& t = weights[i];
      if (!t.name) return fail(ctx, WD_ERR_ARG, "wd_load_encoder: tensor with null name");
      const std::string nm(t.name);
      if (nm.size() >= 4 && nm.compare(nm.size() - 4, 4, ".k.b") == 0)
        return fail(ctx, WD_ERR_ARG, "wd_load_encoder: '" + nm + "': the key projections carry no bias");
      if (byname.count(nm)) return fail(ctx, WD_ERR_ARG, "wd_load_encoder: duplicate tensor '" + nm + "'");
      byname[nm] = &t;
    }
    if (byname.size() != need.size()) return fail(ctx, WD_ERR_ARG, "wd_load_encoder: unexpected tensor count");
    for (const auto& n : need) {
      auto it = byname.find(n.name);
      if (it == byname.end()) return fail(ctx, WD_ERR_ARG, "wd_load_encoder: missing tensor '" + n.name + "'");
      const wd_tensor& t = *it->second;
      if (!t.data || t.numel != n.numel || !valid_dt(t.dtype) || (n.matrix && t.dtype != g.w_dtype))
        return fail(ctx, WD_ERR_ARG, "wd_load_encoder: '" + n.name + "' has a bad pointer, size or dtype");
    }
    char* ws = reinterpret_cast<char*>(workspace);
    hipStream_t s = ctx->stream;
    const int wdt = g.w_dtype;
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    auto T = [&](const std::string& nm) { return byname[nm]; };
    auto vec = [&](const std::string& nm, size_t dst, int64_t n) {
      const wd_tensor* t = T(nm);
      chk(wd::launch_copy_rows(t->data, t->dtype, ws + dst, DT_F32, 1, n, 1, 0, s));
    };
    auto mat = [&](const std::string& nm, size_t dst, int64_t rows, int64_t K, int64_t blk_add) {
      const wd_tensor* t = T(nm);
      chk(wd::launch_pack_frag(t->data, t->dtype, ws + dst, wdt, rows, K, 1, blk_add, s));
    };
    // the stem's kernels [d, C, 3] flattened as (c, tap), columns padded to whole K steps
    chk(wd::launch_pack_pad(T("enc.conv1.w")->data, wdt, d, 3 * n_mels, ws + plan.conv1w, wdt, plan.kp1, s));
    chk(wd::launch_pack_pad(T("enc.conv2.w")->data, wdt, d, 3 * (int)d, ws + plan.conv2w, wdt, 3 * (int)d, s));
    vec("enc.conv1.b", plan.conv1b, d); vec("enc.conv2.b", plan.conv2b, d);
    vec("enc.pos", plan.pos, P * d);
    vec("enc.ln_post.g", plan.lnpg, d); vec("enc.ln_post.b", plan.lnpb, d);
    for (int l = 0; l < n_layers; ++l) {
      const std::string p = "enc." + std::to_string(l) + ".";
      const EncLayer& L = plan.L[l];
      vec(p + "ln1.g", L.ln1g, d); vec(p + "ln1.b", L.ln1b, d); vec(p + "ln2.g", L.ln2g, d); vec(p + "ln2.b", L.ln2b, d);
      mat(p + "attn.q.w", L.wqkv, d, d, 0);
      mat(p + "attn.k.w", L.wqkv, d, d, d / 16);
      mat(p + "attn.v.w", L.wqkv, d, d, 2 * d / 16);
      vec(p + "attn.q.b", L.bq, d); vec(p + "attn.v.b", L.bv, d);
      mat(p + "attn.o.w", L.wo, d, d, 0); vec(p + "attn.o.b", L.bo, d);
      mat(p + "fc1.w", L.w1, d_ff, d, 0); vec(p + "fc1.b", L.b1, d_ff);
      mat(p + "fc2.w", L.w2, d, d_ff, 0); vec(p + "fc2.b", L.b2, d);
    }
    HIPCHK(ctx, e, "wd_load_encoder: weight repack");
    delete ctx->enc;
    ctx->enc = new EncPlan(plan);
    ctx->enc_ws = ws;
    return WD_OK;
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_load_encoder: internal error");
  }
}

wd_status wd_encode(wd_ctx* ctx, const void* mel, int32_t n_sets, void* enc) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    const EncPlan* E = ctx->enc;
    if (!E) return fail(ctx, WD_ERR_STATE, "wd_encode: no encoder loaded (wd_load_encoder)");
    if (!mel || !enc) return fail(ctx, WD_ERR_ARG, "wd_encode: null pointer");
    if (n_sets < 1 || n_sets > E->max_sets) return fail(ctx, WD_ERR_ARG, "wd_encode: n_sets outside [1, max_sets]");
    char* ws = ctx->enc_ws;
    auto at = [&](size_t off) { return reinterpret_cast<void*>(ws + off); };
    auto atf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    hipStream_t s = ctx->stream;
    const int d = g.d_model, H = g.n_heads, hd = g.head_dim, wdt = g.w_dtype, P = E->P;
    const int R1 = n_sets * E->frames, R = n_sets * P;
    auto gemm = [&](const void* W, int N, int K, const void* Ahi, const void* Alo, int rows, int epi, float* out,
                    const float* bias, const float* pos, void* Ohi, void* Olo, const char* what) -> wd_status {
      wd::FgParams f{};
      f.W = W; f.w_dtype = wdt; f.N = N; f.K = K; f.Ahi = Ahi; f.Alo = Alo; f.R = rows; f.epi = epi;
      f.out = out; f.ldo = N; f.Ohi = Ohi; f.Olo = Olo; f.bias = bias; f.pos = pos; f.pos_rows = P;
      HIPCHK(ctx, wd::launch_fgemm(f, s), what);
      return WD_OK;
    };
#define WDCHK(expr) do { const wd_status st_ = (expr); if (st_ != WD_OK) return st_; } while (0)
    // stem: GELU(conv1(mel) + b1), GELU(conv2(.) + b2) + positions
    HIPCHK(ctx, wd::launch_conv_windows(mel, wdt, n_sets, E->frames, E->mels, 1, E->frames, E->kp1, at(E->ah),
                                        at(E->al), wdt, s), "wd_encode: conv1 windows");
    WDCHK(gemm(at(E->conv1w), d, E->kp1, at(E->ah), at(E->al), R1, wd::FG_GELU, atf(E->x1), atf(E->conv1b), nullptr,
               nullptr, nullptr, "wd_encode: conv1"));
    HIPCHK(ctx, wd::launch_conv_windows(atf(E->x1), DT_F32, n_sets, E->frames, d, 2, P, 3 * d, at(E->ah), at(E->al),
                                        wdt, s), "wd_encode: conv2 windows");
    WDCHK(gemm(at(E->conv2w), d, 3 * d, at(E->ah), at(E->al), R, wd::FG_GELU, atf(E->x), atf(E->conv2b), atf(E->pos),
               nullptr, nullptr, "wd_encode: conv2"));
    const float qscale = 1.0f / sqrtf((float)hd);
    for (int l = 0; l < E->layers; ++l) {
      const EncLayer& L = E->L[l];
      HIPCHK(ctx, wd::launch_norm_split(atf(E->x), at(E->ah), at(E->al), wdt, atf(L.ln1g), atf(L.ln1b), R, d,
                                        g.norm_eps, s), "wd_encode: ln1");
      {   // q|k|v with its biases, the q scale and the K/V layout in the GEMM's epilogue
        wd::FgParams f{};
        f.W = at(L.wqkv); f.w_dtype = wdt; f.N = 3 * d; f.K = d; f.Ahi = at(E->ah); f.Alo = at(E->al); f.R = R;
        f.epi = wd::FG_ENC_QKV; f.out = atf(E->q); f.ldo = d; f.bias = atf(L.bq); f.bias2 = atf(L.bv);
        f.scale = qscale; f.Kc = at(E->K); f.Vc = at(E->V); f.kv_P = P; f.kv_H = H; f.kv_hd = hd;
        HIPCHK(ctx, wd::launch_fgemm(f, s), "wd_encode: q|k|v");
      }
      wd::PfAttnParams pa{};
      pa.q = atf(E->q); pa.K = at(E->K); pa.V = at(E->V); pa.cache_dtype = wdt;
      pa.kv_bstride = (int64_t)H * P * hd; pa.ctx = P; pa.B = n_sets; pa.C = P; pa.Cn = P; pa.t0 = 0;
      pa.Hq = H; pa.Hkv = H; pa.hd = hd; pa.o_hi = at(E->ah); pa.o_lo = at(E->al); pa.o_dtype = wdt; pa.full = true;
      HIPCHK(ctx, wd::launch_pf_attn(pa, s), "wd_encode: attention");
      WDCHK(gemm(at(L.wo), d, d, at(E->ah), at(E->al), R, wd::FG_RESID, atf(E->x), atf(L.bo), nullptr, nullptr,
                 nullptr, "wd_encode: out projection"));
      HIPCHK(ctx, wd::launch_norm_split(atf(E->x), at(E->ah), at(E->al), wdt, atf(L.ln2g), atf(L.ln2b), R, d,
                                        g.norm_eps, s), "wd_encode: ln2");
      WDCHK(gemm(at(L.w1), E->dff, d, at(E->ah), at(E->al), R, wd::FG_GELU_SPLIT, nullptr, atf(L.b1), nullptr,
                 at(E->hh), at(E->hl), "wd_encode: fc1"));
      WDCHK(gemm(at(L.w2), d, E->dff, at(E->hh), at(E->hl), R, wd::FG_RESID, atf(E->x), atf(L.b2), nullptr, nullptr,
                 nullptr, "wd_encode: fc2"));
    }
#undef WDCHK
    HIPCHK(ctx, wd::launch_norm(atf(E->x), atf(E->qkv), atf(E->lnpg), atf(E->lnpb), R, d, g.norm_eps, s),
           "wd_encode: final norm");
    HIPCHK(ctx, wd::launch_cast(atf(E->qkv), enc, wdt, (int64_t)R * d, s), "wd_encode: output");
    return WD_OK;
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_encode: internal error");
  }
}

wd_status wd_listen(wd_ctx* ctx, const void* mel) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    const EncPlan* E = ctx->enc;
    if (!E) return fail(ctx, WD_ERR_STATE, "wd_listen: no encoder loaded (wd_load_encoder)");
    if (E->max_sets != g.n_enc) return fail(ctx, WD_ERR_STATE, "wd_listen: the encoder's max_sets must equal n_enc");
    void* states = ctx->enc_ws + E->states;
    const wd_status st = wd_encode(ctx, mel, g.n_enc, states);
    if (st != WD_OK) return st;
    return wd_cross_kv(ctx, states, E->P);
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_listen: internal error");
  }
}

wd_status wd_topk(wd_ctx* ctx, const float* logits, int32_t B, int32_t W, float* top_val, int32_t* top_id,
                  float* lse) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    if (!logits || !top_val || !top_id || !lse) return fail(ctx, WD_ERR_ARG, "wd_topk: null pointer");
    if (B < 1 || B > g.max_batch) return fail(ctx, WD_ERR_ARG, "wd_topk: B outside [1, max_batch]");
    if (W < 1 || W > 8 || W > g.vocab) return fail(ctx, WD_ERR_ARG, "wd_topk: W outside [1, min(8, vocab)]");
    HIPCHK(ctx, wd::launch_topk_lse(logits, B, g.vocab, g.vocab, W, top_val, top_id, lse, ctx->at(ctx->plan.topk),
                                    ctx->stream), "beam candidates");
    return WD_OK;
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_topk: internal error");
  }
}

wd_status wd_beam_step(wd_ctx* ctx, const float* logits, int32_t W, int32_t first, double* scores,
                       int32_t* beam_idx, int32_t* tokens, int32_t n_rows) {
  if (!ctx) return WD_ERR_ARG;
  try {
    const wd_config& g = ctx->cfg;
    if (!logits || !scores || !beam_idx || !tokens) return fail(ctx, WD_ERR_ARG, "wd_beam_step: null pointer");
    if (W < 1 || W > 8 || W > g.max_batch || W > g.vocab)
      return fail(ctx, WD_ERR_ARG, "wd_beam_step: W outside [1, min(8, max_batch, vocab)]");
    if (first != 0 && first != 1) return fail(ctx, WD_ERR_ARG, "wd_beam_step: first must be 0 or 1");
    if (n_rows < 0 || n_rows > g.context) return fail(ctx, WD_ERR_ARG, "wd_beam_step: n_rows outside [0, context]");
    if (n_rows > 0 && ctx->plan.n_bufs < 2)
      return fail(ctx, WD_ERR_STATE, "wd_beam_step: the reorder needs n_enc == 1 and max_batch > 1");
    float* tv = ctx->at<float>(ctx->plan.beam);
    int32_t* ti = reinterpret_cast<int32_t*>(tv + 64);
    float* lse = tv + 128;
    const int rows = first ? 1 : W;
    HIPCHK(ctx, wd::launch_topk_lse(logits, rows, g.vocab, g.vocab, W, tv, ti, lse, ctx->at(ctx->plan.topk),
                                    ctx->stream), "beam candidates");
    HIPCHK(ctx, wd::launch_beam_merge(tv, ti, lse, scores, beam_idx, tokens, W, rows, g.vocab, ctx->stream),
           "beam merge");
    if (n_rows > 0) {
      const int nxt = 1 - ctx->cur;
      HIPCHK(ctx, wd::launch_reorder_dev(ctx->ws + ctx->plan.self[ctx->cur], ctx->ws + ctx->plan.self[nxt],
                                         dtype_bytes(g.cache_dtype), beam_idx, W, g.max_batch, g.n_kv_heads,
                                         g.context, g.head_dim, n_rows, 2 * g.n_layers, ctx->stream),
             "beam reorder");
      ctx->cur = nxt;
    }
    return WD_OK;
  } catch (...) {
    return fail(ctx, WD_ERR_INTERNAL, "wd_beam_step: internal error");
  }
}

wd_status wd_topk_noalloc(const float* logits, int32_t B, int32_t V, int64_t ld, int32_t W, float* top_val,
                          int32_t* top_id, float* lse, void* stream) {
  try {
    if (!logits || !top_val || !top_id || !lse) return fail(nullptr, WD_ERR_ARG, "wd_topk_noalloc: null pointer");
    if (B < 1 || B > WD_TOPK_NOALLOC_MAX_ROWS)
      return fail(nullptr, WD_ERR_ARG, "wd_topk_noalloc: B outside [1, " + std::to_string(WD_TOPK_NOALLOC_MAX_ROWS) +
                                           "] (the size of its static scratch)");
    if (V < 1 || ld < V) return fail(nullptr, WD_ERR_ARG, "wd_topk_noalloc: V < 1 or ld < V");
    if (W < 1 || W > 8 || W > V) return fail(nullptr, WD_ERR_ARG, "wd_topk_noalloc: W outside [1, min(8, V)]");
    if (wd::topk_scratch_bytes(B, V) > kTopkScratchBytes)
      return fail(nullptr, WD_ERR_INTERNAL, "wd_topk_noalloc: scratch too small for this shape");
    void* sp = nullptr;
    const hipError_t e = scratch_address(&sp);
    if (e != hipSuccess) return fail(nullptr, WD_ERR_HIP, std::string("wd_topk_noalloc: scratch address: ") + hipGetErrorString(e));
    const hipError_t l = wd::launch_topk_lse(logits, B, V, ld, W, top_val, top_id, lse, sp,
                                             reinterpret_cast<hipStream_t>(stream));
    if (l != hipSuccess) return fail(nullptr, WD_ERR_HIP, std::string("wd_topk_noalloc: launch: ") + hipGetErrorString(l));
    return WD_OK;
  } catch (...) {
    return fail(nullptr, WD_ERR_INTERNAL, "wd_topk_noalloc: internal error");
  }
}

wd_status wd_check(wd_ctx* ctx) {
  if (!ctx) return WD_ERR_ARG;
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream), "wd_check: stream sync");
  unsigned flag[4] = {0, 0, 0, 0};
  HIPCHK(ctx, hipMemcpy(flag, ctx->ws + ctx->plan.err, sizeof(flag), hipMemcpyDeviceToHost), "wd_check: read flag");
  if (flag[0]) {
    HIPCHK(ctx, wd::launch_fill_u32(reinterpret_cast<uint32_t*>(ctx->ws + ctx->plan.err), 0u, 4, ctx->stream), "wd_check: clear");
    HIPCHK(ctx, hipStreamSynchronize(ctx->stream), "wd_check: stream sync");
    std::string m = "device range flag:";
    if (flag[0] & wd::ERR_TOKEN) m += " token id outside [0, vocab)";
    if (flag[0] & wd::ERR_POS) m += " position outside [0, context)";
    if (flag[0] & wd::ERR_NAN) m += " NaN logit";
    return fail(ctx, WD_ERR_RANGE, m);
  }
  return WD_OK;
}

const char* wd_last_error(const wd_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_load_error.c_str();
}

void wd_free(wd_ctx* ctx) {
  if (!ctx) return;
  // launched graphs and kernels may still be running on the context's stream: wait for it
  // before their graphs are destroyed (and before the caller can release the workspace)
  if (ctx->stream) (void)hipStreamSynchronize(ctx->stream);
  else (void)hipDeviceSynchronize();
  for (auto& e : ctx->graphs) (void)hipGraphExecDestroy(e.exec);
  delete ctx->enc;
  for (auto& pr : ctx->prof) {
    (void)hipEventDestroy(pr.a);
    (void)hipEventDestroy(pr.b);
  }
  delete ctx;
}

wd_status wd_set_option(wd_ctx* ctx, int32_t option, int32_t value) {
  if (!ctx) return WD_ERR_ARG;
  switch (option) {
    case WD_OPT_GRAPHS:
      if (value != 0 && value != 1) return fail(ctx, WD_ERR_ARG, "wd_set_option: WD_OPT_GRAPHS takes 0 or 1");
      ctx->use_graphs = value == 1;
      return WD_OK;
    default:
      return fail(ctx, WD_ERR_ARG, "wd_set_option: unknown option");
  }
}

wd_status wd_get_option(wd_ctx* ctx, int32_t option, int32_t* value) {
  if (!ctx) return WD_ERR_ARG;
  if (!value) return fail(ctx, WD_ERR_ARG, "wd_get_option: value must not be null");
  switch (option) {
    case WD_OPT_GRAPHS: *value = ctx->use_graphs ? 1 : 0; return WD_OK;
    default: return fail(ctx, WD_ERR_ARG, "wd_get_option: unknown option");
  }
}

wd_status wd_profile(wd_ctx* ctx, int32_t kernel, int32_t layer, int32_t repeats) {
  if (!ctx) return WD_ERR_ARG;
  if (kernel < -1 || kernel > 4) return fail(ctx, WD_ERR_ARG, "wd_profile: unknown kernel class");
  if (repeats < 1 || repeats > 64) return fail(ctx, WD_ERR_ARG, "wd_profile: repeats must be in [1, 64]");
  if (ctx->prof.empty() && kernel >= 0) {
    ctx->prof.resize(4096);
    for (auto& pr : ctx->prof) {
      HIPCHK(ctx, hipEventCreate(&pr.a), "wd_profile: event");
      HIPCHK(ctx, hipEventCreate(&pr.b), "wd_profile: event");
    }
  }
  ctx->prof_kernel = kernel;
  ctx->prof_layer = layer;
  ctx->prof_repeats = repeats;
  ctx->prof_used = 0;
  return WD_OK;
}

wd_status wd_profile_read(wd_ctx* ctx, double* total_ms, int64_t* launches) {
  if (!ctx || !total_ms || !launches) return WD_ERR_ARG;
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream), "wd_profile_read: sync");
  double t = 0.0;
  int64_t n = 0;
  for (size_t i = 0; i < ctx->prof_used; ++i) {
    float ms = 0.f;
    HIPCHK(ctx, hipEventElapsedTime(&ms, ctx->prof[i].a, ctx->prof[i].b), "wd_profile_read: elapsed");
    t += ms;
    n += ctx->prof[i].n;
  }
  *total_ms = t;
  *launches = n;
  ctx->prof_used = 0;
  return WD_OK;
}

wd_status wd_debug_cache(wd_ctx* ctx, int32_t which, int32_t layer, void** dev_ptr) {
  if (!ctx) return WD_ERR_ARG;
  if (!dev_ptr || layer < 0 || layer >= ctx->cfg.n_layers || which < 0 || which > 3)
    return fail(ctx, WD_ERR_ARG, "wd_debug_cache: bad argument");
  if (which >= 2 && ctx->cfg.arch != WD_ARCH_WHISPER) return fail(ctx, WD_ERR_ARG, "wd_debug_cache: no cross cache");
  *dev_ptr = which == 0 ? ctx->self_k(layer) : which == 1 ? ctx->self_v(layer)
           : which == 2 ? ctx->cross_k(layer) : ctx->cross_v(layer);
  return WD_OK;
}

wd_status wd_probe(int32_t kind, const void* a, const void* b, int64_t bytes, int32_t iters, float* sink,
                   double* us) {
  if (!us || iters < 1 || iters > 100000 || kind < 0 || kind > 5)
    return fail(nullptr, WD_ERR_ARG, "wd_probe: kind must be in [0, 5], iters in [1, 100000], us not null");
  const bool aligned = !(reinterpret_cast<uintptr_t>(a) % 16) && !(reinterpret_cast<uintptr_t>(b) % 16);
  if (kind == 1 && (!a || !b || !sink || bytes < 16 || bytes % 16 || !aligned))
    return fail(nullptr, WD_ERR_ARG, "wd_probe: stream needs 16-byte aligned a, b, bytes a positive multiple of 16, a sink");
  if ((kind == 2 || kind == 3) && (!a || !b || !aligned || bytes < 16 * kProbeHandoffBlocks ||
                                   bytes % (16 * kProbeHandoffBlocks) || bytes > (int64_t(1) << 28)))
    return fail(nullptr, WD_ERR_ARG, "wd_probe: hand-off needs 16-byte aligned a, b, bytes a multiple of 4096 up to 256 MiB");
  if ((kind == 4 || kind == 5) && (!a || !b || bytes < 4096 || (reinterpret_cast<uintptr_t>(b) % 8)))
    return fail(nullptr, WD_ERR_ARG, "wd_probe: fence needs a of at least 4096 bytes and an 8-byte aligned b");
  struct Res {   // released on every path
    hipStream_t s = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipGraph_t g = nullptr;
    hipGraphExec_t x = nullptr;
    ~Res() {
      if (s) (void)hipStreamSynchronize(s);
      if (x) (void)hipGraphExecDestroy(x);
      if (g) (void)hipGraphDestroy(g);
      if (e0) (void)hipEventDestroy(e0);
      if (e1) (void)hipEventDestroy(e1);
      if (s) (void)hipStreamDestroy(s);
    }
  } r;
#define PCHK(expr) do { const hipError_t e_ = (expr); if (e_ != hipSuccess) \
    return fail(nullptr, WD_ERR_HIP, std::string("wd_probe: ") + hipGetErrorString(e_)); } while (0)
  PCHK(hipStreamCreateWithFlags(&r.s, hipStreamNonBlocking));
  PCHK(hipEventCreate(&r.e0));
  PCHK(hipEventCreate(&r.e1));
  float ms = 0.f;
  if (kind == 0) {   // a graph of `iters` dependent empty launches, replayed like the step graph
    PCHK(hipStreamBeginCapture(r.s, hipStreamCaptureModeThreadLocal));
    for (int i = 0; i < iters; ++i) k_probe_empty<<<kProbeEmptyBlocks, 256, 0, r.s>>>();
    PCHK(hipStreamEndCapture(r.s, &r.g));
    PCHK(hipGraphInstantiate(&r.x, r.g, nullptr, nullptr, 0));
    PCHK(hipGraphLaunch(r.x, r.s));   // warm-up replay
    PCHK(hipEventRecord(r.e0, r.s));
    PCHK(hipGraphLaunch(r.x, r.s));
    PCHK(hipEventRecord(r.e1, r.s));
  } else if (kind == 2 || kind == 3) {   // a graph of `iters` dependent hand-offs, a -> b -> a ...
    const int slab16 = (int)(bytes / 16 / kProbeHandoffBlocks);
    uint4* bufs[2] = {static_cast<uint4*>(const_cast<void*>(a)), static_cast<uint4*>(const_cast<void*>(b))};
    PCHK(hipStreamBeginCapture(r.s, hipStreamCaptureModeThreadLocal));
    for (int i = 0; i < iters; ++i)
      k_probe_handoff<<<kProbeHandoffBlocks, 256, 0, r.s>>>(bufs[i & 1], bufs[(i + 1) & 1], slab16, kind == 3 ? 1 : 0);
    PCHK(hipStreamEndCapture(r.s, &r.g));
    PCHK(hipGraphInstantiate(&r.x, r.g, nullptr, nullptr, 0));
    PCHK(hipGraphLaunch(r.x, r.s));
    PCHK(hipEventRecord(r.e0, r.s));
    PCHK(hipGraphLaunch(r.x, r.s));
    PCHK(hipEventRecord(r.e1, r.s));
  } else if (kind == 4 || kind == 5) {   // `iters` back-to-back fence reductions over 256 / 1024 blocks
    const int blocks = kind == 4 ? 256 : 1024;
    float* part = static_cast<float*>(const_cast<void*>(a));
    unsigned* ctr = static_cast<unsigned*>(const_cast<void*>(b));
    PCHK(hipMemsetAsync(ctr, 0, 8, r.s));   // (a plain stream, not captured)
    k_probe_fence<<<blocks, 256, 0, r.s>>>(part, ctr);
    PCHK(hipGetLastError());
    PCHK(hipEventRecord(r.e0, r.s));
    for (int i = 0; i < iters; ++i) k_probe_fence<<<blocks, 256, 0, r.s>>>(part, ctr);
    PCHK(hipGetLastError());
    PCHK(hipEventRecord(r.e1, r.s));
  } else {           // `iters` back-to-back reads of a and b
    const int64_t n16 = bytes / 16;
    k_probe_stream<<<kProbeStreamBlocks, 512, 0, r.s>>>(static_cast<const uint4*>(a), static_cast<const uint4*>(b), n16, sink);
    PCHK(hipGetLastError());
    PCHK(hipEventRecord(r.e0, r.s));
    for (int i = 0; i < iters; ++i)
      k_probe_stream<<<kProbeStreamBlocks, 512, 0, r.s>>>(static_cast<const uint4*>(a), static_cast<const uint4*>(b), n16, sink);
    PCHK(hipGetLastError());
    PCHK(hipEventRecord(r.e1, r.s));
  }
  PCHK(hipEventSynchronize(r.e1));
  PCHK(hipEventElapsedTime(&ms, r.e0, r.e1));
#undef PCHK
  *us = 1000.0 * ms / iters;
  return WD_OK;
}

}  // extern "C"
