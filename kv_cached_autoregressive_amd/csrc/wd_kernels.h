// Host-side launchers of the decoder-step kernels.  Every launcher checks the
// shapes its kernel assumes before launching and returns hipErrorInvalidValue
// instead of launching when they do not hold.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wd {

enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };  // same values as wd_dtype

// sticky device error bits (reported by wd_check)
enum : unsigned { ERR_TOKEN = 1u, ERR_POS = 2u, ERR_NAN = 4u };

// ---- repack / utility -------------------------------------------------------------------
// dst[(r*row_mul + row_add) * cols + c] = convert(src[r*cols + c]) for r < rows.
hipError_t launch_copy_rows(const void* src, int src_dtype, void* dst, int dst_dtype,
                            int64_t rows, int64_t cols, int64_t row_mul, int64_t row_add,
                            hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);
// Copies one call's inputs into fixed buffers (tokens with stride, positions or a constant,
// and optionally B override rows) so that a captured step reads fixed addresses.
hipError_t launch_stage(const int32_t* tok, int tok_stride, const int32_t* pos, int pos_const, int32_t* tok_out,
                        int32_t* pos_out, int B, const void* rows, int64_t src_stride_bytes, void* rows_out,
                        int64_t row_bytes, hipStream_t s);

// ---- embedding ---------------------------------------------------------------------------
// x[b] = ov ? ov[b*ov_stride ..] : E[tok[b*tok_stride]] + (P ? P[pos[b]] : 0); validates ranges.
// E_frag: E is stored in fragment layout (rows padded to 16) rather than row-major.
hipError_t launch_embed(float* x, const void* E, const void* P, int w_dtype, const int32_t* tok,
                        int tok_stride, const int32_t* pos, const void* ov, int64_t ov_stride,
                        int B, int d, int V, int ctx, unsigned* err, bool E_frag, hipStream_t s);

// ---- row norm: LayerNorm (b != nullptr) or RMSNorm (b == nullptr) ----------------------
hipError_t launch_norm(const float* x, float* y, const float* g, const float* b, int B, int d,
                       float eps, hipStream_t s);

// ---- skinny GEMM (GEMV over B rows) with fused epilogues -----------------------------------
enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_GELU = 2, EPI_QKV = 3, EPI_LOGITS = 4 };
enum YMode : int { Y_PLAIN = 0, Y_SWIGLU = 1 };

struct GemvParams {
  const void* W; int w_dtype; int N; int K;   // W [N, K] row-major
  const float* Y; int ldy; int B; int ymode;  // Y [B, ldy]; SWIGLU reads silu(Y[:,k]) * Y[:,K+k]
  int epi;
  const float* bias;                          // [N] or null
  float* out; int ldo; float scale;           // STORE/GELU/RESID target; STORE multiplies by scale
  // EPI_QKV (Whisper): rows [0,d) -> q (out, times scale), [d,2d) -> K cache, [2d,3d) -> V cache
  int d; int H; int hd; int ctx; const int32_t* pos;
  void* Kc; void* Vc; int cache_dtype; int64_t kv_bstride;
  // EPI_LOGITS: out = logits [B, ldo] or null; per-block argmax keys amax[blockIdx.x * ldp + b]
  unsigned long long* amax; int ldp;
  unsigned* err;
};
// Returns the number of blocks along N (the number of argmax partials per row).
int gemv_blocks(int N, int B);
hipError_t launch_gemv(const GemvParams& p, hipStream_t s);
hipError_t launch_argmax_final(const unsigned long long* amax, int nparts, int ldp, int B,
                               int32_t* out, hipStream_t s);
// Per row b < B of logits [B, ld]: the W (<= 8) largest of the first V values, descending
// (ties: lower index first; NaN as -inf), into top_val / top_id [B, W], and lse[b] =
// log(sum_v exp(logits[b][v])).  scratch: topk_scratch_bytes(B, V) bytes of device memory.
size_t topk_scratch_bytes(int B, int V);
hipError_t launch_topk_lse(const float* logits, int B, int V, int64_t ld, int W, float* top_val, int32_t* top_id,
                           float* lse, void* scratch, hipStream_t s);

// ---- MFMA skinny GEMM (16-bit weights) ------------------------------------------------------
// Weights are stored in MFMA fragment order ("fragment layout"): for W [N, K] with N padded
// to 16 and K % 32 == 0, element (n, k) sits at frag_offset(n, k, K).  One 16 x 32 tile is
// 1 KB contiguous, in the order lane l holds row l%16, columns 8*(l/16)..+7 of the tile.
// Activations feeding the MFMA GEMM use the same layout over [B_pad, K] and are split
// into two 16-bit parts, hi = round(y), lo = round(y - hi), so the products keep ~16
// mantissa bits of the fp32 activation.
__host__ __device__ inline int64_t frag_offset(int64_t r, int64_t k, int64_t K) {
  return ((((r >> 4) * (K >> 5) + (k >> 5)) * 64 + ((r & 15) | (((k >> 3) & 3) << 4))) << 3) + (k & 7);
}

enum Epi2 : int { EPI_GELU_SPLIT = 5, EPI_SWIGLU_SPLIT = 6 };

struct MGemvParams {
  const void* W; int w_dtype; int N; int K;   // W in fragment layout, rows padded to 16
  const void* Yhi; const void* Ylo; int B;    // activations [B_pad, K] fragment layout
  int epi;
  const float* bias;
  float* out; int ldo; float scale;           // STORE / RESID / QKV(q) / LOGITS targets
  int d; int H; int hd; int ctx; const int32_t* pos;   // EPI_QKV (Whisper)
  void* Kc; void* Vc; int cache_dtype; int64_t kv_bstride;
  unsigned long long* amax; int ldp;          // EPI_LOGITS partial keys [blocks][ldp]
  void* yo_hi; void* yo_lo;                   // GELU_SPLIT / SWIGLU_SPLIT output [B_pad, N or N/2]
  unsigned* err;
  float* part; int64_t part_cap;              // K-group partials [G][B][N] fp32 (split-K launches)
  int part_G;                                 // set by the launcher: K groups of this launch
};
// Number of argmax partials (blocks) a logits launch writes: upper bound over K, and exact for K.
int mgemv_blocks(int N, int B);
int mgemv_blocks_k(int N, int K, int B);
// K groups a launch of this shape splits into (1: the epilogue runs in the GEMM).  With G > 1
// the launch writes fp32 partials part[g][b][n] (no bias) and the caller finishes them: a
// residual add is folded into the next norm (launch_norm_split with part), any other
// epilogue runs in launch_mgemv_finish.
int mgemv_groups(int N, int K, int B, int epi);
hipError_t launch_mgemv(const MGemvParams& p, hipStream_t s);
// Sum of the G partials of each output in order g = 0..G-1, then the launch's epilogue.
hipError_t launch_mgemv_finish(const MGemvParams& p, int G, hipStream_t s);

// Row norm writing the split fragment layout (MFMA consumers).
// With part != null, first x += pbias + sum_g part[g][b][:] (G partial slabs of a split-K
// residual projection, added in order g = 0..G-1) and x is written back.
hipError_t launch_norm_split(float* x, void* y_hi, void* y_lo, int act_dtype, const float* g,
                             const float* b, int B, int d, float eps, hipStream_t s,
                             const float* part = nullptr, int G = 0, const float* pbias = nullptr);
// Fragment-layout repack of a [rows, K] matrix into fused row blocks:
// fused row of source row r = (r / 16) * blk_mul * 16 + blk_add * 16 + r % 16.
hipError_t launch_pack_frag(const void* src, int src_dtype, void* dst, int dst_dtype, int64_t rows,
                            int64_t K, int64_t blk_mul, int64_t blk_add, hipStream_t s);

// ---- attention over a K/V cache --------------------------------------------------------------
struct AttnParams {
  const float* q; int q_ld;                   // q [B, q_ld]; head h at h*hd, pre-scaled
  const void* K; const void* V; int cache_dtype;
  int64_t kvb_stride; int rows_cap;           // cache [n_kvb][Hkv][rows_cap][hd]
  const int32_t* pos; int n_rows_fixed;       // pos: rows 0..pos[b]; else n_rows_fixed rows
  const int32_t* rows_kvb;                    // (no pos) rows of each KV set, at most n_rows_fixed
  int B; int Hq; int Hkv; int hd; int q_per_kvb;
  int split_rows; int n_splits;
  int nw;                                     // waves per block: 4 or 8
  float* out; int out_ld;                     // [B, out_ld] (head h at h*hd), or:
  void* o_hi; void* o_lo; int o_dtype;        // split fragment layout [B_pad, Hq*hd] if set
  float* part;                                // [B*Hq][n_splits][hd+2] when n_splits > 1
  // q from the fp32 partials of a split-K projection (then q is ignored):
  //   q[b][h*hd + c] = (sum_g qpart[g][b][q_off + h*hd + c] + qbias[h*hd + c]) * qscale,
  // slabs of B rows x qpart_ld columns, g < qG <= 16
  const float* qpart; int qG; int qpart_ld; int q_off; const float* qbias; float qscale;
  // self-attention append from the same partials (Whisper q|k|v): the block whose split holds
  // row pos[b] writes cache row pos[b] of its head, k = sum_g qpart[..k_off..] (no bias) and
  // v = sum_g qpart[..v_off..] + vbias, rounded to the cache dtype, before reading any row
  int k_off; int v_off; const float* vbias; bool append;
  // Qwen3 (rope): q and the appended k first go through the per-head RMSNorm (gains qn / kn
  // [hd], eps) and the NeoX rotation of the pairs (i, i + hd/2) by the angle pos * base^(-2i/hd),
  // its cos and sin read from rope_cs (launch_rope_table, rows_cap positions); v is appended as
  // summed.  GQA allowed.
  bool rope; const float* qn; const float* kn; float eps; const float* rope_cs;
};
// main kernel (writes o directly when n_splits == 1, else partials) ...
hipError_t launch_attention(const AttnParams& p, hipStream_t s);
// ... and the split combine (no-op when n_splits == 1)
hipError_t launch_attention_combine(const AttnParams& p, hipStream_t s);

// ---- Qwen3: per-head q/k RMSNorm + NeoX RoPE, K/V append -------------------------------------
// With part != null the q|k|v row is the in-order sum of G fp32 partial slabs
// part[g][b][:] ([G][B][(Hq + 2 Hkv) hd]) instead of qkv.  Row b appends to the cache of
// stream b / rows_per_stream at position pos[b] (rows_per_stream > 1: prefill chunks).
// The rotation angles come from rope_cs (launch_rope_table over ctx positions).
hipError_t launch_qk_rope_append(const float* qkv, int B, int Hq, int Hkv, int hd,
                                 const int32_t* pos, int ctx, const float* qn, const float* kn,
                                 float eps, const float* rope_cs, float qscale, float* q_out, void* Kc,
                                 void* Vc, int cache_dtype, int64_t kv_bstride, hipStream_t s,
                                 const float* part = nullptr, int G = 0, int rows_per_stream = 1);

// NeoX RoPE table: cs[p][i] = cos(p * base^(-2i/hd)), then sn[p][i] = sin(...) at cs + ctx * hd/2,
// for p < ctx, i < hd/2 (angles in double, rounded to float).
hipError_t launch_rope_table(float* cs, int ctx, int hd, float base, hipStream_t s);

// ---- batched prefill (Qwen3) --------------------------------------------------------------------
// Chunk rows r = b * C + j (stream b, position t0 + j, j < Cn): x[r] = the audio row or the
// token's embedding (E in fragment layout), pos[r] = t0 + j (-1 and a zero row for j >= Cn).
hipError_t launch_pf_embed(float* x, int32_t* pos, const void* E, int w_dtype, const int32_t* tokens, int T,
                           const void* emb, int A, int offset, int t0, int B, int C, int Cn, int d, int V,
                           unsigned* err, hipStream_t s);
// Dense GEMM over fragment-layout operands: C[R, N] = (Ahi + Alo)[R, K] . W[N, K]^T.
enum FgEpi : int { FG_STORE = 0, FG_RESID = 1, FG_SWIGLU = 2, FG_GELU = 3, FG_GELU_SPLIT = 4, FG_ENC_QKV = 5 };
struct FgParams {
  const void* W; int w_dtype; int N; int K;   // W fragment layout (N % 128 == 0)
  const void* Ahi; const void* Alo; int R;    // A fragment layout [R rounded up to 128, K]
  int epi;
  float* out; int ldo;                        // STORE: out = C; RESID: out += C (fp32 [R, ldo])
                                              // GELU: out = GELU(C) + pos[r % pos_rows] (pos optional)
  void* Ohi; void* Olo;                       // SWIGLU: silu(gate) * up, fragment layout [R_pad, N/2]
                                              // GELU_SPLIT: GELU(C), fragment layout [R_pad, N]
  const float* bias;                          // optional [N], added to C first (STORE, RESID, GELU*)
  const float* pos; int pos_rows;             // GELU: optional [pos_rows, N] added after the GELU
  // ENC_QKV (the encoder's fused q|k|v, N = 3 d, d = kv_H kv_hd, rows r = set * kv_P + frame):
  // columns < d -> out[r][c] = (C + bias[c]) * scale (fp32 [R, d]); the next d -> K, the last d
  // (+ bias2[c]) -> V, both [set][head][frame][hd] in the weight dtype
  const float* bias2; float scale; void* Kc; void* Vc; int kv_P; int kv_H; int kv_hd;
};
hipError_t launch_fgemm(const FgParams& p, hipStream_t s);
// Causal attention of a chunk's rows over cache rows 0..t of their stream (GQA).
struct PfAttnParams {
  const float* q;                             // [B*C, Hq*hd] scaled, normed, rotated
  const void* K; const void* V; int cache_dtype; int64_t kv_bstride; int ctx;   // [B][Hkv][ctx][hd]
  int B; int C; int Cn; int t0; int Hq; int Hkv; int hd;
  void* o_hi; void* o_lo; int o_dtype;        // split fragment layout [B*C rounded up, Hq*hd]
  bool full;                                  // every query attends to all rows 0..t0+Cn-1 (no mask)
};
hipError_t launch_pf_attn(const PfAttnParams& p, hipStream_t s);

// ---- audio encoder (stem and layer glue) ------------------------------------------------------
// Windows of a kernel-3, pad-1 convolution as the split A operand of the dense GEMM: row
// r = b * Lout + o, column c * 3 + k = x[b][o * stride + k - 1][c] (0 outside [0, L)), columns
// >= 3 C zero; x [nb, L, C] in x_dtype (f32, f16 or bf16); A fragment layout [rows, Kp].
hipError_t launch_conv_windows(const void* x, int x_dtype, int nb, int L, int C, int stride, int Lout, int Kp,
                               void* a_hi, void* a_lo, int a_dtype, hipStream_t s);
// Row-major [rows, Ks] (any wd dtype) -> fragment layout [rows, Kp] (Kp >= Ks, columns >= Ks zero).
hipError_t launch_pack_pad(const void* src, int src_dtype, int64_t rows, int Ks, void* dst, int dst_dtype, int Kp,
                           hipStream_t s);
// fp32 [n] -> dtype [n]
hipError_t launch_cast(const float* x, void* y, int y_dtype, int64_t n, hipStream_t s);

// ---- beam reorder: cache-row gather -----------------------------------------------------------
struct BeamIdx { int32_t v[64]; };
hipError_t launch_reorder(const void* src, void* dst, int elt_bytes, const BeamIdx& idx, int B,
                          int Bmax, int H, int ctx, int hd, int n_rows, int n_blocks,
                          hipStream_t s);
// The same copy with the beam indices read from device memory (idx dev int32 [B], each in
// [0, B); an index outside that range is clamped into it).
hipError_t launch_reorder_dev(const void* src, void* dst, int elt_bytes, const int32_t* idx, int B,
                              int Bmax, int H, int ctx, int hd, int n_rows, int n_blocks, hipStream_t s);
// One width-W beam selection from the per-row candidates of launch_topk_lse (top_val, top_id
// [rows, W], lse [rows]): candidate (b, k) scores scores[b] + (top_val[b][k] - lse[b]) in
// float64, the W best kept (score descending, then flat index b * V + id ascending; NaN
// scores last), written as beam_idx[i] = b, tokens[i] = id, scores[i] = its score.  rows is
// 1 at the first generated position (every beam holds the same prefix), else W.  W <= 8.
hipError_t launch_beam_merge(const float* top_val, const int32_t* top_id, const float* lse, double* scores,
                             int32_t* beam_idx, int32_t* tokens, int W, int rows, int V, hipStream_t s);

// ---- cross K/V projection (dense GEMM) with cache scatter ------------------------------------
// C[m, n] = sum_k X[m,k] W[n,k] (+ bias[n]); m = e*frames + f; n < d -> K cache, else V cache;
// caches [n_enc][H][max_frames][hd] in cache_dtype.  fp32: X and W row-major.  16-bit: X in
// fragment order (launch_pack_rows, rows padded to a multiple of 256), W in fragment order,
// hd == 64, d % 128 == 0, 16-bit caches.
hipError_t launch_cross_kv_gemm(const void* X, const void* W, const float* bias, int w_dtype,
                                int M, int d, int frames, int max_frames, int H, int hd,
                                void* Kc, void* Vc, int cache_dtype, hipStream_t s);
// Row-major [M, d] 16-bit rows -> fragment order (the cross-K/V GEMM's X operand).
hipError_t launch_pack_rows(const void* X, int w_dtype, void* Xf, int64_t M, int d, hipStream_t s);

}  // namespace wd
