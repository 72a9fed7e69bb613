/*
 * wd.h -- C ABI of the KV-cached decoder step for AMD Instinct MI355X (gfx950).
 *
 * The library runs one decoder step of a Whisper-style speech-recognition
 * decoder (token embedding + learned position, pre-LN causal self-attention
 * over a K/V cache appended in place, cross-attention over per-window cross
 * K/V, erf-GELU FFN, final LayerNorm, tied-embedding logits and argmax), or of
 * a Qwen3-ASR-style causal LM (RMSNorm, GQA with per-head QK RMSNorm and NeoX
 * RoPE, SwiGLU, tied head).  Every step of the computation runs in the
 * library's own HIP kernels on the device.
 *
 * The calls follow the split the source pages make between weights and
 * per-run state: load the weights once (wavo decoder.rs `Decoder::load`),
 * compute the cross K/V once per audio window (wavo `record_cross`; Whisper
 * tiny (Nest model page) README "Transcribing with caches", entry `listen`),
 * then one call per token (wavo `record_step`; Nest entry `step`;
 * transcribe.cpp qwen3_asr/decoder.h `StepBuildBatched`), with a beam
 * rearrangement of the self caches (mlx-bun whisper.ts
 * `WhisperKvCache.rearrange`) and a prompt prefill (Nest entry `prefill`;
 * decoder.h `PrefillBuild`).
 *
 * Conventions for every call:
 *   - Device pointers are plain HIP device addresses ("dev" below); host
 *     pointers are marked "host".  The caller owns all device memory,
 *     including the workspace; the library never allocates device memory.
 *   - Calls are asynchronous on the stream given to wd_load, except
 *     wd_check (synchronises) and wd_load (returns after its launches are
 *     queued; the source tensors may be freed once the stream has synced).
 *   - A context is bound to one stream and is not thread-safe.
 *   - Errors detectable on the host return a non-zero wd_status at once and
 *     leave the device state unchanged; wd_last_error gives a message.
 *     Errors only visible on the device (a token id outside [0, vocab), a
 *     position outside [0, context), a NaN logit) set a sticky device flag
 *     that wd_check reports as WD_ERR_RANGE; the offending row's cache write
 *     is skipped, so no out-of-bounds access happens.
 *   - No C++ exception crosses this boundary (internal failures return
 *     WD_ERR_INTERNAL).
 */
#ifndef WD_H
#define WD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WD_ABI_VERSION 5
#define WD_MAX_BATCH 64

typedef struct wd_ctx wd_ctx;

typedef enum {
  WD_OK = 0,
  WD_ERR_ARG = 1,      /* bad argument: null pointer, size, dtype, name, shape */
  WD_ERR_STATE = 2,    /* call out of order (e.g. wd_step before wd_cross_kv) */
  WD_ERR_RANGE = 3,    /* device flag: token/position/NaN out of range (wd_check) */
  WD_ERR_HIP = 4,      /* a HIP runtime call failed */
  WD_ERR_OOM = 5,      /* workspace smaller than wd_workspace_bytes */
  WD_ERR_INTERNAL = 6
} wd_status;

typedef enum { WD_F32 = 0, WD_F16 = 1, WD_BF16 = 2 } wd_dtype;
typedef enum { WD_ARCH_WHISPER = 0, WD_ARCH_QWEN3 = 1 } wd_arch;

/* Model and run-size description.
 *   arch        WD_ARCH_WHISPER or WD_ARCH_QWEN3
 *   d_model     residual width d (multiple of 32; Whisper: n_heads * head_dim,
 *               and a multiple of 128 with 16-bit weights, the cross K/V GEMM's
 *               column tile)
 *   n_heads     query heads; head_dim = 64 or 128
 *   n_kv_heads  key/value heads (== n_heads for Whisper; divides n_heads, at
 *               most 8 query heads per kv head)
 *   n_layers, d_ff (multiple of 8), vocab, context (self-cache rows)
 *   max_frames  cross-cache rows per encoder set (Whisper; 0 for Qwen3)
 *   max_batch   rows per step, 1..WD_MAX_BATCH
 *   n_enc       distinct encoder-state sets (Whisper): max_batch (one per
 *               stream) or 1 (one set broadcast to all rows, as for beams;
 *               this also reserves a second self cache for wd_reorder).
 *               Row b reads set b / (max_batch / n_enc), at most 8 rows per
 *               set.  0 for Qwen3.
 *   w_dtype     storage of the weight matrices and encoder states
 *   cache_dtype storage of the self and cross K/V caches
 *   norm_eps    LayerNorm / RMSNorm epsilon; rope_base (Qwen3 only)        */
typedef struct {
  int32_t arch, d_model, n_heads, n_kv_heads, head_dim, n_layers, d_ff, vocab;
  int32_t context, max_frames, max_batch, n_enc;
  int32_t w_dtype, cache_dtype;
  float norm_eps, rope_base;
} wd_config;

/* One named weight tensor in caller device memory, row-major [out, in] for
 * matrices.  Matrices must be in cfg.w_dtype; vectors (biases, norm gains
 * and biases) may be any wd_dtype.  Canonical names (i = layer index):
 *   Whisper: embed [vocab,d]  pos [context,d]  ln_f.g  ln_f.b
 *     dec.i.ln1.g/.b  dec.i.self.q.w/.b  dec.i.self.k.w  dec.i.self.v.w/.b
 *     dec.i.self.o.w/.b  dec.i.ln2.g/.b  dec.i.cross.q.w/.b  dec.i.cross.k.w
 *     dec.i.cross.v.w/.b  dec.i.cross.o.w/.b  dec.i.ln3.g/.b
 *     dec.i.fc1.w [d_ff,d]/.b  dec.i.fc2.w [d,d_ff]/.b
 *   Key projections have no bias (Nest model page, README "The key
 *   projection has no bias"; wavo `Decoder::load` zero-fills the K half of
 *   the fused cross bias): any "*.k.b" name is rejected with WD_ERR_ARG.
 *   Qwen3: embed [vocab,d]  norm_f.g  dec.i.norm1.g  dec.i.self.q.w
 *     [Hq*hd,d]  dec.i.self.k.w/.v.w [Hkv*hd,d]  dec.i.self.o.w [d,Hq*hd]
 *     dec.i.q_norm.g/.k_norm.g [hd]  dec.i.norm2.g  dec.i.mlp.gate.w/.up.w
 *     [d_ff,d]  dec.i.mlp.down.w [d,d_ff]  (no biases).                  */
typedef struct {
  const char* name;
  const void* data;    /* dev */
  int64_t numel;
  int32_t dtype;       /* wd_dtype */
} wd_tensor;

/* Library ABI version (WD_ABI_VERSION). */
int32_t wd_abi_version(void);

/* Bytes of workspace wd_load needs for cfg (repacked weights, self caches,
 * cross caches, step scratch, device error word); 0 if cfg is invalid.  The
 * pages' decoders allocate the same state themselves when they load (wavo
 * decoder.rs `Decoder::load` sizes the self and cross caches from the model
 * dimensions); here the caller allocates it, so the size is a call of its own. */
size_t wd_workspace_bytes(const wd_config* cfg);

/* Validates cfg and the weight list, repacks the weights into `workspace`
 * (dev, 256-byte aligned, ws_bytes >= wd_workspace_bytes(cfg)) on `stream`
 * (a hipStream_t; NULL = the null stream) and returns a host-side context in
 * *out.  Repacking fuses q|k|v (and gate|up) row blocks and the cross [k|v]
 * projection with bias [0 | b_v] (wavo decoder.rs `Decoder::load`).
 * Errors: WD_ERR_ARG (null, invalid dims, missing/unknown/misshaped name,
 * wrong matrix dtype, misaligned workspace), WD_ERR_OOM, WD_ERR_HIP. */
wd_status wd_load(const wd_config* cfg, const wd_tensor* weights, int32_t n_weights,
                  void* workspace, size_t ws_bytes, void* stream, wd_ctx** out);

/* Whisper: computes every layer's cross K/V once per window from encoder
 * states `enc` (dev, [n_enc, frames, d] in w_dtype): K = enc Wk^T, V = enc
 * Wv^T + b_v, rounded to cache_dtype (wavo `record_cross`; mlx-bun
 * `decode` computes crossK/crossV once and reuses them).
 * 1 <= frames <= max_frames.  Errors: ARG, STATE (Qwen3 context). */
wd_status wd_cross_kv(wd_ctx* ctx, const void* enc, int32_t frames);

/* Whisper, a window whose encoder sets have different lengths (batches of audio of
 * different durations, continuous batching): as wd_cross_kv over enc (dev [n_enc, F, d] in
 * w_dtype, F = the largest frames[e]), where set e has frames[e] valid rows (frames: host
 * int32 [n_enc], each in [1, max_frames]) and its rows f >= frames[e] are padding: their
 * K/V are computed but the cross-attention of the rows of set e reads rows 0..frames[e]-1
 * only.  Each row then matches a window of its set alone (Nest `listen` accepts states
 * shorter than 1500 frames).  A later wd_cross_kv returns to one length for all sets.
 * Errors: ARG (null, a frame count out of range), STATE (Qwen3 context), HIP. */
wd_status wd_cross_kv_ragged(wd_ctx* ctx, const void* enc, const int32_t* frames);

/* Audio encoder of a Whisper context (16-bit weights): the step before wd_cross_kv.  It shares
 * d_model, n_heads, head_dim, w_dtype and norm_eps with the decoder and has its own n_layers,
 * d_ff (a multiple of 128) and n_mels.  `frames` mel frames become P = (frames - 1) / 2 + 1
 * states (P <= max_frames): Nest model page, "The convolutional stem" and lib.linnet
 * `encoded`; mlx-bun whisper.ts `encode`:
 *   x = GELU(conv1(mel) + b1)   (kernel 3, stride 1, padding 1, over the mel channels)
 *   x = GELU(conv2(x) + b2) + pos   (kernel 3, stride 2, padding 1; pos the stored table)
 *   per layer: x += attn(LN1(x)) over all P states (no mask, no key bias);
 *              x += W2 GELU(W1 LN2(x) + b1) + b2
 *   out = LN_post(x), in w_dtype.
 * Tensors (i = layer): enc.conv1.w [d, n_mels, 3], enc.conv1.b, enc.conv2.w [d, d, 3],
 * enc.conv2.b, enc.pos [P, d], enc.i.ln1.g/.b, enc.i.attn.q.w/.b, enc.i.attn.k.w,
 * enc.i.attn.v.w/.b, enc.i.attn.o.w/.b, enc.i.ln2.g/.b, enc.i.fc1.w/.b, enc.i.fc2.w/.b,
 * enc.ln_post.g/.b (matrices in w_dtype).  The repacked weights and the encoder's buffers live
 * in a second caller-owned workspace of wd_encoder_workspace_bytes(...) bytes (0: invalid).
 * max_sets bounds the encoder sets per wd_encode call.  Errors: ARG, OOM, HIP. */
size_t wd_encoder_workspace_bytes(const wd_ctx* ctx, int32_t n_mels, int32_t frames, int32_t n_layers,
                                  int32_t d_ff, int32_t max_sets);
wd_status wd_load_encoder(wd_ctx* ctx, int32_t n_mels, int32_t frames, int32_t n_layers, int32_t d_ff,
                          int32_t max_sets, const wd_tensor* weights, int32_t n_weights, void* workspace,
                          size_t ws_bytes);
/* Encoder states of n_sets windows: mel dev [n_sets, frames, n_mels] (positions first) in
 * w_dtype -> enc dev [n_sets, P, d] in w_dtype, ready for wd_cross_kv(ctx, enc, P).
 * Asynchronous on the context's stream.  Errors: ARG, STATE (no encoder loaded), HIP. */
wd_status wd_encode(wd_ctx* ctx, const void* mel, int32_t n_sets, void* enc);
/* wd_encode of all n_enc sets into the encoder workspace, then wd_cross_kv of its P states:
 * one window from mel frames to the cross caches (Nest whisper-tiny model page, README
 * "Transcribing with caches", entry `listen`).  Needs an encoder
 * loaded with max_sets == n_enc.  Errors: ARG, STATE, HIP. */
wd_status wd_listen(wd_ctx* ctx, const void* mel);

/* One decoder step for rows 0..B-1 (1 <= B <= max_batch).
 *   tokens    dev int32 [B]   token id per row (may alias `argmax` for
 *                             on-device greedy decoding)
 *   positions dev int32 [B]   cache row per row; the step writes K/V at that
 *                             row and attends to rows 0..positions[b]
 *                             inclusive (wavo `record_step` attends `pos + 1`
 *                             rows after writing; decoder.h step graph masks
 *                             rows beyond n_past); rows below it must have
 *                             been written by earlier steps or a prefill.
 *   logits    dev float [B, vocab] or NULL (NULL skips the logits write;
 *                             decoder.h `StepBuild::out` returns only the id)
 *   argmax    dev int32 [B]   index of the largest logit, lowest on ties.
 * Whisper requires a prior wd_cross_kv.  Errors: ARG (B, nulls), STATE. */
wd_status wd_step(wd_ctx* ctx, const int32_t* tokens, const int32_t* positions, int32_t B,
                  float* logits, int32_t* argmax);

/* Beam rearrangement: new self-cache row b <- old row beam_idx[b] for cache
 * rows 0..n_rows-1 of every layer (mlx-bun `WhisperKvCache.rearrange`).
 * beam_idx is host int32 [B]; identity returns at once; the broadcast cross
 * cache is not touched.  Needs n_enc == 1 and max_batch > 1 (the spare self
 * cache); the copy goes into the spare cache, which then becomes current.
 * Errors: ARG (index outside [0,B), n_rows outside [0,context]), STATE. */
wd_status wd_reorder(wd_ctx* ctx, const int32_t* beam_idx, int32_t B, int32_t n_rows);

/* Beam candidates on the device, so a beam search need not copy [B, vocab] logits to the
 * host: for each row b < B of `logits` (dev fp32 [B, vocab], as written by wd_step), the W
 * largest logits in descending order (equal values: lower token id first; a NaN counts as
 * -inf) into top_val / top_id (dev [B, W], fp32 / int32), and lse[b] (dev fp32) =
 * log(sum_v exp(logits[b][v])), so log_softmax(v) = logit(v) - lse[b].  Every candidate a
 * width-W beam step keeps (score S_b + log_softmax of row b; mlx-bun `WhisperKvCache.rearrange`
 * consumes the resulting indices) is among the W of its row, so the caller merges W x W
 * candidates instead of B x vocab.  1 <= W <= min(8, vocab).  Asynchronous on the context's
 * stream.  Errors: ARG (null, B or W out of range), HIP. */
wd_status wd_topk(wd_ctx* ctx, const float* logits, int32_t B, int32_t W, float* top_val,
                  int32_t* top_id, float* lse);

/* One whole width-W beam step on the device, with no host round trip: the candidates of
 * rows 0..W-1 of `logits` (dev fp32 [W, vocab], as written by wd_step) as in wd_topk, then
 * the W best of the W x W candidates, then the self-cache rearrangement (mlx-bun
 * `WhisperKvCache.rearrange`).  The selection is the plain width-W beam step with no length
 * penalty and no end token: candidate (b, v) scores scores[b] + logit(b, v) - lse[b] in
 * float64; the W best are kept, best first, equal scores going to the lower b * vocab + v
 * (NaN scores last); with first != 0 (the first generated position, where every beam holds
 * the same prefix) only row 0 is expanded.
 *   scores    dev float64 [W]  in: the beams' scores; out: the kept candidates' scores
 *   beam_idx  dev int32 [W]    out: source beam of each kept candidate
 *   tokens    dev int32 [W]    out: its token, ready as the next wd_step's `tokens`
 *   n_rows    self-cache rows 0..n_rows-1 are copied from beam_idx's rows as by wd_reorder
 *             (0: no copy, as after the last position)
 * 1 <= W <= min(8, max_batch, vocab).  A rearrangement needs n_enc == 1 and max_batch > 1;
 * it always copies (the indices are not known on the host) and makes the spare cache
 * current.  Asynchronous on the context's stream.  Errors: ARG (null, W, first or n_rows out
 * of range), STATE, HIP. */
wd_status wd_beam_step(wd_ctx* ctx, const float* logits, int32_t W, int32_t first, double* scores,
                       int32_t* beam_idx, int32_t* tokens, int32_t n_rows);

/* wd_topk for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation) and hold no decoder context: the same
 * candidates and log-sum-exp from logits dev fp32 [B, ld] (rows of V logits, ld >= V), launched
 * on `stream` (a hipStream_t; NULL = the null stream).  It allocates nothing: its partial lists
 * live in a static device array of the library (147,456 bytes per GPU, held until the process
 * ends), which is why B is limited to WD_TOPK_NOALLOC_MAX_ROWS.  Every call on one GPU shares
 * that array: calls that overlap on one GPU (concurrent streams or threads) race and give
 * undefined results; calls ordered on one stream are safe.  Errors (message from
 * wd_last_error(NULL)): ARG (null pointer, B outside [1, WD_TOPK_NOALLOC_MAX_ROWS], V < 1,
 * ld < V, W outside [1, min(8, V)]), HIP. */
#define WD_TOPK_NOALLOC_MAX_ROWS 64
wd_status wd_topk_noalloc(const float* logits, int32_t B, int32_t V, int64_t ld, int32_t W, float* top_val,
                          int32_t* top_id, float* lse, void* stream);

/* Prompt prefill for rows 0..B-1 at positions 0..T-1 (Nest entry `prefill`;
 * decoder.h `PrefillBuild`).  tokens dev int32 [B, T]; embeds dev [B, A, d]
 * in w_dtype or NULL: rows offset..offset+A-1 take these embeddings instead of
 * the token embeddings (decoder.h "Audio injection").  Fills cache rows
 * 0..T-1 and returns the logits (nullable) and argmax of the last position.
 * Qwen3 with 16-bit weights runs the prompt in chunks of positions through dense
 * GEMMs and a causal prefill attention (decoder.h `PrefillBuildBatched`); Whisper
 * runs one decode step per position.
 * Errors: ARG (T outside [1, context], offset/A outside [0, T]), STATE. */
wd_status wd_prefill(wd_ctx* ctx, const int32_t* tokens, int32_t B, int32_t T,
                     const void* embeds, int32_t A, int32_t offset,
                     float* logits, int32_t* argmax);

/* Run options of a context (wd_set_option / wd_get_option):
 *   WD_OPT_GRAPHS  1 (default): each distinct step (output buffers, row count, current self
 *                  cache, frame count) is captured once into a HIP graph and replayed, since
 *                  positions and tokens live in device memory and the step's launches never
 *                  change (the static-shape step-graph reuse of transcribe.cpp
 *                  qwen3_asr/decoder.h, `build_step_graph` comment); 0: every kernel is
 *                  launched eagerly, on every call.  Both run the same kernels in the same
 *                  order and give bit-identical results.  A context on the null stream never
 *                  captures.
 * Errors: ARG (unknown option, value out of range, null value pointer). */
typedef enum { WD_OPT_GRAPHS = 0 } wd_option;
wd_status wd_set_option(wd_ctx* ctx, int32_t option, int32_t value);
wd_status wd_get_option(wd_ctx* ctx, int32_t option, int32_t* value);

/* Synchronises the stream, reads and clears the sticky device flag:
 * WD_OK, WD_ERR_RANGE (flag was set) or WD_ERR_HIP.  The pages report bad
 * input as a returned error (wavo decoder.rs: `Decoder::load` and the step
 * return `Result`) or a thrown one (mlx-bun whisper.ts); a fault seen only on
 * the device cannot return from an asynchronous launch, so it is collected here. */
wd_status wd_check(wd_ctx* ctx);

/* Message for the last non-OK status of ctx (ctx NULL: of the last failed
 * wd_load on this thread).  Valid until the next call on ctx.  (The text that
 * the pages' `Result` errors and exceptions carry, as a C string.) */
const char* wd_last_error(const wd_ctx* ctx);

/* Waits for the context's stream, then releases the host-side context (captured
 * step graphs, events); never touches caller memory.  After it returns, the caller
 * may free the workspace.  (The pages' decoders drop their state with the object
 * that owns it, wavo `Decoder`; a C caller releases it explicitly.) */
void wd_free(wd_ctx* ctx);

/* --- measurement support (not part of the decoding method) ----------------
 * For benchmarks and profilers only: a decoder never needs these calls, and
 * with recording off (the default) they change nothing on the step path.
 * Records a pair of HIP events on the context's stream around the launches
 * of kernel class `kernel` in layer `layer` (-1: all layers) during later
 * wd_step / wd_cross_kv calls; each such launch is issued `repeats` times back
 * to back between its two events (1..64; every class's launch is idempotent,
 * so results do not change), which spreads the event overhead over the group.
 * wd_profile_read returns the summed elapsed time and the number of kernel
 * launches it covers (synchronising first).  kernel: 0 cross-attention,
 * 1 self-attention, 2 logits + argmax, 3 cross-K/V GEMM, 4 FFN fc1 projection.
 * wd_profile(ctx, -1, 0, 1) disables recording and clears the totals.
 * Errors: ARG (unknown class, repeats out of range).                        */
wd_status wd_profile(wd_ctx* ctx, int32_t kernel, int32_t layer, int32_t repeats);
wd_status wd_profile_read(wd_ctx* ctx, double* total_ms, int64_t* launches);

/* --- machine floors (measurement support, not part of the decoding method) --
 * For benchmarks only: the costs that bound the step's kernels on the device
 * at hand, measured with HIP events on a stream of its own (created and
 * destroyed by the call, default priority; the call synchronises it).
 * kind 0: `iters` dependent launches of an empty kernel of 1280 blocks of 256
 *         threads, captured in one HIP graph and replayed as the decode step's
 *         graph is; *us = time per launch (a, b, bytes, sink unused).
 * kind 1: `iters` back-to-back launches of one kernel that reads `bytes`
 *         bytes of a and `bytes` bytes of b (device buffers, 16-byte aligned,
 *         bytes a positive multiple of 16): 1280 blocks of eight waves, block
 *         i reading the i-th slab of each, with 16-byte nontemporal lane loads
 *         (the large-v3 cross-attention's grid and K/V pattern, without its
 *         arithmetic); *us = time per launch.  sink: device scratch of at
 *         least 1280 floats (practically never written; it keeps the loads).
 * kind 2, 3: a graph of `iters` dependent launches of 256 blocks, each block
 *         reading a slab of bytes / 256 of the previous launch's output (a and
 *         b in turn; 16-byte aligned, bytes a multiple of 4096 up to 256 MiB)
 *         and writing its own: kind 2 the slab its own block index wrote (the
 *         same XCD), kind 3 the next block's (another XCD); *us = time per
 *         launch.  (Both buffers are overwritten.)
 * kind 4, 5: `iters` launches of a kernel of 256 (kind 4) or 1024 (kind 5)
 *         blocks that reduces one value per block inside the kernel: each
 *         block stores its value, fences (__threadfence) and counts itself on
 *         an atomic counter, and the last block adds them up.  a: at least
 *         4096 bytes (bytes >= 4096); b: 8 bytes, 8-byte aligned (counter and
 *         result; zeroed first); *us = time per launch.
 * No device buffer is allocated.  Errors: ARG (kind outside [0, 5], iters
 * outside [1, 100000], null us, or null, misaligned or too small buffers for
 * the kind; wd_last_error(NULL) names it), HIP.                             */
wd_status wd_probe(int32_t kind, const void* a, const void* b, int64_t bytes, int32_t iters, float* sink,
                   double* us);

/* --- test hook (not part of the decoding method) ---------------------------
 * For parity tests only; a decoder never needs it.
 * Device address of one cache block of the current buffer, for checking the
 * caches element by element (in the spirit of named intermediate dumps,
 * transcribe.cpp qwen3_asr/decoder.h `DecoderDumps`).  which: 0 self K,
 * 1 self V ([max_batch][n_kv_heads][context][head_dim]), 2 cross K, 3 cross V
 * ([n_enc][n_heads][max_frames][head_dim]), in cache_dtype.  Errors: ARG.  */
wd_status wd_debug_cache(wd_ctx* ctx, int32_t which, int32_t layer, void** dev_ptr);

#ifdef __cplusplus
}
#endif
#endif /* WD_H */
