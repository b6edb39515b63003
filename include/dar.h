/*
 * dar.h - C ABI of libdar.so: the batch-1 Dual-AR (RQ-Transformer) decode frame
 * on AMD Instinct MI355X (gfx950).
 *
 * What a frame is (tuna-fish README, intro and "Inference estimation"; groxaxo
 * fork README, architecture paragraph; s2-pro-fp8 model card, "Architecture"):
 * one slow-AR token runs through the slow decoder layers against the slow KV
 * cache, the codebook-0 head picks codebook 0 by argmax, then the fast AR runs
 * along depth and emits the residual codebooks one after another, each through
 * the fast layers and a shared head. A frame is 1 + n_res codes. Greedy argmax
 * everywhere (first index among equal maxima).
 *
 * The layer is a pre-RMSNorm decoder block with rotary position embedding and
 * grouped-query attention (pyshine fish-speech tour, "Why You Need This"),
 * SwiGLU FFN, no biases. Weights are bf16, or per-row symmetric
 * float8_e4m3fn with one fp32 scale per output row for every Linear matrix
 * (s2-pro-fp8 model card, "What is this?" and "Quantization Details");
 * tables and norm gains stay bf16 in both modes.
 *
 * Conventions for every entry point:
 *  - Return value: DAR_OK (0) or a negative dar_status. No exceptions cross
 *    the ABI. On DAR_E_HIP the HIP error text is kept in dar_last_error().
 *  - "device" pointers are HIP device memory; "host" pointers are CPU memory.
 *  - Work is stream-ordered on the stream given to dar_create; nothing blocks
 *    the host unless stated. Device outputs are valid after the caller
 *    synchronises that stream.
 *  - Argument checks (null pointers, shapes, alignment, state, capacity)
 *    happen on the host before any HIP call; a failed check changes nothing.
 *  - One dar_ctx is used from one host thread at a time.
 */
#ifndef DAR_H_
#define DAR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DAR_ABI_VERSION 1

typedef enum {
  DAR_OK = 0,
  DAR_E_INVAL = -1,       /* null pointer, bad shape or alignment, id out of range */
  DAR_E_STATE = -2,       /* decode before prefill, use of a destroyed context     */
  DAR_E_CAPACITY = -3,    /* position would reach max_len, batch > max_batch        */
  DAR_E_HIP = -4,         /* a HIP runtime call failed (text in dar_last_error)     */
  DAR_E_WORKSPACE = -5,   /* workspace smaller than dar_workspace_bytes()           */
  DAR_E_UNSUPPORTED = -6  /* valid but not implemented shape or mode                */
} dar_status;

typedef enum {
  DAR_WTYPE_BF16 = 0,           /* every matrix bf16 [rows][cols], row-major                  */
  DAR_WTYPE_FP8_E4M3_ROW = 1,   /* Linear matrices e4m3fn [rows][cols] + fp32 scale [rows]   */
  DAR_WTYPE_INT8_ROW = 2,       /* Linear matrices int8 [rows][cols] + fp32 scale [rows]:
                                   weight-only int8 (the tuna-fish README's int8wo mode),
                                   y_r = scale[r] * sum_j q[r][j] x[j]                       */
  DAR_WTYPE_INT4_G128 = 3       /* Linear matrices int4, two per byte [rows][cols/2] (column
                                   2i in the low nibble of byte i, two's complement), + fp32
                                   scale [rows][cols/128]: weight-only int4 (the tuna-fish
                                   README's int4wo mode), y_r = sum_g scale[r][g] *
                                   sum_{j in group g} q[r][j] x[j]                           */
} dar_wtype;

/* Model geometry and capacity. Checked by dar_workspace_bytes / dar_create.
 * Requirements: head_dim in {64, 128}; n_heads_q a multiple of n_heads_kv;
 * d_model, ffn_dim and n_heads_q*head_dim multiples of 256 and at most 16384;
 * n_res in [0, 15]; n_res > 0 needs n_layers_fast >= 1 and vocab_res >= 1;
 * max_batch in [1, 64] (above 64: DAR_E_UNSUPPORTED). With max_batch > 1 the
 * context decodes that many sequences in lockstep, each with its own prompt
 * length and KV cache; every projection then reads its weights once for all
 * of them (the fish-speech fork README's serving notes: the Dual-AR model
 * takes the batching of ordinary LLM serving). */
typedef struct {
  int32_t n_layers_slow;
  int32_t n_layers_fast;  /* 0 with n_res == 0: slow-AR-only decode (frame = 1 code) */
  int32_t d_model;
  int32_t n_heads_q;
  int32_t n_heads_kv;
  int32_t head_dim;
  int32_t ffn_dim;
  int32_t vocab_c0;       /* codebook-0 entries: rows of the tied table w0           */
  int32_t vocab_res;      /* entries of each residual codebook (fast head rows)      */
  int32_t n_res;          /* residual codebooks per frame                            */
  float rms_eps;
  double rope_base;       /* RoPE angle p * rope_base^(-2i/head_dim), rotate-half    */
  int32_t max_len;        /* slow KV capacity in positions                           */
  int32_t max_batch;
  int32_t wtype;          /* dar_wtype                                               */
} dar_config;

/* One decoder block. All device pointers, 16-byte aligned, caller-owned and
 * unchanged while the context lives. Matrix rows are output features.
 *   attn_norm, ffn_norm : bf16 [d_model]
 *   wqkv : [(n_heads_q + 2*n_heads_kv)*head_dim][d_model]: q rows (head-major),
 *          then k rows, then v rows
 *   wo   : [d_model][n_heads_q*head_dim]
 *   w1, w3 : [ffn_dim][d_model] (gate and up); w2 : [d_model][ffn_dim]
 *   *_scale : fp32 [rows] per-row scales, required for DAR_WTYPE_FP8_E4M3_ROW
 *             and DAR_WTYPE_INT8_ROW; fp32 [rows][cols/128] group scales,
 *             required for DAR_WTYPE_INT4_G128; ignored (may be NULL) for bf16. */
typedef struct {
  const void* attn_norm;
  const void* wqkv;
  const float* wqkv_scale;
  const void* wo;
  const float* wo_scale;
  const void* ffn_norm;
  const void* w1;
  const float* w1_scale;
  const void* w3;
  const float* w3_scale;
  const void* w2;
  const float* w2_scale;
} dar_layer_weights;

/* The whole model. Top-level arrays (slow, fast, fast_emb) are host arrays of
 * device pointers and are copied by dar_create; the device memory they name is
 * referenced, not copied.
 *   w0 : bf16 [vocab_c0][d_model]: slow input table tied to the codebook-0 head
 *   slow_final_norm, fast_final_norm : bf16 [d_model]
 *   fast_emb[k] : bf16 table for codebook k feeding fast step k+1;
 *                 [vocab_c0][d] for k = 0, [vocab_res][d] for k >= 1
 *   fast_head : [vocab_res][d_model] (+ fp32 scales as for a layer matrix when quantised)
 * Fast members are ignored when n_res == 0. */
typedef struct {
  const void* w0;
  const dar_layer_weights* slow;      /* host array [n_layers_slow] */
  const void* slow_final_norm;
  const void* const* fast_emb;        /* host array [n_res]         */
  const dar_layer_weights* fast;      /* host array [n_layers_fast] */
  const void* fast_final_norm;
  const void* fast_head;
  const float* fast_head_scale;
} dar_weights;

typedef struct dar_ctx dar_ctx;

/* Bytes of device workspace the context needs for this config (host only). */
int dar_workspace_bytes(const dar_config* cfg, size_t* bytes_out);

/* Create a decode context. `workspace` is device memory of at least
 * dar_workspace_bytes() bytes, 256-byte aligned, caller-owned, not touched by
 * anyone else while the context lives; it holds the KV caches, activations,
 * the committed-code ring and the RoPE table. `stream` is a hipStream_t (NULL =
 * the null stream). Launches initialisation work on `stream` and waits for it. */
int dar_create(const dar_config* cfg, const dar_weights* weights, void* workspace,
               size_t workspace_bytes, void* stream, dar_ctx** ctx_out);

/* Prefill a prompt and produce frame 0 (the tuna-fish README's
 * "prefill ... decode" run). Positions restart at 0: any previous state is
 * dropped. batch must equal max_batch (DAR_E_CAPACITY above it, DAR_E_INVAL
 * below). tokens: device int32, the batch's prompts one after another
 * (sum of lens_host ids in [0, vocab_c0)); lens_host: host int32 [batch],
 * 1 <= lens_host[b] < max_len (0: DAR_E_INVAL, >= max_len: DAR_E_CAPACITY).
 * Sequence b's frame 0 sits at position lens_host[b] - 1. forced: NULL or device int32
 * [batch][1+n_res], the frame the following steps consume instead of the
 * argmax codes (teacher forcing). codes_out: NULL or device int32
 * [batch][1+n_res] argmax codes of frame 0. logits_out: NULL or device fp32
 * [batch][1+n_res][max(vocab_c0, vocab_res)] (entries past a codebook's size
 * are left untouched). Token ids are not range-checked on the host (they are
 * in device memory); an out-of-range id is clamped to the table and counted
 * with the anomalies dar_nonfinite reports. */
int dar_prefill(dar_ctx* ctx, int32_t batch, const int32_t* tokens, const int32_t* lens_host,
                const int32_t* forced, int32_t* codes_out, float* logits_out);

/* Decode one frame at the next position: the slow AR consumes the previous
 * frame's committed codebook-0 id, then the fast AR emits codebooks 1..n_res.
 * forced / codes_out / logits_out as in dar_prefill. Internally a call commits
 * the frame's codebook 0 (whose slow step ran in the previous call or the
 * prefill), then runs the frame's fast AR and, on a second internal stream at
 * the same time, the slow step and codebook-0 head of the next position. The
 * work is ordered after what is already queued on the ctx's stream, and that
 * stream waits for both internal streams before anything queued later.
 * With a batch every sequence advances one position per call.
 * Errors: DAR_E_STATE before prefill, DAR_E_CAPACITY when the longest
 * sequence's position has reached max_len. */
int dar_decode_frame(dar_ctx* ctx, const int32_t* forced, int32_t* codes_out, float* logits_out);

/* Release the context (graph, events, host state). Waits for the context's
 * stream. Workspace and weights stay with the caller. NULL is a no-op. */
int dar_destroy(dar_ctx* ctx);

/* ---- helpers ---------------------------------------------------------- */

/* Drop the decode state (position 0, needs a new prefill); keeps the graph. */
int dar_reset(dar_ctx* ctx);

/* Next slow position of each sequence, host int32 [max_batch] (host mirror,
 * no synchronisation). */
int dar_position(const dar_ctx* ctx, int32_t* pos_out);

/* Launch each chain of a frame eagerly (0, default) or replay it as a graph
 * captured on first use (1). Same results either way. */
int dar_set_graph(dar_ctx* ctx, int32_t enable);

/* Committed frames [first, first+count) of the ring (index = slow position the
 * frame's codebook 0 was predicted from), copied to device int32
 * [count][max_batch][1+n_res], stream-ordered. */
int dar_codes(dar_ctx* ctx, int32_t first, int32_t count, int32_t* dst);

/* Anomaly counter since create/reset: non-finite logits and out-of-range
 * prompt ids (synchronises the stream). */
int dar_nonfinite(dar_ctx* ctx, int32_t* count_out);

/* Algorithmic bytes of one decode frame that attends over T slow positions:
 * every weight and norm the frame reads (the fast AR once per residual
 * codebook), the scales of quantised weights, the codebook-0 head, T slow KV
 * positions and the fast AR's per-frame KV reads (tuna-fish README,
 * "Inference estimation"). */
int dar_bytes_per_frame(const dar_config* cfg, int32_t T, double* bytes_out);

/* Per-row symmetric e4m3fn quantisation on the device (s2-pro-fp8 model card,
 * "Quantization Details"): scale[r] = max_j |w[r][j]| / 448 in fp32,
 * q[r][j] = e4m3fn(w[r][j] / scale[r]) rounded to nearest even and saturated
 * at 448; a zero row gives scale 0 and codes 0. w: device bf16 [rows][cols];
 * q: device uint8 [rows][cols]; scale: device fp32 [rows]. cols % 16 == 0. */
int dar_quantize_fp8_rows(const void* w, int32_t rows, int32_t cols, void* q, float* scale,
                          void* stream);

/* Per-row symmetric int8 quantisation on the device, for DAR_WTYPE_INT8_ROW.
 * The pages name torchao's int8 weight-only mode but give no formula; the
 * reading taken: scale[r] = max_j |w[r][j]| / 127 in fp32, q[r][j] =
 * round-half-to-even(w[r][j] / scale[r]) (fp32 division) clamped to
 * [-127, 127]; a zero row gives scale 0 and codes 0. w: device bf16
 * [rows][cols]; q: device int8 [rows][cols]; scale: device fp32 [rows].
 * cols % 16 == 0. Stream-ordered. */
int dar_quantize_int8_rows(const void* w, int32_t rows, int32_t cols, void* q, float* scale,
                           void* stream);

/* Group-wise symmetric int4 quantisation on the device, for
 * DAR_WTYPE_INT4_G128. The pages name torchao's int4 weight-only mode but give
 * no formula; the reading taken: groups of 128 consecutive columns of a row,
 * scale[r][g] = max |w| over the group / 7 in fp32, q = round-half-to-even(w /
 * scale) (fp32 division) clamped to [-7, 7]; an all-zero group gives scale 0
 * and codes 0. Codes are packed two per byte, column 2i in the low nibble of
 * byte i. w: device bf16 [rows][cols]; q: device uint8 [rows][cols/2]; scale:
 * device fp32 [rows][cols/128]. cols % 128 == 0. Stream-ordered. */
int dar_quantize_int4_groups(const void* w, int32_t rows, int32_t cols, void* q, float* scale,
                             void* stream);

const char* dar_status_string(int status);
const char* dar_last_error(const dar_ctx* ctx);   /* ctx may be NULL: last create error */

/* ---- paged KV cache and continuous batching ----------------------------
 *
 * The fish-speech fork README's serving notes say the Dual-AR model takes the
 * batching of ordinary LLM serving (requests joining and leaving a running
 * batch, a paged KV cache). A paged context holds max_batch slots. The slow
 * KV cache of every slot comes from one pool of n_pages pages. A page holds
 * page_len consecutive positions of every slow layer and KV head. A slot's
 * block table maps its position p to page (p / page_len), offset
 * (p % page_len). Pages are taken from the pool when a sequence reaches them
 * and returned when it leaves. Workspace:
 *   K, V [n_layers_slow][n_pages][n_heads_kv][page_len][head_dim] bf16
 *   block table int32 [max_batch][ceil(max_len / page_len)]
 * instead of one [max_len] cache per sequence. Page 0 is reserved: a free
 * slot is parked at position 0 of page 0. Its rows still run every frame
 * but change nothing any sequence reads.
 *
 * Frames: dar_seq_add prefills one prompt into a free slot. That slot's
 * frame 0 (at position len - 1) comes out of the next dar_decode_frame.
 * Each dar_decode_frame then returns the next frame of every occupied slot.
 * codes_out / logits_out / forced are [max_batch][...] as for a lockstep
 * batch; rows of free slots are undefined on output and ignored on input.
 * A slot's frames run up to position max_len - 2, because the next frame's
 * slow step is computed ahead. dar_decode_frame returns DAR_E_CAPACITY,
 * and changes nothing, when an occupied slot's frame position has reached
 * max_len - 1 (remove that slot first) or when the pool lacks a page a
 * sequence enters. dar_prefill is refused (DAR_E_STATE). dar_position gives
 * each slot's next frame position, or -1 for a free slot. dar_reset removes
 * every sequence. */
typedef struct {
  int32_t page_len;  /* positions per page: a power of two in [64, 2^20]; at most 64
                        pages per sequence (ceil(max_len / page_len) <= 64) */
  int32_t n_pages;   /* pages in the pool, >= 2 (page 0 is the parking page) */
} dar_paging;

/* Bytes of device workspace of a paged context (host only). Requires
 * max_batch >= 2 (DAR_E_UNSUPPORTED otherwise). */
int dar_workspace_bytes_paged(const dar_config* cfg, const dar_paging* paging, size_t* bytes_out);

/* dar_create for a paged context (arguments and ownership as there). Every
 * slot starts free and all n_pages - 1 usable pages start in the pool. */
int dar_create_paged(const dar_config* cfg, const dar_paging* paging, const dar_weights* weights,
                     void* workspace, size_t workspace_bytes, void* stream, dar_ctx** ctx_out);

/* Prefill a prompt into free slot `slot` (the slow AR over the prompt, on
 * MFMA, and the codebook-0 head on its last position). tokens: device int32
 * [len] with ids in [0, vocab_c0) (clamped otherwise), read on the context's
 * stream. 1 <= len < max_len. Takes ceil(len / page_len) pages from the pool.
 * Errors, all before any change: DAR_E_INVAL (slot out of range, NULL
 * tokens, len < 1), DAR_E_STATE (slot occupied, context not paged),
 * DAR_E_CAPACITY (len >= max_len, too few free pages). Stream-ordered; other
 * slots keep their state and continue with the next dar_decode_frame. */
int dar_seq_add(dar_ctx* ctx, int32_t slot, const int32_t* tokens, int32_t len);

/* Remove the sequence in `slot`. Its pages return to the pool, and the slot
 * is free for dar_seq_add. Work already queued for the slot finishes first
 * (stream order). DAR_E_STATE if the slot is free or the context not paged. */
int dar_seq_remove(dar_ctx* ctx, int32_t slot);

/* Pages left in the pool (host state; 0 for a context that is not paged). */
int dar_pages_free(const dar_ctx* ctx, int32_t* n_free);

/* ---- diagnostics: single operations of the frame, for tests and timing --- */

/* y[m][r] = sum_j W[r][j] * x[m][j] (times scale[r] with fp8 / int8 weights,
 * scale[r][j/128] inside the sum with int4) for m < M, r < rows: the frame's
 * weight-streaming GEMV kernel with no prologue or epilogue. W device
 * [rows][cols] bf16, e4m3fn or int8, or [rows][cols/2] packed int4 (wtype),
 * scale fp32 [rows] ([rows][cols/128] for int4) or NULL for bf16, x device fp32 [M][cols], y device fp32 [M][rows].
 * M in {1, 2}; cols % 256 == 0 and cols <= 16384. */
int dar_op_gemv(int32_t wtype, const void* W, const float* scale, int32_t rows, int32_t cols,
                const float* x, int32_t M, float* y, void* stream);

/* y[m][n] = sum_k x[m][k] * W[n][k] (times scale[n] with fp8 / int8 weights,
 * scale[n][k/128] inside the sum with int4) for m < M, n < N: the prefill's
 * MFMA GEMM, which splits the fp32 inputs into two bf16 parts (hi + lo) and
 * multiplies both. W device [N][K] bf16, e4m3fn or int8, or [N][K/2] packed
 * int4 (wtype), scale fp32 [N] ([N][K/128] for int4) or NULL for bf16, x device fp32 [M][K], y device fp32 [M][N].
 * 1 <= M <= 128; K % 256 == 0 and K <= 16384; N >= 1. Uses its own scratch
 * (allocated per call) and synchronises the stream. */
int dar_op_gemm(int32_t wtype, const void* W, const float* scale, int32_t N, int32_t K, const float* x,
                int32_t M, float* y, void* stream);

/* Bytes of the static device scratch array of dar_op_gemm_noalloc (per GPU). */
#define DAR_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* dar_op_gemm without any allocation, for callers that cannot allocate (code
 * under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
 * Same arguments, shape limits and kernels as dar_op_gemm; the fp32 inputs'
 * hi/lo bf16 halves and the K-split partial sums live in a static device
 * array of DAR_NOALLOC_SCRATCH_BYTES held by each GPU the library runs on
 * until the process ends (the halves take at most 8 MiB; where the rest holds
 * fewer partial sums than dar_op_gemm would use, the product runs with fewer
 * K splits, so sums may round differently). Uses the array of the current
 * device (stream must belong to it). Stream-ordered: no synchronisation and no
 * hipMalloc/hipFree. Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller. Errors:
 * as dar_op_gemm, DAR_E_CAPACITY if the halves exceed the array. */
int dar_op_gemm_noalloc(int32_t wtype, const void* W, const float* scale, int32_t N, int32_t K, const float* x,
                        int32_t M, float* y, void* stream);

/* Decode attention of one layer (the frame's split-K kernel): for query row m
 * at position pos+m, head h, out[m][h] = softmax(q[m][h] . K[kv][0..pos+m] /
 * sqrt(head_dim)) V[kv][0..pos+m] with kv = h / (n_heads_q/n_heads_kv).
 * q device fp32 [M][n_heads_q*head_dim]; K, V device bf16
 * [n_heads_kv][max_len][head_dim]; out device fp32 [M][n_heads_q*head_dim];
 * 0 <= pos, pos + M <= max_len; M in {1, 2}; chunk = positions per split
 * (multiple of 16, 0 = default). One launch: the last split of a (row, KV
 * head) to finish merges the splits. Uses its own scratch (allocated per
 * call). */
int dar_op_attention(const float* q, const void* K, const void* V, int32_t n_heads_q,
                     int32_t n_heads_kv, int32_t head_dim, int32_t max_len, int32_t pos,
                     int32_t M, int32_t chunk, float* out, void* stream);

/* Reference read rate of the GPU: reads `bytes` of device memory at src
 * (16-byte aligned, bytes a multiple of 16) with 16-byte non-temporal loads
 * (as the frame's GEMVs stream their weights, but with no arithmetic) over a
 * grid-stride loop, in each of five launch shapes (384 workgroups x 4 loads
 * in flight per thread, 768 x 2, 256 x 8, 512 x 4, 8192 x 8: HBM on this
 * part streams fastest with about 6-8 MB in flight), each shape one untimed
 * read and then `iters` timed reads back to back, and returns in *ms_out the
 * mean milliseconds per read of the fastest shape (HIP events around the
 * launches; synchronises the stream). sink: device, at least 8 KiB, written
 * only with a value no read produces in practice (it keeps the loads). A
 * measurement aid: the frame's weight rate means most next to it. */
int dar_op_stream_read(const void* src, size_t bytes, int32_t iters, uint32_t* sink, float* ms_out, void* stream);

/* Decode e4m3fn codes with the same conversion the fp8 GEMV uses:
 * out[i] = value of codes[i] (fp32). codes device uint8 [n], out device fp32 [n]. */
int dar_op_fp8_decode(const void* codes, int32_t n, float* out, void* stream);

/* Sampling of the frame's codes instead of the greedy argmax. The pages name
 * top-p and top-k sampling with repetition windows in the generation loop
 * (pyshine fish-speech tour, "Why You Need This") and give no formula; the
 * reading taken, per codebook k of the frame at slow position p of sequence b:
 *   1. every distinct code among codebook k's committed codes of the previous
 *      repetition_window frames (from the sequence's first frame, the one at
 *      its last prompt position) has its logit divided by repetition_penalty
 *      when positive and multiplied by it otherwise;
 *   2. every logit is divided by temperature (fp32);
 *   3. the top_k largest are the candidates (equal values: the lower code);
 *   4. softmax over the candidates, largest first;
 *   5. the candidates are cut after the first one at which the running sum of
 *      probabilities reaches top_p times their total;
 *   6. the code is the first kept candidate whose running sum exceeds
 *      u * (kept total), u = uniforms[(p * max_batch + b) * (1 + n_res) + k].
 * The draws are inputs: uniforms is a caller-owned device fp32 array
 * [max_len][max_batch][1 + n_res] of values in [0, 1), read while the
 * context samples. NaN logits count as -infinity. Limits: 1 <= top_k <= 256,
 * 0 <= repetition_window <= 64, vocabularies up to 8192 (DAR_E_UNSUPPORTED
 * beyond); temperature > 0, top_p in (0, 1], repetition_penalty >= 1
 * (DAR_E_INVAL otherwise). */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p;
  float repetition_penalty;
  int32_t repetition_window;
  const float* uniforms;
} dar_sampling;

/* Switch the context to sampling with these parameters (copied), or back to
 * greedy argmax with NULL. The codes returned and committed from then on are
 * the sampled ones (forced codes still replace the committed ones). Waits for
 * the context's frames in flight; a captured graph is captured again. */
int dar_set_sampling(dar_ctx* ctx, const dar_sampling* sampling);

/* The frame's sampling step alone: codes_out[r] = the code drawn from logits
 * row r with u = sampling->uniforms[r] and window codes history[r][0..n_hist)
 * (entries outside [0, V) ignored; the window length field is not used).
 * logits device fp32 [rows][V], uniforms device fp32 [rows], history device
 * int32 [rows][n_hist] (may be NULL when n_hist == 0), codes_out device int32
 * [rows]. Synchronises the stream. */
int dar_op_sample(const float* logits, int32_t rows, int32_t V, const dar_sampling* sampling,
                  const int32_t* history, int32_t n_hist, int32_t* codes_out, void* stream);

/* Time one kind of launch live: from the next decode call on, every one-row
 * launch of `kind` (the kinds of dar_profile_frame; -1 = off) is timed by a
 * HIP event pair on the stream it runs on, which a single-kernel launch
 * stamps at the kernel's own start and end (hipExtLaunchKernel; a many-row
 * stage of a batched context: recorded around its launches). Eager launches
 * only, not graph replay. dar_kind_time synchronises, returns the summed milliseconds and the
 * number of timed launches since dar_time_kind or the last read, and resets. */
int dar_time_kind(dar_ctx* ctx, int32_t kind);
int dar_kind_time(dar_ctx* ctx, double* ms_total, int32_t* launches);

/* Run one frame eagerly on one stream with a HIP event pair timing every
 * launch (stamped as for dar_time_kind) and report per-launch milliseconds, kind and layer tag (host arrays
 * of capacity cap; *n_out is the number of launches). Kinds: 0 qkv,
 * 1 attention, 2 wo, 3 w13, 4 w2, 5 codebook head, 6 other. Layer tags: slow
 * layer l is l; fast layer l of pass k is 1000k + l. The frame advances the
 * state like dar_decode_frame(ctx, NULL, NULL, NULL). Synchronises. A paged
 * context is refused (DAR_E_STATE): its frames take pages in
 * dar_decode_frame, so time them with dar_time_kind. */
int dar_profile_frame(dar_ctx* ctx, int32_t cap, float* ms_out, int32_t* kind_out,
                      int32_t* layer_out, int32_t* n_out);

#ifdef __cplusplus
}
#endif

#endif /* DAR_H_ */
