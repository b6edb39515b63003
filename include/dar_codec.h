/*
 * dar_codec.h - C ABI of libdar.so, part 2: RVQ codec decode (codes -> audio)
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed (tuna-fish README, intro: a DAC-style RVQ audio codec,
 * timed in its "Audio tokenizer speedtest" on 44.1 kHz mono clips; pyshine
 * fish-speech tour, "Why You Need This": a modified DAC, convolutional, with a
 * residual vector quantiser of ten stacked codebooks at roughly 21 Hz, the
 * first the coarsest and each further one quantising the residual):
 *
 *   z[t]   = sum_k table_k[code[t][k]]                  latent frame t (width D)
 *   x      = conv7(z)                                    D -> C0 channels
 *   block i (stride s_i, C_i -> C_i / 2 channels):
 *     x    = convT(Snake(x))                             kernel 2 s_i, padding s_i / 2,
 *                                                        T rows -> T s_i rows
 *     x    = x + conv1(Snake(conv7_dil(Snake(x))))       dil = 1, 3, 9 (residual units)
 *   audio  = tanh(conv7(Snake(x)))                       -> 1 channel
 *
 * with Snake(x) = x + sin(alpha x)^2 / alpha per channel and zero "same"
 * padding. The pages give no layer widths; the published DAC decoder for
 * 44.1 kHz audio gives them (D 1024, C0 1536, three residual units with
 * dilations 1, 3, 9, 7-tap convolutions), with the strides (8, 8, 8, 4) so that
 * one latent frame becomes 2048 samples (44100 / 2048 = 21.5 Hz).
 *
 * Precision: weights, tables, biases and alphas are bf16; every convolution
 * multiplies bf16 inputs (its input activation, after Snake, rounded to bf16
 * nearest even) on MFMA with fp32 sums; the residual stream, biases, Snake and
 * tanh are fp32 (Snake's sine from the hardware sine after reduction by whole
 * turns: within 4e-7 of sin for |alpha x| <= 1000).
 *
 * Conventions as in dar.h: DAR_OK or a negative dar_status; argument checks on
 * the host before any HIP call; work stream-ordered on the context's stream;
 * one context per host thread at a time.
 */
#ifndef DAR_CODEC_H_
#define DAR_CODEC_H_

#include <stddef.h>
#include <stdint.h>

#include "dar.h" /* dar_status */

#ifdef __cplusplus
extern "C" {
#endif

#define DAR_CODEC_MAX_BLOCKS 8
#define DAR_CODEC_MAX_UNITS 4

/* Geometry. Requirements (DAR_E_INVAL otherwise): n_codebooks in [1, 32];
 * codebook_size >= 1; latent_dim and channels multiples of 32, at most 8192;
 * n_blocks in [1, 8] with channels >> n_blocks >= 32 and a multiple of 32;
 * every rate even, in [2, 16]; n_units in [1, 4], dilations >= 1; kernel_size
 * odd, in [1, 7], with (kernel_size - 1) / 2 * dilation <= 32;
 * max_frames >= 1 with max_frames * prod(rates) * channels < 2^31. */
typedef struct {
  int32_t n_codebooks;
  int32_t codebook_size;
  int32_t latent_dim;
  int32_t channels;          /* width after the input convolution; block i halves it */
  int32_t n_blocks;
  int32_t rates[DAR_CODEC_MAX_BLOCKS];
  int32_t n_units;           /* residual units per block */
  int32_t dilations[DAR_CODEC_MAX_UNITS];
  int32_t kernel_size;       /* taps of the input, residual and output convolutions */
  int32_t max_frames;        /* capacity: latent frames per decode call */
} dar_codec_config;

/* One residual unit: Snake(alpha1), conv w1 [C][C][kernel_size] + b1 [C],
 * Snake(alpha2), conv w2 [C][C][1] + b2 [C]. */
typedef struct {
  const void* alpha1;
  const void* w1;
  const void* b1;
  const void* alpha2;
  const void* w2;
  const void* b2;
} dar_codec_unit;

/* One upsampling block: Snake(alpha) over its C input channels, transposed
 * convolution up_w [C][C/2][2 rate] (PyTorch ConvTranspose1d layout) + up_b
 * [C/2], then its residual units at C/2 channels. */
typedef struct {
  const void* alpha;
  const void* up_w;
  const void* up_b;
  dar_codec_unit units[DAR_CODEC_MAX_UNITS];
} dar_codec_block;

/* Every pointer is device memory holding bf16 values, 16-byte aligned,
 * caller-owned and unchanged while the context lives. Convolution weights in
 * the PyTorch Conv1d layout [Cout][Cin][taps].
 *   tables[k] : [codebook_size][latent_dim]           (host array of n_codebooks pointers)
 *   in_w [channels][latent_dim][kernel_size], in_b [channels]
 *   blocks[i]                                           (host array of n_blocks)
 *   out_alpha [C_last], out_w [1][C_last][kernel_size], out_b [1]
 * Host arrays are copied by dar_codec_create; the context keeps its own
 * re-laid copy of the convolution weights in its workspace (the tables are
 * read in place). */
typedef struct {
  const void* const* tables;
  const void* in_w;
  const void* in_b;
  const dar_codec_block* blocks;
  const void* out_alpha;
  const void* out_w;
  const void* out_b;
} dar_codec_weights;

typedef struct dar_codec dar_codec;

/* Device workspace bytes for this geometry (host only): the re-laid weights
 * and the activations of max_frames frames. */
int dar_codec_workspace_bytes(const dar_codec_config* cfg, size_t* bytes_out);

/* Create a codec context over `workspace` (device, >= dar_codec_workspace_bytes,
 * 256-byte aligned, caller-owned). Re-lays the convolution weights into the
 * workspace on `stream` (a hipStream_t, NULL = null stream) and waits for it. */
int dar_codec_create(const dar_codec_config* cfg, const dar_codec_weights* weights, void* workspace,
                     size_t workspace_bytes, void* stream, dar_codec** out);

/* Decode `frames` latent frames. codes: device int32 [frames][n_codebooks]
 * (frame-major, the Dual-AR model's frame layout; an id outside
 * [0, codebook_size) is clamped and counted, see dar_codec_anomalies).
 * audio: device fp32 [frames * prod(rates)] samples in (-1, 1).
 * 1 <= frames <= max_frames (DAR_E_CAPACITY above). Stream-ordered. */
int dar_codec_decode(dar_codec* ctx, const int32_t* codes, int32_t frames, float* audio);

/* Out-of-range codes seen since create (synchronises the stream). */
int dar_codec_anomalies(dar_codec* ctx, int32_t* count_out);

/* Time each launch of one decode call with HIP event pairs stamped by the
 * launch itself (its kernel's start and end); one stream, synchronises.
 * ms_out, tag_out: host arrays of capacity cap; *n_out launches. Tags: 0 RVQ
 * sum, 1 input conv, 2 transposed conv, 3 residual 7-tap conv, 4 residual
 * 1-tap conv, 5 output conv, 6 residual unit in one launch (blocks of width
 * 32, 64, 96 or 128 run each unit so, the others as tags 3 and 4);
 * block i adds 16 i to tags 2, 3, 4 and 6. */
int dar_codec_profile(dar_codec* ctx, const int32_t* codes, int32_t frames, float* audio, int32_t cap,
                      float* ms_out, int32_t* tag_out, int32_t* n_out);

/* Release the context (waits for its stream). NULL is a no-op. */
int dar_codec_destroy(dar_codec* ctx);

/* Text of the last error of ctx, or of the last failed create, workspace or
 * op call on this thread when ctx is NULL. */
const char* dar_codec_last_error(const dar_codec* ctx);

/* Diagnostic: one convolution of the decoder on its own (the same kernel and
 * launch choice a decode uses). x: device [T][Cin], fp32 (x_bf16 == 0, with
 * Snake(alpha) applied on load when alpha is non-NULL) or bf16 (x_bf16 == 1,
 * used as is); w: device bf16 in the PyTorch layout, [Cout][Cin][taps] for a
 * convolution (stride == 0; same padding, dilation) or [Cin][Cout][2 stride]
 * for a transposed convolution (stride even, padding stride / 2, output
 * T * stride rows); b: device bf16 [Cout]; y: device fp32 [rows][Cout], plus
 * res (device fp32, same shape, may alias y) when non-NULL; tanh_out applies
 * tanh last (fp32 input only). Cin, Cout multiples of 32. Cout == 1 is the
 * output kernel: odd taps <= 7, dilation 1, tanh_out set, no res, and either
 * fp32 input with alpha or bf16 input (the Snake'd operand) without it.
 * Allocates its re-laid weights per call and synchronises the stream. */
int dar_codec_op_conv(const void* x, int32_t x_bf16, const void* alpha, int32_t T, int32_t Cin, int32_t Cout,
                      const void* w, const void* b, int32_t taps, int32_t dilation, int32_t stride,
                      const float* res, int32_t tanh_out, float* y, void* stream);

/* Diagnostic: one residual unit on its own, y = x + conv1(Snake(conv_taps,dil(
 * Snake(x, alpha1)) + b1, alpha2)) + b2, with the hidden activation rounded
 * to bf16 (as in a decode). x, y: device fp32 [T][C]; alpha1, b1, alpha2, b2:
 * device bf16 [C]; w1: bf16 [C][C][taps]; w2: bf16 [C][C][1] (PyTorch
 * layouts). fused == 1 runs the one-launch kernel a decode uses at this width
 * (C in {32, 64, 96, 128}, y != x; DAR_E_INVAL otherwise); fused == 0
 * runs the two convolutions as two launches through a bf16 hidden buffer
 * (any C multiple of 32, up to 8192; y may alias x). Both give the same
 * values bit for bit. Allocates per call and synchronises the stream. */
int dar_codec_op_resunit(const float* x, int32_t T, int32_t C, const void* alpha1, const void* w1, const void* b1,
                         int32_t taps, int32_t dilation, const void* alpha2, const void* w2, const void* b2,
                         int32_t fused, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DAR_CODEC_H_ */
