// Internal interface between the runtime (dar_runtime.hip) and the gfx950
// kernels (dar_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dar {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kMaxM = 2;           // input rows per GEMV launch (fast pass 1 runs two)
constexpr int kAttnChunkDefault = 64;
constexpr int kPrefillRows = 128;  // prompt positions per prefill block (GEMM rows)

// W_FP8, W_INT8: one byte per weight + fp32 row scales; W_INT4: two weights per
// byte + fp32 scales per (row, 128-column group)
enum WType : int { W_BF16 = 0, W_FP8 = 1, W_INT8 = 2, W_INT4 = 3 };

// y[m][r] (+)= scale[r] * sum_j W[r][j] * xin[m][j], xin = x or RMSNorm(x) * gain
struct GemvArgs {
  const void* W;
  const float* scale;       // per-row scales (fp8) or nullptr
  int rows, K, M;
  const float* x;
  int x_stride;
  const uint16_t* gain;     // RMSNorm gain (bf16) or nullptr for no norm
  float eps;
  float* y;
  int y_stride;
  int accumulate;           // 1: y += result (residual stream), 0: y = result
};

// Fused RMSNorm + QKV GEMV + RoPE + KV append.
struct QkvArgs {
  const void* W;
  const float* scale;
  int K, M;
  const float* x;
  int x_stride;
  const uint16_t* gain;
  float eps;
  int n_heads_q, n_heads_kv, head_dim;
  const int* pos;           // device: position of input row 0 (row m is at pos + m)
  const float2* rope;       // [positions][head_dim/2] (cos, sin)
  float* q_out;
  int q_stride;
  uint16_t* kc;             // bf16 [n_kv][cache_len][head_dim]
  uint16_t* vc;
  int cache_len;
};

// Fused RMSNorm + W1/W3 GEMV + SiLU(a) * b.
struct SwigluArgs {
  const void* W1;
  const float* s1;
  const void* W3;
  const float* s3;
  int F, K, M;
  const float* x;
  int x_stride;
  const uint16_t* gain;
  float eps;
  float* h;
  int h_stride;
};

// Fused RMSNorm + head GEMV + per-workgroup argmax.
struct HeadArgs {
  const void* W;
  const float* scale;
  int rows, K;
  const float* x;           // one input row
  const uint16_t* gain;
  float eps;
  float* logits;            // [rows]
  unsigned long long* slots;// [head_grid(rows)] packed (value, index) maximum per workgroup
  int* anomalies;           // +1 per non-finite logit
  float* h_out;             // non-null: workgroup 0 writes the normalised input row here
  int* pos_inc;             // non-null: workgroup 0 does ++*pos_inc (no other reader in the kernel)
};

// Reduce a head's slots to its code and do the frame bookkeeping.
// Sampling of a frame's codes instead of the argmax (u == nullptr: argmax).
// Per codebook: the codes of the previous `window` frames (committed codes,
// from the sequence's first frame on) have their logits divided by `penalty`
// when positive and multiplied otherwise; all logits are divided by
// `temperature`; the top_k largest (ties: lower code) are the candidates;
// softmax over them; cut after the first candidate whose running probability
// sum reaches top_p times the total; the code is the first kept candidate
// whose running sum exceeds u times the kept total.
constexpr int kMaxTopK = 256;          // candidates sorted within one workgroup
constexpr int kMaxSampleVocab = 8192;  // logits held in LDS
constexpr int kMaxWindow = 64;
struct SampleArgs {
  const float* u;     // [max_len][B][frame_codes] draws in [0, 1), by frame position
  float temperature, top_p, penalty;
  int top_k, window;
  const int* win_lo;  // [B] slow position of each sequence's first frame
};
// dynamic LDS of one sampling workgroup over V logits
inline size_t sample_lds_bytes(int V) {
  return ((((size_t)V + 31) / 32 * 4 + 15) & ~(size_t)15) + (size_t)kWaves * 256 * 4 + (size_t)kMaxTopK * 8 +
         256 * 4 + 128;
}

struct CommitArgs {
  const unsigned long long* slots;
  int nslots;
  int code_index;           // k in the frame
  int frame_codes;          // 1 + n_res
  int* pred;                // [frame_codes] argmax codes
  int* committed;           // [frame_codes] codes the next steps consume
  const int* forced;        // [frame_codes]
  const int* force_flag;
  int* ring;                // [max_len][frame_codes]
  const int* pos;           // slow position of this frame
  int* pos_inc;             // non-null: ++*pos_inc at the end (last code of the frame)
  int K;                    // row width of the tables below
  const uint16_t* next_table; // non-null: next_x = next_table[code] (bf16 -> fp32)
  int next_rows;
  float* next_x;
  const uint16_t* slow_table; // non-null: slow_x = slow_table[code] (next frame's slow input)
  int slow_rows;
  float* slow_x;
  const float* copy_src[2];   // optional plain copies done by the same workgroup
  float* copy_dst[2];
  int copy_n[2];
  const float* logits;        // the head's logits [V] (read when sampling)
  int V;
  SampleArgs smp;
};

struct AttnArgs {
  const float* q;
  int q_stride;
  const uint16_t* K;        // bf16 [n_kv][cache_len][head_dim]
  const uint16_t* V;
  int cache_len;
  const int* pos;           // device: position of query row 0
  int n_heads_q, n_heads_kv, head_dim;
  int chunk;                // positions per split (multiple of 16)
  int nsplit_max;           // grid.x
  int M;
  float* part;              // [M][n_kv][nsplit_max][group][head_dim + 2]
  // non-null: the splits merge inside the split launch. The split workgroups
  // of (row m, KV head kvh) count themselves on cnt[m * n_kv + kvh] (zero
  // before the launch, zero again after it) and the last to arrive merges
  // every split's partials into the output; null: a second launch
  // (T_COMBINE) merges them
  unsigned* cnt;
  float* out;
  int out_stride;
  // non-null: the output also as the GEMM input pair hi = bf16(o), lo =
  // bf16(o - hi), same indexing as out (the next projection's input split)
  uint16_t* out_hi;
  uint16_t* out_lo;
  const int* row_pos;       // non-null: position of query row m is row_pos[m] (else *pos + m)
  const int* row_seq;       // non-null: row m reads the cache of sequence row_seq[m]
  long long seq_stride;     // elements between two sequences' caches (paged: between two pages)
  // Paged cache (page_table non-null): position p of sequence s lives in page
  // page_table[s * pages_per_seq + (p >> page_shift)] at offset p & (2^page_shift - 1);
  // cache_len is then the page length. A split never crosses a page (chunk <= page length).
  const int* page_table;
  int page_shift, pages_per_seq;
  int seq0;                 // sequence of every row when row_seq is null (paged prefill)
};

// The same page map for the KV append of many-row stages.
struct PageMap {
  const int* table;         // nullptr: contiguous per-sequence caches
  int shift, per_seq, seq0;
};

// y[m][n] (+)= scale[n] * sum_k x[m][k] W[n][k] for m < M, n < N (prefill
// GEMM on MFMA). The input rows come as two bf16 arrays with x = hi + lo,
// [gemm_mpad(M)][K] (rows past M are never used for an output row).
// K % 64 == 0 (bf16) or % 128 (e4m3), M <= kPrefillRows. With defer set the
// K-split sums stay in part (scaled, [splits][M][N], one split included) for
// the next row kernel to add up; y and accumulate are then unused.
struct GemmArgs {
  const void* W;            // [N][K] bf16 or e4m3fn
  const float* scale;       // [N] (fp8) or nullptr
  int N, K, M;
  const uint16_t* xh;
  const uint16_t* xl;
  float* y;
  int y_stride;
  int accumulate;
  float* part;              // partial sums of the K splits, [splits][M][N]
  int defer;                // leave the sums in part (no second pass)
  int splits, cps;          // set by launch_gemm: K splits, chunks per split
};

// Split-K sums a GEMM left behind: element (m, j) of the product is
// sum over z < n of p[z * stride + m * N + j], N being the product's width.
struct PartSum {
  const float* p;
  int n;                    // 0: nothing pending
  long long stride;         // floats between splits (M * N)
};

// Batched commit of codebook `code_index` for B sequences: argmax of each
// logits row, codes and ring entries, next inputs, position advance.
struct RowsCommitArgs {
  const float* logits;      // [B][ld]
  int ld, V, B;
  int code_index, frame_codes;
  int* pred;                // [B][frame_codes]
  int* committed;           // [B][frame_codes]
  const int* forced;        // [B][frame_codes]
  const int* force_flag;
  int* ring;                // [max_len][B][frame_codes]
  const int* pos;           // [B] slow position of each sequence's frame
  int* pos_inc;             // non-null: ++pos_inc[b] at the end
  int K;                    // row width of the tables and copies
  const uint16_t* next_table;  // non-null: next_x[b * next_stride ...] = next_table[code]
  int next_rows;
  float* next_x;
  int next_stride;
  const uint16_t* slow_table;  // non-null: slow_x[b] = slow_table[code]
  int slow_rows;
  float* slow_x;
  const float* copy_src[2];  // non-null: copy_dst[j][b * dst_stride[j] + i] = copy_src[j][b * src_stride[j] + i]
  float* copy_dst[2];        // for i < copy_n[j]
  int copy_src_stride[2], copy_dst_stride[2], copy_n[2];
  int* anomalies;
  const int* active;         // non-null: rows b with active[b] == 0 keep their position (free slots)
  SampleArgs smp;
};

enum TaskKind : int {
  T_NONE = 0,
  T_QKV,        // QkvArgs
  T_ATTN,       // AttnArgs: split-K attention (direct output when nsplit_max == 1)
  T_COMBINE,    // AttnArgs: merge the splits
  T_GEMV,       // GemvArgs
  T_SWIGLU,     // SwigluArgs
  T_HEAD,       // HeadArgs, weights of the launch's weight type
  T_HEAD_BF16,  // HeadArgs, bf16 weights (the tied codebook-0 head in every mode)
  T_COMMIT,     // CommitArgs, one block
  // many-row stages (batched decode)
  T_NORM_SPLIT,   // NormSplitArgs
  T_GEMM,         // GemmTask
  T_ROPE_ROWS,    // RopeRowsArgs
  T_SILU_SPLIT,   // SiluSplitArgs
  T_COMMIT_ROWS,  // RowsCommitArgs
  T_INC_ROWS      // IncRowsArgs
};

// One stage of a chain: its kind, input rows and arguments.
struct NormSplitArgs {
  float* x;
  int x_stride, M, K;
  const uint16_t* gain;  // nullptr: no norm
  float eps;
  uint16_t* xh;
  uint16_t* xl;
  float* out_f32;        // optional normalised rows
  PartSum add;           // pending residual sums, added into x first
};
struct GemmTask {
  GemmArgs g;
  int wtype;             // the matrix's weight type (the tied codebook-0 head is bf16 in every mode)
  size_t part_cap;       // floats of g.part
};
struct RopeRowsArgs {
  const float* qkv;
  PartSum src;           // when set, the QKV rows are these sums (qkv unused)
  int M;
  const int* row_pos;
  const int* row_seq;
  long long seq_stride;
  int n_heads_q, n_heads_kv, head_dim;
  const float2* rope;
  float* q_out;
  uint16_t* kc;
  uint16_t* vc;
  int cache_len;
  PageMap pages;
};
struct SiluSplitArgs {
  const float* a;
  const float* b;
  PartSum pa, pb;        // when set, a and b are these sums
  int M, F;
  uint16_t* hh;
  uint16_t* hl;
};
struct IncRowsArgs {
  int* v;
  int n;
  const int* active;     // non-null: only entries with active[i] != 0 advance
};

struct Task {
  int kind, M;
  union {
    GemvArgs gemv;
    QkvArgs qkv;
    SwigluArgs swiglu;
    AttnArgs attn;
    HeadArgs head;
    CommitArgs commit;
    NormSplitArgs norm;
    GemmTask gemm;
    RopeRowsArgs rope;
    SiluSplitArgs silu;
    RowsCommitArgs rows;
    IncRowsArgs inc;
  };
};


int head_grid(int rows);
// Launch the kernel specialised for this task (kind, rows M, input width).
// Timing events, when given, are stamped by the launch at the kernel's start
// and end (a many-row stage: recorded before and after its launches).
hipError_t launch_task(int wtype, const Task& t, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// What launch_task needs set up on the host (kernel LDS limits) without
// launching; call before capturing the launch into a graph.
hipError_t prepare_task(int wtype, const Task& t);

// ---- prefill (dar_prefill.hip)
// rows of the GEMM input arrays for M rows
int gemm_mpad(int M);
// K splits gemm_launch_splits picks before the partial-sum limit
// (partial sums: splits * M * N floats)
int gemm_splits(int wtype, int M, int N, int K);
// K splits launch_gemm runs for this product with part_cap floats of partial sums
int gemm_launch_splits(int wtype, int M, int N, int K, size_t part_cap);
// GEMM with K split across workgroups (deterministic second pass, or the
// sums left in part with defer) so that the launch covers the chip; part
// must hold part_cap floats.
hipError_t launch_gemm(int wtype, GemmArgs a, size_t part_cap, hipStream_t s);
// hi/lo bf16 rows of x (RMSNorm(x) * gain when gain is set), gemm_mpad(M)
// rows; out_f32 (optional): the normalised rows in fp32, [M][K]. With add
// pending, x += the sums first (x row stride == K then).
hipError_t launch_norm_split(float* x, int x_stride, int M, int K, const uint16_t* gain, float eps,
                             uint16_t* xh, uint16_t* xl, hipStream_t s, float* out_f32 = nullptr,
                             PartSum add = PartSum{nullptr, 0, 0});
// x[m] = table[clamp(tok[m])] for m < M
hipError_t launch_embed_rows(const uint16_t* table, int rows, int K, const int* tok, int M, float* x,
                             int* anomalies, hipStream_t s);
// RoPE at positions p0 + m (or row_pos[m]) of M rows of QKV output; q out,
// k/v appended to the caches (sequence row_seq[m]'s cache when row_seq is set)
hipError_t launch_rope_rows(const float* qkv, int M, int p0, int n_heads_q, int n_heads_kv, int head_dim,
                            const float2* rope, float* q_out, uint16_t* kc, uint16_t* vc, int cache_len,
                            hipStream_t s, const int* row_pos = nullptr, const int* row_seq = nullptr,
                            long long seq_stride = 0, PartSum src = PartSum{nullptr, 0, 0},
                            PageMap pages = PageMap{nullptr, 0, 0, 0});
// argmax + commit of one codebook for B sequences (k_commit_rows)
hipError_t launch_commit_rows(const RowsCommitArgs& a, hipStream_t s);
// v[i] += 1 for i < n (only where active[i] != 0 when active is set)
hipError_t launch_inc_rows(int* v, int n, hipStream_t s, const int* active = nullptr);
// One slot of a paged context: its block-table row (row[0..per_seq) = pages,
// unused entries the parking page 0), its positions (slow pos_s[b], frame
// pos_f[b], first frame win_lo[b]) and its active flag, in one launch.
constexpr int kMaxPagesPerSeq = 64;
struct SlotState {
  int b, per_seq;
  int pages[kMaxPagesPerSeq];
  int set_state;  // 0: the block-table row only
  int pos_slow, pos_frame, win_lo, active;
};
hipError_t launch_slot_state(int* table, int* pos_s, int* pos_f, int* win_lo, int* active, const SlotState& st,
                             hipStream_t s);
// SiLU(a) * b as hi/lo bf16 rows (a, b: the sums pa, pb when those are set)
hipError_t launch_silu_split(const float* a, const float* b, int M, int F, uint16_t* hh, uint16_t* hl,
                             hipStream_t s, PartSum pa = PartSum{nullptr, 0, 0}, PartSum pb = PartSum{nullptr, 0, 0});

// x = table[clamp(*tok)] as fp32, *pos_out = pos_value (prefill step input)
hipError_t launch_embed(const uint16_t* table, int rows, int K, const int* tok, float* x,
                        int* pos_out, int pos_value, int* anomalies, hipStream_t s);
// forced (nullable) -> dst, *flag = forced != nullptr
hipError_t launch_set_forced(const int* forced, int n, int* dst, int* flag, hipStream_t s);
// dst[i] = value for i < n
hipError_t launch_fill_i32(int* dst, int n, int value, hipStream_t s);
hipError_t launch_fill_u32(unsigned* dst, size_t n, hipStream_t s);
hipError_t launch_quantize_fp8(const uint16_t* w, int rows, int cols, uint8_t* q, float* scale,
                               hipStream_t s);
hipError_t launch_fp8_decode(const uint8_t* codes, int n, float* out, hipStream_t s);
// per-row symmetric int8: scale = rowmax|w| / 127, q = rint(w / scale) in [-127, 127]
hipError_t launch_quantize_int8(const uint16_t* w, int rows, int cols, int8_t* q, float* scale, hipStream_t s);
// int4 in groups of 128 columns: scale [rows][cols/128] = max|w| / 7, codes
// rint(w / scale) in [-7, 7], packed two per byte (even column low)
hipError_t launch_quantize_int4(const uint16_t* w, int rows, int cols, uint8_t* q, float* scale, hipStream_t s);
// codes[r] = the sampled code of logits row r (sample.u[r] the draw,
// history[r][0..n_hist) its window's codes, entries outside [0, V) ignored)
hipError_t launch_sample_rows(const float* logits, int rows, int V, const SampleArgs& sample, const int* history,
                              int n_hist, int* codes, hipStream_t s);
hipError_t launch_copy_i32(const int* src, int* dst, int n, hipStream_t s);

size_t attn_partial_floats(int M, int n_kv, int nsplit_max, int group, int head_dim);

}  // namespace dar
