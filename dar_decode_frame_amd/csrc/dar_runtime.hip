// C-ABI runtime of libdar.so: context, workspace carve-up, RoPE table, the
// frame's launch plans, HIP-graph capture and replay, prefill, helpers.
//
// Frame (tuna-fish README, intro: "slowAR decode + fastAR loop"; "Inference
// estimation": slow AR once, fast AR nine times with a 10-long fast KV):
//   slow layers 0..Ls-1 : QKV(+norm, RoPE, KV append) -> attention (splits
//                         merged in the same launch) -> Wo(+res)
//                         -> W1/W3(+norm, SiLU*mul) -> W2(+res)
//   codebook-0 head     : norm -> W0 -> per-block argmax
//   commit c0           : argmax (or the forced code) -> ring, fast inputs
//                         [h_t, E0[c0]], next frame's slow input W0[c0]
//   fast pass 1         : the fast layers over fast positions 0 and 1 together
//   fast passes 2..R    : the fast layers over position k; after each pass the
//                         shared head and a commit that gathers E_k[c_k]
//
// The slow step of frame i+1 needs only codebook 0 of frame i, not frame i's
// fast AR. A call therefore runs two independent chains of launches on two
// streams: the fast chain finishing frame i (after the commit of its codebook
// 0) and the slow chain computing the slow step and codebook-0 head of frame
// i+1; the slow chain starts once codebook 0 is committed. Their weights are
// nearly equal in size (slow 7.29 GB, fast 9 x 0.83 GB at full shape), and
// the GPU runs kernels of the two streams side by side, so the ramp-up and
// drain of each launch on one stream is covered by the other stream's weight
// traffic. Each chain is a plan of launches built once at create, launched
// eagerly (default: two eager streams overlap better than two replayed graphs
// on ROCm 7.2) or replayed as its own captured graph.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dar.h"
#include "dar_internal.h"

// Device scratch of dar_op_gemm_noalloc: the GEMM's hi/lo input halves and
// its split-K partial sums, for callers that cannot allocate. Each GPU the
// library runs on holds its own copy until the process ends. In host code this
// name is only a stand-in for the device symbol: kernels get the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch()).
static __device__ __align__(256) unsigned char scratch[DAR_NOALLOC_SCRATCH_BYTES];

using namespace dar;

namespace {

thread_local std::string g_create_error;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int frame_codes(const dar_config* c) { return 1 + c->n_res; }
bool has_fast(const dar_config* c) { return c->n_res > 0; }

// the slow chain splits its attention over 64-position chunks once the cache is longer than one chunk
constexpr int kPrefillChunk = 128;  // positions per attention split in the prompt prefill

int nsplit_slow_of(const dar_config* c) { return (c->max_len + kAttnChunkDefault - 1) / kAttnChunkDefault; }

struct Layout {
  size_t x[2], q[2], o[2], h[2], part[2];  // chain scratch: [0] slow (one row), [1] fast (two rows)
  size_t ht, logits0, flogits, slots0, slotsf, pred, committed, forced, flags, acnt, pcnt, pos, seqpos, ring, rope;
  size_t ks, vs, kf, vf;
  // prefill block scratch (kPrefillRows rows): residual, GEMM input halves,
  // QKV output, q, attention output, W1/W3 outputs, GEMM and attention partials
  size_t px, pxh, pxl, pq, po, pgp, patt, ppos, total;
  size_t pgp_floats;
  // batched decode (max_batch > 1): per chain the QKV output, the W3 output,
  // the GEMM input halves and the K-split partial sums; the rows' positions
  // and sequences
  size_t bxh[2], bxl[2], bgp[2], rows;
  size_t bgp_floats[2];
  int nsplit_slow, chunk, rope_len, seq_len, vmax, fast_len, nslots;
  int chunk_rows, nsplit_rows;  // batched slow attention: positions per split, most splits
  // paged slow KV (page_len > 0): K/V pools [L_s][n_pages][n_kv][page_len][hd],
  // block table [max_batch][pages_per_seq], active flags [max_batch]
  int page_len, page_shift, n_pages, pages_per_seq;
  size_t ptable, active;
};

// Paging of a context (page_len 0: one contiguous cache per sequence).
struct Paging {
  int page_len, n_pages;
};

// the kernels' weight type of a dar_wtype (callers have validated it)
int wtype_of(int32_t wtype) {
  switch (wtype) {
    case DAR_WTYPE_FP8_E4M3_ROW: return W_FP8;
    case DAR_WTYPE_INT8_ROW: return W_INT8;
    case DAR_WTYPE_INT4_G128: return W_INT4;
    default: return W_BF16;
  }
}
// quantised Linear matrices, which come with fp32 scales (per row, or per row and 128 columns)
bool has_scales(int32_t wtype) {
  return wtype == DAR_WTYPE_FP8_E4M3_ROW || wtype == DAR_WTYPE_INT8_ROW || wtype == DAR_WTYPE_INT4_G128;
}

Layout make_layout(const dar_config* c, Paging pg = Paging{0, 0}) {
  Layout L{};
  L.page_len = pg.page_len;
  L.n_pages = pg.n_pages;
  if (pg.page_len > 0) {
    while ((1 << L.page_shift) < pg.page_len) ++L.page_shift;
    L.pages_per_seq = (c->max_len + pg.page_len - 1) / pg.page_len;
  }
  const int d = c->d_model, qw = c->n_heads_q * c->head_dim, F = c->ffn_dim;
  const int g = c->n_heads_q / c->n_heads_kv;
  const int fc = frame_codes(c);
  L.chunk = kAttnChunkDefault;
  L.nsplit_slow = nsplit_slow_of(c);
  // batched decode: B x n_kv x splits workgroups for the slow attention, the
  // splits of the longest sequence only (set per frame, eager launches)
  L.chunk_rows = kAttnChunkDefault;
  L.nsplit_rows = (c->max_len + L.chunk_rows - 1) / L.chunk_rows;
  L.fast_len = has_fast(c) ? c->n_res + 1 : 1;
  L.rope_len = std::max(c->max_len, L.fast_len);
  L.seq_len = std::max(c->max_len, L.fast_len + 1);
  L.vmax = std::max(c->vocab_c0, has_fast(c) ? c->vocab_res : 0);
  L.nslots = std::max(head_grid(c->vocab_c0), has_fast(c) ? head_grid(c->vocab_res) : 0);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const int B = c->max_batch;
  for (int ch = 0; ch < 2; ++ch) {
    const int M = (ch == 0 ? 1 : 2) * B;
    const int nsplit = ch == 0 ? L.nsplit_slow : 1;
    L.x[ch] = take(sizeof(float) * M * d);
    L.q[ch] = take(sizeof(float) * M * qw);
    L.o[ch] = take(sizeof(float) * M * qw);
    L.h[ch] = take(sizeof(float) * M * F);
    L.part[ch] = take(sizeof(float) * attn_partial_floats(M, c->n_heads_kv, nsplit, g, c->head_dim));
  }
  L.ht = take(sizeof(float) * (size_t)B * d);
  L.logits0 = take(sizeof(float) * (size_t)B * c->vocab_c0);
  L.flogits = take(sizeof(float) * (size_t)B * fc * L.vmax);
  L.slots0 = take(sizeof(unsigned long long) * L.nslots);
  L.slotsf = take(sizeof(unsigned long long) * L.nslots);
  L.pred = take(sizeof(int) * B * fc);
  L.committed = take(sizeof(int) * B * fc);
  L.forced = take(sizeof(int) * B * fc);
  L.flags = take(sizeof(int) * 4);
  // split counters of the slow decode attention and of the prefill's (zero between launches)
  L.acnt = take(sizeof(unsigned) * B * c->n_heads_kv);
  L.pcnt = take(sizeof(unsigned) * kPrefillRows * c->n_heads_kv);
  L.pos = take(sizeof(int) * (3 * B + 4));  // slow positions [B], frame positions [B], first frames [B]
  L.seqpos = take(sizeof(int) * L.seq_len);
  L.ring = take(sizeof(int) * (size_t)c->max_len * B * fc);
  L.rope = take(sizeof(float) * 2 * (size_t)L.rope_len * (c->head_dim / 2));
  const size_t kv_slow = pg.page_len > 0
                             ? (size_t)c->n_layers_slow * pg.n_pages * c->n_heads_kv * pg.page_len * c->head_dim * 2
                             : (size_t)c->n_layers_slow * B * c->n_heads_kv * c->max_len * c->head_dim * 2;
  L.ks = take(kv_slow);
  L.vs = take(kv_slow);
  const size_t kv_fast =
      has_fast(c) ? (size_t)c->n_layers_fast * B * c->n_heads_kv * L.fast_len * c->head_dim * 2 : 0;
  L.kf = take(kv_fast);
  L.vf = take(kv_fast);
  const size_t R = kPrefillRows;
  const int qkv_rows = (c->n_heads_q + 2 * c->n_heads_kv) * c->head_dim;
  const int kmax = std::max(std::max(d, qw), F);
  L.px = take(sizeof(float) * R * d);
  L.pxh = take(2 * R * kmax);
  L.pxl = take(2 * R * kmax);
  L.pq = take(sizeof(float) * R * qw);
  L.po = take(sizeof(float) * R * qw);
  // partial sums of the widest K split launch_gemm picks for the block's GEMMs
  const int wt = wtype_of(c->wtype);
  L.pgp_floats = 0;
  for (auto nk : {std::pair<int, int>{qkv_rows, d}, {d, qw}, {F, d}, {d, F}}) {
    for (int M = 1; M <= (int)R; ++M)
      L.pgp_floats = std::max(L.pgp_floats, (size_t)gemm_splits(wt, M, nk.first, nk.second) * M * nk.first);
  }
  L.pgp = take(2 * sizeof(float) * L.pgp_floats);  // two regions: W1's and W3's sums live together
  L.patt = take(sizeof(float) * attn_partial_floats((int)R, c->n_heads_kv, L.nsplit_slow, g, c->head_dim));
  L.ppos = take(sizeof(int) * 4);
  if (B > 1) {
    for (int ch = 0; ch < 2; ++ch) {
      const int M = (ch == 0 ? 1 : 2) * B;
      L.bxh[ch] = take(2 * (size_t)gemm_mpad(M) * kmax);
      L.bxl[ch] = take(2 * (size_t)gemm_mpad(M) * kmax);
      L.bgp_floats[ch] = 0;
      for (auto nk : {std::pair<int, int>{qkv_rows, d}, {d, qw}, {F, d}, {d, F}, {c->vocab_c0, d},
                      {has_fast(c) ? c->vocab_res : 1, d}}) {
        for (int m : {M, B})
          L.bgp_floats[ch] =
              std::max(L.bgp_floats[ch], (size_t)gemm_splits(wt, m, nk.first, nk.second) * m * nk.first);
      }
      L.bgp[ch] = take(2 * sizeof(float) * L.bgp_floats[ch]);
    }
    // sequence ids [B], first-pass positions and sequences [2B], pass positions [R+1][B]
    L.rows = take(sizeof(int) * (size_t)(B + 4 * B + (c->n_res + 1) * B));
  }
  if (pg.page_len > 0) {
    L.ptable = take(sizeof(int) * (size_t)B * L.pages_per_seq);
    L.active = take(sizeof(int) * (size_t)B);
  }
  L.total = off;
  return L;
}

int validate_config(const dar_config* c, std::string& why) {
  if (!c) {
    why = "config is NULL";
    return DAR_E_INVAL;
  }
  auto bad = [&](const char* msg) {
    why = msg;
    return DAR_E_INVAL;
  };
  if (c->n_layers_slow < 1) return bad("n_layers_slow must be >= 1");
  if (c->n_layers_fast < 0 || c->n_res < 0) return bad("n_layers_fast and n_res must be >= 0");
  if (c->d_model < 1 || c->n_heads_q < 1 || c->n_heads_kv < 1 || c->head_dim < 1 || c->ffn_dim < 1)
    return bad("dimensions must be positive");
  if (c->n_heads_q % c->n_heads_kv != 0) return bad("n_heads_q must be a multiple of n_heads_kv");
  if (c->vocab_c0 < 1) return bad("vocab_c0 must be >= 1");
  if (c->n_res > 0 && (c->n_layers_fast < 1 || c->vocab_res < 1))
    return bad("n_res > 0 needs n_layers_fast >= 1 and vocab_res >= 1");
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return bad("rms_eps must be positive and finite");
  if (!(c->rope_base > 1.0) || !std::isfinite(c->rope_base)) return bad("rope_base must be > 1");
  if (c->max_len < 2) return bad("max_len must be >= 2");
  if (c->max_batch < 1) return bad("max_batch must be >= 1");
  if (c->wtype != DAR_WTYPE_BF16 && !has_scales(c->wtype)) return bad("unknown wtype");
  const int g = c->n_heads_q / c->n_heads_kv;
  auto unsup = [&](const char* msg) {
    why = msg;
    return DAR_E_UNSUPPORTED;
  };
  if (c->head_dim != 64 && c->head_dim != 128) return unsup("head_dim must be 64 or 128");
  if (g != 1 && g != 2 && g != 4 && g != 8) return unsup("n_heads_q / n_heads_kv must be 1, 2, 4 or 8");
  const int qw = c->n_heads_q * c->head_dim;
  if (c->d_model % 256 || c->ffn_dim % 256 || qw % 256) return unsup("d_model, ffn_dim, n_heads_q*head_dim must be multiples of 256");
  if (c->d_model > 16384 || c->ffn_dim > 16384 || qw > 16384) return unsup("widths above 16384");
  if (c->n_res > 15) return unsup("n_res above 15");
  if (c->max_batch > kPrefillRows / 2) return unsup("max_batch above 64");
  if (c->max_len > (1 << 24)) return unsup("max_len above 2^24");
  return DAR_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }


int check_layer(const dar_layer_weights& w, bool scaled, std::string& why, const char* which, int idx) {
  const void* ptrs[] = {w.attn_norm, w.wqkv, w.wo, w.ffn_norm, w.w1, w.w3, w.w2};
  for (const void* p : ptrs) {
    if (!p || !aligned16(p)) {
      char buf[128];
      snprintf(buf, sizeof buf, "%s layer %d: a weight pointer is NULL or not 16-byte aligned", which, idx);
      why = buf;
      return DAR_E_INVAL;
    }
  }
  if (scaled) {
    const float* s[] = {w.wqkv_scale, w.wo_scale, w.w1_scale, w.w3_scale, w.w2_scale};
    for (const float* p : s) {
      if (!p) {
        char buf[128];
        snprintf(buf, sizeof buf, "%s layer %d: scale pointer is NULL (quantised weights)", which, idx);
        why = buf;
        return DAR_E_INVAL;
      }
    }
  }
  return DAR_OK;
}

typedef uint32_t ru32x4 __attribute__((ext_vector_type(4)));
// Launch shape of the reference read: of the forms timed on this part (1024 to
// 8192 workgroups, four or eight 16-byte loads in flight per thread, ordinary,
// non-temporal or buffer loads), 8192 workgroups with eight non-temporal loads
// in flight per thread read fastest.
// n 16-byte units from p, U non-temporal loads in flight per thread over a
// grid-stride loop
template <int U>
__global__ __launch_bounds__(kBlock) void k_stream_read(const ru32x4* __restrict__ p, size_t n, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kBlock;
  size_t i = blockIdx.x * (size_t)kBlock + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    ru32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x + v[u].y * 3u + v[u].z * 5u + v[u].w * 7u;
  }
  for (; i < n; i += stride) {
    const ru32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x & 2047] = acc;
}

// The read's launch shapes (workgroups, loads in flight per thread). HBM on
// this part streams fastest with about 6-8 MB of loads in flight (384 x 4,
// 768 x 2, 256 x 8 reached 7.2-7.4 TB/s over 1 GiB; 16 MB or more in flight
// fell to 5.2-6.0); the reference takes the fastest shape on the GPU at hand.
struct ReadShape {
  int grid, loads;
};
constexpr ReadShape kReadShapes[] = {{384, 4}, {768, 2}, {256, 8}, {512, 4}, {8192, 8}};


}  // namespace

enum Kind { K_QKV = 0, K_ATTN = 1, K_WO = 2, K_W13 = 3, K_W2 = 4, K_HEAD = 5, K_OTHER = 6 };

struct TaskRec {
  Task t;
  int kind, layer;  // for the profiler
};

// A sequence of launches, one task each.
struct Plan {
  std::vector<Task> tasks;
  std::vector<int> kind, layer;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  size_t launches() const { return tasks.size(); }
};

// Scratch and stream of one chain of launches.
struct Chain {
  float *x = nullptr, *q = nullptr, *o = nullptr, *h = nullptr, *part = nullptr;
  unsigned* cnt = nullptr;  // non-null: split attention merges its splits in its own launch
  hipStream_t s = nullptr;
};

struct dar_ctx {
  dar_config cfg{};
  Layout L{};
  bool quant = false;      // quantised weights with fp32 scales (fp8, int8: per row; int4: per 128 columns)
  int wq = W_BF16;         // the kernels' weight type of the Linear matrices
  std::vector<dar_layer_weights> slow, fast;
  std::vector<const uint16_t*> fast_emb;
  const uint16_t* w0 = nullptr;
  const uint16_t* slow_fn = nullptr;
  const uint16_t* fast_fn = nullptr;
  const void* fast_head = nullptr;
  const float* fast_head_scale = nullptr;

  hipStream_t stream = nullptr;  // the caller's stream
  Chain cs, cf;                  // slow chain (frame i+1) and fast chain (frame i)
  Plan p_c0, p_fast, p_slow;  // commit of c0, fast AR, slow step + c0 head
  hipEvent_t ev_start = nullptr, ev_c0 = nullptr, ev_f_done = nullptr, ev_s_done = nullptr;
  bool use_graph = false;

  char* ws = nullptr;
  float *ht, *logits0, *flogits;
  unsigned long long *slots0, *slotsf;
  int *pred, *committed, *forced, *flags, *pos_s, *pos_f, *seqpos, *ring;
  int* win_lo;                 // [B] slow position of each sequence's first frame (sampling windows)
  SampleArgs smp{};            // sampling of the codes (u == nullptr: greedy argmax)
  int B = 1;                   // sequences decoded in lockstep
  float* bgp[2];
  uint16_t *bxh[2], *bxl[2];
  int *seq_ident, *p1_pos, *p1_seq, *pk_pos;
  std::vector<int> pos_hb;     // host mirror of each sequence's next slow position
  std::vector<int> pos_init;   // host staging of the positions set by a prefill
  float2* rope;
  uint16_t *ks, *vs, *kf, *vf;

  // paged slow KV and continuous batching (dar_create_paged)
  bool paged = false;
  int* ptable = nullptr;        // device block table [B][pages_per_seq]
  int* active = nullptr;        // device flags [B]: slot holds a sequence
  std::vector<int> free_pages;  // host allocator: pages not held by a slot (page 0 never: parking)
  std::vector<std::vector<int>> slot_pages;  // pages of each slot, in position order
  std::vector<char> slot_on;    // host mirror of active

  int pos_host = 0;       // slow position of the next frame to decode
  int attn_splits_live = 0;  // batched slow attention splits for the coming frame (0: all)
  int attn_chunk_live = 0;   // and the positions per split
  bool prefilled = false;
  bool force_dev = false;
  std::string err;

  std::vector<hipEvent_t> events;
  // live timing of one kind of launch in eager decode frames (dar_time_kind)
  int timed_kind = -1;
  std::vector<hipEvent_t> tpool;  // event pairs, reused
  size_t tused = 0;               // events recorded since the last read
};

namespace {

int hip_fail(dar_ctx* c, hipError_t e, const char* what) {
  std::string msg = std::string(what) + ": " + hipGetErrorString(e);
  if (c)
    c->err = msg;
  else
    g_create_error = msg;
  return DAR_E_HIP;
}

#define DAR_HIP(ctx, call, what)                           \
  do {                                                     \
    hipError_t e_ = (call);                                \
    if (e_ != hipSuccess) return hip_fail(ctx, e_, what); \
  } while (0)

Task none_task() {
  Task t;
  std::memset(&t, 0, sizeof t);
  t.kind = T_NONE;
  return t;
}

TaskRec rec(const Task& t, int kind, int layer) {
  TaskRec r;
  r.t = t;
  r.kind = kind;
  r.layer = layer;
  return r;
}

// The five or six stages of one decoder layer over M rows at device position *pos.
void add_layer(dar_ctx* c, std::vector<TaskRec>& out, const Chain& ch, const dar_layer_weights& w, int tag, int M,
               const int* pos, uint16_t* kc, uint16_t* vc, int cache_len, int nsplit_max) {
  const dar_config& g = c->cfg;
  const int d = g.d_model, qw = g.n_heads_q * g.head_dim;
  Task t = none_task();

  t.kind = T_QKV;
  t.M = M;
  QkvArgs& qa = t.qkv;
  qa.W = w.wqkv;
  qa.scale = c->quant ? w.wqkv_scale : nullptr;
  qa.K = d;
  qa.M = M;
  qa.x = ch.x;
  qa.x_stride = d;
  qa.gain = static_cast<const uint16_t*>(w.attn_norm);
  qa.eps = g.rms_eps;
  qa.n_heads_q = g.n_heads_q;
  qa.n_heads_kv = g.n_heads_kv;
  qa.head_dim = g.head_dim;
  qa.pos = pos;
  qa.rope = c->rope;
  qa.q_out = ch.q;
  qa.q_stride = qw;
  qa.kc = kc;
  qa.vc = vc;
  qa.cache_len = cache_len;
  out.push_back(rec(t, K_QKV, tag));

  t = none_task();
  t.kind = T_ATTN;
  t.M = M;
  AttnArgs& aa = t.attn;
  aa.q = ch.q;
  aa.q_stride = qw;
  aa.K = kc;
  aa.V = vc;
  aa.cache_len = cache_len;
  aa.pos = pos;
  aa.n_heads_q = g.n_heads_q;
  aa.n_heads_kv = g.n_heads_kv;
  aa.head_dim = g.head_dim;
  aa.chunk = c->L.chunk;
  aa.nsplit_max = nsplit_max;
  aa.M = M;
  aa.part = ch.part;
  aa.cnt = nsplit_max > 1 ? ch.cnt : nullptr;
  aa.out = ch.o;
  aa.out_stride = qw;
  out.push_back(rec(t, K_ATTN, tag));

  t = none_task();
  t.kind = T_GEMV;
  t.M = M;
  GemvArgs& wo = t.gemv;
  wo.W = w.wo;
  wo.scale = c->quant ? w.wo_scale : nullptr;
  wo.rows = d;
  wo.K = qw;
  wo.M = M;
  wo.x = ch.o;
  wo.x_stride = qw;
  wo.y = ch.x;
  wo.y_stride = d;
  wo.accumulate = 1;
  out.push_back(rec(t, K_WO, tag));

  t = none_task();
  t.kind = T_SWIGLU;
  t.M = M;
  SwigluArgs& sa = t.swiglu;
  sa.W1 = w.w1;
  sa.s1 = c->quant ? w.w1_scale : nullptr;
  sa.W3 = w.w3;
  sa.s3 = c->quant ? w.w3_scale : nullptr;
  sa.F = g.ffn_dim;
  sa.K = d;
  sa.M = M;
  sa.x = ch.x;
  sa.x_stride = d;
  sa.gain = static_cast<const uint16_t*>(w.ffn_norm);
  sa.eps = g.rms_eps;
  sa.h = ch.h;
  sa.h_stride = g.ffn_dim;
  out.push_back(rec(t, K_W13, tag));

  t = none_task();
  t.kind = T_GEMV;
  t.M = M;
  GemvArgs& w2 = t.gemv;
  w2.W = w.w2;
  w2.scale = c->quant ? w.w2_scale : nullptr;
  w2.rows = d;
  w2.K = g.ffn_dim;
  w2.M = M;
  w2.x = ch.h;
  w2.x_stride = g.ffn_dim;
  w2.y = ch.x;
  w2.y_stride = d;
  w2.accumulate = 1;
  out.push_back(rec(t, K_W2, tag));
}

// Slow chain: the slow layers at *pos_s over the slow residual; with_head adds
// the codebook-0 head (logits, per-block maxima, h_t), which also advances pos_s.
std::vector<TaskRec> slow_chain(dar_ctx* c, bool with_head) {
  const dar_config& g = c->cfg;
  std::vector<TaskRec> out;
  const size_t per_layer = (size_t)g.n_heads_kv * g.max_len * g.head_dim;
  for (int l = 0; l < g.n_layers_slow; ++l)
    add_layer(c, out, c->cs, c->slow[l], l, 1, c->pos_s, c->ks + l * per_layer, c->vs + l * per_layer, g.max_len,
              c->L.nsplit_slow);
  if (with_head) {
    Task t = none_task();
    t.kind = T_HEAD_BF16;
    t.M = 1;
    HeadArgs& h0 = t.head;
    h0.W = c->w0;
    h0.scale = nullptr;
    h0.rows = g.vocab_c0;
    h0.K = g.d_model;
    h0.x = c->cs.x;
    h0.gain = c->slow_fn;
    h0.eps = g.rms_eps;
    h0.logits = c->logits0;
    h0.slots = c->slots0;
    h0.anomalies = c->flags + 1;
    h0.h_out = c->ht;
    h0.pos_inc = c->pos_s;
    out.push_back(rec(t, K_HEAD, 0));
  }
  return out;
}

Task commit_task(dar_ctx* c, int k, const unsigned long long* slots, int rows, const float* logits) {
  Task t = none_task();
  t.kind = T_COMMIT;
  t.M = 1;
  CommitArgs& a = t.commit;
  a.slots = slots;
  a.nslots = head_grid(rows);
  a.logits = logits;
  a.V = rows;
  a.smp = c->smp;
  a.code_index = k;
  a.frame_codes = frame_codes(&c->cfg);
  a.pred = c->pred;
  a.committed = c->committed;
  a.forced = c->forced;
  a.force_flag = c->flags + 0;
  a.ring = c->ring;
  a.pos = c->pos_f;
  a.K = c->cfg.d_model;
  return t;
}

// Fast chain: commit codebook 0 of the frame (argmax of the slow head, or the
// forced code), move its logits and h_t into the frame's buffers, write the
// fast inputs [h_t, E0[c0]] and the next slow input W0[c0]; then the fast AR:
// pass 1 over fast positions 0 and 1, passes 2..R over position k, each
// followed by the shared head and its commit.
std::vector<TaskRec> commit0_chain(dar_ctx* c) {
  const dar_config& g = c->cfg;
  const int d = g.d_model;
  const bool fast = has_fast(&g);
  std::vector<TaskRec> out;
  Task t0 = commit_task(c, 0, c->slots0, g.vocab_c0, c->logits0);
  CommitArgs& a = t0.commit;
  a.pos_inc = fast ? nullptr : c->pos_f;
  a.next_table = fast ? c->fast_emb[0] : nullptr;
  a.next_rows = g.vocab_c0;
  a.next_x = c->cf.x + d;
  a.slow_table = c->w0;
  a.slow_rows = g.vocab_c0;
  a.slow_x = c->cs.x;
  a.copy_src[0] = c->logits0;
  a.copy_dst[0] = c->flogits;
  a.copy_n[0] = g.vocab_c0;
  if (fast) {
    a.copy_src[1] = c->ht;
    a.copy_dst[1] = c->cf.x;
    a.copy_n[1] = d;
  }
  out.push_back(rec(t0, K_OTHER, 0));
  return out;
}

std::vector<TaskRec> fast_chain(dar_ctx* c) {
  const dar_config& g = c->cfg;
  const int d = g.d_model;
  std::vector<TaskRec> out;
  if (!has_fast(&g)) return out;
  const size_t per_layer = (size_t)g.n_heads_kv * c->L.fast_len * g.head_dim;
  for (int k = 1; k <= g.n_res; ++k) {
    const int M = (k == 1) ? 2 : 1;
    const int* fpos = c->seqpos + (k == 1 ? 0 : k);
    for (int l = 0; l < g.n_layers_fast; ++l)
      add_layer(c, out, c->cf, c->fast[l], 1000 * k + l, M, fpos, c->kf + l * per_layer, c->vf + l * per_layer,
                c->L.fast_len, 1);
    Task t = none_task();
    t.kind = T_HEAD;
    t.M = 1;
    HeadArgs& hk = t.head;
    hk.W = c->fast_head;
    hk.scale = c->quant ? c->fast_head_scale : nullptr;
    hk.rows = g.vocab_res;
    hk.K = d;
    hk.x = c->cf.x + (size_t)(M - 1) * d;
    hk.gain = c->fast_fn;
    hk.eps = g.rms_eps;
    hk.logits = c->flogits + (size_t)k * c->L.vmax;
    hk.slots = c->slotsf;
    hk.anomalies = c->flags + 1;
    out.push_back(rec(t, K_HEAD, k));
    Task ck = commit_task(c, k, c->slotsf, g.vocab_res, c->flogits + (size_t)k * c->L.vmax);
    ck.commit.pos_inc = (k == g.n_res) ? c->pos_f : nullptr;
    ck.commit.next_table = (k < g.n_res) ? c->fast_emb[k] : nullptr;
    ck.commit.next_rows = g.vocab_res;
    ck.commit.next_x = c->cf.x;
    out.push_back(rec(ck, K_OTHER, k));
  }
  return out;
}

// ---- batched decode (max_batch > 1): every stage runs the chain's rows at
// once (one per sequence; two per sequence in the fast AR's first pass), the
// projections as MFMA GEMMs over the rows.

constexpr PartSum kNoSums{nullptr, 0, 0};

Task t_norm(float* x, int x_stride, int M, int K, const void* gain, float eps, uint16_t* xh, uint16_t* xl,
            float* out_f32 = nullptr, PartSum add = kNoSums) {
  Task t = none_task();
  t.kind = T_NORM_SPLIT;
  t.M = M;
  t.norm = NormSplitArgs{x, x_stride, M, K, static_cast<const uint16_t*>(gain), eps, xh, xl, out_f32, add};
  return t;
}

Task t_gemm(int wtype, const void* W, const float* scale, int N, int K, int M, const uint16_t* xh,
            const uint16_t* xl, float* y, int y_stride, int acc, float* part, size_t cap, int defer = 0) {
  Task t = none_task();
  t.kind = T_GEMM;
  t.M = M;
  GemmArgs& g = t.gemm.g;
  g.W = W;
  g.scale = wtype != W_BF16 ? scale : nullptr;  // one-byte weights carry row scales
  g.N = N;
  g.K = K;
  g.M = M;
  g.xh = xh;
  g.xl = xl;
  g.y = y;
  g.y_stride = y_stride;
  g.accumulate = acc;
  g.part = part;
  g.defer = defer;
  t.gemm.wtype = wtype;
  t.gemm.part_cap = cap;
  return t;
}

// One decoder layer over the chain's M rows: row m is at position row_pos[m]
// of sequence row_seq[m]'s caches (kc/vc: this layer's caches of sequence 0,
// seq_stride elements apart).
void add_layer_rows(dar_ctx* c, std::vector<TaskRec>& out, int ch, const dar_layer_weights& w, int tag, int M,
                    const int* row_pos, const int* row_seq, uint16_t* kc, uint16_t* vc, int cache_len,
                    long long seq_stride, int nsplit_max, int chunk, PartSum& pend, bool defer_w2,
                    PageMap pm = PageMap{nullptr, 0, 0, 0}) {
  const dar_config& g = c->cfg;
  const int d = g.d_model, qw = g.n_heads_q * g.head_dim, F = g.ffn_dim;
  const int qkv_rows = (g.n_heads_q + 2 * g.n_heads_kv) * g.head_dim;
  const int wt = c->wq;
  const Chain& cn = ch == 0 ? c->cs : c->cf;
  uint16_t *xh = c->bxh[ch], *xl = c->bxl[ch];
  float* gp = c->bgp[ch];
  const size_t cap = c->L.bgp_floats[ch];
  float* gp2 = gp + cap;  // second region: W3's sums beside W1's
  // each projection leaves its K-split sums for the row kernel that reads it
  auto sums = [&](float* part, int N, int K) {
    return PartSum{part, gemm_launch_splits(wt, M, N, K, cap), (long long)M * N};
  };
  out.push_back(rec(t_norm(cn.x, d, M, d, w.attn_norm, g.rms_eps, xh, xl, nullptr, pend), K_OTHER, tag));
  out.push_back(rec(t_gemm(wt, w.wqkv, w.wqkv_scale, qkv_rows, d, M, xh, xl, nullptr, 0, 0, gp, cap, 1), K_QKV, tag));
  Task t = none_task();
  t.kind = T_ROPE_ROWS;
  t.M = M;
  t.rope = RopeRowsArgs{nullptr, sums(gp, qkv_rows, d), M, row_pos, row_seq, seq_stride, g.n_heads_q, g.n_heads_kv,
                        g.head_dim, c->rope, cn.q, kc, vc, cache_len, pm};
  out.push_back(rec(t, K_OTHER, tag));
  t = none_task();
  t.kind = T_ATTN;
  t.M = M;
  AttnArgs& aa = t.attn;
  aa.q = cn.q;
  aa.q_stride = qw;
  aa.K = kc;
  aa.V = vc;
  aa.cache_len = cache_len;
  aa.pos = row_pos;
  aa.n_heads_q = g.n_heads_q;
  aa.n_heads_kv = g.n_heads_kv;
  aa.head_dim = g.head_dim;
  aa.chunk = chunk;
  aa.nsplit_max = nsplit_max;
  aa.M = M;
  aa.part = cn.part;
  aa.out = cn.o;
  aa.out_stride = qw;
  aa.row_pos = row_pos;
  aa.row_seq = row_seq;
  aa.seq_stride = seq_stride;
  aa.page_table = pm.table;
  aa.page_shift = pm.shift;
  aa.pages_per_seq = pm.per_seq;
  aa.out_hi = xh;  // the O projection's input split, written by the attention itself
  aa.out_lo = xl;
  out.push_back(rec(t, K_ATTN, tag));
  // a merge launch rather than merging in the split launch: with 64 sequences
  // the in-launch merge made the step slower (5,862 against 6,089 frames/s)
  // although the split and merge kernels alone took longer (31.2 + 7.6 against
  // 36.3 us): its tail of dependent memory round trips overlaps worse with the
  // other chain's kernels
  if (nsplit_max > 1) {
    t.kind = T_COMBINE;
    out.push_back(rec(t, K_ATTN, tag));
  }
  out.push_back(rec(t_gemm(wt, w.wo, w.wo_scale, d, qw, M, xh, xl, nullptr, 0, 0, gp, cap, 1), K_WO, tag));
  out.push_back(rec(t_norm(cn.x, d, M, d, w.ffn_norm, g.rms_eps, xh, xl, nullptr, sums(gp, d, qw)), K_OTHER, tag));
  out.push_back(rec(t_gemm(wt, w.w1, w.w1_scale, F, d, M, xh, xl, nullptr, 0, 0, gp, cap, 1), K_W13, tag));
  out.push_back(rec(t_gemm(wt, w.w3, w.w3_scale, F, d, M, xh, xl, nullptr, 0, 0, gp2, cap, 1), K_W13, tag));
  t = none_task();
  t.kind = T_SILU_SPLIT;
  t.M = M;
  t.silu = SiluSplitArgs{nullptr, nullptr, sums(gp, F, d), sums(gp2, F, d), M, F, xh, xl};
  out.push_back(rec(t, K_OTHER, tag));
  if (defer_w2) {
    out.push_back(rec(t_gemm(wt, w.w2, w.w2_scale, d, F, M, xh, xl, nullptr, 0, 0, gp, cap, 1), K_W2, tag));
    pend = sums(gp, d, F);
  } else {
    out.push_back(rec(t_gemm(wt, w.w2, w.w2_scale, d, F, M, xh, xl, cn.x, d, 1, gp, cap), K_W2, tag));
    pend = kNoSums;
  }
}

// Batched slow chain: the slow layers for every sequence at its position, the
// final norm (h_t kept in fp32) and the codebook-0 head GEMM, then the slow
// positions advance.
std::vector<TaskRec> slow_chain_rows(dar_ctx* c) {
  const dar_config& g = c->cfg;
  const int B = c->B, d = g.d_model;
  std::vector<TaskRec> out;
  PartSum pend = kNoSums;  // the layer's residual sums, added by the next norm
  if (c->paged) {
    // a page holds page_len positions of every KV head; row b's positions go
    // through its block-table row
    const Layout& L = c->L;
    const long long page_stride = (long long)g.n_heads_kv * L.page_len * g.head_dim;
    const PageMap pm{c->ptable, L.page_shift, L.pages_per_seq, 0};
    for (int l = 0; l < g.n_layers_slow; ++l)
      add_layer_rows(c, out, 0, c->slow[l], l, B, c->pos_s, c->seq_ident,
                     c->ks + (size_t)l * L.n_pages * page_stride, c->vs + (size_t)l * L.n_pages * page_stride,
                     L.page_len, page_stride, L.nsplit_rows, L.chunk_rows, pend, true, pm);
  } else {
    const long long seq_stride = (long long)g.n_heads_kv * g.max_len * g.head_dim;
    for (int l = 0; l < g.n_layers_slow; ++l)
      add_layer_rows(c, out, 0, c->slow[l], l, B, c->pos_s, c->seq_ident, c->ks + (size_t)l * B * seq_stride,
                     c->vs + (size_t)l * B * seq_stride, g.max_len, seq_stride, c->L.nsplit_rows, c->L.chunk_rows,
                     pend, true);
  }
  out.push_back(
      rec(t_norm(c->cs.x, d, B, d, c->slow_fn, g.rms_eps, c->bxh[0], c->bxl[0], c->ht, pend), K_OTHER, 0));
  out.push_back(rec(t_gemm(W_BF16, c->w0, nullptr, g.vocab_c0, d, B, c->bxh[0], c->bxl[0], c->logits0, g.vocab_c0, 0,
                           c->bgp[0], c->L.bgp_floats[0]),
                    K_HEAD, 0));
  Task t = none_task();
  t.kind = T_INC_ROWS;
  t.inc = IncRowsArgs{c->pos_s, B, c->active};
  out.push_back(rec(t, K_OTHER, 0));
  return out;
}

RowsCommitArgs rows_commit(dar_ctx* c, int k, const float* logits, int ld, int V) {
  const dar_config& g = c->cfg;
  RowsCommitArgs r{};
  r.logits = logits;
  r.ld = ld;
  r.V = V;
  r.B = c->B;
  r.code_index = k;
  r.frame_codes = frame_codes(&g);
  r.pred = c->pred;
  r.committed = c->committed;
  r.forced = c->forced;
  r.force_flag = c->flags + 0;
  r.ring = c->ring;
  r.pos = c->pos_f;
  r.K = g.d_model;
  r.anomalies = c->flags + 1;
  r.active = c->active;
  r.smp = c->smp;
  return r;
}

// Batched commit of codebook 0: codes, the next slow inputs W0[c0], the fast
// inputs [h_t, E0[c0]] (rows 2b, 2b + 1) and the frame's codebook-0 logits.
std::vector<TaskRec> commit0_chain_rows(dar_ctx* c) {
  const dar_config& g = c->cfg;
  const int d = g.d_model, fc = frame_codes(&g);
  const bool fast = has_fast(&g);
  Task t = none_task();
  t.kind = T_COMMIT_ROWS;
  RowsCommitArgs& r = t.rows;
  r = rows_commit(c, 0, c->logits0, g.vocab_c0, g.vocab_c0);
  r.pos_inc = fast ? nullptr : c->pos_f;
  r.next_table = fast ? c->fast_emb[0] : nullptr;
  r.next_rows = g.vocab_c0;
  r.next_x = c->cf.x + d;
  r.next_stride = 2 * d;
  r.slow_table = c->w0;
  r.slow_rows = g.vocab_c0;
  r.slow_x = c->cs.x;
  if (fast) {
    r.copy_src[0] = c->ht;
    r.copy_dst[0] = c->cf.x;
    r.copy_src_stride[0] = d;
    r.copy_dst_stride[0] = 2 * d;
    r.copy_n[0] = d;
  }
  r.copy_src[1] = c->logits0;
  r.copy_dst[1] = c->flogits;
  r.copy_src_stride[1] = g.vocab_c0;
  r.copy_dst_stride[1] = fc * c->L.vmax;
  r.copy_n[1] = g.vocab_c0;
  return {rec(t, K_OTHER, 0)};
}

// Batched fast AR: pass 1 over 2B rows (positions 0 and 1 of every
// sequence), passes 2..R over B rows, each followed by the head GEMM and the
// commit of c_k for every sequence.
std::vector<TaskRec> fast_chain_rows(dar_ctx* c) {
  const dar_config& g = c->cfg;
  const int B = c->B, d = g.d_model, fc = frame_codes(&g);
  std::vector<TaskRec> out;
  if (!has_fast(&g)) return out;
  const long long seq_stride = (long long)g.n_heads_kv * c->L.fast_len * g.head_dim;
  for (int k = 1; k <= g.n_res; ++k) {
    const int M = k == 1 ? 2 * B : B;
    const int* rp = k == 1 ? c->p1_pos : c->pk_pos + (size_t)k * B;
    const int* rs = k == 1 ? c->p1_seq : c->seq_ident;
    // pass 1's head reads every second row, so its last residual is summed in place
    PartSum pend = kNoSums;
    for (int l = 0; l < g.n_layers_fast; ++l)
      add_layer_rows(c, out, 1, c->fast[l], 1000 * k + l, M, rp, rs, c->kf + (size_t)l * B * seq_stride,
                     c->vf + (size_t)l * B * seq_stride, c->L.fast_len, seq_stride, 1, c->L.chunk, pend,
                     k > 1 || l + 1 < g.n_layers_fast);
    // head on each sequence's last row
    out.push_back(rec(t_norm(c->cf.x + (k == 1 ? d : 0), k == 1 ? 2 * d : d, B, d, c->fast_fn, g.rms_eps, c->bxh[1],
                             c->bxl[1], nullptr, pend),
                      K_OTHER, k));
    out.push_back(rec(t_gemm(c->wq, c->fast_head, c->fast_head_scale, g.vocab_res, d, B, c->bxh[1],
                             c->bxl[1], c->flogits + (size_t)k * c->L.vmax, fc * c->L.vmax, 0, c->bgp[1],
                             c->L.bgp_floats[1]),
                      K_HEAD, k));
    Task t = none_task();
    t.kind = T_COMMIT_ROWS;
    RowsCommitArgs& r = t.rows;
    r = rows_commit(c, k, c->flogits + (size_t)k * c->L.vmax, fc * c->L.vmax, g.vocab_res);
    r.pos_inc = k == g.n_res ? c->pos_f : nullptr;
    r.next_table = k < g.n_res ? c->fast_emb[k] : nullptr;
    r.next_rows = g.vocab_res;
    r.next_x = c->cf.x;
    r.next_stride = d;
    out.push_back(rec(t, K_OTHER, k));
  }
  return out;
}

void plan_single(Plan& p, const std::vector<TaskRec>& chain) {
  for (const TaskRec& r : chain) {
    p.tasks.push_back(r.t);
    p.kind.push_back(r.kind);
    p.layer.push_back(r.layer);
  }
}

// a launch dar_time_kind selected: one-row launches of that kind (the fast
// AR's two-row first pass is left out)
bool timed(const dar_ctx* c, const Plan& p, size_t i) {
  return c->timed_kind >= 0 && p.kind[i] == c->timed_kind && !(p.layer[i] >= 1000 && p.layer[i] < 2000);
}

// Batched slow attention of the coming frame, whose rows attend over at most
// tmax positions: the splits that covers, with longer splits when the launch
// has work enough (measured at 16 and 64 sequences: 64 positions per split
// win at about 1k workgroups, 256 from there on).
void set_live_attention(dar_ctx* c, int tmax) {
  const int n_kv = c->cfg.n_heads_kv;
  int chunk = c->L.chunk_rows;
  for (int cand : {4 * c->L.chunk_rows, 2 * c->L.chunk_rows}) {
    if ((long long)c->B * n_kv * ((tmax + cand - 1) / cand) >= 1024) {
      chunk = cand;
      break;
    }
  }
  if (c->paged) chunk = std::min(chunk, c->L.page_len);  // a split stays within one page
  c->attn_chunk_live = chunk;
  c->attn_splits_live = (tmax + chunk - 1) / chunk;
}

// live: eager launches may trim the batched slow attention to the splits the
// coming frame's longest sequence has (a captured graph keeps them all)
hipError_t enqueue_plan(dar_ctx* c, const Plan& p, hipStream_t s, size_t ev_base = SIZE_MAX, bool live = true) {
  const int wt = c->wq;
  for (size_t i = 0; i < p.launches(); ++i) {
    hipEvent_t before = nullptr, after = nullptr;
    if (ev_base != SIZE_MAX) {
      before = c->events[2 * (ev_base + i)];
      after = c->events[2 * (ev_base + i) + 1];
    } else if (live && timed(c, p, i)) {  // (eager launches only, not under capture)
      while (c->tpool.size() < c->tused + 2) {
        hipEvent_t ev;
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) return e;
        c->tpool.push_back(ev);
      }
      before = c->tpool[c->tused];
      after = c->tpool[c->tused + 1];
      c->tused += 2;
    }
    const Task& t = p.tasks[i];
    hipError_t e;
    // (the batched slow attention: the plan's split attention followed by its
    // combine, nsplit_rows > 1; the fast AR's attention has one split)
    if (live && c->B > 1 && c->attn_splits_live > 0 && c->L.nsplit_rows > 1 &&
        (t.kind == T_ATTN || t.kind == T_COMBINE) && t.attn.nsplit_max == c->L.nsplit_rows) {
      // split s of row m covers positions [s chunk, (s + 1) chunk): rows with
      // fewer positions leave their later splits empty either way; at least
      // two splits, as the combine launch merges split partials
      Task trimmed = t;
      trimmed.attn.chunk = c->attn_chunk_live;
      trimmed.attn.nsplit_max = std::max(2, c->attn_splits_live);
      e = launch_task(wt, trimmed, s, before, after);
    } else {
      e = launch_task(wt, t, s, before, after);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// replay the plan's graph on s (captured on s the first time), or launch eagerly
int run_plan(dar_ctx* c, Plan& p, hipStream_t s, const char* what) {
  if (p.launches() == 0) return DAR_OK;
  if (!c->use_graph) {
    DAR_HIP(c, enqueue_plan(c, p, s), what);
    return DAR_OK;
  }
  if (!p.exec) {
    for (size_t i = 0; i < p.launches(); ++i)
      DAR_HIP(c, prepare_task(c->wq, p.tasks[i]), "prepare launch");
    DAR_HIP(c, hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "begin capture");
    hipError_t e = enqueue_plan(c, p, s, SIZE_MAX, false);
    hipGraph_t g = nullptr;
    hipError_t e2 = hipStreamEndCapture(s, &g);
    if (e != hipSuccess) {
      if (g) (void)hipGraphDestroy(g);
      return hip_fail(c, e, what);
    }
    if (e2 != hipSuccess) return hip_fail(c, e2, "end capture");
    p.graph = g;
    DAR_HIP(c, hipGraphInstantiate(&p.exec, p.graph, nullptr, nullptr, 0), "instantiate graph");
  }
  DAR_HIP(c, hipGraphLaunch(p.exec, s), what);
  return DAR_OK;
}

int copy_outputs(dar_ctx* c, hipStream_t s, int32_t* codes_out, float* logits_out) {
  const dar_config& g = c->cfg;
  const size_t fc = frame_codes(&g);
  if (codes_out) DAR_HIP(c, launch_copy_i32(c->pred, codes_out, (int)fc * c->B, s), "copy codes");
  if (logits_out) {
    for (size_t r = 0; r < fc * c->B; ++r) {
      const int V = (r % fc == 0) ? g.vocab_c0 : g.vocab_res;
      DAR_HIP(c,
              hipMemcpyAsync(logits_out + r * c->L.vmax, c->flogits + r * c->L.vmax, sizeof(float) * V,
                             hipMemcpyDeviceToDevice, s),
              "copy logits");
    }
  }
  return DAR_OK;
}

int set_force(dar_ctx* c, hipStream_t s, const int32_t* forced) {
  const int fc = frame_codes(&c->cfg) * c->B;
  if (forced) {
    DAR_HIP(c, launch_set_forced(forced, fc, c->forced, c->flags + 0, s), "set forced");
    c->force_dev = true;
  } else if (c->force_dev) {
    DAR_HIP(c, launch_set_forced(nullptr, fc, c->forced, c->flags + 0, s), "clear forced");
    c->force_dev = false;
  }
  return DAR_OK;
}

// One pipeline step: the fast chain finishes frame i (commit c0, fast AR,
// outputs) while the slow chain computes the slow step and codebook-0 head of
// frame i+1 (when that position exists), starting once c0 is committed.
int pipeline_step(dar_ctx* c, const int32_t* forced, int32_t* codes_out, float* logits_out, bool run_slow) {
  hipStream_t sf = c->cf.s, ss = c->cs.s;
  DAR_HIP(c, hipEventRecord(c->ev_start, c->stream), "record start");
  DAR_HIP(c, hipStreamWaitEvent(sf, c->ev_start, 0), "wait start");
  DAR_HIP(c, hipStreamWaitEvent(sf, c->ev_s_done, 0), "wait slow chain");
  int st = set_force(c, sf, forced);
  if (st != DAR_OK) return st;
  st = run_plan(c, c->p_c0, sf, "commit codebook 0");
  if (st != DAR_OK) return st;
  DAR_HIP(c, hipEventRecord(c->ev_c0, sf), "record c0");
  if (run_slow) {
    DAR_HIP(c, hipStreamWaitEvent(ss, c->ev_c0, 0), "slow waits c0");
    st = run_plan(c, c->p_slow, ss, "slow chain");
    if (st != DAR_OK) return st;
    DAR_HIP(c, hipEventRecord(c->ev_s_done, ss), "record slow done");
  }
  st = run_plan(c, c->p_fast, sf, "fast chain");
  if (st != DAR_OK) return st;
  st = copy_outputs(c, sf, codes_out, logits_out);
  if (st != DAR_OK) return st;
  DAR_HIP(c, hipEventRecord(c->ev_f_done, sf), "record fast done");
  DAR_HIP(c, hipStreamWaitEvent(c->stream, c->ev_f_done, 0), "join fast");
  DAR_HIP(c, hipStreamWaitEvent(c->stream, c->ev_s_done, 0), "join slow");
  return DAR_OK;
}

// The slow AR over the prompt in blocks of up to kPrefillRows positions:
// every projection is one GEMM over the block's rows (each weight matrix read
// once per block), attention is causal over the cache (earlier blocks) and the
// block itself. Then the codebook-0 head on the last position, which leaves
// pos_s = n; frame 0 sits at position n - 1.
int prefill_blocks(dar_ctx* c, const int32_t* tokens, int n, hipStream_t s, int seq) {
  const dar_config& g = c->cfg;
  const Layout& L = c->L;
  const int d = g.d_model, qw = g.n_heads_q * g.head_dim, F = g.ffn_dim;
  const int qkv_rows = (g.n_heads_q + 2 * g.n_heads_kv) * g.head_dim;
  const int wt = c->wq;
  char* b = c->ws;
  float* px = reinterpret_cast<float*>(b + L.px);
  uint16_t* xh = reinterpret_cast<uint16_t*>(b + L.pxh);
  uint16_t* xl = reinterpret_cast<uint16_t*>(b + L.pxl);
  float* pq = reinterpret_cast<float*>(b + L.pq);
  float* po = reinterpret_cast<float*>(b + L.po);
  float* pgp = reinterpret_cast<float*>(b + L.pgp);
  int* ppos = reinterpret_cast<int*>(b + L.ppos);
  const size_t per_layer = (size_t)g.n_heads_kv * g.max_len * g.head_dim;
  // paged: the layer's page pool, positions through sequence seq's block-table row
  const long long page_stride = (long long)g.n_heads_kv * L.page_len * g.head_dim;
  const PageMap pm = c->paged ? PageMap{c->ptable, L.page_shift, L.pages_per_seq, seq} : PageMap{nullptr, 0, 0, 0};
  float* pgp2 = pgp + L.pgp_floats;  // second region: W3's sums beside W1's
  auto gemm = [&](const void* W, const float* scale, int N, int K, int M, float* y, int acc, float* part,
                  int defer) {
    GemmArgs a{};
    a.W = W;
    a.scale = c->quant ? scale : nullptr;
    a.N = N;
    a.K = K;
    a.M = M;
    a.xh = xh;
    a.xl = xl;
    a.y = y;
    a.y_stride = N;
    a.accumulate = acc;
    a.part = part;
    a.defer = defer;
    return launch_gemm(wt, a, L.pgp_floats, s);
  };
  // K-split sums a deferred projection left in part, for the row kernel that reads it
  auto sums = [&](float* part, int N, int K, int M) {
    return PartSum{part, gemm_launch_splits(wt, M, N, K, L.pgp_floats), (long long)M * N};
  };
  int M = 0;
  for (int p0 = 0; p0 < n; p0 += kPrefillRows) {
    M = std::min(kPrefillRows, n - p0);
    DAR_HIP(c, launch_embed_rows(c->w0, g.vocab_c0, d, tokens + p0, M, px, c->flags + 1, s), "prefill embed");
    DAR_HIP(c, launch_fill_i32(ppos, 1, p0, s), "prefill position");
    PartSum pend{nullptr, 0, 0};  // the previous layer's residual sums
    for (int l = 0; l < g.n_layers_slow; ++l) {
      const dar_layer_weights& w = c->slow[l];
      uint16_t* kc = c->paged ? c->ks + (size_t)l * L.n_pages * page_stride
                              : c->ks + ((size_t)l * c->B + seq) * per_layer;  // layer l of sequence seq
      uint16_t* vc = c->paged ? c->vs + (size_t)l * L.n_pages * page_stride
                              : c->vs + ((size_t)l * c->B + seq) * per_layer;
      const int cache_len = c->paged ? L.page_len : g.max_len;
      DAR_HIP(c,
              launch_norm_split(px, d, M, d, static_cast<const uint16_t*>(w.attn_norm), g.rms_eps, xh, xl, s, nullptr,
                                pend),
              "prefill attn norm");
      DAR_HIP(c, gemm(w.wqkv, w.wqkv_scale, qkv_rows, d, M, nullptr, 0, pgp, 1), "prefill qkv");
      DAR_HIP(c,
              launch_rope_rows(nullptr, M, p0, g.n_heads_q, g.n_heads_kv, g.head_dim, c->rope, pq, kc, vc, cache_len,
                               s, nullptr, nullptr, c->paged ? page_stride : 0, sums(pgp, qkv_rows, d, M), pm),
              "prefill rope");
      Task t = none_task();  // every byte zero: the union's members past the first are not covered by {}
      t.kind = T_ATTN;
      t.M = M;
      AttnArgs& aa = t.attn;
      aa.q = pq;
      aa.q_stride = qw;
      aa.K = kc;
      aa.V = vc;
      aa.cache_len = cache_len;
      if (c->paged) {
        aa.seq_stride = page_stride;
        aa.page_table = pm.table;
        aa.page_shift = pm.shift;
        aa.pages_per_seq = pm.per_seq;
        aa.seq0 = seq;
      }
      aa.pos = ppos;
      aa.n_heads_q = g.n_heads_q;
      aa.n_heads_kv = g.n_heads_kv;
      aa.head_dim = g.head_dim;
      // 128-position splits (within a page when paged): a first block of 128
      // prompt positions is one split with no merge launch (a prompt block
      // 6.4 -> 5.9 ms, 16 prompts of 143..510 ids 301 -> 284 ms against 64)
      aa.chunk = c->paged ? std::min(kPrefillChunk, L.page_len) : kPrefillChunk;
      aa.nsplit_max = (p0 + M + aa.chunk - 1) / aa.chunk;  // splits of the block's longest row
      aa.M = M;
      aa.part = reinterpret_cast<float*>(b + L.patt);
      aa.cnt = aa.nsplit_max > 1 ? reinterpret_cast<unsigned*>(b + L.pcnt) : nullptr;
      aa.out = po;
      aa.out_stride = qw;
      aa.out_hi = xh;  // the O projection's input split
      aa.out_lo = xl;
      DAR_HIP(c, launch_task(wt, t, s), "prefill attention");
      DAR_HIP(c, gemm(w.wo, w.wo_scale, d, qw, M, nullptr, 0, pgp, 1), "prefill wo");
      DAR_HIP(c,
              launch_norm_split(px, d, M, d, static_cast<const uint16_t*>(w.ffn_norm), g.rms_eps, xh, xl, s, nullptr,
                                sums(pgp, d, qw, M)),
              "prefill ffn norm");
      DAR_HIP(c, gemm(w.w1, w.w1_scale, F, d, M, nullptr, 0, pgp, 1), "prefill w1");
      DAR_HIP(c, gemm(w.w3, w.w3_scale, F, d, M, nullptr, 0, pgp2, 1), "prefill w3");
      DAR_HIP(c, launch_silu_split(nullptr, nullptr, M, F, xh, xl, s, sums(pgp, F, d, M), sums(pgp2, F, d, M)),
              "prefill silu");
      // the block's last residual is summed in place (its last row leaves the block)
      const bool last = l + 1 == g.n_layers_slow;
      DAR_HIP(c, gemm(w.w2, w.w2_scale, d, F, M, last ? px : nullptr, 1, pgp, last ? 0 : 1), "prefill w2");
      pend = last ? PartSum{nullptr, 0, 0} : sums(pgp, d, F, M);
    }
  }
  // the last position's residual becomes the sequence's slow row (the head's input)
  DAR_HIP(c, hipMemcpyAsync(c->cs.x + (size_t)seq * d, px + (size_t)(M - 1) * d, sizeof(float) * d,
                            hipMemcpyDeviceToDevice, s),
          "prefill last row");
  return DAR_OK;
}

void free_plan(Plan& p) {
  if (p.exec) (void)hipGraphExecDestroy(p.exec);
  if (p.graph) (void)hipGraphDestroy(p.graph);
  p.exec = nullptr;
  p.graph = nullptr;
}

}  // namespace

extern "C" {

int dar_workspace_bytes(const dar_config* cfg, size_t* bytes_out) {
  std::string why;
  if (!bytes_out) return DAR_E_INVAL;
  const int st = validate_config(cfg, why);
  if (st != DAR_OK) {
    g_create_error = why;
    return st;
  }
  *bytes_out = make_layout(cfg).total;
  return DAR_OK;
}

namespace {

// Paging parameters: page_len a power of two in [64, 2^20], at most
// kMaxPagesPerSeq pages per sequence, page 0 reserved, the many-row path.
int validate_paging(const dar_config* cfg, const dar_paging* pg, std::string& why) {
  if (!pg) {
    why = "paging is NULL";
    return DAR_E_INVAL;
  }
  const int P = pg->page_len;
  if (P < kAttnChunkDefault || P > (1 << 20) || (P & (P - 1))) {
    why = "page_len must be a power of two in [64, 2^20]";
    return DAR_E_INVAL;
  }
  if (pg->n_pages < 2) {
    why = "n_pages must be >= 2 (page 0 parks free slots)";
    return DAR_E_INVAL;
  }
  if ((cfg->max_len + P - 1) / P > kMaxPagesPerSeq) {
    why = "max_len / page_len above 64 pages per sequence";
    return DAR_E_UNSUPPORTED;
  }
  if (cfg->max_batch < 2) {
    why = "a paged context needs max_batch >= 2";
    return DAR_E_UNSUPPORTED;
  }
  return DAR_OK;
}

int create_impl(const dar_config* cfg, const dar_weights* w, void* workspace, size_t ws_bytes, void* stream,
                const dar_paging* paging, dar_ctx** ctx_out);

}  // namespace

int dar_create(const dar_config* cfg, const dar_weights* w, void* workspace, size_t ws_bytes, void* stream,
               dar_ctx** ctx_out) {
  return create_impl(cfg, w, workspace, ws_bytes, stream, nullptr, ctx_out);
}

int dar_workspace_bytes_paged(const dar_config* cfg, const dar_paging* paging, size_t* bytes_out) {
  std::string why;
  int st = validate_config(cfg, why);
  if (st == DAR_OK) st = validate_paging(cfg, paging, why);
  if (st != DAR_OK) {
    g_create_error = why;
    return st;
  }
  if (!bytes_out) return DAR_E_INVAL;
  *bytes_out = make_layout(cfg, Paging{paging->page_len, paging->n_pages}).total;
  return DAR_OK;
}

int dar_create_paged(const dar_config* cfg, const dar_paging* paging, const dar_weights* w, void* workspace,
                     size_t ws_bytes, void* stream, dar_ctx** ctx_out) {
  if (!paging) {
    g_create_error = "paging is NULL";
    if (ctx_out) *ctx_out = nullptr;
    return DAR_E_INVAL;
  }
  return create_impl(cfg, w, workspace, ws_bytes, stream, paging, ctx_out);
}

namespace {

int create_impl(const dar_config* cfg, const dar_weights* w, void* workspace, size_t ws_bytes, void* stream,
                const dar_paging* paging, dar_ctx** ctx_out) {
  std::string why;
  if (!ctx_out) {
    g_create_error = "ctx_out is NULL";
    return DAR_E_INVAL;
  }
  *ctx_out = nullptr;
  int st = validate_config(cfg, why);
  if (st == DAR_OK && paging) st = validate_paging(cfg, paging, why);
  if (st != DAR_OK) {
    g_create_error = why;
    return st;
  }
  if (!w) {
    g_create_error = "weights is NULL";
    return DAR_E_INVAL;
  }
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))) {
    g_create_error = "workspace is NULL or not 256-byte aligned";
    return DAR_E_INVAL;
  }
  const Layout L = make_layout(cfg, paging ? Paging{paging->page_len, paging->n_pages} : Paging{0, 0});
  if (ws_bytes < L.total) {
    g_create_error = "workspace smaller than dar_workspace_bytes()";
    return DAR_E_WORKSPACE;
  }
  const bool scaled = has_scales(cfg->wtype);
  if (!w->w0 || !aligned16(w->w0) || !w->slow || !w->slow_final_norm) {
    g_create_error = "w0, slow layers or slow_final_norm missing or misaligned";
    return DAR_E_INVAL;
  }
  for (int l = 0; l < cfg->n_layers_slow; ++l) {
    st = check_layer(w->slow[l], scaled, why, "slow", l);
    if (st != DAR_OK) {
      g_create_error = why;
      return st;
    }
  }
  if (has_fast(cfg)) {
    if (!w->fast || !w->fast_emb || !w->fast_final_norm || !w->fast_head || !aligned16(w->fast_head) ||
        (scaled && !w->fast_head_scale)) {
      g_create_error = "fast AR weights missing or misaligned";
      return DAR_E_INVAL;
    }
    for (int k = 0; k < cfg->n_res; ++k) {
      if (!w->fast_emb[k]) {
        g_create_error = "fast_emb entry is NULL";
        return DAR_E_INVAL;
      }
    }
    for (int l = 0; l < cfg->n_layers_fast; ++l) {
      st = check_layer(w->fast[l], scaled, why, "fast", l);
      if (st != DAR_OK) {
        g_create_error = why;
        return st;
      }
    }
  }

  dar_ctx* c = new dar_ctx();
  c->cfg = *cfg;
  c->L = L;
  c->quant = scaled;
  c->wq = wtype_of(cfg->wtype);
  c->slow.assign(w->slow, w->slow + cfg->n_layers_slow);
  if (has_fast(cfg)) {
    c->fast.assign(w->fast, w->fast + cfg->n_layers_fast);
    for (int k = 0; k < cfg->n_res; ++k) c->fast_emb.push_back(static_cast<const uint16_t*>(w->fast_emb[k]));
    c->fast_fn = static_cast<const uint16_t*>(w->fast_final_norm);
    c->fast_head = w->fast_head;
    c->fast_head_scale = w->fast_head_scale;
  }
  c->w0 = static_cast<const uint16_t*>(w->w0);
  c->slow_fn = static_cast<const uint16_t*>(w->slow_final_norm);
  c->stream = static_cast<hipStream_t>(stream);
  c->ws = static_cast<char*>(workspace);
  char* b = c->ws;
  Chain* chains[2] = {&c->cs, &c->cf};
  for (int i = 0; i < 2; ++i) {
    chains[i]->x = reinterpret_cast<float*>(b + L.x[i]);
    chains[i]->q = reinterpret_cast<float*>(b + L.q[i]);
    chains[i]->o = reinterpret_cast<float*>(b + L.o[i]);
    chains[i]->h = reinterpret_cast<float*>(b + L.h[i]);
    chains[i]->part = reinterpret_cast<float*>(b + L.part[i]);
  }
  c->cs.cnt = reinterpret_cast<unsigned*>(b + L.acnt);
  c->ht = reinterpret_cast<float*>(b + L.ht);
  c->logits0 = reinterpret_cast<float*>(b + L.logits0);
  c->flogits = reinterpret_cast<float*>(b + L.flogits);
  c->slots0 = reinterpret_cast<unsigned long long*>(b + L.slots0);
  c->slotsf = reinterpret_cast<unsigned long long*>(b + L.slotsf);
  c->pred = reinterpret_cast<int*>(b + L.pred);
  c->committed = reinterpret_cast<int*>(b + L.committed);
  c->forced = reinterpret_cast<int*>(b + L.forced);
  c->flags = reinterpret_cast<int*>(b + L.flags);
  c->B = cfg->max_batch;
  c->pos_hb.assign(c->B, 0);
  c->pos_s = reinterpret_cast<int*>(b + L.pos);
  c->pos_f = c->pos_s + c->B;
  c->win_lo = c->pos_s + 2 * c->B;
  if (c->B > 1) {
    for (int ch = 0; ch < 2; ++ch) {
      c->bgp[ch] = reinterpret_cast<float*>(b + L.bgp[ch]);
      c->bxh[ch] = reinterpret_cast<uint16_t*>(b + L.bxh[ch]);
      c->bxl[ch] = reinterpret_cast<uint16_t*>(b + L.bxl[ch]);
    }
    c->seq_ident = reinterpret_cast<int*>(b + L.rows);
    c->p1_pos = c->seq_ident + c->B;
    c->p1_seq = c->p1_pos + 2 * c->B;
    c->pk_pos = c->p1_seq + 2 * c->B;
  }
  if (paging) {
    c->paged = true;
    c->ptable = reinterpret_cast<int*>(b + L.ptable);
    c->active = reinterpret_cast<int*>(b + L.active);
    for (int p = L.n_pages - 1; p >= 1; --p) c->free_pages.push_back(p);  // handed out from page 1 up
    c->slot_pages.assign(c->B, {});
    c->slot_on.assign(c->B, 0);
  }
  c->seqpos = reinterpret_cast<int*>(b + L.seqpos);
  c->ring = reinterpret_cast<int*>(b + L.ring);
  c->rope = reinterpret_cast<float2*>(b + L.rope);
  c->ks = reinterpret_cast<uint16_t*>(b + L.ks);
  c->vs = reinterpret_cast<uint16_t*>(b + L.vs);
  c->kf = reinterpret_cast<uint16_t*>(b + L.kf);
  c->vf = reinterpret_cast<uint16_t*>(b + L.vf);

  // launch plans: commit of codebook 0, the fast AR, the slow step with its
  // codebook-0 head, and the slow step alone (prompt positions before the last)
  if (c->B == 1) {
    plan_single(c->p_c0, commit0_chain(c));
    plan_single(c->p_fast, fast_chain(c));
    plan_single(c->p_slow, slow_chain(c, true));
  } else {
    plan_single(c->p_c0, commit0_chain_rows(c));
    plan_single(c->p_fast, fast_chain_rows(c));
    plan_single(c->p_slow, slow_chain_rows(c));
  }

  auto fail = [&](hipError_t e, const char* what) {
    g_create_error = std::string(what) + ": " + hipGetErrorString(e);
    for (Chain* ch : chains)
      if (ch->s) (void)hipStreamDestroy(ch->s);
    for (hipEvent_t ev : {c->ev_start, c->ev_c0, c->ev_f_done, c->ev_s_done})
      if (ev) (void)hipEventDestroy(ev);
    delete c;
    return DAR_E_HIP;
  };
  hipError_t e;
  for (Chain* ch : chains)
    if ((e = hipStreamCreateWithFlags(&ch->s, hipStreamNonBlocking)) != hipSuccess) return fail(e, "create stream");
  for (hipEvent_t* ev : {&c->ev_start, &c->ev_c0, &c->ev_f_done, &c->ev_s_done})
    if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return fail(e, "create event");

  // RoPE table: angle p * base^(-2i/hd) in double, cos/sin stored as fp32.
  const int half = cfg->head_dim / 2;
  std::vector<float2> rope((size_t)L.rope_len * half);
  for (int p = 0; p < L.rope_len; ++p) {
    for (int i = 0; i < half; ++i) {
      const double th = (double)p * std::pow(cfg->rope_base, -2.0 * i / cfg->head_dim);
      rope[(size_t)p * half + i] = make_float2((float)std::cos(th), (float)std::sin(th));
    }
  }
  std::vector<int> seq(L.seq_len);
  for (int i = 0; i < L.seq_len; ++i) seq[i] = i;
  // batched rows: sequence ids, first fast pass (positions 0, 1 of each
  // sequence), later passes (position k of each sequence)
  std::vector<int> rows;
  if (c->B > 1) {
    const int B = c->B;
    for (int i = 0; i < B; ++i) rows.push_back(i);
    for (int i = 0; i < 2 * B; ++i) rows.push_back(i % 2);
    for (int i = 0; i < 2 * B; ++i) rows.push_back(i / 2);
    for (int k = 0; k <= cfg->n_res; ++k)
      for (int i = 0; i < B; ++i) rows.push_back(k);
  }
  // zero everything from the activations to the ring (slots, flags, positions included)
  const size_t zero_words = L.rope / 4;
  if ((e = launch_fill_u32(reinterpret_cast<unsigned*>(b), zero_words, c->stream)) != hipSuccess)
    return fail(e, "zero workspace");
  if ((e = hipMemcpyAsync(c->rope, rope.data(), rope.size() * sizeof(float2), hipMemcpyHostToDevice, c->stream)) !=
      hipSuccess)
    return fail(e, "upload rope table");
  if ((e = hipMemcpyAsync(c->seqpos, seq.data(), seq.size() * sizeof(int), hipMemcpyHostToDevice, c->stream)) !=
      hipSuccess)
    return fail(e, "upload positions");
  if (!rows.empty() && (e = hipMemcpyAsync(c->seq_ident, rows.data(), rows.size() * sizeof(int),
                                           hipMemcpyHostToDevice, c->stream)) != hipSuccess)
    return fail(e, "upload rows");
  // paged: every slot free, its block-table row on the parking page
  if (c->paged && ((e = launch_fill_i32(c->ptable, c->B * L.pages_per_seq, 0, c->stream)) != hipSuccess ||
                   (e = launch_fill_i32(c->active, c->B, 0, c->stream)) != hipSuccess))
    return fail(e, "clear block table");
  if ((e = hipStreamSynchronize(c->stream)) != hipSuccess) return fail(e, "synchronize create");
  if ((e = hipEventRecord(c->ev_s_done, c->cs.s)) != hipSuccess) return fail(e, "record event");
  if ((e = hipEventRecord(c->ev_f_done, c->cf.s)) != hipSuccess) return fail(e, "record event");
  *ctx_out = c;
  return DAR_OK;
}

// ---- paged contexts: continuous batching over a shared pool of KV pages

// One launch on the slow stream: slot b's block-table row (its pages, the
// parking page 0 beyond them) and, with set_state, its positions and flag.
hipError_t slot_update(dar_ctx* c, int b, bool set_state, int pos_slow, int pos_frame, int win_lo, int active) {
  SlotState st{};
  st.b = b;
  st.per_seq = c->L.pages_per_seq;
  for (int i = 0; i < st.per_seq; ++i)
    st.pages[i] = i < (int)c->slot_pages[b].size() ? c->slot_pages[b][i] : 0;
  st.set_state = set_state ? 1 : 0;
  st.pos_slow = pos_slow;
  st.pos_frame = pos_frame;
  st.win_lo = win_lo;
  st.active = active;
  return launch_slot_state(c->ptable, c->pos_s, c->pos_f, c->win_lo, c->active, st, c->cs.s);
}

// the slow stream starts after the caller's queued work and the last fast chain
int slow_stream_begin(dar_ctx* c) {
  DAR_HIP(c, hipEventRecord(c->ev_start, c->stream), "record start");
  DAR_HIP(c, hipStreamWaitEvent(c->cs.s, c->ev_start, 0), "wait start");
  DAR_HIP(c, hipStreamWaitEvent(c->cs.s, c->ev_f_done, 0), "wait fast chain");
  return DAR_OK;
}

// ... and the caller's stream waits for it
int slow_stream_end(dar_ctx* c) {
  DAR_HIP(c, hipEventRecord(c->ev_s_done, c->cs.s), "record slow done");
  DAR_HIP(c, hipStreamWaitEvent(c->stream, c->ev_s_done, 0), "join slow");
  return DAR_OK;
}

// A frame of every active slot: slot b returns its frame at position
// pos_hb[b] and its slow step runs at pos_hb[b] + 1, whose page is taken from
// the pool first when the sequence enters a new page.
int paged_frame(dar_ctx* c, const int32_t* forced, int32_t* codes_out, float* logits_out) {
  const int P = c->L.page_len;
  int n_active = 0, need = 0, tmax = 1;
  for (int b = 0; b < c->B; ++b) {
    if (!c->slot_on[b]) continue;
    ++n_active;
    const int next = c->pos_hb[b] + 1;
    if (next >= c->cfg.max_len) {
      c->err = "slot " + std::to_string(b) + " reached max_len - 1 (remove it with dar_seq_remove)";
      return DAR_E_CAPACITY;
    }
    if (next / P >= (int)c->slot_pages[b].size()) ++need;
    tmax = std::max(tmax, next + 1);
  }
  if (n_active == 0) {
    c->err = "no sequence in the context (dar_seq_add)";
    return DAR_E_STATE;
  }
  if (need > (int)c->free_pages.size()) {
    c->err = "KV page pool exhausted: " + std::to_string(need) + " pages needed, " +
             std::to_string(c->free_pages.size()) + " free";
    return DAR_E_CAPACITY;
  }
  // new pages go into the block table on the slow stream, after the previous
  // slow step and before this frame's
  for (int b = 0; b < c->B; ++b) {
    if (!c->slot_on[b] || (c->pos_hb[b] + 1) / P < (int)c->slot_pages[b].size()) continue;
    c->slot_pages[b].push_back(c->free_pages.back());
    c->free_pages.pop_back();
    DAR_HIP(c, slot_update(c, b, false, 0, 0, 0, 0), "block table");
  }
  set_live_attention(c, tmax);
  const int st = pipeline_step(c, forced, codes_out, logits_out, true);
  if (st != DAR_OK) return st;
  for (int b = 0; b < c->B; ++b)
    if (c->slot_on[b]) c->pos_hb[b] += 1;
  return DAR_OK;
}

// dar_seq_add's device work on the slow stream: the slot's table row and
// state, the prompt's prefill through its pages, the codebook-0 head on the
// last prompt position (h_t kept for the fast AR)
int seq_add_launch(dar_ctx* c, int slot, const int32_t* tokens, int len) {
  const dar_config& g = c->cfg;
  const int d = g.d_model;
  int st = slow_stream_begin(c);
  if (st != DAR_OK) return st;
  hipStream_t s = c->cs.s;
  // frame 0 sits at the last prompt position len - 1; the next slow step at len
  DAR_HIP(c, slot_update(c, slot, true, len, len - 1, len - 1, 1), "slot state");
  st = prefill_blocks(c, tokens, len, s, slot);
  if (st != DAR_OK) return st;
  DAR_HIP(c,
          launch_task(c->wq, t_norm(c->cs.x + (size_t)slot * d, d, 1, d, c->slow_fn, g.rms_eps, c->bxh[0], c->bxl[0],
                                    c->ht + (size_t)slot * d),
                      s),
          "slot head norm");
  DAR_HIP(c,
          launch_task(c->wq, t_gemm(W_BF16, c->w0, nullptr, g.vocab_c0, d, 1, c->bxh[0], c->bxl[0],
                                    c->logits0 + (size_t)slot * g.vocab_c0, g.vocab_c0, 0, c->bgp[0],
                                    c->L.bgp_floats[0]),
                      s),
          "slot head");
  return slow_stream_end(c);
}

}  // namespace

int dar_seq_add(dar_ctx* c, int32_t slot, const int32_t* tokens, int32_t len) {
  if (!c) return DAR_E_INVAL;
  if (!c->paged) {
    c->err = "dar_seq_add needs a paged context (dar_create_paged)";
    return DAR_E_STATE;
  }
  if (slot < 0 || slot >= c->B || !tokens || len < 1) {
    c->err = "slot out of range, tokens NULL or len < 1";
    return DAR_E_INVAL;
  }
  if (c->slot_on[slot]) {
    c->err = "slot already holds a sequence";
    return DAR_E_STATE;
  }
  if (len >= c->cfg.max_len) {
    c->err = "prompt length must be below max_len";
    return DAR_E_CAPACITY;
  }
  const int P = c->L.page_len;
  const int need = (len + P - 1) / P;
  if (need > (int)c->free_pages.size()) {
    c->err = "KV page pool exhausted: " + std::to_string(need) + " pages needed, " +
             std::to_string(c->free_pages.size()) + " free";
    return DAR_E_CAPACITY;
  }
  for (int i = 0; i < need; ++i) {
    c->slot_pages[slot].push_back(c->free_pages.back());
    c->free_pages.pop_back();
  }
  c->slot_on[slot] = 1;
  const int st = seq_add_launch(c, slot, tokens, len);
  if (st != DAR_OK) {
    // a HIP failure: the host state goes back to the slot being free (the
    // device may hold part of the work; the context should not be used further)
    for (int p : c->slot_pages[slot]) c->free_pages.push_back(p);
    c->slot_pages[slot].clear();
    c->slot_on[slot] = 0;
    return st;
  }
  c->pos_hb[slot] = len - 1;
  c->prefilled = true;
  return DAR_OK;
}

int dar_seq_remove(dar_ctx* c, int32_t slot) {
  if (!c) return DAR_E_INVAL;
  if (!c->paged) {
    c->err = "dar_seq_remove needs a paged context (dar_create_paged)";
    return DAR_E_STATE;
  }
  if (slot < 0 || slot >= c->B) {
    c->err = "slot out of range";
    return DAR_E_INVAL;
  }
  if (!c->slot_on[slot]) {
    c->err = "slot holds no sequence";
    return DAR_E_STATE;
  }
  int st = slow_stream_begin(c);
  if (st != DAR_OK) return st;
  // the pages return to the pool; the slot parks at position 0 of page 0
  for (int p : c->slot_pages[slot]) c->free_pages.push_back(p);
  c->slot_pages[slot].clear();
  c->slot_on[slot] = 0;
  c->pos_hb[slot] = 0;
  DAR_HIP(c, slot_update(c, slot, true, 0, 0, 0, 0), "slot state");
  return slow_stream_end(c);
}

int dar_pages_free(const dar_ctx* c, int32_t* n_free) {
  if (!c || !n_free) return DAR_E_INVAL;
  *n_free = c->paged ? (int32_t)c->free_pages.size() : 0;
  return DAR_OK;
}

int dar_prefill(dar_ctx* c, int32_t batch, const int32_t* tokens, const int32_t* lens_host, const int32_t* forced,
                int32_t* codes_out, float* logits_out) {
  if (!c) return DAR_E_INVAL;
  if (c->paged) {
    c->err = "a paged context takes its sequences one at a time (dar_seq_add)";
    return DAR_E_STATE;
  }
  if (!tokens || !lens_host) {
    c->err = "tokens and lens_host are required";
    return DAR_E_INVAL;
  }
  if (batch < 1) {
    c->err = "batch must be >= 1";
    return DAR_E_INVAL;
  }
  if (batch > c->cfg.max_batch) {
    c->err = "batch above max_batch";
    return DAR_E_CAPACITY;
  }
  if (batch != c->B) {
    c->err = c->B == 1 ? "batch must be 1" : "batch must equal max_batch (sequences decode in lockstep)";
    return DAR_E_INVAL;
  }
  int nmax = 0;
  for (int b = 0; b < batch; ++b) {
    const int n = lens_host[b];
    if (n < 1 || n >= c->cfg.max_len) {
      c->err = "prompt length must be in [1, max_len)";
      return n < 1 ? DAR_E_INVAL : DAR_E_CAPACITY;
    }
    nmax = std::max(nmax, n);
  }
  c->prefilled = false;
  hipStream_t s = c->cs.s;
  const int wt = c->wq;
  // the slow stream runs the prompts after anything already queued
  DAR_HIP(c, hipEventRecord(c->ev_start, c->stream), "record start");
  DAR_HIP(c, hipStreamWaitEvent(s, c->ev_start, 0), "wait start");
  DAR_HIP(c, hipStreamWaitEvent(s, c->ev_f_done, 0), "wait fast chain");
  size_t off = 0;
  for (int b = 0; b < batch; ++b) {
    const int st0 = prefill_blocks(c, tokens + off, lens_host[b], s, b);
    if (st0 != DAR_OK) return st0;
    off += lens_host[b];
  }
  // codebook-0 head on each sequence's last position (moves pos_s to the
  // prompt length); frame 0 sits at the last prompt position
  c->pos_init.assign(3 * c->B, 0);
  for (int b = 0; b < batch; ++b)
    c->pos_init[b] = c->pos_init[c->B + b] = c->pos_init[2 * c->B + b] = lens_host[b] - 1;
  DAR_HIP(c, hipMemcpyAsync(c->pos_s, c->pos_init.data(), sizeof(int) * 3 * c->B, hipMemcpyHostToDevice, s),
          "prefill positions");
  if (c->B == 1) {
    DAR_HIP(c, launch_task(wt, c->p_slow.tasks.back(), s), "prefill head");
  } else {
    // the slow chain's final norm, head and position step; the prompt rows
    // are complete, so the norm adds no pending layer sums
    const size_t nt = c->p_slow.tasks.size();
    for (size_t i = nt - 3; i < nt; ++i) {
      Task t = c->p_slow.tasks[i];
      if (t.kind == T_NORM_SPLIT) t.norm.add = PartSum{nullptr, 0, 0};
      DAR_HIP(c, launch_task(wt, t, s), "prefill head");
    }
  }
  DAR_HIP(c, hipEventRecord(c->ev_s_done, s), "record slow done");
  // the slow chain runs the longest sequence at position nmax
  set_live_attention(c, nmax + 1);
  const int st = pipeline_step(c, forced, codes_out, logits_out, nmax < c->cfg.max_len);
  if (st != DAR_OK) return st;
  for (int b = 0; b < batch; ++b) c->pos_hb[b] = lens_host[b];
  c->pos_host = nmax;
  c->prefilled = true;
  return DAR_OK;
}

int dar_decode_frame(dar_ctx* c, const int32_t* forced, int32_t* codes_out, float* logits_out) {
  if (!c) return DAR_E_INVAL;
  if (c->paged) return paged_frame(c, forced, codes_out, logits_out);
  if (!c->prefilled) {
    c->err = "decode before prefill";
    return DAR_E_STATE;
  }
  if (c->pos_host >= c->cfg.max_len) {
    c->err = "position reached max_len";
    return DAR_E_CAPACITY;
  }
  // the slow chain runs the longest sequence at position pos_host + 1
  set_live_attention(c, c->pos_host + 2);
  const int st = pipeline_step(c, forced, codes_out, logits_out, c->pos_host + 1 < c->cfg.max_len);
  if (st != DAR_OK) return st;
  c->pos_host += 1;
  for (int& p : c->pos_hb) p += 1;
  return DAR_OK;
}

int dar_destroy(dar_ctx* c) {
  if (!c) return DAR_OK;
  (void)hipStreamSynchronize(c->stream);
  for (Chain* ch : {&c->cs, &c->cf})
    if (ch->s) (void)hipStreamSynchronize(ch->s);
  for (Plan* p : {&c->p_c0, &c->p_fast, &c->p_slow}) free_plan(*p);
  for (hipEvent_t ev : c->events) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : c->tpool) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : {c->ev_start, c->ev_c0, c->ev_f_done, c->ev_s_done})
    if (ev) (void)hipEventDestroy(ev);
  for (Chain* ch : {&c->cs, &c->cf})
    if (ch->s) (void)hipStreamDestroy(ch->s);
  delete c;
  return DAR_OK;
}

int dar_reset(dar_ctx* c) {
  if (!c) return DAR_E_INVAL;
  if (c->paged) {
    for (int b = 0; b < c->B; ++b) {
      if (!c->slot_on[b]) continue;
      const int st = dar_seq_remove(c, b);
      if (st != DAR_OK) return st;
    }
  }
  DAR_HIP(c, launch_fill_i32(c->flags + 1, 1, 0, c->stream), "reset counters");
  c->pos_host = 0;
  std::fill(c->pos_hb.begin(), c->pos_hb.end(), 0);
  c->prefilled = false;
  return DAR_OK;
}

int dar_position(const dar_ctx* c, int32_t* pos_out) {
  if (!c || !pos_out) return DAR_E_INVAL;
  for (int b = 0; b < c->B; ++b) pos_out[b] = c->paged && !c->slot_on[b] ? -1 : c->pos_hb[b];
  return DAR_OK;
}

int dar_set_graph(dar_ctx* c, int32_t enable) {
  if (!c) return DAR_E_INVAL;
  c->use_graph = enable != 0;
  return DAR_OK;
}

int dar_codes(dar_ctx* c, int32_t first, int32_t count, int32_t* dst) {
  if (!c || !dst) return DAR_E_INVAL;
  if (first < 0 || count < 0 || (int64_t)first + count > c->cfg.max_len) {
    c->err = "ring range out of bounds";
    return DAR_E_INVAL;
  }
  if (count == 0) return DAR_OK;
  const int fc = frame_codes(&c->cfg) * c->B;
  DAR_HIP(c, launch_copy_i32(c->ring + (size_t)first * fc, dst, count * fc, c->stream), "copy ring");
  return DAR_OK;
}

int dar_nonfinite(dar_ctx* c, int32_t* count_out) {
  if (!c || !count_out) return DAR_E_INVAL;
  DAR_HIP(c, hipMemcpyAsync(count_out, c->flags + 1, sizeof(int), hipMemcpyDeviceToHost, c->stream), "read counter");
  DAR_HIP(c, hipStreamSynchronize(c->stream), "synchronize");
  return DAR_OK;
}

int dar_bytes_per_frame(const dar_config* cfg, int32_t T, double* bytes_out) {
  std::string why;
  if (!bytes_out || T < 0) return DAR_E_INVAL;
  const int st = validate_config(cfg, why);
  if (st != DAR_OK) return st;
  const double d = cfg->d_model, F = cfg->ffn_dim, qw = (double)cfg->n_heads_q * cfg->head_dim;
  const double qkv = (double)(cfg->n_heads_q + 2 * cfg->n_heads_kv) * cfg->head_dim;
  const double kvw = (double)cfg->n_heads_kv * cfg->head_dim;
  const double mats = qkv * d + d * qw + 3.0 * F * d;
  const double rows = qkv + d + 2.0 * F + d;
  const double norms = 2.0 * d;
  // bytes of a Linear matrix of r rows and e entries: bf16; one byte per
  // weight + an fp32 scale per row (fp8, int8); half a byte per weight + an
  // fp32 scale per 128 entries (int4)
  const int wt = wtype_of(cfg->wtype);
  auto mat = [&](double r, double e) {
    switch (wt) {
      case W_BF16: return 2.0 * e;
      case W_INT4: return 0.5 * e + 4.0 * e / 128.0;
      default: return e + 4.0 * r;
    }
  };
  const double Ls = cfg->n_layers_slow, Lf = cfg->n_layers_fast;
  double slow = Ls * mat(rows, mats) + 2.0 * (Ls * norms + d) + 2.0 * cfg->vocab_c0 * d;
  double fast = 0.0, fast_kv = 0.0;
  if (cfg->n_res > 0) {
    const double head = (double)cfg->vocab_res * d;
    fast = Lf * mat(rows, mats) + mat(cfg->vocab_res, head) + 2.0 * (Lf * norms + d);
    double positions = 0;
    for (int k = 1; k <= cfg->n_res; ++k) positions += k + 1;
    fast_kv = positions * Lf * 2.0 * kvw * 2.0;
  }
  const double kv = (double)cfg->n_layers_slow * 2.0 * kvw * 2.0 * T;
  *bytes_out = slow + cfg->n_res * fast + kv + fast_kv;
  return DAR_OK;
}

int dar_quantize_fp8_rows(const void* w, int32_t rows, int32_t cols, void* q, float* scale, void* stream) {
  if (!w || !q || !scale || rows < 1 || cols < 16 || cols % 16) return DAR_E_INVAL;
  hipError_t e = launch_quantize_fp8(static_cast<const uint16_t*>(w), rows, cols, static_cast<uint8_t*>(q), scale,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "quantize");
  return DAR_OK;
}

int dar_quantize_int8_rows(const void* w, int32_t rows, int32_t cols, void* q, float* scale, void* stream) {
  if (!w || !q || !scale || rows < 1 || cols < 16 || cols % 16) return DAR_E_INVAL;
  hipError_t e = launch_quantize_int8(static_cast<const uint16_t*>(w), rows, cols, static_cast<int8_t*>(q), scale,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "quantize");
  return DAR_OK;
}

int dar_quantize_int4_groups(const void* w, int32_t rows, int32_t cols, void* q, float* scale, void* stream) {
  if (!w || !q || !scale || rows < 1 || cols < 128 || cols % 128) return DAR_E_INVAL;
  hipError_t e = launch_quantize_int4(static_cast<const uint16_t*>(w), rows, cols, static_cast<uint8_t*>(q), scale,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "quantize");
  return DAR_OK;
}

const char* dar_status_string(int status) {
  switch (status) {
    case DAR_OK: return "ok";
    case DAR_E_INVAL: return "invalid argument";
    case DAR_E_STATE: return "invalid state";
    case DAR_E_CAPACITY: return "capacity exceeded";
    case DAR_E_HIP: return "HIP runtime error";
    case DAR_E_WORKSPACE: return "workspace too small";
    case DAR_E_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

const char* dar_last_error(const dar_ctx* c) { return c ? c->err.c_str() : g_create_error.c_str(); }

// Run one task alone (diagnostic entry points); waits for it.
static int run_single_task(const Task& t, int wtype, hipStream_t s, const char* what) {
  hipError_t e = launch_task(wtype, t, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(nullptr, e, what);
  return DAR_OK;
}

int dar_op_gemv(int32_t wtype, const void* W, const float* scale, int32_t rows, int32_t cols, const float* x,
                int32_t M, float* y, void* stream) {
  if (!W || !x || !y || rows < 1 || cols < 256 || cols % 256 || cols > 16384 || (M != 1 && M != 2))
    return DAR_E_INVAL;
  if (wtype != DAR_WTYPE_BF16 && !has_scales(wtype)) return DAR_E_INVAL;
  if (has_scales(wtype) && !scale) return DAR_E_INVAL;
  if (!aligned16(W) || !aligned16(x)) return DAR_E_INVAL;
  Task t = none_task();
  t.kind = T_GEMV;
  t.M = M;
  GemvArgs& a = t.gemv;
  a.W = W;
  a.scale = has_scales(wtype) ? scale : nullptr;
  a.rows = rows;
  a.K = cols;
  a.M = M;
  a.x = x;
  a.x_stride = cols;
  a.gain = nullptr;
  a.y = y;
  a.y_stride = rows;
  a.accumulate = 0;
  return run_single_task(t, wtype_of(wtype), static_cast<hipStream_t>(stream),
                         "gemv");
}

// Address of the current device's copy of `scratch`, looked up once per device
// with that device current (hipGetSymbolAddress) and kept for later calls.
static std::mutex g_noalloc_mu;
static void* g_noalloc_ptr[64] = {};

static hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return hipSuccess;
}

int dar_op_gemm_noalloc(int32_t wtype, const void* W, const float* scale, int32_t N, int32_t K, const float* x,
                        int32_t M, float* y, void* stream) {
  if (!W || !x || !y || N < 1 || K < 256 || K % 256 || K > 16384 || M < 1 || M > kPrefillRows) return DAR_E_INVAL;
  if (wtype != DAR_WTYPE_BF16 && !has_scales(wtype)) return DAR_E_INVAL;
  if (has_scales(wtype) && !scale) return DAR_E_INVAL;
  if (!aligned16(W) || !aligned16(x)) return DAR_E_INVAL;
  const size_t half_bytes = align_up((size_t)gemm_mpad(M) * K * sizeof(uint16_t));
  // the input halves must fit; the partial sums adapt to what is left (one
  // K split needs none). Within the shape limits above the halves take at
  // most 2 x 128 x 16384 x 2 bytes = 8 MiB.
  if (2 * half_bytes > DAR_NOALLOC_SCRATCH_BYTES) {
    g_create_error = "dar_op_gemm_noalloc: the input halves exceed the static scratch";
    return DAR_E_CAPACITY;
  }
  void* base = nullptr;
  hipError_t e = noalloc_scratch(&base);
  if (e != hipSuccess) return hip_fail(nullptr, e, "gemm scratch address");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* sc = static_cast<char*>(base);
  uint16_t* xh = reinterpret_cast<uint16_t*>(sc);
  uint16_t* xl = reinterpret_cast<uint16_t*>(sc + half_bytes);
  GemmArgs a{};
  a.W = W;
  a.scale = has_scales(wtype) ? scale : nullptr;
  a.N = N;
  a.K = K;
  a.M = M;
  a.xh = xh;
  a.xl = xl;
  a.y = y;
  a.y_stride = N;
  a.accumulate = 0;
  a.part = reinterpret_cast<float*>(sc + 2 * half_bytes);
  // fewer K splits when the rest of the scratch holds fewer partial sums (one
  // split needs none: it writes y directly)
  const size_t part_cap = (DAR_NOALLOC_SCRATCH_BYTES - 2 * half_bytes) / sizeof(float);
  // x is only read: no sums are pending
  if ((e = launch_norm_split(const_cast<float*>(x), K, M, K, nullptr, 0.f, xh, xl, s)) == hipSuccess)
    e = launch_gemm(wtype_of(wtype), a, part_cap, s);
  if (e != hipSuccess) return hip_fail(nullptr, e, "gemm (no allocation)");
  return DAR_OK;
}

int dar_op_stream_read(const void* src, size_t bytes, int32_t iters, uint32_t* sink, float* ms_out, void* stream) {
  if (!src || !sink || !ms_out || bytes < 16 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15) || iters < 1)
    return DAR_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  const ru32x4* p = static_cast<const ru32x4*>(src);
  const size_t n = bytes / 16;
  auto pass = [&](const ReadShape& sh) {
    switch (sh.loads) {
      case 2: hipLaunchKernelGGL(k_stream_read<2>, dim3(sh.grid), dim3(kBlock), 0, s, p, n, sink); break;
      case 4: hipLaunchKernelGGL(k_stream_read<4>, dim3(sh.grid), dim3(kBlock), 0, s, p, n, sink); break;
      default: hipLaunchKernelGGL(k_stream_read<8>, dim3(sh.grid), dim3(kBlock), 0, s, p, n, sink); break;
    }
    return hipGetLastError();
  };
  float best = 0.f;
  for (const ReadShape& sh : kReadShapes) {
    if (e == hipSuccess) e = pass(sh);  // untimed: loads the kernel, settles the clocks
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    for (int it = 0; e == hipSuccess && it < iters; ++it) e = pass(sh);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && (best == 0.f || ms < best)) best = ms;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_fail(nullptr, e, "stream read");
  *ms_out = best / iters;
  return DAR_OK;
}

int dar_op_gemm(int32_t wtype, const void* W, const float* scale, int32_t N, int32_t K, const float* x,
                int32_t M, float* y, void* stream) {
  if (!W || !x || !y || N < 1 || K < 256 || K % 256 || K > 16384 || M < 1 || M > kPrefillRows) return DAR_E_INVAL;
  if (wtype != DAR_WTYPE_BF16 && !has_scales(wtype)) return DAR_E_INVAL;
  if (has_scales(wtype) && !scale) return DAR_E_INVAL;
  if (!aligned16(W) || !aligned16(x)) return DAR_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mpad = gemm_mpad(M);
  const size_t half_bytes = align_up((size_t)mpad * K * sizeof(uint16_t));
  const int wt = wtype_of(wtype);
  const size_t part_cap = (size_t)gemm_splits(wt, M, N, K) * M * N;
  char* scratch = nullptr;
  hipError_t e = hipMalloc(&scratch, 2 * half_bytes + part_cap * sizeof(float));
  if (e != hipSuccess) return hip_fail(nullptr, e, "gemm scratch");
  uint16_t* xh = reinterpret_cast<uint16_t*>(scratch);
  uint16_t* xl = reinterpret_cast<uint16_t*>(scratch + half_bytes);
  GemmArgs a{};
  a.W = W;
  a.scale = has_scales(wtype) ? scale : nullptr;
  a.N = N;
  a.K = K;
  a.M = M;
  a.xh = xh;
  a.xl = xl;
  a.y = y;
  a.y_stride = N;
  a.accumulate = 0;
  a.part = reinterpret_cast<float*>(scratch + 2 * half_bytes);
  // x is only read: no sums are pending
  if ((e = launch_norm_split(const_cast<float*>(x), K, M, K, nullptr, 0.f, xh, xl, s)) == hipSuccess &&
      (e = launch_gemm(wt, a, part_cap, s)) == hipSuccess)
    e = hipStreamSynchronize(s);
  (void)hipStreamSynchronize(s);
  (void)hipFree(scratch);
  if (e != hipSuccess) return hip_fail(nullptr, e, "gemm");
  return DAR_OK;
}

int dar_op_attention(const float* q, const void* K, const void* V, int32_t n_heads_q, int32_t n_heads_kv,
                     int32_t head_dim, int32_t max_len, int32_t pos, int32_t M, int32_t chunk, float* out,
                     void* stream) {
  if (!q || !K || !V || !out || n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv) return DAR_E_INVAL;
  const int g = n_heads_q / n_heads_kv;
  if ((head_dim != 64 && head_dim != 128) || (g != 1 && g != 2 && g != 4 && g != 8)) return DAR_E_UNSUPPORTED;
  if ((M != 1 && M != 2) || pos < 0 || pos + M > max_len) return DAR_E_INVAL;
  if (chunk != 0 && (chunk < 16 || chunk % 16)) return DAR_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // chunk 0: one block per (query row, KV head), no split
  const int nsplit_max = chunk == 0 ? 1 : (max_len + chunk - 1) / chunk;
  const size_t pf = attn_partial_floats(M, n_heads_kv, nsplit_max, g, head_dim);
  char* scratch = nullptr;
  const size_t off_pos = align_up(pf * sizeof(float));
  const size_t off_cnt = off_pos + 256;
  hipError_t e = hipMalloc(&scratch, off_cnt + align_up(sizeof(unsigned) * M * n_heads_kv));
  if (e != hipSuccess) return hip_fail(nullptr, e, "attention scratch");
  int* dpos = reinterpret_cast<int*>(scratch + off_pos);
  unsigned* cnt = reinterpret_cast<unsigned*>(scratch + off_cnt);
  Task t = none_task();
  t.kind = T_ATTN;
  t.M = M;
  AttnArgs& a = t.attn;
  a.q = q;
  a.q_stride = n_heads_q * head_dim;
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.cache_len = max_len;
  a.pos = dpos;
  a.n_heads_q = n_heads_q;
  a.n_heads_kv = n_heads_kv;
  a.head_dim = head_dim;
  a.chunk = chunk == 0 ? max_len : chunk;
  a.nsplit_max = nsplit_max;
  a.M = M;
  a.part = reinterpret_cast<float*>(scratch);
  a.cnt = nsplit_max > 1 ? cnt : nullptr;  // the splits merge in the same launch, as in the decode frame
  a.out = out;
  a.out_stride = n_heads_q * head_dim;
  int st = DAR_OK;
  if ((e = launch_fill_i32(dpos, 1, pos, s)) != hipSuccess ||
      (e = launch_fill_i32(reinterpret_cast<int*>(cnt), M * n_heads_kv, 0, s)) != hipSuccess)
    st = hip_fail(nullptr, e, "attention");
  if (st == DAR_OK) st = run_single_task(t, W_BF16, s, "attention");
  (void)hipStreamSynchronize(s);
  (void)hipFree(scratch);
  return st;
}

int dar_op_fp8_decode(const void* codes, int32_t n, float* out, void* stream) {
  if (!codes || !out || n < 1) return DAR_E_INVAL;
  hipError_t e = launch_fp8_decode(static_cast<const uint8_t*>(codes), n, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "fp8 decode");
  return DAR_OK;
}

// checks a dar_sampling against a vocabulary of up to vmax codes; fills sp
static int sampling_args(const dar_sampling* s, int vmax, SampleArgs& sp, std::string& why) {
  if (!s->uniforms || (reinterpret_cast<uintptr_t>(s->uniforms) & 3u)) {
    why = "uniforms NULL or misaligned";
    return DAR_E_INVAL;
  }
  if (!(s->temperature > 0.f) || !std::isfinite(s->temperature)) {
    why = "temperature must be positive and finite";
    return DAR_E_INVAL;
  }
  if (!(s->top_p > 0.f) || !(s->top_p <= 1.f)) {
    why = "top_p must be in (0, 1]";
    return DAR_E_INVAL;
  }
  if (!(s->repetition_penalty >= 1.f) || !std::isfinite(s->repetition_penalty)) {
    why = "repetition_penalty must be >= 1 and finite";
    return DAR_E_INVAL;
  }
  if (s->top_k < 1 || s->repetition_window < 0) {
    why = "top_k must be >= 1 and repetition_window >= 0";
    return DAR_E_INVAL;
  }
  if (s->top_k > kMaxTopK || s->repetition_window > kMaxWindow || vmax > kMaxSampleVocab) {
    why = "top_k above 256, repetition_window above 64 or a vocabulary above 8192";
    return DAR_E_UNSUPPORTED;
  }
  sp.u = s->uniforms;
  sp.temperature = s->temperature;
  sp.top_p = s->top_p;
  sp.penalty = s->repetition_penalty;
  sp.top_k = s->top_k;
  sp.window = s->repetition_window;
  return DAR_OK;
}

int dar_set_sampling(dar_ctx* c, const dar_sampling* s) {
  if (!c) return DAR_E_INVAL;
  SampleArgs sp{};
  if (s) {
    const int vmax = std::max(c->cfg.vocab_c0, has_fast(&c->cfg) ? c->cfg.vocab_res : 0);
    const int st = sampling_args(s, vmax, sp, c->err);
    if (st != DAR_OK) return st;
    sp.win_lo = c->win_lo;
  }
  // no frame of this context may still read the plans' arguments or graphs
  DAR_HIP(c, hipStreamSynchronize(c->cs.s), "synchronize");
  DAR_HIP(c, hipStreamSynchronize(c->cf.s), "synchronize");
  c->smp = sp;
  for (Plan* p : {&c->p_c0, &c->p_fast, &c->p_slow}) {
    bool changed = false;
    for (Task& t : p->tasks) {
      if (t.kind == T_COMMIT) {
        t.commit.smp = sp;
        changed = true;
      } else if (t.kind == T_COMMIT_ROWS) {
        t.rows.smp = sp;
        changed = true;
      }
    }
    if (changed) free_plan(*p);  // a captured graph is captured again with the new arguments
  }
  return DAR_OK;
}

int dar_op_sample(const float* logits, int32_t rows, int32_t V, const dar_sampling* s, const int32_t* history,
                  int32_t n_hist, int32_t* codes_out, void* stream) {
  if (!logits || !s || !codes_out || rows < 1 || V < 1 || n_hist < 0 || (n_hist > 0 && !history))
    return DAR_E_INVAL;
  SampleArgs sp{};
  std::string why;
  const int st = sampling_args(s, V, sp, why);
  if (st != DAR_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = launch_sample_rows(logits, rows, V, sp, history, n_hist, codes_out, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(nullptr, e, "sample");
  return DAR_OK;
}

int dar_time_kind(dar_ctx* c, int32_t kind) {
  if (!c || kind < -1 || kind > K_OTHER) return DAR_E_INVAL;
  c->timed_kind = kind;
  c->tused = 0;
  return DAR_OK;
}

int dar_kind_time(dar_ctx* c, double* ms_total, int32_t* launches) {
  if (!c || !ms_total || !launches) return DAR_E_INVAL;
  DAR_HIP(c, hipStreamSynchronize(c->stream), "synchronize");
  for (Chain* ch : {&c->cs, &c->cf}) DAR_HIP(c, hipStreamSynchronize(ch->s), "synchronize");
  double total = 0.0;
  for (size_t i = 0; i + 1 < c->tused; i += 2) {
    float ms = 0.f;
    DAR_HIP(c, hipEventElapsedTime(&ms, c->tpool[i], c->tpool[i + 1]), "event time");
    total += ms;
  }
  *ms_total = total;
  *launches = (int32_t)(c->tused / 2);
  c->tused = 0;
  return DAR_OK;
}

int dar_profile_frame(dar_ctx* c, int32_t cap, float* ms_out, int32_t* kind_out, int32_t* layer_out,
                      int32_t* n_out) {
  if (!c || !ms_out || !kind_out || !layer_out || !n_out || cap < 1) return DAR_E_INVAL;
  if (c->paged) {
    c->err = "a paged context takes new pages in dar_decode_frame: time it with dar_time_kind";
    return DAR_E_STATE;
  }
  if (!c->prefilled) {
    c->err = "decode before prefill";
    return DAR_E_STATE;
  }
  if (c->pos_host >= c->cfg.max_len) {
    c->err = "position reached max_len";
    return DAR_E_CAPACITY;
  }
  const bool run_slow = c->pos_host + 1 < c->cfg.max_len;
  const Plan* plans[3] = {&c->p_c0, &c->p_fast, run_slow ? &c->p_slow : nullptr};
  size_t launches = 0;
  for (const Plan* p : plans)
    if (p) launches += p->launches();
  if ((size_t)cap < launches) {
    c->err = "profile capacity below the frame's launch count";
    return DAR_E_INVAL;
  }
  while (c->events.size() < 2 * launches) {
    hipEvent_t ev;
    DAR_HIP(c, hipEventCreate(&ev), "create event");
    c->events.push_back(ev);
  }
  // the same frame as dar_decode_frame, every launch on one stream and bracketed by events
  set_live_attention(c, c->pos_host + 2);
  hipStream_t s = c->cf.s;
  DAR_HIP(c, hipEventRecord(c->ev_start, c->stream), "record start");
  DAR_HIP(c, hipStreamWaitEvent(s, c->ev_start, 0), "wait start");
  DAR_HIP(c, hipStreamWaitEvent(s, c->ev_s_done, 0), "wait slow chain");
  int st = set_force(c, s, nullptr);
  if (st != DAR_OK) return st;
  size_t base = 0;
  for (const Plan* p : plans) {
    if (!p) continue;
    DAR_HIP(c, enqueue_plan(c, *p, s, base), "profiled frame");
    base += p->launches();
  }
  DAR_HIP(c, hipEventRecord(c->ev_f_done, s), "record fast done");
  DAR_HIP(c, hipEventRecord(c->ev_s_done, s), "record slow done");
  DAR_HIP(c, hipStreamSynchronize(s), "synchronize profile");
  size_t i = 0;
  for (const Plan* p : plans) {
    if (!p) continue;
    for (size_t j = 0; j < p->launches(); ++j, ++i) {
      float ms = 0.f;
      DAR_HIP(c, hipEventElapsedTime(&ms, c->events[2 * i], c->events[2 * i + 1]), "event time");
      ms_out[i] = ms;
      kind_out[i] = p->kind[j];
      layer_out[i] = p->layer[j];
    }
  }
  *n_out = (int32_t)i;
  c->pos_host += 1;
  for (int& p : c->pos_hb) p += 1;
  return DAR_OK;
}

}  // extern "C"
