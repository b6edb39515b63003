// C-ABI runtime of libdar.so: context, workspace carve-up, RoPE table, the
// frame's launch sequences, HIP-graph capture and replay, prefill, helpers.
//
// Frame (tuna-fish README, intro: "slowAR decode + fastAR loop"; "Inference
// estimation": slow AR once, fast AR nine times with a 10-long fast KV):
//   slow layers 0..Ls-1 : QKV(+norm, RoPE, KV append) -> attention -> Wo(+res)
//                         -> W1/W3(+norm, SiLU*mul) -> W2(+res)
//   codebook-0 head     : norm -> W0 -> per-workgroup argmax
//   commit c0           : argmax (or the forced code) -> ring, fast inputs
//                         [h_t, E0[c0]], next frame's slow input W0[c0]
//   fast pass 1         : the fast layers over fast positions 0 and 1 together
//   fast passes 2..R    : the fast layers over position k; after each pass the
//                         shared head and a commit that gathers E_k[c_k]
//
// The slow step of frame i+1 needs only codebook 0 of frame i, not frame i's
// fast AR, so each call runs two chains concurrently on two streams, each one
// replaying its own captured graph: the fast chain finishes frame i while the
// slow chain computes the slow step and codebook-0 head of frame i+1. Their
// weights are nearly equal in size (slow 7.29 GB, fast 9 x 0.83 GB at full
// shape), so each chain's launch gaps are filled by the other's weight stream.
// Every position and code the chains need lives in device memory.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dar.h"
#include "dar_internal.h"

using namespace dar;

namespace {

thread_local std::string g_create_error;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t x[2], q[2], o[2], h[2], part[2];  // chain scratch: [0] slow (one row), [1] fast (two rows)
  size_t ht, logits0, flogits, slots0, slotsf, pred, committed, forced, flags, pos, seqpos, ring, rope;
  size_t ks, vs, kf, vf, total;
  int nsplit_slow, chunk, rope_len, seq_len, vmax, fast_len, nslots;
};

int frame_codes(const dar_config* c) { return 1 + c->n_res; }
bool has_fast(const dar_config* c) { return c->n_res > 0; }

Layout make_layout(const dar_config* c) {
  Layout L{};
  const int d = c->d_model, qw = c->n_heads_q * c->head_dim, F = c->ffn_dim;
  const int g = c->n_heads_q / c->n_heads_kv;
  const int fc = frame_codes(c);
  L.chunk = kAttnChunkDefault;
  L.nsplit_slow = (c->max_len + L.chunk - 1) / L.chunk;
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
  for (int ch = 0; ch < 2; ++ch) {
    const int M = ch == 0 ? 1 : 2;
    const int nsplit = ch == 0 ? L.nsplit_slow : 1;
    L.x[ch] = take(sizeof(float) * M * d);
    L.q[ch] = take(sizeof(float) * M * qw);
    L.o[ch] = take(sizeof(float) * M * qw);
    L.h[ch] = take(sizeof(float) * M * F);
    L.part[ch] = take(sizeof(float) * attn_partial_floats(M, c->n_heads_kv, nsplit, g, c->head_dim));
  }
  L.ht = take(sizeof(float) * d);
  L.logits0 = take(sizeof(float) * c->vocab_c0);
  L.flogits = take(sizeof(float) * (size_t)fc * L.vmax);
  L.slots0 = take(sizeof(unsigned long long) * L.nslots);
  L.slotsf = take(sizeof(unsigned long long) * L.nslots);
  L.pred = take(sizeof(int) * fc);
  L.committed = take(sizeof(int) * fc);
  L.forced = take(sizeof(int) * fc);
  L.flags = take(sizeof(int) * 4);
  L.pos = take(sizeof(int) * 4);
  L.seqpos = take(sizeof(int) * L.seq_len);
  L.ring = take(sizeof(int) * (size_t)c->max_len * fc);
  L.rope = take(sizeof(float) * 2 * (size_t)L.rope_len * (c->head_dim / 2));
  const size_t kv_slow = (size_t)c->n_layers_slow * c->n_heads_kv * c->max_len * c->head_dim * 2;
  L.ks = take(kv_slow);
  L.vs = take(kv_slow);
  const size_t kv_fast = has_fast(c) ? (size_t)c->n_layers_fast * c->n_heads_kv * L.fast_len * c->head_dim * 2 : 0;
  L.kf = take(kv_fast);
  L.vf = take(kv_fast);
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
  if (c->wtype != DAR_WTYPE_BF16 && c->wtype != DAR_WTYPE_FP8_E4M3_ROW) return bad("unknown wtype");
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
  if (c->max_batch != 1) return unsup("max_batch must be 1 in this version");
  if (c->max_len > (1 << 24)) return unsup("max_len above 2^24");
  return DAR_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_layer(const dar_layer_weights& w, bool fp8, std::string& why, const char* which, int idx) {
  const void* ptrs[] = {w.attn_norm, w.wqkv, w.wo, w.ffn_norm, w.w1, w.w3, w.w2};
  for (const void* p : ptrs) {
    if (!p || !aligned16(p)) {
      char buf[128];
      snprintf(buf, sizeof buf, "%s layer %d: a weight pointer is NULL or not 16-byte aligned", which, idx);
      why = buf;
      return DAR_E_INVAL;
    }
  }
  if (fp8) {
    const float* s[] = {w.wqkv_scale, w.wo_scale, w.w1_scale, w.w3_scale, w.w2_scale};
    for (const float* p : s) {
      if (!p) {
        char buf[128];
        snprintf(buf, sizeof buf, "%s layer %d: fp8 row scale pointer is NULL", which, idx);
        why = buf;
        return DAR_E_INVAL;
      }
    }
  }
  return DAR_OK;
}

}  // namespace

struct LaunchRec {
  int kind, layer;
};

// One dependent chain of launches with its own stream, scratch and graph.
struct Chain {
  float *x = nullptr, *q = nullptr, *o = nullptr, *h = nullptr, *part = nullptr;
  int M = 1;
  hipStream_t s = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

struct dar_ctx {
  dar_config cfg{};
  Layout L{};
  bool fp8 = false;
  std::vector<dar_layer_weights> slow, fast;
  std::vector<const uint16_t*> fast_emb;
  const uint16_t* w0 = nullptr;
  const uint16_t* slow_fn = nullptr;
  const uint16_t* fast_fn = nullptr;
  const void* fast_head = nullptr;
  const float* fast_head_scale = nullptr;

  hipStream_t stream = nullptr;  // the caller's stream
  Chain cs, cf;                  // slow chain (frame i+1) and fast chain (frame i)
  hipEvent_t ev_start = nullptr, ev_c0 = nullptr, ev_f_done = nullptr, ev_s_done = nullptr;
  bool use_graph = true;

  char* ws = nullptr;
  float *ht, *logits0, *flogits;
  unsigned long long *slots0, *slotsf;
  int *pred, *committed, *forced, *flags, *pos_s, *pos_f, *seqpos, *ring;
  float2* rope;
  uint16_t *ks, *vs, *kf, *vf;

  int pos_host = 0;       // slow position of the next frame to decode
  bool prefilled = false;
  bool force_dev = false;
  std::string err;

  std::vector<hipEvent_t> events;
  std::vector<LaunchRec> recs;
  bool profiling = false;
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

// Every launch goes through here so the profiler can bracket it with events.
template <typename F>
hipError_t tracked(dar_ctx* c, hipStream_t s, int kind, int layer, F&& launch) {
  if (c->profiling) {
    const size_t i = c->recs.size();
    if (2 * i + 2 > c->events.size()) return hipErrorOutOfMemory;
    hipError_t e = hipEventRecord(c->events[2 * i], s);
    if (e != hipSuccess) return e;
    e = launch();
    if (e != hipSuccess) return e;
    e = hipEventRecord(c->events[2 * i + 1], s);
    c->recs.push_back({kind, layer});
    return e;
  }
  return launch();
}

enum Kind { K_QKV = 0, K_ATTN = 1, K_WO = 2, K_W13 = 3, K_W2 = 4, K_HEAD = 5, K_OTHER = 6 };

// One decoder layer of a chain over M input rows at device position *pos (row m at +m).
hipError_t enqueue_layer(dar_ctx* c, const Chain& ch, hipStream_t s, const dar_layer_weights& w, int layer_tag,
                         int M, const int* pos, uint16_t* kc, uint16_t* vc, int cache_len, int nsplit_max) {
  const dar_config& g = c->cfg;
  const int d = g.d_model, qw = g.n_heads_q * g.head_dim;
  const int wt = c->fp8 ? W_FP8 : W_BF16;
  hipError_t e;

  QkvArgs qa{};
  qa.W = w.wqkv;
  qa.scale = c->fp8 ? w.wqkv_scale : nullptr;
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
  e = tracked(c, s, K_QKV, layer_tag, [&] { return launch_qkv(wt, qa, s); });
  if (e != hipSuccess) return e;

  AttnArgs aa{};
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
  aa.out = ch.o;
  aa.out_stride = qw;
  e = tracked(c, s, K_ATTN, layer_tag, [&] { return launch_attn(aa, s); });
  if (e != hipSuccess) return e;

  GemvArgs wo{};
  wo.W = w.wo;
  wo.scale = c->fp8 ? w.wo_scale : nullptr;
  wo.rows = d;
  wo.K = qw;
  wo.M = M;
  wo.x = ch.o;
  wo.x_stride = qw;
  wo.y = ch.x;
  wo.y_stride = d;
  wo.accumulate = 1;
  e = tracked(c, s, K_WO, layer_tag, [&] { return launch_gemv(wt, wo, s); });
  if (e != hipSuccess) return e;

  SwigluArgs sa{};
  sa.W1 = w.w1;
  sa.s1 = c->fp8 ? w.w1_scale : nullptr;
  sa.W3 = w.w3;
  sa.s3 = c->fp8 ? w.w3_scale : nullptr;
  sa.F = g.ffn_dim;
  sa.K = d;
  sa.M = M;
  sa.x = ch.x;
  sa.x_stride = d;
  sa.gain = static_cast<const uint16_t*>(w.ffn_norm);
  sa.eps = g.rms_eps;
  sa.h = ch.h;
  sa.h_stride = g.ffn_dim;
  e = tracked(c, s, K_W13, layer_tag, [&] { return launch_swiglu(wt, sa, s); });
  if (e != hipSuccess) return e;

  GemvArgs w2{};
  w2.W = w.w2;
  w2.scale = c->fp8 ? w.w2_scale : nullptr;
  w2.rows = d;
  w2.K = g.ffn_dim;
  w2.M = M;
  w2.x = ch.h;
  w2.x_stride = g.ffn_dim;
  w2.y = ch.x;
  w2.y_stride = d;
  w2.accumulate = 1;
  return tracked(c, s, K_W2, layer_tag, [&] { return launch_gemv(wt, w2, s); });
}

// Slow chain: the slow layers at *pos_s over the slow residual; with_head adds the
// codebook-0 head (logits, per-workgroup maxima, h_t) and advances pos_s.
hipError_t enqueue_slow(dar_ctx* c, hipStream_t s, bool with_head) {
  const dar_config& g = c->cfg;
  const size_t per_layer = (size_t)g.n_heads_kv * g.max_len * g.head_dim;
  for (int l = 0; l < g.n_layers_slow; ++l) {
    hipError_t e = enqueue_layer(c, c->cs, s, c->slow[l], l, 1, c->pos_s, c->ks + l * per_layer,
                                 c->vs + l * per_layer, g.max_len, c->L.nsplit_slow);
    if (e != hipSuccess) return e;
  }
  if (!with_head) return hipSuccess;
  HeadArgs h0{};
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
  return tracked(c, s, K_HEAD, 0, [&] { return launch_head(W_BF16, h0, s); });
}

CommitArgs commit_common(dar_ctx* c, int k, const unsigned long long* slots, int rows) {
  CommitArgs a{};
  a.slots = slots;
  a.nslots = head_grid(rows);
  a.code_index = k;
  a.frame_codes = frame_codes(&c->cfg);
  a.pred = c->pred;
  a.committed = c->committed;
  a.forced = c->forced;
  a.force_flag = c->flags + 0;
  a.ring = c->ring;
  a.pos = c->pos_f;
  a.K = c->cfg.d_model;
  return a;
}

// Start of the fast chain: commit codebook 0 of the frame (argmax of the slow
// head, or the forced code), move its logits and h_t into the frame's buffers,
// write the fast inputs [h_t, E0[c0]] and the next slow input W0[c0].
hipError_t enqueue_commit0(dar_ctx* c, hipStream_t s) {
  const dar_config& g = c->cfg;
  const int d = g.d_model;
  const bool fast = has_fast(&g);
  CommitArgs a = commit_common(c, 0, c->slots0, g.vocab_c0);
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
  return tracked(c, s, K_OTHER, 0, [&] { return launch_commit(a, s); });
}

// The fast AR of one frame: pass 1 over fast positions 0 and 1, passes 2..R
// over position k, each followed by the shared head and its commit.
hipError_t enqueue_fast(dar_ctx* c, hipStream_t s) {
  const dar_config& g = c->cfg;
  const int d = g.d_model;
  const int wt = c->fp8 ? W_FP8 : W_BF16;
  const size_t per_layer = (size_t)g.n_heads_kv * c->L.fast_len * g.head_dim;
  for (int k = 1; k <= g.n_res; ++k) {
    const int M = (k == 1) ? 2 : 1;
    const int* fpos = c->seqpos + (k == 1 ? 0 : k);
    for (int l = 0; l < g.n_layers_fast; ++l) {
      hipError_t e = enqueue_layer(c, c->cf, s, c->fast[l], 1000 * k + l, M, fpos, c->kf + l * per_layer,
                                   c->vf + l * per_layer, c->L.fast_len, 1);
      if (e != hipSuccess) return e;
    }
    HeadArgs hk{};
    hk.W = c->fast_head;
    hk.scale = c->fp8 ? c->fast_head_scale : nullptr;
    hk.rows = g.vocab_res;
    hk.K = d;
    hk.x = c->cf.x + (size_t)(M - 1) * d;
    hk.gain = c->fast_fn;
    hk.eps = g.rms_eps;
    hk.logits = c->flogits + (size_t)k * c->L.vmax;
    hk.slots = c->slotsf;
    hk.anomalies = c->flags + 1;
    hipError_t e = tracked(c, s, K_HEAD, k, [&] { return launch_head(wt, hk, s); });
    if (e != hipSuccess) return e;
    CommitArgs ck = commit_common(c, k, c->slotsf, g.vocab_res);
    ck.pos_inc = (k == g.n_res) ? c->pos_f : nullptr;
    ck.next_table = (k < g.n_res) ? c->fast_emb[k] : nullptr;
    ck.next_rows = g.vocab_res;
    ck.next_x = c->cf.x;
    e = tracked(c, s, K_OTHER, k, [&] { return launch_commit(ck, s); });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int capture(dar_ctx* c, Chain& ch, hipError_t (*body)(dar_ctx*, hipStream_t), const char* what) {
  if (ch.exec) return DAR_OK;
  DAR_HIP(c, hipStreamBeginCapture(ch.s, hipStreamCaptureModeThreadLocal), "begin capture");
  hipError_t e = body(c, ch.s);
  hipGraph_t g = nullptr;
  hipError_t e2 = hipStreamEndCapture(ch.s, &g);
  if (e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return hip_fail(c, e, what);
  }
  if (e2 != hipSuccess) return hip_fail(c, e2, "end capture");
  ch.graph = g;
  DAR_HIP(c, hipGraphInstantiate(&ch.exec, ch.graph, nullptr, nullptr, 0), "instantiate graph");
  return DAR_OK;
}

hipError_t body_fast(dar_ctx* c, hipStream_t s) { return enqueue_fast(c, s); }
hipError_t body_slow(dar_ctx* c, hipStream_t s) { return enqueue_slow(c, s, true); }

int copy_outputs(dar_ctx* c, hipStream_t s, int32_t* codes_out, float* logits_out) {
  const dar_config& g = c->cfg;
  if (codes_out) DAR_HIP(c, launch_copy_i32(c->pred, codes_out, frame_codes(&g), s), "copy codes");
  if (logits_out) {
    const size_t fc = frame_codes(&g);
    for (size_t k = 0; k < fc; ++k) {
      const int V = (k == 0) ? g.vocab_c0 : g.vocab_res;
      DAR_HIP(c,
              hipMemcpyAsync(logits_out + k * c->L.vmax, c->flogits + k * c->L.vmax, sizeof(float) * V,
                             hipMemcpyDeviceToDevice, s),
              "copy logits");
    }
  }
  return DAR_OK;
}

int set_force(dar_ctx* c, hipStream_t s, const int32_t* forced) {
  const int fc = frame_codes(&c->cfg);
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
// frame i+1. The slow chain starts once c0 of frame i is committed (its input).
int pipeline_step(dar_ctx* c, const int32_t* forced, int32_t* codes_out, float* logits_out, bool run_slow) {
  const bool fast = has_fast(&c->cfg);
  if (c->use_graph) {
    int st = fast ? capture(c, c->cf, body_fast, "capture fast chain") : DAR_OK;
    if (st == DAR_OK && run_slow) st = capture(c, c->cs, body_slow, "capture slow chain");
    if (st != DAR_OK) return st;
  }
  hipStream_t sf = c->cf.s, ss = c->cs.s;
  DAR_HIP(c, hipEventRecord(c->ev_start, c->stream), "record start");
  DAR_HIP(c, hipStreamWaitEvent(sf, c->ev_start, 0), "wait start");
  DAR_HIP(c, hipStreamWaitEvent(sf, c->ev_s_done, 0), "wait slow chain");
  int st = set_force(c, sf, forced);
  if (st != DAR_OK) return st;
  DAR_HIP(c, enqueue_commit0(c, sf), "commit codebook 0");
  DAR_HIP(c, hipEventRecord(c->ev_c0, sf), "record c0");
  if (run_slow) {
    DAR_HIP(c, hipStreamWaitEvent(ss, c->ev_c0, 0), "slow waits c0");
    if (c->use_graph) {
      DAR_HIP(c, hipGraphLaunch(c->cs.exec, ss), "slow graph launch");
    } else {
      DAR_HIP(c, enqueue_slow(c, ss, true), "slow chain");
    }
    DAR_HIP(c, hipEventRecord(c->ev_s_done, ss), "record slow done");
  }
  if (fast) {
    if (c->use_graph) {
      DAR_HIP(c, hipGraphLaunch(c->cf.exec, sf), "fast graph launch");
    } else {
      DAR_HIP(c, enqueue_fast(c, sf), "fast chain");
    }
  }
  st = copy_outputs(c, sf, codes_out, logits_out);
  if (st != DAR_OK) return st;
  DAR_HIP(c, hipEventRecord(c->ev_f_done, sf), "record fast done");
  DAR_HIP(c, hipStreamWaitEvent(c->stream, c->ev_f_done, 0), "join fast");
  DAR_HIP(c, hipStreamWaitEvent(c->stream, c->ev_s_done, 0), "join slow");
  return DAR_OK;
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

int dar_create(const dar_config* cfg, const dar_weights* w, void* workspace, size_t ws_bytes, void* stream,
               dar_ctx** ctx_out) {
  std::string why;
  if (!ctx_out) {
    g_create_error = "ctx_out is NULL";
    return DAR_E_INVAL;
  }
  *ctx_out = nullptr;
  int st = validate_config(cfg, why);
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
  const Layout L = make_layout(cfg);
  if (ws_bytes < L.total) {
    g_create_error = "workspace smaller than dar_workspace_bytes()";
    return DAR_E_WORKSPACE;
  }
  const bool fp8 = cfg->wtype == DAR_WTYPE_FP8_E4M3_ROW;
  if (!w->w0 || !aligned16(w->w0) || !w->slow || !w->slow_final_norm) {
    g_create_error = "w0, slow layers or slow_final_norm missing or misaligned";
    return DAR_E_INVAL;
  }
  for (int l = 0; l < cfg->n_layers_slow; ++l) {
    st = check_layer(w->slow[l], fp8, why, "slow", l);
    if (st != DAR_OK) {
      g_create_error = why;
      return st;
    }
  }
  if (has_fast(cfg)) {
    if (!w->fast || !w->fast_emb || !w->fast_final_norm || !w->fast_head || !aligned16(w->fast_head) ||
        (fp8 && !w->fast_head_scale)) {
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
      st = check_layer(w->fast[l], fp8, why, "fast", l);
      if (st != DAR_OK) {
        g_create_error = why;
        return st;
      }
    }
  }

  dar_ctx* c = new dar_ctx();
  c->cfg = *cfg;
  c->L = L;
  c->fp8 = fp8;
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
    chains[i]->M = i == 0 ? 1 : 2;
  }
  c->ht = reinterpret_cast<float*>(b + L.ht);
  c->logits0 = reinterpret_cast<float*>(b + L.logits0);
  c->flogits = reinterpret_cast<float*>(b + L.flogits);
  c->slots0 = reinterpret_cast<unsigned long long*>(b + L.slots0);
  c->slotsf = reinterpret_cast<unsigned long long*>(b + L.slotsf);
  c->pred = reinterpret_cast<int*>(b + L.pred);
  c->committed = reinterpret_cast<int*>(b + L.committed);
  c->forced = reinterpret_cast<int*>(b + L.forced);
  c->flags = reinterpret_cast<int*>(b + L.flags);
  c->pos_s = reinterpret_cast<int*>(b + L.pos);
  c->pos_f = c->pos_s + 1;
  c->seqpos = reinterpret_cast<int*>(b + L.seqpos);
  c->ring = reinterpret_cast<int*>(b + L.ring);
  c->rope = reinterpret_cast<float2*>(b + L.rope);
  c->ks = reinterpret_cast<uint16_t*>(b + L.ks);
  c->vs = reinterpret_cast<uint16_t*>(b + L.vs);
  c->kf = reinterpret_cast<uint16_t*>(b + L.kf);
  c->vf = reinterpret_cast<uint16_t*>(b + L.vf);

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
  if ((e = hipStreamSynchronize(c->stream)) != hipSuccess) return fail(e, "synchronize create");
  if ((e = hipEventRecord(c->ev_s_done, c->cs.s)) != hipSuccess) return fail(e, "record event");
  *ctx_out = c;
  return DAR_OK;
}

int dar_prefill(dar_ctx* c, int32_t batch, const int32_t* tokens, const int32_t* lens_host, const int32_t* forced,
                int32_t* codes_out, float* logits_out) {
  if (!c) return DAR_E_INVAL;
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
  const int n = lens_host[0];
  if (n < 1 || n >= c->cfg.max_len) {
    c->err = "prompt length must be in [1, max_len)";
    return n < 1 ? DAR_E_INVAL : DAR_E_CAPACITY;
  }
  c->prefilled = false;
  const int d = c->cfg.d_model;
  hipStream_t ss = c->cs.s;
  // the slow chain runs the prompt token by token after anything already queued
  DAR_HIP(c, hipEventRecord(c->ev_start, c->stream), "record start");
  DAR_HIP(c, hipStreamWaitEvent(ss, c->ev_start, 0), "wait start");
  DAR_HIP(c, hipStreamWaitEvent(ss, c->ev_f_done, 0), "wait fast chain");
  for (int p = 0; p < n; ++p) {
    DAR_HIP(c, launch_embed(c->w0, c->cfg.vocab_c0, d, tokens + p, c->cs.x, c->pos_s, p, c->flags + 1, ss),
            "prefill embed");
    DAR_HIP(c, enqueue_slow(c, ss, p == n - 1), "prefill layers");
  }
  // frame 0 sits at position n-1; the slow head above moved pos_s to n
  DAR_HIP(c, launch_fill_i32(c->pos_f, 1, n - 1, ss), "set frame position");
  DAR_HIP(c, hipEventRecord(c->ev_s_done, ss), "record slow done");
  const int st = pipeline_step(c, forced, codes_out, logits_out, n < c->cfg.max_len);
  if (st != DAR_OK) return st;
  c->pos_host = n;
  c->prefilled = true;
  return DAR_OK;
}

int dar_decode_frame(dar_ctx* c, const int32_t* forced, int32_t* codes_out, float* logits_out) {
  if (!c) return DAR_E_INVAL;
  if (!c->prefilled) {
    c->err = "decode before prefill";
    return DAR_E_STATE;
  }
  if (c->pos_host >= c->cfg.max_len) {
    c->err = "position reached max_len";
    return DAR_E_CAPACITY;
  }
  const int st = pipeline_step(c, forced, codes_out, logits_out, c->pos_host + 1 < c->cfg.max_len);
  if (st != DAR_OK) return st;
  c->pos_host += 1;
  return DAR_OK;
}

int dar_destroy(dar_ctx* c) {
  if (!c) return DAR_OK;
  (void)hipStreamSynchronize(c->stream);
  for (Chain* ch : {&c->cs, &c->cf}) {
    if (ch->s) (void)hipStreamSynchronize(ch->s);
    if (ch->exec) (void)hipGraphExecDestroy(ch->exec);
    if (ch->graph) (void)hipGraphDestroy(ch->graph);
    if (ch->s) (void)hipStreamDestroy(ch->s);
  }
  for (hipEvent_t ev : c->events) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : {c->ev_start, c->ev_c0, c->ev_f_done, c->ev_s_done})
    if (ev) (void)hipEventDestroy(ev);
  delete c;
  return DAR_OK;
}

int dar_reset(dar_ctx* c) {
  if (!c) return DAR_E_INVAL;
  DAR_HIP(c, launch_fill_i32(c->flags + 1, 1, 0, c->stream), "reset counters");
  c->pos_host = 0;
  c->prefilled = false;
  return DAR_OK;
}

int dar_position(const dar_ctx* c, int32_t* pos_out) {
  if (!c || !pos_out) return DAR_E_INVAL;
  pos_out[0] = c->pos_host;
  return DAR_OK;
}

int dar_set_graph(dar_ctx* c, int32_t enable) {
  if (!c) return DAR_E_INVAL;
  c->use_graph = enable != 0;
  return DAR_OK;
}

int dar_codes(dar_ctx* c, int32_t first, int32_t count, int32_t* dst) {
  if (!c || !dst) return DAR_E_INVAL;
  if (first < 0 || count < 0 || first + count > c->cfg.max_len) {
    c->err = "ring range out of bounds";
    return DAR_E_INVAL;
  }
  if (count == 0) return DAR_OK;
  const int fc = frame_codes(&c->cfg);
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
  const bool fp8 = cfg->wtype == DAR_WTYPE_FP8_E4M3_ROW;
  const double Ls = cfg->n_layers_slow, Lf = cfg->n_layers_fast;
  double slow = (fp8 ? Ls * mats + 4.0 * Ls * rows : 2.0 * Ls * mats) + 2.0 * (Ls * norms + d) +
                2.0 * cfg->vocab_c0 * d;
  double fast = 0.0, fast_kv = 0.0;
  if (cfg->n_res > 0) {
    const double head = (double)cfg->vocab_res * d;
    fast = (fp8 ? Lf * mats + head + 4.0 * (Lf * rows + cfg->vocab_res) : 2.0 * (Lf * mats + head)) +
           2.0 * (Lf * norms + d);
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

int dar_op_gemv(int32_t wtype, const void* W, const float* scale, int32_t rows, int32_t cols, const float* x,
                int32_t M, float* y, void* stream) {
  if (!W || !x || !y || rows < 1 || cols < 256 || cols % 256 || cols > 16384 || (M != 1 && M != 2))
    return DAR_E_INVAL;
  if (wtype != DAR_WTYPE_BF16 && wtype != DAR_WTYPE_FP8_E4M3_ROW) return DAR_E_INVAL;
  if (wtype == DAR_WTYPE_FP8_E4M3_ROW && !scale) return DAR_E_INVAL;
  if (!aligned16(W) || !aligned16(x)) return DAR_E_INVAL;
  GemvArgs a{};
  a.W = W;
  a.scale = wtype == DAR_WTYPE_FP8_E4M3_ROW ? scale : nullptr;
  a.rows = rows;
  a.K = cols;
  a.M = M;
  a.x = x;
  a.x_stride = cols;
  a.gain = nullptr;
  a.y = y;
  a.y_stride = rows;
  a.accumulate = 0;
  hipError_t e = launch_gemv(wtype == DAR_WTYPE_FP8_E4M3_ROW ? W_FP8 : W_BF16, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "gemv");
  return DAR_OK;
}

int dar_op_attention(const float* q, const void* K, const void* V, int32_t n_heads_q, int32_t n_heads_kv,
                     int32_t head_dim, int32_t max_len, int32_t pos, int32_t M, int32_t chunk, float* out,
                     void* stream) {
  if (!q || !K || !V || !out || n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv) return DAR_E_INVAL;
  const int g = n_heads_q / n_heads_kv;
  if ((head_dim != 64 && head_dim != 128) || (g != 1 && g != 2 && g != 4 && g != 8)) return DAR_E_UNSUPPORTED;
  if ((M != 1 && M != 2) || pos < 0 || pos + M > max_len) return DAR_E_INVAL;
  if (chunk == 0) chunk = kAttnChunkDefault;
  if (chunk < 16 || chunk % 16) return DAR_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nsplit_max = (max_len + chunk - 1) / chunk;
  const size_t pf = attn_partial_floats(M, n_heads_kv, nsplit_max, g, head_dim);
  char* scratch = nullptr;
  const size_t off_pos = align_up(pf * sizeof(float));
  const size_t bytes = off_pos + 256;
  hipError_t e = hipMalloc(&scratch, bytes);
  if (e != hipSuccess) return hip_fail(nullptr, e, "attention scratch");
  int* dpos = reinterpret_cast<int*>(scratch + off_pos);
  AttnArgs a{};
  a.q = q;
  a.q_stride = n_heads_q * head_dim;
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.cache_len = max_len;
  a.pos = dpos;
  a.n_heads_q = n_heads_q;
  a.n_heads_kv = n_heads_kv;
  a.head_dim = head_dim;
  a.chunk = chunk;
  a.nsplit_max = nsplit_max;
  a.M = M;
  a.part = reinterpret_cast<float*>(scratch);
  a.out = out;
  a.out_stride = n_heads_q * head_dim;
  if ((e = launch_fill_i32(dpos, 1, pos, s)) == hipSuccess && (e = launch_attn(a, s)) == hipSuccess) {
    e = hipStreamSynchronize(s);
  }
  (void)hipFree(scratch);
  if (e != hipSuccess) return hip_fail(nullptr, e, "attention");
  return DAR_OK;
}

int dar_op_fp8_decode(const void* codes, int32_t n, float* out, void* stream) {
  if (!codes || !out || n < 1) return DAR_E_INVAL;
  hipError_t e = launch_fp8_decode(static_cast<const uint8_t*>(codes), n, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "fp8 decode");
  return DAR_OK;
}

int dar_profile_frame(dar_ctx* c, int32_t cap, float* ms_out, int32_t* kind_out, int32_t* layer_out,
                      int32_t* n_out) {
  if (!c || !ms_out || !kind_out || !layer_out || !n_out || cap < 1) return DAR_E_INVAL;
  if (!c->prefilled) {
    c->err = "decode before prefill";
    return DAR_E_STATE;
  }
  if (c->pos_host >= c->cfg.max_len) {
    c->err = "position reached max_len";
    return DAR_E_CAPACITY;
  }
  const dar_config& g = c->cfg;
  const bool run_slow = c->pos_host + 1 < g.max_len;
  const int launches = 1 + (g.n_res > 0 ? g.n_res * (5 * g.n_layers_fast + 2) : 0) +
                       (run_slow ? 5 * g.n_layers_slow + 1 : 0);
  if (cap < launches) {
    c->err = "profile capacity below the frame's launch count";
    return DAR_E_INVAL;
  }
  while ((int)c->events.size() < 2 * cap) {
    hipEvent_t ev;
    DAR_HIP(c, hipEventCreate(&ev), "create event");
    c->events.push_back(ev);
  }
  // one stream, fast chain of this frame then slow chain of the next, every launch bracketed
  hipStream_t s = c->cf.s;
  DAR_HIP(c, hipEventRecord(c->ev_start, c->stream), "record start");
  DAR_HIP(c, hipStreamWaitEvent(s, c->ev_start, 0), "wait start");
  DAR_HIP(c, hipStreamWaitEvent(s, c->ev_s_done, 0), "wait slow chain");
  int st = set_force(c, s, nullptr);
  if (st != DAR_OK) return st;
  c->recs.clear();
  c->profiling = true;
  hipError_t e = enqueue_commit0(c, s);
  if (e == hipSuccess && has_fast(&g)) e = enqueue_fast(c, s);
  if (e == hipSuccess && run_slow) e = enqueue_slow(c, s, true);
  c->profiling = false;
  if (e != hipSuccess) return hip_fail(c, e, "profiled frame");
  DAR_HIP(c, hipEventRecord(c->ev_f_done, s), "record fast done");
  DAR_HIP(c, hipEventRecord(c->ev_s_done, s), "record slow done");
  DAR_HIP(c, hipStreamSynchronize(s), "synchronize profile");
  const int n = (int)c->recs.size();
  for (int i = 0; i < n && i < cap; ++i) {
    float ms = 0.f;
    DAR_HIP(c, hipEventElapsedTime(&ms, c->events[2 * i], c->events[2 * i + 1]), "event time");
    ms_out[i] = ms;
    kind_out[i] = c->recs[i].kind;
    layer_out[i] = c->recs[i].layer;
  }
  *n_out = n;
  c->pos_host += 1;
  return DAR_OK;
}

}  // extern "C"
