// gfx950 kernels of the batch-1 Dual-AR decode frame.
//
// At batch 1 every projection is a matrix-vector product whose cost is the
// weight stream from HBM (tuna-fish README, "Inference estimation": decode
// time is parameters plus static KV over bandwidth). The kernels below are
// built around that: 16-byte-per-lane coalesced weight loads issued in batches
// before any arithmetic, fp32 accumulation, one 64-lane wave per row group
// reduced with DPP, and the small per-token work (RMSNorm, RoPE, KV append,
// residual add, SiLU*mul, argmax, the next step's embedding gather) folded into
// the prologue or epilogue of the GEMV that needs it, so that a decoder layer is
// five stages: QKV, attention, O-projection, W1/W3, W2. Inputs of up to eight
// 1 KB chunks per row are held in registers by every wave (no LDS, no barrier,
// every weight load of a wave issued at once); wider inputs and two-row passes
// are staged in LDS.
//
// Weights: bf16 (two per 32-bit word) or float8_e4m3fn with one fp32 scale per
// output row (s2-pro-fp8 model card, "Quantization Details"); the scale is
// applied once to the finished dot product. Activations on the residual path
// stay fp32; the slow and fast KV caches are bf16.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <atomic>

#include "dar_internal.h"
#include "dar_sample.h"

namespace dar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Sum within each 16-lane row, result in every lane of the row.
template <int LANES>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "row_sum lanes");
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
  if (LANES >= 8)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  if (LANES >= 16)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Full 64-lane sum, wave-uniform result.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum<16>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Workgroup barrier that orders LDS only (outstanding global loads keep flying).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ------------------------------------------------------- weight dot product --

// Weight types: bits per weight; kGrouped: scales per (row, 128-column group)
// applied to each 16-byte load's partial sum (else one scale per row, or none)
struct BF16 { static constexpr int kBits = 16; static constexpr bool kGrouped = false; };
struct FP8 { static constexpr int kBits = 8; static constexpr bool kGrouped = false; };
struct INT8 { static constexpr int kBits = 8; static constexpr bool kGrouped = false; };
struct INT4 { static constexpr int kBits = 4; static constexpr bool kGrouped = true; };
constexpr int kGroup = 128;  // columns per int4 scale

// byte offset of element n of a weight row
template <typename WT>
__device__ __forceinline__ size_t wbytes(size_t n) { return n * WT::kBits / 8; }

// the per-row scale the epilogue applies (group-scaled types have none)
template <typename WT>
__device__ __forceinline__ float row_scale(const float* scale, int r) {
  return (scale && !WT::kGrouped) ? scale[r] : 1.f;
}
// row r's group scales, [K / kGroup], for group-scaled types
template <typename WT>
__device__ __forceinline__ const float* group_scales(const float* scale, int r, int K) {
  return WT::kGrouped ? scale + (size_t)r * (K / kGroup) : nullptr;
}

template <typename WT>
struct Dot;

// Dot<WT>: V, the per-lane load (E weights, 16 bytes unless stated) and load()
// to fetch it, streaming (nontemporal); run(w, x) = sum_e w_e x[e].
template <>
struct Dot<BF16> {
  static constexpr int E = 8;  // elements per 16-byte load
  using V = u32x4;
  __device__ static __forceinline__ V load(const char* p) { return ld16_nt(p); }
  __device__ static __forceinline__ float run(u32x4 w, const float* x) {
    const float4 a = *reinterpret_cast<const float4*>(x);
    const float4 b = *reinterpret_cast<const float4*>(x + 4);
    float s0 = bf_lo(w.x) * a.x;
    float s1 = bf_hi(w.x) * a.y;
    s0 = fmaf(bf_lo(w.y), a.z, s0);
    s1 = fmaf(bf_hi(w.y), a.w, s1);
    s0 = fmaf(bf_lo(w.z), b.x, s0);
    s1 = fmaf(bf_hi(w.z), b.y, s1);
    s0 = fmaf(bf_lo(w.w), b.z, s0);
    s1 = fmaf(bf_hi(w.w), b.w, s1);
    return s0 + s1;
  }
};

// e4m3fn -> fp32 through the gfx950 packed converter (OCP E4M3).
__device__ __forceinline__ f32x2 fp8x2_lo(uint32_t u) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)u, false); }
__device__ __forceinline__ f32x2 fp8x2_hi(uint32_t u) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)u, true); }

template <>
struct Dot<FP8> {
  static constexpr int E = 16;
  using V = u32x4;
  __device__ static __forceinline__ V load(const char* p) { return ld16_nt(p); }
  __device__ static __forceinline__ float word(uint32_t u, const float4 x, float s) {
    const f32x2 lo = fp8x2_lo(u);
    const f32x2 hi = fp8x2_hi(u);
    s = fmaf(lo.x, x.x, s);
    s = fmaf(lo.y, x.y, s);
    s = fmaf(hi.x, x.z, s);
    s = fmaf(hi.y, x.w, s);
    return s;
  }
  __device__ static __forceinline__ float run(u32x4 w, const float* x) {
    const float4* x4 = reinterpret_cast<const float4*>(x);
    float s0 = word(w.x, x4[0], 0.f);
    float s1 = word(w.y, x4[1], 0.f);
    s0 = word(w.z, x4[2], s0);
    s1 = word(w.w, x4[3], s1);
    return s0 + s1;
  }
};

// Signed int8 codes, four per word, sign-extended and converted exactly to fp32.
template <>
struct Dot<INT8> {
  static constexpr int E = 16;
  using V = u32x4;
  __device__ static __forceinline__ V load(const char* p) { return ld16_nt(p); }
  __device__ static __forceinline__ float word(uint32_t u, const float4 x, float s) {
    const int v = (int)u;
    s = fmaf((float)((v << 24) >> 24), x.x, s);
    s = fmaf((float)((v << 16) >> 24), x.y, s);
    s = fmaf((float)((v << 8) >> 24), x.z, s);
    s = fmaf((float)(v >> 24), x.w, s);
    return s;
  }
  __device__ static __forceinline__ float run(u32x4 w, const float* x) {
    const float4* x4 = reinterpret_cast<const float4*>(x);
    float s0 = word(w.x, x4[0], 0.f);
    float s1 = word(w.y, x4[1], 0.f);
    s0 = word(w.z, x4[2], s0);
    s1 = word(w.w, x4[3], s1);
    return s0 + s1;
  }
};

// Two's complement int4 codes, eight per 4-byte load (column 2i in the low
// nibble of byte i): 64 lanes cover 512 columns, so every width here (a
// multiple of 512 but for the tiny 256 and 768) fills whole chunks, and a
// lane's eight columns sit inside one 128-column scale group.
template <>
struct Dot<INT4> {
  static constexpr int E = 8;
  using V = uint32_t;
  __device__ static __forceinline__ V load(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
  __device__ static __forceinline__ float run(uint32_t w, const float* x) {
    const float4 a = *reinterpret_cast<const float4*>(x);
    const float4 b = *reinterpret_cast<const float4*>(x + 4);
    const int v = (int)w;
    float s0 = (float)((v << 28) >> 28) * a.x;
    float s1 = (float)((v << 24) >> 28) * a.y;
    s0 = fmaf((float)((v << 20) >> 28), a.z, s0);
    s1 = fmaf((float)((v << 16) >> 28), a.w, s1);
    s0 = fmaf((float)((v << 12) >> 28), b.x, s0);
    s1 = fmaf((float)((v << 8) >> 28), b.y, s1);
    s0 = fmaf((float)((v << 4) >> 28), b.z, s0);
    s1 = fmaf((float)(v >> 28), b.w, s1);
    return s0 + s1;
  }
  // sum_e (q_e + 8) x[e]: flipping each nibble's top bit turns q into q + 8 in
  // [0, 15], which converts straight from a byte once the even and odd
  // columns sit in separate bytes; the caller subtracts 8 sum_e x[e]
  __device__ static __forceinline__ float run_biased(uint32_t w, const float* x) {
    const float4 a = *reinterpret_cast<const float4*>(x);
    const float4 b = *reinterpret_cast<const float4*>(x + 4);
    const uint32_t u = w ^ 0x88888888u;
    uint32_t ev = u & 0x0f0f0f0fu;         // columns 0, 2, 4, 6
    uint32_t od = (u >> 4) & 0x0f0f0f0fu;  // columns 1, 3, 5, 7
    // hide the known-zero high nibbles from the optimiser, which would
    // otherwise narrow the byte masks below and lose the one-instruction
    // byte-to-float conversions (v_cvt_f32_ubyte1..3)
    asm("" : "+v"(ev));
    asm("" : "+v"(od));
    float s0 = (float)(ev & 0xffu) * a.x;
    float s1 = (float)(od & 0xffu) * a.y;
    s0 = fmaf((float)((ev >> 8) & 0xffu), a.z, s0);
    s1 = fmaf((float)((od >> 8) & 0xffu), a.w, s1);
    s0 = fmaf((float)((ev >> 16) & 0xffu), b.x, s0);
    s1 = fmaf((float)((od >> 16) & 0xffu), b.y, s1);
    s0 = fmaf((float)(ev >> 24), b.z, s0);
    s1 = fmaf((float)(od >> 24), b.w, s1);
    return s0 + s1;
  }
};

// Streams RPW weight rows (K elements each, starting at base[i]) against M
// input vectors staged in LDS (xs[m*K + j]). Lane l covers one load (E
// elements) of every 64-load chunk of a row. Chunks are fetched in batches of
// U per row (as many bytes for every type), one batch ahead of the arithmetic; the first batch is issued by start(), which
// kernels call before their prologue so the HBM stream overlaps it. Lanes past
// the row end load a clamped (valid) address and skip the arithmetic.
template <typename WT, int M, int RPW>
struct RowStream {
  static constexpr int E = Dot<WT>::E;
  static constexpr int CW = kWave * E;
  using V = typename Dot<WT>::V;
  static constexpr int U = ((RPW >= 4) ? 2 : (8 / RPW)) * 16 / (int)sizeof(V);
  const char* base[RPW];
  const float* sb[RPW];  // group scales of each row (group-scaled types)
  int K, nchunks, lane;
  V buf[U][RPW];
  float gbuf[U][RPW];

  __device__ __forceinline__ void fetch(int c0, V (&w)[U][RPW], float (&g)[U][RPW]) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int col = min((c0 + u) * CW + lane * E, K - E);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        w[u][i] = Dot<WT>::load(base[i] + wbytes<WT>(col));
        if constexpr (WT::kGrouped) g[u][i] = sb[i][col / kGroup];
      }
    }
  }

  __device__ __forceinline__ void start(const char* const (&rows)[RPW], int K_, int lane_,
                                        const float* const* scales = nullptr) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      base[i] = rows[i];
      sb[i] = scales ? scales[i] : nullptr;
    }
    K = K_;
    lane = lane_;
    nchunks = (K + CW - 1) / CW;
    fetch(0, buf, gbuf);
  }

  __device__ __forceinline__ void run(const float* xs, float (&acc)[RPW][M]) {
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[i][m] = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += U) {
      V nxt[U][RPW];
      float gnxt[U][RPW];
      const bool more = c0 + U < nchunks;
      if (more) fetch(c0 + U, nxt, gnxt);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int col = (c0 + u) * CW + lane * E;
        if ((c0 + u < nchunks) && (col < K)) {
#pragma unroll
          for (int m = 0; m < M; ++m) {
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
              const float d = Dot<WT>::run(buf[u][i], xs + m * K + col);
              if constexpr (WT::kGrouped) acc[i][m] = fmaf(gbuf[u][i], d, acc[i][m]);
              else acc[i][m] += d;
            }
          }
        }
      }
      if (more) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < RPW; ++i) {
            buf[u][i] = nxt[u][i];
            gbuf[u][i] = gnxt[u][i];
          }
      }
    }
  }
};

// Stages M fp32 input rows into LDS, applying RMSNorm when a gain is given:
// xs = x / sqrt(mean(x^2) + eps) * gain.
// issue() loads this thread's share (up to NV float4 per row, at clamped
// indices so the loads go out back to back) into registers; bodies call it
// before starting their weight stream, so that waiting for these loads (memory
// counters retire in issue order) never waits for weights. finish() reduces,
// normalises and writes LDS. Rows longer than NV*1024 loop over the rest after
// the first block. `red` is M*kWaves floats of LDS scratch.
template <int M>
struct Stager {
  static constexpr int NV = 4;
  static constexpr int SPAN = kBlock * 4 * NV;
  float4 v[M][NV];
  uint2 g2[NV];
  const float* x;
  const uint16_t* gain;
  int x_stride, K;

  __device__ __forceinline__ void load(int kb) {
    const int tid = threadIdx.x;
    const uint16_t* gsrc = gain ? gain : reinterpret_cast<const uint16_t*>(x);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int kc = min(kb + (j * kBlock + tid) * 4, K - 4);
#pragma unroll
      for (int m = 0; m < M; ++m) v[m][j] = *reinterpret_cast<const float4*>(x + (size_t)m * x_stride + kc);
      g2[j] = *reinterpret_cast<const uint2*>(gsrc + kc);
    }
  }

  __device__ __forceinline__ void issue(const float* x_, int x_stride_, int K_, const uint16_t* gain_) {
    x = x_;
    x_stride = x_stride_;
    K = K_;
    gain = gain_;
    load(0);
  }

  // sum of squares of the block at kb (already in registers); optionally store raw
  __device__ __forceinline__ void absorb(float* xs, int kb, bool store_raw, float (&ss)[M]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int k = kb + (j * kBlock + tid) * 4;
      if (k < K) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          ss[m] += (v[m][j].x * v[m][j].x + v[m][j].y * v[m][j].y) + (v[m][j].z * v[m][j].z + v[m][j].w * v[m][j].w);
          if (store_raw) *reinterpret_cast<float4*>(xs + m * K + k) = v[m][j];
        }
      }
    }
  }

  __device__ __forceinline__ void finish(float* xs, float* red, float eps) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const bool one_pass = K <= SPAN;
    float ss[M];
#pragma unroll
    for (int m = 0; m < M; ++m) ss[m] = 0.f;
    absorb(xs, 0, gain == nullptr || !one_pass, ss);
    if (!one_pass) {
      for (int kb = SPAN; kb < K; kb += SPAN) {
        load(kb);
        absorb(xs, kb, true, ss);
      }
    }
    if (gain == nullptr) {
      lds_barrier();
      return;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float t = wave_sum(ss[m]);
      if (lane == 0) red[m * kWaves + wave] = t;
    }
    lds_barrier();
    float inv[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += red[m * kWaves + w];
      inv[m] = 1.0f / sqrtf(t / (float)K + eps);
    }
    if (one_pass) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int k = (j * kBlock + tid) * 4;
        if (k < K) {
          const float g[4] = {bf_lo(g2[j].x), bf_hi(g2[j].x), bf_lo(g2[j].y), bf_hi(g2[j].y)};
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float4 r;
            r.x = (v[m][j].x * inv[m]) * g[0];
            r.y = (v[m][j].y * inv[m]) * g[1];
            r.z = (v[m][j].z * inv[m]) * g[2];
            r.w = (v[m][j].w * inv[m]) * g[3];
            *reinterpret_cast<float4*>(xs + m * K + k) = r;
          }
        }
      }
    } else {
      for (int k = tid * 4; k < K; k += kBlock * 4) {
        const uint2 gg = *reinterpret_cast<const uint2*>(gain + k);
        const float g[4] = {bf_lo(gg.x), bf_hi(gg.x), bf_lo(gg.y), bf_hi(gg.y)};
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float4* p = reinterpret_cast<float4*>(xs + m * K + k);
          float4 r = *p;
          r.x = (r.x * inv[m]) * g[0];
          r.y = (r.y * inv[m]) * g[1];
          r.z = (r.z * inv[m]) * g[2];
          r.w = (r.w * inv[m]) * g[3];
          *p = r;
        }
      }
    }
    lds_barrier();
  }
};

template <typename WT>
__device__ __forceinline__ const char* row_ptr(const void* W, int r, int K) {
  return reinterpret_cast<const char*>(W) + wbytes<WT>((size_t)r * K);
}

// LDS of the GEMV-shaped bodies: the staged input rows, then small scratch.
__device__ __forceinline__ float* lds_scratch(char* lds, int M, int K) {
  return reinterpret_cast<float*>(lds + (((size_t)M * K * 4 + 15) & ~(size_t)15));
}

// ------------------------------------------------------------------ GEMV --

// y[m][r] (+)= scale[r] * W[r] . x[m]; wave w of block `bid` owns rows
// (bid*kWaves + w)*RPW .. +RPW.
template <typename WT, int M, int RPW>
__device__ __forceinline__ void gemv_body(const GemvArgs& a, int bid, char* lds) {
  float* xs = reinterpret_cast<float*>(lds);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int r0 = (bid * kWaves + wave) * RPW;
  const bool active = r0 < a.rows;
  Stager<M> st;
  st.issue(a.x, a.x_stride, a.K, a.gain);
  // every wave streams (inactive ones a clamped row): no branch around the
  // prefetch, so the staging wait above stays exact
  RowStream<WT, M, RPW> rs;
  {
    const char* base[RPW];
    const float* sc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      base[i] = row_ptr<WT>(a.W, min(r0 + i, a.rows - 1), a.K);
      sc[i] = group_scales<WT>(a.scale, min(r0 + i, a.rows - 1), a.K);
    }
    rs.start(base, a.K, lane, sc);
  }
  st.finish(xs, lds_scratch(lds, M, a.K), a.eps);
  if (!active) return;
  float acc[RPW][M];
  rs.run(xs, acc);
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s = wave_sum(acc[i][m]);
      const int r = r0 + i;
      if (lane == 0 && r < a.rows) {
        s *= row_scale<WT>(a.scale, r);
        float* y = a.y + (size_t)m * a.y_stride + r;
        *y = a.accumulate ? (*y + s) : s;
      }
    }
  }
}

// --------------------------------------------------- RMSNorm+QKV+RoPE+KV --

// Wave w handles rotation pairs (head, i) and (head, i + hd/2) so RoPE is
// applied where both halves are known. Pair p: head = p / (hd/2), i = p % (hd/2).
template <typename WT, int M>
__device__ __forceinline__ void qkv_body(const QkvArgs& a, int bid, char* lds) {
  float* xs = reinterpret_cast<float*>(lds);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int half = a.head_dim / 2;
  const int n_heads = a.n_heads_q + 2 * a.n_heads_kv;
  const int p = bid * kWaves + wave;
  const bool active = p < n_heads * half;
  const int pc = min(p, n_heads * half - 1);
  const int head = pc / half, i = pc % half;
  const int r1 = head * a.head_dim + i, r2 = r1 + half;
  Stager<M> st;
  st.issue(a.x, a.x_stride, a.K, a.gain);
  RowStream<WT, M, 2> rs;
  {
    const char* base[2] = {row_ptr<WT>(a.W, r1, a.K), row_ptr<WT>(a.W, r2, a.K)};
    const float* sc[2] = {group_scales<WT>(a.scale, r1, a.K), group_scales<WT>(a.scale, r2, a.K)};
    rs.start(base, a.K, lane, sc);
  }
  st.finish(xs, lds_scratch(lds, M, a.K), a.eps);
  if (!active) return;
  float acc[2][M];
  rs.run(xs, acc);
  float y1[M], y2[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    y1[m] = wave_sum(acc[0][m]);
    y2[m] = wave_sum(acc[1][m]);
  }
  if (lane != 0) return;
  const float sc1 = row_scale<WT>(a.scale, r1), sc2 = row_scale<WT>(a.scale, r2);
  const int pos0 = *a.pos;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float u = y1[m] * sc1, v = y2[m] * sc2;
    const int pos = pos0 + m;
    if (head < a.n_heads_q + a.n_heads_kv) {
      const float2 cs = a.rope[(size_t)pos * half + i];
      const float o1 = u * cs.x - v * cs.y;
      const float o2 = u * cs.y + v * cs.x;
      if (head < a.n_heads_q) {
        a.q_out[(size_t)m * a.q_stride + r1] = o1;
        a.q_out[(size_t)m * a.q_stride + r2] = o2;
      } else {
        uint16_t* kp = a.kc + ((size_t)(head - a.n_heads_q) * a.cache_len + pos) * a.head_dim;
        kp[i] = f2bf(o1);
        kp[i + half] = f2bf(o2);
      }
    } else {
      uint16_t* vp = a.vc + ((size_t)(head - a.n_heads_q - a.n_heads_kv) * a.cache_len + pos) * a.head_dim;
      vp[i] = f2bf(u);
      vp[i + half] = f2bf(v);
    }
  }
}

// ------------------------------------------------ RMSNorm + W1/W3 + SwiGLU --

template <typename WT, int M>
__device__ __forceinline__ void swiglu_body(const SwigluArgs& a, int bid, char* lds) {
  float* xs = reinterpret_cast<float*>(lds);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int r = bid * kWaves + wave;
  const bool active = r < a.F;
  Stager<M> st;
  st.issue(a.x, a.x_stride, a.K, a.gain);
  RowStream<WT, M, 2> rs;
  {
    const int rc = min(r, a.F - 1);
    const char* base[2] = {row_ptr<WT>(a.W1, rc, a.K), row_ptr<WT>(a.W3, rc, a.K)};
    const float* sc[2] = {group_scales<WT>(a.s1, rc, a.K), group_scales<WT>(a.s3, rc, a.K)};
    rs.start(base, a.K, lane, sc);
  }
  st.finish(xs, lds_scratch(lds, M, a.K), a.eps);
  if (!active) return;
  float acc[2][M];
  rs.run(xs, acc);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float g = wave_sum(acc[0][m]);
    float u = wave_sum(acc[1][m]);
    if (lane == 0) {
      g *= row_scale<WT>(a.s1, r);
      u *= row_scale<WT>(a.s3, r);
      const float silu = g / (1.0f + expf(-g));
      a.h[(size_t)m * a.h_stride + r] = silu * u;
    }
  }
}

// ----------------------------------------- RMSNorm + head + per-block argmax --

// Order-preserving key: larger float -> larger key; NaN -> smallest key.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  uint32_t k;
  if (v != v) {
    k = 0u;
  } else {
    k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((unsigned long long)k << 32) | (unsigned long long)(0xffffffffu - (uint32_t)idx);
}

template <typename WT>
__device__ __forceinline__ void head_body(const HeadArgs& a, int bid, char* lds) {
  float* xs = reinterpret_cast<float*>(lds);
  float* red = lds_scratch(lds, 1, a.K);
  unsigned long long* wbest = reinterpret_cast<unsigned long long*>(red + 2 * kWaves);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  constexpr int RPW = 2;
  const int r0 = (bid * kWaves + wave) * RPW;
  Stager<1> st;
  st.issue(a.x, a.K, a.K, a.gain);
  RowStream<WT, 1, RPW> rs;
  {
    const char* base[RPW];
    const float* sc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      base[i] = row_ptr<WT>(a.W, min(r0 + i, a.rows - 1), a.K);
      sc[i] = group_scales<WT>(a.scale, min(r0 + i, a.rows - 1), a.K);
    }
    rs.start(base, a.K, lane, sc);
  }
  st.finish(xs, red, a.eps);
  if (a.h_out && bid == 0) {
    for (int k = tid; k < a.K; k += kBlock) a.h_out[k] = xs[k];
  }
  unsigned long long best = 0ull;
  if (r0 < a.rows) {
    float acc[RPW][1];
    rs.run(xs, acc);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      float s = wave_sum(acc[i][0]);
      const int r = r0 + i;
      if (r < a.rows) {
        s *= row_scale<WT>(a.scale, r);
        if (lane == 0) {
          a.logits[r] = s;
          if (!isfinite(s)) atomicAdd(a.anomalies, 1);
        }
        const unsigned long long k = argmax_key(s, r);
        best = k > best ? k : best;
      }
    }
  }
  if (lane == 0) wbest[wave] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = wbest[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) b = wbest[w] > b ? wbest[w] : b;
    a.slots[bid] = b;  // reduced by the commit that follows
    if (a.pos_inc && bid == 0) *a.pos_inc = *a.pos_inc + 1;
  }
}

// One workgroup after each head: reduce the per-block maxima to the code (or
// sample it from the head's logits), record it (the model's code and the
// committed/forced one), gather the next step's inputs and, after the frame's
// last head, advance the position.
__device__ __forceinline__ void commit_body(const CommitArgs& a, char* lds) {
  unsigned long long* red = reinterpret_cast<unsigned long long*>(lds);
  int* code_sh = reinterpret_cast<int*>(lds + kWaves * sizeof(unsigned long long));
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // independent loads first: they overlap the slot reduction
  const int force = *a.force_flag, forced = a.forced[a.code_index], pos = *a.pos;
  int sampled = 0;
  if (a.smp.u) {
    // window: this codebook's committed codes at positions [lo, pos)
    const int lo = max(*a.smp.win_lo, pos - a.smp.window);
    sampled = sample_row(a.logits, a.V, a.smp, a.smp.u[(size_t)pos * a.frame_codes + a.code_index],
                         a.ring + (size_t)lo * a.frame_codes + a.code_index, a.frame_codes, max(pos - lo, 0), lds);
    __syncthreads();  // the LDS is reused below
  }
  unsigned long long b = 0ull;
  for (int i = tid; i < a.nslots; i += kBlock) b = a.slots[i] > b ? a.slots[i] : b;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(b, off);
    b = o > b ? o : b;
  }
  if (lane == 0) red[wave] = b;
  __syncthreads();
  if (tid == 0) {
    unsigned long long m = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = red[w] > m ? red[w] : m;
    const int pred = a.smp.u ? sampled : (int)(0xffffffffu - (uint32_t)(m & 0xffffffffull));
    const int code = force ? forced : pred;
    a.pred[a.code_index] = pred;
    a.committed[a.code_index] = code;
    a.ring[(size_t)pos * a.frame_codes + a.code_index] = code;
    *code_sh = code;
  }
  __syncthreads();
  const int code = *code_sh;
  if (a.next_table) {
    const int c = min(max(code, 0), a.next_rows - 1);
    const uint16_t* row = a.next_table + (size_t)c * a.K;
    for (int k = tid; k < a.K; k += kBlock) a.next_x[k] = bf2f(row[k]);
  }
  if (a.slow_table) {
    const int c = min(max(code, 0), a.slow_rows - 1);
    const uint16_t* row = a.slow_table + (size_t)c * a.K;
    for (int k = tid; k < a.K; k += kBlock) a.slow_x[k] = bf2f(row[k]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (a.copy_src[j]) {
      for (int k = tid; k < a.copy_n[j]; k += kBlock) a.copy_dst[j][k] = a.copy_src[j][k];
    }
  }
  __syncthreads();
  if (a.pos_inc && tid == 0) *a.pos_inc = *a.pos_inc + 1;
}

// Positions attended by query row m (its own position + 1, causal) and the
// offset of its sequence's cache: rows at *pos + m of one cache by default,
// or per-row positions and sequences (batched decode, fast AR first pass).
__device__ __forceinline__ int attn_len(const AttnArgs& a, int m) {
  return (a.row_pos ? a.row_pos[m] : *a.pos + m) + 1;
}
// Offset of the cache block holding position j0 of row m's sequence and, in
// jb0, the first position that block holds: a sequence's whole cache
// (jb0 = 0), or with a page table the page of j0 (positions j0 .. the page's
// end are then at j - jb0 within it).
__device__ __forceinline__ size_t attn_kv_base(const AttnArgs& a, int m, int j0, int& jb0) {
  const int sq = a.row_seq ? a.row_seq[m] : a.seq0;
  if (a.page_table) {
    const int pi = j0 >> a.page_shift;
    jb0 = pi << a.page_shift;
    return (size_t)a.page_table[(size_t)sq * a.pages_per_seq + pi] * a.seq_stride;
  }
  jb0 = 0;
  return (size_t)sq * a.seq_stride;
}

// One output value of the attention, and its hi/lo bf16 pair when asked for.
__device__ __forceinline__ void attn_store(const AttnArgs& a, size_t idx, float v) {
  a.out[idx] = v;
  if (a.out_hi) {
    const uint16_t h = f2bf(v);
    a.out_hi[idx] = h;
    a.out_lo[idx] = f2bf(v - bf2f(h));
  }
}

// Stores and loads of data that another workgroup, possibly on another XCD,
// reads or wrote inside the same launch: system scope (sc0 sc1), so the store
// writes through to memory and the load does not take a line one XCD's L2
// held from before.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ------------------------------------------------ split-K decode attention --

// One block = one KV head x one split of `chunk` positions for one query row
// (bid = (m * n_kv + kvh) * nsplit_max + s). hd/8 lanes cover one key row (16
// bytes each); a wave covers 64/(hd/8) positions per step and keeps an online
// softmax per lane group; groups and waves are merged at the end. With one
// split the block writes the output; otherwise it writes the split's (max,
// sum, acc), and either combine_body merges the splits in the following
// launch (a.cnt null) or the last split of the (row, KV head) to finish
// merges them in this one (a.cnt set). The merging split reads partials that
// workgroups on other XCDs wrote; those are exchanged with system-coherent
// stores and loads (written through to memory, not held in one XCD's L2), the
// writers wait for their stores to complete before they count themselves, and
// the count is an agent-scope atomic, so no cache-wide fence is needed.
template <int HD, int G>
__device__ __forceinline__ void attn_body(const AttnArgs& a, int bid, char* lds) {
  constexpr int LPP = HD / 8;
  constexpr int PPW = kWave / LPP;
  constexpr int U = 4;
  const int s = bid % a.nsplit_max;
  const int kvh = (bid / a.nsplit_max) % a.n_heads_kv;
  const int m = bid / (a.nsplit_max * a.n_heads_kv);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int T = attn_len(a, m);
  const int nsplit = (T + a.chunk - 1) / a.chunk;
  if (s >= nsplit) return;
  const int j0 = s * a.chunk, j1 = min(T, j0 + a.chunk);
  const int grp = lane / LPP, sub = lane % LPP;
  float* sm_acc = reinterpret_cast<float*>(lds);            // [kWaves][G][HD]
  float* sm_ml = sm_acc + kWaves * G * HD;                   // [kWaves][G][2]

  const float qscale = 1.4426950408889634f / sqrtf((float)HD);  // log2(e)/sqrt(hd)
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qp = a.q + (size_t)m * a.q_stride + (kvh * G + h) * HD + sub * 8;
    const float4 q0 = *reinterpret_cast<const float4*>(qp);
    const float4 q1 = *reinterpret_cast<const float4*>(qp + 4);
    qv[h][0] = q0.x * qscale; qv[h][1] = q0.y * qscale; qv[h][2] = q0.z * qscale; qv[h][3] = q0.w * qscale;
    qv[h][4] = q1.x * qscale; qv[h][5] = q1.y * qscale; qv[h][6] = q1.z * qscale; qv[h][7] = q1.w * qscale;
  }
  float mx[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mx[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  // the split's positions lie in one cache block (a page never ends inside a split)
  int jb0;
  const size_t kv0 = attn_kv_base(a, m, j0, jb0) + (size_t)kvh * a.cache_len * HD + sub * 8;
  const uint16_t* Kb = a.K + kv0;
  const uint16_t* Vb = a.V + kv0;
  constexpr int STEP = kWaves * PPW;
  for (int jb = j0 + wave * PPW; jb < j1; jb += STEP * U) {
    u32x4 kk[U], vv[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * STEP + grp;
      ok[u] = j < j1;
      kk[u] = ok[u] ? ld16(Kb + (size_t)(j - jb0) * HD) : u32x4{0u, 0u, 0u, 0u};
      vv[u] = ok[u] ? ld16(Vb + (size_t)(j - jb0) * HD) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float kf[8] = {bf_lo(kk[u].x), bf_hi(kk[u].x), bf_lo(kk[u].y), bf_hi(kk[u].y),
                           bf_lo(kk[u].z), bf_hi(kk[u].z), bf_lo(kk[u].w), bf_hi(kk[u].w)};
      const float vf[8] = {bf_lo(vv[u].x), bf_hi(vv[u].x), bf_lo(vv[u].y), bf_hi(vv[u].y),
                           bf_lo(vv[u].z), bf_hi(vv[u].z), bf_lo(vv[u].w), bf_hi(vv[u].w)};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sc = fmaf(qv[h][e], kf[e], sc);
        sc = row_sum<LPP>(sc);
        if (ok[u]) {
          const float mn = fmaxf(mx[h], sc);
          const float corr = exp2f(mx[h] - mn);
          const float pr = exp2f(sc - mn);
          l[h] = l[h] * corr + pr;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e] * corr);
          mx[h] = mn;
        }
      }
    }
  }
  // merge the PPW lane groups of this wave (xor over the group bits of the lane id)
#pragma unroll
  for (int off = LPP; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(mx[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(mx[h], mo);
      const float ca = (mx[h] == -INFINITY) ? 0.f : exp2f(mx[h] - mn);
      const float cb = (mo == -INFINITY) ? 0.f : exp2f(mo - mn);
      l[h] = l[h] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * ca + ao * cb;
      }
      mx[h] = mn;
    }
  }
  // merge the waves through LDS
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[(wave * G + h) * HD + sub * 8 + e] = acc[h][e];
      if (sub == 0) {
        sm_ml[(wave * G + h) * 2 + 0] = mx[h];
        sm_ml[(wave * G + h) * 2 + 1] = l[h];
      }
    }
  }
  __syncthreads();
  const bool merge_here = a.cnt != nullptr;
  const bool direct = a.nsplit_max == 1 || (merge_here && nsplit == 1);
  const int stride_s = G * (HD + 2);
  float* part = a.part + (((size_t)m * a.n_heads_kv + kvh) * a.nsplit_max) * stride_s;
  for (int idx = tid; idx < G * HD; idx += kBlock) {
    const int h = idx / HD, e = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[(w * G + h) * 2]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_ml[(w * G + h) * 2];
      const float c = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      num += sm_acc[(w * G + h) * HD + e] * c;
      den += sm_ml[(w * G + h) * 2 + 1] * c;
    }
    if (direct) {
      // a single split covers every position: normalise and write the output
      attn_store(a, (size_t)m * a.out_stride + (kvh * G + h) * HD + e, num / den);
    } else if (merge_here) {
      float* ps = part + (size_t)s * stride_s + h * (HD + 2);
      st_coherent(ps + e, num);
      if (e == 0) {
        st_coherent(ps + HD, M);
        st_coherent(ps + HD + 1, den);
      }
    } else {
      float* ps = part + (size_t)s * stride_s + h * (HD + 2);
      ps[e] = num;
      if (e == 0) {
        ps[HD] = M;
        ps[HD + 1] = den;
      }
    }
  }
  if (direct || !merge_here) return;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partials have reached memory
  __syncthreads();                // ... and every wave's (the LDS above is free again)
  int* last = reinterpret_cast<int*>(lds);
  if (tid == 0) {
    unsigned* c = a.cnt + (size_t)m * a.n_heads_kv + kvh;
    const unsigned before = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool is_last = before + 1u == (unsigned)nsplit;
    if (is_last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next launch
    *last = is_last;
  }
  __syncthreads();
  if (!*last) return;
  // every split has written its partials: merge them in split order (the
  // same sums whichever split arrives last), MU splits' loads in flight per
  // step, with the running maximum rescaling the sums as in the splits
  constexpr int MU = 4;
#pragma unroll
  for (int i = 0; i < (G * HD + kBlock - 1) / kBlock; ++i) {
    const int idx = tid + i * kBlock;
    if (idx >= G * HD) break;
    const int h = idx / HD, e = idx % HD;
    const float* ph = part + h * (HD + 2);
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int t0 = 0; t0 < nsplit; t0 += MU) {
      float mv[MU], lv[MU], av[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const float* pt = ph + (size_t)min(t0 + u, nsplit - 1) * stride_s;
        mv[u] = ld_coherent(pt + HD);
        lv[u] = ld_coherent(pt + HD + 1);
        av[u] = ld_coherent(pt + e);
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        if (t0 + u < nsplit) {
          const float mn = fmaxf(M, mv[u]);
          const float ca = exp2f(M - mn);  // 0 for the first split (M = -inf)
          const float cb = exp2f(mv[u] - mn);
          num = num * ca + av[u] * cb;
          den = den * ca + lv[u] * cb;
          M = mn;
        }
      }
    }
    attn_store(a, (size_t)m * a.out_stride + (kvh * G + h) * HD + e, num / den);
  }
}

// Combine the splits of one query head (bid = (m * n_kv + kvh) * G + h):
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s. Latency first: the
// split maxima are loaded in one pass and reduced across wave 0, then every
// thread issues all its accumulator loads before summing them.
template <int HD, int G>
__device__ __forceinline__ void combine_body(const AttnArgs& a, int bid, char* lds) {
  constexpr int R = kBlock / HD;  // threads per output element
  constexpr int U = 8;            // loads in flight per thread
  const int h = bid % G, kvh = (bid / G) % a.n_heads_kv, m = bid / (G * a.n_heads_kv);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int T = attn_len(a, m);
  const int nsplit = (T + a.chunk - 1) / a.chunk;
  const int stride_s = G * (HD + 2);
  const float* part = a.part + (((size_t)m * a.n_heads_kv + kvh) * a.nsplit_max) * stride_s + h * (HD + 2);
  float* wsh = reinterpret_cast<float*>(lds);  // [nsplit_max] split weights, then the denominator
  float* red = wsh + a.nsplit_max + 1;         // [R][HD]
  if (wave == 0) {
    float mx = -INFINITY;
    for (int t = lane; t < nsplit; t += kWave) mx = fmaxf(mx, part[(size_t)t * stride_s + HD]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float den = 0.f;
    for (int t = lane; t < nsplit; t += kWave) {
      const float* ps = part + (size_t)t * stride_s;
      const float c = exp2f(ps[HD] - mx);
      wsh[t] = c;
      den += c * ps[HD + 1];
    }
    den = wave_sum(den);
    if (lane == 0) wsh[a.nsplit_max] = den;
  }
  __syncthreads();
  const int e = tid % HD, r = tid / HD;
  float num = 0.f;
  for (int t0 = r; t0 < nsplit; t0 += R * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = part[(size_t)min(t0 + u * R, nsplit - 1) * stride_s + e];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t0 + u * R < nsplit) num = fmaf(wsh[t0 + u * R], v[u], num);
  }
  red[r * HD + e] = num;
  __syncthreads();
  if (r == 0) {
    float sum = red[e];
#pragma unroll
    for (int q = 1; q < R; ++q) sum += red[q * HD + e];
    attn_store(a, (size_t)m * a.out_stride + (kvh * G + h) * HD + e, sum / wsh[a.nsplit_max]);
  }
}

// -------------------------------------------- register-input weight streaming --

// Wave-independent GEMV machinery for inputs of at most NCH chunks (NCH*64*E
// columns, E = 8 bf16 or 16 fp8 / int8 per 16-byte load, 8 int4 per 4-byte
// load). Each lane keeps its own
// slice of the input row in registers (the same columns for every weight row
// it touches), so no LDS staging and no workgroup barrier are needed: a wave
// issues its input loads, then every weight load of all its rows at once (one
// memory round trip), normalises its slice with one wave reduction, and
// consumes the weights as they arrive. Lanes past the row end load a clamped
// address and hold a zero input, so they add nothing.
template <typename WT, int NCH, int RPW>
struct RegStream {
  static constexpr int E = Dot<WT>::E;
  static constexpr int CW = kWave * E;
  static constexpr int NX = E / 4;   // float4 of input per chunk
  static constexpr int NG = E / 8;   // 16-byte loads of bf16 gain per chunk
  static constexpr bool kBiased = WT::kGrouped;  // int4: offset-binary products, see Dot<INT4>
  float4 x[NCH][NX];
  u32x4 g[NCH][NG];
  typename Dot<WT>::V w[RPW][NCH];
  float gs[RPW][NCH];  // group scale of each row's chunk slice (group-scaled types)
  float xb[NCH];       // 8 * the sum of this lane's slice of chunk c (kBiased)
  int lane, K;
  int c0 = 0, cs = 1;  // this wave's chunk c is input chunk c0 + c * cs

  // column of this lane's slice of chunk c
  __device__ __forceinline__ int col_of(int c) const { return (c0 + c * cs) * CW + lane * E; }

  __device__ __forceinline__ void load_x(const float* xp, const uint16_t* gain, int K_, int lane_) {
    lane = lane_;
    K = K_;
    const uint16_t* gsrc = gain ? gain : reinterpret_cast<const uint16_t*>(xp);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int col = min(col_of(c), K - E);
#pragma unroll
      for (int j = 0; j < NX; ++j) x[c][j] = *reinterpret_cast<const float4*>(xp + col + 4 * j);
#pragma unroll
      for (int j = 0; j < NG; ++j) g[c][j] = *reinterpret_cast<const u32x4*>(gsrc + col + 8 * j);
    }
  }

  __device__ __forceinline__ void load_w(const char* const (&base)[RPW], const float* const* scales = nullptr) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int col = min(col_of(c), K - E);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        w[i][c] = Dot<WT>::load(base[i] + wbytes<WT>(col));
        if constexpr (WT::kGrouped) gs[i][c] = scales[i][col / kGroup];
      }
    }
  }

  // zero the slices past the row end; with a gain, x <- x / sqrt(mean(x^2) + eps) * gain
  __device__ __forceinline__ void prepare(bool has_gain, float eps) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const bool valid = col_of(c) < K;
#pragma unroll
      for (int j = 0; j < NX; ++j) {
        if (!valid) x[c][j] = make_float4(0.f, 0.f, 0.f, 0.f);
        ss += (x[c][j].x * x[c][j].x + x[c][j].y * x[c][j].y) + (x[c][j].z * x[c][j].z + x[c][j].w * x[c][j].w);
      }
    }
    if (!has_gain) {
      slice_bias();
      return;
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const u32x4 gg = g[c][j];
        float4& a = x[c][2 * j];
        float4& b = x[c][2 * j + 1];
        a.x = (a.x * inv) * bf_lo(gg.x);
        a.y = (a.y * inv) * bf_hi(gg.x);
        a.z = (a.z * inv) * bf_lo(gg.y);
        a.w = (a.w * inv) * bf_hi(gg.y);
        b.x = (b.x * inv) * bf_lo(gg.z);
        b.y = (b.y * inv) * bf_hi(gg.z);
        b.z = (b.z * inv) * bf_lo(gg.w);
        b.w = (b.w * inv) * bf_hi(gg.w);
      }
    }
    slice_bias();
  }

  __device__ __forceinline__ void slice_bias() {
    if constexpr (kBiased) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < NX; ++j) t += (x[c][j].x + x[c][j].y) + (x[c][j].z + x[c][j].w);
        xb[c] = 8.f * t;
      }
    }
  }

  __device__ __forceinline__ float dot_row(int i) const {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const float* xc = reinterpret_cast<const float*>(&x[c][0]);
      if constexpr (kBiased) {
        acc = fmaf(gs[i][c], Dot<WT>::run_biased(w[i][c], xc) - xb[c], acc);
      } else if constexpr (WT::kGrouped) {
        acc = fmaf(gs[i][c], Dot<WT>::run(w[i][c], xc), acc);
      } else {
        acc += Dot<WT>::run(w[i][c], xc);
      }
    }
    return acc;
  }

  // write this lane's (normalised) slice of the input to dst (valid columns only)
  __device__ __forceinline__ void store_x(float* dst) const {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int col = col_of(c);
      if (col < K) {
#pragma unroll
        for (int j = 0; j < NX; ++j) *reinterpret_cast<float4*>(dst + col + 4 * j) = x[c][j];
      }
    }
  }
};

// Outputs per wave of the register kernels: an fp8 row is half the bytes of a
// bf16 row, so fp8 waves take two outputs to keep the weight bytes per input
// slice (read from L2 by every wave) the same.
template <typename WT>
struct PerWave {
  static constexpr int v = 1;
};
// One-byte weights: three outputs per wave (fewer, wider workgroups share the
// chip better with the other chain's launches: fp8 frame 396 -> 410 frames/s,
// although a W13 launch alone takes 14.9 instead of 13.9 us), two QKV
// rotation pairs per wave.
template <>
struct PerWave<FP8> {
  static constexpr int v = 3;
};
template <>
struct PerWave<INT8> {
  static constexpr int v = 3;
};
template <>
struct PerWave<INT4> {
  static constexpr int v = 2;  // more waves rather than more rows each: the int4 dot is ALU-heavy
};
// Rows per wave of the plain GEMV (Wo, fast first pass) and of the fused QKV
// (rotation pairs per wave) where they differ from the SwiGLU's PerWave.
template <typename WT>
struct PerWaveGemv {
  static constexpr int v = PerWave<WT>::v;
};
template <typename WT>
struct PerWaveQkv {
  static constexpr int v = PerWave<WT>::v;
};
// Inputs of at least this many chunks go to the split-K GEMV (four waves share
// a row's chunks) when there is no RMSNorm prologue.
template <typename WT>
struct SplitFrom {
  static constexpr int v = 9;
};
template <>
struct PerWaveQkv<FP8> {
  static constexpr int v = 2;
};
template <>
struct PerWaveQkv<INT8> {
  static constexpr int v = 2;
};

// y[r] (+)= scale[r] * W[r] . x, P rows per wave
template <typename WT, int NCH>
__device__ __forceinline__ void gemv_reg_body(const GemvArgs& a, int bid) {
  constexpr int P = PerWaveGemv<WT>::v;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int r0 = (bid * kWaves + wave) * P;
  RegStream<WT, NCH, P> rs;
  rs.load_x(a.x, a.gain, a.K, lane);
  const char* base[P];
  const float* sc[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    base[i] = row_ptr<WT>(a.W, min(r0 + i, a.rows - 1), a.K);
    sc[i] = group_scales<WT>(a.scale, min(r0 + i, a.rows - 1), a.K);
  }
  rs.load_w(base, sc);
  rs.prepare(a.gain != nullptr, a.eps);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int r = r0 + i;
    if (r >= a.rows) return;
    float s = wave_sum(rs.dot_row(i));
    if (lane == 0) {
      s *= row_scale<WT>(a.scale, r);
      float* y = a.y + r;
      *y = a.accumulate ? (*y + s) : s;
    }
  }
}

// fused RMSNorm + QKV + RoPE + KV append; a wave takes P rotation pairs
// (head, i), (head, i + hd/2)
template <typename WT, int NCH>
__device__ __forceinline__ void qkv_reg_body(const QkvArgs& a, int bid) {
  constexpr int P = PerWaveQkv<WT>::v;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int half = a.head_dim / 2;
  const int n_heads = a.n_heads_q + 2 * a.n_heads_kv;
  const int npairs = n_heads * half;
  const int p0 = (bid * kWaves + wave) * P;
  RegStream<WT, NCH, 2 * P> rs;
  rs.load_x(a.x, a.gain, a.K, lane);
  const char* base[2 * P];
  const float* sc[2 * P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int pc = min(p0 + j, npairs - 1);
    const int r1 = (pc / half) * a.head_dim + pc % half;
    base[2 * j] = row_ptr<WT>(a.W, r1, a.K);
    base[2 * j + 1] = row_ptr<WT>(a.W, r1 + half, a.K);
    sc[2 * j] = group_scales<WT>(a.scale, r1, a.K);
    sc[2 * j + 1] = group_scales<WT>(a.scale, r1 + half, a.K);
  }
  rs.load_w(base, sc);
  rs.prepare(true, a.eps);
  const int pos = *a.pos;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int p = p0 + j;
    if (p >= npairs) return;
    const int head = p / half, i = p % half;
    const int r1 = head * a.head_dim + i, r2 = r1 + half;
    const float y1 = wave_sum(rs.dot_row(2 * j));
    const float y2 = wave_sum(rs.dot_row(2 * j + 1));
    if (lane != 0) continue;
    const float u = y1 * row_scale<WT>(a.scale, r1), v = y2 * row_scale<WT>(a.scale, r2);
    if (head < a.n_heads_q + a.n_heads_kv) {
      const float2 cs = a.rope[(size_t)pos * half + i];
      const float o1 = u * cs.x - v * cs.y;
      const float o2 = u * cs.y + v * cs.x;
      if (head < a.n_heads_q) {
        a.q_out[r1] = o1;
        a.q_out[r2] = o2;
      } else {
        uint16_t* kp = a.kc + ((size_t)(head - a.n_heads_q) * a.cache_len + pos) * a.head_dim;
        kp[i] = f2bf(o1);
        kp[i + half] = f2bf(o2);
      }
    } else {
      uint16_t* vp = a.vc + ((size_t)(head - a.n_heads_q - a.n_heads_kv) * a.cache_len + pos) * a.head_dim;
      vp[i] = f2bf(u);
      vp[i + half] = f2bf(v);
    }
  }
}

// fused RMSNorm + W1/W3 + SiLU(a)*b; a wave takes P outputs r (rows W1[r], W3[r])
template <typename WT, int NCH>
__device__ __forceinline__ void swiglu_reg_body(const SwigluArgs& a, int bid) {
  constexpr int P = PerWave<WT>::v;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int r0 = (bid * kWaves + wave) * P;
  RegStream<WT, NCH, 2 * P> rs;
  rs.load_x(a.x, a.gain, a.K, lane);
  const char* base[2 * P];
  const float* sc[2 * P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int rc = min(r0 + j, a.F - 1);
    base[2 * j] = row_ptr<WT>(a.W1, rc, a.K);
    base[2 * j + 1] = row_ptr<WT>(a.W3, rc, a.K);
    sc[2 * j] = group_scales<WT>(a.s1, rc, a.K);
    sc[2 * j + 1] = group_scales<WT>(a.s3, rc, a.K);
  }
  rs.load_w(base, sc);
  rs.prepare(true, a.eps);
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int r = r0 + j;
    if (r >= a.F) return;
    float g = wave_sum(rs.dot_row(2 * j));
    float u = wave_sum(rs.dot_row(2 * j + 1));
    if (lane == 0) {
      g *= row_scale<WT>(a.s1, r);
      u *= row_scale<WT>(a.s3, r);
      const float silu = g / (1.0f + expf(-g));
      a.h[r] = silu * u;
    }
  }
}

// Inputs wider than the register path (the FFN down-projection): the block's
// waves split the input's chunks (wave w takes chunks w, w + 4, ...) over R
// rows, so each wave holds a quarter of the input in registers and issues all
// its row loads at once; the partial sums meet in LDS. No input norm.
template <typename WT, int NCW, int R>
__device__ __forceinline__ void gemv_split_body(const GemvArgs& a, int bid, char* lds) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int r0 = bid * R;
  RegStream<WT, NCW, R> rs;
  rs.c0 = wave;
  rs.cs = kWaves;
  rs.load_x(a.x, nullptr, a.K, lane);
  const char* base[R];
  const float* sc[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    base[i] = row_ptr<WT>(a.W, min(r0 + i, a.rows - 1), a.K);
    sc[i] = group_scales<WT>(a.scale, min(r0 + i, a.rows - 1), a.K);
  }
  rs.load_w(base, sc);
  rs.prepare(false, 0.f);
  float* part = reinterpret_cast<float*>(lds);  // [kWaves][R]
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float p = wave_sum(rs.dot_row(i));
    if (lane == 0) part[wave * R + i] = p;
  }
  __syncthreads();
  if (wave == 0 && lane < R && r0 + lane < a.rows) {
    const int r = r0 + lane;
    float s = part[lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += part[w * R + lane];
    s *= row_scale<WT>(a.scale, r);
    float* y = a.y + r;
    *y = a.accumulate ? (*y + s) : s;
  }
}

// fused RMSNorm + head GEMV + per-block argmax (two rows per wave)
template <typename WT, int NCH>
__device__ __forceinline__ void head_reg_body(const HeadArgs& a, int bid, char* lds) {
  unsigned long long* wbest = reinterpret_cast<unsigned long long*>(lds);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int r0 = (bid * kWaves + wave) * 2;
  RegStream<WT, NCH, 2> rs;
  rs.load_x(a.x, a.gain, a.K, lane);
  const char* base[2] = {row_ptr<WT>(a.W, min(r0, a.rows - 1), a.K), row_ptr<WT>(a.W, min(r0 + 1, a.rows - 1), a.K)};
  const float* sc[2] = {group_scales<WT>(a.scale, min(r0, a.rows - 1), a.K),
                        group_scales<WT>(a.scale, min(r0 + 1, a.rows - 1), a.K)};
  rs.load_w(base, sc);
  rs.prepare(true, a.eps);
  if (a.h_out && bid == 0 && wave == 0) rs.store_x(a.h_out);
  unsigned long long best = 0ull;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = r0 + i;
    float s = wave_sum(rs.dot_row(i));
    if (r < a.rows) {
      s *= row_scale<WT>(a.scale, r);
      if (lane == 0) {
        a.logits[r] = s;
        if (!isfinite(s)) atomicAdd(a.anomalies, 1);
      }
      const unsigned long long k = argmax_key(s, r);
      best = k > best ? k : best;
    }
  }
  if (lane == 0) wbest[wave] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = wbest[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) b = wbest[w] > b ? wbest[w] : b;
    a.slots[bid] = b;  // reduced by the commit that follows
    if (a.pos_inc && bid == 0) *a.pos_inc = *a.pos_inc + 1;
  }
}

// ------------------------------------------- one-workgroup-per-head attention --

// Decode attention without splits: block = (query row m, KV head kvh), NW
// waves; wave w takes passes w, w+NW, ... of PPW positions each, U passes of
// K/V loads in flight; per-lane online softmax, merged across lane groups with
// shuffles and across waves through LDS; the block writes the g heads' output.
template <int HD, int G, int NW, int U>
__device__ __forceinline__ void attn_wide_body(const AttnArgs& a, int bid, char* lds) {
  constexpr int LPP = HD / 8;
  constexpr int PPW = kWave / LPP;
  constexpr int STEP = NW * PPW;
  constexpr int NT = NW * kWave;
  const int kvh = bid % a.n_heads_kv, m = bid / a.n_heads_kv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int T = attn_len(a, m);
  const int grp = lane / LPP, sub = lane % LPP;
  float* sm_acc = reinterpret_cast<float*>(lds);  // [NW][G][HD]
  float* sm_ml = sm_acc + NW * G * HD;            // [NW][G][2]

  const float qscale = 1.4426950408889634f / sqrtf((float)HD);  // log2(e)/sqrt(hd)
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qp = a.q + (size_t)m * a.q_stride + (kvh * G + h) * HD + sub * 8;
    const float4 q0 = *reinterpret_cast<const float4*>(qp);
    const float4 q1 = *reinterpret_cast<const float4*>(qp + 4);
    qv[h][0] = q0.x * qscale; qv[h][1] = q0.y * qscale; qv[h][2] = q0.z * qscale; qv[h][3] = q0.w * qscale;
    qv[h][4] = q1.x * qscale; qv[h][5] = q1.y * qscale; qv[h][6] = q1.z * qscale; qv[h][7] = q1.w * qscale;
  }
  float mx[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mx[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  // every position of a one-split launch lies in the first cache block (with
  // a page table: T <= one split <= the page length)
  int jb0;
  const size_t kv0 = attn_kv_base(a, m, 0, jb0) + (size_t)kvh * a.cache_len * HD + sub * 8;
  const uint16_t* Kb = a.K + kv0;
  const uint16_t* Vb = a.V + kv0;
  for (int jb = wave * PPW; jb < T; jb += STEP * U) {
    u32x4 kk[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(jb + u * STEP + grp, T - 1);  // clamped: always a valid row
      kk[u] = ld16(Kb + (size_t)j * HD);
      vv[u] = ld16(Vb + (size_t)j * HD);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = jb + u * STEP + grp < T;
      const float kf[8] = {bf_lo(kk[u].x), bf_hi(kk[u].x), bf_lo(kk[u].y), bf_hi(kk[u].y),
                           bf_lo(kk[u].z), bf_hi(kk[u].z), bf_lo(kk[u].w), bf_hi(kk[u].w)};
      const float vf[8] = {bf_lo(vv[u].x), bf_hi(vv[u].x), bf_lo(vv[u].y), bf_hi(vv[u].y),
                           bf_lo(vv[u].z), bf_hi(vv[u].z), bf_lo(vv[u].w), bf_hi(vv[u].w)};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sc = fmaf(qv[h][e], kf[e], sc);
        sc = row_sum<LPP>(sc);
        if (ok) {
          const float mn = fmaxf(mx[h], sc);
          const float corr = exp2f(mx[h] - mn);
          const float pr = exp2f(sc - mn);
          l[h] = l[h] * corr + pr;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e] * corr);
          mx[h] = mn;
        }
      }
    }
  }
#pragma unroll
  for (int off = LPP; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(mx[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(mx[h], mo);
      const float ca = (mx[h] == -INFINITY) ? 0.f : exp2f(mx[h] - mn);
      const float cb = (mo == -INFINITY) ? 0.f : exp2f(mo - mn);
      l[h] = l[h] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * ca + ao * cb;
      }
      mx[h] = mn;
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[(wave * G + h) * HD + sub * 8 + e] = acc[h][e];
      if (sub == 0) {
        sm_ml[(wave * G + h) * 2 + 0] = mx[h];
        sm_ml[(wave * G + h) * 2 + 1] = l[h];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * HD; idx += NT) {
    const int h = idx / HD, e = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_ml[(w * G + h) * 2]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_ml[(w * G + h) * 2];
      const float c = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      num += sm_acc[(w * G + h) * HD + e] * c;
      den += sm_ml[(w * G + h) * 2 + 1] * c;
    }
    attn_store(a, (size_t)m * a.out_stride + (kvh * G + h) * HD + e, num / den);
  }
}

// --------------------------------------------------------- stage bodies --
//
// Every stage is a body run by one 256-lane workgroup given its block index
// within the stage; k_one<Body> launches one stage.

template <typename WT, int NCH>
struct GemvR {
  using Args = GemvArgs;
  __device__ static void run(const Args& a, int bid, char*) { gemv_reg_body<WT, NCH>(a, bid); }
};
template <typename WT, int NCW, int R>
struct GemvS {
  using Args = GemvArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { gemv_split_body<WT, NCW, R>(a, bid, lds); }
};
template <typename WT, int M>
struct GemvL {
  using Args = GemvArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { gemv_body<WT, M, 2>(a, bid, lds); }
};
template <typename WT, int NCH>
struct QkvR {
  using Args = QkvArgs;
  __device__ static void run(const Args& a, int bid, char*) { qkv_reg_body<WT, NCH>(a, bid); }
};
template <typename WT, int M>
struct QkvL {
  using Args = QkvArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { qkv_body<WT, M>(a, bid, lds); }
};
template <typename WT, int NCH>
struct SwiR {
  using Args = SwigluArgs;
  __device__ static void run(const Args& a, int bid, char*) { swiglu_reg_body<WT, NCH>(a, bid); }
};
template <typename WT, int M>
struct SwiL {
  using Args = SwigluArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { swiglu_body<WT, M>(a, bid, lds); }
};
template <typename WT, int NCH>
struct HeadR {
  using Args = HeadArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { head_reg_body<WT, NCH>(a, bid, lds); }
};
template <typename WT>
struct HeadL {
  using Args = HeadArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { head_body<WT>(a, bid, lds); }
};
struct Commit {
  using Args = CommitArgs;
  __device__ static void run(const Args& a, int, char* lds) { commit_body(a, lds); }
};
template <int HD, int G>
struct AttS {
  using Args = AttnArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { attn_body<HD, G>(a, bid, lds); }
};
template <int HD, int G>
struct AttC {
  using Args = AttnArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { combine_body<HD, G>(a, bid, lds); }
};
template <int HD, int G>
struct AttW {
  using Args = AttnArgs;
  __device__ static void run(const Args& a, int bid, char* lds) { attn_wide_body<HD, G, 4, 2>(a, bid, lds); }
};

template <class A>
__global__ __launch_bounds__(kBlock) void k_one(typename A::Args a) {
  extern __shared__ __align__(16) char lds[];
  A::run(a, blockIdx.x, lds);
}


// ---------------------------------------------------------- small kernels --

__global__ void k_embed(const uint16_t* table, int rows, int K, const int* tok, float* x, int* pos_out,
                        int pos_value, int* anomalies) {
  const int t = *tok;
  const int c = min(max(t, 0), rows - 1);
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    if (t != c) atomicAdd(anomalies, 1);
    if (pos_out) *pos_out = pos_value;
  }
  const uint16_t* row = table + (size_t)c * K;
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < K; k += gridDim.x * blockDim.x) x[k] = bf2f(row[k]);
}

__global__ void k_set_forced(const int* forced, int n, int* dst, int* flag) {
  if (forced)
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = forced[i];
  if (threadIdx.x == 0) *flag = forced ? 1 : 0;
}

__global__ void k_fill_i32(int* dst, int n, int value) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) dst[i] = value;
}

__global__ void k_fill_u32(unsigned* dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = 0u;
}

__global__ void k_copy_i32(const int* src, int* dst, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) dst[i] = src[i];
}

// e4m3fn encode of a finite fp32 value: nearest, ties to even, saturate at 448.
// Every step is exact in fp32 (scaling by powers of two), so the result is the
// correctly rounded code.
__device__ __forceinline__ uint8_t e4m3_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal step 2^-9
    code = (uint32_t)rintf(a * 512.0f);  // 8 here is the smallest normal's code
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // a normal fp32 here
    const float mant = __uint_as_float(__float_as_uint(a) & 0x807fffffu | 0x3f800000u) - 1.0f;
    uint32_t mq = (uint32_t)rintf(mant * 8.0f);
    if (mq == 8u) {
      mq = 0u;
      e += 1;
    }
    code = ((uint32_t)(e + 7) << 3) | mq;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return (uint8_t)(code | sign);
}

// One workgroup per row: scale = rowmax|w| / 448, codes = e4m3(w / scale).
__global__ __launch_bounds__(kBlock) void k_quantize_fp8(const uint16_t* w, int rows, int cols, uint8_t* q,
                                                        float* scale) {
  __shared__ float red[kWaves];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const uint16_t* row = w + (size_t)r * cols;
  float mx = 0.f;
  for (int k = tid; k < cols; k += kBlock) mx = fmaxf(mx, fabsf(bf2f(row[k])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float amax = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) amax = fmaxf(amax, red[i]);
  const float s = amax / 448.0f;
  if (tid == 0) scale[r] = s;
  uint8_t* qr = q + (size_t)r * cols;
  for (int k = tid; k < cols; k += kBlock) {
    qr[k] = (s > 0.f) ? e4m3_encode(bf2f(row[k]) / s) : (uint8_t)0;
  }
}

// One workgroup per row: scale = rowmax|w| / 127, codes = rint(w / scale)
// clamped to [-127, 127] (fp32 division, round half to even).
__global__ __launch_bounds__(kBlock) void k_quantize_int8(const uint16_t* w, int rows, int cols, int8_t* q,
                                                         float* scale) {
  __shared__ float red[kWaves];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const uint16_t* row = w + (size_t)r * cols;
  float mx = 0.f;
  for (int k = tid; k < cols; k += kBlock) mx = fmaxf(mx, fabsf(bf2f(row[k])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float amax = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) amax = fmaxf(amax, red[i]);
  const float s = amax / 127.0f;
  if (tid == 0) scale[r] = s;
  int8_t* qr = q + (size_t)r * cols;
  for (int k = tid; k < cols; k += kBlock)
    qr[k] = (s > 0.f) ? (int8_t)fminf(fmaxf(rintf(bf2f(row[k]) / s), -127.f), 127.f) : (int8_t)0;
}

// One workgroup per row; a wave per 128-column group at a time: scale =
// max|w| / 7 over the group, codes = rint(w / scale) clamped to [-7, 7], two
// per byte (the even column in the low nibble).
__global__ __launch_bounds__(kBlock) void k_quantize_int4(const uint16_t* w, int rows, int cols, uint8_t* q,
                                                         float* scale) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const uint16_t* row = w + (size_t)r * cols;
  const int ngroups = cols / kGroup;
  for (int gi = wave; gi < ngroups; gi += kWaves) {
    const int c = gi * kGroup + 2 * lane;  // this lane's pair of columns
    const float a = bf2f(row[c]), b = bf2f(row[c + 1]);
    float mx = fmaxf(fabsf(a), fabsf(b));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float s = mx / 7.0f;
    if (lane == 0) scale[(size_t)r * ngroups + gi] = s;
    int qa = 0, qb = 0;
    if (s > 0.f) {
      qa = (int)fminf(fmaxf(rintf(a / s), -7.f), 7.f);
      qb = (int)fminf(fmaxf(rintf(b / s), -7.f), 7.f);
    }
    q[((size_t)r * cols + c) / 2] = (uint8_t)((qa & 0xF) | ((qb & 0xF) << 4));
  }
}

// codes[r] = the code sampled from logits row r (one workgroup per row)
__global__ __launch_bounds__(kBlock) void k_sample_rows(const float* logits, int V, SampleArgs sp, const int* history,
                                                       int n_hist, int* codes) {
  extern __shared__ __align__(16) char lds[];
  const int r = blockIdx.x;
  const int c = sample_row(logits + (size_t)r * V, V, sp, sp.u[r], history + (size_t)r * n_hist, 1, n_hist, lds);
  if (threadIdx.x == 0) codes[r] = c;
}

__global__ void k_fp8_decode(const uint8_t* codes, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const uint32_t u = codes[i];
    out[i] = fp8x2_lo(u).x;
  }
}

// ---------------------------------------------------------------- launchers --

int head_grid(int rows) { return (rows + kWaves * 2 - 1) / (kWaves * 2); }

static size_t gemv_lds(int M, int K) { return (((size_t)M * K * 4 + 15) & ~(size_t)15) + 64; }

template <typename WT>
static int nch_of(int K) {
  constexpr int CW = kWave * Dot<WT>::E;
  return (K + CW - 1) / CW;
}

// grid and dynamic LDS of one task
struct Geo {
  int grid;
  size_t lds;
};

// Calls f(Body{}, args, geo) with the body that runs task t (weights of type
// WT, the codebook-0 head always bf16); false when t has no body.
#define DAR_NCH_CASES(CALL)    \
  case 1: CALL(1); return true; \
  case 2: CALL(2); return true; \
  case 3: CALL(3); return true; \
  case 4: CALL(4); return true; \
  case 5: CALL(5); return true; \
  case 8: CALL(8); return true; \
  default: break;

template <typename WT, typename HWT, typename F>
static bool head_body_for(const HeadArgs& a, F&& f) {
  const Geo g{head_grid(a.rows), 64};
#define CALL(N) f(HeadR<HWT, N>{}, a, g)
  switch (nch_of<HWT>(a.K)) { DAR_NCH_CASES(CALL) }
#undef CALL
  f(HeadL<HWT>{}, a, Geo{g.grid, gemv_lds(1, a.K)});
  return true;
}

template <int HD, int G, typename F>
static bool attn_body_for(const Task& t, F&& f) {
  const AttnArgs& a = t.attn;
  if (t.kind == T_COMBINE) {
    f(AttC<HD, G>{}, a, Geo{a.n_heads_kv * G * a.M, ((size_t)a.nsplit_max + 1 + kBlock) * 4});
  } else if (a.nsplit_max > 1) {
    f(AttS<HD, G>{}, a, Geo{a.nsplit_max * a.n_heads_kv * a.M, (size_t)kWaves * G * (HD + 2) * 4});
  } else {
    // one block per (query row, KV head): the fast AR's <= R+1 positions
    f(AttW<HD, G>{}, a, Geo{a.n_heads_kv * a.M, (size_t)4 * G * (HD + 2) * 4});
  }
  return true;
}

template <typename WT, typename F>
static bool with_body(const Task& t, F&& f) {
  switch (t.kind) {
    case T_GEMV: {
      const GemvArgs& a = t.gemv;
      if (t.M == 1) {
        const Geo g{(a.rows + kWaves * PerWaveGemv<WT>::v - 1) / (kWaves * PerWaveGemv<WT>::v), 0};
#define CALL(N) f(GemvR<WT, N>{}, a, g)
        if (a.gain || nch_of<WT>(a.K) < SplitFrom<WT>::v) {
          switch (nch_of<WT>(a.K)) { DAR_NCH_CASES(CALL) }
        }
#undef CALL
        if (!a.gain) {
          // wider inputs: four waves split the chunks, two rows per block
          const Geo gs{(a.rows + 1) / 2, 64};
#define CALL(N) f(GemvS<WT, N, 2>{}, a, gs)
          switch ((nch_of<WT>(a.K) + kWaves - 1) / kWaves) {
            DAR_NCH_CASES(CALL)
            case 6:
            case 7: f(GemvS<WT, 8, 2>{}, a, gs); return true;
          }
#undef CALL
        }
      }
      const Geo g{(a.rows + kWaves * 2 - 1) / (kWaves * 2), gemv_lds(t.M, a.K)};
      if (t.M == 2)
        f(GemvL<WT, 2>{}, a, g);
      else
        f(GemvL<WT, 1>{}, a, g);
      return true;
    }
    case T_QKV: {
      const QkvArgs& a = t.qkv;
      const int pairs = (a.n_heads_q + 2 * a.n_heads_kv) * a.head_dim / 2;
      const int grid = (pairs + kWaves - 1) / kWaves;
      if (t.M == 1) {
        const int rgrid = (pairs + kWaves * PerWaveQkv<WT>::v - 1) / (kWaves * PerWaveQkv<WT>::v);
#define CALL(N) f(QkvR<WT, N>{}, a, Geo{rgrid, 0})
        switch (nch_of<WT>(a.K)) { DAR_NCH_CASES(CALL) }
#undef CALL
      }
      if (t.M == 2)
        f(QkvL<WT, 2>{}, a, Geo{grid, gemv_lds(2, a.K)});
      else
        f(QkvL<WT, 1>{}, a, Geo{grid, gemv_lds(1, a.K)});
      return true;
    }
    case T_SWIGLU: {
      const SwigluArgs& a = t.swiglu;
      const int grid = (a.F + kWaves - 1) / kWaves;
      if (t.M == 1) {
        const int rgrid = (a.F + kWaves * PerWave<WT>::v - 1) / (kWaves * PerWave<WT>::v);
#define CALL(N) f(SwiR<WT, N>{}, a, Geo{rgrid, 0})
        switch (nch_of<WT>(a.K)) { DAR_NCH_CASES(CALL) }
#undef CALL
      }
      if (t.M == 2)
        f(SwiL<WT, 2>{}, a, Geo{grid, gemv_lds(2, a.K)});
      else
        f(SwiL<WT, 1>{}, a, Geo{grid, gemv_lds(1, a.K)});
      return true;
    }
    case T_HEAD: return head_body_for<WT, WT>(t.head, f);
    case T_HEAD_BF16: return head_body_for<WT, BF16>(t.head, f);
    case T_COMMIT:
      f(Commit{}, t.commit, Geo{1, t.commit.smp.u ? sample_lds_bytes(t.commit.V) : (size_t)64});
      return true;
    case T_ATTN:
    case T_COMBINE: {
      const int g = t.attn.n_heads_q / t.attn.n_heads_kv;
      if (t.attn.head_dim == 128) {
        switch (g) {
          case 1: return attn_body_for<128, 1>(t, f);
          case 2: return attn_body_for<128, 2>(t, f);
          case 4: return attn_body_for<128, 4>(t, f);
          case 8: return attn_body_for<128, 8>(t, f);
        }
      } else if (t.attn.head_dim == 64) {
        switch (g) {
          case 1: return attn_body_for<64, 1>(t, f);
          case 2: return attn_body_for<64, 2>(t, f);
          case 4: return attn_body_for<64, 4>(t, f);
          case 8: return attn_body_for<64, 8>(t, f);
        }
      }
      return false;
    }
    default: return false;
  }
}
#undef DAR_NCH_CASES

// kernels whose dynamic LDS may exceed the default 64 KB get the 160 KB limit
// once per kernel; the flag is atomic because contexts on other host threads
// launch the same kernels (setting the attribute twice is harmless)
template <typename KernelT>
static hipError_t allow_lds(KernelT kern, size_t lds, std::atomic<bool>& done) {
  if (lds <= 65536 || done.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.store(true, std::memory_order_release);
  return e;
}

// prep: only raise the LDS limit (before graph capture), no launch. With
// events, the launch itself stamps them at the kernel's start and end.
template <class A>
static hipError_t go1(const typename A::Args& a, const Geo& g, hipStream_t s, bool prep, hipEvent_t ev0,
                      hipEvent_t ev1) {
  static std::atomic<bool> big{false};  // one flag per kernel instantiation
  hipError_t e = allow_lds(k_one<A>, g.lds, big);
  if (e != hipSuccess || prep) return e;
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(k_one<A>, dim3(g.grid), dim3(kBlock), g.lds, s, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL(k_one<A>, dim3(g.grid), dim3(kBlock), g.lds, s, a);
  return hipGetLastError();
}

template <typename WT>
static hipError_t single_launch(const Task& t, hipStream_t s, bool prep, hipEvent_t ev0 = nullptr,
                                hipEvent_t ev1 = nullptr) {
  if (t.kind == T_NONE) return hipSuccess;
  hipError_t err = hipErrorInvalidValue;
  with_body<WT>(t, [&](auto body, const auto& args, const Geo& g) {
    err = go1<decltype(body)>(args, g, s, prep, ev0, ev1);
  });
  return err;
}

// the many-row stages (dar_prefill.hip); false when t is not one of them
static bool row_stage(const Task& t, hipStream_t s, hipError_t& e) {
  switch (t.kind) {
    case T_NORM_SPLIT: {
      const NormSplitArgs& a = t.norm;
      e = launch_norm_split(a.x, a.x_stride, a.M, a.K, a.gain, a.eps, a.xh, a.xl, s, a.out_f32, a.add);
      return true;
    }
    case T_GEMM: e = launch_gemm(t.gemm.wtype, t.gemm.g, t.gemm.part_cap, s); return true;
    case T_ROPE_ROWS: {
      const RopeRowsArgs& a = t.rope;
      e = launch_rope_rows(a.qkv, a.M, 0, a.n_heads_q, a.n_heads_kv, a.head_dim, a.rope, a.q_out, a.kc, a.vc,
                           a.cache_len, s, a.row_pos, a.row_seq, a.seq_stride, a.src, a.pages);
      return true;
    }
    case T_SILU_SPLIT:
      e = launch_silu_split(t.silu.a, t.silu.b, t.silu.M, t.silu.F, t.silu.hh, t.silu.hl, s, t.silu.pa, t.silu.pb);
      return true;
    case T_COMMIT_ROWS: e = launch_commit_rows(t.rows, s); return true;
    case T_INC_ROWS: e = launch_inc_rows(t.inc.v, t.inc.n, s, t.inc.active); return true;
    default: return false;
  }
}

hipError_t launch_task(int wtype, const Task& t, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e = hipSuccess;
  if (t.kind >= T_NORM_SPLIT) {
    // a many-row stage may take several launches: events around all of them
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
    if (!row_stage(t, s, e)) return hipErrorInvalidValue;
    if (e == hipSuccess && ev1) e = hipEventRecord(ev1, s);
    return e;
  }
  if (wtype == W_FP8) return single_launch<FP8>(t, s, false, ev0, ev1);
  if (wtype == W_INT8) return single_launch<INT8>(t, s, false, ev0, ev1);
  if (wtype == W_INT4) return single_launch<INT4>(t, s, false, ev0, ev1);
  return single_launch<BF16>(t, s, false, ev0, ev1);
}

hipError_t prepare_task(int wtype, const Task& t) {
  if (t.kind >= T_NORM_SPLIT) return hipSuccess;  // the many-row kernels need no set-up
  if (wtype == W_FP8) return single_launch<FP8>(t, nullptr, true);
  if (wtype == W_INT8) return single_launch<INT8>(t, nullptr, true);
  if (wtype == W_INT4) return single_launch<INT4>(t, nullptr, true);
  return single_launch<BF16>(t, nullptr, true);
}

size_t attn_partial_floats(int M, int n_kv, int nsplit_max, int group, int head_dim) {
  return (size_t)M * n_kv * nsplit_max * group * (head_dim + 2);
}

hipError_t launch_embed(const uint16_t* table, int rows, int K, const int* tok, float* x, int* pos_out,
                        int pos_value, int* anomalies, hipStream_t s) {
  const int grid = (K + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(k_embed, dim3(grid), dim3(kBlock), 0, s, table, rows, K, tok, x, pos_out, pos_value,
                     anomalies);
  return hipGetLastError();
}

hipError_t launch_set_forced(const int* forced, int n, int* dst, int* flag, hipStream_t s) {
  hipLaunchKernelGGL(k_set_forced, dim3(1), dim3(64), 0, s, forced, n, dst, flag);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* dst, int n, int value, hipStream_t s) {
  const int grid = n > 0 ? (n + kBlock - 1) / kBlock : 1;
  hipLaunchKernelGGL(k_fill_i32, dim3(grid < 1024 ? grid : 1024), dim3(kBlock), 0, s, dst, n, value);
  return hipGetLastError();
}

hipError_t launch_fill_u32(unsigned* dst, size_t n, hipStream_t s) {
  size_t grid = n > 0 ? (n + kBlock - 1) / kBlock : 1;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)grid), dim3(kBlock), 0, s, dst, n);
  return hipGetLastError();
}

hipError_t launch_copy_i32(const int* src, int* dst, int n, hipStream_t s) {
  const int grid = n > 0 ? (n + kBlock - 1) / kBlock : 1;
  hipLaunchKernelGGL(k_copy_i32, dim3(grid < 1024 ? grid : 1024), dim3(kBlock), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const uint16_t* w, int rows, int cols, uint8_t* q, float* scale, hipStream_t s) {
  hipLaunchKernelGGL(k_quantize_fp8, dim3(rows), dim3(kBlock), 0, s, w, rows, cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_quantize_int8(const uint16_t* w, int rows, int cols, int8_t* q, float* scale, hipStream_t s) {
  hipLaunchKernelGGL(k_quantize_int8, dim3(rows), dim3(kBlock), 0, s, w, rows, cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_quantize_int4(const uint16_t* w, int rows, int cols, uint8_t* q, float* scale, hipStream_t s) {
  if (cols % kGroup) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quantize_int4, dim3(rows), dim3(kBlock), 0, s, w, rows, cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_sample_rows(const float* logits, int rows, int V, const SampleArgs& sample, const int* history,
                              int n_hist, int* codes, hipStream_t s) {
  if (rows < 1 || V < 1 || V > kMaxSampleVocab || sample.top_k < 1 || sample.top_k > kMaxTopK || n_hist < 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sample_rows, dim3(rows), dim3(kBlock), sample_lds_bytes(V), s, logits, V, sample, history,
                     n_hist, codes);
  return hipGetLastError();
}

hipError_t launch_fp8_decode(const uint8_t* codes, int n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_fp8_decode, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, codes, n, out);
  return hipGetLastError();
}

}  // namespace dar
