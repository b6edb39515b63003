// RVQ codec decode on gfx950: codes -> 44.1 kHz audio (include/dar_codec.h).
//
// What is computed (tuna-fish README, intro and "Audio tokenizer speedtest";
// pyshine fish-speech tour, "Why You Need This"): the ten selected codebook
// vectors of a frame are summed into the latent frame, then a DAC-style
// convolutional decoder upsamples it 2048-fold: an input convolution, blocks of
// Snake + transposed convolution + residual units, and Snake + an output
// convolution + tanh.
//
// Every convolution with more than one output channel is one implicit GEMM on
// MFMA (v_mfma_f32_32x32x16_bf16): output rows (time) x output channels, the
// sum over input channels and taps. A transposed convolution with kernel
// 2 stride and padding stride / 2 splits into `stride` phases: output row
// t stride + r is a two-tap convolution of input rows {t, t - 1} or
// {t + 1, t} with the kernel taps that land on phase r, so each phase is the
// same GEMM with its own two taps (blockIdx.z). A workgroup stages, per chunk of
// 32 input channels, the input window its output rows need under every tap
// (rows t0 + min offset .. t0 + BM + max offset, Snake applied and rounded to
// bf16 on the way in, zeros outside [0, T)) and the chunk of every tap's
// weights into LDS, then each wave runs its 32-row x 32 NT-column MFMA tiles
// over the taps. Activations are time-major [T][C], so a window row is one
// contiguous run of channels. The epilogue adds the bias and either the
// residual (fp32 out) or applies the next Snake and rounds to bf16 (the input
// of the residual unit's 1-tap convolution).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/dar.h"
#include "../../include/dar_codec.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kChunk = 32;      // input channels per staged chunk (two MFMA k-steps)
constexpr int kMaxTaps = 7;
constexpr int kMaxOff = 32;     // largest |tap offset| of a convolution
constexpr int kMaxOffs = 32;    // taps x phases of one launch

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, nearest even (gfx950 converts in one instruction)
__device__ __forceinline__ uint32_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Snake(x) = x + sin(a x)^2 / a. The sine: a x reduced by whole turns with a
// two-part 2 pi (the high part 6.28125 is exact in 8 bits, so k times it is
// exact for |k| < 2^16), then the hardware sine of the remaining fraction of a
// turn. Measured on this part within 4e-7 of sin for |a x| <= 1000 (the
// library sinf: 7e-8), several times cheaper, and far below the bf16 step
// that every Snake output is rounded to next.
// ra = 1 / a, which the epilogues compute once per channel (a multiply per
// value instead of a division).
__device__ __forceinline__ float snake(float x, float a, float ra) {
  const float t = a * x;
  const float k = rintf(t * 0.15915494309189535f);
  float f = fmaf(-k, 6.28125f, t);
  f = fmaf(-k, 1.9353071795864769e-3f, f);
  const float s = __builtin_amdgcn_sinf(f * 0.15915494309189535f);  // sin(2 pi turns)
  return x + (s * s) * ra;
}
__device__ __forceinline__ float snake(float x, float a) { return snake(x, a, 1.0f / a); }

struct ConvArgs {
  const float* xf;          // fp32 input [T][Cin] (or null)
  const uint16_t* xb;       // bf16 input [T][Cin] (or null)
  const uint16_t* alpha_in; // Snake of the fp32 input on load (null: none)
  int T, Cin, Cout;
  const uint16_t* W;        // [nphase][ntap][Cout][Cin] bf16
  int nphase, ntap;
  int off[kMaxOffs];        // input row offset of tap j of phase z: off[z * ntap + j]
  const uint16_t* bias;     // bf16 [Cout]
  float* yf;                // fp32 output [T * nphase][Cout], row t * nphase + z
  const float* res;         // added to the fp32 output (may alias yf)
  int tanh_out;
  uint16_t* yb;             // bf16 output: Snake(acc + bias, alpha_out), rounded
  const uint16_t* alpha_out;
  uint16_t* ys;             // beside the fp32 output (bf16 input only): bf16(Snake(y, alpha_s)), the
  const uint16_t* alpha_s;  // next residual unit's operand
};

// LDS row r of 32 bf16 (64 B, four 16-byte units): unit u sits at slot
// u ^ ((r >> 2) & 3). The LDS serves 16-byte reads sixteen lanes at a time
// from 64 four-byte banks (256 B): sixteen consecutive rows read at one unit
// then hit sixteen distinct 16-byte bank groups (row r % 4 picks the 64-byte
// quarter, the swizzle the unit within it).
__device__ __forceinline__ int lds_at(int r, int u) { return r * 64 + ((u ^ ((r >> 2) & 3)) << 4); }

// The MFMA tiles of one workgroup: rows t0 .. t0 + 32 WM of phase z times
// columns n0 .. n0 + 32 NT WN, summed over every input channel and tap, then
// handed to epi(acc) (wave (wm, wn) holds rows t0 + 32 wm .., columns
// n0 + 32 (wn NT + nt) ..). Uses the LDS at smem (window rows, then every
// tap's weights); epi runs after a barrier, so it may reuse that LDS. (The
// accumulators stay local to this function: passed in by reference instead,
// they cost the compiler about fifty more registers and a wave per SIMD.)
template <int WM, int WN, int NT, bool XB16, typename Epi>
__device__ __forceinline__ void conv_accumulate(const ConvArgs& a, int z, int t0, int n0, char* smem, Epi&& epi) {
  f32x16 acc[NT];
  constexpr int BM = 32 * WM, BN = 32 * NT * WN;
  static_assert(WM * WN == 4, "four waves");
  // 16-byte units a thread stages per chunk: window rows x 4, tap rows x 4
  constexpr int XN = ((BM + 2 * kMaxOff) * 4 + kThreads - 1) / kThreads;
  constexpr int WNU = (kMaxTaps * BN * 4 + kThreads - 1) / kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int* off = a.off + z * a.ntap;
  int omin = off[0], omax = off[0];
  for (int j = 1; j < a.ntap; ++j) {
    omin = min(omin, off[j]);
    omax = max(omax, off[j]);
  }
  const int wrows = BM + omax - omin;
  const int xunits = wrows * 4, wunits = a.ntap * BN * 4;
  char* xs = smem;
  char* ws = smem + wrows * 64;
  const uint16_t* Wz = a.W + (size_t)z * a.ntap * a.Cout * a.Cin;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[nt][v] = 0.f;
  const int half = lane >> 5, l32 = lane & 31;
  // A chunk of 32 input channels is staged in two steps, so that its global
  // loads are all in flight together and overlap the previous chunk's MFMAs:
  // load() issues every load of the chunk into registers, store() converts
  // (Snake, bf16) and writes them to LDS once they have landed.
  // window unit i: row w = i / 4 (input row t0 + omin + w), channels c0 + 8 (i % 4) ..
  f32x4 xv[XN][2];
  u32x4 xa[XN];
  u32x4 wv[WNU];
  auto load = [&](int c0) {
#pragma unroll
    for (int k = 0; k < XN; ++k) {
      const int i = tid + k * kThreads;
      const int w = i >> 2, u = i & 3;
      const int row = t0 + omin + w;
      const bool in = i < xunits && row >= 0 && row < a.T;
      if constexpr (XB16) {
        xa[k] = in ? *reinterpret_cast<const u32x4*>(a.xb + (size_t)row * a.Cin + c0 + 8 * u) : u32x4{0u, 0u, 0u, 0u};
      } else {
        const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
        const f32x4* src = reinterpret_cast<const f32x4*>(a.xf + (size_t)(in ? row : 0) * a.Cin + c0 + 8 * u);
        xv[k][0] = in ? src[0] : zf;
        xv[k][1] = in ? src[1] : zf;
        if (a.alpha_in && i < xunits) xa[k] = *reinterpret_cast<const u32x4*>(a.alpha_in + c0 + 8 * u);
      }
    }
    // tap unit i: LDS row r = i / 4 = j BN + n holds output channel n0 + n of tap j
#pragma unroll
    for (int k = 0; k < WNU; ++k) {
      const int i = tid + k * kThreads;
      const int r = i >> 2, u = i & 3;
      const int j = r / BN, n = n0 + r % BN;
      wv[k] = (i < wunits && n < a.Cout)
                  ? *reinterpret_cast<const u32x4*>(Wz + ((size_t)j * a.Cout + n) * a.Cin + c0 + 8 * u)
                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int k = 0; k < XN; ++k) {
      const int i = tid + k * kThreads;
      if (i >= xunits) continue;
      const int w = i >> 2, u = i & 3;
      u32x4 v;
      if constexpr (XB16) {
        v = xa[k];
      } else {
        const int row = t0 + omin + w;
        float f[8] = {xv[k][0].x, xv[k][0].y, xv[k][0].z, xv[k][0].w, xv[k][1].x, xv[k][1].y, xv[k][1].z, xv[k][1].w};
        if (a.alpha_in && row >= 0 && row < a.T) {
          const uint32_t aw[4] = {xa[k].x, xa[k].y, xa[k].z, xa[k].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = snake(f[e], bf2f((uint16_t)(aw[e >> 1] >> (16 * (e & 1)))));
        }
        v.x = f2bf(f[0]) | (f2bf(f[1]) << 16);
        v.y = f2bf(f[2]) | (f2bf(f[3]) << 16);
        v.z = f2bf(f[4]) | (f2bf(f[5]) << 16);
        v.w = f2bf(f[6]) | (f2bf(f[7]) << 16);
      }
      *reinterpret_cast<u32x4*>(xs + lds_at(w, u)) = v;
    }
#pragma unroll
    for (int k = 0; k < WNU; ++k) {
      const int i = tid + k * kThreads;
      if (i < wunits) *reinterpret_cast<u32x4*>(ws + lds_at(i >> 2, i & 3)) = wv[k];
    }
  };
  load(0);
  for (int c0 = 0; c0 < a.Cin; c0 += kChunk) {
    store();
    __syncthreads();
    if (c0 + kChunk < a.Cin) load(c0 + kChunk);
    for (int j = 0; j < a.ntap; ++j) {
      const int xr = wm * 32 + l32 + off[j] - omin;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int u = 2 * ks + half;
        const bf16x8 A = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + lds_at(xr, u)));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int wr = j * BN + (wn * NT + nt) * 32 + l32;
          const bf16x8 B = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ws + lds_at(wr, u)));
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  epi(acc);
}

template <int WM, int WN, int NT, bool XB16, bool YB16>
__global__ __launch_bounds__(kThreads) void k_conv(ConvArgs a) {
  constexpr int BM = 32 * WM, BN = 32 * NT * WN;
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int z = blockIdx.z;
  const int t0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int half = lane >> 5, l32 = lane & 31;
  conv_accumulate<WM, WN, NT, XB16>(a, z, t0, n0, smem, [&](f32x16 (&acc)[NT]) {
    if constexpr (XB16) {
      if (t0 + BM <= a.T && n0 + BN <= a.Cout) {
        // A whole tile: the sums go through LDS (the staging area, free
        // again; the launch sizes it for this) so that the residual is read
        // and the outputs written 16 or 8 bytes per lane along the rows: the
        // fp32 rows and the next operand (a transposed convolution, an
        // unfused unit's 1-tap convolution), or one bf16 operand (the input
        // convolution, a 7-tap convolution's hidden rows, a block's last
        // 1-tap convolution). The values are the per-element path's.
        constexpr int YP = BN + 8;  // floats per staged row: the two half-waves' rows 32 banks apart
        float* yl = reinterpret_cast<float*>(smem);
        float* al = yl + BM * YP;   // [BN] alpha, [BN] 1/alpha of the tile's channels
        const uint16_t* alpha = YB16 ? a.alpha_out : a.ys ? a.alpha_s : nullptr;
        const int tid = threadIdx.x;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = (wn * NT + nt) * 32 + l32;
          const float b = bf2f(a.bias[n0 + col]);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            yl[(wm * 32 + (v & 3) + 4 * half + 8 * (v >> 2)) * YP + col] = acc[nt][v] + b;
        }
        if (alpha) {
          for (int c = tid; c < BN; c += kThreads) {
            const float ao = bf2f(alpha[n0 + c]);
            al[c] = ao;
            al[BN + c] = 1.0f / ao;
          }
        }
        __syncthreads();
        constexpr int Q = BN / 4;  // 16-byte units of a staged row
        for (int i = tid; i < BM * Q; i += kThreads) {
          const int row = i / Q, q = i % Q;
          const size_t at = ((size_t)(t0 + row) * a.nphase + z) * a.Cout + n0 + 4 * q;
          f32x4 val = *reinterpret_cast<const f32x4*>(yl + row * YP + 4 * q);
          if (a.res) {
            const f32x4 rv = *reinterpret_cast<const f32x4*>(a.res + at);
            val = f32x4{val.x + rv.x, val.y + rv.y, val.z + rv.z, val.w + rv.w};
          }
          if constexpr (!YB16) *reinterpret_cast<f32x4*>(a.yf + at) = val;
          if (alpha) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(al + 4 * q);
            const f32x4 rv = *reinterpret_cast<const f32x4*>(al + BN + 4 * q);
            uint2 o;
            o.x = f2bf(snake(val.x, av.x, rv.x)) | (f2bf(snake(val.y, av.y, rv.y)) << 16);
            o.y = f2bf(snake(val.z, av.z, rv.z)) | (f2bf(snake(val.w, av.w, rv.w)) << 16);
            *reinterpret_cast<uint2*>((YB16 ? a.yb : a.ys) + at) = o;
          }
        }
        return;
      }
    }
    // lane holds output channel n of its tiles; accumulator v holds output row
    // t0 + 32 wm + (v % 4) + 4 half + 8 (v / 4)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + (wn * NT + nt) * 32 + l32;
      if (n >= a.Cout) continue;
      const float b = bf2f(a.bias[n]);
      const float ao = YB16 ? bf2f(a.alpha_out[n]) : (XB16 && a.ys ? bf2f(a.alpha_s[n]) : 1.f);
      const float rao = 1.0f / ao;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + wm * 32 + (v & 3) + 4 * half + 8 * (v >> 2);
        if (t >= a.T) continue;
        const size_t at = ((size_t)t * a.nphase + z) * a.Cout + n;
        float val = acc[nt][v] + b;
        if constexpr (YB16) {
          if constexpr (XB16) {  // a block's last 1-tap conv: residual, then the next layer's Snake
            if (a.res) val += a.res[at];
          }
          a.yb[at] = (uint16_t)f2bf(snake(val, ao, rao));
        } else {
          if (a.res) val += a.res[at];
          if constexpr (XB16) {  // (tanh is the fp32-input path's only: it keeps this epilogue's code small)
            a.yf[at] = val;
            if (a.ys) a.ys[at] = (uint16_t)f2bf(snake(val, ao, rao));
          } else {
            if (a.tanh_out) val = tanhf(val);
            a.yf[at] = val;
          }
        }
      }
    }
  });
}

// The output convolution (one channel): y[t] = tanh(b + sum_j sum_c w[c][j]
// u[t + j - h][c]), u the operand rows (Snake, rounded to bf16; zeros outside
// [0, T)), h = (K - 1) / 2. The double sum splits into per-row tap projections
// p_j[r] = sum_c w[c][j] u[r][c] -- a [rows x C] by [C x K] product, run on
// MFMA with the taps as the tile's columns -- and then y[t] needs only
// p_j[t + j - h] over the K taps. A workgroup projects kOutP consecutive rows
// (each wave two 32-row tiles; every operand load of a pass over the channels
// is issued at once, straight into the A registers, so each row is read from
// memory once and no staging sits between the loads and the MFMAs), parks the
// projections in LDS and sums them into kOutP - (K - 1) output samples.
constexpr int kOutP = 256;     // projected rows per workgroup (4 waves x 2 tiles of 32)
constexpr int kOutPitch = 9;   // LDS floats per projected row: odd, so a wave's reads of one tap hit 64 banks
constexpr int kOutSteps = 6;   // MFMA k-steps (16 channels each) per pass over the channels
static_assert(kMaxTaps < kOutPitch, "every tap's projection needs its own LDS slot");

// XB16: the operand rows are given (bf16, Snake applied); otherwise fp32 rows
// take Snake(alpha) and the bf16 rounding on load
template <bool XB16>
__global__ __launch_bounds__(kThreads) void k_conv_out(const float* x, const uint16_t* xb16, const uint16_t* alpha,
                                                     int T, int C, const uint16_t* w, const uint16_t* b, int K,
                                                     float* y) {
  __shared__ float ps[kOutP * kOutPitch];  // ps[r * kOutPitch + j] = p_j[p0 + r]
  __shared__ bf16x8 bs[kOutSteps * 64];    // the B operand of each k-step, per lane
  const int halfk = (K - 1) / 2, TM = kOutP - (K - 1);
  const int t0 = blockIdx.x * TM, p0 = t0 - halfk;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, hk = lane >> 5;  // this lane's MFMA row / column (tap) and k half
  const bool whole = p0 >= 0 && p0 + kOutP <= T;
  f32x16 acc[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[m][v] = 0.f;
  const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  for (int c0 = 0; c0 < C; c0 += 16 * kOutSteps) {
    const int S = min(kOutSteps, (C - c0) / 16);
    // A: row (tile base + n), channels c0 + 16 s + 8 hk .. + 8
    bf16x8 A[2][kOutSteps];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int row = p0 + 32 * (2 * wv + m) + n;
      const bool in = whole || (row >= 0 && row < T);
#pragma unroll
      for (int st = 0; st < kOutSteps; ++st) {
        A[m][st] = zero;
        if (st >= S || !in) continue;
        const int c = c0 + 16 * st + 8 * hk;
        if constexpr (XB16) {
          A[m][st] = *reinterpret_cast<const bf16x8*>(xb16 + (size_t)row * C + c);
        } else {
          const f32x4 lo = *reinterpret_cast<const f32x4*>(x + (size_t)row * C + c);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(x + (size_t)row * C + c + 4);
          const float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) A[m][st][e] = (__bf16)snake(f[e], bf2f(alpha[c + e]));
        }
      }
    }
    // B: column j of k-step s holds w[c][j] for the step's 16 channels (zero past the taps)
    for (int i = tid; i < S * 64; i += kThreads) {
      const int st = i >> 6, nn = i & 31, hh = (i >> 5) & 1;
      bf16x8 v = zero;
      if (nn < K) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = __builtin_bit_cast(__bf16, w[(size_t)(c0 + 16 * st + 8 * hh + e) * K + nn]);
      }
      bs[i] = v;
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < kOutSteps; ++st) {
      if (st >= S) break;
      const bf16x8 B = bs[st * 64 + lane];
#pragma unroll
      for (int m = 0; m < 2; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m][st], B, acc[m], 0, 0, 0);
    }
    __syncthreads();  // bs is rewritten by the next pass
  }
  if (n < K) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * (2 * wv + m) + (v & 3) + 4 * hk + 8 * (v >> 2);
        ps[r * kOutPitch + n] = acc[m][v];
      }
  }
  __syncthreads();
  const int t = t0 + tid;
  if (tid < TM && t < T) {
    float sum = 0.f;
    for (int j = 0; j < K; ++j) sum += ps[(tid + j) * kOutPitch + j];
    y[t] = tanhf(sum + bf2f(b[0]));
  }
}

// z[t] = sum_k table_k[code[t][k]] over the codebooks in order, fp32 sums
// rounded to bf16 (the input convolution's operand). A thread makes eight
// channels of one frame.
struct RvqArgs {
  const uint16_t* tab[32];
  const int* codes;  // [T][nq]
  int T, nq, V, D;
  uint16_t* z;       // [T][D]
  int* anomalies;
};

__global__ __launch_bounds__(kThreads) void k_rvq(RvqArgs a) {
  const int per = a.D / 8;
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)a.T * per) return;
  const int t = (int)(idx / per), u = (int)(idx % per);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (k >= a.nq) break;
    int c = a.codes[(size_t)t * a.nq + k];
    if (c < 0 || c >= a.V) {
      if (u == 0) atomicAdd(a.anomalies, 1);
      c = c < 0 ? 0 : a.V - 1;
    }
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.tab[k] + (size_t)c * a.D + 8 * u);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += bf2f((uint16_t)(wv[e >> 1] >> (16 * (e & 1))));
  }
  u32x4 o;
  o.x = f2bf(s[0]) | (f2bf(s[1]) << 16);
  o.y = f2bf(s[2]) | (f2bf(s[3]) << 16);
  o.z = f2bf(s[4]) | (f2bf(s[5]) << 16);
  o.w = f2bf(s[6]) | (f2bf(s[7]) << 16);
  *reinterpret_cast<u32x4*>(a.z + (size_t)t * a.D + 8 * u) = o;
}

// [Cout][Cin][K] -> [K][Cout][Cin]
__global__ void k_relayout_conv(const uint16_t* src, int Cout, int Cin, int K, uint16_t* dst) {
  const long long n = (long long)Cout * Cin * K;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(i % Cin);
    const long long r = i / Cin;
    const int o = (int)(r % Cout), j = (int)(r / Cout);
    dst[i] = src[((size_t)o * Cin + c) * K + j];
  }
}

// transposed convolution [Cin][Cout][2s] -> [phase r][tap j][Cout][Cin], tap j
// of phase r being kernel index kidx[2 r + j]
struct PhaseTaps {
  int k[kMaxOffs];
};
__global__ void k_relayout_convT(const uint16_t* src, int Cin, int Cout, int s, PhaseTaps taps, uint16_t* dst) {
  const long long n = (long long)2 * s * Cout * Cin;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(i % Cin);
    const long long r = i / Cin;
    const int o = (int)(r % Cout), pj = (int)(r / Cout);
    dst[i] = src[((size_t)c * Cout + o) * (2 * s) + taps.k[pj]];
  }
}

// ---- host side -----------------------------------------------------------

struct TileCfg {
  int wm, wn, nt;
  int bm() const { return 32 * wm; }
  int bn() const { return 32 * nt * wn; }
};
// largest tiles first (a 128 x 128 tile needs more registers than a wave has
// room for with the staged chunk in flight)
constexpr TileCfg kCfgs[] = {{4, 1, 3}, {2, 2, 2}, {2, 2, 1}, {1, 4, 1}, {4, 1, 1}};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

long long cfg_grid(const TileCfg& c, int rows, int Cout, int nphase) {
  return (long long)((rows + c.bm() - 1) / c.bm()) * ((Cout + c.bn() - 1) / c.bn()) * nphase;
}

// The tile shape of a convolution: among the shapes whose column width
// divides Cout (else all), the largest that still gives every CU two
// workgroups, else the one with the most workgroups.
int pick_cfg(int rows, int Cout, int nphase) {
  bool any_exact = false;
  for (int i = 0; i < kNumCfgs; ++i) any_exact |= Cout % kCfgs[i].bn() == 0;
  int best = -1;
  long long best_grid = -1;
  for (int i = 0; i < kNumCfgs; ++i) {
    if (any_exact && Cout % kCfgs[i].bn() != 0) continue;
    const long long g = cfg_grid(kCfgs[i], rows, Cout, nphase);
    if (g >= 512) return i;
    if (g > best_grid) {
      best_grid = g;
      best = i;
    }
  }
  return best;
}

size_t conv_lds(const TileCfg& c, int span, int ntap) {
  return (size_t)(c.bm() + span) * 64 + (size_t)ntap * c.bn() * 64;
}

template <typename KernelT>
hipError_t allow_lds(KernelT kern, size_t lds, std::atomic<bool>& done) {
  if (lds <= 65536 || done.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.store(true, std::memory_order_release);
  return e;
}

// One residual unit in one launch, for widths a workgroup's tile spans
// (C = 32 NT WN): h = Snake(conv_K,dil(Snake(x, alpha1)) + b1, alpha2) is
// rounded to bf16 and kept in LDS, then y = x + conv_1(h) + b2. The 1-tap
// convolution needs only the workgroup's own rows of h, so h never goes to
// HBM. y and x are different buffers: the neighbouring workgroups still read
// the rows of x around their tiles.
struct ResArgs {
  ConvArgs c1;              // the 7-tap convolution (fp32 x with Snake alpha1, [K][C][C] weights, b1)
  const uint16_t* alpha2;   // Snake of the hidden rows
  const uint16_t* W2;       // [C][C] bf16 (the 1-tap convolution)
  const uint16_t* b2;
  float* y;                 // [T][C] = x + conv_1(h) + b2
  uint16_t* ys;             // with y (optional): bf16(Snake(y, alpha_s)), the next unit's operand
  const uint16_t* alpha_s;
  uint16_t* yb;             // or, in y's place, bf16(Snake(y, alpha_out)): the next layer's operand
  const uint16_t* alpha_out;
  int h_at;                 // LDS byte offset of h (past the 7-tap convolution's staging)
};

// XB16: the 7-tap convolution stages c1.xb (its operand, bf16(Snake(x,
// alpha1)), written by the layer before) instead of Snake'ing c1.xf itself;
// the residual add reads c1.xf either way. OUT: 0 writes y, 1 y and ys, 2 yb
// (one output form per instantiation keeps the epilogue's Snake code small
// enough to stay inline).
template <int WM, int WN, int NT, bool XB16, int OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_resunit(ResArgs r) {
  constexpr int BM = 32 * WM, C = 32 * NT * WN;
  constexpr int CH = C / 32;                       // 32-channel chunks of h
  constexpr int WU = (C * 4 + kThreads - 1) / kThreads;  // 16-byte units of a W2 chunk per thread
  extern __shared__ __align__(16) char smem[];
  const ConvArgs& a = r.c1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int t0 = blockIdx.x * BM;
  const int half = lane >> 5, l32 = lane & 31;
  // h: chunk c's rows at hs + c BM 64, laid out as a staged window (lds_at)
  char* hs = smem + r.h_at;
  // the 1-tap convolution's weights, every chunk at once: chunk c's rows at
  // ws + c C 64 (the 7-tap staging area, free once its loop has ended; the
  // launch sizes it for at least a whole tile's fp32 sums, BM (C + 8) 4 bytes)
  char* ws = smem;
  static_assert(CH * C * 64 <= BM * (C + 8) * 4, "the 1-tap weights fit in the staging area");
  conv_accumulate<WM, WN, NT, XB16>(a, 0, t0, 0, smem, [&](f32x16 (&acc)[NT]) {
    // issued before the hidden rows' Snake, so that their latency hides behind it
    u32x4 wv[CH][WU];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int k = 0; k < WU; ++k) {
        const int i = tid + k * kThreads;
        wv[c][k] = i < C * 4 ? *reinterpret_cast<const u32x4*>(r.W2 + (size_t)(i >> 2) * C + 32 * c + 8 * (i & 3))
                             : u32x4{0u, 0u, 0u, 0u};
      }
    const bool whole = t0 + BM <= a.T;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = (wn * NT + nt) * 32 + l32;  // chunk wn NT + nt, channel l32 of it
      const float b = bf2f(a.bias[n]), ao = bf2f(r.alpha2[n]), rao = 1.0f / ao;
      char* hc = hs + (size_t)(wn * NT + nt) * BM * 64;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 32 + (v & 3) + 4 * half + 8 * (v >> 2);
        // rows past the end hold zero (a select, not a branch)
        const float h = snake(acc[nt][v] + b, ao, rao);
        const uint16_t hv = (whole || t0 + row < a.T) ? (uint16_t)f2bf(h) : (uint16_t)0;
        *reinterpret_cast<uint16_t*>(hc + lds_at(row, l32 >> 3) + 2 * (l32 & 7)) = hv;
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int k = 0; k < WU; ++k) {
        const int i = tid + k * kThreads;
        if (i < C * 4) *reinterpret_cast<u32x4*>(ws + (size_t)c * C * 64 + lds_at(i >> 2, i & 3)) = wv[c][k];
      }
  });
  __syncthreads();  // h and the 1-tap weights are complete
  // the 1-tap convolution over h, chunk by chunk
  f32x16 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[nt][v] = 0.f;
  for (int c = 0; c < CH; ++c) {
    const char* wc = ws + (size_t)c * C * 64;
    const char* hc = hs + (size_t)c * BM * 64;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int u = 2 * ks + half;
      const bf16x8 A = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(hc + lds_at(wm * 32 + l32, u)));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 B =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wc + lds_at((wn * NT + nt) * 32 + l32, u)));
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[nt], 0, 0, 0);
      }
    }
  }
  if (OUT != 2 && t0 + BM <= a.T) {
    // A whole tile's sums go through LDS (the 7-tap staging area, free again)
    // so that the residual rows are read and the outputs written 16 bytes per
    // lane along the rows instead of one value per lane and instruction; the
    // channels' 1/alpha sit in the hidden rows' area, free after the 1-tap
    // convolution. The values are the per-element path's.
    constexpr int YP = C + 8;  // floats per staged row: the two half-waves' rows 32 banks apart
    float* yl = reinterpret_cast<float*>(smem);
    float* al = reinterpret_cast<float*>(hs);  // [C] alpha, [C] 1/alpha
    __syncthreads();  // every wave is done with the 1-tap convolution's LDS
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = (wn * NT + nt) * 32 + l32;
      const float b = bf2f(r.b2[col]);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        yl[(wm * 32 + (v & 3) + 4 * half + 8 * (v >> 2)) * YP + col] = acc[nt][v] + b;
    }
    if constexpr (OUT != 0) {
      for (int n = tid; n < C; n += kThreads) {
        const float ao = bf2f(OUT == 2 ? r.alpha_out[n] : r.alpha_s[n]);
        al[n] = ao;
        al[C + n] = 1.0f / ao;
      }
    }
    __syncthreads();
    constexpr int Q = C / 4;  // 16-byte units of a row
    for (int i = tid; i < BM * Q; i += kThreads) {
      const int row = i / Q, q = i % Q;
      const size_t at = (size_t)(t0 + row) * C + 4 * q;
      const f32x4 xv = *reinterpret_cast<const f32x4*>(a.xf + at);
      const f32x4 sv = *reinterpret_cast<const f32x4*>(yl + row * YP + 4 * q);
      const f32x4 val = {sv.x + xv.x, sv.y + xv.y, sv.z + xv.z, sv.w + xv.w};  // (sum + b2) + x
      if constexpr (OUT != 2) *reinterpret_cast<f32x4*>(r.y + at) = val;
      if constexpr (OUT != 0) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(al + 4 * q);
        const f32x4 rv = *reinterpret_cast<const f32x4*>(al + C + 4 * q);
        uint2 o;
        o.x = f2bf(snake(val.x, av.x, rv.x)) | (f2bf(snake(val.y, av.y, rv.y)) << 16);
        o.y = f2bf(snake(val.z, av.z, rv.z)) | (f2bf(snake(val.w, av.w, rv.w)) << 16);
        *reinterpret_cast<uint2*>((OUT == 2 ? r.yb : r.ys) + at) = o;
      }
    }
    return;
  }
  // one value per lane (a block's last unit, whose bf16 output is a quarter
  // of the rows' bytes, measured faster this way; and the partial last
  // tile, whose rows past the end are skipped)
  auto epilogue = [&](auto whole) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = (wn * NT + nt) * 32 + l32;
      const float b = bf2f(r.b2[n]);
      const float ao = OUT == 2 ? bf2f(r.alpha_out[n]) : (OUT == 1 ? bf2f(r.alpha_s[n]) : 1.f), rao = 1.0f / ao;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + wm * 32 + (v & 3) + 4 * half + 8 * (v >> 2);
        if (!decltype(whole)::value && t >= a.T) continue;
        const size_t at = (size_t)t * C + n;
        const float val = (acc[nt][v] + b) + a.xf[at];  // the two-launch path's order of the sums
        if constexpr (OUT == 2) {
          r.yb[at] = (uint16_t)f2bf(snake(val, ao, rao));
        } else {
          r.y[at] = val;
          if constexpr (OUT == 1) r.ys[at] = (uint16_t)f2bf(snake(val, ao, rao));
        }
      }
    }
  };
  if (t0 + BM <= a.T)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
}

template <int WM, int WN, int NT, bool XB16, bool YB16>
hipError_t go_conv(const ConvArgs& a, dim3 grid, size_t lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  static std::atomic<bool> big{false};  // one flag per kernel instantiation
  hipError_t e = allow_lds(k_conv<WM, WN, NT, XB16, YB16>, lds, big);
  if (e != hipSuccess) return e;
  if (e0 || e1)
    hipExtLaunchKernelGGL((k_conv<WM, WN, NT, XB16, YB16>), grid, dim3(kThreads), lds, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((k_conv<WM, WN, NT, XB16, YB16>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <bool XB16, bool YB16>
hipError_t go_conv_cfg(int ci, const ConvArgs& a, dim3 grid, size_t lds, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1) {
  switch (ci) {
    case 0: return go_conv<4, 1, 3, XB16, YB16>(a, grid, lds, s, e0, e1);
    case 1: return go_conv<2, 2, 2, XB16, YB16>(a, grid, lds, s, e0, e1);
    case 2: return go_conv<2, 2, 1, XB16, YB16>(a, grid, lds, s, e0, e1);
    case 3: return go_conv<1, 4, 1, XB16, YB16>(a, grid, lds, s, e0, e1);
    default: return go_conv<4, 1, 1, XB16, YB16>(a, grid, lds, s, e0, e1);
  }
}

// Launch one convolution (rows = input rows per phase).
hipError_t launch_conv(const ConvArgs& a, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  const int ci = pick_cfg(a.T, a.Cout, a.nphase);
  const TileCfg& c = kCfgs[ci];
  int span = 0;
  for (int z = 0; z < a.nphase; ++z) {
    int lo = a.off[z * a.ntap], hi = lo;
    for (int j = 1; j < a.ntap; ++j) {
      lo = std::min(lo, a.off[z * a.ntap + j]);
      hi = std::max(hi, a.off[z * a.ntap + j]);
    }
    span = std::max(span, hi - lo);
  }
  size_t lds = conv_lds(c, span, a.ntap);
  if (a.xb)  // whole tiles stage their fp32 sums and the channels' alphas at the end
    lds = std::max(lds, (size_t)c.bm() * (c.bn() + 8) * 4 + (size_t)c.bn() * 8);
  const dim3 grid((a.T + c.bm() - 1) / c.bm(), (a.Cout + c.bn() - 1) / c.bn(), a.nphase);
  const bool xb = a.xb != nullptr, yb = a.yb != nullptr;
  if (xb && !yb) return go_conv_cfg<true, false>(ci, a, grid, lds, s, e0, e1);
  if (!xb && yb) return go_conv_cfg<false, true>(ci, a, grid, lds, s, e0, e1);
  if (!xb && !yb) return go_conv_cfg<false, false>(ci, a, grid, lds, s, e0, e1);
  return go_conv_cfg<true, true>(ci, a, grid, lds, s, e0, e1);  // a block's last 1-tap conv to the next operand
}

// Tile of the one-launch residual unit at width C: the workgroup spans all C
// output channels (index into kCfgs, or -1: C is run as two launches).
int resunit_cfg(int C) {
  switch (C) {
    case 32: return 4;   // 128 x 32
    case 64: return 2;   // 64 x 64
    case 96: return 0;   // 128 x 96
    case 128: return 1;  // 64 x 128
    default: return -1;  // (a 64 x 192 tile runs at one wave per SIMD: slower than two launches)
  }
}

template <int WM, int WN, int NT, bool XB16, int OUT>
hipError_t go_resunit(const ResArgs& r, dim3 grid, size_t lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  static std::atomic<bool> big{false};
  hipError_t e = allow_lds(k_resunit<WM, WN, NT, XB16, OUT>, lds, big);
  if (e != hipSuccess) return e;
  if (e0 || e1)
    hipExtLaunchKernelGGL((k_resunit<WM, WN, NT, XB16, OUT>), grid, dim3(kThreads), lds, s, e0, e1, 0, r);
  else
    hipLaunchKernelGGL((k_resunit<WM, WN, NT, XB16, OUT>), grid, dim3(kThreads), lds, s, r);
  return hipGetLastError();
}

template <bool XB16, int OUT>
hipError_t go_resunit_cfg(int ci, const ResArgs& r, dim3 grid, size_t lds, hipStream_t s, hipEvent_t e0,
                          hipEvent_t e1) {
  switch (ci) {
    case 0: return go_resunit<4, 1, 3, XB16, OUT>(r, grid, lds, s, e0, e1);
    case 1: return go_resunit<2, 2, 2, XB16, OUT>(r, grid, lds, s, e0, e1);
    case 2: return go_resunit<2, 2, 1, XB16, OUT>(r, grid, lds, s, e0, e1);
    default: return go_resunit<4, 1, 1, XB16, OUT>(r, grid, lds, s, e0, e1);
  }
}

// One residual unit in one launch (r.c1 describes the 7-tap convolution:
// fp32 input xf, which the residual add reads, staged either from its
// operand xb or from xf with Snake(alpha1); C in and out, one phase; the
// output y (fp32, optionally with ys) or yb in a buffer other than xf).
hipError_t launch_resunit(ResArgs r, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  const ConvArgs& a = r.c1;
  const int ci = resunit_cfg(a.Cout);
  if (ci < 0 || a.Cin != a.Cout || a.nphase != 1 || !a.xf || (!a.xb && !a.alpha_in) || !r.y == !r.yb ||
      (r.yb && !r.alpha_out) || (r.ys && (!r.y || !r.alpha_s)) ||
      static_cast<const void*>(r.y ? static_cast<const void*>(r.y) : r.yb) == a.xf)
    return hipErrorInvalidValue;
  const TileCfg& c = kCfgs[ci];
  const int span = a.off[a.ntap - 1] - a.off[0];
  // the 7-tap staging area also holds a whole tile's fp32 sums at the end
  const size_t conv = std::max(conv_lds(c, span, a.ntap), (size_t)c.bm() * (a.Cout + 8) * 4);
  r.h_at = (int)conv;
  const size_t lds = conv + (size_t)c.bm() * a.Cout * 2;
  const dim3 grid((a.T + c.bm() - 1) / c.bm());
  // the decode's forms (operand staged, output with its operand or as the
  // next layer's operand) and the diagnostic's (fp32 staged, fp32 out)
  if (a.xb && r.ys) return go_resunit_cfg<true, 1>(ci, r, grid, lds, s, e0, e1);
  if (a.xb && r.yb) return go_resunit_cfg<true, 2>(ci, r, grid, lds, s, e0, e1);
  if (!a.xb && !r.ys && !r.yb) return go_resunit_cfg<false, 0>(ci, r, grid, lds, s, e0, e1);
  return hipErrorInvalidValue;
}

// x: fp32 rows with Snake(alpha) applied on load, or xb16: bf16 rows already
// Snake'd and rounded (alpha unused)
hipError_t launch_conv_out(const float* x, const uint16_t* xb16, const uint16_t* alpha, int T, int C,
                           const uint16_t* w, const uint16_t* b, int K, float* y, hipStream_t s,
                           hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  const dim3 grid((T + kOutP - K) / (kOutP - (K - 1)));
  auto go = [&](auto kern) {
    if (e0 || e1)
      hipExtLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, e0, e1, 0, x, xb16, alpha, T, C, w, b, K, y);
    else
      hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, x, xb16, alpha, T, C, w, b, K, y);
  };
  if (xb16)
    go(k_conv_out<true>);
  else
    go(k_conv_out<false>);
  return hipGetLastError();
}

// kernel taps of a transposed convolution (kernel 2s, padding s/2) that land on
// output phase r: input rows t and t - 1 (first half of the phases) or t + 1
// and t (second half)
void convT_taps(int s, int* kidx, int* offs) {
  for (int r = 0; r < s; ++r) {
    const int q = r + s / 2;
    if (q < s) {
      kidx[2 * r] = q;
      offs[2 * r] = 0;
      kidx[2 * r + 1] = q + s;
      offs[2 * r + 1] = -1;
    } else {
      kidx[2 * r] = q - s;
      offs[2 * r] = 1;
      kidx[2 * r + 1] = q;
      offs[2 * r + 1] = 0;
    }
  }
}

void conv_taps(int K, int dil, int* offs) {
  for (int j = 0; j < K; ++j) offs[j] = dil * (j - (K - 1) / 2);
}

hipError_t relayout_conv(const uint16_t* src, int Cout, int Cin, int K, uint16_t* dst, hipStream_t s) {
  hipLaunchKernelGGL(k_relayout_conv, dim3(1024), dim3(kThreads), 0, s, src, Cout, Cin, K, dst);
  return hipGetLastError();
}

hipError_t relayout_convT(const uint16_t* src, int Cin, int Cout, int st, uint16_t* dst, hipStream_t s) {
  PhaseTaps t{};
  int offs[kMaxOffs];
  convT_taps(st, t.k, offs);
  hipLaunchKernelGGL(k_relayout_convT, dim3(1024), dim3(kThreads), 0, s, src, Cin, Cout, st, t, dst);
  return hipGetLastError();
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

thread_local std::string g_codec_error;

struct CodecLayout {
  size_t in_w;
  size_t up_w[DAR_CODEC_MAX_BLOCKS];
  size_t w1[DAR_CODEC_MAX_BLOCKS][DAR_CODEC_MAX_UNITS], w2[DAR_CODEC_MAX_BLOCKS][DAR_CODEC_MAX_UNITS];
  size_t z, xa, xb, h, sa, sb, anom, total;
  size_t act_elems;  // largest rows x channels of any activation
};

int width(const dar_codec_config* c, int i) { return c->channels >> i; }

CodecLayout codec_layout(const dar_codec_config* c) {
  CodecLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const int K = c->kernel_size;
  L.in_w = take((size_t)2 * K * c->channels * c->latent_dim);
  size_t rows = (size_t)c->max_frames;
  L.act_elems = rows * c->channels;
  for (int i = 0; i < c->n_blocks; ++i) {
    const int cin = width(c, i), cout = width(c, i + 1), s = c->rates[i];
    L.up_w[i] = take((size_t)2 * 2 * s * cout * cin);
    for (int u = 0; u < c->n_units; ++u) {
      L.w1[i][u] = take((size_t)2 * K * cout * cout);
      L.w2[i][u] = take((size_t)2 * cout * cout);
    }
    rows *= s;
    L.act_elems = std::max(L.act_elems, rows * cout);
  }
  L.z = take((size_t)2 * c->max_frames * c->latent_dim);
  L.xa = take(4 * L.act_elems);
  L.xb = take(4 * L.act_elems);
  L.h = take(2 * L.act_elems);
  L.sa = take(2 * L.act_elems);  // residual units' operands, bf16(Snake(x, alpha1)), alternating
  L.sb = take(2 * L.act_elems);
  L.anom = take(sizeof(int) * 4);
  L.total = off;
  return L;
}

int validate_codec(const dar_codec_config* c, std::string& why) {
  if (!c) {
    why = "config is NULL";
    return DAR_E_INVAL;
  }
  auto bad = [&](const char* m) {
    why = m;
    return DAR_E_INVAL;
  };
  if (c->n_codebooks < 1 || c->n_codebooks > 32) return bad("n_codebooks must be in [1, 32]");
  if (c->codebook_size < 1) return bad("codebook_size must be >= 1");
  if (c->latent_dim < 32 || c->latent_dim % 32 || c->latent_dim > 8192) return bad("latent_dim: multiple of 32 in [32, 8192]");
  if (c->channels < 32 || c->channels % 32 || c->channels > 8192) return bad("channels: multiple of 32 in [32, 8192]");
  if (c->n_blocks < 1 || c->n_blocks > DAR_CODEC_MAX_BLOCKS) return bad("n_blocks must be in [1, 8]");
  const int last = c->channels >> c->n_blocks;
  if (last < 32 || last % 32 || (last << c->n_blocks) != c->channels)
    return bad("every block width (channels >> i) must be a multiple of 32");
  if (c->n_units < 1 || c->n_units > DAR_CODEC_MAX_UNITS) return bad("n_units must be in [1, 4]");
  const int K = c->kernel_size;
  if (K < 1 || K > kMaxTaps || K % 2 == 0) return bad("kernel_size must be odd, in [1, 7]");
  for (int u = 0; u < c->n_units; ++u)
    if (c->dilations[u] < 1 || (long long)(K - 1) / 2 * c->dilations[u] > kMaxOff)
      return bad("dilations must be >= 1 with (kernel_size - 1) / 2 * dilation <= 32");
  long long hop = 1;
  for (int i = 0; i < c->n_blocks; ++i) {
    if (c->rates[i] < 2 || c->rates[i] > 16 || c->rates[i] % 2) return bad("rates must be even, in [2, 16]");
    hop *= c->rates[i];
  }
  if (c->max_frames < 1) return bad("max_frames must be >= 1");
  if ((long long)c->max_frames * hop * c->channels >= (1LL << 31)) return bad("max_frames * hop * channels must be < 2^31");
  return DAR_OK;
}

bool al16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct dar_codec {
  dar_codec_config cfg{};
  CodecLayout L{};
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  std::vector<const uint16_t*> tables;
  const uint16_t* in_b = nullptr;
  dar_codec_block blocks[DAR_CODEC_MAX_BLOCKS];
  const uint16_t *out_alpha = nullptr, *out_w = nullptr, *out_b = nullptr;
  std::string err;
  std::vector<hipEvent_t> events;
};

namespace {

int codec_hip_fail(dar_codec* c, hipError_t e, const char* what) {
  const std::string msg = std::string(what) + ": " + hipGetErrorString(e);
  if (c)
    c->err = msg;
  else
    g_codec_error = msg;
  return DAR_E_HIP;
}

#define CODEC_HIP(ctx, call, what)                              \
  do {                                                          \
    hipError_t e_ = (call);                                     \
    if (e_ != hipSuccess) return codec_hip_fail(ctx, e_, what); \
  } while (0)

const uint16_t* U16(const void* p) { return static_cast<const uint16_t*>(p); }

// One decode: every launch in order, each optionally timed (events[2i], [2i+1]).
int run_decode(dar_codec* c, const int32_t* codes, int frames, float* audio, bool timed, std::vector<int>* tags) {
  const dar_codec_config& g = c->cfg;
  const CodecLayout& L = c->L;
  hipStream_t s = c->stream;
  const int K = g.kernel_size;
  size_t ev = 0;
  auto evs = [&](hipEvent_t*& e0, hipEvent_t*& e1) {
    if (!timed) return;
    while (c->events.size() < 2 * (ev + 1)) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return;
      c->events.push_back(e);
    }
    e0 = &c->events[2 * ev];
    e1 = &c->events[2 * ev + 1];
    ++ev;
  };
  auto tag = [&](int t) {
    if (tags) tags->push_back(t);
  };
  uint16_t* z = reinterpret_cast<uint16_t*>(c->ws + L.z);
  float* bufs[2] = {reinterpret_cast<float*>(c->ws + L.xa), reinterpret_cast<float*>(c->ws + L.xb)};
  uint16_t* h = reinterpret_cast<uint16_t*>(c->ws + L.h);
  uint16_t* ops[2] = {reinterpret_cast<uint16_t*>(c->ws + L.sa), reinterpret_cast<uint16_t*>(c->ws + L.sb)};
  int* anom = reinterpret_cast<int*>(c->ws + L.anom);

  RvqArgs ra{};
  for (int k = 0; k < g.n_codebooks; ++k) ra.tab[k] = c->tables[k];
  ra.codes = codes;
  ra.T = frames;
  ra.nq = g.n_codebooks;
  ra.V = g.codebook_size;
  ra.D = g.latent_dim;
  ra.z = z;
  ra.anomalies = anom;
  {
    hipEvent_t *e0 = nullptr, *e1 = nullptr;
    evs(e0, e1);
    const long long n = (long long)frames * (g.latent_dim / 8);
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (timed && e0)
      hipExtLaunchKernelGGL(k_rvq, grid, dim3(kThreads), 0, s, *e0, *e1, 0, ra);
    else
      hipLaunchKernelGGL(k_rvq, grid, dim3(kThreads), 0, s, ra);
    CODEC_HIP(c, hipGetLastError(), "rvq sum");
    tag(0);
  }
  auto conv = [&](ConvArgs& a, int t) -> int {
    hipEvent_t *e0 = nullptr, *e1 = nullptr;
    evs(e0, e1);
    CODEC_HIP(c, launch_conv(a, s, e0 ? *e0 : nullptr, e1 ? *e1 : nullptr), "codec convolution");
    tag(t);
    return DAR_OK;
  };
  int st;
  {
    ConvArgs a{};
    a.xb = z;
    a.T = frames;
    a.Cin = g.latent_dim;
    a.Cout = g.channels;
    a.W = reinterpret_cast<const uint16_t*>(c->ws + L.in_w);
    a.nphase = 1;
    a.ntap = K;
    conv_taps(K, 1, a.off);
    a.bias = c->in_b;
    // the first transposed convolution's operand, bf16(Snake(x, its alpha)), as below
    a.yb = reinterpret_cast<uint16_t*>(bufs[0]);
    a.alpha_out = U16(c->blocks[0].alpha);
    if ((st = conv(a, 1)) != DAR_OK) return st;
  }
  // Every convolution's operand is bf16(Snake(x, its alpha)) of the fp32
  // rows before it. The layer that makes those rows writes that operand too
  // (the same values the convolution would compute when staging the rows,
  // once per element instead of once per workgroup that stages it): the
  // input convolution and each block's last residual unit write only the
  // operand (nothing else reads their rows), the transposed convolutions and
  // the other residual units write it beside their fp32 rows, which the next
  // residual add reads.
  const uint16_t* xb_next = reinterpret_cast<const uint16_t*>(bufs[0]);
  int cur = 0, rows = frames, so = 0;
  for (int i = 0; i < g.n_blocks; ++i) {
    const dar_codec_block& B = c->blocks[i];
    const int cin = width(&g, i), cout = width(&g, i + 1), sr = g.rates[i];
    const uint16_t* alpha_next = U16(i + 1 < g.n_blocks ? c->blocks[i + 1].alpha : c->out_alpha);
    ConvArgs a{};
    a.xb = xb_next;
    a.T = rows;
    a.Cin = cin;
    a.Cout = cout;
    a.W = reinterpret_cast<const uint16_t*>(c->ws + L.up_w[i]);
    a.nphase = sr;
    a.ntap = 2;
    int kidx[kMaxOffs];
    convT_taps(sr, kidx, a.off);
    a.bias = U16(B.up_b);
    a.yf = bufs[cur ^ 1];
    a.ys = ops[so];
    a.alpha_s = U16(B.units[0].alpha1);
    if ((st = conv(a, 2 + 16 * i)) != DAR_OK) return st;
    cur ^= 1;
    rows *= sr;
    const bool fuse = resunit_cfg(cout) >= 0;
    for (int u = 0; u < g.n_units; ++u) {
      const dar_codec_unit& U = B.units[u];
      const bool last = u + 1 == g.n_units;
      uint16_t* hand = reinterpret_cast<uint16_t*>(bufs[cur ^ 1]);  // the last unit's operand for the next layer
      const uint16_t* alpha_s = last ? nullptr : U16(B.units[u + 1].alpha1);
      ConvArgs a1{};
      a1.xf = bufs[cur];  // the residual add's rows
      a1.xb = ops[so];    // the 7-tap convolution's operand
      a1.T = rows;
      a1.Cin = cout;
      a1.Cout = cout;
      a1.W = reinterpret_cast<const uint16_t*>(c->ws + L.w1[i][u]);
      a1.nphase = 1;
      a1.ntap = K;
      conv_taps(K, g.dilations[u], a1.off);
      a1.bias = U16(U.b1);
      if (fuse) {
        ResArgs r{};
        r.c1 = a1;
        r.alpha2 = U16(U.alpha2);
        r.W2 = reinterpret_cast<const uint16_t*>(c->ws + L.w2[i][u]);
        r.b2 = U16(U.b2);
        if (last) {
          r.yb = hand;
          r.alpha_out = alpha_next;
        } else {
          r.y = bufs[cur ^ 1];
          r.ys = ops[so ^ 1];
          r.alpha_s = alpha_s;
        }
        hipEvent_t *e0 = nullptr, *e1 = nullptr;
        evs(e0, e1);
        CODEC_HIP(c, launch_resunit(r, s, e0 ? *e0 : nullptr, e1 ? *e1 : nullptr), "codec residual unit");
        tag(6 + 16 * i);
        cur ^= 1;
        so ^= 1;
        if (last) xb_next = hand;
        continue;
      }
      a1.xf = nullptr;
      a1.yb = h;
      a1.alpha_out = U16(U.alpha2);
      if ((st = conv(a1, 3 + 16 * i)) != DAR_OK) return st;
      ConvArgs a2{};
      a2.xb = h;
      a2.T = rows;
      a2.Cin = cout;
      a2.Cout = cout;
      a2.W = reinterpret_cast<const uint16_t*>(c->ws + L.w2[i][u]);
      a2.nphase = 1;
      a2.ntap = 1;
      a2.off[0] = 0;
      a2.bias = U16(U.b2);
      a2.res = bufs[cur];
      if (last) {
        a2.yb = hand;
        a2.alpha_out = alpha_next;
      } else {
        a2.yf = bufs[cur];
        a2.ys = ops[so ^ 1];
        a2.alpha_s = alpha_s;
      }
      if ((st = conv(a2, 4 + 16 * i)) != DAR_OK) return st;
      so ^= 1;
      if (last) {
        cur ^= 1;
        xb_next = hand;
      }
    }
  }
  {
    hipEvent_t *e0 = nullptr, *e1 = nullptr;
    evs(e0, e1);
    CODEC_HIP(c,
              launch_conv_out(xb_next ? nullptr : bufs[cur], xb_next, c->out_alpha, rows, width(&g, g.n_blocks),
                              c->out_w, c->out_b, K, audio, s, e0 ? *e0 : nullptr, e1 ? *e1 : nullptr),
              "codec output convolution");
    tag(5);
  }
  return DAR_OK;
}

}  // namespace

extern "C" {

int dar_codec_workspace_bytes(const dar_codec_config* cfg, size_t* bytes_out) {
  std::string why;
  const int st = validate_codec(cfg, why);
  if (st != DAR_OK) {
    g_codec_error = why;
    return st;
  }
  if (!bytes_out) return DAR_E_INVAL;
  *bytes_out = codec_layout(cfg).total;
  return DAR_OK;
}

int dar_codec_create(const dar_codec_config* cfg, const dar_codec_weights* w, void* workspace, size_t workspace_bytes,
                     void* stream, dar_codec** out) {
  std::string why;
  int st = validate_codec(cfg, why);
  if (st != DAR_OK) {
    g_codec_error = why;
    return st;
  }
  if (!w || !out || !workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))) {
    g_codec_error = "weights, out and a 256-byte aligned workspace are required";
    return DAR_E_INVAL;
  }
  const CodecLayout L = codec_layout(cfg);
  if (workspace_bytes < L.total) {
    g_codec_error = "workspace smaller than dar_codec_workspace_bytes";
    return DAR_E_WORKSPACE;
  }
  if (!w->tables || !w->blocks || !al16(w->in_w) || !al16(w->in_b) || !al16(w->out_alpha) || !al16(w->out_w) ||
      !al16(w->out_b)) {
    g_codec_error = "a weight pointer is NULL or not 16-byte aligned";
    return DAR_E_INVAL;
  }
  for (int k = 0; k < cfg->n_codebooks; ++k)
    if (!al16(w->tables[k])) {
      g_codec_error = "a codebook table pointer is NULL or not 16-byte aligned";
      return DAR_E_INVAL;
    }
  for (int i = 0; i < cfg->n_blocks; ++i) {
    const dar_codec_block& B = w->blocks[i];
    bool ok = al16(B.alpha) && al16(B.up_w) && al16(B.up_b);
    for (int u = 0; u < cfg->n_units; ++u) {
      const dar_codec_unit& U = B.units[u];
      ok = ok && al16(U.alpha1) && al16(U.w1) && al16(U.b1) && al16(U.alpha2) && al16(U.w2) && al16(U.b2);
    }
    if (!ok) {
      g_codec_error = "a block weight pointer is NULL or not 16-byte aligned";
      return DAR_E_INVAL;
    }
  }
  dar_codec* c = new dar_codec();
  c->cfg = *cfg;
  c->L = L;
  c->stream = static_cast<hipStream_t>(stream);
  c->ws = static_cast<char*>(workspace);
  c->tables.assign(reinterpret_cast<const uint16_t* const*>(w->tables),
                   reinterpret_cast<const uint16_t* const*>(w->tables) + cfg->n_codebooks);
  c->in_b = U16(w->in_b);
  for (int i = 0; i < cfg->n_blocks; ++i) c->blocks[i] = w->blocks[i];
  c->out_alpha = U16(w->out_alpha);
  c->out_w = U16(w->out_w);
  c->out_b = U16(w->out_b);
  hipStream_t s = c->stream;
  const int K = cfg->kernel_size;
  auto fail = [&](hipError_t e, const char* what) {
    codec_hip_fail(nullptr, e, what);
    delete c;
    return DAR_E_HIP;
  };
  hipError_t e;
  if ((e = relayout_conv(U16(w->in_w), cfg->channels, cfg->latent_dim, K,
                         reinterpret_cast<uint16_t*>(c->ws + L.in_w), s)) != hipSuccess)
    return fail(e, "relayout input conv");
  for (int i = 0; i < cfg->n_blocks; ++i) {
    const int cin = width(cfg, i), cout = width(cfg, i + 1);
    if ((e = relayout_convT(U16(w->blocks[i].up_w), cin, cout, cfg->rates[i],
                            reinterpret_cast<uint16_t*>(c->ws + L.up_w[i]), s)) != hipSuccess)
      return fail(e, "relayout transposed conv");
    for (int u = 0; u < cfg->n_units; ++u) {
      if ((e = relayout_conv(U16(w->blocks[i].units[u].w1), cout, cout, K,
                             reinterpret_cast<uint16_t*>(c->ws + L.w1[i][u]), s)) != hipSuccess ||
          (e = relayout_conv(U16(w->blocks[i].units[u].w2), cout, cout, 1,
                             reinterpret_cast<uint16_t*>(c->ws + L.w2[i][u]), s)) != hipSuccess)
        return fail(e, "relayout residual conv");
    }
  }
  if ((e = hipMemsetAsync(c->ws + L.anom, 0, sizeof(int) * 4, s)) != hipSuccess) return fail(e, "clear counter");
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail(e, "create synchronize");
  *out = c;
  return DAR_OK;
}

int dar_codec_decode(dar_codec* c, const int32_t* codes, int32_t frames, float* audio) {
  if (!c || !codes || !audio) return DAR_E_INVAL;
  if (frames < 1) {
    c->err = "frames must be >= 1";
    return DAR_E_INVAL;
  }
  if (frames > c->cfg.max_frames) {
    c->err = "frames above max_frames";
    return DAR_E_CAPACITY;
  }
  return run_decode(c, codes, frames, audio, false, nullptr);
}

int dar_codec_anomalies(dar_codec* c, int32_t* count_out) {
  if (!c || !count_out) return DAR_E_INVAL;
  int v = 0;
  CODEC_HIP(c, hipMemcpyAsync(&v, c->ws + c->L.anom, sizeof(int), hipMemcpyDeviceToHost, c->stream), "read counter");
  CODEC_HIP(c, hipStreamSynchronize(c->stream), "synchronize");
  *count_out = v;
  return DAR_OK;
}

int dar_codec_profile(dar_codec* c, const int32_t* codes, int32_t frames, float* audio, int32_t cap, float* ms_out,
                      int32_t* tag_out, int32_t* n_out) {
  if (!c || !codes || !audio || !ms_out || !tag_out || !n_out || cap < 1) return DAR_E_INVAL;
  if (frames < 1 || frames > c->cfg.max_frames) return frames < 1 ? DAR_E_INVAL : DAR_E_CAPACITY;
  const int launches = 3 + c->cfg.n_blocks * (1 + 2 * c->cfg.n_units);
  if (cap < launches) {
    c->err = "cap below the launches of one decode";
    return DAR_E_INVAL;
  }
  std::vector<int> tags;
  const int st = run_decode(c, codes, frames, audio, true, &tags);
  if (st != DAR_OK) return st;
  CODEC_HIP(c, hipStreamSynchronize(c->stream), "profile synchronize");
  if (c->events.size() < 2 * tags.size()) {
    c->err = "event creation failed";
    return DAR_E_HIP;
  }
  for (size_t i = 0; i < tags.size(); ++i) {
    float ms = 0.f;
    CODEC_HIP(c, hipEventElapsedTime(&ms, c->events[2 * i], c->events[2 * i + 1]), "event time");
    ms_out[i] = ms;
    tag_out[i] = tags[i];
  }
  *n_out = (int32_t)tags.size();
  return DAR_OK;
}

const char* dar_codec_last_error(const dar_codec* c) { return c ? c->err.c_str() : g_codec_error.c_str(); }

int dar_codec_destroy(dar_codec* c) {
  if (!c) return DAR_OK;
  (void)hipStreamSynchronize(c->stream);
  for (hipEvent_t e : c->events) (void)hipEventDestroy(e);
  delete c;
  return DAR_OK;
}

int dar_codec_op_conv(const void* x, int32_t x_bf16, const void* alpha, int32_t T, int32_t Cin, int32_t Cout,
                      const void* w, const void* b, int32_t taps, int32_t dilation, int32_t stride, const float* res,
                      int32_t tanh_out, float* y, void* stream) {
  if (!x || !w || !b || !y || T < 1 || Cin < 1) return DAR_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Cout == 1) {
    if ((x_bf16 != 0) == (alpha != nullptr) || stride != 0 || dilation != 1 || taps < 1 || taps > kMaxTaps ||
        taps % 2 == 0 || !tanh_out || res || Cin % 32)
      return DAR_E_INVAL;
    hipError_t e = x_bf16 ? launch_conv_out(nullptr, U16(x), nullptr, T, Cin, U16(w), U16(b), taps, y, s)
                          : launch_conv_out(static_cast<const float*>(x), nullptr, U16(alpha), T, Cin, U16(w), U16(b),
                                            taps, y, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e == hipSuccess ? DAR_OK : codec_hip_fail(nullptr, e, "op conv out");
  }
  if (Cin % 32 || Cout % 32 || (x_bf16 && (alpha || tanh_out))) return DAR_E_INVAL;
  ConvArgs a{};
  if (x_bf16)
    a.xb = U16(x);
  else
    a.xf = static_cast<const float*>(x);
  a.alpha_in = U16(alpha);
  a.T = T;
  a.Cin = Cin;
  a.Cout = Cout;
  a.bias = U16(b);
  a.yf = y;
  a.res = res;
  a.tanh_out = tanh_out;
  size_t wbytes;
  if (stride == 0) {
    if (taps < 1 || taps > kMaxTaps || taps % 2 == 0 || dilation < 1 || (taps - 1) / 2 * dilation > kMaxOff)
      return DAR_E_INVAL;
    a.nphase = 1;
    a.ntap = taps;
    conv_taps(taps, dilation, a.off);
    wbytes = (size_t)2 * taps * Cout * Cin;
  } else {
    if (stride < 2 || stride > 16 || stride % 2) return DAR_E_INVAL;
    a.nphase = stride;
    a.ntap = 2;
    int kidx[kMaxOffs];
    convT_taps(stride, kidx, a.off);
    wbytes = (size_t)2 * 2 * stride * Cout * Cin;
  }
  void* wr = nullptr;
  hipError_t e = hipMalloc(&wr, wbytes);
  if (e != hipSuccess) return codec_hip_fail(nullptr, e, "op conv alloc");
  e = stride == 0 ? relayout_conv(U16(w), Cout, Cin, taps, static_cast<uint16_t*>(wr), s)
                  : relayout_convT(U16(w), Cin, Cout, stride, static_cast<uint16_t*>(wr), s);
  a.W = static_cast<const uint16_t*>(wr);
  if (e == hipSuccess) e = launch_conv(a, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(wr);
  return e == hipSuccess ? DAR_OK : codec_hip_fail(nullptr, e, "op conv");
}

int dar_codec_op_resunit(const float* x, int32_t T, int32_t C, const void* alpha1, const void* w1, const void* b1,
                         int32_t taps, int32_t dilation, const void* alpha2, const void* w2, const void* b2,
                         int32_t fused, float* y, void* stream) {
  if (!x || !alpha1 || !w1 || !b1 || !alpha2 || !w2 || !b2 || !y || T < 1 || C < 32 || C % 32 || C > 8192 ||
      taps < 1 || taps > kMaxTaps || taps % 2 == 0 || dilation < 1 || (taps - 1) / 2 * dilation > kMaxOff) {
    g_codec_error = "op resunit: bad pointer, width or taps";
    return DAR_E_INVAL;
  }
  if (fused && (resunit_cfg(C) < 0 || y == x)) {
    g_codec_error = "op resunit: the one-launch unit needs C in {32, 64, 96, 128} and y != x";
    return DAR_E_INVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t w1b = (size_t)2 * taps * C * C, w2b = (size_t)2 * C * C, hb = fused ? 0 : (size_t)2 * T * C;
  char* buf = nullptr;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&buf), w1b + w2b + hb);
  if (e != hipSuccess) return codec_hip_fail(nullptr, e, "op resunit alloc");
  uint16_t* W1 = reinterpret_cast<uint16_t*>(buf);
  uint16_t* W2 = reinterpret_cast<uint16_t*>(buf + w1b);
  uint16_t* h = reinterpret_cast<uint16_t*>(buf + w1b + w2b);
  e = relayout_conv(U16(w1), C, C, taps, W1, s);
  if (e == hipSuccess) e = relayout_conv(U16(w2), C, C, 1, W2, s);
  ConvArgs a1{};
  a1.xf = x;
  a1.alpha_in = U16(alpha1);
  a1.T = T;
  a1.Cin = C;
  a1.Cout = C;
  a1.W = W1;
  a1.nphase = 1;
  a1.ntap = taps;
  conv_taps(taps, dilation, a1.off);
  a1.bias = U16(b1);
  if (e == hipSuccess && fused) {
    ResArgs r{};
    r.c1 = a1;
    r.alpha2 = U16(alpha2);
    r.W2 = W2;
    r.b2 = U16(b2);
    r.y = y;
    e = launch_resunit(r, s);
  } else if (e == hipSuccess) {
    a1.yb = h;
    a1.alpha_out = U16(alpha2);
    e = launch_conv(a1, s);
    ConvArgs a2{};
    a2.xb = h;
    a2.T = T;
    a2.Cin = C;
    a2.Cout = C;
    a2.W = W2;
    a2.nphase = 1;
    a2.ntap = 1;
    a2.bias = U16(b2);
    a2.yf = y;
    a2.res = x;
    if (e == hipSuccess) e = launch_conv(a2, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(buf);
  return e == hipSuccess ? DAR_OK : codec_hip_fail(nullptr, e, "op resunit");
}

}  // extern "C"
