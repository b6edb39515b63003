// gfx950 kernels that run a layer over many rows at once: the prompt prefill
// (a block of up to kPrefillRows prompt positions) and batched decode (one
// row per sequence, two in the fast AR's first pass), so every weight matrix
// is read once per launch instead of once per row.
//
// The projections become GEMMs y[m][n] = sum_k x[m][k] W[n][k] with m over the
// block's positions, run on MFMA (v_mfma_f32_32x32x16_bf16). The weights are
// bf16 or e4m3fn (widened exactly to bf16 in registers, the per-row scale
// applied to the finished sum). The inputs are split into two bf16 parts
// x = hi + lo (|x - hi - lo| <= 2^-16 |x|) and both parts are multiplied, so
// the GEMM keeps the fp32 inputs of the decode path to within fp32 rounding
// noise. Attention over the block (causal, the cache holding earlier blocks)
// reuses the decode attention kernels with one query row per position.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "dar_internal.h"
#include "dar_sample.h"

namespace dar {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTileN = 128;    // weight rows per workgroup (32 per wave)
constexpr int kRowChunk = 128; // bytes of every weight row per GEMM chunk
constexpr int kStages = 3;     // chunks in the LDS ring of the GEMM

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 16 bytes per lane moved from global memory straight into LDS (no register
// staging): lane l's bytes land at lds + 16 l, lds being the same for the
// whole wave.
__device__ __forceinline__ void load_lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)lds, 16, 0, 0);
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order); the other counters are left alone.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A staged chunk holds 128 B of each of 128 weight rows; the 16-byte units of
// row r sit XOR-swizzled, unit u at slot u ^ swz8(r). The LDS serves 16-byte
// reads sixteen lanes at a time from 64 four-byte banks (256 B), and sixteen
// consecutive 128-byte rows read at one unit then land in sixteen distinct
// 16-byte bank groups (r % 2 picks the half of the 256 B, swz8 the unit).
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
// the same for the staged input rows of XU units: 128-byte rows (XU = 8) as
// above; rows of 256 or 512 bytes (XU = 16, 32) start on the same bank, so
// the unit is swizzled by r % 16
template <int XU>
__device__ __forceinline__ int swzx(int r) {
  return XU >= 16 ? (r & 15) : ((r >> 1) & 7);
}
struct BF16T {
  static constexpr int kBits = 16;
  static constexpr bool kGrouped = false;
  // eight consecutive weights of row r at k = 16 s + 8 half, as the MFMA B operand
  __device__ static __forceinline__ bf16x8 frag(const char* st, int r, int s, int half) {
    const int u = (2 * s + half) ^ swz8(r);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + (r * 8 + u) * 16));
  }
};

struct FP8T {
  static constexpr int kBits = 8;
  static constexpr bool kGrouped = false;
  // e4m3fn values are exact in bf16: widen through fp32 and keep the top half
  __device__ static __forceinline__ uint32_t pack2(f32x2 v) {
    return (__float_as_uint(v.x) >> 16) | (__float_as_uint(v.y) & 0xffff0000u);
  }
  __device__ static __forceinline__ bf16x8 frag(const char* st, int r, int s, int half) {
    const int u = s ^ swz8(r);
    const u32x2 w = *reinterpret_cast<const u32x2*>(st + (r * 8 + u) * 16 + 8 * half);
    u32x4 o;
    o.x = pack2(__builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false));
    o.y = pack2(__builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true));
    o.z = pack2(__builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false));
    o.w = pack2(__builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true));
    return __builtin_bit_cast(bf16x8, o);
  }
};

struct INT8T {
  static constexpr int kBits = 8;
  static constexpr bool kGrouped = false;
  // int8 codes (|q| <= 127) are exact in bf16: sign-extend, convert, keep the top half
  __device__ static __forceinline__ uint32_t pack2(int a, int b) {
    return (__float_as_uint((float)a) >> 16) | (__float_as_uint((float)b) & 0xffff0000u);
  }
  __device__ static __forceinline__ bf16x8 frag(const char* st, int r, int s, int half) {
    const int u = s ^ swz8(r);
    const u32x2 w = *reinterpret_cast<const u32x2*>(st + (r * 8 + u) * 16 + 8 * half);
    const int x = (int)w.x, y = (int)w.y;
    u32x4 o;
    o.x = pack2((x << 24) >> 24, (x << 16) >> 24);
    o.y = pack2((x << 8) >> 24, x >> 24);
    o.z = pack2((y << 24) >> 24, (y << 16) >> 24);
    o.w = pack2((y << 8) >> 24, y >> 24);
    return __builtin_bit_cast(bf16x8, o);
  }
};

// Two's complement int4 codes, two per byte (even column in the low nibble),
// with an fp32 scale per (row, 128 columns): a 128-byte chunk of a row is two
// scale groups of 128 codes. A k-step's eight codes are one 32-bit word.
struct INT4T {
  static constexpr int kBits = 4;
  static constexpr bool kGrouped = true;
  __device__ static __forceinline__ uint32_t pack2(int a, int b) {
    return (__float_as_uint((float)a) >> 16) | (__float_as_uint((float)b) & 0xffff0000u);
  }
  __device__ static __forceinline__ bf16x8 frag(const char* st, int r, int s, int half) {
    const int u = (s >> 1) ^ swz8(r);
    const int w = *reinterpret_cast<const int*>(st + (r * 8 + u) * 16 + (s & 1) * 8 + 4 * half);
    u32x4 o;
    o.x = pack2((w << 28) >> 28, (w << 24) >> 28);
    o.y = pack2((w << 20) >> 28, (w << 16) >> 28);
    o.z = pack2((w << 12) >> 28, (w << 8) >> 28);
    o.w = pack2((w << 4) >> 28, w >> 28);
    return __builtin_bit_cast(bf16x8, o);
  }
};

// The workgroup's finished sums: lane l holds weight row (output column) n =
// its tile row, and accumulator v of tile mt holds input row
// m0 + 32 mt + (v % 4) + 4 (l / 32) + 8 (v / 4). Split partials carry the row
// scale when deferred (the reduce pass applies it otherwise).
template <int MT>
__device__ __forceinline__ void gemm_store(const GemmArgs& a, const f32x16 (&acc)[MT], int n, int m0, int lane) {
  if (n >= a.N) return;
  const float sc = (a.scale && (a.splits == 1 || a.defer)) ? a.scale[n] : 1.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + mt * 32 + (v % 4) + 4 * (lane >> 5) + 8 * (v / 4);
      if (m >= a.M) continue;
      if (a.defer) {
        a.part[((size_t)blockIdx.z * a.M + m) * a.N + n] = acc[mt][v] * sc;
      } else if (a.splits == 1) {
        float* y = a.y + (size_t)m * a.y_stride + n;
        const float val = acc[mt][v] * sc;
        *y = a.accumulate ? *y + val : val;
      } else {
        a.part[((size_t)blockIdx.z * a.M + m) * a.N + n] = acc[mt][v];
      }
    }
  }
}

// k per chunk (128 bytes of a weight row)
template <typename WT>
constexpr int kChunkK = kRowChunk * 8 / WT::kBits;

// One workgroup: weight rows [128 bx, +128) (wave w: 32 rows) x input rows
// [32 MT by, +32 MT) x the chunks of split bz. A chunk is 128 B of each
// weight row (64 bf16, 128 e4m3 or int8, 256 int4 weights) and the matching
// hi and lo input columns (same swizzle, per input row). Chunks stream
// through a ring of kStages LDS buffers by direct loads, issued kStages - 1
// chunks ahead; a chunk costs one barrier, after which every wave runs its
// MFMAs from LDS. Group-scaled weights (int4) sum each 128-column group on its
// own and add it times the group's scale, loaded with the chunk.
template <typename WT, int MT>
__global__ __launch_bounds__(kBlock) void k_gemm(GemmArgs a) {
  constexpr int KC = kChunkK<WT>;                      // k per chunk
  constexpr int ST = KC / 16;                          // MFMA k-steps per chunk
  constexpr int XU = KC / 8;                           // 16-byte units of an input row per chunk
  constexpr int WB = kTileN * kRowChunk;               // weight bytes per stage
  constexpr int XB = 2 * 32 * MT * XU * 16;            // input bytes per stage (hi, lo)
  constexpr int SB = WB + XB;
  constexpr int XL = XB / (16 * 64 * kWaves);          // input loads per wave per stage
  constexpr int LPS = 4 + XL + (WT::kGrouped ? 1 : 0); // loads per wave per stage
  static_assert(XL * 16 * 64 * kWaves == XB, "input staging split");
  static_assert(!WT::kGrouped || (MT == 1 && KC == 256), "group scales: two 128-column groups per chunk");
  __shared__ __align__(16) char sm[kStages * SB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = blockIdx.x * kTileN;
  const int m0 = blockIdx.y * 32 * MT;
  const int c_begin = blockIdx.z * a.cps;
  const int nc = min(a.K / KC, c_begin + a.cps) - c_begin;
  // weight load i of this wave fills rows 32 wave + 8 i + lane / 8, slot lane % 8
  const char* wsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + 8 * i + (lane >> 3);
    wsrc[i] = reinterpret_cast<const char*>(a.W) + (size_t)min(nb + r, a.N - 1) * a.K * WT::kBits / 8 +
              (size_t)c_begin * kRowChunk + 16 * ((lane & 7) ^ swz8(r));
  }
  // group scales of this lane's weight row, two per chunk
  const f32x2* gsrc = nullptr;
  if constexpr (WT::kGrouped)
    gsrc = reinterpret_cast<const f32x2*>(a.scale + (size_t)min(nb + wave * 32 + (lane & 31), a.N - 1) * (a.K / 128)) +
           c_begin;
  f32x2 gsc[kStages];
  // input load j of this wave fills 64 consecutive slots of the hi or lo part
  const char* xsrc[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int q0 = (wave * XL + j) * 64;
    const int part = q0 / (32 * MT * XU);
    const int q = q0 % (32 * MT * XU) + lane;
    const int row = q / XU, u = (q % XU) ^ swzx<XU>(row);
    xsrc[j] = reinterpret_cast<const char*>(part ? a.xl : a.xh) +
              ((size_t)(m0 + row) * a.K + (size_t)c_begin * KC) * 2 + 16 * u;
  }
  auto issue = [&](int t, int stage) {
    char* base = sm + stage * SB;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_lds16(wsrc[i] + (size_t)t * kRowChunk, base + wave * 4096 + i * 1024);
#pragma unroll
    for (int j = 0; j < XL; ++j) load_lds16(xsrc[j] + (size_t)t * KC * 2, base + WB + (wave * XL + j) * 1024);
    if constexpr (WT::kGrouped) gsc[stage] = gsrc[t];
  };
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[mt][v] = 0.f;
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j)
    if (j < nc) issue(j, j);
  const int half = lane >> 5;
  for (int t0 = 0; t0 < nc; t0 += kStages) {
#pragma unroll
    for (int j = 0; j < kStages; ++j) {
      const int t = t0 + j;
      if (t < nc) {
        // chunk t has landed for this wave once only the later chunks' loads are outstanding
        static_assert(kStages == 3, "wait counts below assume three stages");
        if (t + 1 < nc) wait_loads<LPS>();
        else wait_loads<0>();
        // every wave's chunk t has landed, and every wave is done with chunk t - 1's buffer
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t + kStages - 1 < nc) issue(t + kStages - 1, (j + kStages - 1) % kStages);
        const char* ws = sm + j * SB;
        const char* xs = ws + WB;
        if constexpr (WT::kGrouped) {
          const int row = lane & 31;
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            f32x16 gh, gl;
#pragma unroll
            for (int v = 0; v < 16; ++v) gh[v] = gl[v] = 0.f;
#pragma unroll
            for (int s = 8 * g; s < 8 * g + 8; ++s) {
              const bf16x8 b = WT::frag(ws, wave * 32 + row, s, half);
              const int u = (2 * s + half) ^ swzx<XU>(row);
              const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + (row * XU + u) * 16));
              const bf16x8 al =
                  __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + ((32 + row) * XU + u) * 16));
              gh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b, gh, 0, 0, 0);
              gl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, gl, 0, 0, 0);
            }
            const float sc = g ? gsc[j].y : gsc[j].x;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[0][v] = fmaf(gh[v] + gl[v], sc, acc[0][v]);
          }
        } else {
#pragma unroll
          for (int s = 0; s < ST; ++s) {
            const bf16x8 b = WT::frag(ws, wave * 32 + (lane & 31), s, half);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const int row = mt * 32 + (lane & 31);
              const int u = (2 * s + half) ^ swzx<XU>(row);
              const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + (row * XU + u) * 16));
              const bf16x8 al =
                  __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + ((32 * MT + row) * XU + u) * 16));
              acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b, acc[mt], 0, 0, 0);
              acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, acc[mt], 0, 0, 0);
            }
          }
        }
      }
    }
  }
  if constexpr (WT::kGrouped) {
    GemmArgs b = a;
    b.scale = nullptr;  // already applied per group
    gemm_store<MT>(b, acc, nb + wave * 32 + (lane & 31), m0, lane);
  } else {
    gemm_store<MT>(a, acc, nb + wave * 32 + (lane & 31), m0, lane);
  }
}

// The same product with eight waves per workgroup (two per SIMD, so one
// wave's MFMAs cover the other's LDS reads and waits) over 64 or 128 input
// rows: the staged chunk and its layout are k_gemm's; each wave multiplies
// 32 input rows by 32 NT weight rows (NT = 2 at 128 input rows: a k-step
// reads two weight fragments and one hi/lo pair for four MFMAs), with the hi
// and lo products in separate accumulators.
constexpr int kWaves8 = 8;
template <typename WT, int MT>
__global__ __launch_bounds__(kWaves8 * kWave) void k_gemm8(GemmArgs a) {
  static_assert(!WT::kGrouped && (MT == 2 || MT == 4), "row-scaled or unscaled weights, 64 or 128 rows");
  constexpr int KC = kChunkK<WT>;
  constexpr int ST = KC / 16;
  constexpr int XU = KC / 8;
  constexpr int WB = kTileN * kRowChunk;
  constexpr int XB = 2 * 32 * MT * XU * 16;
  constexpr int SB = WB + XB;
  constexpr int WL = WB / (16 * 64 * kWaves8);         // weight loads per wave per stage
  constexpr int XL = XB / (16 * 64 * kWaves8);         // input loads per wave per stage
  constexpr int LPS = WL + XL;
  constexpr int WMW = MT;                              // waves along the input rows (32 rows each)
  constexpr int WNW = kWaves8 / WMW;                   // waves along the weight rows
  constexpr int NT = kTileN / 32 / WNW;                // 32-row weight tiles per wave
  static_assert(WL * 16 * 64 * kWaves8 == WB && XL * 16 * 64 * kWaves8 == XB, "staging split");
  static_assert(kStages * SB <= 160 * 1024, "LDS");
  __shared__ __align__(16) char sm[kStages * SB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WNW, wm = wave / WNW;
  const int nb = blockIdx.x * kTileN;
  const int m0 = blockIdx.y * 32 * MT;
  const int c_begin = blockIdx.z * a.cps;
  const int nc = min(a.K / KC, c_begin + a.cps) - c_begin;
  // weight load i of this wave fills rows 16 wave + 8 i + lane / 8, slot lane % 8
  const char* wsrc[WL];
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int r = wave * 8 * WL + 8 * i + (lane >> 3);
    wsrc[i] = reinterpret_cast<const char*>(a.W) + (size_t)min(nb + r, a.N - 1) * a.K * WT::kBits / 8 +
              (size_t)c_begin * kRowChunk + 16 * ((lane & 7) ^ swz8(r));
  }
  const char* xsrc[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int q0 = (wave * XL + j) * 64;
    const int part = q0 / (32 * MT * XU);
    const int q = q0 % (32 * MT * XU) + lane;
    const int row = q / XU, u = (q % XU) ^ swzx<XU>(row);
    xsrc[j] = reinterpret_cast<const char*>(part ? a.xl : a.xh) +
              ((size_t)(m0 + row) * a.K + (size_t)c_begin * KC) * 2 + 16 * u;
  }
  auto issue = [&](int t, int stage) {
    char* base = sm + stage * SB;
#pragma unroll
    for (int i = 0; i < WL; ++i)
      load_lds16(wsrc[i] + (size_t)t * kRowChunk, base + (wave * WL + i) * 1024);
#pragma unroll
    for (int j = 0; j < XL; ++j) load_lds16(xsrc[j] + (size_t)t * KC * 2, base + WB + (wave * XL + j) * 1024);
  };
  f32x16 acc_h[NT], acc_l[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_h[nt][v] = acc_l[nt][v] = 0.f;
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j)
    if (j < nc) issue(j, j);
  const int half = lane >> 5;
  const int row = wm * 32 + (lane & 31);
  for (int t0 = 0; t0 < nc; t0 += kStages) {
#pragma unroll
    for (int j = 0; j < kStages; ++j) {
      const int t = t0 + j;
      if (t < nc) {
        static_assert(kStages == 3, "wait counts below assume three stages");
        if (t + 1 < nc) wait_loads<LPS>();
        else wait_loads<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t + kStages - 1 < nc) issue(t + kStages - 1, (j + kStages - 1) % kStages);
        const char* ws = sm + j * SB;
        const char* xs = ws + WB;
#pragma unroll
        for (int s = 0; s < ST; ++s) {
          bf16x8 b[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) b[nt] = WT::frag(ws, (wn * NT + nt) * 32 + (lane & 31), s, half);
          const int u = (2 * s + half) ^ swzx<XU>(row);
          const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + (row * XU + u) * 16));
          const bf16x8 al =
              __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + ((32 * MT + row) * XU + u) * 16));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc_h[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b[nt], acc_h[nt], 0, 0, 0);
            acc_l[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b[nt], acc_l[nt], 0, 0, 0);
          }
        }
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x16 acc[1];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[0][v] = acc_h[nt][v] + acc_l[nt][v];
    gemm_store<1>(a, acc, nb + (wn * NT + nt) * 32 + (lane & 31), m0 + wm * 32, lane);
  }
}

// s_waitcnt vmcnt(4 n) for a count n in [0, 5] known only at run time
__device__ __forceinline__ void wait_loads_x4(int n) {
  switch (n) {
    case 0: wait_loads<0>(); break;
    case 1: wait_loads<4>(); break;
    case 2: wait_loads<8>(); break;
    case 3: wait_loads<12>(); break;
    case 4: wait_loads<16>(); break;
    default: wait_loads<20>(); break;
  }
}

// Up to 32 input rows (MT = 1) with the split's input resident: the
// workgroup first moves all of its split's input chunks into LDS (one
// barrier), then every wave streams only its own 32 weight rows through its
// own ring of kStages chunk slots, waiting on its own loads alone: no
// workgroup barrier per chunk. The hi and lo products accumulate separately
// so that consecutive MFMAs do not wait on each other. Same LDS layouts as
// k_gemm. Needs a.cps <= kResidentChunks<WT>. (Staging only 16 input rows
// for a six-slot ring was tried at 16 sequences: no faster.)
template <typename WT>
constexpr int kResidentChunks = WT::kBits == 16 ? 14 : 7;  // a one-byte chunk spans twice the input columns

template <typename WT>
__global__ __launch_bounds__(kBlock) void k_gemm_x(GemmArgs a) {
  static_assert(!WT::kGrouped, "row-scaled or unscaled weights only");
  constexpr int KC = kChunkK<WT>;
  constexpr int ST = KC / 16;
  constexpr int XU = KC / 8;
  constexpr int XROWS = 32;                            // staged input rows
  constexpr int XB = 2 * XROWS * XU * 16;              // input bytes per chunk (hi, lo)
  constexpr int XL = XB / (16 * 64 * kWaves);          // input loads per wave per chunk
  constexpr int WS = 32 * kRowChunk;                   // one wave's weight bytes per chunk
  constexpr int S = kStages;                           // ring slots per wave
  constexpr int XR = kResidentChunks<WT> * XB;
  static_assert(XL * 16 * 64 * kWaves == XB, "input staging split");
  static_assert(XR + kWaves * S * WS <= 160 * 1024, "LDS");
  __shared__ __align__(16) char sm[XR + kWaves * S * WS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = blockIdx.x * kTileN;
  const int c_begin = blockIdx.z * a.cps;
  const int nc = min(a.K / KC, c_begin + a.cps) - c_begin;
  char* ring = sm + XR + wave * S * WS;
  const char* wsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + 8 * i + (lane >> 3);
    wsrc[i] = reinterpret_cast<const char*>(a.W) + (size_t)min(nb + r, a.N - 1) * a.K * WT::kBits / 8 +
              (size_t)c_begin * kRowChunk + 16 * ((lane & 7) ^ swz8(r));
  }
  auto issue_w = [&](int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) load_lds16(wsrc[i] + (size_t)t * kRowChunk, ring + (t % S) * WS + i * 1024);
  };
  // the split's input, chunk t at sm + t XB
  for (int t = 0; t < nc; ++t) {
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int q0 = (wave * XL + j) * 64;
      const int part = q0 / (XROWS * XU);
      const int q = q0 % (XROWS * XU) + lane;
      const int row = q / XU, u = (q % XU) ^ swzx<XU>(row);
      load_lds16(reinterpret_cast<const char*>(part ? a.xl : a.xh) +
                     ((size_t)row * a.K + (size_t)(c_begin + t) * KC) * 2 + 16 * u,
                 sm + t * XB + (wave * XL + j) * 1024);
    }
  }
  for (int j = 0; j < S - 1 && j < nc; ++j) issue_w(j);
  // the input has landed for this wave once only its weight loads are outstanding
  wait_loads_x4(min(S - 1, nc));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  f32x16 acc[1], acc_lo;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[0][v] = acc_lo[v] = 0.f;
  const int half = lane >> 5;
  const int xrow = lane & 31;
  for (int t = 0; t < nc; ++t) {
    // this wave's chunk t has landed once only its later chunks' loads are outstanding
    wait_loads_x4(min(S - 2, nc - 1 - t));
    asm volatile("" ::: "memory");
    // the slot refilled here held chunk t - 1, whose reads this wave finished
    if (t + S - 1 < nc) issue_w(t + S - 1);
    const char* ws = ring + (t % S) * WS;
    const char* xs = sm + t * XB;
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      const bf16x8 b = WT::frag(ws, lane & 31, s, half);
      const int u = (2 * s + half) ^ swzx<XU>(xrow);
      const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + (xrow * XU + u) * 16));
      const bf16x8 al =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + ((XROWS + xrow) * XU + u) * 16));
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b, acc[0], 0, 0, 0);
      acc_lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, acc_lo, 0, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[0][v] += acc_lo[v];
  gemm_store<1>(a, acc, nb + wave * 32 + (lane & 31), 0, lane);
}

// y[m][n] (+)= scale[n] * sum over splits (fixed order) of the partial sums
__global__ void k_gemm_reduce(GemmArgs a) {
  const size_t total = (size_t)a.M * a.N;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / a.N), n = (int)(i % a.N);
    float s = 0.f;
    for (int z = 0; z < a.splits; ++z) s += a.part[(size_t)z * total + i];
    if (a.scale) s *= a.scale[n];
    float* y = a.y + (size_t)m * a.y_stride + n;
    *y = a.accumulate ? *y + s : s;
  }
}

// Block reduction of one value per thread; result in every thread.
template <int NW = kWaves>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += red[w];
  __syncthreads();
  return t;
}

constexpr int kNormBlock = 1024;  // threads per row of k_norm_split (a float4 each at d = 4096)

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// Four consecutive elements of a pending split-K sum starting at element idx
// (fixed order: splits in groups of eight, each group summed pairwise), so
// that up to eight splits' loads are in flight together.
__device__ __forceinline__ float4 part_sum4(const PartSum& ps, size_t idx) {
  const float* p = ps.p + idx;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  int z = 0;
  for (; z + 8 <= ps.n; z += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld4(p + (size_t)(z + u) * ps.stride);
    s = add4(s, add4(add4(add4(v[0], v[1]), add4(v[2], v[3])), add4(add4(v[4], v[5]), add4(v[6], v[7]))));
  }
  if (z + 4 <= ps.n) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ld4(p + (size_t)(z + u) * ps.stride);
    s = add4(s, add4(add4(v[0], v[1]), add4(v[2], v[3])));
    z += 4;
  }
  for (; z < ps.n; ++z) s = add4(s, ld4(p + (size_t)z * ps.stride));
  return s;
}

// hi/lo bf16 of four values, stored as 8 bytes each
__device__ __forceinline__ void split_store4(float4 v, uint16_t* oh, uint16_t* ol) {
  const uint16_t h0 = f2bf(v.x), h1 = f2bf(v.y), h2 = f2bf(v.z), h3 = f2bf(v.w);
  const uint16_t l0 = f2bf(v.x - bf2f(h0)), l1 = f2bf(v.y - bf2f(h1));
  const uint16_t l2 = f2bf(v.z - bf2f(h2)), l3 = f2bf(v.w - bf2f(h3));
  *reinterpret_cast<u32x2*>(oh) = u32x2{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
  *reinterpret_cast<u32x2*>(ol) = u32x2{(uint32_t)l0 | ((uint32_t)l1 << 16), (uint32_t)l2 | ((uint32_t)l3 << 16)};
}

// Row m of the GEMM input: v = x[m] (RMSNorm(x[m]) * gain when gain is set),
// written as hi = bf16(v), lo = bf16(v - hi); rows M..Mpad-1 are zero. With
// residual sums pending, x[m] += their sum first (written back). With out_f32
// set, v is also written there in fp32 (row stride K). Columns in fours, at
// most kNormCols4 per thread, kept in registers from the load to the split
// (no second read of the row after the norm's block sum).
constexpr int kNormCols4 = 4;  // K <= 4 * kNormCols4 * kNormBlock
__global__ __launch_bounds__(kNormBlock) void k_norm_split(float* x, int x_stride, int M, int K,
                                                            const uint16_t* gain, float eps, uint16_t* xh,
                                                            uint16_t* xl, float* out_f32, PartSum add) {
  constexpr int NW = kNormBlock / kWave;
  __shared__ float red[NW];
  const int m = blockIdx.x, tid = threadIdx.x;
  uint16_t* oh = xh + (size_t)m * K;
  uint16_t* ol = xl + (size_t)m * K;
  if (m >= M) {
    for (int k = tid; k < K; k += kNormBlock) oh[k] = ol[k] = 0;
    return;
  }
  float* xr = x + (size_t)m * x_stride;
  float ss = 0.f;
  float4 xv[kNormCols4];
  u32x2 gv[kNormCols4];
#pragma unroll
  for (int j = 0; j < kNormCols4; ++j) {
    const int k = 4 * tid + j * 4 * kNormBlock;
    if (k >= K) break;
    if (gain) gv[j] = *reinterpret_cast<const u32x2*>(gain + k);  // in flight with the row's loads
    float4 v = ld4(xr + k);
    if (add.n > 0) {
      v = add4(v, part_sum4(add, (size_t)m * K + k));
      *reinterpret_cast<float4*>(xr + k) = v;
    }
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    xv[j] = v;
  }
  float inv = 1.f;
  if (gain) {
    ss = block_sum<NW>(ss, red);
    inv = 1.0f / sqrtf(ss / (float)K + eps);
  }
#pragma unroll
  for (int j = 0; j < kNormCols4; ++j) {
    const int k = 4 * tid + j * 4 * kNormBlock;
    if (k >= K) break;
    float4 v = xv[j];
    if (gain) {
      const u32x2 g = gv[j];
      v.x = (v.x * inv) * bf2f((uint16_t)(g.x & 0xffffu));
      v.y = (v.y * inv) * bf2f((uint16_t)(g.x >> 16));
      v.z = (v.z * inv) * bf2f((uint16_t)(g.y & 0xffffu));
      v.w = (v.w * inv) * bf2f((uint16_t)(g.y >> 16));
    }
    split_store4(v, oh + k, ol + k);
    if (out_f32) *reinterpret_cast<float4*>(out_f32 + (size_t)m * K + k) = v;
  }
}

// x[m] = table[clamp(tok[m])] as fp32 for the block's prompt ids
__global__ __launch_bounds__(kBlock) void k_embed_rows(const uint16_t* table, int rows, int K, const int* tok,
                                                        float* x, int* anomalies) {
  const int m = blockIdx.x;
  const int t = tok[m];
  const int c = min(max(t, 0), rows - 1);
  if (threadIdx.x == 0 && t != c) atomicAdd(anomalies, 1);
  const uint16_t* row = table + (size_t)c * K;
  for (int k = threadIdx.x; k < K; k += kBlock) x[(size_t)m * K + k] = bf2f(row[k]);
}

// RoPE at positions p0 + m (or row_pos[m]) on q and k of the rows' QKV output
// (or of the pending split-K sums src), q to q_out, k and v appended to the
// bf16 caches (rotate-half pairs (i, i + hd/2)); with row_seq, row m appends
// to sequence row_seq[m]'s cache; with a page map, position p of sequence s
// goes to page table[s][p >> shift] (seq_stride elements per page) at offset
// p within the page. One wave per (row, head), lane i: pair i.
__global__ __launch_bounds__(kWave) void k_rope_rows(const float* qkv, PartSum src, int M, int p0,
                                                      const int* row_pos, const int* row_seq, long long seq_stride,
                                                      int n_heads_q, int n_heads_kv, int head_dim, const float2* rope,
                                                      float* q_out, uint16_t* kc, uint16_t* vc, int cache_len,
                                                      PageMap pm) {
  const int m = blockIdx.x, head = blockIdx.y, i = threadIdx.x;
  const int half = head_dim / 2;
  if (i >= half) return;
  const int width = (n_heads_q + 2 * n_heads_kv) * head_dim;
  const int pos_abs = row_pos ? row_pos[m] : p0 + m;
  int pos = pos_abs;  // position within the cache block written
  if (pm.table) {
    const int sq = row_seq ? row_seq[m] : pm.seq0;
    const size_t page = (size_t)pm.table[(size_t)sq * pm.per_seq + (pos_abs >> pm.shift)];
    kc += page * seq_stride;
    vc += page * seq_stride;
    pos = pos_abs & ((1 << pm.shift) - 1);
  } else if (row_seq) {
    kc += (size_t)row_seq[m] * seq_stride;
    vc += (size_t)row_seq[m] * seq_stride;
  }
  const int r1 = head * head_dim + i, r2 = r1 + half;
  float u, v;
  if (src.n > 0) {
    const float* p = src.p + (size_t)m * width;
    u = p[r1];
    v = p[r2];
    for (int z = 1; z < src.n; ++z) {
      u += p[(size_t)z * src.stride + r1];
      v += p[(size_t)z * src.stride + r2];
    }
  } else {
    u = qkv[(size_t)m * width + r1];
    v = qkv[(size_t)m * width + r2];
  }
  if (head < n_heads_q + n_heads_kv) {
    const float2 cs = rope[(size_t)pos_abs * half + i];
    const float o1 = u * cs.x - v * cs.y;
    const float o2 = u * cs.y + v * cs.x;
    if (head < n_heads_q) {
      q_out[(size_t)m * n_heads_q * head_dim + r1] = o1;
      q_out[(size_t)m * n_heads_q * head_dim + r2] = o2;
    } else {
      uint16_t* kp = kc + ((size_t)(head - n_heads_q) * cache_len + pos) * head_dim;
      kp[i] = f2bf(o1);
      kp[i + half] = f2bf(o2);
    }
  } else {
    uint16_t* vp = vc + ((size_t)(head - n_heads_q - n_heads_kv) * cache_len + pos) * head_dim;
    vp[i] = f2bf(u);
    vp[i + half] = f2bf(v);
  }
}

// h = SiLU(a) * b per element (a, b: the pending sums pa, pb when set), split
// into bf16 hi/lo rows (rows M..Mpad-1 zero). Block (row, 1024 columns).
__global__ __launch_bounds__(kBlock) void k_silu_split(const float* a, const float* b, PartSum pa, PartSum pb, int M,
                                                        int F, uint16_t* hh, uint16_t* hl) {
  const int m = blockIdx.x, k = 4 * (blockIdx.y * kBlock + threadIdx.x);
  if (k >= F) return;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (m < M) {
    const size_t idx = (size_t)m * F + k;
    const float4 g = pa.n > 0 ? part_sum4(pa, idx) : ld4(a + idx);
    const float4 u = pb.n > 0 ? part_sum4(pb, idx) : ld4(b + idx);
    v.x = g.x / (1.0f + expf(-g.x)) * u.x;
    v.y = g.y / (1.0f + expf(-g.y)) * u.y;
    v.z = g.z / (1.0f + expf(-g.z)) * u.z;
    v.w = g.w / (1.0f + expf(-g.w)) * u.w;
  }
  split_store4(v, hh + (size_t)m * F + k, hl + (size_t)m * F + k);
}

// Batched codebook commit, one workgroup per sequence b: the first index of
// the maximum of logits[b] (NaN counts as -inf and as an anomaly), recorded as
// the argmax and (or the forced code) as the committed code, then the next
// inputs gathered from the tables and the position advanced.
__global__ __launch_bounds__(kBlock) void k_commit_rows(RowsCommitArgs a) {
  __shared__ unsigned long long red[kWaves];
  __shared__ int code_sh;
  extern __shared__ __align__(16) char sample_lds[];  // sample_lds_bytes(V) when sampling
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* lg = a.logits + (size_t)b * a.ld;
  int sampled = 0;
  if (a.smp.u) {
    // window: sequence b's committed codes of this codebook at positions [lo, pos)
    const int pos = a.pos[b], lo = max(a.smp.win_lo[b], pos - a.smp.window);
    sampled = sample_row(lg, a.V, a.smp, a.smp.u[((size_t)pos * a.B + b) * a.frame_codes + a.code_index],
                         a.ring + ((size_t)lo * a.B + b) * a.frame_codes + a.code_index,
                         (long long)a.B * a.frame_codes, max(pos - lo, 0), sample_lds);
  }
  unsigned long long best = 0ull;
  int bad = 0;
  for (int i = tid; i < a.V; i += kBlock) {
    float v = lg[i];
    if (!isfinite(v)) {
      ++bad;
      if (v != v) v = -INFINITY;
    }
    // order-preserving key of the value, ties to the lower index
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    const unsigned long long k = ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
    best = k > best ? k : best;
  }
  if (bad) atomicAdd(a.anomalies, bad);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long m = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = red[w] > m ? red[w] : m;
    const int pred = a.smp.u ? sampled : (int)(0xffffffffu - (uint32_t)(m & 0xffffffffull));
    const int slot = b * a.frame_codes + a.code_index;
    const int code = *a.force_flag ? a.forced[slot] : pred;
    a.pred[slot] = pred;
    a.committed[slot] = code;
    a.ring[((size_t)a.pos[b] * a.B + b) * a.frame_codes + a.code_index] = code;
    code_sh = code;
  }
  __syncthreads();
  const int code = code_sh;
  if (a.next_table) {
    const uint16_t* row = a.next_table + (size_t)min(max(code, 0), a.next_rows - 1) * a.K;
    for (int k = tid; k < a.K; k += kBlock) a.next_x[(size_t)b * a.next_stride + k] = bf2f(row[k]);
  }
  if (a.slow_table) {
    const uint16_t* row = a.slow_table + (size_t)min(max(code, 0), a.slow_rows - 1) * a.K;
    for (int k = tid; k < a.K; k += kBlock) a.slow_x[(size_t)b * a.K + k] = bf2f(row[k]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (a.copy_src[j]) {
      for (int k = tid; k < a.copy_n[j]; k += kBlock)
        a.copy_dst[j][(size_t)b * a.copy_dst_stride[j] + k] = a.copy_src[j][(size_t)b * a.copy_src_stride[j] + k];
    }
  }
  __syncthreads();
  if (a.pos_inc && tid == 0 && (!a.active || a.active[b])) a.pos_inc[b] = a.pos_inc[b] + 1;
}

__global__ void k_inc_rows(int* v, int n, const int* active) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n && (!active || active[i])) v[i] = v[i] + 1;
}

// one slot of a paged context: block-table row, positions, active flag
__global__ void k_slot_state(int* table, int* pos_s, int* pos_f, int* win_lo, int* active, SlotState st) {
  const int i = threadIdx.x;
  if (i < st.per_seq) table[(size_t)st.b * st.per_seq + i] = st.pages[i];
  if (i == 0 && st.set_state) {
    pos_s[st.b] = st.pos_slow;
    pos_f[st.b] = st.pos_frame;
    win_lo[st.b] = st.win_lo;
    active[st.b] = st.active;
  }
}

hipError_t gemm_dispatch(int wtype, const GemmArgs& a, int mt, dim3 grid, hipStream_t s) {
  if (wtype == W_INT4) {
    hipLaunchKernelGGL((k_gemm<INT4T, 1>), grid, dim3(kBlock), 0, s, a);
  } else if (wtype == W_INT8) {
    if (mt == 1 && a.cps <= kResidentChunks<INT8T>)
      hipLaunchKernelGGL((k_gemm_x<INT8T>), grid, dim3(kBlock), 0, s, a);
    else if (mt == 1)
      hipLaunchKernelGGL((k_gemm<INT8T, 1>), grid, dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm8<INT8T, 2>), grid, dim3(kWaves8 * kWave), 0, s, a);
  } else if (wtype == W_FP8) {
    if (mt == 1 && a.cps <= kResidentChunks<FP8T>)
      hipLaunchKernelGGL((k_gemm_x<FP8T>), grid, dim3(kBlock), 0, s, a);
    else if (mt == 1)
      hipLaunchKernelGGL((k_gemm<FP8T, 1>), grid, dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm8<FP8T, 2>), grid, dim3(kWaves8 * kWave), 0, s, a);
  } else {
    switch (mt) {
      case 1:
        if (a.cps <= kResidentChunks<BF16T>)
          hipLaunchKernelGGL((k_gemm_x<BF16T>), grid, dim3(kBlock), 0, s, a);
        else
          hipLaunchKernelGGL((k_gemm<BF16T, 1>), grid, dim3(kBlock), 0, s, a);
        break;
      case 2: hipLaunchKernelGGL((k_gemm8<BF16T, 2>), grid, dim3(kWaves8 * kWave), 0, s, a); break;
      default: hipLaunchKernelGGL((k_gemm8<BF16T, 4>), grid, dim3(kWaves8 * kWave), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

int gemm_mpad(int M) { return M <= 32 ? 32 : (M <= 64 ? 64 : ((M + 127) / 128) * 128); }

// input rows per workgroup / 32: the one-byte kernels (e4m3, int8) stage
// twice the input columns per chunk, so their LDS ring holds at most 64 input
// rows; int4 stages four times as many, so 32
static int gemm_mt(int wtype, int M) {
  const int mt = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  if (wtype == W_INT4) return 1;
  return (wtype != W_BF16 && mt > 2) ? 2 : mt;
}

// k per chunk of a weight type
static int gemm_kc(int wtype) {
  return wtype == W_BF16 ? kChunkK<BF16T> : (wtype == W_INT4 ? kChunkK<INT4T> : kChunkK<FP8T>);
}

// K splits: as many as keep the launch within one workgroup per CU (a
// workgroup's LDS ring and loads in flight are what stream the weights; a
// second one on a CU adds no bandwidth), each split at least one chunk; up
// to 32 rows, few enough chunks per split for the resident-input kernel
int gemm_splits(int wtype, int M, int N, int K) {
  const int mt = gemm_mt(wtype, M);
  const int tiles = ((N + kTileN - 1) / kTileN) * ((M + 32 * mt - 1) / (32 * mt));
  const int nchunks = K / gemm_kc(wtype);
  int splits = 256 / tiles;
  if (mt == 1 && wtype != W_INT4) {
    const int resident = wtype == W_BF16 ? kResidentChunks<BF16T> : kResidentChunks<FP8T>;
    splits = std::max(splits, (nchunks + resident - 1) / resident);
  }
  splits = splits < 1 ? 1 : (splits > nchunks ? nchunks : splits);
  const int cps = (nchunks + splits - 1) / splits;
  return (nchunks + cps - 1) / cps;
}

int gemm_launch_splits(int wtype, int M, int N, int K, size_t part_cap) {
  const int nchunks = K / gemm_kc(wtype);
  int splits = gemm_splits(wtype, M, N, K);
  while (splits > 1 && (size_t)splits * M * N > part_cap) --splits;
  const int cps = (nchunks + splits - 1) / splits;
  return (nchunks + cps - 1) / cps;
}

hipError_t launch_gemm(int wtype, GemmArgs a, size_t part_cap, hipStream_t s) {
  const int kc = gemm_kc(wtype);
  if (wtype == W_INT4 && !a.scale) return hipErrorInvalidValue;
  if (a.M < 1 || a.M > kPrefillRows || a.K < kc || a.K % kc || a.N < 1) return hipErrorInvalidValue;
  if (a.defer && (size_t)a.M * a.N > part_cap) return hipErrorInvalidValue;
  const int mt = gemm_mt(wtype, a.M);
  const int gx = (a.N + kTileN - 1) / kTileN, gy = (a.M + 32 * mt - 1) / (32 * mt);
  const int nchunks = a.K / kc;
  a.splits = gemm_launch_splits(wtype, a.M, a.N, a.K, part_cap);
  a.cps = (nchunks + a.splits - 1) / a.splits;
  const dim3 grid(gx, gy, a.splits);
  hipError_t e = gemm_dispatch(wtype, a, mt, grid, s);
  if (e != hipSuccess || a.splits == 1 || a.defer) return e;
  if (wtype == W_INT4) a.scale = nullptr;  // the partials carry the group scales
  const size_t total = (size_t)a.M * a.N;
  size_t blocks = (total + kBlock - 1) / kBlock;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_split(float* x, int x_stride, int M, int K, const uint16_t* gain, float eps, uint16_t* xh,
                             uint16_t* xl, hipStream_t s, float* out_f32, PartSum add) {
  if (K % 4 || K > 4 * kNormCols4 * kNormBlock || x_stride % 4 || (add.n > 0 && x_stride != K))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_norm_split, dim3(gemm_mpad(M)), dim3(kNormBlock), 0, s, x, x_stride, M, K, gain, eps, xh, xl,
                     out_f32, add);
  return hipGetLastError();
}

hipError_t launch_embed_rows(const uint16_t* table, int rows, int K, const int* tok, int M, float* x,
                             int* anomalies, hipStream_t s) {
  hipLaunchKernelGGL(k_embed_rows, dim3(M), dim3(kBlock), 0, s, table, rows, K, tok, x, anomalies);
  return hipGetLastError();
}

hipError_t launch_rope_rows(const float* qkv, int M, int p0, int n_heads_q, int n_heads_kv, int head_dim,
                            const float2* rope, float* q_out, uint16_t* kc, uint16_t* vc, int cache_len,
                            hipStream_t s, const int* row_pos, const int* row_seq, long long seq_stride,
                            PartSum src, PageMap pages) {
  if (head_dim / 2 > kWave) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rope_rows, dim3(M, n_heads_q + 2 * n_heads_kv), dim3(kWave), 0, s, qkv, src, M, p0, row_pos,
                     row_seq, seq_stride, n_heads_q, n_heads_kv, head_dim, rope, q_out, kc, vc, cache_len, pages);
  return hipGetLastError();
}

hipError_t launch_inc_rows(int* v, int n, hipStream_t s, const int* active) {
  hipLaunchKernelGGL(k_inc_rows, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, v, n, active);
  return hipGetLastError();
}

hipError_t launch_slot_state(int* table, int* pos_s, int* pos_f, int* win_lo, int* active, const SlotState& st,
                             hipStream_t s) {
  if (st.per_seq < 1 || st.per_seq > kMaxPagesPerSeq || st.b < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_slot_state, dim3(1), dim3(kMaxPagesPerSeq), 0, s, table, pos_s, pos_f, win_lo, active, st);
  return hipGetLastError();
}

hipError_t launch_commit_rows(const RowsCommitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_commit_rows, dim3(a.B), dim3(kBlock), a.smp.u ? sample_lds_bytes(a.V) : 0, s, a);
  return hipGetLastError();
}

hipError_t launch_silu_split(const float* a, const float* b, int M, int F, uint16_t* hh, uint16_t* hl,
                             hipStream_t s, PartSum pa, PartSum pb) {
  if (F % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_silu_split, dim3(gemm_mpad(M), (F + 4 * kBlock - 1) / (4 * kBlock)), dim3(kBlock), 0, s, a, b,
                     pa, pb, M, F, hh, hl);
  return hipGetLastError();
}

}  // namespace dar
