// Sampling of one code by one workgroup of kBlock threads (device code shared
// by the decode commit and the batched commit). Steps, per the generation
// loop's top-p / top-k sampling with repetition windows (pyshine fish-speech
// tour, "Why You Need This"; the reading is stated with SampleArgs):
//   1. window codes marked in an LDS bitmap; each logit penalised if marked,
//      then divided by the temperature, and kept as an order-preserving key in
//      registers (thread t owns the contiguous codes [t per, (t + 1) per));
//   2. top-k: radix select of the k-th largest key, MSB first, 8 bits a pass
//      (integer histograms, one per wave so that keys sharing their top byte
//      spread their LDS atomics; the result does not depend on thread timing);
//   3. the k candidates (larger keys, then equal keys by lower code) compacted
//      with block scans and sorted by (value desc, code asc) with a bitonic
//      network, one element per thread: lane shuffles within a wave, LDS and
//      a barrier only for the strides of 64 and 128;
//   4. exp(v - vmax) per candidate, a block scan for the running sums, then
//      the top-p cut and the draw as counts over the running sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dar_internal.h"

namespace dar {

__device__ __forceinline__ uint32_t sample_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float sample_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// exclusive prefix sum over the block's threads (thread order); *total = the sum
__device__ __forceinline__ int sample_scan_excl(int v, int* red, int* total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) red[wave] = x;
  __syncthreads();
  int base = 0, t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    base += w < wave ? red[w] : 0;
    t += red[w];
  }
  __syncthreads();
  *total = t;
  return base + x - v;
}

// inclusive prefix sum of floats over the block's threads
__device__ __forceinline__ float sample_scan_incl(float v, float* red) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) red[wave] = x;
  __syncthreads();
  float base = 0.f;
  for (int w = 0; w < wave; ++w) base += red[w];
  __syncthreads();
  return base + x;
}

// The sampled code of logits lg[0..V) with draw u; hist[i * hist_stride],
// i < nh, are the window's codes. Every thread returns the code. lds holds
// sample_lds_bytes(V) bytes. Needs 1 <= top_k <= kMaxTopK, V <= kMaxSampleVocab.
__device__ __forceinline__ int sample_row(const float* lg, int V, const SampleArgs& sp, float u, const int* hist,
                                          long long hist_stride, int nh, char* lds) {
  static_assert(kBlock == 256 && kMaxTopK == kBlock, "one candidate per thread, one histogram bin per thread");
  constexpr int kPer = kMaxSampleVocab / kBlock;  // codes per thread at most
  const int tid = threadIdx.x;
  char* p = lds;
  const int nwords = (V + 31) / 32;
  uint32_t* bits = reinterpret_cast<uint32_t*>(p);
  p += ((size_t)nwords * 4 + 15) & ~(size_t)15;
  int* hcount = reinterpret_cast<int*>(p);  // [kWaves][256]
  p += kWaves * 256 * 4;
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(p);
  p += (size_t)kMaxTopK * 8;
  float* cum = reinterpret_cast<float*>(p);
  p += 256 * 4;
  int* red = reinterpret_cast<int*>(p);         // kWaves ints of scan scratch
  float* redf = reinterpret_cast<float*>(p + 32);
  int* bcast = reinterpret_cast<int*>(p + 64);  // digit, count above

  // 1. window bitmap, penalty, temperature, keys
  for (int i = tid; i < nwords; i += kBlock) bits[i] = 0u;
  __syncthreads();
  for (int i = tid; i < nh; i += kBlock) {
    const int c = hist[(long long)i * hist_stride];
    if (c >= 0 && c < V) atomicOr(&bits[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  const int per = (V + kBlock - 1) / kBlock;
  const int i0 = min(tid * per, V), n_own = min(per, V - i0);
  uint32_t kr[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    kr[j] = 0u;
    if (j < n_own) {
      const int i = i0 + j;
      float v = lg[i];
      if (v != v) v = -INFINITY;
      if ((bits[i >> 5] >> (i & 31)) & 1u) v = v > 0.f ? v / sp.penalty : v * sp.penalty;
      kr[j] = sample_key(v / sp.temperature);
    }
  }

  // 2. the k-th largest key: digit by digit from the top, `want` = how many of
  // the keys matching the digits so far are still to be taken
  const int k = min(sp.top_k, V);
  uint32_t prefix = 0u, mask = 0u;
  int want = k;
  int* hwave = hcount + (tid / kWave) * 256;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) hcount[w * 256 + tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < n_own && (kr[j] & mask) == prefix) atomicAdd(&hwave[(kr[j] >> shift) & 255u], 1);
    __syncthreads();
    // thread t looks at digit 255 - t: the keys above it are the scan's prefix
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c += hcount[w * 256 + 255 - tid];
    int tot;
    const int above = sample_scan_excl(c, red, &tot);
    if (above < want && above + c >= want) {
      bcast[0] = 255 - tid;
      bcast[1] = above;
    }
    __syncthreads();
    const int d = bcast[0];
    want -= bcast[1];
    prefix |= (uint32_t)d << shift;
    mask |= 0xffu << shift;
    __syncthreads();
  }

  // 3. candidates: the keys above the threshold, then `want` keys equal to it
  // (lowest codes first)
  const uint32_t T = prefix;
  int ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (j < n_own) {
      ngt += kr[j] > T;
      neq += kr[j] == T;
    }
  }
  int tot_gt, tot_eq;
  int off_gt = sample_scan_excl(ngt, red, &tot_gt);
  int off_eq = sample_scan_excl(neq, red, &tot_eq);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (j >= n_own) continue;
    const uint32_t key = kr[j];
    int slot = -1;
    if (key > T) {
      slot = off_gt++;
    } else if (key == T) {
      if (off_eq < want) slot = tot_gt + off_eq;
      ++off_eq;
    }
    // ascending order of (~key, code) = descending value, ascending code
    if (slot >= 0) cand[slot] = ((unsigned long long)(~key) << 32) | (unsigned long long)(uint32_t)(i0 + j);
  }
  if (tid >= k) cand[tid] = ~0ull;
  __syncthreads();
  // ascending sort, element tid in a register: at each compare-exchange the
  // lower element of a pair keeps the minimum when its block of `size` runs up
  unsigned long long x = cand[tid];
  for (int size = 2; size <= kMaxTopK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      unsigned long long y;
      if (stride >= kWave) {
        __syncthreads();  // every lane's previous value read
        cand[tid] = x;
        __syncthreads();
        y = cand[tid ^ stride];
      } else {
        y = __shfl_xor(x, stride);
      }
      const bool keep_min = ((tid & stride) == 0) == ((tid & size) == 0);
      x = keep_min ? (x < y ? x : y) : (x < y ? y : x);
    }
  }
  __syncthreads();
  cand[tid] = x;
  __syncthreads();

  // 4. probabilities, running sums, top-p cut, draw
  const bool valid = tid < k;
  const float vmax = sample_value(~(uint32_t)(cand[0] >> 32));
  const float w = valid ? expf(sample_value(~(uint32_t)(cand[tid] >> 32)) - vmax) : 0.f;
  const float run = sample_scan_incl(w, redf);
  cum[tid] = run;
  __syncthreads();
  const float total = cum[k - 1];
  const float thr = sp.top_p * total;
  const int before_cut = __syncthreads_count(valid && run < thr);
  const int m = min(before_cut + 1, k);
  const float target = u * cum[m - 1];
  const int pick = min(__syncthreads_count(tid < m && run <= target), m - 1);
  return (int)(uint32_t)(cand[pick] & 0xffffffffull);
}

}  // namespace dar
