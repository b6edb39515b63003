// Sampling of one code by one workgroup of kBlock threads (device code shared
// by the decode commit and the batched commit). Steps, per the generation
// loop's top-p / top-k sampling with repetition windows (pyshine fish-speech
// tour, "Why You Need This"; the reading is stated with SampleArgs):
//   1. window codes marked in an LDS bitmap; each logit penalised if marked,
//      then divided by the temperature, and stored as an order-preserving key;
//   2. top-k: radix select of the k-th largest key, MSB first, 8 bits a pass
//      (integer histograms, so the result does not depend on thread timing);
//   3. the k candidates (larger keys, then equal keys by lower code) compacted
//      with block scans and sorted by (value desc, code asc) with a bitonic
//      network in LDS;
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
  const int tid = threadIdx.x;
  char* p = lds;
  uint32_t* keys = reinterpret_cast<uint32_t*>(p);
  p += ((size_t)V * 4 + 15) & ~(size_t)15;
  const int nwords = (V + 31) / 32;
  uint32_t* bits = reinterpret_cast<uint32_t*>(p);
  p += ((size_t)nwords * 4 + 15) & ~(size_t)15;
  int* hcount = reinterpret_cast<int*>(p);
  p += 256 * 4;
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
  for (int i = tid; i < V; i += kBlock) {
    float v = lg[i];
    if (v != v) v = -INFINITY;
    if ((bits[i >> 5] >> (i & 31)) & 1u) v = v > 0.f ? v / sp.penalty : v * sp.penalty;
    keys[i] = sample_key(v / sp.temperature);
  }
  __syncthreads();

  // 2. the k-th largest key: digit by digit from the top, `want` = how many of
  // the keys matching the digits so far are still to be taken
  const int k = min(sp.top_k, V);
  uint32_t prefix = 0u, mask = 0u;
  int want = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hcount[tid] = 0;
    __syncthreads();
    for (int i = tid; i < V; i += kBlock) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hcount[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    // thread t looks at digit 255 - t: the keys above it are the scan's prefix
    const int c = hcount[255 - tid];
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
  // (lowest codes first); thread t scans codes [t per, (t + 1) per)
  const uint32_t T = prefix;
  const int per = (V + kBlock - 1) / kBlock;
  const int i0 = min(tid * per, V), i1 = min(i0 + per, V);
  int ngt = 0, neq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    ngt += key > T;
    neq += key == T;
  }
  int tot_gt, tot_eq;
  int off_gt = sample_scan_excl(ngt, red, &tot_gt);
  int off_eq = sample_scan_excl(neq, red, &tot_eq);
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    int slot = -1;
    if (key > T) {
      slot = off_gt++;
    } else if (key == T) {
      if (off_eq < want) slot = tot_gt + off_eq;
      ++off_eq;
    }
    // ascending order of (~key, code) = descending value, ascending code
    if (slot >= 0) cand[slot] = ((unsigned long long)(~key) << 32) | (unsigned long long)(uint32_t)i;
  }
  if (tid >= k) cand[tid] = ~0ull;
  __syncthreads();
  for (int size = 2; size <= kMaxTopK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int j = tid ^ stride;
      if (j > tid) {
        const unsigned long long a = cand[tid], b = cand[j];
        if ((a > b) == ((tid & size) == 0)) {
          cand[tid] = b;
          cand[j] = a;
        }
      }
      __syncthreads();
    }
  }

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
