// Workgroup-level exact selection primitives (LDS radix select, threshold bins).
#pragma once

#include "common.hpp"

namespace idxtopk {

// LDS scratch for wg_radix_select: 256 histogram bins + 4 broadcast words.
struct SelectLds {
  uint32_t hist[256];
  uint32_t bcast[4];
};

// Exact k-th largest of a set of DISTINCT 64-bit keys spread over the
// workgroup. `for_each(f)` must call f(key) once for every key this thread
// owns, the same set on every call. Precondition: the set holds more than k
// keys, and k >= 1.
//
// Returns T such that exactly k keys are >= T (T is the shortest digit prefix
// that separates them, so it need not be one of the keys). MSB-first radix
// select over 8-bit digits: each pass histograms the keys that still match
// the prefix, then finds the digit where the count from the top reaches the
// remaining rank. Stops as soon as the keys matching the prefix are exactly
// the ones still needed.
template <int WG, class ForEach>
__device__ uint64_t wg_radix_select(ForEach&& for_each, uint32_t k, SelectLds& s) {
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  uint64_t prefix = 0, mask = 0;
  uint32_t kk = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += WG) s.hist[i] = 0;
    __syncthreads();
    for_each([&](uint64_t key) {
      if ((key & mask) == prefix) atomicAdd(&s.hist[(key >> shift) & 0xffu], 1u);
    });
    __syncthreads();
    if (wave == 0) {
      const uint32_t c0 = s.hist[4 * lane + 0], c1 = s.hist[4 * lane + 1];
      const uint32_t c2 = s.hist[4 * lane + 2], c3 = s.hist[4 * lane + 3];
      const uint32_t incl = wave_suffix_sum(c0 + c1 + c2 + c3);
      const uint32_t above_lane = incl - (c0 + c1 + c2 + c3);  // keys in bins of higher lanes
      if (above_lane < kk && incl >= kk) {
        uint32_t above = above_lane;
        uint32_t c[4] = {c0, c1, c2, c3};
        int d = 3;
        for (; d > 0; --d) {
          if (above + c[d] >= kk) break;
          above += c[d];
        }
        s.bcast[0] = 4 * lane + d;
        s.bcast[1] = above;
        s.bcast[2] = c[d];
      }
    }
    __syncthreads();
    const uint32_t d = s.bcast[0], above = s.bcast[1], cnt = s.bcast[2];
    kk -= above;
    prefix |= static_cast<uint64_t>(d) << shift;
    mask |= 0xffull << shift;
    if (cnt == kk) break;
  }
  __syncthreads();
  return prefix;
}

// Threshold bin of a histogram for rank k: the highest bin b with
// sum(bins >= b) >= k. Returns above = sum(bins > b) and the total count.
// When total < k, returns bin 0 with all=true (everything is selected).
struct BinThreshold {
  uint32_t bin;
  uint32_t above;
  uint32_t total;
  bool all;
};

// `load(i)` returns the count of bin i (0 <= i < NBINS). Every thread of the
// workgroup must call this. Uses `scratch` (LDS, >= WG/64 + 4 words).
template <int WG, int NBINS, class Load>
__device__ BinThreshold wg_threshold_bin(Load&& load, uint32_t k, uint32_t* scratch) {
  static_assert(NBINS % WG == 0, "bins per thread");
  constexpr int PER = NBINS / WG;
  constexpr int NW = WG / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  // thread t owns bins [t*PER, (t+1)*PER)
  uint32_t c[PER];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = load(tid * PER + i);
    local += c[i];
  }
  const uint32_t incl_w = wave_suffix_sum(local);  // within wave, lanes >= lane
  if (lane == 0) scratch[wave] = incl_w;            // wave total
  __syncthreads();
  uint32_t higher_waves = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = scratch[w];
    total += t;
    if (w > wave) higher_waves += t;
  }
  const uint32_t incl = incl_w + higher_waves;  // bins of threads >= tid
  const uint32_t above_t = incl - local;
  __syncthreads();
  if (total >= k && above_t < k && incl >= k) {
    uint32_t above = above_t;
    int i = PER - 1;
    for (; i > 0; --i) {
      if (above + c[i] >= k) break;
      above += c[i];
    }
    scratch[NW + 0] = tid * PER + i;
    scratch[NW + 1] = above;
  }
  __syncthreads();
  BinThreshold r;
  r.total = total;
  if (total < k) {
    r.bin = 0;
    r.above = 0;
    r.all = true;
  } else {
    r.bin = scratch[NW + 0];
    r.above = scratch[NW + 1];
    r.all = false;
  }
  __syncthreads();
  return r;
}

}  // namespace idxtopk
