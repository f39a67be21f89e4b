// Workgroup-level exact selection primitives (adaptive-bin select, threshold bins).
#pragma once

#include "common.hpp"

namespace idxtopk {

// ---------------------------------------------------------------------------
// Exact selection over distinct 64-bit keys
// ---------------------------------------------------------------------------

constexpr int kSelBins = 1024;    // histogram bins of one select iteration
constexpr int kSelMembers = 64;   // threshold-bin size a single wave resolves

// LDS state of wg_select. `hist` and `mcnt` must be zero when a select starts
// (wg_select_init once per kernel) and every select leaves them zero again.
// Bin b lives at word sel_slot(b): the 16 bins lane l of wave 0 scans
// (16 l .. 16 l + 15) then sit in 16 rows of 64 consecutive words, one per
// lane, so the scan reads and clears without bank conflicts.
struct SelectLds {
  alignas(16) uint32_t hist[kSelBins];  // wave_select clears it 16 bytes per lane
  uint64_t red[2][16];
  uint64_t members[kSelMembers];
  uint64_t result;
  uint32_t bcast[4];
  uint32_t mcnt;
};

static_assert(kSelBins == 16 * kWave, "sel_slot assumes 16 bins per lane of one wave");
__device__ __forceinline__ uint32_t sel_slot(uint32_t bin) { return ((bin & 15u) << 6) | (bin >> 4); }

template <int WG>
__device__ __forceinline__ void wg_select_init(SelectLds& s) {
  for (int i = threadIdx.x; i < kSelBins; i += WG) s.hist[i] = 0;
  if (threadIdx.x == 0) s.mcnt = 0;
}

// Calls f(buf[i]) for i = tid, tid + WG, ... below n, CH loads in flight per
// thread: the loads of a chunk are issued together (an index past n re-reads
// the chunk's first entry, which is in range) before any is used.
template <int WG, int CH, class F>
__device__ __forceinline__ void lds_for_each(const uint64_t* buf, uint32_t n, F&& f) {
  for (uint32_t b = threadIdx.x; b < n; b += CH * WG) {
    uint64_t x[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t i = b + j * WG;
      x[j] = buf[i < n ? i : b];
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (b + j * WG < n) f(x[j]);
  }
}

// Workgroup min and max of per-thread values (one barrier). Every thread
// gets the results.
template <int WG>
__device__ __forceinline__ void wg_range(uint64_t& mn, uint64_t& mx, SelectLds& s) {
  constexpr int NW = WG / kWave;
  const int wave = threadIdx.x / kWave;
  mn = wave_min_u64(mn);
  mx = wave_max_u64(mx);
  if (lane_id() == 0) {
    s.red[0][wave] = mn;
    s.red[1][wave] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint64_t a = s.red[0][w], b = s.red[1][w];
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
}

// Pick from the kSelBins histogram in s.hist (every thread has added its
// counts; the call starts with the barrier that completes them): the highest
// bin b whose count from the top reaches kk (which the total must). Returns
// b, the count above it and its own count, and leaves the histogram zeroed.
// Wave 0 alone reads (16 bins per lane, conflict-free through sel_slot),
// clears and scans.
struct HistPick {
  uint32_t bin;
  uint32_t above;
  uint32_t cnt;
};

template <int WG>
__device__ __forceinline__ HistPick wg_hist_pick(uint32_t kk, SelectLds& s) {
  constexpr int PL = kSelBins / kWave;  // bins per lane of wave 0
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = lane_id();
    uint32_t c[PL];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      c[i] = s.hist[i * kWave + lane];  // bin lane * PL + i
      local += c[i];
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) s.hist[i * kWave + lane] = 0;
    const uint32_t pre = wave_prefix_incl(local);
    const uint32_t tot = __builtin_amdgcn_readlane(pre, kWave - 1);
    const uint32_t incl = tot - pre + local;  // bins of lanes >= lane
    const uint32_t above_l = incl - local;
    if (above_l < kk && incl >= kk) {
      uint32_t above = above_l;
      int i = PL - 1;
      for (; i > 0; --i) {
        if (above + c[i] >= kk) break;
        above += c[i];
      }
      s.bcast[0] = lane * PL + i;
      s.bcast[1] = above;
      s.bcast[2] = c[i];
    }
  }
  __syncthreads();
  return HistPick{s.bcast[0], s.bcast[1], s.bcast[2]};
}

// k-th largest of a set of DISTINCT 64-bit keys spread over the workgroup,
// all within [lo, hi] (wg_range gives these). `for_each(f)` must call f(key)
// once for every key this thread owns, the same set on every call.
// Precondition: the set holds more than k keys, k >= 1.
//
// Returns T such that exactly k keys are >= T. With slack > 0 it may stop
// earlier, at a bound T with k <= (keys >= T) <= k + slack: it stops as soon
// as the keys in and above the current range are few enough (slack = ~0u
// stops after the first histogram).
//
// Method: each iteration histograms the undecided keys into kSelBins equal
// bins covering exactly their range [lo, hi], so they spread over many bins
// whatever their magnitude. The bin where the count from the top reaches the
// remaining rank becomes the new range, and the keys above it are decided.
// The loop ends when the bin's keys are exactly the ones still needed. When
// the bin holds at most 64 keys, wave 0 instead ranks them against each other
// by broadcast. Each iteration shrinks the range by a factor of kSelBins, so
// at most 7 run; one or two are typical.
template <int WG, class ForEach>
__device__ __forceinline__ uint64_t wg_select(ForEach&& for_each, uint32_t k, uint64_t lo, uint64_t hi, SelectLds& s,
                              uint32_t slack = 0) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  uint32_t kk = k;
  for (int it = 0; it < 8; ++it) {
    const uint64_t span = hi - lo;
    if (span == 0) break;  // one key left, and it is the k-th
    const int bits = 64 - __clzll(span);
    const int shift = bits > 10 ? bits - 10 : 0;
    for_each([&](uint64_t key) {
      if (key >= lo && key <= hi) atomicAdd(&s.hist[sel_slot(static_cast<uint32_t>((key - lo) >> shift))], 1u);
    });
    const HistPick p = wg_hist_pick<WG>(kk, s);
    const uint32_t cnt = p.cnt;
    kk -= p.above;
    lo += static_cast<uint64_t>(p.bin) << shift;
    const uint64_t top = lo + ((1ull << shift) - 1ull);
    hi = top < hi ? top : hi;
    if (cnt - kk <= slack) break;  // keys >= lo: (k - kk) + cnt
    if (cnt <= static_cast<uint32_t>(kSelMembers)) {
      // few keys left: gather them and let one wave rank them
      const uint64_t blo = lo, bhi = hi;
      for_each([&](uint64_t key) {
        if (key >= blo && key <= bhi) s.members[atomicAdd(&s.mcnt, 1u)] = key;
      });
      __syncthreads();
      if (wave == 0) {
        const uint64_t m = lane < static_cast<int>(cnt) ? s.members[lane] : 0ull;
        uint32_t rank = 0;  // members greater than m
        for (uint32_t j = 0; j < cnt; ++j) {
          const uint32_t olo = __builtin_amdgcn_readlane(static_cast<uint32_t>(m), j);
          const uint32_t ohi = __builtin_amdgcn_readlane(static_cast<uint32_t>(m >> 32), j);
          rank += ((static_cast<uint64_t>(ohi) << 32) | olo) > m;
        }
        if (lane < static_cast<int>(cnt) && rank == kk - 1) s.result = m;
        if (lane == 0) s.mcnt = 0;
      }
      __syncthreads();
      lo = s.result;
      break;
    }
  }
  return lo;
}

// k-th largest of at most PER * 64 DISTINCT 64-bit keys held by one wave
// (key[e] counts where valid[e]), with 1 <= k < the number of keys: returns
// T such that exactly k keys are >= T. Wave-synchronous, no workgroup
// barrier: `hist` is 256 words of LDS that only this wave uses.
//
// Method as wg_select's, with 256 bins per round: histogram the keys in
// [lo, hi] into 256 equal bins, find the bin where the count from the top
// reaches the remaining rank, narrow [lo, hi] to it. Each round shrinks the
// range by 2^8, so at most 8 rounds run on 64-bit keys. The wave's LDS
// operations complete in order, so no barrier separates the rounds.
template <int PER>
__device__ __forceinline__ uint64_t wave_select(const uint64_t (&key)[PER], const bool (&valid)[PER], uint32_t k,
                                                uint32_t* hist) {
  const int lane = lane_id();
  uint64_t lo = ~0ull, hi = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (valid[e]) {
      lo = key[e] < lo ? key[e] : lo;
      hi = key[e] > hi ? key[e] : hi;
    }
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  uint32_t kk = k;
  for (int it = 0; it < 8; ++it) {
    const uint64_t span = hi - lo;
    if (span == 0) break;  // one key left, and it is the k-th
    const int bits = 64 - __clzll(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (valid[e] && key[e] >= lo && key[e] <= hi) atomicAdd(&hist[static_cast<uint32_t>((key[e] - lo) >> shift)], 1u);
    const uint4 c4 = reinterpret_cast<const uint4*>(hist)[lane];  // bins 4 lane .. 4 lane + 3
    const uint32_t c[4] = {c4.x, c4.y, c4.z, c4.w};
    const uint32_t local = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_prefix_incl(local);
    const uint32_t tot = __builtin_amdgcn_readlane(incl, kWave - 1);
    const uint32_t above_l = tot - incl;  // keys in the bins of higher lanes
    // the lane whose bins hold the kk-th key from the top
    const bool mine = above_l < kk && above_l + local >= kk;
    uint32_t bin = 0, above = above_l, cnt = 0;
    if (mine) {
      int i = 3;
      for (; i > 0; --i) {
        if (above + c[i] >= kk) break;
        above += c[i];
      }
      bin = 4 * lane + i;
      cnt = c[i];
    }
    const int src = __builtin_ctzll(ballot(mine));
    bin = __builtin_amdgcn_readlane(bin, src);
    above = __builtin_amdgcn_readlane(above, src);
    cnt = __builtin_amdgcn_readlane(cnt, src);
    kk -= above;
    lo += static_cast<uint64_t>(bin) << shift;
    const uint64_t top = lo + ((1ull << shift) - 1ull);
    hi = top < hi ? top : hi;
    if (cnt == kk) break;  // every key of the bin is taken: keys >= lo are exactly k
  }
  return lo;
}

// A lower bound T for the rank-th largest of at most PER * 64 32-bit keys
// held by one wave (key[e] counts where valid[e]; 1 <= rank <= their
// number): at least `rank` keys are >= T, and at most rank + slack unless
// two rounds were not enough to narrow it. Each round histograms the keys
// of the current range [lo, hi] into 256 equal bins (the `hist` words of
// LDS that only this wave uses) and keeps the bin where the count from the
// top reaches the remaining rank; T is that bin's lower edge. Wave-
// synchronous, no barrier (the wave's LDS operations complete in order).
template <int PER>
__device__ __forceinline__ uint32_t wave_lower_bound(const uint32_t (&key)[PER], const bool (&valid)[PER],
                                                     uint32_t rank, uint32_t slack, uint32_t* hist) {
  const int lane = lane_id();
  uint32_t lo = ~0u, hi = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (valid[e]) {
      lo = key[e] < lo ? key[e] : lo;
      hi = key[e] > hi ? key[e] : hi;
    }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  uint32_t kk = rank;
  for (int it = 0; it < 2; ++it) {
    const uint32_t span = hi - lo;
    if (span == 0u) break;
    const int bits = 32 - __clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (valid[e] && key[e] >= lo && key[e] <= hi) atomicAdd(&hist[(key[e] - lo) >> shift], 1u);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const uint4 c4 = reinterpret_cast<const uint4*>(hist)[lane];  // bins 4 lane .. 4 lane + 3
    const uint32_t c[4] = {c4.x, c4.y, c4.z, c4.w};
    const uint32_t local = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_prefix_incl(local);
    const uint32_t tot = __builtin_amdgcn_readlane(incl, kWave - 1);
    const uint32_t above_l = tot - incl;  // keys in the bins of higher lanes
    const bool mine = above_l < kk && above_l + local >= kk;
    uint32_t bin = 0, above = above_l, cnt = 0;
    if (mine) {
      int i = 3;
      for (; i > 0; --i) {
        if (above + c[i] >= kk) break;
        above += c[i];
      }
      bin = 4 * lane + i;
      cnt = c[i];
    }
    const int src = __builtin_ctzll(ballot(mine));
    bin = __builtin_amdgcn_readlane(bin, src);
    above = __builtin_amdgcn_readlane(above, src);
    cnt = __builtin_amdgcn_readlane(cnt, src);
    kk -= above;
    lo += bin << shift;
    const uint32_t top = lo + ((1u << shift) - 1u);
    hi = top < hi ? top : hi;
    if (cnt - kk <= slack) break;  // keys >= lo: (rank - kk) + cnt
  }
  return lo;
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

// Threshold bin from counts already in registers: thread t holds the counts
// of bins [t * PER, (t + 1) * PER) in c[]. Every thread of the workgroup must
// call this. Uses `scratch` (LDS, >= WG/64 + 4 words).
template <int WG, int PER>
__device__ BinThreshold wg_threshold_counts(const uint32_t (&c)[PER], uint32_t k, uint32_t* scratch) {
  constexpr int NW = WG / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += c[i];
  const uint32_t pre = wave_prefix_incl(local);
  const uint32_t wtot = __builtin_amdgcn_readlane(pre, kWave - 1);
  const uint32_t incl_w = wtot - pre + local;  // within wave, lanes >= lane
  if (lane == 0) scratch[wave] = wtot;         // wave total
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

// `load(i)` returns the count of bin i (0 <= i < NBINS); all of a thread's
// loads are issued before any count is used. Every thread of the workgroup
// must call this. Uses `scratch` (LDS, >= WG/64 + 4 words).
template <int WG, int NBINS, class Load>
__device__ BinThreshold wg_threshold_bin(Load&& load, uint32_t k, uint32_t* scratch) {
  static_assert(NBINS % WG == 0, "bins per thread");
  constexpr int PER = NBINS / WG;
  // thread t owns bins [t*PER, (t+1)*PER)
  uint32_t c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) c[i] = load(static_cast<int>(threadIdx.x) * PER + i);
  return wg_threshold_counts<WG, PER>(c, k, scratch);
}

}  // namespace idxtopk
