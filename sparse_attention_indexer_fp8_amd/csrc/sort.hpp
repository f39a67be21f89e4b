// Workgroup bitonic sort of 64-bit keys into descending order.
//
// The network is the uniform-direction form of the bitonic sort: merging two
// sorted blocks of size/2 into one of `size` first compares element i with
// its mirror i ^ (size - 1), then runs half-cleaners at strides size/4 .. 1
// (i against i ^ stride); every comparison puts the larger key at the lower
// index, so no step needs a direction. Thread t holds logical elements
// t*E .. t*E + E - 1 in registers. Steps whose partner is in the same thread
// are register compare-exchanges, partners in the same wave come by
// ds_bpermute (all of a step's shuffles issued before any result is used),
// and partners in another wave go through LDS.
#pragma once

#include "common.hpp"

namespace idxtopk {

// larger key to a, smaller to b
__device__ __forceinline__ void ce_desc(uint64_t& a, uint64_t& b) {
  const bool sw = a < b;
  const uint64_t x = a;
  a = sw ? b : a;
  b = sw ? x : b;
}

// the larger of x, y on the lower index of a pair, the smaller on the upper
__device__ __forceinline__ uint64_t keep_side(uint64_t x, uint64_t y, bool lower) {
  return (x > y) == lower ? x : y;
}

// y[e] = partner thread's r[MIRROR ? E - 1 - e : e], partner = tid ^ m
// (m < 64: the partner is in this wave).
template <int E, bool MIRROR>
__device__ __forceinline__ void xchg_wave(const uint64_t (&r)[E], uint64_t (&y)[E], int m) {
  const int addr = (static_cast<int>(lane_id()) ^ m) << 2;
  uint32_t lo[E], hi[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t v = r[MIRROR ? E - 1 - e : e];
    lo[e] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(static_cast<uint32_t>(v))));
    hi[e] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(static_cast<uint32_t>(v >> 32))));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = (static_cast<uint64_t>(hi[e]) << 32) | lo[e];
}

// The same through LDS (xs holds WG * E keys, element-major so that a wave's
// accesses are contiguous). Every thread of the workgroup must call.
template <int WG, int E, bool MIRROR>
__device__ __forceinline__ void xchg_lds(const uint64_t (&r)[E], uint64_t (&y)[E], int m, uint64_t* xs) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < E; ++e) xs[e * WG + tid] = r[e];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = xs[(MIRROR ? E - 1 - e : e) * WG + (tid ^ m)];
  __syncthreads();
}

template <int WG, int E, bool MIRROR>
__device__ __forceinline__ void cross_step(uint64_t (&r)[E], int m, bool lower, uint64_t* xs) {
  uint64_t y[E];
  if (m < kWave)
    xchg_wave<E, MIRROR>(r, y, m);
  else
    xchg_lds<WG, E, MIRROR>(r, y, m, xs);
#pragma unroll
  for (int e = 0; e < E; ++e) r[e] = keep_side(r[e], y[e], lower);
}

// half-cleaners at strides E/2 .. 1 inside the thread
template <int E>
__device__ __forceinline__ void thread_clean(uint64_t (&r)[E]) {
#pragma unroll
  for (int stride = E / 2; stride > 0; stride >>= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (!(e & stride)) ce_desc(r[e], r[e | stride]);
  }
}

// Sorts the WG * E keys held in r (any placement) so that thread t ends with
// the keys of ranks t*E .. t*E + E - 1 in r[0 .. E). xs: LDS scratch of
// WG * E keys (unused when WG <= 64). Every thread of the workgroup calls.
template <int WG, int E>
__device__ __forceinline__ void block_sort_desc(uint64_t (&r)[E], uint64_t* xs) {
  // blocks of up to E elements: inside the thread
#pragma unroll
  for (int size = 2; size <= E; size <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int p = e ^ (size - 1);
      if (e < p) ce_desc(r[e], r[p]);
    }
#pragma unroll
    for (int stride = size / 4; stride > 0; stride >>= 1) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (!(e & stride)) ce_desc(r[e], r[e | stride]);
    }
  }
  const int base = static_cast<int>(threadIdx.x) * E;
  for (int size = 2 * E; size <= WG * E; size <<= 1) {
    cross_step<WG, E, true>(r, size / E - 1, (base & (size >> 1)) == 0, xs);
    for (int stride = size >> 2; stride >= E; stride >>= 1)
      cross_step<WG, E, false>(r, stride / E, (base & stride) == 0, xs);
    thread_clean<E>(r);
  }
}

}  // namespace idxtopk
