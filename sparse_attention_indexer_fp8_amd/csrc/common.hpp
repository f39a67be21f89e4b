// Shared device helpers for libidxtopk (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxtopk {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Checked builds (IDXTOPK_CHECKS=1, libidxtopk_checked.so): device-side
// checks of the callers' preconditions and of internal bounds. A failed
// check sets its bit in this source file's error word (one word per source
// file: each is its own code object), which idxtopk_check_status reads;
// the kernels then carry on exactly as a release build does. In a release
// build a check compiles to nothing and its arguments are not evaluated.
// ---------------------------------------------------------------------------
#ifndef IDXTOPK_CHECKS
#define IDXTOPK_CHECKS 0
#endif

constexpr uint32_t kChkWindow = 1u << 0;        // topk_rows: a window outside its buffer row
constexpr uint32_t kChkCandOverflow = 1u << 1;  // topk_rows: candidate buffer overrun
constexpr uint32_t kChkPosition = 1u << 2;      // a selected position outside its row, before the lookup
constexpr uint32_t kChkSeqLen = 1u << 3;        // seq_lens[b] < 0 or above max_seq_len
constexpr uint32_t kChkRowToBatch = 1u << 4;    // row_to_batch[b] < 0
constexpr uint32_t kChkPageId = 1u << 5;        // a block-table or page-table entry < 0
constexpr uint32_t kChkChunkCount = 1u << 6;    // fused: a chunk header's count above the chunk's tokens
constexpr uint32_t kChkBlock = 1u << 7;         // block top-k: a selected block outside the row
constexpr uint32_t kChkMergeCount = 1u << 8;    // fused merge: histogram or threshold sub-bin counts inconsistent

#if IDXTOPK_CHECKS
static __device__ uint32_t g_check_word;
__device__ __forceinline__ void check_failed(uint32_t bit) { atomicOr(&g_check_word, bit); }
#define IDXTOPK_CHECK(ok, bit)                  \
  do {                                          \
    if (!(ok)) ::idxtopk::check_failed((bit));  \
  } while (0)
// This source file's error word (host side; synchronous), cleared if asked.
static inline uint32_t read_check_word(bool clear) {
  uint32_t v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_word), sizeof(v)) != hipSuccess) return 0xffffffffu;
  if (clear) {
    const uint32_t z = 0;
    (void)hipMemcpyToSymbol(HIP_SYMBOL(g_check_word), &z, sizeof(z));
  }
  return v;
}
#else
#define IDXTOPK_CHECK(ok, bit) ((void)0)
#endif

// ---------------------------------------------------------------------------
// Ordered keys
// ---------------------------------------------------------------------------

// Order-preserving map from an fp32 value to uint32: a larger float gives a
// larger key, -0.0 and +0.0 give the same key (they tie), denormals keep their
// order, and +-inf sit at the ends of the finite range.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t mag = u & 0x7fffffffu;
  return (u >> 31) ? (0x80000000u - mag) : (0x80000000u + mag);
}

// Inverse of float_key (zero comes back as +0.0).
__device__ __forceinline__ float key_float(uint32_t key) {
  return (key >= 0x80000000u) ? __uint_as_float(key - 0x80000000u)
                              : __uint_as_float((0x80000000u - key) | 0x80000000u);
}

// Total order used by every selection: value first, then the lower position
// wins. The 64-bit key is unique per position, so "the k largest keys" is
// exactly the top-k with ties resolved toward the lower position.
__device__ __forceinline__ uint64_t rank_key(uint32_t vkey, uint32_t pos) {
  return (static_cast<uint64_t>(vkey) << 32) | static_cast<uint32_t>(~pos);
}
__device__ __forceinline__ uint32_t rank_pos(uint64_t key) {
  return ~static_cast<uint32_t>(key);
}
__device__ __forceinline__ uint32_t rank_vkey(uint64_t key) {
  return static_cast<uint32_t>(key >> 32);
}

// ---------------------------------------------------------------------------
// Division by a runtime-invariant divisor (numerators below 2^31)
// Granlund & Montgomery, "Division by invariant integers using
// multiplication" (PLDI 1994): q = (umulhi(n, m) + n) >> l with
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1.
// ---------------------------------------------------------------------------
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1ull;
  return FastDiv{d, static_cast<uint32_t>(m), l};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.l;
}

// Load of a uniform address through the scalar unit (constant address space).
// Only for data no kernel of the launch writes (row metadata, tables).
template <class T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// ---------------------------------------------------------------------------
// Wave helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// s_waitcnt vmcnt(0): wait until every vector memory operation of the wave
// has completed (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and
// lgkmcnt 11:8 left at their maximum). A loop that streams loads ahead must
// not carry a store into its next iteration: loads and stores share this
// counter and complete out of order with respect to each other, so the
// compiler would then wait for every load in flight before the next use.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Inclusive prefix sum across the wave with DPP row shifts and row
// broadcasts (no LDS traffic).
// Inclusive prefix sum within each 16-lane row of the wave (DPP row shifts).
__device__ __forceinline__ uint32_t row16_prefix_incl(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  return x;
}

__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Reserve `mine` consecutive output slots for this thread: one DPP prefix
// and at most one atomic per wave on the LDS counter `ctr`. Returns the
// thread's first slot. Every lane of the wave must call.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t mine, uint32_t* ctr) {
  const uint32_t pre = wave_prefix_incl(mine);
  const uint32_t tot = __builtin_amdgcn_readlane(pre, kWave - 1);
  uint32_t base = 0;
  if (lane_id() == kWave - 1 && tot) base = atomicAdd(ctr, tot);
  base = __builtin_amdgcn_readlane(base, kWave - 1);
  return base + pre - mine;
}

// DPP lane moves of 32- and 64-bit values (every lane valid for the
// controls used here: quad permutes and row rotations).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x) {
  return __builtin_amdgcn_update_dpp(0u, x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_move(uint64_t x) {
  const uint32_t lo = dpp_move<CTRL>(static_cast<uint32_t>(x));
  const uint32_t hi = dpp_move<CTRL>(static_cast<uint32_t>(x >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint32_t read_lane(uint32_t x, int lane) { return __builtin_amdgcn_readlane(x, lane); }
__device__ __forceinline__ uint64_t read_lane(uint64_t x, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(x >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Wave-wide reduction: two quad permutes and two row rotations reduce each
// row of 16 lanes in place, then the four row results (lanes 0, 16, 32, 48)
// are combined. The result is uniform.
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  x = op(x, dpp_move<0xb1>(x));   // quad_perm:[1,0,3,2]
  x = op(x, dpp_move<0x4e>(x));   // quad_perm:[2,3,0,1]
  x = op(x, dpp_move<0x124>(x));  // row_ror:4
  x = op(x, dpp_move<0x128>(x));  // row_ror:8
  return op(op(read_lane(x, 0), read_lane(x, 16)), op(read_lane(x, 32), read_lane(x, 48)));
}

// Maximum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ uint32_t row16_max(uint32_t x) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  x = mx(x, dpp_move<0xb1>(x));   // quad_perm:[1,0,3,2]
  x = mx(x, dpp_move<0x4e>(x));   // quad_perm:[2,3,0,1]
  x = mx(x, dpp_move<0x124>(x));  // row_ror:4
  x = mx(x, dpp_move<0x128>(x));  // row_ror:8
  return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  return wave_reduce(v, [](uint64_t a, uint64_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  return wave_reduce(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

// Device-scope relaxed atomics on workspace words.
__device__ __forceinline__ uint32_t ld_acquire_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace idxtopk
