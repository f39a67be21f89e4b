// topk_rows: exact top-k over a given fp32 score buffer, with page transform.
//
// Addressing ([SGL-37889] "[AMD] Enable GLM DSA prefill top-k to the v2
// kernel", section Modifications, addressing table): row i reads
// scores[i, rs_i : rs_i + n_i] with rs_i = row_starts[i] (or 0), and uses
// page-table row row_to_batch[i] (or i). Selected positions stay row-local
// until the page transform in the epilogue.
//
// Design (one workgroup per row, one pass over HBM):
//  * The window is streamed in tiles of TR_TILE floats with 16-byte loads, with
//    TR_RING tiles in flight. A scalar head (up to 3 elements, up to the first
//    16-byte boundary) and tail (up to 3 elements) make the stride and the
//    start column free: no alignment is required.
//  * A running lower bound L on the row's k-th value filters each element with
//    one float compare. Survivors are appended to an LDS candidate buffer as
//    unique 64-bit keys (value key, inverted position), using a wave ballot
//    plus prefix count and one LDS atomic per wave.
//  * The first tile sets L with one histogram pass over its elements in
//    registers (the edge of the bin where the count from the top reaches k).
//    When the buffer would overflow, an exact select keeps its k best keys,
//    and L becomes the smallest kept value. L never exceeds the row's true
//    k-th value, so no winner is dropped.
//  * At the end an exact select over the buffer gives the top k. The epilogue
//    maps positions through the page table and writes them.
//  * Rows with n <= k need no scores: every position is selected.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace idxtopk {

constexpr int TR_WG = 256;
constexpr int TR_VEC = 2;                    // float4 loads per thread per tile
constexpr int TR_TILE = TR_WG * TR_VEC * 4;  // floats per tile (8 KB)
constexpr int TR_RING = 4;                   // tiles in flight per workgroup

struct RowsArgs {
  const float* scores;
  int64_t stride;
  const int32_t* seq_lens;
  const int32_t* row_starts;
  const int32_t* row_to_batch;
  const int32_t* page_table;
  int64_t pt_stride;
  int32_t page_size;
  FastDiv pdiv;
  int32_t k;
  int32_t* out;
  int32_t cap;  // candidate buffer entries
};

__device__ __forceinline__ int32_t map_slot(const int32_t* pt_row, uint32_t pos, uint32_t P,
                                            const FastDiv& pdiv) {
  if (pt_row == nullptr) return static_cast<int32_t>(pos);
  const uint32_t pg = fdiv(pos, pdiv);
  const uint32_t off = pos - pg * P;
  return static_cast<int32_t>(static_cast<int64_t>(pt_row[pg]) * P + off);
}

typedef float f4 __attribute__((ext_vector_type(4)));

struct TopkRowsLds {
  SelectLds sel;
  uint32_t cnt;
  uint32_t ocnt;
  uint32_t minkey;
};

// Valid elements of one tile of this thread: vector v holds positions
// head + 4 * vi + c with vi = vi0 + v * TR_WG + tid; vectors past the window
// (vi >= nv) were loaded from a clamped address and are ignored.
struct TileView {
  int vi0;
  int nv;
  int head;
  __device__ __forceinline__ bool valid(int v) const {
    return vi0 + v * TR_WG + static_cast<int>(threadIdx.x) < nv;
  }
  __device__ __forceinline__ uint32_t pos(int v, int c) const {
    return static_cast<uint32_t>(head) +
           4u * static_cast<uint32_t>(vi0 + v * TR_WG + static_cast<int>(threadIdx.x)) + c;
  }
};

// Append, in wave-ballot order, every valid element of the thread's tile
// that is >= lf, plus the optional extra (head / tail) element.
__device__ __forceinline__ void append_tile(const f4 (&x)[TR_VEC], const TileView& tv, bool has_e, float xe,
                                            uint32_t pe, float lf, uint64_t* cand, uint32_t* cnt) {
  bool keep[TR_VEC][4];
  uint64_t m[TR_VEC][4];
  uint32_t total = 0;
#pragma unroll
  for (int v = 0; v < TR_VEC; ++v) {
    const bool valid = tv.valid(v);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      keep[v][c] = valid && x[v][c] >= lf;
      m[v][c] = ballot(keep[v][c]);
      total += __popcll(m[v][c]);
    }
  }
  const bool keep_e = has_e && xe >= lf;
  const uint64_t me = ballot(keep_e);
  total += __popcll(me);
  if (total == 0) return;
  uint32_t base = 0;
  if (lane_id() == 0) base = atomicAdd(cnt, total);
  base = uniform(base);
  uint32_t run = 0;
#pragma unroll
  for (int v = 0; v < TR_VEC; ++v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (keep[v][c]) cand[base + run + lanes_below(m[v][c])] = rank_key(float_key(x[v][c]), tv.pos(v, c));
      run += __popcll(m[v][c]);
    }
  }
  if (keep_e) cand[base + run + lanes_below(me)] = rank_key(float_key(xe), pe);
}

// Load this thread's share of cand[0, n) into registers (entries tid + e*WG).
template <int MAXE>
__device__ __forceinline__ int gather_entries(const uint64_t* cand, uint32_t n, uint64_t (&keys)[MAXE]) {
  int nv = 0;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const uint32_t i = threadIdx.x + e * TR_WG;
    if (i < n) {
      keys[e] = cand[i];
      nv = e + 1;
    }
  }
  return nv;
}

template <int MAXE>
__global__ __launch_bounds__(TR_WG, 3) void topk_rows_kernel(RowsArgs a) {
  extern __shared__ uint64_t cand[];
  __shared__ TopkRowsLds s;
  // The select histogram overlays the candidate buffer: every select first
  // copies the buffer's keys to registers.
  uint32_t* hist = reinterpret_cast<uint32_t*>(cand);

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = a.seq_lens[row];
  const int64_t rs = a.row_starts ? a.row_starts[row] : 0;
  const int prow = a.row_to_batch ? a.row_to_batch[row] : row;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  int32_t* out = a.out + static_cast<int64_t>(row) * a.k;
  const int32_t* pt_row = a.page_table ? a.page_table + static_cast<int64_t>(prow) * a.pt_stride : nullptr;

  if (n <= a.k) {  // every visible key is selected
    for (int i = tid; i < a.k; i += TR_WG)
      out[i] = (i < n) ? map_slot(pt_row, static_cast<uint32_t>(i), P, a.pdiv) : -1;
    return;
  }

  const float* base = a.scores + static_cast<int64_t>(row) * a.stride + rs;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(base);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) >> 2);
  head = head < n ? head : n;
  const int nv = (n - head) >> 2;  // full float4 vectors
  const int tail0 = head + 4 * nv;
  const int ntail = n - tail0;
  const f4* vbase = reinterpret_cast<const f4*>(base + head);
  const int ntiles = (nv + TR_WG * TR_VEC - 1) / (TR_WG * TR_VEC);

  // scalar head and tail elements ride along with the first tile
  const bool has_e = tid < head + ntail;
  uint32_t pe = 0;
  float xe = 0.0f;
  if (has_e) {
    pe = static_cast<uint32_t>(tid < head ? tid : tail0 + (tid - head));
    xe = base[pe];
  }

  // tile t, vector v of this thread; loads past the window use a clamped
  // (in-bounds) address and are masked out by TileView
  auto load_tile = [&](int t, f4 (&x)[TR_VEC]) {
#pragma unroll
    for (int v = 0; v < TR_VEC; ++v) {
      int vi = t * TR_WG * TR_VEC + v * TR_WG + tid;
      vi = vi < nv ? vi : nv - 1;
      x[v] = __builtin_nontemporal_load(vbase + vi);
    }
  };
  auto view = [&](int t) { return TileView{t * TR_WG * TR_VEC, nv, head}; };

  // exact top-k of the buffer; returns the separating key T
  auto select_buffer = [&](uint32_t c, uint64_t (&keys)[MAXE], int& nvk) -> uint64_t {
    nvk = gather_entries<MAXE>(cand, c, keys);
    __syncthreads();  // every thread holds its keys before the histogram overlays them
    return wg_select<TR_WG>(
        [&](auto&& f) {
#pragma unroll
          for (int e = 0; e < MAXE; ++e)
            if (e < nvk) f(keys[e]);
        },
        k, hist, s.sel);
  };

  if (tid == 0) s.cnt = 0;
  float lf = -__builtin_inff();

  // After tile t: when the buffer would not take another tile, keep exactly
  // the k best keys and raise the bound to the smallest kept value.
  auto after_tile = [&](int t) {
    __syncthreads();
    const uint32_t c = s.cnt;
    __syncthreads();
    const bool last = (t + 1 == ntiles);
    if (!last && c > k && c + TR_TILE > static_cast<uint32_t>(a.cap)) {
      uint64_t keys[MAXE];
      int nvk;
      const uint64_t T = select_buffer(c, keys, nvk);
      if (tid == 0) {
        s.cnt = 0;
        s.minkey = 0xffffffffu;
      }
      __syncthreads();
      uint32_t mymin = 0xffffffffu;
#pragma unroll
      for (int e = 0; e < MAXE; ++e) {
        const bool keep = (e < nvk) && keys[e] >= T;
        const uint64_t mk = ballot(keep);
        if (mk == 0) continue;
        uint32_t wb = 0;
        if (lane_id() == 0) wb = atomicAdd(&s.cnt, static_cast<uint32_t>(__popcll(mk)));
        wb = uniform(wb);
        const uint32_t at = wb + lanes_below(mk);
        if (keep && at < static_cast<uint32_t>(a.cap)) {
          cand[at] = keys[e];
          const uint32_t vk = rank_vkey(keys[e]);
          mymin = vk < mymin ? vk : mymin;
        }
      }
      mymin = wave_min_u32(mymin);
      if (lane_id() == 0) atomicMin(&s.minkey, mymin);
      __syncthreads();
      lf = key_float(s.minkey);
      __syncthreads();
    }
  };

  // Ring of TR_RING tiles in flight: tile t lives in slot t % TR_RING, is
  // consumed in place, and its slot is refilled with tile t + TR_RING right
  // after (no register copies, so a tile only waits for its own loads).
  f4 ring[TR_RING][TR_VEC];
  if (ntiles > 0) {
#pragma unroll
    for (int u = 0; u < TR_RING; ++u) load_tile(u < ntiles ? u : ntiles - 1, ring[u]);
  }
  __syncthreads();

  // First tile (plus the head / tail elements): when more data follows, one
  // histogram pass over these elements bounds the k-th value; then append
  // what passes the bound.
  {
    const TileView tv = view(0);
    const bool has_tile = ntiles > 0;
    const int n0 = 4 * min(nv, TR_WG * TR_VEC) + head + ntail;
    if (ntiles > 1 && n0 > a.k) {
      const uint64_t bound = wg_select<TR_WG>(
          [&](auto&& f) {
#pragma unroll
            for (int v = 0; v < TR_VEC; ++v)
              if (tv.valid(v)) {
#pragma unroll
                for (int c = 0; c < 4; ++c) f(rank_key(float_key(ring[0][v][c]), tv.pos(v, c)));
              }
            if (has_e) f(rank_key(float_key(xe), pe));
          },
          k, hist, s.sel, 1);
      lf = key_float(rank_vkey(bound));
    }
    if (has_tile) {
      append_tile(ring[0], tv, has_e, xe, pe, lf, cand, &s.cnt);
      __builtin_amdgcn_sched_barrier(0);
      if (TR_RING < ntiles) load_tile(TR_RING, ring[0]);
      after_tile(0);
    } else {
      const f4 none[TR_VEC] = {};
      append_tile(none, TileView{0, 0, head}, has_e, xe, pe, lf, cand, &s.cnt);
      __syncthreads();
    }
  }

  // steady state: tiles t0 .. t0 + TR_RING - 1 (slot t % TR_RING), every
  // refill in range, so control flow is uniform
  int t0 = 1;
  for (; t0 + 2 * TR_RING <= ntiles; t0 += TR_RING) {
#pragma unroll
    for (int u = 0; u < TR_RING; ++u) {
      const int t = t0 + u;
      const int slot = (1 + u) % TR_RING;
      append_tile(ring[slot], view(t), false, 0.0f, 0u, lf, cand, &s.cnt);
      __builtin_amdgcn_sched_barrier(0);
      load_tile(t + TR_RING, ring[slot]);
      after_tile(t);
    }
  }
  // drain: fewer than 2 * TR_RING tiles remain
#pragma unroll
  for (int u = 0; u < 2 * TR_RING; ++u) {
    const int t = t0 + u;
    const int slot = (1 + u) % TR_RING;
    if (t < ntiles) {
      append_tile(ring[slot], view(t), false, 0.0f, 0u, lf, cand, &s.cnt);
      if (t + TR_RING < ntiles) load_tile(t + TR_RING, ring[slot]);
      after_tile(t);
    }
  }

  // final selection over the buffer
  const uint32_t c = s.cnt;
  if (tid == 0) s.ocnt = 0;
  __syncthreads();
  if (c <= k) {
    // only reachable with NaN inputs (outside the domain): emit what is there
    for (uint32_t i = tid; i < k; i += TR_WG)
      out[i] = (i < c) ? map_slot(pt_row, rank_pos(cand[i]), P, a.pdiv) : -1;
    return;
  }
  uint64_t keys[MAXE];
  int nvk;
  const uint64_t T = select_buffer(c, keys, nvk);
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const bool keep = (e < nvk) && keys[e] >= T;
    const uint64_t mk = ballot(keep);
    if (mk == 0) continue;
    uint32_t wb = 0;
    if (lane_id() == 0) wb = atomicAdd(&s.ocnt, static_cast<uint32_t>(__popcll(mk)));
    wb = uniform(wb);
    const uint32_t at = wb + lanes_below(mk);
    if (keep && at < k) out[at] = map_slot(pt_row, rank_pos(keys[e]), P, a.pdiv);
  }
}

// Candidate buffer sizing: room for the k kept keys plus two whole tiles
// (one tile of slack between compactions), and never less than the select
// histogram that overlays it.
static inline int rows_cap(int k) {
  const int c = (k > TR_TILE ? k : TR_TILE) + 2 * TR_TILE + 8;
  return c > kSelBins / 2 ? c : kSelBins / 2;
}

int launch_topk_rows(const float* scores, int64_t stride, int rows, const int32_t* seq_lens,
                     const int32_t* row_starts, const int32_t* row_to_batch,
                     const int32_t* page_table, int64_t pt_stride, int page_size, int k,
                     int32_t* out, hipStream_t stream) {
  RowsArgs a;
  a.scores = scores;
  a.stride = stride;
  a.seq_lens = seq_lens;
  a.row_starts = row_starts;
  a.row_to_batch = row_to_batch;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.page_size = page_size > 0 ? page_size : 1;
  a.pdiv = make_fastdiv(static_cast<uint32_t>(a.page_size));
  a.k = k;
  a.out = out;
  a.cap = rows_cap(k);
  const size_t lds = static_cast<size_t>(a.cap) * sizeof(uint64_t);
  const int maxe_needed = (a.cap + TR_WG - 1) / TR_WG;
  if (maxe_needed <= 25) {  // k <= 2048
    static std::atomic<size_t> granted25{0};
    if (allow_dynamic_lds(reinterpret_cast<const void*>(&topk_rows_kernel<25>), lds, granted25) != hipSuccess)
      return -4;
    (void)hipGetLastError();
    hipLaunchKernelGGL(topk_rows_kernel<25>, dim3(rows), dim3(TR_WG), lds, stream, a);
  } else {  // k <= 8192
    static std::atomic<size_t> granted49{0};
    if (allow_dynamic_lds(reinterpret_cast<const void*>(&topk_rows_kernel<49>), lds, granted49) != hipSuccess)
      return -4;
    (void)hipGetLastError();
    hipLaunchKernelGGL(topk_rows_kernel<49>, dim3(rows), dim3(TR_WG), lds, stream, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace idxtopk
