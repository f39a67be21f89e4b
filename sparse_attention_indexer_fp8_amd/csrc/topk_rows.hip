// topk_rows: exact top-k over a given fp32 score buffer, with page transform.
//
// Addressing ([SGL-37889] "[AMD] Enable GLM DSA prefill top-k to the v2
// kernel", section Modifications, addressing table): row i reads
// scores[i, rs_i : rs_i + n_i] with rs_i = row_starts[i] (or 0), and uses
// page-table row row_to_batch[i] (or i). Selected positions stay row-local
// until the page transform in the epilogue.
//
// Design (one workgroup per row, one pass over HBM):
//  * Workgroups are dispatched in row order, several resident per compute
//    unit, so while one runs its selects the others keep loads in flight.
//  * A row's window is streamed in tiles of TR_TILE floats with 16-byte
//    loads, TR_RING tiles in flight. A scalar head (up to 3 elements, up to
//    the first 16-byte boundary) and tail (up to 3 elements) make the stride
//    and the start column free: no alignment is required.
//  * A running lower bound L filters each element with one float compare.
//    Survivors are appended to an LDS candidate buffer as unique 64-bit keys
//    (value key, inverted position): a wave ballot plus prefix count and one
//    LDS atomic per wave.
//  * The first tile sets L with one histogram pass over its n0 elements in
//    registers: the edge of the bin where the count from the top reaches a
//    rank r. With r = k, L is a proven lower bound on the row's k-th value.
//    A long row first tries r ~ 1.5 k n0 / n + 8 (about 1.5 k of the row's
//    n values are expected above it), binned by value (equal-width bins
//    over the tile's range) rather than by key. The buffer then holds every
//    element >= L, so if it ends with at least k keys, L was below the k-th
//    value and the result is exact; otherwise the row is streamed again with
//    r = k.
//  * When the buffer would overflow, a select finds a bound with between k
//    and k + slack keys above it, the buffer keeps those, and L becomes the
//    smallest kept value (never above the row's k-th value).
//  * At the end an exact select gives the key T of the k-th best; the keys
//    >= T go through the page table to the output (slots reserved per wave,
//    all page-table gathers of a round issued before any is used).
//  * Rows with n <= k need no scores: every position is selected.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"
#include "sort.hpp"


namespace idxtopk {

constexpr int TR_WG = 256;
constexpr int TR_VEC = 2;                    // float4 loads per thread per tile
constexpr int TR_TILE = TR_WG * TR_VEC * 4;  // floats per tile (8 KB)
constexpr int TR_RING = 4;                   // tiles in flight per workgroup
constexpr int TR_BATCH = 4;                  // buffer entries per thread per compaction batch
constexpr int TR_EMIT = 8;                   // outputs per thread per emission round

struct RowsArgs {
  const float* scores;
  int64_t stride;
  const int32_t* seq_lens;
  const int32_t* row_starts;
  const int32_t* row_to_batch;
  const int32_t* kv_offset;  // per row: KV position of the window's column 0, or null (0)
  const int32_t* page_table;
  int64_t pt_stride;
  int32_t page_size;
  FastDiv pdiv;
  int32_t k;
  int32_t* out;
  int32_t cap;   // candidate buffer entries
  int32_t npow;  // sorted output: power of two >= k (<= cap)
  int32_t rows;
  int32_t short_rows;  // rows of at most SR_MAX_N keys take one wave each
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

// Geometry of one row (all values uniform across the workgroup).
struct RowCtx {
  int row;
  int n;
  int head;    // scalar elements before the first 16-byte boundary
  int nv;      // full float4 vectors after the head
  int tail0;   // first tail element
  int ntail;
  int ntiles;
  const float* base;
  const f4* vbase;
  const int32_t* pt_row;
  int32_t* out;
  uint32_t off;  // added to every selected row-local position before the transform
  bool trivial;  // n <= k: every position is selected
};

__device__ __forceinline__ RowCtx row_setup(const RowsArgs& a, int row) {
  RowCtx r;
  r.row = row;
  r.n = load_uniform(a.seq_lens + row);
  const int64_t rs = a.row_starts ? load_uniform(a.row_starts + row) : 0;
  const int prow = a.row_to_batch ? load_uniform(a.row_to_batch + row) : row;
  r.pt_row = a.page_table ? a.page_table + static_cast<int64_t>(prow) * a.pt_stride : nullptr;
  r.out = a.out + static_cast<int64_t>(row) * a.k;
  r.off = a.kv_offset ? static_cast<uint32_t>(load_uniform(a.kv_offset + row)) : 0u;
  r.trivial = r.n <= a.k;
  IDXTOPK_CHECK(r.n >= 0 && rs >= 0 && rs + r.n <= a.stride, kChkWindow);
  IDXTOPK_CHECK(prow >= 0, kChkRowToBatch);
  r.base = a.scores + static_cast<int64_t>(row) * a.stride + rs;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(r.base);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) >> 2);
  r.head = head < r.n ? head : r.n;
  r.nv = (r.n - r.head) >> 2;
  r.tail0 = r.head + 4 * r.nv;
  r.ntail = r.n - r.tail0;
  r.vbase = reinterpret_cast<const f4*>(r.base + r.head);
  r.ntiles = r.trivial ? 0 : (r.nv + TR_WG * TR_VEC - 1) / (TR_WG * TR_VEC);
  return r;
}

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

__device__ __forceinline__ TileView tile_view(const RowCtx& r, int t) {
  return TileView{t * TR_WG * TR_VEC, r.nv, r.head};
}

// Tile t of row r, this thread's vectors; loads past the window use a clamped
// (in-bounds) address and are masked out by TileView.
__device__ __forceinline__ void load_tile(const RowCtx& r, int t, f4 (&x)[TR_VEC]) {
#pragma unroll
  for (int v = 0; v < TR_VEC; ++v) {
    int vi = t * TR_WG * TR_VEC + v * TR_WG + static_cast<int>(threadIdx.x);
    vi = vi < r.nv ? vi : r.nv - 1;
    x[v] = __builtin_nontemporal_load(r.vbase + vi);
  }
}

// The scalar head / tail element this thread carries (if any).
struct Extra {
  bool has;
  uint32_t pos;
  float x;
};

// Request the start of a row: its head / tail element (if this thread has
// one) and tiles [0, TR_RING) (slots past the row's last tile repeat it; the
// duplicates are never read).
__device__ __forceinline__ void prefetch_row(const RowCtx& r, f4 (&ring)[TR_RING][TR_VEC], Extra& e) {
  const int tid = threadIdx.x;
  e.has = tid < r.head + r.ntail;
  e.pos = static_cast<uint32_t>(tid < r.head ? tid : r.tail0 + (tid - r.head));
  e.x = e.has ? r.base[e.pos] : 0.0f;
  if (r.ntiles > 0) {
#pragma unroll
    for (int u = 0; u < TR_RING; ++u) load_tile(r, u < r.ntiles ? u : r.ntiles - 1, ring[u]);
  }
}

// Append, in wave-ballot order, every valid element of the thread's tile
// that is >= lf, plus the optional extra (head / tail) element.
__device__ __forceinline__ void append_tile(const f4 (&x)[TR_VEC], const TileView& tv, const Extra& e,
                                            bool with_extra, float lf, uint64_t* cand, uint32_t* cnt) {
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
  const bool keep_e = with_extra && e.has && e.x >= lf;
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
  if (keep_e) cand[base + run + lanes_below(me)] = rank_key(float_key(e.x), e.pos);
}

// Select over cand[0, c) (c > k): a key T with k <= (keys >= T) <= k + slack
// (exactly k for slack 0). The keys stay in LDS; every histogram pass
// re-reads them there.
__device__ __forceinline__ uint64_t select_buffer(const uint64_t* cand, uint32_t c, uint32_t k,
                                                  uint32_t slack, TopkRowsLds& s) {
  uint64_t mn = ~0ull, mx = 0;
  lds_for_each<TR_WG, 4>(cand, c, [&](uint64_t x) {
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  });
  wg_range<TR_WG>(mn, mx, s.sel);
  return wg_select<TR_WG>([&](auto&& f) { lds_for_each<TR_WG, 4>(cand, c, f); }, k, mn, mx, s.sel, slack);
}

// Keep the keys >= T of cand[0, c), packed to the front of the buffer (in no
// particular order); s.cnt becomes their count. Returns the smallest kept
// value key. Every thread must have read c before the call.
// In place, in batches of TR_BATCH * TR_WG entries: a batch is read
// completely (barrier) before its kept keys are written, and they land below
// the batch's end, where every entry has been read already.
__device__ __forceinline__ uint32_t keep_compact(uint64_t* cand, uint32_t c, uint64_t T, TopkRowsLds& s) {
  const uint32_t tid = threadIdx.x;
  if (tid == 0) {
    s.cnt = 0;
    s.minkey = 0xffffffffu;
  }
  __syncthreads();
  uint32_t mymin = 0xffffffffu;
  for (uint32_t b0 = 0; b0 < c; b0 += TR_BATCH * TR_WG) {
    uint64_t key[TR_BATCH];
    bool keep[TR_BATCH];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < TR_BATCH; ++j) {
      const uint32_t i = b0 + j * TR_WG + tid;
      key[j] = cand[i < c ? i : 0];
      keep[j] = i < c && key[j] >= T;
      mine += keep[j];
    }
    __syncthreads();
    uint32_t at = wave_reserve(mine, &s.cnt);
#pragma unroll
    for (int j = 0; j < TR_BATCH; ++j) {
      if (keep[j]) {
        cand[at++] = key[j];
        const uint32_t vk = rank_vkey(key[j]);
        mymin = vk < mymin ? vk : mymin;
      }
    }
  }
  mymin = wave_min_u32(mymin);
  if (lane_id() == 0) atomicMin(&s.minkey, mymin);
  __syncthreads();
  return s.minkey;
}

// After tile t of row r: when the buffer would not take another tile, keep
// between k and k + (cap - TR_TILE - k) / 2 of its best keys (so at least
// half the spare room is freed) and raise the bound to the smallest kept
// value.
__device__ __forceinline__ void after_tile(const RowCtx& r, int t, uint32_t k, int cap, float& lf,
                                           uint64_t* cand, TopkRowsLds& s) {
  __syncthreads();
  const uint32_t c = s.cnt;
  __syncthreads();
  IDXTOPK_CHECK(c <= static_cast<uint32_t>(cap), kChkCandOverflow);
  if (t + 1 == r.ntiles || c <= k || c + TR_TILE <= static_cast<uint32_t>(cap)) return;
  const uint32_t slack = (static_cast<uint32_t>(cap) - TR_TILE - k) / 2;
  const uint64_t T = select_buffer(cand, c, k, slack, s);
  lf = key_float(keep_compact(cand, c, T, s));
}

// Stream all tiles of row r (its first TR_RING tiles and the extra element are
// already requested) into the candidate buffer. With `estimate`, a long row's
// first-tile bound uses the rank r ~ 1.5 k n0 / n + 8 instead of k; returns
// whether it did (then the caller must check that at least k keys were kept).
__device__ __forceinline__ bool stream_row(const RowCtx& r, f4 (&ring)[TR_RING][TR_VEC], const Extra& ex,
                                           uint32_t k, int cap, bool estimate, uint64_t* cand,
                                           TopkRowsLds& s) {
  float lf = -__builtin_inff();
  bool estimated = false;
  // First tile (plus the head / tail elements): when more data follows, one
  // histogram pass over these elements bounds the rank-r value; then append
  // what passes the bound.
  {
    const TileView tv = tile_view(r, 0);
    const int n0 = 4 * min(r.nv, TR_WG * TR_VEC) + r.head + r.ntail;
    if (r.ntiles > 1 && n0 > static_cast<int>(k)) {
      uint32_t rank = k;
      if (estimate) {
        const uint64_t n = static_cast<uint64_t>(r.n);
        const uint64_t want = (3ull * k * static_cast<uint64_t>(n0) + 2 * n - 1) / (2 * n) + 8u;
        if (want < k) {
          rank = static_cast<uint32_t>(want);
          estimated = true;
        }
      }
      auto each = [&](auto&& f) {
#pragma unroll
        for (int v = 0; v < TR_VEC; ++v)
          if (tv.valid(v)) {
#pragma unroll
            for (int c = 0; c < 4; ++c) f(rank_key(float_key(ring[0][v][c]), tv.pos(v, c)));
          }
        if (ex.has) f(rank_key(float_key(ex.x), ex.pos));
      };
      uint64_t mn = ~0ull, mx = 0;
      each([&](uint64_t key) {
        mn = key < mn ? key : mn;
        mx = key > mx ? key : mx;
      });
      wg_range<TR_WG>(mn, mx, s.sel);
      const float vmin = key_float(rank_vkey(mn)), vmax = key_float(rank_vkey(mx));
      const float width = vmax - vmin;
      if (estimated && width > 0.0f && width < __builtin_inff()) {
        // estimate: kSelBins equal-width value bins over the tile's range;
        // the bound is the lower edge of the bin where the count from the
        // top reaches the rank
        const float scale = static_cast<float>(kSelBins) / width;
        auto add = [&](float x) {
          float f = (x - vmin) * scale;
          f = f < static_cast<float>(kSelBins - 1) ? f : static_cast<float>(kSelBins - 1);
          f = f > 0.0f ? f : 0.0f;
          atomicAdd(&s.sel.hist[sel_slot(static_cast<uint32_t>(f))], 1u);
        };
#pragma unroll
        for (int v = 0; v < TR_VEC; ++v)
          if (tv.valid(v)) {
#pragma unroll
            for (int c = 0; c < 4; ++c) add(ring[0][v][c]);
          }
        if (ex.has) add(ex.x);
        const HistPick p = wg_hist_pick<TR_WG>(rank, s.sel);
        lf = vmin + static_cast<float>(p.bin) / scale;
      } else {
        // proven: at least rank keys of the tile are >= the bound
        const uint64_t bound = wg_select<TR_WG>(each, rank, mn, mx, s.sel, ~0u);
        lf = key_float(rank_vkey(bound));
      }
    }
    if (r.ntiles > 0) {
      append_tile(ring[0], tv, ex, true, lf, cand, &s.cnt);
      __builtin_amdgcn_sched_barrier(0);
      if (TR_RING < r.ntiles) load_tile(r, TR_RING, ring[0]);
      after_tile(r, 0, k, cap, lf, cand, s);
    } else {
      const f4 none[TR_VEC] = {};
      append_tile(none, TileView{0, 0, r.head}, ex, true, lf, cand, &s.cnt);
      __syncthreads();
    }
  }
  // steady state: tiles t0 .. t0 + TR_RING - 1 (slot t % TR_RING), every
  // refill in range, so control flow is uniform
  const Extra none_e{false, 0u, 0.0f};
  int t0 = 1;
  for (; t0 + 2 * TR_RING <= r.ntiles; t0 += TR_RING) {
#pragma unroll
    for (int u = 0; u < TR_RING; ++u) {
      const int t = t0 + u;
      const int slot = (1 + u) % TR_RING;
      append_tile(ring[slot], tile_view(r, t), none_e, false, lf, cand, &s.cnt);
      __builtin_amdgcn_sched_barrier(0);
      load_tile(r, t + TR_RING, ring[slot]);
      after_tile(r, t, k, cap, lf, cand, s);
    }
  }
  // drain: fewer than 2 * TR_RING tiles remain
#pragma unroll
  for (int u = 0; u < 2 * TR_RING; ++u) {
    const int t = t0 + u;
    const int slot = (1 + u) % TR_RING;
    if (t < r.ntiles) {
      append_tile(ring[slot], tile_view(r, t), none_e, false, lf, cand, &s.cnt);
      if (t + TR_RING < r.ntiles) load_tile(r, t + TR_RING, ring[slot]);
      after_tile(r, t, k, cap, lf, cand, s);
    }
  }
  return estimated;
}

// Outputs of a row with n <= k: positions 0 .. n - 1 mapped, then -1.
__device__ __forceinline__ void emit_all(const RowCtx& r, const RowsArgs& a) {
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  for (int i = threadIdx.x; i < a.k; i += TR_WG)
    r.out[i] = (i < r.n) ? map_slot(r.pt_row, static_cast<uint32_t>(i) + r.off, P, a.pdiv) : -1;
}

// Sorted output: keys[0, npow) (real entries first, then zeros) are put in
// descending order, and entry i of the row's output is the key of rank i
// mapped to its slot (-1 for a zero key). A larger key is the better entry
// (higher score, then lower position), so the order is score descending,
// equal scores by ascending position.
//
// Up to 2048 keys: E per thread in registers (block_sort_desc; `keys` then
// serves as its exchange scratch), ranks tid*E .. tid*E + E - 1 written by
// thread tid with all page lookups issued first.
template <int E>
__device__ __forceinline__ void sort_emit_reg(const RowCtx& r, const RowsArgs& a, uint64_t* keys) {
  const int tid = threadIdx.x;
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = keys[e * TR_WG + tid];
  __syncthreads();
  block_sort_desc<TR_WG, E>(x, keys);
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  uint32_t pg[E];
  int32_t page[E];
#pragma unroll
  for (int e = 0; e < E; ++e) pg[e] = x[e] ? fdiv(rank_pos(x[e]) + r.off, a.pdiv) : 0u;
  if (r.pt_row && x[0]) {
    // zero keys read page 0, which exists when this thread holds any entry
#pragma unroll
    for (int e = 0; e < E; ++e) page[e] = r.pt_row[pg[e]];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    if (i < a.k) {
      const uint32_t pos = rank_pos(x[e]) + r.off;
      r.out[i] = !x[e] ? -1
               : r.pt_row ? static_cast<int32_t>(static_cast<int64_t>(page[e]) * P + (pos - pg[e] * P))
                          : static_cast<int32_t>(pos);
    }
  }
}

// Larger sizes: a bitonic network in LDS, one barrier per step.
__device__ __forceinline__ void sort_emit_lds(const RowCtx& r, const RowsArgs& a, uint64_t* keys) {
  const int tid = threadIdx.x;
  const int npow = a.npow;
  for (int size = 2; size <= npow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (npow >> 1); t += TR_WG) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = keys[lo], y = keys[hi];
        if ((x < y) == desc) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  for (int i0 = 0; i0 < a.k; i0 += TR_EMIT * TR_WG) {
    uint64_t kk[TR_EMIT];
    int32_t base[TR_EMIT];
    uint32_t pg[TR_EMIT];
#pragma unroll
    for (int j = 0; j < TR_EMIT; ++j) {
      const int i = i0 + j * TR_WG + tid;
      kk[j] = i < a.k ? keys[i] : 0ull;
      pg[j] = kk[j] ? fdiv(rank_pos(kk[j]) + r.off, a.pdiv) : 0u;
    }
    if (r.pt_row) {
      // all lookups issued before any is used; zero keys read page 0
#pragma unroll
      for (int j = 0; j < TR_EMIT; ++j) base[j] = kk[j] || r.n > 0 ? r.pt_row[pg[j]] : 0;
    }
#pragma unroll
    for (int j = 0; j < TR_EMIT; ++j) {
      const int i = i0 + j * TR_WG + tid;
      if (i < a.k) {
        const uint32_t pos = rank_pos(kk[j]) + r.off;
        r.out[i] = !kk[j] ? -1
                 : r.pt_row ? static_cast<int32_t>(static_cast<int64_t>(base[j]) * P + (pos - pg[j] * P))
                            : static_cast<int32_t>(pos);
      }
    }
  }
}

__device__ __forceinline__ void sort_emit(const RowCtx& r, const RowsArgs& a, uint64_t* keys) {
  switch (a.npow) {
    case 512: sort_emit_reg<2>(r, a, keys); break;
    case 1024: sort_emit_reg<4>(r, a, keys); break;
    case 2048: sort_emit_reg<8>(r, a, keys); break;
    default: sort_emit_lds(r, a, keys); break;
  }
}

// The whole workgroup selects the k best keys of row `cur` (any length) and
// writes its output row.
template <bool SORTED>
__device__ __forceinline__ void wg_row(const RowsArgs& a, const RowCtx& cur, uint64_t* cand, TopkRowsLds& s) {
  const uint32_t tid = threadIdx.x;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  if (cur.trivial) {
    if (SORTED) {
      // every position is selected: its keys, then the sort
      for (int i = tid; i < a.npow; i += TR_WG)
        cand[i] = i < cur.n ? rank_key(float_key(cur.base[i]), static_cast<uint32_t>(i)) : 0ull;
      __syncthreads();
      sort_emit(cur, a, cand);
    } else {
      emit_all(cur, a);
    }
    return;
  }
  f4 ring[TR_RING][TR_VEC];
  Extra ex;
  prefetch_row(cur, ring, ex);
  wg_select_init<TR_WG>(s.sel);
  if (tid == 0) {
    s.cnt = 0;
    s.ocnt = 0;
  }
  __syncthreads();

  const bool estimated = stream_row(cur, ring, ex, k, a.cap, true, cand, s);
  uint32_t c = s.cnt;  // stable: the last after_tile ended with a barrier
  if (estimated && c < k) {
    // the estimated bound was above the row's k-th value: stream the row
    // again with the proven first-tile bound
    __syncthreads();
    if (tid == 0) s.cnt = 0;
    __syncthreads();
    prefetch_row(cur, ring, ex);
    stream_row(cur, ring, ex, k, a.cap, false, cand, s);
    c = s.cnt;
  }
  // the k best keys are those >= T (all of them when c <= k, which with
  // c < k happens only for NaN inputs, outside the domain: the rest of the
  // row is padded with -1). Each round reserves output slots per wave, then
  // issues all its page-table gathers before using any.
  const uint64_t T = c > k ? select_buffer(cand, c, k, 0, s) : 0ull;
  if (SORTED) {
    // the kept keys move to the front of the buffer, in place: a round
    // writes only below what all rounds so far have read (the barrier
    // separates this round's reads from its writes), so nothing unread is
    // overwritten
    for (uint32_t b0 = 0; b0 < c; b0 += TR_EMIT * TR_WG) {
      uint64_t key[TR_EMIT];
      bool keep[TR_EMIT];
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < TR_EMIT; ++j) {
        const uint32_t i = b0 + j * TR_WG + tid;
        key[j] = cand[i < c ? i : 0];
        keep[j] = i < c && key[j] >= T;
        mine += keep[j];
      }
      uint32_t at = wave_reserve(mine, &s.ocnt);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < TR_EMIT; ++j) {
        if (keep[j]) {
          if (at < k) cand[at] = key[j];
          ++at;
        }
      }
    }
    __syncthreads();
    const uint32_t kept = s.ocnt < k ? s.ocnt : k;
    for (uint32_t i = kept + tid; i < static_cast<uint32_t>(a.npow); i += TR_WG) cand[i] = 0ull;
    __syncthreads();
    sort_emit(cur, a, cand);
    return;
  }
  for (uint32_t b0 = 0; b0 < c; b0 += TR_EMIT * TR_WG) {
    bool keep[TR_EMIT];
    uint32_t pos[TR_EMIT];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < TR_EMIT; ++j) {
      const uint32_t i = b0 + j * TR_WG + tid;
      const uint64_t key = cand[i < c ? i : 0];
      keep[j] = i < c && key >= T;
      IDXTOPK_CHECK(!keep[j] || rank_pos(key) < static_cast<uint32_t>(cur.n), kChkPosition);
      pos[j] = rank_pos(key) + cur.off;
      mine += keep[j];
    }
    uint32_t at = wave_reserve(mine, &s.ocnt);
    // entries not kept read page 0 (in range)
    uint32_t pg[TR_EMIT];
    int32_t base[TR_EMIT];
    const bool paged = cur.pt_row != nullptr;
    if (paged) {
#pragma unroll
      for (int j = 0; j < TR_EMIT; ++j) {
        pg[j] = keep[j] ? fdiv(pos[j], a.pdiv) : 0u;
        base[j] = cur.pt_row[pg[j]];
      }
#pragma unroll
      for (int j = 0; j < TR_EMIT; ++j) IDXTOPK_CHECK(!keep[j] || base[j] >= 0, kChkPageId);
    }
#pragma unroll
    for (int j = 0; j < TR_EMIT; ++j) {
      if (keep[j]) {
        const int32_t slot = paged ? static_cast<int32_t>(static_cast<int64_t>(base[j]) * P + (pos[j] - pg[j] * P))
                                   : static_cast<int32_t>(pos[j]);
        if (at < k) __builtin_nontemporal_store(slot, cur.out + at);  // read by the next kernel, not by this one
        ++at;
      }
    }
  }
  for (uint32_t i = c + tid; i < k; i += TR_WG) cur.out[i] = -1;
}

// ---------------------------------------------------------------------------
// Short rows: one wave per row, no workgroup barrier
// ---------------------------------------------------------------------------
//
// A row of at most SR_MAX_N keys (with k <= SR_MAX_K) is read by one wave in
// quarters of SR_QV float4 vectors, two quarters in flight. The first
// quarter (plus the scalar head and tail) sets an estimated bound L, as the
// workgroup path's first tile does: 256 equal-width value bins over the
// quarter's range, L the lower edge of the bin where the count from the top
// reaches ~1.5 k n0 / n + 8. Every element >= L goes, as a unique 64-bit
// key, to the wave's own SR_CAP-entry LDS area by ballot compaction. If
// between k and SR_CAP keys were kept, L lies at or below the row's k-th
// value, so every element of the top k is among them: wave_select finds the
// k-th key T exactly and the keys >= T are emitted. Otherwise the row goes
// to the workgroup path afterwards.

constexpr int SR_MAX_N = 8192;
constexpr int SR_MAX_K = 512;
constexpr int SR_V = 8;                 // float4 per lane per quarter
constexpr int SR_QV = SR_V * kWave;     // vectors per quarter (2048 floats)
constexpr int SR_CAP = 1024;            // candidates per wave
constexpr int SR_PER = SR_CAP / kWave;  // candidates per lane in the select
constexpr int SR_EMIT = 8;              // outputs per lane per emission round
constexpr int SR_MIN_ROWS = 2048;       // launches with fewer rows keep a workgroup per row
static_assert(SR_MAX_N <= 4 * SR_QV * 4, "four quarters cover a short row");
static_assert(SR_PER % SR_EMIT == 0, "whole emission rounds");

// Returns false when the row needs the workgroup path.
__device__ __forceinline__ bool short_row(const RowsArgs& a, const RowCtx& r, uint64_t* wc, uint32_t* hist) {
  const int lane = lane_id();
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  const int n = r.n;
  if (n <= static_cast<int>(k)) {
    for (int i = lane; i < static_cast<int>(k); i += kWave)
      r.out[i] = i < n ? map_slot(r.pt_row, static_cast<uint32_t>(i) + r.off, P, a.pdiv) : -1;
    return true;
  }
  // the head / tail element of this lane, if any
  const bool has_x = lane < r.head + r.ntail;
  const uint32_t xpos = static_cast<uint32_t>(lane < r.head ? lane : r.tail0 + (lane - r.head));
  const float xv = has_x ? r.base[xpos] : 0.0f;
  const int nq = (r.nv + SR_QV - 1) / SR_QV;  // quarters holding vectors (0 .. 4)
  f4 A[SR_V], B[SR_V];
  auto load_q = [&](int q, f4 (&X)[SR_V]) {
#pragma unroll
    for (int v = 0; v < SR_V; ++v) {
      int vi = q * SR_QV + v * kWave + lane;
      vi = vi < r.nv ? vi : r.nv - 1;
      X[v] = __builtin_nontemporal_load(r.vbase + vi);
    }
  };
  if (nq > 0) load_q(0, A);
  if (nq > 1) load_q(1, B);

  // Estimated bound from the first quarter and the head / tail elements.
  const int n0 = 4 * min(r.nv, SR_QV) + r.head + r.ntail;
  const uint64_t want = (3ull * k * static_cast<uint64_t>(n0) + 2ull * n - 1) / (2ull * n) + 8u;
  float lf = -__builtin_inff();
  if (want < static_cast<uint64_t>(n0)) {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    auto see = [&](bool ok, float x) {
      const uint32_t key = ok ? float_key(x) : 0u;
      kmax = key > kmax ? key : kmax;
      kmin = ok && key < kmin ? key : kmin;
    };
    see(has_x, xv);
#pragma unroll
    for (int v = 0; v < SR_V; ++v) {
      const bool ok = v * kWave + lane < r.nv;
#pragma unroll
      for (int c = 0; c < 4; ++c) see(ok, A[v][c]);
    }
    const float vmin = key_float(wave_min_u32(kmin)), vmax = key_float(wave_max_u32(kmax));
    const float width = vmax - vmin;
    if (width > 0.0f && width < __builtin_inff()) {
      const float scale = 256.0f / width;
      reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      auto add = [&](bool ok, float x) {
        if (ok) {
          float f = (x - vmin) * scale;
          f = f < 255.0f ? f : 255.0f;
          f = f > 0.0f ? f : 0.0f;
          atomicAdd(&hist[static_cast<uint32_t>(f)], 1u);
        }
      };
      add(has_x, xv);
#pragma unroll
      for (int v = 0; v < SR_V; ++v) {
        const bool ok = v * kWave + lane < r.nv;
#pragma unroll
        for (int c = 0; c < 4; ++c) add(ok, A[v][c]);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const uint4 c4 = reinterpret_cast<const uint4*>(hist)[lane];  // bins 4 lane .. 4 lane + 3
      const uint32_t cb[4] = {c4.x, c4.y, c4.z, c4.w};
      const uint32_t local = cb[0] + cb[1] + cb[2] + cb[3];
      const uint32_t incl = wave_prefix_incl(local);
      const uint32_t tot = __builtin_amdgcn_readlane(incl, kWave - 1);
      const uint32_t above = tot - incl;  // counts of higher lanes' bins
      const uint32_t rank = static_cast<uint32_t>(want);
      const bool mine = above < rank && above + local >= rank;
      uint32_t bin = 0;
      if (mine) {
        uint32_t acc = above;
        int i = 3;
        for (; i > 0; --i) {
          if (acc + cb[i] >= rank) break;
          acc += cb[i];
        }
        bin = 4 * lane + i;
      }
      bin = __builtin_amdgcn_readlane(bin, __builtin_ctzll(ballot(mine)));
      lf = vmin + static_cast<float>(bin) / scale;
    }
  }

  // Keep every element >= lf (ballot compaction; the count is uniform).
  uint32_t cnt = 0;
  auto take = [&](bool keep, float x, uint32_t pos) {
    const uint64_t m = ballot(keep);
    const uint32_t at = cnt + lanes_below(m);
    if (keep && at < static_cast<uint32_t>(SR_CAP)) wc[at] = rank_key(float_key(x), pos);
    cnt += static_cast<uint32_t>(__popcll(m));
  };
  auto filter_q = [&](int q, const f4 (&X)[SR_V]) {
#pragma unroll
    for (int v = 0; v < SR_V; ++v) {
      const int vi = q * SR_QV + v * kWave + lane;
      const bool ok = vi < r.nv;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        take(ok && X[v][c] >= lf, X[v][c], static_cast<uint32_t>(r.head + 4 * vi + c));
    }
  };
  take(has_x && xv >= lf, xv, xpos);
  if (nq > 0) filter_q(0, A);
  if (nq > 2) load_q(2, A);
  if (nq > 1) filter_q(1, B);
  if (nq > 3) load_q(3, B);
  if (nq > 2) filter_q(2, A);
  if (nq > 3) filter_q(3, B);
  if (cnt < k || cnt > static_cast<uint32_t>(SR_CAP)) return false;

  // The k-th key T of the kept ones, then the keys >= T (exactly k) out.
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  uint64_t keys[SR_PER];
  bool valid[SR_PER];
#pragma unroll
  for (int e = 0; e < SR_PER; ++e) {
    const uint32_t i = e * kWave + lane;
    valid[e] = i < cnt;
    keys[e] = valid[e] ? wc[i] : 0ull;
  }
  const uint64_t T = cnt > k ? wave_select<SR_PER>(keys, valid, k, hist) : 0ull;
  uint32_t at = 0;
#pragma unroll
  for (int e0 = 0; e0 < SR_PER; e0 += SR_EMIT) {
    bool keep[SR_EMIT];
    uint32_t pos[SR_EMIT], idx[SR_EMIT], pg[SR_EMIT];
    int32_t page[SR_EMIT];
#pragma unroll
    for (int e = 0; e < SR_EMIT; ++e) {
      keep[e] = valid[e0 + e] && keys[e0 + e] >= T;
      const uint64_t m = ballot(keep[e]);
      idx[e] = at + lanes_below(m);
      at += static_cast<uint32_t>(__popcll(m));
      IDXTOPK_CHECK(!keep[e] || rank_pos(keys[e0 + e]) < static_cast<uint32_t>(n), kChkPosition);
      pos[e] = rank_pos(keys[e0 + e]) + r.off;
      pg[e] = keep[e] ? fdiv(pos[e], a.pdiv) : 0u;
    }
    if (r.pt_row) {
      // all lookups issued before any is used; entries not kept read page 0
#pragma unroll
      for (int e = 0; e < SR_EMIT; ++e) page[e] = r.pt_row[pg[e]];
#pragma unroll
      for (int e = 0; e < SR_EMIT; ++e) IDXTOPK_CHECK(!keep[e] || page[e] >= 0, kChkPageId);
    }
#pragma unroll
    for (int e = 0; e < SR_EMIT; ++e)
      if (keep[e])
        __builtin_nontemporal_store(r.pt_row ? static_cast<int32_t>(static_cast<int64_t>(page[e]) * P + (pos[e] - pg[e] * P))
                                            : static_cast<int32_t>(pos[e]),
                                    r.out + idx[e]);
  }
  return true;
}

// Short rows are taken four to a workgroup, one wave per row. A group is
// the rows 32 m + x + 8 j (j = 0..3) for x = row % 8: workgroups are dealt
// to the 8 XCDs round-robin by index, so a group's rows, and the workgroup
// that takes them, sit on one XCD, and the groups spread over all eight.
// Inside an XCD, consecutive workgroups go to its shader engines in turn,
// so the workgroup that takes a group's short rows is its first short row
// counting from member m % 4: the taking workgroups then spread over the
// engines. The group's other short-row workgroups leave at once (a long row
// keeps its own workgroup). Rows whose estimate failed are then selected by
// the whole workgroup, one after another.
__device__ __forceinline__ int group_row(int base, int j) { return base + 8 * j; }

__device__ __forceinline__ void short_group(const RowsArgs& a, uint64_t* cand, TopkRowsLds& s) {
  const int base = (static_cast<int>(blockIdx.x) / 32) * 32 + static_cast<int>(blockIdx.x) % 8;
  const int wave = uniform(static_cast<int>(threadIdx.x) / kWave);
  const int m = static_cast<int>(blockIdx.x) / 32;
  int leader = -1;
  bool my_short = false;  // this wave's row is short
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int w = (m + t) & 3;
    const int row = group_row(base, w);
    const bool sh = row < a.rows && load_uniform(a.seq_lens + row) <= SR_MAX_N;
    if (leader < 0 && sh) leader = row;
    my_short = w == wave ? sh : my_short;
  }
  if (leader != static_cast<int>(blockIdx.x)) return;
  bool ok = true;
  if (my_short) {
    const RowCtx r = row_setup(a, group_row(base, wave));
    ok = short_row(a, r, cand + wave * SR_CAP, s.sel.hist + wave * (kSelBins / 4));
  }
  if (lane_id() == 0) s.sel.bcast[wave] = ok ? 0u : 1u;
  __syncthreads();
  uint32_t failed = 0;  // bit w: row g0 + w needs the workgroup path
#pragma unroll
  for (int w = 0; w < 4; ++w) failed |= s.sel.bcast[w] << w;
  failed = static_cast<uint32_t>(uniform(static_cast<int>(failed)));
  __syncthreads();
  while (failed) {
    const int w = __builtin_ctz(failed);
    failed &= failed - 1;
    wg_row<false>(a, row_setup(a, group_row(base, w)), cand, s);
    __syncthreads();
  }
}

template <bool SORTED>
__global__ __launch_bounds__(TR_WG, 4) void topk_rows_kernel(RowsArgs a) {
  extern __shared__ uint64_t cand[];
  __shared__ TopkRowsLds s;
  if (!SORTED && a.short_rows && load_uniform(a.seq_lens + blockIdx.x) <= SR_MAX_N) {
    short_group(a, cand, s);
    return;
  }
  wg_row<SORTED>(a, row_setup(a, blockIdx.x), cand, s);
}

// ---------------------------------------------------------------------------
// Launches of few short rows: one 1024-thread workgroup per row
// ---------------------------------------------------------------------------
//
// Rows of at most SM_MAX_N keys (every window of a score buffer whose row
// stride is at most SM_MAX_N), in launches too small to fill the chip. Each
// thread holds SM_PER consecutive keys in registers after one load round
// trip, and the k-th value key is located by a radix select over the 32-bit
// value keys, 8 bits per round from the top: each round histograms the digit
// of the keys that match the bits found so far (the prefix), and one wave
// finds the digit where the count from the top reaches the remaining rank.
// The select stops early when the keys matching the prefix number exactly
// the remaining rank. Every key above the prefix (in its bits) is kept, and
// of the keys matching it the remaining rank's count with the lowest
// positions (all of them after an early stop); one workgroup scan of the
// packed (above, matching) counts gives each thread both its output offset
// and its ties' ranks. The kept positions then go through the page table,
// their lookups issued together.
constexpr int SM_WG = 1024;
constexpr int SM_PER = 4;
constexpr int SM_MAX_N = SM_WG * SM_PER;
constexpr int SM_WAVES = SM_WG / kWave;

struct SmallRowLds {
  uint32_t hist[256];
  uint32_t wsum[SM_WAVES];
  uint32_t digit;
  uint32_t above;
  uint32_t count;  // keys with the found digit
};

__global__ __launch_bounds__(SM_WG) void topk_small_rows_kernel(RowsArgs a) {
  __shared__ SmallRowLds s;
  const RowCtx r = row_setup(a, blockIdx.x);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = uniform(tid / kWave);
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  IDXTOPK_CHECK(r.n <= SM_MAX_N, kChkWindow);
  const int n = r.n < SM_MAX_N ? r.n : SM_MAX_N;
  if (static_cast<uint32_t>(n) <= k) {
    for (int i = tid; i < static_cast<int>(k); i += SM_WG)
      r.out[i] = i < n ? map_slot(r.pt_row, static_cast<uint32_t>(i) + r.off, P, a.pdiv) : -1;
    return;
  }

  // this thread's keys: positions SM_PER tid .. SM_PER tid + SM_PER - 1
  uint32_t vk[SM_PER];
  bool ok[SM_PER];
#pragma unroll
  for (int e = 0; e < SM_PER; ++e) {
    const int p = SM_PER * tid + e;
    ok[e] = p < n;
    const float x = r.base[ok[e] ? p : 0];  // n > k >= 1 here, so position 0 exists
    vk[e] = ok[e] ? float_key(x) : 0u;
  }

  // Radix select: (prefix, pmask) ends as the bits of the k-th largest value
  // key that the rounds resolved, kk as the number of keys matching them
  // that are kept.
  uint32_t prefix = 0u, pmask = 0u, kk = k;
  for (int d = 0; d < 4; ++d) {
    const int shift = 24 - 8 * d;
    if (tid < 256) s.hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < SM_PER; ++e)
      if (ok[e] && (vk[e] & pmask) == prefix) atomicAdd(&s.hist[(vk[e] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 4 l .. 4 l + 3; counts from the top
      const uint4 c4 = reinterpret_cast<const uint4*>(s.hist)[lane];
      const uint32_t c[4] = {c4.x, c4.y, c4.z, c4.w};
      const uint32_t local = c[0] + c[1] + c[2] + c[3];
      const uint32_t incl = wave_prefix_incl(local);
      const uint32_t tot = __builtin_amdgcn_readlane(incl, kWave - 1);
      uint32_t above = tot - incl;  // keys in the digits of higher lanes
      if (above < kk && above + local >= kk) {
        int i = 3;
        for (; i > 0; --i) {
          if (above + c[i] >= kk) break;
          above += c[i];
        }
        s.digit = 4u * static_cast<uint32_t>(lane) + static_cast<uint32_t>(i);
        s.above = above;
        s.count = c[i];
      }
    }
    __syncthreads();
    kk -= s.above;
    prefix |= s.digit << shift;
    pmask |= 255u << shift;
    if (s.count == kk) break;  // every key matching the prefix is kept
  }

  // Offsets: one scan of (above the prefix) << 16 | (matching it) in
  // position order.
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int e = 0; e < SM_PER; ++e) {
    gt += ok[e] && (vk[e] & pmask) > prefix;
    eq += ok[e] && (vk[e] & pmask) == prefix;
  }
  const uint32_t mine = (gt << 16) | eq;
  const uint32_t incl = wave_prefix_incl(mine);
  if (lane == kWave - 1) s.wsum[wave] = incl;
  __syncthreads();
  uint32_t before = incl - mine;
  for (int w = 0; w < wave; ++w) before += s.wsum[w];
  const uint32_t eq_before = before & 0xffffu;
  uint32_t at = (before >> 16) + (eq_before < kk ? eq_before : kk);
  uint32_t tie = eq_before;

  bool keep[SM_PER];
  uint32_t idx[SM_PER], pos[SM_PER], pg[SM_PER];
  int32_t page[SM_PER];
#pragma unroll
  for (int e = 0; e < SM_PER; ++e) {
    keep[e] = false;
    if (ok[e] && (vk[e] & pmask) > prefix) {
      keep[e] = true;
    } else if (ok[e] && (vk[e] & pmask) == prefix) {
      keep[e] = tie < kk;
      ++tie;
    }
    idx[e] = at;
    at += keep[e];
    pos[e] = static_cast<uint32_t>(SM_PER * tid + e) + r.off;
    pg[e] = keep[e] && r.pt_row ? fdiv(pos[e], a.pdiv) : 0u;
    IDXTOPK_CHECK(!keep[e] || idx[e] < k, kChkPosition);
  }
  if (r.pt_row) {
    // all lookups issued before any is used; entries not kept read page 0
#pragma unroll
    for (int e = 0; e < SM_PER; ++e) page[e] = r.pt_row[pg[e]];
#pragma unroll
    for (int e = 0; e < SM_PER; ++e) IDXTOPK_CHECK(!keep[e] || page[e] >= 0, kChkPageId);
  }
#pragma unroll
  for (int e = 0; e < SM_PER; ++e)
    if (keep[e] && idx[e] < k)
      r.out[idx[e]] = r.pt_row ? static_cast<int32_t>(static_cast<int64_t>(page[e]) * P + (pos[e] - pg[e] * P))
                               : static_cast<int32_t>(pos[e]);
}

// Candidate buffer entries: at least two tiles (the first tile is appended
// whole in the worst case), and k plus one and a half tiles so that a
// compaction frees at least a quarter tile beyond the next tile.
static inline int rows_cap(int k) {
  const int a = k + TR_TILE + TR_TILE / 2, b = 2 * TR_TILE;
  return (a > b ? a : b) + 8;
}

// What the streaming loop relies on (checked before every launch):
//  * the first tile plus the scalar head and tail (at most 3 each) fits
//    before any compaction: cap >= TR_TILE + 6;
//  * after_tile's slack (cap - TR_TILE - k) / 2, computed in uint32, is at
//    least 1: a smaller buffer would wrap it to ~2^31, the compaction select
//    would stop after one histogram and keep nearly every key, and the next
//    tile would be appended past the end of the buffer;
//  * after a compaction the buffer holds at most k + slack keys, so the next
//    tile fits: k + slack + TR_TILE <= cap, which the slack's definition
//    gives for any cap above.
static inline bool rows_cap_ok(int cap, int k) {
  return cap >= TR_TILE + 6 && static_cast<int64_t>(cap) - TR_TILE - k >= 2;
}

uint32_t check_word_topk_rows(bool clear) {
#if IDXTOPK_CHECKS
  return read_check_word(clear);
#else
  (void)clear;
  return 0;
#endif
}

int launch_topk_rows(const float* scores, int64_t stride, int rows, const int32_t* seq_lens,
                     const int32_t* row_starts, const int32_t* row_to_batch, const int32_t* kv_offset,
                     const int32_t* page_table, int64_t pt_stride, int page_size, int k,
                     int32_t* out, bool sorted, hipStream_t stream) {
  RowsArgs a;
  a.scores = scores;
  a.stride = stride;
  a.seq_lens = seq_lens;
  a.row_starts = row_starts;
  a.row_to_batch = row_to_batch;
  a.kv_offset = kv_offset;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.page_size = page_size > 0 ? page_size : 1;
  a.pdiv = make_fastdiv(static_cast<uint32_t>(a.page_size));
  a.k = k;
  a.out = out;
  a.cap = rows_cap(k);
  int npow = 512;  // at least two keys per thread
  while (npow < k) npow <<= 1;
  a.npow = npow;
  if (sorted && a.cap < npow) a.cap = npow;
  if (!rows_cap_ok(a.cap, k)) return -4;
  a.rows = rows;
  // Launches of few rows whose windows hold at most SM_MAX_N keys (the row
  // stride bounds every window): one 1024-thread workgroup per row.
  if (!sorted && rows < SR_MIN_ROWS && stride <= SM_MAX_N) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(topk_small_rows_kernel, dim3(rows), dim3(SM_WG), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -4;
  }
  // One wave per short row: it takes longer per row than a workgroup does,
  // so it pays only when there are rows enough to fill the chip (and it
  // needs four wave areas in the candidate buffer).
  a.short_rows = !sorted && k <= SR_MAX_K && a.cap >= 4 * SR_CAP && rows >= SR_MIN_ROWS;
  const size_t lds = static_cast<size_t>(a.cap) * sizeof(uint64_t);
  const void* kern = sorted ? reinterpret_cast<const void*>(&topk_rows_kernel<true>)
                            : reinterpret_cast<const void*>(&topk_rows_kernel<false>);
  static std::atomic<size_t> granted[2] = {{0}, {0}};
  if (allow_dynamic_lds(kern, lds, granted[sorted]) != hipSuccess) return -4;
  (void)hipGetLastError();
  if (sorted)
    hipLaunchKernelGGL(topk_rows_kernel<true>, dim3(rows), dim3(TR_WG), lds, stream, a);
  else
    hipLaunchKernelGGL(topk_rows_kernel<false>, dim3(rows), dim3(TR_WG), lds, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace idxtopk
