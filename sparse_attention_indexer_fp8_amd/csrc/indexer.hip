// Paged fp8 indexer kernels: unfused scores, fused decode top-k, block top-k.
//
// Pages:
//  [ATOM-1473] ROCm/ATOM PR 1473 "enable minimax m3 fp8 index cache and fuse
//   index_score_kernel with partial_topk kernel": fp8 index cache, fp8 dot
//   products, the decode kernel's block-table walk with a causal-length mask,
//   and a fused score + partial top-k kernel whose grid has a chunk axis and
//   whose chunk results go to caller-visible partial buffers.
//  [ATOM-1282] ROCm/ATOM PR 1282 "merge build sparse block into topk":
//   128-token blocks; the sparse block list is built inside the top-k kernel.
//
// Grid: one workgroup per (row, chunk) pair, chunk-major (all rows' chunk 0
// first), the row index rotated per chunk so each row's chunks spread over
// all XCDs. Chunks past a row's length exit at once. Every workgroup scores
// its chunk with the fp8 MFMA core (score_mfma.hpp).
//
// Fused decode (idx_score_topk_fused), per chunk:
//  1. Scores stay in LDS. A 4096-bin LDS histogram of the value keys' top 12
//     bits is built on the fly.
//  2. The chunk adds its histogram into the row's global histogram, then reads
//     the global histogram back. The highest bin whose count from the top
//     reaches k is a valid lower bound on the row's k-th score: every count
//     seen belongs to a real token, whichever chunks have added so far.
//  3. The chunk emits only tokens in bins >= that bound, as unique 64-bit
//     keys (score key, inverted position), to the row's candidate list in
//     the workspace.
//  4. A second kernel merges, one workgroup per row, once every chunk is
//     done. The complete histogram names the exact threshold bin.
//     Candidates above it are emitted directly. Candidates in it go to LDS,
//     and an exact select takes the remaining count. Output goes through the
//     block table to slots. The merging workgroup then zeroes the row's
//     histogram, counters and candidates, so the workspace is clean for the
//     next call.
// The score row never exists in HBM.
#include "common.hpp"
#include "launch.hpp"
#include "score_mfma.hpp"
#include "select.hpp"

namespace idxtopk {

constexpr int IX_WG = 256;
constexpr int IX_RING = 4;  // 16-token key groups in flight per wave
constexpr int HIST_BITS = 12;
constexpr int HIST_BINS = 1 << HIST_BITS;
constexpr int HIST_SHIFT = 32 - HIST_BITS;
constexpr int FU_CH_MAX = 8192;
constexpr int IX_PAGES = 512;

static_assert(IX_PAGES <= kMaxChunkPages, "page staging");

// ---------------------------------------------------------------------------
// Workspace layouts
// ---------------------------------------------------------------------------

static inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct FusedWs {
  uint32_t* hist;  // [rows][HIST_BINS]
  uint32_t* ctr;   // [rows][4]: candidate count, done chunks
  uint64_t* cand;  // [rows][cap]
  int64_t cap;
};

static inline FusedWs fused_ws(void* base, int rows, int max_seq_len) {
  char* p = static_cast<char*>(base);
  FusedWs w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(rows) * HIST_BINS * 4);
  w.ctr = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(rows) * 16);
  w.cand = reinterpret_cast<uint64_t*>(p);
  w.cap = max_seq_len > 0 ? max_seq_len : 1;
  return w;
}

size_t fused_workspace_bytes(int rows, int k, int max_seq_len) {
  (void)k;
  const int64_t cap = max_seq_len > 0 ? max_seq_len : 1;
  return align256(static_cast<size_t>(rows) * HIST_BINS * 4) + align256(static_cast<size_t>(rows) * 16) +
         align256(static_cast<size_t>(rows) * cap * 8);
}

struct BlockWs {
  uint32_t* bscore;  // [rows][nblk_max] value keys of the block maxima
  uint32_t* ctr;     // [rows][4]: done chunks
  int64_t nblk_max;
};

static inline BlockWs block_ws(void* base, int rows, int block_size, int max_seq_len) {
  char* p = static_cast<char*>(base);
  BlockWs w;
  w.nblk_max = max_seq_len > 0 ? (max_seq_len + block_size - 1) / block_size : 1;
  w.bscore = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(rows) * w.nblk_max * 4);
  w.ctr = reinterpret_cast<uint32_t*>(p);
  return w;
}

size_t block_workspace_bytes(int rows, int block_size, int max_seq_len) {
  const int64_t nblk = max_seq_len > 0 ? (max_seq_len + block_size - 1) / block_size : 1;
  return align256(static_cast<size_t>(rows) * nblk * 4) + align256(static_cast<size_t>(rows) * 16);
}

// Workgroup -> (row b, chunk c), chunk-major. Workgroups are dealt to the
// XCDs round-robin by index; with a plain b = index % batch each XCD would
// own a fixed subset of rows (every row whose index is congruent to it modulo
// the XCD count) and the XCDs holding the longest rows would finish last. The
// row index is therefore rotated by the chunk index: a row's chunks land on
// every XCD in turn.
__device__ __forceinline__ void chunk_of(const IndexerArgs& a, int& b, int& c) {
  c = blockIdx.x / a.batch;
  b = (blockIdx.x + c) % a.batch;
}

// First token and token count of chunk c under the guided schedule: the
// grid is chunk-major, so the last workgroups dispatched are the short ones
// and the tail of the launch stays short.
__device__ __forceinline__ void chunk_span(const IndexerArgs& a, int c, int& tb, int& len) {
  if (c < a.n_full) {
    tb = c * a.chunk;
    len = a.chunk;
  } else if (c < a.n_full + a.n_half) {
    len = a.chunk / 2;
    tb = a.tok_half + (c - a.n_full) * len;
  } else {
    len = a.chunk / 4;
    tb = a.tok_quarter + (c - a.n_full - a.n_half) * len;
  }
}

__device__ __forceinline__ int32_t token_slot(const IndexerArgs& a, int b, uint32_t pos) {
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  const uint32_t pg = fdiv(pos, a.pdiv);
  const uint32_t off = pos - pg * P;
  const int32_t page = a.block_table[static_cast<int64_t>(b) * a.bt_stride + pg];
  return static_cast<int32_t>(static_cast<int64_t>(page) * P + off);
}

// ---------------------------------------------------------------------------
// Unfused scores
// ---------------------------------------------------------------------------

template <int NT>
__global__ __launch_bounds__(IX_WG) void score_kernel(IndexerArgs a, float* scores, int64_t sstride) {
  __shared__ int32_t pages[IX_PAGES];
  int b, c;
  chunk_of(a, b, c);
  const int n = a.seq_lens[b];
  int tb, clen;
  chunk_span(a, c, tb, clen);
  if (tb >= n) return;
  const int te = min(n, tb + clen);
  float* srow = scores + static_cast<int64_t>(b) * sstride;
  score_chunk<NT, IX_WG, IX_RING>(a, b, tb, te, pages, [&](int j, float s, bool valid) {
    if (valid) srow[j] = s;
  });
}

// ---------------------------------------------------------------------------
// Fused decode score + top-k: chunk kernel, then per-row merge kernel
// ---------------------------------------------------------------------------

constexpr int MG_WG = 512;                      // merge workgroup
constexpr int MG_BUF = 6144;                    // threshold-bin entries held in LDS (48 KB)
constexpr int MG_MAXE = MG_BUF / MG_WG;

static_assert(HIST_BINS == 16 * IX_WG, "16 histogram bins per thread");

// The 16 counts of bins [16 t, 16 t + 16) of an LDS histogram, for thread t
// (four 16-byte reads).
__device__ __forceinline__ void own_bins16(const uint32_t* hist, uint32_t (&c)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(hist) + threadIdx.x * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 v = p[j];
    c[4 * j + 0] = v.x;
    c[4 * j + 1] = v.y;
    c[4 * j + 2] = v.z;
    c[4 * j + 3] = v.w;
  }
}

constexpr uint32_t FU_STAGE = HIST_BINS / 2;  // candidates staged in the histogram's LDS

struct ChunkLds {
  union {
    alignas(16) uint32_t hist[HIST_BINS];  // the chunk's histogram, until its bound is known
    uint64_t stage[FU_STAGE];              // then the chunk's candidates
  };
  int32_t pages[IX_PAGES];
  uint32_t scratch[16];
  uint32_t lcnt;
  uint32_t lcnt2;
  uint32_t gbase;
};

struct FusedOut {
  int32_t* slots;
  float* scores;
  int k;
};

// Dynamic LDS: the chunk's scores (a.chunk floats).
template <int NT>
__global__ __launch_bounds__(IX_WG) void fused_chunk_kernel(IndexerArgs a, FusedWs ws, int k) {
  extern __shared__ float sc[];
  __shared__ ChunkLds s;
  const int tid = threadIdx.x;
  int b, c;
  chunk_of(a, b, c);
  const int n = a.seq_lens[b];
  int tb, clen;
  chunk_span(a, c, tb, clen);
  if (tb >= n) return;
  const int te = min(n, tb + clen);
  const int cnt = te - tb;
  uint32_t* Hg = ws.hist + static_cast<int64_t>(b) * HIST_BINS;
  uint32_t* ctr = ws.ctr + static_cast<int64_t>(b) * 4;
  uint64_t* cand = ws.cand + static_cast<int64_t>(b) * ws.cap;

  for (int i = tid; i < HIST_BINS; i += IX_WG) s.hist[i] = 0;
  if (tid == 0) {
    s.lcnt = 0;
    s.lcnt2 = 0;
  }
  // (score_chunk synchronises before its first emit)
  score_chunk<NT, IX_WG, IX_RING>(a, b, tb, te, s.pages, [&](int j, float v, bool valid) {
    if (valid) {
      sc[j - tb] = v;
      atomicAdd(&s.hist[float_key(v) >> HIST_SHIFT], 1u);
    }
  });
  __syncthreads();

  // 1. The chunk's own threshold bin: the row holds these tokens, so the
  //    row's threshold bin is at least this one, and counts of lower bins
  //    can never decide it.
  uint32_t c16[16];
  own_bins16(s.hist, c16);
  const BinThreshold own = wg_threshold_counts<IX_WG, 16>(c16, static_cast<uint32_t>(k), s.scratch);
  const uint32_t lo_bin = own.all ? 0u : own.bin;
  // 2. Publish the counts of bins >= lo_bin to the row's histogram, then read
  //    the row's counts back (coalesced: bin i * IX_WG + tid; all loads issued
  //    before any is used; bins below lo_bin re-read lo_bin's counter).
  uint32_t g16[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t bin = i * IX_WG + tid;
    const uint32_t h = s.hist[bin];
    if (h && bin >= lo_bin) add_dev(&Hg[bin], h);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t bin = i * IX_WG + tid;
    g16[i] = ld_acquire_dev(&Hg[bin >= lo_bin ? bin : lo_bin]);
  }
  // 3. Bound the row's k-th score with what the row's histogram holds so far.
  //    Per bin, max(row count seen, own count) never exceeds the number of
  //    real tokens in that bin, so the threshold bin of these counts is a
  //    valid lower bound whatever has become visible; bins below lo_bin
  //    cannot hold it. (Each thread rewrites only the bins it read.)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t bin = i * IX_WG + tid;
    const uint32_t l = s.hist[bin];
    s.hist[bin] = bin >= lo_bin ? (g16[i] > l ? g16[i] : l) : 0u;
  }
  __syncthreads();
  own_bins16(s.hist, c16);
  const BinThreshold bound = wg_threshold_counts<IX_WG, 16>(c16, static_cast<uint32_t>(k), s.scratch);
  const uint32_t bin_g = bound.all ? 0u : bound.bin;

  // 4. Emit this chunk's candidates (bin >= bound) to the row's list: staged
  //    in LDS (over the histogram, which is no longer read) with one slot
  //    reservation per wave per batch, then one global reservation and a
  //    coalesced copy. If more than FU_STAGE pass, a second pass writes them
  //    straight to the list instead.
  constexpr int EB = 8;
  for (int i0 = 0; i0 < cnt; i0 += EB * IX_WG) {
    uint32_t key[EB];
    bool keep[EB];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int i = i0 + j * IX_WG + tid;
      key[j] = float_key(sc[i < cnt ? i : 0]);
      keep[j] = i < cnt && (key[j] >> HIST_SHIFT) >= bin_g;
      mine += keep[j];
    }
    uint32_t at = wave_reserve(mine, &s.lcnt);
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      if (keep[j]) {
        if (at < FU_STAGE) s.stage[at] = rank_key(key[j], static_cast<uint32_t>(tb + i0 + j * IX_WG + tid));
        ++at;
      }
    }
  }
  __syncthreads();
  const uint32_t m = s.lcnt;
  if (tid == 0) s.gbase = m ? add_dev(&ctr[0], m) : 0u;
  __syncthreads();
  const uint32_t gbase = s.gbase;
  if (m <= FU_STAGE) {
    for (uint32_t i = tid; i < m; i += IX_WG) cand[gbase + i] = s.stage[i];
  } else {
    for (int i0 = 0; i0 < cnt; i0 += EB * IX_WG) {
      uint32_t key[EB];
      bool keep[EB];
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        const int i = i0 + j * IX_WG + tid;
        key[j] = float_key(sc[i < cnt ? i : 0]);
        keep[j] = i < cnt && (key[j] >> HIST_SHIFT) >= bin_g;
        mine += keep[j];
      }
      uint32_t at = gbase + wave_reserve(mine, &s.lcnt2);
#pragma unroll
      for (int j = 0; j < EB; ++j)
        if (keep[j]) cand[at++] = rank_key(key[j], static_cast<uint32_t>(tb + i0 + j * IX_WG + tid));
    }
  }
}

struct MergeLds {
  uint64_t buf[MG_BUF];
  SelectLds sel;
  uint32_t scratch[24];
  uint32_t ocnt;
  uint32_t bcnt;
};

// Emit this thread's keys with keep[e] set: one slot reservation per wave,
// then independent block-table gathers and stores. All lanes of the wave must
// call.
template <int N>
__device__ __forceinline__ void emit_batch(const uint64_t (&keys)[N], const bool (&keep)[N],
                                           const IndexerArgs& a, int b, const FusedOut& o,
                                           uint32_t* ocnt) {
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) mine += keep[e];
  uint32_t at = wave_reserve(mine, ocnt);
  int32_t sl[N];
#pragma unroll
  for (int e = 0; e < N; ++e)
    if (keep[e]) sl[e] = token_slot(a, b, rank_pos(keys[e]));
  const int64_t row = static_cast<int64_t>(b) * o.k;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if (keep[e]) {
      if (at < static_cast<uint32_t>(o.k)) {
        o.slots[row + at] = sl[e];
        if (o.scores) o.scores[row + at] = key_float(rank_vkey(keys[e]));
      }
      ++at;
    }
  }
}

constexpr int MG_BATCH = 8;  // candidates per thread per pass of the merge

// One workgroup per row. The row's histogram is complete now (previous
// kernel), so it names the exact threshold bin: candidates above it are
// selected outright, candidates inside it go through an exact radix select
// for the remaining count. Then every workspace byte the row used is zeroed.
__global__ __launch_bounds__(MG_WG) void fused_merge_kernel(IndexerArgs a, FusedWs ws, FusedOut o) {
  __shared__ MergeLds s;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int n = a.seq_lens[b];
  const uint32_t k = static_cast<uint32_t>(o.k);
  uint32_t* Hg = ws.hist + static_cast<int64_t>(b) * HIST_BINS;
  uint32_t* ctr = ws.ctr + static_cast<int64_t>(b) * 4;
  uint64_t* cand = ws.cand + static_cast<int64_t>(b) * ws.cap;
  const uint32_t ncand = n > 0 ? ctr[0] : 0u;

  wg_select_init<MG_WG>(s.sel);
  if (tid == 0) {
    s.ocnt = 0;
    s.bcnt = 0;
  }
  const BinThreshold th = wg_threshold_bin<MG_WG, HIST_BINS>([&](int i) { return Hg[i]; }, k, s.scratch);
  const uint32_t bstar = th.all ? 0u : th.bin;
  const uint32_t need = th.all ? 0u : k - th.above;
  // Pass over the candidates: keys above the threshold bin (or all keys when
  // the row holds fewer than k) are emitted, keys inside it go to LDS.
  for (uint32_t i0 = 0; i0 < ncand; i0 += MG_WG * MG_BATCH) {
    uint64_t key[MG_BATCH];
    bool keep[MG_BATCH], mid[MG_BATCH];
    uint32_t nmid = 0;
#pragma unroll
    for (int j = 0; j < MG_BATCH; ++j) {
      const uint32_t i = i0 + j * MG_WG + tid;
      const bool valid = i < ncand;
      key[j] = valid ? cand[i] : 0ull;
      const uint32_t bin = rank_vkey(key[j]) >> HIST_SHIFT;
      keep[j] = valid && (th.all || bin > bstar);
      mid[j] = valid && !th.all && bin == bstar;
      nmid += mid[j];
    }
    emit_batch<MG_BATCH>(key, keep, a, b, o, &s.ocnt);
    uint32_t at = wave_reserve(nmid, &s.bcnt);
#pragma unroll
    for (int j = 0; j < MG_BATCH; ++j) {
      if (mid[j]) {
        if (at < static_cast<uint32_t>(MG_BUF)) s.buf[at] = key[j];
        ++at;
      }
    }
  }
  __syncthreads();
  const uint32_t nb = s.bcnt;
  if (!th.all && nb > 0) {
    if (nb <= static_cast<uint32_t>(MG_BUF)) {
      uint64_t keys[MG_MAXE];
      int nvk = 0;
#pragma unroll
      for (int e = 0; e < MG_MAXE; ++e) {
        const uint32_t i = tid + e * MG_WG;
        keys[e] = 0;
        if (i < nb) {
          keys[e] = s.buf[i];
          nvk = e + 1;
        }
      }
      uint64_t T = 0;  // keys >= T are selected
      if (nb > need) {
        uint64_t mn = ~0ull, mx = 0;
#pragma unroll
        for (int e = 0; e < MG_MAXE; ++e)
          if (e < nvk) {
            mn = keys[e] < mn ? keys[e] : mn;
            mx = keys[e] > mx ? keys[e] : mx;
          }
        wg_range<MG_WG>(mn, mx, s.sel);
        T = wg_select<MG_WG>(
            [&](auto&& f) {
#pragma unroll
              for (int e = 0; e < MG_MAXE; ++e)
                if (e < nvk) f(keys[e]);
            },
            need, mn, mx, s.sel);
      }
      bool keep[MG_MAXE];
#pragma unroll
      for (int e = 0; e < MG_MAXE; ++e) keep[e] = e < nvk && keys[e] >= T;
      emit_batch<MG_MAXE>(keys, keep, a, b, o, &s.ocnt);
    } else {
      // threshold bin larger than the LDS buffer: select straight from the
      // candidate list (several passes over it)
      auto each_mid = [&](auto&& f) {
        for (uint32_t i = tid; i < ncand; i += MG_WG) {
          const uint64_t key = cand[i];
          if ((rank_vkey(key) >> HIST_SHIFT) == bstar) f(key);
        }
      };
      uint64_t mn = ~0ull, mx = 0;
      each_mid([&](uint64_t key) {
        mn = key < mn ? key : mn;
        mx = key > mx ? key : mx;
      });
      wg_range<MG_WG>(mn, mx, s.sel);
      const uint64_t T = wg_select<MG_WG>(each_mid, need, mn, mx, s.sel);
      for (uint32_t i0 = 0; i0 < ncand; i0 += MG_WG * MG_BATCH) {
        uint64_t key[MG_BATCH];
        bool keep[MG_BATCH];
#pragma unroll
        for (int j = 0; j < MG_BATCH; ++j) {
          const uint32_t i = i0 + j * MG_WG + tid;
          key[j] = i < ncand ? cand[i] : 0ull;
          keep[j] = i < ncand && (rank_vkey(key[j]) >> HIST_SHIFT) == bstar && key[j] >= T;
        }
        emit_batch<MG_BATCH>(key, keep, a, b, o, &s.ocnt);
      }
    }
  }
  __syncthreads();
  // padding for rows shorter than k
  for (uint32_t i = min(s.ocnt, k) + tid; i < k; i += MG_WG) {
    o.slots[static_cast<int64_t>(b) * o.k + i] = -1;
    if (o.scores) o.scores[static_cast<int64_t>(b) * o.k + i] = -__builtin_inff();
  }
  // leave every workspace byte of this row zero again (any later call, of any
  // shape or op, may lay its counters over these bytes)
  for (uint32_t i = tid; i < ncand; i += MG_WG) cand[i] = 0;
  if (n > 0)
    for (int i = tid; i < HIST_BINS; i += MG_WG) Hg[i] = 0;
  if (tid == 0) ctr[0] = 0;
}

// ---------------------------------------------------------------------------
// Block-sparse top-k: chunk kernel (block maxima), then per-row merge kernel
// ---------------------------------------------------------------------------

constexpr int BK_MAX_BLOCKS_PER_CHUNK = 512;
constexpr int BK_MAX_TOP = 4096;  // IDXTOPK_MAX_TOP_BLOCKS

struct BlockChunkLds {
  int32_t pages[IX_PAGES];
  uint32_t bmax[BK_MAX_BLOCKS_PER_CHUNK];
};

struct BlockMergeLds {
  int32_t sel_blocks[BK_MAX_TOP];
  SelectLds sel;
  uint32_t ocnt;
};

struct BlockOut {
  int32_t* blocks;
  int32_t* slots;
  int top;
  int bs;
};

template <int NT>
__global__ __launch_bounds__(IX_WG) void block_chunk_kernel(IndexerArgs a, BlockWs ws, int bs) {
  __shared__ BlockChunkLds s;
  const int tid = threadIdx.x;
  int b, c;
  chunk_of(a, b, c);
  const int n = a.seq_lens[b];
  int tb, clen;
  chunk_span(a, c, tb, clen);
  if (tb >= n) return;
  const int te = min(n, tb + clen);
  const int nbc = (te - tb + bs - 1) / bs;
  uint32_t* bsc = ws.bscore + static_cast<int64_t>(b) * ws.nblk_max;

  for (int i = tid; i < nbc; i += IX_WG) s.bmax[i] = 0;
  // block size equals page size, so the page division gives the block index
  // A 16-token group lies inside one block (block size and chunk starts are
  // multiples of 16), so the group's maximum is taken in registers (DPP over
  // the 16 lanes of each row) and one lane updates the block.
  score_chunk<NT, IX_WG, IX_RING>(a, b, tb, te, s.pages, [&](int j, float v, bool valid) {
    uint32_t key = valid ? float_key(v) : 0u;
    key = row16_max(key);
    if (lane_id() == 0 && key) atomicMax(&s.bmax[fdiv(static_cast<uint32_t>(j - tb), a.pdiv)], key);
  });
  __syncthreads();
  const int blk0 = tb / bs;
  for (int i = tid; i < nbc; i += IX_WG) bsc[blk0 + i] = s.bmax[i];
}

__global__ __launch_bounds__(MG_WG) void block_merge_kernel(IndexerArgs a, BlockWs ws, BlockOut o) {
  __shared__ BlockMergeLds s;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int n = a.seq_lens[b];
  const int bs = o.bs;
  const int top = o.top;
  const int nblk = (n + bs - 1) / bs;
  uint32_t* bsc = ws.bscore + static_cast<int64_t>(b) * ws.nblk_max;

  wg_select_init<MG_WG>(s.sel);
  if (tid == 0) s.ocnt = 0;
  __syncthreads();
  if (nblk <= top) {
    for (int i = tid; i < nblk; i += MG_WG) s.sel_blocks[i] = i;
    if (tid == 0) s.ocnt = static_cast<uint32_t>(nblk);
  } else {
    auto each = [&](auto&& f) {
      for (int cb = tid; cb < nblk; cb += MG_WG) f(rank_key(bsc[cb], static_cast<uint32_t>(cb)));
    };
    uint64_t mn = ~0ull, mx = 0;
    each([&](uint64_t key) {
      mn = key < mn ? key : mn;
      mx = key > mx ? key : mx;
    });
    wg_range<MG_WG>(mn, mx, s.sel);
    const uint64_t T = wg_select<MG_WG>(each, static_cast<uint32_t>(top), mn, mx, s.sel);
    for (int c0 = 0; c0 < nblk; c0 += MG_WG) {
      const int cb = c0 + tid;
      const bool keep = cb < nblk && rank_key(bsc[cb], static_cast<uint32_t>(cb)) >= T;
      const uint64_t mk = ballot(keep);
      if (mk == 0) continue;
      uint32_t wb = 0;
      if (lane_id() == 0) wb = atomicAdd(&s.ocnt, static_cast<uint32_t>(__popcll(mk)));
      wb = uniform(wb);
      const uint32_t at = wb + lanes_below(mk);
      if (keep && at < static_cast<uint32_t>(top)) s.sel_blocks[at] = cb;
    }
  }
  __syncthreads();
  const int nsel = min(static_cast<int>(s.ocnt), top);
  const int32_t* bt_row = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  for (int i = tid; i < top; i += MG_WG)
    o.blocks[static_cast<int64_t>(b) * top + i] = i < nsel ? bt_row[s.sel_blocks[i]] : -1;
  if (o.slots) {
    const int64_t slot_row = static_cast<int64_t>(b) * top * bs;
    for (int e = tid; e < top * bs; e += MG_WG) {
      const int i = e / bs;
      const int t = e - i * bs;
      int32_t v = -1;
      if (i < nsel) {
        const int cb = s.sel_blocks[i];
        if (cb * bs + t < n) v = static_cast<int32_t>(static_cast<int64_t>(bt_row[cb]) * bs + t);
      }
      o.slots[slot_row + e] = v;
    }
  }
  // leave every workspace byte of this row zero again
  __syncthreads();
  for (int cb = tid; cb < nblk; cb += MG_WG) bsc[cb] = 0;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static IndexerArgs make_args(const IndexerInputs& in, int chunk, bool guided = false, int guide_align = 16) {
  IndexerArgs a;
  a.q = in.q;
  a.q_scale = in.q_scale;
  a.w = in.w;
  a.kcache = in.kcache;
  a.k_scale = in.k_scale;
  a.block_table = in.block_table;
  a.bt_stride = in.bt_stride;
  a.page_size = in.page_size;
  a.pdiv = make_fastdiv(static_cast<uint32_t>(in.page_size));
  a.seq_lens = in.seq_lens;
  a.batch = in.batch;
  a.heads = in.heads;
  a.chunk = chunk;
  const int msl = in.max_seq_len > 0 ? in.max_seq_len : 1;
  // Guided schedule when quarter chunks stay large (and aligned): full-size
  // chunks up to half the longest row, halves up to three quarters, then
  // quarters.
  const int quarter = chunk / 4;
  if (guided && chunk % 4 == 0 && quarter >= 1024 && quarter % guide_align == 0 && msl > 2 * chunk) {
    a.n_full = (msl / 2) / chunk;
    a.tok_half = a.n_full * chunk;
    a.n_half = ((msl - a.tok_half) / 2) / (chunk / 2);
    a.tok_quarter = a.tok_half + a.n_half * (chunk / 2);
    a.nchunk_max = a.n_full + a.n_half + (msl - a.tok_quarter + quarter - 1) / quarter;
  } else {
    a.n_full = (msl + chunk - 1) / chunk;
    a.n_half = 0;
    a.tok_half = a.tok_quarter = a.n_full * chunk;
    a.nchunk_max = a.n_full;
  }
  return a;
}

// Tokens per workgroup: aim for ~2048 workgroups over the whole batch, keep
// the chunk's block-table entries within the LDS staging area, keep it a
// multiple of `align`, and stay within [lo, hi].
static int choose_chunk(int batch, int max_seq_len, int page_size, int align, int lo, int hi) {
  const int64_t total = static_cast<int64_t>(batch) * (max_seq_len > 0 ? max_seq_len : 1);
  int64_t ch = lo;
  while (ch < hi && total / ch > 2048) ch *= 2;
  const int64_t page_cap = static_cast<int64_t>(IX_PAGES - 2) * page_size;
  if (ch > page_cap) ch = page_cap;
  ch = (ch / align) * align;
  if (ch < align) ch = align;
  return static_cast<int>(ch);
}

#define IDXTOPK_DISPATCH_NT_LDS(KERNEL, heads, grid, lds, stream, ...)                               \
  do {                                                                                            \
    switch (heads) {                                                                              \
      case 16: hipLaunchKernelGGL(KERNEL<1>, grid, dim3(IX_WG), lds, stream, __VA_ARGS__); break;   \
      case 32: hipLaunchKernelGGL(KERNEL<2>, grid, dim3(IX_WG), lds, stream, __VA_ARGS__); break;   \
      case 64: hipLaunchKernelGGL(KERNEL<4>, grid, dim3(IX_WG), lds, stream, __VA_ARGS__); break;   \
      case 128: hipLaunchKernelGGL(KERNEL<8>, grid, dim3(IX_WG), lds, stream, __VA_ARGS__); break;  \
      default: return -2;                                                                         \
    }                                                                                             \
  } while (0)
#define IDXTOPK_DISPATCH_NT(KERNEL, heads, grid, stream, ...) \
  IDXTOPK_DISPATCH_NT_LDS(KERNEL, heads, grid, 0, stream, __VA_ARGS__)

int launch_idx_score(const IndexerInputs& in, float* scores, int64_t score_stride, hipStream_t stream) {
  if (in.batch == 0) return 0;
  const int chunk = choose_chunk(in.batch, in.max_seq_len, in.page_size, kGroup, 512, 8192);
  const IndexerArgs a = make_args(in, chunk, true);
  const dim3 grid(static_cast<unsigned>(a.nchunk_max * in.batch));
  (void)hipGetLastError();
  IDXTOPK_DISPATCH_NT(score_kernel, in.heads, grid, stream, a, scores, score_stride);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_fused(const IndexerInputs& in, int k, int32_t* out_slots, float* out_scores, void* ws,
                 hipStream_t stream) {
  if (in.batch == 0) return 0;
  const int chunk = choose_chunk(in.batch, in.max_seq_len, in.page_size, kGroup, 512, FU_CH_MAX);
  const IndexerArgs a = make_args(in, chunk, true);
  const FusedWs w = fused_ws(ws, in.batch, in.max_seq_len);
  FusedOut o;
  o.slots = out_slots;
  o.scores = out_scores;
  o.k = k;
  const dim3 grid(static_cast<unsigned>(a.nchunk_max * in.batch));
  (void)hipGetLastError();
  // the scores' dynamic LDS plus the static part stay within 64 KB
  static_assert(FU_CH_MAX * 4 + sizeof(ChunkLds) <= 64 * 1024, "fused chunk LDS");
  const size_t lds = static_cast<size_t>(chunk) * sizeof(float);
  IDXTOPK_DISPATCH_NT_LDS(fused_chunk_kernel, in.heads, grid, lds, stream, a, w, k);
  hipLaunchKernelGGL(fused_merge_kernel, dim3(in.batch), dim3(MG_WG), 0, stream, a, w, o);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_block_topk(const IndexerInputs& in, int block_size, int top_blocks, int32_t* out_blocks,
                      int32_t* out_slots, void* ws, hipStream_t stream) {
  if (in.batch == 0) return 0;
  int chunk = choose_chunk(in.batch, in.max_seq_len, in.page_size, block_size, 512, 8192);
  if (chunk / block_size > BK_MAX_BLOCKS_PER_CHUNK) chunk = BK_MAX_BLOCKS_PER_CHUNK * block_size;
  const IndexerArgs a = make_args(in, chunk, true, block_size);
  const BlockWs w = block_ws(ws, in.batch, block_size, in.max_seq_len);
  BlockOut o;
  o.blocks = out_blocks;
  o.slots = out_slots;
  o.top = top_blocks;
  o.bs = block_size;
  const dim3 grid(static_cast<unsigned>(a.nchunk_max * in.batch));
  (void)hipGetLastError();
  IDXTOPK_DISPATCH_NT(block_chunk_kernel, in.heads, grid, stream, a, w, block_size);
  hipLaunchKernelGGL(block_merge_kernel, dim3(in.batch), dim3(MG_WG), 0, stream, a, w, o);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace idxtopk
