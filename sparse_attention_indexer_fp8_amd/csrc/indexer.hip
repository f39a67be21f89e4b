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
// The score row never exists in HBM on this path. Batches of at most
// FS_MAX_TOKENS tokens take a variant whose chunks write their scores to the
// workspace instead (see "Fused decode, small batches" below).
#include "../../include/idxtopk.h"
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
  float* sval;     // [rows][k]: scores of the selection for the sort pass
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
  p += align256(static_cast<size_t>(rows) * w.cap * 8);
  w.sval = reinterpret_cast<float*>(p);
  return w;
}

size_t fused_workspace_bytes(int rows, int k, int max_seq_len) {
  const int64_t cap = max_seq_len > 0 ? max_seq_len : 1;
  return align256(static_cast<size_t>(rows) * HIST_BINS * 4) + align256(static_cast<size_t>(rows) * 16) +
         align256(static_cast<size_t>(rows) * cap * 8) + align256(static_cast<size_t>(rows) * k * 4);
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
//
// With quad_map, rows 4q..4q+3 (query rows of one request sit next to each
// other and read the same keys) take the same chunk on one XCD back to back:
// quad-slot Q = (quad, chunk) maps to workgroups 32 (Q / 8) + Q % 8 + 8 r,
// r = 0..3, which the dispatcher sends to XCD Q % 8 one after another, so the
// XCD's L2 fetches the chunk's keys once for all four. Quad-slots past the
// grid's chunks get a chunk index >= nchunk_max, whose span starts past
// every row's end.
__device__ __forceinline__ void chunk_of(const IndexerArgs& a, int& b, int& c) {
  if (a.quad_map) {
    const int i = blockIdx.x;
    const int r = (i >> 3) & 3;
    const int Q = ((i >> 5) << 3) | (i & 7);
    const int nq = a.batch >> 2;
    c = Q / nq;
    b = 4 * ((Q + c) % nq) + r;
    return;
  }
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

// ---------------------------------------------------------------------------
// Unfused scores
// ---------------------------------------------------------------------------

template <int NT, bool BF = false>
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
  score_chunk_any<BF, NT, IX_WG, IX_RING>(a, b, tb, te, pages, [&](int j, float s, bool valid) {
    if (valid) srow[j] = s;
  });
}

// ---------------------------------------------------------------------------
// Unfused scores, rows in groups (prefill and multi-token rows)
// ---------------------------------------------------------------------------
//
// Query rows that map to one block-table row (a request's prefill rows or its
// multi-token decode rows) read the same keys. Each wave here takes four
// consecutive rows: every 16-token key group is loaded once and scored
// against all four rows' queries, and the head sums of the four rows reduce
// together (score16x4), so lane group g ends up holding row g's scores and
// every lane stores. If the four rows do not share a block-table row, the
// wave scores pairs (score16x2) or single rows instead. The grid is
// chunk-major, so all workgroups stream the same 64-page key chunk at about
// the same time and share it through the caches. A chunk's page ids sit one
// per lane in a VGPR, so a group's page is one readlane: no LDS and no
// barrier. Used when pages hold whole 16-token groups (page_size % 16 == 0).
//
// On the packed-prefill geometry (16384 rows, 573M row-keys) the four-row
// path runs at ~1.67 PFLOP/s of fp8 products, a third of the matrix peak;
// the per-head weighted ReLU costs two vector instructions per product
// element, about as much issue time as the products themselves. Two rows
// per wave (2 waves per SIMD) ran 5.75 ms, four rows (1 wave per SIMD,
// 52 AGPRs) 5.61 ms, one row 10.6 ms; issuing the next group's products
// before the current group's head sums did not help.

constexpr int PR_WG = 256;  // 4 waves, each up to 4 rows
constexpr int PR_RING = 4;  // key groups in flight per wave
constexpr int PR_CHUNK_PAGES = kWave;

// Score R rows (R = 1, 2 or 4, all reading block-table row bt_row) over the
// keys [kb, ke) of one chunk; row r's scores go to rows[r][j] for j < n[r].
template <int NT, int R>
__device__ __forceinline__ void rows_range(const IndexerArgs& a, const QOperand<NT> (&q)[R], float* const (&rows)[R],
                                           const int (&n)[R], const int32_t* bt_row, int kb, int ke) {
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  const int l = lane_id();
  const int c = l & 15, g = l >> 4;
  const uint32_t pg0 = fdiv(static_cast<uint32_t>(kb), a.pdiv);
  const uint32_t npg = fdiv(static_cast<uint32_t>(ke - 1), a.pdiv) - pg0 + 1;  // <= PR_CHUNK_PAGES
  const int32_t pv = static_cast<uint32_t>(l) < npg ? bt_row[pg0 + l] : 0;
  const int ngroups = (ke - kb + kGroup - 1) / kGroup;

  // group gi -> this lane's 32 key bytes in the operand layout (bytes
  // [32g, 32g + 32) of token c) and the token's scale. The group lies in one
  // page, and tokens past ke read that page's bytes. Keys come mostly from
  // the caches here (many rows read them), so the operand layout is loaded
  // directly rather than as whole lines plus a permute: fewer instructions.
  auto fetch = [&](int gi, KeyPieces& kp, float& ks) {
    const int j0 = kb + gi * kGroup;
    const uint32_t pg = fdiv(static_cast<uint32_t>(j0), a.pdiv);
    uint32_t m = (static_cast<uint32_t>(__builtin_amdgcn_readlane(pv, pg - pg0)) - pg) * P;
    asm volatile("" : "+s"(m));
    const uint32_t s0 = m + static_cast<uint32_t>(j0);
    const uint8_t* kp0 = a.kcache + (static_cast<uint64_t>(s0 + c) << 7) + 32 * g;
    kp.x0 = load_v4i_stream(kp0);
    kp.x1 = load_v4i_stream(kp0 + 16);
    ks = a.k_scale[s0 + c];
  };
  // lane group g holds row (g % R)'s scores; groups g >= R repeat rows
  float* const dst = rows[g % R];
  const int nd = n[g % R];
  const bool writer = g < R;
  auto consume = [&](int gi, float sc) {
    const int j = kb + gi * kGroup + c;
    if (writer && j < nd) dst[j] = sc;
  };
  auto score = [&](const KeyPieces& kp, float ks) {
    v8i kbv;
    kbv[0] = kp.x0[0]; kbv[1] = kp.x0[1]; kbv[2] = kp.x0[2]; kbv[3] = kp.x0[3];
    kbv[4] = kp.x1[0]; kbv[5] = kp.x1[1]; kbv[6] = kp.x1[2]; kbv[7] = kp.x1[3];
    if constexpr (R == 4) return score16x4<NT>(q, kbv, ks);
    else if constexpr (R == 2) return score16x2<NT>(q[0], q[1], kbv, ks);
    else return score16<NT>(q[0], kbv, ks);
  };

  typedef float vks __attribute__((ext_vector_type(PR_RING)));
  KeyPieces ring[PR_RING];
  vks ksr;
  const int gmax = ngroups - 1;
#pragma unroll
  for (int u = 0; u < PR_RING; ++u) {
    float t;
    fetch(min(u, gmax), ring[u], t);
    ksr[u] = t;
  }
  int gi0 = 0;
  for (; gi0 + 2 * PR_RING <= ngroups; gi0 += PR_RING) {
#pragma unroll
    for (int u = 0; u < PR_RING; ++u) {
      float sc = score(ring[u], ksr[u]);
      // the score is final before the slot is refilled (see score_chunk)
      asm volatile("" : "+v"(sc));
      __builtin_amdgcn_sched_barrier(0);
      float t;
      fetch(gi0 + u + PR_RING, ring[u], t);
      ksr[u] = t;
      consume(gi0 + u, sc);
    }
  }
#pragma unroll
  for (int u = 0; u < PR_RING; ++u) {
    const int gi = gi0 + u;
    if (gi < ngroups) {
      const float sc = score(ring[u], ksr[u]);
      if (gi + PR_RING < ngroups) {
        float t;
        fetch(gi + PR_RING, ring[u], t);
        ksr[u] = t;
      }
      consume(gi, sc);
    }
  }
#pragma unroll
  for (int u = 0; u < PR_RING; ++u) {
    const int gi = gi0 + PR_RING + u;
    if (gi < ngroups) consume(gi, score(ring[u], ksr[u]));
  }
}

template <int NT, int R>
__device__ __forceinline__ void score_rows(const IndexerArgs& a, float* scores, int64_t sstride, int b0,
                                           const int (&nn)[4], const int (&pr)[4], int i0, int kb, int chunk) {
  QOperand<NT> q[R];
  float* rows[R];
  int n[R];
  int nmax = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int b = b0 + i0 + r;
    load_query<NT>(q[r], a.q + static_cast<int64_t>(b) * a.heads * kDim, a.w + static_cast<int64_t>(b) * a.heads,
                   a.q_scale[b]);
    rows[r] = scores + static_cast<int64_t>(b) * sstride;
    n[r] = nn[i0 + r];
    nmax = max(nmax, n[r]);
  }
  const int ke = min(kb + chunk, nmax);
  if (kb < ke) rows_range<NT, R>(a, q, rows, n, a.block_table + static_cast<int64_t>(pr[i0]) * a.bt_stride, kb, ke);
}

template <int NT>
__global__ __launch_bounds__(PR_WG) void pair_score_kernel(IndexerArgs a, float* scores, int64_t sstride,
                                                           int ntiles, int chunk) {
  const int tile = blockIdx.x % ntiles;
  const int kc = blockIdx.x / ntiles;
  const int quad = tile * (PR_WG / kWave) + uniform(static_cast<int>(threadIdx.x) / kWave);
  const int b0 = 4 * quad;
  if (b0 >= a.batch) return;
  const int nr = min(4, a.batch - b0);
  int nn[4], pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = b0 + (i < nr ? i : 0);
    nn[i] = i < nr ? load_uniform(a.seq_lens + b) : 0;
    pr[i] = a.row_to_batch ? load_uniform(a.row_to_batch + b) : b;
  }
  const int kb = kc * chunk;
  if (nr == 4 && pr[0] == pr[1] && pr[1] == pr[2] && pr[2] == pr[3]) {
    score_rows<NT, 4>(a, scores, sstride, b0, nn, pr, 0, kb, chunk);
    return;
  }
  for (int i0 = 0; i0 < nr; i0 += 2) {
    if (i0 + 1 < nr && pr[i0] == pr[i0 + 1]) {
      score_rows<NT, 2>(a, scores, sstride, b0, nn, pr, i0, kb, chunk);
    } else {
      score_rows<NT, 1>(a, scores, sstride, b0, nn, pr, i0, kb, chunk);
      if (i0 + 1 < nr) score_rows<NT, 1>(a, scores, sstride, b0, nn, pr, i0 + 1, kb, chunk);
    }
  }
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
  int keep_positions;  // leave row-local positions in `slots` (the sort pass maps them)
};

// Dynamic LDS: the chunk's scores (a.chunk floats).
template <int NT, bool BF = false>
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
  score_chunk_any<BF, NT, IX_WG, IX_RING, true>(a, b, tb, te, s.pages, [&](int j, float v, bool valid) {
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

// Emit this thread's keys with keep[e] set: one output reservation per
// wave, then each key's row-local position (and score) is stored. The merge
// turns positions into slots in one pass at the end (positions_to_slots).
// All lanes of the wave must call.
template <int N>
__device__ __forceinline__ void emit_batch(const uint64_t (&keys)[N], const bool (&keep)[N], int b,
                                           const FusedOut& o, uint32_t* ocnt) {
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) mine += keep[e];
  uint32_t at = wave_reserve(mine, ocnt);
  const int64_t row = static_cast<int64_t>(b) * o.k;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if (keep[e]) {
      if (at < static_cast<uint32_t>(o.k)) {
        o.slots[row + at] = static_cast<int32_t>(rank_pos(keys[e]));
        if (o.scores) o.scores[row + at] = key_float(rank_vkey(keys[e]));
      }
      ++at;
    }
  }
}

// Row b's first nout output entries hold row-local positions written by this
// workgroup (a barrier must separate the writes from this call): map them to
// slots through the block table (page_of(logical page) gives the physical
// page). Each thread reads PER positions, issues all their block-table
// lookups, then forms and stores the slots. slot =
// (page - pg) * P + pos, with the multiply and the add kept apart by an empty
// asm: fused, they become a 64-bit mad whose unused high addend half can
// alias a register with a load in flight, and the wait for it would drain
// every load.
template <int WG, int PER, class PageOf>
__device__ __forceinline__ void positions_to_slots(const IndexerArgs& a, int b, const FusedOut& o, uint32_t nout,
                                                   PageOf&& page_of) {
  const int tid = threadIdx.x;
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  const int64_t row = static_cast<int64_t>(b) * o.k;
  for (uint32_t i0 = 0; i0 < nout; i0 += PER * WG) {
    uint32_t pos[PER], pg[PER];
    int32_t page[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const uint32_t i = i0 + e * WG + tid;
      pos[e] = i < nout ? static_cast<uint32_t>(o.slots[row + i]) : 0u;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      pg[e] = fdiv(pos[e], a.pdiv);
      page[e] = page_of(pg[e]);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      uint32_t x = (static_cast<uint32_t>(page[e]) - pg[e]) * P;
      asm volatile("" : "+v"(x));
      const uint32_t i = i0 + e * WG + tid;
      if (i < nout) o.slots[row + i] = static_cast<int32_t>(x + pos[e]);
    }
  }
}

constexpr int MG_BATCH = 8;  // candidates per thread per pass of the merge
constexpr int WS_PER = 16;   // threshold-bin keys per lane when one wave selects

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
    emit_batch<MG_BATCH>(key, keep, b, o, &s.ocnt);
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
  if (!th.all && nb > 0 && nb <= static_cast<uint32_t>(kWave * WS_PER)) {
    // a small threshold bin: wave 0 alone selects and emits it
    if (tid < kWave) {
      uint64_t keys[WS_PER];
      bool valid[WS_PER], keep[WS_PER];
#pragma unroll
      for (int e = 0; e < WS_PER; ++e) {
        const uint32_t i = e * kWave + tid;
        valid[e] = i < nb;
        keys[e] = valid[e] ? s.buf[i] : 0ull;
      }
      const uint64_t T = nb > need ? wave_select<WS_PER>(keys, valid, need, s.sel.hist) : 0ull;
#pragma unroll
      for (int e = 0; e < WS_PER; ++e) keep[e] = valid[e] && keys[e] >= T;
      emit_batch<WS_PER>(keys, keep, b, o, &s.ocnt);
    }
  } else if (!th.all && nb > 0) {
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
      emit_batch<MG_MAXE>(keys, keep, b, o, &s.ocnt);
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
        emit_batch<MG_BATCH>(key, keep, b, o, &s.ocnt);
      }
    }
  }
  __syncthreads();
  if (!o.keep_positions) {
    const int32_t* bt_row = bt_row_of(a, b);
    positions_to_slots<MG_WG, 8>(a, b, o, min(s.ocnt, k), [&](uint32_t pg) { return bt_row[pg]; });
  }
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
// Fused decode, small batches: score buffer instead of candidates
// ---------------------------------------------------------------------------
//
// When the batch holds few tokens (batch * max_seq_len <= FS_MAX_TOKENS) the
// chunks are sized so that every chunk workgroup is resident at once, and a
// chunk ends without waiting on anything: it writes its scores to the
// workspace (the candidate area, as fp32 [rows][cap]) and adds its histogram
// to the row's with fire-and-forget atomics. The per-chunk bound, the
// read-back and the candidate reservation of the path above each cost a
// dependent round trip that a short chunk cannot hide. One workgroup per row
// then issues the histogram, the block table and its first scores together,
// takes the exact threshold bin, emits the scores above it and selects
// inside it. The extra bytes (scores written, read back and zeroed: 12 B per
// token against 132 B of key and scale) stay in the last-level cache at
// these sizes.

constexpr int64_t FS_MAX_TOKENS = int64_t{1} << 21;
constexpr int FS_CH_MAX = 4096;  // chunk tokens (dynamic LDS for the scores)
constexpr int FS_CH_MIN = 256;
constexpr int FS_RING = 4;       // key groups in flight per wave
constexpr int FS_WG = 1024;      // merge workgroup
constexpr int FS_PER = 8;        // scores per thread per pass of the merge
constexpr int FS_BUF = 4096;     // threshold-bin keys held in LDS (32 KB)
constexpr int FS_MAXE = FS_BUF / FS_WG;
static_assert(FS_MAXE <= FS_PER, "slot lookups of one emission");
constexpr int FS_PAGES = 4096;   // block-table entries staged in LDS
constexpr int FS_PG_PER = FS_PAGES / FS_WG;

__device__ __forceinline__ float* fused_scores_row(const FusedWs& w, int b) {
  return reinterpret_cast<float*>(w.cand) + static_cast<int64_t>(b) * w.cap;
}

struct ScoresChunkLds {
  alignas(16) uint32_t hist[HIST_BINS];
  int32_t pages[IX_PAGES];
};

template <int NT, bool BF = false>
__global__ __launch_bounds__(IX_WG) void fused_scores_chunk_kernel(IndexerArgs a, FusedWs ws) {
  extern __shared__ float4 sc4[];
  float* sc = reinterpret_cast<float*>(sc4);
  __shared__ ScoresChunkLds s;
  const int tid = threadIdx.x;
  int b, c;
  chunk_of(a, b, c);
  const int n = a.seq_lens[b];
  int tb, clen;
  chunk_span(a, c, tb, clen);
  if (tb >= n) return;
  const int te = min(n, tb + clen);
  const int cnt = te - tb;

  for (int i = tid; i < HIST_BINS; i += IX_WG) s.hist[i] = 0;
  // (score_chunk synchronises before its first emit)
  score_chunk_any<BF, NT, IX_WG, FS_RING>(a, b, tb, te, s.pages, [&](int j, float v, bool valid) {
    if (valid) {
      sc[j - tb] = v;
      atomicAdd(&s.hist[float_key(v) >> HIST_SHIFT], 1u);
    }
  });
  __syncthreads();
  // scores out, 16 bytes per lane where the row's base allows it
  float* srow = fused_scores_row(ws, b) + tb;
  if ((reinterpret_cast<uintptr_t>(srow) & 15u) == 0) {
    for (int i = 4 * tid; i < cnt; i += 4 * IX_WG) {
      if (i + 4 <= cnt) {
        *reinterpret_cast<float4*>(srow + i) = sc4[i / 4];
      } else {
        for (int e = i; e < cnt; ++e) srow[e] = sc[e];
      }
    }
  } else {
    for (int i = tid; i < cnt; i += IX_WG) srow[i] = sc[i];
  }
  uint32_t* Hg = ws.hist + static_cast<int64_t>(b) * HIST_BINS;
#pragma unroll
  for (int i = 0; i < HIST_BINS / IX_WG; ++i) {
    const int bin = i * IX_WG + tid;
    const uint32_t h = s.hist[bin];
    if (h) add_dev(&Hg[bin], h);
  }
}

struct ScoresMergeLds {
  uint64_t buf[FS_BUF];
  int32_t pages[FS_PAGES];
  SelectLds sel;
  uint32_t scratch[24];
  uint32_t ocnt;
  uint32_t bcnt;
};

// One workgroup per row: exact top-k of the row's scores from its complete
// histogram, then the row's scores and histogram are zeroed again. STAGED:
// the row's block table fits in LDS (else slots are looked up in HBM).
template <bool STAGED>
__device__ __forceinline__ void fused_scores_merge_row(const IndexerArgs& a, const FusedWs& ws, const FusedOut& o,
                                                       ScoresMergeLds& s, int b, int n, int npages) {
  const int tid = threadIdx.x;
  const uint32_t k = static_cast<uint32_t>(o.k);
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  uint32_t* Hg = ws.hist + static_cast<int64_t>(b) * HIST_BINS;
  float* srow = fused_scores_row(ws, b);
  const int32_t* bt_row = bt_row_of(a, b);
  const int64_t orow = static_cast<int64_t>(b) * o.k;

  wg_select_init<FS_WG>(s.sel);
  if (tid == 0) {
    s.ocnt = 0;
    s.bcnt = 0;
  }
  // In flight together: the first pass of scores, the block table, the
  // histogram (indices past the row re-read entry 0, which exists).
  float v0[FS_PER];
#pragma unroll
  for (int e = 0; e < FS_PER; ++e) {
    const int i = e * FS_WG + tid;
    v0[e] = srow[i < n ? i : 0];
  }
  if (STAGED && npages > 0) {
    int32_t pg[FS_PG_PER];
#pragma unroll
    for (int r = 0; r < FS_PG_PER; ++r) {
      const int i = r * FS_WG + tid;
      pg[r] = bt_row[i < npages ? i : 0];
    }
#pragma unroll
    for (int r = 0; r < FS_PG_PER; ++r)
      if (r * FS_WG + tid < npages) s.pages[r * FS_WG + tid] = pg[r];
  }
  const BinThreshold th = wg_threshold_bin<FS_WG, HIST_BINS>([&](int i) { return Hg[i]; }, k, s.scratch);
  const uint32_t bstar = th.all ? 0u : th.bin;
  const uint32_t need = th.all ? 0u : k - th.above;

  // Selected tokens are first written to the output row as positions (and
  // scores); one coalesced pass at the end turns positions into slots, so
  // no block-table lookup sits on the selection passes.
  auto emit = [&](const uint64_t* key, const bool* keep, int m) {
    uint32_t mine = 0;
    for (int e = 0; e < m; ++e) mine += keep[e];
    uint32_t at = wave_reserve(mine, &s.ocnt);
    for (int e = 0; e < m; ++e) {
      if (keep[e]) {
        if (at < k) {
          o.slots[orow + at] = static_cast<int32_t>(rank_pos(key[e]));
          if (o.scores) o.scores[orow + at] = key_float(rank_vkey(key[e]));
        }
        ++at;
      }
    }
  };
  // One pass: scores above the threshold bin (all of them when the row holds
  // at most k) are emitted, scores inside it go to LDS as unique keys.
  auto pass = [&](const float (&v)[FS_PER], int base) {
    static_assert(FS_PER <= 32, "bit masks");
    uint32_t keepm = 0, midm = 0;
#pragma unroll
    for (int e = 0; e < FS_PER; ++e) {
      const bool valid = base + e * FS_WG + tid < n;
      const uint32_t bin = float_key(v[e]) >> HIST_SHIFT;
      keepm |= static_cast<uint32_t>(valid && (th.all || bin > bstar)) << e;
      midm |= static_cast<uint32_t>(valid && !th.all && bin == bstar) << e;
    }
    uint32_t at = wave_reserve(__builtin_popcount(keepm), &s.ocnt);
#pragma unroll
    for (int e = 0; e < FS_PER; ++e) {
      if ((keepm >> e) & 1u) {
        if (at < k) {
          o.slots[orow + at] = base + e * FS_WG + tid;
          if (o.scores) o.scores[orow + at] = v[e];
        }
        ++at;
      }
    }
    uint32_t bt = wave_reserve(__builtin_popcount(midm), &s.bcnt);
#pragma unroll
    for (int e = 0; e < FS_PER; ++e) {
      if ((midm >> e) & 1u) {
        if (bt < static_cast<uint32_t>(FS_BUF))
          s.buf[bt] = rank_key(float_key(v[e]), static_cast<uint32_t>(base + e * FS_WG + tid));
        ++bt;
      }
    }
  };
  // the next pass's scores are in flight while this pass is processed
  for (int base = 0; base == 0 || base < n; base += FS_PER * FS_WG) {
    float nx[FS_PER];
    const int nb0 = base + FS_PER * FS_WG;
    if (nb0 < n) {
#pragma unroll
      for (int e = 0; e < FS_PER; ++e) {
        const int i = nb0 + e * FS_WG + tid;
        nx[e] = srow[i < n ? i : 0];
      }
    }
    pass(v0, base);
    if (nb0 < n) {
#pragma unroll
      for (int e = 0; e < FS_PER; ++e) v0[e] = nx[e];
    }
  }
  __syncthreads();
  const uint32_t nb = s.bcnt;
  if (!th.all && nb > 0 && nb <= static_cast<uint32_t>(kWave * WS_PER)) {
    // a small threshold bin: wave 0 alone selects and emits it (no
    // workgroup barrier inside the select)
    if (tid < kWave) {
      uint64_t keys[WS_PER];
      bool valid[WS_PER], keep[WS_PER];
#pragma unroll
      for (int e = 0; e < WS_PER; ++e) {
        const uint32_t i = e * kWave + tid;
        valid[e] = i < nb;
        keys[e] = valid[e] ? s.buf[i] : 0ull;
      }
      const uint64_t T = nb > need ? wave_select<WS_PER>(keys, valid, need, s.sel.hist) : 0ull;
#pragma unroll
      for (int e = 0; e < WS_PER; ++e) keep[e] = valid[e] && keys[e] >= T;
      emit(keys, keep, WS_PER);
    }
  } else if (!th.all && nb > 0) {
    if (nb <= static_cast<uint32_t>(FS_BUF)) {
      uint64_t keys[FS_MAXE];
      bool keep[FS_MAXE];
      uint64_t mn = ~0ull, mx = 0;
#pragma unroll
      for (int e = 0; e < FS_MAXE; ++e) {
        const uint32_t i = tid + e * FS_WG;
        keys[e] = i < nb ? s.buf[i] : 0ull;
        if (i < nb) {
          mn = keys[e] < mn ? keys[e] : mn;
          mx = keys[e] > mx ? keys[e] : mx;
        }
      }
      uint64_t T = 0;  // keys >= T are selected
      if (nb > need) {
        wg_range<FS_WG>(mn, mx, s.sel);
        T = wg_select<FS_WG>(
            [&](auto&& f) {
#pragma unroll
              for (int e = 0; e < FS_MAXE; ++e)
                if (tid + e * FS_WG < nb) f(keys[e]);
            },
            need, mn, mx, s.sel);
      }
#pragma unroll
      for (int e = 0; e < FS_MAXE; ++e) keep[e] = tid + e * FS_WG < nb && keys[e] >= T;
      emit(keys, keep, FS_MAXE);
    } else {
      // threshold bin larger than the LDS buffer: select straight from the
      // row's scores (several passes over them)
      auto each_mid = [&](auto&& f) {
        for (int i = tid; i < n; i += FS_WG) {
          const uint32_t vk = float_key(srow[i]);
          if ((vk >> HIST_SHIFT) == bstar) f(rank_key(vk, static_cast<uint32_t>(i)));
        }
      };
      uint64_t mn = ~0ull, mx = 0;
      each_mid([&](uint64_t key) {
        mn = key < mn ? key : mn;
        mx = key > mx ? key : mx;
      });
      wg_range<FS_WG>(mn, mx, s.sel);
      const uint64_t T = wg_select<FS_WG>(each_mid, need, mn, mx, s.sel);
      for (int i0 = 0; i0 < n; i0 += FS_WG) {
        const int i = i0 + tid;
        uint64_t key = 0;
        bool keep = false;
        if (i < n) {
          const uint32_t vk = float_key(srow[i]);
          key = rank_key(vk, static_cast<uint32_t>(i));
          keep = (vk >> HIST_SHIFT) == bstar && key >= T;
        }
        emit(&key, &keep, 1);
      }
    }
  }
  __syncthreads();
  const uint32_t nout = min(s.ocnt, k);
  // positions -> slots (this workgroup wrote them; the barrier orders it)
  if (!o.keep_positions)
    positions_to_slots<FS_WG, FS_PER>(a, b, o, nout, [&](uint32_t pg) {
      return STAGED ? s.pages[pg] : bt_row[pg];
    });
  // padding for rows shorter than k
  for (uint32_t i = nout + tid; i < k; i += FS_WG) {
    o.slots[orow + i] = -1;
    if (o.scores) o.scores[orow + i] = -__builtin_inff();
  }
  // leave the row's workspace bytes zero again
  for (int i = tid; i < n; i += FS_WG) srow[i] = 0.0f;
  if (n > 0)
    for (int i = tid; i < HIST_BINS; i += FS_WG) Hg[i] = 0;
}

__global__ __launch_bounds__(FS_WG) void fused_scores_merge_kernel(IndexerArgs a, FusedWs ws, FusedOut o) {
  __shared__ ScoresMergeLds s;
  const int b = blockIdx.x;
  const int n = a.seq_lens[b];
  const int npages = n > 0 ? static_cast<int>(fdiv(static_cast<uint32_t>(n - 1), a.pdiv)) + 1 : 0;
  if (npages <= FS_PAGES)
    fused_scores_merge_row<true>(a, ws, o, s, b, n, npages);
  else
    fused_scores_merge_row<false>(a, ws, o, s, b, n, npages);
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
  int32_t phys[BK_MAX_TOP];  // physical block id of each selected block
  SelectLds sel;
  uint32_t ocnt;
};

struct BlockOut {
  int32_t* blocks;
  int32_t* slots;
  int top;
  int bs;
  int hp;  // selections per query row: 1, or the head count (per-head variant)
};

template <int NT, bool BF = false>
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
  score_chunk_any<BF, NT, IX_WG, IX_RING>(a, b, tb, te, s.pages, [&](int j, float v, bool valid) {
    uint32_t key = valid ? float_key(v) : 0u;
    key = row16_max(key);
    if (lane_id() == 0 && key) atomicMax(&s.bmax[fdiv(static_cast<uint32_t>(j - tb), a.pdiv)], key);
  });
  __syncthreads();
  const int blk0 = tb / bs;
  for (int i = tid; i < nbc; i += IX_WG) bsc[blk0 + i] = s.bmax[i];
}

// Slot list of one selection: entry e of its top * bs entries is token
// t = e % bs of selected block i = e / bs, i.e. slot phys[i] * bs + t when
// block i exists (i < nsel) and its token is visible (cbs[i] * bs + t < n),
// else -1. Thread `me` of NTH writes four consecutive entries per 16-byte
// nontemporal store (the lists are written once) when the output is 16-byte
// aligned (bs is a multiple of 16, so every selection's list then is too).
// Slot ids are int32 outputs: the arithmetic wraps as their int32
// conversion would.
template <int NTH>
__device__ __forceinline__ void write_slot_list(int32_t* srow, int top, int bs, int nsel, int n,
                                                const int32_t* cbs, const int32_t* phys, const FastDiv& bdiv,
                                                int me, bool vec) {
  const int total = top * bs;
  auto slot = [&](int i, int t) -> int32_t {
    if (i >= nsel || cbs[i] * bs + t >= n) return -1;
    return static_cast<int32_t>(static_cast<uint32_t>(phys[i]) * static_cast<uint32_t>(bs) +
                                static_cast<uint32_t>(t));
  };
  if (vec) {
    for (int e = 4 * me; e < total; e += 4 * NTH) {
      const int i = static_cast<int>(fdiv(static_cast<uint32_t>(e), bdiv));
      const int t = e - i * bs;
      v4i v;
      v.x = slot(i, t);
      v.y = slot(i, t + 1);
      v.z = slot(i, t + 2);
      v.w = slot(i, t + 3);
      __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(srow + e));
    }
  } else {
    for (int e = me; e < total; e += NTH) {
      const int i = static_cast<int>(fdiv(static_cast<uint32_t>(e), bdiv));
      srow[e] = slot(i, e - i * bs);
    }
  }
}

// One workgroup per selection: query row b, or (row b, head) in the per-head
// variant, whose block maxima and outputs are laid out [rows * hp].
__global__ __launch_bounds__(MG_WG) void block_merge_kernel(IndexerArgs a, BlockWs ws, BlockOut o) {
  __shared__ BlockMergeLds s;
  const int tid = threadIdx.x;
  const int sel_row = blockIdx.x;
  const int b = sel_row / o.hp;
  const int n = a.seq_lens[b];
  const int bs = o.bs;
  const int top = o.top;
  const int nblk = (n + bs - 1) / bs;
  uint32_t* bsc = ws.bscore + static_cast<int64_t>(sel_row) * ws.nblk_max;

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
  const int32_t* bt_row = bt_row_of(a, b);
  for (int i = tid; i < top; i += MG_WG) {
    const int32_t pb = i < nsel ? bt_row[s.sel_blocks[i]] : -1;
    o.blocks[static_cast<int64_t>(sel_row) * top + i] = pb;
    s.phys[i] = pb;
  }
  if (o.slots) {
    __syncthreads();
    write_slot_list<MG_WG>(o.slots + static_cast<int64_t>(sel_row) * top * bs, top, bs, nsel, n, s.sel_blocks,
                           s.phys, a.pdiv, tid, (reinterpret_cast<uintptr_t>(o.slots) & 15u) == 0);
  }
  // leave every workspace byte of this row zero again
  __syncthreads();
  for (int cb = tid; cb < nblk; cb += MG_WG) bsc[cb] = 0;
}

// Per-head block maxima (fp8 cache): each head's term of the score, maxed
// over the block's visible tokens, for every (head, block) of the chunk:
// the 16 tokens of a group are reduced in registers per head (DPP over each
// 16-lane row, which holds four heads of the tile), and lane 0 of the row
// raises the (head, block) entry in LDS.
constexpr int BKH_MAX_BLOCKS = 64;  // blocks per chunk

struct BlockHeadsLds {
  int32_t pages[IX_PAGES];
  uint32_t hmax[128 * BKH_MAX_BLOCKS];
};

template <int NT>
__global__ __launch_bounds__(IX_WG) void block_heads_chunk_kernel(IndexerArgs a, BlockWs ws, int bs) {
  __shared__ BlockHeadsLds s;
  constexpr int H = 16 * NT;
  const int tid = threadIdx.x;
  int b, c;
  chunk_of(a, b, c);
  const int n = a.seq_lens[b];
  int tb, clen;
  chunk_span(a, c, tb, clen);
  if (tb >= n) return;
  const int te = min(n, tb + clen);
  const int nbc = (te - tb + bs - 1) / bs;
  for (int i = tid; i < H * BKH_MAX_BLOCKS; i += IX_WG) s.hmax[i] = 0;
  // (score_chunk_heads synchronises before its first emit)
  const int l = lane_id();
  const int lc = l & 15, lg = l >> 4;
  score_chunk_heads<NT, IX_WG, IX_RING>(a, b, tb, te, s.pages, [&](int j0, const float (&v)[NT][4]) {
    const bool valid = j0 + lc < te;
    // a group lies inside one block (block size and chunk start are
    // multiples of 16)
    const uint32_t blk = fdiv(static_cast<uint32_t>(j0 - tb), a.pdiv);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t key = row16_max(valid ? float_key(v[t][r]) : 0u);
        if (lc == 0 && key) atomicMax(&s.hmax[(16 * t + 4 * lg + r) * BKH_MAX_BLOCKS + blk], key);
      }
    }
  });
  __syncthreads();
  const int blk0 = tb / bs;
  for (int i = tid; i < H * nbc; i += IX_WG) {
    const int h = i / nbc, cb = i - h * nbc;
    ws.bscore[(static_cast<int64_t>(b) * H + h) * ws.nblk_max + blk0 + cb] = s.hmax[h * BKH_MAX_BLOCKS + cb];
  }
}

// Per-head merge with one wave per (row, head) selection (there are batch x
// heads of them, enough waves to fill the chip), for rows of at most
// BH_MAX_BLOCKS blocks and at most BH_MAX_TOP kept blocks: the selection's
// block keys sit 16 per lane, wave_select finds the top-th, a ballot compacts
// the kept block ids into this wave's LDS list, and the wave writes the
// block ids, the slot lists and the zeros. No workgroup barrier: a wave whose
// selection is past the end leaves at once.
constexpr int BH_WAVES = 4;
constexpr int BH_PER = 16;
constexpr int BH_MAX_BLOCKS = BH_PER * kWave;
constexpr int BH_MAX_TOP = 256;

struct BlockHeadsMergeLds {
  alignas(16) uint32_t hist[BH_WAVES][256];  // wave_select clears it 16 bytes per lane
  int32_t sel[BH_WAVES][BH_MAX_TOP];
  int32_t phys[BH_WAVES][BH_MAX_TOP];
};

__global__ __launch_bounds__(BH_WAVES * kWave) void block_heads_merge_kernel(IndexerArgs a, BlockWs ws,
                                                                              BlockOut o) {
  __shared__ BlockHeadsMergeLds s;
  const int wave = static_cast<int>(threadIdx.x) / kWave;
  const int lane = lane_id();
  const int sel_row = static_cast<int>(blockIdx.x) * BH_WAVES + wave;
  if (sel_row >= a.batch * o.hp) return;
  const int b = sel_row / o.hp;
  const int n = a.seq_lens[b];
  const int bs = o.bs;
  const int top = o.top;
  const int nblk = (n + bs - 1) / bs;
  uint32_t* bsc = ws.bscore + static_cast<int64_t>(sel_row) * ws.nblk_max;
  uint64_t keys[BH_PER];
  bool valid[BH_PER];
#pragma unroll
  for (int e = 0; e < BH_PER; ++e) {
    const int cb = e * kWave + lane;
    valid[e] = cb < nblk;
    keys[e] = valid[e] ? rank_key(bsc[cb], static_cast<uint32_t>(cb)) : 0ull;
  }
  const uint64_t T = nblk > top ? wave_select<BH_PER>(keys, valid, static_cast<uint32_t>(top), s.hist[wave]) : 0ull;
  const int nsel = min(nblk, top);
  uint32_t at = 0;
#pragma unroll
  for (int e = 0; e < BH_PER; ++e) {
    const bool keep = valid[e] && keys[e] >= T;
    const uint64_t mk = ballot(keep);
    if (keep) s.sel[wave][at + lanes_below(mk)] = e * kWave + lane;
    at += static_cast<uint32_t>(__popcll(mk));
  }
  // the wave's LDS writes complete before its reads (in-order LDS queue);
  // keep the compiler from moving the reads up
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int32_t* bt_row = bt_row_of(a, b);
  for (int i = lane; i < top; i += kWave) {
    const int32_t pb = i < nsel ? bt_row[s.sel[wave][i]] : -1;
    o.blocks[static_cast<int64_t>(sel_row) * top + i] = pb;
    s.phys[wave][i] = pb;
  }
  if (o.slots) {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    write_slot_list<kWave>(o.slots + static_cast<int64_t>(sel_row) * top * bs, top, bs, nsel, n, s.sel[wave],
                           s.phys[wave], a.pdiv, lane, (reinterpret_cast<uintptr_t>(o.slots) & 15u) == 0);
  }
  // leave this selection's workspace entries zero again
#pragma unroll
  for (int e = 0; e < BH_PER; ++e)
    if (valid[e]) bsc[e * kWave + lane] = 0;
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
  a.row_to_batch = in.row_to_batch;
  a.bt_stride = in.bt_stride;
  a.page_size = in.page_size;
  a.pdiv = make_fastdiv(static_cast<uint32_t>(in.page_size));
  a.seq_lens = in.seq_lens;
  a.batch = in.batch;
  a.heads = in.heads;
  a.chunk = chunk;
  a.quad_map = in.row_to_batch != nullptr && in.batch % 4 == 0 && in.batch >= 8;
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

// Workgroups of a chunk-major grid (chunk_of): every (row, chunk) pair, in
// whole groups of 32 under quad_map.
static unsigned chunk_grid(const IndexerArgs& a) {
  const int64_t n = static_cast<int64_t>(a.nchunk_max) * a.batch;
  return static_cast<unsigned>(a.quad_map ? (n + 31) / 32 * 32 : n);
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

#define IDXTOPK_SWITCH_NT(KERNEL, BFV, heads, grid, lds, stream, ...)                                  \
  switch (heads) {                                                                                  \
    case 16: hipLaunchKernelGGL((KERNEL<1, BFV>), grid, dim3(IX_WG), lds, stream, __VA_ARGS__); break; \
    case 32: hipLaunchKernelGGL((KERNEL<2, BFV>), grid, dim3(IX_WG), lds, stream, __VA_ARGS__); break; \
    case 64: hipLaunchKernelGGL((KERNEL<4, BFV>), grid, dim3(IX_WG), lds, stream, __VA_ARGS__); break; \
    case 128: hipLaunchKernelGGL((KERNEL<8, BFV>), grid, dim3(IX_WG), lds, stream, __VA_ARGS__); break; \
    default: return -2;                                                                             \
  }
// KERNEL<NT, bf16 cache> for the head count
#define IDXTOPK_DISPATCH_NT_LDS(KERNEL, bf, heads, grid, lds, stream, ...)    \
  do {                                                                        \
    if (bf) {                                                                 \
      IDXTOPK_SWITCH_NT(KERNEL, true, heads, grid, lds, stream, __VA_ARGS__)  \
    } else {                                                                  \
      IDXTOPK_SWITCH_NT(KERNEL, false, heads, grid, lds, stream, __VA_ARGS__) \
    }                                                                         \
  } while (0)
#define IDXTOPK_DISPATCH_NT(KERNEL, bf, heads, grid, stream, ...) \
  IDXTOPK_DISPATCH_NT_LDS(KERNEL, bf, heads, grid, 0, stream, __VA_ARGS__)

int launch_idx_score(const IndexerInputs& in, float* scores, int64_t score_stride, hipStream_t stream) {
  if (in.batch == 0) return 0;
  if (in.row_to_batch && !in.bf16 && in.page_size % kGroup == 0 && in.heads <= 64) {
    // rows sharing block-table rows: two rows per wave against one key load
    int64_t chunk = static_cast<int64_t>(PR_CHUNK_PAGES) * in.page_size;
    if (chunk > 8192) chunk = 8192 / in.page_size * in.page_size;
    const IndexerArgs a = make_args(in, static_cast<int>(chunk), false);
    const int quads = (in.batch + 3) / 4;
    const int ntiles = (quads + PR_WG / kWave - 1) / (PR_WG / kWave);
    const int nkc = static_cast<int>((static_cast<int64_t>(in.max_seq_len > 0 ? in.max_seq_len : 1) + chunk - 1) / chunk);
    const dim3 grid(static_cast<unsigned>(ntiles * nkc));
    (void)hipGetLastError();
    switch (in.heads) {
      case 16: hipLaunchKernelGGL(pair_score_kernel<1>, grid, dim3(PR_WG), 0, stream, a, scores, score_stride, ntiles, static_cast<int>(chunk)); break;
      case 32: hipLaunchKernelGGL(pair_score_kernel<2>, grid, dim3(PR_WG), 0, stream, a, scores, score_stride, ntiles, static_cast<int>(chunk)); break;
      default: hipLaunchKernelGGL(pair_score_kernel<4>, grid, dim3(PR_WG), 0, stream, a, scores, score_stride, ntiles, static_cast<int>(chunk)); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
  }
  const int chunk = choose_chunk(in.batch, in.max_seq_len, in.page_size, kGroup, 512, 8192);
  const IndexerArgs a = make_args(in, chunk, true);
  const dim3 grid(chunk_grid(a));
  (void)hipGetLastError();
  IDXTOPK_DISPATCH_NT(score_kernel, in.bf16, in.heads, grid, stream, a, scores, score_stride);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Workgroups of fused_scores_chunk_kernel that the current device holds at
// once (all compute units, launched with the largest score LDS). Cached per
// device and head count.
static int fs_resident_wgs(int heads, bool bf) {
  static int cache[2][4][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int ti = heads == 16 ? 0 : heads == 32 ? 1 : heads == 64 ? 2 : 3;
  if (cache[bf][ti][dev] > 0) return cache[bf][ti][dev];
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const size_t lds = static_cast<size_t>(FS_CH_MAX) * sizeof(float);
  hipError_t e = hipErrorInvalidValue;
#define IDXTOPK_OCC(B)                                                                                          \
  switch (heads) {                                                                                            \
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_scores_chunk_kernel<1, B>, IX_WG, lds); break;   \
    case 32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_scores_chunk_kernel<2, B>, IX_WG, lds); break;   \
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_scores_chunk_kernel<4, B>, IX_WG, lds); break;   \
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_scores_chunk_kernel<8, B>, IX_WG, lds); break;  \
    default: break;                                                                                           \
  }
  if (bf) {
    IDXTOPK_OCC(true)
  } else {
    IDXTOPK_OCC(false)
  }
#undef IDXTOPK_OCC
  if (e != hipSuccess || per < 1) per = 1;
  cache[bf][ti][dev] = cus * per;
  return cache[bf][ti][dev];
}

// Score-buffer path: chunks sized so the whole grid is resident at once.
static int launch_fused_scores(const IndexerInputs& in, const FusedWs& w, const FusedOut& o, hipStream_t stream) {
  const int64_t tokens = static_cast<int64_t>(in.batch) * (in.max_seq_len > 0 ? in.max_seq_len : 1);
  const int64_t nwg = fs_resident_wgs(in.heads, in.bf16);
  int64_t ch = nwg > 0 ? (tokens + nwg - 1) / nwg : FS_CH_MAX;
  ch = (ch + kGroup - 1) / kGroup * kGroup;
  if (ch < FS_CH_MIN) ch = FS_CH_MIN;
  if (ch > FS_CH_MAX) ch = FS_CH_MAX;
  const int64_t page_cap = (static_cast<int64_t>(IX_PAGES - 2) * in.page_size) / kGroup * kGroup;
  if (ch > page_cap) ch = page_cap > kGroup ? page_cap : kGroup;
  const IndexerArgs a = make_args(in, static_cast<int>(ch), false);
  const dim3 grid(chunk_grid(a));
  const size_t lds = static_cast<size_t>(ch) * sizeof(float);
  (void)hipGetLastError();
  IDXTOPK_DISPATCH_NT_LDS(fused_scores_chunk_kernel, in.bf16, in.heads, grid, lds, stream, a, w);
  hipLaunchKernelGGL(fused_scores_merge_kernel, dim3(in.batch), dim3(FS_WG), 0, stream, a, w, o);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

static int launch_fused_select(const IndexerInputs& in, const FusedWs& w, const FusedOut& o, hipStream_t stream);

// Sorted output: the merges leave positions and scores (in the workspace's
// score area when the caller wants none), then the sort pass orders and maps
// them and clears that area again.
int launch_fused(const IndexerInputs& in, int k, int32_t* out_slots, float* out_scores, void* ws,
                 bool sorted, hipStream_t stream) {
  if (in.batch == 0) return 0;
  const FusedWs w = fused_ws(ws, in.batch, in.max_seq_len);
  FusedOut o;
  o.slots = out_slots;
  o.scores = sorted && !out_scores ? w.sval : out_scores;
  o.k = k;
  o.keep_positions = sorted;
  const int e = launch_fused_select(in, w, o, stream);
  if (e || !sorted) return e;
  return launch_sort_rows(in.batch, k, out_slots, o.scores, nullptr, 0, nullptr, nullptr, in.block_table,
                          in.bt_stride, in.page_size, in.row_to_batch, out_scores,
                          out_scores ? nullptr : w.sval, stream);
}

static int launch_fused_select(const IndexerInputs& in, const FusedWs& w, const FusedOut& o, hipStream_t stream) {
  if (static_cast<int64_t>(in.batch) * in.max_seq_len <= FS_MAX_TOKENS) return launch_fused_scores(in, w, o, stream);
  const int chunk = choose_chunk(in.batch, in.max_seq_len, in.page_size, kGroup, 512, FU_CH_MAX);
  const IndexerArgs a = make_args(in, chunk, true);
  const int k = o.k;
  const dim3 grid(chunk_grid(a));
  (void)hipGetLastError();
  // the scores' dynamic LDS plus the static part stay within 64 KB
  static_assert(FU_CH_MAX * 4 + sizeof(ChunkLds) <= 64 * 1024, "fused chunk LDS");
  const size_t lds = static_cast<size_t>(chunk) * sizeof(float);
  IDXTOPK_DISPATCH_NT_LDS(fused_chunk_kernel, in.bf16, in.heads, grid, lds, stream, a, w, k);
  hipLaunchKernelGGL(fused_merge_kernel, dim3(in.batch), dim3(MG_WG), 0, stream, a, w, o);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Workgroups of block_chunk_kernel that the current device holds at once.
static int bk_resident_wgs(int heads, bool bf) {
  static int cache[2][4][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int ti = heads == 16 ? 0 : heads == 32 ? 1 : heads == 64 ? 2 : 3;
  if (cache[bf][ti][dev] > 0) return cache[bf][ti][dev];
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  hipError_t e = hipErrorInvalidValue;
#define IDXTOPK_OCC(B)                                                                                          \
  switch (heads) {                                                                                            \
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, block_chunk_kernel<1, B>, IX_WG, 0); break;   \
    case 32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, block_chunk_kernel<2, B>, IX_WG, 0); break;   \
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, block_chunk_kernel<4, B>, IX_WG, 0); break;   \
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, block_chunk_kernel<8, B>, IX_WG, 0); break;  \
    default: break;                                                                                           \
  }
  if (bf) {
    IDXTOPK_OCC(true)
  } else {
    IDXTOPK_OCC(false)
  }
#undef IDXTOPK_OCC
  if (e != hipSuccess || per < 1) per = 1;
  cache[bf][ti][dev] = cus * per;
  return cache[bf][ti][dev];
}

int launch_block_topk(const IndexerInputs& in, int block_size, int top_blocks, int32_t* out_blocks,
                      int32_t* out_slots, void* ws, hipStream_t stream) {
  if (in.batch == 0) return 0;
  int chunk = choose_chunk(in.batch, in.max_seq_len, in.page_size, block_size, 512, 8192);
  // When one resident wave of workgroups can hold the whole batch at chunks
  // of at most 8192 tokens, size the chunks for exactly that: every chunk
  // then runs at once, and each amortises its setup over more tokens.
  const int64_t tokens = static_cast<int64_t>(in.batch) * (in.max_seq_len > 0 ? in.max_seq_len : 1);
  const int64_t nwg = bk_resident_wgs(in.heads, in.bf16);
  if (nwg > 0 && tokens <= nwg * 8192) {
    int64_t ch = (tokens + nwg - 1) / nwg;
    ch = (ch + block_size - 1) / block_size * block_size;
    const int64_t page_cap = static_cast<int64_t>(IX_PAGES - 2) * in.page_size / block_size * block_size;
    if (ch > page_cap) ch = page_cap;
    if (ch > chunk) chunk = static_cast<int>(ch);
  }
  if (chunk / block_size > BK_MAX_BLOCKS_PER_CHUNK) chunk = BK_MAX_BLOCKS_PER_CHUNK * block_size;
  const IndexerArgs a = make_args(in, chunk, true, block_size);
  const BlockWs w = block_ws(ws, in.batch, block_size, in.max_seq_len);
  BlockOut o;
  o.blocks = out_blocks;
  o.slots = out_slots;
  o.top = top_blocks;
  o.bs = block_size;
  o.hp = 1;
  const dim3 grid(chunk_grid(a));
  (void)hipGetLastError();
  IDXTOPK_DISPATCH_NT(block_chunk_kernel, in.bf16, in.heads, grid, stream, a, w, block_size);
  // one workgroup per row: with one selection per row there are too few
  // selections for the one-wave merge (block-sparse B64: 72 vs 81 us)
  hipLaunchKernelGGL(block_merge_kernel, dim3(in.batch), dim3(MG_WG), 0, stream, a, w, o);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Per-head block selection: chunks of at most BKH_MAX_BLOCKS blocks, one
// selection per (row, head) in the merge.
int launch_block_topk_heads(const IndexerInputs& in, int block_size, int top_blocks, int32_t* out_blocks,
                            int32_t* out_slots, void* ws, hipStream_t stream) {
  if (in.batch == 0) return 0;
  int chunk = choose_chunk(in.batch, in.max_seq_len, in.page_size, block_size, 512, 8192);
  if (chunk / block_size > BKH_MAX_BLOCKS) chunk = BKH_MAX_BLOCKS * block_size;
  if (chunk < block_size) chunk = block_size;
  const IndexerArgs a = make_args(in, chunk, true, block_size);
  const BlockWs w = block_ws(ws, in.batch * in.heads, block_size, in.max_seq_len);
  BlockOut o;
  o.blocks = out_blocks;
  o.slots = out_slots;
  o.top = top_blocks;
  o.bs = block_size;
  o.hp = in.heads;
  const dim3 grid(chunk_grid(a));
  (void)hipGetLastError();
  switch (in.heads) {
    case 16: hipLaunchKernelGGL(block_heads_chunk_kernel<1>, grid, dim3(IX_WG), 0, stream, a, w, block_size); break;
    case 32: hipLaunchKernelGGL(block_heads_chunk_kernel<2>, grid, dim3(IX_WG), 0, stream, a, w, block_size); break;
    case 64: hipLaunchKernelGGL(block_heads_chunk_kernel<4>, grid, dim3(IX_WG), 0, stream, a, w, block_size); break;
    case 128: hipLaunchKernelGGL(block_heads_chunk_kernel<8>, grid, dim3(IX_WG), 0, stream, a, w, block_size); break;
    default: return -2;
  }
  const int64_t sels = static_cast<int64_t>(in.batch) * in.heads;
  if (w.nblk_max <= BH_MAX_BLOCKS && top_blocks <= BH_MAX_TOP)
    hipLaunchKernelGGL(block_heads_merge_kernel, dim3(static_cast<unsigned>((sels + BH_WAVES - 1) / BH_WAVES)),
                       dim3(BH_WAVES * kWave), 0, stream, a, w, o);
  else
    hipLaunchKernelGGL(block_merge_kernel, dim3(static_cast<unsigned>(sels)), dim3(MG_WG), 0, stream, a, w, o);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace idxtopk
