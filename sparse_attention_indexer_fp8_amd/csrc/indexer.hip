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
// Fused decode (idx_score_topk_fused):
//  1. Per chunk: scores stay in LDS, with a 4096-bin LDS histogram of the
//     value keys' top 12 bits. The chunk's bound is the bin where its own
//     count from the top reaches a rank with a wide statistical margin over
//     its expected share of the row's k best. Its tokens in bins at or above
//     that bin go, as unique 64-bit keys (score key, inverted position), to
//     the chunk's own range of the row's candidate area, (count, bound) to
//     the chunk's header, and its counts of the 64 bins from the bound up to
//     a window beside it. No chunk waits on another.
//  2. Per row, once every chunk is done: the merge gathers the candidates,
//     histograms them (long rows add the chunks' windows instead of
//     counting each candidate) and takes the threshold bin for rank k. When
//     that bin is at or above every chunk's bound, every token of the row
//     in it and above is a candidate, so the selection is exact: candidates
//     above the bin are emitted, and those in it are split once more by the
//     next 8 bits of their value key, the keys of the one sub-bin holding
//     the k-th going through an exact select. Otherwise
//     (best tokens crowded into a few chunks far beyond the margin) the
//     merge scores the row again itself, keeping every token at or above
//     the candidates' threshold bin, a proven lower bound, and selects from
//     those. Output goes through the block table to slots.
// The score row never exists in HBM, and the workspace needs no initial
// contents: each entry the merge reads was written earlier in the call.
#include "../../include/idxtopk.h"
#include "common.hpp"
#include "launch.hpp"
#include "score_mfma.hpp"
#include "select.hpp"
#include "indexer_shared.hpp"

namespace idxtopk {


// ---------------------------------------------------------------------------
// Workspace layouts
// ---------------------------------------------------------------------------


// Fused decode: the candidates of chunk c of row b sit at its own tokens'
// positions of the row's area, cand[b][tb_c, tb_c + count); hdr[b][c] holds
// (count, bound bin). Every entry the merge reads was written earlier in the
// same call, so the area needs no initial contents.
constexpr int FE_CH_MIN = 256;         // shortest chunk: bounds the chunks of a row
constexpr int FE_RESIDENT_MAX = 2048;  // longest chunk of the one-resident-wave sizing
constexpr int FE_WIN = 64;             // bins of a chunk's candidate-count window
constexpr size_t FE_PAIR_LDS = 53 * 1024;  // LDS of a two-row chunk workgroup: three per CU

// win[b][c][i]: how many of chunk c's candidates lie in histogram bin
// bound_c + i, i < FE_WIN (16-bit counts, two per word: a chunk holds at
// most FU_CH_MAX = 8192 tokens; entries of bins past the last are not
// written). For rows of many candidates the merge adds
// these instead of counting each candidate of those bins.
struct FusedWs {
  uint64_t* cand;  // [rows][cap]
  int64_t cap;
  uint2* hdr;      // [rows][hcap]
  int32_t hcap;
  uint32_t* win;   // [rows][hcap][FE_WIN / 2]
  float* sval;     // [rows][k]: scores of the selection for the sort pass
};

// Chunk headers per row: enough for chunks of FE_CH_MIN tokens or more,
// whichever schedule (chunks of a guided schedule are at least a quarter of
// a chunk of 4096 tokens or more).
static inline int32_t fused_hcap(int max_seq_len) {
  return (max_seq_len > 0 ? max_seq_len : 1) / FE_CH_MIN + 8;
}

static inline FusedWs fused_ws(void* base, int rows, int max_seq_len) {
  char* p = static_cast<char*>(base);
  FusedWs w;
  w.cap = max_seq_len > 0 ? max_seq_len : 1;
  w.hcap = fused_hcap(max_seq_len);
  w.cand = reinterpret_cast<uint64_t*>(p);
  p += align256(static_cast<size_t>(rows) * w.cap * 8);
  w.hdr = reinterpret_cast<uint2*>(p);
  p += align256(static_cast<size_t>(rows) * w.hcap * 8);
  w.win = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(rows) * w.hcap * FE_WIN * 2);
  w.sval = reinterpret_cast<float*>(p);
  return w;
}

size_t fused_workspace_bytes(int rows, int k, int max_seq_len) {
  const int64_t cap = max_seq_len > 0 ? max_seq_len : 1;
  return align256(static_cast<size_t>(rows) * cap * 8) +
         align256(static_cast<size_t>(rows) * fused_hcap(max_seq_len) * 8) +
         align256(static_cast<size_t>(rows) * fused_hcap(max_seq_len) * FE_WIN * 2) +
         align256(static_cast<size_t>(rows) * k * 4);
}

// Block top-k: bscore[r][c] is the value key of block c's maximum for
// selection r. The chunks covering a row write every block entry the merge
// reads, so the area needs no initial contents.
struct BlockWs {
  uint32_t* bscore;  // [rows][nblk_max]
  int64_t nblk_max;
};

static inline BlockWs block_ws(void* base, int block_size, int max_seq_len) {
  BlockWs w;
  w.nblk_max = max_seq_len > 0 ? (max_seq_len + block_size - 1) / block_size : 1;
  w.bscore = static_cast<uint32_t*>(base);
  return w;
}

size_t block_workspace_bytes(int rows, int block_size, int max_seq_len) {
  const int64_t nblk = max_seq_len > 0 ? (max_seq_len + block_size - 1) / block_size : 1;
  return align256(static_cast<size_t>(rows) * nblk * 4);
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

// A wave's scores wait in LDS and go out SK_STAGE groups at a time (a wave
// scores consecutive groups, so a run of staged groups is one contiguous
// stretch of the row): full-line stores instead of one 64-byte store per
// group.
constexpr int SK_STAGE = 32;

template <int NT, bool BF = false>
__global__ __launch_bounds__(IX_WG) void score_kernel(IndexerArgs a, float* scores, int64_t sstride) {
  __shared__ int32_t pages[IX_PAGES];
  __shared__ float stage[IX_WG / kWave][SK_STAGE * kGroup];
  int b, c;
  chunk_of(a, b, c);
  const int n = row_len(a, b);
  int tb, clen;
  chunk_span(a, c, tb, clen);
  if (tb >= n) return;
  const int te = min(n, tb + clen);
  float* srow = scores + static_cast<int64_t>(b) * sstride;
  const int l = lane_id();
  float* st = stage[uniform(static_cast<int>(threadIdx.x) / kWave)];
  int ns = 0;     // groups staged (the same in every lane)
  int first = 0;  // first token of the staged run
  auto flush = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int lim = min(ns * kGroup, te - first);
    for (int i = l; i < lim; i += kWave) srow[first + i] = st[i];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    ns = 0;
  };
  score_chunk_any<BF, NT, IX_WG, IX_RING>(a, b, tb, te, pages, [&](int j, float s, bool) {
    if (ns == 0) first = __builtin_amdgcn_readfirstlane(j - (l & 15));
    if (l < kGroup) st[ns * kGroup + l] = s;
    if (++ns == SK_STAGE) flush();
  });
  if (ns > 0) flush();
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
// chunk-major, so all workgroups stream the same key chunk (64 pages, 4096
// tokens at page 64) at about the same time and share it through the
// caches. A chunk's page ids sit in VGPRs, so a group's page is a readlane:
// no LDS and no barrier. Used when pages hold whole 16-token groups
// (page_size % 16 == 0).
//
// On the packed-prefill geometry (16384 rows, 573M row-keys) the four-row
// path runs at ~1.67 PFLOP/s of fp8 products, a third of the matrix peak;
// the per-head weighted ReLU costs two vector instructions per product
// element, about as much issue time as the products themselves. Two rows
// per wave (2 waves per SIMD) ran 5.75 ms, four rows (1 wave per SIMD,
// 52 AGPRs) 5.61 ms, one row 10.6 ms; issuing the next group's products
// before the current group's head sums did not help. The key stream itself
// is RowGroupStream (indexer_shared.hpp).

// Scores wait in LDS (PR_STAGE groups per row) and go out together, so
// stores are in flight into the key stream only once per PR_STAGE groups.
constexpr int PR_STAGE = 32;

template <int NT, int R>
__device__ __forceinline__ void score_rows(const IndexerArgs& a, float* scores, int64_t sstride, int b0,
                                           const int (&nn)[4], const int (&pr)[4], int i0, int kb, int chunk,
                                           float (&stage)[4][PR_STAGE * kGroup]) {
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
  if (kb >= ke) return;
  RowGroupStream<NT, R> st(a, q, a.block_table + static_cast<int64_t>(pr[i0]) * a.bt_stride, kb, ke);
  // lane group g holds row (g % R)'s scores; groups g >= R repeat rows
  const int l = lane_id();
  const int c = l & 15, g = l >> 4;
  auto in_order = [](int s) { return s; };
  st.prime(in_order);
  for (int s0 = 0; s0 < st.ngroups; s0 += PR_STAGE) {
    const int s1 = min(st.ngroups, s0 + PR_STAGE);
    st.run(s0, s1, in_order, [&](int s, int, float sc) {
      if (g < R) stage[g][(s - s0) * kGroup + c] = sc;
    });
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int t0 = kb + s0 * kGroup;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int lim = min(n[r] - t0, (s1 - s0) * kGroup);
      for (int i = l; i < lim; i += kWave) rows[r][t0 + i] = stage[r][i];
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    wait_vmem_all();
  }
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
    IDXTOPK_CHECK(nn[i] >= 0 && nn[i] <= a.max_seq_len, kChkSeqLen);
    pr[i] = a.row_to_batch ? load_uniform(a.row_to_batch + b) : b;
  }
  const int kb = kc * chunk;
  __shared__ float stage[PR_WG / kWave][4][PR_STAGE * kGroup];
  auto& sw = stage[uniform(static_cast<int>(threadIdx.x) / kWave)];
  if (nr == 4 && pr[0] == pr[1] && pr[1] == pr[2] && pr[2] == pr[3]) {
    score_rows<NT, 4>(a, scores, sstride, b0, nn, pr, 0, kb, chunk, sw);
    return;
  }
  for (int i0 = 0; i0 < nr; i0 += 2) {
    if (i0 + 1 < nr && pr[i0] == pr[i0 + 1]) {
      score_rows<NT, 2>(a, scores, sstride, b0, nn, pr, i0, kb, chunk, sw);
    } else {
      score_rows<NT, 1>(a, scores, sstride, b0, nn, pr, i0, kb, chunk, sw);
      if (i0 + 1 < nr) score_rows<NT, 1>(a, scores, sstride, b0, nn, pr, i0 + 1, kb, chunk, sw);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused decode score + top-k: chunk kernel, then per-row merge kernel
// ---------------------------------------------------------------------------

constexpr int MG_WG = 512;        // block merge workgroup
constexpr int FM_WG = 1024;       // fused merge workgroup
constexpr int MG_BUF = 10240;     // candidates of a row gathered in LDS (80 KB)
constexpr int MG_MID = HIST_BINS / 2;  // threshold-bin keys held in LDS (over the histogram)
constexpr int MG_MAXE = MG_MID / FM_WG;
constexpr int MG_CHUNKS = 1024;   // chunk headers of a row held in LDS
constexpr int MG_BATCH = 8;       // candidates per thread per pass of the merge
constexpr int MG_HIST_MAX = 4096;  // candidates beyond which the merge counts them through the chunks' windows
constexpr int MG_WPT = 2;          // window words per merge thread (rows of up to 64 chunks)
constexpr int MG_WIN_CHUNKS = 32;  // rows of fewer chunks count every candidate on its own
constexpr int MG_SUB_BITS = 8;    // sub-bins of the threshold bin: the next 8 bits of the value key
constexpr int MG_SUB = 1 << MG_SUB_BITS;
static_assert(MG_SUB == 4 * kWave, "one wave scans the sub-histogram, four sub-bins per lane");
static_assert(MG_CHUNKS >= MG_SUB, "the sub-histogram reuses the chunk counts");

static_assert(HIST_BINS == 16 * IX_WG, "16 histogram bins per thread");
constexpr int MG_HPER = HIST_BINS / FM_WG;  // histogram bins per merge thread
static_assert(MG_HPER % 4 == 0, "whole 16-byte histogram reads");

// Sub-bin of a candidate key inside its histogram bin.
__device__ __forceinline__ uint32_t sub_bin(uint64_t key) {
  return (rank_vkey(key) >> (HIST_SHIFT - MG_SUB_BITS)) & static_cast<uint32_t>(MG_SUB - 1);
}

// The PER counts of bins [PER t, PER t + PER) of an LDS histogram, for
// thread t (16-byte reads).
template <int PER>
__device__ __forceinline__ void own_bins(const uint32_t* hist, uint32_t (&c)[PER]) {
  static_assert(PER % 4 == 0, "whole 16-byte reads");
  const uint4* p = reinterpret_cast<const uint4*>(hist) + threadIdx.x * (PER / 4);
#pragma unroll
  for (int j = 0; j < PER / 4; ++j) {
    const uint4 v = p[j];
    c[4 * j + 0] = v.x;
    c[4 * j + 1] = v.y;
    c[4 * j + 2] = v.z;
    c[4 * j + 3] = v.w;
  }
}

constexpr uint32_t FU_STAGE = HIST_BINS / 2;  // candidates staged in the histogram's LDS

// Selection state of one (row, chunk) in LDS.
struct ChunkSel {
  union {
    alignas(16) uint32_t hist[HIST_BINS];  // the chunk's histogram, until its bound is known
    uint64_t stage[FU_STAGE];              // then the chunk's candidates
  };
  uint32_t scratch[16];
  uint32_t lcnt;
  uint32_t lcnt2;
};

struct ChunkLds {
  ChunkSel sel;
  int32_t pages[IX_PAGES];
};


// How many of its own best tokens a chunk sends to the merge: of the row's n
// tokens, the chunk holds cnt, so on average mu = k * cnt / n of the row's k
// best (fewer than that when the chunk is a random part of the row: the
// count is binomial, its standard deviation below sqrt(mu)). Sending mu +
// 6 sqrt(mu) + 16 leaves a margin of more than six standard deviations; a
// row whose best tokens crowd into some chunks beyond that is caught by the
// merge's check and scored again there. When the rank reaches cnt (always
// when n <= k) the chunk sends every token.
__device__ __forceinline__ uint32_t chunk_rank(int k, int cnt, int n) {
  const float mu = static_cast<float>(k) * static_cast<float>(cnt) / static_cast<float>(n);
  const float r = mu + 6.0f * sqrtf(mu) + 16.0f;
  return r >= static_cast<float>(cnt) ? static_cast<uint32_t>(cnt) + 1u : static_cast<uint32_t>(r);
}

// After a chunk's scores (scr[0 .. cnt), tokens tb .. tb + cnt - 1 of row
// b, which has n tokens) and their histogram (s.hist) are in LDS, and s.lcnt
// and s.lcnt2 are zero: the chunk's bound, its window of per-bin counts, its
// candidates and its header. Every thread of the workgroup calls.
__device__ __forceinline__ void chunk_emit(const FusedWs& ws, int k, int b, int c, int tb, int cnt, int n,
                                           const float* scr, ChunkSel& s) {
  const int tid = threadIdx.x;
  uint64_t* cand = ws.cand + static_cast<int64_t>(b) * ws.cap + tb;
  // The chunk's bound: the highest bin whose count from the top reaches
  // chunk_rank (bin 0, every token, when the chunk holds fewer).
  uint32_t c16[16];
  own_bins<16>(s.hist, c16);
  const BinThreshold own = wg_threshold_counts<IX_WG, 16>(c16, chunk_rank(k, cnt, n), s.scratch);
  const uint32_t bin_c = own.all ? 0u : own.bin;
  // the candidates per bin for bins bin_c .. bin_c + FE_WIN - 1 (this
  // thread holds the counts of bins 16 tid .. 16 tid + 15)
  uint16_t* win = reinterpret_cast<uint16_t*>(ws.win + (static_cast<int64_t>(b) * ws.hcap + c) * (FE_WIN / 2));
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t bin = 16u * static_cast<uint32_t>(tid) + static_cast<uint32_t>(i);
    if (bin >= bin_c && bin < bin_c + static_cast<uint32_t>(FE_WIN)) win[bin - bin_c] = static_cast<uint16_t>(c16[i]);
  }

  // Every token in bins >= bin_c, as unique keys: staged in LDS (over the
  // histogram, no longer read) with one slot reservation per wave per batch,
  // then copied out coalesced. If more than FU_STAGE pass, a second pass
  // writes them straight out instead.
  constexpr int EB = 8;
  for (int i0 = 0; i0 < cnt; i0 += EB * IX_WG) {
    uint32_t key[EB];
    bool keep[EB];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int i = i0 + j * IX_WG + tid;
      key[j] = float_key(scr[i < cnt ? i : 0]);
      keep[j] = i < cnt && (key[j] >> HIST_SHIFT) >= bin_c;
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
  if (m <= FU_STAGE) {
    for (uint32_t i = tid; i < m; i += IX_WG) cand[i] = s.stage[i];
  } else {
    for (int i0 = 0; i0 < cnt; i0 += EB * IX_WG) {
      uint32_t key[EB];
      bool keep[EB];
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        const int i = i0 + j * IX_WG + tid;
        key[j] = float_key(scr[i < cnt ? i : 0]);
        keep[j] = i < cnt && (key[j] >> HIST_SHIFT) >= bin_c;
        mine += keep[j];
      }
      uint32_t at = wave_reserve(mine, &s.lcnt2);
#pragma unroll
      for (int j = 0; j < EB; ++j)
        if (keep[j]) cand[at++] = rank_key(key[j], static_cast<uint32_t>(tb + i0 + j * IX_WG + tid));
    }
  }
  if (tid == 0) ws.hdr[static_cast<int64_t>(b) * ws.hcap + c] = make_uint2(m, bin_c);
}

// One workgroup per (row, chunk). Dynamic LDS: the chunk's scores (a.chunk
// floats). Nothing here waits on another workgroup: the chunk's bound comes
// from its own histogram, its candidates go to its own tokens' range of the
// row's candidate area, its count and bound to its own header.
template <int NT, bool BF = false>
__global__ __launch_bounds__(IX_WG) void fused_chunk_kernel(IndexerArgs a, FusedWs ws, int k) {
  extern __shared__ float sc[];
  __shared__ ChunkLds s;
  const int tid = threadIdx.x;
  int b, c;
  chunk_of(a, b, c);
  const int n = row_len(a, b);
  int tb, clen;
  chunk_span(a, c, tb, clen);
  if (tb >= n) return;
  const int te = min(n, tb + clen);
  const int cnt = te - tb;

  for (int i = tid; i < HIST_BINS; i += IX_WG) s.sel.hist[i] = 0;
  if (tid == 0) {
    s.sel.lcnt = 0;
    s.sel.lcnt2 = 0;
  }
  // (score_chunk synchronises before its first emit). A bf16 cache is read
  // with ordinary loads for large batches (the second half of each line then
  // comes from the cache) and nontemporal ones for decode batches.
  auto emit = [&](int j, float v, bool valid) {
    if (valid) {
      sc[j - tb] = v;
      atomicAdd(&s.sel.hist[float_key(v) >> HIST_SHIFT], 1u);
    }
  };
  if (a.cached_keys)
    score_chunk_any<BF, NT, IX_WG, IX_RING, true>(a, b, tb, te, s.pages, emit);
  else
    score_chunk_any<BF, NT, IX_WG, IX_RING, false>(a, b, tb, te, s.pages, emit);
  __syncthreads();

  chunk_emit(ws, k, b, c, tb, cnt, n, sc, s.sel);
}

// ---------------------------------------------------------------------------
// Fused decode, two rows of one request per workgroup
// ---------------------------------------------------------------------------
//
// Multi-token decode rows (row_to_batch; a request's rows next to each
// other) read the same keys. Here a workgroup takes rows b0 and b0 + 1 over
// one chunk: its four waves split the chunk's 16-token groups, and each
// group is loaded once per wave and scored against both rows
// (RowGroupStream with score16x2, whose sums run in the per-row scorer's
// order, so the scores are bit-identical). Each row keeps its own scores and
// histogram in LDS; its chunk bound, window, candidates and header then
// follow as in fused_chunk_kernel, so the merge reads the same workspace.
// Rows of a pair that do not share a block-table row are scored one after
// the other.
//
// Pair slot P = (quad, chunk) is taken by workgroups 16 (P / 8) + P % 8 + 8 h
// for the rows 4 quad + 2 h and 4 quad + 2 h + 1 (h = 0, 1): the dispatcher
// sends both to XCD P % 8, so a quad's four rows read the chunk's keys
// through one L2. The row index rotates with the chunk as in chunk_of.
// Requires batch % 4 == 0 (quad_map).
__device__ __forceinline__ void pair_chunk_of(const IndexerArgs& a, int& b0, int& c) {
  const int i = blockIdx.x;
  const int h = (i >> 3) & 1;
  const int Q = ((i >> 4) << 3) | (i & 7);
  const int nq = a.batch >> 2;
  c = Q / nq;
  b0 = 4 * ((Q + c) % nq) + 2 * h;
}

// Workgroups of the pair grid: every (pair, chunk), in whole groups of 16.
static inline unsigned pair_chunk_grid(const IndexerArgs& a) {
  const int64_t n = static_cast<int64_t>(a.nchunk_max) * (a.batch / 2);
  return static_cast<unsigned>((n + 15) / 16 * 16);
}

// Rows b0 + r0 .. b0 + r0 + R - 1 (block-table row prow) over tokens
// [kb, ke) of the chunk that starts at tb: score j of pair row r goes to
// sc[r * chunk + j - tb] and into sel[r]'s histogram, for j < te[r].
template <int NT, int R>
__device__ __forceinline__ void pair_score_rows(const IndexerArgs& a, int b0, int r0, int prow, int kb, int ke,
                                                int tb, const int (&te)[2], float* sc, ChunkSel (&sel)[2]) {
  QOperand<NT> q[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int b = b0 + r0 + r;
    load_query<NT>(q[r], a.q + static_cast<int64_t>(b) * a.heads * kDim, a.w + static_cast<int64_t>(b) * a.heads,
                   a.q_scale[b]);
  }
  RowGroupStream<NT, R> st(a, q, a.block_table + static_cast<int64_t>(prow) * a.bt_stride, kb, ke);
  // lane group g holds row (g % R)'s scores; groups g >= R repeat rows
  const int l = lane_id();
  const int c = l & 15, g = l >> 4;
  const int r = r0 + (g < R ? g : 0);
  const int lim = g < R ? te[r] : INT32_MIN;
  float* srow = sc + r * a.chunk - tb;
  uint32_t* hist = sel[r].hist;
  auto in_order = [](int s) { return s; };
  st.prime(in_order);
  st.run(0, st.ngroups, in_order, [&](int, int gi, float v) {
    const int j = kb + gi * kGroup + c;
    if (j < lim) {
      srow[j] = v;
      atomicAdd(&hist[float_key(v) >> HIST_SHIFT], 1u);
    }
  });
}

// Dynamic LDS: the two rows' scores (2 a.chunk floats).
template <int NT>
__global__ __launch_bounds__(IX_WG, 3) void fused_pair_chunk_kernel(IndexerArgs a, FusedWs ws, int k) {
  extern __shared__ float sc[];
  __shared__ ChunkSel sel[2];
  const int tid = threadIdx.x;
  int b0, c;
  pair_chunk_of(a, b0, c);
  int tb, clen;
  chunk_span(a, c, tb, clen);
  const int n[2] = {row_len(a, b0), row_len(a, b0 + 1)};
  const int nmax = max(n[0], n[1]);
  if (tb >= nmax) return;
  // a row with te[r] <= tb has no token in this chunk
  const int te[2] = {min(n[0], tb + clen), min(n[1], tb + clen)};
  for (int i = tid; i < HIST_BINS; i += IX_WG) {
    sel[0].hist[i] = 0;
    sel[1].hist[i] = 0;
  }
  if (tid == 0) {
    sel[0].lcnt = 0;
    sel[0].lcnt2 = 0;
    sel[1].lcnt = 0;
    sel[1].lcnt2 = 0;
  }
  __syncthreads();

  const int ke = min(nmax, tb + clen);
  const int G = (ke - tb + kGroup - 1) / kGroup;
  const int wave = uniform(tid / kWave);
  const int per = (G + IX_WG / kWave - 1) / (IX_WG / kWave);
  const int g_lo = wave * per;
  const int g_hi = min(G, g_lo + per);
  if (g_lo < g_hi) {
    const int kb = tb + g_lo * kGroup;
    const int kw = min(ke, tb + g_hi * kGroup);
    const int pr[2] = {load_uniform(a.row_to_batch + b0), load_uniform(a.row_to_batch + b0 + 1)};
    IDXTOPK_CHECK(pr[0] >= 0 && pr[1] >= 0, kChkRowToBatch);
    if (pr[0] == pr[1]) {
      pair_score_rows<NT, 2>(a, b0, 0, pr[0], kb, kw, tb, te, sc, sel);
    } else {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int kr = min(kw, te[r]);
        if (kb < kr) pair_score_rows<NT, 1>(a, b0, r, pr[r], kb, kr, tb, te, sc, sel);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (te[r] > tb) chunk_emit(ws, k, b0 + r, c, tb, te[r] - tb, n[r], sc + r * a.chunk, sel[r]);
}

constexpr int MG_SPEC = 8;  // candidate loads per thread issued with the headers
static_assert(MG_SPEC * FM_WG <= MG_BUF, "the first loads fit the gather buffer");
constexpr int MG_PAGES = 8192;           // block-table entries of a row staged in LDS
constexpr int MG_PG_PER = MG_PAGES / FM_WG;

struct MergeLds {
  uint64_t buf[MG_BUF];  // the row's candidates (or, rescoring, the staged pages)
  union {
    alignas(16) uint32_t hist[HIST_BINS];  // histogram of the candidates' bins
    uint64_t mid[MG_MID];                  // then the threshold bin's keys
  };
  int32_t pages[MG_PAGES];       // the row's block-table entries (rows of at most MG_PAGES pages)
  uint32_t coff[MG_CHUNKS + 1];  // first candidate of each chunk in the gathered order
  uint32_t ctb[MG_CHUNKS];       // first token of each chunk
  alignas(16) uint32_t ccnt[MG_CHUNKS];  // candidates of each chunk (then the sub-histogram)
  uint32_t cbin[MG_CHUNKS];       // bound bin of each chunk
  SelectLds sel;
  uint32_t scratch[24];
  uint32_t ocnt;
  uint32_t mcnt;
  uint32_t fcnt;
  uint32_t maxbin;
};


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

// Workgroup-wide exclusive prefix sum of one value per thread (every thread
// must call); `scratch` holds at least WG/64 words. Returns the thread's
// offset, and the total in `total`.
template <int WG>
__device__ __forceinline__ uint32_t wg_exclusive_sum(uint32_t x, uint32_t* scratch, uint32_t& total) {
  constexpr int NW = WG / kWave;
  const int wave = threadIdx.x / kWave;
  const uint32_t incl = wave_prefix_incl(x);
  if (lane_id() == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = scratch[w];
    before += w < wave ? t : 0u;
    total += t;
  }
  __syncthreads();
  return before + incl - x;
}

// Where the merge reads the row's candidates: gathered in LDS, in the
// chunks' ranges of the row's candidate area (too many to gather), or,
// after rescoring, packed at the start of that area.
struct CandSource {
  const uint64_t* lds;      // gathered (or null)
  const uint64_t* list;     // packed list in the workspace (or null)
  const uint64_t* regions;  // the row's candidate area, chunk ranges
  const uint32_t* coff;     // chunk offsets in the gathered order (LDS)
  const uint32_t* ctb;      // chunk first tokens (LDS)
  int nch;
  __device__ __forceinline__ uint64_t at(uint32_t i) const {
    if (lds) return lds[i];
    if (list) return list[i];
    // the chunk holding flat index i: the last c with coff[c] <= i
    int lo = 0, hi = nch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (coff[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    return regions[ctb[lo] + (i - coff[lo])];
  }
};

// Number of chunks of the schedule whose first token lies below n
// (chunk_span grows with the chunk index).
__device__ __forceinline__ int chunks_below(const IndexerArgs& a, int n) {
  if (n <= 0) return 0;
  int c;
  if (n <= a.tok_half) {
    c = (n + a.chunk - 1) / a.chunk;
  } else if (n <= a.tok_quarter) {
    const int h = a.chunk / 2;
    c = a.n_full + (n - a.tok_half + h - 1) / h;
  } else {
    const int q = a.chunk / 4;
    c = a.n_full + a.n_half + (n - a.tok_quarter + q - 1) / q;
  }
  return c < a.nchunk_max ? c : a.nchunk_max;
}

// One workgroup per row (see the section comment above). Leaves nothing in
// the workspace that a later call depends on.
template <int NT, bool BF = false>
__global__ __launch_bounds__(FM_WG) void fused_merge_kernel(IndexerArgs a, FusedWs ws, FusedOut o) {
  __shared__ MergeLds s;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int b = blockIdx.x;
  const int n = row_len(a, b);
  const uint32_t k = static_cast<uint32_t>(o.k);
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  uint64_t* cand = ws.cand + static_cast<int64_t>(b) * ws.cap;
  const uint2* hdr = ws.hdr + static_cast<int64_t>(b) * ws.hcap;
  const int32_t* bt_row = bt_row_of(a, b);
  const int nch = chunks_below(a, n);
  const bool staged = n > 0 && nch <= MG_CHUNKS;
  const int npages = n > 0 ? static_cast<int>(fdiv(static_cast<uint32_t>(n - 1), a.pdiv)) + 1 : 0;
  const bool pages_staged = !o.keep_positions && npages <= MG_PAGES;

  wg_select_init<FM_WG>(s.sel);
  for (int i = tid; i < HIST_BINS; i += FM_WG) s.hist[i] = 0;
  if (tid == 0) {
    s.ocnt = 0;
    s.mcnt = 0;
    s.fcnt = 0;
    s.maxbin = 0;
  }

  // In flight together: the chunk headers, the first `spec` candidates of
  // every chunk (MG_SPEC * FM_WG entries spread evenly over the row's chunks;
  // most chunks send fewer), and the row's block table.
  constexpr int PC = MG_CHUNKS / FM_WG;
  uint2 h[PC];
  const int spec = staged ? MG_SPEC * FM_WG / nch : 1;
  const float rspec = 1.0f / static_cast<float>(spec);
  // flat index f -> (chunk c, entry j): a float estimate of f / spec (f <
  // 2^14), corrected by one step
  auto split = [&](int f, int& c, int& j) {
    c = static_cast<int>(static_cast<float>(f) * rspec);
    c -= c * spec > f;
    c += (c + 1) * spec <= f;
    j = f - c * spec;
  };
  uint64_t sk[MG_SPEC];
  int32_t pg[MG_PG_PER];
  // the chunks' candidate-count windows, for rows of many chunks (long rows,
  // whose candidates crowd into few bins) when they fit MG_WPT words per thread
  constexpr int WW = FE_WIN / 2;  // window words per chunk
  const bool windows = staged && nch >= MG_WIN_CHUNKS && nch * WW <= MG_WPT * FM_WG;
  uint32_t wv[MG_WPT];
  if (staged) {
#pragma unroll
    for (int e = 0; e < PC; ++e) {
      const int c = tid * PC + e;
      h[e] = c < nch ? hdr[c] : make_uint2(0u, 0u);
    }
    const uint32_t* wrow = ws.win + static_cast<int64_t>(b) * ws.hcap * WW;
#pragma unroll
    for (int r = 0; r < MG_WPT; ++r) {
      const int f = r * FM_WG + tid;
      wv[r] = windows && f < nch * WW ? wrow[f] : 0u;
    }
#pragma unroll
    for (int e = 0; e < MG_SPEC; ++e) {
      int c, j;
      split(e * FM_WG + tid, c, j);
      int tb, clen;
      chunk_span(a, c < nch ? c : 0, tb, clen);
      // within the chunk's own tokens, so inside the row's area
      sk[e] = c < nch && j < clen && tb + j < n ? cand[tb + j] : 0ull;
    }
  }
  if (pages_staged) {
#pragma unroll
    for (int r = 0; r < MG_PG_PER; ++r) {
      const int i = r * FM_WG + tid;
      pg[r] = i < npages ? bt_row[i] : 0;
    }
  }

  // Chunk counts prefix-summed into coff; the highest chunk bound.
  uint32_t total = 0;
  if (staged) {
    uint32_t sum = 0, mx = 0;
#pragma unroll
    for (int e = 0; e < PC; ++e) {
      sum += h[e].x;
      mx = h[e].y > mx ? h[e].y : mx;
    }
    uint32_t off = wg_exclusive_sum<FM_WG>(sum, s.scratch, total);
#pragma unroll
    for (int e = 0; e < PC; ++e) {
      const int c = tid * PC + e;
      if (c < nch) {
        int tb, clen;
        chunk_span(a, c, tb, clen);
        IDXTOPK_CHECK(h[e].x <= static_cast<uint32_t>(min(clen, n - tb)), kChkChunkCount);
        s.coff[c] = off;
        s.ctb[c] = static_cast<uint32_t>(tb);
        s.ccnt[c] = h[e].x;
        s.cbin[c] = h[e].y;
      }
      off += h[e].x;
    }
    if (tid == 0) s.coff[nch] = total;
    mx = wave_max_u32(mx);
    if (lane == 0) atomicMax(&s.maxbin, mx);
  }
  __syncthreads();
  const bool gathered = staged && total <= static_cast<uint32_t>(MG_BUF);
  // Many candidates crowd into few histogram bins (long rows: the row's top
  // sliver), where per-candidate atomics serialise on those bins; such rows
  // add their chunks' windows instead (one add per chunk and bin) and count
  // on their own only the candidates past their chunk's window.
  const bool use_win = windows && total > static_cast<uint32_t>(MG_HIST_MAX);
  auto count = [&](uint64_t key, int c) {
    const uint32_t bin = rank_vkey(key) >> HIST_SHIFT;
    if (!use_win || bin >= s.cbin[c] + static_cast<uint32_t>(FE_WIN)) atomicAdd(&s.hist[bin], 1u);
  };
  // Place the loaded candidates: into the histogram of their bins, and into
  // LDS when they all fit; then load what the first loads did not cover
  // (chunks that sent more than `spec`), one wave per chunk.
  if (staged) {
#pragma unroll
    for (int e = 0; e < MG_SPEC; ++e) {
      int c, j;
      split(e * FM_WG + tid, c, j);
      if (c < nch && static_cast<uint32_t>(j) < s.ccnt[c]) {
        if (gathered) s.buf[s.coff[c] + j] = sk[e];
        count(sk[e], c);
      }
    }
    if (use_win) {
#pragma unroll
      for (int r = 0; r < MG_WPT; ++r) {
        const int f = r * FM_WG + tid;
        if (f < nch * WW) {
          // window entries of bins past the last were never written
          const uint32_t bin = s.cbin[f / WW] + 2u * static_cast<uint32_t>(f % WW);
          const uint32_t lo = wv[r] & 0xFFFFu, hi = wv[r] >> 16;
          if (lo != 0u && bin < static_cast<uint32_t>(HIST_BINS)) atomicAdd(&s.hist[bin], lo);
          if (hi != 0u && bin + 1u < static_cast<uint32_t>(HIST_BINS)) atomicAdd(&s.hist[bin + 1u], hi);
        }
      }
    }
    for (int c = wave; c < nch; c += FM_WG / kWave) {
      const uint32_t cnt = s.ccnt[c];
      if (cnt <= static_cast<uint32_t>(spec)) continue;
      const uint32_t tb = s.ctb[c], off = s.coff[c];
      for (uint32_t j = spec + lane; j < cnt; j += kWave) {
        const uint64_t key = cand[tb + j];
        if (gathered) s.buf[off + j] = key;
        count(key, c);
      }
    }
  }
  if (pages_staged) {
#pragma unroll
    for (int r = 0; r < MG_PG_PER; ++r) {
      const int i = r * FM_WG + tid;
      if (i < npages) s.pages[i] = pg[r];
    }
  }
  __syncthreads();

  // Output of a selected position: its slot when the row's block table is
  // staged in LDS; otherwise the position itself (for the sort pass, or for
  // positions_to_slots below, which batches the block-table lookups).
  auto out_of = [&](uint32_t pos) -> int32_t {
    IDXTOPK_CHECK(pos < static_cast<uint32_t>(n), kChkPosition);
    if (!pages_staged) return static_cast<int32_t>(pos);
    const uint32_t lp = fdiv(pos, a.pdiv);
    uint32_t x = (static_cast<uint32_t>(s.pages[lp]) - lp) * P;
    asm volatile("" : "+v"(x));  // a 64-bit mad here would wait on loads in flight
    return static_cast<int32_t>(x + pos);
  };

  // The threshold bin: the bin of the candidates' k-th best key, from the
  // histogram of their bins. The selection is the row's when that bin is at
  // or above every chunk's bound (each chunk sent all of its tokens in bins
  // >= its bound, so every token of the row in bins above it, and every
  // token of the bin at or above the k-th key, is a candidate), or, with at
  // most k candidates, when every token was sent. Then the keys above the
  // bin are emitted and those in it selected exactly, from LDS when the
  // candidates were gathered there, else from the chunks' ranges.
  // The chunk counts are not read again: their words hold the threshold
  // bin's sub-histogram (the next MG_SUB_BITS bits of the value key), built
  // while classifying (the barriers below order the clearing before it).
  uint32_t* sub = s.ccnt;
  for (int i = tid; i < MG_SUB; i += FM_WG) sub[i] = 0u;
  CandSource src{gathered ? s.buf : nullptr, nullptr, cand, s.coff, s.ctb, nch};
  uint32_t ncand = total;
  BinThreshold th{0u, 0u, 0u, true};
  bool ok = false;
  uint32_t lo_bin = 0u;  // rescoring keeps the tokens in bins >= lo_bin
  if (staged) {
    uint32_t h8[MG_HPER];
    own_bins<MG_HPER>(s.hist, h8);
    th = wg_threshold_counts<FM_WG, MG_HPER>(h8, k, s.scratch);
    // the histogram (windows included) counts every candidate once
    IDXTOPK_CHECK(th.total == total, kChkMergeCount);
    ok = th.all ? total == static_cast<uint32_t>(n) : th.bin >= s.maxbin;
    lo_bin = th.all ? 0u : th.bin;  // the candidates' k-th best key is at or below the row's
  }
  if (!ok && n > 0) {
    // Score the row again and keep every token in bins >= lo_bin: the
    // candidates' k-th best key is at or below the row's k-th best, so no
    // token of the row's top k is dropped.
    __syncthreads();
    for (int i = tid; i < HIST_BINS; i += FM_WG) s.hist[i] = 0;
    if (tid == 0) s.fcnt = 0;
    int32_t* spages = reinterpret_cast<int32_t*>(s.buf);
    const int64_t span64 = (static_cast<int64_t>(IX_PAGES - 2) * a.page_size) / kGroup * kGroup;
    const int span = static_cast<int>(span64 > kGroup ? span64 : kGroup);
    for (int t0 = 0; t0 < n; t0 += span) {
      const int t1 = min(n, t0 + span);
      score_chunk_any<BF, NT, FM_WG, 1, true>(a, b, t0, t1, spages, [&](int j, float v, bool valid) {
        const uint32_t key = float_key(v);
        const bool keep = valid && (key >> HIST_SHIFT) >= lo_bin;
        const uint64_t mk = ballot(keep);
        if (mk) {
          uint32_t base = 0;
          if (lane_id() == 0) base = atomicAdd(&s.fcnt, static_cast<uint32_t>(__popcll(mk)));
          base = uniform(base);
          if (keep) {
            cand[base + lanes_below(mk)] = rank_key(key, static_cast<uint32_t>(j));
            atomicAdd(&s.hist[key >> HIST_SHIFT], 1u);
          }
        }
      });
      __syncthreads();  // the staged pages are replaced by the next span's
    }
    ncand = s.fcnt;
    src = CandSource{nullptr, cand, cand, s.coff, s.ctb, 0};
    uint32_t h8[MG_HPER];
    own_bins<MG_HPER>(s.hist, h8);
    th = wg_threshold_counts<FM_WG, MG_HPER>(h8, k, s.scratch);
  }
  const uint32_t bstar = th.all ? 0u : th.bin;
  const uint32_t need = th.all ? 0u : k - th.above;

  // Classify: keys above the threshold bin (all keys when the row holds at
  // most k) are emitted, keys inside it go to LDS (over the histogram).
  for (uint32_t i0 = 0; i0 < ncand; i0 += FM_WG * MG_BATCH) {
    uint64_t key[MG_BATCH];
    bool keep[MG_BATCH], mid[MG_BATCH];
    uint32_t nmid = 0;
#pragma unroll
    for (int j = 0; j < MG_BATCH; ++j) {
      const uint32_t i = i0 + j * FM_WG + tid;
      key[j] = i < ncand ? src.at(i) : 0ull;
    }
#pragma unroll
    for (int j = 0; j < MG_BATCH; ++j) {
      const bool valid = i0 + j * FM_WG + tid < ncand;
      const uint32_t bin = rank_vkey(key[j]) >> HIST_SHIFT;
      keep[j] = valid && (th.all || bin > bstar);
      mid[j] = valid && !th.all && bin == bstar;
      nmid += mid[j];
    }
    emit_batch<MG_BATCH>(key, keep, b, o, &s.ocnt, out_of);
    uint32_t at = wave_reserve(nmid, &s.mcnt);
#pragma unroll
    for (int j = 0; j < MG_BATCH; ++j) {
      if (mid[j]) {
        if (at < static_cast<uint32_t>(MG_MID)) s.mid[at] = key[j];
        ++at;
        atomicAdd(&sub[sub_bin(key[j])], 1u);
      }
    }
  }
  __syncthreads();
  const uint32_t nb = s.mcnt;
  if (!th.all && nb > 0 && nb <= static_cast<uint32_t>(MG_MID)) {
    // A threshold bin held in LDS (MG_MAXE keys per thread at most). Its
    // sub-histogram gives the sub-bin sb holding the need-th key from the
    // top (every wave finds it on its own): keys in higher sub-bins are
    // taken, and need2 of the cnt2 keys of sb: all of them, or the best
    // need2 by their rank among them (gathered in LDS), or, when more than
    // kSelMembers keys share sb (equal scores), by the workgroup select
    // over those keys alone.
    const uint4 c4 = reinterpret_cast<const uint4*>(sub)[lane];  // sub-bins 4 lane .. 4 lane + 3
    const uint32_t cb[4] = {c4.x, c4.y, c4.z, c4.w};
    const uint32_t local = cb[0] + cb[1] + cb[2] + cb[3];
    const uint32_t incl = wave_prefix_incl(local);
    const uint32_t above_l = __builtin_amdgcn_readlane(incl, kWave - 1) - incl;
    const bool mine = above_l < need && above_l + local >= need;
    uint32_t sbl = 0u, above2 = above_l, cnt2 = 0u;
    if (mine) {
      int i = 3;
      for (; i > 0; --i) {
        if (above2 + cb[i] >= need) break;
        above2 += cb[i];
      }
      sbl = 4u * static_cast<uint32_t>(lane) + static_cast<uint32_t>(i);
      cnt2 = cb[i];
    }
    const int srcl = __builtin_ctzll(ballot(mine));
    const uint32_t sb = __builtin_amdgcn_readlane(sbl, srcl);
    const uint32_t need2 = need - __builtin_amdgcn_readlane(above2, srcl);
    cnt2 = __builtin_amdgcn_readlane(cnt2, srcl);
    const bool all2 = cnt2 == need2;
    IDXTOPK_CHECK(need2 >= 1u && cnt2 >= need2, kChkMergeCount);
    uint64_t keys[MG_MAXE];
    bool keep[MG_MAXE], tie[MG_MAXE];
#pragma unroll
    for (int e = 0; e < MG_MAXE; ++e) {
      const uint32_t i = tid + e * FM_WG;
      const bool valid = i < nb;
      keys[e] = valid ? s.mid[i] : 0ull;
      const uint32_t sbk = sub_bin(keys[e]);
      keep[e] = valid && (sbk > sb || (sbk == sb && all2));
      tie[e] = valid && sbk == sb && !all2;
    }
    emit_batch<MG_MAXE>(keys, keep, b, o, &s.ocnt, out_of);
    if (!all2 && cnt2 <= static_cast<uint32_t>(kSelMembers)) {
      // s.sel.mcnt is zero here (wg_select_init) and is left zero again
#pragma unroll
      for (int e = 0; e < MG_MAXE; ++e)
        if (tie[e]) s.sel.members[atomicAdd(&s.sel.mcnt, 1u)] = keys[e];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < MG_MAXE; ++e) {
        uint32_t rank = 0u;
        if (tie[e])
          for (uint32_t j = 0; j < cnt2; ++j) rank += s.sel.members[j] > keys[e];
        keep[e] = tie[e] && rank < need2;
      }
      emit_batch<MG_MAXE>(keys, keep, b, o, &s.ocnt, out_of);
      if (tid == 0) s.sel.mcnt = 0u;
    } else if (!all2) {
      uint64_t mn = ~0ull, mx = 0;
#pragma unroll
      for (int e = 0; e < MG_MAXE; ++e)
        if (tie[e]) {
          mn = keys[e] < mn ? keys[e] : mn;
          mx = keys[e] > mx ? keys[e] : mx;
        }
      wg_range<FM_WG>(mn, mx, s.sel);
      const uint64_t T = wg_select<FM_WG>(
          [&](auto&& f) {
#pragma unroll
            for (int e = 0; e < MG_MAXE; ++e)
              if (tie[e]) f(keys[e]);
          },
          need2, mn, mx, s.sel);
#pragma unroll
      for (int e = 0; e < MG_MAXE; ++e) keep[e] = tie[e] && keys[e] >= T;
      emit_batch<MG_MAXE>(keys, keep, b, o, &s.ocnt, out_of);
    }
  } else if (!th.all && nb > 0) {
    // threshold bin larger than its LDS area: select straight from the
    // candidates (several passes over them)
    auto each_mid = [&](auto&& f) {
      for (uint32_t i = tid; i < ncand; i += FM_WG) {
        const uint64_t key = src.at(i);
        if ((rank_vkey(key) >> HIST_SHIFT) == bstar) f(key);
      }
    };
    uint64_t mn = ~0ull, mx = 0;
    each_mid([&](uint64_t key) {
      mn = key < mn ? key : mn;
      mx = key > mx ? key : mx;
    });
    wg_range<FM_WG>(mn, mx, s.sel);
    const uint64_t T = wg_select<FM_WG>(each_mid, need, mn, mx, s.sel);
    for (uint32_t i0 = 0; i0 < ncand; i0 += FM_WG * MG_BATCH) {
      uint64_t key[MG_BATCH];
      bool keep[MG_BATCH];
#pragma unroll
      for (int j = 0; j < MG_BATCH; ++j) {
        const uint32_t i = i0 + j * FM_WG + tid;
        key[j] = i < ncand ? src.at(i) : 0ull;
        keep[j] = i < ncand && (rank_vkey(key[j]) >> HIST_SHIFT) == bstar && key[j] >= T;
      }
      emit_batch<MG_BATCH>(key, keep, b, o, &s.ocnt, out_of);
    }
  }
  __syncthreads();
  if (!pages_staged && !o.keep_positions)
    positions_to_slots<FM_WG, 8>(a, b, o, min(s.ocnt, k), [&](uint32_t lp) { return bt_row[lp]; });
  // padding for rows shorter than k
  for (uint32_t i = min(s.ocnt, k) + tid; i < k; i += FM_WG) {
    o.slots[static_cast<int64_t>(b) * o.k + i] = -1;
    if (o.scores) o.scores[static_cast<int64_t>(b) * o.k + i] = -__builtin_inff();
  }
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
  const int n = row_len(a, b);
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
  const int n = row_len(a, b);
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
    IDXTOPK_CHECK(i >= nsel || s.sel_blocks[i] < nblk, kChkBlock);
    const int32_t pb = i < nsel ? bt_row[s.sel_blocks[i]] : -1;
    IDXTOPK_CHECK(i >= nsel || pb >= 0, kChkPageId);
    o.blocks[static_cast<int64_t>(sel_row) * top + i] = pb;
    s.phys[i] = pb;
  }
  if (o.slots) {
    __syncthreads();
    write_slot_list<MG_WG>(o.slots + static_cast<int64_t>(sel_row) * top * bs, top, bs, nsel, n, s.sel_blocks,
                           s.phys, a.pdiv, tid, (reinterpret_cast<uintptr_t>(o.slots) & 15u) == 0);
  }
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
  const int n = row_len(a, b);
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
// block ids and the slot lists. No workgroup barrier: a wave whose
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
  const int n = row_len(a, b);
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
    IDXTOPK_CHECK(i >= nsel || s.sel[wave][i] < nblk, kChkBlock);
    const int32_t pb = i < nsel ? bt_row[s.sel[wave][i]] : -1;
    IDXTOPK_CHECK(i >= nsel || pb >= 0, kChkPageId);
    o.blocks[static_cast<int64_t>(sel_row) * top + i] = pb;
    s.phys[wave][i] = pb;
  }
  if (o.slots) {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    write_slot_list<kWave>(o.slots + static_cast<int64_t>(sel_row) * top * bs, top, bs, nsel, n, s.sel[wave],
                           s.phys[wave], a.pdiv, lane, (reinterpret_cast<uintptr_t>(o.slots) & 15u) == 0);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------


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

uint32_t check_word_indexer(bool clear) {
#if IDXTOPK_CHECKS
  return read_check_word(clear);
#else
  (void)clear;
  return 0;
#endif
}

int launch_idx_score(const IndexerInputs& in, float* scores, int64_t score_stride, hipStream_t stream) {
  if (in.batch == 0) return 0;
  if (in.row_to_batch && !in.bf16 && in.page_size % kGroup == 0 && in.heads <= 64) {
    // rows sharing block-table rows: up to four rows per wave against one
    // key load. Chunks of 64 pages (4096 tokens at page 64), half the
    // stream's capacity: the score rows written here share the L2 with the
    // chunk's keys, and 128-page chunks measured 3.6% slower (more key
    // re-fetches), where the fused prefill call, which writes no score rows,
    // gains from them.
    int64_t chunk = static_cast<int64_t>(PR_CHUNK_PAGES / 2) * in.page_size;
    if (chunk > 4096) chunk = 4096 / in.page_size * in.page_size;
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

// Workgroups of fused_chunk_kernel that the current device holds at once
// (all compute units, with the score LDS of a FE_RESIDENT_MAX-token chunk).
// Cached per device, head count and cache format.
static int fused_resident_wgs(int heads, bool bf) {
  static int cache[2][4][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int ti = heads == 16 ? 0 : heads == 32 ? 1 : heads == 64 ? 2 : 3;
  if (cache[bf][ti][dev] > 0) return cache[bf][ti][dev];
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const size_t lds = static_cast<size_t>(FE_RESIDENT_MAX) * sizeof(float);
  hipError_t e = hipErrorInvalidValue;
#define IDXTOPK_OCC(B)                                                                                         \
  switch (heads) {                                                                                           \
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_chunk_kernel<1, B>, IX_WG, lds); break;   \
    case 32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_chunk_kernel<2, B>, IX_WG, lds); break;   \
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_chunk_kernel<4, B>, IX_WG, lds); break;   \
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_chunk_kernel<8, B>, IX_WG, lds); break;  \
    default: break;                                                                                          \
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

#define IDXTOPK_MERGE_NT(BFV, heads, grid, stream, ...)                                                        \
  switch (heads) {                                                                                            \
    case 16: hipLaunchKernelGGL((fused_merge_kernel<1, BFV>), grid, dim3(FM_WG), 0, stream, __VA_ARGS__); break; \
    case 32: hipLaunchKernelGGL((fused_merge_kernel<2, BFV>), grid, dim3(FM_WG), 0, stream, __VA_ARGS__); break; \
    case 64: hipLaunchKernelGGL((fused_merge_kernel<4, BFV>), grid, dim3(FM_WG), 0, stream, __VA_ARGS__); break; \
    case 128: hipLaunchKernelGGL((fused_merge_kernel<8, BFV>), grid, dim3(FM_WG), 0, stream, __VA_ARGS__); break; \
    default: return -2;                                                                                       \
  }

// Chunk size: when the batch fits one resident wave of chunk workgroups at
// up to FE_RESIDENT_MAX tokens each (decode batches), chunks are sized so
// that the whole grid runs at once; larger batches take chunks of up to
// FU_CH_MAX tokens on the guided schedule (about 2048 workgroups).
static IndexerArgs fused_args(const IndexerInputs& in) {
  const int64_t tokens = static_cast<int64_t>(in.batch) * (in.max_seq_len > 0 ? in.max_seq_len : 1);
  const int64_t nwg = fused_resident_wgs(in.heads, in.bf16);
  const int64_t page_cap = (static_cast<int64_t>(IX_PAGES - 2) * in.page_size) / kGroup * kGroup;
  if (nwg > 0 && tokens <= nwg * FE_RESIDENT_MAX) {
    int64_t ch = (tokens + nwg - 1) / nwg;
    ch = (ch + kGroup - 1) / kGroup * kGroup;
    if (ch < FE_CH_MIN) ch = FE_CH_MIN;
    if (ch > page_cap) ch = page_cap;
    if (ch < kGroup) ch = kGroup;
    return make_args(in, static_cast<int>(ch), false);
  }
  IndexerArgs a = make_args(in, choose_chunk(in.batch, in.max_seq_len, in.page_size, kGroup, 512, FU_CH_MAX), true);
  a.cached_keys = 1;
  return a;
}

// Two rows per chunk workgroup (fused_pair_chunk_kernel): rows in quads of
// a request (quad_map), an fp8 cache whose pages hold whole 16-token groups,
// at most 64 heads, two rows' scores within the LDS budget, and a wave's
// quarter of a chunk within the key stream's 128 page ids.
static bool fused_pairs(const IndexerInputs& in, const IndexerArgs& a) {
  if (!a.quad_map || in.bf16 || in.page_size % kGroup != 0 || in.heads > 64) return false;
  if (2 * static_cast<size_t>(a.chunk) * sizeof(float) + 2 * sizeof(ChunkSel) > FE_PAIR_LDS) return false;
  const int64_t wave_tokens = (static_cast<int64_t>(a.chunk) / kGroup + 3) / 4 * kGroup;
  return wave_tokens / in.page_size + 2 <= PR_CHUNK_PAGES;
}

// Sorted output: the merge leaves positions and scores (in the workspace's
// score area when the caller wants none), then the sort pass orders and maps
// them.
int launch_fused(const IndexerInputs& in, int k, int32_t* out_slots, float* out_scores, void* ws,
                 bool sorted, hipStream_t stream) {
  if (in.batch == 0) return 0;
  const FusedWs w = fused_ws(ws, in.batch, in.max_seq_len);
  FusedOut o;
  o.slots = out_slots;
  o.scores = sorted && !out_scores ? w.sval : out_scores;
  o.k = k;
  o.keep_positions = sorted;
  const IndexerArgs a = fused_args(in);
  // every chunk of a row has a header (chunks are at least FE_CH_MIN tokens:
  // the page-staging cap is 496 tokens or more)
  if (a.nchunk_max > w.hcap) return -4;
  (void)hipGetLastError();
  // the scores' dynamic LDS plus the static part stay within 64 KB
  static_assert(FU_CH_MAX * 4 + sizeof(ChunkLds) <= 64 * 1024, "fused chunk LDS");
  if (fused_pairs(in, a)) {
    const size_t lds = 2 * static_cast<size_t>(a.chunk) * sizeof(float);
    const dim3 grid(pair_chunk_grid(a));
    switch (in.heads) {
      case 16: hipLaunchKernelGGL(fused_pair_chunk_kernel<1>, grid, dim3(IX_WG), lds, stream, a, w, k); break;
      case 32: hipLaunchKernelGGL(fused_pair_chunk_kernel<2>, grid, dim3(IX_WG), lds, stream, a, w, k); break;
      default: hipLaunchKernelGGL(fused_pair_chunk_kernel<4>, grid, dim3(IX_WG), lds, stream, a, w, k); break;
    }
  } else {
    const dim3 grid(chunk_grid(a));
    const size_t lds = static_cast<size_t>(a.chunk) * sizeof(float);
    IDXTOPK_DISPATCH_NT_LDS(fused_chunk_kernel, in.bf16, in.heads, grid, lds, stream, a, w, k);
  }
  if (in.bf16) {
    IDXTOPK_MERGE_NT(true, in.heads, dim3(in.batch), stream, a, w, o)
  } else {
    IDXTOPK_MERGE_NT(false, in.heads, dim3(in.batch), stream, a, w, o)
  }
  if (hipGetLastError() != hipSuccess) return -4;
  if (!sorted) return 0;
  return launch_sort_rows(in.batch, k, out_slots, o.scores, nullptr, 0, nullptr, nullptr, in.block_table,
                          in.bt_stride, in.page_size, in.row_to_batch, out_scores, stream);
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
  const BlockWs w = block_ws(ws, block_size, in.max_seq_len);
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
  const BlockWs w = block_ws(ws, block_size, in.max_seq_len);
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
