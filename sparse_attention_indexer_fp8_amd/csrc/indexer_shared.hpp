// Pieces shared by the indexer kernels (indexer.hip) and the fused prefill
// indexer (prefill.hip): sizes, the selection output, the host-side chunk
// schedule, and the row-group key stream that scores up to four query rows
// against every key load.
#pragma once

#include "common.hpp"
#include "launch.hpp"
#include "score_mfma.hpp"

namespace idxtopk {

constexpr int IX_WG = 256;
constexpr int IX_RING = 4;  // 16-token key groups in flight per wave
constexpr int HIST_BITS = 12;
constexpr int HIST_BINS = 1 << HIST_BITS;
constexpr int HIST_SHIFT = 32 - HIST_BITS;
constexpr int FU_CH_MAX = 8192;
constexpr int IX_PAGES = 512;

static_assert(IX_PAGES <= kMaxChunkPages, "page staging");

static inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Where a selection goes: slots (or row-local positions) and scores.
struct FusedOut {
  int32_t* slots;
  float* scores;
  int k;
  int keep_positions;  // leave row-local positions in `slots` (the sort pass maps them)
};

// Emit this thread's keys with keep[e] set: one output reservation per
// wave, then out_of(position) (its slot, or the position itself) and the
// score are stored. All lanes of the wave must call.
template <int N, class OutOf>
__device__ __forceinline__ void emit_batch(const uint64_t (&keys)[N], const bool (&keep)[N], int b,
                                           const FusedOut& o, uint32_t* ocnt, OutOf&& out_of) {
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) mine += keep[e];
  uint32_t at = wave_reserve(mine, ocnt);
  const int64_t row = static_cast<int64_t>(b) * o.k;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if (keep[e]) {
      if (at < static_cast<uint32_t>(o.k)) {
        o.slots[row + at] = out_of(rank_pos(keys[e]));
        if (o.scores) o.scores[row + at] = key_float(rank_vkey(keys[e]));
      }
      ++at;
    }
  }
}

// ---------------------------------------------------------------------------
// Row-group key stream
// ---------------------------------------------------------------------------
//
// R query rows (R = 1, 2 or 4) that read one block-table row are scored
// together over the keys [kb, ke) of one chunk: every 16-token key group is
// loaded once and goes through the MFMA core against all R queries
// (score16x4 / score16x2 / score16), so lane (g, c) = (lane / 16, lane % 16)
// ends up holding row (g % R)'s score of the group's token c. The chunk's
// page ids sit in two VGPRs, two per lane (at most 128 pages), so a group's
// page is a readlane: no LDS and no barrier. Pages hold whole 16-token groups
// (page_size % 16 == 0). Keys come mostly from the caches here (many rows
// read them), so the operand layout is loaded directly rather than as whole
// lines plus a permute: fewer instructions.
//
// Groups are visited in the order gi = order(s), s = 0 .. ngroups - 1 (a
// permutation of the groups). A ring of RING groups' key loads is kept in
// flight: slot u holds the group of sequence index s with s % RING == u, and
// is refilled with the group RING ahead right after its scores are taken.
// run() may be called several times over consecutive ranges of s that
// start at multiples of RING; loads for the next range are already in
// flight while the caller works between two ranges.

constexpr int PR_WG = 256;  // 4 waves, each up to 4 rows
constexpr int PR_RING = 4;  // key groups in flight per wave
constexpr int PR_CHUNK_PAGES = 2 * kWave;  // page ids of a chunk: two per lane

template <int NT, int R, int RING = PR_RING>
struct RowGroupStream {
  const IndexerArgs& a;
  const QOperand<NT> (&q)[R];
  uint32_t pg0;
  int32_t pv0, pv1;  // the chunk's page ids: page i at lane i (pv0) or i - 64 (pv1)
  int kb;
  int ngroups;
  KeyPieces ring[RING];
  float ks[RING];

  __device__ __forceinline__ RowGroupStream(const IndexerArgs& a_, const QOperand<NT> (&q_)[R],
                                            const int32_t* bt_row, int kb_, int ke)
      : a(a_), q(q_), kb(kb_) {
    const int l = lane_id();
    pg0 = fdiv(static_cast<uint32_t>(kb), a.pdiv);
    const uint32_t npg = fdiv(static_cast<uint32_t>(ke - 1), a.pdiv) - pg0 + 1;  // <= PR_CHUNK_PAGES
    pv0 = static_cast<uint32_t>(l) < npg ? bt_row[pg0 + l] : 0;
    pv1 = static_cast<uint32_t>(l + kWave) < npg ? bt_row[pg0 + kWave + l] : 0;
    ngroups = (ke - kb + kGroup - 1) / kGroup;
  }

  // group gi -> this lane's 32 key bytes in the operand layout (bytes
  // [32g, 32g + 32) of token c) and the token's scale, into slot u. The
  // group lies in one page, and tokens past ke read that page's bytes.
  __device__ __forceinline__ void fetch(int gi, int u) {
    const int l = lane_id();
    const int c = l & 15, g = l >> 4;
    const uint32_t P = static_cast<uint32_t>(a.page_size);
    const int j0 = kb + gi * kGroup;
    const uint32_t pg = fdiv(static_cast<uint32_t>(j0), a.pdiv);
    const uint32_t i = pg - pg0;
    const uint32_t page = i < static_cast<uint32_t>(kWave) ? __builtin_amdgcn_readlane(pv0, i)
                                                           : __builtin_amdgcn_readlane(pv1, i - kWave);
    uint32_t m = (page - pg) * P;
    asm volatile("" : "+s"(m));
    const uint32_t s0 = m + static_cast<uint32_t>(j0);
    const uint8_t* kp0 = a.kcache + (static_cast<uint64_t>(s0 + c) << 7) + 32 * g;
    ring[u].x0 = load_v4i_stream(kp0);
    ring[u].x1 = load_v4i_stream(kp0 + 16);
    ks[u] = a.k_scale[s0 + c];
  }

  __device__ __forceinline__ float score(int u) const {
    v8i kbv;
    kbv[0] = ring[u].x0[0]; kbv[1] = ring[u].x0[1]; kbv[2] = ring[u].x0[2]; kbv[3] = ring[u].x0[3];
    kbv[4] = ring[u].x1[0]; kbv[5] = ring[u].x1[1]; kbv[6] = ring[u].x1[2]; kbv[7] = ring[u].x1[3];
    if constexpr (R == 4) return score16x4<NT>(q, kbv, ks[u]);
    else if constexpr (R == 2) return score16x2<NT>(q[0], q[1], kbv, ks[u]);
    else return score16<NT>(q[0], kbv, ks[u]);
  }

  // Issue the loads of s = 0 .. RING - 1 (repeating the last group when
  // there are fewer).
  template <class Order>
  __device__ __forceinline__ void prime(Order&& order) {
#pragma unroll
    for (int u = 0; u < RING; ++u) fetch(order(min(u, ngroups - 1)), u);
  }

  // consume(s, gi, score) for s in [s0, s1), s0 % RING == 0.
  template <class Order, class Consume>
  __device__ __forceinline__ void run(int s0, int s1, Order&& order, Consume&& consume) {
    auto step = [&](int s, int u, bool refill) __attribute__((always_inline)) {
      float sc = score(u);
      // the score is final before the slot is refilled (see score_chunk)
      asm volatile("" : "+v"(sc));
      __builtin_amdgcn_sched_barrier(0);
      if (refill) fetch(order(s + RING), u);
      consume(s, order(s), sc);
    };
    int s = s0;
    // refills below ngroups without a check
    for (; s + RING <= s1 && s + 2 * RING <= ngroups; s += RING) {
#pragma unroll
      for (int u = 0; u < RING; ++u) step(s + u, u, true);
    }
    for (; s < s1; s += RING) {
#pragma unroll
      for (int u = 0; u < RING; ++u)
        if (s + u < s1) step(s + u, u, s + u + RING < ngroups);
    }
  }
};

// ---------------------------------------------------------------------------
// Host side: chunk schedule
// ---------------------------------------------------------------------------

static inline IndexerArgs make_args(const IndexerInputs& in, int chunk, bool guided = false, int guide_align = 16) {
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
  a.max_seq_len = in.max_seq_len;
  a.chunk = chunk;
  a.quad_map = in.row_to_batch != nullptr && in.batch % 4 == 0 && in.batch >= 8;
  a.cached_keys = 0;
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
static inline unsigned chunk_grid(const IndexerArgs& a) {
  const int64_t n = static_cast<int64_t>(a.nchunk_max) * a.batch;
  return static_cast<unsigned>(a.quad_map ? (n + 31) / 32 * 32 : n);
}

// Tokens per workgroup: aim for ~2048 workgroups over the whole batch, keep
// the chunk's block-table entries within the LDS staging area, keep it a
// multiple of `align`, and stay within [lo, hi].
static inline int choose_chunk(int batch, int max_seq_len, int page_size, int align, int lo, int hi) {
  const int64_t total = static_cast<int64_t>(batch) * (max_seq_len > 0 ? max_seq_len : 1);
  int64_t ch = lo;
  while (ch < hi && total / ch > 2048) ch *= 2;
  const int64_t page_cap = static_cast<int64_t>(IX_PAGES - 2) * page_size;
  if (ch > page_cap) ch = page_cap;
  ch = (ch / align) * align;
  if (ch < align) ch = align;
  return static_cast<int>(ch);
}

}  // namespace idxtopk
