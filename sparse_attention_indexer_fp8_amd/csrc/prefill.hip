// Fused prefill indexer: the top k keys of every packed prefill row, scored
// from the paged fp8 index cache, with no score row in HBM.
//
// Pages:
//  [SGL-37889] sgl-project/sglang PR 37889 "[AMD] Enable GLM DSA prefill
//   top-k to the v2 kernel" (Motivation, Modifications): the query rows of
//   all requests of a prefill batch are packed; row_to_batch names each
//   row's request (its block-table row), each row keeps the top 512 of its
//   causal window, and the selection goes through the page table to slots.
//  [ATOM-1473] ROCm/ATOM PR 1473 "enable minimax m3 fp8 index cache and fuse
//   index_score_kernel with partial_topk kernel" (Pull request overview):
//   fusing the scores with a partial top-k removes the intermediate score
//   tensor; here that is carried from decode rows to packed prefill rows.
//
// One call, four kernels on the caller's stream:
//  0. prefill_zero_kernel clears each row's candidate count and bound and
//     the fallback queue (the workspace needs no initial contents).
//  1. prefill_chunk_kernel, one wave per (two query rows of one request,
//     chunk of keys), chunk-major, three waves per SIMD (calls of few rows:
//     four rows per wave under the balanced schedule): each 16-token key
//     group is loaded once per wave and scored against its rows
//     (RowGroupStream). The chunk's groups
//     are visited strided first: every S-th group (about 1024 tokens) is the
//     sample, whose value keys go to LDS. Per row, the sample holds on
//     average mu = k m / n of the row's k best (m sampled of the row's n
//     tokens); a lower bound of its r-th best key with r = mu + 6 sqrt(mu)
//     + 6 (the edge of a histogram bin, two 256-bin rounds at most) becomes
//     the chunk's bound for the row (no bound when r would not fit in the
//     sample or the row has at most k tokens). The chunk then keeps every
//     token at or above its bound, sampled ones included, as unique 64-bit
//     keys (value key, inverted position): staged per row in LDS by ballot
//     compaction and appended to the row's candidate list with one atomic
//     add per flush. The largest bound of a row goes to its bound word.
//  2. prefill_merge_kernel, one workgroup per row: the exact k-th key T of
//     the candidates (wg_select). When T's value key is at or above every
//     chunk's bound, every token of the row at or above T was kept by its
//     chunk, so the candidates' top k is the row's top k, and it is emitted
//     through the block table. Otherwise (a chunk's bound above the row's
//     k-th value, too few candidates, or more than the list holds) the row
//     goes to the fallback queue.
//  3. prefill_fallback_kernel: a few workgroups take the queued rows one by
//     one, score each whole row again into their own area of the workspace,
//     and select exactly from it. With no queued row it ends at once.
// The sorted-output flag adds the sort pass of sort_rows.hip.
#include <cmath>

#include "../../include/idxtopk.h"
#include "common.hpp"
#include "indexer_shared.hpp"
#include "launch.hpp"
#include "score_mfma.hpp"
#include "select.hpp"

namespace idxtopk {

constexpr int PF_SAMPLE = 64;       // sampled 16-token groups per (row, chunk), at most
constexpr int PF_RING = PR_RING;    // key groups in flight per wave
constexpr int PF_STAGE = 256;       // staged candidates per (wave, row)
constexpr int PF_MERGE_WG = 512;
constexpr int PF_MERGE_PER_MAX = 32;
constexpr int PF_FB_WGS = 16;       // workgroups of the fallback kernel
constexpr int64_t PF_MIN_WAVES = 2048;  // chunk waves a launch should hold (two per SIMD)
constexpr int64_t PF_CAP_MAX = static_cast<int64_t>(PF_MERGE_WG) * PF_MERGE_PER_MAX;

#if IDXTOPK_CHECKS
uint32_t check_word_prefill(bool clear) { return read_check_word(clear); }
#else
uint32_t check_word_prefill(bool) { return 0; }
#endif

// ---------------------------------------------------------------------------
// Workspace
// ---------------------------------------------------------------------------
//
// cand [rows][cap]  candidates (64-bit keys), in no particular order
// cnt  [rows]       candidates appended (may exceed cap: then the row is
//                   selected by the fallback)
// bound[rows]       largest chunk bound (value key; 0 = none)
// fb   [2 + rows]   fallback queue: length, next taken, row ids
// area [PF_FB_WGS][max_seq_len]  fallback rows' keys
// sval [rows][k]    selection scores for the sort pass
struct PrefillWs {
  uint64_t* cand;
  int64_t cap;
  uint32_t* cnt;
  uint32_t* bound;
  uint32_t* fb;
  uint64_t* area;
  int64_t area_cap;
  float* sval;
};

// Candidates a row of n tokens sends on average, for samples of 1024
// tokens per chunk: the k best plus each chunk's margin (6 sqrt(mu) + 6
// sampled tokens, each standing for n_chunk / 1024 tokens). The list holds
// a quarter more plus 1024, capped by what one merge workgroup holds; a row
// beyond it is selected by the fallback.
static int64_t prefill_cap(int k, int max_seq_len) {
  const double n = max_seq_len > 0 ? max_seq_len : 1;
  const double e = k + 6.0 * std::sqrt(k * n / 1024.0) + 6.0 * n / 1024.0;
  int64_t cap = (static_cast<int64_t>(1.25 * e) + 1024 + 255) / 256 * 256;
  const int64_t whole = (static_cast<int64_t>(n) + 255) / 256 * 256;
  if (cap > whole) cap = whole;
  if (cap > PF_CAP_MAX) cap = PF_CAP_MAX;
  return cap;
}

static PrefillWs prefill_ws(void* base, int rows, int k, int max_seq_len) {
  char* p = static_cast<char*>(base);
  PrefillWs w;
  w.cap = prefill_cap(k, max_seq_len);
  w.area_cap = max_seq_len > 0 ? max_seq_len : 1;
  w.cand = reinterpret_cast<uint64_t*>(p);
  p += align256(static_cast<size_t>(rows) * w.cap * 8);
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(rows) * 4);
  w.bound = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(rows) * 4);
  w.fb = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(rows + 2) * 4);
  w.area = reinterpret_cast<uint64_t*>(p);
  p += align256(static_cast<size_t>(PF_FB_WGS) * w.area_cap * 8);
  w.sval = reinterpret_cast<float*>(p);
  return w;
}

size_t prefill_workspace_bytes(int rows, int k, int max_seq_len) {
  const int64_t cap = prefill_cap(k, max_seq_len);
  const int64_t area = max_seq_len > 0 ? max_seq_len : 1;
  return align256(static_cast<size_t>(rows) * cap * 8) + 2 * align256(static_cast<size_t>(rows) * 4) +
         align256(static_cast<size_t>(rows + 2) * 4) + align256(static_cast<size_t>(PF_FB_WGS) * area * 8) +
         align256(static_cast<size_t>(rows) * k * 4);
}

// ---------------------------------------------------------------------------
// 0. Clear the counters
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void prefill_zero_kernel(PrefillWs w, int rows) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < rows) {
    w.cnt[i] = 0u;
    w.bound[i] = 0u;
  }
  if (i < 2) w.fb[i] = 0u;
}

// ---------------------------------------------------------------------------
// 1. Chunk kernel
// ---------------------------------------------------------------------------

struct PrefillParams {
  int k;
  int chunk;      // tokens per chunk
  int stride;     // S: one sampled group in S (1 when a chunk has at most PF_SAMPLE groups)
  FastDiv sdiv1;  // division by S - 1 (by 1 when S = 1)
  int ntiles;     // workgroups per chunk
  int balanced;   // nonzero: waves take (quad, chunk) pairs of the balanced schedule (prefill_chunk_kernel<NT, true>)
};

// Balanced schedule for calls of few rows (at most PF_BAL_QUADS quads, e.g.
// multi-token decode). A chunk-major grid over max_seq_len leaves the waves
// past each request's context idle and gives the others whole chunks of
// PF_SAMPLE groups. Here every wave reads the quads' lengths (lane q: quad
// q's longest row), sizes the chunks from the actual total of 16-token
// groups so that the grid's waves share it evenly (at most PF_SAMPLE groups,
// so a chunk is all sample), and takes the i-th (quad, chunk) pair in quad
// order. Every wave computes the same schedule on its own: no LDS, no
// barrier.
constexpr int PF_BAL_QUADS = kWave;

// ceil(x / d) for x < 2^24 and d >= 1, from a float estimate corrected by one
// step each way (rd = 1 / d up to rounding).
__device__ __forceinline__ uint32_t ceil_div_small(uint32_t x, uint32_t d, float rd) {
  const uint32_t y = x + d - 1u;
  uint32_t q = static_cast<uint32_t>(static_cast<float>(y) * rd);
  q -= q * d > y;
  q += (q + 1u) * d <= y;
  return q;
}

// Pair of wave index i: quad `quad`, keys from kb, `chunk` tokens per chunk.
// Returns false past the last pair. The pairs number at most the grid's
// waves W: with g = ceil(G / (W - nq)) groups per chunk, the quads' chunks
// number at most G / g + nq <= W; with g capped at PF_SAMPLE, at most nq
// ceil(max_seq_len / (16 PF_SAMPLE)), which the host's grid holds.
__device__ __forceinline__ bool balanced_pair(const IndexerArgs& a, uint32_t i, int& quad, int& kb, int& chunk) {
  const int l = lane_id();
  const int nq = (a.batch + 3) / 4;
  uint32_t gq = 0u;  // 16-token groups of quad l's longest row
  if (l < nq) {
    int m = 0;
    for (int r = 0; r < 4 && 4 * l + r < a.batch; ++r) m = max(m, row_len(a, 4 * l + r));
    gq = static_cast<uint32_t>((m + kGroup - 1) / kGroup);
  }
  const uint32_t G = wave_sum(gq);
  const uint32_t W = gridDim.x * (PR_WG / kWave);
  uint32_t g = (G + (W - nq) - 1u) / (W - nq);
  g = g < 1u ? 1u : g > static_cast<uint32_t>(PF_SAMPLE) ? static_cast<uint32_t>(PF_SAMPLE) : g;
  const uint32_t nc = gq > 0u ? ceil_div_small(gq, g, 1.0f / static_cast<float>(g)) : 0u;
  const uint32_t incl = wave_prefix_incl(nc);
  if (i >= __builtin_amdgcn_readlane(incl, kWave - 1)) return false;
  const bool here = incl - nc <= i && i < incl;
  const int src = static_cast<int>(__builtin_ctzll(ballot(here)));
  quad = src;
  kb = static_cast<int>((i - __builtin_amdgcn_readlane(incl - nc, src)) * g * kGroup);
  chunk = static_cast<int>(g * kGroup);
  return true;
}

// Per-lane lists of kept tokens: pf_list<RM>() entries (score, group) per
// lane, for waves of up to RM rows. A wave whose rows keep more than a
// quarter of that per lane on average (dense: short rows, or rows without a
// bound) flushes after every list length of groups, so no list can
// overflow; the others flush once, after the chunk, and a lane that
// outgrows its list (far beyond its average) sends its row to the fallback.
// Pair waves keep shorter lists: their LDS then leaves room for four waves
// per SIMD.
template <int RM>
constexpr int pf_list() { return RM == 4 ? 32 : 16; }

template <int RM>
struct PrefillWaveLds {
  union {
    uint32_t samp[RM][PF_SAMPLE * kGroup + kGroup];  // sampled value keys per row (0: no token); rows
                                                     // padded so the rows' lanes write distinct banks
    struct {
      float sc[pf_list<RM>() * kWave];     // then: lane l's kept scores at [i * 64 + l]
      uint32_t gi[pf_list<RM>() * kWave];  // and their groups
    } list;
  };
  alignas(16) uint32_t hist[256];          // wave_lower_bound
};

// Rows b0 + i0 .. + R - 1 (one block-table row, prow) over the chunk at kb,
// in a wave of up to RM rows.
template <int NT, int R, int RM>
__device__ __forceinline__ void prefill_rows(const IndexerArgs& a, const PrefillWs& w, const PrefillParams& pp,
                                             PrefillWaveLds<RM>& L, int b0, const int (&nn)[4], int i0, int prow,
                                             int kb) {
  static_assert(R <= RM, "rows of the wave");
  constexpr int LIST = pf_list<RM>();
  QOperand<NT> q[R];
  int n[R];
  int nmax = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int b = b0 + i0 + r;
    load_query<NT>(q[r], a.q + static_cast<int64_t>(b) * a.heads * kDim, a.w + static_cast<int64_t>(b) * a.heads,
                   a.q_scale[b]);
    n[r] = nn[i0 + r];
    nmax = max(nmax, n[r]);
  }
  const int ke = min(kb + pp.chunk, nmax);
  if (kb >= ke) return;
  static_assert(LIST % PF_RING == 0, "list segments start at multiples of the ring");
  RowGroupStream<NT, R, PF_RING> st(a, q, a.block_table + static_cast<int64_t>(prow) * a.bt_stride, kb, ke);
  const int G = st.ngroups;
  const int S = pp.stride;
  // Visiting order: the sampled groups 0, S, 2S, ... first, then the others
  // in increasing order. A chunk of at most PF_SAMPLE groups is all sample.
  const bool whole = G <= PF_SAMPLE;
  const int Se = whole ? 1 : S;
  const int cnt0 = whole ? G : (G + S - 1) / S;
  const int nA = whole ? G : min(PF_SAMPLE, (cnt0 + PF_RING - 1) / PF_RING * PF_RING);
  // after the sample, the t-th other group is t + t / (S - 1) + 1 (no
  // branches: both forms are computed and one is selected)
  auto later = [&](int s) -> int {
    const int t = s - cnt0;
    return t + static_cast<int>(fdiv(static_cast<uint32_t>(t), pp.sdiv1)) + 1;
  };
  auto order = [&](int s) -> int { return s < cnt0 ? s * Se : later(s); };

  const int l = lane_id();
  const int c = l & 15, g = l >> 4;
  const bool writer = g < R;
  int my_n = n[0];
#pragma unroll
  for (int r = 1; r < R; ++r) my_n = g == r ? n[r] : my_n;

  // Sample: value keys to LDS.
  st.prime(order);
  st.run(0, nA, order, [&](int s, int gi, float sc) {
    const int j = kb + gi * kGroup + c;
    if (writer) L.samp[g][s * kGroup + c] = j < my_n ? float_key(sc) : 0u;
  });
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  // Per row: the bound from the sample, and the sampled tokens at or above
  // it straight to the row's candidate list (one atomic round trip for all
  // rows).
  constexpr int SP = PF_SAMPLE * kGroup / kWave;  // sample entries per lane
  const uint32_t k = static_cast<uint32_t>(pp.k);
  const int m_all = nA * kGroup;
  uint32_t T[R], pre[R], kept[R], kbits[R];
  float per_lane = 0.0f;  // expected kept tokens per lane over the other groups (largest row)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    uint32_t key[SP];
    bool valid[SP];
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < SP; ++e) {
      const int i = e * kWave + l;
      key[e] = i < m_all ? L.samp[r][i] : 0u;
      valid[e] = key[e] != 0u;
      mine += valid[e];
    }
    const uint32_t m = wave_sum(mine);
    T[r] = 0u;
    float rank_f = static_cast<float>(m);
    if (n[r] > static_cast<int>(k) && m > 0u) {
      const float mu = static_cast<float>(k) * static_cast<float>(m) / static_cast<float>(n[r]);
      const uint32_t rank = static_cast<uint32_t>(ceilf(mu + 6.0f * sqrtf(mu) + 6.0f));
      if (rank < m) {
        // a lower bound is enough: a few more sampled tokens above it only
        // lower the bound further
        T[r] = wave_lower_bound<SP>(key, valid, rank, rank / 8u + 8u, L.hist);
        rank_f = static_cast<float>(rank);
      }
    }
    const float share = m > 0u ? rank_f / static_cast<float>(m) : 1.0f;
    per_lane = fmaxf(per_lane, share * static_cast<float>(G - nA));
    // this lane's sampled tokens at or above the bound, as a bit mask
    kbits[r] = 0u;
#pragma unroll
    for (int e = 0; e < SP; ++e) kbits[r] |= (valid[e] && key[e] >= T[r] ? 1u : 0u) << e;
    kept[r] = static_cast<uint32_t>(__builtin_popcount(kbits[r]));
    pre[r] = wave_prefix_incl(kept[r]);
  }
  uint32_t tot = 0u, bnd = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t t = __builtin_amdgcn_readlane(pre[r], kWave - 1);
    tot = l == r ? t : tot;
    bnd = l == r ? T[r] : bnd;
  }
  uint32_t base = 0u;
  if (l < R && tot != 0u) base = atomicAdd(w.cnt + b0 + i0 + l, tot);
  if (l < R && bnd != 0u) atomicMax(w.bound + b0 + i0 + l, bnd);
  float thr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    thr[r] = T[r] == 0u ? -__builtin_inff() : key_float(T[r]);
    if (__builtin_amdgcn_readlane(pre[r], kWave - 1) == 0u) continue;
    uint32_t at = __builtin_amdgcn_readlane(base, r) + pre[r] - kept[r];
    uint64_t* dst = w.cand + static_cast<int64_t>(b0 + i0 + r) * w.cap;
    // only this lane's kept entries (a few), not all SP of them
    for (uint32_t bits = kbits[r]; bits != 0u; bits &= bits - 1u) {
      const int i = __builtin_ctz(bits) * kWave + l;
      const uint32_t v = L.samp[r][i];
      const int j = kb + order(i >> 4) * kGroup + (i & 15);
      if (at < static_cast<uint32_t>(w.cap)) dst[at] = rank_key(v, static_cast<uint32_t>(j));
      ++at;
    }
  }
  float my_thr = thr[0];
#pragma unroll
  for (int r = 1; r < R; ++r) my_thr = g == r ? thr[r] : my_thr;
  wait_vmem_all();  // no store in flight into the key stream
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // the lists replace the sample in LDS

  // The other groups: each lane keeps its tokens at or above its row's
  // bound in its own LDS list (a float compare: it may keep a -0 against a
  // +0 bound, never drop a token); the lists then go to the rows' candidate
  // lists.
  uint32_t my_cnt = 0u;
  uint64_t* my_dst = w.cand + static_cast<int64_t>(b0 + i0 + (writer ? g : 0)) * w.cap;
  const int lim = writer ? my_n - kb - c : INT32_MIN;  // group gi holds this lane's token iff 16 gi < lim
  const int seg = per_lane > static_cast<float>(LIST / 4) ? LIST : G;
  for (int s0 = nA; s0 < G; s0 += seg) {
    st.run(s0, min(G, s0 + seg), later, [&](int, int gi, float sc) {
      if (gi * kGroup < lim && sc >= my_thr) {
        if (my_cnt < static_cast<uint32_t>(LIST)) {
          L.list.sc[my_cnt * kWave + l] = sc;
          L.list.gi[my_cnt * kWave + l] = static_cast<uint32_t>(gi);
        }
        ++my_cnt;
      }
    });
    // lanes 16 g .. 16 g + 15 hold row g's lists; a list that overflowed
    // makes its row's count exceed the candidate capacity (fallback)
    const uint32_t held = min(my_cnt, static_cast<uint32_t>(LIST));
    const uint32_t over = my_cnt > static_cast<uint32_t>(LIST) ? static_cast<uint32_t>(w.cap) + 1u : 0u;
    const uint32_t p = row16_prefix_incl(held + over);
    uint32_t fbase = 0u;
    if (c == 15 && writer && p != 0u) fbase = atomicAdd(w.cnt + b0 + i0 + g, p);
    uint32_t my_base = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t br = __builtin_amdgcn_readlane(fbase, 16 * r + 15);
      my_base = g == r ? br : my_base;
    }
    my_base += p - held - over;
    const uint32_t most = wave_max_u32(held);
    for (uint32_t i = 0; i < most; ++i)
      if (i < held && my_base + i < static_cast<uint32_t>(w.cap)) {
        const uint32_t j = static_cast<uint32_t>(kb + c) + L.list.gi[i * kWave + l] * kGroup;
        my_dst[my_base + i] = rank_key(float_key(L.list.sc[i * kWave + l]), j);
      }
    my_cnt = 0u;
    wait_vmem_all();  // no store in flight into the key stream
  }
}

// One wave per (RM rows, chunk): RM = 4 (quads, one wave per SIMD: the four
// rows' query operands take most of the registers) or RM = 2 (pairs, three
// waves per SIMD). Per group of 16 keys a quad issues 16 products and their
// ReLU and weighted sums from one wave, which leaves the matrix core idle
// while that wave waits on its own results; three pair waves per SIMD keep
// it busy from the others. A quad's two pairs sit in one workgroup and read
// the same keys on the same compute unit.
template <int NT, bool BAL, int RM>
__global__ __launch_bounds__(PR_WG, RM == 4 ? 1 : 3) void prefill_chunk_kernel(IndexerArgs a, PrefillWs w,
                                                                                PrefillParams pp) {
  static_assert(RM == 4 || (RM == 2 && !BAL), "rows per wave");
  __shared__ PrefillWaveLds<RM> lds[PR_WG / kWave];
  const int wave = uniform(static_cast<int>(threadIdx.x) / kWave);
  int unit, kb;
  if constexpr (BAL) {
    if (!balanced_pair(a, blockIdx.x * (PR_WG / kWave) + wave, unit, kb, pp.chunk)) return;
  } else {
    unit = static_cast<int>(blockIdx.x % pp.ntiles) * (PR_WG / kWave) + wave;
    kb = static_cast<int>(blockIdx.x / pp.ntiles) * pp.chunk;
  }
  const int b0 = RM * unit;
  if (b0 >= a.batch) return;
  const int nr = min(RM, a.batch - b0);
  int nn[4] = {0, 0, 0, 0}, pr[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int b = b0 + (i < nr ? i : 0);
    nn[i] = i < nr ? load_uniform(a.seq_lens + b) : 0;
    IDXTOPK_CHECK(nn[i] >= 0 && nn[i] <= a.max_seq_len, kChkSeqLen);
    pr[i] = a.row_to_batch ? load_uniform(a.row_to_batch + b) : b;
    IDXTOPK_CHECK(pr[i] >= 0, kChkRowToBatch);
  }
  PrefillWaveLds<RM>& L = lds[wave];
  if constexpr (RM == 4) {
    if (nr == 4 && pr[0] == pr[1] && pr[1] == pr[2] && pr[2] == pr[3]) {
      prefill_rows<NT, 4, RM>(a, w, pp, L, b0, nn, 0, pr[0], kb);
      return;
    }
  }
  for (int i0 = 0; i0 < nr; i0 += 2) {
    if (i0 + 1 < nr && pr[i0] == pr[i0 + 1]) {
      prefill_rows<NT, 2, RM>(a, w, pp, L, b0, nn, i0, pr[i0], kb);
    } else {
      prefill_rows<NT, 1, RM>(a, w, pp, L, b0, nn, i0, pr[i0], kb);
      if (i0 + 1 < nr) prefill_rows<NT, 1, RM>(a, w, pp, L, b0, nn, i0 + 1, pr[i0 + 1], kb);
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Merge
// ---------------------------------------------------------------------------

__device__ __forceinline__ void prefill_enqueue(const PrefillWs& w, int b) {
  if (threadIdx.x == 0) {
    const uint32_t i = atomicAdd(w.fb, 1u);
    w.fb[2 + i] = static_cast<uint32_t>(b);
  }
}

// Output entry of position pos of row b: its slot through the block table,
// or the position itself when the sort pass maps it later.
struct SlotOf {
  const IndexerArgs& a;
  const int32_t* bt_row;
  bool keep_positions;
  int n;
  __device__ __forceinline__ int32_t operator()(uint32_t pos) const {
    IDXTOPK_CHECK(pos < static_cast<uint32_t>(n), kChkPosition);
    if (keep_positions) return static_cast<int32_t>(pos);
    const uint32_t pg = fdiv(pos, a.pdiv);
    const int32_t page = bt_row[pg];
    IDXTOPK_CHECK(page >= 0, kChkPageId);
    return static_cast<int32_t>(static_cast<int64_t>(page) * a.page_size + (pos - pg * a.page_size));
  }
};

template <int WG>
__device__ __forceinline__ void pad_row(const FusedOut& o, int b, uint32_t from) {
  const int64_t row = static_cast<int64_t>(b) * o.k;
  for (uint32_t i = from + threadIdx.x; i < static_cast<uint32_t>(o.k); i += WG) {
    o.slots[row + i] = -1;
    if (o.scores) o.scores[row + i] = -__builtin_inff();
  }
}

template <int PER>
__global__ __launch_bounds__(PF_MERGE_WG) void prefill_merge_kernel(IndexerArgs a, PrefillWs w, FusedOut o) {
  __shared__ SelectLds sel;
  __shared__ uint32_t ocnt;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int n = row_len(a, b);
  const uint32_t k = static_cast<uint32_t>(o.k);
  wg_select_init<PF_MERGE_WG>(sel);
  if (tid == 0) ocnt = 0u;
  const uint32_t c = w.cnt[b];
  const uint32_t bound = w.bound[b];
  const bool small = static_cast<uint32_t>(n) <= k;
  if (c > static_cast<uint32_t>(w.cap) || (small ? c != static_cast<uint32_t>(n) : c < k)) {
    prefill_enqueue(w, b);
    return;
  }
  const uint64_t* cand = w.cand + static_cast<int64_t>(b) * w.cap;
  uint64_t key[PER];
  bool valid[PER];
  uint64_t mn = ~0ull, mx = 0ull;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const uint32_t i = e * PF_MERGE_WG + tid;
    valid[e] = i < c;
    key[e] = valid[e] ? cand[i] : 0ull;
    if (valid[e]) {
      mn = key[e] < mn ? key[e] : mn;
      mx = key[e] > mx ? key[e] : mx;
    }
  }
  wg_range<PF_MERGE_WG>(mn, mx, sel);  // (its barrier also publishes the LDS initialisation)
  uint64_t T = 0ull;
  if (!small) {
    T = c > k ? wg_select<PF_MERGE_WG>(
                    [&](auto&& f) {
#pragma unroll
                      for (int e = 0; e < PER; ++e)
                        if (valid[e]) f(key[e]);
                    },
                    k, mn, mx, sel)
              : mn;
    if (rank_vkey(T) < bound) {
      prefill_enqueue(w, b);
      return;
    }
  }
  bool keep[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) keep[e] = valid[e] && key[e] >= T;
  const SlotOf slot_of{a, bt_row_of(a, b), o.keep_positions != 0, n};
  emit_batch<PER>(key, keep, b, o, &ocnt, slot_of);
  if (small) pad_row<PF_MERGE_WG>(o, b, static_cast<uint32_t>(n));
}

// ---------------------------------------------------------------------------
// 3. Fallback: whole rows scored again
// ---------------------------------------------------------------------------

constexpr int PF_FB_BATCH = 8;

template <int NT>
__global__ __launch_bounds__(IX_WG) void prefill_fallback_kernel(IndexerArgs a, PrefillWs w, FusedOut o) {
  __shared__ int32_t pages[IX_PAGES];
  __shared__ SelectLds sel;
  __shared__ uint32_t ocnt;
  __shared__ int32_t next_row;
  const int tid = threadIdx.x;
  uint64_t* area = w.area + static_cast<int64_t>(blockIdx.x) * w.area_cap;
  const uint32_t k = static_cast<uint32_t>(o.k);
  const int64_t span64 = (static_cast<int64_t>(IX_PAGES - 2) * a.page_size) / kGroup * kGroup;
  const int span = static_cast<int>(span64 > kGroup ? span64 : kGroup);
  wg_select_init<IX_WG>(sel);
  for (;;) {
    if (tid == 0) {
      const uint32_t i = atomicAdd(w.fb + 1, 1u);
      next_row = i < w.fb[0] ? static_cast<int32_t>(w.fb[2 + i]) : -1;
      ocnt = 0u;
    }
    __syncthreads();
    const int b = next_row;
    if (b < 0) break;
    const int n = row_len(a, b);
    // every token's key at its position
    for (int t0 = 0; t0 < n; t0 += span) {
      const int t1 = min(n, t0 + span);
      score_chunk_any<false, NT, IX_WG, IX_RING>(a, b, t0, t1, pages, [&](int j, float v, bool ok) {
        if (ok) area[j] = rank_key(float_key(v), static_cast<uint32_t>(j));
      });
      __syncthreads();  // the staged pages are replaced by the next span's
    }
    uint64_t T = 0ull;
    if (static_cast<uint32_t>(n) > k) {
      uint64_t mn = ~0ull, mx = 0ull;
      for (int i = tid; i < n; i += IX_WG) {
        const uint64_t x = area[i];
        mn = x < mn ? x : mn;
        mx = x > mx ? x : mx;
      }
      wg_range<IX_WG>(mn, mx, sel);
      T = wg_select<IX_WG>(
          [&](auto&& f) {
            for (int i = tid; i < n; i += IX_WG) f(area[i]);
          },
          k, mn, mx, sel);
    }
    const SlotOf slot_of{a, bt_row_of(a, b), o.keep_positions != 0, n};
    for (int i0 = 0; i0 < n; i0 += IX_WG * PF_FB_BATCH) {
      uint64_t key[PF_FB_BATCH];
      bool keep[PF_FB_BATCH];
#pragma unroll
      for (int e = 0; e < PF_FB_BATCH; ++e) {
        const int i = i0 + e * IX_WG + tid;
        key[e] = i < n ? area[i] : 0ull;
        keep[e] = i < n && key[e] >= T;
      }
      emit_batch<PF_FB_BATCH>(key, keep, b, o, &ocnt, slot_of);
    }
    if (static_cast<uint32_t>(n) < k) pad_row<IX_WG>(o, b, static_cast<uint32_t>(max(n, 0)));
    __syncthreads();  // next_row, ocnt and the area are reused
  }
}

// ---------------------------------------------------------------------------
// Launcher
// ---------------------------------------------------------------------------

// SIMDs of the current device (four per compute unit), cached per device.
static int64_t prefill_simds() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cache[dev] = 4 * cus;
  }
  return cache[dev];
}

int launch_prefill_fused(const IndexerInputs& in, int k, int32_t* out_slots, float* out_scores, void* ws,
                         bool sorted, hipStream_t stream) {
  if (in.batch == 0) return 0;
  if (in.bf16 || in.page_size % kGroup != 0 || (in.heads != 16 && in.heads != 32 && in.heads != 64)) return -2;
  const PrefillWs w = prefill_ws(ws, in.batch, k, in.max_seq_len);
  FusedOut o;
  o.slots = out_slots;
  o.scores = sorted && !out_scores ? w.sval : out_scores;
  o.k = k;
  o.keep_positions = sorted;

  // Chunks of up to PR_CHUNK_PAGES pages (8192 tokens at most), halved
  // while the grid would hold fewer than PF_MIN_WAVES waves and a chunk
  // keeps at least 1024 tokens (few rows, e.g. multi-token decode).
  int64_t chunk = static_cast<int64_t>(PR_CHUNK_PAGES) * in.page_size;
  if (chunk > 8192) chunk = 8192 / in.page_size * in.page_size;
  const int64_t quads = (in.batch + 3) / 4;
  const int64_t msl = in.max_seq_len > 0 ? in.max_seq_len : 1;
  while (chunk / 2 >= 1024 && (chunk / 2) % in.page_size == 0 && quads * ((msl + chunk - 1) / chunk) < PF_MIN_WAVES)
    chunk /= 2;
  const IndexerArgs a = make_args(in, static_cast<int>(chunk), false);
  PrefillParams pp;
  pp.k = k;
  pp.chunk = static_cast<int>(chunk);
  const int gfull = static_cast<int>(chunk / kGroup);
  pp.stride = (gfull + PF_SAMPLE - 1) / PF_SAMPLE;
  pp.sdiv1 = make_fastdiv(static_cast<uint32_t>(pp.stride > 1 ? pp.stride - 1 : 1));  // S - 1 (1 when S = 1)
  // Few quads: the balanced schedule (quad waves); otherwise pair waves.
  pp.balanced = quads <= PF_BAL_QUADS;
  const int64_t units = pp.balanced ? quads : (in.batch + 1) / 2;
  pp.ntiles = static_cast<int>((units + PR_WG / kWave - 1) / (PR_WG / kWave));
  const int nkc = static_cast<int>((static_cast<int64_t>(in.max_seq_len > 0 ? in.max_seq_len : 1) + chunk - 1) / chunk);
  // The balanced schedule runs over a grid of at least one wave per SIMD,
  // and at least nq chunks of PF_SAMPLE groups per quad's bound.
  int64_t nwg = static_cast<int64_t>(pp.ntiles) * nkc;
  if (pp.balanced) {
    const int64_t full = quads * ((msl + PF_SAMPLE * kGroup - 1) / (PF_SAMPLE * kGroup));
    int64_t waves = prefill_simds();
    if (waves < full) waves = full;
    if (waves < 2 * quads) waves = 2 * quads;
    nwg = (waves + PR_WG / kWave - 1) / (PR_WG / kWave);
  }

  (void)hipGetLastError();
  hipLaunchKernelGGL(prefill_zero_kernel, dim3((in.batch + 255) / 256), dim3(256), 0, stream, w, in.batch);
  const dim3 grid(static_cast<unsigned>(nwg));
#define IDXTOPK_PF_CHUNK(BAL, RM)                                                                          \
  switch (in.heads) {                                                                                      \
    case 16: hipLaunchKernelGGL((prefill_chunk_kernel<1, BAL, RM>), grid, dim3(PR_WG), 0, stream, a, w, pp); break; \
    case 32: hipLaunchKernelGGL((prefill_chunk_kernel<2, BAL, RM>), grid, dim3(PR_WG), 0, stream, a, w, pp); break; \
    default: hipLaunchKernelGGL((prefill_chunk_kernel<4, BAL, RM>), grid, dim3(PR_WG), 0, stream, a, w, pp); break; \
  }
  if (pp.balanced) {
    IDXTOPK_PF_CHUNK(true, 4)
  } else {
    IDXTOPK_PF_CHUNK(false, 2)
  }
#undef IDXTOPK_PF_CHUNK
  const int64_t per = (w.cap + PF_MERGE_WG - 1) / PF_MERGE_WG;
  const dim3 rows(static_cast<unsigned>(in.batch));
  if (per <= 2) hipLaunchKernelGGL(prefill_merge_kernel<2>, rows, dim3(PF_MERGE_WG), 0, stream, a, w, o);
  else if (per <= 4) hipLaunchKernelGGL(prefill_merge_kernel<4>, rows, dim3(PF_MERGE_WG), 0, stream, a, w, o);
  else if (per <= 8) hipLaunchKernelGGL(prefill_merge_kernel<8>, rows, dim3(PF_MERGE_WG), 0, stream, a, w, o);
  else if (per <= 16) hipLaunchKernelGGL(prefill_merge_kernel<16>, rows, dim3(PF_MERGE_WG), 0, stream, a, w, o);
  else hipLaunchKernelGGL(prefill_merge_kernel<32>, rows, dim3(PF_MERGE_WG), 0, stream, a, w, o);
  const dim3 fb(PF_FB_WGS);
  switch (in.heads) {
    case 16: hipLaunchKernelGGL(prefill_fallback_kernel<1>, fb, dim3(IX_WG), 0, stream, a, w, o); break;
    case 32: hipLaunchKernelGGL(prefill_fallback_kernel<2>, fb, dim3(IX_WG), 0, stream, a, w, o); break;
    default: hipLaunchKernelGGL(prefill_fallback_kernel<4>, fb, dim3(IX_WG), 0, stream, a, w, o); break;
  }
  if (hipGetLastError() != hipSuccess) return -4;
  if (!sorted) return 0;
  return launch_sort_rows(in.batch, k, out_slots, o.scores, nullptr, 0, nullptr, nullptr, in.block_table,
                          in.bt_stride, in.page_size, in.row_to_batch, out_scores, stream);
}

}  // namespace idxtopk
