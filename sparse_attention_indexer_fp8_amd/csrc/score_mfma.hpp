// fp8 indexer scoring on gfx950 matrix cores.
//
// For one query row b and 16 consecutive key tokens at a time, one wave
// computes logits[h, j] = q[b, h, :] . key[slot_j, :] with
// v_mfma_f32_16x16x128_f8f6f4. The 16 tokens are the N columns, 16 heads are
// the M rows, and K = 128 = the whole head dimension in one instruction. It
// then reduces the heads in registers:
//   S[j] = k_scale[slot_j] * sum_h (w[b, h] * q_scale[b]) * max(0, logits[h, j]).
// (The scales are > 0, so folding them outside the ReLU is exact algebra.)
//
// Operand layout (both operands, lane l, c = l & 15, g = l >> 4):
//   A (query):  row c of the 16-head tile, bytes [32g, 32g + 32) of the head vector
//   B (keys):   column c = token tok0 + c, bytes [32g, 32g + 32) of its key
// A and B use the same K grouping, so the product sums the full 128-term dot
// whatever order the hardware assigns to the K index inside a group.
// The key operand is not loaded in this layout (16 scattered half-lines per
// instruction stream at ~80% of the rate of whole lines): keys_to_operand
// builds it from whole-line loads.
// Result: lane l holds D[4g + r][c], r = 0..3, i.e. heads 4g + r of the tile
// for token c.
#pragma once

#include "common.hpp"

namespace idxtopk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kDim = 128;
constexpr int kGroup = 16;  // tokens per MFMA column block

struct IndexerArgs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  const uint8_t* kcache;
  const float* k_scale;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t page_size;
  FastDiv pdiv;
  const int32_t* row_to_batch;  // block-table row of each query row, or null (row b -> b)
  const int32_t* seq_lens;
  int32_t batch;
  int32_t heads;
  int32_t max_seq_len;  // the caller's bound on every seq_lens[b]
  int32_t chunk;       // tokens per full-size chunk
  int32_t nchunk_max;  // chunks per row in the grid
  // Guided chunk schedule: chunks [0, n_full) have `chunk` tokens, the next
  // n_half have chunk / 2 from token tok_half, the rest chunk / 4 from token
  // tok_quarter (n_half = 0 and tok_half = tok_quarter = n_full * chunk when
  // every chunk is full size).
  int32_t n_full;
  int32_t n_half;
  int32_t tok_half;
  int32_t tok_quarter;
  // Nonzero: consecutive query rows may share block-table rows, and the grid
  // deals (row, chunk) pairs to workgroups in quads of rows (batch % 4 == 0,
  // grid rounded up to a multiple of 32).
  int32_t quad_map;
  // Nonzero: a bf16 cache is read with ordinary (cached) loads in the fused
  // chunk kernel, else with nontemporal ones.
  int32_t cached_keys;
};

struct KeyPieces {
  v4i x0, x1;
};

// Block-table row of query row b (several query rows may share one).
__device__ __forceinline__ const int32_t* bt_row_of(const IndexerArgs& a, int b) {
  const int prow = a.row_to_batch ? load_uniform(a.row_to_batch + b) : b;
  IDXTOPK_CHECK(prow >= 0, kChkRowToBatch);
  return a.block_table + static_cast<int64_t>(prow) * a.bt_stride;
}

// seq_lens[b], the number of visible keys of row b (checked builds check it
// against the caller's bound).
__device__ __forceinline__ int row_len(const IndexerArgs& a, int b) {
  const int n = a.seq_lens[b];
  IDXTOPK_CHECK(n >= 0 && n <= a.max_seq_len, kChkSeqLen);
  return n;
}

template <int NT>
struct QOperand {
  v8i a[NT];
  float wt[NT][4];
};

__device__ __forceinline__ v8i load_v8i(const uint8_t* p) {
  const uint4* p4 = reinterpret_cast<const uint4*>(p);
  const uint4 x = p4[0];
  const uint4 y = p4[1];
  v8i r;
  r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
  r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
  return r;
}

// Key bytes are read once per call: load them without keeping them in cache.
__device__ __forceinline__ v4i load_v4i_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

// Keys are fetched in whole lines: for a group of 16 tokens, lane l loads the
// 16-byte piece (l & 7) of token (l >> 3) (x0) and of token 8 + (l >> 3) (x1),
// so each load instruction covers eight complete 128-byte keys. The B operand
// wants lane (c, g) to hold pieces 2g and 2g + 1 of token c; two steps of
// ds_bpermute move them. In step 0 a lane with c < 8 pulls piece 2g from x0
// of lane 8c + 2g, and a lane with c >= 8 pulls piece 2g + 1 from x1 of lane
// 8(c - 8) + 2g + 1; step 1 pulls the other piece from the other parity.
// Even lanes offer x0 in step 0 and x1 in step 1, odd lanes the reverse, so
// every piece is sent once. Lanes with c >= 8 receive their pieces in swapped
// order and put them back.
__device__ __forceinline__ v8i keys_to_operand(const v4i x0, const v4i x1) {
  const int l = lane_id();
  const int c = l & 15, g = l >> 4, hi = c >> 3;
  const int a0 = 4 * (8 * (c & 7) + 2 * g + hi);
  const int a1 = 4 * (8 * (c & 7) + 2 * g + 1 - hi);
  const bool even = (l & 1) == 0;
  const v4i r0 = even ? x0 : x1, r1 = even ? x1 : x0;
  v4i t0, t1;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    t0[d] = __builtin_amdgcn_ds_bpermute(a0, r0[d]);
    t1[d] = __builtin_amdgcn_ds_bpermute(a1, r1[d]);
  }
  const v4i lo = hi ? t1 : t0, up = hi ? t0 : t1;
  v8i kb;
  kb[0] = lo[0]; kb[1] = lo[1]; kb[2] = lo[2]; kb[3] = lo[3];
  kb[4] = up[0]; kb[5] = up[1]; kb[6] = up[2]; kb[7] = up[3];
  return kb;
}

template <int NT>
__device__ __forceinline__ void load_query(QOperand<NT>& qo, const uint8_t* q_row,
                                           const float* w_row, float s_q) {
  const int l = lane_id();
  const int c = l & 15, g = l >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    qo.a[t] = load_v8i(q_row + (16 * t + c) * kDim + 32 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) qo.wt[t][r] = w_row[16 * t + 4 * g + r] * s_q;
  }
}

// max(x, 0) for a float that is not NaN, as one integer max on its bits:
// positive floats are positive integers, negative ones (and -0) negative.
__device__ __forceinline__ float relu_bits(float x) {
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

// Score of token (tok0 + (lane & 15)), returned in every lane of the wave.
template <int NT>
__device__ __forceinline__ float score16(const QOperand<NT>& qo, const v8i kb, float ks) {
  // all tiles' products first, so no result is waited on while another
  // product could still be issued
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[t], kb, zero, 0, 0, 0, 0, 0, 0);
  }
  float part = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) part = fmaf(qo.wt[t][r], relu_bits(acc[t][r]), part);
  }
  // sum the four 16-lane groups (heads 4g..4g+3 of every tile)
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part),
                                                    false, false);
  part = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                    false, false);
  part = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  return part * ks;
}

// Scores of token (tok0 + (lane & 15)) for two query rows against one key
// operand: lanes 0-15 and 32-47 return row A's, lanes 16-31 and 48-63 row
// B's. The permlane16 swap of A's partial sums against B's leaves A's and
// B's pairwise sums in alternate 16-lane rows, so one permlane32 swap
// finishes both; each row is summed in the same order as score16, so the
// results are bit-identical to it.
template <int NT>
__device__ __forceinline__ float score16x2(const QOperand<NT>& qa, const QOperand<NT>& qb, const v8i kb,
                                           float ks) {
  v4f acc[2][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    acc[0][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa.a[t], kb, zero, 0, 0, 0, 0, 0, 0);
    acc[1][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qb.a[t], kb, zero, 0, 0, 0, 0, 0, 0);
  }
  float pa = 0.0f, pb = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pa = fmaf(qa.wt[t][r], relu_bits(acc[0][t][r]), pa);
      pb = fmaf(qb.wt[t][r], relu_bits(acc[1][t][r]), pb);
    }
  }
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
  float part = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                    false, false);
  part = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  return part * ks;
}

// Scores of token (tok0 + (lane & 15)) for four query rows against one key
// operand: lane group g (lanes 16g..16g+15) returns row g's. Two permlane16
// swaps (rows 0 with 1, rows 2 with 3) and one permlane32 swap put every
// row's four 16-lane partial sums together, in score16's order, so the
// results are bit-identical to it.
template <int NT>
__device__ __forceinline__ float score16x4(const QOperand<NT> (&q)[4], const v8i kb, float ks) {
  // Products i = 4 t + r (row r, head tile t). A wave issues one instruction
  // at a time, so the vector work of product i - 2 (ReLU and weighted sum,
  // 8 instructions) is placed after product i: it runs while the matrix
  // core works on products i - 1 and i, whose results it does not need,
  // and only about three products' results are live at once. Each row's sum
  // still runs over t, then the tile's four heads, as in score16.
  constexpr int N = 4 * NT;
  v4f acc[N];
  float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto fold = [&](int i) __attribute__((always_inline)) {
    const int t = i / 4, r = i % 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) p[r] = fmaf(q[r].wt[t][j], relu_bits(acc[i][j]), p[r]);
  };
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q[i % 4].a[i / 4], kb, zero, 0, 0, 0, 0, 0, 0);
    if (i >= 2) fold(i - 2);
  }
  fold(N - 2);
  fold(N - 1);
  // the order above, for the scheduler: product, then 8 vector instructions
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
  }
  const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
  const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[2]), __float_as_uint(p[3]), false, false);
  const float x = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
  const float y = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return (__uint_as_float(s32[0]) + __uint_as_float(s32[1])) * ks;
}

// Max number of page ids a chunk stages in LDS.
constexpr int kMaxChunkPages = 1024;

// Score the tokens [tok_begin, tok_end) of row b with a WG-thread workgroup.
// The chunk's block-table entries are staged in LDS once (`lds_pages`).
// Waves take contiguous ranges of 16-token groups. Each wave keeps a ring of
// RING groups of key loads in flight: a slot is consumed in place and refilled
// with the group RING ahead right after, so no register copy ever forces the
// wave to wait for loads it has only just issued.
// emit(j, score, valid) is called by every lane of the wave for each 16-token
// group: lane l carries token j = group start + (l & 15) and its score, and
// valid is true for exactly one lane per token in the chunk ((l >> 4) == 0
// and j < tok_end).
template <int NT, int WG, int RING, bool WHOLE, class Emit>
__device__ __forceinline__ void score_chunk_impl(const IndexerArgs& a, int b, int tok_begin, int tok_end,
                                                 int32_t* lds_pages, Emit&& emit) {
  constexpr int NW = WG / kWave;
  const int tid = threadIdx.x;
  const int wave = uniform(tid / kWave);
  const int l = lane_id();
  const int c = l & 15, g = l >> 4;
  const uint32_t P = static_cast<uint32_t>(a.page_size);

  const uint32_t p0 = fdiv(static_cast<uint32_t>(tok_begin), a.pdiv);
  const uint32_t p1 = fdiv(static_cast<uint32_t>(tok_end - 1), a.pdiv);
  const int32_t* bt_row = bt_row_of(a, b);
  for (int i = tid; i <= static_cast<int>(p1 - p0); i += WG) {
    lds_pages[i] = bt_row[p0 + i];
    IDXTOPK_CHECK(lds_pages[i] >= 0, kChkPageId);
  }

  QOperand<NT> qo;
  load_query<NT>(qo, a.q + static_cast<int64_t>(b) * a.heads * kDim,
                 a.w + static_cast<int64_t>(b) * a.heads, a.q_scale[b]);
  __syncthreads();

  const int ngroups = (tok_end - tok_begin + kGroup - 1) / kGroup;
  const int per = (ngroups + NW - 1) / NW;
  const int g_lo = wave * per;
  const int g_hi = min(ngroups, g_lo + per);
  const int last = tok_end - 1;

  // token j (clamped into the chunk) -> its cache slot. Slot ids fit in 32
  // bits (they are returned as int32), so only byte offsets are widened.
  // slot = page * P + (j - pg * P) = (page - pg) * P + j. The empty asm keeps
  // the multiply and the add apart: fused, they become a 64-bit mad whose
  // unused high addend half may alias a register with a key load still in
  // flight, and the wait for that load would stall the ring.
  auto slot_of = [&](int j) {
    j = j < last ? j : last;
    const uint32_t pg = fdiv(static_cast<uint32_t>(j), a.pdiv);
    uint32_t m = (static_cast<uint32_t>(lds_pages[pg - p0]) - pg) * P;
    asm volatile("" : "+v"(m));
    return m + static_cast<uint32_t>(j);
  };
  auto key_piece = [&](uint32_t slot, int lp) {
    return load_v4i_stream(a.kcache + (static_cast<uint64_t>(slot) << 7) + lp);
  };
  // group gi of this chunk -> this lane's two whole-line key pieces and the
  // scale of token c. When pages hold whole groups and the chunk starts on a
  // group boundary, a group never straddles a page: one lookup gives the
  // group's first slot, and tokens past the chunk's end read bytes of that
  // same page (never used), so nothing is clamped.
  const int lt = l >> 3, lp = 16 * (l & 7);
  auto fetch = [&](int gi, KeyPieces& kp, float& ks) {
    const int j0 = tok_begin + gi * kGroup;
    if (WHOLE) {
      const uint32_t pg = fdiv(static_cast<uint32_t>(j0), a.pdiv);
      uint32_t m = (static_cast<uint32_t>(uniform(lds_pages[pg - p0])) - pg) * P;
      asm volatile("" : "+s"(m));
      const uint32_t s0 = m + static_cast<uint32_t>(j0);
      kp.x0 = key_piece(s0 + lt, lp);
      kp.x1 = key_piece(s0 + 8 + lt, lp);
      ks = a.k_scale[s0 + c];
    } else {
      kp.x0 = key_piece(slot_of(j0 + lt), lp);
      kp.x1 = key_piece(slot_of(j0 + 8 + lt), lp);
      ks = a.k_scale[slot_of(j0 + c)];
    }
  };

  if (g_lo >= g_hi) return;
  const int gmax = g_hi - 1;
  auto consume = [&](int gi, float s) {
    const int j = tok_begin + gi * kGroup + c;
    emit(j, s, g == 0 && j < tok_end);
  };

  typedef float vks __attribute__((ext_vector_type(RING)));
  KeyPieces ring[RING];
  vks ksr;
#pragma unroll
  for (int u = 0; u < RING; ++u) {
    float t;
    fetch(min(g_lo + u, gmax), ring[u], t);
    ksr[u] = t;
  }

  // steady state: every refill is in range, so control flow is uniform and
  // each group only waits for its own loads
  int gi0 = g_lo;
  for (; gi0 + 2 * RING <= g_hi; gi0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      float s = score16<NT>(qo, keys_to_operand(ring[u].x0, ring[u].x1), ksr[u]);
      // slot u is fully consumed before its refill is issued, so the refill can
      // reuse the slot's registers (no copies, no early waits). The empty asm
      // makes the score final here, so the scale multiply cannot sink past the
      // refill and keep the old scale alive beside the new one.
      asm volatile("" : "+v"(s));
      __builtin_amdgcn_sched_barrier(0);
      float t;
      fetch(gi0 + u + RING, ring[u], t);
      ksr[u] = t;
      consume(gi0 + u, s);
    }
  }
  // drain: fewer than 2 * RING groups remain; the ring holds gi0 .. gi0 + RING - 1
#pragma unroll
  for (int u = 0; u < RING; ++u) {
    const int gi = gi0 + u;
    if (gi < g_hi) {
      const float s = score16<NT>(qo, keys_to_operand(ring[u].x0, ring[u].x1), ksr[u]);
      if (gi + RING < g_hi) {
        float t;
        fetch(gi + RING, ring[u], t);
        ksr[u] = t;
      }
      consume(gi, s);
    }
  }
#pragma unroll
  for (int u = 0; u < RING; ++u) {
    const int gi = gi0 + RING + u;
    if (gi < g_hi) consume(gi, score16<NT>(qo, keys_to_operand(ring[u].x0, ring[u].x1), ksr[u]));
  }
}

// Score the tokens [tok_begin, tok_end) of row b with a WG-thread workgroup
// (see score_chunk_impl). Chunks whose pages hold whole 16-token groups, and
// that start on a group boundary, take the one-lookup-per-group fetch.
template <int NT, int WG, int RING, class Emit>
__device__ void score_chunk(const IndexerArgs& a, int b, int tok_begin, int tok_end, int32_t* lds_pages,
                            Emit&& emit) {
  if (a.page_size % kGroup == 0 && tok_begin % kGroup == 0)
    score_chunk_impl<NT, WG, RING, true>(a, b, tok_begin, tok_end, lds_pages, emit);
  else
    score_chunk_impl<NT, WG, RING, false>(a, b, tok_begin, tok_end, lds_pages, emit);
}

// ---------------------------------------------------------------------------
// bf16 index cache: bf16 queries [B][H][128] and keys [slot][128] (256 bytes
// per token), no scales. v_mfma_f32_16x16x32_bf16 contracts 32 dimensions:
// lane (c, g) of the B operand holds 8 dimensions of token c, and the four
// instructions of a 16-token group take dimensions [32s, 32s + 32), lane
// group g the eight at 32s + 8g. One load instruction per s then covers 64
// contiguous bytes of each of the group's 16 tokens. The accumulator layout
// is the fp8 instruction's (lane (c, g) holds heads 4g .. 4g + 3 of token
// c), so the weighted-ReLU head sum is score16's.
// ---------------------------------------------------------------------------

template <int NT>
struct QOperandBF {
  v4i a[NT][4];
  float wt[NT][4];
};

struct KeyPiecesBF {
  v4i x[4];
};

template <int NT>
__device__ __forceinline__ void load_query_bf16(QOperandBF<NT>& qo, const uint8_t* q_row, const float* w_row) {
  const int l = lane_id();
  const int c = l & 15, g = l >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
      qo.a[t][sl] = *reinterpret_cast<const v4i*>(q_row + ((16 * t + c) * kDim + 32 * sl + 8 * g) * 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) qo.wt[t][r] = w_row[16 * t + 4 * g + r];
  }
}

// Score of token (tok0 + (lane & 15)) from a bf16 key group, in every lane.
template <int NT>
__device__ __forceinline__ float score16_bf16(const QOperandBF<NT>& qo, const KeyPiecesBF& kp) {
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qo.a[t][sl]),
                                                       __builtin_bit_cast(v8bf, kp.x[sl]), acc[t], 0, 0, 0);
  }
  float part = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) part = fmaf(qo.wt[t][r], relu_bits(acc[t][r]), part);
  }
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part),
                                                    false, false);
  part = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                    false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// score_chunk_impl for a bf16 cache: the same chunk staging, wave split,
// ring discipline and emit contract; a group's keys are four 16-byte loads
// per lane (token c, dimensions 32s + 8g .. + 8) and need no rearranging.
// One load instruction covers half of each token's two 128-byte lines, so
// each line is fetched by two instructions. CACHED: ordinary loads, which
// keep the line for its second half (faster for long rows); otherwise
// nontemporal loads, which leave the caches to the data that follows (the
// score-buffer variant's score rows).
template <int NT, int WG, int RING, bool WHOLE, bool CACHED, class Emit>
__device__ __forceinline__ void score_chunk_bf16_impl(const IndexerArgs& a, int b, int tok_begin, int tok_end,
                                                      int32_t* lds_pages, Emit&& emit) {
  constexpr int NW = WG / kWave;
  const int tid = threadIdx.x;
  const int wave = uniform(tid / kWave);
  const int l = lane_id();
  const int c = l & 15, g = l >> 4;
  const uint32_t P = static_cast<uint32_t>(a.page_size);

  const uint32_t p0 = fdiv(static_cast<uint32_t>(tok_begin), a.pdiv);
  const uint32_t p1 = fdiv(static_cast<uint32_t>(tok_end - 1), a.pdiv);
  const int32_t* bt_row = bt_row_of(a, b);
  for (int i = tid; i <= static_cast<int>(p1 - p0); i += WG) {
    lds_pages[i] = bt_row[p0 + i];
    IDXTOPK_CHECK(lds_pages[i] >= 0, kChkPageId);
  }

  QOperandBF<NT> qo;
  load_query_bf16<NT>(qo, a.q + static_cast<int64_t>(b) * a.heads * kDim * 2, a.w + static_cast<int64_t>(b) * a.heads);
  __syncthreads();

  const int ngroups = (tok_end - tok_begin + kGroup - 1) / kGroup;
  const int per = (ngroups + NW - 1) / NW;
  const int g_lo = wave * per;
  const int g_hi = min(ngroups, g_lo + per);
  const int last = tok_end - 1;

  // token j (clamped into the chunk) -> its cache slot (multiply and add kept
  // apart, as in score_chunk_impl)
  auto slot_of = [&](int j) {
    j = j < last ? j : last;
    const uint32_t pg = fdiv(static_cast<uint32_t>(j), a.pdiv);
    uint32_t m = (static_cast<uint32_t>(lds_pages[pg - p0]) - pg) * P;
    asm volatile("" : "+v"(m));
    return m + static_cast<uint32_t>(j);
  };
  const int lp = 16 * g;
  auto fetch = [&](int gi, KeyPiecesBF& kp) {
    const int j0 = tok_begin + gi * kGroup;
    uint32_t slot;
    if (WHOLE) {
      const uint32_t pg = fdiv(static_cast<uint32_t>(j0), a.pdiv);
      uint32_t m = (static_cast<uint32_t>(uniform(lds_pages[pg - p0])) - pg) * P;
      asm volatile("" : "+s"(m));
      slot = m + static_cast<uint32_t>(j0) + c;
    } else {
      slot = slot_of(j0 + c);
    }
    const uint8_t* row = a.kcache + (static_cast<uint64_t>(slot) << 8) + lp;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
      kp.x[sl] = CACHED ? *reinterpret_cast<const v4i*>(row + 64 * sl) : load_v4i_stream(row + 64 * sl);
  };

  if (g_lo >= g_hi) return;
  const int gmax = g_hi - 1;
  auto consume = [&](int gi, float s) {
    const int j = tok_begin + gi * kGroup + c;
    emit(j, s, g == 0 && j < tok_end);
  };

  KeyPiecesBF ring[RING];
#pragma unroll
  for (int u = 0; u < RING; ++u) fetch(min(g_lo + u, gmax), ring[u]);

  int gi0 = g_lo;
  for (; gi0 + 2 * RING <= g_hi; gi0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      float s = score16_bf16<NT>(qo, ring[u]);
      asm volatile("" : "+v"(s));
      __builtin_amdgcn_sched_barrier(0);
      fetch(gi0 + u + RING, ring[u]);
      consume(gi0 + u, s);
    }
  }
#pragma unroll
  for (int u = 0; u < RING; ++u) {
    const int gi = gi0 + u;
    if (gi < g_hi) {
      const float s = score16_bf16<NT>(qo, ring[u]);
      if (gi + RING < g_hi) fetch(gi + RING, ring[u]);
      consume(gi, s);
    }
  }
#pragma unroll
  for (int u = 0; u < RING; ++u) {
    const int gi = gi0 + RING + u;
    if (gi < g_hi) consume(gi, score16_bf16<NT>(qo, ring[u]));
  }
}

// Score a chunk from a bf16 cache. A bf16 group is twice an fp8 group's
// bytes, so half the ring depth keeps the same bytes in flight.
template <int NT, int WG, int RING, bool CACHED, class Emit>
__device__ void score_chunk_bf16(const IndexerArgs& a, int b, int tok_begin, int tok_end, int32_t* lds_pages,
                                 Emit&& emit) {
  constexpr int R = RING > 2 ? RING / 2 : RING;
  if (a.page_size % kGroup == 0 && tok_begin % kGroup == 0)
    score_chunk_bf16_impl<NT, WG, R, true, CACHED>(a, b, tok_begin, tok_end, lds_pages, emit);
  else
    score_chunk_bf16_impl<NT, WG, R, false, CACHED>(a, b, tok_begin, tok_end, lds_pages, emit);
}

// ---------------------------------------------------------------------------
// Per-head terms (fp8 cache): the block variant that selects per index head
// needs every head's term of the score, not their sum.
// ---------------------------------------------------------------------------

// Lane (c, g) gets, for tile t and r = 0..3, the term of head 16t + 4g + r
// for token c of the group: w * s_q (folded into wt) * relu(logit) * s_k.
template <int NT>
__device__ __forceinline__ void heads16(const QOperand<NT>& qo, const v8i kb, float ks, float (&v)[NT][4]) {
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[t], kb, zero, 0, 0, 0, 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[t][r] = qo.wt[t][r] * relu_bits(acc[t][r]) * ks;
  }
}

// The chunk loop of score_chunk_impl (staged pages, waves on contiguous
// group ranges, a ring of RING groups refilled right after use) with the
// per-head terms: emit_heads(j0, v) is called by every lane for each group,
// j0 the group's first token; lane (c, g) holds token j0 + c's terms of
// heads 16t + 4g + r. Tokens at or past tok_end carry terms of unrelated
// keys and must be ignored.
template <int NT, int WG, int RING, bool WHOLE, class Emit>
__device__ __forceinline__ void score_chunk_heads_impl(const IndexerArgs& a, int b, int tok_begin, int tok_end,
                                                       int32_t* lds_pages, Emit&& emit_heads) {
  constexpr int NW = WG / kWave;
  const int tid = threadIdx.x;
  const int wave = uniform(tid / kWave);
  const int l = lane_id();
  const int c = l & 15;
  const uint32_t P = static_cast<uint32_t>(a.page_size);

  const uint32_t p0 = fdiv(static_cast<uint32_t>(tok_begin), a.pdiv);
  const uint32_t p1 = fdiv(static_cast<uint32_t>(tok_end - 1), a.pdiv);
  const int32_t* bt_row = bt_row_of(a, b);
  for (int i = tid; i <= static_cast<int>(p1 - p0); i += WG) {
    lds_pages[i] = bt_row[p0 + i];
    IDXTOPK_CHECK(lds_pages[i] >= 0, kChkPageId);
  }

  QOperand<NT> qo;
  load_query<NT>(qo, a.q + static_cast<int64_t>(b) * a.heads * kDim,
                 a.w + static_cast<int64_t>(b) * a.heads, a.q_scale[b]);
  __syncthreads();

  const int ngroups = (tok_end - tok_begin + kGroup - 1) / kGroup;
  const int per = (ngroups + NW - 1) / NW;
  const int g_lo = wave * per;
  const int g_hi = min(ngroups, g_lo + per);
  const int last = tok_end - 1;
  auto slot_of = [&](int j) {
    j = j < last ? j : last;
    const uint32_t pg = fdiv(static_cast<uint32_t>(j), a.pdiv);
    uint32_t m = (static_cast<uint32_t>(lds_pages[pg - p0]) - pg) * P;
    asm volatile("" : "+v"(m));
    return m + static_cast<uint32_t>(j);
  };
  auto key_piece = [&](uint32_t slot, int lp) {
    return load_v4i_stream(a.kcache + (static_cast<uint64_t>(slot) << 7) + lp);
  };
  const int lt = l >> 3, lp = 16 * (l & 7);
  auto fetch = [&](int gi, KeyPieces& kp, float& ks) {
    const int j0 = tok_begin + gi * kGroup;
    if (WHOLE) {
      const uint32_t pg = fdiv(static_cast<uint32_t>(j0), a.pdiv);
      uint32_t m = (static_cast<uint32_t>(uniform(lds_pages[pg - p0])) - pg) * P;
      asm volatile("" : "+s"(m));
      const uint32_t s0 = m + static_cast<uint32_t>(j0);
      kp.x0 = key_piece(s0 + lt, lp);
      kp.x1 = key_piece(s0 + 8 + lt, lp);
      ks = a.k_scale[s0 + c];
    } else {
      kp.x0 = key_piece(slot_of(j0 + lt), lp);
      kp.x1 = key_piece(slot_of(j0 + 8 + lt), lp);
      ks = a.k_scale[slot_of(j0 + c)];
    }
  };
  if (g_lo >= g_hi) return;
  const int gmax = g_hi - 1;
  KeyPieces ring[RING];
  float ksr[RING];
#pragma unroll
  for (int u = 0; u < RING; ++u) fetch(min(g_lo + u, gmax), ring[u], ksr[u]);
  for (int gi0 = g_lo; gi0 < g_hi; gi0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      const int gi = gi0 + u;
      if (gi < g_hi) {
        float v[NT][4];
        heads16<NT>(qo, keys_to_operand(ring[u].x0, ring[u].x1), ksr[u], v);
        if (gi + RING < g_hi) fetch(gi + RING, ring[u], ksr[u]);
        emit_heads(tok_begin + gi * kGroup, v);
      }
    }
  }
}

template <int NT, int WG, int RING, class Emit>
__device__ void score_chunk_heads(const IndexerArgs& a, int b, int tok_begin, int tok_end, int32_t* lds_pages,
                                  Emit&& emit_heads) {
  if (a.page_size % kGroup == 0 && tok_begin % kGroup == 0)
    score_chunk_heads_impl<NT, WG, RING, true>(a, b, tok_begin, tok_end, lds_pages, emit_heads);
  else
    score_chunk_heads_impl<NT, WG, RING, false>(a, b, tok_begin, tok_end, lds_pages, emit_heads);
}

// Either cache format (CACHED: see score_chunk_bf16_impl; fp8 keys are
// always read nontemporally).
template <bool BF, int NT, int WG, int RING, bool CACHED = false, class Emit>
__device__ __forceinline__ void score_chunk_any(const IndexerArgs& a, int b, int tok_begin, int tok_end,
                                                int32_t* lds_pages, Emit&& emit) {
  if constexpr (BF)
    score_chunk_bf16<NT, WG, RING, CACHED>(a, b, tok_begin, tok_end, lds_pages, emit);
  else
    score_chunk<NT, WG, RING>(a, b, tok_begin, tok_end, lds_pages, emit);
}

}  // namespace idxtopk
