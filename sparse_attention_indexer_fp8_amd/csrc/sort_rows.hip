// Sorted output: each row's selected entries in descending score order,
// equal scores by ascending row-local position, then the page transform
// ([SGL-37889] Modifications: the selected index stays row-local until the
// transform maps it through the page table). The selection kernels leave
// positions; this pass orders and maps them.
#include "common.hpp"
#include "launch.hpp"
#include "sort.hpp"

namespace idxtopk {

struct SortArgs {
  int32_t* pos;                // [rows][k] positions in (-1 = padding), slots or positions out
  const float* vals;           // [rows][k] score of each entry, or null: read from the score buffer
  const float* scores;         // score buffer: entry p of row i is scores[i * stride + rs_i + p]
  int64_t stride;
  const int32_t* row_starts;   // rs_i, or null (0)
  const int32_t* seq_lens;     // only with `scores`: positions are below seq_lens[i]
  const int32_t* page_table;   // null: positions are written back as they are
  int64_t pt_stride;
  int32_t page_size;
  FastDiv pdiv;
  const int32_t* row_to_batch;  // page-table row of each row, or null (row i -> i)
  float* out_vals;             // sorted scores out (may alias vals; -inf pads), or null
  int32_t k;
  int32_t npow;                // power of two >= k, at least 256
};

constexpr int SR_MIN_NPOW = 256;

// One workgroup of npow / E threads per row. The row's k entries become
// 64-bit keys (score key high, complemented position low: a larger key is a
// better entry, padding is key 0, below every real entry), block_sort_desc
// orders them, and each sorted entry is written back mapped to its slot.
template <int WG, int E>
__global__ __launch_bounds__(WG) void sort_rows_kernel(SortArgs a) {
  __shared__ uint64_t xs[WG * E];
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int64_t row = static_cast<int64_t>(i) * a.k;
  const float* srow = nullptr;
  int n = 0;
  if (a.scores) {
    srow = a.scores + static_cast<int64_t>(i) * a.stride + (a.row_starts ? a.row_starts[i] : 0);
    n = a.seq_lens[i];
  }
  // The initial placement is free: entry e * WG + tid goes to r[e]
  // (coalesced). Every load of a step is issued before any is used, at
  // clamped addresses, so no load waits behind another's branch.
  int32_t p[E];
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * WG + tid;
    p[e] = a.pos[row + (j < a.k ? j : a.k - 1)];
  }
  if (a.vals) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = e * WG + tid;
      v[e] = a.vals[row + (j < a.k ? j : a.k - 1)];
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = e * WG + tid < a.k && p[e] >= 0 && p[e] < n;
      v[e] = *(ok ? srow + p[e] : a.scores);
    }
  }
  uint64_t r[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * WG + tid;
    const bool real = j < a.k && p[e] >= 0 && (a.vals || p[e] < n);
    r[e] = real ? rank_key(float_key(v[e]), static_cast<uint32_t>(p[e])) : 0ull;
  }
  block_sort_desc<WG, E>(r, xs);
  const int base = tid * E;  // rank of r[0]
  const int32_t* pt_row = nullptr;
  if (a.page_table) {
    const int prow = a.row_to_batch ? a.row_to_batch[i] : i;
    pt_row = a.page_table + static_cast<int64_t>(prow) * a.pt_stride;
  }
  // positions -> slots: all page lookups issued first (padding looks up
  // page 0 of the row, which exists when the row has any entry)
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  uint32_t pos[E], pg[E];
  int32_t page[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    pos[e] = r[e] ? rank_pos(r[e]) : 0u;
    pg[e] = fdiv(pos[e], a.pdiv);
  }
  if (pt_row && r[0]) {
#pragma unroll
    for (int e = 0; e < E; ++e) page[e] = pt_row[pg[e]];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int t = base + e;
    if (t < a.k) {
      int32_t o = -1;
      if (r[e]) o = pt_row ? static_cast<int32_t>(static_cast<uint32_t>(page[e]) * P + (pos[e] - pg[e] * P))
                           : static_cast<int32_t>(pos[e]);
      a.pos[row + t] = o;
      if (a.out_vals) a.out_vals[row + t] = r[e] ? key_float(rank_vkey(r[e])) : -__builtin_inff();
    }
  }
}

int launch_sort_rows(int rows, int k, int32_t* pos, const float* vals, const float* scores, int64_t stride,
                     const int32_t* row_starts, const int32_t* seq_lens, const int32_t* page_table,
                     int64_t pt_stride, int page_size, const int32_t* row_to_batch, float* out_vals,
                     hipStream_t stream) {
  if (rows == 0) return 0;
  SortArgs a;
  a.pos = pos;
  a.vals = vals;
  a.scores = scores;
  a.stride = stride;
  a.row_starts = row_starts;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.page_size = page_size > 0 ? page_size : 1;
  a.pdiv = make_fastdiv(static_cast<uint32_t>(a.page_size));
  a.row_to_batch = row_to_batch;
  a.out_vals = out_vals;
  a.k = k;
  int npow = SR_MIN_NPOW;
  while (npow < k) npow <<= 1;
  a.npow = npow;
  (void)hipGetLastError();
  // four keys per thread (eight at the largest size, for 1024 threads)
  switch (npow) {
    case 256: hipLaunchKernelGGL((sort_rows_kernel<64, 4>), dim3(rows), dim3(64), 0, stream, a); break;
    case 512: hipLaunchKernelGGL((sort_rows_kernel<128, 4>), dim3(rows), dim3(128), 0, stream, a); break;
    case 1024: hipLaunchKernelGGL((sort_rows_kernel<256, 4>), dim3(rows), dim3(256), 0, stream, a); break;
    case 2048: hipLaunchKernelGGL((sort_rows_kernel<512, 4>), dim3(rows), dim3(512), 0, stream, a); break;
    case 4096: hipLaunchKernelGGL((sort_rows_kernel<1024, 4>), dim3(rows), dim3(1024), 0, stream, a); break;
    case 8192: hipLaunchKernelGGL((sort_rows_kernel<1024, 8>), dim3(rows), dim3(1024), 0, stream, a); break;
    default: return -4;  // k above 8192 is refused before this
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace idxtopk
