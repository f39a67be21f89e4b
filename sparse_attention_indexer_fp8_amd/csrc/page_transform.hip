// topk_page_transform: row-local positions -> physical KV-cache slots.
//
// [SGL-37889] "[AMD] Enable GLM DSA prefill top-k to the v2 kernel", sections
// Motivation and Modifications: the selected index stays row-local and the
// transform maps it through the page-table row (row_to_batch[i], or i).
// Elementwise; -1 padding passes through. One thread per output entry, a
// 256-thread workgroup covers 256 consecutive entries (coalesced in and out).
#include "common.hpp"
#include "launch.hpp"

namespace idxtopk {

constexpr int PT_WG = 256;

__global__ __launch_bounds__(PT_WG) void page_transform_kernel(
    const int32_t* idx, int64_t total, int k, const int32_t* page_table, int64_t pt_stride,
    uint32_t P, FastDiv pdiv, const int32_t* row_to_batch, int32_t* out) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * PT_WG + threadIdx.x;
  if (e >= total) return;
  const int row = static_cast<int>(e / k);
  const int32_t p = idx[e];
  int32_t r = -1;
  if (p >= 0) {
    const int prow = row_to_batch ? row_to_batch[row] : row;
    const uint32_t pg = fdiv(static_cast<uint32_t>(p), pdiv);
    const uint32_t off = static_cast<uint32_t>(p) - pg * P;
    r = static_cast<int32_t>(static_cast<int64_t>(page_table[static_cast<int64_t>(prow) * pt_stride + pg]) * P + off);
  }
  out[e] = r;
}

int launch_page_transform(const int32_t* idx, int rows, int k, const int32_t* page_table,
                          int64_t pt_stride, int page_size, const int32_t* row_to_batch,
                          int32_t* out, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(rows) * k;
  if (total == 0) return 0;
  const int64_t blocks = (total + PT_WG - 1) / PT_WG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(page_transform_kernel, dim3(static_cast<unsigned>(blocks)), dim3(PT_WG), 0,
                     stream, idx, total, k, page_table, pt_stride, static_cast<uint32_t>(page_size),
                     make_fastdiv(static_cast<uint32_t>(page_size)), row_to_batch, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace idxtopk
