// Host-side launchers behind the C ABI (api.hip validates, these enqueue).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace idxtopk {

// Lets `kernel` take `bytes` of dynamic LDS (above the 64 KB default; gfx950
// has 160 KB per CU). `granted` caches the largest size already granted for
// this kernel, so the runtime is asked only when a call needs more. The
// runtime's recorded error state is cleared either way.
inline hipError_t allow_dynamic_lds(const void* kernel, size_t bytes, std::atomic<size_t>& granted) {
  if (bytes <= granted.load(std::memory_order_relaxed)) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  (void)hipGetLastError();
  if (e == hipSuccess) granted.store(bytes, std::memory_order_relaxed);
  return e;
}

// Error words of the checked build, one per source file with checks
// (read, and cleared if asked; 0 in a release build, which has none).
uint32_t check_word_topk_rows(bool clear);
uint32_t check_word_indexer(bool clear);
uint32_t check_word_prefill(bool clear);

// All return 0 or -4 (launch failure); arguments are already validated.
int launch_topk_rows(const float* scores, int64_t stride, int rows, const int32_t* seq_lens,
                     const int32_t* row_starts, const int32_t* row_to_batch, const int32_t* kv_offset,
                     const int32_t* page_table, int64_t pt_stride, int page_size, int k,
                     int32_t* out, bool sorted, hipStream_t stream);

// Sorted output pass: orders each row's k entries (score descending, equal
// scores by ascending position; -1 entries last) and maps them to slots.
// Scores come from `vals` ([rows][k]) or, when it is null, from the score
// buffer `scores` at the entry's position.
int launch_sort_rows(int rows, int k, int32_t* pos, const float* vals, const float* scores, int64_t stride,
                     const int32_t* row_starts, const int32_t* seq_lens, const int32_t* page_table,
                     int64_t pt_stride, int page_size, const int32_t* row_to_batch, float* out_vals,
                     hipStream_t stream);

int launch_page_transform(const int32_t* idx, int rows, int k, const int32_t* page_table,
                          int64_t pt_stride, int page_size, const int32_t* row_to_batch,
                          int32_t* out, hipStream_t stream);

struct IndexerInputs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  const uint8_t* kcache;
  const float* k_scale;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t page_size;
  const int32_t* row_to_batch;  // block-table row of each query row, or null (row b -> b)
  const int32_t* seq_lens;
  int32_t batch;
  int32_t heads;
  int32_t max_seq_len;
  bool bf16 = false;  // bf16 index cache: q and kcache hold bf16, no scales
};

int launch_idx_score(const IndexerInputs& in, float* scores, int64_t score_stride, hipStream_t stream);

size_t fused_workspace_bytes(int rows, int k, int max_seq_len);
int launch_fused(const IndexerInputs& in, int k, int32_t* out_slots, float* out_scores, void* ws,
                 bool sorted, hipStream_t stream);

size_t prefill_workspace_bytes(int rows, int k, int max_seq_len);
int launch_prefill_fused(const IndexerInputs& in, int k, int32_t* out_slots, float* out_scores, void* ws,
                         bool sorted, hipStream_t stream);

size_t block_workspace_bytes(int rows, int block_size, int max_seq_len);

int launch_cache_write(const void* keys, bool bf16, int64_t stride, int tokens, const int32_t* slots,
                       uint8_t* kcache, float* kscale, hipStream_t stream);
int launch_cache_write_bf16(const void* keys, bool bf16_in, int64_t stride, int tokens, const int32_t* slots,
                            uint16_t* kcache, hipStream_t stream);
int launch_block_topk(const IndexerInputs& in, int block_size, int top_blocks, int32_t* out_blocks,
                      int32_t* out_slots, void* ws, hipStream_t stream);
int launch_block_topk_heads(const IndexerInputs& in, int block_size, int top_blocks, int32_t* out_blocks,
                            int32_t* out_slots, void* ws, hipStream_t stream);

}  // namespace idxtopk
