// C ABI of libidxtopk: argument validation, then the launchers.
// Declarations and the meaning of every argument: include/idxtopk.h.
#include "../../include/idxtopk.h"
#include "launch.hpp"

#include <mutex>

namespace {

// ---------------------------------------------------------------------------
// Built-in workspace of idx_score_topk_fused_noalloc
// ---------------------------------------------------------------------------
//
// One array per GPU the library runs on, held until the process ends. Host
// code never passes `scratch` itself to a kernel (on the host that name is
// only a stand-in, not a device address): the first call on a device
// resolves the device's own address with hipGetSymbolAddress, and every
// later use goes through that pointer. The fused path needs no particular
// workspace contents, so the array is never cleared.
constexpr size_t kScratchBytes = IDXTOPK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // the device address of `scratch` on each device

// The current device's scratch address (resolved once per device), or null.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

using idxtopk::IndexerInputs;

bool heads_ok(int32_t h) { return h == 16 || h == 32 || h == 64 || h == 128; }

// Shared checks of the paged indexer inputs (no device access). A bf16 cache
// has no scales, and its query and key rows are read 16 bytes at a time.
int check_indexer(const void* q, const float* q_scale, const float* w, const void* kcache,
                  const float* k_scale, const int32_t* block_table, int64_t bt_stride,
                  int32_t page_size, const int32_t* seq_lens, int32_t batch, int32_t heads,
                  int32_t dim, int32_t max_seq_len, bool bf16 = false) {
  if (batch < 0 || heads <= 0 || dim <= 0 || page_size <= 0 || bt_stride < 0 || max_seq_len < 0)
    return IDXTOPK_EINVAL;
  if (batch > 0 && (!q || !w || !kcache || !block_table || !seq_lens)) return IDXTOPK_EINVAL;
  if (batch > 0 && !bf16 && (!q_scale || !k_scale)) return IDXTOPK_EINVAL;
  if (batch > 0 && bf16 &&
      (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(kcache) % 16 != 0))
    return IDXTOPK_EINVAL;
  if (dim != IDXTOPK_DIM || !heads_ok(heads)) return IDXTOPK_EUNSUPPORTED;
  // every visible token's logical page must exist in the block-table row
  if (static_cast<int64_t>(max_seq_len) > bt_stride * static_cast<int64_t>(page_size))
    return IDXTOPK_EINVAL;
  return IDXTOPK_OK;
}

IndexerInputs pack(const void* q, const float* q_scale, const float* w, const void* kcache,
                   const float* k_scale, const int32_t* block_table, int64_t bt_stride,
                   int32_t page_size, const int32_t* row_to_batch, const int32_t* seq_lens,
                   int32_t batch, int32_t heads, int32_t max_seq_len, bool bf16 = false) {
  IndexerInputs in;
  in.bf16 = bf16;
  in.q = static_cast<const uint8_t*>(q);
  in.q_scale = q_scale;
  in.w = w;
  in.kcache = static_cast<const uint8_t*>(kcache);
  in.k_scale = k_scale;
  in.block_table = block_table;
  in.bt_stride = bt_stride;
  in.page_size = page_size;
  in.row_to_batch = row_to_batch;
  in.seq_lens = seq_lens;
  in.batch = batch;
  in.heads = heads;
  in.max_seq_len = max_seq_len;
  return in;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int idx_score_fp8(const uint8_t* q, const float* q_scale, const float* w, const uint8_t* kcache,
                  const float* k_scale, const int32_t* block_table, int64_t bt_stride,
                  int32_t page_size, const int32_t* row_to_batch, const int32_t* seq_lens,
                  int32_t batch, int32_t heads,
                  int32_t dim, int32_t max_seq_len, float* scores, int64_t score_stride,
                  void* stream) {
  const int st = check_indexer(q, q_scale, w, kcache, k_scale, block_table, bt_stride, page_size,
                               seq_lens, batch, heads, dim, max_seq_len);
  if (st != IDXTOPK_OK) return st;
  if (score_stride < 0 || (batch > 0 && !scores)) return IDXTOPK_EINVAL;
  if (static_cast<int64_t>(max_seq_len) > score_stride) return IDXTOPK_EINVAL;
  if (batch == 0 || max_seq_len == 0) return IDXTOPK_OK;
  return idxtopk::launch_idx_score(
      pack(q, q_scale, w, kcache, k_scale, block_table, bt_stride, page_size, row_to_batch, seq_lens,
           batch, heads, max_seq_len),
      scores, score_stride, static_cast<hipStream_t>(stream));
}

int topk_rows(const float* scores, int64_t score_stride, int32_t rows, const int32_t* seq_lens,
              const int32_t* row_starts, const int32_t* row_to_batch, const int32_t* kv_offset,
              const int32_t* page_table,
              int64_t pt_stride, int32_t page_size, int32_t k, int32_t* out, int32_t flags, void* stream) {
  if (rows < 0 || k <= 0 || score_stride < 0 || (flags & ~IDXTOPK_SORTED)) return IDXTOPK_EINVAL;
  if (rows > 0 && (!scores || !seq_lens || !out)) return IDXTOPK_EINVAL;
  if (page_table && (pt_stride < 0 || page_size <= 0)) return IDXTOPK_EINVAL;
  if (k > IDXTOPK_MAX_K_ROWS) return IDXTOPK_EUNSUPPORTED;
  if (rows == 0) return IDXTOPK_OK;
  return idxtopk::launch_topk_rows(scores, score_stride, rows, seq_lens, row_starts, row_to_batch, kv_offset,
                                   page_table, pt_stride, page_table ? page_size : 1, k, out,
                                   (flags & IDXTOPK_SORTED) != 0, static_cast<hipStream_t>(stream));
}

int topk_page_transform(const int32_t* idx, int32_t rows, int32_t k, const int32_t* page_table,
                        int64_t pt_stride, int32_t page_size, const int32_t* row_to_batch,
                        int32_t* out, void* stream) {
  if (rows < 0 || k <= 0 || pt_stride < 0 || page_size <= 0) return IDXTOPK_EINVAL;
  if (rows > 0 && (!idx || !page_table || !out)) return IDXTOPK_EINVAL;
  if (rows == 0) return IDXTOPK_OK;
  return idxtopk::launch_page_transform(idx, rows, k, page_table, pt_stride, page_size,
                                        row_to_batch, out, static_cast<hipStream_t>(stream));
}

int idx_score_topk_fused(const uint8_t* q, const float* q_scale, const float* w,
                         const uint8_t* kcache, const float* k_scale, const int32_t* block_table,
                         int64_t bt_stride, int32_t page_size, const int32_t* row_to_batch,
                         const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t dim, int32_t max_seq_len, int32_t k,
                         int32_t* out_slots, float* out_scores, void* workspace,
                         size_t workspace_bytes, int32_t flags, void* stream) {
  if (flags & ~IDXTOPK_SORTED) return IDXTOPK_EINVAL;
  const int st = check_indexer(q, q_scale, w, kcache, k_scale, block_table, bt_stride, page_size,
                               seq_lens, batch, heads, dim, max_seq_len);
  if (st != IDXTOPK_OK) return st;
  if (k <= 0 || (batch > 0 && !out_slots)) return IDXTOPK_EINVAL;
  if (k > IDXTOPK_MAX_K_FUSED) return IDXTOPK_EUNSUPPORTED;
  if (batch == 0) return IDXTOPK_OK;
  if (!workspace || workspace_bytes < idxtopk::fused_workspace_bytes(batch, k, max_seq_len))
    return IDXTOPK_EWORKSPACE;
  return idxtopk::launch_fused(pack(q, q_scale, w, kcache, k_scale, block_table, bt_stride,
                                    page_size, row_to_batch, seq_lens, batch, heads, max_seq_len),
                               k, out_slots, out_scores, workspace, (flags & IDXTOPK_SORTED) != 0,
                               static_cast<hipStream_t>(stream));
}

int idx_score_topk_fused_noalloc(const uint8_t* q, const float* q_scale, const float* w,
                                 const uint8_t* kcache, const float* k_scale, const int32_t* block_table,
                                 int64_t bt_stride, int32_t page_size, const int32_t* row_to_batch,
                                 const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t dim,
                                 int32_t max_seq_len, int32_t k, int32_t* out_slots, float* out_scores,
                                 int32_t flags, void* stream) {
  if (flags & ~IDXTOPK_SORTED) return IDXTOPK_EINVAL;
  const int st = check_indexer(q, q_scale, w, kcache, k_scale, block_table, bt_stride, page_size,
                               seq_lens, batch, heads, dim, max_seq_len);
  if (st != IDXTOPK_OK) return st;
  if (k <= 0 || (batch > 0 && !out_slots)) return IDXTOPK_EINVAL;
  if (k > IDXTOPK_MAX_K_FUSED) return IDXTOPK_EUNSUPPORTED;
  if (batch == 0) return IDXTOPK_OK;
  const size_t need = idxtopk::fused_workspace_bytes(batch, k, max_seq_len);
  if (need > kScratchBytes) return IDXTOPK_EWORKSPACE;
  void* ws = scratch_ptr();
  if (ws == nullptr) return IDXTOPK_ELAUNCH;
  return idxtopk::launch_fused(pack(q, q_scale, w, kcache, k_scale, block_table, bt_stride, page_size,
                                    row_to_batch, seq_lens, batch, heads, max_seq_len),
                               k, out_slots, out_scores, ws, (flags & IDXTOPK_SORTED) != 0,
                               static_cast<hipStream_t>(stream));
}

int idx_score_topk_prefill(const uint8_t* q, const float* q_scale, const float* w,
                           const uint8_t* kcache, const float* k_scale, const int32_t* block_table,
                           int64_t bt_stride, int32_t page_size, const int32_t* row_to_batch,
                           const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t dim,
                           int32_t max_seq_len, int32_t k, int32_t* out_slots, float* out_scores,
                           void* workspace, size_t workspace_bytes, int32_t flags, void* stream) {
  if (flags & ~IDXTOPK_SORTED) return IDXTOPK_EINVAL;
  const int st = check_indexer(q, q_scale, w, kcache, k_scale, block_table, bt_stride, page_size,
                               seq_lens, batch, heads, dim, max_seq_len);
  if (st != IDXTOPK_OK) return st;
  if (k <= 0 || (batch > 0 && !out_slots)) return IDXTOPK_EINVAL;
  if (k > IDXTOPK_MAX_K_PREFILL || page_size % 16 != 0 || (heads != 16 && heads != 32 && heads != 64))
    return IDXTOPK_EUNSUPPORTED;
  if (batch == 0) return IDXTOPK_OK;
  if (!workspace || workspace_bytes < idxtopk::prefill_workspace_bytes(batch, k, max_seq_len))
    return IDXTOPK_EWORKSPACE;
  return idxtopk::launch_prefill_fused(pack(q, q_scale, w, kcache, k_scale, block_table, bt_stride,
                                            page_size, row_to_batch, seq_lens, batch, heads, max_seq_len),
                                       k, out_slots, out_scores, workspace, (flags & IDXTOPK_SORTED) != 0,
                                       static_cast<hipStream_t>(stream));
}

int block_topk(const uint8_t* q, const float* q_scale, const float* w, const uint8_t* kcache,
               const float* k_scale, const int32_t* block_table, int64_t bt_stride,
               int32_t page_size, const int32_t* row_to_batch, const int32_t* seq_lens,
               int32_t batch, int32_t heads,
               int32_t dim, int32_t max_seq_len, int32_t block_size, int32_t top_blocks,
               int32_t* out_blocks, int32_t* out_slots, void* workspace, size_t workspace_bytes,
               void* stream) {
  const int st = check_indexer(q, q_scale, w, kcache, k_scale, block_table, bt_stride, page_size,
                               seq_lens, batch, heads, dim, max_seq_len);
  if (st != IDXTOPK_OK) return st;
  if (block_size <= 0 || top_blocks <= 0 || (batch > 0 && !out_blocks)) return IDXTOPK_EINVAL;
  if (block_size != page_size || top_blocks > IDXTOPK_MAX_TOP_BLOCKS || block_size % 16 != 0 ||
      block_size > 8192)
    return IDXTOPK_EUNSUPPORTED;
  if (batch == 0) return IDXTOPK_OK;
  if (!workspace ||
      workspace_bytes < idxtopk::block_workspace_bytes(batch, block_size, max_seq_len))
    return IDXTOPK_EWORKSPACE;
  return idxtopk::launch_block_topk(pack(q, q_scale, w, kcache, k_scale, block_table, bt_stride,
                                         page_size, row_to_batch, seq_lens, batch, heads,
                                         max_seq_len),
                                    block_size, top_blocks, out_blocks, out_slots, workspace,
                                    static_cast<hipStream_t>(stream));
}

int idx_cache_write(const void* keys, int32_t key_dtype, int64_t key_stride, int32_t tokens,
                    int32_t dim, const int32_t* slot_mapping, uint8_t* kcache, float* k_scale,
                    void* stream) {
  if (tokens < 0 || dim <= 0) return IDXTOPK_EINVAL;
  if (dim != IDXTOPK_DIM) return IDXTOPK_EUNSUPPORTED;
  if (key_dtype != IDXTOPK_KEY_F32 && key_dtype != IDXTOPK_KEY_BF16) return IDXTOPK_EUNSUPPORTED;
  if (tokens == 0) return IDXTOPK_OK;
  if (!keys || !slot_mapping || !kcache || !k_scale || key_stride < dim) return IDXTOPK_EINVAL;
  // every row must start on a whole pair of elements (8 bytes fp32, 4 bf16)
  const uintptr_t align = key_dtype == IDXTOPK_KEY_F32 ? 8u : 4u;
  if (reinterpret_cast<uintptr_t>(keys) % align != 0 || key_stride % 2 != 0) return IDXTOPK_EINVAL;
  return idxtopk::launch_cache_write(keys, key_dtype == IDXTOPK_KEY_BF16, key_stride, tokens, slot_mapping,
                                     kcache, k_scale, static_cast<hipStream_t>(stream));
}

int block_topk_heads(const uint8_t* q, const float* q_scale, const float* w, const uint8_t* kcache,
                     const float* k_scale, const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                     const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch, int32_t heads,
                     int32_t dim, int32_t max_seq_len, int32_t block_size, int32_t top_blocks,
                     int32_t* out_blocks, int32_t* out_slots, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const int st = check_indexer(q, q_scale, w, kcache, k_scale, block_table, bt_stride, page_size,
                               seq_lens, batch, heads, dim, max_seq_len);
  if (st != IDXTOPK_OK) return st;
  if (block_size <= 0 || top_blocks <= 0 || (batch > 0 && !out_blocks)) return IDXTOPK_EINVAL;
  if (block_size != page_size || top_blocks > IDXTOPK_MAX_TOP_BLOCKS || block_size % 16 != 0 ||
      block_size > 8192)
    return IDXTOPK_EUNSUPPORTED;
  if (batch == 0) return IDXTOPK_OK;
  if (!workspace ||
      workspace_bytes < idxtopk::block_workspace_bytes(batch * heads, block_size, max_seq_len))
    return IDXTOPK_EWORKSPACE;
  return idxtopk::launch_block_topk_heads(pack(q, q_scale, w, kcache, k_scale, block_table, bt_stride,
                                               page_size, row_to_batch, seq_lens, batch, heads, max_seq_len),
                                          block_size, top_blocks, out_blocks, out_slots, workspace,
                                          static_cast<hipStream_t>(stream));
}

int idx_score_bf16(const uint16_t* q, const float* w, const uint16_t* kcache, const int32_t* block_table,
                   int64_t bt_stride, int32_t page_size, const int32_t* row_to_batch, const int32_t* seq_lens,
                   int32_t batch, int32_t heads, int32_t dim, int32_t max_seq_len, float* scores,
                   int64_t score_stride, void* stream) {
  const int st = check_indexer(q, nullptr, w, kcache, nullptr, block_table, bt_stride, page_size, seq_lens, batch,
                               heads, dim, max_seq_len, true);
  if (st != IDXTOPK_OK) return st;
  if (score_stride < 0 || (batch > 0 && !scores)) return IDXTOPK_EINVAL;
  if (static_cast<int64_t>(max_seq_len) > score_stride) return IDXTOPK_EINVAL;
  if (batch == 0 || max_seq_len == 0) return IDXTOPK_OK;
  return idxtopk::launch_idx_score(pack(q, nullptr, w, kcache, nullptr, block_table, bt_stride, page_size,
                                        row_to_batch, seq_lens, batch, heads, max_seq_len, true),
                                   scores, score_stride, static_cast<hipStream_t>(stream));
}

int idx_score_topk_fused_bf16(const uint16_t* q, const float* w, const uint16_t* kcache,
                              const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                              const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch, int32_t heads,
                              int32_t dim, int32_t max_seq_len, int32_t k, int32_t* out_slots, float* out_scores,
                              void* workspace, size_t workspace_bytes, int32_t flags, void* stream) {
  if (flags & ~IDXTOPK_SORTED) return IDXTOPK_EINVAL;
  const int st = check_indexer(q, nullptr, w, kcache, nullptr, block_table, bt_stride, page_size, seq_lens, batch,
                               heads, dim, max_seq_len, true);
  if (st != IDXTOPK_OK) return st;
  if (k <= 0 || (batch > 0 && !out_slots)) return IDXTOPK_EINVAL;
  if (k > IDXTOPK_MAX_K_FUSED) return IDXTOPK_EUNSUPPORTED;
  if (batch == 0) return IDXTOPK_OK;
  if (!workspace || workspace_bytes < idxtopk::fused_workspace_bytes(batch, k, max_seq_len))
    return IDXTOPK_EWORKSPACE;
  return idxtopk::launch_fused(pack(q, nullptr, w, kcache, nullptr, block_table, bt_stride, page_size, row_to_batch,
                                    seq_lens, batch, heads, max_seq_len, true),
                               k, out_slots, out_scores, workspace, (flags & IDXTOPK_SORTED) != 0,
                               static_cast<hipStream_t>(stream));
}

int block_topk_bf16(const uint16_t* q, const float* w, const uint16_t* kcache, const int32_t* block_table,
                    int64_t bt_stride, int32_t page_size, const int32_t* row_to_batch, const int32_t* seq_lens,
                    int32_t batch, int32_t heads, int32_t dim, int32_t max_seq_len, int32_t block_size,
                    int32_t top_blocks, int32_t* out_blocks, int32_t* out_slots, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const int st = check_indexer(q, nullptr, w, kcache, nullptr, block_table, bt_stride, page_size, seq_lens, batch,
                               heads, dim, max_seq_len, true);
  if (st != IDXTOPK_OK) return st;
  if (block_size <= 0 || top_blocks <= 0 || (batch > 0 && !out_blocks)) return IDXTOPK_EINVAL;
  if (block_size != page_size || top_blocks > IDXTOPK_MAX_TOP_BLOCKS || block_size % 16 != 0 ||
      block_size > 8192)
    return IDXTOPK_EUNSUPPORTED;
  if (batch == 0) return IDXTOPK_OK;
  if (!workspace ||
      workspace_bytes < idxtopk::block_workspace_bytes(batch, block_size, max_seq_len))
    return IDXTOPK_EWORKSPACE;
  return idxtopk::launch_block_topk(pack(q, nullptr, w, kcache, nullptr, block_table, bt_stride, page_size,
                                         row_to_batch, seq_lens, batch, heads, max_seq_len, true),
                                    block_size, top_blocks, out_blocks, out_slots, workspace,
                                    static_cast<hipStream_t>(stream));
}

int idx_cache_write_bf16(const void* keys, int32_t key_dtype, int64_t key_stride, int32_t tokens, int32_t dim,
                         const int32_t* slot_mapping, uint16_t* kcache, void* stream) {
  if (tokens < 0 || dim <= 0) return IDXTOPK_EINVAL;
  if (dim != IDXTOPK_DIM) return IDXTOPK_EUNSUPPORTED;
  if (key_dtype != IDXTOPK_KEY_F32 && key_dtype != IDXTOPK_KEY_BF16) return IDXTOPK_EUNSUPPORTED;
  if (tokens == 0) return IDXTOPK_OK;
  if (!keys || !slot_mapping || !kcache || key_stride < dim) return IDXTOPK_EINVAL;
  // every row starts on 16 bytes of the input and of the cache
  const int64_t esize = key_dtype == IDXTOPK_KEY_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(keys) % 16 != 0 || (key_stride * esize) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(kcache) % 16 != 0)
    return IDXTOPK_EINVAL;
  return idxtopk::launch_cache_write_bf16(keys, key_dtype == IDXTOPK_KEY_BF16, key_stride, tokens, slot_mapping,
                                          kcache, static_cast<hipStream_t>(stream));
}

size_t idxtopk_workspace_bytes(int32_t op, int32_t rows, int32_t k, int32_t max_seq_len) {
  if (rows < 0 || max_seq_len < 0) return 0;
  switch (op) {
    case IDXTOPK_OP_SCORE_TOPK_FUSED:
      return rows > 0 ? idxtopk::fused_workspace_bytes(rows, k, max_seq_len) : 0;
    case IDXTOPK_OP_SCORE_TOPK_PREFILL:
      if (k <= 0) return 0;
      return rows > 0 ? idxtopk::prefill_workspace_bytes(rows, k, max_seq_len) : 0;
    case IDXTOPK_OP_BLOCK_TOPK:
    case IDXTOPK_OP_BLOCK_TOPK_HEADS:  // rows = batch * heads
      if (k <= 0) return 0;
      return rows > 0 ? idxtopk::block_workspace_bytes(rows, k, max_seq_len) : 0;
    default:
      return 0;
  }
}

const char* idxtopk_status_str(int32_t status) {
  switch (status) {
    case IDXTOPK_OK: return "ok";
    case IDXTOPK_EINVAL: return "invalid argument";
    case IDXTOPK_EUNSUPPORTED: return "unsupported shape or size";
    case IDXTOPK_EWORKSPACE: return "workspace missing or too small";
    case IDXTOPK_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int32_t idxtopk_version(void) { return IDXTOPK_VERSION; }

uint32_t idxtopk_check_status(int32_t clear) {
#if IDXTOPK_CHECKS
  // synchronous: waits for the device's queued work, then reads the words
  (void)hipDeviceSynchronize();
  return idxtopk::check_word_topk_rows(clear != 0) | idxtopk::check_word_indexer(clear != 0) |
         idxtopk::check_word_prefill(clear != 0);
#else
  (void)clear;
  return IDXTOPK_CHECKS_OFF;
#endif
}

}  // extern "C"
#pragma GCC visibility pop
