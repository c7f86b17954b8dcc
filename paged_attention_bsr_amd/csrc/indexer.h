// Launch interface of the sparse-attention indexer (scores + exact Top-K).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace bsa {

// Top-K: a threshold from a sample of at most kIdxSample scores per row; at
// most kIdxCandCap candidates (keys at or above the threshold) per row in LDS.
constexpr int kIdxSample = 4096;
constexpr int kIdxCandCap = 8192;

// Pointers are device addresses; strides in elements.
struct IndexerArgs {
  const void* q;               // [num_rows][head_dim] fp16 / bf16
  const void* key_cache;       // [num_slots][head_dim], same type
  const int32_t* block_table;  // [num_reqs][max_pages]
  const int32_t* req_row_ptr;  // [num_reqs + 1]
  const int32_t* ctx_len;      // [num_rows]
  const int32_t* req_kv_len;   // [num_reqs]
  float* scores;               // [num_rows][ld_scores]
  int32_t* out;                // [num_rows][topk]
  int64_t num_slots, max_ctx, ld_scores, q_stride, k_stride;  // ld_scores: max_ctx rounded up to 64
  int32_t num_rows, num_reqs, max_pages, page_size, head_dim, topk;
  int32_t page_shift;          // log2(page_size) when it is a power of two, else -1
};

// The scores kernel (unless there are no rows), then, unless scores_only, the
// Top-K kernel.  head_dim in {64, 128, 256}.
hipError_t launch_indexer(const IndexerArgs& a, bool bf16, bool scores_only, hipStream_t stream);

}  // namespace bsa
