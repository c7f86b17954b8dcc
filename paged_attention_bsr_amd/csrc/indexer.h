// Launch interface of the sparse-attention indexer (scores + exact Top-K).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace bsa {

// Top-K: chunks of kIdxChunk positions per workgroup; a threshold from a sample
// of at most kIdxSample scores per row; at most kIdxCandCap candidates (keys at
// or above the threshold) per chunk and per row.
constexpr int kIdxChunk = 16384;
constexpr int kIdxSample = 2048;
constexpr int kIdxCandCap = 12288;
constexpr int kIdxMaxChunks = 1024;  // max_ctx <= 8388480 (65535 score workgroups of 128 keys) spans at most 512 chunks

// Workspace: per (row, chunk) a candidate count, then per (row, chunk) a region of
// kIdxCandCap (key, position) pairs.  Nothing in it needs initialising.
inline size_t indexer_workspace_bytes(int64_t num_rows, int64_t max_ctx) {
  if (num_rows <= 0 || max_ctx <= 0) return 0;
  const size_t chunks = static_cast<size_t>(num_rows) * static_cast<size_t>((max_ctx + kIdxChunk - 1) / kIdxChunk);
  return (chunks * 4 + 255) / 256 * 256 + chunks * kIdxCandCap * 8;
}

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
  int32_t* ws_count;           // [num_rows][nch_max] candidates per chunk
  uint2* ws_cand;              // [num_rows][nch_max][kIdxCandCap] (key, position)
  int64_t num_slots, max_ctx, ld_scores, q_stride, k_stride;  // ld_scores: max_ctx rounded up to 64
  int32_t num_rows, num_reqs, max_pages, page_size, head_dim, topk;
  int32_t page_shift;          // log2(page_size) when it is a power of two, else -1
  int32_t nch_max;             // chunks of the longest row: ceil(max_ctx / kIdxChunk)
};

// The scores kernel (unless there are no rows), then, unless scores_only, the
// two Top-K kernels.  head_dim in {64, 128, 256}.
hipError_t launch_indexer(const IndexerArgs& a, bool bf16, bool scores_only, hipStream_t stream);

}  // namespace bsa
