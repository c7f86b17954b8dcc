// Launch interface of the sparse-attention indexer (scores + exact Top-K).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace bsa {

// Top-K work split: chunks of kIdxChunk score positions per workgroup, a
// histogram of the keys' top kIdxHistBits bits per row, at most kIdxCandCap
// keys of the K-th key's bin collected per row (more take the slow path).
constexpr int kIdxChunk = 16384;
constexpr int kIdxHistBits = 12;
constexpr int kIdxHistBins = 1 << kIdxHistBits;
constexpr int kIdxCandCap = 4096;
constexpr int kIdxMaxChunks = 1024;  // max_ctx <= 16776960 (65535 score workgroups of 256 keys) spans at most 1024 chunks
constexpr int kIdxStateWords = 16;

// words of a row's state in the workspace
enum : int {
  kStArrive0 = 0,  // histogram workgroups finished (back to 0 when the row's step is done)
  kStArrive1,      // collection workgroups finished (likewise)
  kStBin,          // histogram bin of the K-th largest key
  kStNeed,         // keys to take from that bin
  kStInBin,        // keys in that bin
  kStNcand,        // candidates appended (back to 0 after the selection)
  kStT,            // the K-th largest key
  kStPLast,        // last kept position among keys equal to it (0x7fffffff: all)
  kStFallback,     // 1: the bin overflows the candidate buffer
};

// The workspace holds one block of kIdxRowBytes per row, at row * kIdxRowBytes
// whatever the call's sizes, so the words that must start at zero (the two
// arrival counters, the candidate count and the histogram, all reset by the
// call that used them) sit at the same place in every call:
//   state  kIdxStateWords uint32 words
//   hist   kIdxHistBins uint32 counts
//   cand   kIdxCandCap (key, position) pairs
//   chunk  kIdxMaxChunks int32: keys above the bin per chunk, then the chunk's output offset
constexpr size_t kIdxRowState = 0;
constexpr size_t kIdxRowHist = 256;
constexpr size_t kIdxRowCand = kIdxRowHist + kIdxHistBins * 4;
constexpr size_t kIdxRowChunk = kIdxRowCand + kIdxCandCap * 8;
constexpr size_t kIdxRowBytes = kIdxRowChunk + kIdxMaxChunks * 4;
static_assert(kIdxRowBytes % 256 == 0, "row blocks stay 256-byte aligned");

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
  char* ws;                    // [num_rows][kIdxRowBytes]
  int64_t num_slots, max_ctx, ld_scores, q_stride, k_stride;  // ld_scores: max_ctx rounded up to 64
  int32_t num_rows, num_reqs, max_pages, page_size, head_dim, topk;
  int32_t page_shift;          // log2(page_size) when it is a power of two, else -1
  int32_t nch_max;             // chunks of the longest row: ceil(max_ctx / kIdxChunk)
};

// The scores kernel (unless there are no rows), then, unless scores_only, the
// three Top-K kernels.  head_dim in {64, 128, 256}.
hipError_t launch_indexer(const IndexerArgs& a, bool bf16, bool scores_only, hipStream_t stream);

}  // namespace bsa
