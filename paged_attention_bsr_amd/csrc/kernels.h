// Launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsa {

// Arguments of the attention kernels.  Pointers are device addresses.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // may be null
  const int32_t* tiles;    // 8 ints per tile (planner layout)
  const int32_t* wg_ptr;   // workgroup w runs tiles wg_ptr[w] .. wg_ptr[w+1]-1 (decode kernel)
  const int32_t* cols;     // column blocks per row block
  const int32_t* lens;     // valid length of each cols entry, or null (all blocks full)
  float* part;             // split partial region
  const void* zero_row;    // >= 1 KB of zeros in the workspace (loads of masked keys)
  int64_t q_stride, k_stride, v_stride, o_stride;  // elements per token
  int32_t R, C, group, num_qo_heads;
  int32_t causal_off;      // N - M
  float scale_log2;        // sm_scale * q_descale * k_descale * log2(e)
  float out_scale;         // v_descale
  int32_t num_tiles;
  int32_t num_wgs;         // workgroups of the launch (decode kernel)
  int32_t heads_per_wg;    // decode kernel: kv heads of one workgroup (a power of two <= 8)
  // per-head dequant scales (device float arrays, or null = 1): q per qo head,
  // k and v per kv head (decode and tile kernels)
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  // element-mask bit planes (tile kernel): plane r, bit e*C + c = row r of
  // column-list entry e's row block sees key c of that block; null = none
  const uint32_t* mbits;
  int64_t mask_plane_words;
  int32_t* trace;          // trace build only: per-tile records (planner.h), else null
  int64_t num_keys;        // N: key tokens are in [0, N) (checked by the trace build)
};

struct MergeArgs {
  const int32_t* merges;   // 8 ints per merge (planner layout)
  const float* part;
  void* o;
  float* lse;              // may be null
  int64_t o_stride;        // elements per token
  int32_t R, group, num_qo_heads, dv;
  int32_t num_merges;
};

// Generic MFMA tile kernel, head_dim 128, q/o fp16 or bf16, K/V in the same
// type or fp8 e4m3 (kv8).  tile_rows in {32, 128, 256}.
hipError_t launch_attn_tile(const AttnArgs& a, bool bf16, bool kv8, int tile_rows, bool causal, bool has_lens,
                            bool has_mask, hipStream_t stream);

// Paged-decode kernel: R = 1, C >= 16, head_dim 128, q/o fp16 or bf16, K/V in
// the same type or fp8 e4m3 (kv8), g <= 16; workgroup w runs the tile groups
// wg_ptr[w] .. wg_ptr[w+1]-1 (heads_per_wg tiles each).
hipError_t launch_attn_decode(const AttnArgs& a, bool bf16, bool kv8, bool causal, bool has_lens,
                              hipStream_t stream);

// Sparse-MLA kernel: bf16 q/o, fp8 e4m3 kv, Dqk 576, Dv 512, one kv head.
hipError_t launch_attn_mla(const AttnArgs& a, bool causal, bool has_lens, hipStream_t stream);

// LSE merge of split partials into o / lse.
hipError_t launch_merge(const MergeArgs& a, int o_dtype, hipStream_t stream);

// Standalone merge of attention states, layout [seq][state][head][dim].
hipError_t launch_merge_states(const float* v, const float* s, void* v_out, float* s_out,
                               int64_t seq_len, int32_t num_states, int32_t num_heads,
                               int32_t head_dim, int32_t out_dtype, hipStream_t stream);

}  // namespace bsa
