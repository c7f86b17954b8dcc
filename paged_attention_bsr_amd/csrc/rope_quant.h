// Launch interface of the MLA RoPE + FP8 quantize kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsa {

// MLA RoPE + FP8 quantize.  Pointers are device addresses; strides in elements
// (bf16 inputs) or bytes (fp8 outputs): [0] per token, [1] per head.
struct RopeArgs {
  const void* q_rope;      // bf16 [nnz][H][64]
  const void* k_rope;      // bf16 [nnz][64]
  const void* q_nope;      // bf16 [nnz][H][512]
  const void* k_nope;      // bf16 [nnz][512]
  const void* cos_sin;     // [max_seq_len][64] fp32 or bf16 (cache_bf16)
  const void* pos;         // [nnz] int32 or int64 (pos_int64)
  void* q_rope_out;
  void* k_rope_out;
  void* q_nope_out;
  void* k_nope_out;
  int64_t qr_s[2], qn_s[2], kr_s, kn_s;
  int64_t qro_s[2], qno_s[2], kro_s, kno_s;
  int64_t nnz, max_seq_len;
  int32_t num_heads;
  int32_t is_neox, cache_bf16, pos_int64;
  float scale_q, scale_kv;
};

hipError_t launch_rope_quant(const RopeArgs& a, hipStream_t stream);

}  // namespace bsa
