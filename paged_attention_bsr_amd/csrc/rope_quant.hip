// MLA RoPE + FP8 E4M3 quantize on gfx950 (MATE sparse-MLA API and FlashInfer
// wrapper pages, "RoPE and FP8 quantization": mla_rope_quantize_fp8).
//
// Per token: the 64-value RoPE tails of q (every head) and k are turned by the
// token's position (cosines and sines from a [max_seq_len, 64] cache, columns
// 0..31 and 32..63; pair i = values (i, i + 32) for the NeoX layout, (2i, 2i + 1)
// otherwise), then every value of q is multiplied by quant_scale_q and every
// value of k by quant_scale_kv and cast to FP8 E4M3.  Each float32 product and
// sum is rounded on its own (contraction is off here), so the float32 value a
// code is cast from is fixed (every product passes an empty asm barrier, so the
// compiler cannot fuse it into the following sum, whatever contraction mode
// the build uses); the cast rounds to nearest even and saturates (magnitudes
// are clamped to 448 before the hardware conversion).
//
// The op is a pure stream (2 bytes read per byte written): a workgroup takes one
// token and up to 16 heads; each lane moves 8 values at a time (a 16-byte bf16
// load, an 8-byte fp8 store), consecutive lanes covering consecutive chunks of a
// row, so every wave access is contiguous.  The token's cache row is read by the
// lanes that rotate a tail (L2-resident: positions repeat across heads).
#include "device_common.h"
#include "kernels.h"
#include "rope_quant.h"

namespace bsa {

namespace {

constexpr int kRopeHeadsPerWg = 16;
constexpr int kRopeThreads = 256;
constexpr float kFp8Max = 448.f;

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// a float32 product as its own rounded value (no fused multiply-add downstream)
__device__ __forceinline__ float rounded(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Saturate to the largest finite E4M3 magnitude; NaN passes through (min/max
// return their non-NaN operand, so it is selected around them) and becomes a
// NaN code in the cast, infinities become +-448 like any other magnitude.
__device__ __forceinline__ float sat448(float x) {
  const float c = fminf(fmaxf(x, -kFp8Max), kFp8Max);
  return x != x ? x : c;
}

// eight float32 values -> eight E4M3 codes (little-endian byte order = value order)
__device__ __forceinline__ u32x2_t fp8x8(const float (&v)[8]) {
  u32x2_t out;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int w = 0;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(v[4 * i]), sat448(v[4 * i + 1]), w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(v[4 * i + 2]), sat448(v[4 * i + 3]), w, true);
    out[i] = static_cast<uint32_t>(w);
  }
  return out;
}

__device__ __forceinline__ void load8(const unsigned short* p, float (&v)[8]) {
  const u16x8 raw = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = bf16_bits_to_f32(raw[i]);
}

// cosines and sines of cache columns j0 .. j0 + 7
__device__ __forceinline__ void load_cos_sin(const RopeArgs& a, int64_t pos, int j0, float (&c)[8], float (&s)[8]) {
  if (a.cache_bf16) {
    const unsigned short* row = static_cast<const unsigned short*>(a.cos_sin) + pos * 64;
    load8(row + j0, c);
    load8(row + 32 + j0, s);
  } else {
    const float* row = static_cast<const float*>(a.cos_sin) + pos * 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4_t cv = *reinterpret_cast<const f32x4_t*>(row + j0 + 4 * h);
      const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(row + 32 + j0 + 4 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[4 * h + i] = cv[i];
        s[4 * h + i] = sv[i];
      }
    }
  }
}

// a 64-value row times `scale` -> codes, chunk `chunk` (8 values) of a latent row
__device__ __forceinline__ void quant_chunk(const unsigned short* src, unsigned char* dst, float scale) {
  float v[8];
  load8(src, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * scale;
  *reinterpret_cast<u32x2_t*>(dst) = fp8x8(v);
}

// quarter u (16 values) of a 64-value RoPE tail: rotate, scale, cast.  NeoX: values
// 8u..8u+7 pair with 32+8u..32+8u+7 (columns 8u..8u+7); otherwise values 16u..16u+15
// form pairs (16u + 2j, 16u + 2j + 1) with column 8u + j.
__device__ __forceinline__ void rope_quarter(const RopeArgs& a, const unsigned short* src, unsigned char* dst, int u,
                                             int64_t pos, bool pos_ok, float scale) {
  if (!pos_ok) {  // the caller broke the position contract: NaN codes, no cache read
    const u32x2_t nan = {0x7f7f7f7fu, 0x7f7f7f7fu};
    *reinterpret_cast<u32x2_t*>(dst + (a.is_neox ? 8 * u : 16 * u)) = nan;
    *reinterpret_cast<u32x2_t*>(dst + (a.is_neox ? 32 + 8 * u : 16 * u + 8)) = nan;
    return;
  }
  float c[8], s[8], x0[8], x1[8], y0[8], y1[8];
  load_cos_sin(a, pos, 8 * u, c, s);
  if (a.is_neox) {
    load8(src + 8 * u, x0);        // first members of pairs 8u .. 8u+7
    load8(src + 32 + 8 * u, x1);   // their partners
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float ac = rounded(x0[j] * c[j]), bs = rounded(x1[j] * s[j]);
      const float bc = rounded(x1[j] * c[j]), as = rounded(x0[j] * s[j]);
      y0[j] = (ac - bs) * scale;
      y1[j] = (bc + as) * scale;
    }
    *reinterpret_cast<u32x2_t*>(dst + 8 * u) = fp8x8(y0);
    *reinterpret_cast<u32x2_t*>(dst + 32 + 8 * u) = fp8x8(y1);
  } else {
    load8(src + 16 * u, x0);       // pairs 8u .. 8u+3
    load8(src + 16 * u + 8, x1);   // pairs 8u+4 .. 8u+7
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      {
        const float ac = rounded(x0[2 * j] * c[j]), bs = rounded(x0[2 * j + 1] * s[j]);
        const float bc = rounded(x0[2 * j + 1] * c[j]), as = rounded(x0[2 * j] * s[j]);
        y0[2 * j] = (ac - bs) * scale;
        y0[2 * j + 1] = (bc + as) * scale;
      }
      {
        const float ac = rounded(x1[2 * j] * c[4 + j]), bs = rounded(x1[2 * j + 1] * s[4 + j]);
        const float bc = rounded(x1[2 * j + 1] * c[4 + j]), as = rounded(x1[2 * j] * s[4 + j]);
        y1[2 * j] = (ac - bs) * scale;
        y1[2 * j + 1] = (bc + as) * scale;
      }
    }
    *reinterpret_cast<u32x2_t*>(dst + 16 * u) = fp8x8(y0);
    *reinterpret_cast<u32x2_t*>(dst + 16 * u + 8) = fp8x8(y1);
  }
}

__global__ __launch_bounds__(kRopeThreads) void rope_quant_kernel(RopeArgs a) {
  const int64_t t = blockIdx.x;
  const int h0 = blockIdx.y * kRopeHeadsPerWg;
  const int nh = min(kRopeHeadsPerWg, a.num_heads - h0);
  const int tid = threadIdx.x;
  const int64_t pos = a.pos_int64 ? static_cast<const int64_t*>(a.pos)[t]
                                  : static_cast<int64_t>(static_cast<const int32_t*>(a.pos)[t]);
  const bool pos_ok = pos >= 0 && pos < a.max_seq_len;
  const unsigned short* qn = static_cast<const unsigned short*>(a.q_nope);
  const unsigned short* qr = static_cast<const unsigned short*>(a.q_rope);
  unsigned char* qno = static_cast<unsigned char*>(a.q_nope_out);
  unsigned char* qro = static_cast<unsigned char*>(a.q_rope_out);
  // q latent rows of this workgroup's heads: 64 chunks of 8 values per head
  for (int i = tid; i < nh * 64; i += kRopeThreads) {
    const int64_t h = h0 + (i >> 6);
    const int ch = i & 63;
    quant_chunk(qn + t * a.qn_s[0] + h * a.qn_s[1] + ch * 8, qno + t * a.qno_s[0] + h * a.qno_s[1] + ch * 8,
                a.scale_q);
  }
  // q RoPE tails: four quarters per head
  for (int i = tid; i < nh * 4; i += kRopeThreads) {
    const int64_t h = h0 + (i >> 2);
    rope_quarter(a, qr + t * a.qr_s[0] + h * a.qr_s[1], qro + t * a.qro_s[0] + h * a.qro_s[1], i & 3, pos, pos_ok,
                 a.scale_q);
  }
  // the token's key row, once (head chunk 0)
  if (blockIdx.y == 0) {
    if (tid < 64) {
      quant_chunk(static_cast<const unsigned short*>(a.k_nope) + t * a.kn_s + tid * 8,
                  static_cast<unsigned char*>(a.k_nope_out) + t * a.kno_s + tid * 8, a.scale_kv);
    } else if (tid < 68) {
      rope_quarter(a, static_cast<const unsigned short*>(a.k_rope) + t * a.kr_s,
                   static_cast<unsigned char*>(a.k_rope_out) + t * a.kro_s, tid - 64, pos, pos_ok, a.scale_kv);
    }
  }
}

}  // namespace

hipError_t launch_rope_quant(const RopeArgs& a, hipStream_t stream) {
  if (a.nnz == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(a.nnz), static_cast<uint32_t>((a.num_heads + kRopeHeadsPerWg - 1) / kRopeHeadsPerWg));
  rope_quant_kernel<<<grid, dim3(kRopeThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace bsa
