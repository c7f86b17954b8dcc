// LSE merge of attention states on gfx950 (flashinfer.cascade merge_state /
// merge_states; the split-KV combine step of BlockSparseAttentionWrapper's
// kv_splits).  For one query row with states (o_s, lse_s) over disjoint key
// sets:  lse = M + ln sum_s exp(lse_s - M) with M = max_s lse_s, and
// o = sum_s exp(lse_s - lse) o_s.  States with lse_s = -inf weigh 0; if all
// are -inf the row is o = 0, lse = -inf.  Bandwidth-bound: every thread owns
// four consecutive output values of one row and reads the matching float4
// of each state; the per-row weights are recomputed by each thread from the
// (cached) lse values instead of being staged through LDS.
#include "device_common.h"
#include "kernels.h"

namespace bsa {

namespace {

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
  typedef T v4t __attribute__((ext_vector_type(4)));
  v4t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = static_cast<T>(v[e]);
  *reinterpret_cast<v4t*>(p) = o;
}

template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

// Merge `n` states of one row: lse of state s at lse_p[s * lse_step], its
// 4-vector at o_p[s * o_step].  Returns the merged 4-vector, *lse_out the
// merged lse.  One pass with a running maximum (the accumulator is rescaled
// when it grows); the loads of up to eight states are issued together before
// any of them is merged (a split row has at most a few partitions, so this is
// usually a single memory round trip), and a state with lse = -inf is skipped
// by a select, so whatever its values hold never reaches the sum.
__device__ __forceinline__ void merge_one(float l, f32x4 o, float& mx, float& tot, f32x4& acc) {
  const bool live = l != -INFINITY;
  const float m_new = live ? fmaxf(mx, l) : mx;
  const float scale = m_new == mx ? 1.f : fast_exp2((mx - m_new) * kLog2e);  // mx = -inf: 0
  const float w = live ? fast_exp2((l - m_new) * kLog2e) : 0.f;
  tot = tot * scale + w;
  acc = live ? acc * scale + w * o : acc;
  mx = m_new;
}

__device__ __forceinline__ f32x4 merge_row4(const float* lse_p, int64_t lse_step, const float* o_p,
                                            int64_t o_step, int n, float* lse_out) {
  constexpr int kBatch = 8;
  float mx = -INFINITY, tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n; s0 += kBatch) {
    float l[kBatch];
    f32x4 o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      // states past n read state s0 (in bounds) and are dropped below
      const int s = s0 + j < n ? s0 + j : s0;
      l[j] = lse_p[s * lse_step];
      o[j] = *reinterpret_cast<const f32x4*>(o_p + s * o_step);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) merge_one(s0 + j < n ? l[j] : -INFINITY, o[j], mx, tot, acc);
  }
  if (mx == -INFINITY) {
    *lse_out = -INFINITY;
    return f32x4{0.f, 0.f, 0.f, 0.f};
  }
  *lse_out = mx + __logf(tot);
  return acc * (1.f / tot);
}

template <typename T>
__global__ __launch_bounds__(256) void merge_partials_kernel(MergeArgs a) {
  const int32_t* m = a.merges + static_cast<int64_t>(blockIdx.x) * 8;
  const int I = m[0], kvh = m[1], row0 = m[2], nrows = m[3], p0 = m[4], ns = m[5], stride = m[6];
  const int chunks = a.dv / 4;
  const float* base = a.part + p0;
  for (int item = threadIdx.x; item < nrows * chunks; item += blockDim.x) {
    const int rl = item / chunks;
    const int c4 = (item - rl * chunks) * 4;
    float lse;
    const f32x4 o = merge_row4(base + static_cast<int64_t>(nrows) * a.dv + rl, stride,
                               base + static_cast<int64_t>(rl) * a.dv + c4, stride, ns, &lse);
    const int r = row0 + rl;
    const int tok = I * a.R + r / a.group;
    const int head = kvh * a.group + r % a.group;
    store4(static_cast<T*>(a.o) + static_cast<int64_t>(tok) * a.o_stride + static_cast<int64_t>(head) * a.dv + c4, o);
    if (c4 == 0 && a.lse) a.lse[static_cast<int64_t>(tok) * a.num_qo_heads + head] = lse;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void merge_states_kernel(const float* v, const float* s, T* v_out,
                                                           float* s_out, int64_t rows, int ns,
                                                           int heads, int dim) {
  const int chunks = dim / 4;
  const int64_t total = rows * chunks;
  for (int64_t item = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; item < total;
       item += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = item / chunks;  // row = seq * heads + head
    const int c4 = static_cast<int>(item - row * chunks) * 4;
    const int64_t seq = row / heads;
    const int head = static_cast<int>(row - seq * heads);
    float lse;
    const f32x4 o = merge_row4(s + seq * ns * heads + head, heads,
                               v + (seq * ns * heads + head) * static_cast<int64_t>(dim) + c4,
                               static_cast<int64_t>(heads) * dim, ns, &lse);
    store4(v_out + row * dim + c4, o);
    if (c4 == 0 && s_out) s_out[row] = lse;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int o_dtype, hipStream_t st) {
  if (a.num_merges == 0) return hipSuccess;
  const dim3 grid(a.num_merges), block(256);
  if (o_dtype == 1) merge_partials_kernel<__bf16><<<grid, block, 0, st>>>(a);
  else merge_partials_kernel<_Float16><<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge_states(const float* v, const float* s, void* v_out, float* s_out,
                               int64_t seq_len, int32_t num_states, int32_t num_heads,
                               int32_t head_dim, int32_t out_dtype, hipStream_t st) {
  const int64_t rows = seq_len * num_heads;
  const int64_t items = rows * (head_dim / 4);
  if (items == 0) return hipSuccess;
  int64_t blocks = (items + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (out_dtype) {
    case 0:
      merge_states_kernel<_Float16><<<grid, block, 0, st>>>(v, s, static_cast<_Float16*>(v_out), s_out, rows,
                                                             num_states, num_heads, head_dim);
      break;
    case 1:
      merge_states_kernel<__bf16><<<grid, block, 0, st>>>(v, s, static_cast<__bf16*>(v_out), s_out, rows,
                                                           num_states, num_heads, head_dim);
      break;
    default:
      merge_states_kernel<float><<<grid, block, 0, st>>>(v, s, static_cast<float*>(v_out), s_out, rows,
                                                          num_states, num_heads, head_dim);
      break;
  }
  return hipGetLastError();
}

}  // namespace bsa
