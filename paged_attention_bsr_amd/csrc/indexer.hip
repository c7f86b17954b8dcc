// Sparse-attention indexer on gfx950: FP32 scores of query rows against their
// request's paged keys, then each row's exact Top-K keys (flashinfer.sparse
// 0.7.4, "SDSA Indexer": indexer_scores, top_k_from_candidates; one query
// head, no head weights).  Its output -- int32 physical cache rows -- is the
// index list that index-selected sparse MLA decode consumes.
//
// Scores: a workgroup takes 16 query rows of one request (grid x) against
// 256 key positions (grid y; four waves of 64).  The dot products run on
// v_mfma_f32_16x16x32 with the query rows as the A operand (lane l: row
// l % 16, dims 8 (l / 16) .. + 7 of the k-step) and the keys as B (the same
// dims of key l % 16), so lane l ends with rows 4 (l / 16) + v of key l % 16
// and the 16 lanes of a group store 16 consecutive scores of one row.  Key
// rows are fetched through the block table with 16-byte loads; a page id
// outside the cache reads as a zero key.
//
// Top-K: one workgroup per row.  A score maps to an unsigned key that orders
// like the float (sign bit flipped for positives, all bits for negatives;
// -0 becomes +0), and four 8-bit radix passes over the row find the K-th
// largest key T and how many keys equal to T the row keeps (the lowest
// positions among them).  Then every thread owns a contiguous segment of the
// row: one pass counts its keys equal to T, a workgroup scan gives each
// segment its rank among the equal keys and, with its keys above T, its
// count of kept keys; a second scan gives each segment its first output slot,
// and the thread writes the kept positions' cache rows in position order.
#include "device_common.h"
#include "indexer.h"

namespace bsa {

namespace {

constexpr int kRowsPerGroup = 16;
constexpr int kKeysPerWg = 256;
constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 256;  // one thread per radix bin

template <typename T>
struct IdxOps;
template <>
struct IdxOps<_Float16> {
  using v8 = f16x8;
  static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct IdxOps<__bf16> {
  using v8 = bf16x8;
  static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// physical cache row of position p of request r, or -1 when the position has no page
// in the table or its page id is outside the cache
__device__ __forceinline__ int64_t idx_slot(const IndexerArgs& a, int r, int64_t p) {
  const int64_t pi = p / a.page_size;
  if (pi >= a.max_pages) return -1;
  const int32_t page = a.block_table[static_cast<int64_t>(r) * a.max_pages + pi];
  const int64_t slot = static_cast<int64_t>(page) * a.page_size + p % a.page_size;
  return (page < 0 || slot >= a.num_slots) ? -1 : slot;
}

template <typename T, int KSTEPS>
__global__ __launch_bounds__(kScoreThreads) void indexer_scores_kernel(IndexerArgs a) {
  using Ops = IdxOps<T>;
  using v8 = typename Ops::v8;
  const int groups_per_req = (a.max_rows_per_req + kRowsPerGroup - 1) / kRowsPerGroup;
  const int r = blockIdx.x / groups_per_req;
  const int g = blockIdx.x - r * groups_per_req;
  const int rb = a.req_row_ptr[r];
  const int re = a.req_row_ptr[r + 1];
  const int row0 = rb + g * kRowsPerGroup;
  if (row0 >= re || row0 >= a.num_rows) return;
  const int64_t kv_len = a.req_kv_len[r];
  const int64_t p_wg = static_cast<int64_t>(blockIdx.y) * kKeysPerWg;
  if (p_wg >= kv_len || p_wg >= a.max_ctx) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int nrows = min(min(re, a.num_rows) - row0, kRowsPerGroup);

  // A: query row c16 (rows past the group read row0: their results are never stored)
  const T* qp = static_cast<const T*>(a.q) + static_cast<int64_t>(row0 + (c16 < nrows ? c16 : 0)) * a.q_stride +
                quad * 8;
  v8 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const v8*>(qp + ks * 32);

  // B: four 16-key blocks of this wave's 64 positions
  constexpr int KB = 4;
  f32x4 acc[KB];
  v8 kf[KB][KSTEPS];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t p = p_wg + wave * 64 + kb * 16 + c16;
    const int64_t slot = p < kv_len ? idx_slot(a, r, p) : -1;
    // a key past the request or outside the cache loads cache row 0 and counts as zeros
    const T* kp = static_cast<const T*>(a.key_cache) + (slot >= 0 ? slot : 0) * a.k_stride + quad * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const v8 x = *reinterpret_cast<const v8*>(kp + ks * 32);
      kf[kb][ks] = slot >= 0 ? x : v8{};
    }
  }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) acc[kb] = Ops::mfma(qf[ks], kf[kb][ks], acc[kb]);
  }
  // lane (c16, quad) holds rows 4 quad + v of key c16 of each block
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rl = 4 * quad + v;
    if (rl >= nrows) continue;
    const int row = row0 + rl;
    const int64_t n = min(static_cast<int64_t>(a.ctx_len[row]), a.max_ctx);
    float* sp = a.scores + static_cast<int64_t>(row) * a.max_ctx;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int64_t p = p_wg + wave * 64 + kb * 16 + c16;
      if (p < n) sp[p] = acc[kb][v];
    }
  }
}

// order-preserving unsigned key of a float score (-0 and +0 equal)
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// exclusive scan of one value per thread over the workgroup; returns the
// thread's exclusive prefix, *total the sum
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTopkThreads; off <<= 1) {
    const int add = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += add;
    __syncthreads();
  }
  const int incl = lds[tid];
  *total = lds[kTopkThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kTopkThreads) void indexer_topk_kernel(IndexerArgs a) {
  __shared__ int hist[256];
  __shared__ int scan[kTopkThreads];
  __shared__ int pick[2];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  // request of this row: the last r with req_row_ptr[r] <= row (rows outside every request keep no key)
  int lo = 0, hi = a.num_reqs;  // num_reqs >= 1 (checked on the host)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.req_row_ptr[mid] <= row) lo = mid;
    else hi = mid;
  }
  const int r = lo;
  const bool in_req = a.req_row_ptr[r] <= row && row < a.req_row_ptr[r + 1];
  int64_t n = in_req ? a.ctx_len[row] : 0;
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  if (in_req && n > a.req_kv_len[r]) n = a.req_kv_len[r];
  const int K = a.topk;
  int32_t* out = a.out + static_cast<int64_t>(row) * K;
  if (n <= K) {
    for (int i = tid; i < K; i += kTopkThreads) out[i] = i < n ? static_cast<int32_t>(idx_slot(a, r, i)) : -1;
    return;
  }
  const float* s = a.scores + static_cast<int64_t>(row) * a.max_ctx;

  // radix select of the K-th largest key, 8 bits per pass from the top
  uint32_t prefix = 0, mask = 0;
  int need = K;  // keys still to take among those matching prefix
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kTopkThreads) {
      const uint32_t u = score_key(s[i]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    // the digit d whose bin holds the need-th largest key: the count of keys in
    // the bins above d (thread 255 - d's exclusive prefix over the bins taken
    // from the top) is below need and reaches it with bin d
    if (tid == 0) {
      pick[0] = 0;
      pick[1] = need;
    }
    {
      const int d = 255 - tid;
      const int h = hist[d];
      int tot;
      const int above = block_exclusive_scan(h, scan, &tot);
      if (above < need && above + h >= need) {
        pick[0] = d;
        pick[1] = need - above;
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(pick[0]) << shift;
    mask |= 0xFFu << shift;
    need = pick[1];
    __syncthreads();
  }
  const uint32_t T = prefix;  // the K-th largest key; `need` keys equal to it are kept

  // segments in position order: ranks among the keys equal to T, then output slots
  const int64_t seg = (n + kTopkThreads - 1) / kTopkThreads;
  const int64_t b = tid * seg < n ? tid * seg : n;
  const int64_t e = b + seg < n ? b + seg : n;
  int gt = 0, eq = 0;
  for (int64_t i = b; i < e; ++i) {
    const uint32_t u = score_key(s[i]);
    gt += u > T;
    eq += u == T;
  }
  int tot;
  const int eq_before = block_exclusive_scan(eq, scan, &tot);
  int eq_take = need - eq_before;
  eq_take = eq_take < 0 ? 0 : (eq_take > eq ? eq : eq_take);
  const int out0 = block_exclusive_scan(gt + eq_take, scan, &tot);
  int o = out0, taken = 0;
  for (int64_t i = b; i < e; ++i) {
    const uint32_t u = score_key(s[i]);
    bool keep = u > T;
    if (u == T) {
      keep = taken < eq_take;
      taken += 1;
    }
    if (keep && o < K) out[o++] = static_cast<int32_t>(idx_slot(a, r, i));
  }
}

template <typename T>
hipError_t launch_scores(const IndexerArgs& a, hipStream_t st) {
  const int groups = (a.max_rows_per_req + kRowsPerGroup - 1) / kRowsPerGroup;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.num_reqs) * groups),
                  static_cast<unsigned>((a.max_ctx + kKeysPerWg - 1) / kKeysPerWg));
  switch (a.head_dim) {
    case 64: indexer_scores_kernel<T, 2><<<grid, kScoreThreads, 0, st>>>(a); break;
    case 128: indexer_scores_kernel<T, 4><<<grid, kScoreThreads, 0, st>>>(a); break;
    case 256: indexer_scores_kernel<T, 8><<<grid, kScoreThreads, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, bool bf16, bool scores_only, hipStream_t st) {
  if (a.num_rows == 0) return hipSuccess;
  if (a.num_reqs > 0 && a.max_rows_per_req > 0) {
    const hipError_t e = bf16 ? launch_scores<__bf16>(a, st) : launch_scores<_Float16>(a, st);
    if (e != hipSuccess) return e;
  }
  if (scores_only) return hipSuccess;
  indexer_topk_kernel<<<a.num_rows, kTopkThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace bsa
