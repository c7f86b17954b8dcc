// Sparse-attention indexer on gfx950: a float32 score for every key position
// a query row sees in its request's paged cache, then the row's exact Top-K
// keys (flashinfer.sparse 0.7.4, "SDSA Indexer": indexer_scores,
// top_k_from_candidates; one query head, no head weights).  Its output --
// int32 physical cache rows -- is the index list that index-selected sparse
// MLA decode consumes.
//
// Scores: a workgroup takes one request (grid x) and 256 of its key positions
// (grid y; four waves of 64): it loads the keys once into registers, stages
// the request's query rows in LDS 64 at a time, and runs them against the
// keys 16 at a time.  The dot products run on
// v_mfma_f32_16x16x32 with the query rows as the A operand (lane l: row
// l % 16, dims 8 (l / 16) .. + 7 of the k-step) and the keys as B (the same
// dims of key l % 16), so lane l ends with rows 4 (l / 16) + v of key l % 16
// and the 16 lanes of a group store 16 consecutive scores of one row.  Key
// rows are fetched through the block table with 16-byte loads; a page id
// outside the cache reads as a zero key.
//
// Top-K: a score maps to an unsigned key that orders like the float (sign bit
// flipped for positives, all bits for negatives; -0 becomes +0).  Each row is
// cut into chunks of 16384 positions, one 1024-thread workgroup per (row,
// chunk), in three kernels:
//   (1) histogram of the keys' top 12 bits in LDS, added to the row's
//       histogram in the workspace; the row's last workgroup to finish finds
//       the bin of the K-th largest key;
//   (2) each chunk counts its keys in the bins above (kept outright) and
//       appends that bin's keys with their positions to the row's candidates;
//       the last workgroup selects among the candidates the exact K-th largest
//       key T (radix passes over the remaining bits) and, when not every key
//       equal to T is kept, the last kept position among them (ties to the
//       lower position), then turns the chunks' kept counts into output
//       offsets;
//   (3) each chunk writes its kept positions' cache rows in position order
//       from its offset (ballots within a wave, wave totals through LDS).
// "Last workgroup" is decided by a per-row arrival counter; the data it reads
// from the others goes through device-scope atomics (see last_to_arrive), and
// it resets the counters and the histogram, so the workspace is ready for the
// next call.  A bin with more keys than the candidate buffer holds (heavy
// ties) sends the row down a slower path: its first chunk's workgroup in (3)
// does the whole row by four 8-bit radix passes and per-thread segments.
#include <algorithm>

#include "device_common.h"
#include "indexer.h"

namespace bsa {

namespace {

constexpr int kRowsPerGroup = 16;
constexpr int kKeyBlocks = 4;               // 16-key blocks per wave
constexpr int kQRows = 64;                  // query rows staged in LDS at a time
constexpr int kKeysPerWg = 4 * 16 * kKeyBlocks;
constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 1024;

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

// page index of position p (< 2^24): a shift when the page size is a power of two
__device__ __forceinline__ uint32_t page_of(const IndexerArgs& a, uint32_t p) {
  return a.page_shift >= 0 ? p >> a.page_shift : p / static_cast<uint32_t>(a.page_size);
}

// physical cache row of position p of request r, or -1 when the position has no page
// in the table or its page id is outside the cache
__device__ __forceinline__ int64_t idx_slot(const IndexerArgs& a, int r, int64_t p) {
  const uint32_t pi = page_of(a, static_cast<uint32_t>(p));
  if (static_cast<int32_t>(pi) >= a.max_pages) return -1;
  const int32_t page = a.block_table[static_cast<int64_t>(r) * a.max_pages + pi];
  const int64_t slot = static_cast<int64_t>(page) * a.page_size + (p - static_cast<int64_t>(pi) * a.page_size);
  return (page < 0 || slot >= a.num_slots) ? -1 : slot;
}

template <typename T, int KSTEPS>
__global__ __launch_bounds__(kScoreThreads) void indexer_scores_kernel(IndexerArgs a) {
  using Ops = IdxOps<T>;
  using v8 = typename Ops::v8;
  constexpr int D = 32 * KSTEPS;     // head_dim
  constexpr int LDQ = D + 8;         // padded LDS row: the 16 rows a k-step reads fall in distinct banks
  __shared__ __attribute__((aligned(16))) T qs[kQRows * LDQ];
  __shared__ int lens[kQRows];
  const int r = blockIdx.x;
  const int rb = a.req_row_ptr[r];
  const int re = min(a.req_row_ptr[r + 1], a.num_rows);
  if (rb >= re) return;
  const int64_t kv_len = a.req_kv_len[r];
  const int64_t p_wg = static_cast<int64_t>(blockIdx.y) * kKeysPerWg;
  if (p_wg >= kv_len || p_wg >= a.max_ctx) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int quad = lane >> 4;

  // B: this wave's kKeyBlocks 16-key blocks, loaded once for every query row of the request.
  // A key past the request or outside the cache loads cache row 0 and its scores are
  // stored as 0 (a zero key), so nothing waits on the loads before the first product.
  // All block-table entries are read before any key row is requested (a position
  // without a page reads entry 0 and is marked as a zero key).
  v8 kf[kKeyBlocks][KSTEPS];
  int32_t page[kKeyBlocks];
  uint32_t pidx[kKeyBlocks];
  uint32_t zero_key = 0;  // bit kb: this lane's key of block kb counts as zeros
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb) {
    const int64_t p = p_wg + wave * (16 * kKeyBlocks) + kb * 16 + c16;
    pidx[kb] = page_of(a, static_cast<uint32_t>(p));
    const bool has_page = p < kv_len && static_cast<int32_t>(pidx[kb]) < a.max_pages;
    zero_key |= has_page ? 0u : 1u << kb;
    page[kb] = a.block_table[static_cast<int64_t>(r) * a.max_pages + (has_page ? pidx[kb] : 0)];
  }
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb) {
    const int64_t p = p_wg + wave * (16 * kKeyBlocks) + kb * 16 + c16;
    const int64_t slot = static_cast<int64_t>(page[kb]) * a.page_size + (p - static_cast<int64_t>(pidx[kb]) * a.page_size);
    const bool ok = !((zero_key >> kb) & 1u) && page[kb] >= 0 && slot < a.num_slots;
    zero_key |= ok ? 0u : 1u << kb;
    const T* kp = static_cast<const T*>(a.key_cache) + (ok ? slot : 0) * a.k_stride + quad * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) kf[kb][ks] = *reinterpret_cast<const v8*>(kp + ks * 32);
  }
  // A: the request's query rows, kQRows at a time through LDS (the next block's rows are
  // requested while the current one multiplies), then 16 at a time into the MFMAs
  constexpr int CPR = D / 8;                         // 16-byte pieces per row
  constexpr int PPT = kQRows * CPR / kScoreThreads;  // pieces per thread
  v8 stage[PPT];
  int len_t;
  // (rows past the block re-read its last row; they are never used)
  auto request_block = [&](int rblk) {
    const int nblk = min(re - rblk, kQRows);
    len_t = a.ctx_len[rblk + min(tid, nblk - 1)];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int i = tid + j * kScoreThreads;
      const int rr = min(i / CPR, nblk - 1), cc = i % CPR;
      stage[j] = *reinterpret_cast<const v8*>(static_cast<const T*>(a.q) + static_cast<int64_t>(rblk + rr) * a.q_stride +
                                              cc * 8);
    }
  };
  request_block(rb);
  // the keys are in registers before the loop starts (the loop then never waits on them, and
  // the next block's rows stay in flight while the current block multiplies)
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) asm volatile("" ::"v"(kf[kb][ks]));
#pragma unroll 1
  for (int rblk = rb; rblk < re; rblk += kQRows) {
    const int nblk = min(re - rblk, kQRows);
    __syncthreads();  // the previous block's rows are no longer read
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int i = tid + j * kScoreThreads;
      const int rr = i / CPR, cc = i % CPR;
      *reinterpret_cast<v8*>(&qs[rr * LDQ + cc * 8]) = stage[j];
    }
    if (tid < kQRows) lens[tid] = len_t;
    __syncthreads();
    if (rblk + kQRows < re) request_block(rblk + kQRows);
    // unrolled: a loop here would make the compiler wait for the requested rows first
#pragma unroll
    for (int g = 0; g < kQRows / kRowsPerGroup; ++g) {
      const int g0 = g * kRowsPerGroup;
      if (g0 >= nblk) break;
      // rows past the block read its first row: their results are never stored
      const int rl = g0 + c16 < nblk ? g0 + c16 : 0;
      v8 qf[KSTEPS];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const v8*>(&qs[rl * LDQ + ks * 32 + quad * 8]);
      f32x4 acc[kKeyBlocks];
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb) {
        acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) acc[kb] = Ops::mfma(qf[ks], kf[kb][ks], acc[kb]);
      }
      // lane (c16, quad) holds rows 4 quad + v of key c16 of each block
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int bl = g0 + 4 * quad + v;
        if (bl >= nblk) continue;
        const int64_t n = min(static_cast<int64_t>(lens[bl]), a.max_ctx);
        float* sp = a.scores + static_cast<int64_t>(rblk + bl) * a.ld_scores;
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb) {
          const int64_t p = p_wg + wave * (16 * kKeyBlocks) + kb * 16 + c16;
          if (p < n) sp[p] = (zero_key >> kb) & 1u ? 0.f : acc[kb][v];
        }
      }
    }
  }
}

// order-preserving unsigned key of a float score (-0 and +0 equal)
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// exclusive scan of one value per thread over a workgroup of kTopkThreads: a
// shuffle scan inside each wave, then the waves' totals through LDS (lds holds
// one int per wave).  Returns the thread's exclusive prefix, *total the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds, int* total) {
  constexpr int NW = kTopkThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int x = __shfl_up(incl, off);
    if (lane >= off) incl += x;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = lds[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return before + incl - v;
}

// Thread t holds the count v of the bin `bin` that comes t-th in scan order.
// Returns the bin holding the need-th key in that order; need becomes the
// key's rank inside it and *count the bin's size.  Requires 1 <= need <= the
// total count.
__device__ __forceinline__ int pick_bin(int v, int bin, int& need, int* count, int* scan, int* pick) {
  int tot;
  const int before = block_exclusive_scan(v, scan, &tot);
  if (before < need && before + v >= need) {
    pick[0] = bin;
    pick[1] = need - before;
    pick[2] = v;
  }
  __syncthreads();
  const int b = pick[0];
  need = pick[1];
  *count = pick[2];
  __syncthreads();
  return b;
}

// request of a row (the last r with req_row_ptr[r] <= row) and the row's key
// count n = min(ctx_len, req_kv_len, max_ctx), 0 for a row outside every request
__device__ __forceinline__ int64_t row_keys(const IndexerArgs& a, int row, int* r_out) {
  const int64_t len = a.ctx_len[row];  // requested alongside the search
  int lo = 0, hi = a.num_reqs;         // num_reqs >= 1 (checked on the host)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.req_row_ptr[mid] <= row) lo = mid;
    else hi = mid;
  }
  const bool in_req = a.req_row_ptr[lo] <= row && row < a.req_row_ptr[lo + 1];
  int64_t n = in_req ? len : 0;
  if (in_req && n > a.req_kv_len[lo]) n = a.req_kv_len[lo];
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  *r_out = lo;
  return n;
}

// the row's block of the workspace and its parts
__device__ __forceinline__ char* row_ws(const IndexerArgs& a, int row) { return a.ws + static_cast<int64_t>(row) * kIdxRowBytes; }
__device__ __forceinline__ uint32_t* row_state(const IndexerArgs& a, int row) {
  return reinterpret_cast<uint32_t*>(row_ws(a, row) + kIdxRowState);
}

// Workgroups of one row pass data to the row's last workgroup only through
// device-scope atomics: read-modify-writes whose returned value each thread
// waits for (an atomic returns after it has been performed at the device's
// coherence point), and atomic loads in the reader.  No fence is needed, and
// none is taken: a device-scope fence writes back and invalidates the L2 of
// the caller's XCD.
__device__ __forceinline__ uint32_t dev_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_xchg(uint32_t* p, uint32_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t dev_xchg(uint64_t* p, uint64_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T dev_load(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True in the one workgroup that completes a row's step.  `sink` folds the
// values the thread's device atomics returned: using it makes the thread wait
// for them, so when the workgroup counts itself in, its atomics are performed.
__device__ __forceinline__ bool last_to_arrive(uint32_t* counter, int count, uint32_t sink, int* flag) {
  asm volatile("" ::"v"(sink));
  __syncthreads();
  if (threadIdx.x == 0) *flag = dev_add(counter, 1u) == static_cast<uint32_t>(count - 1) ? 1 : 0;
  __syncthreads();
  return *flag != 0;
}

// Top-K of one row by four 8-bit radix passes over the scores in global
// memory and per-thread contiguous segments for the ordered output: one
// workgroup does the whole row (the path for a row whose bin of the K-th
// largest key holds more keys than the candidate buffer, i.e. heavy ties).
__device__ void topk_by_radix_passes(const IndexerArgs& a, int r, const float* s, int64_t n, int K, int32_t* out,
                                     int* hist, int* scan, int* pick) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int need = K;  // keys still to take among those matching prefix
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kTopkThreads) {
      const uint32_t u = score_key(s[i]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    // the digit whose bin holds the need-th largest key, bins taken from the top
    const int d = 255 - tid;
    int cnt;
    const int digit = pick_bin(tid < 256 ? hist[d] : 0, d, need, &cnt, scan, pick);
    prefix |= static_cast<uint32_t>(digit) << shift;
    mask |= 0xFFu << shift;
  }
  const uint32_t T = prefix;  // the K-th largest key; `need` keys equal to it are kept
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

constexpr int kHistShift = 32 - kIdxHistBits;  // a key's histogram bin is key >> kHistShift
constexpr int kChunkShift = 14;                 // log2(kIdxChunk)
constexpr int kPer = kIdxChunk / (4 * kTopkThreads);  // 16-byte groups per thread and chunk
constexpr int kWaveSpan = kIdxChunk / (kTopkThreads / 64);  // positions per wave and chunk
static_assert(kQRows * 8 % kScoreThreads == 0, "whole 16-byte pieces per thread");
static_assert((1 << kChunkShift) == kIdxChunk && kPer == 4 && kWaveSpan == 4 * 64 * kPer, "chunk layout");
static_assert(kIdxHistBits == 12, "candidates are resolved by two 10-bit passes over the low 20 bits");

// first of the four positions that thread tid takes in step j of chunk c: wave w owns
// the chunk's positions kWaveSpan w .. + kWaveSpan - 1, 256 of them per step
__device__ __forceinline__ int64_t chunk_pos(int c, int tid, int j) {
  return (static_cast<int64_t>(c) << kChunkShift) + (tid >> 6) * kWaveSpan + j * 256 + 4 * (tid & 63);
}

// the thread's kPer 16-byte groups of the chunk (zeros past n; score rows are padded
// to 64 floats, so a group that starts below n lies in the row)
__device__ __forceinline__ void load_chunk(const float* srow, int c, int tid, int64_t n, f32x4 (&v)[kPer]) {
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = chunk_pos(c, tid, j);
    v[j] = p < n ? *reinterpret_cast<const f32x4*>(srow + p) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// (1) per chunk: a histogram of the keys' top 12 bits in LDS, added to the
// row's histogram in the workspace; the last chunk to finish locates the bin
// of the K-th largest key and clears the histogram for the next call
__global__ __launch_bounds__(kTopkThreads) void topk_hist_kernel(IndexerArgs a) {
  __shared__ int hist[kIdxHistBins];
  __shared__ int scan[kTopkThreads / 64];
  __shared__ int flag;
  const int row = blockIdx.x;
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  int r;
  const int64_t n = row_keys(a, row, &r);
  const int K = a.topk;
  if (n <= K) return;
  const int nch = static_cast<int>((n + kIdxChunk - 1) >> kChunkShift);
  if (c >= nch) return;
  f32x4 v[kPer];
  load_chunk(a.scores + static_cast<int64_t>(row) * a.ld_scores, c, tid, n, v);
  for (int i = tid; i < kIdxHistBins; i += kTopkThreads) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = chunk_pos(c, tid, j);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (p + e < n) atomicAdd(&hist[score_key(v[j][e]) >> kHistShift], 1);
  }
  __syncthreads();
  uint32_t* gh = reinterpret_cast<uint32_t*>(row_ws(a, row) + kIdxRowHist);
  uint32_t sink = 0;
  for (int i = tid; i < kIdxHistBins; i += kTopkThreads) {
    const int h = hist[i];
    if (h != 0) sink ^= dev_add(&gh[i], static_cast<uint32_t>(h));
  }
  uint32_t* st = row_state(a, row);
  if (!last_to_arrive(&st[kStArrive0], nch, sink, &flag)) return;
  // the row's last chunk: thread t takes bins 4095 - 4t .. 4092 - 4t (from the top)
  constexpr int BPT = kIdxHistBins / kTopkThreads;
  int h[BPT], sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    h[j] = static_cast<int>(dev_load(&gh[kIdxHistBins - 1 - (tid * BPT + j)]));
    sum += h[j];
  }
  int tot;
  int above = block_exclusive_scan(sum, scan, &tot);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    if (above < K && above + h[j] >= K) {
      st[kStBin] = static_cast<uint32_t>(kIdxHistBins - 1 - (tid * BPT + j));
      st[kStNeed] = static_cast<uint32_t>(K - above);  // keys to take from that bin
      st[kStInBin] = static_cast<uint32_t>(h[j]);      // keys in that bin
      st[kStFallback] = h[j] > kIdxCandCap ? 1u : 0u;
    }
    above += h[j];
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) gh[kIdxHistBins - 1 - (tid * BPT + j)] = 0;
  if (tid == 0) st[kStArrive0] = 0;
}

// (2) per chunk: the count of keys in the bins above the K-th key's bin (all
// kept) and that bin's keys appended, with their positions, to the row's
// candidates (one reservation per workgroup).  The last chunk to finish
// selects among the candidates the exact K-th largest key T (two 10-bit radix
// passes over the bits below the bin's) and, when not every key equal to T is
// kept, the position of the last one kept (ties to the lower position: 10-,
// 10- and 4-bit passes over the tied keys' positions, lowest first); it then
// turns each chunk's kept count into the chunk's offset in the row's output.
__global__ __launch_bounds__(kTopkThreads) void topk_collect_kernel(IndexerArgs a) {
  __shared__ uint32_t cu[kIdxCandCap];
  __shared__ int32_t cp[kIdxCandCap];
  __shared__ int kc[kIdxMaxChunks];
  __shared__ int h[kTopkThreads];
  __shared__ int scan[kTopkThreads / 64];
  __shared__ int pick[3];
  __shared__ int flag;
  __shared__ uint32_t base_lds;
  const int row = blockIdx.x;
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  int r;
  const int64_t n = row_keys(a, row, &r);
  const int K = a.topk;
  if (n <= K) return;
  const int nch = static_cast<int>((n + kIdxChunk - 1) >> kChunkShift);
  if (c >= nch) return;
  f32x4 v[kPer];
  load_chunk(a.scores + static_cast<int64_t>(row) * a.ld_scores, c, tid, n, v);
  uint32_t* st = row_state(a, row);
  const uint32_t bin = st[kStBin];
  const bool collect = st[kStFallback] == 0;
  int above = 0, mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = chunk_pos(c, tid, j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t hb = score_key(v[j][e]) >> kHistShift;
      if (p + e < n) {
        above += hb > bin ? 1 : 0;
        mine += hb == bin ? 1 : 0;
      }
    }
  }
  // one scan for both counts: a chunk holds at most 2^14 keys, so the low 16 bits never carry
  int tot;
  const int pre = block_exclusive_scan(above | mine << 16, scan, &tot);
  const int above_c = tot & 0xffff;
  const int mine_c = tot >> 16;
  uint64_t* cand = reinterpret_cast<uint64_t*>(row_ws(a, row) + kIdxRowCand);  // key | position << 32
  uint32_t sink = 0;
  if (collect && mine_c > 0) {
    if (tid == 0) base_lds = dev_add(&st[kStNcand], static_cast<uint32_t>(mine_c));
    __syncthreads();
    // the bin holds at most kIdxCandCap keys, so every append fits
    uint32_t idx = base_lds + static_cast<uint32_t>(pre >> 16);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t p = chunk_pos(c, tid, j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = score_key(v[j][e]);
        if (p + e < n && (u >> kHistShift) == bin) {
          if (idx < static_cast<uint32_t>(kIdxCandCap))
            sink ^= static_cast<uint32_t>(dev_xchg(&cand[idx], u | static_cast<uint64_t>(p + e) << 32));
          ++idx;
        }
      }
    }
  }
  uint32_t* chunk = reinterpret_cast<uint32_t*>(row_ws(a, row) + kIdxRowChunk);
  if (tid == 0) sink ^= dev_xchg(&chunk[c], static_cast<uint32_t>(above_c));
  if (!last_to_arrive(&st[kStArrive1], nch, sink, &flag)) return;
  if (!collect) {  // the output kernel takes the whole row by radix passes
    if (tid == 0) st[kStArrive1] = 0;
    return;
  }
  const int m = min(static_cast<int>(st[kStInBin]), kIdxCandCap);
  for (int j = tid; j < m; j += kTopkThreads) {
    const uint64_t x = dev_load(&cand[j]);
    cu[j] = static_cast<uint32_t>(x);
    cp[j] = static_cast<int32_t>(x >> 32);
  }
  // each chunk's keys above the bin: its kept count before the candidates
  if (tid < nch) kc[tid] = static_cast<int>(dev_load(&chunk[tid]));
  int need = static_cast<int>(st[kStNeed]);
  uint32_t T = bin << kHistShift;
  int ties = 0;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = 10 - 10 * pass;
    const uint32_t msk = ~0u << (shift + 10);
    h[tid] = 0;
    __syncthreads();
    for (int j = tid; j < m; j += kTopkThreads) {
      const uint32_t u = cu[j];
      if ((u & msk) == T) atomicAdd(&h[(u >> shift) & 1023], 1);
    }
    __syncthreads();
    const int d = pick_bin(h[1023 - tid], 1023 - tid, need, &ties, scan, pick);
    T |= static_cast<uint32_t>(d) << shift;
  }
  // `ties` keys equal T; the `need` of them with the lowest positions are kept
  int32_t p_last = 0x7fffffff;
  if (need < ties) {
    uint32_t ppre = 0, pmsk = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 14 : (pass == 1 ? 4 : 0);
      const uint32_t dm = pass < 2 ? 1023u : 15u;
      h[tid] = 0;
      __syncthreads();
      for (int j = tid; j < m; j += kTopkThreads) {
        const uint32_t pj = static_cast<uint32_t>(cp[j]);
        if (cu[j] == T && (pj & pmsk) == ppre) atomicAdd(&h[(pj >> shift) & dm], 1);
      }
      __syncthreads();
      int cnt;
      const int d = pick_bin(h[tid], tid, need, &cnt, scan, pick);
      ppre |= static_cast<uint32_t>(d) << shift;
      pmsk |= dm << shift;
    }
    p_last = static_cast<int32_t>(ppre);
  }
  // kept keys per chunk: those above the bin plus the kept candidates
  static_assert(kIdxMaxChunks == kTopkThreads, "one chunk per thread");
  for (int j = tid; j < m; j += kTopkThreads) {
    const uint32_t u = cu[j];
    const int32_t pj = cp[j];
    if (u > T || (u == T && pj <= p_last)) atomicAdd(&kc[pj >> kChunkShift], 1);
  }
  __syncthreads();
  const int mine_k = tid < nch ? kc[tid] : 0;
  const int off = block_exclusive_scan(mine_k, scan, &tot);
  if (tid < nch) chunk[tid] = static_cast<uint32_t>(off);
  if (tid == 0) {
    st[kStT] = T;
    st[kStPLast] = static_cast<uint32_t>(p_last);
    st[kStNcand] = 0;
    st[kStArrive1] = 0;
  }
}

// (3) per chunk: the kept keys' cache rows, in position order, from the
// chunk's offset.  A wave's keys rank after the kept keys of the waves
// before it; inside a wave, step j's keys after those of steps j' < j, and
// lane l's four keys after the kept keys of lanes below it (one ballot per
// key of the group).  A row with n <= K writes its n slots and the -1 padding
// here; a row on the slow path is done whole by its first chunk's workgroup.
__global__ __launch_bounds__(kTopkThreads) void topk_out_kernel(IndexerArgs a) {
  __shared__ int wc[kTopkThreads / 64];
  __shared__ int hist[256];
  __shared__ int scan[kTopkThreads / 64];
  __shared__ int pick[3];
  const int row = blockIdx.x;
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int r;
  const int64_t n = row_keys(a, row, &r);
  const int K = a.topk;
  int32_t* out = a.out + static_cast<int64_t>(row) * K;
  if (n <= K) {
    const int64_t i0 = static_cast<int64_t>(c) << kChunkShift;
    for (int64_t i = i0 + tid; i < i0 + kIdxChunk && i < K; i += kTopkThreads)
      out[i] = i < n ? static_cast<int32_t>(idx_slot(a, r, i)) : -1;
    return;
  }
  const int nch = static_cast<int>((n + kIdxChunk - 1) >> kChunkShift);
  if (c >= nch) return;
  const float* s = a.scores + static_cast<int64_t>(row) * a.ld_scores;
  f32x4 v[kPer];
  load_chunk(s, c, tid, n, v);
  const uint32_t* st = row_state(a, row);
  if (st[kStFallback] != 0) {
    if (c == 0) topk_by_radix_passes(a, r, s, n, K, out, hist, scan, pick);
    return;
  }
  const uint32_t T = st[kStT];
  const int64_t p_last = static_cast<int32_t>(st[kStPLast]);
  const int base = static_cast<int>(reinterpret_cast<const uint32_t*>(row_ws(a, row) + kIdxRowChunk)[c]);
  uint32_t keep = 0;  // bit 4 j + e: key e of step j is kept
  int rank[kPer];     // kept keys of the wave before lane's group in step j
  int w_total = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = chunk_pos(c, tid, j);
    int below = 0, step = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = score_key(v[j][e]);
      const bool k = p + e < n && (u > T || (u == T && p + e <= p_last));
      keep |= k ? 1u << (4 * j + e) : 0u;
      const uint64_t bal = __ballot(k);
      below += __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                         __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
      step += __popcll(bal);
    }
    rank[j] = w_total + below;
    w_total += step;
  }
  if (lane == 0) wc[wave] = w_total;
  __syncthreads();
  int o0 = base;
  for (int w = 0; w < wave; ++w) o0 += wc[w];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = chunk_pos(c, tid, j);
    int o = o0 + rank[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (keep & (1u << (4 * j + e))) {
        if (o < K) out[o] = static_cast<int32_t>(idx_slot(a, r, p + e));
        ++o;
      }
    }
  }
}

template <typename T>
hipError_t launch_scores(const IndexerArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.num_reqs), static_cast<unsigned>((a.max_ctx + kKeysPerWg - 1) / kKeysPerWg));
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
  if (a.num_reqs > 0) {
    const hipError_t e = bf16 ? launch_scores<__bf16>(a, st) : launch_scores<_Float16>(a, st);
    if (e != hipSuccess) return e;
  }
  if (scores_only) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(a.num_rows), static_cast<unsigned>(a.nch_max));
  topk_hist_kernel<<<grid, kTopkThreads, 0, st>>>(a);
  topk_collect_kernel<<<grid, kTopkThreads, 0, st>>>(a);
  const int64_t out_chunks = std::max<int64_t>(a.nch_max, (a.topk + kIdxChunk - 1) / kIdxChunk);
  topk_out_kernel<<<dim3(static_cast<unsigned>(a.num_rows), static_cast<unsigned>(out_chunks)), kTopkThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace bsa
