// Sparse-attention indexer on gfx950: a float32 score for every key position
// a query row sees in its request's paged cache, then the row's exact Top-K
// keys (flashinfer.sparse 0.7.4, "SDSA Indexer": indexer_scores,
// top_k_from_candidates; one query head, no head weights).  Its output --
// int32 physical cache rows -- is the index list that index-selected sparse
// MLA decode consumes.
//
// Scores: a workgroup takes one request (grid x) and 128 of its key positions
// (grid y; four waves of 32): it loads the keys once into registers, stages
// the request's query rows in LDS 64 at a time, and runs them against the
// keys 16 at a time.  The dot products run on v_mfma_f32_16x16x32 with the
// query rows as the A operand (lane l: row l % 16, dims 8 (l / 16) .. + 7 of
// the k-step) and the keys as B (the same dims of key l % 16), so lane l ends
// with rows 4 (l / 16) + v of key l % 16 and the 16 lanes of a group store 16
// consecutive scores of one row.  Key rows are fetched through the block
// table with 16-byte loads; a position whose page is missing or outside the
// cache scores as a zero key.
//
// Top-K: a score maps to an unsigned key that orders like the float (sign bit
// flipped for positives, all bits for negatives; -0 becomes +0).  Every
// workgroup of a row takes the same threshold from a sample of the row's
// scores; one workgroup per (row, chunk of 16384 positions) writes the chunk's
// keys at or above it, in position order, to the chunk's region of the
// workspace; then one workgroup per row gathers them, finds the exact K-th
// largest key among them and writes the kept keys' cache rows in position
// order.  A row whose sample misses (fewer than K keys reach the threshold, or
// more than the candidate buffer holds, as with heavy ties) is done by radix
// passes over the whole row in one workgroup.
#include <algorithm>

#include "device_common.h"
#include "indexer.h"

namespace bsa {

namespace {

constexpr int kRowsPerGroup = 16;
constexpr int kKeyBlocks = 2;               // 16-key blocks per wave
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
  const int64_t p_wg = static_cast<int64_t>(blockIdx.y) * kKeysPerWg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int quad = lane >> 4;

  // B: this wave's kKeyBlocks 16-key blocks, loaded once for every query row of the request.
  // The block-table entries depend only on the grid position, so they are requested
  // together with the request's bounds (a position without a page reads entry 0); then
  // every key row.  A key past the request or outside the cache loads cache row 0 and its
  // scores are stored as 0 (a zero key), so nothing waits on the key loads before the
  // first product.
  int32_t page[kKeyBlocks];
  uint32_t pidx[kKeyBlocks];
  uint32_t zero_key = 0;  // bit kb: this lane's key of block kb counts as zeros
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb) {
    const int64_t p = p_wg + wave * (16 * kKeyBlocks) + kb * 16 + c16;
    pidx[kb] = page_of(a, static_cast<uint32_t>(p < a.max_ctx ? p : 0));
    const bool has_page = p < a.max_ctx && static_cast<int32_t>(pidx[kb]) < a.max_pages;
    zero_key |= has_page ? 0u : 1u << kb;
    page[kb] = a.block_table[static_cast<int64_t>(r) * a.max_pages + (has_page ? pidx[kb] : 0)];
  }
  const int rb = a.req_row_ptr[r];
  const int re = min(a.req_row_ptr[r + 1], a.num_rows);
  const int64_t kv_len = a.req_kv_len[r];
  if (rb >= re || p_wg >= kv_len || p_wg >= a.max_ctx) return;
  v8 kf[kKeyBlocks][KSTEPS];
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb) {
    const int64_t p = p_wg + wave * (16 * kKeyBlocks) + kb * 16 + c16;
    const int64_t slot = static_cast<int64_t>(page[kb]) * a.page_size + (p - static_cast<int64_t>(pidx[kb]) * a.page_size);
    const bool ok = !((zero_key >> kb) & 1u) && p < kv_len && page[kb] >= 0 && slot < a.num_slots;
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

// Top-K of one row in one workgroup, for a row whose sample misses (e.g.
// heavy ties).  Every pass reads the row in steps of 4096 positions: wave w
// takes positions 256 w .. 256 w + 255 of a step (lane l the four from 4 l),
// with 16-byte loads.  The bits that all the row's keys share (above the
// highest bit where the smallest and the largest differ) are fixed by a first
// pass, so a row of equal scores needs no radix pass; the rest are resolved 8
// bits at a time from the top, giving the K-th largest key T and the number of
// keys equal to T to keep.  The output pass ranks the keys equal to T in
// position order (ballots inside a wave, wave totals through LDS, a running
// count across steps), keeps the lowest ones, and writes every kept key's
// cache row at its rank among the kept keys.
__device__ void topk_by_radix_passes(const IndexerArgs& a, int r, const float* s, int64_t n, int K, int32_t* out,
                                     int* hist, int* scan, int* pick) {
  constexpr int kStep = 4096;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // thread's 4 keys of the step at `base` (positions p0 + e); keys past n read as 0
  auto load_step = [&](int64_t base, uint32_t (&u)[4], int64_t& p0) {
    p0 = base + wave * 256 + 4 * lane;
    // score rows are padded to 64 floats: a 16-byte group that starts below n lies in the row
    const f32x4 v = p0 < n ? *reinterpret_cast<const f32x4*>(s + p0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = score_key(v[e]);
  };
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll 1
  for (int64_t base = 0; base < n; base += kStep) {
    uint32_t u[4];
    int64_t p0;
    load_step(base, u, p0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (p0 + i < n) {
        lo = min(lo, u[i]);
        hi = max(hi, u[i]);
      }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off)));
  }
  if (lane == 0) {
    hist[2 * wave] = static_cast<int>(lo);
    hist[2 * wave + 1] = static_cast<int>(hi);
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    lo = min(lo, static_cast<uint32_t>(hist[2 * w]));
    hi = max(hi, static_cast<uint32_t>(hist[2 * w + 1]));
  }
  __syncthreads();
  int bits = lo == hi ? 0 : 32 - __clz(static_cast<int>(lo ^ hi));  // bits [0, bits) still to decide
  const uint32_t low_mask = bits == 32 ? 0xFFFFFFFFu : (1u << bits) - 1u;
  uint32_t prefix = lo & ~low_mask, mask = ~low_mask;
  int need = K;  // keys still to take among those matching prefix
#pragma unroll 1
  while (bits > 0) {
    const int w = bits < 8 ? bits : 8;
    const int shift = bits - w;
    const int nb = 1 << w;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll 1
    for (int64_t base = 0; base < n; base += kStep) {
      uint32_t u[4];
      int64_t p0;
      load_step(base, u, p0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p0 + i < n && (u[i] & mask) == prefix) atomicAdd(&hist[(u[i] >> shift) & (nb - 1)], 1);
    }
    __syncthreads();
    // the digit whose bin holds the need-th largest key, bins taken from the top
    int cnt;
    const int digit = pick_bin(tid < nb ? hist[nb - 1 - tid] : 0, nb - 1 - tid, need, &cnt, scan, pick);
    prefix |= static_cast<uint32_t>(digit) << shift;
    mask |= static_cast<uint32_t>(nb - 1) << shift;
    bits = shift;
  }
  const uint32_t T = prefix;  // the K-th largest key; the `need` lowest-positioned keys equal to it are kept
  int* w_eq = hist;           // per wave: keys equal to T in this step
  int* w_keep = hist + 32;    // per wave: keys kept in this step
  int eq_base = 0, out_base = 0;  // over the steps before
#pragma unroll 1
  for (int64_t base = 0; base < n; base += kStep) {
    uint32_t u[4];
    int64_t p0;
    load_step(base, u, p0);
    // ranks of the keys equal to T: lanes below, then this lane's earlier keys
    uint32_t eqm = 0, gtm = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = p0 + i < n;
      eqm |= in && u[i] == T ? 1u << i : 0u;
      gtm |= in && u[i] > T ? 1u << i : 0u;
    }
    int below = 0, eq_w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t bal = __ballot((eqm >> e) & 1u);
      below += __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                         __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
      eq_w += __popcll(bal);
    }
    if (lane == 0) w_eq[wave] = eq_w;
    __syncthreads();
    int eq_off = eq_base, eq_step = 0;
#pragma unroll
    for (int w = 0; w < kTopkThreads / 64; ++w) {
      eq_off += w < wave ? w_eq[w] : 0;
      eq_step += w_eq[w];
    }
    uint32_t keepm = gtm;
    int rk = eq_off + below;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((eqm >> e) & 1u) {
        keepm |= rk < need ? 1u << e : 0u;
        ++rk;
      }
    // output ranks of the kept keys, in the same order
    int kbelow = 0, keep_w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t bal = __ballot((keepm >> e) & 1u);
      kbelow += __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
      keep_w += __popcll(bal);
    }
    if (lane == 0) w_keep[wave] = keep_w;
    __syncthreads();
    int o = out_base + kbelow, keep_step = 0;
#pragma unroll
    for (int w = 0; w < kTopkThreads / 64; ++w) {
      o += w < wave ? w_keep[w] : 0;
      keep_step += w_keep[w];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((keepm >> e) & 1u) {
        if (o < K) out[o] = static_cast<int32_t>(idx_slot(a, r, p0 + e));
        ++o;
      }
    eq_base += eq_step;
    out_base += keep_step;
    __syncthreads();  // w_eq / w_keep are rewritten by the next step
  }
}

constexpr int kChunkShift = 14;                                // log2(kIdxChunk)
constexpr int kCSteps = kIdxChunk / (4 * kTopkThreads);        // 16-byte groups per thread per chunk
constexpr int kCWaveSpan = kIdxChunk / (kTopkThreads / 64);    // positions per wave per chunk
static_assert((1 << kChunkShift) == kIdxChunk && kCSteps == 4 && kCWaveSpan == 256 * kCSteps, "chunk layout");
static_assert(kIdxSample % kTopkThreads == 0 && kIdxMaxChunks <= kTopkThreads, "one chunk per thread");
static_assert(kIdxCandCap % kTopkThreads == 0, "whole candidates per thread");

// The key that `rank` keys of keys[0 .. S) reach (the rank-th largest).  The bits all
// keys share (above the highest bit where the smallest and the largest differ) are
// fixed first; the rest are resolved by 8-bit radix passes from the top (so the first
// histogram spreads over its bins even when the keys lie close together, as the
// candidates above a threshold do).  Requires 1 <= rank <= S.
__device__ __forceinline__ uint32_t select_rank(const uint32_t* keys, int S, int rank, int* hist, int* scan,
                                                int* pick) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = tid; i < S; i += kTopkThreads) {
    lo = min(lo, keys[i]);
    hi = max(hi, keys[i]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off)));
  }
  if (lane == 0) {
    hist[2 * wave] = static_cast<int>(lo);
    hist[2 * wave + 1] = static_cast<int>(hi);
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    lo = min(lo, static_cast<uint32_t>(hist[2 * w]));
    hi = max(hi, static_cast<uint32_t>(hist[2 * w + 1]));
  }
  __syncthreads();
  if (lo == hi) return lo;
  int bits = 32 - __clz(static_cast<int>(lo ^ hi));  // bits [0, bits) still to decide
  const uint32_t low_mask = bits == 32 ? 0xFFFFFFFFu : (1u << bits) - 1u;
  uint32_t pre = lo & ~low_mask, msk = ~low_mask;
  int need = rank, cnt;
#pragma unroll 1
  while (bits > 0) {
    const int w = bits < 8 ? bits : 8;
    const int shift = bits - w;
    const int nb = 1 << w;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < S; i += kTopkThreads) {
      const uint32_t u = keys[i];
      if ((u & msk) == pre) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1);
    }
    __syncthreads();
    const int d = pick_bin(tid < nb ? hist[nb - 1 - tid] : 0, nb - 1 - tid, need, &cnt, scan, pick);
    pre |= static_cast<uint32_t>(d) << shift;
    msk |= static_cast<uint32_t>(nb - 1) << shift;
    bits = shift;
  }
  return pre;
}

// The row's threshold key, the same in every workgroup of the row: from a sample of
// S = min(n, 2048) scores (the whole row when n <= 2048, else 128 runs of 16
// consecutive scores spread evenly over the row), the lower edge of the 12-bit key bin
// that holds the sample's rank-th largest key.  With the whole row as the sample,
// rank = K; otherwise K's share of the sample plus four standard deviations and 8, so
// that at least K keys of the row reach the threshold unless the sample is far from
// typical.  hist holds 4096 ints.
__device__ __forceinline__ uint32_t sample_threshold(const float* s, int64_t n, int K, int* hist, int* scan,
                                                     int* pick) {
  const int tid = threadIdx.x;
  const int S = n < kIdxSample ? static_cast<int>(n) : kIdxSample;
  uint32_t smp[kIdxSample / kTopkThreads];
#pragma unroll
  for (int j = 0; j < kIdxSample / kTopkThreads; ++j) {
    const int i = tid + j * kTopkThreads;
    const int64_t p = S < n ? (i >> 4) * (n >> 7) + (i & 15) : i;  // n > 2048: the runs are n / 128 apart
    smp[j] = i < S ? score_key(s[p]) : 0u;
  }
  int rank = K;
  if (S < n) {
    const double f = static_cast<double>(K) / static_cast<double>(n);
    const double m = S * f;
    rank = min(S, static_cast<int>(ceil(m + 4.0 * sqrt(m * (1.0 - f)) + 8.0)));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) hist[tid * 4 + j] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kIdxSample / kTopkThreads; ++j)
    if (tid + j * kTopkThreads < S) atomicAdd(&hist[smp[j] >> 20], 1);
  __syncthreads();
  // thread t takes bins 4095 - 4t .. 4092 - 4t (from the top)
  int h[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = hist[4095 - (tid * 4 + j)];
    sum += h[j];
  }
  int tot;
  int above = block_exclusive_scan(sum, scan, &tot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (above < rank && above + h[j] >= rank) pick[0] = 4095 - (tid * 4 + j);
    above += h[j];
  }
  __syncthreads();
  const uint32_t thr = static_cast<uint32_t>(pick[0]) << 20;
  __syncthreads();
  return thr;
}

// (1) One 1024-thread workgroup per (row, chunk of 16384 positions): wave w takes
// positions 1024 w .. 1024 w + 1023 of the chunk, 256 per step (lane l the four from
// 4 l).  It writes the chunk's keys at or above the row's threshold, with their
// positions, in position order (per-wave counts, then ballot ranks inside each step)
// into the chunk's own region of the workspace, and their number beside it.
__global__ __launch_bounds__(kTopkThreads) void topk_candidates_kernel(IndexerArgs a) {
  __shared__ int hist[4096];
  __shared__ int scan[kTopkThreads / 64];
  __shared__ int wcnt[kTopkThreads / 64];
  __shared__ int pick[3];
  const int row = blockIdx.x;
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int r;
  const int64_t n = row_keys(a, row, &r);
  if (n <= a.topk) return;
  const int nch = static_cast<int>((n + kIdxChunk - 1) >> kChunkShift);
  if (c >= nch) return;
  const float* s = a.scores + static_cast<int64_t>(row) * a.ld_scores;
  const int64_t p0 = (static_cast<int64_t>(c) << kChunkShift) + wave * kCWaveSpan + 4 * lane;
  // score rows are padded to 64 floats, so a 16-byte group that starts below n lies in the row
  f32x4 v[kCSteps];
#pragma unroll
  for (int j = 0; j < kCSteps; ++j)
    v[j] = p0 + j * 256 < n ? *reinterpret_cast<const f32x4*>(s + p0 + j * 256) : f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t thr = sample_threshold(s, n, a.topk, hist, scan, pick);
  uint32_t sel = 0;  // bit 4 j + e: position p0 + 256 j + e is a candidate
#pragma unroll
  for (int j = 0; j < kCSteps; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sel |= p0 + j * 256 + e < n && score_key(v[j][e]) >= thr ? 1u << (4 * j + e) : 0u;
  int w_cnt = 0;
#pragma unroll
  for (int b = 0; b < 4 * kCSteps; ++b) w_cnt += __popcll(__ballot((sel >> b) & 1u));
  if (lane == 0) wcnt[wave] = w_cnt;
  __syncthreads();
  int o = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const int cw = wcnt[w];
    o += w < wave ? cw : 0;
    tot += cw;
  }
  const int64_t chunk_id = static_cast<int64_t>(row) * a.nch_max + c;
  uint2* reg = a.ws_cand + chunk_id * kIdxCandCap;
#pragma unroll
  for (int j = 0; j < kCSteps; ++j) {
    int below = 0, step = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t bal = __ballot((sel >> (4 * j + e)) & 1u);
      below += __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                         __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
      step += __popcll(bal);
    }
    int idx = o + below;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((sel >> (4 * j + e)) & 1u) {
        if (idx < kIdxCandCap)
          reg[idx] = make_uint2(score_key(v[j][e]), static_cast<uint32_t>(p0 + j * 256 + e));
        ++idx;
      }
    }
    o += step;
  }
  if (tid == 0) a.ws_count[chunk_id] = tot;
}

// (2) One 1024-thread workgroup per row: the chunks' candidates in position order
// into LDS (each chunk's count, then an exclusive scan over the chunks gives where
// its candidates start), the exact K-th largest key T among them (four 8-bit radix
// passes), and the kept keys' cache rows in position order: the keys above T, and of
// those equal to T the lowest-positioned ones.  A row whose candidates number fewer
// than K or more than kIdxCandCap (in total or in one chunk) is done by radix passes
// over the whole row.  Rows with n <= K write their n slots and the -1 padding.
__global__ __launch_bounds__(kTopkThreads) void topk_finish_kernel(IndexerArgs a) {
  __shared__ uint32_t ck[kIdxCandCap];
  __shared__ int32_t cpos[kIdxCandCap];
  __shared__ int coff[kIdxMaxChunks];
  __shared__ int hist[256];
  __shared__ int scan[kTopkThreads / 64];
  __shared__ int pick[3];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  int r;
  const int64_t n = row_keys(a, row, &r);
  const int K = a.topk;
  int32_t* out = a.out + static_cast<int64_t>(row) * K;
  if (n <= K) {
    for (int i = tid; i < K; i += kTopkThreads) out[i] = i < n ? static_cast<int32_t>(idx_slot(a, r, i)) : -1;
    return;
  }
  const float* s = a.scores + static_cast<int64_t>(row) * a.ld_scores;
  const int nch = static_cast<int>((n + kIdxChunk - 1) >> kChunkShift);
  const int64_t chunk0 = static_cast<int64_t>(row) * a.nch_max;
  const int cnt = tid < nch ? a.ws_count[chunk0 + tid] : 0;
  int total;
  const int off = block_exclusive_scan(cnt, scan, &total);
  const bool over = __syncthreads_or(cnt > kIdxCandCap);
  if (over || total < K || total > kIdxCandCap) {
    topk_by_radix_passes(a, r, s, n, K, out, hist, scan, pick);
    return;
  }
  if (tid < nch) coff[tid] = off;
  __syncthreads();
  // candidate j (position order) is entry j - coff[c] of chunk c, the last chunk with coff[c] <= j
  constexpr int PER = kIdxCandCap / kTopkThreads;
  uint2 x[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int j = tid + u * kTopkThreads;
    if (j < total) {
      int lo = 0, hi = nch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (coff[mid] <= j) lo = mid;
        else hi = mid;
      }
      x[u] = a.ws_cand[(chunk0 + lo) * kIdxCandCap + (j - coff[lo])];
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int j = tid + u * kTopkThreads;
    if (j < total) {
      ck[j] = x[u].x;
      cpos[j] = static_cast<int32_t>(x[u].y);
    }
  }
  __syncthreads();
  const uint32_t T = select_rank(ck, total, K, hist, scan, pick);
  // thread t takes the candidates t R .. t R + R - 1
  const int R = (total + kTopkThreads - 1) / kTopkThreads;
  const int j0 = min(tid * R, total), j1 = min(j0 + R, total);
  int gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    gt += ck[j] > T ? 1 : 0;
    eq += ck[j] == T ? 1 : 0;
  }
  int gt_all, t3;
  block_exclusive_scan(gt, scan, &gt_all);
  const int eq_before = block_exclusive_scan(eq, scan, &t3);
  const int need_eq = K - gt_all;  // tied keys to keep, lowest positions first
  const int take_eq = min(max(need_eq - eq_before, 0), eq);
  int o = block_exclusive_scan(gt + take_eq, scan, &t3);
  int taken = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = ck[j];
    bool keep = u > T;
    if (u == T) {
      keep = taken < take_eq;
      ++taken;
    }
    if (keep) {
      if (o < K) out[o] = static_cast<int32_t>(idx_slot(a, r, cpos[j]));
      ++o;
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
  topk_candidates_kernel<<<dim3(static_cast<unsigned>(a.num_rows), static_cast<unsigned>(a.nch_max)), kTopkThreads, 0,
                           st>>>(a);
  topk_finish_kernel<<<static_cast<unsigned>(a.num_rows), kTopkThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace bsa
