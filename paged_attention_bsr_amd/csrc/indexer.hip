// Sparse-attention indexer on gfx950: FP32 scores of query rows against their
// request's paged keys, then each row's exact Top-K keys (flashinfer.sparse
// 0.7.4, "SDSA Indexer": indexer_scores, top_k_from_candidates; one query
// head, no head weights).  Its output -- int32 physical cache rows -- is the
// index list that index-selected sparse MLA decode consumes.
//
// Scores: a workgroup takes one request (grid x) and 256 of its key positions
// (grid y; four waves of 64): it loads the keys once and runs the request's
// query rows against them 16 at a time.  The dot products run on
// v_mfma_f32_16x16x32 with the query rows as the A operand (lane l: row
// l % 16, dims 8 (l / 16) .. + 7 of the k-step) and the keys as B (the same
// dims of key l % 16), so lane l ends with rows 4 (l / 16) + v of key l % 16
// and the 16 lanes of a group store 16 consecutive scores of one row.  Key
// rows are fetched through the block table with 16-byte loads; a page id
// outside the cache reads as a zero key.
//
// Top-K: one workgroup per row.  A score maps to an unsigned key that orders
// like the float (sign bit flipped for positives, all bits for negatives;
// -0 becomes +0).  One pass over the row builds a histogram of the keys' top
// 11 bits and locates the bin of the K-th largest key.  A second pass, each
// wave over its own segment of the row, counts the keys of the bins above
// (kept outright) and collects the bin's keys with their positions into LDS
// (the candidates).  One wave then finds, among the candidates, the exact
// K-th largest key T by radix passes over its remaining bits and, when not all
// keys equal to T are kept, the position of the last one kept (ties to the
// lower position).  Each wave adds its kept candidates to its count, takes
// its offset from the waves before it, and writes its kept positions' cache
// rows in position order, 256 positions per step by ballot.  A bin with more
// keys than the candidate buffer holds (heavy ties) takes a slower path: four
// 8-bit radix passes over the row and per-thread segments for the output.
// The passes over the row keep four independent 16-byte loads in flight per
// thread.
#include "device_common.h"
#include "indexer.h"

namespace bsa {

namespace {

constexpr int kRowsPerGroup = 16;
constexpr int kKeysPerWg = 256;
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
  const int r = blockIdx.x;
  const int rb = a.req_row_ptr[r];
  const int re = min(a.req_row_ptr[r + 1], a.num_rows);
  if (rb >= re) return;
  const int64_t kv_len = a.req_kv_len[r];
  const int64_t p_wg = static_cast<int64_t>(blockIdx.y) * kKeysPerWg;
  if (p_wg >= kv_len || p_wg >= a.max_ctx) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int quad = lane >> 4;

  // B: this wave's four 16-key blocks, loaded once for every row group of the request
  constexpr int KB = 4;
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
  // A: the request's query rows, 16 at a time (rows past the request read its first row:
  // their results are never stored)
#pragma unroll 1
  for (int row0 = rb; row0 < re; row0 += kRowsPerGroup) {
    const int nrows = min(re - row0, kRowsPerGroup);
    const T* qp = static_cast<const T*>(a.q) + static_cast<int64_t>(row0 + (c16 < nrows ? c16 : 0)) * a.q_stride +
                  quad * 8;
    v8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const v8*>(qp + ks * 32);
    f32x4 acc[KB];
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
      float* sp = a.scores + static_cast<int64_t>(row) * a.ld_scores;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int64_t p = p_wg + wave * 64 + kb * 16 + c16;
        if (p < n) sp[p] = acc[kb][v];
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

// Top-K of one row by four 8-bit radix passes over the scores in global
// memory and per-thread contiguous segments for the ordered output (the
// fallback when the bin of the K-th score is too full to collect in LDS).
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
    // the digit d whose bin holds the need-th largest key: the count of keys in
    // the bins above d (thread 255 - d's exclusive prefix over the bins taken
    // from the top) is below need and reaches it with bin d
    if (tid == 0) {
      pick[0] = 0;
      pick[1] = need;
    }
    {
      const int d = 255 - tid;
      const int h = tid < 256 ? hist[d] : 0;
      int tot;
      const int above = block_exclusive_scan(h, scan, &tot);
      if (tid < 256 && above < need && above + h >= need) {
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

constexpr int kTopBits = 11;              // histogram of the top 11 key bits
constexpr int kBins = 1 << kTopBits;
constexpr int kCand = 4096;               // candidates collected in LDS
constexpr int kUnroll = 4;                // independent 16-byte loads in flight per thread
constexpr int kBtCap = 4096;              // block-table entries staged in LDS for the output

__global__ __launch_bounds__(kTopkThreads) void indexer_topk_kernel(IndexerArgs a) {
  __shared__ int hist[kBins];
  __shared__ uint32_t cu[kCand];          // candidates: keys of the bin of the K-th largest key ...
  __shared__ int32_t cp[kCand];           // ... and their positions
  __shared__ int h256[256];               // wave 0's radix histograms over the candidates
  __shared__ int scan[kTopkThreads];
  __shared__ int pick[4];
  __shared__ int seg[2 * (kTopkThreads / 64)];  // per wave: keys above the bin, then kept keys
  __shared__ uint32_t sel_key[1];
  __shared__ int64_t sel_pos[1];
  __shared__ int32_t btl[kBtCap];         // the row's pages (rows that need at most kBtCap of them)
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const float* s = a.scores + static_cast<int64_t>(row) * a.ld_scores;
  const f32x4* s4 = reinterpret_cast<const f32x4*>(s);  // rows are 256-byte aligned
  const int64_t n4 = (n + 3) / 4;                       // 16-byte groups (the row is padded past n)
  // the pages of positions 0 .. n - 1, staged for the output's slot lookups (-1: no page)
  const int64_t npg = (n + a.page_size - 1) / a.page_size;
  const bool bt_lds = npg <= kBtCap;
  if (bt_lds)
    for (int i = tid; i < npg; i += kTopkThreads)
      btl[i] = i < a.max_pages ? a.block_table[static_cast<int64_t>(r) * a.max_pages + i] : -1;
  auto slot_of = [&](int64_t pos) -> int32_t {
    if (!bt_lds) return static_cast<int32_t>(idx_slot(a, r, pos));
    const uint32_t pi = page_of(a, static_cast<uint32_t>(pos));
    const int32_t page = btl[pi];
    const int64_t slot = static_cast<int64_t>(page) * a.page_size + (pos - static_cast<int64_t>(pi) * a.page_size);
    return (page < 0 || slot >= a.num_slots) ? -1 : static_cast<int32_t>(slot);
  };

  // (1) histogram of the top bits; kUnroll 16-byte loads per thread in flight
  for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
  __syncthreads();
  for (int64_t g0 = tid; g0 < n4; g0 += kTopkThreads * kUnroll) {
    f32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t g = g0 + j * kTopkThreads;
      v[j] = s4[g < n4 ? g : 0];
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * (g0 + j * kTopkThreads) + e < n) atomicAdd(&hist[score_key(v[j][e]) >> (32 - kTopBits)], 1);
  }
  __syncthreads();
  // (2) the bin of the K-th largest key: thread t sums bins kBins-1-BPT t .. (from the top),
  // a scan gives the count above its first bin, and the thread walks its bins
  constexpr int BPT = kBins / kTopkThreads;
  {
    int h[BPT], sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      h[j] = hist[kBins - 1 - (tid * BPT + j)];
      sum += h[j];
    }
    int tot;
    int above = block_exclusive_scan(sum, scan, &tot);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (above < K && above + h[j] >= K) {
        pick[0] = kBins - 1 - (tid * BPT + j);
        pick[1] = K - above;   // keys to take from that bin
        pick[2] = h[j];        // keys in that bin
      }
      above += h[j];
    }
  }
  if (tid == 0) pick[3] = 0;
  __syncthreads();
  const uint32_t bin = static_cast<uint32_t>(pick[0]);
  const int need = pick[1];
  const int in_bin = pick[2];
  if (in_bin > kCand) {
    topk_by_radix_passes(a, r, s, n, K, out, hist, scan, pick);
    return;
  }
  // (3) wave w owns the 16-byte groups [w n4 / NWV, (w + 1) n4 / NWV): it counts its keys in the
  // bins above `bin` (kept outright) and collects the bin's keys with their positions
  constexpr int NWV = kTopkThreads / 64;
  const int64_t gb = n4 * wave / NWV, ge = n4 * (wave + 1) / NWV;
  int above_w = 0;
  for (int64_t g0 = gb + lane; g0 < ge; g0 += 64 * kUnroll) {
    f32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t g = g0 + j * 64;
      v[j] = s4[g < ge ? g : gb];
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t g = g0 + j * 64;
        const int64_t i = 4 * g + e;
        const uint32_t u = score_key(v[j][e]);
        const uint32_t hb = u >> (32 - kTopBits);
        if (g < ge && i < n) {
          above_w += hb > bin ? 1 : 0;
          if (hb == bin) {
            const int c = atomicAdd(&pick[3], 1);
            if (c < kCand) {
              cu[c] = u;
              cp[c] = static_cast<int32_t>(i);
            }
          }
        }
      }
  }
  for (int off = 32; off > 0; off >>= 1) above_w += __shfl_xor(above_w, off);
  if (lane == 0) seg[wave] = above_w;
  __syncthreads();
  // (4) wave 0 finds, among the candidates, the need-th largest key T (three 7-bit radix passes
  // over the bits below the bin's) and, when not every key equal to T is kept, the position of
  // the last one kept (three 8-bit passes over the tied keys' positions, smallest first)
  if (wave == 0) {
    const int c = in_bin;
    uint32_t pre = bin << (32 - kTopBits), msk = ~0u << (32 - kTopBits);
    int nd = need;
    // the digit (of 2^bits bins) holding the nd-th key counted from the top (desc) or bottom
    auto select_digit = [&](int bits, bool desc, int& nd_io) -> int {
      const int nb = 1 << bits;
      const int per = nb / 64;
      int hv[4], sum = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < per) {
          const int b = desc ? nb - 1 - (lane * per + k) : lane * per + k;
          hv[k] = h256[b];
          sum += hv[k];
        } else {
          hv[k] = 0;
        }
      }
      int incl = sum;
      for (int off = 1; off < 64; off <<= 1) {
        const int x = __shfl_up(incl, off);
        if (lane >= off) incl += x;
      }
      int below = incl - sum, digit = -1, rest = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < per && digit < 0 && below < nd_io && below + hv[k] >= nd_io) {
          digit = desc ? nb - 1 - (lane * per + k) : lane * per + k;
          rest = nd_io - below;
        }
        below += hv[k];
      }
      const uint64_t who = __ballot(digit >= 0);
      const int src = __ffsll(static_cast<unsigned long long>(who)) - 1;
      nd_io = __shfl(rest, src);
      return __shfl(digit, src);
    };
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = 14 - 7 * pass;
      h256[lane] = 0;
      h256[lane + 64] = 0;
      for (int j = lane; j < c; j += 64) {
        const uint32_t u = cu[j];
        if ((u & msk) == pre) atomicAdd(&h256[(u >> shift) & 127], 1);
      }
      const int d = select_digit(7, true, nd);
      pre |= static_cast<uint32_t>(d) << shift;
      msk |= 127u << shift;
    }
    const uint32_t T = pre;
    // ties at T: keep the nd of them with the lowest positions
    int ties = 0;
    for (int j = lane; j < c; j += 64) ties += cu[j] == T ? 1 : 0;
    for (int off = 32; off > 0; off >>= 1) ties += __shfl_xor(ties, off);
    int64_t p_last = 0x7fffffffffffffffll;
    if (nd < ties) {
      uint32_t ppre = 0, pmsk = 0;
#pragma unroll 1
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = 16 - 8 * pass;
#pragma unroll
        for (int k = 0; k < 4; ++k) h256[lane + 64 * k] = 0;
        for (int j = lane; j < c; j += 64) {
          const uint32_t pj = static_cast<uint32_t>(cp[j]);
          if (cu[j] == T && (pj & pmsk) == ppre) atomicAdd(&h256[(pj >> shift) & 255], 1);
        }
        const int d = select_digit(8, false, nd);
        ppre |= static_cast<uint32_t>(d) << shift;
        pmsk |= 255u << shift;
      }
      p_last = ppre;
    }
    if (lane == 0) {
      sel_key[0] = T;
      sel_pos[0] = p_last;
    }
  }
  __syncthreads();
  const uint32_t T = sel_key[0];
  const int64_t p_last = sel_pos[0];
  auto kept = [&](float v, int64_t i) {
    const uint32_t u = score_key(v);
    return i < n && (u > T || (u == T && i <= p_last));
  };
  // (5) each wave's kept count: its keys above the bin plus its kept candidates; offsets in wave order
  {
    int kc = 0;
    for (int j = lane; j < in_bin; j += 64) {
      const int64_t pj = cp[j];
      const uint32_t u = cu[j];
      if (pj >= 4 * gb && pj < 4 * ge && (u > T || (u == T && pj <= p_last))) ++kc;
    }
    for (int off = 32; off > 0; off >>= 1) kc += __shfl_xor(kc, off);
    if (lane == 0) seg[NWV + wave] = seg[wave] + kc;
  }
  __syncthreads();
  int o = 0;
  for (int w = 0; w < wave; ++w) o += seg[NWV + w];
  // (6) ordered output, 256 positions per step: lane l's four keys 4 l + e rank after the kept
  // keys of the lanes below it (one ballot per e) and after its own kept keys e' < e
  for (int64_t g0 = gb; g0 < ge; g0 += 64 * kUnroll) {
    f32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t g = g0 + j * 64 + lane;
      v[j] = s4[g < ge ? g : gb];
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t g = g0 + j * 64 + lane;
      bool keep[4];
      int below = 0, step = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        keep[e] = g < ge && kept(v[j][e], 4 * g + e);
        const uint64_t bal = __ballot(keep[e]);
        below += __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                           __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
        step += __popcll(bal);
      }
      int mine = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (keep[e] && o + below + mine < K) out[o + below + mine] = slot_of(4 * g + e);
        mine += keep[e] ? 1 : 0;
      }
      o += step;
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
  indexer_topk_kernel<<<a.num_rows, kTopkThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace bsa
