// Generic MFMA tile kernel for BSR block-sparse attention on gfx950.
//
// One workgroup processes one planner tile: up to 32 * NW query rows of one
// (row block, kv head) work unit -- the g qo heads of each query token are
// packed as rows, so grouped-query heads share every K/V load -- against the
// keys of a contiguous range of the row block's column blocks
// (flashinfer.sparse BlockSparseAttentionWrapper: BSR mask, GQA head
// grouping; the key loop is ordinary flash-style online softmax).
//
// Per key tile of KT keys (64, or 128 for 256-row tiles over blocks of a
// multiple of 128 keys):
//   * the K and V rows of the tile are gathered by block index straight into
//     LDS with global_load_lds (16 bytes per lane, each wave instruction
//     filling 1 KB = 4 rows; keys outside a block's valid length, or past the
//     range, read a zero row); the 16-byte chunks of each row are XOR-
//     swizzled by key, each lane fetching the chunk that belongs in its slot.
//     The DMA of tile t+1 lands in the other of two LDS stages while tile t
//     is computed; one wait + barrier per tile;
//   * fp8 e4m3 K/V (KV8; run()'s per-head scale_k / scale_v with FP8 KV):
//     the tile is staged through registers instead -- loaded one tile ahead
//     as 16-byte pieces (16 values), widened exactly to the 16-bit type
//     (every e4m3 value is an fp16 and a bf16 value) and stored into the
//     same swizzled LDS layout at the end of the step, so every later read
//     is unchanged; the dequant scales fold into the logit and output scales;
//   * each wave computes S^T = K Q^T for its 32 rows with
//     v_mfma_f32_32x32x16 (K from LDS as the A operand, Q^T held in
//     registers as B), so every lane owns one query row and its row max
//     needs one cross-half exchange only; K rows enter in an order (bits 2
//     and 3 of the row index swapped) that makes the S^T accumulators line
//     up with the transposed V fragments below;
//   * causal / valid-length masking runs only on tiles that need it, and a
//     wave skips tiles that lie wholly above its causal diagonal;
//   * element masks inside blocks (MASK): the planner's bit planes hold, per
//     row offset in the row block, one bit per key position of the column
//     list; each lane loads the KT + 32 bits around its tile from its row's
//     plane (a funnel shift aligns them) and ANDs them into the score mask;
//   * online softmax in the log2 domain (scale folded into one FMA); the
//     running max only moves when a tile exceeds it by more than 2^8, so
//     the rescale of O is rare (probabilities stay below 256);
//   * O^T += V^T P^T with v_mfma_f32_32x32x16: V^T fragments come straight
//     from the row-major V tile through ds_read_b64_tr_b16, P^T straight
//     from the S^T accumulator registers.
// The result is o = O / l (rounded to the storage type) and
// lse = (m + log2 l) ln 2, or, for a split tile, the fp32 partial (O / l,
// lse) in the workspace for the merge kernel.
#include "device_common.h"
#include "kernels.h"

namespace bsa {

namespace {

constexpr int kD = 128;            // q/k and v/o head dim of this kernel
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may lag behind


typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int KT>
struct TileLds {
  static constexpr int kKBytes = KT * kD * 2;   // K: KT rows of 256 B
  static constexpr int kVBytes = KT * kD * 2;   // V: KT rows of 256 B
};

// LDS layouts for 64 banks x 4 B (a 16-byte-per-lane access is served 16
// lanes at a time, an 8-byte one up to 32 lanes at a time).  Both tiles are
// row-major, 256 B per key, with the 16-byte chunks of a row permuted by an
// XOR (so a DMA that fills 1 KB = 4 rows per wave instruction can place them:
// each lane fetches the chunk that belongs in its slot).  K: the 16 lanes of
// a read phase fetch 16 different rows at one chunk, so the chunk is XORed
// with the row's low 4 bits.  V: a transposing read touches 4 consecutive
// rows x 2 chunks per 16-lane group and a neighbouring group the next 2
// chunks of the same rows, so the chunk is XORed with 4 * (row % 4).
__device__ __forceinline__ int k_swz(int key) { return key & 15; }
__device__ __forceinline__ int v_swz(int key) { return (key & 3) << 2; }
__device__ __forceinline__ int k_off(int key, int c) { return key * 256 + ((c ^ k_swz(key)) << 4); }
__device__ __forceinline__ int v_off(int key, int c) { return key * 256 + ((c ^ v_swz(key)) << 4); }

// S^T row m of a 32-key block holds key swap23(m) (bits 2 and 3 exchanged).
__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <typename T, int NW, int KT, bool CAUSAL, bool LENS, bool BLOCKTILE, bool MASK, bool KV8>
__global__ __launch_bounds__(NW * 64, 2) void attn_tile_kernel(AttnArgs a) {
  using Ops = MfmaType<T>;
  using v8 = typename Ops::v8;
  using v4 = typename Ops::v4;
  using L = TileLds<KT>;
  constexpr int NTHR = NW * 64;
  constexpr int NKB = KT / 32;

  // two LDS stages as separate arrays: the compiler then knows that reading
  // one stage does not depend on the DMA in flight into the other
  __shared__ __attribute__((aligned(16))) unsigned char st0[L::kKBytes + L::kVBytes];
  __shared__ __attribute__((aligned(16))) unsigned char st1[L::kKBytes + L::kVBytes];
  // the key tokens (written by ordinary stores) live apart from the DMA target
  __shared__ __attribute__((aligned(16))) int tk0[KT];
  __shared__ __attribute__((aligned(16))) int tk1[KT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave branches scalar
  const int half = lane >> 5;
  const int ql = lane & 31;

  // read-only tables through the constant address space: their wave-uniform
  // lookups inside the key loop become scalar loads
  const cint32_t* cols = (const cint32_t*)(a.cols);
  const cint32_t* lens = (const cint32_t*)(a.lens);
  const int32_t* trec = a.tiles + static_cast<int64_t>(blockIdx.x) * 8;
  const int I = trec[0];
  const int kvh = trec[1];
  const int row0 = trec[2];
  const int nrows = trec[3];
  const int cb = trec[4];
  const int ce = trec[5];
  const int part = trec[6];
  const int C = a.C;
  const int g = a.group;
  const int nblk = ce - cb;
  const int npos = nblk * C;
  const int ntiles = (npos + KT - 1) / KT;

  // ---- this lane's query row
  const int rloc = wave * 32 + ql;
  const bool row_ok = rloc < nrows;
  const int r = row0 + rloc;
  const int qtok = I * a.R + r / g;
  const int qhead = kvh * g + r % g;
  const int wave_rows = nrows - wave * 32;
  const bool wave_active = wave_rows > 0;
  const int wave_min_tok = I * a.R + (row0 + wave * 32) / g;
  const int wave_max_tok = I * a.R + (row0 + wave * 32 + (wave_rows < 32 ? wave_rows : 32) - 1) / g;
  // key token t is visible to this row iff (unsigned)t < qbound: masked slots
  // carry t = -1, and causal rows see t <= qtok + N - M
  uint32_t qbound = 0x80000000u;
  if (CAUSAL) {
    const int64_t l = static_cast<int64_t>(qtok) + a.causal_off;
    qbound = l >= 0x7fffffff ? 0x80000000u : (l < -1 ? 0u : static_cast<uint32_t>(l + 1));
  }
  const int64_t wave_lim = static_cast<int64_t>(wave_max_tok) + a.causal_off;
  const int64_t wave_lim_lo = static_cast<int64_t>(wave_min_tok) + a.causal_off;

  v8 qf[8];
  if (row_ok) {
    const T* qp = static_cast<const T*>(a.q) + static_cast<int64_t>(qtok) * a.q_stride +
                  static_cast<int64_t>(qhead) * kD + half * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const v8*>(qp + ks * 16);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = v8{};
  }

  TraceAcc tr;  // trace build: column entries and valid keys this thread loaded

  // ---- key tokens.  BLOCKTILE (C a multiple of KT): a key tile lies inside one
  // block, whose id and length are uniform scalar loads.  Otherwise each key
  // looks its block up.  Tiles past the end (only ever loaded, never used)
  // resolve to masked keys.
  struct TileInfo {
    int base;   // token of the tile's first key slot
    int off0;   // offset of that slot inside its block
    int len;    // valid length of the block
  };
  auto tile_info = [&](int kt) {
    TileInfo ti;
    const int t0 = kt * KT;
    int blk = t0 / C;
    blk = blk < nblk ? blk : nblk - 1;
    ti.off0 = t0 - blk * C;
    ti.base = cols[cb + blk] * C + ti.off0;
    ti.len = LENS ? lens[cb + blk] : C;
    return ti;
  };
  // (trace build: tokens outside [0, N) are masked, and counted where `count`: one
  // lane per key)
  auto key_tok = [&](int kt, const TileInfo& ti, int key, bool count = false) -> int {
    const int t = kt * KT + key;
    if (BLOCKTILE) {
      bool ok = t < npos;
      if (LENS) ok = ok && ti.off0 + key < ti.len;
      return tr.check(ok ? ti.base + key : -1, a.num_keys, count);
    } else {
      if (t >= npos) return -1;
      const int blk = t / C;
      const int off = t - blk * C;
      if (LENS && off >= lens[cb + blk]) return -1;
      return tr.check(cols[cb + blk] * C + off, a.num_keys, count);
    }
  };

  constexpr int kElt = KV8 ? 1 : 2;  // bytes per stored K/V value
  const T* kbase = static_cast<const T*>(a.k) + static_cast<int64_t>(kvh) * kD;
  const T* vbase = static_cast<const T*>(a.v) + static_cast<int64_t>(kvh) * kD;
  const T* zrow = static_cast<const T*>(a.zero_row);
  const unsigned char* kbase8 = static_cast<const unsigned char*>(a.k) + static_cast<int64_t>(kvh) * kD * kElt;
  const unsigned char* vbase8 = static_cast<const unsigned char*>(a.v) + static_cast<int64_t>(kvh) * kD * kElt;
  const unsigned char* zrow8 = static_cast<const unsigned char*>(a.zero_row);
  // ---- global -> LDS by DMA (global_load_lds, 16 B per lane): a K or V tile
  // is KT/4 blocks of 1 KB = 4 rows; wave w fills blocks w*BPW .. (w+1)*BPW-1
  // of both.  Lane l of a block serves row 4b + l/16 and slot l%16, i.e. it
  // fetches chunk (l%16) ^ swz(row) of that row.  Masked keys read the zero row.
  constexpr int KBLK = KT / 4;
  constexpr int BPW = KBLK / NW;
  static_assert(KBLK % NW == 0, "DMA blocks per wave");
  auto dma_tile = [&](int kt, unsigned char* st, int* ktok) {
    const TileInfo ti = tile_info(kt);
    const int u = lane & 15;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int b = wave * BPW + j;
      const int row = 4 * b + (lane >> 4);
      const int tok = key_tok(kt, ti, row, u == 0);
      const T* pk = tok >= 0 ? kbase + static_cast<int64_t>(tok) * a.k_stride : zrow;
      const T* pv = tok >= 0 ? vbase + static_cast<int64_t>(tok) * a.v_stride : zrow;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(pk + (u ^ k_swz(row)) * 8),
                                       (__attribute__((address_space(3))) void*)(st + b * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(pv + (u ^ v_swz(row)) * 8),
                                       (__attribute__((address_space(3))) void*)(st + L::kKBytes + b * 1024), 16, 0,
                                       0);
      if (u == 0) {
        ktok[row] = tok;
        if (kTrace && tok >= 0) tr.keys(cb + (kt * KT + row) / C, 1);
      }
    }
  };

  // ---- KV8 staging: a tile's fp8 K (and V) rows are KT x 8 pieces of 16 bytes;
  // thread tid takes pieces tid, tid + NTHR, ... (8 consecutive threads read one
  // 128-byte row), keeps them in registers while the current tile is computed,
  // then widens each piece to two 16-byte chunks of the 16-bit row and stores
  // them where the DMA would have put those chunks.  Masked keys read the zero row.
  constexpr int PPT = KV8 ? KT * 8 / NTHR : 1;  // pieces per thread
  static_assert(!KV8 || (KT * 8) % NTHR == 0, "fp8 pieces per thread");
  u32x4 k8[PPT], v8r[PPT];
  int tok8[PPT];
  auto load8 = [&](int kt) {
    const TileInfo ti = tile_info(kt);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = tid + i * NTHR;
      const int row = piece >> 3;
      const int pc = (piece & 7) * 16;
      const int tok = key_tok(kt, ti, row, (piece & 7) == 0);
      const unsigned char* pk = tok >= 0 ? kbase8 + static_cast<int64_t>(tok) * a.k_stride : zrow8;
      const unsigned char* pv = tok >= 0 ? vbase8 + static_cast<int64_t>(tok) * a.v_stride : zrow8;
      k8[i] = *reinterpret_cast<const u32x4*>(pk + pc);
      v8r[i] = *reinterpret_cast<const u32x4*>(pv + pc);
      tok8[i] = tok;
      if (kTrace && (piece & 7) == 0 && tok >= 0) tr.keys(cb + (kt * KT + row) / C, 1);
    }
  };
  auto store8 = [&](unsigned char* st, int* ktok) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = tid + i * NTHR;
      const int row = piece >> 3;
      const int c = (piece & 7) * 2;  // its two 16-bit chunks
      // pieces 4-7 of a row store their odd chunk first: a ds_write_b128 serves
      // 8 consecutive lanes per pass, conflict-free when their chunks differ mod
      // 8 (measured on gfx950), and chunks 2p, p = 0..7, do so only in pairs
      const bool h = (piece & 4) != 0;
      const u32x2 k0 = h ? u32x2{k8[i][2], k8[i][3]} : u32x2{k8[i][0], k8[i][1]};
      const u32x2 k1 = h ? u32x2{k8[i][0], k8[i][1]} : u32x2{k8[i][2], k8[i][3]};
      const u32x2 v0 = h ? u32x2{v8r[i][2], v8r[i][3]} : u32x2{v8r[i][0], v8r[i][1]};
      const u32x2 v1 = h ? u32x2{v8r[i][0], v8r[i][1]} : u32x2{v8r[i][2], v8r[i][3]};
      const int c0 = c + (h ? 1 : 0), c1 = c + (h ? 0 : 1);
      *reinterpret_cast<u32x4*>(st + k_off(row, c0)) = fp8x8_widen<T>(k0);
      *reinterpret_cast<u32x4*>(st + k_off(row, c1)) = fp8x8_widen<T>(k1);
      *reinterpret_cast<u32x4*>(st + L::kKBytes + v_off(row, c0)) = fp8x8_widen<T>(v0);
      *reinterpret_cast<u32x4*>(st + L::kKBytes + v_off(row, c1)) = fp8x8_widen<T>(v1);
      // the whole-tile path (full blocks, whole key tiles) keeps no token array
      if (!(BLOCKTILE && !LENS))
        if ((piece & 7) == 0) ktok[row] = tok8[i];
    }
  };

  // this lane's element-mask plane (row offset inside the row block; rows past
  // the tile read plane 0 and are never stored)
  const uint32_t* mplane = nullptr;
  if (MASK) mplane = a.mbits + static_cast<int64_t>(row_ok ? qtok - I * a.R : 0) * a.mask_plane_words;
  constexpr int NMW = KT / 32 + 1;  // words covering a tile at any bit offset

  // Full blocks that each hold whole key tiles (BLOCKTILE without lengths):
  // every key of a tile is valid and its tokens are consecutive, so the DMA
  // needs one scalar base per tile plus per-lane byte offsets fixed for the
  // whole loop, blocks advance without a division, and masks follow from the
  // tile's first token (no token array).
  constexpr bool FAST = BLOCKTILE && !LENS;
  uint32_t koff[BPW], voff[BPW];
  if (FAST) {
    const int u = lane & 15;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int row = 4 * (wave * BPW + j) + (lane >> 4);
      koff[j] = static_cast<uint32_t>(row) * static_cast<uint32_t>(a.k_stride * 2) + ((u ^ k_swz(row)) << 4);
      voff[j] = static_cast<uint32_t>(row) * static_cast<uint32_t>(a.v_stride * 2) + ((u ^ v_swz(row)) << 4);
    }
  }
  const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(kbase);
  const unsigned char* vbytes = reinterpret_cast<const unsigned char*>(vbase);
  int dblk = 0, doff = 0;  // block and offset of the next tile to load (FAST)
  // (trace build: a tile whose tokens leave [0, N) counts its KT keys and loads tile 0's
  // rows instead, so no load leaves the cache; this path has no per-key mask)
  auto fast_check = [&](int lo) -> int {
    if (kTrace && (lo < 0 || static_cast<int64_t>(lo) + KT > a.num_keys)) {
      if (tid == 0) tr.bad += KT;
      return 0;
    }
    return lo;
  };
  auto dma_fast = [&](unsigned char* st) -> int {
    if (kTrace && tid == 0) tr.keys(cb + dblk, KT);
    const int lo = fast_check(cols[cb + dblk] * C + doff);
    doff += KT;
    if (doff == C) {
      doff = 0;
      ++dblk;
    }
    const unsigned char* kt = kbytes + static_cast<int64_t>(lo) * (a.k_stride * 2);
    const unsigned char* vt = vbytes + static_cast<int64_t>(lo) * (a.v_stride * 2);
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int b = wave * BPW + j;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(kt + koff[j]),
                                       (__attribute__((address_space(3))) void*)(st + b * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(vt + voff[j]),
                                       (__attribute__((address_space(3))) void*)(st + L::kKBytes + b * 1024), 16, 0,
                                       0);
    }
    return lo;
  };

  // wave-uniform token range of key tile kt (the column list is ascending)
  auto tile_tok_range = [&](int kt, int64_t& lo, int64_t& hi) {
    const int t0 = kt * KT;
    const int t1 = (t0 + KT < npos ? t0 + KT : npos) - 1;
    const int blk0 = t0 / C, blk1 = t1 / C;
    lo = static_cast<int64_t>(cols[cb + blk0]) * C + (t0 - blk0 * C);
    hi = static_cast<int64_t>(cols[cb + blk1]) * C + (t1 - blk1 * C);
  };

  // the eight K fragments of the first 32-key block are read before its
  // products; those of block kb + 1 are read one by one between the products
  // of block kb (each into the register the product before it consumed), so
  // the LDS latency is paid once per tile
  auto qk = [&](const unsigned char* kl, f32x16 (&sacc)[NKB]) {
    v8 kf[NKB][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[0][ks] = *reinterpret_cast<const v8*>(kl + k_off(swap23(ql), 2 * ks + half));
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sacc[kb] = Ops::mfma32(kf[kb][ks], qf[ks], sacc[kb]);
        if (kb + 1 < NKB)
          kf[kb + 1][ks] = *reinterpret_cast<const v8*>(kl + k_off((kb + 1) * 32 + swap23(ql), 2 * ks + half));
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // block 0's reads
#pragma unroll
    for (int kb = 0; kb + 1 < NKB; ++kb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a product of block kb
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a read of block kb + 1
      }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // the last block's products
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  // logit scale of this lane's row (run()'s per-head scales multiply the plan's)
  float sl2 = a.scale_log2;
  if (a.q_scale) sl2 *= a.q_scale[qhead];
  if (a.k_scale) sl2 *= a.k_scale[kvh];
  const float out_scale = a.v_scale ? a.out_scale * a.v_scale[kvh] : a.out_scale;

  // element mask: bits mw[0..NMW) of this row's plane start at bit `sh` of mw[0]
  auto mask_bits = [&](const uint32_t (&mw)[NMW], int sh, f32x16 (&sacc)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // the 32 keys of block kb; this lane's keys sit 8*half further up
      const uint64_t pair = (static_cast<uint64_t>(mw[kb + 1]) << 32) | mw[kb];
      const uint32_t w = static_cast<uint32_t>(pair >> sh) >> (8 * half);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int b = 16 * (g4 >> 1) + 4 * (g4 & 1) + e;
          sacc[kb][g4 * 4 + e] = (w >> b) & 1u ? sacc[kb][g4 * 4 + e] : -INFINITY;
        }
    }
  };
  // causal / length mask of S (only on tiles that need it), and the element mask
  auto mask_scores = [&](bool need_mask, const int* ktok, const uint32_t (&mw)[NMW], int sh,
                         f32x16 (&sacc)[NKB]) {
    if (!need_mask) return;
    // value 4*g4 + e of this lane is S^T row 8*g4 + 4*half + e, i.e. key
    // 16*(g4/2) + 8*half + 4*(g4%2) + e of the block
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int4 tk = *reinterpret_cast<const int4*>(ktok + kb * 32 + 16 * (g4 >> 1) + 8 * half + 4 * (g4 & 1));
        const uint32_t tt[4] = {static_cast<uint32_t>(tk.x), static_cast<uint32_t>(tk.y),
                                static_cast<uint32_t>(tk.z), static_cast<uint32_t>(tk.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[kb][g4 * 4 + e] = tt[e] < qbound ? sacc[kb][g4 * 4 + e] : -INFINITY;
      }
    }
    if (MASK) mask_bits(mw, sh, sacc);
  };
  // FAST causal mask: key idx of the tile is visible iff idx <= qtok + N - M - lo
  auto mask_fast = [&](int lo, f32x16 (&sacc)[NKB]) {
    const int limh = qtok + a.causal_off - lo - 8 * half;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = kb * 32 + 16 * (g4 >> 1) + 4 * (g4 & 1) + e;
          sacc[kb][g4 * 4 + e] = c <= limh ? sacc[kb][g4 * 4 + e] : -INFINITY;
        }
  };
  // scores -> probabilities with a lagging running max (branch-free, so it can
  // be interleaved with the next tile's QK^T); `live` = false leaves the running
  // state untouched.  Returns alpha; sets `upd` when the running max moved.
  // probabilities of the current tile, rounded to the storage type, in pairs
  // (pair j of block kb = S^T values 2j, 2j+1 of this lane)
  typedef T T2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  constexpr bool kIsHalf = sizeof(T) == 2 && static_cast<T>(1.0009765625f) != static_cast<T>(1.f);
  T2 pp[NKB][8];
  auto softmax_core = [&](f32x16 (&sacc)[NKB], bool live, bool& upd) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = max_xor32(mx);
    const float mt = mx * sl2;
    upd = live && mt > m_run + kRescaleSlack;
    const float m_new = upd ? mt : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float p0 = fast_exp2(fmaf(sacc[kb][v], sl2, -m_use));
        const float p1 = fast_exp2(fmaf(sacc[kb][v + 1], sl2, -m_use));
        T2 pr;
        pr[0] = static_cast<T>(p0);
        pr[1] = static_cast<T>(p1);
        pp[kb][v >> 1] = pr;
        // fp16: the row sum adds exactly the rounded probabilities the PV
        // product uses (one dot2 per pair); bf16 rounding is too coarse for
        // the sum, which stays in fp32
        if (kIsHalf) ls = __builtin_amdgcn_fdot2(bitcast<h2>(pr), h2{1, 1}, ls, false);
        else ls += p0 + p1;
      }
    m_run = m_new;
    l_run = live ? l_run * alpha + ls : l_run;
    return alpha;
  };

  // lane -> transposed-read coordinates (16-lane group G, lane L within it)
  const int G = lane >> 4;
  const int Lg = lane & 15;
  const int vrow = 8 * half + (Lg >> 2);          // + ks*16 + 4*j
  const int vdim = 16 * (G & 1) + 4 * (Lg & 3);   // + db*32
  auto pv = [&](const unsigned char* st, const f32x16 (&sacc)[NKB]) {
    const unsigned char* vl = st + L::kKBytes;
    // k-step ks covers keys ks*16 .. +16: lane half h holds keys ks*16 + 8h + e
    // (e = 0..7), from S^T values hv*8 + e of block ks/2
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      const int kb = ks >> 1;
      const int hv = ks & 1;
      v8 pf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pf[2 * j] = pp[kb][hv * 4 + j][0];
        pf[2 * j + 1] = pp[kb][hv * 4 + j][1];
      }
      const int row = ks * 16 + vrow;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + vdim;
        const int boff = (d & 7) * 2;
        const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vl + v_off(row, d >> 3) + boff));
        const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vl + v_off(row + 4, d >> 3) + boff));
        const v8 vf = __builtin_shufflevector(bitcast<v4>(lo), bitcast<v4>(hi), 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = Ops::mfma32(vf, pf, oacc[db]);
      }
    }
  };

  // element-mask words of key tile t (positions cb*C + t*KT ..); returns the bit offset
  auto load_mask_words = [&](int t, uint32_t (&mw)[NMW]) -> int {
    if (!MASK) {
#pragma unroll
      for (int i = 0; i < NMW; ++i) mw[i] = 0u;
      return 0;
    }
    const int64_t p0 = static_cast<int64_t>(cb) * C + static_cast<int64_t>(t) * KT;
    const uint32_t* src = mplane + (p0 >> 5);
#pragma unroll
    for (int i = 0; i < NMW; ++i) mw[i] = src[i];
    return static_cast<int>(p0 & 31);
  };

  // ---- key loop: two LDS stages, one barrier per tile; the DMA of tile t+1
  // is in flight while tile t is computed
  auto step = [&](int t, unsigned char* cur, const int* curtok, unsigned char* nxt, int* nxttok) {
    if (!KV8) __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMA into `cur` has landed
    __syncthreads();                     // ... and every other wave's (KV8: their stores)
    // every scalar table read of the iteration happens here, before the LDS
    // math: an outstanding scalar load would turn each LDS wait into a full
    // drain (both share one counter)
    int64_t lo = 0, hi = 0;
    if (CAUSAL) tile_tok_range(t, lo, hi);
    // this tile's mask words, loaded ahead of the next tile's DMA so that
    // waiting for them does not wait for that DMA
    uint32_t mw[NMW];
    const int sh = load_mask_words(t, mw);
    if (t + 1 < ntiles) {
      if (KV8) load8(t + 1);
      else dma_tile(t + 1, nxt, nxttok);
    }
    // tiles above this wave's diagonal are skipped
    if (wave_active && !(CAUSAL && lo > wave_lim)) {
      const bool need_mask = MASK || LENS || (t * KT + KT > npos) || (CAUSAL && hi > wave_lim_lo);
      f32x16 sc[NKB];
      qk(cur, sc);
      mask_scores(need_mask, curtok, mw, sh, sc);
      bool upd;
      const float alpha = softmax_core(sc, true, upd);
      if (__ballot(upd) != 0) {
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      }
      pv(cur, sc);
    }
    if (KV8 && t + 1 < ntiles) store8(nxt, nxttok);
  };
  int lo_next = 0;  // first token of the tile in flight (FAST)
  // FAST + KV8: the tile's first token, then fixed per-thread byte offsets
  uint32_t koff8[PPT], voff8[PPT];
  if (FAST && KV8) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = tid + i * NTHR;
      koff8[i] = static_cast<uint32_t>(piece >> 3) * static_cast<uint32_t>(a.k_stride) + (piece & 7) * 16;
      voff8[i] = static_cast<uint32_t>(piece >> 3) * static_cast<uint32_t>(a.v_stride) + (piece & 7) * 16;
    }
  }
  auto load8_fast = [&]() -> int {
    if (kTrace && tid == 0) tr.keys(cb + dblk, KT);
    const int lo = fast_check(cols[cb + dblk] * C + doff);
    doff += KT;
    if (doff == C) {
      doff = 0;
      ++dblk;
    }
    const unsigned char* kt = kbase8 + static_cast<int64_t>(lo) * a.k_stride;
    const unsigned char* vt = vbase8 + static_cast<int64_t>(lo) * a.v_stride;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      k8[i] = *reinterpret_cast<const u32x4*>(kt + koff8[i]);
      v8r[i] = *reinterpret_cast<const u32x4*>(vt + voff8[i]);
    }
    return lo;
  };
  auto step_fast = [&](int t, unsigned char* cur, unsigned char* nxt) {
    if (!KV8) __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMA into `cur` has landed
    __syncthreads();                     // ... and every other wave's (KV8: their stores)
    const int lo = lo_next;
    uint32_t mw[NMW];
    const int sh = load_mask_words(t, mw);
    if (t + 1 < ntiles) lo_next = KV8 ? load8_fast() : dma_fast(nxt);
    // tiles above this wave's diagonal are skipped
    if (wave_active && !(CAUSAL && lo > wave_lim)) {
      f32x16 sc[NKB];
      qk(cur, sc);
      if (CAUSAL && static_cast<int64_t>(lo) + (KT - 1) > wave_lim_lo) mask_fast(lo, sc);
      if (MASK) mask_bits(mw, sh, sc);
      bool upd;
      const float alpha = softmax_core(sc, true, upd);
      if (__ballot(upd) != 0) {
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      }
      pv(cur, sc);
    }
    if (KV8 && t + 1 < ntiles) store8(nxt, nullptr);
  };
  if (ntiles > 0) {
    if (FAST) {
      if (KV8) {
        lo_next = load8_fast();
        store8(st0, nullptr);
      } else {
        lo_next = dma_fast(st0);
      }
      for (int t = 0; t < ntiles; t += 2) {
        step_fast(t, st0, st1);
        if (t + 1 < ntiles) step_fast(t + 1, st1, st0);
      }
    } else {
      if (KV8) {
        load8(0);
        store8(st0, tk0);
      } else {
        dma_tile(0, st0, tk0);
      }
      for (int t = 0; t < ntiles; t += 2) {
        step(t, st0, tk0, st1, tk1);
        if (t + 1 < ntiles) step(t + 1, st1, tk1, st0, tk0);
      }
    }
  }

  trace_flush(a.trace, blockIdx.x, tr, tid == 0, part, kvh, row0, nrows);

  // ---- finalize this lane's row
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? out_scale / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (!row_ok) return;
  if (part < 0) {
    T* op = static_cast<T*>(a.o) + static_cast<int64_t>(qtok) * a.o_stride + static_cast<int64_t>(qhead) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        v4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(oacc[db][g4 * 4 + e] * inv);
        *reinterpret_cast<v4*>(op + db * 32 + 8 * g4 + 4 * half) = out;
      }
    if (half == 0 && a.lse) a.lse[static_cast<int64_t>(qtok) * a.num_qo_heads + qhead] = lse_v;
  } else {
    float* pp = a.part + part;
    float* po = pp + static_cast<int64_t>(rloc) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = oacc[db][g4 * 4 + e] * inv;
        *reinterpret_cast<f32x4*>(po + db * 32 + 8 * g4 + 4 * half) = out;
      }
    if (half == 0) pp[static_cast<int64_t>(nrows) * kD + rloc] = lse_v;
  }
}

template <typename T, int NW, int KT, bool KV8>
hipError_t launch_variant(const AttnArgs& a, bool causal, bool lens, bool mask, hipStream_t st) {
  const dim3 grid(a.num_tiles), block(NW * 64);
  // block tiles also need every row offset of a tile (KT rows) to fit 31 bits
  const int64_t max_stride = a.k_stride > a.v_stride ? a.k_stride : a.v_stride;
  const bool bt = a.C % KT == 0 && static_cast<int64_t>(KT) * 2 * max_stride < (int64_t{1} << 31);
  // element masks come without block lengths (the planner folds neither in)
  if (mask && (lens || !a.mbits || a.mask_plane_words < 1)) return hipErrorInvalidValue;
#define BSA_TILE_LAUNCH(CA, LE)                                                                  \
  if (bt) attn_tile_kernel<T, NW, KT, CA, LE, true, false, KV8><<<grid, block, 0, st>>>(a);      \
  else attn_tile_kernel<T, NW, KT, CA, LE, false, false, KV8><<<grid, block, 0, st>>>(a);
#define BSA_TILE_LAUNCH_MASK(CA)                                                                 \
  if (bt) attn_tile_kernel<T, NW, KT, CA, false, true, true, KV8><<<grid, block, 0, st>>>(a);    \
  else attn_tile_kernel<T, NW, KT, CA, false, false, true, KV8><<<grid, block, 0, st>>>(a);
  if (mask) {
    // masked plans run 64-key tiles (the mask words of 128-key ones spill)
    if constexpr (KT == 128) return hipErrorInvalidValue;
    else if (causal) { BSA_TILE_LAUNCH_MASK(true) } else { BSA_TILE_LAUNCH_MASK(false) }
  } else if (causal) {
    if (lens) { BSA_TILE_LAUNCH(true, true) } else { BSA_TILE_LAUNCH(true, false) }
  } else {
    if (lens) { BSA_TILE_LAUNCH(false, true) } else { BSA_TILE_LAUNCH(false, false) }
  }
#undef BSA_TILE_LAUNCH
#undef BSA_TILE_LAUNCH_MASK
  return hipGetLastError();
}

template <typename T, bool KV8>
hipError_t launch_typed(const AttnArgs& a, int tile_rows, bool causal, bool lens, bool mask, hipStream_t st) {
  switch (tile_rows) {
    case 32: return launch_variant<T, 1, 32, KV8>(a, causal, lens, mask, st);
    case 128: return launch_variant<T, 4, 64, KV8>(a, causal, lens, mask, st);
    case 256:
      // 128-key tiles (two 64 KB LDS stages) when every tile lies in one block; fp8
      // staging keeps 64-key tiles (the registers of the 128-key variant are full)
      if constexpr (!KV8)
        if (a.C % 128 == 0 && !mask) return launch_variant<T, 8, 128, false>(a, causal, lens, mask, st);
      return launch_variant<T, 8, 64, KV8>(a, causal, lens, mask, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_tile(const AttnArgs& a, bool bf16, bool kv8, int tile_rows, bool causal, bool has_lens,
                            bool has_mask, hipStream_t stream) {
  if (a.num_tiles == 0) return hipSuccess;
  if (kv8)
    return bf16 ? launch_typed<__bf16, true>(a, tile_rows, causal, has_lens, has_mask, stream)
                : launch_typed<_Float16, true>(a, tile_rows, causal, has_lens, has_mask, stream);
  return bf16 ? launch_typed<__bf16, false>(a, tile_rows, causal, has_lens, has_mask, stream)
              : launch_typed<_Float16, false>(a, tile_rows, causal, has_lens, has_mask, stream);
}

}  // namespace bsa
