// Sparse-MLA attention kernel on gfx950: BSR with R = 1, one shared latent
// KV head stored as OCP fp8 e4m3 rows of 576 values (512 latent + 64 rope),
// V = the first 512 values of each row, bf16 queries and outputs
// (MATE sparse_mla_fp8_decode / FlashInfer MLA decode conventions: 576-wide
// query and cache rows, indices shared by all heads, bf16 out, fp32 lse;
// per-tensor scales folded as bmm1 = sm_scale * q_descale * k_descale and
// bmm2 = v_descale).
//
// The work is two dense products per query token (S = Q K^T over 576 dims,
// O = P V over 512), so it is shaped around operand reuse: every 16-byte
// fragment a wave reads from LDS feeds two MFMAs, because each wave holds 32
// heads' operands in registers (Q^T for QK^T, P^T for PV).  One workgroup =
// one planner tile = 64 heads of one query token, 4 waves (one per SIMD, so
// a wave may hold Q of 32 heads x 576 dims and O of 32 heads x 256 dims):
// wave (hg, hf) serves heads 32 hg .. 32 hg + 31.  Per key tile of 32 keys:
//   * the selected fp8 rows are gathered with 16-byte loads two tiles ahead
//     (the per-key index one tile ahead of its use), widened exactly to bf16
//     (every e4m3 value is a bf16 value; the dequant scales are applied to
//     the logits and the output instead) and stored as row-major bf16 rows
//     with XOR-swizzled 16-byte units into the LDS buffer of the next tile
//     while this tile is computed.  The same rows serve as K and, through
//     their first 512 values, as V: there is no separate V tile;
//   * wave (hg, hf) computes the part of S^T = K Q^T over dims 288 hf ..
//     288 hf + 287 for all 32 keys of the tile and its 32 heads with
//     v_mfma_f32_16x16x32_bf16 (its half of Q^T resident in registers); the
//     pair (hg, 0), (hg, 1) swaps the fp32 partial scores through LDS and adds
//     them, both run the same softmax step (log2 domain, probabilities
//     against a fixed reference per row, so O is never rescaled inside the
//     loop) on all 32 keys, and wave (hg, hf) accumulates O^T += V^T P^T for
//     value dims 256 hf .. 256 hf + 255.  P^T is the S^T accumulator itself
//     (rounded to bf16; the row sum l keeps the unrounded fp32
//     probabilities): lane (head col, quad) holds keys 4 quad + v and
//     16 + 4 quad + v, and the V^T fragments are read from the row-major tile
//     by ds_read_b64_tr_b16 in that same key order.
// The two 64-head tiles of a token are dealt to workgroups that the hardware
// places on the same XCD (workgroups go to XCDs round-robin), so the second
// gather of each row is served by that XCD's L2.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace bsa {

namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kKT = 32;
constexpr int kNW = 4;                 // waves: 2 head groups x 2
constexpr int kThreads = kNW * 64;
constexpr int kUnits = kDqk / 16;      // 16-byte fp8 units per cache row (36)
constexpr int kLdRounds = 5;           // gather rounds per thread (8 units per round per key)
// A row's probabilities are taken against a fixed reference: the maximum of
// its first tile with a visible key.  A later tile may exceed it by up to
// kOverflowLog2 (probabilities up to 2^64: exact enough in bf16, and the fp32
// sums stay far from overflow); a tile beyond that flags the workgroup, which
// then runs its key loop a second time against each row's true maximum.
constexpr float kOverflowLog2 = 64.f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct MlaLds {
  // 1152 B of bf16 per key (72 16-byte units, no padding)
  static constexpr int kKRow = kDqk * 2;
  static constexpr int kKBytes = kKT * kKRow;
  static constexpr int kTokBytes = kKT * 4;
  static constexpr int kBuf = kKBytes + kTokBytes;
  // stores of the round past a row's 36 units (waves 2, 3) go here: 2 x 128 lanes x 16 B
  static constexpr int kDummy = 2 * 128 * 16;
  // partial-score exchange: per wave 4 planes of [64 lanes] x 16 B (a plane
  // per (key block, head block) accumulator), so 16 lanes of a pass touch 256
  // contiguous bytes
  static constexpr int kXsWave = 4 * 64 * 16;
  static constexpr int kXsBytes = kNW * kXsWave;
};

// Two OCP e4m3 bytes (the selected 16-bit half of `w`) -> two bf16 values
// packed in one dword, low value in the low half, with gfx950's direct scaled
// conversion at scale 1.0 (exact: every e4m3 value is a bf16 value).
// (Reinterpreting the second float of v_cvt_pk_f32_fp8's result as bits was
// miscompiled by this toolchain -- element 1 came back as a copy of element 0
// -- so the f32 round trip is avoided.)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Unit u of key k's row sits at unit u ^ kx(k), kx(k) = k & 7, so the XOR
// stays inside an aligned group of 8 units.  LDS has 64 banks of 4 B; a row is
// 72 units of 16 B, so even keys start at bank 0 and odd keys at bank 32.
// Measured on gfx950 (SQ_LDS_BANK_CONFLICT): a ds_write_b128 serves 8
// consecutive lanes per pass and is conflict-free when their units differ mod
// 8; a ds_read_b128 serves 16 lanes per pass, lanes 0-7 of one quad (16-lane
// group) with lanes 8-15 of another, and is conflict-free when their units
// differ mod 16.  Then
//   * the tile stores (8 consecutive keys at one unit) hit units U ^ k mod 8:
//     all different;
//   * the QK reads (lane (col, quad) at key col, unit B + quad): keys of one
//     quad hit different units; for keys c < 8 of one quad and d >= 8 of the
//     quad read with it, both even or both odd (else their rows start in
//     different bank halves), the units differ because (c ^ d) & 7 is even
//     while quad ^ quad' is odd (1 or 3 for the quads read together);
//   * a transposed read (32 lanes x 8 B per pass: 8 consecutive keys 8p ..
//     8p + 7, each at the two units 2m, 2m + 1 before the XOR) hits 8
//     different aligned unit pairs: bit 0 of the key picks the bank half,
//     bits 1 and 2 (kx bits 1 and 2) the pair; kx bit 0 only swaps the two
//     units of a pair.
__device__ __forceinline__ int kx(int key) { return key & 7; }
__device__ __forceinline__ int k_off(int key, int u) { return key * MlaLds::kKRow + ((u ^ kx(key)) << 4); }

// Workgroup -> tile: within each run of 16 workgroups, b and b + 8 (which the
// hardware places on one XCD) take tiles 2p and 2p + 1, the two head halves
// of one token in the planner's order; a ragged tail maps to itself.
__device__ __forceinline__ int xcd_paired_tile(int b, int num_tiles) {
  if (b >= (num_tiles & ~15)) return b;
  const int r = b & 15;
  return ((((b >> 4) << 3) + (r & 7)) << 1) + (r >> 3);
}

// C1: blocks of one key (index-selected rows), so positions are block ids
template <bool CAUSAL, bool LENS, bool C1>
__global__ __launch_bounds__(kThreads, 1) void attn_mla_kernel(AttnArgs a) {
  using L = MlaLds;
  // two LDS tile buffers (tile kt + 1 is stored while tile kt is computed) as separate
  // arrays, so the compiler sees that the stores into one never alias the reads of the other
  __shared__ __attribute__((aligned(16))) unsigned char lds_b0[L::kBuf + L::kDummy];
  __shared__ __attribute__((aligned(16))) unsigned char lds_b1[L::kBuf + L::kDummy];
  __shared__ __attribute__((aligned(16))) unsigned char lds_xs[L::kXsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave >> 1;  // head group: 32 heads
  const int hf = wave & 1;   // which half of the key tile (scores) and of dv (output)
  const int quad = lane >> 4;
  const int col = lane & 15;

  // read-only tables through the constant address space (scalar loads)
  const cint32_t* cols = (const cint32_t*)(a.cols);
  const cint32_t* lens = (const cint32_t*)(a.lens);
  const int tile = xcd_paired_tile(blockIdx.x, a.num_tiles);
  const int32_t* trec = a.tiles + static_cast<int64_t>(tile) * 8;
  const int I = trec[0];
  const int row0 = trec[2];
  const int nrows = trec[3];
  const int cb = trec[4];
  const int ce = trec[5];
  const int part = trec[6];
  const int C = C1 ? 1 : a.C;
  const int npos = (ce - cb) * C;
  const int ntiles = (npos + kKT - 1) / kKT;

  // rows of a unit are the g qo heads of token I (R = 1); lane column = head
  // of a 16-head block: heads 32 hg + 16 hb + col, hb = 0, 1
  const int qtok = I;
  const bool group_active = hg * 32 < nrows;
  // key token t is visible to this row iff (unsigned)t < qbound (masked slots carry -1)
  uint32_t qbound = 0x80000000u;
  if (CAUSAL) {
    const int64_t l = static_cast<int64_t>(qtok) + a.causal_off;
    qbound = l >= 0x7fffffff ? 0x80000000u : (l < -1 ? 0u : static_cast<uint32_t>(l + 1));
  }

  // Q^T operands of this wave's dim half: head block hb, k-step ks = dims
  // 288 hf + 32 ks + 8 quad .. + 8
  constexpr int kSteps = kDqk / 2 / 32;  // 9
  bf16x8 qf[2][kSteps];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int rloc = hg * 32 + hb * 16 + col;
    if (rloc < nrows) {
      const __bf16* qp = static_cast<const __bf16*>(a.q) + static_cast<int64_t>(qtok) * a.q_stride +
                         static_cast<int64_t>(row0 + rloc) * kDqk + hf * (kDqk / 2) + quad * 8;
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) qf[hb][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) qf[hb][ks] = bf16x8{};
    }
  }

  // trace build: one thread per key (waves 0, 1, lanes 0-15) counts the keys
  // and column entries of every tile it loads, in the last pass
  TraceAcc tr;
  // token of key position t (-1 past the range or past a block's valid
  // length), in two steps: fetch_blk issues the (unconditional, clamped)
  // table loads, finish_tok uses them -- a tile later for the prefetched
  // index, so that waiting for it never drains the row loads in flight
  struct BlkRef {
    int J;    // column block
    int len;  // its valid length (LENS)
  };
  auto fetch_blk = [&](int t) -> BlkRef {
    const int tc = t < npos ? t : npos - 1;
    const int blk = C1 ? tc : tc / C;
    BlkRef r;
    r.J = cols[cb + blk];
    r.len = LENS ? lens[cb + blk] : C;
    return r;
  };
  auto finish_tok = [&](int t, const BlkRef& r) -> int {
    const int off = C1 ? 0 : t - (t / C) * C;
    bool ok = t < npos;
    if (LENS) ok = ok && off < r.len;
    // trace build: tokens outside [0, N) are counted (by the key's counting lane) and masked
    return tr.check(ok ? r.J * C + off : -1, a.num_keys, tid < 128 && quad == 0);
  };
  auto key_tok = [&](int t) -> int { return finish_tok(t, fetch_blk(t)); };
  auto trace_key = [&](int t, int tok) {
    if (kTrace && tid < 128 && quad == 0 && tok >= 0) tr.keys(cb + (C1 ? t : t / C), 1);
  };
  const uint8_t* kv = static_cast<const uint8_t*>(a.k);
  // gather mapping: lane l of wave w takes key l % 16 (+ 16 for odd waves) and
  // 16-byte unit l / 16 (+ 4 for waves 2, 3, + 8 per round), so one load
  // instruction covers 16 keys x 64 contiguous bytes and one 16-lane store pass
  // 16 keys at one unit; each thread keeps one key.  Waves 0, 1 gather 5 units
  // per key, waves 2, 3 four (units past 35 load the row's last unit again and
  // are not stored, so every load is unconditional).
  const int my_key = (tid & 15) + 16 * (wave & 1);
  const int unit0 = quad + 4 * (wave >> 1);
  // two register sets: the rows of tile kt + 2 are in flight while tile kt is
  // stored and computed
  u32x4 creg_a[kLdRounds], creg_b[kLdRounds];
  int tok_a = -1, tok_b = -1;
  BlkRef blk_next{};  // table entries of the next tile to be fetched
  // unconditional loads (masked keys read the workspace's zero row), so the
  // wait counters keep the prefetch in flight
  const uint8_t* zrow = static_cast<const uint8_t*>(a.zero_row);
  auto load_tile = [&](u32x4 (&creg)[kLdRounds], int tok) {
    const uint8_t* src = tok >= 0 ? kv + static_cast<int64_t>(tok) * a.k_stride : zrow;
#pragma unroll
    for (int i = 0; i < kLdRounds; ++i) {
      const int u = unit0 + 8 * i;
      creg[i] = *reinterpret_cast<const u32x4*>(src + (u < kUnits ? u : kUnits - 1) * 16);
    }
  };
  // widen a tile's rows to bf16 and store them into `base` (no branch: the round
  // past a row's last unit stores into the buffer's dummy area)
  auto store_rows = [&](unsigned char* base, const u32x4 (&creg)[kLdRounds]) {
#pragma unroll
    for (int i = 0; i < kLdRounds; ++i) {
      const int u = unit0 + 8 * i;
      uint32_t b[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        b[2 * w] = fp8x2_to_bf16x2<false>(creg[i][w]);
        b[2 * w + 1] = fp8x2_to_bf16x2<true>(creg[i][w]);
      }
      // bf16 units 2u and 2u + 1 of this key's row
      const bool real = i < kLdRounds - 1 || u < kUnits;
      unsigned char* p0 = real ? base + k_off(my_key, 2 * u) : base + L::kBuf + (tid & 127) * 16;
      unsigned char* p1 = real ? base + k_off(my_key, 2 * u + 1) : base + L::kBuf + (128 + (tid & 127)) * 16;
      *reinterpret_cast<u32x4*>(p0) = u32x4{b[0], b[1], b[2], b[3]};
      *reinterpret_cast<u32x4*>(p1) = u32x4{b[4], b[5], b[6], b[7]};
    }
  };
  auto store_tok = [&](unsigned char* base, int tok) {
    if (tid < 128 && quad == 0) reinterpret_cast<int*>(base + L::kKBytes)[my_key] = tok;
  };
  auto store_tile = [&](unsigned char* base, const u32x4 (&creg)[kLdRounds], int tok) {
    store_rows(base, creg);
    store_tok(base, tok);
  };

  // this wave's output: O^T for dv in [256 hf, 256 hf + 256) of its 32 heads
  constexpr int NDB = kDv / 2 / 16;
  f32x4 oacc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db][0] = oacc[db][1] = f32x4{};
  float m_ref[2] = {-INFINITY, -INFINITY};  // reference of the probabilities (log2 units)
  float m_max[2] = {-INFINITY, -INFINITY};  // true running maximum (log2 units)
  float l_run[2] = {0.f, 0.f};  // this lane's share (keys 4 quad + v, 16 + 4 quad + v of every tile)
  bool over = false;            // some tile exceeded its row's reference by more than 2^kOverflowLog2
  const float sl2 = a.scale_log2;
  // this wave's exchange planes and its partner's
  unsigned char* xs_own = lds_xs + wave * L::kXsWave + lane * 16;
  const unsigned char* xs_peer = lds_xs + (wave ^ 1) * L::kXsWave + lane * 16;

  // One tile.  `ld`: registers of tile kt (stored last iteration), refilled
  // with the rows of tile kt + 2; `nx`: registers of tile kt + 1, widened and
  // stored into the other LDS buffer while this tile's products run.  Barrier
  // A: tile kt is in LDS and every wave is done with tile kt - 1 (its buffer
  // and the score exchange area are free).  Barrier B: scores exchanged,
  // tile kt + 1 stored.
  auto tile_step = [&](int kt, unsigned char* kl, unsigned char* knx, u32x4 (&ld)[kLdRounds], int& ld_tok,
                       const u32x4 (&nx)[kLdRounds], int nx_tok) {
    __syncthreads();
    {
      // index of tile kt + 3 first, then the rows of tile kt + 2 (whose index
      // arrived during the previous tile): waiting for the index next time
      // leaves these row loads in flight.  Past the last tile both resolve
      // to masked keys.
      const int t2 = finish_tok((kt + 2) * kKT + my_key, blk_next);
      blk_next = fetch_blk((kt + 3) * kKT + my_key);
      load_tile(ld, t2);
      ld_tok = t2;
      trace_key((kt + 2) * kKT + my_key, t2);
    }
    if (kt >= ntiles) return;  // the odd step after the last tile: loads only

    // tile-level decisions are the same for every wave (one query token)
    const int t0 = kt * kKT;
    const int t1 = (t0 + kKT < npos ? t0 + kKT : npos) - 1;
    const int blk0 = C1 ? t0 : t0 / C, blk1 = C1 ? t1 : t1 / C;
    const int64_t tok_lo = static_cast<int64_t>(cols[cb + blk0]) * C + (t0 - blk0 * C);
    const int64_t tok_hi = static_cast<int64_t>(cols[cb + blk1]) * C + (t1 - blk1 * C);
    const bool skip = CAUSAL && tok_lo > static_cast<int64_t>(qtok) + a.causal_off;
    const bool need_mask = LENS || (t0 + kKT > npos) || (CAUSAL && tok_hi > static_cast<int64_t>(qtok) + a.causal_off);

    const int* ktok = reinterpret_cast<const int*>(kl + L::kKBytes);

    // (1) this wave's part of S^T: all 32 keys (key blocks kb) x 32 heads (head
    // blocks hb) over its 288 dims, 9 k-steps; each K fragment is read once for
    // both head blocks
    f32x4 sacc[2][2] = {{f32x4{}, f32x4{}}, {f32x4{}, f32x4{}}};
    {
      // bf16 unit 32 hf + 4 j + quad (j = ks + hf) of key 16 kb + col.  The XOR
      // touches the low three unit bits only, so step ks reads at a per-wave
      // base plus an immediate offset: even ks at pa + 64 ks, odd ks at
      // pb + 64 (ks - 1), with pa / pb the units of j = 0 / 1 for hf = 0 and of
      // j = 1 / 2 for hf = 1.  The products run for every wave and tile (an
      // inactive head group multiplies zero Q rows, a tile above the causal
      // diagonal is dropped after the exchange), so the block has no branch and
      // the next tile's widening and stores interleave with the products.
      constexpr int kRing = 6;
      const unsigned char* pa[2];
      const unsigned char* pb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const unsigned char* ke = kl + k_off(16 * kb + col, 32 * hf + quad);
        const unsigned char* ko = kl + k_off(16 * kb + col, 32 * hf + quad + 4);
        pa[kb] = hf ? ko : ke;
        pb[kb] = hf ? ke + 128 : ko;
      }
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>((ks & 1) ? pb[kb] + (ks >> 1) * 128
                                                                      : pa[kb] + (ks >> 1) * 128);
          sacc[kb][0] = MfmaType<__bf16>::mfma16(kf, qf[0][ks], sacc[kb][0]);
          sacc[kb][1] = MfmaType<__bf16>::mfma16(kf, qf[1][ks], sacc[kb][1]);
        }
      // the next tile's rows, widened and stored between the products (the
      // store buffer is another array than the one read here)
      store_rows(knx, nx);
      __builtin_amdgcn_sched_group_barrier(0x100, kRing, 0);
#pragma unroll
      for (int i = 0; i < 2 * kSteps - kRing; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kRing, 0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          *reinterpret_cast<f32x4*>(xs_own + (kb * 2 + hb) * 1024) = sacc[kb][hb];
    }
    store_tok(knx, nx_tok);
    __syncthreads();
    if (!group_active || skip) return;

    // (2) add the partner's partial scores; lane (col, quad) now holds, for head
    // 32 hg + 16 hb + col, the scores of keys 4 quad + v (kb = 0) and 16 + 4 quad
    // + v (kb = 1).  Both waves of the pair run the same softmax.
    int tt[8];
    if (need_mask) {
      const int4 ta = *reinterpret_cast<const int4*>(ktok + 4 * quad);
      const int4 tb = *reinterpret_cast<const int4*>(ktok + 16 + 4 * quad);
      tt[0] = ta.x, tt[1] = ta.y, tt[2] = ta.z, tt[3] = ta.w, tt[4] = tb.x, tt[5] = tb.y, tt[6] = tb.z, tt[7] = tb.w;
    }
    bf16x8 pf[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float sv[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x4 peer = *reinterpret_cast<const f32x4*>(xs_peer + (kb * 2 + hb) * 1024);
        // one addition of two partials: commutative, so both waves get the same bits
        const f32x4 tot = sacc[kb][hb] + peer;
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[kb * 4 + v] = tot[v];
      }
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = static_cast<uint32_t>(tt[e]) < qbound ? sv[e] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = max_rows4(mx);
      const float mt = mx * sl2;
      m_max[hb] = fmaxf(m_max[hb], mt);
      // the first tile with a visible key sets the reference (O and l are
      // still zero then: every earlier probability was exp2(-inf) = 0)
      if (m_ref[hb] == -INFINITY) m_ref[hb] = mt;
      over = over || mt > m_ref[hb] + kOverflowLog2;
      const float m_use = m_ref[hb] == -INFINITY ? 0.f : m_ref[hb];
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(fmaf(sv[e], sl2, -m_use));
        ls += p;
        pf[hb][e] = static_cast<__bf16>(p);
      }
      l_run[hb] += ls;
    }
    // (3) O^T += V^T P^T for this wave's dv half and both head blocks.  A =
    // V^T (16 dv x 32 keys) with its keys in the order of P^T's registers: lane
    // (col, quad) needs dv 16 db + col of keys 4 quad + 0..3 and 16 + 4 quad +
    // 0..3.  A transposed read of 16 lanes takes 4 keys x 16 dv (lane col
    // addresses key col / 4, dv 4 (col % 4) .. + 3) and hands lane col that
    // 4-key column of dv col.  Each fragment feeds both head blocks.
    {
      const int vr = 4 * quad + (col >> 2);
      const int c1 = (col & 3) >> 1;
      const int xa = kx(vr), xb = kx(vr + 16);
      const unsigned char* va = kl + vr * L::kKRow + hf * (kDv / 2) * 2 + (col & 1) * 8;
      const unsigned char* vb = va + 16 * L::kKRow;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int ul = 2 * (db & 3) + c1;  // low three unit bits before the XOR
        const int hi = (db >> 2) * 128;
        const auto lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(va + (((ul ^ xa)) << 4) + hi));
        const auto hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vb + (((ul ^ xb)) << 4) + hi));
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db][0] = MfmaType<__bf16>::mfma16(vf, pf[0], oacc[db][0]);
        oacc[db][1] = MfmaType<__bf16>::mfma16(vf, pf[1], oacc[db][1]);
      }
      // the transposed reads run kVRing fragments ahead of the products
      constexpr int kVRing = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVRing, 0);
#pragma unroll
      for (int db = 0; db < NDB - kVRing; ++db) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kVRing, 0);
    }
  };
  for (int pass = 0;; ++pass) {
    tr = TraceAcc{};
    if (ntiles > 0) {
      tok_a = key_tok(my_key);
      load_tile(creg_a, tok_a);
      tok_b = key_tok(kKT + my_key);
      load_tile(creg_b, tok_b);
      trace_key(my_key, tok_a);
      trace_key(kKT + my_key, tok_b);
      blk_next = fetch_blk(2 * kKT + my_key);
      store_tile(lds_b0, creg_a, tok_a);
    }
    for (int kt = 0; kt < ntiles; kt += 2) {
      tile_step(kt, lds_b0, lds_b1, creg_a, tok_a, creg_b, tok_b);
      tile_step(kt + 1, lds_b1, lds_b0, creg_b, tok_b, creg_a, tok_a);
    }
    // a second pass, against each row's true maximum, only if some row of the
    // workgroup overflowed its first reference (its result is then discarded);
    // the barrier also frees the LDS buffers for the second prologue
    if (pass == 1 || !__syncthreads_or(over)) break;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      m_ref[hb] = m_max[hb];
      l_run[hb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db][hb] = f32x4{};
    }
    over = false;
  }

  trace_flush(a.trace, tile, tr, tid == 0, part, 0, row0, nrows);

  const int dv0 = hf * (kDv / 2);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float l_tot = sum_rows4(l_run[hb]);
    const float inv = l_tot > 0.f ? a.out_scale / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_ref[hb] + __log2f(l_tot)) * kLn2 : -INFINITY;
    const int rloc = hg * 32 + hb * 16 + col;
    if (rloc >= nrows) continue;
    const int head = row0 + rloc;
    if (part < 0) {
      __bf16* op = static_cast<__bf16*>(a.o) + static_cast<int64_t>(qtok) * a.o_stride +
                   static_cast<int64_t>(head) * kDv + dv0;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 out;
#pragma unroll
        for (int v = 0; v < 4; ++v) out[v] = static_cast<__bf16>(oacc[db][hb][v] * inv);
        *reinterpret_cast<bf16x4*>(op + db * 16 + 4 * quad) = out;
      }
      if (hf == 0 && quad == 0 && a.lse) a.lse[static_cast<int64_t>(qtok) * a.num_qo_heads + head] = lse_v;
    } else {
      float* pp = a.part + part;
      float* po = pp + static_cast<int64_t>(rloc) * kDv + dv0;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const f32x4 out = oacc[db][hb] * inv;
        *reinterpret_cast<f32x4*>(po + db * 16 + 4 * quad) = out;
      }
      if (hf == 0 && quad == 0) pp[static_cast<int64_t>(nrows) * kDv + rloc] = lse_v;
    }
  }
}

}  // namespace

hipError_t launch_attn_mla(const AttnArgs& a, bool causal, bool has_lens, hipStream_t st) {
  if (a.num_tiles == 0) return hipSuccess;
  const dim3 grid(a.num_tiles), block(kThreads);
  if (causal) {
    if (has_lens) attn_mla_kernel<true, true, false><<<grid, block, 0, st>>>(a);
    else if (a.C == 1) attn_mla_kernel<true, false, true><<<grid, block, 0, st>>>(a);
    else attn_mla_kernel<true, false, false><<<grid, block, 0, st>>>(a);
  } else {
    if (has_lens) attn_mla_kernel<false, true, false><<<grid, block, 0, st>>>(a);
    else if (a.C == 1) attn_mla_kernel<false, false, true><<<grid, block, 0, st>>>(a);
    else attn_mla_kernel<false, false, false><<<grid, block, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace bsa
