// Sparse-MLA attention kernel on gfx950: BSR with R = 1, one shared latent
// KV head stored as OCP fp8 e4m3 rows of 576 values (512 latent + 64 rope),
// V = the first 512 values of each row, bf16 queries and outputs
// (MATE sparse_mla_fp8_decode / FlashInfer MLA decode conventions: 576-wide
// query and cache rows, indices shared by all heads, bf16 out, fp32 lse;
// per-tensor scales folded as bmm1 = sm_scale * q_descale * k_descale and
// bmm2 = v_descale).
//
// One workgroup = one planner tile = 64 heads of one query token, 8 waves:
// four groups of 16 heads, two waves per group.  The heads are the MFMA
// column dimension, so every gathered cache row is used by all heads of the
// tile.  Per key tile of 32 keys:
//   * the selected fp8 rows are gathered with 16-byte loads two tiles ahead
//     (the per-key index one tile ahead of its use), widened exactly to bf16
//     (every e4m3 value is a bf16 value; the dequant scale is applied to the
//     logits and the output instead) and stored as row-major bf16 rows with
//     XOR-swizzled 16-byte units into the LDS buffer of the next tile while
//     this tile's scores are computed.  The same rows serve as K and, through
//     their first 512 values, as V: there is no separate V tile;
//   * wave h of a pair computes S^T = K Q^T for keys 16h .. 16h+15 of the
//     tile with v_mfma_f32_16x16x32_bf16 (Q^T resident in registers); the
//     pair swaps its fp32 scores through LDS, both waves run the same online
//     softmax (log2 domain, lagging running max) on all 32 keys, and wave h
//     accumulates O^T += V^T P^T for value dims 256h .. 256h+255 with
//     v_mfma_f32_16x16x32_bf16, the V^T fragments read from the row-major
//     tile by ds_read_b64_tr_b16 and P rounded to bf16 (the row sum l keeps
//     the unrounded fp32 probabilities).
#include "device_common.h"
#include "kernels.h"

namespace bsa {

namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kKT = 32;
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may lag behind

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct MlaLds {
  // 1152 B of bf16 per key (72 16-byte units, no padding)
  static constexpr int kKRow = kDqk * 2;
  static constexpr int kKBytes = kKT * kKRow;
  static constexpr int kTokBytes = kKT * 4;
  static constexpr int kBuf = kKBytes + kTokBytes;
  // score exchange of a wave pair: [16 heads][kXsRow] fp32, rows padded to
  // 36 floats so that 16 heads at one key offset hit distinct banks
  static constexpr int kXsRow = kKT + 4;
  static constexpr int kXsBytes = 16 * kXsRow * 4;
};

// Two OCP e4m3 bytes (the selected 16-bit half of `w`) -> two bf16 / two fp16
// values packed in one dword, low value in the low half, with gfx950's direct
// scaled conversions at scale 1.0.  Both are exact: every e4m3 value is a
// bf16 value, and e4m3 magnitudes (2^-9 .. 448, 3 mantissa bits) are fp16
// values too.  (Reinterpreting the second float of v_cvt_pk_f32_fp8's result
// as bits was miscompiled by this toolchain -- element 1 came back as a copy
// of element 0 -- so the f32 round trip is avoided.)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Unit u of key k's row sits at unit u ^ kx(k), with kx(k) a permutation of
// bits 1-3 of the key into the low three bits of the unit (bit 1 -> bit 1,
// bit 2 -> bit 0, bit 3 -> bit 2), so the XOR stays inside an aligned group
// of 8 units.  LDS has 64 banks of 4 B, 16 units per pass; a row is 72 units,
// so even keys start at bank unit 0 and odd keys at 8.  Then
//   * 16 consecutive keys at one unit (the QK reads and the tile stores, 16
//     lanes x 16 B per pass) hit 16 different bank units: the key's bit 0
//     picks the half, kx a distinct unit inside it;
//   * a transposed read (32 lanes x 8 B per pass: keys 8q + {0..3} of two
//     neighbouring q, or + {4..7}, two aligned units each) hits 8 different
//     aligned unit pairs: bit 0 picks the half, bits 1 and 3 (kx bits 1 and 2)
//     the pair.
__device__ __forceinline__ int kx(int key) {
  return (((key >> 1) & 1) << 1) | (((key >> 3) & 1) << 2) | ((key >> 2) & 1);
}
__device__ __forceinline__ int k_off(int key, int u) { return key * MlaLds::kKRow + ((u ^ kx(key)) << 4); }


// C1: blocks of one key (index-selected rows), so positions are block ids
template <int NW, bool CAUSAL, bool LENS, bool C1>
__global__ __launch_bounds__(NW * 64) void attn_mla_kernel(AttnArgs a) {
  constexpr int NBUF = 2;  // LDS tile buffers: tile kt + 1 is stored while tile kt is computed
  using L = MlaLds;
  constexpr int NTHR = NW * 64;
  constexpr int NCHUNK = kKT * (kDqk / 16);  // 16-byte fp8 chunks per key tile
  constexpr int CH_PER_T = (NCHUNK + NTHR - 1) / NTHR;
  constexpr int NGROUP = NW / 2;             // 16-head groups per tile
  static_assert(NTHR % kKT == 0 && NW % 2 == 0, "loader maps one key per thread; waves pair up");
  static_assert(NW == 8, "the gather mapping below covers 32 keys x 16 chunks per round with 512 threads");

  __shared__ __attribute__((aligned(16))) unsigned char lds[NBUF * L::kBuf + NGROUP * L::kXsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave >> 1;  // head group: 16 heads
  const int hf = wave & 1;   // which half of the key tile (scores) and of dv (output)
  const int quad = lane >> 4;
  const int col = lane & 15;

  // read-only tables through the constant address space (scalar loads)
  const cint32_t* cols = (const cint32_t*)(a.cols);
  const cint32_t* lens = (const cint32_t*)(a.lens);
  const int32_t* trec = a.tiles + static_cast<int64_t>(blockIdx.x) * 8;
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
  const int rloc = hg * 16 + col;
  const bool row_ok = rloc < nrows;
  const int head = row0 + rloc;
  const int qtok = I;
  const bool group_active = hg * 16 < nrows;
  // key token t is visible to this row iff (unsigned)t < qbound (masked slots carry -1)
  uint32_t qbound = 0x80000000u;
  if (CAUSAL) {
    const int64_t l = static_cast<int64_t>(qtok) + a.causal_off;
    qbound = l >= 0x7fffffff ? 0x80000000u : (l < -1 ? 0u : static_cast<uint32_t>(l + 1));
  }

  bf16x8 qf[kDqk / 32];
  if (row_ok) {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + static_cast<int64_t>(qtok) * a.q_stride +
                       static_cast<int64_t>(head) * kDqk + quad * 8;
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
  } else {
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) qf[ks] = bf16x8{};
  }

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
    return ok ? r.J * C + off : -1;
  };
  auto key_tok = [&](int t) -> int { return finish_tok(t, fetch_blk(t)); };
  const uint8_t* kv = static_cast<const uint8_t*>(a.k);
  // gather mapping: lane l of a wave takes key l % 16 (+ 16 for odd waves) and
  // 16-byte chunk l / 16 (+ 4 per pair of waves, + 16 per round), so one load
  // instruction covers 16 keys x 64 contiguous bytes and one 16-lane store pass
  // 16 keys at one unit; each thread keeps one key
  const int my_key = (tid & 15) + 16 * ((tid >> 6) & 1);
  auto chunk_of = [&](int i) { return ((tid & 63) >> 4) + 4 * (tid >> 7) + 16 * i; };
  // two register sets: the rows of tile kt + 2 are in flight while tile kt is
  // stored and computed
  u32x4 creg_a[CH_PER_T], creg_b[CH_PER_T];
  int tok_a = -1, tok_b = -1;
  BlkRef blk_next{};  // table entries of the next tile to be fetched
  // unconditional loads (masked keys and idle lanes read the workspace's zero
  // row), so the wait counters keep the prefetch in flight
  const uint8_t* zrow = static_cast<const uint8_t*>(a.zero_row);
  auto load_tile = [&](u32x4 (&creg)[CH_PER_T], int tok) {
#pragma unroll
    for (int i = 0; i < CH_PER_T; ++i) {
      const int ci = tid + i * NTHR;
      const int c = chunk_of(i);  // 16-byte chunk of the fp8 row (< 48, inside the 1 KB zero row)
      const uint8_t* src = (ci < NCHUNK && tok >= 0) ? kv + static_cast<int64_t>(tok) * a.k_stride : zrow;
      creg[i] = *reinterpret_cast<const u32x4*>(src + c * 16);
    }
  };
  auto store_tile = [&](int buf, const u32x4 (&creg)[CH_PER_T], int tok) {
    unsigned char* base = lds + buf * L::kBuf;
#pragma unroll
    for (int i = 0; i < CH_PER_T; ++i) {
      const int ci = tid + i * NTHR;
      if (ci >= NCHUNK) continue;
      const int c = chunk_of(i);
      uint32_t b[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        b[2 * w] = fp8x2_to_bf16x2<false>(creg[i][w]);
        b[2 * w + 1] = fp8x2_to_bf16x2<true>(creg[i][w]);
      }
      // bf16 units 2c and 2c + 1 of this key's row
      *reinterpret_cast<u32x4*>(base + k_off(my_key, 2 * c)) = u32x4{b[0], b[1], b[2], b[3]};
      *reinterpret_cast<u32x4*>(base + k_off(my_key, 2 * c + 1)) = u32x4{b[4], b[5], b[6], b[7]};
    }
    if (tid < 128 && ((tid >> 4) & 3) == 0) reinterpret_cast<int*>(base + L::kKBytes)[my_key] = tok;
  };

  // this wave's output: O^T for dv in [256 * hf, 256 * hf + 256), its 16 heads
  constexpr int NDB = kDv / 2 / 16;
  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's share (keys 8 * quad .. + 8 of every tile)
  const float sl2 = a.scale_log2;
  float* xs = reinterpret_cast<float*>(lds + NBUF * L::kBuf + hg * L::kXsBytes);  // [16 heads][kXsRow]

  // One tile.  `ld`: registers of tile kt (stored last iteration), refilled
  // with the rows of tile kt + 2; `nx`: registers of tile kt + 1, widened and
  // stored into the other LDS buffer while this tile's products run.  Barrier
  // A: tile kt is in LDS and every wave is done with tile kt - 1 (its buffer
  // and the score exchange area are free).  Barrier B: scores exchanged,
  // tile kt + 1 stored.
  auto tile_step = [&](int kt, u32x4 (&ld)[CH_PER_T], int& ld_tok, const u32x4 (&nx)[CH_PER_T], int nx_tok) {
    const int buf = kt & 1;
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

    const unsigned char* kl = lds + buf * L::kBuf;
    const int* ktok = reinterpret_cast<const int*>(kl + L::kKBytes);

    // (1) S^T of this wave's 16 keys (16 * hf ..) x 16 heads over all 576
    // dims, 18 k-steps; K fragments through a small register ring
    if (group_active && !skip) {
      constexpr int kSteps = kDqk / 32;
      constexpr int kRing = 8;
      // unit quad + 4 ks of key 16 hf + col: the XOR touches the low three
      // unit bits only, so even and odd ks each have one base and
      // immediate offsets
      const int key = hf * 16 + col;
      const unsigned char* kev = kl + k_off(key, quad);
      const unsigned char* kod = kl + k_off(key, quad + 4);
      auto kfrag = [&](int ks) {
        return *reinterpret_cast<const bf16x8*>((ks & 1 ? kod : kev) + (ks >> 1) * 128);
      };
      f32x4 sacc = f32x4{};
      bf16x8 kr[kSteps];
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) kr[ks] = kfrag(ks);
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) sacc = MfmaType<__bf16>::mfma16(kr[ks], qf[ks], sacc);
      // reads run kRing fragments ahead of the products (the scheduler would
      // otherwise issue each read one or two products before its use)
      __builtin_amdgcn_sched_group_barrier(0x100, kRing, 0);
#pragma unroll
      for (int ks = 0; ks < kSteps - kRing; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kRing, 0);
      // lane holds head col, keys 16 * hf + 4 * quad + v
      *reinterpret_cast<f32x4*>(xs + col * L::kXsRow + hf * 16 + 4 * quad) = sacc;
    }
    if (kt + 1 < ntiles) store_tile(buf ^ 1, nx, nx_tok);
    __syncthreads();
    if (!group_active || skip) return;

    // (2) both waves of the pair read all 32 scores of their heads in the
    // P^T operand layout (head col, keys 8 * quad + e) and run the same softmax
    float sv[8];
    {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(xs + col * L::kXsRow + 8 * quad);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(xs + col * L::kXsRow + 8 * quad + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[e] = lo[e];
        sv[e + 4] = hi[e];
      }
    }
    if (need_mask) {
      const int4 ta = *reinterpret_cast<const int4*>(ktok + 8 * quad);
      const int4 tb = *reinterpret_cast<const int4*>(ktok + 8 * quad + 4);
      const int tt[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = static_cast<uint32_t>(tt[e]) < qbound ? sv[e] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // lagging running max: it only moves when the tile exceeds it by more
    // than 2^kRescaleSlack, so the rescale of O is rare
    const float mt = mx * sl2;
    const bool upd = mt > m_run + kRescaleSlack;
    const float m_new = upd ? mt : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
    m_run = m_new;
    float ls = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(fmaf(sv[e], sl2, -m_use));
      ls += p;
      pf[e] = static_cast<__bf16>(p);
    }
    l_run = l_run * alpha + ls;
    if (__ballot(upd) != 0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    // (3) O^T += V^T P^T for this wave's dv half.  A = V^T (16 dv x 32 keys):
    // lane (col, quad) needs dv 16 db + col of keys 8 quad .. 8 quad + 7.  A
    // transposed read of 16 lanes takes 4 keys x 16 dv (lane col addresses key
    // col / 4, dv 4 (col % 4) .. + 3) and hands lane col that 4-key column of
    // dv col; two reads cover keys 8 quad + 0..3 and + 4..7.
    {
      const int vr = 8 * quad + (col >> 2);
      const int c1 = (col & 3) >> 1;
      const int xa = kx(vr), xb = kx(vr + 4);
      const unsigned char* va = kl + vr * L::kKRow + hf * (kDv / 2) * 2 + (col & 1) * 8;
      const unsigned char* vb = va + 4 * L::kKRow;
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
        oacc[db] = MfmaType<__bf16>::mfma16(vf, pf, oacc[db]);
      }
      // the transposed reads run kVRing products ahead
      constexpr int kVRing = 6;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVRing, 0);
#pragma unroll
      for (int db = 0; db < NDB - kVRing; ++db) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kVRing, 0);
    }
  };
  if (ntiles > 0) {
    tok_a = key_tok(my_key);
    load_tile(creg_a, tok_a);
    tok_b = key_tok(kKT + my_key);
    load_tile(creg_b, tok_b);
    blk_next = fetch_blk(2 * kKT + my_key);
    store_tile(0, creg_a, tok_a);
  }
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile_step(kt, creg_a, tok_a, creg_b, tok_b);
    tile_step(kt + 1, creg_b, tok_b, creg_a, tok_a);
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? a.out_scale / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (!row_ok) return;
  const int dv0 = hf * (kDv / 2);
  if (part < 0) {
    __bf16* op = static_cast<__bf16*>(a.o) + static_cast<int64_t>(qtok) * a.o_stride +
                 static_cast<int64_t>(head) * kDv + dv0;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x4 out;
#pragma unroll
      for (int v = 0; v < 4; ++v) out[v] = static_cast<__bf16>(oacc[db][v] * inv);
      *reinterpret_cast<bf16x4*>(op + db * 16 + 4 * quad) = out;
    }
    if (hf == 0 && quad == 0 && a.lse) a.lse[static_cast<int64_t>(qtok) * a.num_qo_heads + head] = lse_v;
  } else {
    float* pp = a.part + part;
    float* po = pp + static_cast<int64_t>(rloc) * kDv + dv0;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      f32x4 out = oacc[db] * inv;
      *reinterpret_cast<f32x4*>(po + db * 16 + 4 * quad) = out;
    }
    if (hf == 0 && quad == 0) pp[static_cast<int64_t>(nrows) * kDv + rloc] = lse_v;
  }
}

}  // namespace

hipError_t launch_attn_mla(const AttnArgs& a, bool causal, bool has_lens, hipStream_t st) {
  if (a.num_tiles == 0) return hipSuccess;
  constexpr int NW = 8;
  const dim3 grid(a.num_tiles), block(NW * 64);
  if (causal) {
    if (has_lens) attn_mla_kernel<NW, true, true, false><<<grid, block, 0, st>>>(a);
    else if (a.C == 1) attn_mla_kernel<NW, true, false, true><<<grid, block, 0, st>>>(a);
    else attn_mla_kernel<NW, true, false, false><<<grid, block, 0, st>>>(a);
  } else {
    if (has_lens) attn_mla_kernel<NW, false, true, false><<<grid, block, 0, st>>>(a);
    else if (a.C == 1) attn_mla_kernel<NW, false, false, true><<<grid, block, 0, st>>>(a);
    else attn_mla_kernel<NW, false, false, false><<<grid, block, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace bsa
