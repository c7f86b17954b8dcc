// Paged-decode kernel on gfx950: BSR with R = 1 (one query token per row
// block), block size C a multiple of 16 (C = page size), head_dim 128,
// fp16/bf16, up to 16 qo heads per kv head (flashinfer.sparse
// BlockSparseAttentionWrapper with R = 1, C = page size; the FlashInfer
// BatchDecodeWithPagedKVCacheWrapper workload written as BSR).
//
// Decode reads every unmasked K/V row exactly once and does ~4 flops per
// byte, so the kernel is built around bytes in flight, not arithmetic:
//   * a workgroup of NW = 8 waves takes groups of HG tiles (the planner's
//     head groups: same token and pages, HG consecutive kv heads, HG a power
//     of two up to 8); wave w serves kv head w % HG of the group and takes
//     its 32-key tiles w / HG, w / HG + NW / HG, ...  With 8 kv heads each
//     wave owns one head, so one workgroup reads whole token rows of K and V
//     (all heads of a page) at once: pages read in lockstep by workgroups on
//     different XCDs stream markedly slower;
//   * the workgroups stay resident and run their groups back to back, the
//     next group's first keys loading while the current group's waves merge
//     their softmax states through LDS;
//   * K goes from HBM straight into MFMA A-operand registers (16-byte loads,
//     no LDS); S^T = K Q^T runs on v_mfma_f32_16x16x32 with the g heads as
//     the (zero-padded) 16 columns;
//   * V is staged row-major in a wave-private 8 KB LDS tile (chunks XOR-
//     swizzled by key) and read back transposed with ds_read_b64_tr_b16 as
//     the A operand of O^T += V^T P^T; the key order of S^T's rows is chosen
//     so that P^T comes straight from the S^T accumulators in the order the
//     transposed reads deliver V;
//   * the next key tile's K and V loads are issued before the current one's
//     math (register double buffering), and no workgroup barrier is needed
//     inside the key loop;
//   * keys outside a page's valid length (or past the range) load from a
//     zero row in the workspace, so unused cache slots never reach the
//     arithmetic, and are masked to -inf in the scores.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace bsa {

namespace {

#ifndef BSA_DECODE_NW
#define BSA_DECODE_NW 8            // waves per workgroup
#endif
#ifndef BSA_DECODE_MIN_WAVES
#define BSA_DECODE_MIN_WAVES 2     // occupancy target (waves per SIMD) given to the register allocator
#endif

constexpr int kD = 128;
constexpr int kKT = 32;                 // keys per tile
constexpr int kVBytes = kKT * kD * 2;   // wave-private V tile

typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS byte offset of 16-byte chunk `c` of key row `k` in a V tile: chunk
// c ^ s(k), s(k) = 2 (k & 3) + 9 bit3(k).  A V store writes one chunk of keys
// {0..3, 8..11} (+ 4) from 8 consecutive lanes, which a ds_write_b128 serves
// in one pass when the chunks differ mod 8 (measured on gfx950): s(k) mod 8 =
// 0, 2, 4, 6, 1, 3, 5, 7.  A transposed read takes the aligned chunk pair
// (2m, 2m + 1) of the same 8 rows: pair m ^ (s(k) >> 1) = m ^ 0..7, all
// different.
__device__ __forceinline__ int v_chunk_off(int k, int c) {
  return k * (kD * 2) + ((c ^ (((k & 3) << 1) | (((k >> 3) & 1) * 9))) << 4);
}

// KV8: K and V are stored as OCP fp8 e4m3 (one byte per value) and widened
// exactly to T where they are used (K before its products, V before its LDS
// store); per-head dequant scales fold into the logit and output scales.
template <typename T, bool KV8, int NW, bool CAUSAL, bool LENS, bool POW2C>
__global__ __launch_bounds__(NW * 64, BSA_DECODE_MIN_WAVES) void attn_decode_kernel(AttnArgs a) {
  using Ops = MfmaType<T>;
  using v8 = typename Ops::v8;
  using v4 = typename Ops::v4;

  __shared__ __attribute__((aligned(16))) unsigned char lds[NW * kVBytes];
  __shared__ float red_m[NW][16], red_l[NW][16];
  __shared__ int head_kvh[NW], head_part[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quad = lane >> 4;
  const int col = lane & 15;
  // head slot hw of the group and key-tile phase sub of this wave; WPH waves share a head
  const int HG = a.heads_per_wg;
  const int lg_hg = __builtin_ctz(HG);
  const int WPH = NW >> lg_hg;
  const int lg_wph = __builtin_ctz(WPH);
  const int hw = wave & (HG - 1);
  const int sub = wave >> lg_hg;
  const int C = a.C;
  const int cshift = POW2C ? __builtin_ctz(C) : 0;  // C = 1 << cshift when POW2C
  const int g = a.group;
  const cint32_t* cols = (const cint32_t*)(a.cols);
  const cint32_t* lens = (const cint32_t*)(a.lens);
  const cint32_t* zints = (const cint32_t*)(a.zero_row);

  // One planner tile as scalars (R = 1: the query token is the row block).
  // A tile index past the end gives an empty context: no keys, and every
  // load it leads to reads the zero row.
  struct Ctx {
    int I, kvh, row0, nrows, cb, nblk, part, ntiles, qlim;
  };
  // this workgroup's tiles: t_begin .. t_end-1 of the plan's tile list, in
  // groups of HG; this wave's tile of the group starting at g0 is g0 + hw
  const cint32_t* wgp = (const cint32_t*)(a.wg_ptr) + blockIdx.x;
  const int t_begin = wgp[0], t_end = wgp[1];
  if (t_begin >= t_end) return;
  auto read_ctx = [&](int g0) {
    Ctx c{0, 0, 0, 0, 0, 0, -1, 0, -1};
    if (g0 < t_end) {
      const cint32_t* tr = (const cint32_t*)(a.tiles) + static_cast<int64_t>(g0 + hw) * 8;
      c.I = tr[0];
      c.kvh = tr[1];
      c.row0 = tr[2];
      c.nrows = tr[3];
      c.cb = tr[4];
      c.nblk = tr[5] - c.cb;
      c.part = tr[6];
      c.ntiles = (c.nblk * C + kKT - 1) / kKT;
      if (CAUSAL) {
        const int64_t lim64 = static_cast<int64_t>(c.I) + a.causal_off;
        c.qlim = lim64 > 0x7fffffff ? 0x7fffffff : (lim64 < -1 ? -1 : static_cast<int>(lim64));
      }
    }
    return c;
  };

  // Key tile kt of a tile context with its (uniform, scalar-loaded) column
  // blocks and their valid lengths: a 32-key tile spans at most 3 blocks
  // when C >= 16.  Tiles past the end of the range only feed dummy loads.
  struct Src {
    int t0, npos, qlim, kvh;
    int base;            // first key position of the key tile's first block
    int J0, J1, J2;      // its first three column blocks (clamped to the range)
    int L0, L1, L2;      // their valid lengths
  };
  auto make_src = [&](const Ctx& c, int kt) {
    Src s;
    s.t0 = kt * kKT;
    s.npos = c.nblk * C;
    s.qlim = c.qlim;
    s.kvh = c.kvh;
    const int last = c.nblk > 0 ? c.nblk - 1 : 0;
    const cint32_t* cp = c.nblk > 0 ? cols + c.cb : zints;
    int blk0 = POW2C ? (s.t0 >> cshift) : s.t0 / C;
    blk0 = blk0 < last ? blk0 : last;
    const int b1 = blk0 + 1 < last ? blk0 + 1 : last;
    const int b2 = blk0 + 2 < last ? blk0 + 2 : last;
    s.base = blk0 * C;
    s.J0 = cp[blk0];
    s.J1 = cp[b1];
    s.J2 = cp[b2];
    if (LENS) {
      const cint32_t* lp = c.nblk > 0 ? lens + c.cb : zints;
      s.L0 = lp[blk0];
      s.L1 = lp[b1];
      s.L2 = lp[b2];
    } else {
      s.L0 = s.L1 = s.L2 = C;
    }
    return s;
  };
  TraceAcc tr_chk;  // trace build: out-of-range key tokens (counted into each tile's record)
  // branch-free, so every stage issues the same loads and the compiler can
  // wait for exactly the older stage
  auto key_token = [&](const Src& b, int t) -> int {
    const int r = t - b.base;                      // < 32 + C, so at most two block steps
    // select block 0, 1 or 2 with masks (a plain ?: chain of these uniform
    // values was lowered to an indexed load from a stack copy)
    const int s1 = r >= C ? -1 : 0;
    const int s2 = r >= 2 * C ? -1 : 0;
    const int off = r - (C & s1) - (C & s2);
    int J = b.J0 ^ ((b.J0 ^ b.J1) & s1);
    J ^= (J ^ b.J2) & s2;
    int len = b.L0 ^ ((b.L0 ^ b.L1) & s1);
    len ^= (len ^ b.L2) & s2;
    const int tok = J * C + off;
    bool ok = t < b.npos;
    if (LENS) ok = ok && off < len;
    if (CAUSAL) ok = ok && tok <= b.qlim;
    // trace build: tokens outside [0, N) are counted (by quad 0, one lane per key) and masked
    return tr_chk.check(ok ? tok : -1, a.num_keys, quad == 0);
  };

  // per-key-tile registers: K fragments and V chunks, both indexed (kb, ks):
  // lane (col, quad) holds dims ks*32 + quad*8 .. +8 of key (kb, col)
  // Raw K/V bytes of a key, as 16-byte loads.  16-bit storage: four loads,
  // load j = dims j*32 + quad*8 .. +8 (k-step j).  fp8: two loads, load j =
  // dims j*64 + quad*16 .. +16, so every load covers whole 64-byte sectors;
  // k-step ks then takes half ks % 2 of load ks / 2.  Q is loaded in the same
  // dim order (the dot product is indifferent to it), and V goes back to its
  // own chunks in LDS.
  constexpr int NLD = KV8 ? 2 : 4;
  struct Stage {
    u32x4 k[2][NLD];
    u32x4 v[2][NLD];
    uint32_t valid[2];  // bit m: key (kb, m) valid
  };
  // key of S^T row m in block kb: 8*(m/4) + 4*kb + m%4
  constexpr int kElt = KV8 ? 1 : 2;  // bytes per K/V value
  auto load_stage = [&](Stage& s, const Src& b) {
    const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + static_cast<int64_t>(b.kvh) * kD * kElt;
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + static_cast<int64_t>(b.kvh) * kD * kElt;
    const unsigned char* zb = static_cast<const unsigned char*>(a.zero_row);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 8 * (col >> 2) + 4 * kb + (col & 3);
      const int tok = key_token(b, b.t0 + key);
      const unsigned char* pk = tok >= 0 ? kbase + static_cast<int64_t>(tok) * a.k_stride * kElt : zb;
      const unsigned char* pv = tok >= 0 ? vbase + static_cast<int64_t>(tok) * a.v_stride * kElt : zb;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int off = KV8 ? j * 64 + quad * 16 : (j * 32 + quad * 8) * 2;
        s.k[kb][j] = *reinterpret_cast<const u32x4*>(pk + off);
        s.v[kb][j] = *reinterpret_cast<const u32x4*>(pv + off);
      }
      const uint64_t bal = __ballot(tok >= 0);
      s.valid[kb] = static_cast<uint32_t>(bal & 0xffffu);
    }
  };
  // the eight K values of k-step ks, in T
  auto kfrag = [&](const Stage& s, int kb, int ks) -> v8 {
    if constexpr (KV8) {
      const u32x4 r = s.k[kb][ks >> 1];
      return bitcast<v8>(fp8x8_widen<T>((ks & 1) ? u32x2{r[2], r[3]} : u32x2{r[0], r[1]}));
    } else {
      return bitcast<v8>(s.k[kb][ks]);
    }
  };

  // Q^T as the B operand: column `col` is qo head kvh*g + row0 + col.  Columns
  // at or beyond nrows load the tile's last row instead (a plain, unconditional
  // load): columns never mix, and those columns are never written.
  v8 qf[4], qn[4];  // this group's Q and the next group's (loaded one group ahead)
  auto load_q = [&](const Ctx& c, v8 (&q)[4]) {
    const int cc = col < c.nrows ? col : (c.nrows > 0 ? c.nrows - 1 : 0);
    const T* qp = static_cast<const T*>(a.q) + static_cast<int64_t>(c.I) * a.q_stride +
                  static_cast<int64_t>(c.kvh * g + c.row0 + cc) * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      q[ks] = *reinterpret_cast<const v8*>(qp + (KV8 ? (ks >> 1) * 64 + quad * 16 + (ks & 1) * 8 : ks * 32 + quad * 8));
  };

  unsigned char* vl = lds + wave * kVBytes;
  f32x4 oacc[8];
  float m_run, l_run;
  // logit scale of this lane's column (qo head) in the current group:
  // sm_scale * q/k dequant scales * log2(e); sln is the next group's
  float sl2 = a.scale_log2, sln = a.scale_log2;
  auto lane_scale = [&](const Ctx& c) -> float {
    const int cc = col < c.nrows ? col : (c.nrows > 0 ? c.nrows - 1 : 0);
    float s = a.scale_log2;
    if (a.q_scale) s *= a.q_scale[c.kvh * g + c.row0 + cc];
    if (a.k_scale) s *= a.k_scale[c.kvh];
    return s;
  };
  auto out_scale = [&](int kvh) -> float { return a.v_scale ? a.out_scale * a.v_scale[kvh] : a.out_scale; };

  // First half of a key tile's math: stage V into this wave's LDS tile
  // (row-major, swizzled chunks) and form the masked scores S^T = K Q^T.
  // After it the stage's registers are free for the next loads.
  auto scores = [&](const Stage& s, f32x4 (&sc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 8 * (col >> 2) + 4 * kb + (col & 3);
      if constexpr (KV8) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 r = s.v[kb][j];
          *reinterpret_cast<u32x4*>(vl + v_chunk_off(key, j * 8 + quad * 2)) = fp8x8_widen<T>(u32x2{r[0], r[1]});
          *reinterpret_cast<u32x4*>(vl + v_chunk_off(key, j * 8 + quad * 2 + 1)) = fp8x8_widen<T>(u32x2{r[2], r[3]});
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<u32x4*>(vl + v_chunk_off(key, ks * 4 + quad)) = s.v[kb][ks];
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[kb] = Ops::mfma16(kfrag(s, kb, ks), qf[ks], sc[kb]);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (!((s.valid[kb] >> (4 * quad + v)) & 1u)) sc[kb][v] = -INFINITY;
    }
  };
  // Second half: online softmax update and O^T += V^T P^T.
  auto accumulate = [&](const f32x4 (&sc)[2]) {
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = max_rows4(mx);
    const float m_new = fmaxf(m_run, mx * sl2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float ls = 0.f;
    v8 pf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = fast_exp2(fmaf(sc[kb][v], sl2, -m_use));
        ls += p;
        pf[4 * kb + v] = static_cast<T>(p);
      }
    l_run = l_run * alpha + ls;
    // transposed reads: lane L of this quad reads key row 8*quad + 4*j + L/4
    // at dims d0 + 4*(L%4) .. +3
    const int rrow = 8 * quad + (col >> 2);
    const int dsub = 4 * (col & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = db * 16 + dsub;
      const int c = d >> 3;
      const int boff = (d & 7) * 2;
      const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vl + v_chunk_off(rrow, c) + boff));
      const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vl + v_chunk_off(rrow + 4, c) + boff));
      const v4 vlo = bitcast<v4>(lo), vhi = bitcast<v4>(hi);
      const v8 vf = __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[db] = Ops::mfma16(vf, pf, oacc[db] * alpha);
    }
  };

  // Merge the softmax states of the waves that share a head (WPH of them)
  // for the finished group and write each head's output (or split partial);
  // c is this wave's tile of the group.
  auto finish_tile = [&](const Ctx& c) {
    const float l_tot = sum_rows4(l_run);
    if (WPH == 1) {
      // the wave owns its head: normalise and store straight from the
      // accumulators (lane (col, quad) holds dims db*16 + 4*quad .. +3 of
      // column col).  Columns at or beyond nrows replicate column nrows - 1
      // bit for bit (same Q), so every lane stores, to that column's place,
      // the same bytes: no predicated stores.
      const int cc = col < c.nrows ? col : c.nrows - 1;
      const int head = c.kvh * g + c.row0 + cc;
      const float inv = l_tot > 0.f ? out_scale(c.kvh) / l_tot : 0.f;
      const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
      if (c.part < 0) {
        T* op = static_cast<T*>(a.o) + static_cast<int64_t>(c.I) * a.o_stride + static_cast<int64_t>(head) * kD + 4 * quad;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          v4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(oacc[db][e] * inv);
          *reinterpret_cast<v4*>(op + db * 16) = out;
        }
        if (a.lse) a.lse[static_cast<int64_t>(c.I) * a.num_qo_heads + head] = lse_v;
      } else {
        float* pp = a.part + c.part;
#pragma unroll
        for (int db = 0; db < 8; ++db)
          *reinterpret_cast<f32x4*>(pp + static_cast<int64_t>(cc) * kD + db * 16 + 4 * quad) = oacc[db] * inv;
        pp[static_cast<int64_t>(c.nrows) * kD + cc] = lse_v;
      }
      return;
    }
    __syncthreads();  // every wave is done with its V tile: reuse LDS for the merge
    float* ob = reinterpret_cast<float*>(lds);  // [NW][16 cols][128 d]
    if (quad == 0) {
      red_m[wave][col] = m_run;
      red_l[wave][col] = l_tot;
    }
    if (sub == 0 && lane == 0) {
      head_kvh[hw] = c.kvh;
      head_part[hw] = c.part;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<f32x4*>(ob + (wave * 16 + col) * kD + db * 16 + 4 * quad) = oacc[db];
    __syncthreads();
    // thread -> (head slot, column, 4 dims): HG * 16 * 32 items over NW * 64 threads
    for (int item = tid; item < HG * 16 * (kD / 4); item += NW * 64) {
      const int hs = item >> 9;
      const int cq = (item >> 5) & 15;
      const int d4 = (item & 31) * 4;
      if (cq >= c.nrows) continue;
      float M = -INFINITY;
      for (int s2 = 0; s2 < WPH; ++s2) M = fmaxf(M, red_m[hs + (s2 << lg_hg)][cq]);
      const float Mu = M == -INFINITY ? 0.f : M;
      float L = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int s2 = 0; s2 < WPH; ++s2) {
        const int w2 = hs + (s2 << lg_hg);
        const float sc = fast_exp2(red_m[w2][cq] - Mu);
        L += red_l[w2][cq] * sc;
        acc += sc * *reinterpret_cast<const f32x4*>(ob + (w2 * 16 + cq) * kD + d4);
      }
      const float inv = L > 0.f ? out_scale(head_kvh[hs]) / L : 0.f;
      const float lse_v = L > 0.f ? (Mu + __log2f(L)) * kLn2 : -INFINITY;
      const int head = head_kvh[hs] * g + c.row0 + cq;
      const int part = head_part[hs];
      acc *= inv;
      if (part < 0) {
        v4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(acc[e]);
        *reinterpret_cast<v4*>(static_cast<T*>(a.o) + static_cast<int64_t>(c.I) * a.o_stride +
                               static_cast<int64_t>(head) * kD + d4) = out;
        if (d4 == 0 && a.lse) a.lse[static_cast<int64_t>(c.I) * a.num_qo_heads + head] = lse_v;
      } else {
        float* pp = a.part + part;
        *reinterpret_cast<f32x4*>(pp + static_cast<int64_t>(cq) * kD + d4) = acc;
        if (d4 == 0) pp[static_cast<int64_t>(c.nrows) * kD + cq] = lse_v;
      }
    }
    __syncthreads();  // the merge buffer is the next group's V staging area
  };

  // The workgroup runs its groups in order.  Within a group the WPH waves of
  // a head take its 32-key tiles sub, sub+WPH, ...; each wave's sequence is
  // padded to a multiple of NS (at least NS) with key tiles past the end, which
  // load the zero row and are fully masked (so computing them leaves the
  // softmax state unchanged), and the loads run two items ahead across tile
  // boundaries, so the next group's first keys are in flight during the
  // current group's merge.  Every load and every use is unconditional, so each
  // wait covers exactly the older stage.
  Ctx cur = read_ctx(t_begin);
  load_q(cur, qf);
  sl2 = lane_scale(cur);
  // NS register stages of key tiles in flight (three or four fp8 stages measured slower)
  constexpr int NS = 2;
  Stage stg[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) load_stage(stg[i], make_src(cur, sub + i * WPH));
  for (int gn = t_begin + HG;; gn += HG) {
    const Ctx nxt = read_ctx(gn);
    load_q(nxt, qn);
    sln = lane_scale(nxt);
    const int nT = cur.ntiles > sub ? (cur.ntiles - sub + WPH - 1) >> lg_wph : 0;
    const int nTe = nT < NS ? NS : (nT + NS - 1) / NS * NS;
    // key tile loaded for item q: item q of this group for q < nTe, else item
    // q - nTe of the next one
    auto src_of = [&](int q) {
      const bool in = q < nTe;
      const Ctx c = in ? cur : nxt;
      return make_src(c, sub + ((in ? q : q - nTe) << lg_wph));
    };
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = f32x4{};
    m_run = -INFINITY;
    l_run = 0.f;
    // stage i holds item p + i at the top of each pass; it is reloaded (item
    // p + NS + i) as soon as its scores are formed
    int p = 0;
    TraceAcc tr;  // trace build: column entries and keys (before the causal mask) of this wave's items
    do {  // nTe >= NS: at least one pass, so the waits never see a skipped body
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if constexpr (kTrace) {
          // this lane's two keys of the item (quad 0 only), inside the range
          // and their block's valid length
          const int kt = sub + ((p + i) << lg_wph);
          for (int kb = 0; kb < 2 && quad == 0; ++kb) {
            const int t = kt * kKT + 8 * (col >> 2) + 4 * kb + (col & 3);
            if (t < cur.nblk * C && t % C < (LENS ? lens[cur.cb + t / C] : C)) tr.keys(cur.cb + t / C, 1);
          }
        }
        f32x4 sc[2];
        const Src sn = src_of(p + NS + i);
        scores(stg[i], sc);
        load_stage(stg[i], sn);
        accumulate(sc);
      }
      p += NS;
    } while (p < nTe);
    if constexpr (kTrace) {
      tr.bad = tr_chk.bad;  // met while loading this group's keys (and the next group's first ones)
      tr_chk.bad = 0;
      trace_flush(a.trace, gn - HG + hw, tr, sub == 0 && lane == 0, cur.part, cur.kvh, cur.row0, cur.nrows);
    }
    finish_tile(cur);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = qn[ks];
    sl2 = sln;
    if (gn >= t_end) break;
    cur = nxt;
  }
}

template <typename T, bool KV8, int NW, bool CAUSAL, bool LENS, bool POW2C>
hipError_t launch_variant(const AttnArgs& a, hipStream_t st) {
  attn_decode_kernel<T, KV8, NW, CAUSAL, LENS, POW2C><<<dim3(a.num_wgs), dim3(NW * 64), 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, bool KV8, int NW, bool POW2C>
hipError_t launch_nw(const AttnArgs& a, bool causal, bool lens, hipStream_t st) {
  if (causal)
    return lens ? launch_variant<T, KV8, NW, true, true, POW2C>(a, st) : launch_variant<T, KV8, NW, true, false, POW2C>(a, st);
  return lens ? launch_variant<T, KV8, NW, false, true, POW2C>(a, st) : launch_variant<T, KV8, NW, false, false, POW2C>(a, st);
}

template <typename T, bool KV8>
hipError_t launch_typed(const AttnArgs& a, bool causal, bool lens, hipStream_t st) {
  if ((a.C & (a.C - 1)) == 0) return launch_nw<T, KV8, BSA_DECODE_NW, true>(a, causal, lens, st);
  return launch_nw<T, KV8, BSA_DECODE_NW, false>(a, causal, lens, st);
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, bool bf16, bool kv8, bool causal, bool has_lens,
                              hipStream_t stream) {
  if (a.num_tiles == 0 || a.num_wgs <= 0) return hipSuccess;
  if (kv8)
    return bf16 ? launch_typed<__bf16, true>(a, causal, has_lens, stream)
                : launch_typed<_Float16, true>(a, causal, has_lens, stream);
  return bf16 ? launch_typed<__bf16, false>(a, causal, has_lens, stream)
              : launch_typed<_Float16, false>(a, causal, has_lens, stream);
}

}  // namespace bsa
