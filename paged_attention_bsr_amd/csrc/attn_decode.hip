// Paged-decode kernel on gfx950: BSR with R = 1 (one query token per row
// block), block size C a multiple of 16 (C = page size), head_dim 128,
// fp16/bf16, up to 16 qo heads per kv head (flashinfer.sparse
// BlockSparseAttentionWrapper with R = 1, C = page size; the FlashInfer
// BatchDecodeWithPagedKVCacheWrapper workload written as BSR).
//
// Decode reads every unmasked K/V row exactly once and does ~4 flops per
// byte, so the kernel is built around bytes in flight, not arithmetic:
//   * one workgroup = one planner tile = the g query heads of one token
//     and one kv head, over a range of pages; its NW waves take 32-key
//     tiles in turn and merge their softmax states through LDS at the end;
//   * K goes from HBM straight into MFMA A-operand registers (16-byte loads,
//     no LDS); S^T = K Q^T runs on v_mfma_f32_16x16x32 with the g heads as
//     the (zero-padded) 16 columns;
//   * V is staged row-major in a wave-private 8 KB LDS tile (chunks XOR-
//     swizzled by key) and read back transposed with ds_read_b64_tr_b16 as
//     the A operand of O^T += V^T P^T; the key order of S^T's rows is chosen
//     so that P^T comes straight from the S^T accumulators in the order the
//     transposed reads deliver V;
//   * the next tile's K and V loads are issued before the current tile's
//     math (register double buffering), and no workgroup barrier is needed
//     inside the key loop;
//   * keys outside a page's valid length (or past the range) load from a
//     zero row in the workspace, so unused cache slots never reach the
//     arithmetic, and are masked to -inf in the scores.
#include "device_common.h"
#include "kernels.h"

namespace bsa {

namespace {

#ifndef BSA_DECODE_NW
#define BSA_DECODE_NW 4            // waves per workgroup
#endif
#ifndef BSA_DECODE_MIN_WAVES
#define BSA_DECODE_MIN_WAVES 2     // occupancy target (waves per SIMD) given to the register allocator
#endif

constexpr int kD = 128;
constexpr int kKT = 32;                 // keys per tile
constexpr int kVBytes = kKT * kD * 2;   // wave-private V tile

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ u32x4 load_kv(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// LDS byte offset of 16-byte chunk `c` of key row `k` in a V tile.
__device__ __forceinline__ int v_chunk_off(int k, int c) {
  return k * (kD * 2) + ((c ^ (((k & 3) << 1) | (((k >> 3) & 1) << 3))) << 4);
}

template <typename T, int NW, bool CAUSAL, bool LENS, bool POW2C>
__global__ __launch_bounds__(NW * 64, BSA_DECODE_MIN_WAVES) void attn_decode_kernel(AttnArgs a) {
  using Ops = MfmaType<T>;
  using v8 = typename Ops::v8;
  using v4 = typename Ops::v4;

  __shared__ __attribute__((aligned(16))) unsigned char lds[NW * kVBytes];
  __shared__ float red_m[NW][16], red_l[NW][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quad = lane >> 4;
  const int col = lane & 15;

  const int32_t* trec = a.tiles + static_cast<int64_t>(blockIdx.x) * 8;
  const int I = trec[0];
  const int kvh = trec[1];
  const int row0 = trec[2];
  const int nrows = trec[3];
  const int cb = trec[4];
  const int ce = trec[5];
  const int part = trec[6];
  const int C = a.C;
  const int cshift = POW2C ? __builtin_ctz(C) : 0;  // C = 1 << cshift when POW2C
  const int npos = (ce - cb) * C;
  const int ntiles = (npos + kKT - 1) / kKT;
  const int g = a.group;
  const int qtok = I;                     // R = 1
  int64_t lim64 = CAUSAL ? static_cast<int64_t>(qtok) + a.causal_off : 0;
  const int qlim = CAUSAL ? (lim64 > 0x7fffffff ? 0x7fffffff : (lim64 < -1 ? -1 : static_cast<int>(lim64))) : 0;

  // Q^T as the B operand: column `col` is qo head kvh*g + row0 + col (zero beyond nrows)
  const bool col_ok = col < nrows;
  v8 qf[4];
  {
    const T* qp = static_cast<const T*>(a.q) + static_cast<int64_t>(qtok) * a.q_stride +
                  static_cast<int64_t>(kvh * g + row0 + col) * kD + quad * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = col_ok ? *reinterpret_cast<const v8*>(qp + ks * 32) : v8{};
  }

  const T* kbase = static_cast<const T*>(a.k) + static_cast<int64_t>(kvh) * kD;
  const T* vbase = static_cast<const T*>(a.v) + static_cast<int64_t>(kvh) * kD;
  const T* zrow = static_cast<const T*>(a.zero_row);

  // Token of key position t of this tile range (-1 = masked), from the
  // tile's (uniform, scalar-loaded) column blocks and their valid lengths:
  // a 32-key tile spans at most 3 blocks when C >= 16.
  struct TileBlocks {
    int base;              // first key position of the tile's first block
    int J0, J1, J2;        // its first three column blocks (clamped to the range)
    int L0, L1, L2;        // their valid lengths
  };
  const int nblk = ce - cb;
  auto tile_blocks = [&](int kt) {
    TileBlocks b;
    const int t0 = kt * kKT;
    int blk0 = POW2C ? (t0 >> cshift) : t0 / C;
    blk0 = blk0 < nblk ? blk0 : nblk - 1;  // tiles past the end only feed dummy loads
    const int b1 = blk0 + 1 < nblk ? blk0 + 1 : nblk - 1;
    const int b2 = blk0 + 2 < nblk ? blk0 + 2 : nblk - 1;
    b.base = blk0 * C;
    b.J0 = a.cols[cb + blk0];
    b.J1 = a.cols[cb + b1];
    b.J2 = a.cols[cb + b2];
    b.L0 = LENS ? a.lens[cb + blk0] : C;
    b.L1 = LENS ? a.lens[cb + b1] : C;
    b.L2 = LENS ? a.lens[cb + b2] : C;
    return b;
  };
  // branch-free, so every stage issues the same loads and the compiler can
  // wait for exactly the older stage
  auto key_token = [&](const TileBlocks& b, int t) -> int {
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
    bool ok = t < npos;
    if (LENS) ok = ok && off < len;
    if (CAUSAL) ok = ok && tok <= qlim;
    return ok ? tok : -1;
  };

  // per-tile registers: K fragments and V chunks, both indexed (kb, ks):
  // lane (col, quad) holds dims ks*32 + quad*8 .. +8 of key (kb, col)
  struct Stage {
    v8 k[2][4];
    u32x4 v[2][4];
    uint32_t valid[2];  // bit m: key (kb, m) valid
  };
  // key of S^T row m in block kb: 8*(m/4) + 4*kb + m%4
  auto load_stage = [&](Stage& s, int kt, const TileBlocks& b) {
    const int t0 = kt * kKT;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 8 * (col >> 2) + 4 * kb + (col & 3);
      const int tok = key_token(b, t0 + key);
      const T* pk = tok >= 0 ? kbase + static_cast<int64_t>(tok) * a.k_stride : zrow;
      const T* pv = tok >= 0 ? vbase + static_cast<int64_t>(tok) * a.v_stride : zrow;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s.k[kb][ks] = bitcast<v8>(load_kv(pk + ks * 32 + quad * 8));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s.v[kb][ks] = load_kv(pv + ks * 32 + quad * 8);
      const uint64_t bal = __ballot(tok >= 0);
      s.valid[kb] = static_cast<uint32_t>(bal & 0xffffu);
    }
  };

  unsigned char* vl = lds + wave * kVBytes;
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;

  auto compute = [&](const Stage& s) {
    // stage V into this wave's LDS tile (row-major, swizzled chunks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 8 * (col >> 2) + 4 * kb + (col & 3);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<u32x4*>(vl + v_chunk_off(key, ks * 4 + quad)) = s.v[kb][ks];
    }
    // S^T = K Q^T
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[kb] = Ops::mfma16(s.k[kb][ks], qf[ks], sc[kb]);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (!((s.valid[kb] >> (4 * quad + v)) & 1u)) sc[kb][v] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
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
    // O^T += V^T P^T; transposed reads: lane L of this quad reads key row
    // 8*quad + 4*j + L/4 at dims d0 + 4*(L%4) .. +3.
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

  // key loop: this wave's tiles wave, wave + NW, ...; the K/V loads of the
  // next tile and the block ids of the one after are in flight during each
  // tile's math
  // Every stage issues its loads unconditionally (tiles past the end read
  // the zero row), so the wait before each tile's math covers exactly the
  // older stage.
  if (ntiles > 0) {
    Stage s0, s1;
    TileBlocks bA = tile_blocks(wave), bB = tile_blocks(wave + NW);
    load_stage(s0, wave, bA);
    for (int kt = wave; kt < ntiles; kt += 2 * NW) {
      load_stage(s1, kt + NW, bB);
      bA = tile_blocks(kt + 2 * NW);
      compute(s0);
      load_stage(s0, kt + 2 * NW, bA);
      bB = tile_blocks(kt + 3 * NW);
      if (kt + NW < ntiles) compute(s1);
    }
  }

  // ---- merge the waves' states (all waves, every query column)
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  __syncthreads();  // every wave is done with its V tile: reuse LDS for the merge
  float* ob = reinterpret_cast<float*>(lds);  // [NW][16 cols][128 d]
  if (quad == 0) {
    red_m[wave][col] = m_run;
    red_l[wave][col] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<f32x4*>(ob + (wave * 16 + col) * kD + db * 16 + 4 * quad) = oacc[db];
  __syncthreads();
  // thread -> (column, 4 dims): 16 * 32 items over NW * 64 threads
  for (int item = tid; item < 16 * (kD / 4); item += NW * 64) {
    const int cq = item / (kD / 4);
    const int d4 = (item - cq * (kD / 4)) * 4;
    if (cq >= nrows) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][cq]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = fast_exp2(red_m[w][cq] - Mu);
      L += red_l[w][cq] * sc;
      acc += sc * *reinterpret_cast<const f32x4*>(ob + (w * 16 + cq) * kD + d4);
    }
    const float inv = L > 0.f ? a.out_scale / L : 0.f;
    const float lse_v = L > 0.f ? (Mu + __log2f(L)) * kLn2 : -INFINITY;
    const int head = kvh * g + row0 + cq;
    acc *= inv;
    if (part < 0) {
      v4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(acc[e]);
      *reinterpret_cast<v4*>(static_cast<T*>(a.o) + static_cast<int64_t>(qtok) * a.o_stride +
                             static_cast<int64_t>(head) * kD + d4) = out;
      if (d4 == 0 && a.lse) a.lse[static_cast<int64_t>(qtok) * a.num_qo_heads + head] = lse_v;
    } else {
      float* pp = a.part + part;
      *reinterpret_cast<f32x4*>(pp + static_cast<int64_t>(cq) * kD + d4) = acc;
      if (d4 == 0) pp[static_cast<int64_t>(nrows) * kD + cq] = lse_v;
    }
  }
}

template <typename T, int NW, bool POW2C>
hipError_t launch_nw(const AttnArgs& a, bool causal, bool lens, hipStream_t st) {
  const dim3 grid(a.num_tiles), block(NW * 64);
  if (causal) {
    if (lens) attn_decode_kernel<T, NW, true, true, POW2C><<<grid, block, 0, st>>>(a);
    else attn_decode_kernel<T, NW, true, false, POW2C><<<grid, block, 0, st>>>(a);
  } else {
    if (lens) attn_decode_kernel<T, NW, false, true, POW2C><<<grid, block, 0, st>>>(a);
    else attn_decode_kernel<T, NW, false, false, POW2C><<<grid, block, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const AttnArgs& a, bool causal, bool lens, hipStream_t st) {
  if ((a.C & (a.C - 1)) == 0) return launch_nw<T, BSA_DECODE_NW, true>(a, causal, lens, st);
  return launch_nw<T, BSA_DECODE_NW, false>(a, causal, lens, st);
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, bool bf16, bool causal, bool has_lens, hipStream_t stream) {
  if (a.num_tiles == 0) return hipSuccess;
  return bf16 ? launch_typed<__bf16>(a, causal, has_lens, stream)
              : launch_typed<_Float16>(a, causal, has_lens, stream);
}

}  // namespace bsa
