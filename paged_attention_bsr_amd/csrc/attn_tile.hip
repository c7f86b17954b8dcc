// Generic MFMA tile kernel for BSR block-sparse attention on gfx950.
//
// One workgroup processes one planner tile: up to 32 * NW query rows of one
// (row block, kv head) work unit -- the g qo heads of each query token are
// packed as rows, so grouped-query heads share every K/V load -- against the
// keys of a contiguous range of the row block's column blocks
// (flashinfer.sparse BlockSparseAttentionWrapper: BSR mask, GQA head
// grouping; the key loop is ordinary flash-style online softmax).
//
// Per key tile of KT keys:
//   * the whole workgroup gathers K and V rows by block index with 16-byte
//     global loads (keys outside a block's valid length, or past the range,
//     are loaded as zeros and masked), K into a row-major LDS tile whose
//     16-byte chunks are XOR-swizzled by key, V transposed into a padded
//     (head_dim x KT) LDS tile; loads for tile t+1 are in flight while tile t
//     is computed (two LDS buffers, one barrier per tile);
//   * each wave computes S^T = K Q^T for its 32 rows with
//     v_mfma_f32_32x32x16 (K from LDS as the A operand, Q^T held in
//     registers as B), so every lane owns one query row and its row max
//     needs one cross-half exchange only;
//   * causal / valid-length masking runs only on tiles that need it;
//   * online softmax in the log2 domain (scale folded into one FMA);
//   * O^T += V^T P^T with v_mfma_f32_32x32x16, P^T straight from the S^T
//     accumulator registers, so the per-row rescale is a per-lane multiply.
// The result is o = O / l (rounded to the storage type) and
// lse = (m + log2 l) ln 2, or, for a split tile, the fp32 partial (O / l,
// lse) in the workspace for the merge kernel.
#include "device_common.h"
#include "kernels.h"

namespace bsa {

namespace {

constexpr int kD = 128;  // q/k and v/o head dim of this kernel

template <int KT>
struct TileLds {
  static constexpr int kKBytes = KT * kD * 2;       // K: KT rows of 256 B, swizzled chunks
  static constexpr int kVtStride = KT * 2 + 8;      // V^T: one padded row of KT keys per dim
  static constexpr int kVtBytes = kD * kVtStride;
  static constexpr int kTokBytes = KT * 4;          // token of each key slot, -1 = masked
  static constexpr int kBuf = kKBytes + kVtBytes + kTokBytes;
};

template <typename T, int NW, int KT, bool CAUSAL, bool LENS>
__global__ __launch_bounds__(NW * 64) void attn_tile_kernel(AttnArgs a) {
  using Ops = MfmaType<T>;
  using v8 = typename Ops::v8;
  using v4 = typename Ops::v4;
  using L = TileLds<KT>;
  constexpr int NTHR = NW * 64;
  constexpr int KCH = KT * 16 / NTHR;  // 16-byte chunks per thread per tile, for K and for V
  static_assert(KCH >= 1 && KT * 16 % NTHR == 0, "loader shape");
  static_assert(NTHR % KT == 0, "V loader assumes one key per thread");
  constexpr int NKB = KT / 32;

  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * L::kBuf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int ql = lane & 31;

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
  const int npos = (ce - cb) * C;
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
  int qlim = 0x7fffffff;
  if (CAUSAL) {
    const int64_t l = static_cast<int64_t>(qtok) + a.causal_off;
    qlim = l > 0x7fffffff ? 0x7fffffff : (l < -1 ? -1 : static_cast<int>(l));
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

  // ---- key-slot -> token (-1: masked / outside the range)
  auto key_tok = [&](int t) -> int {
    if (t >= npos) return -1;
    const int blk = t / C;
    const int off = t - blk * C;
    const int J = a.cols[cb + blk];
    if (LENS && off >= a.lens[cb + blk]) return -1;
    return J * C + off;
  };

  const T* kbase = static_cast<const T*>(a.k) + static_cast<int64_t>(kvh) * kD;
  const T* vbase = static_cast<const T*>(a.v) + static_cast<int64_t>(kvh) * kD;
  u32x4 kreg[KCH], vreg[KCH];
  int vtok = -1;
  const int vkey = tid % KT;
  auto load_tile = [&](int kt) {
    const int t0 = kt * KT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int key = (tid >> 4) + i * (NTHR / 16);
      const int c = tid & 15;
      const int tok = key_tok(t0 + key);
      kreg[i] = tok >= 0 ? *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(tok) * a.k_stride + c * 8)
                         : u32x4{0, 0, 0, 0};
    }
    vtok = key_tok(t0 + vkey);
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid / KT + i * (NTHR / KT);
      vreg[i] = vtok >= 0 ? *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(vtok) * a.v_stride + c * 8)
                          : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* base = lds + buf * L::kBuf;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int key = (tid >> 4) + i * (NTHR / 16);
      const int c = tid & 15;
      *reinterpret_cast<u32x4*>(base + key * 256 + ((c ^ (key & 7)) << 4)) = kreg[i];
    }
    unsigned char* vt = base + L::kKBytes;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid / KT + i * (NTHR / KT);
      const uint32_t w[4] = {vreg[i][0], vreg[i][1], vreg[i][2], vreg[i][3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t hv = static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16));
        *reinterpret_cast<uint16_t*>(vt + (c * 8 + e) * L::kVtStride + vkey * 2) = hv;
      }
    }
    if (tid < KT) reinterpret_cast<int*>(base + L::kKBytes + L::kVtBytes)[tid] = vtok;
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float sl2 = a.scale_log2;

  if (ntiles > 0) load_tile(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    store_tile(buf);
    __syncthreads();
    if (kt + 1 < ntiles) load_tile(kt + 1);
    if (!wave_active) continue;

    // wave-uniform range of key tokens in this tile (columns are ascending)
    const int t0 = kt * KT;
    const int t1 = (t0 + KT < npos ? t0 + KT : npos) - 1;
    const int blk0 = t0 / C, blk1 = t1 / C;
    const int64_t tok_lo = static_cast<int64_t>(a.cols[cb + blk0]) * C + (t0 - blk0 * C);
    const int64_t tok_hi = static_cast<int64_t>(a.cols[cb + blk1]) * C + (t1 - blk1 * C);
    if (CAUSAL && tok_lo > wave_lim) continue;  // every key of the tile is above this wave's diagonal
    const bool need_mask = LENS || (t0 + KT > npos) || (CAUSAL && tok_hi > wave_lim_lo);

    const unsigned char* kl = lds + buf * L::kBuf;
    const unsigned char* vt = kl + L::kKBytes;
    const int* ktok = reinterpret_cast<const int*>(kl + L::kKBytes + L::kVtBytes);

    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      const int key = kb * 32 + ql;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int c = 2 * ks + half;
        const v8 kf = *reinterpret_cast<const v8*>(kl + key * 256 + ((c ^ (key & 7)) << 4));
        s[kb] = Ops::mfma32(kf, qf[ks], s[kb]);
      }
    }
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int4 tk = *reinterpret_cast<const int4*>(ktok + kb * 32 + 8 * g4 + 4 * half);
          const int tt[4] = {tk.x, tk.y, tk.z, tk.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = tt[e] >= 0 && (!CAUSAL || tt[e] <= qlim);
            if (!ok) s[kb][g4 * 4 + e] = -INFINITY;
          }
        }
      }
    }
    // online softmax (log2 domain)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, xor_lane32(mx));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(fmaf(s[kb][v], sl2, -m_use));
        s[kb][v] = p;
        ls += p;
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      const int kb = ks >> 1;
      const int hv = ks & 1;
      v8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = static_cast<T>(s[kb][hv * 8 + e]);
      const int kcol = kb * 32 + hv * 16 + 4 * half;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const unsigned char* row = vt + (db * 32 + ql) * L::kVtStride;
        const v4 lo = *reinterpret_cast<const v4*>(row + kcol * 2);
        const v4 hi = *reinterpret_cast<const v4*>(row + (kcol + 8) * 2);
        const v8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = Ops::mfma32(vf, pf, oacc[db]);
      }
    }
  }

  // ---- finalize this lane's row
  const float l_tot = l_run + xor_lane32(l_run);
  const float inv = l_tot > 0.f ? a.out_scale / l_tot : 0.f;
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

template <typename T, int NW, int KT>
hipError_t launch_variant(const AttnArgs& a, bool causal, bool lens, hipStream_t st) {
  const dim3 grid(a.num_tiles), block(NW * 64);
  if (causal) {
    if (lens) attn_tile_kernel<T, NW, KT, true, true><<<grid, block, 0, st>>>(a);
    else attn_tile_kernel<T, NW, KT, true, false><<<grid, block, 0, st>>>(a);
  } else {
    if (lens) attn_tile_kernel<T, NW, KT, false, true><<<grid, block, 0, st>>>(a);
    else attn_tile_kernel<T, NW, KT, false, false><<<grid, block, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const AttnArgs& a, int tile_rows, bool causal, bool lens, hipStream_t st) {
  switch (tile_rows) {
    case 32: return launch_variant<T, 1, 32>(a, causal, lens, st);
    case 128: return launch_variant<T, 4, 64>(a, causal, lens, st);
    case 256: return launch_variant<T, 8, 64>(a, causal, lens, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_tile(const AttnArgs& a, bool bf16, int tile_rows, bool causal, bool has_lens,
                            hipStream_t stream) {
  if (a.num_tiles == 0) return hipSuccess;
  return bf16 ? launch_typed<__bf16>(a, tile_rows, causal, has_lens, stream)
              : launch_typed<_Float16>(a, tile_rows, causal, has_lens, stream);
}

}  // namespace bsa
