// Host planner for BSR block-sparse attention.
//
// flashinfer.sparse, BlockSparseAttentionWrapper.plan: the structure
// (indptr over MB = ceil_div(M, R) row blocks, indices below NB = N / C,
// optional per-block valid lengths) is turned once into auxiliary tables
// that many runs reuse; kv_splits (None/int/"auto") selects split-KV with
// the partials kept in the float workspace.
//
// The partition rule (pinned bit-exactly by a Python model in the tests):
//  1. cols: per row block, its column blocks in ascending order; with a
//     causal mask, blocks whose first key lies beyond the row block's last
//     allowed key (last token + N - M) are dropped.
//  2. A work unit is (row block I, kv head h): rows_I * g query rows in
//     token-major order (row r = token I*R + r / g, qo head h*g + r % g).
//     It is cut into row tiles of tile_rows consecutive rows; a causal row
//     tile only keeps the prefix of cols whose first key is within its own
//     last token's limit.
//  3. Work of a row tile = key positions x ceil(nrows / 32).
//  4. Splits s: kv_splits = 1 -> 1; k > 1 -> min(k, #blocks); 0 -> auto:
//     chunk = ceil(total work / (kAutoTilesPerCu * num_cus)),
//     s = ceil(work / chunk) clamped to [1, min(#blocks, kMaxSplits,
//     max(1, keys / kAutoMinSplitKeys))].
//  5. Boundaries b_j (0 < j < s): first block index p with
//     prefix_keys[p] * s >= j * keys, then forced strictly increasing and
//     leaving at least one block per later split.
//  6. Tiles are emitted in (I, row tile, h, split) order, then stably sorted
//     by descending work (longest processing time first); workgroup t runs
//     tile t.
//  Per-head structure (block_mask or q2k selections): every kv head has its
//     own column lists (step 1 per kv head, then per row block), row tiles
//     are made per (kv head, row block) in that order and each is emitted
//     for its own head only (G = 1 below); the rest is unchanged.
//  Decode kernel: a workgroup takes G = decode_heads_per_wg(Hkv) kv heads at
//     once, so the unit of steps 4-6 is (I, head group gi) and every piece
//     emits G tiles (heads gi*G .. gi*G+G-1, same blocks) as one group; head
//     i's partial of piece j of s is at base + (i*s + j) * psize.  Groups are
//     sorted as in 6 and workgroup t runs group t, except with kv_splits = 0:
//     then the partition is balanced over W = min(kDecodeWgPerCu * num_cus,
//     max(1, K / kBalancedMinKeys)) resident workgroups, K = total keys over
//     all units taken in (I, gi) order.  The block starting at key position X
//     of that sequence goes to workgroup floor(X * W / K), a unit without keys
//     to the workgroup of its position (at most W - 1); a unit's maximal runs
//     of blocks with one workgroup are its pieces, emitted in order, which is
//     workgroup order.
//  Element masks (mask of the BSR blocks, or variable block sizes mapped onto
//     a fixed R x C grid): the structure and the partition are those of the
//     blocks; the masks become bit planes over the column lists (Plan::mbits)
//     that the tile kernel ANDs into each key tile.  A mask of the BSR form
//     follows its block through the sort of step 1 and turns the causal flag
//     off; a variable-block map first marks every fixed block that a set
//     variable block touches (a per-kv-head block mask), and each bit of such
//     a block is then looked up through the token -> variable block maps.
// Kernel choice: sparse-MLA shape -> MLA kernel (64-row tiles); R = 1 with
// g <= 16 and C >= 16 -> decode kernel (16-row tiles, i.e. one per unit);
// otherwise the generic tile kernel with 32, 128 or 256-row tiles for units
// of <= 32, <= 128 or more rows; 128 also for larger units when 256-row tiles
// would leave fewer than kTileSmallGridPerCu tiles per CU.
#include "planner.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <numeric>

namespace bsa {

namespace {

std::atomic<uint64_t> g_next_plan_id{1};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

bool is_mla_shape(const bsa_plan_desc_t& d) {
  return d.kv_dtype == BSA_FP8_E4M3 && d.head_dim_qk != 128;
}

bsa_status_t fail(std::string& err, bsa_status_t st, const std::string& msg) {
  err = msg;
  return st;
}

// Where element visibility inside blocks comes from.
struct MaskSrc {
  int kind = 0;                    // 0: whole blocks; 1: masks of the BSR blocks; 2: variable blocks
  const uint8_t* mask = nullptr;   // kind 1: entry (p*R + r)*C + c of BSR block p
  bool packed = false;             // kind 1: eight entries a byte, least significant bit first
  const uint8_t* vmap = nullptr;   // kind 2: [kv head][var row block][var col block]
  int64_t vmb = 0, vnb = 0;
  std::vector<std::vector<int32_t>> row_block, col_block;  // kind 2: per kv head, token -> variable block
};

bsa_status_t build_plan_impl(const bsa_plan_desc_t& desc, int32_t num_cus, Plan& P, std::string& err,
                             const MaskSrc& ms) {
  const bsa_plan_desc_t& d = desc;
  // ---- validation of sizes and structure (plan() parameter contract)
  if (d.R < 1 || d.C < 1) return fail(err, BSA_ERR_INVALID_ARGUMENT, "R and C must be >= 1");
  if (d.M < 0 || d.N < 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "M and N must be >= 0");
  if (d.M > INT32_MAX || d.N > INT32_MAX)
    return fail(err, BSA_ERR_UNSUPPORTED, "M and N above 2^31 - 1 are not supported");
  if (d.N % d.C != 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "N must be divisible by C");
  if (d.num_qo_heads < 1 || d.num_kv_heads < 1)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
  if (d.num_qo_heads % d.num_kv_heads != 0)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "num_qo_heads must be a multiple of num_kv_heads");
  if (d.head_dim_qk < 1 || d.head_dim_vo < 1)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "head dims must be >= 1");
  if (d.kv_splits < 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "kv_splits must be >= 0");
  if (num_cus < 1) return fail(err, BSA_ERR_INVALID_ARGUMENT, "num_cus must be >= 1");
  if (!(d.q_descale > 0.f) || !(d.k_descale > 0.f) || !(d.v_descale > 0.f) ||
      !std::isfinite(d.q_descale) || !std::isfinite(d.k_descale) || !std::isfinite(d.v_descale))
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "descales must be finite and > 0");
  if (!std::isfinite(d.sm_scale)) return fail(err, BSA_ERR_INVALID_ARGUMENT, "sm_scale must be finite");

  const int64_t MB = ceil_div(d.M, d.R);
  const int64_t NB = d.N / d.C;
  // The structure as one CSR per structure head: HS = 1 (the BSR indptr /
  // indices, shared by every kv head) or HS = num_kv_heads (block_mask or
  // q2k selections, one list per kv head).  List (hs, I) is
  // sidx[sptr[hs * MB + I] .. sptr[hs * MB + I + 1]).
  const bool per_head = d.block_mask || d.q2k_indices;
  const int32_t g0 = d.num_qo_heads / d.num_kv_heads;
  const int64_t HS = per_head ? d.num_kv_heads : 1;
  std::vector<int64_t> sptr(static_cast<size_t>(HS * MB + 1), 0);
  std::vector<int32_t> sidx;
  if (!per_head) {
    if (!d.indptr) return fail(err, BSA_ERR_INVALID_ARGUMENT, "indptr is NULL");
    if (d.indptr[0] != 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "indptr[0] must be 0");
    for (int64_t I = 0; I < MB; ++I)
      if (d.indptr[I + 1] < d.indptr[I])
        return fail(err, BSA_ERR_INVALID_ARGUMENT, "indptr must be non-decreasing");
    const int64_t nnz0 = d.indptr[MB];
    if (nnz0 > 0 && !d.indices) return fail(err, BSA_ERR_INVALID_ARGUMENT, "indices is NULL");
    for (int64_t I = 0; I <= MB; ++I) sptr[I] = d.indptr[I];
    sidx.assign(d.indices, d.indices + nnz0);
  } else {
    if (d.block_mask && d.q2k_indices)
      return fail(err, BSA_ERR_INVALID_ARGUMENT, "block_mask and q2k_indices are mutually exclusive");
    if (d.struct_heads != d.num_kv_heads && d.struct_heads != d.num_qo_heads)
      return fail(err, BSA_ERR_INVALID_ARGUMENT, "struct_heads must be num_kv_heads or num_qo_heads");
    if (d.q2k_indices && d.q2k_topk < 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "q2k_topk must be >= 0");
    // the selected blocks of structure head sh, row block I, in given order
    std::vector<int32_t> row, other;
    auto get_row = [&](int64_t sh, int64_t I, std::vector<int32_t>& out) -> bool {
      out.clear();
      if (d.block_mask) {
        const uint8_t* m = d.block_mask + (sh * MB + I) * NB;
        for (int64_t J = 0; J < NB; ++J)
          if (m[J]) out.push_back(static_cast<int32_t>(J));
        return true;
      }
      const int64_t n = d.q2k_num ? d.q2k_num[sh * MB + I] : d.q2k_topk;
      if (n < 0 || n > d.q2k_topk) return false;
      const int32_t* q = d.q2k_indices + (sh * MB + I) * d.q2k_topk;
      out.assign(q, q + n);
      return true;
    };
    const int32_t per_kv = d.struct_heads == d.num_kv_heads ? 1 : g0;
    for (int64_t h = 0; h < HS; ++h) {
      for (int64_t I = 0; I < MB; ++I) {
        if (!get_row(h * per_kv, I, row))
          return fail(err, BSA_ERR_INVALID_ARGUMENT, "q2k_num entries must lie in [0, q2k_topk]");
        // the qo heads of one kv head must select the same blocks
        for (int32_t j = 1; j < per_kv; ++j) {
          if (!get_row(h * per_kv + j, I, other))
            return fail(err, BSA_ERR_INVALID_ARGUMENT, "q2k_num entries must lie in [0, q2k_topk]");
          std::vector<int32_t> a = row, b = other;
          std::sort(a.begin(), a.end());
          std::sort(b.begin(), b.end());
          if (a != b)
            return fail(err, BSA_ERR_INVALID_ARGUMENT,
                        "the qo heads of one kv head must select the same key blocks");
        }
        sidx.insert(sidx.end(), row.begin(), row.end());
        sptr[h * MB + I + 1] = static_cast<int64_t>(sidx.size());
      }
    }
  }
  const int64_t nnz = static_cast<int64_t>(sidx.size());
  std::vector<uint8_t> seen(static_cast<size_t>(NB), 0);
  for (int64_t u = 0; u < HS * MB; ++u) {
    for (int64_t p = sptr[u]; p < sptr[u + 1]; ++p) {
      const int32_t J = sidx[p];
      if (J < 0 || J >= NB) return fail(err, BSA_ERR_INVALID_ARGUMENT, "indices must lie in [0, NB)");
      if (seen[J]) return fail(err, BSA_ERR_INVALID_ARGUMENT, "duplicate column index within a row block");
      seen[J] = 1;
    }
    for (int64_t p = sptr[u]; p < sptr[u + 1]; ++p) seen[sidx[p]] = 0;
  }
  if (d.kv_block_lens) {
    for (int64_t J = 0; J < NB; ++J)
      if (d.kv_block_lens[J] < 1 || d.kv_block_lens[J] > d.C)
        return fail(err, BSA_ERR_INVALID_ARGUMENT, "kv_block_lens entries must lie in [1, C]");
  }

  // a mask given per element replaces the causal flag
  const bool causal = d.causal && ms.kind != 1;

  // ---- kernel selection (supported dtype / head_dim sets)
  const int32_t g = d.num_qo_heads / d.num_kv_heads;
  int32_t kernel, tile_rows, key_tile;
  if (is_mla_shape(d)) {
    if (d.q_dtype != BSA_BF16 || d.o_dtype != BSA_BF16 || d.head_dim_qk != 576 ||
        d.head_dim_vo != 512 || d.num_kv_heads != 1 || d.R != 1)
      return fail(err, BSA_ERR_UNSUPPORTED,
                  "fp8 e4m3 KV is supported for the sparse-MLA shape only: bf16 q/o, head_dim_qk 576, "
                  "head_dim_vo 512, one kv head, R = 1");
    kernel = BSA_KERNEL_MLA;
    tile_rows = 64;
    key_tile = 32;
  } else {
    const bool kv8 = d.kv_dtype == BSA_FP8_E4M3;
    const bool f16 = d.q_dtype == BSA_F16 && (d.kv_dtype == BSA_F16 || kv8) && d.o_dtype == BSA_F16;
    const bool bf16 = d.q_dtype == BSA_BF16 && (d.kv_dtype == BSA_BF16 || kv8) && d.o_dtype == BSA_BF16;
    if (!(f16 || bf16))
      return fail(err, BSA_ERR_UNSUPPORTED,
                  "q/o must both be fp16 or both bf16, with k/v in the same type or fp8 e4m3, for this head_dim");
    if (d.head_dim_qk != 128 || d.head_dim_vo != 128)
      return fail(err, BSA_ERR_UNSUPPORTED, "head_dim 128 (q/k and v/o) is the supported size");
    if (!kv8 && (d.q_descale != 1.f || d.k_descale != 1.f || d.v_descale != 1.f))
      return fail(err, BSA_ERR_UNSUPPORTED, "dequant scales apply to fp8 KV only");
    if (d.R == 1 && g <= 16 && d.C >= 16 && ms.kind == 0) {
      kernel = BSA_KERNEL_DECODE;
      tile_rows = 16;
      key_tile = 32;
    } else {
      kernel = BSA_KERNEL_TILE;
      const int64_t umax = std::min<int64_t>(d.R, std::max<int64_t>(d.M, 1)) * g;
      if (umax <= 32) {
        tile_rows = 32;
      } else if (umax <= 128 || kTileMaxRows == 128) {
        tile_rows = 128;
      } else {
        const int64_t rows_last = d.M - (MB - 1) * d.R;
        const int64_t n256 = ((MB - 1) * ceil_div((int64_t)d.R * g, 256) + ceil_div(rows_last * g, 256)) *
                             d.num_kv_heads;
        tile_rows = n256 < (int64_t)kTileSmallGridPerCu * num_cus ? 128 : 256;
      }
      key_tile = tile_rows == 32 ? 32 : 64;
    }
  }

  P.d = d;
  // the host arrays are read during planning only
  P.d.indptr = P.d.indices = P.d.kv_block_lens = P.d.q2k_indices = P.d.q2k_num = nullptr;
  P.d.block_mask = P.d.mask = nullptr;
  P.d.block_row_sz = P.d.block_col_sz = nullptr;
  P.d.causal = causal;
  P.MB = MB;
  P.NB = NB;
  P.group = g;
  P.sm_scale = d.sm_scale > 0.f ? d.sm_scale : static_cast<float>(1.0 / std::sqrt((double)d.head_dim_qk));
  P.kernel = kernel;
  P.tile_rows = tile_rows;
  P.key_tile = key_tile;
  P.num_cus = num_cus;
  P.id = g_next_plan_id.fetch_add(1);

  auto blen = [&](int32_t J) -> int64_t { return d.kv_block_lens ? d.kv_block_lens[J] : d.C; };
  const int64_t off = d.N - d.M;  // causal offset: key j allowed for query i iff j <= i + off

  // ---- 1. sorted, causally trimmed column lists
  // (per structure head, then per row block: list hs * MB + I)
  // (csrc: the sidx position each entry came from, for masks of the BSR blocks)
  std::vector<int64_t> bptr(static_cast<size_t>(HS * MB + 1), 0);
  std::vector<int64_t> csrc, ord;
  P.cols.clear();
  P.cols.reserve(static_cast<size_t>(nnz));
  for (int64_t u = 0; u < HS * MB; ++u) {
    const int64_t I = u % MB;
    ord.resize(static_cast<size_t>(sptr[u + 1] - sptr[u]));
    std::iota(ord.begin(), ord.end(), sptr[u]);
    std::sort(ord.begin(), ord.end(), [&](int64_t x, int64_t y) { return sidx[x] < sidx[y]; });
    const int64_t last_tok = std::min<int64_t>(d.M, (I + 1) * d.R) - 1;
    for (int64_t x : ord) {
      const int32_t J = sidx[x];
      if (causal && static_cast<int64_t>(J) * d.C > last_tok + off) break;
      P.cols.push_back(J);
      if (ms.kind == 1) csrc.push_back(x);
    }
    bptr[u + 1] = static_cast<int64_t>(P.cols.size());
  }
  // valid length of each column-list entry (parallel to cols), so kernels
  // read a block's length with the same index as the block itself
  P.lens.clear();
  if (d.kv_block_lens) {
    P.lens.resize(P.cols.size());
    for (size_t p = 0; p < P.cols.size(); ++p) P.lens[p] = d.kv_block_lens[P.cols[p]];
  }
  // element-mask bit planes (layout in planner.h)
  P.mbits.clear();
  P.mask_plane_words = 0;
  if (ms.kind != 0) {
    const int64_t W = ceil_div(static_cast<int64_t>(P.cols.size()) * d.C, 32) + 8;
    if (static_cast<int64_t>(d.R) * W > (int64_t{1} << 29))
      return fail(err, BSA_ERR_UNSUPPORTED, "element-mask bit planes would exceed 2 GiB");
    P.mask_plane_words = W;
    P.mbits.assign(static_cast<size_t>(d.R * W), 0u);
    for (int64_t u = 0; u < HS * MB; ++u) {
      const int64_t I = u % MB, hs = u / MB;
      const int64_t rows_I = std::min<int64_t>(d.R, d.M - I * d.R);
      for (int64_t e = bptr[u]; e < bptr[u + 1]; ++e) {
        const int64_t J = P.cols[e];
        for (int64_t r = 0; r < rows_I; ++r) {
          uint32_t* plane = P.mbits.data() + r * W;
          const uint8_t* vrow =
              ms.kind == 2 ? ms.vmap + (hs * ms.vmb + ms.row_block[hs][I * d.R + r]) * ms.vnb : nullptr;
          for (int64_t c = 0; c < d.C; ++c) {
            bool bit;
            if (ms.kind == 1) {
              const int64_t i = (csrc[e] * d.R + r) * d.C + c;
              bit = ms.packed ? ((ms.mask[i >> 3] >> (i & 7)) & 1) != 0 : ms.mask[i] != 0;
            } else {
              bit = vrow[ms.col_block[hs][J * d.C + c]] != 0;
            }
            const int64_t pos = e * d.C + c;
            if (bit) plane[pos >> 5] |= 1u << (pos & 31);
          }
        }
      }
    }
  }

  // ---- 2./3. row tiles with their (prefix) column ranges and work
  // (hs = the structure head of the row tile's columns: 0 when shared)
  struct RowTile {
    int64_t I, row0, nrows, cb, n, keys, work, hs;
  };
  std::vector<RowTile> rts;
  std::vector<int64_t> pref;  // prefix key counts, reused
  for (int64_t u = 0; u < HS * MB; ++u) {
    const int64_t I = u % MB;
    const int64_t rows_I = std::min<int64_t>(d.R, d.M - I * d.R);
    const int64_t U = rows_I * g;
    for (int64_t r0 = 0; r0 < U; r0 += tile_rows) {
      const int64_t nr = std::min<int64_t>(tile_rows, U - r0);
      int64_t n = bptr[u + 1] - bptr[u];
      if (causal) {
        const int64_t lim = I * d.R + (r0 + nr - 1) / g + off;
        int64_t k = 0;
        while (k < n && static_cast<int64_t>(P.cols[bptr[u] + k]) * d.C <= lim) ++k;
        n = k;
      }
      int64_t keys = 0;
      for (int64_t k = 0; k < n; ++k) keys += blen(P.cols[bptr[u] + k]);
      rts.push_back({I, r0, nr, bptr[u], n, keys, keys * ceil_div(nr, 32), u / MB});
    }
  }

  // Tiles come in groups: one group per (row tile, head group, key range)
  // holds the tiles of G consecutive kv heads (G = 1 except for the decode
  // kernel, whose workgroup gives each of its waves one kv head of the group).
  // With a per-head structure every kv head has its own columns, so groups
  // hold one head and a row tile serves only its own head.
  const int32_t G = kernel == BSA_KERNEL_DECODE && !per_head ? decode_heads_per_wg(d.num_kv_heads) : 1;
  const int32_t NG = d.num_kv_heads / G;
  const int32_t units_per_rt = per_head ? 1 : NG;  // head groups each row tile is emitted for
  auto group_of = [&](const RowTile& rt, int32_t k) -> int32_t {
    return per_head ? static_cast<int32_t>(rt.hs) : k;
  };
  struct TileRec {
    int32_t f[kTileInts];
  };
  struct GroupRec {
    size_t first;   // its G tiles are recs[first .. first + G)
    int64_t work;   // keys x ceil(rows / 32)
    int64_t wg;     // workgroup (balanced partition)
  };
  std::vector<TileRec> recs;
  std::vector<GroupRec> groups;
  P.merges.clear();
  int64_t part = 0;
  int32_t max_s = 1;
  const int64_t dv = d.head_dim_vo;
  P.valid_pairs = 0;
  // Tiles of head group gi of row tile rt cut at blocks b[0] < ... < b[s]
  // (pref = the row tile's prefix key counts).  Head i's partial of piece j
  // sits at base + (i * s + j) * psize; false if the partials overflow.
  auto emit_unit = [&](const RowTile& rt, int32_t gi, const int64_t* b, const int64_t* wg, int64_t s) {
    const int64_t psize = round_up(rt.nrows * (dv + 1), 64);
    const int64_t base = part;
    for (int64_t j = 0; j < s; ++j) {
      const int64_t keys_j = pref[b[j + 1]] - pref[b[j]];
      groups.push_back({recs.size(), keys_j * ceil_div(rt.nrows, 32), wg ? wg[j] : 0});
      for (int32_t i = 0; i < G; ++i) {
        TileRec r{};
        r.f[T_ROWBLOCK] = static_cast<int32_t>(rt.I);
        r.f[T_KVHEAD] = gi * G + i;
        r.f[T_ROW0] = static_cast<int32_t>(rt.row0);
        r.f[T_NROWS] = static_cast<int32_t>(rt.nrows);
        r.f[T_COLB] = static_cast<int32_t>(rt.cb + b[j]);
        r.f[T_COLE] = static_cast<int32_t>(rt.cb + b[j + 1]);
        r.f[T_PART] = s > 1 ? static_cast<int32_t>(base + (i * s + j) * psize) : -1;
        r.f[T_KEYS] = static_cast<int32_t>(keys_j);
        recs.push_back(r);
        P.valid_pairs += keys_j * rt.nrows;
      }
    }
    max_s = std::max<int32_t>(max_s, static_cast<int32_t>(s));
    if (s > 1) {
      part += G * s * psize;
      if (part > INT32_MAX) return false;
      for (int32_t i = 0; i < G; ++i) {
        int32_t m[kMergeInts] = {static_cast<int32_t>(rt.I), gi * G + i, static_cast<int32_t>(rt.row0),
                                 static_cast<int32_t>(rt.nrows), static_cast<int32_t>(base + i * s * psize),
                                 static_cast<int32_t>(s), static_cast<int32_t>(psize), 0};
        P.merges.insert(P.merges.end(), m, m + kMergeInts);
      }
    }
    return true;
  };
  auto row_prefix = [&](const RowTile& rt) {
    pref.assign(static_cast<size_t>(rt.n + 1), 0);
    for (int64_t k = 0; k < rt.n; ++k) pref[k + 1] = pref[k] + blen(P.cols[rt.cb + k]);
  };
  std::vector<int64_t> cut, cut_wg;
  int64_t W = 0;
  if (kernel == BSA_KERNEL_DECODE && d.kv_splits == 0) {
    // ---- 4.-6. balanced partition over resident workgroups
    int64_t K = 0;
    for (const auto& rt : rts) K += rt.keys * units_per_rt;
    W = std::max<int64_t>(1, std::min<int64_t>((int64_t)kDecodeWgPerCu * num_cus, K / kBalancedMinKeys));
    auto wg_of = [&](int64_t X) -> int64_t {
      if (K == 0) return 0;
      const int64_t w = static_cast<int64_t>((static_cast<__int128>(X) * W) / K);
      return std::min<int64_t>(w, W - 1);
    };
    int64_t X = 0;
    for (const auto& rt : rts) {
      row_prefix(rt);
      for (int32_t k = 0; k < units_per_rt; ++k) {
        const int32_t gi = group_of(rt, k);
        // maximal runs of blocks with one workgroup
        cut.assign(1, 0);
        cut_wg.assign(1, wg_of(X));
        for (int64_t k = 1; k < rt.n; ++k) {
          const int64_t wk = wg_of(X + pref[k]);
          if (wk != cut_wg.back()) {
            cut.push_back(k);
            cut_wg.push_back(wk);
          }
        }
        cut.push_back(rt.n);
        if (!emit_unit(rt, gi, cut.data(), cut_wg.data(), static_cast<int64_t>(cut_wg.size())))
          return fail(err, BSA_ERR_UNSUPPORTED, "split partials exceed 2^31 floats");
        X += rt.keys;
      }
    }
  } else {
    // ---- 4. split counts
    int64_t total_work = 0;
    for (const auto& rt : rts) total_work += rt.work * (per_head ? 1 : d.num_kv_heads);
    const int64_t chunk = std::max<int64_t>(1, ceil_div(total_work, (int64_t)kAutoTilesPerCu * num_cus));
    for (const auto& rt : rts) {
      int64_t s = 1;
      if (d.kv_splits > 1) {
        s = std::min<int64_t>(d.kv_splits, rt.n);
      } else if (d.kv_splits == 0) {
        const int64_t cap = std::min<int64_t>({rt.n, (int64_t)kMaxSplits,
                                               std::max<int64_t>(1, rt.keys / kAutoMinSplitKeys)});
        s = std::min<int64_t>(ceil_div(rt.work, chunk), cap);
      }
      s = std::max<int64_t>(1, s);
      // ---- 5. boundaries
      row_prefix(rt);
      cut.assign(static_cast<size_t>(s + 1), 0);
      cut[s] = rt.n;
      for (int64_t j = 1; j < s; ++j) {
        int64_t p = 0;
        while (p < rt.n && pref[p] * s < j * rt.keys) ++p;
        p = std::max<int64_t>(p, cut[j - 1] + 1);
        p = std::min<int64_t>(p, rt.n - (s - j));
        cut[j] = p;
      }
      for (int32_t k = 0; k < units_per_rt; ++k)
        if (!emit_unit(rt, group_of(rt, k), cut.data(), nullptr, s))
          return fail(err, BSA_ERR_UNSUPPORTED, "split partials exceed 2^31 floats");
    }
    // ---- 6. longest first, one group per workgroup
    std::stable_sort(groups.begin(), groups.end(),
                     [](const GroupRec& a, const GroupRec& b) { return a.work > b.work; });
    W = static_cast<int64_t>(groups.size());
    for (int64_t w = 0; w < W; ++w) groups[static_cast<size_t>(w)].wg = w;
  }
  if (recs.size() > static_cast<size_t>(INT32_MAX / kTileInts))
    return fail(err, BSA_ERR_UNSUPPORTED, "too many tiles");
  P.tiles.clear();
  P.tiles.reserve(recs.size() * kTileInts);
  P.wg_ptr.assign(static_cast<size_t>(W + 1), 0);
  for (const auto& gr : groups) {
    for (int32_t i = 0; i < G; ++i) P.tiles.insert(P.tiles.end(), recs[gr.first + i].f, recs[gr.first + i].f + kTileInts);
    P.wg_ptr[static_cast<size_t>(gr.wg + 1)] += G;
  }
  for (int64_t w = 0; w < W; ++w) P.wg_ptr[w + 1] += P.wg_ptr[w];
  P.heads_per_wg = G;
  P.max_splits = max_s;
  P.partial_floats = part;

  // ---- workspace layout: [tiles | merges | cols | lens | wg_ptr | zero row | mask bits] then partials
  int64_t o = 0;
  P.off_tiles = o;
  o = round_up(o + (int64_t)P.tiles.size() * 4, 256);
  P.off_merges = o;
  o = round_up(o + (int64_t)P.merges.size() * 4, 256);
  P.off_cols = o;
  o = round_up(o + (int64_t)P.cols.size() * 4, 256);
  P.off_lens = o;
  o = round_up(o + (int64_t)P.lens.size() * 4, 256);
  P.off_wg = o;
  o = round_up(o + (int64_t)P.wg_ptr.size() * 4, 256);
  P.off_zero = o;  // zero row: masked keys load from here
  o = round_up(o + 1024, 256);
  P.off_mbits = o;
  o = round_up(o + (int64_t)P.mbits.size() * 4, 256);
  P.table_bytes = std::max<int64_t>(o, 256);
  P.partial_bytes = round_up(P.partial_floats * 4, 256);
  P.workspace_bytes = P.table_bytes + P.partial_bytes;
#ifdef BSA_TRACE
  // trace build: one record of kTraceInts int32 per tile after the partials
  P.workspace_bytes += round_up(static_cast<int64_t>(P.tiles.size() / kTileInts) * kTraceInts * 4, 256);
#endif
  P.table_blob.assign(static_cast<size_t>(P.table_bytes), 0);
  auto put = [&](int64_t at, const std::vector<int32_t>& v) {
    if (!v.empty()) std::copy(reinterpret_cast<const uint8_t*>(v.data()),
                              reinterpret_cast<const uint8_t*>(v.data()) + v.size() * 4,
                              P.table_blob.begin() + at);
  };
  put(P.off_tiles, P.tiles);
  put(P.off_merges, P.merges);
  put(P.off_cols, P.cols);
  put(P.off_lens, P.lens);
  put(P.off_wg, P.wg_ptr);
  if (!P.mbits.empty())
    std::copy(reinterpret_cast<const uint8_t*>(P.mbits.data()),
              reinterpret_cast<const uint8_t*>(P.mbits.data()) + P.mbits.size() * 4, P.table_blob.begin() + P.off_mbits);
  return BSA_OK;
}

}  // namespace

bsa_status_t build_plan(const bsa_plan_desc_t& desc, int32_t num_cus, Plan& P, std::string& err) {
  const bool var = desc.block_row_sz || desc.block_col_sz;
  MaskSrc ms;
  if (!desc.mask && !var) return build_plan_impl(desc, num_cus, P, err, ms);
  if (desc.head_dim_qk != 128 || desc.head_dim_vo != 128)
    return fail(err, BSA_ERR_UNSUPPORTED, "element masks and variable block sizes are supported for head_dim 128");
  if (desc.kv_block_lens)
    return fail(err, BSA_ERR_INVALID_ARGUMENT,
                "kv_block_lens must be NULL with element masks or variable block sizes (lengths belong in the mask)");
  if (desc.mask && var)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "mask applies to fixed-size BSR blocks, not to variable block sizes");
  if (desc.mask) {
    if (desc.block_mask || desc.q2k_indices)
      return fail(err, BSA_ERR_INVALID_ARGUMENT,
                  "element masks apply to the BSR form (indptr / indices), not to block_mask or q2k selections");
    if (desc.mask_packed != 0 && desc.mask_packed != 1)
      return fail(err, BSA_ERR_INVALID_ARGUMENT, "mask_packed must be 0 or 1");
    ms.kind = 1;
    ms.mask = desc.mask;
    ms.packed = desc.mask_packed != 0;
    return build_plan_impl(desc, num_cus, P, err, ms);
  }
  // ---- variable block sizes -> per-kv-head fixed blocks with element masks
  if (!desc.block_row_sz || !desc.block_col_sz || !desc.block_mask)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "variable block sizes need block_row_sz, block_col_sz and block_mask");
  if (desc.q2k_indices)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "q2k selections do not combine with variable block sizes");
  if (desc.num_kv_heads < 1 || desc.num_qo_heads < 1 || desc.num_qo_heads % desc.num_kv_heads != 0)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "num_qo_heads must be a positive multiple of num_kv_heads");
  if (desc.struct_heads != desc.num_kv_heads)
    return fail(err, BSA_ERR_INVALID_ARGUMENT,
                "variable block sizes take one pattern per kv head (struct_heads = num_kv_heads)");
  if (desc.var_row_blocks < 1 || desc.var_col_blocks < 1)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "var_row_blocks and var_col_blocks must be >= 1");
  if (desc.M < 0 || desc.N < 0 || desc.M > INT32_MAX || desc.N > INT32_MAX)
    return fail(err, BSA_ERR_INVALID_ARGUMENT, "M and N must lie in [0, 2^31)");
  if (desc.R < 0 || desc.C < 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "R and C must be >= 0");
  const int64_t H = desc.num_kv_heads, VMB = desc.var_row_blocks, VNB = desc.var_col_blocks;
  for (int64_t h = 0; h < H; ++h) {
    int64_t sr = 0, sc = 0;
    for (int64_t a = 0; a < VMB; ++a) {
      if (desc.block_row_sz[h * VMB + a] < 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "block sizes must be >= 0");
      sr += desc.block_row_sz[h * VMB + a];
    }
    for (int64_t b = 0; b < VNB; ++b) {
      if (desc.block_col_sz[h * VNB + b] < 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "block sizes must be >= 0");
      sc += desc.block_col_sz[h * VNB + b];
    }
    if (sr != desc.M || sc != desc.N)
      return fail(err, BSA_ERR_INVALID_ARGUMENT,
                  "every kv head's block_row_sz must sum to M and its block_col_sz to N");
  }
  // Default grid: R*g = 128 query rows per row block (one 4-wave tile); C the
  // largest power of two up to min(64, a quarter of the mean non-empty column
  // block) that divides N -- finer blocks waste fewer masked keys, coarser ones
  // keep whole key tiles inside a block.
  const int64_t g = desc.num_qo_heads / desc.num_kv_heads;
  int32_t C = desc.C;
  if (C == 0) {
    int64_t nonempty = 0;
    for (int64_t i = 0; i < H * VNB; ++i) nonempty += desc.block_col_sz[i] > 0;
    const int64_t quarter = nonempty > 0 ? desc.N * H / nonempty / 4 : 64;
    C = 64;
    while (C > 1 && (C > quarter || desc.N % C != 0)) C /= 2;
  }
  const int32_t R = desc.R > 0 ? desc.R : static_cast<int32_t>(std::max<int64_t>(1, 128 / g));
  if (desc.N % C != 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "N must be divisible by C");
  const int64_t MB = ceil_div(desc.M, R), NB = desc.N / C;
  ms.kind = 2;
  ms.vmap = desc.block_mask;
  ms.vmb = VMB;
  ms.vnb = VNB;
  ms.row_block.assign(static_cast<size_t>(H), {});
  ms.col_block.assign(static_cast<size_t>(H), {});
  std::vector<uint8_t> fixed(static_cast<size_t>(H * MB * NB), 0);
  std::vector<int64_t> c0(static_cast<size_t>(VNB + 1));
  for (int64_t h = 0; h < H; ++h) {
    auto& rb = ms.row_block[h];
    auto& cbk = ms.col_block[h];
    rb.reserve(static_cast<size_t>(desc.M));
    cbk.reserve(static_cast<size_t>(desc.N));
    for (int64_t a = 0; a < VMB; ++a) rb.insert(rb.end(), desc.block_row_sz[h * VMB + a], static_cast<int32_t>(a));
    c0[0] = 0;
    for (int64_t b = 0; b < VNB; ++b) {
      cbk.insert(cbk.end(), desc.block_col_sz[h * VNB + b], static_cast<int32_t>(b));
      c0[b + 1] = c0[b] + desc.block_col_sz[h * VNB + b];
    }
    int64_t r0 = 0;
    for (int64_t a = 0; a < VMB; ++a) {
      const int64_t r1 = r0 + desc.block_row_sz[h * VMB + a];
      for (int64_t b = 0; r1 > r0 && b < VNB; ++b) {
        if (!desc.block_mask[(h * VMB + a) * VNB + b] || c0[b + 1] == c0[b]) continue;
        for (int64_t I = r0 / R; I <= (r1 - 1) / R; ++I)
          for (int64_t J = c0[b] / C; J <= (c0[b + 1] - 1) / C; ++J) fixed[(h * MB + I) * NB + J] = 1;
      }
      r0 = r1;
    }
  }
  bsa_plan_desc_t dl = desc;
  dl.R = R;
  dl.C = C;
  dl.indptr = dl.indices = nullptr;
  dl.block_mask = fixed.data();
  dl.struct_heads = desc.num_kv_heads;
  dl.block_row_sz = dl.block_col_sz = nullptr;
  return build_plan_impl(dl, num_cus, P, err, ms);
}

}  // namespace bsa
