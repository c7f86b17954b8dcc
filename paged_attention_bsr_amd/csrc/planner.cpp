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
//     by descending work (longest processing time first).
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
  return d.kv_dtype == BSA_FP8_E4M3;
}

bsa_status_t fail(std::string& err, bsa_status_t st, const std::string& msg) {
  err = msg;
  return st;
}

}  // namespace

bsa_status_t build_plan(const bsa_plan_desc_t& desc, int32_t num_cus, Plan& P, std::string& err) {
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
  if (!d.indptr) return fail(err, BSA_ERR_INVALID_ARGUMENT, "indptr is NULL");
  if (d.indptr[0] != 0) return fail(err, BSA_ERR_INVALID_ARGUMENT, "indptr[0] must be 0");
  for (int64_t I = 0; I < MB; ++I)
    if (d.indptr[I + 1] < d.indptr[I])
      return fail(err, BSA_ERR_INVALID_ARGUMENT, "indptr must be non-decreasing");
  const int64_t nnz = d.indptr[MB];
  if (nnz > 0 && !d.indices) return fail(err, BSA_ERR_INVALID_ARGUMENT, "indices is NULL");
  std::vector<uint8_t> seen(static_cast<size_t>(NB), 0);
  for (int64_t I = 0; I < MB; ++I) {
    for (int64_t p = d.indptr[I]; p < d.indptr[I + 1]; ++p) {
      const int32_t J = d.indices[p];
      if (J < 0 || J >= NB) return fail(err, BSA_ERR_INVALID_ARGUMENT, "indices must lie in [0, NB)");
      if (seen[J]) return fail(err, BSA_ERR_INVALID_ARGUMENT, "duplicate column index within a row block");
      seen[J] = 1;
    }
    for (int64_t p = d.indptr[I]; p < d.indptr[I + 1]; ++p) seen[d.indices[p]] = 0;
  }
  if (d.kv_block_lens) {
    for (int64_t J = 0; J < NB; ++J)
      if (d.kv_block_lens[J] < 1 || d.kv_block_lens[J] > d.C)
        return fail(err, BSA_ERR_INVALID_ARGUMENT, "kv_block_lens entries must lie in [1, C]");
  }

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
    const bool f16 = d.q_dtype == BSA_F16 && d.kv_dtype == BSA_F16 && d.o_dtype == BSA_F16;
    const bool bf16 = d.q_dtype == BSA_BF16 && d.kv_dtype == BSA_BF16 && d.o_dtype == BSA_BF16;
    if (!(f16 || bf16))
      return fail(err, BSA_ERR_UNSUPPORTED, "q/k/v/o must all be fp16 or all bf16 for this head_dim");
    if (d.head_dim_qk != 128 || d.head_dim_vo != 128)
      return fail(err, BSA_ERR_UNSUPPORTED, "head_dim 128 (q/k and v/o) is the supported size");
    if (d.q_descale != 1.f || d.k_descale != 1.f || d.v_descale != 1.f)
      return fail(err, BSA_ERR_UNSUPPORTED, "dequant scales apply to fp8 KV only");
    if (d.R == 1 && g <= 16 && d.C >= 16) {
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
  std::vector<int64_t> bptr(MB + 1, 0);
  P.cols.clear();
  P.cols.reserve(static_cast<size_t>(nnz));
  for (int64_t I = 0; I < MB; ++I) {
    std::vector<int32_t> row(d.indices + d.indptr[I], d.indices + d.indptr[I + 1]);
    std::sort(row.begin(), row.end());
    const int64_t last_tok = std::min<int64_t>(d.M, (I + 1) * d.R) - 1;
    for (int32_t J : row) {
      if (d.causal && static_cast<int64_t>(J) * d.C > last_tok + off) break;
      P.cols.push_back(J);
    }
    bptr[I + 1] = static_cast<int64_t>(P.cols.size());
  }
  // valid length of each column-list entry (parallel to cols), so kernels
  // read a block's length with the same index as the block itself
  P.lens.clear();
  if (d.kv_block_lens) {
    P.lens.resize(P.cols.size());
    for (size_t p = 0; p < P.cols.size(); ++p) P.lens[p] = d.kv_block_lens[P.cols[p]];
  }

  // ---- 2./3. row tiles with their (prefix) column ranges and work
  struct RowTile {
    int64_t I, row0, nrows, cb, n, keys, work;
  };
  std::vector<RowTile> rts;
  std::vector<int64_t> pref;  // prefix key counts, reused
  for (int64_t I = 0; I < MB; ++I) {
    const int64_t rows_I = std::min<int64_t>(d.R, d.M - I * d.R);
    const int64_t U = rows_I * g;
    for (int64_t r0 = 0; r0 < U; r0 += tile_rows) {
      const int64_t nr = std::min<int64_t>(tile_rows, U - r0);
      int64_t n = bptr[I + 1] - bptr[I];
      if (d.causal) {
        const int64_t lim = I * d.R + (r0 + nr - 1) / g + off;
        int64_t k = 0;
        while (k < n && static_cast<int64_t>(P.cols[bptr[I] + k]) * d.C <= lim) ++k;
        n = k;
      }
      int64_t keys = 0;
      for (int64_t k = 0; k < n; ++k) keys += blen(P.cols[bptr[I] + k]);
      rts.push_back({I, r0, nr, bptr[I], n, keys, keys * ceil_div(nr, 32)});
    }
  }

  // ---- 4. split counts
  int64_t total_work = 0;
  for (const auto& rt : rts) total_work += rt.work * d.num_kv_heads;
  const int64_t chunk = std::max<int64_t>(1, ceil_div(total_work, (int64_t)kAutoTilesPerCu * num_cus));
  std::vector<int64_t> splits(rts.size(), 1);
  for (size_t t = 0; t < rts.size(); ++t) {
    const auto& rt = rts[t];
    int64_t s = 1;
    if (d.kv_splits > 1) {
      s = std::min<int64_t>(d.kv_splits, rt.n);
    } else if (d.kv_splits == 0) {
      const int64_t cap = std::min<int64_t>({rt.n, (int64_t)kMaxSplits,
                                             std::max<int64_t>(1, rt.keys / kAutoMinSplitKeys)});
      s = std::min<int64_t>(ceil_div(rt.work, chunk), cap);
    }
    splits[t] = std::max<int64_t>(1, s);
  }

  // ---- 5./6. emit tiles and merges
  struct TileRec {
    int32_t f[kTileInts];
    int64_t work;
  };
  std::vector<TileRec> recs;
  P.merges.clear();
  int64_t part = 0;
  int32_t max_s = 1;
  const int64_t dv = d.head_dim_vo;
  P.valid_pairs = 0;
  for (size_t t = 0; t < rts.size(); ++t) {
    const auto& rt = rts[t];
    const int64_t s = splits[t];
    max_s = std::max<int32_t>(max_s, static_cast<int32_t>(s));
    // prefix key counts over the row tile's blocks
    pref.assign(static_cast<size_t>(rt.n + 1), 0);
    for (int64_t k = 0; k < rt.n; ++k) pref[k + 1] = pref[k] + blen(P.cols[rt.cb + k]);
    std::vector<int64_t> b(static_cast<size_t>(s + 1), 0);
    b[s] = rt.n;
    for (int64_t j = 1; j < s; ++j) {
      int64_t p = 0;
      while (p < rt.n && pref[p] * s < j * rt.keys) ++p;
      p = std::max<int64_t>(p, b[j - 1] + 1);
      p = std::min<int64_t>(p, rt.n - (s - j));
      b[j] = p;
    }
    const int64_t psize = round_up(rt.nrows * (dv + 1), 64);
    for (int32_t h = 0; h < d.num_kv_heads; ++h) {
      const int64_t first = part;
      for (int64_t j = 0; j < s; ++j) {
        TileRec r{};
        const int64_t keys_j = pref[b[j + 1]] - pref[b[j]];
        r.f[T_ROWBLOCK] = static_cast<int32_t>(rt.I);
        r.f[T_KVHEAD] = h;
        r.f[T_ROW0] = static_cast<int32_t>(rt.row0);
        r.f[T_NROWS] = static_cast<int32_t>(rt.nrows);
        r.f[T_COLB] = static_cast<int32_t>(rt.cb + b[j]);
        r.f[T_COLE] = static_cast<int32_t>(rt.cb + b[j + 1]);
        r.f[T_PART] = s > 1 ? static_cast<int32_t>(part) : -1;
        r.f[T_KEYS] = static_cast<int32_t>(keys_j);
        r.work = keys_j * ceil_div(rt.nrows, 32);
        P.valid_pairs += keys_j * rt.nrows;
        if (s > 1) part += psize;
        if (part > INT32_MAX) return fail(err, BSA_ERR_UNSUPPORTED, "split partials exceed 2^31 floats");
        recs.push_back(r);
      }
      if (s > 1) {
        int32_t m[kMergeInts] = {static_cast<int32_t>(rt.I), h, static_cast<int32_t>(rt.row0),
                                 static_cast<int32_t>(rt.nrows), static_cast<int32_t>(first),
                                 static_cast<int32_t>(s), static_cast<int32_t>(psize), 0};
        P.merges.insert(P.merges.end(), m, m + kMergeInts);
      }
    }
  }
  std::stable_sort(recs.begin(), recs.end(),
                   [](const TileRec& a, const TileRec& b) { return a.work > b.work; });
  if (recs.size() > static_cast<size_t>(INT32_MAX / kTileInts))
    return fail(err, BSA_ERR_UNSUPPORTED, "too many tiles");
  P.tiles.clear();
  P.tiles.reserve(recs.size() * kTileInts);
  for (const auto& r : recs) P.tiles.insert(P.tiles.end(), r.f, r.f + kTileInts);
  P.max_splits = max_s;
  P.partial_floats = part;

  // ---- workspace layout: [tiles | merges | cols | lens] then partials
  int64_t o = 0;
  P.off_tiles = o;
  o = round_up(o + (int64_t)P.tiles.size() * 4, 256);
  P.off_merges = o;
  o = round_up(o + (int64_t)P.merges.size() * 4, 256);
  P.off_cols = o;
  o = round_up(o + (int64_t)P.cols.size() * 4, 256);
  P.off_lens = o;
  o = round_up(o + (int64_t)P.lens.size() * 4, 256);
  P.off_zero = o;  // zero row: masked keys load from here
  o = round_up(o + 1024, 256);
  P.table_bytes = std::max<int64_t>(o, 256);
  P.partial_bytes = round_up(P.partial_floats * 4, 256);
  P.workspace_bytes = P.table_bytes + P.partial_bytes;
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
  return BSA_OK;
}

}  // namespace bsa
