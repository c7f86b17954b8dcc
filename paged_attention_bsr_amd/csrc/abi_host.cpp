// C ABI of libbsa.so, host half: plan descriptors, planning, plan inspection
// and lifetime, the error string.  No HIP runtime call happens here; the two
// device facts planning needs (the current device's CU count, forgetting a
// destroyed plan's workspace bindings) come through the hooks of
// abi_internal.h.
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "abi_internal.h"

namespace bsa {

namespace {
thread_local std::string g_err;
int elt_bytes(bsa_dtype_t t) { return t == BSA_FP8_E4M3 ? 1 : 2; }
}  // namespace

bsa_status_t set_err(bsa_status_t st, const std::string& msg) {
  g_err = msg;
  return st;
}

void clear_err() { g_err.clear(); }

namespace {
// BSA_LOG set (and not "0"): one line per planning call on stderr -- the plan's
// statistics, or the error it failed with
bool log_on() {
  static const bool on = [] {
    const char* v = std::getenv("BSA_LOG");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}

void log_plan(const bsa_plan_desc_t& d, const Plan* P, bsa_status_t st, double us) {
  if (!log_on()) return;
  if (!P) {
    std::fprintf(stderr, "[bsa] plan M=%lld N=%lld R=%d C=%d Hq=%d Hkv=%d D=%d/%d failed (%d): %s\n",
                 static_cast<long long>(d.M), static_cast<long long>(d.N), d.R, d.C, d.num_qo_heads,
                 d.num_kv_heads, d.head_dim_qk, d.head_dim_vo, static_cast<int>(st), g_err.c_str());
    return;
  }
  static const char* kNames[] = {"tile", "mla", "decode"};
  const int k = P->kernel >= 0 && P->kernel <= 2 ? P->kernel : 0;
  std::fprintf(stderr,
               "[bsa] plan M=%lld N=%lld R=%d C=%d Hq=%d Hkv=%d D=%d/%d causal=%d kv_splits=%d: kernel=%s "
               "tile_rows=%d key_tile=%d tiles=%zu merges=%zu max_splits=%d workgroups=%zu cols=%zu "
               "valid_pairs=%lld workspace=%lld B (tables %lld) in %.1f us\n",
               static_cast<long long>(d.M), static_cast<long long>(d.N), P->d.R, P->d.C, d.num_qo_heads,
               d.num_kv_heads, d.head_dim_qk, d.head_dim_vo, d.causal, d.kv_splits, kNames[k], P->tile_rows,
               P->key_tile, P->tiles.size() / kTileInts, P->merges.size() / kMergeInts, P->max_splits,
               P->wg_ptr.size() - 1, P->cols.size(), static_cast<long long>(P->valid_pairs),
               static_cast<long long>(P->workspace_bytes), static_cast<long long>(P->table_bytes), us);
}
}  // namespace

}  // namespace bsa

using bsa::clear_err;
using bsa::elt_bytes;
using bsa::set_err;

extern "C" {

void bsa_plan_desc_init(bsa_plan_desc_t* d) {
  if (!d) return;
  std::memset(d, 0, sizeof(*d));
  d->R = 1;
  d->C = 1;
  d->num_qo_heads = 1;
  d->num_kv_heads = 1;
  d->head_dim_qk = 128;
  d->head_dim_vo = 0;
  d->sm_scale = 0.f;
  d->kv_splits = 1;
  d->q_dtype = d->kv_dtype = d->o_dtype = BSA_F16;
  d->q_descale = d->k_descale = d->v_descale = 1.f;
}

size_t bsa_plan_desc_sizeof(void) { return sizeof(bsa_plan_desc_t); }

bsa_status_t bsa_plan_ex(const bsa_plan_desc_t* desc, bsa_plan_t* out_plan) {
  clear_err();
  if (!desc || !out_plan) return set_err(BSA_ERR_INVALID_ARGUMENT, "desc and out_plan must be non-NULL");
  *out_plan = nullptr;
  bsa_plan_desc_t d = *desc;
  if (d.head_dim_vo == 0) d.head_dim_vo = d.head_dim_qk;
  if (d.q_token_stride == 0) d.q_token_stride = static_cast<int64_t>(d.num_qo_heads) * d.head_dim_qk;
  if (d.k_token_stride == 0) d.k_token_stride = static_cast<int64_t>(d.num_kv_heads) * d.head_dim_qk;
  if (d.v_token_stride == 0) d.v_token_stride = static_cast<int64_t>(d.num_kv_heads) * d.head_dim_vo;
  if (d.o_token_stride == 0) d.o_token_stride = static_cast<int64_t>(d.num_qo_heads) * d.head_dim_vo;
  if (d.q_token_stride < static_cast<int64_t>(d.num_qo_heads) * d.head_dim_qk ||
      d.k_token_stride < static_cast<int64_t>(d.num_kv_heads) * d.head_dim_qk ||
      d.v_token_stride < static_cast<int64_t>(d.num_kv_heads) * d.head_dim_vo ||
      d.o_token_stride < static_cast<int64_t>(d.num_qo_heads) * d.head_dim_vo)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "token strides must cover all heads of a token");
  const int vec = 16 / elt_bytes(d.kv_dtype);
  if (d.k_token_stride % vec || d.v_token_stride % vec || d.q_token_stride % 8 || d.o_token_stride % 8)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "token strides must keep every row 16-byte aligned");
  int32_t cus = d.num_cus;
  if (cus == 0) {
    const bsa_status_t s = bsa::current_device_cus(&cus);
    if (s != BSA_OK) return s;
  }
  bsa_plan_s* plan = nullptr;
  const auto t0 = std::chrono::steady_clock::now();
  auto elapsed_us = [&] {
    return std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  };
  try {
    plan = new bsa_plan_s();
    std::string err;
    const bsa_status_t st = bsa::build_plan(d, cus, plan->p, err);
    if (st != BSA_OK) {
      delete plan;
      set_err(st, err);
      bsa::log_plan(d, nullptr, st, elapsed_us());
      return st;
    }
  } catch (const std::bad_alloc&) {
    delete plan;
    set_err(BSA_ERR_HOST_ALLOC, "host allocation failed while planning");
    bsa::log_plan(d, nullptr, BSA_ERR_HOST_ALLOC, elapsed_us());
    return BSA_ERR_HOST_ALLOC;
  }
  bsa::log_plan(d, &plan->p, BSA_OK, elapsed_us());
  *out_plan = plan;
  return BSA_OK;
}

bsa_status_t bsa_plan(const int32_t* indptr, const int32_t* indices, int64_t M, int64_t N, int32_t R,
                      int32_t C, int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t causal, float sm_scale, int32_t kv_splits, bsa_plan_t* out_plan) {
  bsa_plan_desc_t d;
  bsa_plan_desc_init(&d);
  d.indptr = indptr;
  d.indices = indices;
  d.M = M;
  d.N = N;
  d.R = R;
  d.C = C;
  d.num_qo_heads = num_qo_heads;
  d.num_kv_heads = num_kv_heads;
  d.head_dim_qk = head_dim;
  d.head_dim_vo = head_dim;
  d.causal = causal;
  d.sm_scale = sm_scale;
  d.kv_splits = kv_splits;
  return bsa_plan_ex(&d, out_plan);
}

size_t bsa_workspace_size(bsa_plan_t plan) {
  return plan ? static_cast<size_t>(plan->p.workspace_bytes) : 0;
}

bsa_status_t bsa_plan_info(bsa_plan_t plan, bsa_plan_info_t* info) {
  clear_err();
  if (!plan || !info) return set_err(BSA_ERR_INVALID_ARGUMENT, "plan and info must be non-NULL");
  const bsa::Plan& P = plan->p;
  info->kernel = P.kernel;
  info->tile_rows = P.tile_rows;
  info->key_tile = P.key_tile;
  info->num_tiles = static_cast<int32_t>(P.tiles.size() / bsa::kTileInts);
  info->num_merges = static_cast<int32_t>(P.merges.size() / bsa::kMergeInts);
  info->num_cols = static_cast<int32_t>(P.cols.size());
  info->max_splits = P.max_splits;
  info->num_cus = P.num_cus;
  info->num_workgroups = static_cast<int32_t>(P.wg_ptr.size()) - 1;
  info->heads_per_wg = P.heads_per_wg;
  info->table_bytes = P.table_bytes;
  info->partial_bytes = P.partial_bytes;
  info->workspace_bytes = P.workspace_bytes;
  info->valid_pairs = P.valid_pairs;
  info->R = P.d.R;
  info->C = P.d.C;
  info->mask_plane_words = P.mask_plane_words;
  return BSA_OK;
}

bsa_status_t bsa_plan_export_mask_bits(bsa_plan_t plan, uint32_t* bits) {
  clear_err();
  if (!plan || !bits) return set_err(BSA_ERR_INVALID_ARGUMENT, "plan and bits must be non-NULL");
  const bsa::Plan& P = plan->p;
  if (!P.mbits.empty()) std::memcpy(bits, P.mbits.data(), P.mbits.size() * 4);
  return BSA_OK;
}

bsa_status_t bsa_plan_export(bsa_plan_t plan, int32_t* tiles, int32_t* merges, int32_t* cols) {
  clear_err();
  if (!plan) return set_err(BSA_ERR_INVALID_ARGUMENT, "plan is NULL");
  const bsa::Plan& P = plan->p;
  if (tiles && !P.tiles.empty()) std::memcpy(tiles, P.tiles.data(), P.tiles.size() * 4);
  if (merges && !P.merges.empty()) std::memcpy(merges, P.merges.data(), P.merges.size() * 4);
  if (cols && !P.cols.empty()) std::memcpy(cols, P.cols.data(), P.cols.size() * 4);
  return BSA_OK;
}

bsa_status_t bsa_plan_export_workgroups(bsa_plan_t plan, int32_t* wg_ptr) {
  clear_err();
  if (!plan || !wg_ptr) return set_err(BSA_ERR_INVALID_ARGUMENT, "plan and wg_ptr must be non-NULL");
  const bsa::Plan& P = plan->p;
  std::memcpy(wg_ptr, P.wg_ptr.data(), P.wg_ptr.size() * 4);
  return BSA_OK;
}

void bsa_plan_destroy(bsa_plan_t plan) {
  if (!plan) return;
  bsa::forget_plan(plan->p.id);
  delete plan;
}

const char* bsa_last_error(void) { return bsa::g_err.c_str(); }

void bsa_rope_quant_init(bsa_rope_quant_t* args) {
  if (!args) return;
  std::memset(args, 0, sizeof(*args));
  args->is_neox = 1;
  args->quant_scale_q = args->quant_scale_kv = 1.f;
}

size_t bsa_rope_quant_sizeof(void) { return sizeof(bsa_rope_quant_t); }

void bsa_indexer_init(bsa_indexer_t* args) {
  if (!args) return;
  std::memset(args, 0, sizeof(*args));
  args->dtype = BSA_BF16;
}

size_t bsa_indexer_sizeof(void) { return sizeof(bsa_indexer_t); }

}  // extern "C"
