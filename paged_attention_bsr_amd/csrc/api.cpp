// C ABI of libbsa.so, device half: workspace tables, runs, launches (the
// host half -- planning, plan inspection and lifetime -- is abi_host.cpp).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>

#include "abi_internal.h"
#include "kernels.h"
#include "indexer.h"
#include "rope_quant.h"

namespace {

using bsa::set_err;

// Which plan's tables each (device, workspace address) currently holds, and
// whether the caller pinned them there with bsa_upload.  Only a pinned entry
// lets bsa_run skip the upload: an address alone says nothing about the
// memory's contents once the caller may have freed and reused it.
struct Binding {
  uint64_t plan_id;
  bool pinned;
};
std::mutex g_reg_mu;
std::map<std::pair<int, uintptr_t>, Binding> g_registry;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_bytes(bsa_dtype_t t) { return t == BSA_FP8_E4M3 ? 1 : 2; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return an && bn && x < y + bn && y < x + an;
}

bsa_status_t hip_fail(hipError_t e, const char* what) {
  return set_err(BSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Copies the plan's tables into `ws` and records them there, pinned or not
// (an unpinned upload also drops any other plan's pin at that address: its
// tables are gone).
bsa_status_t do_upload(const bsa::Plan& P, void* ws, hipStream_t st, bool pin) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipMemcpyAsync(ws, P.table_blob.data(), static_cast<size_t>(P.table_bytes), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "table upload");
  std::lock_guard<std::mutex> lk(g_reg_mu);
  g_registry[{dev, reinterpret_cast<uintptr_t>(ws)}] = Binding{P.id, pin};
  return BSA_OK;
}

// Library-owned workspace for bsa_run_noalloc: a file-scope device array
// (each device holds its own copy for the life of the process).  In host code
// `scratch` names a host-side stand-in, never the device memory: host code
// only uses the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = BSA_NOALLOC_MAX_WORKSPACE;
static_assert(kScratchBytes % 256 == 0, "scratch holds 256-byte aligned workspaces");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> address of its copy of `scratch`

// The current device's copy of `scratch` (looked up once per device, with that
// device current).
bsa_status_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return set_err(BSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return BSA_OK;
}

bool pinned_here(const bsa::Plan& P, void* ws) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lk(g_reg_mu);
  auto it = g_registry.find({dev, reinterpret_cast<uintptr_t>(ws)});
  return it != g_registry.end() && it->second.plan_id == P.id && it->second.pinned;
}

}  // namespace

namespace bsa {

bsa_status_t current_device_cus(int32_t* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "querying the CU count (pass num_cus > 0 to plan without a GPU)");
  return BSA_OK;
}

void forget_plan(uint64_t plan_id) {
  std::lock_guard<std::mutex> lk(g_reg_mu);
  for (auto it = g_registry.begin(); it != g_registry.end();) {
    if (it->second.plan_id == plan_id) it = g_registry.erase(it);
    else ++it;
  }
}

}  // namespace bsa

extern "C" {

bsa_status_t bsa_upload(bsa_plan_t plan, void* workspace, size_t workspace_bytes, void* stream) {
  bsa::clear_err();
  if (!plan || !workspace) return set_err(BSA_ERR_INVALID_ARGUMENT, "plan and workspace must be non-NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < static_cast<size_t>(plan->p.workspace_bytes))
    return set_err(BSA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than bsa_workspace_size(plan)");
  return do_upload(plan->p, workspace, static_cast<hipStream_t>(stream), true);
}

bsa_status_t bsa_unpin(bsa_plan_t plan, void* workspace) {
  bsa::clear_err();
  if (!plan || !workspace) return set_err(BSA_ERR_INVALID_ARGUMENT, "plan and workspace must be non-NULL");
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_reg_mu);
  auto it = g_registry.find({dev, reinterpret_cast<uintptr_t>(workspace)});
  if (it != g_registry.end() && it->second.plan_id == plan->p.id) g_registry.erase(it);
  return BSA_OK;
}

bsa_status_t bsa_run(bsa_plan_t plan, const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return bsa_run_phase(plan, BSA_PHASE_ALL, q, k, v, o, lse, workspace, workspace_bytes, stream);
}

bsa_status_t bsa_run_phase(bsa_plan_t plan, int32_t phase, const void* q, const void* k, const void* v, void* o,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return bsa_run_ex(plan, phase, q, k, v, o, lse, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
}

bsa_status_t bsa_run_ex(bsa_plan_t plan, int32_t phase, const void* q, const void* k, const void* v, void* o,
                        float* lse, const float* scale_q, const float* scale_k, const float* scale_v,
                        void* workspace, size_t workspace_bytes, void* stream) {
  bsa::clear_err();
  if (!plan) return set_err(BSA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (phase < BSA_PHASE_ATTENTION || phase > BSA_PHASE_ALL)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "phase must be BSA_PHASE_ATTENTION, BSA_PHASE_MERGE or BSA_PHASE_ALL");
  const bsa::Plan& P = plan->p;
  const bsa_plan_desc_t& d = P.d;
  if ((scale_q || scale_k || scale_v) && P.kernel == BSA_KERNEL_MLA)
    return set_err(BSA_ERR_UNSUPPORTED, "per-head scales apply to head_dim 128 plans (the sparse-MLA shape has "
                                        "one kv head: use the plan's per-tensor descales)");
  if ((reinterpret_cast<uintptr_t>(scale_q) | reinterpret_cast<uintptr_t>(scale_k) |
       reinterpret_cast<uintptr_t>(scale_v)) & 3u)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "scale arrays must be 4-byte aligned");
  if (!q || !k || !v || !o || !workspace)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "q, k, v, o and workspace must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return set_err(BSA_ERR_INVALID_ARGUMENT, "q, k, v and o must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return set_err(BSA_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < static_cast<size_t>(P.workspace_bytes))
    return set_err(BSA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than bsa_workspace_size(plan)");
  const size_t o_bytes = static_cast<size_t>(d.M) * d.o_token_stride * elt_bytes(d.o_dtype);
  const size_t lse_bytes = lse ? static_cast<size_t>(d.M) * d.num_qo_heads * 4 : 0;
  if (overlaps(o, o_bytes, workspace, P.workspace_bytes) || overlaps(lse, lse_bytes, workspace, P.workspace_bytes))
    return set_err(BSA_ERR_INVALID_ARGUMENT, "o and lse must not overlap the workspace");
  if (overlaps(o, o_bytes, q, static_cast<size_t>(d.M) * d.q_token_stride * elt_bytes(d.q_dtype)))
    return set_err(BSA_ERR_INVALID_ARGUMENT, "o must not overlap q");

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!pinned_here(P, workspace)) {
    const bsa_status_t s = do_upload(P, workspace, st, false);
    if (s != BSA_OK) return s;
  }
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  bsa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.tiles = reinterpret_cast<const int32_t*>(ws + P.off_tiles);
  a.wg_ptr = reinterpret_cast<const int32_t*>(ws + P.off_wg);
  a.cols = reinterpret_cast<const int32_t*>(ws + P.off_cols);
  a.lens = P.lens.empty() ? nullptr : reinterpret_cast<const int32_t*>(ws + P.off_lens);
  a.part = reinterpret_cast<float*>(ws + P.table_bytes);
  a.zero_row = ws + P.off_zero;
  a.q_stride = d.q_token_stride;
  a.k_stride = d.k_token_stride;
  a.v_stride = d.v_token_stride;
  a.o_stride = d.o_token_stride;
  a.R = d.R;
  a.C = d.C;
  a.group = P.group;
  a.num_qo_heads = d.num_qo_heads;
  a.causal_off = static_cast<int32_t>(d.N - d.M);
  a.scale_log2 = static_cast<float>(static_cast<double>(P.sm_scale) * d.q_descale * d.k_descale * 1.4426950408889634);
  a.out_scale = d.v_descale;
  a.num_tiles = static_cast<int32_t>(P.tiles.size() / bsa::kTileInts);
  a.num_wgs = static_cast<int32_t>(P.wg_ptr.size()) - 1;
  a.heads_per_wg = P.heads_per_wg;
  a.mbits = P.mbits.empty() ? nullptr : reinterpret_cast<const uint32_t*>(ws + P.off_mbits);
  a.mask_plane_words = P.mask_plane_words;
#ifdef BSA_TRACE
  a.trace = reinterpret_cast<int32_t*>(ws + P.table_bytes + P.partial_bytes);
#endif
  a.num_keys = d.N;
  a.q_scale = scale_q;
  a.k_scale = scale_k;
  a.v_scale = scale_v;

  hipError_t e;
#ifdef BSA_TRACE
  if (phase & BSA_PHASE_ATTENTION) {
    // every record starts as {0, INT32_MAX, 0, 0, -2, -2, -2, -2, 0, -2 ...}
    std::vector<int32_t> init(static_cast<size_t>(a.num_tiles) * bsa::kTraceInts, -2);
    for (int32_t t = 0; t < a.num_tiles; ++t) {
      int32_t* r = init.data() + static_cast<size_t>(t) * bsa::kTraceInts;
      r[0] = 0, r[1] = INT32_MAX, r[2] = 0, r[3] = 0, r[8] = 0;
    }
    e = hipMemcpyAsync(a.trace, init.data(), init.size() * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return set_err(BSA_ERR_HIP, std::string("trace reset: ") + hipGetErrorString(e));
  }
#endif
  if (phase & BSA_PHASE_ATTENTION) {
    if (P.kernel == BSA_KERNEL_MLA) e = bsa::launch_attn_mla(a, d.causal != 0, a.lens != nullptr, st);
    else if (P.kernel == BSA_KERNEL_DECODE)
      e = bsa::launch_attn_decode(a, d.q_dtype == BSA_BF16, d.kv_dtype == BSA_FP8_E4M3, d.causal != 0,
                                  a.lens != nullptr, st);
    else e = bsa::launch_attn_tile(a, d.q_dtype == BSA_BF16, d.kv_dtype == BSA_FP8_E4M3, P.tile_rows,
                                   d.causal != 0, a.lens != nullptr, a.mbits != nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  }
  if (!(phase & BSA_PHASE_MERGE)) return BSA_OK;

  bsa::MergeArgs m{};
  m.merges = reinterpret_cast<const int32_t*>(ws + P.off_merges);
  m.part = a.part;
  m.o = o;
  m.lse = lse;
  m.o_stride = d.o_token_stride;
  m.R = d.R;
  m.group = P.group;
  m.num_qo_heads = d.num_qo_heads;
  m.dv = d.head_dim_vo;
  m.num_merges = static_cast<int32_t>(P.merges.size() / bsa::kMergeInts);
  e = bsa::launch_merge(m, d.o_dtype == BSA_BF16 ? 1 : 0, st);
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return BSA_OK;
}

bsa_status_t bsa_run_noalloc(bsa_plan_t plan, const void* q, const void* k, const void* v, void* o, float* lse,
                             void* stream) {
  bsa::clear_err();
  if (!plan) return set_err(BSA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (static_cast<size_t>(plan->p.workspace_bytes) > kScratchBytes)
    return set_err(BSA_ERR_WORKSPACE_TOO_SMALL,
                   "plan needs " + std::to_string(plan->p.workspace_bytes) + " bytes of workspace; bsa_run_noalloc "
                   "has " + std::to_string(kScratchBytes) + " (use bsa_run with a caller workspace)");
  void* ws = nullptr;
  const bsa_status_t st = scratch_address(&ws);
  if (st != BSA_OK) return st;
  // the library alone writes `scratch`, so a pin there is exact: copy the tables only
  // when another plan ran here last
  if (!pinned_here(plan->p, ws)) {
    const bsa_status_t su = do_upload(plan->p, ws, static_cast<hipStream_t>(stream), true);
    if (su != BSA_OK) return su;
  }
  return bsa_run_ex(plan, BSA_PHASE_ALL, q, k, v, o, lse, nullptr, nullptr, nullptr, ws, kScratchBytes, stream);
}

bsa_status_t bsa_merge_states(const float* v, const float* s, void* v_out, float* s_out, int64_t seq_len,
                              int32_t num_states, int32_t num_heads, int32_t head_dim, int32_t out_dtype,
                              void* stream) {
  bsa::clear_err();
  if (seq_len < 0 || num_states < 1 || num_heads < 1 || head_dim < 4 || head_dim % 4)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "need seq_len >= 0, num_states >= 1, num_heads >= 1, head_dim % 4 == 0");
  if (out_dtype != BSA_F16 && out_dtype != BSA_BF16 && out_dtype != BSA_FP32_OUT)
    return set_err(BSA_ERR_UNSUPPORTED, "out_dtype must be BSA_F16, BSA_BF16 or BSA_FP32_OUT");
  if (seq_len == 0) return BSA_OK;
  if (!v || !s || !v_out) return set_err(BSA_ERR_INVALID_ARGUMENT, "v, s and v_out must be non-NULL");
  if (!aligned16(v) || !aligned16(v_out)) return set_err(BSA_ERR_INVALID_ARGUMENT, "v and v_out must be 16-byte aligned");
  const hipError_t e = bsa::launch_merge_states(v, s, v_out, s_out, seq_len, num_states, num_heads, head_dim,
                                                out_dtype == BSA_FP32_OUT ? 2 : out_dtype,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge_states launch");
  return BSA_OK;
}

bsa_status_t bsa_trace_records(bsa_plan_t plan, const void* workspace, int32_t* records, void* stream) {
  bsa::clear_err();
  if (!plan || !workspace || !records)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "plan, workspace and records must be non-NULL");
#ifdef BSA_TRACE
  const bsa::Plan& P = plan->p;
  const size_t n = P.tiles.size() / bsa::kTileInts * bsa::kTraceInts;
  if (n == 0) return BSA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned char* src = static_cast<const unsigned char*>(workspace) + P.table_bytes + P.partial_bytes;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess) e = hipMemcpy(records, src, n * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return set_err(BSA_ERR_HIP, std::string("trace copy: ") + hipGetErrorString(e));
  return BSA_OK;
#else
  (void)stream;
  return set_err(BSA_ERR_UNSUPPORTED, "library built without per-tile trace records (BSA_TRACE)");
#endif
}

bsa_status_t bsa_mla_rope_quantize_fp8(const bsa_rope_quant_t* p, void* stream) {
  bsa::clear_err();
  if (!p) return set_err(BSA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (p->nnz < 0 || p->nnz > 0x7fffffff) return set_err(BSA_ERR_INVALID_ARGUMENT, "nnz must lie in [0, 2^31)");
  if (p->num_heads < 1 || p->num_heads > 65535 * 16)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "num_heads must lie in [1, 1048560]");
  if (p->max_seq_len < 1) return set_err(BSA_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 1");
  if (!std::isfinite(p->quant_scale_q) || !std::isfinite(p->quant_scale_kv))
    return set_err(BSA_ERR_INVALID_ARGUMENT, "quantization scales must be finite");
  if (p->nnz == 0) return BSA_OK;
  const void* in[] = {p->q_rope, p->k_rope, p->q_nope, p->k_nope, p->cos_sin_cache, p->pos_ids};
  const void* out[] = {p->q_rope_out, p->k_rope_out, p->q_nope_out, p->k_nope_out};
  for (const void* q : in)
    if (!q || reinterpret_cast<uintptr_t>(q) % 16 != 0)
      return set_err(BSA_ERR_INVALID_ARGUMENT, "inputs and the cache must be non-NULL and 16-byte aligned");
  for (const void* q : out)
    if (!q || reinterpret_cast<uintptr_t>(q) % 8 != 0)
      return set_err(BSA_ERR_INVALID_ARGUMENT, "outputs must be non-NULL and 8-byte aligned");
  const int64_t H = p->num_heads;
  bsa::RopeArgs a{};
  a.q_rope = p->q_rope;
  a.k_rope = p->k_rope;
  a.q_nope = p->q_nope;
  a.k_nope = p->k_nope;
  a.cos_sin = p->cos_sin_cache;
  a.pos = p->pos_ids;
  a.q_rope_out = p->q_rope_out;
  a.k_rope_out = p->k_rope_out;
  a.q_nope_out = p->q_nope_out;
  a.k_nope_out = p->k_nope_out;
  // a zero stride selects the dense one
  auto pick = [](int64_t s, int64_t dense) { return s != 0 ? s : dense; };
  a.qr_s[0] = pick(p->q_rope_stride[0], H * 64);
  a.qr_s[1] = pick(p->q_rope_stride[1], 64);
  a.qn_s[0] = pick(p->q_nope_stride[0], H * 512);
  a.qn_s[1] = pick(p->q_nope_stride[1], 512);
  a.kr_s = pick(p->k_rope_stride, 64);
  a.kn_s = pick(p->k_nope_stride, 512);
  a.qro_s[0] = pick(p->q_rope_out_stride[0], H * 64);
  a.qro_s[1] = pick(p->q_rope_out_stride[1], 64);
  a.qno_s[0] = pick(p->q_nope_out_stride[0], H * 512);
  a.qno_s[1] = pick(p->q_nope_out_stride[1], 512);
  a.kro_s = pick(p->k_rope_out_stride, 64);
  a.kno_s = pick(p->k_nope_out_stride, 512);
  const int64_t strides[] = {a.qr_s[0], a.qr_s[1], a.qn_s[0], a.qn_s[1], a.kr_s, a.kn_s,
                             a.qro_s[0], a.qro_s[1], a.qno_s[0], a.qno_s[1], a.kro_s, a.kno_s};
  for (int64_t st : strides)
    if (st < 0 || st % 8 != 0) return set_err(BSA_ERR_INVALID_ARGUMENT, "strides must be non-negative multiples of 8");
  a.nnz = p->nnz;
  a.max_seq_len = p->max_seq_len;
  a.num_heads = p->num_heads;
  a.is_neox = p->is_neox != 0;
  a.cache_bf16 = p->cache_bf16 != 0;
  a.pos_int64 = p->pos_int64 != 0;
  a.scale_q = p->quant_scale_q;
  a.scale_kv = p->quant_scale_kv;
  const hipError_t e = bsa::launch_rope_quant(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope quantize kernel launch");
  return BSA_OK;
}


size_t bsa_indexer_workspace_size(int32_t num_rows, int64_t max_ctx) {
  return bsa::indexer_workspace_bytes(num_rows, max_ctx);
}

bsa_status_t bsa_indexer_topk(const bsa_indexer_t* p, void* stream) {
  bsa::clear_err();
  if (!p) return set_err(BSA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (p->num_rows < 0) return set_err(BSA_ERR_INVALID_ARGUMENT, "num_rows must be >= 0");
  if (p->num_reqs < 1) return set_err(BSA_ERR_INVALID_ARGUMENT, "num_reqs must be >= 1");
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "head_dim must be 64, 128 or 256");
  if (p->page_size < 1 || p->max_pages < 1)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "page_size and max_pages must be >= 1");
  if (p->topk < 1 || p->topk > (1 << 24)) return set_err(BSA_ERR_INVALID_ARGUMENT, "topk must lie in [1, 2^24]");
  if (p->num_slots < 1 || p->num_slots > 0x7fffffff)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "num_slots must lie in [1, 2^31)");
  if (p->max_ctx < 1) return set_err(BSA_ERR_INVALID_ARGUMENT, "max_ctx must be >= 1");
  if (p->dtype != BSA_F16 && p->dtype != BSA_BF16)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "dtype must be BSA_F16 or BSA_BF16");
  const int64_t qs = p->q_stride != 0 ? p->q_stride : p->head_dim;
  const int64_t ks = p->k_stride != 0 ? p->k_stride : p->head_dim;
  if (qs < p->head_dim || ks < p->head_dim || qs % 8 != 0 || ks % 8 != 0)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "strides must be multiples of 8 and at least head_dim");
  if (p->max_ctx > 8388480) return set_err(BSA_ERR_INVALID_ARGUMENT, "max_ctx must be at most 8388480");
  if (p->num_rows == 0) return BSA_OK;
  if (!p->q || !p->key_cache || reinterpret_cast<uintptr_t>(p->q) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(p->key_cache) % 16 != 0)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "q and key_cache must be non-NULL and 16-byte aligned");
  if (!p->scores || reinterpret_cast<uintptr_t>(p->scores) % 16 != 0)
    return set_err(BSA_ERR_INVALID_ARGUMENT, "scores must be non-NULL and 16-byte aligned");
  const void* ints[] = {p->block_table, p->req_row_ptr, p->ctx_len, p->req_kv_len, p->out};
  for (const void* x : ints)
    if (!x || reinterpret_cast<uintptr_t>(x) % 4 != 0)
      return set_err(BSA_ERR_INVALID_ARGUMENT, "table and output arrays must be non-NULL and 4-byte aligned");
  const size_t ws_need = bsa::indexer_workspace_bytes(p->num_rows, p->max_ctx);
  if (!p->scores_only) {
    if (!p->workspace || reinterpret_cast<uintptr_t>(p->workspace) % 256 != 0)
      return set_err(BSA_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    if (p->workspace_bytes < ws_need)
      return set_err(BSA_ERR_INVALID_ARGUMENT, "workspace is smaller than bsa_indexer_workspace_size");
  }
  bsa::IndexerArgs a{};
  a.q = p->q;
  a.key_cache = p->key_cache;
  a.block_table = p->block_table;
  a.req_row_ptr = p->req_row_ptr;
  a.ctx_len = p->ctx_len;
  a.req_kv_len = p->req_kv_len;
  a.scores = p->scores;
  a.out = p->out;
  a.num_slots = p->num_slots;
  a.max_ctx = p->max_ctx;
  a.ld_scores = (p->max_ctx + 63) / 64 * 64;
  a.q_stride = qs;
  a.k_stride = ks;
  a.num_rows = p->num_rows;
  a.num_reqs = p->num_reqs;
  a.max_pages = p->max_pages;
  a.page_size = p->page_size;
  a.page_shift = (p->page_size & (p->page_size - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(p->page_size)) : -1;
  a.head_dim = p->head_dim;
  a.topk = p->topk;
  a.nch_max = static_cast<int32_t>((p->max_ctx + bsa::kIdxChunk - 1) / bsa::kIdxChunk);
  if (!p->scores_only) {
    const size_t chunks = static_cast<size_t>(p->num_rows) * static_cast<size_t>(a.nch_max);
    a.ws_count = static_cast<int32_t*>(p->workspace);
    a.ws_cand = reinterpret_cast<uint2*>(static_cast<char*>(p->workspace) + (chunks * 4 + 255) / 256 * 256);
  }
  const hipError_t e = bsa::launch_indexer(a, p->dtype == BSA_BF16, p->scores_only != 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "indexer kernel launch");
  return BSA_OK;
}
}  // extern "C"
