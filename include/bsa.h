/*
 * bsa.h -- block-sparse (BSR) attention over a KV cache on AMD MI355X (gfx950).
 *
 * C ABI of libbsa.so.  Plain pointers and sizes only; device pointers are
 * HIP device addresses on the current device, streams are hipStream_t
 * passed as void*.
 *
 * The operation (flashinfer.sparse, BlockSparseAttentionWrapper: class
 * description, the worked example and plan()/run() parameters):
 *   A BSR matrix in the SciPy bsr_matrix convention -- indptr over
 *   MB = ceil_div(M, R) row blocks, indices of column blocks below
 *   NB = N / C -- is an attention mask over M query rows and N key rows.
 *   Query row i attends to key j iff the row block i / R lists a column
 *   block J with J*C <= j < J*C + len_J (len_J = kv_block_lens[J], or C),
 *   and, if causal, j <= i + (N - M).  For every qo head h (kv head
 *   h / (num_qo_heads / num_kv_heads)):
 *       o[i,h,:]  = sum_j softmax_j(sm_scale * q[i,h,:] . k[j,kvh,:]) v[j,kvh,:]
 *       lse[i,h]  = ln sum_j exp(sm_scale * q[i,h,:] . k[j,kvh,:])
 *   over the unmasked keys; a row with no unmasked key gets o = 0 and
 *   lse = -inf.  Paged batch decode is the case R = 1, C = page size;
 *   index-selected sparse MLA decode (MATE sparse_mla_fp8_decode) is the
 *   case R = C = 1, one KV head of 576 = 512 latent + 64 rope values stored
 *   as fp8 e4m3, V = the first 512 values of each K row.
 *
 * Plan / run split (BlockSparseAttentionWrapper.plan notes; MATE decode
 * "metadata reuse"): bsa_plan* turns the structure into work tiles once,
 * on the host; bsa_run launches the kernels for one set of q/k/v and may
 * be called many times per plan.  A plan must not be shared by overlapping
 * runs on the same workspace.
 *
 * Errors: every call returns a bsa_status_t; bsa_last_error() gives the
 * calling thread's text for the last failure.  Nothing aborts, throws or
 * prints.  A failed bsa_run launches nothing and writes no output.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_VERSION_MAJOR 0
#define BSA_VERSION_MINOR 3

typedef struct bsa_plan_s* bsa_plan_t;

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARGUMENT = 1,   /* malformed structure, bad sizes, null/misaligned pointer */
  BSA_ERR_UNSUPPORTED = 2,        /* valid request the library has no kernel for */
  BSA_ERR_WORKSPACE_TOO_SMALL = 3,
  BSA_ERR_HIP = 4,                /* a HIP runtime call or kernel launch failed */
  BSA_ERR_HOST_ALLOC = 5          /* host memory allocation failed */
} bsa_status_t;

typedef enum { BSA_F16 = 0, BSA_BF16 = 1, BSA_FP8_E4M3 = 2 } bsa_dtype_t;

/* Kernel family a plan selected (informational). */
typedef enum {
  BSA_KERNEL_TILE = 0,    /* MFMA tile kernel: head_dim 128, fp16/bf16 (kv also fp8 e4m3), any R, C */
  BSA_KERNEL_MLA = 1,     /* MFMA sparse-MLA kernel: Dqk 576 / Dv 512, bf16 q/o, fp8 e4m3 kv, R = 1 */
  BSA_KERNEL_DECODE = 2   /* paged-decode kernel: R = 1, C >= 16, head_dim 128, fp16/bf16 (kv also fp8 e4m3), <= 16 qo heads per kv head */
} bsa_kernel_t;

/*
 * Full plan description.  Fill with bsa_plan_desc_init() first, then set
 * fields.  All arrays are HOST memory, read only during the call.
 *
 *   indptr         int32[MB + 1]; indptr[0] = 0, non-decreasing, indptr[MB] = nnz
 *   indices        int32[nnz]; column block of each non-zero block, 0 <= J < NB,
 *                  no duplicate within a row block; any order within a row
 *   M, N           query rows / key rows; N % C == 0
 *   R, C           block rows / block columns, >= 1 (variable blocks: see below)
 *   num_qo_heads   multiple of num_kv_heads (grouped-query attention)
 *   head_dim_qk    q/k head dim; head_dim_vo: v/o head dim (0 = head_dim_qk)
 *   causal         0/1: also mask key j > i + (N - M)
 *   sm_scale       softmax scale; <= 0 selects 1/sqrt(head_dim_qk)
 *   kv_splits      1 = no split-KV; k > 1 = at most k contiguous partitions of
 *                  each row's blocks; 0 = automatic (from the sparsity and
 *                  num_cus; for the decode kernel an equal share of all keys
 *                  per resident workgroup, see bsa_plan_export_workgroups).
 *                  Split partials live in the workspace and are LSE-merged by
 *                  a second kernel.
 *   kv_block_lens  NULL, or int32[NB] valid tokens per key block, each in [1, C]
 *   q/kv/o_dtype   storage types.  Supported: all BSA_F16, or all BSA_BF16
 *                  (head_dim 128); q/o BSA_F16 or BSA_BF16 with kv BSA_FP8_E4M3
 *                  for head_dim 128, any R and C (decode and prefill shapes;
 *                  BlockSparseAttentionWrapper.run: scale_k / scale_v "used with
 *                  FP8 Quantization"); or q/o BSA_BF16 with kv BSA_FP8_E4M3 and
 *                  head_dim_qk 576 / head_dim_vo 512 / one kv head / R = 1.
 *   q_descale etc. per-tensor dequant scales: real value = stored * descale
 *                  (MATE scale folding: the logit scale becomes
 *                  sm_scale * q_descale * k_descale, the output scale v_descale)
 *   *_token_stride elements between consecutive tokens; 0 = dense
 *                  (q: num_qo_heads*head_dim_qk, k: num_kv_heads*head_dim_qk,
 *                  v: num_kv_heads*head_dim_vo, o: num_qo_heads*head_dim_vo).
 *                  For the MLA shape v may alias k (v pointer == k pointer,
 *                  v_token_stride == k_token_stride).
 *   num_cus        0 = query the current device; > 0 = plan for that many CUs
 *                  without touching the GPU (host-only planning)
 *
 * Per-head structure (BlockSparseAttentionWrapper.plan: block_mask,
 * q2k_indices / q2k_num; VariableBlockSparseAttentionWrapper: each kv head
 * its own pattern).  Set at most one of block_mask and q2k_indices; then
 * indptr / indices are ignored and kv head h attends by its own structure:
 *   struct_heads   heads of the structure arrays: num_kv_heads, or
 *                  num_qo_heads -- then the qo heads of one kv head (h*g ..
 *                  h*g+g-1) must describe the same blocks (the kv head shares
 *                  every K/V load between them); a mismatch is
 *                  BSA_ERR_INVALID_ARGUMENT
 *   block_mask     NULL, or uint8[struct_heads][MB][NB]: nonzero = query
 *                  block I attends to key block J for that head
 *   q2k_indices    NULL, or int32[struct_heads][MB][q2k_topk]: the selected key
 *                  blocks of each (head, query block), each in [0, NB), no
 *                  duplicate among a row's first q2k_num entries, any order
 *   q2k_num        NULL (every row uses all q2k_topk entries), or
 *                  int32[struct_heads][MB] with entries in [0, q2k_topk]
 *   q2k_topk       entries per selection row (>= 0)
 * kv_block_lens, causal, kv_splits and everything else apply as for BSR.
 *
 * Element masks inside blocks (BlockSparseAttentionWrapper.plan: mask of
 * shape (nnz, R, C), packed_mask from flashinfer.quantization.packbits).
 * BSR form only (not with block_mask / q2k):
 *   mask           NULL (every block full), or the visibility of each element of
 *                  each BSR block: row r, column c of the block indices[p] (the
 *                  p-th entry as given, before any sorting) is entry
 *                  i = (p*R + r)*C + c; query I*R + r sees key J*C + c iff it is set
 *   mask_packed    0: uint8[nnz*R*C], nonzero = visible; 1: uint8[ceil(nnz*R*C / 8)],
 *                  entry i in bit i % 8 (least significant first) of byte i / 8
 * With a mask the causal flag has no effect (the pages: causal applies only
 * when no mask is given); kv_block_lens must be NULL (lengths belong in the
 * mask).  Element masks run on the tile kernel (head_dim 128, fp16/bf16, K/V
 * also fp8 e4m3), also for R = 1 shapes.
 *
 * Variable block sizes (VariableBlockSparseAttentionWrapper.plan:
 * block_mask_map, block_row_sz, block_col_sz; each kv head its own pattern):
 *   block_row_sz   NULL (fixed R x C blocks), or int32[num_kv_heads][var_row_blocks]:
 *                  row block a of kv head h covers the block_row_sz[h][a] query
 *                  rows after those of blocks 0..a-1; entries >= 0, each head's
 *                  sum equal to M
 *   block_col_sz   int32[num_kv_heads][var_col_blocks], the same for keys; each
 *                  head's sum equal to N
 *   var_row_blocks, var_col_blocks  >= 1
 *   block_mask     then uint8[num_kv_heads][var_row_blocks][var_col_blocks]
 *                  (struct_heads must be num_kv_heads; q2k, indptr / indices,
 *                  mask and kv_block_lens unused and must be NULL where listed)
 *   R, C           the fixed grid the planner maps the variable blocks onto (each
 *                  fixed block touched by a set variable block becomes a block
 *                  with an element mask): 0 = chosen by the planner (R =
 *                  max(1, 128 / g); C the largest power of two up to min(64, a
 *                  quarter of the mean non-empty column block size) dividing N)
 * causal applies on top of the block map (key j <= i + N - M).
 */
typedef struct {
  const int32_t* indptr;
  const int32_t* indices;
  int64_t M, N;
  int32_t R, C;
  int32_t num_qo_heads, num_kv_heads;
  int32_t head_dim_qk, head_dim_vo;
  int32_t causal;
  float sm_scale;
  int32_t kv_splits;
  const int32_t* kv_block_lens;
  bsa_dtype_t q_dtype, kv_dtype, o_dtype;
  float q_descale, k_descale, v_descale;
  int64_t q_token_stride, k_token_stride, v_token_stride, o_token_stride;
  int32_t num_cus;
  int32_t struct_heads;
  const uint8_t* block_mask;
  const int32_t* q2k_indices;
  const int32_t* q2k_num;
  int32_t q2k_topk;
  const uint8_t* mask;
  int32_t mask_packed;
  const int32_t* block_row_sz;
  const int32_t* block_col_sz;
  int32_t var_row_blocks, var_col_blocks;
} bsa_plan_desc_t;

/* Defaults: fp16 everywhere, head_dim_vo = head_dim_qk, non-causal, default
 * sm_scale, kv_splits = 1, descales 1, dense strides, num_cus from device. */
void bsa_plan_desc_init(bsa_plan_desc_t* desc);

/* sizeof(bsa_plan_desc_t) as compiled into the library, so that foreign
 * bindings can check their copy of the struct layout. */
size_t bsa_plan_desc_sizeof(void);

/* North-star form: fp16 q/k/v/o of shape (M, Hq, D) / (N, Hkv, D) / (N, Hkv, D)
 * / (M, Hq, D), all blocks full, num_cus from the current device.
 * sm_scale <= 0 selects 1/sqrt(head_dim).  On success *out_plan owns host
 * memory only; release it with bsa_plan_destroy. */
bsa_status_t bsa_plan(const int32_t* indptr, const int32_t* indices, int64_t M, int64_t N,
                      int32_t R, int32_t C, int32_t num_qo_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t causal, float sm_scale, int32_t kv_splits,
                      bsa_plan_t* out_plan);

/* Extended form (partial blocks, other dtypes, fp8 scales, strides, CU count).  *
 * With the environment variable BSA_LOG set (to anything but "0"), every call
 * of bsa_plan / bsa_plan_ex that reaches the planner prints one line to
 * stderr: the plan's kernel, tiles, merges, splits, workgroups, workspace and
 * planning time, or the error it failed with (the plan() conventions: fail
 * explicitly, and say why).
 */
bsa_status_t bsa_plan_ex(const bsa_plan_desc_t* desc, bsa_plan_t* out_plan);

/* Bytes of device workspace bsa_run needs for this plan (multiple of 256).
 * The caller owns and allocates the workspace, as the wrappers of
 * flashinfer.sparse take a user-reserved float_workspace_buffer in their
 * constructor (BlockSparseAttentionWrapper.__init__: it stores the
 * intermediate results of the split-k algorithm).  Here it holds the plan's
 * tables followed by the split-KV partials; the library never allocates
 * device memory.  Returns 0 for a NULL plan. */
size_t bsa_workspace_size(bsa_plan_t plan);

/* Bind `workspace` (device memory of at least bsa_workspace_size bytes,
 * 256-byte aligned) to the plan: copy the plan's tables into it on `stream`
 * and pin them there, so that later bsa_run calls on this workspace skip the
 * copy (BlockSparseAttentionWrapper.plan copies its auxiliary structures to
 * the device once and every run reuses them; reset_workspace_buffer hands a
 * wrapper new buffers).  The pin is remembered per device and workspace
 * address, and it is the caller's promise that the memory keeps the tables:
 * while pinned, nothing else may write it, and it must not be freed and
 * reused.  A pin ends with bsa_unpin, bsa_plan_destroy, a bsa_upload of
 * another plan to the same address, or any bsa_run of another plan on it.
 * bsa_run on a workspace that is not pinned to its plan copies the tables
 * itself, every time: that is always correct, only slower.  Pin before
 * capturing runs in a HIP graph (the copy is then not part of the run). */
bsa_status_t bsa_upload(bsa_plan_t plan, void* workspace, size_t workspace_bytes, void* stream);

/* End the plan's pin on `workspace` (see bsa_upload), e.g. before freeing
 * the memory; nothing happens if the plan is not pinned there.  Host-only:
 * launches nothing.  BSA_ERR_INVALID_ARGUMENT for NULL arguments. */
bsa_status_t bsa_unpin(bsa_plan_t plan, void* workspace);

/*
 * Run the planned attention on `stream` (hipStream_t; NULL = default stream).
 *   q    device, q_dtype,  [M][q_token_stride] with head h at h*head_dim_qk
 *   k    device, kv_dtype, [N][k_token_stride] with kv head h at h*head_dim_qk
 *   v    device, kv_dtype, [N][v_token_stride] with kv head h at h*head_dim_vo
 *   o    device, o_dtype,  [M][o_token_stride] with head h at h*head_dim_vo (written)
 *   lse  device float32 [M][num_qo_heads] natural-log LSE (written), or NULL
 *   workspace  device, >= bsa_workspace_size(plan) bytes, 256-byte aligned
 * q, k, v, o must be 16-byte aligned and must not overlap the workspace.
 * Every one of the M * num_qo_heads output rows is written; rows with no
 * unmasked key get o = 0 and lse = -inf.  The call only enqueues work on
 * `stream`: it neither synchronises nor allocates device memory.  Unless the
 * workspace is pinned to this plan (bsa_upload), the plan's tables are first
 * copied into it on `stream` (BlockSparseAttentionWrapper.run reuses what
 * plan() prepared; run() takes q, k, v and returns o and, with return_lse,
 * the lse).
 */
bsa_status_t bsa_run(bsa_plan_t plan, const void* q, const void* k, const void* v, void* o,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two phases of bsa_run, for callers that schedule them separately (or
 * time them separately).  phase = BSA_PHASE_ATTENTION launches the attention
 * kernel only (tiles without a split write o/lse, split tiles write their
 * partials into the workspace); BSA_PHASE_MERGE launches the LSE merge of the
 * split partials only (it must follow an attention phase of the same plan on
 * the same workspace, in stream order); BSA_PHASE_ALL is bsa_run.  Arguments
 * and errors as for bsa_run.
 */
#define BSA_PHASE_ATTENTION 1
#define BSA_PHASE_MERGE 2
#define BSA_PHASE_ALL 3
bsa_status_t bsa_run_phase(bsa_plan_t plan, int32_t phase, const void* q, const void* k, const void* v,
                           void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsa_run for callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and results as bsa_run without the workspace:
 * the library runs the plan in its own workspace, a static device array of
 * BSA_NOALLOC_MAX_WORKSPACE bytes per GPU, held from the library's load
 * until the process ends.  No call allocates or frees device memory.  The
 * plan's tables are copied into that array on `stream` when another plan
 * used it last, else reused.  Every call on one GPU shares the array: calls
 * that overlap on one GPU (other threads, other streams) race, and the
 * caller must order them.  A plan with bsa_workspace_size(plan) >
 * BSA_NOALLOC_MAX_WORKSPACE is refused with BSA_ERR_WORKSPACE_TOO_SMALL,
 * before anything touches the GPU; other errors as for bsa_run.
 */
#define BSA_NOALLOC_MAX_WORKSPACE (32u << 20)
bsa_status_t bsa_run_noalloc(bsa_plan_t plan, const void* q, const void* k, const void* v, void* o,
                             float* lse, void* stream);

/*
 * bsa_run_phase with per-head dequant scales (BlockSparseAttentionWrapper.run:
 * scale_q (num_qo_heads), scale_k and scale_v (num_kv_heads), per-head
 * quantization used with FP8): device float32 arrays, each NULL for 1.0.  The
 * value a kernel uses is stored value * descale of the plan * scale of the
 * head, i.e. logits are scaled by sm_scale * q_descale * k_descale *
 * scale_q[h] * scale_k[h / g] and outputs by v_descale * scale_v[h / g].
 * Supported by every head_dim 128 plan (tile and paged-decode kernels; K/V
 * fp16, bf16 or fp8 e4m3); BSA_ERR_UNSUPPORTED for the sparse-MLA shape (one
 * kv head: its per-tensor descales are the plan's) when any scale is given.
 */
bsa_status_t bsa_run_ex(bsa_plan_t plan, int32_t phase, const void* q, const void* k, const void* v,
                        void* o, float* lse, const float* scale_q, const float* scale_k, const float* scale_v,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * LSE merge of attention states (flashinfer.cascade merge_states): for each
 * of seq_len * num_heads rows, combine num_states partial results computed
 * over disjoint key sets:
 *     s_out = ln sum_k exp(s_k),   v_out = sum_k exp(s_k - s_out) v_k
 * States with s_k = -inf have weight 0; if all are -inf, v_out = 0 and
 * s_out = -inf.
 *   v      device float32 [seq_len][num_states][num_heads][head_dim]
 *   s      device float32 [seq_len][num_states][num_heads]   (natural log)
 *   v_out  device, out_dtype (BSA_F16, BSA_BF16 or float32 via BSA_FP32_OUT)
 *          [seq_len][num_heads][head_dim]
 *   s_out  device float32 [seq_len][num_heads], or NULL
 * head_dim must be a multiple of 4; pointers 16-byte aligned.
 */
#define BSA_FP32_OUT 3
bsa_status_t bsa_merge_states(const float* v, const float* s, void* v_out, float* s_out,
                              int64_t seq_len, int32_t num_states, int32_t num_heads,
                              int32_t head_dim, int32_t out_dtype, void* stream);

/*
 * MLA RoPE + FP8 quantize: the producer of the sparse-MLA decode inputs (MATE
 * sparse-MLA API page and its FlashInfer-wrapper page, "RoPE and FP8
 * quantization", mla_rope_quantize_fp8).  For every token t (position
 * pos_ids[t]) it turns the 64-value RoPE tails of q (each of num_heads heads)
 * and k by the position's angles, multiplies every q value (latent 512 and
 * tail 64) by quant_scale_q and every k value by quant_scale_kv, and casts to
 * FP8 E4M3.  Rotation: cache row pos holds cosines in columns 0..31 and sines in
 * 32..63; pair i uses column i and is values (i, i + 32) when is_neox, else
 * (2i, 2i + 1); a' = a cos - b sin, b' = b cos + a sin, each product and sum a
 * float32 operation of its own.  The cast rounds to nearest even and saturates
 * at +-448 (inputs are finite).
 *
 *   q_rope, q_nope   bf16 device arrays [nnz][num_heads][64] / [nnz][num_heads][512]
 *   k_rope, k_nope   bf16 device arrays [nnz][64] / [nnz][512]
 *   cos_sin_cache    device [max_seq_len][64], float32 (cache_bf16 = 0) or bf16 (1), contiguous
 *   pos_ids          device [nnz] int32 (pos_int64 = 0) or int64 (1); each in [0, max_seq_len):
 *                    a token whose position lies outside gets NaN codes (0x7F) in both its
 *                    rotated tails and never reads the cache
 *   *_out            fp8 e4m3 device arrays of the same shapes; may be slices of merged
 *                    [..., 576] rows (q_nope_out = row[:512], q_rope_out = row[512:])
 *   *_stride         leading-dimension strides, in elements of the array's own type (bf16
 *                    inputs, 1-byte outputs): [0] between tokens, [1] between heads; 0 =
 *                    dense.  Every stride must be a multiple of 8, inputs and the cache
 *                    16-byte aligned, outputs 8-byte aligned; the last dimension is always
 *                    contiguous.  Output rows must not overlap one another (not checked).
 * Runs one kernel on `stream`; nnz = 0 launches nothing.  BSA_ERR_INVALID_ARGUMENT for a
 * NULL argument struct or array, a bad size, stride or alignment, or a non-finite scale.
 */
typedef struct {
  const void* q_rope;
  const void* k_rope;
  const void* q_nope;
  const void* k_nope;
  const void* cos_sin_cache;
  int32_t cache_bf16;
  const void* pos_ids;
  int32_t pos_int64;
  int64_t nnz;
  int32_t num_heads;
  int64_t max_seq_len;
  int32_t is_neox;
  float quant_scale_q, quant_scale_kv;
  void* q_rope_out;
  void* k_rope_out;
  void* q_nope_out;
  void* k_nope_out;
  int64_t q_rope_stride[2], q_nope_stride[2], k_rope_stride, k_nope_stride;
  int64_t q_rope_out_stride[2], q_nope_out_stride[2], k_rope_out_stride, k_nope_out_stride;
} bsa_rope_quant_t;

/* Defaults: everything zero / NULL (dense strides), is_neox = 1, scales 1. */
void bsa_rope_quant_init(bsa_rope_quant_t* args);
/* sizeof(bsa_rope_quant_t) as compiled into the library. */
size_t bsa_rope_quant_sizeof(void);
bsa_status_t bsa_mla_rope_quantize_fp8(const bsa_rope_quant_t* args, void* stream);

/*
 * Sparse-attention indexer: FP32 scores and each query row's exact Top-K keys
 * (flashinfer.sparse 0.7.4 API page, "SDSA Indexer": indexer_scores gives a
 * float32 score per query row and key position of the row's request in the
 * paged cache; top_k_from_candidates keeps the row's exact Top-K; one query
 * head, no head weights).  The output, int32 physical cache rows, is the index list
 * of index-selected sparse MLA decode.
 *
 *   score(row, p) = sum_d q[row][d] * key_cache[slot(r, p)][d], accumulated in float32,
 *   slot(r, p)    = block_table[r][p / page_size] * page_size + p % page_size,
 * for the positions p = 0 .. n - 1 of the row's request r, n = min(ctx_len[row],
 * req_kv_len[r], max_ctx).  A row keeps the K = topk positions of highest score;
 * among equal scores the lower position wins (-0 and +0 are equal).  out[row] holds
 * their slots in ascending position order; a row with n <= K keeps all n and pads
 * with -1.  A position whose page index reaches max_pages or whose page id lies
 * outside [0, num_slots / page_size) is scored as a zero key and, if kept, written
 * as -1 (no read leaves the arrays).
 *
 *   q            device [num_rows][head_dim] fp16 or bf16 (dtype = BSA_F16 / BSA_BF16),
 *                row stride q_stride elements (0 = head_dim), 16-byte aligned rows
 *   key_cache    device [num_slots][head_dim], the same type, row stride k_stride (0 = dense)
 *   block_table  device int32 [num_reqs][max_pages]
 *   req_row_ptr  device int32 [num_reqs + 1], ascending in [0, num_rows]: the rows of
 *                request r are req_row_ptr[r] .. req_row_ptr[r + 1] - 1
 *   ctx_len      device int32 [num_rows]; req_kv_len device int32 [num_reqs]
 *   scores       device float32 [num_rows][ld], ld = max_ctx rounded up to a multiple of 64,
 *                16-byte aligned, caller-owned output: afterwards scores[row][p] holds
 *                score(row, p) for p < n (the rest of the row is unspecified)
 *   out          device int32 [num_rows][topk]
 *   workspace    device, >= bsa_indexer_workspace_size(num_rows, max_ctx) bytes, 256-byte
 *                aligned, caller-owned scratch of the Top-K step (per chunk of 16384
 *                positions a candidate count and up to 12288 candidates); no initial
 *                contents are needed.  Calls that share a workspace must not overlap.
 *                Not read when scores_only is set (may then be NULL).
 *   scores_only  non-zero: compute the scores only
 * Sizes: num_reqs >= 1, head_dim in {64, 128, 256}, page_size >= 1, max_pages >= 1,
 * 1 <= topk <= 2^24, 1 <= num_slots < 2^31, 1 <= max_ctx <= 8388480, strides multiples of
 * 8 and >= head_dim.
 * Runs three kernels on `stream` (scores; candidates per chunk of 16384 positions above a
 * threshold taken from a sample of the row's scores; the exact selection per row);
 * num_rows = 0 launches nothing.
 * BSA_ERR_INVALID_ARGUMENT for a NULL argument struct or array, a bad size, stride,
 * type or alignment.
 */
typedef struct {
  const void* q;
  const void* key_cache;
  const int32_t* block_table;
  const int32_t* req_row_ptr;
  const int32_t* ctx_len;
  const int32_t* req_kv_len;
  float* scores;
  int32_t* out;
  void* workspace;
  size_t workspace_bytes;
  int64_t num_slots, max_ctx, q_stride, k_stride;
  int32_t num_rows, num_reqs, max_pages, page_size, head_dim, topk, dtype;
  int32_t scores_only;
} bsa_indexer_t;

/* Defaults: everything zero / NULL (dense strides), dtype BSA_BF16. */
void bsa_indexer_init(bsa_indexer_t* args);
/* sizeof(bsa_indexer_t) as compiled into the library. */
size_t bsa_indexer_sizeof(void);
/* Bytes of workspace bsa_indexer_topk needs for num_rows rows of at most max_ctx keys
 * (0 when either is <= 0). */
size_t bsa_indexer_workspace_size(int32_t num_rows, int64_t max_ctx);
bsa_status_t bsa_indexer_topk(const bsa_indexer_t* args, void* stream);

/* Plan statistics, and the tables themselves, for inspection and tests. */
typedef struct {
  int32_t kernel;          /* bsa_kernel_t */
  int32_t tile_rows;       /* query rows (token, head pairs) per work tile */
  int32_t key_tile;        /* keys per inner step */
  int32_t num_tiles;
  int32_t num_merges;      /* row tiles split over > 1 partition */
  int32_t num_cols;        /* entries of the column table */
  int32_t max_splits;
  int32_t num_cus;
  int32_t num_workgroups;  /* workgroups of the attention launch */
  int32_t heads_per_wg;    /* kv heads per tile group (1 except for the decode kernel) */
  int64_t table_bytes;     /* int tables at the start of the workspace */
  int64_t partial_bytes;   /* split partials after the tables */
  int64_t workspace_bytes;
  int64_t valid_pairs;     /* block-level key positions x query rows, summed over tiles */
  int32_t R, C;            /* block grid the plan runs on (for variable blocks: the one chosen) */
  int64_t mask_plane_words; /* words per element-mask bit plane; 0 = no element masks */
} bsa_plan_info_t;

bsa_status_t bsa_plan_info(bsa_plan_t plan, bsa_plan_info_t* info);

/*
 * Copy the plan's tables to caller-owned host arrays sized from
 * bsa_plan_info (any pointer may be NULL to skip it):
 *   tiles   int32[num_tiles][8]  = {row_block, kv_head, row0, nrows,
 *                                   col_begin, col_end, partial_offset, key_count}
 *           in launch order (see bsa_plan_export_workgroups); row r of a tile (row0 <= r < row0 + nrows) is
 *           query token row_block*R + r / g and qo head kv_head*g + r % g
 *           (g = num_qo_heads / num_kv_heads); its keys are the blocks
 *           cols[col_begin .. col_end); partial_offset is -1 when the tile
 *           writes o/lse directly, else the float offset of its partial in
 *           the workspace's partial region.
 *   merges  int32[num_merges][8] = {row_block, kv_head, row0, nrows,
 *                                   first_partial, num_splits, partial_stride, 0}
 *   cols    int32[num_cols]: per row block, its column blocks in ascending
 *           order, without blocks that the causal mask removes entirely
 *           (with a per-head structure: per kv head, then per row block).
 */
bsa_status_t bsa_plan_export(bsa_plan_t plan, int32_t* tiles, int32_t* merges, int32_t* cols);

/*
 * Copy the workgroup table, int32[num_workgroups + 1], to a caller-owned host
 * array: workgroup w of the attention launch runs tiles wg_ptr[w] ..
 * wg_ptr[w+1]-1 in that order.  Tiles come in groups of heads_per_wg tiles
 * (same row block and blocks, consecutive kv heads: the decode kernel gives
 * each kv head of a group its own waves); each workgroup runs one group (the
 * hardware handing out groups longest first), except for the decode kernel
 * with kv_splits = 0: there the automatic split-KV partition
 * (BlockSparseAttentionWrapper.plan, kv_splits "auto") gives each of a fixed
 * number of resident workgroups an equal share of all keys, cutting rows
 * where the shares end.  Returns BSA_ERR_INVALID_ARGUMENT for a NULL plan or
 * array.
 */
bsa_status_t bsa_plan_export_workgroups(bsa_plan_t plan, int32_t* wg_ptr);

/* Copy the element-mask bit planes (R * mask_plane_words uint32 words, see
 * bsa_plan_info) into host `bits`.  Plane r holds, for entry e of the column
 * table (bsa_plan_export) and key c < C of that block, whether query row
 * I*R + r of the entry's row block sees key cols[e]*C + c: bit (e*C + c) % 32
 * of word (e*C + c) / 32.  BSA_ERR_INVALID_ARGUMENT for a NULL plan or array;
 * nothing is copied for a plan without element masks. */
bsa_status_t bsa_plan_export_mask_bits(bsa_plan_t plan, uint32_t* bits);

/*
 * Per-tile trace records of the last attention phase run with `workspace`
 * (a check that the kernels walk exactly the tables bsa_plan_export returns).
 * Only a library built with BSA_TRACE keeps them: there the workspace
 * (bsa_workspace_size) ends with int32[num_tiles][16] records, after the split
 * partials, which each run's attention phase resets and its kernel fills in,
 * tile t (launch order) =
 *   {times the tile was processed, first column entry whose keys it loaded,
 *    last such entry + 1, keys it loaded that lie inside their block's valid
 *    length (before the causal mask), partial_offset it wrote (-1: o/lse
 *    directly), kv_head, row0, nrows, key tokens outside [0, N) it met,
 *    7 unused}
 * and a tile with no valid key reads {1, INT32_MAX, 0, 0, ...}.  That build
 * checks every key token its kernels derive from the tables against [0, N):
 * one outside is counted in field 8 and read as a masked key, never loaded.
 * Waits for `stream`, then copies the records to host `records`
 * (int32[num_tiles * 16]).
 * The product library returns BSA_ERR_UNSUPPORTED; BSA_ERR_INVALID_ARGUMENT
 * for NULL arguments, BSA_ERR_HIP when the copy fails.
 */
bsa_status_t bsa_trace_records(bsa_plan_t plan, const void* workspace, int32_t* records, void* stream);

/* Free the plan's host memory and end its workspace pins.  A plan is made
 * once and reused across runs until the structure changes (MATE sparse-MLA
 * decode, "Metadata reuse": a new metadata object for new sequence lengths,
 * query shape or top-k); destroying it is the end of that reuse.  The caller
 * must not destroy a plan whose runs are still being enqueued on another
 * thread.  NULL is a no-op. */
void bsa_plan_destroy(bsa_plan_t plan);

/* Text of the calling thread's last error ("" if none).  Valid until the
 * thread's next bsa_* call.  Unsupported shapes, dtypes or layouts are
 * reported, never silently run another way (MATE FlashInfer wrapper, FP8
 * sparse MLA decode: unsupported inputs "fail explicitly"; flashinfer.sparse
 * plan(): a GQA ratio the kernel lacks raises an error). */
const char* bsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
