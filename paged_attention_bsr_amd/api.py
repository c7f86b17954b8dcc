"""Python binding of libbsa: plan once, run many times.

Argument marshalling only -- every step of the attention runs in the HIP
library.  PyTorch supplies device memory and the current stream.  The call
names follow the C ABI (bsa_plan / bsa_run) and, for the arguments, the
flashinfer.sparse BlockSparseAttentionWrapper plan()/run() parameters.
"""
from __future__ import annotations

import ctypes
import weakref
from typing import Optional

import numpy as np
import torch

from . import _lib as L

_DTYPE_CODES = {torch.float16: L.BSA_F16, torch.bfloat16: L.BSA_BF16, torch.float8_e4m3fn: L.BSA_FP8_E4M3}


def _i32(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _np(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.asarray(a)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class Plan:
    """A planned BSR attention problem (bsa_plan_ex).

    indptr / indices / kv_block_lens are host arrays (numpy or CPU tensors).
    ``kv_splits``: 1 = none, k = at most k partitions per row tile, 0 or
    "auto" = automatic.  ``num_cus`` = 0 asks the current device.

    Per-head structure (plan(): block_mask, q2k_indices / q2k_num): pass
    ``block_mask`` (heads, MB, NB) bool, or ``q2k_indices`` (heads, MB, topk)
    int with optional ``q2k_num`` (heads, MB); heads = num_kv_heads or
    num_qo_heads.  indptr / indices are then ignored (may be None).

    Element masks inside blocks (plan(): mask, packed_mask): ``mask`` (nnz, R, C)
    bool, mask[p] belonging to block indices[p]; or ``packed_mask``, its
    flattening eight entries a byte, least significant bit first (then
    ``mask`` is ignored).  With either, ``causal`` has no effect.

    Variable block sizes: use ``Plan.variable``.

    ``trace=True`` plans and runs with libbsa_trace.so, whose kernels record
    per tile what they walked (trace_records); tests only.
    """

    def __init__(self, indptr, indices, M: int, N: int, R: int, C: int, num_qo_heads: int,
                 num_kv_heads: int, head_dim: int, *, head_dim_vo: Optional[int] = None,
                 causal: bool = False, sm_scale: Optional[float] = None, kv_splits=1,
                 kv_block_lens=None, q_dtype: torch.dtype = torch.float16,
                 kv_dtype: Optional[torch.dtype] = None, o_dtype: Optional[torch.dtype] = None,
                 q_descale: float = 1.0, k_descale: float = 1.0, v_descale: float = 1.0,
                 q_token_stride: int = 0, k_token_stride: int = 0, v_token_stride: int = 0,
                 o_token_stride: int = 0, num_cus: int = 0, block_mask=None, q2k_indices=None,
                 q2k_num=None, mask=None, packed_mask=None, block_row_sz=None, block_col_sz=None,
                 trace: bool = False):
        lib = self._lib = L.trace_lib() if trace else L.lib()
        self._handle = ctypes.c_void_p()
        self._indptr = _i32(np.zeros(1) if indptr is None else indptr)
        self._indices = _i32(np.zeros(0) if indices is None else indices)
        self._mask = None if block_mask is None else np.ascontiguousarray(_np(block_mask), dtype=np.uint8)
        self._q2k = None if q2k_indices is None else _i32(q2k_indices)
        self._q2k_num = None if q2k_num is None else _i32(q2k_num)
        self._lens = None if kv_block_lens is None else _i32(kv_block_lens)
        if packed_mask is not None:
            self._emask = np.ascontiguousarray(_np(packed_mask).ravel(), dtype=np.uint8)
        elif mask is not None:
            self._emask = np.ascontiguousarray(_np(mask).astype(bool), dtype=np.uint8)
            if self._emask.shape != (int(self._indptr[-1]), int(R), int(C)):
                raise ValueError(f"mask must have shape (nnz, R, C) = ({int(self._indptr[-1])}, {int(R)}, {int(C)})")
        else:
            self._emask = None
        if self._emask is not None and packed_mask is not None:
            nbits = int(self._indptr[-1]) * int(R) * int(C)
            if self._emask.size < -(-nbits // 8):
                raise ValueError(f"packed_mask needs {-(-nbits // 8)} bytes for nnz * R * C = {nbits} entries")
        self._row_sz = None if block_row_sz is None else _i32(block_row_sz)
        self._col_sz = None if block_col_sz is None else _i32(block_col_sz)
        kv_dtype = q_dtype if kv_dtype is None else kv_dtype
        o_dtype = q_dtype if o_dtype is None else o_dtype
        for t in (q_dtype, kv_dtype, o_dtype):
            if t not in _DTYPE_CODES:
                raise ValueError(f"unsupported dtype {t}")
        d = L.PlanDesc()
        lib.bsa_plan_desc_init(ctypes.byref(d))
        d.indptr = _ptr(self._indptr)
        d.indices = _ptr(self._indices) if self._indices.size else None
        d.M, d.N, d.R, d.C = int(M), int(N), int(R), int(C)
        d.num_qo_heads, d.num_kv_heads = int(num_qo_heads), int(num_kv_heads)
        d.head_dim_qk = int(head_dim)
        d.head_dim_vo = int(head_dim if head_dim_vo is None else head_dim_vo)
        d.causal = int(bool(causal))
        d.sm_scale = float(sm_scale) if sm_scale is not None else 0.0
        d.kv_splits = 0 if kv_splits == "auto" else (1 if kv_splits is None else int(kv_splits))
        d.kv_block_lens = _ptr(self._lens) if self._lens is not None else None
        d.q_dtype, d.kv_dtype, d.o_dtype = _DTYPE_CODES[q_dtype], _DTYPE_CODES[kv_dtype], _DTYPE_CODES[o_dtype]
        d.q_descale, d.k_descale, d.v_descale = float(q_descale), float(k_descale), float(v_descale)
        d.q_token_stride, d.k_token_stride = int(q_token_stride), int(k_token_stride)
        d.v_token_stride, d.o_token_stride = int(v_token_stride), int(o_token_stride)
        d.num_cus = int(num_cus)
        if self._mask is not None:
            if self._mask.ndim != 3:
                raise ValueError("block_mask must have shape (heads, MB, NB)")
            d.struct_heads = int(self._mask.shape[0])
            d.block_mask = self._mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        if self._q2k is not None:
            if self._q2k.ndim != 3:
                raise ValueError("q2k_indices must have shape (heads, MB, topk)")
            d.struct_heads = int(self._q2k.shape[0])
            d.q2k_topk = int(self._q2k.shape[2])
            if self._q2k.size == 0:  # topk = 0: a valid pointer that is never read
                self._q2k = np.zeros(1, np.int32)
            d.q2k_indices = _ptr(self._q2k)
            if self._q2k_num is not None:
                if self._q2k_num.shape != self._q2k.shape[:2]:
                    raise ValueError("q2k_num must have shape (heads, MB)")
                d.q2k_num = _ptr(self._q2k_num)
        if self._emask is not None:
            if self._emask.size == 0:  # nnz = 0: a valid pointer that is never read
                self._emask = np.zeros(1, np.uint8)
            d.mask = self._emask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
            d.mask_packed = int(packed_mask is not None)
        if self._row_sz is not None or self._col_sz is not None:
            if self._row_sz is None or self._col_sz is None or self._row_sz.ndim != 2 or self._col_sz.ndim != 2:
                raise ValueError("block_row_sz (heads, MB) and block_col_sz (heads, NB) go together")
            d.block_row_sz, d.block_col_sz = _ptr(self._row_sz), _ptr(self._col_sz)
            d.var_row_blocks, d.var_col_blocks = int(self._row_sz.shape[1]), int(self._col_sz.shape[1])
        self._check(lib.bsa_plan_ex(ctypes.byref(d), ctypes.byref(self._handle)))
        inf = self.info()
        self.M, self.N, self.R, self.C = int(M), int(N), int(inf["R"]), int(inf["C"])
        self.num_qo_heads, self.num_kv_heads = int(num_qo_heads), int(num_kv_heads)
        self.head_dim, self.head_dim_vo = int(head_dim), int(d.head_dim_vo)
        self.q_dtype, self.kv_dtype, self.o_dtype = q_dtype, kv_dtype, o_dtype
        self.k_token_stride = int(k_token_stride) or self.num_kv_heads * self.head_dim
        self.v_token_stride = int(v_token_stride) or self.num_kv_heads * self.head_dim_vo
        self._workspace: Optional[torch.Tensor] = None
        # the workspace tensor this plan's tables are pinned in (bsa_upload), held weakly:
        # a freed tensor whose memory comes back at the same address is a new workspace
        self._pinned: Optional[tuple] = None

    @classmethod
    def variable(cls, block_mask_map, block_row_sz, block_col_sz, num_qo_heads: int, num_kv_heads: int,
                 head_dim: int, *, R: int = 0, C: int = 0, **kw) -> "Plan":
        """Variable block sizes (VariableBlockSparseAttentionWrapper.plan): block_mask_map
        (num_kv_heads, MB, NB) bool, block_row_sz (num_kv_heads, MB) and block_col_sz
        (num_kv_heads, NB) int, each head's sizes summing to the query / key counts.
        q, k, v, o keep the token-major (tokens, heads, dim) layout of run().  R, C:
        the fixed grid the library maps the blocks onto (0 = its choice); other keyword
        arguments as for Plan."""
        rs, cs = _i32(block_row_sz), _i32(block_col_sz)
        if rs.ndim != 2 or cs.ndim != 2 or rs.shape[0] < 1:
            raise ValueError("block_row_sz must be (heads, MB) and block_col_sz (heads, NB)")
        return cls(None, None, int(rs[0].sum()), int(cs[0].sum()), R, C, num_qo_heads, num_kv_heads, head_dim,
                   block_mask=block_mask_map, block_row_sz=rs, block_col_sz=cs, **kw)

    def _check(self, status: int) -> None:
        L.check(status, self._lib)

    # ------------------------------------------------------------------ info
    def info(self) -> dict:
        inf = L.PlanInfo()
        self._check(self._lib.bsa_plan_info(self._handle, ctypes.byref(inf)))
        return {name: getattr(inf, name) for name, _ in inf._fields_}

    @property
    def workspace_size(self) -> int:
        return int(self._lib.bsa_workspace_size(self._handle))

    def tables(self) -> dict:
        """The planner's tables (tiles (T, 8), merges (S, 8), cols, wg_ptr (W + 1)) as int32 numpy arrays."""
        inf = self.info()
        tiles = np.zeros((inf["num_tiles"], 8), np.int32)
        merges = np.zeros((inf["num_merges"], 8), np.int32)
        cols = np.zeros(inf["num_cols"], np.int32)
        wg_ptr = np.zeros(inf["num_workgroups"] + 1, np.int32)
        self._check(self._lib.bsa_plan_export(self._handle, _ptr(tiles), _ptr(merges), _ptr(cols)))
        self._check(self._lib.bsa_plan_export_workgroups(self._handle, _ptr(wg_ptr)))
        out = {"tiles": tiles, "merges": merges, "cols": cols, "wg_ptr": wg_ptr}
        if inf["mask_plane_words"] > 0:
            bits = np.zeros((inf["R"], inf["mask_plane_words"]), np.uint32)
            self._check(self._lib.bsa_plan_export_mask_bits(self._handle,
                                                      bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))))
            out["mask_bits"] = bits
        return out

    # ------------------------------------------------------------------ run
    def workspace(self, device=None) -> torch.Tensor:
        """A device workspace owned by this plan (kept alive with it)."""
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        ws = self._workspace
        if ws is None or ws.device != dev or ws.numel() < self.workspace_size:
            self._workspace = torch.empty(max(self.workspace_size, 256), dtype=torch.uint8, device=dev)
        return self._workspace

    def upload(self, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
        """Copy the tables into ``workspace`` and pin them there (bsa_upload); later runs on
        the same tensor skip the copy."""
        ws = self.workspace() if workspace is None else workspace
        st = torch.cuda.current_stream(ws.device).cuda_stream if stream is None else stream
        self._check(self._lib.bsa_upload(self._handle, ws.data_ptr(), ws.numel() * ws.element_size(), st))
        self._pinned = (weakref.ref(ws), ws.data_ptr(), ws.numel() * ws.element_size())

    def _ensure_pinned(self, ws: torch.Tensor, stream) -> None:
        """Pin the tables in ``ws`` unless this very tensor (alive, same memory) holds them."""
        pin = self._pinned
        if pin is not None and pin[0]() is ws and pin[1] == ws.data_ptr() and \
                pin[2] == ws.numel() * ws.element_size():
            return
        self.upload(ws, stream)

    def run(self, q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            return_lse: bool = True, workspace: Optional[torch.Tensor] = None, stream=None,
            phase: int = L.BSA_PHASE_ALL, scale_q: Optional[torch.Tensor] = None,
            scale_k: Optional[torch.Tensor] = None, scale_v: Optional[torch.Tensor] = None):
        """o (M, Hq, Dv) and, if requested, lse (M, Hq) float32.  v=None aliases k (MLA).

        ``phase`` selects bsa_run_phase's attention-only / merge-only halves.
        ``scale_q`` (num_qo_heads,), ``scale_k`` / ``scale_v`` (num_kv_heads,): per-head
        float32 dequant scales on the device (run(): scale_q/k/v), None = 1."""
        call, out, lse = self._prepare(q, k, v, out, lse, return_lse, workspace, stream, phase,
                                       scale_q, scale_k, scale_v)
        call()
        return (out, lse) if return_lse else out

    def bind(self, q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             return_lse: bool = True, workspace: Optional[torch.Tensor] = None, stream=None,
             phase: int = L.BSA_PHASE_ALL, scale_q: Optional[torch.Tensor] = None,
             scale_k: Optional[torch.Tensor] = None, scale_v: Optional[torch.Tensor] = None):
        """Validate the arguments of run() once, pin the tables in the workspace and
        return (fn, out, lse): fn() runs the attention into out / lse with nothing
        but the C call (bsa_run_ex), for loops that run the same buffers many
        times.  fn keeps every tensor it uses alive; the caller must not resize,
        free or re-pin the workspace to another plan while using it."""
        return self._prepare(q, k, v, out, lse, return_lse, workspace, stream, phase, scale_q, scale_k, scale_v)

    def _prepare(self, q, k, v, out, lse, return_lse, workspace, stream, phase, scale_q, scale_k, scale_v):
        if v is None:
            v = k
        for name, t, dt in (("q", q, self.q_dtype), ("k", k, self.kv_dtype), ("v", v, self.kv_dtype)):
            if not t.is_cuda:
                raise ValueError(f"{name} must be a device tensor")
            if t.dtype != dt:
                raise ValueError(f"{name} dtype {t.dtype} does not match the plan ({dt})")
        if q.shape != (self.M, self.num_qo_heads, self.head_dim) or not q.is_contiguous():
            raise ValueError(f"q must be a contiguous ({self.M}, {self.num_qo_heads}, {self.head_dim}) tensor")
        if k.shape[0] != self.N or v.shape[0] != self.N:
            raise ValueError(f"k and v need {self.N} rows")
        if k.stride(-1) != 1 or v.stride(-1) != 1 or k.stride(0) != self.k_token_stride or \
                v.stride(0) != self.v_token_stride:
            raise ValueError(f"k/v token strides must be {self.k_token_stride}/{self.v_token_stride} "
                             "elements with a contiguous last dimension")
        if out is None:
            out = torch.empty((self.M, self.num_qo_heads, self.head_dim_vo), dtype=self.o_dtype, device=q.device)
        elif out.shape != (self.M, self.num_qo_heads, self.head_dim_vo) or out.dtype != self.o_dtype or not out.is_contiguous():
            raise ValueError("out has the wrong shape, dtype or layout")
        if lse is None and return_lse:
            lse = torch.empty((self.M, self.num_qo_heads), dtype=torch.float32, device=q.device)
        ws = self.workspace(q.device) if workspace is None else workspace
        st = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
        self._ensure_pinned(ws, st)
        scales = []
        for name, t, n in (("scale_q", scale_q, self.num_qo_heads), ("scale_k", scale_k, self.num_kv_heads),
                           ("scale_v", scale_v, self.num_kv_heads)):
            if t is None:
                scales.append(None)
                continue
            if not t.is_cuda or t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 device tensor of {n} entries")
            scales.append(t.data_ptr())
        fn, args = self._lib.bsa_run_ex, (self._handle, int(phase), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), lse.data_ptr() if lse is not None else None, *scales,
                                          ws.data_ptr(), ws.numel() * ws.element_size(), st)
        keep = (q, k, v, out, lse, ws, scale_q, scale_k, scale_v)  # alive as long as the call

        def call(_keep=keep):
            self._check(fn(*args))

        return call, out, lse

    def trace_records(self, workspace: torch.Tensor, stream=None) -> np.ndarray:
        """(num_tiles, 16) int32 records of the last attention phase run in ``workspace``
        (bsa_trace_records; trace=True plans only)."""
        st = torch.cuda.current_stream(workspace.device).cuda_stream if stream is None else stream
        rec = np.zeros((self.info()["num_tiles"], 16), np.int32)
        self._check(self._lib.bsa_trace_records(self._handle, workspace.data_ptr(), _ptr(rec), st))
        return rec

    def __del__(self):
        h = getattr(self, "_handle", None)
        lib = getattr(self, "_lib", None)
        if h is not None and h.value and lib is not None:
            try:
                lib.bsa_plan_destroy(h)
            except Exception:  # interpreter shutdown
                pass
            self._handle = None


def merge_states(v: torch.Tensor, s: torch.Tensor, out_dtype: torch.dtype = torch.float32, stream=None):
    """LSE merge of attention states (bsa_merge_states).

    v: float32 (seq_len, num_states, num_heads, head_dim), s: float32
    (seq_len, num_states, num_heads).  Returns (v_merged, s_merged).
    """
    if v.dtype != torch.float32 or s.dtype != torch.float32 or not v.is_contiguous() or not s.is_contiguous():
        raise ValueError("v and s must be contiguous float32 device tensors")
    seq, ns, heads, dim = v.shape
    if s.shape != (seq, ns, heads):
        raise ValueError("s must have shape (seq_len, num_states, num_heads)")
    code = {torch.float16: L.BSA_F16, torch.bfloat16: L.BSA_BF16, torch.float32: L.BSA_FP32_OUT}[out_dtype]
    v_out = torch.empty((seq, heads, dim), dtype=out_dtype, device=v.device)
    s_out = torch.empty((seq, heads), dtype=torch.float32, device=v.device)
    st = torch.cuda.current_stream(v.device).cuda_stream if stream is None else stream
    L.check(L.lib().bsa_merge_states(v.data_ptr(), s.data_ptr(), v_out.data_ptr(), s_out.data_ptr(),
                                     seq, ns, heads, dim, code, st))
    return v_out, s_out


def indexer_topk(q: torch.Tensor, key_cache: torch.Tensor, block_table: torch.Tensor, req_row_ptr: torch.Tensor,
                 ctx_len: torch.Tensor, req_kv_len: torch.Tensor, topk: int, page_size: int,
                 max_ctx: Optional[int] = None,
                 scores: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 scores_only: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Sparse-attention indexer (bsa_indexer_topk; flashinfer.sparse "SDSA Indexer":
    indexer_scores, top_k_from_candidates): a float32 score for each key position a query row
    sees in its request's paged cache, and the row's exact Top-K keys (ties to the lower position) as
    int32 physical cache rows in ascending position order, padded with -1.

    q (num_rows, head_dim) and key_cache (num_slots, head_dim): fp16 or bf16 device
    tensors with contiguous rows; block_table (num_reqs, max_pages), req_row_ptr
    (num_reqs + 1,), ctx_len (num_rows,), req_kv_len (num_reqs,): int32 device tensors.
    max_ctx defaults to the largest ctx_len, read back from the device (a synchronising
    copy); pass it to avoid that.  workspace: a device tensor of at least
    bsa_indexer_workspace_size(num_rows, max_ctx) bytes (default: a fresh one from torch's
    allocator).  Returns (out, scores); scores has
    max_ctx rounded up to a multiple of 64 columns (row i's scores are scores[i, :n])."""
    for name, t in (("q", q), ("key_cache", key_cache)):
        if not t.is_cuda or t.dim() != 2 or t.stride(1) != 1 or t.dtype not in (torch.float16, torch.bfloat16):
            raise ValueError(f"{name} must be a 2-D fp16 / bf16 device tensor with contiguous rows")
    if q.dtype != key_cache.dtype or q.shape[1] != key_cache.shape[1]:
        raise ValueError("q and key_cache must share dtype and head_dim")
    for name, t, nd in (("block_table", block_table, 2), ("req_row_ptr", req_row_ptr, 1), ("ctx_len", ctx_len, 1),
                        ("req_kv_len", req_kv_len, 1)):
        if not t.is_cuda or t.dtype != torch.int32 or t.dim() != nd or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {nd}-D int32 device tensor")
    num_rows, num_reqs = q.shape[0], block_table.shape[0]
    if req_row_ptr.shape[0] != num_reqs + 1 or ctx_len.shape[0] != num_rows or req_kv_len.shape[0] != num_reqs:
        raise ValueError("req_row_ptr, ctx_len and req_kv_len do not match num_reqs / num_rows")
    if max_ctx is None:
        max_ctx = max(1, int(ctx_len.max().item())) if num_rows else 1
    ld = (max_ctx + 63) // 64 * 64  # score rows are padded to a multiple of 64 floats
    if scores is None:
        scores = torch.empty((num_rows, ld), dtype=torch.float32, device=q.device)
    elif scores.dtype != torch.float32 or scores.shape != (num_rows, ld) or not scores.is_contiguous():
        raise ValueError(f"scores must be a contiguous ({num_rows}, {ld}) float32 tensor")
    if out is None:
        out = torch.empty((num_rows, topk), dtype=torch.int32, device=q.device)
    elif out.dtype != torch.int32 or out.shape != (num_rows, topk) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous ({num_rows}, {topk}) int32 tensor")
    lib = L.lib()
    if not scores_only:
        need = int(lib.bsa_indexer_workspace_size(num_rows, max_ctx))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        elif (not workspace.is_cuda or not workspace.is_contiguous()
              or workspace.numel() * workspace.element_size() < need):
            raise ValueError(f"workspace must be a contiguous device tensor of at least {need} bytes")
    a = L.Indexer()
    lib.bsa_indexer_init(ctypes.byref(a))
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    a.q, a.key_cache = q.data_ptr(), key_cache.data_ptr()
    a.block_table, a.req_row_ptr = block_table.data_ptr(), req_row_ptr.data_ptr()
    a.ctx_len, a.req_kv_len = ctx_len.data_ptr(), req_kv_len.data_ptr()
    a.scores, a.out = scores.data_ptr(), out.data_ptr()
    a.num_slots, a.max_ctx = key_cache.shape[0], max_ctx
    a.q_stride, a.k_stride = q.stride(0), key_cache.stride(0)
    a.num_rows, a.num_reqs = num_rows, num_reqs
    a.max_pages, a.page_size, a.head_dim, a.topk = block_table.shape[1], page_size, q.shape[1], topk
    a.dtype = L.BSA_BF16 if q.dtype == torch.bfloat16 else L.BSA_F16
    a.scores_only = 1 if scores_only else 0
    st = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    L.check(lib.bsa_indexer_topk(ctypes.byref(a), st))
    return out, scores


def mla_rope_quantize_fp8(q_rope: torch.Tensor, k_rope: torch.Tensor, q_nope: torch.Tensor, k_nope: torch.Tensor,
                          cos_sin_cache: torch.Tensor, pos_ids: torch.Tensor, is_neox: bool = True,
                          quant_scale_q: float = 1.0, quant_scale_kv: float = 1.0,
                          q_rope_out: Optional[torch.Tensor] = None, k_rope_out: Optional[torch.Tensor] = None,
                          q_nope_out: Optional[torch.Tensor] = None, k_nope_out: Optional[torch.Tensor] = None,
                          stream=None):
    """RoPE on the 64-value tails and per-tensor FP8 E4M3 quantization of MLA q / k
    (bsa_mla_rope_quantize_fp8; MATE mla_rope_quantize_fp8).  q_rope (nnz, H, 64),
    k_rope (nnz, 64), q_nope (nnz, H, 512), k_nope (nnz, 512): bf16 device tensors with a
    contiguous last dimension; cos_sin_cache (max_seq_len, 64) fp32 or bf16; pos_ids (nnz,)
    int32 or int64.  Outputs may be given (fp8 views, e.g. slices of [..., 576] rows) or are
    allocated.  Returns (q_rope_out, k_rope_out, q_nope_out, k_nope_out)."""
    nnz, H = q_rope.shape[0], q_rope.shape[1]
    shapes = {"q_rope": (q_rope, (nnz, H, 64)), "k_rope": (k_rope, (nnz, 64)),
              "q_nope": (q_nope, (nnz, H, 512)), "k_nope": (k_nope, (nnz, 512))}
    for name, (t, shp) in shapes.items():
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shp or not t.is_cuda or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a bf16 device tensor of shape {shp} with a contiguous last dimension")
    if cos_sin_cache.dtype not in (torch.float32, torch.bfloat16) or cos_sin_cache.dim() != 2 or \
            cos_sin_cache.shape[1] != 64 or not cos_sin_cache.is_contiguous():
        raise ValueError("cos_sin_cache must be a contiguous (max_seq_len, 64) float32 or bf16 tensor")
    if pos_ids.dtype not in (torch.int32, torch.int64) or tuple(pos_ids.shape) != (nnz,) or not pos_ids.is_contiguous():
        raise ValueError("pos_ids must be a contiguous int32 or int64 tensor of nnz entries")
    f8 = torch.float8_e4m3fn
    outs = []
    for name, t in (("q_rope", q_rope_out), ("k_rope", k_rope_out), ("q_nope", q_nope_out), ("k_nope", k_nope_out)):
        shp = shapes[name][1]
        if t is None:
            t = torch.empty(shp, dtype=f8, device=q_rope.device)
        elif t.dtype != f8 or tuple(t.shape) != shp or t.stride(-1) != 1:
            raise ValueError(f"{name}_out must be a float8_e4m3fn tensor of shape {shp} with a contiguous last dimension")
        outs.append(t)
    a = L.RopeQuant()
    lib = L.lib()
    lib.bsa_rope_quant_init(ctypes.byref(a))
    a.q_rope, a.k_rope, a.q_nope, a.k_nope = (t.data_ptr() for t in (q_rope, k_rope, q_nope, k_nope))
    a.cos_sin_cache, a.cache_bf16 = cos_sin_cache.data_ptr(), int(cos_sin_cache.dtype == torch.bfloat16)
    a.pos_ids, a.pos_int64 = pos_ids.data_ptr(), int(pos_ids.dtype == torch.int64)
    a.nnz, a.num_heads, a.max_seq_len = nnz, H, cos_sin_cache.shape[0]
    a.is_neox = int(bool(is_neox))
    a.quant_scale_q, a.quant_scale_kv = float(quant_scale_q), float(quant_scale_kv)
    a.q_rope_out, a.k_rope_out, a.q_nope_out, a.k_nope_out = (t.data_ptr() for t in outs)
    a.q_rope_stride[0], a.q_rope_stride[1] = q_rope.stride(0), q_rope.stride(1)
    a.q_nope_stride[0], a.q_nope_stride[1] = q_nope.stride(0), q_nope.stride(1)
    a.k_rope_stride, a.k_nope_stride = k_rope.stride(0), k_nope.stride(0)
    a.q_rope_out_stride[0], a.q_rope_out_stride[1] = outs[0].stride(0), outs[0].stride(1)
    a.q_nope_out_stride[0], a.q_nope_out_stride[1] = outs[2].stride(0), outs[2].stride(1)
    a.k_rope_out_stride, a.k_nope_out_stride = outs[1].stride(0), outs[3].stride(0)
    st = torch.cuda.current_stream(q_rope.device).cuda_stream if stream is None else stream
    L.check(lib.bsa_mla_rope_quantize_fp8(ctypes.byref(a), st))
    return tuple(outs)

