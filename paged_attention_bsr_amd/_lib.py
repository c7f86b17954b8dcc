"""ctypes declarations of libbsa.so (include/bsa.h).  Loading fails loudly if
the library has not been built; there is no fallback implementation.

trace_lib() loads libbsa_trace.so, the same sources built with BSA_TRACE
(per-tile trace records, bsa_trace_records), which only tests use."""
from __future__ import annotations

import ctypes
import os

# BSA_LIBRARY names another build of the same C ABI to load instead (the planner's
# sanitizer tests use a host-only one that lacks the device entry points)
LIB_PATH = os.environ.get("BSA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsa.so")
TRACE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsa_trace.so")

BSA_OK = 0
BSA_ERR_INVALID_ARGUMENT = 1
BSA_ERR_UNSUPPORTED = 2
BSA_ERR_WORKSPACE_TOO_SMALL = 3
BSA_ERR_HIP = 4
BSA_ERR_HOST_ALLOC = 5

BSA_F16, BSA_BF16, BSA_FP8_E4M3, BSA_FP32_OUT = 0, 1, 2, 3
BSA_KERNEL_TILE, BSA_KERNEL_MLA, BSA_KERNEL_DECODE = 0, 1, 2
BSA_PHASE_ATTENTION, BSA_PHASE_MERGE, BSA_PHASE_ALL = 1, 2, 3
BSA_NOALLOC_MAX_WORKSPACE = 32 << 20   # bytes of bsa_run_noalloc's own workspace (bsa.h)

_i32p = ctypes.POINTER(ctypes.c_int32)


class PlanDesc(ctypes.Structure):
    _fields_ = [
        ("indptr", _i32p),
        ("indices", _i32p),
        ("M", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("R", ctypes.c_int32),
        ("C", ctypes.c_int32),
        ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_vo", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("kv_splits", ctypes.c_int32),
        ("kv_block_lens", _i32p),
        ("q_dtype", ctypes.c_int),
        ("kv_dtype", ctypes.c_int),
        ("o_dtype", ctypes.c_int),
        ("q_descale", ctypes.c_float),
        ("k_descale", ctypes.c_float),
        ("v_descale", ctypes.c_float),
        ("q_token_stride", ctypes.c_int64),
        ("k_token_stride", ctypes.c_int64),
        ("v_token_stride", ctypes.c_int64),
        ("o_token_stride", ctypes.c_int64),
        ("num_cus", ctypes.c_int32),
        ("struct_heads", ctypes.c_int32),
        ("block_mask", ctypes.POINTER(ctypes.c_uint8)),
        ("q2k_indices", _i32p),
        ("q2k_num", _i32p),
        ("q2k_topk", ctypes.c_int32),
        ("mask", ctypes.POINTER(ctypes.c_uint8)),
        ("mask_packed", ctypes.c_int32),
        ("block_row_sz", _i32p),
        ("block_col_sz", _i32p),
        ("var_row_blocks", ctypes.c_int32),
        ("var_col_blocks", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("tile_rows", ctypes.c_int32),
        ("key_tile", ctypes.c_int32),
        ("num_tiles", ctypes.c_int32),
        ("num_merges", ctypes.c_int32),
        ("num_cols", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int32),
        ("heads_per_wg", ctypes.c_int32),
        ("table_bytes", ctypes.c_int64),
        ("partial_bytes", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("valid_pairs", ctypes.c_int64),
        ("R", ctypes.c_int32),
        ("C", ctypes.c_int32),
        ("mask_plane_words", ctypes.c_int64),
    ]


class RopeQuant(ctypes.Structure):
    _fields_ = [
        ("q_rope", ctypes.c_void_p),
        ("k_rope", ctypes.c_void_p),
        ("q_nope", ctypes.c_void_p),
        ("k_nope", ctypes.c_void_p),
        ("cos_sin_cache", ctypes.c_void_p),
        ("cache_bf16", ctypes.c_int32),
        ("pos_ids", ctypes.c_void_p),
        ("pos_int64", ctypes.c_int32),
        ("nnz", ctypes.c_int64),
        ("num_heads", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int64),
        ("is_neox", ctypes.c_int32),
        ("quant_scale_q", ctypes.c_float),
        ("quant_scale_kv", ctypes.c_float),
        ("q_rope_out", ctypes.c_void_p),
        ("k_rope_out", ctypes.c_void_p),
        ("q_nope_out", ctypes.c_void_p),
        ("k_nope_out", ctypes.c_void_p),
        ("q_rope_stride", ctypes.c_int64 * 2),
        ("q_nope_stride", ctypes.c_int64 * 2),
        ("k_rope_stride", ctypes.c_int64),
        ("k_nope_stride", ctypes.c_int64),
        ("q_rope_out_stride", ctypes.c_int64 * 2),
        ("q_nope_out_stride", ctypes.c_int64 * 2),
        ("k_rope_out_stride", ctypes.c_int64),
        ("k_nope_out_stride", ctypes.c_int64),
    ]



class Indexer(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("key_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("req_row_ptr", ctypes.c_void_p),
        ("ctx_len", ctypes.c_void_p),
        ("req_kv_len", ctypes.c_void_p),
        ("scores", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("num_slots", ctypes.c_int64),
        ("max_ctx", ctypes.c_int64),
        ("q_stride", ctypes.c_int64),
        ("k_stride", ctypes.c_int64),
        ("num_rows", ctypes.c_int32),
        ("num_reqs", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scores_only", ctypes.c_int32),
    ]


_lib = None
_trace_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libbsa.so, with argument/return types declared."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def trace_lib() -> ctypes.CDLL:
    """The loaded libbsa_trace.so (test builds with per-tile trace records)."""
    global _trace_lib
    if _trace_lib is None:
        _trace_lib = _load(TRACE_LIB_PATH)
    return _trace_lib


class _Declarer:
    """Attribute setter that skips functions a host-only build does not export."""

    def __init__(self, lib: ctypes.CDLL, host_only: bool):
        self._lib, self._host_only = lib, host_only

    def __getattr__(self, name):
        try:
            return getattr(self._lib, name)
        except AttributeError:
            if not self._host_only:
                raise
            return _Sink()


class _Sink:
    """Absorbs argtypes / restype of a function the loaded build does not have."""

    argtypes = restype = None


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_attention_bsr_amd.build`")
    lib = ctypes.CDLL(path)
    host_only = not hasattr(lib, "bsa_run")
    L = _Declarer(lib, host_only)
    vp, st, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.bsa_plan_desc_init.argtypes = [ctypes.POINTER(PlanDesc)]
    L.bsa_plan_desc_init.restype = None
    L.bsa_plan_desc_sizeof.argtypes = []
    L.bsa_plan_desc_sizeof.restype = sz
    L.bsa_plan.argtypes = [_i32p, _i32p, i64, i64, i32, i32, i32, i32, i32, i32, f32, i32, ctypes.POINTER(vp)]
    L.bsa_plan.restype = st
    L.bsa_plan_ex.argtypes = [ctypes.POINTER(PlanDesc), ctypes.POINTER(vp)]
    L.bsa_plan_ex.restype = st
    L.bsa_workspace_size.argtypes = [vp]
    L.bsa_workspace_size.restype = sz
    L.bsa_upload.argtypes = [vp, vp, sz, vp]
    L.bsa_upload.restype = st
    L.bsa_unpin.argtypes = [vp, vp]
    L.bsa_unpin.restype = st
    L.bsa_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.bsa_run.restype = st
    L.bsa_run_phase.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.bsa_run_phase.restype = st
    L.bsa_run_ex.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.bsa_run_ex.restype = st
    L.bsa_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.bsa_run_noalloc.restype = st
    L.bsa_merge_states.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, vp]
    L.bsa_merge_states.restype = st
    L.bsa_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.bsa_plan_info.restype = st
    L.bsa_plan_export.argtypes = [vp, _i32p, _i32p, _i32p]
    L.bsa_plan_export.restype = st
    L.bsa_plan_export_workgroups.argtypes = [vp, _i32p]
    L.bsa_plan_export_workgroups.restype = st
    L.bsa_plan_export_mask_bits.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32)]
    L.bsa_plan_export_mask_bits.restype = st
    L.bsa_rope_quant_init.argtypes = [ctypes.POINTER(RopeQuant)]
    L.bsa_rope_quant_init.restype = None
    L.bsa_rope_quant_sizeof.argtypes = []
    L.bsa_rope_quant_sizeof.restype = sz
    L.bsa_mla_rope_quantize_fp8.argtypes = [ctypes.POINTER(RopeQuant), vp]
    L.bsa_mla_rope_quantize_fp8.restype = st
    L.bsa_indexer_init.argtypes = [ctypes.POINTER(Indexer)]
    L.bsa_indexer_init.restype = None
    L.bsa_indexer_sizeof.argtypes = []
    L.bsa_indexer_sizeof.restype = sz
    L.bsa_indexer_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64]
    L.bsa_indexer_workspace_size.restype = sz
    L.bsa_indexer_topk.argtypes = [ctypes.POINTER(Indexer), vp]
    L.bsa_indexer_topk.restype = st
    L.bsa_plan_destroy.argtypes = [vp]
    L.bsa_plan_destroy.restype = None
    L.bsa_last_error.argtypes = []
    L.bsa_last_error.restype = ctypes.c_char_p
    L.bsa_trace_records.argtypes = [vp, vp, _i32p, vp]
    L.bsa_trace_records.restype = st
    if L.bsa_plan_desc_sizeof() != ctypes.sizeof(PlanDesc):
        raise RuntimeError("bsa_plan_desc_t layout mismatch between bsa.h and the Python binding")
    return lib


class BsaError(RuntimeError):
    """A libbsa call returned a status other than BSA_OK."""

    def __init__(self, status: int, message: str):
        super().__init__(f"bsa status {status}: {message}")
        self.status = status


def check(status: int, library: ctypes.CDLL | None = None) -> None:
    """Raise BsaError with the last error message of ``library`` (default libbsa.so)."""
    if status != BSA_OK:
        raise BsaError(status, (library or lib()).bsa_last_error().decode(errors="replace"))
