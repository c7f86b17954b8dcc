"""The C ABI library loads, exports every declared symbol, and validates
its arguments on the host (no GPU work is started by these tests)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from paged_attention_bsr_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in bsa.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(bsa_[a-z0-9_]+)\b", out))
    assert set(names) <= exported


@pytest.mark.parametrize("path", [L.LIB_PATH, L.TRACE_LIB_PATH], ids=["product", "trace"])
def test_both_builds_export_the_same_declared_functions(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(bsa_[a-z0-9_]+)\b", out))
    assert set(_declared_functions()) <= exported


def _tiny_plan(lib):
    indptr = np.array([0, 1], np.int32)
    indices = np.array([0], np.int32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    d = L.PlanDesc()
    lib.bsa_plan_desc_init(ctypes.byref(d))
    d.indptr, d.indices = indptr.ctypes.data_as(i32p), indices.ctypes.data_as(i32p)
    d.M = d.N = d.R = d.C = 4
    d.num_qo_heads = d.num_kv_heads = 2
    d.head_dim_qk = d.head_dim_vo = 128
    d.num_cus = 256
    h = ctypes.c_void_p()
    st = lib.bsa_plan_ex(ctypes.byref(d), ctypes.byref(h))
    assert st == L.BSA_OK, lib.bsa_last_error()
    return h


def test_trace_records_only_in_the_trace_build():
    # the product build refuses on the host, before touching any device memory
    lib = L.lib()
    h = _tiny_plan(lib)
    rec = np.zeros(8, np.int32)
    st = lib.bsa_trace_records(h, ctypes.c_void_p(256), rec.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None)
    assert st == L.BSA_ERR_UNSUPPORTED and b"BSA_TRACE" in lib.bsa_last_error()
    assert lib.bsa_trace_records(h, None, rec.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None) == \
        L.BSA_ERR_INVALID_ARGUMENT
    lib.bsa_plan_destroy(h)
    # the trace build reserves one record of 8 int32 per tile after the partials
    tl = L.trace_lib()
    ht, hp = _tiny_plan(tl), _tiny_plan(lib)
    it, ip = L.PlanInfo(), L.PlanInfo()
    assert tl.bsa_plan_info(ht, ctypes.byref(it)) == 0 and lib.bsa_plan_info(hp, ctypes.byref(ip)) == 0
    assert it.table_bytes == ip.table_bytes and it.partial_bytes == ip.partial_bytes
    assert it.workspace_bytes == ip.workspace_bytes + -(-it.num_tiles * 32 // 256) * 256
    tl.bsa_plan_destroy(ht)
    lib.bsa_plan_destroy(hp)


def test_desc_layout_matches_binding():
    assert L.lib().bsa_plan_desc_sizeof() == ctypes.sizeof(L.PlanDesc)


def _desc(**kw):
    d = L.PlanDesc()
    L.lib().bsa_plan_desc_init(ctypes.byref(d))
    keep = []
    for k, v in kw.items():
        if isinstance(v, np.ndarray):
            v = np.ascontiguousarray(v, dtype=np.int32)
            keep.append(v)
            v = v.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        setattr(d, k, v)
    d._keep = keep
    return d


def _plan_status(**kw):
    kw.setdefault("num_cus", 4)
    d = _desc(**kw)
    h = ctypes.c_void_p()
    st = L.lib().bsa_plan_ex(ctypes.byref(d), ctypes.byref(h))
    msg = L.lib().bsa_last_error().decode()
    if st == 0:
        L.lib().bsa_plan_destroy(h)
    return st, msg


GOOD = dict(indptr=np.array([0, 1, 3, 5]), indices=np.array([2, 0, 2, 1, 2]), M=3, N=3, R=1, C=1,
            num_qo_heads=32, num_kv_heads=8, head_dim_qk=128)


def test_plan_without_gpu_succeeds():
    st, msg = _plan_status(**GOOD)
    assert st == L.BSA_OK, msg


@pytest.mark.parametrize("change,status", [
    (dict(indptr=np.array([1, 1, 3, 5])), L.BSA_ERR_INVALID_ARGUMENT),
    (dict(indptr=np.array([0, 3, 1, 5])), L.BSA_ERR_INVALID_ARGUMENT),
    (dict(indices=np.array([2, 0, 3, 1, 2])), L.BSA_ERR_INVALID_ARGUMENT),
    (dict(indices=np.array([2, 0, -1, 1, 2])), L.BSA_ERR_INVALID_ARGUMENT),
    (dict(indices=np.array([2, 0, 0, 1, 2])), L.BSA_ERR_INVALID_ARGUMENT),   # duplicate in row 1
    (dict(N=4, C=3), L.BSA_ERR_INVALID_ARGUMENT),                   # N % C
    (dict(R=0), L.BSA_ERR_INVALID_ARGUMENT),
    (dict(num_qo_heads=30), L.BSA_ERR_INVALID_ARGUMENT),            # not a multiple
    (dict(head_dim_qk=64), L.BSA_ERR_UNSUPPORTED),
    (dict(q_dtype=L.BSA_BF16), L.BSA_ERR_UNSUPPORTED),              # mixed dtypes
    (dict(q_dtype=L.BSA_FP8_E4M3, kv_dtype=L.BSA_FP8_E4M3), L.BSA_ERR_UNSUPPORTED),  # fp8 queries
    (dict(kv_splits=-1), L.BSA_ERR_INVALID_ARGUMENT),
    (dict(k_descale=0.0), L.BSA_ERR_INVALID_ARGUMENT),
    (dict(kv_block_lens=np.array([1, 2, 1]), N=3), L.BSA_ERR_INVALID_ARGUMENT),  # len > C
])
def test_plan_rejects(change, status):
    args = dict(GOOD)
    args.update(change)
    st, msg = _plan_status(**args)
    assert st == status, msg
    assert msg


def test_run_validates_before_touching_the_gpu():
    lib = L.lib()
    d = _desc(num_cus=4, **GOOD)
    h = ctypes.c_void_p()
    assert lib.bsa_plan_ex(ctypes.byref(d), ctypes.byref(h)) == 0
    ws_need = lib.bsa_workspace_size(h)
    assert ws_need % 256 == 0 and ws_need > 0
    fake = 1 << 40  # never dereferenced: every case below fails validation first
    cases = [
        ((None, fake, fake, fake, None, fake, ws_need), L.BSA_ERR_INVALID_ARGUMENT),     # null q
        ((fake + 8, fake, fake, fake, None, fake, ws_need), L.BSA_ERR_INVALID_ARGUMENT),  # misaligned q
        ((fake, fake, fake, fake, None, fake + 16, ws_need), L.BSA_ERR_INVALID_ARGUMENT),  # ws alignment
        ((fake, fake, fake, fake, None, fake, ws_need - 256), L.BSA_ERR_WORKSPACE_TOO_SMALL),
        ((fake, fake, fake, fake, fake + 2, fake, ws_need), L.BSA_ERR_INVALID_ARGUMENT),   # lse alignment
    ]
    for (q, k, v, o, lse, ws, n), want in cases:
        st = lib.bsa_run(h, q, k, v, o, lse, ws, n, None)
        assert st == want, lib.bsa_last_error()
    # o overlapping the workspace (q, k, v far away)
    ws = fake + (1 << 30)
    st = lib.bsa_run(h, fake, fake, fake, ws + 256, None, ws, ws_need, None)
    assert st == L.BSA_ERR_INVALID_ARGUMENT and "workspace" in lib.bsa_last_error().decode()
    # o overlapping q
    st = lib.bsa_run(h, fake, fake, fake, fake + 1024, None, ws, ws_need, None)
    assert st == L.BSA_ERR_INVALID_ARGUMENT and "q" in lib.bsa_last_error().decode()
    lib.bsa_plan_destroy(h)
    assert lib.bsa_run(None, fake, fake, fake, fake, None, fake, 1 << 20, None) == L.BSA_ERR_INVALID_ARGUMENT


def test_merge_states_validates():
    lib = L.lib()
    assert lib.bsa_merge_states(None, None, None, None, 4, 0, 2, 8, 0, None) == L.BSA_ERR_INVALID_ARGUMENT
    assert lib.bsa_merge_states(None, None, None, None, 4, 2, 2, 6, 0, None) == L.BSA_ERR_INVALID_ARGUMENT
    assert lib.bsa_merge_states(None, None, None, None, 4, 2, 2, 8, 9, None) == L.BSA_ERR_UNSUPPORTED
    assert lib.bsa_merge_states(None, None, None, None, 0, 2, 2, 8, 0, None) == L.BSA_OK


def test_rope_quant_layout_matches_binding():
    import ctypes
    from paged_attention_bsr_amd import _lib as L
    assert L.lib().bsa_rope_quant_sizeof() == ctypes.sizeof(L.RopeQuant)
    a = L.RopeQuant()
    L.lib().bsa_rope_quant_init(ctypes.byref(a))
    assert (a.is_neox, a.quant_scale_q, a.quant_scale_kv, a.nnz) == (1, 1.0, 1.0, 0)


def test_indexer_layout_matches_binding():
    import ctypes
    from paged_attention_bsr_amd import _lib as L
    assert L.lib().bsa_indexer_sizeof() == ctypes.sizeof(L.Indexer)
    a = L.Indexer()
    L.lib().bsa_indexer_init(ctypes.byref(a))
    assert (a.dtype, a.num_rows, a.topk, a.q_stride, a.scores_only) == (L.BSA_BF16, 0, 0, 0, 0)


def test_indexer_validates_before_touching_the_gpu():
    import ctypes
    from paged_attention_bsr_amd import _lib as L
    lib = L.lib()

    def base():
        a = L.Indexer()
        lib.bsa_indexer_init(ctypes.byref(a))
        a.num_rows, a.num_reqs, a.max_pages, a.page_size = 0, 1, 4, 16
        a.head_dim, a.topk, a.num_slots, a.max_ctx = 128, 8, 64, 64
        return a

    a = base()
    assert lib.bsa_indexer_topk(ctypes.byref(a), None) == L.BSA_OK          # no rows: nothing to do
    a.num_rows = 2
    assert lib.bsa_indexer_topk(ctypes.byref(a), None) == L.BSA_ERR_INVALID_ARGUMENT  # NULL arrays
    assert b"16-byte aligned" in lib.bsa_last_error()
    assert lib.bsa_indexer_topk(None, None) == L.BSA_ERR_INVALID_ARGUMENT
    # the workspace: per (row, chunk of 16384 positions) a count and 12288 candidates
    ws = lib.bsa_indexer_workspace_size
    assert ws(0, 100) == 0 and ws(3, 0) == 0
    assert ws(1, 16384) == 256 + 12288 * 8 and ws(2, 16385) == 256 + 4 * 12288 * 8
    a = base()
    a.num_rows = 2
    # host-side checks up to the workspace (16-byte aligned fake device addresses, never dereferenced)
    for f in ("q", "key_cache", "scores", "block_table", "req_row_ptr", "ctx_len", "req_kv_len", "out"):
        setattr(a, f, 1 << 20)
    assert lib.bsa_indexer_topk(ctypes.byref(a), None) == L.BSA_ERR_INVALID_ARGUMENT
    assert b"workspace" in lib.bsa_last_error()
    a.workspace, a.workspace_bytes = 1 << 20, ws(2, 64) - 1
    assert lib.bsa_indexer_topk(ctypes.byref(a), None) == L.BSA_ERR_INVALID_ARGUMENT
    assert b"workspace" in lib.bsa_last_error()
    for field, value in (("head_dim", 96), ("topk", 0), ("topk", (1 << 24) + 1), ("num_reqs", 0), ("page_size", 0), ("max_pages", 0),
                         ("num_slots", 0), ("max_ctx", 0), ("dtype", L.BSA_FP8_E4M3), ("q_stride", 100),
                         ("k_stride", 64), ("max_ctx", 1 << 25)):
        a = base()
        setattr(a, field, value)
        assert lib.bsa_indexer_topk(ctypes.byref(a), None) == L.BSA_ERR_INVALID_ARGUMENT, field


def test_rope_quant_validates_before_touching_the_gpu():
    import ctypes
    from paged_attention_bsr_amd import _lib as L
    lib = L.lib()
    a = L.RopeQuant()
    lib.bsa_rope_quant_init(ctypes.byref(a))
    a.num_heads, a.max_seq_len, a.nnz = 4, 16, 0
    assert lib.bsa_mla_rope_quantize_fp8(ctypes.byref(a), None) == L.BSA_OK      # nothing to do
    a.nnz = 3
    assert lib.bsa_mla_rope_quantize_fp8(ctypes.byref(a), None) == L.BSA_ERR_INVALID_ARGUMENT  # NULL arrays
    a.nnz, a.num_heads = 0, 0
    assert lib.bsa_mla_rope_quantize_fp8(ctypes.byref(a), None) == L.BSA_ERR_INVALID_ARGUMENT
    a.num_heads, a.quant_scale_q = 4, float("inf")
    assert lib.bsa_mla_rope_quantize_fp8(ctypes.byref(a), None) == L.BSA_ERR_INVALID_ARGUMENT
    assert lib.bsa_mla_rope_quantize_fp8(None, None) == L.BSA_ERR_INVALID_ARGUMENT


def test_noalloc_limit_matches_header_and_refuses_large_plans_on_the_host():
    """bsa_run_noalloc's workspace limit is the header's BSA_NOALLOC_MAX_WORKSPACE; a plan
    needing more is refused before anything touches the GPU (fake pointers: never used)."""
    text = open(HEADER).read()
    m = re.search(r"#define BSA_NOALLOC_MAX_WORKSPACE \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == L.BSA_NOALLOC_MAX_WORKSPACE
    from paged_attention_bsr_amd import workloads as W
    w = W.bsr_prefill(M=8192, values=False)
    d = _desc(indptr=w.indptr, indices=w.indices, M=w.M, N=w.N, R=w.R, C=w.C, num_qo_heads=32, num_kv_heads=8,
              head_dim_qk=128, causal=1, kv_splits=8, num_cus=256)
    lib = L.lib()
    h = ctypes.c_void_p()
    assert lib.bsa_plan_ex(ctypes.byref(d), ctypes.byref(h)) == L.BSA_OK
    assert lib.bsa_workspace_size(h) > L.BSA_NOALLOC_MAX_WORKSPACE
    fake = 1 << 40
    st = lib.bsa_run_noalloc(h, fake, fake, fake, fake + (1 << 32), None, None)
    assert st == L.BSA_ERR_WORKSPACE_TOO_SMALL and "bsa_run_noalloc" in lib.bsa_last_error().decode()
    lib.bsa_plan_destroy(h)
    assert lib.bsa_run_noalloc(None, fake, fake, fake, fake, None, None) == L.BSA_ERR_INVALID_ARGUMENT


def test_bsa_log_prints_plan_statistics():
    # BSA_LOG=1: one line per planning call on stderr, with the plan's statistics or the error
    code = (
        "import ctypes, numpy as np\n"
        "from paged_attention_bsr_amd import _lib as L\n"
        "lib = L.lib()\n"
        "d = L.PlanDesc(); lib.bsa_plan_desc_init(ctypes.byref(d))\n"
        "ip = np.array([0, 2], np.int32); ix = np.array([0, 1], np.int32)\n"
        "P = ctypes.POINTER(ctypes.c_int32)\n"
        "d.indptr, d.indices = ip.ctypes.data_as(P), ix.ctypes.data_as(P)\n"
        "d.M, d.N, d.R, d.C, d.num_cus = 4, 8, 4, 4, 8\n"
        "h = ctypes.c_void_p()\n"
        "assert lib.bsa_plan_ex(ctypes.byref(d), ctypes.byref(h)) == 0\n"
        "d.N = 6\n"
        "assert lib.bsa_plan_ex(ctypes.byref(d), ctypes.byref(h)) != 0\n"
    )
    env = dict(os.environ, BSA_LOG="1")
    r = subprocess.run([__import__("sys").executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[bsa] plan")]
    assert len(lines) == 2, r.stderr
    assert "kernel=tile" in lines[0] and "tiles=" in lines[0] and "workspace=" in lines[0]
    assert "failed" in lines[1]
    env["BSA_LOG"] = "0"
    r = subprocess.run([__import__("sys").executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and "[bsa] plan" not in r.stderr
