"""bsa_run_noalloc (the library's own static workspace, no allocation) against
bsa_run (a caller workspace) through the C ABI: two calls in a row, the second
with a smaller input, each compared with bsa_run's result and with the oracle."""
import ctypes

import pytest
import torch

from paged_attention_bsr_amd import Plan
from paged_attention_bsr_amd import _lib as L
from paged_attention_bsr_amd import workloads as W
from tests.parity_util import compare, oracle_result, say, tol_for

pytestmark = pytest.mark.gpu


def _plan(w, kv_splits):
    return Plan(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                head_dim_vo=w.head_dim_vo, causal=w.causal, kv_splits=kv_splits, kv_block_lens=w.kv_block_lens,
                q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, o_dtype=w.o_dtype, k_descale=w.k_descale,
                v_descale=w.v_descale, k_token_stride=w.k_token_stride, v_token_stride=w.v_token_stride)


def _both(w, kv_splits):
    """(o, lse) from bsa_run with its own workspace and from bsa_run_noalloc."""
    lib = L.lib()
    p = _plan(w, kv_splits)
    assert p.workspace_size <= L.BSA_NOALLOC_MAX_WORKSPACE
    dev = torch.device("cuda")
    q, k = w.q.to(dev), w.k.to(dev)
    v = k if w.v_aliases_k else w.v.to(dev)
    st = torch.cuda.current_stream().cuda_stream
    res = []
    for noalloc in (False, True):
        o = torch.full((w.M, w.num_qo_heads, w.head_dim_vo), float("nan"), dtype=w.o_dtype, device=dev)
        lse = torch.full((w.M, w.num_qo_heads), float("nan"), dtype=torch.float32, device=dev)
        if noalloc:
            L.check(lib.bsa_run_noalloc(p._handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        lse.data_ptr(), st))
        else:
            ws = torch.empty(p.workspace_size, dtype=torch.uint8, device=dev)
            L.check(lib.bsa_run(p._handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), ws.data_ptr(), p.workspace_size, st))
        torch.cuda.synchronize()
        res.append((o, lse))
    return res


CASES = [
    # two calls in a row on one kernel family, the second smaller (fewer rows and keys)
    ("decode", lambda: W.paged_decode(seed=81, batch=40, min_len=100, max_len=3000),
     lambda: W.paged_decode(seed=82, batch=9, min_len=20, max_len=700), 0),
    ("prefill", lambda: W.bsr_prefill(seed=83, M=1024, density=0.3),   # 31.3 MiB of 32: near the limit
     lambda: W.bsr_prefill(seed=84, M=512, density=0.5), 3),
    ("mla", lambda: W.sparse_mla(seed=85, num_tokens=8, num_heads=128, cache_rows=4096, topk=512, min_ctx=1024,
                                 max_ctx=4096),
     lambda: W.sparse_mla(seed=86, num_tokens=3, num_heads=64, cache_rows=2048, topk=96, min_ctx=512,
                          max_ctx=2048), 2),
]


@pytest.mark.parametrize("name,big,small,kv_splits", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_run(name, big, small, kv_splits):
    for label, make in (("first", big), ("second, smaller", small)):
        w = make()
        what = f"noalloc {name} {label} M={w.M} N={w.N} splits={kv_splits}"
        say(f"[parity] {what}")
        (o1, l1), (o2, l2) = _both(w, kv_splits)
        # the same kernels on the same tables and inputs: identical bits
        assert torch.equal(o1, o2) and torch.equal(l1, l2), what
        o_ref, lse_ref = oracle_result(w)
        compare(o2, l2, o_ref, lse_ref, tol_for(w), what)


def test_noalloc_runs_again_after_another_plan():
    """Plan A, plan B, plan A again through bsa_run_noalloc: the shared array's tables
    follow the plan of each call."""
    wa = W.bsr_prefill(seed=87, M=1024, density=0.4)
    wb = W.paged_decode(seed=88, batch=12, min_len=50, max_len=900)
    pa, pb = _plan(wa, 2), _plan(wb, 0)
    dev = torch.device("cuda")
    lib = L.lib()
    st = torch.cuda.current_stream().cuda_stream
    outs = []
    for p, w in ((pa, wa), (pb, wb), (pa, wa)):
        q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
        o = torch.empty(w.M, w.num_qo_heads, w.head_dim_vo, dtype=w.o_dtype, device=dev)
        lse = torch.empty(w.M, w.num_qo_heads, dtype=torch.float32, device=dev)
        L.check(lib.bsa_run_noalloc(p._handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), st))
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[0][1], outs[2][1])
    for (o, lse), w in ((outs[1], wb), (outs[2], wa)):
        o_ref, lse_ref = oracle_result(w)
        compare(o, lse, o_ref, lse_ref, tol_for(w), "noalloc A/B/A")
