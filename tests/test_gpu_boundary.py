"""The boundary calls themselves on real work: bsa_plan (the 12-argument form),
bsa_workspace_size, bsa_upload / bsa_unpin and bsa_run through ctypes with
device pointers, checked against the oracle; and the workspace-binding rules
(a run on a workspace that is not pinned to its plan copies the tables)."""
import ctypes

import numpy as np
import pytest
import torch

from paged_attention_bsr_amd import Plan
from paged_attention_bsr_amd import _lib as L
from paged_attention_bsr_amd import workloads as W
from tests.parity_util import compare, oracle_result, say, tol_for

pytestmark = pytest.mark.gpu


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _north_star_run(w, kv_splits, pin):
    """bsa_plan + bsa_workspace_size + (bsa_upload) + bsa_run on w's fp16 tensors."""
    lib = L.lib()
    indptr = np.ascontiguousarray(w.indptr, np.int32)
    indices = np.ascontiguousarray(w.indices, np.int32)
    h = ctypes.c_void_p()
    L.check(lib.bsa_plan(_i32p(indptr), _i32p(indices), w.M, w.N, w.R, w.C, w.num_qo_heads, w.num_kv_heads,
                         w.head_dim, int(w.causal), 0.0, kv_splits, ctypes.byref(h)))
    try:
        nbytes = lib.bsa_workspace_size(h)
        assert nbytes > 0 and nbytes % 256 == 0
        dev = torch.device("cuda")
        q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
        o = torch.empty(w.M, w.num_qo_heads, w.head_dim, dtype=torch.float16, device=dev)
        lse = torch.empty(w.M, w.num_qo_heads, dtype=torch.float32, device=dev)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        st = torch.cuda.current_stream().cuda_stream
        if pin:
            L.check(lib.bsa_upload(h, ws.data_ptr(), nbytes, st))
        for _ in range(2):   # the second run reuses (pinned) or re-copies (unpinned) the tables
            L.check(lib.bsa_run(h, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                ws.data_ptr(), nbytes, st))
        torch.cuda.synchronize()
        if pin:
            L.check(lib.bsa_unpin(h, ws.data_ptr()))
        return o, lse
    finally:
        lib.bsa_plan_destroy(h)


NORTH_STAR = [
    ("worked_example", lambda: W.worked_example(), 1),
    ("worked_example_auto", lambda: W.worked_example(), 0),
    ("bsr_prefill_1024", lambda: W.bsr_prefill(seed=71, M=1024, density=0.3), 1),
    ("bsr_prefill_1024_split", lambda: W.bsr_prefill(seed=72, M=1024, density=0.3), 3),
    ("decode_full_pages", lambda: W.random_bsr(73, 24, 60 * 16, 1, 16, 32, 8, density=0.4), 0),
]


@pytest.mark.parametrize("pin", [False, True])
@pytest.mark.parametrize("name,make,kv_splits", NORTH_STAR, ids=[c[0] for c in NORTH_STAR])
def test_north_star_plan_and_run(name, make, kv_splits, pin):
    w = make()
    assert w.kv_block_lens is None and w.q_dtype == torch.float16
    what = f"north-star bsa_plan/bsa_run {name} splits={kv_splits} pin={pin}"
    say(f"[parity] {what}")
    o, lse = _north_star_run(w, kv_splits, pin)
    o_ref, lse_ref = oracle_result(w)
    compare(o, lse, o_ref, lse_ref, tol_for(w), what)


def test_workspace_freed_and_reused_at_the_same_address():
    """Plan.run pins its tables in a caller's workspace tensor.  When that tensor is freed,
    its memory refilled with other data, and a new workspace tensor comes back at the same
    address, the binding must copy the tables again (the address alone proves nothing)."""
    w = W.bsr_prefill(seed=74, M=512, density=0.5)
    p = Plan(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.num_qo_heads, w.num_kv_heads, w.head_dim,
             causal=w.causal, kv_splits=3)
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    n = p.workspace_size
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    addr = ws.data_ptr()
    o1, l1 = p.run(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    del ws
    junk = torch.full((n,), 0x7F, dtype=torch.uint8, device=dev)   # tile indices of 0x7F7F7F7F
    reused = junk.data_ptr() == addr
    del junk
    ws2 = torch.empty(n, dtype=torch.uint8, device=dev)
    say(f"[parity] workspace reuse: same address {reused and ws2.data_ptr() == addr}")
    o2, l2 = p.run(q, k, v, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle_result(w)
    compare(o2, l2, o_ref, lse_ref, tol_for(w), "workspace reuse")


def test_two_plans_alternating_on_one_workspace():
    """Plan A pinned in a workspace; a run of plan B there replaces A's tables (and ends A's
    pin); the next run of A must copy its own tables back."""
    wa = W.bsr_prefill(seed=75, M=512, density=0.4)
    wb = W.random_bsr(76, 40, 30 * 16, 1, 16, 32, 8, density=0.5)
    pa = Plan(wa.indptr, wa.indices, wa.M, wa.N, wa.R, wa.C, wa.num_qo_heads, wa.num_kv_heads, wa.head_dim,
              causal=wa.causal, kv_splits=2)
    pb = Plan(wb.indptr, wb.indices, wb.M, wb.N, wb.R, wb.C, wb.num_qo_heads, wb.num_kv_heads, wb.head_dim,
              kv_splits=0)
    dev = torch.device("cuda")
    ws = torch.empty(max(pa.workspace_size, pb.workspace_size), dtype=torch.uint8, device=dev)
    qa, ka, va = (t.to(dev) for t in (wa.q, wa.k, wa.v))
    qb, kb, vb = (t.to(dev) for t in (wb.q, wb.k, wb.v))
    lib = L.lib()
    st = torch.cuda.current_stream().cuda_stream
    L.check(lib.bsa_upload(pa._handle, ws.data_ptr(), ws.numel(), st))
    outs = []
    for plan, (q, k, v), w in ((pa, (qa, ka, va), wa), (pb, (qb, kb, vb), wb), (pa, (qa, ka, va), wa)):
        o = torch.empty(w.M, w.num_qo_heads, w.head_dim, dtype=torch.float16, device=dev)
        lse = torch.empty(w.M, w.num_qo_heads, dtype=torch.float32, device=dev)
        # straight through the C ABI: no binding-side bookkeeping
        L.check(lib.bsa_run(plan._handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), ws.data_ptr(), ws.numel(), st))
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[0][1], outs[2][1])
    for (o, lse), w, what in ((outs[1], wb, "plan B"), (outs[2], wa, "plan A again")):
        o_ref, lse_ref = oracle_result(w)
        compare(o, lse, o_ref, lse_ref, tol_for(w), what)


@pytest.mark.parametrize("kv_splits", [1, 0])
def test_bound_run_matches_run(kv_splits):
    # Plan.bind validates once and then only calls bsa_run_ex: same bits as run(),
    # call after call, also for the attention phase alone followed by the merge phase
    w = W.paged_decode(seed=61, batch=9, min_len=5, max_len=900)
    say(f"[boundary] bind vs run, splits={kv_splits}")
    plan = Plan(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                kv_splits=kv_splits, kv_block_lens=w.kv_block_lens, q_dtype=w.q_dtype)
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    o_ref, l_ref = plan.run(q, k, v)
    fn, o, lse = plan.bind(q, k, v)
    attn, o2, l2 = plan.bind(q, k, v, phase=L.BSA_PHASE_ATTENTION)
    merge, _, _ = plan.bind(q, k, v, out=o2, lse=l2, phase=L.BSA_PHASE_MERGE)
    for _ in range(3):
        o.zero_(), lse.zero_(), o2.zero_(), l2.zero_()
        fn()
        attn()
        merge()
        torch.cuda.synchronize()
        for a, b in ((o, o_ref), (lse, l_ref), (o2, o_ref), (l2, l_ref)):
            assert torch.equal(a, b)
