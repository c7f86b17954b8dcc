"""The kernels walk exactly the planner's tables.

The trace build of the library (libbsa_trace.so, the same sources compiled
with BSA_TRACE) has every kernel record, per planner tile, how often it ran
the tile, the first and last column entries whose keys it loaded, how many
keys inside their blocks' valid lengths it loaded, and where it wrote
(bsa_trace_records).  These records must equal what bsa_plan_export says
each tile covers, bit for bit, for the five reduced workloads and the
structural variants, at kv_splits 1, 3 and automatic; and the trace build's
outputs must equal the product build's bit for bit (the records change
nothing else)."""
import numpy as np
import pytest
import torch

from paged_attention_bsr_amd import workloads as W
from tests.parity_util import plan_for, say, scales_for, to_device

pytestmark = pytest.mark.gpu

INT32_MAX = np.iinfo(np.int32).max


def _expected(w, tables):
    """Per-tile records implied by the exported tables: {1, first entry with a
    valid key, last such entry + 1, key_count, partial_offset, kv_head, row0, nrows}."""
    tiles, cols = tables["tiles"], tables["cols"]
    lens = w.kv_block_lens
    ent_len = (np.full(cols.shape, w.C, np.int64) if lens is None
               else np.asarray(lens, np.int64)[cols.astype(np.int64)])
    exp = np.zeros_like(tiles)
    exp[:, 0] = 1
    for t, (_, kvh, row0, nrows, cb, ce, part, keys) in enumerate(tiles):
        live = np.nonzero(ent_len[cb:ce] > 0)[0]
        exp[t, 1] = cb + live[0] if live.size else INT32_MAX
        exp[t, 2] = cb + live[-1] + 1 if live.size else 0
        exp[t, 3:] = (keys, part, kvh, row0, nrows)
    return exp


def _check_trace(w, kv_splits):
    what = f"{w.name} M={w.M} N={w.N} R={w.R} C={w.C} splits={kv_splits}"
    say(f"[trace] {what}")
    pt = plan_for(w, kv_splits, trace=True)
    pp = plan_for(w, kv_splits)
    tt, tp = pt.tables(), pp.tables()
    for key in tp:
        assert np.array_equal(tt[key], tp[key]), f"{what}: trace build planned {key} differently"
    q, k, v = to_device(w)
    sc = scales_for(w)
    ws = pt.workspace(q.device)
    ws.fill_(0xA5)  # records and partials start from garbage; the run resets the records
    o_t, l_t = pt.run(q, k, v, workspace=ws, **sc)
    rec = pt.trace_records(ws)
    o_p, l_p = pp.run(q, k, v, **sc)
    torch.cuda.synchronize()
    exp = _expected(w, tt)
    bad = np.nonzero((rec != exp).any(axis=1))[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {len(rec)} tiles differ; first tile {bad[0]}:\n"
                           f"  kernel  {rec[bad[0]].tolist()}\n  planner {exp[bad[0]].tolist()}")
    assert torch.equal(o_t.view(torch.int16) if o_t.dtype != torch.float32 else o_t.view(torch.int32),
                       o_p.view(torch.int16) if o_p.dtype != torch.float32 else o_p.view(torch.int32)), \
        f"{what}: trace build output differs from the product build"
    assert torch.equal(l_t.view(torch.int32), l_p.view(torch.int32)), f"{what}: lse differs between builds"
    say(f"[trace] {what}: {len(rec)} tiles, {int(rec[:, 3].sum())} keys, records equal the tables")


REDUCED = {
    "worked_example": lambda: W.worked_example(),
    "paged_decode": lambda: W.paged_decode(seed=31, batch=12, min_len=1, max_len=700),
    "bsr_prefill": lambda: W.bsr_prefill(seed=32, M=1024, density=0.3),
    "window_prefill": lambda: W.window_prefill(seed=33, M=2048, num_qo_heads=16, num_kv_heads=2, window=3,
                                               stride=5),
    "sparse_mla": lambda: W.sparse_mla(seed=34, num_tokens=6, num_heads=128, cache_rows=4096, topk=256,
                                       min_ctx=512, max_ctx=4096),
}


@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("kv_splits", [1, 3, 0])
def test_trace_reduced_workloads(name, kv_splits):
    _check_trace(REDUCED[name](), kv_splits)


def _fp8_prefill():
    w = W.bsr_prefill(seed=100, M=1024, density=0.3)
    W.fp8_kv(w, 100)
    return w


VARIANTS = {
    # causal + partial block lengths on the tile kernel, odd sizes
    "causal_lens": lambda: W.random_bsr(7, 33, 12 * 16, 11, 16, 12, 3, causal=True, partial_lens=True,
                                        density=0.5, garbage=6e4),
    # C = 3 with lengths (key tiles spanning many blocks)
    "c3_lens": lambda: W.random_bsr(10, 70, 30 * 3, 70, 3, 4, 4, partial_lens=True, density=0.5, garbage=6e4),
    # decode shape with partial pages through the decode kernel
    "decode_lens": lambda: W.random_bsr(5, 9, 40 * 16, 1, 16, 32, 8, partial_lens=True, density=0.4,
                                        garbage=6e4),
    "empty_rows": lambda: W.random_bsr(21, 40, 8 * 4, 4, 4, 8, 2, density=0.15),
    "fp8_prefill": _fp8_prefill,
    "head_sparse": lambda: W.head_sparse_prefill(seed=48, M=1024),
    "element_mask": lambda: W.element_mask_prefill(seed=58, M=1024),
    "variable_block": lambda: W.variable_block_prefill(seed=59, M=1024),
}


@pytest.mark.parametrize("name", list(VARIANTS))
@pytest.mark.parametrize("kv_splits", [1, 0])
def test_trace_structural_variants(name, kv_splits):
    _check_trace(VARIANTS[name](), kv_splits)


@pytest.mark.parametrize("name", W.WORKLOAD_NAMES)
def test_trace_full_size_bench_launch(name):
    # every workload at its full size, in the launch configuration the benchmark times
    _check_trace(W.by_name(name), W.BENCH_KV_SPLITS[name])
