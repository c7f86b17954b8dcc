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
    valid key, last such entry + 1, key_count, partial_offset, kv_head, row0, nrows,
    0 key tokens outside [0, N), 7 x the host's fill -2}."""
    tiles, cols = tables["tiles"], tables["cols"]
    lens = w.kv_block_lens
    ent_len = (np.full(cols.shape, w.C, np.int64) if lens is None
               else np.asarray(lens, np.int64)[cols.astype(np.int64)])
    exp = np.full((len(tiles), 16), -2, np.int32)
    exp[:, 0] = 1
    exp[:, 8] = 0
    for t, (_, kvh, row0, nrows, cb, ce, part, keys) in enumerate(tiles):
        live = np.nonzero(ent_len[cb:ce] > 0)[0]
        exp[t, 1] = cb + live[0] if live.size else INT32_MAX
        exp[t, 2] = cb + live[-1] + 1 if live.size else 0
        exp[t, 3:8] = (keys, part, kvh, row0, nrows)
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


def _corrupt_case(kind):
    """A small plan of each kernel path, with K/V tensors whose storage holds `extra`
    rows past N (so a token up to N + extra - 1 is still inside memory)."""
    if kind == "decode":
        w, extra = W.random_bsr(81, 9, 40 * 16, 1, 16, 32, 8, partial_lens=False, density=0.4), 16
    elif kind == "tile_fast":      # 64-key tiles inside 64-key blocks: the whole-tile path
        w, extra = W.random_bsr(82, 256, 12 * 64, 64, 64, 16, 4, density=0.5), 64
    elif kind == "tile_generic":   # 48-key blocks: per-key tokens
        w, extra = W.random_bsr(83, 96, 20 * 48, 32, 48, 32, 4, density=0.5), 48
    else:                          # sparse MLA, one token per block
        w, extra = W.sparse_mla(seed=84, num_tokens=4, num_heads=64, cache_rows=2048, topk=128, min_ctx=256,
                                max_ctx=2048), 1
    return w, extra


@pytest.mark.parametrize("kind", ["decode", "tile_fast", "tile_generic", "mla"])
def test_trace_build_masks_out_of_range_tokens(kind):
    # a column entry overwritten in the device tables to point one block past N: the
    # trace build counts the keys it meets there, reads them as masked, and leaves every
    # row that does not use the entry bit-identical to the uncorrupted run
    w, extra = _corrupt_case(kind)
    say(f"[trace] out-of-range tokens, {kind}")
    dev = torch.device("cuda")
    p = plan_for(w, 1, trace=True)
    tab = p.tables()
    cols, tiles = tab["cols"], tab["tiles"]

    def with_room(t):
        full = torch.zeros((t.shape[0] + extra,) + tuple(t.shape[1:]), dtype=t.dtype)
        full[: t.shape[0]] = t
        return full.to(dev)[: t.shape[0]]

    q = w.q.to(dev)
    k = with_room(w.k)
    v = None if w.v_aliases_k else with_room(w.v)
    sc = scales_for(w)
    ws = p.workspace(dev)
    p.upload(ws)
    o_ref, l_ref = p.run(q, k, v, workspace=ws, **sc)
    o_ref, l_ref = o_ref.clone(), l_ref.clone()
    assert int(p.trace_records(ws)[:, 8].sum()) == 0
    # find the column table in the uploaded tables and redirect its entry e
    table = ws[: p.info()["table_bytes"]].cpu().numpy().view(np.int32)
    starts = [i for i in range(len(table) - len(cols) + 1) if np.array_equal(table[i:i + len(cols)], cols)]
    assert len(starts) >= 1
    e = len(cols) // 2
    nb = w.N // (1 if kind == "mla" else w.C)
    off = starts[0] + e
    patch = torch.tensor([nb], dtype=torch.int32)
    ws.view(torch.int32)[off:off + 1].copy_(patch.to(dev))
    torch.cuda.synchronize()
    o, lse = p.run(q, k, v, workspace=ws, **sc)
    rec = p.trace_records(ws)
    bad = int(rec[:, 8].sum())
    assert bad > 0, f"{kind}: no out-of-range token counted"
    assert torch.isfinite(o.float()).all()
    # rows whose tiles do not walk entry e are untouched
    touched = np.zeros(w.M, bool)
    g = w.num_qo_heads // w.num_kv_heads
    for (I, kvh, row0, nrows, cb, ce, part, keys) in tiles:
        if cb <= e < ce:
            for r in range(row0, row0 + nrows):
                tok = I * w.R + r // g
                if tok < w.M:
                    touched[tok] = True
    assert touched.any() and not touched.all()
    keep = torch.from_numpy(~touched).to(dev)
    assert torch.equal(o[keep].view(torch.int16), o_ref[keep].view(torch.int16))
    assert torch.equal(lse[keep], l_ref[keep])
    say(f"[trace] {kind}: {bad} out-of-range key loads masked, {int(touched.sum())} of {w.M} rows affected")
