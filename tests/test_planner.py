"""Host planner: bit-exact against a Python model of its documented rule,
plus coverage invariants (every unmasked (row, key-block) pair is visited by
exactly one tile).  Runs on the CPU: planning never touches the GPU when the
CU count is given."""
import math

import numpy as np
import pytest
import torch

from paged_attention_bsr_amd import Plan
from paged_attention_bsr_amd import workloads as W

AUTO_TILES_PER_CU = 4
AUTO_MIN_SPLIT_KEYS = 256
MAX_SPLITS = 64
DECODE_WG_PER_CU = 1
BALANCED_MIN_KEYS = 256


def _cdiv(a, b):
    return -(-a // b)


def model_plan(w, kv_splits, num_cus, tile_rows, head_lists=None):
    """Python model of the planner's partition rule (steps 1-6 of planner.cpp,
    and the balanced partition of the decode kernel with kv_splits = 0).
    ``head_lists``: None (the BSR rows of ``w``, shared by every kv head) or,
    for a per-head structure, head_lists[h][I] = the blocks of kv head h.
    Returns (tiles, merges, cols, wg_ptr)."""
    M, N, R, C = w.M, w.N, w.R, w.C
    g = w.num_qo_heads // w.num_kv_heads
    MB = _cdiv(M, R)
    off = N - M
    blen = (lambda J: int(w.kv_block_lens[J])) if w.kv_block_lens is not None else (lambda J: C)
    per_head = head_lists is not None
    if not per_head:
        head_lists = [[w.indices[w.indptr[I]:w.indptr[I + 1]] for I in range(MB)]]
    HS = len(head_lists)
    cols, bptr = [], [0]
    for hs in range(HS):
        for I in range(MB):
            row = sorted(int(x) for x in head_lists[hs][I])
            last = min(M, (I + 1) * R) - 1
            for J in row:
                if w.causal and J * C > last + off:
                    break
                cols.append(J)
            bptr.append(len(cols))
    rts = []
    for u in range(HS * MB):
        I, hs = u % MB, u // MB
        U = min(R, M - I * R) * g
        for r0 in range(0, U, tile_rows):
            nr = min(tile_rows, U - r0)
            n = bptr[u + 1] - bptr[u]
            if w.causal:
                lim = I * R + (r0 + nr - 1) // g + off
                k = 0
                while k < n and cols[bptr[u] + k] * C <= lim:
                    k += 1
                n = k
            keys = sum(blen(cols[bptr[u] + k]) for k in range(n))
            rts.append((I, r0, nr, bptr[u], n, keys, keys * _cdiv(nr, 32), hs))
    decode = model_kernel(w, num_cus)[0] == 2
    G = min(8, w.num_kv_heads & -w.num_kv_heads) if decode and not per_head else 1
    NG = w.num_kv_heads // G
    heads_of = (lambda rt: [rt[7]]) if per_head else (lambda rt: range(NG))
    st = {"part": 0, "tiles": [], "merges": [], "groups": []}

    def emit_unit(rt, gi, pref, b, wgs):
        """Pieces b[j]..b[j+1] of head group gi; head i's partial of piece j at base + (i*s + j)*psize."""
        (I, r0, nr, cb, n, keys, work, _) = rt
        s = len(b) - 1
        psize = _cdiv(nr * (w.head_dim_vo + 1), 64) * 64
        base = st["part"]
        for j in range(s):
            kj = pref[b[j + 1]] - pref[b[j]]
            grp = [[I, gi * G + i, r0, nr, cb + b[j], cb + b[j + 1],
                    base + (i * s + j) * psize if s > 1 else -1, kj] for i in range(G)]
            st["groups"].append((grp, kj * _cdiv(nr, 32), wgs[j] if wgs else 0))
        if s > 1:
            st["part"] += G * s * psize
            for i in range(G):
                st["merges"].append([I, gi * G + i, r0, nr, base + i * s * psize, s, psize, 0])

    def prefix(rt):
        pref = [0]
        for k in range(rt[4]):
            pref.append(pref[-1] + blen(cols[rt[3] + k]))
        return pref

    if kv_splits == 0 and decode:
        K = sum(rt[5] * len(heads_of(rt)) for rt in rts)
        Wn = max(1, min(DECODE_WG_PER_CU * num_cus, K // BALANCED_MIN_KEYS))
        wg_of = (lambda X: min(Wn - 1, X * Wn // K)) if K > 0 else (lambda X: 0)
        X = 0
        for rt in rts:
            pref = prefix(rt)
            n = rt[4]
            for gi in heads_of(rt):
                b, wgs = [0], [wg_of(X)]
                for k in range(1, n):
                    if wg_of(X + pref[k]) != wgs[-1]:
                        b.append(k)
                        wgs.append(wg_of(X + pref[k]))
                b.append(n)
                emit_unit(rt, gi, pref, b, wgs)
                X += rt[5]
        order = st["groups"]
        count = [0] * Wn
        for (_, _, wg) in order:
            count[wg] += G
        wg_ptr = np.concatenate([[0], np.cumsum(count)]).astype(np.int32)
    else:
        total = sum(rt[6] for rt in rts) * (1 if per_head else w.num_kv_heads)
        chunk = max(1, _cdiv(total, AUTO_TILES_PER_CU * num_cus))
        for rt in rts:
            (I, r0, nr, cb, n, keys, work, _) = rt
            if kv_splits == 1:
                s = 1
            elif kv_splits > 1:
                s = min(kv_splits, n)
            else:
                cap = min(n, MAX_SPLITS, max(1, keys // AUTO_MIN_SPLIT_KEYS))
                s = min(_cdiv(work, chunk), cap)
            s = max(1, s)
            pref = prefix(rt)
            b = [0] * (s + 1)
            b[s] = n
            for j in range(1, s):
                p = 0
                while p < n and pref[p] * s < j * keys:
                    p += 1
                p = max(p, b[j - 1] + 1)
                p = min(p, n - (s - j))
                b[j] = p
            for gi in heads_of(rt):
                emit_unit(rt, gi, pref, b, None)
        order = sorted(st["groups"], key=lambda gr: -gr[1])  # stable
        wg_ptr = (np.arange(len(order) + 1) * G).astype(np.int32)
    tiles = [t for (grp, _, _) in order for t in grp]
    return (np.array(tiles, np.int32).reshape(-1, 8), np.array(st["merges"], np.int32).reshape(-1, 8),
            np.array(cols, np.int32), wg_ptr)


def _plan(w, kv_splits, num_cus=256):
    return Plan(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                head_dim_vo=w.head_dim_vo, causal=w.causal, kv_block_lens=w.kv_block_lens,
                q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, o_dtype=w.o_dtype, kv_splits=kv_splits,
                num_cus=num_cus)


def _small_cases():
    cases = []
    for seed in range(10):
        rng = np.random.default_rng(seed)
        R, C = int(rng.choice([1, 2, 3, 16, 64])), int(rng.choice([1, 3, 16, 64]))
        g = int(rng.choice([1, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        M = int(rng.integers(1, 300))
        NB = int(rng.integers(1, 40))
        cases.append(W.random_bsr(seed, M, NB * C, R, C, Hkv * g, Hkv, causal=bool(seed % 2),
                                  partial_lens=seed % 3 == 0, density=0.4, values=False))
    return cases


@pytest.mark.parametrize("kv_splits", [1, 2, 7, 0])
@pytest.mark.parametrize("case", range(10))
def test_planner_matches_model_small(case, kv_splits):
    w = _small_cases()[case]
    p = _plan(w, kv_splits, num_cus=8)
    t = p.tables()
    tiles, merges, cols, wg_ptr = model_plan(w, kv_splits, 8, p.info()["tile_rows"])
    np.testing.assert_array_equal(t["cols"], cols)
    np.testing.assert_array_equal(t["tiles"], tiles)
    np.testing.assert_array_equal(t["merges"], merges)
    np.testing.assert_array_equal(t["wg_ptr"], wg_ptr)


@pytest.mark.parametrize("name", ["worked_example", "paged_decode", "bsr_prefill", "window_prefill", "sparse_mla"])
@pytest.mark.parametrize("kv_splits", [1, 0])
def test_planner_matches_model_full_workloads(name, kv_splits):
    w = W.by_name(name, values=False)
    p = _plan(w, kv_splits)
    t = p.tables()
    tiles, merges, cols, wg_ptr = model_plan(w, kv_splits, 256, p.info()["tile_rows"])
    np.testing.assert_array_equal(t["cols"], cols)
    np.testing.assert_array_equal(t["tiles"], tiles)
    np.testing.assert_array_equal(t["merges"], merges)
    np.testing.assert_array_equal(t["wg_ptr"], wg_ptr)


def _coverage(w, tables, g):
    """Count how often each (query row, qo head, key block) is visited by the tiles."""
    cols = tables["cols"]
    seen = {}
    for (I, h, r0, nr, cb, ce, part, keys) in tables["tiles"]:
        for r in range(r0, r0 + nr):
            tok, head = I * w.R + r // g, h * g + r % g
            for p in range(cb, ce):
                key = (tok, head, int(cols[p]))
                seen[key] = seen.get(key, 0) + 1
    return seen


@pytest.mark.parametrize("case", range(6))
@pytest.mark.parametrize("kv_splits", [1, 3, 0])
def test_every_unmasked_pair_is_covered_exactly_once(case, kv_splits):
    w = _small_cases()[case]
    p = _plan(w, kv_splits, num_cus=4)
    t = p.tables()
    g = w.num_qo_heads // w.num_kv_heads
    seen = _coverage(w, t, g)
    assert all(v == 1 for v in seen.values())
    # every (row, head, block) whose block has an unmasked key appears
    lens = w.kv_block_lens
    for i in range(w.M):
        I = i // w.R
        for J in w.indices[w.indptr[I]:w.indptr[I + 1]]:
            first = J * w.C
            if w.causal and first > i + (w.N - w.M):
                continue
            for head in range(w.num_qo_heads):
                assert seen.get((i, head, int(J))) == 1
    # merges reference exactly the split tiles
    tiles = t["tiles"]
    split = tiles[tiles[:, 6] >= 0]
    assert sum(int(m[5]) for m in t["merges"]) == len(split)
    assert set(split[:, 6].tolist()) == {int(m[4]) + j * int(m[6]) for m in t["merges"] for j in range(m[5])}


def _decode_cases():
    """R = 1, C >= 16 problems (decode kernel) with short and empty rows."""
    cases = []
    for seed in range(8):
        rng = np.random.default_rng(100 + seed)
        C = int(rng.choice([16, 32, 64]))
        g = int(rng.choice([1, 4, 16]))
        Hkv = int(rng.choice([1, 2, 3]))
        M = int(rng.integers(1, 40))
        NB = int(rng.integers(1, 60))
        cases.append(W.random_bsr(200 + seed, M, NB * C, 1, C, Hkv * g, Hkv, causal=bool(seed % 2),
                                  partial_lens=seed % 3 != 2, density=float(rng.choice([0.05, 0.3, 0.9])),
                                  values=False))
    return cases


@pytest.mark.parametrize("num_cus", [1, 3, 8, 256])
@pytest.mark.parametrize("case", range(8))
def test_balanced_partition_matches_model(case, num_cus):
    w = _decode_cases()[case]
    p = _plan(w, 0, num_cus=num_cus)
    assert p.info()["kernel"] == 2
    t = p.tables()
    tiles, merges, cols, wg_ptr = model_plan(w, 0, num_cus, 16)
    np.testing.assert_array_equal(t["tiles"], tiles)
    np.testing.assert_array_equal(t["merges"], merges)
    np.testing.assert_array_equal(t["wg_ptr"], wg_ptr)


@pytest.mark.parametrize("case", range(8))
def test_balanced_partition_shares_and_coverage(case):
    """Every workgroup gets its share of all keys to within one block, each
    workgroup's tiles are one contiguous run of the (I, h) key sequence, and
    every unmasked pair is visited exactly once."""
    w = _decode_cases()[case]
    num_cus = 3
    p = _plan(w, 0, num_cus=num_cus)
    t, inf = p.tables(), p.info()
    tiles, wg_ptr = t["tiles"], t["wg_ptr"]
    G = inf["heads_per_wg"]
    assert G == min(8, w.num_kv_heads & -w.num_kv_heads)
    K = int(tiles[:, 7].sum()) // G          # keys of the (I, head group) sequence
    Wn = inf["num_workgroups"]
    assert Wn == max(1, min(DECODE_WG_PER_CU * num_cus, K // BALANCED_MIN_KEYS))
    assert wg_ptr[0] == 0 and wg_ptr[-1] == len(tiles) and np.all(np.diff(wg_ptr) >= 0)
    assert np.all(wg_ptr % G == 0)
    # a group's G tiles share row block and blocks, heads gi*G .. gi*G+G-1
    for q in range(0, len(tiles), G):
        grp = tiles[q:q + G]
        assert np.all(grp[:, [0, 2, 3, 4, 5, 7]] == grp[0, [0, 2, 3, 4, 5, 7]])
        assert list(grp[:, 1]) == list(range(grp[0, 1], grp[0, 1] + G)) and grp[0, 1] % G == 0
    share = [int(tiles[wg_ptr[i]:wg_ptr[i + 1], 7].sum()) // G for i in range(Wn)]
    assert sum(share) == K
    if K > 0:
        assert max(share) <= -(-K // Wn) + w.C and min(share) >= K // Wn - w.C
    # tiles follow the (I, head group) sequence: (row block, group, first block, head) never decreases
    keyseq = [(int(r[0]), int(r[1]) // G, int(r[4]), int(r[1]) % G) for r in tiles]
    assert keyseq == sorted(keyseq)
    g = w.num_qo_heads // w.num_kv_heads
    assert all(v == 1 for v in _coverage(w, t, g).values())
    # every (token, kv head) unit has exactly one unsplit tile or one merge
    split = tiles[tiles[:, 6] >= 0]
    assert sum(int(m[5]) for m in t["merges"]) == len(split)
    units = {(int(r[0]), int(r[1])) for r in tiles}
    assert len(units) == w.M * w.num_kv_heads


def test_plan_is_deterministic_and_order_free():
    w = W.random_bsr(3, 200, 64 * 16, 16, 16, 8, 2, causal=True, values=False)
    a = _plan(w, 0, num_cus=16).tables()
    b = _plan(w, 0, num_cus=16).tables()
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    rng = np.random.default_rng(0)
    perm = w.indices.copy()
    for I in range(len(w.indptr) - 1):
        seg = perm[w.indptr[I]:w.indptr[I + 1]]
        perm[w.indptr[I]:w.indptr[I + 1]] = seg[rng.permutation(seg.size)]
    w.indices = perm
    c = _plan(w, 0, num_cus=16).tables()
    for k in a:
        np.testing.assert_array_equal(a[k], c[k])


def test_workspace_layout():
    w = W.paged_decode(values=False)
    p = _plan(w, 0)
    inf = p.info()
    assert inf["workspace_bytes"] == inf["table_bytes"] + inf["partial_bytes"]
    assert inf["workspace_bytes"] % 256 == 0 and inf["table_bytes"] % 256 == 0
    assert p.workspace_size == inf["workspace_bytes"]
    assert inf["num_merges"] > 0 and inf["max_splits"] > 1


TILE_SMALL_GRID_PER_CU = 8


def model_kernel(w, num_cus):
    """Python model of the planner's kernel / row-tile choice."""
    g = w.num_qo_heads // w.num_kv_heads
    if w.kv_dtype == torch.float8_e4m3fn and w.head_dim != 128:
        return 1, 64
    if w.R == 1 and g <= 16 and w.C >= 16:
        return 2, 16
    MB = _cdiv(w.M, w.R)
    umax = min(w.R, max(w.M, 1)) * g
    if umax <= 32:
        return 0, 32
    if umax <= 128:
        return 0, 128
    n256 = w.num_kv_heads * sum(_cdiv(min(w.R, w.M - I * w.R) * g, 256) for I in range(MB))
    return 0, (128 if n256 < TILE_SMALL_GRID_PER_CU * num_cus else 256)


@pytest.mark.parametrize("num_cus", [4, 64, 256])
def test_kernel_and_tile_rows_rule(num_cus):
    ws = [W.by_name(n, values=False) for n in W.WORKLOAD_NAMES] + _small_cases()
    ws.append(W.random_bsr(11, 4096, 4096, 128, 128, 32, 4, causal=True, density=0.2, values=False))
    seen = set()
    for w in ws:
        inf = _plan(w, 1, num_cus=num_cus).info()
        want = model_kernel(w, num_cus)
        assert (inf["kernel"], inf["tile_rows"]) == want
        seen.add(want)
    # the rule's branches are all exercised at some CU count
    assert {(0, 32), (0, 128), (2, 16), (1, 64)} <= seen


def test_small_grids_use_128_row_tiles():
    w = W.by_name("bsr_prefill", values=False)   # 1024 tiles of 256 rows: 4 per CU at 256 CUs
    assert _plan(w, 1, num_cus=256).info()["tile_rows"] == 128
    assert _plan(w, 1, num_cus=64).info()["tile_rows"] == 256
    w = W.by_name("window_prefill", values=False)  # 8192 tiles of 256 rows
    assert _plan(w, 1, num_cus=256).info()["tile_rows"] == 256


# ---------------------------------------------------------------- per-head structure
def _per_head_case(seed, decode):
    """A random problem with one block mask per kv head (tile or decode kernel shapes)."""
    rng = np.random.default_rng(900 + seed)
    if decode:
        R, C = 1, int(rng.choice([16, 32]))
        g = int(rng.choice([1, 4, 8]))
    else:
        R, C = int(rng.choice([2, 16, 64])), int(rng.choice([1, 16, 64]))
        g = int(rng.choice([1, 4]))
    Hkv = int(rng.choice([1, 2, 4]))
    M = int(rng.integers(1, 200 if not decode else 30))
    NB = int(rng.integers(1, 30))
    w = W.random_bsr(seed, M, NB * C, R, C, Hkv * g, Hkv, causal=bool(seed % 2), partial_lens=seed % 3 == 0,
                     density=0.3, values=False)
    bm = rng.random((Hkv, w.MB, w.NB)) < float(rng.choice([0.1, 0.4, 0.8]))
    return w, bm


def _plan_heads(w, kv_splits, num_cus, **kw):
    return Plan(None, None, w.M, w.N, w.R, w.C, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                head_dim_vo=w.head_dim_vo, causal=w.causal, kv_block_lens=w.kv_block_lens,
                q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, o_dtype=w.o_dtype, kv_splits=kv_splits,
                num_cus=num_cus, **kw)


def _lists(bm):
    return [[np.nonzero(bm[h, I])[0] for I in range(bm.shape[1])] for h in range(bm.shape[0])]


@pytest.mark.parametrize("kv_splits", [1, 2, 0])
@pytest.mark.parametrize("case", range(8))
def test_per_head_planner_matches_model(case, kv_splits):
    w, bm = _per_head_case(case, decode=case % 2 == 1)
    p = _plan_heads(w, kv_splits, 8, block_mask=bm)
    t = p.tables()
    tiles, merges, cols, wg_ptr = model_plan(w, kv_splits, 8, p.info()["tile_rows"], _lists(bm))
    np.testing.assert_array_equal(t["cols"], cols)
    np.testing.assert_array_equal(t["tiles"], tiles)
    np.testing.assert_array_equal(t["merges"], merges)
    np.testing.assert_array_equal(t["wg_ptr"], wg_ptr)
    assert p.info()["heads_per_wg"] == 1


@pytest.mark.parametrize("case", range(6))
def test_per_head_forms_agree(case):
    """block_mask per kv head, the same mask per qo head, and q2k selections of the same
    blocks (shuffled, padded past q2k_num) give identical tables."""
    w, bm = _per_head_case(case, decode=case % 2 == 1)
    g = w.num_qo_heads // w.num_kv_heads
    ref = _plan_heads(w, 0, 16, block_mask=bm).tables()
    by_qo = _plan_heads(w, 0, 16, block_mask=np.repeat(bm, g, axis=0)).tables()
    rng = np.random.default_rng(case)
    topk = max(1, int(bm.sum(axis=2).max()) + 2)
    sel = np.full(bm.shape[:2] + (topk,), -5, np.int32)      # padding past q2k_num is never read
    num = bm.sum(axis=2).astype(np.int32)
    for h in range(bm.shape[0]):
        for I in range(bm.shape[1]):
            js = rng.permutation(np.nonzero(bm[h, I])[0])
            sel[h, I, :js.size] = js
    by_q2k = _plan_heads(w, 0, 16, q2k_indices=np.repeat(sel, g, axis=0), q2k_num=np.repeat(num, g, axis=0)).tables()
    for k in ref:
        np.testing.assert_array_equal(ref[k], by_qo[k])
        np.testing.assert_array_equal(ref[k], by_q2k[k])


@pytest.mark.parametrize("case", range(6))
@pytest.mark.parametrize("kv_splits", [1, 3, 0])
def test_per_head_coverage_exactly_once(case, kv_splits):
    w, bm = _per_head_case(case, decode=case % 3 == 0)
    p = _plan_heads(w, kv_splits, 4, block_mask=bm)
    t = p.tables()
    g = w.num_qo_heads // w.num_kv_heads
    seen = _coverage(w, t, g)
    assert all(v == 1 for v in seen.values())
    want = set()
    for i in range(w.M):
        for h in range(w.num_kv_heads):
            for J in np.nonzero(bm[h, i // w.R])[0]:
                if w.causal and J * w.C > i + (w.N - w.M):
                    continue
                want.update((i, h * g + j, int(J)) for j in range(g))
    assert want <= set(seen)
    # a tile visits only blocks of its own head's structure (rows past their causal limit are masked
    # inside the kernel)
    assert all(bm[hq // g, int(i) // w.R, J] for (i, hq, J) in seen)


def test_per_head_structure_errors():
    w, bm = _per_head_case(0, decode=False)
    g = w.num_qo_heads // w.num_kv_heads
    with pytest.raises(RuntimeError, match="mutually exclusive"):
        _plan_heads(w, 1, 8, block_mask=bm, q2k_indices=np.zeros((w.num_kv_heads, w.MB, 1), np.int32))
    with pytest.raises(RuntimeError, match="struct_heads"):
        _plan_heads(w, 1, 8, block_mask=np.concatenate([bm, bm[:1]]))
    sel = np.zeros((w.num_kv_heads, w.MB, 2), np.int32)
    with pytest.raises(RuntimeError, match="duplicate"):
        _plan_heads(w, 1, 8, q2k_indices=sel)
    with pytest.raises(RuntimeError, match="q2k_num"):
        _plan_heads(w, 1, 8, q2k_indices=sel, q2k_num=np.full((w.num_kv_heads, w.MB), 3, np.int32))
    sel[..., 1] = w.NB
    with pytest.raises(RuntimeError, match=r"\[0, NB\)"):
        _plan_heads(w, 1, 8, q2k_indices=sel)
    if g > 1:
        bq = np.repeat(bm, g, axis=0)
        bq[1, 0] = ~bq[1, 0]
        with pytest.raises(RuntimeError, match="same key blocks"):
            _plan_heads(w, 1, 8, block_mask=bq)



def test_fp8_kv_head_dim_128_kernel_choice():
    """fp8 e4m3 K/V at head_dim 128: decode shapes (R = 1, C >= 16) run the decode kernel,
    every other shape -- prefill blocks, C < 16, element masks -- the tile kernel."""
    w = W.by_name("paged_decode_fp8", values=False)
    assert _plan(w, 0).info()["kernel"] == 2
    w2 = W.random_bsr(5, 64, 64 * 4, 16, 16, 8, 2, values=False)
    w2.kv_dtype = torch.float8_e4m3fn
    assert _plan(w2, 1).info()["kernel"] == 0
    w3 = W.random_bsr(7, 9, 8 * 4, 1, 4, 8, 2, values=False)   # R = 1 but C < 16
    w3.kv_dtype = torch.float8_e4m3fn
    assert _plan(w3, 1).info()["kernel"] == 0
    # fp8 queries have no kernel
    w4 = W.random_bsr(8, 64, 64 * 4, 16, 16, 8, 2, values=False)
    w4.kv_dtype = w4.q_dtype = w4.o_dtype = torch.float8_e4m3fn
    with pytest.raises(RuntimeError, match="q/o must both be fp16 or both bf16"):
        _plan(w4, 1)


def test_run_scales_rejected_for_the_mla_shape():
    """Per-head run scales apply to head_dim 128 plans; the sparse-MLA plan (one kv head,
    per-tensor descales) refuses them before touching any pointer."""
    import ctypes
    from paged_attention_bsr_amd import _lib as L
    w = W.sparse_mla(seed=9, num_tokens=4, num_heads=16, cache_rows=256, topk=32, min_ctx=64, max_ctx=256,
                     values=False)
    p = _plan(w, 1)
    lib = L.lib()
    if not hasattr(lib, "bsa_run_ex"):
        pytest.skip("host-only build of the planner (no device entry points)")
    st = lib.bsa_run_ex(p._handle, L.BSA_PHASE_ALL, None, None, None, None, None, 16, None, None, None, 0, None)
    assert st == L.BSA_ERR_UNSUPPORTED
    assert b"per-head scales" in lib.bsa_last_error()
