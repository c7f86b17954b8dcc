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


def _cdiv(a, b):
    return -(-a // b)


def model_plan(w, kv_splits, num_cus, tile_rows):
    """Python model of the planner's partition rule (steps 1-6 of planner.cpp)."""
    M, N, R, C = w.M, w.N, w.R, w.C
    g = w.num_qo_heads // w.num_kv_heads
    MB = _cdiv(M, R)
    off = N - M
    blen = (lambda J: int(w.kv_block_lens[J])) if w.kv_block_lens is not None else (lambda J: C)
    cols, bptr = [], [0]
    for I in range(MB):
        row = sorted(int(x) for x in w.indices[w.indptr[I]:w.indptr[I + 1]])
        last = min(M, (I + 1) * R) - 1
        for J in row:
            if w.causal and J * C > last + off:
                break
            cols.append(J)
        bptr.append(len(cols))
    rts = []
    for I in range(MB):
        U = min(R, M - I * R) * g
        for r0 in range(0, U, tile_rows):
            nr = min(tile_rows, U - r0)
            n = bptr[I + 1] - bptr[I]
            if w.causal:
                lim = I * R + (r0 + nr - 1) // g + off
                k = 0
                while k < n and cols[bptr[I] + k] * C <= lim:
                    k += 1
                n = k
            keys = sum(blen(cols[bptr[I] + k]) for k in range(n))
            rts.append((I, r0, nr, bptr[I], n, keys, keys * _cdiv(nr, 32)))
    total = sum(rt[6] for rt in rts) * w.num_kv_heads
    chunk = max(1, _cdiv(total, AUTO_TILES_PER_CU * num_cus))
    tiles, merges, part = [], [], 0
    dv = w.head_dim_vo
    for (I, r0, nr, cb, n, keys, work) in rts:
        if kv_splits == 1:
            s = 1
        elif kv_splits > 1:
            s = min(kv_splits, n)
        else:
            cap = min(n, MAX_SPLITS, max(1, keys // AUTO_MIN_SPLIT_KEYS))
            s = min(_cdiv(work, chunk), cap)
        s = max(1, s)
        pref = [0]
        for k in range(n):
            pref.append(pref[-1] + blen(cols[cb + k]))
        b = [0] * (s + 1)
        b[s] = n
        for j in range(1, s):
            p = 0
            while p < n and pref[p] * s < j * keys:
                p += 1
            p = max(p, b[j - 1] + 1)
            p = min(p, n - (s - j))
            b[j] = p
        psize = _cdiv(nr * (dv + 1), 64) * 64
        for h in range(w.num_kv_heads):
            first = part
            for j in range(s):
                kj = pref[b[j + 1]] - pref[b[j]]
                tiles.append(([I, h, r0, nr, cb + b[j], cb + b[j + 1], part if s > 1 else -1, kj],
                              kj * _cdiv(nr, 32)))
                if s > 1:
                    part += psize
            if s > 1:
                merges.append([I, h, r0, nr, first, s, psize, 0])
    order = sorted(range(len(tiles)), key=lambda t: -tiles[t][1])  # stable
    return (np.array([tiles[t][0] for t in order], np.int32).reshape(-1, 8),
            np.array(merges, np.int32).reshape(-1, 8), np.array(cols, np.int32))


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
    tiles, merges, cols = model_plan(w, kv_splits, 8, p.info()["tile_rows"])
    np.testing.assert_array_equal(t["cols"], cols)
    np.testing.assert_array_equal(t["tiles"], tiles)
    np.testing.assert_array_equal(t["merges"], merges)


@pytest.mark.parametrize("name", ["worked_example", "paged_decode", "bsr_prefill", "window_prefill", "sparse_mla"])
@pytest.mark.parametrize("kv_splits", [1, 0])
def test_planner_matches_model_full_workloads(name, kv_splits):
    w = W.by_name(name, values=False)
    p = _plan(w, kv_splits)
    t = p.tables()
    tiles, merges, cols = model_plan(w, kv_splits, 256, p.info()["tile_rows"])
    np.testing.assert_array_equal(t["cols"], cols)
    np.testing.assert_array_equal(t["tiles"], tiles)
    np.testing.assert_array_equal(t["merges"], merges)


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
    if w.kv_dtype == torch.float8_e4m3fn:
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
