"""Pins of the indexer oracle (oracle/indexer.py): float32 scores of each query
row over the key positions of its request's paged cache and the exact Top-K with ties to the
lower position (flashinfer.sparse 0.7.4, "SDSA Indexer": indexer_scores,
top_k_from_candidates).

The pins do not re-run the oracle's own formulas: the brute force below forms
each score with Python float arithmetic and rounds it through a 4-byte float
pack, walks the pages position by position, and selects by repeatedly taking
the highest remaining score (lowest position among equals), a different
algorithm from the oracle's sort.  Closed cases fix the tie rule, the short
rows and the paging; planted mistakes in a copy of the oracle must fail at
least one pin."""
import os
import struct
import types

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "indexer.py")


def _f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _brute_force(q, key_cache, block_table, page_size, req_row_ptr, ctx_len, k):
    rows = []
    for r in range(len(req_row_ptr) - 1):
        for row in range(int(req_row_ptr[r]), int(req_row_ptr[r + 1])):
            n = int(ctx_len[row])
            slots, scores = [], []
            for p in range(n):
                slot = int(block_table[r][p // page_size]) * page_size + p % page_size
                acc = 0.0
                for d in range(len(q[row])):
                    acc += float(q[row][d]) * float(key_cache[slot][d])
                slots.append(slot)
                scores.append(_f32(acc))
            left = list(range(n))
            chosen = []
            while left and len(chosen) < k:
                best = left[0]
                for p in left[1:]:
                    if scores[p] > scores[best]:
                        best = p
                chosen.append(best)
                left.remove(best)
            out = [slots[p] for p in sorted(chosen)] + [-1] * (k - len(chosen))
            rows.append(out)
    return np.array(rows, dtype=np.int64)


def _case(seed, num_reqs=3, rows_per_req=(1, 3, 2), dim=8, page=4, max_pages=6, integer=True):
    rng = np.random.default_rng(seed)
    num_slots = num_reqs * max_pages * page
    if integer:
        key_cache = rng.integers(-3, 4, size=(num_slots, dim)).astype(np.float64)
        q = rng.integers(-3, 4, size=(sum(rows_per_req), dim)).astype(np.float64)
    else:
        key_cache = rng.standard_normal((num_slots, dim))
        q = rng.standard_normal((sum(rows_per_req), dim))
    # every request owns max_pages distinct pages, in random order
    perm = rng.permutation(num_reqs * max_pages).reshape(num_reqs, max_pages).astype(np.int32)
    req_row_ptr = np.concatenate([[0], np.cumsum(rows_per_req)]).astype(np.int32)
    ctx = rng.integers(0, max_pages * page + 1, size=req_row_ptr[-1]).astype(np.int32)
    return q, key_cache, perm, page, req_row_ptr, ctx


@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("seed", range(6))
def test_matches_brute_force(seed, integer):
    q, kc, bt, page, rp, ctx = _case(seed, integer=integer)
    for k in (1, 5, 9):
        got = oracle.indexer_topk(q, kc, bt, page, rp, ctx, k)
        ref = _brute_force(q.tolist(), kc.tolist(), bt.tolist(), page, rp.tolist(), ctx.tolist(), k)
        assert np.array_equal(got, ref), (seed, integer, k)


def test_scores_are_dot_products_rounded_to_float32():
    q, kc, bt, page, rp, ctx = _case(7, integer=False)
    s = oracle.indexer_scores(q, kc, bt, page, rp, ctx)
    for r in range(len(rp) - 1):
        for row in range(rp[r], rp[r + 1]):
            for p in range(int(ctx[row])):
                slot = int(bt[r][p // page]) * page + p % page
                acc = sum(float(a) * float(b) for a, b in zip(q[row], kc[slot]))
                assert s[row].dtype == np.float32 and s[row][p] == np.float32(_f32(acc))


def test_equal_scores_keep_the_lowest_positions():
    # every key equal: the K kept keys are positions 0 .. K-1
    kc = np.ones((32, 4))
    bt = np.arange(8, dtype=np.int32)[None, :]
    got = oracle.indexer_topk(np.ones((1, 4)), kc, bt, 4, np.array([0, 1]), np.array([32]), 5)
    assert got.tolist() == [[0, 1, 2, 3, 4]]
    # -0 and +0 are the same score
    assert oracle.topk_positions(np.array([-0.0, 0.0, -1.0], np.float32), 1).tolist() == [0]
    assert oracle.topk_positions(np.array([0.0, -0.0, -1.0], np.float32), 1).tolist() == [0]


def test_increasing_scores_keep_the_last_positions():
    n, k = 40, 7
    kc = np.arange(n, dtype=np.float64)[:, None] * np.ones((1, 2))
    bt = np.arange(10, dtype=np.int32)[None, :]
    got = oracle.indexer_topk(np.ones((1, 2)), kc, bt, 4, np.array([0, 1]), np.array([n]), k)
    assert got.tolist() == [list(range(n - k, n))]


def test_short_and_empty_rows_pad_with_minus_one():
    kc = np.random.default_rng(1).standard_normal((16, 3))
    bt = np.array([[3, 1, 2, 0]], dtype=np.int32)
    got = oracle.indexer_topk(np.ones((3, 3)), kc, bt, 4, np.array([0, 3]), np.array([0, 3, 6]), 6)
    assert got[0].tolist() == [-1] * 6
    assert got[1].tolist() == [12, 13, 14, -1, -1, -1]           # page 3, positions 0..2
    assert got[2].tolist() == [12, 13, 14, 15, 4, 5]             # page 3, then page 1


def test_float32_rounding_decides_ties():
    # two keys whose exact scores differ below float32 resolution tie in float32,
    # so the lower position is kept although its exact score is smaller
    kc = np.array([[1.0], [1.0 + 2.0 ** -30], [0.5], [0.25]])
    bt = np.array([[0]], dtype=np.int32)
    got = oracle.indexer_topk(np.ones((1, 1)), kc, bt, 4, np.array([0, 1]), np.array([4]), 1)
    assert got.tolist() == [[0]]
    # the selection itself compares float32 values, whatever precision it is handed
    assert oracle.topk_positions(np.array([1.0, 1.0 + 2.0 ** -30, 0.5]), 1).tolist() == [0]


def test_paging_follows_the_block_table():
    # the same keys laid out through a permuted table give the same selected key vectors
    rng = np.random.default_rng(3)
    page, pages, dim, n, k = 4, 5, 6, 19, 6
    keys = rng.standard_normal((pages * page, dim))
    q = rng.standard_normal((1, dim))
    ident = oracle.indexer_topk(q, keys, np.arange(pages, dtype=np.int32)[None, :], page, np.array([0, 1]),
                                np.array([n]), k)
    perm = rng.permutation(pages).astype(np.int32)
    paged = np.zeros_like(keys)
    for p in range(pages):
        paged[perm[p] * page:(perm[p] + 1) * page] = keys[p * page:(p + 1) * page]
    got = oracle.indexer_topk(q, paged, perm[None, :], page, np.array([0, 1]), np.array([n]), k)
    assert np.array_equal(paged[got[0]], keys[ident[0]])


MUTATIONS = {
    "ties_to_higher": ("order = np.lexsort((np.arange(n), -s))", "order = np.lexsort((-np.arange(n), -s))"),
    "lowest_scores": ("order = np.lexsort((np.arange(n), -s))", "order = np.lexsort((np.arange(n), s))"),
    "page_offset_dropped": ("block_table[req, p // page_size].astype(np.int64) * page_size + p % page_size",
                            "block_table[req, p // page_size].astype(np.int64) * page_size"),
    "page_index_by_position": ("block_table[req, p // page_size]", "block_table[req, p % block_table.shape[1]]"),
    "no_float32_rounding": ("s = np.asarray(scores, dtype=np.float32).astype(np.float64)",
                            "s = np.asarray(scores, dtype=np.float64)"),
    "scores_in_float64": ("out[row] = (k64[slots] @ q64[row]).astype(np.float32)", "out[row] = k64[slots] @ q64[row]"),
    "short_rows_truncated": ("    if n <= k:\n        return np.arange(n, dtype=np.int64)",
                             "    if n <= k:\n        return np.arange(max(n - 1, 0), dtype=np.int64)"),
    "unsorted_output": ("return np.sort(order[:k])", "return order[:k]"),
}


def _mutant(name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"indexer_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


PINS = [lambda: test_matches_brute_force(0, True), lambda: test_matches_brute_force(1, False),
        test_scores_are_dot_products_rounded_to_float32, test_equal_scores_keep_the_lowest_positions,
        test_increasing_scores_keep_the_last_positions, test_short_and_empty_rows_pad_with_minus_one,
        test_float32_rounding_decides_ties, test_paging_follows_the_block_table]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod = _mutant(name)
    for f in ("key_slots", "indexer_scores", "topk_positions", "indexer_topk"):
        monkeypatch.setattr(oracle, f, getattr(mod, f))
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught {name}"
