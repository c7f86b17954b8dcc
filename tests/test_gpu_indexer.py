"""GPU parity of the sparse-attention indexer (bsa_indexer_topk through the C ABI)
against the oracle (oracle/indexer.py).

With integer-valued inputs every float32 dot product is exact in any summation
order, so the kernels' scores and index lists must equal the oracle's bit for
bit, ties included.  With normal inputs the scores must agree within the
float32 accumulation bound, and the kept sets may differ only in keys whose
scores lie within that bound of the row's K-th score."""
import numpy as np
import pytest
import torch

import oracle
from paged_attention_bsr_amd import indexer_topk
from paged_attention_bsr_amd import workloads as W
from tests.parity_util import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def _run(w, **kw):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out, scores = indexer_topk(w["q"].to(DEV), w["key_cache"].to(DEV), t(w["block_table"]), t(w["req_row_ptr"]),
                               t(w["ctx_len"]), t(w["req_kv_len"]), w["topk"], w["page_size"],
                               max_ctx=w["max_ctx"], **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64), scores.cpu().numpy()


def _oracle_inputs(w):
    return (w["q"].float().numpy(), w["key_cache"].float().numpy(), w["block_table"], w["page_size"],
            w["req_row_ptr"], np.minimum(w["ctx_len"], np.repeat(w["req_kv_len"], np.diff(w["req_row_ptr"]))))


SMALL = {
    # (seed, rows, cache rows, requests, page, head_dim, topk, min_ctx, max_ctx, dtype)
    "one_request_tiles": (1, 40, 3000, 1, 64, 128, 300, 0, 3000, torch.bfloat16),
    "three_requests_odd_page": (2, 40, 3000, 3, 12, 128, 50, 0, 1100, torch.bfloat16),
    "rows_over_two_groups": (3, 37, 2048, 1, 16, 64, 100, 200, 2048, torch.float16),
    "head_dim_256": (4, 20, 1500, 2, 32, 256, 64, 10, 800, torch.bfloat16),
    "many_requests_decode": (5, 64, 8192, 64, 16, 128, 32, 0, 128, torch.float16),
    "topk_one": (6, 18, 1024, 2, 8, 128, 1, 0, 512, torch.bfloat16),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_exact_on_integer_inputs(name):
    seed, rows, cache, reqs, page, dim, k, lo, hi, dt = SMALL[name]
    w = W.indexer(seed=seed, num_tokens=rows, cache_rows=cache, num_reqs=reqs, page_size=page, head_dim=dim,
                  topk=k, min_ctx=lo, max_ctx=hi, dtype=dt, integer=True)
    say(f"[indexer] exact {name}")
    out, scores = _run(w)
    args = _oracle_inputs(w)
    ref = oracle.indexer_topk(*args, k)
    ref_s = oracle.indexer_scores(*args)
    for row in range(rows):
        n = len(ref_s[row])
        assert np.array_equal(scores[row, :n], ref_s[row]), f"{name}: scores of row {row} differ"
    bad = np.nonzero((out != ref).any(axis=1))[0]
    assert bad.size == 0, f"{name}: {bad.size} rows differ; row {bad[0]}: {out[bad[0]][:12]} vs {ref[bad[0]][:12]}"


def _check_within_bound(w, out, scores, rows):
    """Scores within the float32 accumulation bound; kept sets equal except near the K-th score."""
    q, kc, bt, page, rp, ctx = _oracle_inputs(w)
    k = w["topk"]
    q64, k64 = q.astype(np.float64), kc.astype(np.float64)
    req_of = np.repeat(np.arange(len(rp) - 1), np.diff(rp))
    for row in rows:
        r, n = int(req_of[row]), int(ctx[row])
        slots = oracle.key_slots(bt, page, r, n)
        exact = k64[slots] @ q64[row]
        bound = (q.shape[1] + 2) * 2.0 ** -24 * (np.abs(k64[slots]) @ np.abs(q64[row])) + 1e-30
        assert np.all(np.abs(scores[row, :n] - exact) <= bound), f"row {row}: score outside the float32 bound"
        if n <= k:
            assert np.array_equal(out[row, :n], slots) and np.all(out[row, n:] == -1)
            continue
        kth = np.sort(exact)[::-1][k - 1]
        kept = set(out[row].tolist())
        assert -1 not in kept and len(kept) == k, f"row {row}: output is not K distinct slots"
        pos_of = {int(s): i for i, s in enumerate(slots)}
        kept_pos = np.array(sorted(pos_of[s] for s in kept))
        assert np.array_equal(np.array([pos_of[s] for s in out[row]]), kept_pos), f"row {row}: not in position order"
        must = set(np.nonzero(exact > kth + 2 * bound)[0].tolist())
        never = set(np.nonzero(exact < kth - 2 * bound)[0].tolist())
        assert must <= set(kept_pos.tolist()), f"row {row}: a key clearly above the K-th score was dropped"
        assert not (never & set(kept_pos.tolist())), f"row {row}: a key clearly below the K-th score was kept"


def test_within_bound_on_normal_inputs():
    w = W.indexer(seed=11, num_tokens=48, cache_rows=6000, num_reqs=2, page_size=32, head_dim=128, topk=256,
                  min_ctx=100, max_ctx=3000)
    say("[indexer] normal inputs, 48 rows")
    out, scores = _run(w)
    _check_within_bound(w, out, scores, range(48))


def test_full_size_sampled_rows():
    # the sparse-MLA pipeline's indexer: 128 rows, 65536 keys of head_dim 128, Top-2048
    w = W.indexer()
    say("[indexer] full size: 128 rows x up to 65536 keys, top 2048")
    out, scores = _run(w)
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 127] + rng.choice(128, 10, replace=False).tolist()))
    _check_within_bound(w, out, scores, rows)


def test_full_size_exact_on_integer_inputs():
    w = W.indexer(integer=True)
    say("[indexer] full size, integer inputs")
    out, scores = _run(w)
    args = _oracle_inputs(w)
    rows = [0, 5, 64, 127]
    sub_ptr = np.array([0, len(rows)], np.int32)
    # the oracle on the sampled rows only (one request)
    ref = oracle.indexer_topk(args[0][rows], args[1], args[2], args[3], sub_ptr, args[5][rows], w["topk"])
    assert np.array_equal(out[rows], ref)


def test_equal_scores_keep_the_lowest_positions():
    w = W.indexer(seed=2, num_tokens=4, cache_rows=4096, num_reqs=1, page_size=16, head_dim=64, topk=100,
                  min_ctx=1000, max_ctx=4096, integer=True)
    w["key_cache"] = torch.ones_like(w["key_cache"])
    out, _ = _run(w)
    for row in range(4):
        slots = oracle.key_slots(w["block_table"], 16, 0, 100)
        assert np.array_equal(out[row], slots)


def test_invalid_pages_score_zero_and_are_written_as_minus_one():
    # keys all score -1 except where the table points outside the cache: those read as zero
    # keys (score 0, the highest) and come back as -1
    w = W.indexer(seed=3, num_tokens=2, cache_rows=1024, num_reqs=1, page_size=16, head_dim=64, topk=20,
                  min_ctx=1024, max_ctx=1024, integer=True)
    w["q"] = torch.ones_like(w["q"])
    w["key_cache"] = torch.full_like(w["key_cache"], -1.0 / 64)
    w["block_table"] = w["block_table"].copy()
    w["block_table"][0, 3] = -5                  # positions 48..63
    w["block_table"][0, 10] = 1 << 20            # positions 160..175
    out, scores = _run(w)
    for row in range(2):
        assert np.all(scores[row, 48:64] == 0) and np.all(scores[row, 160:176] == 0)
        assert np.all(scores[row, :48] == -1)
        assert out[row].tolist()[:16] == [-1] * 16 and out[row].tolist()[16:] == [-1] * 4


@pytest.mark.parametrize("k", [100, 5000])
def test_heavy_ties_take_the_slow_path(k):
    # every score equal: the K-th key's bin holds all n > 4096 keys, more than the candidate
    # buffer, so the row is done by radix passes over the whole row
    w = W.indexer(seed=7, num_tokens=3, cache_rows=16384, num_reqs=1, page_size=64, head_dim=128, topk=k,
                  min_ctx=9000, max_ctx=16000, integer=True)
    w["key_cache"] = torch.ones_like(w["key_cache"])
    say(f"[indexer] heavy ties, top {k}")
    out, _ = _run(w)
    for row in range(3):
        assert np.array_equal(out[row], oracle.key_slots(w["block_table"], 64, 0, k))


def test_calls_are_independent():
    # two shapes in a row, then the first again
    a = W.indexer(seed=21, num_tokens=24, cache_rows=20000, num_reqs=2, page_size=16, head_dim=64, topk=300,
                  min_ctx=5000, max_ctx=20000, integer=True)
    b = W.indexer(seed=22, num_tokens=9, cache_rows=9000, num_reqs=3, page_size=32, head_dim=128, topk=64,
                  min_ctx=100, max_ctx=9000, integer=True)
    say("[indexer] A, B, A")
    out_a, _ = _run(a)
    out_b, _ = _run(b)
    again, _ = _run(a)
    assert np.array_equal(out_a, again)
    assert np.array_equal(out_a, oracle.indexer_topk(*_oracle_inputs(a), 300))
    assert np.array_equal(out_b, oracle.indexer_topk(*_oracle_inputs(b), 64))


def test_rows_longer_than_one_segment():
    # 32768 positions per step of the pass over the row: rows of up to 150000 keys take five
    w = W.indexer(seed=23, num_tokens=6, cache_rows=150000, num_reqs=1, page_size=64, head_dim=64, topk=1000,
                  min_ctx=60000, max_ctx=150000, integer=True)
    say("[indexer] rows over several segments")
    out, _ = _run(w)
    assert np.array_equal(out, oracle.indexer_topk(*_oracle_inputs(w), 1000))


def test_sample_that_misses_takes_the_slow_path():
    # the sampled positions (128 runs of 16, n / 128 apart) hold the row's only high scores, all
    # distinct, so the threshold from the sample is met by fewer than K keys of the row: the
    # selection must notice and do the row by radix passes
    n, S, k, D = 20000, 2048, 2000, 64
    w = W.indexer(seed=9, num_tokens=1, cache_rows=n, num_reqs=1, page_size=16, head_dim=D, topk=k,
                  min_ctx=n, max_ctx=n, integer=True)
    q = torch.zeros(1, D)
    q[0, 0], q[0, 1] = 256.0, 1.0
    slots = oracle.key_slots(w["block_table"], 16, 0, n)
    kc = torch.zeros(n, D)
    kc[:, 0] = -1.0
    for i in range(S):
        v, p = S - i, (i >> 4) * (n >> 7) + (i & 15)
        kc[slots[p], 0], kc[slots[p], 1] = v // 256, v % 256
    w["q"], w["key_cache"] = q.to(torch.bfloat16), kc.to(torch.bfloat16)
    say("[indexer] sample that misses")
    out, scores = _run(w)
    args = _oracle_inputs(w)
    assert np.array_equal(scores[0, :n], oracle.indexer_scores(*args)[0])
    assert np.array_equal(out, oracle.indexer_topk(*args, k))


# the sampled threshold across K / n: tiny K on long rows (the margin's +8 dominates), K near n
# (the threshold admits most of the row), and K so close to n that the candidates overflow the
# buffer (the row takes the slow path)
REGIMES = {
    "k16_long_rows": (31, 4, 70000, 16, 60000, 70000),
    "k6000_of_8000": (32, 3, 8000, 6000, 8000, 8000),
    "k8000_of_9000": (33, 2, 9000, 8000, 9000, 9000),
    "k2048_mixed": (34, 24, 40000, 2048, 100, 40000),
}


@pytest.mark.parametrize("name", sorted(REGIMES))
def test_sampled_threshold_regimes(name):
    seed, rows, cache, k, lo, hi = REGIMES[name]
    w = W.indexer(seed=seed, num_tokens=rows, cache_rows=cache, num_reqs=1, page_size=32, head_dim=128, topk=k,
                  min_ctx=lo, max_ctx=hi, integer=True)
    say(f"[indexer] threshold regime {name}")
    out, _ = _run(w)
    assert np.array_equal(out, oracle.indexer_topk(*_oracle_inputs(w), k))
    wn = W.indexer(seed=seed, num_tokens=rows, cache_rows=cache, num_reqs=1, page_size=32, head_dim=128, topk=k,
                   min_ctx=lo, max_ctx=hi)
    out_n, scores_n = _run(wn)
    _check_within_bound(wn, out_n, scores_n, range(rows))


def test_many_requests_short_rows():
    # a decode-like batch: 2048 rows over 512 requests, contexts up to 3000, top 256 (many rows
    # keep all their keys and pad, the others select from one chunk)
    w = W.indexer(seed=41, num_tokens=2048, cache_rows=512 * 3072, num_reqs=512, page_size=64, head_dim=64,
                  topk=256, min_ctx=1, max_ctx=3000, integer=True)
    say("[indexer] 2048 rows over 512 requests")
    out, _ = _run(w)
    assert np.array_equal(out, oracle.indexer_topk(*_oracle_inputs(w), 256))


def test_rows_outside_every_request_keep_nothing():
    # req_row_ptr ends before num_rows: rows 7..9 belong to no request and come back as -1
    w = W.indexer(seed=43, num_tokens=10, cache_rows=4000, num_reqs=2, page_size=16, head_dim=64, topk=50,
                  min_ctx=20, max_ctx=2000, integer=True)
    w["req_row_ptr"] = np.array([0, 3, 7], np.int32)
    out, _ = _run(w)
    assert np.all(out[7:] == -1)
    ctx = np.minimum(w["ctx_len"][:7], np.repeat(w["req_kv_len"], np.diff(w["req_row_ptr"])))
    ref = oracle.indexer_topk(w["q"].float().numpy()[:7], w["key_cache"].float().numpy(), w["block_table"],
                              w["page_size"], w["req_row_ptr"], ctx, 50)
    assert np.array_equal(out[:7], ref)


def test_full_size_large_k():
    # K = 7000 of up to 65536 keys: the candidates above the sampled threshold exceed 8192 and
    # stay within the buffer
    w = W.indexer(integer=True, topk=7000)
    say("[indexer] full size, top 7000")
    out, _ = _run(w)
    args = _oracle_inputs(w)
    rows = [0, 17, 64, 127]
    ref = oracle.indexer_topk(args[0][rows], args[1], args[2], args[3], np.array([0, len(rows)], np.int32),
                              args[5][rows], 7000)
    assert np.array_equal(out[rows], ref)
