"""The benchmark's algorithmic pair counts equal the number of visible (query,
key) pairs of the oracle's masks (summed over kv heads).  CPU only."""
import numpy as np
import pytest

import bench
import oracle
from paged_attention_bsr_amd import workloads as W


@pytest.mark.parametrize("name,kw,rows", [
    ("element_mask_prefill", dict(M=512), None),
    ("element_mask_prefill", dict(M=512), [0, 5, 63, 64, 300, 511]),
    ("variable_block_prefill", dict(M=700), None),
    ("variable_block_prefill", dict(M=700, causal=True), [0, 1, 99, 350, 699]),
])
def test_masked_pair_counts(name, kw, rows):
    w = W.by_name(name, values=False, **kw)
    if "mask" in w.meta:
        want = int(oracle.element_mask(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.meta["mask"], rows).sum())
        want *= w.num_kv_heads
    else:
        bm, rs, cs = w.meta["variable"]
        want = int(oracle.variable_block_masks(bm, rs, cs, w.causal, rows).sum())
    assert bench.masked_kv_pairs(w, rows) == want


def test_bsr_pair_counts():
    w = W.random_bsr(3, 70, 9 * 8, 16, 8, 4, 2, causal=True, partial_lens=True, values=False)
    want = int(oracle.bsr_mask(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.kv_block_lens, True).sum())
    assert bench.unmasked_pairs(w) == want
    assert bench.masked_kv_pairs(w) is None
