"""Pins of the oracle's element masks inside blocks (plan(): mask (nnz, R, C)
and packed_mask) and variable block sizes (VariableBlockSparseAttentionWrapper:
block_mask_map with block_row_sz / block_col_sz).  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import (bsr_attention, element_mask, element_mask_attention, head_block_masks,
                    unpack_block_masks, variable_block_attention, variable_block_masks)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, k, v, dense, sm_scale):
    """fp64 torch SDPA per qo head under dense masks (kv heads, M, N); qo head h
    uses kv head h // g.  Rows without a key are left out of the comparison."""
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv
    d = torch.from_numpy(dense).repeat_interleave(g, dim=0)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(g, 1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(g, 1).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=d, scale=sm_scale)
    logits = sm_scale * (tq @ tk.transpose(1, 2))
    lse = torch.logsumexp(logits.masked_fill(~d, float("-inf")), dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


# ---- variable block sizes

def test_variable_worked_example_token_mask():
    with open(os.path.join(GOLDEN, "variable_block_example_6x6.json")) as f:
        gd = json.load(f)
    got = variable_block_masks(gd["block_mask_map"], gd["block_row_sz"], gd["block_col_sz"])
    assert np.array_equal(got[0], np.array(gd["token_mask"], bool))


def test_variable_worked_example_attention():
    with open(os.path.join(GOLDEN, "variable_block_example_6x6.json")) as f:
        gd = json.load(f)
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((6, 1, 16)) for _ in range(3))
    o, lse = variable_block_attention(gd["block_mask_map"], gd["block_row_sz"], gd["block_col_sz"], q, k, v)
    ro, rl = _sdpa(q, k, v, np.array(gd["token_mask"], bool)[None], 0.25)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-13)


def _loop_token_mask(bm, rs, cs, causal):
    """Pure-Python: walk the block boundaries and fill each visible block."""
    H, MB, NB = len(bm), len(bm[0]), len(bm[0][0])
    M, N = sum(rs[0]), sum(cs[0])
    out = np.zeros((H, M, N), bool)
    for h in range(H):
        r0 = 0
        for a in range(MB):
            c0 = 0
            for b in range(NB):
                if bm[h][a][b]:
                    for i in range(r0, r0 + rs[h][a]):
                        for j in range(c0, c0 + cs[h][b]):
                            out[h, i, j] = (not causal) or j <= i + N - M
                c0 += cs[h][b]
            r0 += rs[h][a]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_variable_masks_loop(seed):
    rng = np.random.default_rng(40 + seed)
    H, MB, NB = 1 + seed % 3, int(rng.integers(1, 5)), int(rng.integers(1, 5))
    rs = rng.integers(0, 4, (H, MB))
    cs = rng.integers(0, 4, (H, NB))
    # every head covers the same counts: put the difference into each head's last block
    rs[:, -1] += rs.sum(1).max() - rs.sum(1)
    cs[:, -1] += cs.sum(1).max() - cs.sum(1)
    bm = rng.random((H, MB, NB)) < 0.5
    causal = seed % 2 == 1
    want = _loop_token_mask(bm.tolist(), rs.tolist(), cs.tolist(), causal)
    assert np.array_equal(variable_block_masks(bm, rs, cs, causal), want)


def test_variable_uniform_sizes_equal_fixed_blocks():
    rng = np.random.default_rng(3)
    bm = rng.random((2, 4, 3)) < 0.5
    got = variable_block_masks(bm, np.full((2, 4), 3), np.full((2, 3), 5), causal=True)
    assert np.array_equal(got, head_block_masks(bm, 12, 15, 3, 5, causal=True))


def test_variable_attention_gqa_sdpa():
    rng = np.random.default_rng(8)
    H, g = 2, 3
    rs = np.array([[2, 5, 3], [4, 4, 2]])
    cs = np.array([[6, 1, 5], [3, 3, 6]])
    bm = rng.random((H, 3, 3)) < 0.6
    bm[:, :, 0] = True
    q, k, v = rng.standard_normal((10, H * g, 8)), rng.standard_normal((12, H, 8)), rng.standard_normal((12, H, 5))
    o, lse = variable_block_attention(bm, rs, cs, q, k, v, sm_scale=0.3)
    ro, rl = _sdpa(q, k, v, _loop_token_mask(bm.tolist(), rs.tolist(), cs.tolist(), False), 0.3)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("rs,cs", [
    ([[1, 2]], [[3, 1, 1]]),            # shapes do not match the (1, 2, 2) map
    ([[1, 2], [2, 2]], [[3, 1], [3, 1]]),  # heads disagree on the query count
    ([[-1, 4]], [[3, 1]]),
])
def test_variable_rejects(rs, cs):
    bm = np.ones((len(rs), 2, 2), bool)
    with pytest.raises(ValueError):
        variable_block_masks(bm, np.array(rs), np.array(cs))


# ---- element masks inside blocks

def test_packed_bit_order_hand_example():
    # entries 0, 2 and 8 set in a (1, 3, 3) mask: byte 0 = 0b00000101, byte 1 = 0b00000001
    got = unpack_block_masks(np.array([0b101, 0b1], np.uint8), 1, 3, 3)
    want = np.zeros((1, 3, 3), bool)
    want[0, 0, 0] = want[0, 0, 2] = want[0, 2, 2] = True
    assert np.array_equal(got, want)


def test_packed_matches_numpy_unpackbits_little():
    rng = np.random.default_rng(2)
    packed = rng.integers(0, 256, 23).astype(np.uint8)
    got = unpack_block_masks(packed, 5, 4, 9)          # 180 bits of 184
    assert np.array_equal(got.ravel(), np.unpackbits(packed, bitorder="little")[:180].astype(bool))


def _random_bsr(rng, M, NB, R, density):
    MB = -(-M // R)
    rows = [rng.permutation(np.nonzero(rng.random(NB) < density)[0]) for _ in range(MB)]
    indptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    indices = (np.concatenate(rows) if indptr[-1] else np.zeros(0)).astype(np.int32)
    return indptr, indices


def test_full_element_masks_equal_plain_bsr():
    rng = np.random.default_rng(4)
    M, R, C, NB = 11, 3, 4, 5
    indptr, indices = _random_bsr(rng, M, NB, R, 0.6)
    q, k, v = rng.standard_normal((M, 4, 6)), rng.standard_normal((NB * C, 2, 6)), rng.standard_normal((NB * C, 2, 3))
    full = np.ones((int(indptr[-1]), R, C), bool)
    o1, l1 = element_mask_attention(indptr, indices, M, NB * C, R, C, full, q, k, v, sm_scale=0.4)
    o2, l2 = bsr_attention(indptr, indices, M, NB * C, R, C, q, k, v, sm_scale=0.4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_causal_band_as_element_masks_equals_causal_bsr():
    """An element mask holding exactly the causal band (key J*C + c <= row I*R + r + N - M)
    reproduces causal BSR attention, empty rows included."""
    rng = np.random.default_rng(5)
    M, R, C, NB = 10, 4, 3, 6
    N = NB * C
    indptr, indices = _random_bsr(rng, M, NB, R, 0.5)
    mask = np.zeros((int(indptr[-1]), R, C), bool)
    for I in range(len(indptr) - 1):
        for p in range(indptr[I], indptr[I + 1]):
            for r in range(R):
                for c in range(C):
                    mask[p, r, c] = indices[p] * C + c <= I * R + r + N - M
    q, k, v = rng.standard_normal((M, 2, 5)), rng.standard_normal((N, 1, 5)), rng.standard_normal((N, 1, 4))
    o1, l1 = element_mask_attention(indptr, indices, M, N, R, C, mask, q, k, v, sm_scale=0.6)
    o2, l2 = bsr_attention(indptr, indices, M, N, R, C, q, k, v, sm_scale=0.6, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("seed", range(4))
def test_element_masks_sdpa(seed):
    """Dense mask assembled with torch ops (each block's R x C mask written at its
    place) against the oracle; then SDPA on it."""
    rng = np.random.default_rng(60 + seed)
    M, R, C, NB = int(rng.integers(5, 14)), int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(2, 6))
    N = NB * C
    indptr, indices = _random_bsr(rng, M, NB, R, 0.7)
    mask = rng.random((int(indptr[-1]), R, C)) < 0.6
    dense = torch.zeros(-(-M // R) * R, N, dtype=torch.bool)
    for I in range(len(indptr) - 1):
        for p in range(indptr[I], indptr[I + 1]):
            dense[I * R:(I + 1) * R, indices[p] * C:(indices[p] + 1) * C] = torch.from_numpy(mask[p])
    dense = dense[:M].numpy()
    assert np.array_equal(element_mask(indptr, indices, M, N, R, C, mask), dense)
    q, k, v = rng.standard_normal((M, 2, 6)), rng.standard_normal((N, 2, 6)), rng.standard_normal((N, 2, 4))
    o, lse = element_mask_attention(indptr, indices, M, N, R, C, mask, q, k, v, sm_scale=0.5)
    live = dense.any(axis=1)
    ro, rl = _sdpa(q[live], k, v, dense[live][None].repeat(2, axis=0), 0.5)
    np.testing.assert_allclose(o[live], ro, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse[live], rl, rtol=1e-12, atol=1e-12)
    assert np.all(o[~live] == 0) and np.all(np.isneginf(lse[~live]))


def test_element_masks_follow_given_index_order():
    """Mask p belongs to indices[p]: permuting a row's indices together with its masks
    changes nothing; permuting the indices alone changes the result."""
    rng = np.random.default_rng(9)
    M, R, C, N = 4, 4, 2, 6
    indptr, indices = np.array([0, 3], np.int32), np.array([2, 0, 1], np.int32)
    mask = rng.random((3, R, C)) < 0.5
    mask[:, :, 0] = True
    q, k, v = rng.standard_normal((M, 1, 4)), rng.standard_normal((N, 1, 4)), rng.standard_normal((N, 1, 4))
    base = element_mask(indptr, indices, M, N, R, C, mask)
    perm = np.array([1, 2, 0])
    assert np.array_equal(element_mask(indptr, indices[perm], M, N, R, C, mask[perm]), base)
    assert not np.array_equal(element_mask(indptr, indices[perm], M, N, R, C, mask), base)
    o1, _ = element_mask_attention(indptr, indices, M, N, R, C, mask, q, k, v)
    o2, _ = element_mask_attention(indptr, indices[perm], M, N, R, C, mask[perm], q, k, v)
    assert np.array_equal(o1, o2)


def test_element_mask_rejects_wrong_shape():
    with pytest.raises(ValueError):
        element_mask(np.array([0, 1]), np.array([0]), 2, 2, 2, 2, np.ones((1, 2, 3), bool))
    with pytest.raises(ValueError):
        unpack_block_masks(np.zeros(1, np.uint8), 1, 3, 3)   # 9 bits need 2 bytes
