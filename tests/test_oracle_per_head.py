"""Pins of the oracle's per-head structure (block_mask per kv or qo head, and
q2k_indices / q2k_num direct selections; flashinfer.sparse
BlockSparseAttentionWrapper.plan parameters, VariableBlockSparseAttentionWrapper:
each kv head its own pattern).  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import block_mask_attention, bsr_attention, head_block_masks, q2k_block_mask
from tests.test_oracle import _brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dense_masks_torch(bm, M, N, R, C, lens, causal):
    """Dense (heads, M, N) masks built with torch ops alone: block (I, J) covers
    rows I*R.. and columns J*C.., cropped to M; block lengths and the causal
    band are applied as separate masks."""
    t = torch.from_numpy(bm.astype(bool))
    dense = t.repeat_interleave(R, dim=1).repeat_interleave(C, dim=2)[:, :M, :N]
    if lens is not None:
        pos = torch.arange(N)
        dense = dense & ((pos % C) < torch.from_numpy(lens).long()[pos // C])[None, None, :]
    if causal:
        dense = dense & torch.ones(M, N, dtype=torch.bool).tril(N - M)[None]
    return dense


def _case(seed, Hkv, g, R, C, M, NB, density, lens, causal):
    rng = np.random.default_rng(seed)
    MB = -(-M // R)
    N = NB * C
    bm = rng.random((Hkv, MB, NB)) < density
    bm[:, :, 0] = True          # every row keeps a key (SDPA gives NaN on empty rows)
    ln = rng.integers(1, C + 1, NB).astype(np.int32) if lens else None
    q = rng.standard_normal((M, Hkv * g, 6))
    k = rng.standard_normal((N, Hkv, 6))
    v = rng.standard_normal((N, Hkv, 5))
    return bm, ln, q, k, v, N


@pytest.mark.parametrize("seed,Hkv,g,R,C,M,NB,lens,causal", [
    (1, 2, 2, 2, 3, 7, 4, False, False),
    (2, 3, 1, 1, 4, 9, 5, True, False),
    (3, 2, 4, 3, 2, 8, 6, True, True),
    (4, 4, 2, 4, 4, 16, 4, False, True),
])
def test_per_head_masks_equal_sdpa(seed, Hkv, g, R, C, M, NB, lens, causal):
    """Each qo head attends under its kv head's own dense mask (torch SDPA, fp64)."""
    bm, ln, q, k, v, N = _case(seed, Hkv, g, R, C, M, NB, 0.5, lens, causal)
    if causal:   # keep a visible key in every row: block 0 holds key 0 <= i + N - M
        assert N >= M
    o, lse = block_mask_attention(bm, M, N, R, C, q, k, v, sm_scale=0.4, causal=causal, kv_block_lens=ln)
    dense = _dense_masks_torch(bm, M, N, R, C, ln, causal).repeat_interleave(g, dim=0)  # (Hq, M, N)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=dense, scale=0.4)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
    logits = 0.4 * torch.einsum("hmd,hnd->hmn", tq, tk).masked_fill(~dense, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).permute(1, 0).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", range(8))
def test_per_head_brute_force_tiny(case):
    """Per kv head, the pure-Python brute force on that head's own BSR rows."""
    rng = np.random.default_rng(700 + case)
    Hkv, g = 1 + case % 3, [1, 2, 3][case % 3]
    R, C = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    M = int(rng.integers(1, 12))
    NB = int(rng.integers(1, 12 // C + 1))
    N, MB = NB * C, -(-M // R)
    bm = rng.random((Hkv, MB, NB)) < 0.5
    ln = rng.integers(1, C + 1, NB).astype(np.int32) if case % 2 else None
    causal = case % 4 >= 2
    q = rng.standard_normal((M, Hkv * g, 4))
    k = rng.standard_normal((N, Hkv, 4))
    v = rng.standard_normal((N, Hkv, 3))
    o, lse = block_mask_attention(bm, M, N, R, C, q, k, v, sm_scale=0.6, causal=causal, kv_block_lens=ln)
    for h in range(Hkv):
        rows = [rng.permutation(np.nonzero(bm[h, I])[0]) for I in range(MB)]
        indptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
        indices = (np.concatenate(rows) if indptr[-1] else np.zeros(0)).astype(np.int32)
        ob, lb = _brute_force(indptr, indices, M, N, R, C, g, 1, q[:, h * g:(h + 1) * g], k[:, h:h + 1],
                              v[:, h:h + 1], 0.6, causal, ln)
        np.testing.assert_allclose(o[:, h * g:(h + 1) * g], ob, rtol=1e-9, atol=1e-12)
        got = lse[:, h * g:(h + 1) * g]
        assert np.array_equal(np.isneginf(got), np.isneginf(lb))
        fin = np.isfinite(lb)
        np.testing.assert_allclose(got[fin], lb[fin], rtol=1e-9, atol=1e-12)


def test_worked_example_as_block_mask():
    """The BSR worked example written as a block mask (R = C = 1) gives the BSR result bit for bit."""
    with open(os.path.join(GOLDEN, "worked_example_3x3.json")) as f:
        gd = json.load(f)
    rng = np.random.default_rng(5)
    Hq, Hkv, D = gd["num_qo_heads"], gd["num_kv_heads"], gd["head_dim"]
    q, k, v = rng.standard_normal((3, Hq, D)), rng.standard_normal((3, Hkv, D)), rng.standard_normal((3, Hkv, D))
    bm = np.repeat(np.array(gd["mask"], bool)[None], Hkv, axis=0)
    o1, l1 = block_mask_attention(bm, 3, 3, 1, 1, q, k, v)
    o2, l2 = bsr_attention(gd["indptr"], gd["indices"], 3, 3, 1, 1, q, k, v)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_qo_shaped_mask_with_agreeing_groups_equals_kv_shaped():
    bm, ln, q, k, v, N = _case(9, 2, 3, 2, 2, 6, 5, 0.5, True, False)
    o1, l1 = block_mask_attention(bm, 6, N, 2, 2, q, k, v, kv_block_lens=ln)
    o2, l2 = block_mask_attention(np.repeat(bm, 3, axis=0), 6, N, 2, 2, q, k, v, kv_block_lens=ln)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_empty_head_rows_give_zero_and_neg_inf():
    rng = np.random.default_rng(3)
    bm = np.zeros((2, 2, 2), bool)
    bm[0, 1, 0] = True               # kv head 0: only row block 1 sees block 0; kv head 1: nothing
    q, k, v = rng.standard_normal((4, 2, 3)), rng.standard_normal((4, 2, 3)), rng.standard_normal((4, 2, 3))
    o, lse = block_mask_attention(bm, 4, 4, 2, 2, q, k, v)
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse[:2]))
    assert np.all(o[:, 1] == 0) and np.all(np.isneginf(lse[:, 1]))
    assert np.all(np.isfinite(lse[2:, 0]))


def test_q2k_block_mask_closed_form():
    sel = np.array([[[2, 0, 5], [1, 3, 3]], [[4, 5, 0], [0, 1, 2]]], np.int32)
    num = np.array([[2, 1], [3, 0]], np.int32)
    bm = q2k_block_mask(sel, num, 6)
    want = np.zeros((2, 2, 6), bool)
    want[0, 0, [0, 2]] = True
    want[0, 1, 1] = True
    want[1, 0, [0, 4, 5]] = True
    assert np.array_equal(bm, want)
    # without q2k_num every entry counts
    assert np.array_equal(q2k_block_mask(np.array([[[3, 1]]]), None, 4), np.array([[[0, 1, 0, 1]]], bool))


@pytest.mark.parametrize("sel,num", [
    ([[[0, 0]]], None),          # repeat
    ([[[0, 7]]], None),          # out of range (NB = 4)
    ([[[0, 1]]], [[3]]),         # num > topk
    ([[[0, 1]]], [[-1]]),
])
def test_q2k_rejects(sel, num):
    with pytest.raises(ValueError):
        q2k_block_mask(np.array(sel), None if num is None else np.array(num), 4)


def test_head_block_masks_rejects_bad_shape():
    with pytest.raises(ValueError):
        head_block_masks(np.ones((1, 2, 3), bool), 4, 4, 2, 2)   # NB is 2, not 3
