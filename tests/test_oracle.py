"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what pins it: the worked example of the flashinfer.sparse
BlockSparseAttentionWrapper documentation (golden fixture), closed forms,
a library routine (torch's scaled_dot_product_attention on the CPU, torch's
float8_e4m3fn decode), invariants of the definition, or an independent
pure-Python brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (bf16_bits_decode, bsr_attention, bsr_mask, e4m3fn_decode,
                    masked_attention, merge_states, validate_bsr)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- P1: worked example
def test_worked_example_mask_expansion():
    g = _golden("worked_example_3x3.json")
    mask = bsr_mask(g["indptr"], g["indices"], g["M"], g["N"], g["R"], g["C"])
    assert mask.dtype == bool
    assert mask.tolist() == [[bool(x) for x in r] for r in g["mask"]]


def test_worked_example_equals_dense_masked_sdpa():
    """BSR result == dense attention with the same boolean mask (torch SDPA, fp64)."""
    g = _golden("worked_example_3x3.json")
    rng = np.random.default_rng(0)
    M, N, Hq, Hkv, D = g["M"], g["N"], g["num_qo_heads"], g["num_kv_heads"], g["head_dim"]
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    o, lse = bsr_attention(g["indptr"], g["indices"], M, N, 1, 1, q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
    tm = torch.tensor(g["mask"], dtype=torch.bool)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    # log-sum-exp of the scaled logits, by direct summation
    for i in range(M):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            logits = [q[i, h] @ k[j, kvh] / math.sqrt(D) for j in range(N) if g["mask"][i][j]]
            assert lse[i, h] == pytest.approx(math.log(sum(math.exp(x) for x in logits)), abs=1e-12)


# ---------------------------------------------------------------- P2 / P3: closed forms
def test_single_key_returns_that_value_row():
    rng = np.random.default_rng(1)
    M, N, Hq, Hkv, D = 5, 7, 4, 2, 16
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    # row block i selects exactly column (3 * i) % N
    indptr = np.arange(M + 1, dtype=np.int32)
    indices = np.array([(3 * i) % N for i in range(M)], dtype=np.int32)
    o, lse = bsr_attention(indptr, indices, M, N, 1, 1, q, k, v, sm_scale=0.3)
    for i in range(M):
        j = indices[i]
        for h in range(Hq):
            kvh = h // 2
            np.testing.assert_array_equal(o[i, h], v[j, kvh])
            assert lse[i, h] == pytest.approx(0.3 * float(q[i, h] @ k[j, kvh]), rel=1e-14, abs=1e-14)


def test_equal_scores_give_mean_of_values():
    rng = np.random.default_rng(2)
    M, N, R, C, Hq, Hkv, D = 6, 12, 2, 3, 6, 3, 8
    q = np.zeros((M, Hq, D))                       # every logit is 0
    k, v = _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    indptr = np.array([0, 2, 3, 4], np.int32)
    indices = np.array([0, 3, 1, 2], np.int32)
    lens = np.array([3, 2, 1, 3], np.int32)
    o, lse = bsr_attention(indptr, indices, M, N, R, C, q, k, v, kv_block_lens=lens)
    for i in range(M):
        I = i // R
        keys = [J * C + t for J in indices[indptr[I]:indptr[I + 1]] for t in range(lens[J])]
        for h in range(Hq):
            np.testing.assert_allclose(o[i, h], v[keys, h // 2].mean(axis=0), rtol=1e-13, atol=1e-14)
            assert lse[i, h] == pytest.approx(math.log(len(keys)), abs=1e-13)
    # and a constant non-zero logit s: lse = s + ln n
    k1 = np.ones((N, Hkv, D))
    q1 = np.full((M, Hq, D), 0.25)
    _, lse1 = bsr_attention(indptr, indices, M, N, R, C, q1, k1, v, sm_scale=0.5, kv_block_lens=lens)
    s = 0.5 * 0.25 * D
    for i in range(M):
        I = i // R
        n = sum(int(lens[J]) for J in indices[indptr[I]:indptr[I + 1]])
        np.testing.assert_allclose(lse1[i], s + math.log(n), rtol=1e-14)


def test_empty_row_gives_zero_and_neg_inf():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 4, 2, 8), _rand(rng, 4, 1, 8), _rand(rng, 4, 1, 8)
    indptr = np.array([0, 1, 1, 2, 2], np.int32)
    indices = np.array([1, 3], np.int32)
    o, lse = bsr_attention(indptr, indices, 4, 4, 1, 1, q, k, v)
    assert np.all(o[1] == 0) and np.all(o[3] == 0)
    assert np.all(np.isneginf(lse[1])) and np.all(np.isneginf(lse[3]))
    assert np.all(np.isfinite(lse[0])) and np.all(np.isfinite(lse[2]))


# ---------------------------------------------------------------- P4: library routine
@pytest.mark.parametrize("g", [1, 4])
def test_all_blocks_equals_full_attention(g):
    rng = np.random.default_rng(4 + g)
    M, N, R, C, Hkv, D = 10, 12, 3, 4, 2, 16
    Hq = Hkv * g
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    MB, NB = -(-M // R), N // C
    indptr = (np.arange(MB + 1) * NB).astype(np.int32)
    indices = np.tile(np.arange(NB), MB).astype(np.int32)
    o, _ = bsr_attention(indptr, indices, M, N, R, C, q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_lower_blocks_causal_equals_sdpa_causal():
    rng = np.random.default_rng(7)
    M = N = 12
    R = C = 4
    Hq, Hkv, D = 4, 2, 8
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    rows = [list(range(I + 1)) for I in range(M // R)]
    indptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    indices = np.concatenate(rows).astype(np.int32)
    o, _ = bsr_attention(indptr, indices, M, N, R, C, q, k, v, causal=True)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(2, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(2, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P5 / P6 / P9: invariants
def test_permuting_indices_within_rows_is_bitwise_invariant():
    rng = np.random.default_rng(8)
    M, N, R, C, Hq, Hkv, D = 9, 16, 2, 4, 4, 2, 8
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    indptr = np.array([0, 2, 5, 5, 7, 8], np.int32)
    indices = np.array([3, 0, 1, 2, 3, 0, 2, 1], np.int32)
    o1, l1 = bsr_attention(indptr, indices, M, N, R, C, q, k, v)
    perm = indices.copy()
    for I in range(len(indptr) - 1):
        seg = perm[indptr[I]:indptr[I + 1]]
        perm[indptr[I]:indptr[I + 1]] = seg[rng.permutation(seg.size)]
    o2, l2 = bsr_attention(indptr, perm, M, N, R, C, q, k, v)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_causal_upper_blocks_contribute_nothing():
    rng = np.random.default_rng(9)
    M = N = 16
    R = C = 4
    Hq, Hkv, D = 2, 1, 8
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    lower = [[0], [0, 1], [1, 2], [0, 3]]
    full = [[0, 2, 3], [0, 1, 3], [1, 2, 3], [0, 3]]
    def csr(rows):
        return (np.cumsum([0] + [len(r) for r in rows]).astype(np.int32),
                np.concatenate(rows).astype(np.int32))
    o1, l1 = bsr_attention(*csr(lower), M, N, R, C, q, k, v, causal=True)
    o2, l2 = bsr_attention(*csr(full), M, N, R, C, q, k, v, causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_block_lens_equal_deleting_masked_columns():
    rng = np.random.default_rng(10)
    M, R, C, Hq, Hkv, D = 4, 2, 4, 2, 1, 8
    NB = 3
    N = NB * C
    lens = np.array([4, 1, 3], np.int32)
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    indptr = np.array([0, 3, 5], np.int32)
    indices = np.array([2, 0, 1, 1, 2], np.int32)
    o1, l1 = bsr_attention(indptr, indices, M, N, R, C, q, k, v, kv_block_lens=lens)
    # physically delete the masked columns and use one key per block (R = 2, C = 1)
    keep = [J * C + t for J in range(NB) for t in range(lens[J])]
    owner = {J: [keep.index(J * C + t) for t in range(lens[J])] for J in range(NB)}
    rows = [sum((owner[J] for J in indices[indptr[I]:indptr[I + 1]]), []) for I in range(2)]
    ip2 = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    ix2 = np.concatenate(rows).astype(np.int32)
    o2, l2 = bsr_attention(ip2, ix2, M, len(keep), R, 1, q, k[keep], v[keep])
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- P7: brute force
def _brute_force(indptr, indices, M, N, R, C, Hq, Hkv, q, k, v, sm_scale, causal, lens):
    """Independent pure-Python evaluation: walk the blocks of each row, no mask matrix."""
    g = Hq // Hkv
    Dv = v.shape[2]
    o = [[[0.0] * Dv for _ in range(Hq)] for _ in range(M)]
    lse = [[-math.inf] * Hq for _ in range(M)]
    for i in range(M):
        I = i // R
        keys = []
        for p in range(indptr[I], indptr[I + 1]):
            J = int(indices[p])
            n = C if lens is None else int(lens[J])
            for t in range(n):
                j = J * C + t
                if causal and j > i + (N - M):
                    continue
                keys.append(j)
        if not keys:
            continue
        for h in range(Hq):
            kvh = h // g
            logits = [sm_scale * sum(float(q[i, h, d]) * float(k[j, kvh, d]) for d in range(q.shape[2]))
                      for j in keys]
            top = max(logits)
            w = [math.exp(x - top) for x in logits]
            tot = sum(w)
            for d in range(Dv):
                o[i][h][d] = sum(wi * float(v[j, kvh, d]) for wi, j in zip(w, keys)) / tot
            lse[i][h] = top + math.log(tot)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("case", range(12))
def test_brute_force_tiny(case):
    rng = np.random.default_rng(100 + case)
    R = int(rng.integers(1, 4))
    C = int(rng.integers(1, 4))
    g = [1, 2, 4][case % 3]
    Hkv = 1 + case % 2
    Hq = Hkv * g
    M = int(rng.integers(1, 13))
    NB = int(rng.integers(1, 13 // C + 1))
    N = NB * C
    D, Dv = 5, 3 + case % 3
    MB = -(-M // R)
    rows = [rng.permutation(np.nonzero(rng.random(NB) < 0.5)[0]) for _ in range(MB)]
    indptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    indices = (np.concatenate(rows) if sum(len(r) for r in rows) else np.zeros(0)).astype(np.int32)
    lens = rng.integers(1, C + 1, size=NB).astype(np.int32) if case % 4 == 1 else None
    causal = case % 2 == 1
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, Dv)
    sm = 0.7
    o, lse = bsr_attention(indptr, indices, M, N, R, C, q, k, v, sm_scale=sm, causal=causal,
                           kv_block_lens=lens)
    ob, lb = _brute_force(indptr, indices, M, N, R, C, Hq, Hkv, q, k, v, sm, causal, lens)
    np.testing.assert_allclose(o, ob, rtol=1e-9, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-9, atol=1e-12)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(11)
    M, N, R, C, Hq, Hkv, D = 11, 12, 3, 2, 4, 2, 8
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    MB, NB = 4, 6
    rows = [rng.permutation(np.nonzero(rng.random(NB) < 0.6)[0]) for _ in range(MB)]
    indptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    indices = np.concatenate(rows).astype(np.int32)
    o, lse = bsr_attention(indptr, indices, M, N, R, C, q, k, v, causal=True)
    sel = [10, 0, 5, 5]
    o2, l2 = bsr_attention(indptr, indices, M, N, R, C, q, k, v, causal=True, rows=sel)
    np.testing.assert_array_equal(o2, o[sel])
    np.testing.assert_array_equal(l2, lse[sel])


# ---------------------------------------------------------------- P8: merge identity
def test_merge_of_column_partition_reproduces_unsplit():
    rng = np.random.default_rng(12)
    M, N, Hq, Hkv, D = 6, 20, 4, 2, 8
    q, k, v = _rand(rng, M, Hq, D), _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D)
    mask = rng.random((M, N)) < 0.6
    mask[2] = False                                   # an empty row
    o_full, lse_full = masked_attention(q, k, v, mask, 0.4)
    cuts = [0, 3, 4, 11, 20]
    os_, ls_ = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = np.zeros_like(mask)
        part[:, a:b] = mask[:, a:b]
        o_p, l_p = masked_attention(q, k, v, part, 0.4)
        os_.append(o_p)
        ls_.append(l_p)
    o_m, l_m = merge_states(np.stack(os_), np.stack(ls_))
    np.testing.assert_allclose(o_m, o_full, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isneginf(l_m), np.isneginf(lse_full))
    fin = np.isfinite(lse_full)
    np.testing.assert_allclose(l_m[fin], lse_full[fin], rtol=1e-13)


def test_merge_two_states_closed_form():
    o = np.array([[[1.0, 2.0]], [[3.0, -1.0]]])
    lse = np.array([[0.0], [math.log(3.0)]])
    om, lm = merge_states(o, lse)
    np.testing.assert_allclose(om[0], [(1 + 3 * 3) / 4, (2 - 3) / 4])
    assert lm[0] == pytest.approx(math.log(4.0))
    om, lm = merge_states(np.array([[[5.0]], [[7.0]]]), np.array([[-np.inf], [-np.inf]]))
    assert om[0, 0] == 0.0 and np.isneginf(lm[0])


# ---------------------------------------------------------------- P10: fp8 / bf16 decode
def test_e4m3fn_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.nanmax(ours) == 448.0 and ours[1] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(13)
    t = torch.from_numpy(rng.standard_normal(1000).astype(np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits_decode(bits), t.double().numpy())


# ---------------------------------------------------------------- O1: validation
@pytest.mark.parametrize("bad", [
    dict(indptr=[0, 1, 2], indices=[0, 1], M=3, N=3, R=1, C=1),          # too few row blocks
    dict(indptr=[1, 1, 2, 2], indices=[0, 1], M=3, N=3, R=1, C=1),       # indptr[0] != 0
    dict(indptr=[0, 2, 1, 2], indices=[0, 1], M=3, N=3, R=1, C=1),       # decreasing
    dict(indptr=[0, 1, 2, 3], indices=[0, 1], M=3, N=3, R=1, C=1),       # end != nnz
    dict(indptr=[0, 1, 2, 2], indices=[0, 3], M=3, N=3, R=1, C=1),       # index >= NB
    dict(indptr=[0, 2, 2, 2], indices=[1, 1], M=3, N=3, R=1, C=1),       # duplicate
    dict(indptr=[0, 1], indices=[0], M=2, N=3, R=2, C=2),                # N % C != 0
])
def test_validation_rejects(bad):
    with pytest.raises(ValueError):
        validate_bsr(np.array(bad["indptr"]), np.array(bad["indices"]), bad["M"], bad["N"],
                     bad["R"], bad["C"])


def test_validation_rejects_bad_lens():
    with pytest.raises(ValueError):
        validate_bsr(np.array([0, 1]), np.array([0]), 1, 4, 1, 2, kv_block_lens=np.array([0, 2]))
    with pytest.raises(ValueError):
        validate_bsr(np.array([0, 1]), np.array([0]), 1, 4, 1, 2, kv_block_lens=np.array([3, 2]))


# ---------------------------------------------------------------- fp8 KV with per-head scales
def test_fp8_dequant_matches_torch_with_head_scales():
    """O4 with per-head scales: torch's e4m3fn decode times the head's scale and the descale."""
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 256, size=(7, 3, 16)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0          # no NaN codes in KV data
    scales = np.array([0.5, 2.0, 3.25], np.float32)
    got = oracle.fp8_dequant(codes, scales, descale=0.75)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = ref * 0.75 * scales.astype(np.float64)[None, :, None]
    assert np.array_equal(got, ref)
    assert np.array_equal(oracle.fp8_dequant(codes), torch.from_numpy(codes).view(torch.float8_e4m3fn)
                          .to(torch.float64).numpy())
    with pytest.raises(ValueError):
        oracle.fp8_dequant(codes, scales[:2])
