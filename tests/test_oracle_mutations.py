"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake into a private copy of the oracle's source (a
dropped term, a wrong index, a wrong log base, a wrong fp8 bias, ...),
loads that copy as a separate module, and checks that at least one pin
fails on it.  The oracle on disk is never modified.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

from tests.test_oracle import _brute_force

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "bsr_attention.py")

MUTATIONS = {
    "gqa_modulo": ("kvh = h // group\n        s = sm_scale", "kvh = h % Hkv\n        s = sm_scale"),
    "per_head_gqa_modulo": ("kvh = h // group\n        mh = ", "kvh = h % Hkv\n        mh = "),
    "ignore_block_lens": ("mask[out_row, J * C:J * C + length] = True",
                          "mask[out_row, J * C:J * C + C] = True"),
    "causal_top_left": ("mask[out_row, max(0, i + (N - M) + 1):] = False",
                        "mask[out_row, max(0, i + 1):] = False"),
    "lse_base2": ("m + np.log(safe_l)", "m + np.log2(safe_l)"),
    "no_sm_scale": ("s = sm_scale * (q[:, h, :] @ k[:, kvh, :].T)", "s = (q[:, h, :] @ k[:, kvh, :].T)"),
    "row_block_index": ("        I = i // R\n        for p in range(int(indptr[I]), int(indptr[I + 1])):\n            J = int(indices[p])\n            length",
                        "        I = min(i, len(indptr) - 2)\n        for p in range(int(indptr[I]), int(indptr[I + 1])):\n            J = int(indices[p])\n            length"),
    "fp8_bias8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "fp8_subnormal": ("sub = (m / 8.0) * 2.0 ** -6", "sub = (1.0 + m / 8.0) * 2.0 ** -7"),
    "merge_unweighted": ("w = np.where(np.isfinite(lse_states), np.exp(lse_states - top_safe), 0.0)",
                         "w = np.where(np.isfinite(lse_states), 1.0, 0.0)"),
    "merge_lse_max_only": ("lse = np.where(any_keys, top_safe + np.log(total_safe), -np.inf)",
                           "lse = np.where(any_keys, top_safe, -np.inf)"),
    "no_max_subtraction": ("p = np.where(mask, np.exp(s - m[:, None]), 0.0)",
                           "p = np.where(mask, np.exp(s), 0.0)"),
    "off_by_one_block_end": ("mask[out_row, J * C:J * C + length] = True",
                             "mask[out_row, J * C:J * C + length - 1] = True"),
    # per-head structure (block_mask / q2k selections)
    "per_head_modulo": ("mh = masks[kvh] if masks.shape[0] == Hkv else masks[h]",
                        "mh = masks[h % masks.shape[0]]"),
    "q2k_ignore_num": ("row = [int(x) for x in sel[h, I, :n]]", "row = [int(x) for x in sel[h, I, :topk]]"),
    "per_head_ignore_lens": ("key_ok = (np.arange(N) % C) < lens[np.arange(N) // C]",
                             "key_ok = np.ones(N, dtype=bool)"),
    "per_head_causal_top_left": ("out[h, out_row, max(0, i + (N - M) + 1):] = False\n    return out\n\n\ndef block_mask_attention",
                                 "out[h, out_row, max(0, i + 1):] = False\n    return out\n\n\ndef block_mask_attention"),
    "per_head_rows_by_C": ("blocks = bm[h, i // R]", "blocks = bm[h, min(i // C, bm.shape[1] - 1)]"),
    "fp8_scale_axis": ("vals = vals * sc[None, :, None]", "vals = vals * sc[None, None, :1]"),
    # element masks and variable block sizes
    "packed_big_endian": ("((packed[i // 8] >> (i % 8)) & 1)", "((packed[i // 8] >> (7 - i % 8)) & 1)"),
    "elem_mask_row_shift": ("out[out_row, J * C:(J + 1) * C] = mask[p, i % R]",
                            "out[out_row, J * C:(J + 1) * C] = mask[p, (i + 1) % R]"),
    "elem_mask_sorted_order": ("out[out_row, J * C:(J + 1) * C] = mask[p, i % R]",
                               "out[out_row, J * C:(J + 1) * C] = mask[int(indptr[I]) + sorted(indices[int(indptr[I]):int(indptr[I + 1])]).index(J), i % R]"),
    "variable_sizes_swapped": ("row_block = np.repeat(np.arange(bm.shape[1]), rs[h])",
                               "row_block = np.repeat(np.arange(bm.shape[1]), rs[h][::-1])"),
    "variable_head_zero_sizes": ("col_block = np.repeat(np.arange(bm.shape[2]), cs[h])",
                                 "col_block = np.repeat(np.arange(bm.shape[2]), cs[0])"),
    "variable_causal_top_left": ("                out[h, out_row, max(0, i + (N - M) + 1):] = False\n    return out\n\n\ndef variable_block_attention",
                                 "                out[h, out_row, max(0, i + 1):] = False\n    return out\n\n\ndef variable_block_attention"),
}


def _load(name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _pin_brute_force(mod):
    for case in range(12):
        rng = np.random.default_rng(500 + case)
        R, C = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        Hkv, g = 1 + case % 2, [1, 2, 4][case % 3]
        Hq = Hkv * g
        M = int(rng.integers(2, 13))
        NB = int(rng.integers(1, 13 // C + 1))
        N = NB * C
        MB = -(-M // R)
        rows = [rng.permutation(np.nonzero(rng.random(NB) < 0.6)[0]) for _ in range(MB)]
        indptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
        indices = (np.concatenate(rows) if indptr[-1] else np.zeros(0)).astype(np.int32)
        lens = rng.integers(1, C + 1, size=NB).astype(np.int32) if case % 4 == 1 else None
        causal = case % 2 == 1
        q, k, v = (rng.standard_normal(s) for s in [(M, Hq, 4), (N, Hkv, 4), (N, Hkv, 3)])
        o, lse = mod.bsr_attention(indptr, indices, M, N, R, C, q, k, v, sm_scale=0.7,
                                   causal=causal, kv_block_lens=lens)
        ob, lb = _brute_force(indptr, indices, M, N, R, C, Hq, Hkv, q, k, v, 0.7, causal, lens)
        if not np.allclose(o, ob, rtol=1e-9, atol=1e-12):
            return False
        if not np.array_equal(np.isneginf(lse), np.isneginf(lb)):
            return False
        fin = np.isfinite(lb)
        if not np.allclose(lse[fin], lb[fin], rtol=1e-9, atol=1e-12):
            return False
    return True


def _pin_equal_scores(mod):
    rng = np.random.default_rng(1)
    v = rng.standard_normal((4, 1, 3))
    q = np.zeros((1, 1, 3))
    k = rng.standard_normal((4, 1, 3))
    o, lse = mod.bsr_attention(np.array([0, 1]), np.array([0]), 1, 4, 1, 4, q, k, v)
    return np.allclose(o[0, 0], v[:, 0].mean(0)) and abs(lse[0, 0] - math.log(4)) < 1e-12


def _pin_sdpa(mod):
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal(s) for s in [(6, 4, 8), (8, 2, 8), (8, 2, 8)])
    o, _ = mod.bsr_attention(np.array([0, 2, 4, 6]), np.array([0, 1, 0, 1, 0, 1]), 6, 8, 2, 4, q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(2, 1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(2, 1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    return np.allclose(o, ref, rtol=1e-11, atol=1e-12)


def _pin_fp8(mod):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = mod.e4m3fn_decode(codes)
    nan = np.isnan(ref)
    return np.array_equal(np.isnan(ours), nan) and np.array_equal(ours[~nan], ref[~nan])


def _pin_merge(mod):
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal(s) for s in [(3, 2, 4), (10, 1, 4), (10, 1, 4)])
    mask = rng.random((3, 10)) < 0.7
    mask[:, 0] = True
    o_full, l_full = mod.masked_attention(q, k, v, mask, 0.5)
    parts = []
    for a, b in [(0, 4), (4, 10)]:
        m = np.zeros_like(mask)
        m[:, a:b] = mask[:, a:b]
        parts.append(mod.masked_attention(q, k, v, m, 0.5))
    om, lm = mod.merge_states(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    return np.allclose(om, o_full, rtol=1e-12) and np.allclose(lm, l_full, rtol=1e-12)


def _pin_per_head_sdpa(mod):
    """Per-kv-head block masks (R != C, M < N, lengths, causal) against torch SDPA on a dense
    per-head mask built with torch ops."""
    from tests.test_oracle_per_head import _dense_masks_torch
    rng = np.random.default_rng(4)
    Hkv, g, R, C, M, NB = 3, 2, 3, 2, 8, 6
    N, MB = NB * C, -(-M // R)
    bm = rng.random((Hkv, MB, NB)) < 0.5
    bm[:, :, 0] = True
    ln = rng.integers(1, C + 1, NB).astype(np.int32)
    q, k, v = rng.standard_normal((M, Hkv * g, 4)), rng.standard_normal((N, Hkv, 4)), rng.standard_normal((N, Hkv, 3))
    try:
        o, _ = mod.block_mask_attention(bm, M, N, R, C, q, k, v, sm_scale=0.5, causal=True, kv_block_lens=ln)
    except (ValueError, IndexError):
        return False
    dense = _dense_masks_torch(bm, M, N, R, C, ln, True).repeat_interleave(g, dim=0)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(g, 1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(g, 1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=dense, scale=0.5)
    return np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def _pin_q2k(mod):
    sel = np.array([[[2, 0, 0], [1, 3, 3]]], np.int32)
    try:
        bm = mod.q2k_block_mask(sel, np.array([[2, 1]], np.int32), 4)
    except ValueError:
        return False
    want = np.zeros((1, 2, 4), bool)
    want[0, 0, [0, 2]] = True
    want[0, 1, 1] = True
    return np.array_equal(bm, want)


def _pin_fp8_heads(mod):
    codes = np.arange(96, dtype=np.uint8).reshape(4, 3, 8)
    scales = np.array([0.5, 2.0, 3.0])
    try:
        got = mod.fp8_dequant(codes, scales, descale=0.25)
    except (ValueError, IndexError):
        return False
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 0.25 * scales[None, :, None]
    return np.array_equal(got, ref)


def _pin_packed_bits(mod):
    try:
        got = mod.unpack_block_masks(np.array([0b101, 0b1], np.uint8), 1, 3, 3)
    except (ValueError, IndexError):
        return False
    want = np.zeros((1, 3, 3), bool)
    want[0, 0, 0] = want[0, 0, 2] = want[0, 2, 2] = True
    return np.array_equal(got, want)


def _pin_element_masks(mod):
    """Element masks (unsorted indices, R != C, partial last row block) against a dense
    mask written block by block with torch ops."""
    rng = np.random.default_rng(61)
    M, R, C, NB = 11, 3, 2, 5
    N = NB * C
    rows = [rng.permutation(np.nonzero(rng.random(NB) < 0.7)[0]) for _ in range(-(-M // R))]
    indptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    indices = np.concatenate(rows).astype(np.int32)
    mask = rng.random((int(indptr[-1]), R, C)) < 0.6
    dense = torch.zeros(-(-M // R) * R, N, dtype=torch.bool)
    for I in range(len(indptr) - 1):
        for p in range(indptr[I], indptr[I + 1]):
            dense[I * R:(I + 1) * R, indices[p] * C:(indices[p] + 1) * C] = torch.from_numpy(mask[p])
    try:
        got = mod.element_mask(indptr, indices, M, N, R, C, mask)
    except (ValueError, IndexError):
        return False
    return np.array_equal(got, dense[:M].numpy())


def _pin_variable_blocks(mod):
    """The variable-block worked example's hand-written token mask, and a two-head causal
    case against a pure-Python walk over the block boundaries."""
    from tests.test_oracle_masks import _loop_token_mask
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "variable_block_example_6x6.json")) as f:
        gd = json.load(f)
    rs = np.array([[2, 5, 0, 3], [4, 4, 1, 1]])
    cs = np.array([[6, 1, 5], [3, 3, 6]])
    bm = np.random.default_rng(8).random((2, 4, 3)) < 0.6
    try:
        ex = mod.variable_block_masks(gd["block_mask_map"], gd["block_row_sz"], gd["block_col_sz"])
        got = [mod.variable_block_masks(bm, rs, cs, causal=c) for c in (False, True)]
    except (ValueError, IndexError):
        return False
    return (np.array_equal(ex[0], np.array(gd["token_mask"], bool)) and
            all(np.array_equal(got[c], _loop_token_mask(bm.tolist(), rs.tolist(), cs.tolist(), bool(c)))
                for c in (0, 1)))


PINS = [_pin_brute_force, _pin_equal_scores, _pin_sdpa, _pin_fp8, _pin_merge, _pin_per_head_sdpa, _pin_q2k,
        _pin_fp8_heads, _pin_packed_bits, _pin_element_masks, _pin_variable_blocks]


def test_unmutated_copy_passes_every_pin():
    src = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "<copy>", "exec"), mod.__dict__)
    assert all(pin(mod) for pin in PINS)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _load(name)
    with np.errstate(all="ignore"):
        results = [pin(mod) for pin in PINS]
    assert not all(results), f"no pin caught mutation {name}"
