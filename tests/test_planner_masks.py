"""Host planner with element masks inside blocks and variable block sizes.

The token-level mask a plan encodes -- every tile's rows against its column
range, each key's bit taken from the exported bit planes, the causal band on
top as the kernel applies it -- must equal the oracle's mask exactly.  CPU
only: planning with a given CU count never touches the GPU."""
import numpy as np
import pytest

import oracle
from paged_attention_bsr_amd import Plan
from paged_attention_bsr_amd._lib import BsaError, BSA_KERNEL_TILE

CUS = 16


def plan_mask(p: Plan, M, N, g, Hkv, causal):
    """(Hkv, M, N) visibility the plan encodes (rows I*R + r of a tile's row block,
    keys of its column range, bits from the planes, causal band)."""
    inf, t = p.info(), p.tables()
    R, C = inf["R"], inf["C"]
    bits = t.get("mask_bits")
    out = np.zeros((Hkv, M, N), bool)
    for I, h, row0, nrows, cb, ce, _, _ in t["tiles"]:
        toks = sorted({int(I) * R + r // g for r in range(row0, row0 + nrows)})
        for e in range(cb, ce):
            J = int(t["cols"][e])
            for tok in toks:
                r = tok - int(I) * R
                for c in range(C):
                    pos = e * C + c
                    ok = True if bits is None else bool((bits[r, pos >> 5] >> (pos & 31)) & 1)
                    if causal and J * C + c > tok + N - M:
                        ok = False
                    if ok:
                        out[h, tok, J * C + c] = True
    return out


def _bsr(rng, M, NB, R, density):
    MB = -(-M // R)
    rows = [rng.permutation(np.nonzero(rng.random(NB) < density)[0]) for _ in range(MB)]
    indptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    indices = (np.concatenate(rows) if indptr[-1] else np.zeros(0)).astype(np.int32)
    return indptr, indices


@pytest.mark.parametrize("seed,M,NB,R,C,g,packed,splits", [
    (0, 13, 5, 4, 3, 1, False, 1),
    (1, 40, 6, 16, 8, 2, True, 2),
    (2, 200, 7, 64, 64, 4, False, 0),
    (3, 70, 9, 32, 16, 8, True, 3),
    (4, 9, 4, 1, 32, 4, True, 1),      # a decode shape: masks go to the tile kernel
])
def test_element_mask_planes_match_oracle(seed, M, NB, R, C, g, packed, splits):
    rng = np.random.default_rng(seed)
    N = NB * C
    indptr, indices = _bsr(rng, M, NB, R, 0.6)
    mask = rng.random((int(indptr[-1]), R, C)) < 0.5
    kw = {"packed_mask": np.packbits(mask.ravel(), bitorder="little")} if packed else {"mask": mask}
    p = Plan(indptr, indices, M, N, R, C, 2 * g, 2, 128, causal=True, kv_splits=splits, num_cus=CUS, **kw)
    assert p.info()["kernel"] == BSA_KERNEL_TILE
    want = oracle.element_mask(indptr, indices, M, N, R, C, mask)   # the causal flag has no effect
    got = plan_mask(p, M, N, g, 2, causal=False)
    assert np.array_equal(got[0], want) and np.array_equal(got[1], want)


@pytest.mark.parametrize("seed,H,g,causal,R,C", [
    (0, 1, 1, False, 0, 0),
    (1, 2, 2, True, 0, 0),
    (2, 3, 1, True, 4, 2),
    (3, 2, 4, False, 8, 0),
])
def test_variable_block_planes_match_oracle(seed, H, g, causal, R, C):
    rng = np.random.default_rng(30 + seed)
    MBv, NBv = int(rng.integers(2, 6)), int(rng.integers(2, 6))
    rs = rng.integers(0, 9, (H, MBv))
    cs = rng.integers(0, 9, (H, NBv))
    rs[:, -1] += rs.sum(1).max() - rs.sum(1) + 1
    cs[:, -1] += 32 - cs.sum(1) % 32 if cs.sum(1).max() % 32 else 0
    cs[:, -1] += cs.sum(1).max() - cs.sum(1)
    bm = rng.random((H, MBv, NBv)) < 0.5
    p = Plan.variable(bm, rs, cs, H * g, H, 128, R=R, C=C, causal=causal, num_cus=CUS)
    M, N = int(rs[0].sum()), int(cs[0].sum())
    want = oracle.variable_block_masks(bm, rs, cs, causal)
    assert np.array_equal(plan_mask(p, M, N, g, H, causal), want)


def test_variable_worked_example_plan():
    bm = np.array([[[0, 0, 1], [1, 0, 1], [0, 1, 1]]], bool)
    p = Plan.variable(bm, [[1, 2, 3]], [[3, 1, 2]], 1, 1, 128, num_cus=CUS)
    want = np.array([[0, 0, 0, 0, 1, 1], [1, 1, 1, 0, 1, 1], [1, 1, 1, 0, 1, 1],
                     [0, 0, 0, 1, 1, 1], [0, 0, 0, 1, 1, 1], [0, 0, 0, 1, 1, 1]], bool)
    assert np.array_equal(plan_mask(p, 6, 6, 1, 1, False)[0], want)


def test_variable_default_grid():
    # g = 4: R = 128 / 4; mean column block 96 * 2 / 4 = 48, a quarter 12 -> C = 8 (divides N = 96)
    p = Plan.variable(np.ones((2, 1, 2), bool), [[100], [100]], [[40, 56], [90, 6]], 8, 2, 128, num_cus=CUS)
    assert (p.info()["R"], p.info()["C"]) == (32, 8)
    assert (p.R, p.C, p.M, p.N) == (32, 8, 100, 96)
    # large blocks keep 64-key blocks; N = 4100 is not a multiple of 8 -> C = 4
    p = Plan.variable(np.ones((1, 1, 2), bool), [[10]], [[2048, 2048]], 1, 1, 128, num_cus=CUS)
    assert (p.info()["R"], p.info()["C"]) == (128, 64)
    p = Plan.variable(np.ones((1, 1, 2), bool), [[10]], [[2050, 2050]], 1, 1, 128, num_cus=CUS)
    assert p.info()["C"] == 4


def _expect_error(**kw):
    base = dict(indptr=np.array([0, 1], np.int32), indices=np.array([0], np.int32), M=4, N=4, R=4, C=4,
                num_qo_heads=2, num_kv_heads=2, head_dim=128, num_cus=CUS)
    base.update(kw)
    with pytest.raises((BsaError, ValueError)):
        Plan(**base)


def test_mask_rejections():
    m = np.ones((1, 4, 4), bool)
    _expect_error(mask=m, kv_block_lens=np.array([4], np.int32))
    _expect_error(mask=m, block_mask=np.ones((2, 1, 1), bool))
    # element masks run on the head_dim 128 tile kernel (fp16 / bf16, K/V also fp8), not the MLA shape
    _expect_error(mask=m, kv_dtype=__import__("torch").float8_e4m3fn, head_dim=576)
    _expect_error(mask=np.ones((2, 4, 4), bool))                 # nnz is 1
    _expect_error(packed_mask=np.zeros(1, np.uint8))             # 16 bits need 2 bytes
    _expect_error(mask=m, head_dim=64)


def test_variable_rejections():
    ok = dict(block_mask_map=np.ones((2, 1, 1), bool), block_row_sz=[[4], [4]], block_col_sz=[[8], [8]])

    def expect(**kw):
        a = dict(ok)
        a.update(kw)
        with pytest.raises((BsaError, ValueError)):
            Plan.variable(a.pop("block_mask_map"), a.pop("block_row_sz"), a.pop("block_col_sz"), 2, 2, 128,
                          num_cus=CUS, **a)
    Plan.variable(ok["block_mask_map"], ok["block_row_sz"], ok["block_col_sz"], 2, 2, 128, num_cus=CUS)
    expect(block_row_sz=[[4], [5]])                  # heads disagree on M
    expect(block_col_sz=[[8], [-1]])
    expect(block_mask_map=np.ones((1, 1, 1), bool))  # one pattern for two kv heads
    expect(C=3)                                      # N = 8 not divisible by 3
    expect(kv_block_lens=np.array([8], np.int32))
