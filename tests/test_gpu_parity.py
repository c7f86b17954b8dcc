"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases are compared on every output; the five full-size workloads are
compared on sampled query rows that the oracle computes one by one, in the
same launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import oracle
from paged_attention_bsr_amd import workloads as W
from paged_attention_bsr_amd import merge_states
from tests.parity_util import (TOL_F16, compare, oracle_inputs, oracle_result, plan_for, run_gpu, say,
                               to_device, tol_for)

pytestmark = pytest.mark.gpu


def _check(w, kv_splits=1, rows=None, what=None):
    what = what or f"{w.name} M={w.M} N={w.N} R={w.R} C={w.C} splits={kv_splits}"
    say(f"[parity] {what}")
    o, lse = run_gpu(w, kv_splits)
    o_ref, lse_ref = oracle_result(w, rows=rows)
    if rows is not None:
        o, lse = o[rows], lse[rows]
    return compare(o, lse, o_ref, lse_ref, tol_for(w), what)


def test_worked_example():
    _check(W.worked_example())


def test_worked_example_bf16():
    _check(W.worked_example(dtype=torch.bfloat16))


SMALL = [
    # (seed, M, NB, R, C, Hq, Hkv, causal, partial_lens, density)
    (1, 37, 9, 5, 7, 8, 2, False, False, 0.5),
    (2, 64, 8, 64, 64, 32, 8, True, False, 0.6),
    (3, 130, 6, 64, 64, 4, 1, True, False, 0.7),      # M % R != 0, g = 4, one kv head
    (4, 256, 2, 128, 128, 16, 2, True, False, 1.0),   # R = C = 128, g = 8
    (5, 9, 40, 1, 16, 32, 8, False, True, 0.4),       # paged decode shape, partial pages
    (6, 50, 70, 3, 1, 8, 8, False, False, 0.3),       # C = 1, g = 1
    (7, 33, 12, 11, 16, 12, 3, True, True, 0.5),      # odd everything, causal + lens
    (8, 300, 10, 100, 30, 2, 1, False, False, 0.5),   # tile rows > 128 per unit
    (9, 17, 5, 17, 48, 64, 8, True, False, 0.8),      # 136 rows per unit, C = 48
    (10, 70, 30, 70, 3, 4, 4, False, True, 0.5),      # C = 3 with lens
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}" for c in SMALL])
@pytest.mark.parametrize("kv_splits", [1, 3, 0])
def test_random_bsr(case, kv_splits):
    seed, M, NB, R, C, Hq, Hkv, causal, lens, dens = case
    w = W.random_bsr(seed, M, NB * C, R, C, Hq, Hkv, causal=causal, partial_lens=lens,
                     density=dens, garbage=6e4 if lens else 0.0)
    _check(w, kv_splits)


@pytest.mark.parametrize("seed", [11, 12])
def test_random_bsr_bf16(seed):
    w = W.random_bsr(seed, 90, 12 * 32, 32, 32, 16, 4, causal=seed % 2 == 0, partial_lens=True,
                     dtype=torch.bfloat16, garbage=3e4)
    _check(w, 0)


def test_empty_rows_and_empty_structure():
    w = W.random_bsr(21, 40, 8 * 4, 4, 4, 8, 2, density=0.15)
    assert (np.diff(w.indptr) == 0).any()
    _check(w, 1)
    w0 = W.random_bsr(22, 10, 4, 2, 2, 4, 2, density=0.0)
    assert w0.nnz == 0
    o, lse = run_gpu(w0)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_causal_rows_before_the_key_window():
    # M > N: early query rows have no allowed key at all (bottom-right alignment)
    w = W.random_bsr(23, 48, 16, 8, 4, 8, 2, causal=True, density=1.0)
    _check(w, 2)


def test_reduced_paged_decode():
    _check(W.paged_decode(seed=31, batch=12, min_len=1, max_len=700), 0)


def test_reduced_bsr_prefill():
    _check(W.bsr_prefill(seed=32, M=1024, density=0.3), 1)


def test_reduced_window_prefill():
    _check(W.window_prefill(seed=33, M=2048, num_qo_heads=16, num_kv_heads=2, window=3, stride=5), 1)


def test_reduced_sparse_mla():
    _check(W.sparse_mla(seed=34, num_tokens=6, num_heads=128, cache_rows=4096, topk=256, min_ctx=512,
                        max_ctx=4096), 1)
    _check(W.sparse_mla(seed=35, num_tokens=4, num_heads=64, cache_rows=2048, topk=200, min_ctx=300,
                        max_ctx=2048), 3)


def test_mla_every_fp8_code_decodes_exactly():
    """One key per query: o must be that key's V row (every e4m3 code appears)."""
    w = W.sparse_mla(seed=36, num_tokens=4, num_heads=16, cache_rows=64, topk=1, min_ctx=64, max_ctx=64)
    codes = torch.arange(256, dtype=torch.int32).remainder(256).to(torch.uint8)
    codes[codes == 0x7F] = 0x7E       # no NaN inputs
    codes[codes == 0xFF] = 0xFE
    kv = torch.zeros(64, 576, dtype=torch.uint8)
    for r in range(64):
        kv[r, :512] = codes.roll(r).repeat(2)
        kv[r, 512:] = codes[:64]
    w.k = kv.view(torch.float8_e4m3fn)
    w.k_descale = w.v_descale = 1.0
    _check(w, 1, what="mla fp8 codes")
    o, _ = run_gpu(w)
    q, k, v = oracle_inputs(w)
    for t in range(w.M):
        J = int(w.indices[t])
        ref = torch.from_numpy(v[J, 0]).to(torch.bfloat16)
        assert torch.equal(o[t].cpu(), ref.expand(w.num_qo_heads, -1)), f"token {t}"


def test_permuted_indices_give_identical_bits():
    w = W.random_bsr(41, 64, 20 * 16, 16, 16, 8, 2, causal=True, density=0.5, shuffle=False)
    o1, l1 = run_gpu(w, 0)
    rng = np.random.default_rng(0)
    for I in range(len(w.indptr) - 1):
        seg = w.indices[w.indptr[I]:w.indptr[I + 1]]
        w.indices[w.indptr[I]:w.indptr[I + 1]] = seg[rng.permutation(seg.size)]
    o2, l2 = run_gpu(w, 0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_runs_are_deterministic_and_splits_agree():
    w = W.paged_decode(seed=42, batch=16, min_len=100, max_len=3000)
    p = plan_for(w, 0)
    dev = to_device(w)
    o1, l1 = run_gpu(w, plan=p, dev=dev)
    o2, l2 = run_gpu(w, plan=p, dev=dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = run_gpu(w, 1, dev=dev)
    assert (o1.float() - o3.float()).abs().max().item() < 4e-3
    assert (l1 - l3).abs().max().item() < 1e-4


def test_merge_states_matches_oracle():
    g = torch.Generator().manual_seed(5)
    seq, ns, heads, dim = 7, 5, 3, 64
    v = torch.randn(seq, ns, heads, dim, generator=g)
    s = torch.randn(seq, ns, heads, generator=g) * 3
    s[0, :, 0] = -float("inf")          # all states empty
    s[1, 2, 1] = -float("inf")          # one empty state
    v[1, 2, 1] = float("nan")           # its values must not leak
    o_ref, s_ref = oracle.merge_states(v.double().numpy().transpose(1, 0, 2, 3), s.double().numpy().transpose(1, 0, 2))
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        say(f"[parity] merge_states {dt}")
        vo, so = merge_states(v.cuda(), s.cuda(), out_dtype=dt)
        torch.cuda.synchronize()
        tol = (1e-6, 1e-5) if dt == torch.float32 else TOL_F16
        compare(vo, so, o_ref, s_ref, tol, f"merge_states {dt}")


# ---------------------------------------------------------------- full-size workloads
FULL_ROWS = {
    "worked_example": None,
    "paged_decode": None,                                       # all 64 requests
    "bsr_prefill": [0, 1, 63, 64, 127, 4095, 4096, 6000, 8190, 8191],
    "window_prefill": [0, 1, 127, 128, 1100, 1151, 2048, 16383, 30000, 32767],
    "sparse_mla": [0, 1, 17, 64, 100, 127],
    "head_sparse_prefill": [0, 1, 63, 64, 127, 4095, 4096, 6000, 8190, 8191],
    "paged_decode_fp8": None,                                   # all 64 requests
    "element_mask_prefill": [0, 1, 63, 64, 127, 4095, 4096, 6000, 8190, 8191],
    "variable_block_prefill": [0, 1, 31, 95, 160, 4095, 4096, 6000, 8190, 8191],
    "bsr_prefill_fp8": [0, 1, 63, 64, 127, 4095, 4096, 6000, 8190, 8191],
}


@pytest.mark.parametrize("name", list(FULL_ROWS))
def test_full_size_workload(name):
    kv_splits, rows = W.BENCH_KV_SPLITS[name], FULL_ROWS[name]
    w = W.by_name(name)
    if rows is not None:
        # the fixed rows (edges of tiles and blocks) plus six drawn with a seed per workload
        rng = np.random.default_rng(sum(map(ord, name)))
        drawn = rng.choice(np.setdiff1d(np.arange(w.M), rows), 6, replace=False)
        rows = sorted(set(rows) | set(int(r) for r in drawn))
    _check(w, kv_splits, rows=rows, what=f"full {name} splits={kv_splits} rows={rows}")


DETERMINISM = {
    # tile kernel with split rows merged by LSE, fixed and automatic splits
    "bsr_prefill_s3": (lambda: W.bsr_prefill(seed=70, M=1024, density=0.3), 3),
    "bsr_prefill_auto": (lambda: W.bsr_prefill(seed=71, M=1024, density=0.3), 0),
    "fp8_prefill_auto": (lambda: W.fp8_kv(W.bsr_prefill(seed=72, M=1024, density=0.3), 72), 0),
    # decode kernel, balanced partition over the device
    "paged_decode_auto": (lambda: W.paged_decode(seed=73, batch=12, min_len=1, max_len=900), 0),
    # sparse MLA, head pairs on one XCD, unsplit and split
    "sparse_mla": (lambda: W.sparse_mla(seed=74, num_tokens=6, num_heads=128, cache_rows=4096, topk=256,
                                        min_ctx=512, max_ctx=4096), 1),
    "sparse_mla_s3": (lambda: W.sparse_mla(seed=75, num_tokens=4, num_heads=64, cache_rows=2048, topk=200,
                                           min_ctx=300, max_ctx=2048), 3),
}


@pytest.mark.parametrize("name", list(DETERMINISM))
def test_bitwise_determinism(name):
    # no atomics and a fixed reduction order: repeated runs give the same bits, also
    # after other work has run on the device in between
    make, kv_splits = DETERMINISM[name]
    w = make()
    say(f"[determinism] {name} splits={kv_splits}")
    plan = plan_for(w, kv_splits)
    q, k, v = to_device(w)
    o0, l0 = run_gpu(w, kv_splits, plan=plan, dev=(q, k, v))
    o0, l0 = o0.clone(), l0.clone()
    for i in range(3):
        if i == 1:
            torch.randn(1 << 22, device=q.device).sum()  # unrelated work in between
        o, lse = run_gpu(w, kv_splits, plan=plan, dev=(q, k, v))
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16)), f"{name}: output bits differ on run {i + 1}"
        assert torch.equal(lse.view(torch.int32), l0.view(torch.int32)), f"{name}: lse bits differ on run {i + 1}"


# Every launch variant of the generic tile kernel: (rows per tile, keys per
# tile, whole tiles inside one block or not, causal, valid lengths, dtype).
# Planning for 1 CU keeps the planner from shrinking 256-row tiles to 128.
TILE_VARIANTS = [
    # (seed, M, NB, R, C, Hq, Hkv, causal, lens, dtype, expected tile_rows)
    (31, 128, 6, 64, 64, 16, 4, True, False, torch.float16, 256),     # 64-key tiles, whole blocks
    (32, 96, 20, 32, 48, 32, 4, False, True, torch.float16, 256),     # 64-key tiles over 48-key blocks
    (33, 192, 4, 64, 256, 32, 4, True, True, torch.float16, 256),     # 128-key tiles, 2 per block, lens
    (34, 256, 3, 128, 128, 16, 4, False, False, torch.bfloat16, 256), # 128-key tiles, bf16
    (35, 96, 12, 32, 32, 16, 4, True, False, torch.float16, 128),     # 128-row tiles over 32-key blocks
    (36, 40, 30, 8, 16, 16, 4, True, True, torch.float16, 32),        # 32-row tiles
]


@pytest.mark.parametrize("case", TILE_VARIANTS, ids=[f"v{c[0]}" for c in TILE_VARIANTS])
@pytest.mark.parametrize("kv_splits", [1, 3])
def test_tile_kernel_variants(case, kv_splits):
    seed, M, NB, R, C, Hq, Hkv, causal, lens, dtype, rows = case
    w = W.random_bsr(seed, M, NB * C, R, C, Hq, Hkv, causal=causal, partial_lens=lens, density=0.6,
                     dtype=dtype, garbage=6e4 if lens else 0.0)
    p = plan_for(w, kv_splits, num_cus=1)
    assert p.info()["kernel"] == 0 and p.info()["tile_rows"] == rows
    what = f"tile variant s{seed} rows={rows} C={C} splits={kv_splits}"
    say(f"[parity] {what}")
    o, lse = run_gpu(w, kv_splits, plan=p)
    o_ref, lse_ref = oracle_result(w)
    compare(o, lse, o_ref, lse_ref, tol_for(w), what)


# The decode kernel for 1 to 16 kv heads (1, 2, 4 or 8 heads per workgroup),
# under the balanced partition planned for a few CUs, so that each resident
# workgroup runs many tile groups in a row (units cut at workgroup
# boundaries, units without keys, the next group's keys prefetched across
# every boundary), and with fixed splits (one group per workgroup).
DECODE_VARIANTS = [
    # (seed, M, NB, C, Hq, Hkv, causal, lens, density, dtype, num_cus)
    (51, 30, 40, 16, 32, 8, False, True, 0.3, torch.float16, 1),   # 2 workgroups, partial pages
    (52, 25, 30, 32, 16, 1, True, True, 0.5, torch.bfloat16, 2),   # g = 16, one kv head, causal
    (53, 40, 50, 64, 3, 3, False, False, 0.2, torch.float16, 3),   # g = 1, three kv heads, C = 64
    (54, 12, 80, 16, 8, 2, True, False, 0.9, torch.bfloat16, 5),
    (55, 48, 1, 16, 8, 2, True, False, 1.0, torch.float16, 1),     # M > N: early rows see no key
    (56, 9, 4, 16, 4, 1, False, True, 0.1, torch.float16, 2),      # nearly empty: one workgroup
    (57, 20, 24, 16, 16, 4, True, True, 0.6, torch.float16, 2),    # 4 kv heads: two waves per head
    (58, 10, 30, 32, 64, 16, False, True, 0.5, torch.bfloat16, 3), # 16 kv heads: two head groups
]


@pytest.mark.parametrize("case", DECODE_VARIANTS, ids=[f"d{c[0]}" for c in DECODE_VARIANTS])
@pytest.mark.parametrize("kv_splits", [0, 3])
def test_decode_balanced_partition(case, kv_splits):
    seed, M, NB, C, Hq, Hkv, causal, lens, dens, dtype, num_cus = case
    w = W.random_bsr(seed, M, NB * C, 1, C, Hq, Hkv, causal=causal, partial_lens=lens, density=dens,
                     dtype=dtype, garbage=6e4 if lens else 0.0)
    p = plan_for(w, kv_splits, num_cus=num_cus)
    inf = p.info()
    assert inf["kernel"] == 2
    what = (f"decode s{seed} splits={kv_splits} C={C} g={Hq // Hkv} heads/wg={inf['heads_per_wg']} "
            f"wgs={inf['num_workgroups']} tiles={inf['num_tiles']}")
    say(f"[parity] {what}")
    o, lse = run_gpu(w, kv_splits, plan=p)
    o_ref, lse_ref = oracle_result(w)
    compare(o, lse, o_ref, lse_ref, tol_for(w), what)


@pytest.mark.parametrize("causal,lens", [(True, False), (False, True), (True, True)])
def test_mla_kernel_variants(causal, lens):
    """Causal masking (early tokens lose the newest selected rows), per-block valid lengths
    (all 1 for R = C = 1: the masked path with nothing to mask), 40 heads (a partial
    16-head group) and 96 keys per token (an odd number of 32-key tiles)."""
    w = W.sparse_mla(seed=37, num_tokens=64, num_heads=40, cache_rows=1024, topk=96, min_ctx=1024,
                     max_ctx=1024)
    w.causal = causal
    if lens:
        w.kv_block_lens = np.ones(w.N // w.C, np.int32)
    if causal:  # make sure some selected rows lie above the diagonal of some token
        off = w.N - w.M
        assert any(int(j) > t + off for t in range(w.M) for j in w.indices[w.indptr[t]:w.indptr[t + 1]])
    _check(w, 1, what=f"mla variant causal={causal} lens={lens}")
    _check(w, 3, what=f"mla variant causal={causal} lens={lens} splits=3")


def _mla_logit_jump(seed, q_rope_value):
    """Sparse MLA where every token's first 32 selected rows (its first key tile) have
    nothing in their 64 rope dims, while later rows hold +448 there and q holds
    q_rope_value: those later keys' logits exceed the first tile's by about
    q_rope_value * 448 s * 64 / 24 (s the dequant scale)."""
    w = W.sparse_mla(seed=seed, num_tokens=5, num_heads=64, cache_rows=512, topk=128, min_ctx=512, max_ctx=512)
    rng = np.random.default_rng(seed)
    small, big = np.arange(0, 256), np.arange(256, 512)
    rows = [np.concatenate([rng.permutation(small)[:32], rng.permutation(np.concatenate([small, big]))[:200]])
            for _ in range(w.M)]
    rows = [np.concatenate([r[:32], [j for j in r[32:] if j not in set(r[:32])][:96]]) for r in rows]
    w.indices = np.concatenate(rows).astype(np.int32)
    codes = w.k.view(torch.uint8).clone()
    codes[small, 512:] = 0
    codes[big, 512:] = 0x7E
    w.k = codes.view(torch.float8_e4m3fn)
    w.q[:, :, 512:] = q_rope_value
    return w


def test_mla_reference_overflow_runs_a_second_pass():
    """Later keys beat the first tile's reference by ~580 log2 units: the first pass
    overflows and the workgroup redoes its key loop against the true maximum."""
    w = _mla_logit_jump(39, 30.0)
    _check(w, 1, what="mla logit jump (second pass)")
    _check(w, 2, what="mla logit jump (second pass) splits=2")


def test_mla_large_logit_growth_in_one_pass():
    """Later keys beat the first tile by ~38 log2 units: probabilities up to 2^38 in the
    single pass."""
    w = _mla_logit_jump(40, 2.0)
    _check(w, 1, what="mla logit growth")


def test_mla_paired_tiles_and_ragged_tail():
    """18 tiles: 16 dealt in XCD pairs, 2 in the ragged tail."""
    w = W.sparse_mla(seed=41, num_tokens=9, num_heads=128, cache_rows=2048, topk=160, min_ctx=512, max_ctx=2048)
    assert plan_for(w, 1).info()["num_tiles"] == 18
    _check(w, 1, what="mla 18 tiles")


@pytest.mark.parametrize("causal,lens", [(False, False), (True, True)])
def test_mla_kernel_multi_row_blocks(causal, lens):
    """The sparse-MLA kernel with blocks of 4 latent rows (C = 4) instead of single rows: key
    positions map to blocks by division, and with lengths the last rows of some blocks are
    masked (their cache slots hold garbage that must not reach the output)."""
    w = W.sparse_mla(seed=38, num_tokens=48, num_heads=64, cache_rows=1024, topk=8, min_ctx=1024,
                     max_ctx=1024)
    rng = np.random.default_rng(38)
    C, nb = 4, 1024 // 4
    w.C = C
    w.indptr = (np.arange(w.M + 1) * 24).astype(np.int32)
    w.indices = np.concatenate([rng.choice(nb, 24, replace=False) for _ in range(w.M)]).astype(np.int32)
    w.causal = causal
    if lens:
        w.kv_block_lens = rng.integers(1, C + 1, nb).astype(np.int32)
    _check(w, 1, what=f"mla C=4 causal={causal} lens={lens}")
    _check(w, 2, what=f"mla C=4 causal={causal} lens={lens} splits=2")



# ---------------------------------------------------------------- per-head structure
# Each kv head attends by its own block pattern (block_mask per kv or qo head, or
# q2k_indices / q2k_num selections); tile kernel and decode kernel shapes.
PER_HEAD = [
    # (seed, M, NB, R, C, Hq, Hkv, causal, lens, density, form)
    (41, 130, 6, 64, 64, 16, 4, True, False, 0.5, "kv"),     # M % R != 0, whole 64-key block tiles
    (42, 256, 4, 128, 128, 16, 2, True, False, 0.7, "qo"),   # 128-key tiles; mask given per qo head
    (43, 37, 9, 5, 7, 8, 2, False, True, 0.5, "q2k"),        # generic key lookup, garbage past lengths
    (44, 20, 40, 1, 16, 32, 8, False, True, 0.3, "kv"),      # decode kernel, one kv head per workgroup
    (45, 12, 30, 1, 32, 16, 4, True, True, 0.5, "q2k"),      # decode kernel, causal, lengths
    (46, 96, 12, 32, 32, 8, 8, True, False, 0.4, "qo"),      # g = 1: qo and kv heads coincide
]


def _per_head_workload(case):
    seed, M, NB, R, C, Hq, Hkv, causal, lens, dens, form = case
    w = W.random_bsr(seed, M, NB * C, R, C, Hq, Hkv, causal=causal, partial_lens=lens, density=dens,
                     garbage=6e4 if lens else 0.0)
    rng = np.random.default_rng(seed)
    bm = rng.random((Hkv, w.MB, NB)) < dens
    bm[:, -1, :] = False                      # an empty row block for every head
    if Hkv > 1:
        bm[1] = rng.random((w.MB, NB)) < 0.9  # a head far denser than the others
    g = Hq // Hkv
    if form == "kv":
        w.meta["block_mask"] = bm
    elif form == "qo":
        w.meta["block_mask"] = np.repeat(bm, g, axis=0)
    else:
        topk = int(bm.sum(axis=2).max()) + 1
        sel = np.full((Hkv, w.MB, topk), NB + 7, np.int32)   # entries past q2k_num are never read
        num = bm.sum(axis=2).astype(np.int32)
        for h in range(Hkv):
            for I in range(w.MB):
                js = rng.permutation(np.nonzero(bm[h, I])[0])
                sel[h, I, :js.size] = js
        w.meta["q2k"] = (np.repeat(sel, g, axis=0), np.repeat(num, g, axis=0))
    return w


@pytest.mark.parametrize("case", PER_HEAD, ids=[f"h{c[0]}" for c in PER_HEAD])
@pytest.mark.parametrize("kv_splits", [1, 3, 0])
def test_per_head_structure(case, kv_splits):
    w = _per_head_workload(case)
    kern = plan_for(w, kv_splits).info()["kernel"]
    _check(w, kv_splits, what=f"per-head {case[-1]} s{case[0]} kernel={kern} splits={kv_splits}")


def test_per_head_identical_heads_match_shared_plan_bitwise():
    """A per-head mask that repeats the shared rows for every head runs the same tiles through the
    tile kernel as the shared plan: the outputs agree bit for bit."""
    w = W.random_bsr(47, 200, 10 * 64, 64, 64, 32, 4, causal=True, density=0.6)
    bm = np.zeros((w.num_kv_heads, w.MB, w.NB), bool)
    for I in range(w.MB):
        bm[:, I, w.indices[w.indptr[I]:w.indptr[I + 1]]] = True
    o1, l1 = run_gpu(w, 1)
    w.meta["block_mask"] = bm
    o2, l2 = run_gpu(w, 1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_reduced_head_sparse_prefill():
    w = W.head_sparse_prefill(seed=48, M=1024)
    _check(w, 1)
    _check(w, 0)



# ---------------------------------------------------------------- fp8 e4m3 KV, head_dim 128 (decode kernel)
FP8_DECODE = [
    # (seed, M, NB, C, Hq, Hkv, causal, lens, dtype, q_scales)
    (51, 9, 40, 16, 32, 8, False, True, torch.float16, False),
    (52, 20, 30, 32, 16, 4, True, True, torch.float16, True),
    (53, 7, 50, 16, 16, 1, False, False, torch.bfloat16, True),   # one kv head, 16 qo heads
    (54, 33, 20, 48, 24, 3, False, True, torch.bfloat16, False),  # odd kv heads, C not a power of two
]


@pytest.mark.parametrize("case", FP8_DECODE, ids=[f"f{c[0]}" for c in FP8_DECODE])
@pytest.mark.parametrize("kv_splits", [1, 3, 0])
def test_fp8_kv_decode(case, kv_splits):
    """fp8 e4m3 K/V with per-kv-head scales (and per-qo-head q scales) through the decode
    kernel; unused slots of partial pages hold the largest finite codes (+-448)."""
    seed, M, NB, C, Hq, Hkv, causal, lens, dtype, qs = case
    w = W.random_bsr(seed, M, NB * C, 1, C, Hq, Hkv, causal=causal, partial_lens=lens, density=0.5, dtype=dtype)
    W.fp8_kv(w, seed, q_scales=qs)
    if lens:
        kb, vb = w.k.view(torch.uint8), w.v.view(torch.uint8)
        for J in range(NB):
            n = int(w.kv_block_lens[J])
            if n < C:
                kb[J * C + n:(J + 1) * C] = 0x7E      # +448
                vb[J * C + n:(J + 1) * C] = 0xFE      # -448
    assert plan_for(w, kv_splits).info()["kernel"] == 2
    _check(w, kv_splits, what=f"fp8 decode s{seed} {dtype} splits={kv_splits}")


# ---------------------------------------------------------------- fp8 e4m3 KV, head_dim 128 (tile kernel)
# Every launch shape of the tile kernel with fp8 K/V staged through registers: 32-, 128-
# and 256-row tiles (the 256-row ones on 64-key tiles also where C is a multiple of 128),
# whole-tile and generic key lookup, causal, valid lengths (the unused slots hold the
# largest codes), per-kv-head scale_k / scale_v and per-qo-head scale_q.
FP8_TILE = [
    # (seed, M, NB, R, C, Hq, Hkv, causal, lens, dtype, q_scales, expected tile_rows)
    (91, 128, 6, 64, 64, 16, 4, True, False, torch.float16, False, 256),    # whole 64-key block tiles
    (92, 96, 20, 32, 48, 32, 4, False, True, torch.float16, True, 256),     # generic lookup over 48-key blocks
    (93, 192, 4, 64, 256, 32, 4, True, True, torch.float16, False, 256),    # C = 256: 64-key tiles, lens
    (94, 256, 3, 128, 128, 16, 4, False, False, torch.bfloat16, True, 256), # bf16 q/o
    (95, 96, 12, 32, 32, 16, 4, True, False, torch.float16, True, 128),     # 128-row tiles over 32-key blocks
    (96, 40, 30, 8, 16, 16, 4, True, True, torch.float16, False, 32),       # 32-row tiles
    (97, 37, 9, 5, 7, 8, 2, False, True, torch.bfloat16, False, 32),        # odd everything
    (98, 9, 40, 1, 4, 32, 8, False, True, torch.float16, True, 32),         # R = 1, C < 16: not the decode kernel
]


def _fp8_tile_workload(case):
    seed, M, NB, R, C, Hq, Hkv, causal, lens, dtype, qs, _ = case
    w = W.random_bsr(seed, M, NB * C, R, C, Hq, Hkv, causal=causal, partial_lens=lens, density=0.6, dtype=dtype)
    W.fp8_kv(w, seed, q_scales=qs)
    if lens:
        kb, vb = w.k.view(torch.uint8), w.v.view(torch.uint8)
        for J in range(NB):
            n = int(w.kv_block_lens[J])
            if n < C:
                kb[J * C + n:(J + 1) * C] = 0x7E      # +448
                vb[J * C + n:(J + 1) * C] = 0xFE      # -448
    return w


@pytest.mark.parametrize("case", FP8_TILE, ids=[f"t{c[0]}" for c in FP8_TILE])
@pytest.mark.parametrize("kv_splits", [1, 3])
def test_fp8_kv_tile_kernel(case, kv_splits):
    w = _fp8_tile_workload(case)
    p = plan_for(w, kv_splits, num_cus=1)
    inf = p.info()
    assert inf["kernel"] == 0 and inf["tile_rows"] == case[-1], inf
    what = f"fp8 tile s{case[0]} rows={case[-1]} C={case[4]} {case[9]} splits={kv_splits}"
    say(f"[parity] {what}")
    o, lse = run_gpu(w, kv_splits, plan=p)
    o_ref, lse_ref = oracle_result(w)
    compare(o, lse, o_ref, lse_ref, tol_for(w), what)


def test_fp8_kv_with_element_masks():
    """fp8 K/V through the tile kernel's masked path (packed element masks)."""
    case = (99, 130, 6, 64, 64, 16, 4, 0.6, True, False)
    w = _masked_workload(case)
    W.fp8_kv(w, 99, q_scales=True)
    _check(w, 1, what="fp8 element masks")
    _check(w, 3, what="fp8 element masks splits=3")


def test_reduced_bsr_prefill_fp8():
    w = W.bsr_prefill(seed=100, M=1024, density=0.3)
    W.fp8_kv(w, 100)
    _check(w, 1, what="bsr_prefill fp8 M=1024")
    _check(w, 0, what="bsr_prefill fp8 M=1024 auto splits")


# ---------------------------------------------------------------- element masks and variable blocks
# Element masks inside BSR blocks (mask / packed_mask; the causal flag has no effect
# with them) and variable block sizes mapped onto a fixed grid with masks.
MASKED = [
    # (seed, M, NB, R, C, Hq, Hkv, keep, packed, bf16)
    (51, 130, 6, 64, 64, 16, 4, 0.6, True, False),     # M % R != 0, whole 64-key block tiles
    (52, 256, 4, 128, 128, 16, 2, 0.5, False, False),  # 256-row tiles: 64-key tiles when masked
    (53, 37, 9, 5, 7, 8, 2, 0.5, True, True),          # generic key lookup, bf16
    (54, 20, 40, 1, 16, 32, 8, 0.7, False, False),     # decode shape, run by the tile kernel
    (55, 96, 12, 32, 32, 8, 8, 0.3, True, False),      # g = 1
]


def _masked_workload(case):
    seed, M, NB, R, C, Hq, Hkv, keep, packed, bf16 = case
    w = W.random_bsr(seed, M, NB * C, R, C, Hq, Hkv, causal=True, density=0.6,
                     dtype=torch.bfloat16 if bf16 else torch.float16)
    rng = np.random.default_rng(seed)
    mask = rng.random((w.nnz, R, C)) < keep
    if w.nnz:
        mask[0] = False                                              # a block with nothing visible
        mask[w.indptr[-2]:] = False                                  # last row block: rows without keys
    if packed:
        w.meta["packed_mask"] = np.packbits(mask.ravel(), bitorder="little")
    else:
        w.meta["mask"] = mask
    return w


@pytest.mark.parametrize("case", MASKED, ids=[f"m{c[0]}" for c in MASKED])
@pytest.mark.parametrize("kv_splits", [1, 3, 0])
def test_element_masks(case, kv_splits):
    w = _masked_workload(case)
    _check(w, kv_splits, what=f"element masks s{case[0]} packed={case[8]} splits={kv_splits}")


VARIABLE = [
    # (seed, M, min_block, max_block, density, causal, Hq, Hkv, grid, dtype)
    (61, 300, 8, 40, 0.3, False, 8, 2, {}, torch.float16),
    (62, 257, 20, 90, 0.25, True, 16, 4, {}, torch.float16),            # N odd: a grid of 1-key blocks
    (63, 512, 1, 200, 0.2, True, 4, 4, {"R": 32, "C": 16}, torch.float16),
    (64, 200, 50, 50, 0.5, False, 32, 8, {"C": 8}, torch.float16),
    # causal on grids whose key blocks hold whole key tiles: the masked whole-tile path
    # with the causal mask on top (128-row tiles over 64-key blocks; 32-row tiles over
    # 32-key blocks), fp16 and bf16
    (65, 512, 20, 120, 0.3, True, 16, 4, {"R": 32, "C": 64}, torch.bfloat16),
    (66, 384, 20, 120, 0.3, True, 8, 2, {"R": 32, "C": 64}, torch.float16),
    (67, 256, 10, 60, 0.3, True, 8, 8, {"R": 32, "C": 32}, torch.float16),
]


@pytest.mark.parametrize("case", VARIABLE, ids=[f"v{c[0]}" for c in VARIABLE])
@pytest.mark.parametrize("kv_splits", [1, 0])
def test_variable_blocks(case, kv_splits):
    seed, M, lo, hi, dens, causal, Hq, Hkv, grid, dtype = case
    w = W.variable_block_prefill(seed=seed, M=M, min_block=lo, max_block=hi, density=dens, causal=causal,
                                 num_qo_heads=Hq, num_kv_heads=Hkv, dtype=dtype)
    w.meta["grid"] = grid
    if grid.get("C") in (32, 64):
        inf = plan_for(w, kv_splits).info()
        assert inf["kernel"] == 0 and inf["key_tile"] == grid["C"], inf
    _check(w, kv_splits, what=f"variable blocks s{seed} grid={grid} {dtype} splits={kv_splits}")


def test_variable_worked_example():
    bm = np.array([[[0, 0, 1], [1, 0, 1], [0, 1, 1]]], bool)
    w = W.Workload("variable_example", np.zeros(1, np.int32), np.zeros(0, np.int32), 6, 6, 1, 1, 1, 1, 128, 128,
                   False, 128 ** -0.5, meta={"variable": (bm, np.array([[1, 2, 3]]), np.array([[3, 1, 2]]))})
    g = torch.Generator().manual_seed(12)
    w.q, w.k, w.v = (torch.randn(6, 1, 128, generator=g).half() for _ in range(3))
    _check(w, 1, what="variable-block worked example")


def test_reduced_element_mask_prefill():
    _check(W.element_mask_prefill(seed=58, M=1024), 1, what="element_mask_prefill M=1024")


def test_reduced_variable_block_prefill():
    _check(W.variable_block_prefill(seed=59, M=1024), 1, what="variable_block_prefill M=1024")
