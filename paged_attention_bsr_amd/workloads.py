"""Seeded synthetic workloads for BSR block-sparse attention.

This module only draws inputs: sparsity structures (indptr / indices /
per-block valid lengths) and value tensors.  It holds none of the attention
arithmetic, so both the oracle-based tests and the GPU path can consume the
same bytes without sharing any code of the method itself.

Structures are drawn with ``numpy.random.default_rng(seed)``; values with
``torch.Generator().manual_seed(seed)`` as float32 standard normals, then
rounded (round-to-nearest-even) to the storage dtype.  Everything is made on
the host, so the device copy and the oracle's copy are the same bytes.

The five workloads follow the shapes the flashinfer.sparse documentation
(BlockSparseAttentionWrapper: worked example and plan parameters) and the
MATE sparse-MLA decode documentation describe:

1. ``worked_example``  -- the 3x3 mask of the BlockSparseAttentionWrapper
   example (R = C = 1, 32 qo / 8 kv heads, head_dim 128).
2. ``paged_decode``    -- paged batch decode written as BSR with R = 1 and
   C = page size 16: one query token per request, each request owning a run
   of pages drawn from a randomly permuted shared pool, last page partial.
3. ``bsr_prefill``     -- 64x64 blocks, all diagonal blocks plus Bernoulli
   lower blocks, causal.
4. ``window_prefill``  -- 128x128 blocks, a local window of preceding blocks
   plus a stride-16 set of global column blocks, causal.
5. ``sparse_mla``      -- R = C = 1, one shared latent KV head (576 = 512 +
   64), fp8 e4m3 KV cache with a per-tensor scale, 2048 selected rows per
   query token.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = [
    "Workload",
    "worked_example",
    "paged_decode",
    "bsr_prefill",
    "window_prefill",
    "sparse_mla",
    "head_sparse_prefill",
    "paged_decode_fp8",
    "bsr_prefill_fp8",
    "fp8_kv",
    "random_bsr",
    "by_name",
    "WORKLOAD_NAMES",
]


@dataclasses.dataclass
class Workload:
    """A BSR attention problem: structure, parameters and host tensors."""

    name: str
    indptr: np.ndarray            # int32 (MB + 1,)
    indices: np.ndarray           # int32 (nnz,)
    M: int
    N: int
    R: int
    C: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int                 # q/k head dim
    head_dim_vo: int              # v/o head dim
    causal: bool
    sm_scale: float
    kv_block_lens: Optional[np.ndarray] = None   # int32 (NB,) or None
    q_dtype: torch.dtype = torch.float16
    kv_dtype: torch.dtype = torch.float16
    o_dtype: torch.dtype = torch.float16
    q: Optional[torch.Tensor] = None      # (M, Hq, D)
    k: Optional[torch.Tensor] = None      # (N, Hkv, D) or (N, D) for MLA
    v: Optional[torch.Tensor] = None      # (N, Hkv, Dv) or None (v aliases k)
    k_descale: float = 1.0
    v_descale: float = 1.0
    v_aliases_k: bool = False     # MLA: V = first head_dim_vo components of K
    k_token_stride: int = 0       # elements; 0 = contiguous
    v_token_stride: int = 0
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.indptr[-1])

    @property
    def MB(self) -> int:
        return -(-self.M // self.R)

    @property
    def NB(self) -> int:
        return self.N // self.C


def _randn(gen: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(dtype)


def _csr_from_rows(rows) -> tuple[np.ndarray, np.ndarray]:
    indptr = np.zeros(len(rows) + 1, dtype=np.int64)
    for i, r in enumerate(rows):
        indptr[i + 1] = indptr[i] + len(r)
    indices = np.concatenate([np.asarray(r, dtype=np.int64) for r in rows]) if rows else np.zeros(0)
    return indptr.astype(np.int32), indices.astype(np.int32)


def worked_example(seed: int = 1, dtype: torch.dtype = torch.float16,
                   values: bool = True) -> Workload:
    """The 3x3 BSR example of BlockSparseAttentionWrapper (R = C = 1)."""
    M = N = 3
    Hq, Hkv, D = 32, 8, 128
    w = Workload("worked_example", np.array([0, 1, 3, 5], np.int32),
                 np.array([2, 0, 2, 1, 2], np.int32), M, N, 1, 1, Hq, Hkv, D, D,
                 False, 1.0 / np.sqrt(D), q_dtype=dtype, kv_dtype=dtype, o_dtype=dtype)
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (M, Hq, D), dtype)
        w.k = _randn(g, (N, Hkv, D), dtype)
        w.v = _randn(g, (N, Hkv, D), dtype)
    return w


def paged_decode(seed: int = 2, batch: int = 64, min_len: int = 512, max_len: int = 4096,
                 page: int = 16, num_qo_heads: int = 32, num_kv_heads: int = 8,
                 head_dim: int = 128, dtype: torch.dtype = torch.float16,
                 values: bool = True) -> Workload:
    """Paged batch decode as BSR: R = 1, C = page size, last page partial.

    Request lengths are uniform in [min_len, max_len]; request i owns
    ceil(len_i / page) pages taken, in order, from one random permutation of
    the shared pool; its last page holds len_i - page * (pages_i - 1) tokens.
    Unused slots of partial pages hold random values like every other slot.
    """
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len + 1, size=batch)
    pages = -(-lens // page)
    P = int(pages.sum())
    perm = rng.permutation(P)
    rows, pos = [], 0
    block_lens = np.full(P, page, dtype=np.int32)
    for i in range(batch):
        own = perm[pos:pos + pages[i]]
        pos += pages[i]
        rows.append(own)
        block_lens[own[-1]] = lens[i] - page * (pages[i] - 1)
    indptr, indices = _csr_from_rows(rows)
    N = P * page
    w = Workload("paged_decode", indptr, indices, batch, N, 1, page, num_qo_heads,
                 num_kv_heads, head_dim, head_dim, False, 1.0 / np.sqrt(head_dim),
                 kv_block_lens=block_lens, q_dtype=dtype, kv_dtype=dtype, o_dtype=dtype,
                 meta={"seq_lens": lens.astype(np.int64)})
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (batch, num_qo_heads, head_dim), dtype)
        w.k = _randn(g, (N, num_kv_heads, head_dim), dtype)
        w.v = _randn(g, (N, num_kv_heads, head_dim), dtype)
    return w


def fp8_kv(w: Workload, seed: int, q_scales: bool = False) -> Workload:
    """Give ``w`` fp8 e4m3 K and V with one dequant scale per kv head
    (BlockSparseAttentionWrapper.run: scale_k / scale_v, per-head quantization).

    K and V are float32 normals; head h's scale is s_h = max |x[:, h, :]| / 448 and
    its stored values are x / s_h rounded to e4m3 (torch.float8_e4m3fn); the
    scales go to ``meta["scale_k"]`` / ``meta["scale_v"]`` (float32).  q keeps its
    16-bit type; with ``q_scales`` a per-qo-head multiplier in [0.5, 2) is drawn
    into ``meta["scale_q"]`` too.  Returns ``w``.
    """
    g = torch.Generator().manual_seed(seed)
    for name in ("k", "v"):
        x = torch.randn(w.N, w.num_kv_heads, w.head_dim, generator=g, dtype=torch.float32)
        s = x.abs().amax(dim=(0, 2)) / 448.0
        setattr(w, name, (x / s[None, :, None]).to(torch.float8_e4m3fn))
        w.meta[f"scale_{name}"] = s.numpy().astype(np.float32)
    if q_scales:
        w.meta["scale_q"] = (0.5 + 1.5 * torch.rand(w.num_qo_heads, generator=g)).numpy().astype(np.float32)
    w.kv_dtype = torch.float8_e4m3fn
    return w


def paged_decode_fp8(seed: int = 7, values: bool = True) -> Workload:
    """paged_decode's structure (same requests, lengths and pages) with fp8 e4m3 K/V
    and per-kv-head dequant scales (see fp8_kv); q and o fp16."""
    w = paged_decode(values=values)
    w.name = "paged_decode_fp8"
    w.kv_dtype = torch.float8_e4m3fn
    if values:
        fp8_kv(w, seed)
    return w


def bsr_prefill_fp8(seed: int = 11, values: bool = True) -> Workload:
    """bsr_prefill's structure (same blocks, causal) with fp8 e4m3 K/V and per-kv-head
    dequant scales (see fp8_kv); q and o fp16."""
    w = bsr_prefill(values=values)
    w.name = "bsr_prefill_fp8"
    w.kv_dtype = torch.float8_e4m3fn
    if values:
        fp8_kv(w, seed)
    return w


def bsr_prefill(seed: int = 3, M: int = 8192, block: int = 64, density: float = 0.10,
                num_qo_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                dtype: torch.dtype = torch.float16, values: bool = True) -> Workload:
    """All diagonal blocks plus i.i.d. Bernoulli(density) strictly-lower blocks; causal."""
    rng = np.random.default_rng(seed)
    MB = M // block
    rows = []
    for i in range(MB):
        lower = np.nonzero(rng.random(i) < density)[0]
        rows.append(np.concatenate([lower, [i]]))
    indptr, indices = _csr_from_rows(rows)
    w = Workload("bsr_prefill", indptr, indices, M, M, block, block, num_qo_heads,
                 num_kv_heads, head_dim, head_dim, True, 1.0 / np.sqrt(head_dim),
                 q_dtype=dtype, kv_dtype=dtype, o_dtype=dtype)
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (M, num_qo_heads, head_dim), dtype)
        w.k = _randn(g, (M, num_kv_heads, head_dim), dtype)
        w.v = _randn(g, (M, num_kv_heads, head_dim), dtype)
    return w


def head_sparse_prefill(seed: int = 6, M: int = 8192, block: int = 64, density: float = 0.10,
                        num_qo_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                        dtype: torch.dtype = torch.float16, values: bool = True) -> Workload:
    """bsr_prefill with a pattern of its own for every kv head: all diagonal blocks plus
    i.i.d. Bernoulli(density) strictly-lower blocks drawn per (kv head, block); causal.

    The per-head block mask (num_kv_heads, MB, MB) is in ``meta["block_mask"]``; the
    workload's indptr / indices hold the union over heads (a BSR view for sizing only).
    """
    rng = np.random.default_rng(seed)
    MB = M // block
    bm = np.zeros((num_kv_heads, MB, MB), dtype=bool)
    for h in range(num_kv_heads):
        for i in range(MB):
            bm[h, i, np.nonzero(rng.random(i) < density)[0]] = True
            bm[h, i, i] = True
    union = bm.any(axis=0)
    indptr, indices = _csr_from_rows([np.nonzero(union[i])[0] for i in range(MB)])
    w = Workload("head_sparse_prefill", indptr, indices, M, M, block, block, num_qo_heads,
                 num_kv_heads, head_dim, head_dim, True, 1.0 / np.sqrt(head_dim),
                 q_dtype=dtype, kv_dtype=dtype, o_dtype=dtype, meta={"block_mask": bm})
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (M, num_qo_heads, head_dim), dtype)
        w.k = _randn(g, (M, num_kv_heads, head_dim), dtype)
        w.v = _randn(g, (M, num_kv_heads, head_dim), dtype)
    return w


def element_mask_prefill(seed: int = 8, M: int = 8192, block: int = 64, density: float = 0.10,
                         keep: float = 0.75, num_qo_heads: int = 32, num_kv_heads: int = 8,
                         head_dim: int = 128, dtype: torch.dtype = torch.float16,
                         values: bool = True) -> Workload:
    """bsr_prefill's block pattern (all diagonal blocks plus i.i.d. Bernoulli(density)
    strictly-lower blocks, each row's blocks in random order) with an element mask in
    every block: each (query, key) entry kept i.i.d. with probability ``keep``; the
    diagonal blocks keep only entries with key <= query and always the key equal to
    the query, so every row sees a key.  Not causal (the masks take its place).

    ``meta["mask"]``: (nnz, R, C) bool, mask[p] for block indices[p];
    ``meta["packed_mask"]``: its flattening packed eight entries a byte, least
    significant bit first.
    """
    rng = np.random.default_rng(seed)
    MB = M // block
    rows = []
    for i in range(MB):
        lower = np.nonzero(rng.random(i) < density)[0]
        rows.append(rng.permutation(np.concatenate([lower, [i]]).astype(np.int64)))
    indptr, indices = _csr_from_rows(rows)
    mask = rng.random((int(indptr[-1]), block, block)) < keep
    tri = np.tril(np.ones((block, block), bool))
    for I in range(MB):
        for p in range(indptr[I], indptr[I + 1]):
            if indices[p] == I:
                mask[p] &= tri
                mask[p][np.arange(block), np.arange(block)] = True
    w = Workload("element_mask_prefill", indptr, indices, M, M, block, block, num_qo_heads,
                 num_kv_heads, head_dim, head_dim, False, 1.0 / np.sqrt(head_dim),
                 q_dtype=dtype, kv_dtype=dtype, o_dtype=dtype,
                 meta={"mask": mask, "packed_mask": np.packbits(mask.ravel(), bitorder="little")})
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (M, num_qo_heads, head_dim), dtype)
        w.k = _randn(g, (M, num_kv_heads, head_dim), dtype)
        w.v = _randn(g, (M, num_kv_heads, head_dim), dtype)
    return w


def _variable_sizes(rng, total: int, lo: int, hi: int) -> list:
    """Block sizes drawn uniformly from [lo, hi] until they cover ``total``; the
    last one is cut to fit."""
    sizes, acc = [], 0
    while acc < total:
        s = int(min(rng.integers(lo, hi + 1), total - acc))
        sizes.append(s)
        acc += s
    return sizes


def variable_block_prefill(seed: int = 9, M: int = 8192, min_block: int = 32, max_block: int = 160,
                           density: float = 0.15, causal: bool = False, num_qo_heads: int = 32,
                           num_kv_heads: int = 8, head_dim: int = 128, dtype: torch.dtype = torch.float16,
                           values: bool = True) -> Workload:
    """Variable block sizes with a pattern per kv head (VariableBlockSparseAttentionWrapper):
    each kv head cuts the M query rows and the M keys into blocks of sizes drawn
    uniformly from [min_block, max_block] (its own cuts for rows and for keys), padded
    with empty blocks to the longest head's count; each (row block, column block)
    pair is set i.i.d. with probability ``density``, and so is the column block
    holding a row block's first row (every row sees a key).

    ``meta["variable"]`` = (block_mask_map, block_row_sz, block_col_sz); the workload's
    R = C = 64 BSR arrays are the union of the fixed 64 x 64 blocks the map touches
    (a view for sizing only).
    """
    rng = np.random.default_rng(seed)
    rs = [_variable_sizes(rng, M, min_block, max_block) for _ in range(num_kv_heads)]
    cs = [_variable_sizes(rng, M, min_block, max_block) for _ in range(num_kv_heads)]
    MBv, NBv = max(map(len, rs)), max(map(len, cs))
    rsz = np.zeros((num_kv_heads, MBv), np.int32)
    csz = np.zeros((num_kv_heads, NBv), np.int32)
    bm = np.zeros((num_kv_heads, MBv, NBv), bool)
    for h in range(num_kv_heads):
        rsz[h, :len(rs[h])] = rs[h]
        csz[h, :len(cs[h])] = cs[h]
        bm[h, :len(rs[h]), :len(cs[h])] = rng.random((len(rs[h]), len(cs[h]))) < density
        col_start = np.cumsum([0] + cs[h])
        for a, r0 in enumerate(np.cumsum([0] + rs[h])[:-1]):
            bm[h, a, int(np.searchsorted(col_start, r0, side="right")) - 1] = True
    # union of touched 64 x 64 blocks
    blk = 64
    MB = -(-M // blk)
    touched = np.zeros((MB, MB), bool)
    for h in range(num_kv_heads):
        r0s, c0s = np.cumsum(np.r_[0, rsz[h]]), np.cumsum(np.r_[0, csz[h]])
        for a, b in zip(*np.nonzero(bm[h])):
            if rsz[h, a] and csz[h, b]:
                touched[r0s[a] // blk:(r0s[a + 1] - 1) // blk + 1, c0s[b] // blk:(c0s[b + 1] - 1) // blk + 1] = True
    indptr, indices = _csr_from_rows([np.nonzero(touched[i])[0] for i in range(MB)])
    w = Workload("variable_block_prefill", indptr, indices, M, M, blk, blk, num_qo_heads, num_kv_heads,
                 head_dim, head_dim, causal, 1.0 / np.sqrt(head_dim), q_dtype=dtype, kv_dtype=dtype,
                 o_dtype=dtype, meta={"variable": (bm, rsz, csz)})
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (M, num_qo_heads, head_dim), dtype)
        w.k = _randn(g, (M, num_kv_heads, head_dim), dtype)
        w.v = _randn(g, (M, num_kv_heads, head_dim), dtype)
    return w


def window_prefill(seed: int = 4, M: int = 32768, block: int = 128, window: int = 8,
                   stride: int = 16, num_qo_heads: int = 64, num_kv_heads: int = 8,
                   head_dim: int = 128, dtype: torch.dtype = torch.float16,
                   values: bool = True) -> Workload:
    """Row block i attends to {max(0, i - window) .. i} and {j <= i : j % stride == 0}; causal."""
    MB = M // block
    rows = []
    for i in range(MB):
        cols = set(range(max(0, i - window), i + 1))
        cols.update(range(0, i + 1, stride))
        rows.append(sorted(cols))
    indptr, indices = _csr_from_rows(rows)
    w = Workload("window_prefill", indptr, indices, M, M, block, block, num_qo_heads,
                 num_kv_heads, head_dim, head_dim, True, 1.0 / np.sqrt(head_dim),
                 q_dtype=dtype, kv_dtype=dtype, o_dtype=dtype)
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (M, num_qo_heads, head_dim), dtype)
        w.k = _randn(g, (M, num_kv_heads, head_dim), dtype)
        w.v = _randn(g, (M, num_kv_heads, head_dim), dtype)
    return w


def sparse_mla(seed: int = 5, num_tokens: int = 128, num_heads: int = 128,
               cache_rows: int = 65536, topk: int = 2048, min_ctx: int = 4096,
               max_ctx: int = 65536, latent: int = 512, rope: int = 64,
               values: bool = True) -> Workload:
    """Index-selected sparse MLA decode as BSR with R = C = 1 and one KV head.

    Query token t attends to ``topk`` cache rows drawn without replacement
    from [0, ctx_t), ctx_t uniform in [min_ctx, max_ctx], kept in drawn
    order.  The cache is float32 normals quantised with one per-tensor
    scale s = max|kv| / 448 to OCP fp8 e4m3 (torch.float8_e4m3fn); the
    dequant scale handed to the kernel is s for both K and V.
    """
    rng = np.random.default_rng(seed)
    D = latent + rope
    ctx = rng.integers(min_ctx, max_ctx + 1, size=num_tokens)
    rows = [rng.choice(int(c), size=topk, replace=False) for c in ctx]
    indptr, indices = _csr_from_rows(rows)
    w = Workload("sparse_mla", indptr, indices, num_tokens, cache_rows, 1, 1, num_heads, 1,
                 D, latent, False, 1.0 / np.sqrt(D), q_dtype=torch.bfloat16,
                 kv_dtype=torch.float8_e4m3fn, o_dtype=torch.bfloat16, v_aliases_k=True,
                 k_token_stride=D, v_token_stride=D, meta={"ctx_lens": ctx.astype(np.int64)})
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (num_tokens, num_heads, D), torch.bfloat16)
        kv32 = torch.randn(cache_rows, D, generator=g, dtype=torch.float32)
        s = float(kv32.abs().max()) / 448.0
        w.k = (kv32 / s).to(torch.float8_e4m3fn)
        w.v = None
        w.k_descale = s
        w.v_descale = s
    return w


def random_bsr(seed: int, M: int, N: int, R: int, C: int, num_qo_heads: int,
               num_kv_heads: int, head_dim: int = 128, density: float = 0.5,
               causal: bool = False, partial_lens: bool = False, empty_rows: bool = True,
               shuffle: bool = True, dtype: torch.dtype = torch.float16,
               garbage: float = 0.0, values: bool = True) -> Workload:
    """A small random BSR problem for parity and edge cases.

    ``partial_lens`` draws per-block valid lengths in [1, C];
    ``garbage`` > 0 overwrites the unused slots of partial blocks with
    +-garbage (finite) so that masking them is exercised; ``shuffle`` leaves
    the column indices of a row in random order.
    """
    assert N % C == 0
    rng = np.random.default_rng(seed)
    MB, NB = -(-M // R), N // C
    rows = []
    for i in range(MB):
        sel = np.nonzero(rng.random(NB) < density)[0]
        if empty_rows is False and sel.size == 0:
            sel = np.array([rng.integers(NB)])
        if shuffle:
            sel = rng.permutation(sel)
        rows.append(sel)
    indptr, indices = _csr_from_rows(rows)
    lens = rng.integers(1, C + 1, size=NB).astype(np.int32) if partial_lens else None
    w = Workload("random_bsr", indptr, indices, M, N, R, C, num_qo_heads, num_kv_heads,
                 head_dim, head_dim, causal, 1.0 / np.sqrt(head_dim), kv_block_lens=lens,
                 q_dtype=dtype, kv_dtype=dtype, o_dtype=dtype)
    if values:
        g = torch.Generator().manual_seed(seed)
        w.q = _randn(g, (M, num_qo_heads, head_dim), dtype)
        w.k = _randn(g, (N, num_kv_heads, head_dim), dtype)
        w.v = _randn(g, (N, num_kv_heads, head_dim), dtype)
        if lens is not None and garbage > 0:
            for J in range(NB):
                if lens[J] < C:
                    sl = slice(J * C + int(lens[J]), (J + 1) * C)
                    sign = torch.where(torch.rand(w.k[sl].shape, generator=g) < 0.5, -1.0, 1.0)
                    w.k[sl] = (sign * garbage).to(dtype)
                    w.v[sl] = (-sign * garbage).to(dtype)
    return w


def rope_cache(max_seq_len: int, theta: float = 10000.0, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """(max_seq_len, 64) rotary cache: column i < 32 = cos(p * theta^(-i/32)), column 32 + i = its sine."""
    inv = theta ** (-np.arange(32, dtype=np.float64) / 32.0)
    ang = np.arange(max_seq_len, dtype=np.float64)[:, None] * inv[None, :]
    return torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)).to(dtype)


def rope_quantize(seed: int = 10, nnz: int = 4096, num_heads: int = 128, max_seq_len: int = 32768,
                  is_neox: bool = True, scale: float = 64.0, cache_dtype: torch.dtype = torch.float32,
                  values: bool = True) -> dict:
    """The producer of the sparse-MLA inputs for a chunk of ``nnz`` tokens: bf16 q (nnz, H, 512 latent
    + 64 RoPE) and k (nnz, 512 + 64) standard normals, int32 positions uniform in
    [0, max_seq_len), an fp32 rotary cache (theta 10000), NeoX layout, quant scales ``scale``
    for q and kv (a unit normal's tail beyond 7 saturates)."""
    w = {"name": "rope_quantize", "nnz": nnz, "num_heads": num_heads, "max_seq_len": max_seq_len,
         "is_neox": is_neox, "quant_scale_q": scale, "quant_scale_kv": scale}
    if values:
        g = torch.Generator().manual_seed(seed)
        bf = lambda *shape: torch.randn(*shape, generator=g).to(torch.bfloat16)
        w.update(q_rope=bf(nnz, num_heads, 64), k_rope=bf(nnz, 64), q_nope=bf(nnz, num_heads, 512),
                 k_nope=bf(nnz, 512), cos_sin_cache=rope_cache(max_seq_len, dtype=cache_dtype),
                 pos_ids=torch.randint(0, max_seq_len, (nnz,), generator=g, dtype=torch.int32))
    return w


def indexer(seed: int = 5, num_tokens: int = 128, cache_rows: int = 65536, head_dim: int = 128,
            topk: int = 2048, page_size: int = 64, min_ctx: int = 4096, max_ctx: int = 65536,
            num_reqs: int = 1, dtype: torch.dtype = torch.bfloat16, integer: bool = False,
            values: bool = True) -> dict:
    """The indexer upstream of sparse MLA decode: ``num_tokens`` query rows (one index head of
    ``head_dim``) split evenly over ``num_reqs`` requests, each request owning
    cache_rows / num_reqs keys laid out over pages of ``page_size`` in a random page order.  Row t
    scores positions [0, ctx_t) of its request, ctx_t uniform in [min_ctx, max_ctx] (capped at the
    request's keys) and drawn first from the seed as in sparse_mla, and keeps ``topk`` of them.
    Values: standard normals in ``dtype``, or (``integer``) integers in [-4, 4], whose float32
    dot products are exact in any summation order."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(min_ctx, max_ctx + 1, size=num_tokens).astype(np.int64)
    per_req = cache_rows // num_reqs
    pages_per_req = (per_req + page_size - 1) // page_size
    num_pages = pages_per_req * num_reqs
    table = rng.permutation(num_pages).astype(np.int32).reshape(num_reqs, pages_per_req)
    bounds = np.linspace(0, num_tokens, num_reqs + 1).round().astype(np.int32)
    ctx = np.minimum(ctx, per_req).astype(np.int32)
    w = {"name": "indexer", "num_rows": num_tokens, "num_reqs": num_reqs, "head_dim": head_dim, "topk": topk,
         "page_size": page_size, "num_slots": num_pages * page_size, "block_table": table,
         "req_row_ptr": bounds, "ctx_len": ctx, "req_kv_len": np.full(num_reqs, per_req, np.int32),
         "max_ctx": int(ctx.max()) if num_tokens else 1}
    if values:
        g = torch.Generator().manual_seed(seed)
        if integer:
            w["q"] = torch.randint(-4, 5, (num_tokens, head_dim), generator=g).to(dtype)
            w["key_cache"] = torch.randint(-4, 5, (num_pages * page_size, head_dim), generator=g).to(dtype)
        else:
            w["q"] = torch.randn(num_tokens, head_dim, generator=g).to(dtype)
            w["key_cache"] = torch.randn(num_pages * page_size, head_dim, generator=g).to(dtype)
    return w


# Split-KV setting each workload is timed (and parity-checked at full size) with:
# 0 = automatic, 1 = no split.
BENCH_KV_SPLITS = {"worked_example": 1, "paged_decode": 0, "bsr_prefill": 1, "window_prefill": 1,
                   "sparse_mla": 1, "head_sparse_prefill": 1, "paged_decode_fp8": 0,
                   "element_mask_prefill": 1, "variable_block_prefill": 1, "bsr_prefill_fp8": 1}

WORKLOAD_NAMES = ["worked_example", "paged_decode", "bsr_prefill", "window_prefill", "sparse_mla",
                  "head_sparse_prefill", "paged_decode_fp8", "element_mask_prefill", "variable_block_prefill",
                  "bsr_prefill_fp8"]


def by_name(name: str, **kw) -> Workload:
    return {"worked_example": worked_example, "paged_decode": paged_decode,
            "bsr_prefill": bsr_prefill, "window_prefill": window_prefill,
            "sparse_mla": sparse_mla, "head_sparse_prefill": head_sparse_prefill,
            "paged_decode_fp8": paged_decode_fp8, "element_mask_prefill": element_mask_prefill,
            "variable_block_prefill": variable_block_prefill, "bsr_prefill_fp8": bsr_prefill_fp8}[name](**kw)
