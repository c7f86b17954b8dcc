"""CPU oracle for BSR block-sparse attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library.

What it computes is the plain definition the flashinfer.sparse documentation
gives for BlockSparseAttentionWrapper: the BSR structure (SciPy bsr_matrix
convention: indptr over row blocks, indices of column blocks, R x C blocks)
is an attention mask, and the result is ordinary masked softmax attention
(the worked example there compares the BSR result with dense attention under
the same boolean mask).  Every step is written out plainly in float64:

  O1  validate the structure              (plan(): indptr/indices, M, N, R, C)
  O2  expand BSR -> dense boolean mask    (plan(): MB = ceil_div(M, R), NB = N / C;
                                           kv_block_lens: valid tokens per KV block)
  O3  causal mask on top of the blocks    (plan(): causal; bottom-right aligned)
  O4  decode fp8 e4m3 storage             (OCP E4M3 / torch.float8_e4m3fn; per-tensor
                                           dequant scale as in the MATE sparse-MLA
                                           decode scale folding)
  O5  scores  S = sm_scale * q k^T        (plan(): sm_scale, default 1/sqrt(head_dim);
                                           GQA: qo head h reads kv head h // (Hq / Hkv))
  O6  softmax over unmasked keys, o = P v / l, lse = m + ln l
                                          (run(): o and the log-sum-exp of the logits)
  O7  merge of (o, lse) attention states  (flashinfer.cascade merge_state(s))
  O8  per-head structure                  (plan(): block_mask (heads, MB, NB) and
                                           q2k_indices / q2k_num; VariableBlockSparse-
                                           AttentionWrapper: each kv head its own pattern)
  O9  element masks inside blocks         (plan(): mask (nnz, R, C), packed_mask from
                                           flashinfer.quantization.packbits)
  O10 variable block sizes                (VariableBlockSparseAttentionWrapper.plan:
                                           block_mask_map, block_row_sz, block_col_sz)

Readings taken where the pages are silent:
  * lse is the natural log of sum(exp(sm_scale * q.k)) over unmasked keys;
  * a row with no unmasked key has o = 0 and lse = -inf;
  * causal masking keeps key j for query i iff j <= i + (N - M);
  * duplicate column indices within a row are rejected;
  * rows i >= M of a partial last row block do not exist;
  * a per-head structure given per qo head applies to that qo head (the
    library requires the qo heads of one kv head to agree, which makes this
    the same as using the first qo head of each group);
  * element mask p belongs to the block indices[p] of the BSR arrays as
    given (before any sorting), its entry [r, c] to query row I*R + r and key
    J*C + c; with an element mask the causal flag has no effect (plan()
    documents causal as ignored whenever a mask or packed mask is passed);
  * packed_mask holds the flattened (nnz, R, C) mask eight entries a byte,
    entry i in bit i % 8 (least significant first) of byte i // 8;
  * variable blocks: row block a of kv head h covers the block_row_sz[h, a]
    query rows after those of blocks 0..a-1 (columns likewise), the sizes of
    each head sum to the query / key counts, and causal masking (j <= i + N - M)
    applies on top of the block map.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "validate_bsr",
    "bsr_mask",
    "e4m3fn_decode",
    "fp8_dequant",
    "bf16_bits_decode",
    "masked_attention",
    "bsr_attention",
    "merge_states",
    "q2k_block_mask",
    "head_block_masks",
    "block_mask_attention",
    "unpack_block_masks",
    "element_mask",
    "element_mask_attention",
    "variable_block_masks",
    "variable_block_attention",
]


def validate_bsr(indptr, indices, M: int, N: int, R: int, C: int,
                 kv_block_lens=None) -> None:
    """O1: reject a malformed BSR structure with ValueError.

    flashinfer.sparse, BlockSparseAttentionWrapper.plan parameters: indptr has
    MB + 1 entries with MB = ceil_div(M, R); every index is below
    NB = N // C; N must be divisible by C; kv_block_lens has NB entries in
    [1, C].
    """
    indptr = np.asarray(indptr)
    indices = np.asarray(indices)
    if R < 1 or C < 1 or M < 0 or N < 0:
        raise ValueError("R, C must be >= 1 and M, N >= 0")
    if N % C != 0:
        raise ValueError("N must be divisible by C")
    MB = -(-M // R)
    NB = N // C
    if indptr.ndim != 1 or indptr.shape[0] != MB + 1:
        raise ValueError(f"indptr must have MB + 1 = {MB + 1} entries")
    if indptr[0] != 0 or np.any(np.diff(indptr) < 0) or indptr[-1] != indices.shape[0]:
        raise ValueError("indptr must start at 0, be non-decreasing and end at nnz")
    if indices.size and (indices.min() < 0 or indices.max() >= NB):
        raise ValueError("indices must lie in [0, NB)")
    for I in range(MB):
        row = indices[indptr[I]:indptr[I + 1]]
        if np.unique(row).size != row.size:
            raise ValueError(f"duplicate column index in row block {I}")
    if kv_block_lens is not None:
        lens = np.asarray(kv_block_lens)
        if lens.shape != (NB,) or lens.min(initial=1) < 1 or lens.max(initial=1) > C:
            raise ValueError("kv_block_lens must have NB entries in [1, C]")


def bsr_mask(indptr, indices, M: int, N: int, R: int, C: int, kv_block_lens=None,
             causal: bool = False, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O2 + O3: the boolean attention mask the BSR structure defines.

    Entry (i, j) is True iff query row i lies in row block I = i // R, some
    column index J of row block I has j in [J*C, J*C + len_J) with
    len_J = kv_block_lens[J] (or C when absent), and, when causal, also
    j <= i + (N - M).  ``rows`` restricts the expansion to the listed query
    rows (the result then has one mask row per listed row, in that order).
    """
    validate_bsr(indptr, indices, M, N, R, C, kv_block_lens)
    row_list = list(range(M)) if rows is None else [int(r) for r in rows]
    mask = np.zeros((len(row_list), N), dtype=bool)
    for out_row, i in enumerate(row_list):
        if not 0 <= i < M:
            raise ValueError("row out of range")
        I = i // R
        for p in range(int(indptr[I]), int(indptr[I + 1])):
            J = int(indices[p])
            length = C if kv_block_lens is None else int(kv_block_lens[J])
            mask[out_row, J * C:J * C + length] = True
        if causal:
            mask[out_row, max(0, i + (N - M) + 1):] = False
    return mask


def e4m3fn_decode(codes) -> np.ndarray:
    """O4: value of each OCP FP8 E4M3 ("fn": finite, no infinities) byte.

    Layout: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
    Exponent field 0 encodes subnormals m/8 * 2^-6; exponent 15 with mantissa
    7 is NaN (there is no infinity), every other code is (1 + m/8) * 2^(e-7).
    Largest finite magnitude: 448.
    """
    codes = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = codes & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def fp8_dequant(codes, head_scales=None, descale: float = 1.0) -> np.ndarray:
    """O4 with per-head scales: e4m3 codes (tokens, heads, dim) -> float64 values.

    value = decode(code) * descale * head_scales[head] (BlockSparseAttentionWrapper.run:
    scale_k / scale_v per kv head, scale_q per qo head, "per-head quantization"; the
    plan's per-tensor descale as in the MATE scale folding).  head_scales None = 1.
    """
    vals = e4m3fn_decode(codes) * float(descale)
    if head_scales is not None:
        sc = np.asarray(head_scales, dtype=np.float64)
        if sc.shape != (vals.shape[1],):
            raise ValueError("one scale per head")
        vals = vals * sc[None, :, None]
    return vals


def bf16_bits_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: bf16 is the top half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def masked_attention(q, k, v, mask, sm_scale: float):
    """O5 + O6: softmax attention of q over k/v restricted to ``mask``.

    q: (M, Hq, Dqk), k: (N, Hkv, Dqk), v: (N, Hkv, Dv), mask: (M, N) bool,
    all float64.  Grouped-query attention: qo head h uses kv head
    h // (Hq // Hkv) (flashinfer.sparse plan notes: num_qo_heads is a multiple
    of num_kv_heads).  Returns o (M, Hq, Dv) and lse (M, Hq), natural log.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    M, Hq, _ = q.shape
    N, Hkv, _ = k.shape
    Dv = v.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    group = Hq // Hkv
    o = np.zeros((M, Hq, Dv), dtype=np.float64)
    lse = np.full((M, Hq), -np.inf, dtype=np.float64)
    has_key = mask.any(axis=1)
    for h in range(Hq):
        kvh = h // group
        s = sm_scale * (q[:, h, :] @ k[:, kvh, :].T)          # (M, N)
        s = np.where(mask, s, -np.inf)
        m = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
        p = np.where(mask, np.exp(s - m[:, None]), 0.0)
        l = p.sum(axis=1)
        safe_l = np.where(has_key, l, 1.0)
        o[:, h, :] = np.where(has_key[:, None], (p @ v[:, kvh, :]) / safe_l[:, None], 0.0)
        lse[:, h] = np.where(has_key, m + np.log(safe_l), -np.inf)
    return o, lse


def bsr_attention(indptr, indices, M: int, N: int, R: int, C: int, q, k, v,
                  sm_scale: Optional[float] = None, causal: bool = False,
                  kv_block_lens=None, rows: Optional[Iterable[int]] = None):
    """BSR attention = masked attention under the expanded mask (O1-O6).

    q/k/v are float64 arrays (already decoded from their storage dtype with
    any dequant scale applied).  ``sm_scale`` defaults to 1/sqrt(head_dim)
    (plan(): sm_scale).  With ``rows``, only those query rows are computed;
    the returned o/lse then have one entry per listed row.
    """
    q = np.asarray(q, dtype=np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    row_list = None if rows is None else [int(r) for r in rows]
    mask = bsr_mask(indptr, indices, M, N, R, C, kv_block_lens, causal, row_list)
    if row_list is not None:
        q = q[row_list]
    return masked_attention(q, k, v, mask, sm_scale)


def merge_states(o_states, lse_states):
    """O7: merge attention states computed over disjoint key sets.

    flashinfer.cascade merge_state(s): given per-state outputs o_s (already
    normalised by their own softmax sums) and log-sum-exps lse_s of the same
    query over disjoint key sets, the state over the union is
        lse = log(sum_s exp(lse_s)),  o = sum_s exp(lse_s - lse) * o_s.
    States with lse_s = -inf (no keys) carry weight 0; if every state is
    empty the result is o = 0, lse = -inf.
    o_states: (S, ..., D), lse_states: (S, ...); float64.
    """
    o_states = np.asarray(o_states, dtype=np.float64)
    lse_states = np.asarray(lse_states, dtype=np.float64)
    top = lse_states.max(axis=0)
    any_keys = np.isfinite(top)
    top_safe = np.where(any_keys, top, 0.0)
    w = np.where(np.isfinite(lse_states), np.exp(lse_states - top_safe), 0.0)
    total = w.sum(axis=0)
    total_safe = np.where(any_keys, total, 1.0)
    contrib = np.where(np.isfinite(lse_states)[..., None], w[..., None] * o_states, 0.0)
    o = contrib.sum(axis=0) / total_safe[..., None]
    o = np.where(any_keys[..., None], o, 0.0)
    lse = np.where(any_keys, top_safe + np.log(total_safe), -np.inf)
    return o, lse


def q2k_block_mask(q2k_indices, q2k_num, NB: int) -> np.ndarray:
    """O8: direct selections -> block mask.

    flashinfer.sparse plan(): q2k_indices (heads, MB, topk) lists the selected
    KV blocks of each (head, query block); q2k_num (heads, MB) says how many
    leading entries of each row are valid (all topk when absent).  Entry
    (h, I, J) of the result is True iff J is among the first q2k_num[h, I]
    entries of row (h, I).  Entries must lie in [0, NB) and not repeat.
    """
    sel = np.asarray(q2k_indices)
    H, MB, topk = sel.shape
    num = np.full((H, MB), topk) if q2k_num is None else np.asarray(q2k_num)
    out = np.zeros((H, MB, NB), dtype=bool)
    for h in range(H):
        for I in range(MB):
            n = int(num[h, I])
            if not 0 <= n <= topk:
                raise ValueError("q2k_num entries must lie in [0, topk]")
            row = [int(x) for x in sel[h, I, :n]]
            if any(not 0 <= J < NB for J in row) or len(set(row)) != len(row):
                raise ValueError("selections must lie in [0, NB) without repeats")
            out[h, I, row] = True
    return out


def head_block_masks(block_mask, M: int, N: int, R: int, C: int, kv_block_lens=None,
                     causal: bool = False, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O8 with O2 + O3: per-head block mask -> dense boolean masks (heads, rows, N).

    Entry (h, i, j) is True iff block_mask[h, i // R, j // C] is set,
    j % C < len_J for J = j // C (kv_block_lens, or C when absent), and, when
    causal, j <= i + (N - M).
    """
    bm = np.asarray(block_mask).astype(bool)
    if C < 1 or R < 1 or N % C != 0:
        raise ValueError("R, C must be >= 1 and N divisible by C")
    MB, NB = -(-M // R), N // C
    if bm.ndim != 3 or bm.shape[1:] != (MB, NB):
        raise ValueError(f"block_mask must have shape (heads, {MB}, {NB})")
    row_list = list(range(M)) if rows is None else [int(r) for r in rows]
    lens = np.full(NB, C) if kv_block_lens is None else np.asarray(kv_block_lens)
    key_ok = (np.arange(N) % C) < lens[np.arange(N) // C]       # position inside its block's length
    out = np.zeros((bm.shape[0], len(row_list), N), dtype=bool)
    for h in range(bm.shape[0]):
        for out_row, i in enumerate(row_list):
            if not 0 <= i < M:
                raise ValueError("row out of range")
            blocks = bm[h, i // R]                               # (NB,) selected key blocks
            out[h, out_row] = np.repeat(blocks, C) & key_ok
            if causal:
                out[h, out_row, max(0, i + (N - M) + 1):] = False
    return out


def block_mask_attention(block_mask, M: int, N: int, R: int, C: int, q, k, v,
                         sm_scale: Optional[float] = None, causal: bool = False,
                         kv_block_lens=None, rows: Optional[Iterable[int]] = None):
    """Attention under a per-head block mask (O8, then O5 + O6 head by head).

    block_mask has num_kv_heads or num_qo_heads heads; qo head h uses mask
    h // (Hq / Hkv) in the first case (the heads of a kv group share its
    pattern) and mask h in the second.  Returns o (rows, Hq, Dv), lse (rows, Hq).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    group = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    row_list = None if rows is None else [int(r) for r in rows]
    masks = head_block_masks(block_mask, M, N, R, C, kv_block_lens, causal, row_list)
    if masks.shape[0] not in (Hkv, Hq):
        raise ValueError("block_mask must have num_kv_heads or num_qo_heads heads")
    if row_list is not None:
        q = q[row_list]
    o = np.zeros((q.shape[0], Hq, v.shape[2]))
    lse = np.zeros((q.shape[0], Hq))
    for h in range(Hq):
        kvh = h // group
        mh = masks[kvh] if masks.shape[0] == Hkv else masks[h]
        oh, lh = masked_attention(q[:, h:h + 1], k[:, kvh:kvh + 1], v[:, kvh:kvh + 1], mh, sm_scale)
        o[:, h], lse[:, h] = oh[:, 0], lh[:, 0]
    return o, lse


def unpack_block_masks(packed, nnz: int, R: int, C: int) -> np.ndarray:
    """O9: packed_mask -> the (nnz, R, C) boolean element masks.

    Entry i of the flattened mask is bit i % 8, least significant first, of
    byte i // 8 (the reading of packbits' bit order stated above); trailing
    bits of the last byte are ignored.
    """
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    n = nnz * R * C
    if packed.size < -(-n // 8):
        raise ValueError("packed_mask is shorter than nnz * R * C bits")
    i = np.arange(n)
    return ((packed[i // 8] >> (i % 8)) & 1).astype(bool).reshape(nnz, R, C)


def element_mask(indptr, indices, M: int, N: int, R: int, C: int, mask,
                 rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O9 + O2: dense boolean mask of a BSR structure with element masks.

    Entry (i, j) is True iff, for I = i // R, some p in indptr[I] ..
    indptr[I + 1] - 1 has indices[p] == j // C and mask[p, i % R, j % C].
    """
    validate_bsr(indptr, indices, M, N, R, C)
    mask = np.asarray(mask).astype(bool)
    nnz = int(indptr[-1])
    if mask.shape != (nnz, R, C):
        raise ValueError(f"mask must have shape ({nnz}, {R}, {C})")
    row_list = list(range(M)) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(row_list), N), dtype=bool)
    for out_row, i in enumerate(row_list):
        if not 0 <= i < M:
            raise ValueError("row out of range")
        I = i // R
        for p in range(int(indptr[I]), int(indptr[I + 1])):
            J = int(indices[p])
            out[out_row, J * C:(J + 1) * C] = mask[p, i % R]
    return out


def element_mask_attention(indptr, indices, M: int, N: int, R: int, C: int, mask, q, k, v,
                           sm_scale: Optional[float] = None, rows: Optional[Iterable[int]] = None):
    """Attention under BSR blocks with element masks (O9, then O5 + O6).

    ``mask`` is the (nnz, R, C) boolean array (unpack a packed_mask with
    unpack_block_masks first).  No causal flag: the mask replaces it.
    """
    q = np.asarray(q, dtype=np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    row_list = None if rows is None else [int(r) for r in rows]
    dense = element_mask(indptr, indices, M, N, R, C, mask, row_list)
    if row_list is not None:
        q = q[row_list]
    return masked_attention(q, k, v, dense, sm_scale)


def variable_block_masks(block_mask_map, block_row_sz, block_col_sz, causal: bool = False,
                         rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O10: variable-size block map -> dense boolean masks (kv heads, rows, N).

    Token row i of head h lies in the row block a whose row range (the sizes
    of blocks before it summed, plus its own) holds i, key j in column block b
    likewise; (h, i, j) is True iff block_mask_map[h, a, b], and, when causal,
    j <= i + (N - M).
    """
    bm = np.asarray(block_mask_map).astype(bool)
    rs = np.asarray(block_row_sz, dtype=np.int64)
    cs = np.asarray(block_col_sz, dtype=np.int64)
    if bm.ndim != 3 or rs.shape != bm.shape[:2] or cs.shape != (bm.shape[0], bm.shape[2]):
        raise ValueError("block_row_sz must be (heads, MB) and block_col_sz (heads, NB) for a (heads, MB, NB) map")
    if (rs < 0).any() or (cs < 0).any():
        raise ValueError("block sizes must be >= 0")
    M, N = int(rs[0].sum()), int(cs[0].sum())
    if (rs.sum(axis=1) != M).any() or (cs.sum(axis=1) != N).any():
        raise ValueError("every head's block sizes must sum to the same query / key counts")
    row_list = list(range(M)) if rows is None else [int(r) for r in rows]
    out = np.zeros((bm.shape[0], len(row_list), N), dtype=bool)
    for h in range(bm.shape[0]):
        row_block = np.repeat(np.arange(bm.shape[1]), rs[h])    # token row -> its row block
        col_block = np.repeat(np.arange(bm.shape[2]), cs[h])    # key -> its column block
        for out_row, i in enumerate(row_list):
            if not 0 <= i < M:
                raise ValueError("row out of range")
            out[h, out_row] = bm[h, row_block[i], col_block]
            if causal:
                out[h, out_row, max(0, i + (N - M) + 1):] = False
    return out


def variable_block_attention(block_mask_map, block_row_sz, block_col_sz, q, k, v,
                             sm_scale: Optional[float] = None, causal: bool = False,
                             rows: Optional[Iterable[int]] = None):
    """Attention under variable-size blocks, each kv head its own map (O10, then
    O5 + O6 head by head; the qo heads of a kv group share its map).
    q (M, Hq, D), k (N, Hkv, D), v (N, Hkv, Dv) float64; returns o, lse."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    group = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    row_list = None if rows is None else [int(r) for r in rows]
    masks = variable_block_masks(block_mask_map, block_row_sz, block_col_sz, causal, row_list)
    if masks.shape[0] != Hkv:
        raise ValueError("block_mask_map must have num_kv_heads heads")
    if row_list is not None:
        q = q[row_list]
    o = np.zeros((q.shape[0], Hq, v.shape[2]))
    lse = np.zeros((q.shape[0], Hq))
    for h in range(Hq):
        kvh = h // group
        oh, lh = masked_attention(q[:, h:h + 1], k[:, kvh:kvh + 1], v[:, kvh:kvh + 1], masks[kvh], sm_scale)
        o[:, h], lse[:, h] = oh[:, 0], lh[:, 0]
    return o, lse
