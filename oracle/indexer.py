"""CPU oracle for the sparse-attention indexer: scores and exact Top-K (test infrastructure only).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library.

What it computes follows the FlashInfer sparse API page (flashinfer.sparse
0.7.4, section "SDSA Indexer"), the indexer upstream of index-selected
sparse MLA decode (whose int32 physical-token index lists it produces):

  I1  indexer_scores: FP32 scores of query rows against their request's paged
      keys.  The indexer has one query head and no head weights, so a score
      is the dot product of the row's query vector with the key vector;
  I2  exact Top-K: each query row keeps the K keys of highest score
      (top_k_from_candidates writes every row's exact Top-K from the
      candidates and the tied keys the selection stored, so a tie at the
      K-th score has to be resolved by a rule).

Readings taken where the pages are silent:
  * a request's key position p lives in cache row
    block_table[r][p // page_size] * page_size + p % page_size (the paged
    layout of the pages' KV caches); a row with context length n sees the
    positions 0 .. n - 1 of its request;
  * "FP32 scores": the exact dot product rounded once to float32 (here: the
    products and their sum in float64, which is exact for the bf16 inputs of
    the tests up to the final rounding whenever the sum fits 53 bits);
  * ties: among equal float32 scores the lower position wins (-0 and +0
    are equal scores);
  * output: the K kept keys' physical cache rows in ascending position order;
    a row with n < K keys keeps all n and pads with -1.
"""
from __future__ import annotations

import numpy as np


def key_slots(block_table: np.ndarray, page_size: int, req: int, n: int) -> np.ndarray:
    """Physical cache rows of positions 0 .. n - 1 of request `req` (reading: paged layout)."""
    p = np.arange(n, dtype=np.int64)
    return block_table[req, p // page_size].astype(np.int64) * page_size + p % page_size


def indexer_scores(q: np.ndarray, key_cache: np.ndarray, block_table: np.ndarray, page_size: int,
                   req_row_ptr: np.ndarray, ctx_len: np.ndarray) -> list:
    """I1: per query row, the float32 scores of positions 0 .. ctx_len[row] - 1 of its request.

    q: [num_rows, D]; key_cache: [num_slots, D] (any float dtype; values are
    used exactly); req_row_ptr: rows of request r are req_row_ptr[r] ..
    req_row_ptr[r + 1] - 1.  Returns a list of float32 arrays, one per row."""
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(key_cache, dtype=np.float64)
    out = [None] * q64.shape[0]
    for r in range(len(req_row_ptr) - 1):
        for row in range(int(req_row_ptr[r]), int(req_row_ptr[r + 1])):
            n = int(ctx_len[row])
            slots = key_slots(block_table, page_size, r, n)
            out[row] = (k64[slots] @ q64[row]).astype(np.float32)
    return out


def topk_positions(scores: np.ndarray, k: int) -> np.ndarray:
    """I2: positions of the K highest float32 scores, ties to the lower position,
    returned in ascending position order (all positions when there are <= K)."""
    s = np.asarray(scores, dtype=np.float32).astype(np.float64)  # -0 == +0 as values
    n = s.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -s))   # primary: score descending; then position ascending
    return np.sort(order[:k])


def indexer_topk(q: np.ndarray, key_cache: np.ndarray, block_table: np.ndarray, page_size: int,
                 req_row_ptr: np.ndarray, ctx_len: np.ndarray, k: int) -> np.ndarray:
    """I1 + I2: int64 [num_rows, K] physical cache rows of each row's exact Top-K keys,
    ascending by position, padded with -1."""
    scores = indexer_scores(q, key_cache, block_table, page_size, req_row_ptr, ctx_len)
    out = np.full((len(scores), k), -1, dtype=np.int64)
    for r in range(len(req_row_ptr) - 1):
        for row in range(int(req_row_ptr[r]), int(req_row_ptr[r + 1])):
            pos = topk_positions(scores[row], k)
            out[row, :len(pos)] = key_slots(block_table, page_size, r, int(ctx_len[row]))[pos]
    return out
