"""Helpers for GPU-vs-oracle parity tests: run a workload through the HIP
library, run the oracle on the same host bytes, compare element by element."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from paged_attention_bsr_amd import Plan

# Tolerances: |gpu - ref| <= ATOL + RTOL * |ref| elementwise on o; |dlse| <= LSE_TOL.
# fp16 storage: the stated fp16 bound.  fp8 KV (MLA shape): the stated 2e-2
# relative bound with the fp16 clause's absolute floor.  bf16 storage (no bound
# stated): the probabilities feed the PV product as bf16 (relative rounding
# 2^-9) and o is rounded to bf16 (2^-9), so |err| <= 2^-9 * max|v| + 2^-9 |o|
# plus fp32 accumulation noise; for unit-normal V (max |v| < 5) that is below
# 1e-2 + 1e-2 |ref|.
TOL_F16 = (2e-3, 1e-2)
TOL_BF16 = (1e-2, 1e-2)
TOL_FP8 = (2e-3, 2e-2)
LSE_TOL = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def plan_for(w, kv_splits=1, num_cus=0, trace=False) -> Plan:
    """The library plan of a workload; a per-head structure (w.meta["block_mask"], or
    w.meta["q2k"] = (q2k_indices, q2k_num)) replaces the shared BSR rows; element masks
    come from w.meta["packed_mask"] (else w.meta["mask"]); w.meta["variable"] =
    (block_mask_map, block_row_sz, block_col_sz) plans variable block sizes.  ``trace``
    plans with the trace build of the library (per-tile records)."""
    if "variable" in w.meta:
        bm, rs, cs = w.meta["variable"]
        return Plan.variable(bm, rs, cs, w.num_qo_heads, w.num_kv_heads, w.head_dim, causal=w.causal,
                             sm_scale=w.sm_scale, kv_splits=kv_splits, q_dtype=w.q_dtype, num_cus=num_cus,
                             trace=trace, **w.meta.get("grid", {}))
    extra = {}
    if "packed_mask" in w.meta:
        extra["packed_mask"] = w.meta["packed_mask"]
    elif "mask" in w.meta:
        extra["mask"] = w.meta["mask"]
    if "block_mask" in w.meta:
        extra["block_mask"] = w.meta["block_mask"]
    if "q2k" in w.meta:
        extra["q2k_indices"], extra["q2k_num"] = w.meta["q2k"]
    return Plan(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                head_dim_vo=w.head_dim_vo, causal=w.causal, sm_scale=w.sm_scale,
                kv_splits=kv_splits, kv_block_lens=w.kv_block_lens, q_dtype=w.q_dtype,
                kv_dtype=w.kv_dtype, o_dtype=w.o_dtype, k_descale=w.k_descale,
                v_descale=w.v_descale, k_token_stride=w.k_token_stride,
                v_token_stride=w.v_token_stride, num_cus=num_cus, trace=trace, **extra)


def to_device(w, device="cuda"):
    q = w.q.to(device)
    k = w.k.to(device)
    v = None if w.v_aliases_k else w.v.to(device)
    return q, k, v


def scales_for(w, device="cuda"):
    """Per-head run() scales of a workload as device tensors (None where absent)."""
    return {f"scale_{n}": (torch.from_numpy(w.meta[f"scale_{n}"]).to(device) if f"scale_{n}" in w.meta else None)
            for n in ("q", "k", "v")}


def run_gpu(w, kv_splits=1, plan=None, dev=None):
    p = plan if plan is not None else plan_for(w, kv_splits)
    q, k, v = dev if dev is not None else to_device(w)
    o, lse = p.run(q, k, v, **scales_for(w))
    torch.cuda.synchronize()
    return o, lse


def oracle_inputs(w):
    """float64 q, k, v as the oracle sees them (fp8 decoded by the oracle itself)."""
    q = w.q.double().numpy()
    if "scale_q" in w.meta:   # a per-qo-head logit multiplier is a scale of q
        q = q * w.meta["scale_q"].astype(np.float64)[None, :, None]
    if w.kv_dtype == torch.float8_e4m3fn and not w.v_aliases_k:
        k = oracle.fp8_dequant(w.k.view(torch.uint8).numpy(), w.meta.get("scale_k"), w.k_descale)
        v = oracle.fp8_dequant(w.v.view(torch.uint8).numpy(), w.meta.get("scale_v"), w.v_descale)
    elif w.kv_dtype == torch.float8_e4m3fn:
        codes = w.k.view(torch.uint8).numpy()
        kf = oracle.e4m3fn_decode(codes)
        k = (kf * w.k_descale)[:, None, :]
        v = (kf[:, :w.head_dim_vo] * w.v_descale)[:, None, :]
    else:
        k = w.k.double().numpy()
        v = w.v.double().numpy()
    return q, k, v


def oracle_result(w, rows=None, inputs=None):
    q, k, v = oracle_inputs(w) if inputs is None else inputs
    if "variable" in w.meta:
        bm, rs, cs = w.meta["variable"]
        return oracle.variable_block_attention(bm, rs, cs, q, k, v, sm_scale=w.sm_scale, causal=w.causal, rows=rows)
    if "mask" in w.meta or "packed_mask" in w.meta:
        mask = (w.meta["mask"] if "mask" in w.meta
                else oracle.unpack_block_masks(w.meta["packed_mask"], w.nnz, w.R, w.C))
        return oracle.element_mask_attention(w.indptr, w.indices, w.M, w.N, w.R, w.C, mask, q, k, v,
                                             sm_scale=w.sm_scale, rows=rows)
    if "block_mask" in w.meta or "q2k" in w.meta:
        bm = (w.meta["block_mask"] if "block_mask" in w.meta
              else oracle.q2k_block_mask(w.meta["q2k"][0], w.meta["q2k"][1], w.NB))
        return oracle.block_mask_attention(bm, w.M, w.N, w.R, w.C, q, k, v, sm_scale=w.sm_scale,
                                           causal=w.causal, kv_block_lens=w.kv_block_lens, rows=rows)
    return oracle.bsr_attention(w.indptr, w.indices, w.M, w.N, w.R, w.C, q, k, v, sm_scale=w.sm_scale,
                                causal=w.causal, kv_block_lens=w.kv_block_lens, rows=rows)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, tol, what=""):
    """Assert elementwise closeness; returns (max abs err, max lse err)."""
    o = o_gpu.float().cpu().double().numpy()
    atol, rtol = tol
    err = np.abs(o - o_ref)
    bound = atol + rtol * np.abs(o_ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs out of tolerance; "
                             f"max err {err.max():.3e}; first at {idx}: gpu {o[tuple(idx[0])]:.6f} "
                             f"ref {o_ref[tuple(idx[0])]:.6f}")
    assert not np.isnan(o).any(), f"{what}: NaN in output"
    lse_err = 0.0
    if lse_gpu is not None:
        l = lse_gpu.cpu().double().numpy()
        inf_ref = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(l), inf_ref), f"{what}: -inf lse pattern differs"
        if (~inf_ref).any():
            lse_err = float(np.abs(l[~inf_ref] - lse_ref[~inf_ref]).max())
            assert lse_err <= LSE_TOL, f"{what}: lse error {lse_err:.3e}"
    return float(err.max()) if err.size else 0.0, lse_err


def tol_for(w):
    if w.kv_dtype == torch.float8_e4m3fn:
        # the fp8 bound with the output type's own rounding floor for 16-bit outputs
        return TOL_FP8 if w.o_dtype != torch.bfloat16 or w.v_aliases_k else TOL_BF16
    return TOL_BF16 if w.q_dtype == torch.bfloat16 else TOL_F16
