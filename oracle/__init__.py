"""CPU oracle for BSR block-sparse attention (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the HIP library and its Python binding never do.
"""
from .bsr_attention import (  # noqa: F401
    validate_bsr,
    bsr_mask,
    e4m3fn_decode,
    fp8_dequant,
    bf16_bits_decode,
    masked_attention,
    bsr_attention,
    merge_states,
    q2k_block_mask,
    head_block_masks,
    block_mask_attention,
    unpack_block_masks,
    element_mask,
    element_mask_attention,
    variable_block_masks,
    variable_block_attention,
)
from .rope_quantize import (  # noqa: F401
    e4m3fn_encode,
    rope_fp32,
    mla_rope_quantize_fp8,
)
from .indexer import (  # noqa: F401
    key_slots,
    indexer_scores,
    topk_positions,
    indexer_topk,
)
