"""fp64 CPU oracle (test infrastructure only; never imported by the library)."""
from .seer_oracle import (  # noqa: F401
    BLOCK, as_f64, n_blocks, pool_q, pool_k, block_rope, gate_scores, gate_distill, threshold_mask, topk_mask,
    attention_rows, attention, maxpool_gt_rows, maxpool_gt,
    decode_kcomp, decode_gate_scores, decode_threshold_mask, decode_topk_mask, decode_attention, decode_gt,
)
