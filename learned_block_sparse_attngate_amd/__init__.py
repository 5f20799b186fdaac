"""MI355X (gfx950) SeerAttention hot path: AttnGate block scoring and mask
(with optional block-level RoPE), causal GQA block-sparse attention, dense
attention with the 2D-maxpooled ground-truth map, and the gate's
self-distillation step (KL loss and weight gradients), and the decode stage
(compressed K cache, per-token gate, block-sparse decode attention), and
varlen (packed, unpadded) prefill batches. The computation lives in libseer.so (HIP); this package is a
thin ctypes binding over its C ABI (include/seer.h)."""
from ._binding import (  # noqa: F401
    BLOCK, EXPORTED, LIB_PATH, SeerError, SeerShape, load_library, make_shape, nblocks,
    seer_gate_fwd, seer_gate_distill_bwd, seer_block_sparse_attn_fwd, seer_attn_maxpool_gt,
    seer_decode_compress_k, seer_decode_gate_fwd, seer_decode_attn_fwd, decode_attn_workspace_bytes,
    seer_decode_attn_fwd_noalloc, NOALLOC_SCRATCH_BYTES,
    SeerVarlen, make_varlen, varlen_map_offsets, seer_gate_varlen_fwd, seer_block_sparse_attn_varlen_fwd,
    seer_attn_maxpool_gt_varlen,
    gate_workspace_bytes, gate_varlen_workspace_bytes, distill_workspace_bytes, gt_workspace_bytes,
    attn_workspace_bytes, version,
    SEER_OK, SEER_ERR_INVALID_ARG, SEER_ERR_SHAPE, SEER_ERR_UNSUPPORTED, SEER_ERR_WORKSPACE, SEER_ERR_HIP,
    SEER_MASK_THRESHOLD, SEER_MASK_TOPK, SEER_F32, SEER_BF16,
)
