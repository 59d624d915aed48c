"""fp64 CPU oracle for DSV-style dynamic block-sparse attention -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may use it.
The product (the HIP library and its Python binding) never imports it.
"""
from .dsa_oracle import (  # noqa: F401
    Geometry, pooled_features, block_scores, predict_head, select_row, select_head, kept_keys,
    attn_tile, attn_fwd_head, attn_bwd_tile, attn_bwd_head, attn_bwd_key_block,
    predict, select, attn_fwd, attn_bwd,
    tile_means, pooled_logits, predictor_loss_head, predictor_grad_head, predictor_grad,
    rope_sections, rope_angles, rope3d,
)
