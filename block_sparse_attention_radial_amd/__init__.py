"""Radial Attention forward pass for MI355X (gfx950).

    from block_sparse_attention_radial_amd import build_mask, attn_fwd
    mask = build_mask(frames, tokens_per_frame, w0).to("cuda")
    o = attn_fwd(q, k, v, mask)            # q, k, v: bf16 [B, H, n, D] on the GPU

Variants: attn_fwd(..., element=True) applies the rule to single entries inside the
active blocks (from stored decisions once mask.with_element_table() has built them on
the GPU); build_mask(..., grid_w=W) takes the 2-D grid distance on frames of W
columns; rule_mask(...) lets the kernel derive the blocks itself (no CSR);
attention(...) adds the backward pass for autograd; build_varlen_mask + attn_fwd_varlen
(attention_varlen with autograd) run a packed batch of videos of different lengths.

The mask builder and the kernels live in libradial.so (C ABI: include/radial_attn.h),
built in-tree by `python -m block_sparse_attention_radial_amd.build`.
"""
from .api import (BLOCK, Mask, RadialAttentionFunction, RadialAttentionVarlenFunction,
                  RadialError, RuleMask, VarlenMask, VarlenRuleMask, attention, attention_varlen,
                  attn_bwd, attn_bwd_noalloc,
                  attn_bwd_varlen, attn_fwd, attn_fwd_varlen, build_element_table, build_mask,
                  build_pairs,
                  build_varlen_mask, concat_masks, dense_mask, error_string, lib, mask_dims,
                  rule_mask)

__all__ = ["BLOCK", "Mask", "RadialAttentionFunction", "RadialAttentionVarlenFunction",
           "RadialError", "RuleMask", "VarlenMask", "VarlenRuleMask", "attention",
           "attention_varlen", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_varlen", "attn_fwd", "attn_fwd_varlen", "build_element_table", "build_mask", "build_pairs",
           "build_varlen_mask", "concat_masks", "dense_mask", "error_string", "lib",
           "mask_dims", "rule_mask"]
