"""Hiera stage stack, float64 numpy oracle (test infrastructure: only tests/,
the smoke check and the benchmark's CPU baseline may import it).

The Hiera plan ("Phase 4: Hiera Backbone MLX Port", "Architecture Summary"
and "Implementation Plan" item 8) assembles the backbone as: Unroll the
token grid once, run the 24 blocks in order (the first block of stages 1-3
is a transition whose 2x2 query max-pool cuts the tokens 4x), and at each
stage end Reroll the current tokens back to a spatial [B, H, W, C] map.
Patch embedding and the positional embedding come before this and are not
part of it: the stack starts from tokens in raster order.

Each 2x2 pooling consumes one level of the unrolled order (the pooled order
is the (L-1)-level unroll of the half-size grid, see ``index_maps``), so a
feature map taken after k transitions is rerolled with L - k levels.

A tower without unrolling (levels 0) is the same loop: the SAM3 trunk runs
its LayerNorm ``ln_pre`` and then the blocks (SAM3 page, trunk block loop);
the SigLIP tower runs the blocks and then ``post_layernorm`` (SigLIP page,
``forward_frame``) -- ``tower_forward``.

Pins (tests/test_oracle.py): the 512x512 shape contract of the plan
("Sub-phase 4d": 128x128x112, 64x64x224, 32x32x448, 16x16x896); a stack of
global blocks without pooling equals the same blocks on raster-order tokens
(global attention does not see the token order, so unroll and reroll must
cancel exactly); a one-block stack equals unroll -> block -> reroll;
``tower_forward``'s post_layernorm against the pure-Python LayerNorm of the
last block's output and its gamma 1 / beta 0 closed form, and its ln_pre
against the pure-Python LayerNorm feeding the first block.
"""
import numpy as np

from oracle import block as ob
from oracle import index_maps as im


def stack_forward(x, blocks, specs, levels, taps):
    """x [B, H*W, D_0] raster order; blocks: per-block weight dicts; specs:
    per-block specs (block i's output grid is block i+1's input grid);
    levels: unroll levels; taps: block indices whose outputs are returned.
    Returns the rerolled features, each [B, H_k*W_k, D_k] in raster order."""
    H, W = specs[0]["grid_h"], specs[0]["grid_w"]
    t = im.unroll(np.asarray(x, dtype=np.float64), H, W, levels)
    feats = []
    for i, (w, sp) in enumerate(zip(blocks, specs)):
        t = ob.block_forward(t, w, sp)["y"]
        if sp["q_stride"] == 4:
            levels -= 1
            H, W = H // 2, W // 2
        if i in taps:
            feats.append(im.reroll(t, H, W, levels))
    return feats


def tower_forward(x, blocks, specs, pre_ln=None, post_ln=None, eps=1e-6):
    """Blocks applied in order to raster-order tokens, with an optional
    LayerNorm (gamma, beta) before the first block and after the last."""
    t = np.asarray(x, dtype=np.float64)
    if pre_ln is not None:
        t = ob.layer_norm(t, np.asarray(pre_ln[0], dtype=np.float64), np.asarray(pre_ln[1], dtype=np.float64), eps)
    (t,) = stack_forward(t, blocks, specs, 0, [len(specs) - 1])
    if post_ln is not None:
        t = ob.layer_norm(t, np.asarray(post_ln[0], dtype=np.float64), np.asarray(post_ln[1], dtype=np.float64), eps)
    return t
