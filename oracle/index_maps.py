"""Token orders and window membership for the encoder block (oracle side; test
infrastructure: only tests/, the smoke check and the benchmark's CPU baseline
may import it).

Integer index arithmetic only. Every map here is compared bit-exactly with
the HIP permute kernels and with the window addressing of the HIP attention
kernel.

Hiera unroll/reroll. The Hiera plan ("Phase 4: Hiera Backbone MLX Port",
"Architecture Summary" and "Sub-phase 4a") says only that Unroll permutes the
tokens so that mask-unit attention can work on them, and that Reroll undoes
the permutation back to a spatial [B, H, W, C] map; the order itself is not
printed. The reading taken here: at each of L levels, the 2x2 offset of a
token inside its 2x2 cell is moved out in front of the coarser grid, finest
level first, so that after L levels the token at spatial (y, x) sits at

    n = (((s_0 * 4 + s_1) * 4 + ...) * 4 + s_{L-1}) * (H_L * W_L)
        + (y >> L) * W_L + (x >> L),
    s_k = 2 * ((y >> k) & 1) + ((x >> k) & 1),   H_L = H / 2^L, W_L = W / 2^L.

Consequences that the tests check (they tie the reading to what the plan
states): the map is a bijection; ``n mod (H_L * W_L)`` is the index of the
2^L x 2^L spatial block (the mask unit: 8x8 at L = 3, hence 64-token windows
at stage 0 and 16-token windows after one 2x2 pooling); the four tokens
``m + s * N/4`` (s = 0..3) are one 2x2 spatial cell, so a max over them is a
2x2 max-pool that cuts the tokens 4x; and the pooled order is again the
(L-1)-level unroll of the half-size grid.
"""
import numpy as np


def unroll_positions(H, W, L):
    """Unrolled position n of every spatial token, as an [H*W] int64 array
    indexed by the row-major spatial index y*W + x.

    Implements the level loop described in the module header: at each level
    the token's 2x2 offset is appended to an outer (batch-like) index and the
    coordinates are halved."""
    if H % (1 << L) or W % (1 << L):
        raise ValueError("grid %dx%d not divisible by 2^%d" % (H, W, L))
    HL, WL = H >> L, W >> L
    pos = np.empty(H * W, dtype=np.int64)
    for y in range(H):
        for x in range(W):
            outer, yy, xx = 0, y, x
            for _ in range(L):
                outer = outer * 4 + 2 * (yy & 1) + (xx & 1)
                yy >>= 1
                xx >>= 1
            pos[y * W + x] = outer * (HL * WL) + yy * WL + xx
    return pos


def unroll(x, H, W, L):
    """Spatial row-major tokens [B, H*W, C] -> unrolled order (Hiera Unroll,
    as read in the module header)."""
    pos = unroll_positions(H, W, L)
    out = np.empty_like(x)
    out[:, pos, :] = x
    return out


def reroll(x, H, W, L):
    """Unrolled order [B, H*W, C] -> spatial row-major (the inverse map:
    Hiera Reroll / undo_windowing, as read in the module header)."""
    pos = unroll_positions(H, W, L)
    return x[:, pos, :]


def mask_unit_windows(n_tokens, n_windows, q_stride):
    """Hiera MaskUnitAttention windows on unrolled tokens.

    Window w holds the kv tokens n with n mod n_windows == w, and the
    (pooled, when q_stride = 4) query tokens m with m mod n_windows == w.
    Returns a list of (q_tokens, kv_tokens) int64 arrays, windows in order."""
    if n_tokens % n_windows or (n_tokens // q_stride) % n_windows:
        raise ValueError("tokens not divisible into windows")
    nq = n_tokens // q_stride
    return [(np.arange(w, nq, n_windows, dtype=np.int64),
             np.arange(w, n_tokens, n_windows, dtype=np.int64))
            for w in range(n_windows)]


def spatial_windows(H, W, win_h, win_w):
    """SAM3 trunk windows (sam3.rs, ``vit_windows``): the row-major grid is
    cut into win_h x win_w blocks, taken in raster order; inside a block the
    tokens are in raster order too, so in-window index y*win_w + x is also the
    row of the windowed RoPE table. Returns a list of token-index arrays."""
    if H % win_h or W % win_w:
        raise ValueError("grid not divisible by window")
    wins = []
    for wy in range(H // win_h):
        for wx in range(W // win_w):
            idx = [(wy * win_h + y) * W + wx * win_w + x
                   for y in range(win_h) for x in range(win_w)]
            wins.append(np.array(idx, dtype=np.int64))
    return wins


def pool_groups(n_tokens):
    """Rows pooled together by the 4x query/residual max-pool, per output
    token m: [m, m + N/4, m + 2N/4, m + 3N/4] (the q_stride axis of the
    unrolled order; see the module header). Returns an [N/4, 4] array."""
    if n_tokens % 4:
        raise ValueError("token count not divisible by 4")
    q = n_tokens // 4
    return np.stack([np.arange(q) + s * q for s in range(4)], axis=1).astype(np.int64)
