"""Pre-LayerNorm ViT encoder block, float64 numpy oracle (test infrastructure:
only tests/, the smoke check and the benchmark's CPU baseline may import it).

What the block computes, in the order the pages give it:

  1. h  = LN1(x)                                  SAM3 ``layer_norm_rows``;
                                                  SigLIP ``encoder_block``
  2. r  = x, or at a Hiera stage transition       Hiera plan, "Architecture
          r = pool4(h W_res^T + b_res)            Summary" (stage transitions)
  3. qkv = h W_qkv^T + b_qkv (row = [q | k | v]), SAM3 ``run_attn`` (fused);
          or three separate projections          SigLIP ``self_attention``
  4. axial RoPE on q and k (SAM3 trunk only)      SAM3 ``apply_rope``
  5. q <- pool4(q) at a transition                Hiera plan, "MaskUnitAttention"
  6. per frame, window and head:                  SAM3 ``run_attn`` (stable
          S = Q K^T * scale, P = softmax(S - rowmax), softmax); SigLIP
          O = P V                                 ``self_attention`` (non-causal)
  7. x1 = r + ctx W_o^T + b_o
  8. y  = x1 + GELU(LN2(x1) W_1^T + b_1) W_2^T + b_2   SigLIP ``encoder_block``;
                                                  SAM3 trunk block loop (LN2
                                                  reads a copy of the residual)

Each function states the passage it follows. The arithmetic is the plain
definition: one step per line, library matmul / erf / tanh / exp as the only
primitives, no blocking or fusion.

Pins (tests/test_oracle.py): LN closed form and torch's layer_norm; GELU-tanh
values printed by the SigLIP test ``gelu_tanh_reference_values``; GELU-erf
against Phi(u)*u from math.erf; softmax rows summing to 1 and shift
invariance; attention against a pure-Python double loop (``brute``) on all of
the tiny configuration, against torch's scaled_dot_product_attention, and the
identical-keys / single-key special cases; RoPE norm preservation, identity
at position 0, relative-position property; the block's RoPE step against a
pure-Python block that turns only the q and k parts (spatial and global), v
equal to the plain projection, and a position-independent rotation dropping
out of attention exactly; pool groups and window maps against the spatial
definitions. The whole block, every seam, is pinned against pure-Python loop
blocks (``brute``) on tiny inputs: mask-unit windows with fused qkv and
erf-GELU, global windows with separate q/k/v and tanh-GELU, spatial and
global windows with RoPE, and a stage transition with the pooled residual
and pooled queries; planted mistakes in the composition (a dropped residual,
LN2 reading the wrong tensor, RoPE on v) fail those comparisons
(``tests/test_oracle_mutations.py``). No page prints a block output for a
known input, so brute force on tiny inputs is the pin of the composition.
"""
import numpy as np
from scipy.special import erf as _erf

from . import index_maps


def layer_norm(x, gamma, beta, eps):
    """Row LayerNorm (SAM3 ``layer_norm_rows``): mean over the row, biased
    variance (divide by D), (x - mean) / sqrt(var + eps) * gamma + beta."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def linear(x, w, b):
    """PyTorch-style Linear: w is [out, in] row-major, y = x w^T + b
    (SigLIP ``Linear``; SAM3 ``matmat`` followed by ``add_bias``)."""
    return x @ np.asarray(w, dtype=np.float64).T + b


def gelu_erf(u):
    """Exact GELU, u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)) (SAM3 ``gelu_erf``,
    applied by ``gelu_slice`` after fc1)."""
    return 0.5 * u * (1.0 + _erf(u / np.sqrt(2.0)))


def gelu_tanh(u):
    """tanh-approximated GELU, 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))
    (SigLIP ``encoder_block`` uses ``nn::gelu_tanh``; its test
    ``gelu_tanh_reference_values`` prints values for this form)."""
    return 0.5 * u * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (u + 0.044715 * u ** 3)))


def softmax_rows(s):
    """Stable softmax over the last axis: subtract the row maximum before
    exponentiating (SAM3 ``run_attn``: trunk scores reach about 155, so the
    unshifted exponential would overflow)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def rope_rows_for(spec):
    """Table row used by each token of one frame (SAM3 ``vit_windows`` and the
    global trunk layers): in SPATIAL mode the token's in-window raster index,
    in GLOBAL mode its raster index in the grid."""
    H, W = spec["grid_h"], spec["grid_w"]
    n = np.arange(H * W)
    if spec["mode"] == "spatial":
        y, x = n // W, n % W
        return (y % spec["win_h"]) * spec["win_w"] + (x % spec["win_w"])
    return n


def apply_rope(t, table, rows, head_dim):
    """Axial RoPE on q or k (SAM3 ``apply_rope``): every head block of
    head_dim columns is rotated pair by pair; pair j is columns (2j, 2j+1),
    with (c, s) = table[row, j]: a' = a c - b s, b' = b c + a s. The table's
    first half of pairs carries the x (width) angle and the second half the y
    angle; that split is baked into the table, not into this rotation."""
    n, width = t.shape
    out = t.copy()
    for h0 in range(0, width, head_dim):
        for j in range(head_dim // 2):
            c = table[rows, j, 0]
            s = table[rows, j, 1]
            a = t[:, h0 + 2 * j]
            b = t[:, h0 + 2 * j + 1]
            out[:, h0 + 2 * j] = a * c - b * s
            out[:, h0 + 2 * j + 1] = b * c + a * s
    return out


def rope_qk(qkv, table, rows, dim, head_dim):
    """The block's RoPE step (SAM3 ``apply_rope``, called on the fused qkv
    rows of the trunk's attention): the q part (columns 0..dim-1) and the k
    part (dim..2*dim-1) are each rotated per head; the v part is left as it
    is. Returns a new array."""
    out = qkv.copy()
    out[:, :dim] = apply_rope(qkv[:, :dim], table, rows, head_dim)
    out[:, dim:2 * dim] = apply_rope(qkv[:, dim:2 * dim], table, rows, head_dim)
    return out


def pool4(z):
    """4x max-pool over the q_stride axis of the unrolled order (Hiera plan,
    "MaskUnitAttention" and the stage-transition line): output token m is the
    elementwise max of tokens m + s*N/4, s = 0..3. z is [N, C]."""
    g = index_maps.pool_groups(z.shape[0])
    return z[g].max(axis=1)


def windows_for(spec):
    """(q_tokens, kv_tokens) index pairs of one frame, per attention mode."""
    N = spec["grid_h"] * spec["grid_w"]
    mode = spec["mode"]
    if mode == "mask_unit":
        return index_maps.mask_unit_windows(N, spec["n_windows"], spec["q_stride"])
    if mode == "spatial":
        return [(w, w) for w in index_maps.spatial_windows(
            spec["grid_h"], spec["grid_w"], spec["win_h"], spec["win_w"])]
    nq = N // spec["q_stride"]
    return [(np.arange(nq), np.arange(N))]


def attention(q, k, v, windows, heads, scale):
    """Non-causal multi-head scaled-dot-product attention of one frame
    (SAM3 ``run_attn``; SigLIP ``self_attention`` with causal = false).

    q is [Nq, D], k and v are [N, D]; head t owns columns t*hd .. t*hd+hd-1.
    Inside each window and head: S = Q K^T * scale, P = softmax(S), O = P V,
    written into that head's columns of the window's query rows."""
    D = q.shape[1]
    hd = D // heads
    ctx = np.zeros_like(q)
    for qi, ki in windows:
        for t in range(heads):
            c = slice(t * hd, (t + 1) * hd)
            S = (q[qi, c] @ k[ki, c].T) * scale
            P = softmax_rows(S)
            ctx[np.ix_(qi, np.arange(t * hd, (t + 1) * hd))] = P @ v[ki, c]
    return ctx


def block_forward(x, w, spec):
    """Forward one pre-LN encoder block and return every intermediate.

    x: [B, N_in, D_in]; w: dict of float arrays (PyTorch Linear layout);
    spec: dict with batch, grid_h, grid_w, dim_in, dim_out, heads, mlp, mode
    ('global' | 'mask_unit' | 'spatial'), n_windows, win_h, win_w, q_stride
    (1 or 4), gelu ('erf' | 'tanh'), eps, scale (None: head_dim^-1/2),
    rope (bool), qkv ('fused' | 'separate').

    Returns a dict of float64 arrays, each [B, rows, cols]: h, qkv, q_pooled
    (transitions), r, ctx, attn_branch, x1, h2, u, mlp_branch, y."""
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    x = f64(x)
    B = x.shape[0]
    D, heads = spec["dim_out"], spec["heads"]
    hd = D // heads
    scale = spec.get("scale") or hd ** -0.5
    gelu = gelu_erf if spec["gelu"] == "erf" else gelu_tanh
    wins = windows_for(spec)
    seams = {k: [] for k in ("h", "qkv", "q_pooled", "r", "ctx", "attn_branch",
                             "x1", "h2", "u", "mlp_branch", "y")}
    for b in range(B):
        xb = x[b]
        h = layer_norm(xb, f64(w["ln1_g"]), f64(w["ln1_b"]), spec["eps"])
        if spec["q_stride"] == 4:
            r = pool4(linear(h, w["res_w"], f64(w["res_b"])))
        else:
            r = xb
        if spec.get("qkv", "fused") == "separate":
            qkv = np.concatenate([linear(h, w["q_w"], f64(w["q_b"])),
                                  linear(h, w["k_w"], f64(w["k_b"])),
                                  linear(h, w["v_w"], f64(w["v_b"]))], axis=1)
        else:
            qkv = linear(h, w["qkv_w"], f64(w["qkv_b"]))
        if spec.get("rope"):
            qkv = rope_qk(qkv, f64(w["rope"]), rope_rows_for(spec), D, hd)
        q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
        if spec["q_stride"] == 4:
            q = pool4(q)
            seams["q_pooled"].append(q)
        ctx = attention(q, k, v, wins, heads, scale)
        attn_branch = linear(ctx, w["o_w"], f64(w["o_b"]))
        x1 = r + attn_branch
        h2 = layer_norm(x1, f64(w["ln2_g"]), f64(w["ln2_b"]), spec["eps"])
        u = gelu(linear(h2, w["fc1_w"], f64(w["fc1_b"])))
        mlp_branch = linear(u, w["fc2_w"], f64(w["fc2_b"]))
        y = x1 + mlp_branch
        for name, val in (("h", h), ("qkv", qkv), ("r", r), ("ctx", ctx),
                          ("attn_branch", attn_branch), ("x1", x1), ("h2", h2),
                          ("u", u), ("mlp_branch", mlp_branch), ("y", y)):
            seams[name].append(val)
    return {k: np.stack(v) for k, v in seams.items() if v}


def block_forward_rows(x, w, spec, rows):
    """The same block, evaluated only at the output token rows ``rows`` of
    every frame (for full-size workloads, where all rows would take too long).

    Exactly the steps of ``block_forward``: LN1 and the projections run over
    every token (keys and values of every window are needed), attention and
    everything after it only for the chosen query rows. Returns the seams
    restricted to those rows: qkv/h rows are not returned; ctx, attn_branch,
    r, x1, h2, u, mlp_branch, y are [B, len(rows), cols]."""
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    x = f64(x)
    rows = np.asarray(rows, dtype=np.int64)
    D, heads = spec["dim_out"], spec["heads"]
    hd = D // heads
    scale = spec.get("scale") or hd ** -0.5
    gelu = gelu_erf if spec["gelu"] == "erf" else gelu_tanh
    wins = windows_for(spec)
    owner = {}
    for wi, (qi, _) in enumerate(wins):
        for pos, t in enumerate(qi):
            owner[int(t)] = (wi, pos)
    out = {k: [] for k in ("r", "ctx", "attn_branch", "x1", "h2", "u", "mlp_branch", "y")}
    for b in range(x.shape[0]):
        xb = x[b]
        h = layer_norm(xb, f64(w["ln1_g"]), f64(w["ln1_b"]), spec["eps"])
        if spec["q_stride"] == 4:
            r = pool4(linear(h, w["res_w"], f64(w["res_b"])))[rows]
        else:
            r = xb[rows]
        if spec.get("qkv", "fused") == "separate":
            qkv = np.concatenate([linear(h, w["q_w"], f64(w["q_b"])),
                                  linear(h, w["k_w"], f64(w["k_b"])),
                                  linear(h, w["v_w"], f64(w["v_b"]))], axis=1)
        else:
            qkv = linear(h, w["qkv_w"], f64(w["qkv_b"]))
        if spec.get("rope"):
            qkv = rope_qk(qkv, f64(w["rope"]), rope_rows_for(spec), D, hd)
        q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
        if spec["q_stride"] == 4:
            q = pool4(q)
        ctx = np.zeros((len(rows), D))
        for a, t in enumerate(rows):
            wi, _ = owner[int(t)]
            ki = wins[wi][1]
            ctx[a] = attention(q[[t]], k[ki], v[ki], [(np.array([0]), np.arange(len(ki)))],
                               heads, scale)[0]
        ab = linear(ctx, w["o_w"], f64(w["o_b"]))
        x1 = r + ab
        h2 = layer_norm(x1, f64(w["ln2_g"]), f64(w["ln2_b"]), spec["eps"])
        u = gelu(linear(h2, w["fc1_w"], f64(w["fc1_b"])))
        mb = linear(u, w["fc2_w"], f64(w["fc2_b"]))
        for name, val in (("r", r), ("ctx", ctx), ("attn_branch", ab), ("x1", x1), ("h2", h2),
                          ("u", u), ("mlp_branch", mb), ("y", x1 + mb)):
            out[name].append(val)
    return {k: np.stack(v) for k, v in out.items()}
