"""Pure-Python loop versions of the block's steps, for tiny shapes only
(test infrastructure, imported by tests/ only; pins for ``oracle.block``).

No numpy arithmetic here: every sum, product, maximum and exponential is a
Python float operation on one scalar, so an indexing or transposition slip in
the vectorised oracle cannot be repeated here by the same library call.
Follows the same passages as ``oracle.block`` (SAM3 ``layer_norm_rows``,
``run_attn``; SigLIP ``encoder_block``; Hiera plan "MaskUnitAttention").
"""
import math


def layer_norm(rows, gamma, beta, eps):
    out = []
    for r in rows:
        d = len(r)
        mean = sum(r) / d
        var = sum((v - mean) * (v - mean) for v in r) / d
        inv = 1.0 / math.sqrt(var + eps)
        out.append([(r[i] - mean) * inv * gamma[i] + beta[i] for i in range(d)])
    return out


def linear(rows, w, b):
    """y[i][o] = sum_k rows[i][k] * w[o][k] + b[o] (w is [out, in])."""
    return [[sum(r[k] * w[o][k] for k in range(len(r))) + b[o]
             for o in range(len(w))] for r in rows]


def gelu_erf(v):
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def gelu_tanh(v):
    return 0.5 * v * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3)))


def attention_head(q_rows, k_rows, v_rows, scale):
    """One (window, head): for each query, scores against every key, stable
    softmax, weighted sum of the values."""
    out = []
    for q in q_rows:
        s = [sum(q[d] * k[d] for d in range(len(q))) * scale for k in k_rows]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        p = [v / z for v in e]
        out.append([sum(p[j] * v_rows[j][d] for j in range(len(v_rows)))
                    for d in range(len(v_rows[0]))])
    return out


def block_forward_mask_unit(x, w, n_windows, heads, eps, gelu="erf"):
    """Whole block for one frame with mask-unit windows, q_stride 1, fused
    qkv, no RoPE (the tiny configuration's shape). x is a list of token rows
    in unrolled order; w holds nested lists. Returns (ctx, y)."""
    n = len(x)
    h = layer_norm(x, w["ln1_g"], w["ln1_b"], eps)
    qkv = linear(h, w["qkv_w"], w["qkv_b"])
    D = len(qkv[0]) // 3
    hd = D // heads
    scale = 1.0 / math.sqrt(hd)
    ctx = [[0.0] * D for _ in range(n)]
    for win in range(n_windows):
        toks = list(range(win, n, n_windows))
        for t in range(heads):
            lo = t * hd
            qr = [qkv[i][lo:lo + hd] for i in toks]
            kr = [qkv[i][D + lo:D + lo + hd] for i in toks]
            vr = [qkv[i][2 * D + lo:2 * D + lo + hd] for i in toks]
            o = attention_head(qr, kr, vr, scale)
            for a, i in enumerate(toks):
                ctx[i][lo:lo + hd] = o[a]
    ab = linear(ctx, w["o_w"], w["o_b"])
    x1 = [[x[i][c] + ab[i][c] for c in range(D)] for i in range(n)]
    h2 = layer_norm(x1, w["ln2_g"], w["ln2_b"], eps)
    g = gelu_erf if gelu == "erf" else gelu_tanh
    u = [[g(v) for v in row] for row in linear(h2, w["fc1_w"], w["fc1_b"])]
    mb = linear(u, w["fc2_w"], w["fc2_b"])
    y = [[x1[i][c] + mb[i][c] for c in range(D)] for i in range(n)]
    return ctx, y


def rotate_pairs(vec, cs):
    """One head's q or k vector turned pair by pair (SAM3 ``apply_rope``):
    pair j is elements (2j, 2j+1) and turns by the angle whose (cos, sin) is
    cs[j]; (a, b) -> (a cos - b sin, a sin + b cos)."""
    out = list(vec)
    for j, (c, s) in enumerate(cs):
        a, b = vec[2 * j], vec[2 * j + 1]
        out[2 * j] = a * c - b * s
        out[2 * j + 1] = a * s + b * c
    return out


def block_forward_rope(x, w, grid_h, grid_w, win_h, win_w, heads, eps, table):
    """Whole block for one frame of raster-order tokens with fused qkv,
    axial RoPE on q and k and erf-GELU (the SAM3 trunk's block), q_stride 1.
    win_h = win_w = 0 means one global window and table rows are grid raster
    indices; otherwise windows are the win_h x win_w tiles of the grid and a
    token's table row is its raster index inside its tile. Returns
    (qkv_after_rope, ctx, y) as nested lists."""
    n = grid_h * grid_w
    h = layer_norm(x, w["ln1_g"], w["ln1_b"], eps)
    qkv = linear(h, w["qkv_w"], w["qkv_b"])
    D = len(qkv[0]) // 3
    hd = D // heads
    spatial = win_h > 0
    win_of, row_of = [], []
    for i in range(n):
        gy, gx = i // grid_w, i % grid_w
        if spatial:
            win_of.append((gy // win_h, gx // win_w))
            row_of.append((gy % win_h) * win_w + (gx % win_w))
        else:
            win_of.append((0, 0))
            row_of.append(i)
    rot = []
    for i in range(n):
        cs = [(table[row_of[i]][j][0], table[row_of[i]][j][1]) for j in range(hd // 2)]
        r = list(qkv[i])
        for t in range(heads):
            q0, k0 = t * hd, D + t * hd
            r[q0:q0 + hd] = rotate_pairs(qkv[i][q0:q0 + hd], cs)
            r[k0:k0 + hd] = rotate_pairs(qkv[i][k0:k0 + hd], cs)
        rot.append(r)
    scale = 1.0 / math.sqrt(hd)
    ctx = [[0.0] * D for _ in range(n)]
    for win in sorted(set(win_of)):
        toks = [i for i in range(n) if win_of[i] == win]
        for t in range(heads):
            lo = t * hd
            qr = [rot[i][lo:lo + hd] for i in toks]
            kr = [rot[i][D + lo:D + lo + hd] for i in toks]
            vr = [rot[i][2 * D + lo:2 * D + lo + hd] for i in toks]
            o = attention_head(qr, kr, vr, scale)
            for a, i in enumerate(toks):
                ctx[i][lo:lo + hd] = o[a]
    ab = linear(ctx, w["o_w"], w["o_b"])
    x1 = [[x[i][c] + ab[i][c] for c in range(D)] for i in range(n)]
    h2 = layer_norm(x1, w["ln2_g"], w["ln2_b"], eps)
    u = [[gelu_erf(v) for v in row] for row in linear(h2, w["fc1_w"], w["fc1_b"])]
    mb = linear(u, w["fc2_w"], w["fc2_b"])
    y = [[x1[i][c] + mb[i][c] for c in range(D)] for i in range(n)]
    return rot, ctx, y
