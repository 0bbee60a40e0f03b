"""The oracle's pins have teeth: plant a plausible mistake in one oracle
step (on the CPU, by monkeypatching) and check that a pin in test_oracle
fails. A pin that still passed with the mistake in place would pin nothing."""
import numpy as np
import pytest

import tests.test_oracle as pins
from oracle import block as ob
from oracle import index_maps as im


def _ln_unbiased(x, g, b, eps):
    x = np.asarray(x, dtype=np.float64)
    m = x.mean(axis=-1, keepdims=True)
    v = x.var(axis=-1, ddof=1, keepdims=True)
    return (x - m) / np.sqrt(v + eps) * g + b


def _ln_eps_outside(x, g, b, eps):
    x = np.asarray(x, dtype=np.float64)
    m = x.mean(axis=-1, keepdims=True)
    v = x.var(axis=-1, keepdims=True)
    return (x - m) / (np.sqrt(v) + eps) * g + b


def _softmax_unshifted(s):
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def _rope_wrong_sign(t, table, rows, hd):
    neg = table.copy()
    neg[..., 1] *= -1
    return _orig_rope(t, neg, rows, hd)


def _rope_half_split(t, table, rows, hd):
    # pairs (j, j + hd/2) instead of (2j, 2j + 1)
    out = t.copy()
    for h0 in range(0, t.shape[1], hd):
        for j in range(hd // 2):
            c, s = table[rows, j, 0], table[rows, j, 1]
            a, b = t[:, h0 + j], t[:, h0 + j + hd // 2]
            out[:, h0 + j] = a * c - b * s
            out[:, h0 + j + hd // 2] = b * c + a * s
    return out


def _gelu_erf_as_tanh(u):
    return ob.gelu_tanh(u)


def _mask_unit_contiguous(n, nw, qs):
    per = n // nw
    return [(np.arange(w * per // qs, (w + 1) * per // qs), np.arange(w * per, (w + 1) * per)) for w in range(nw)]


def _attention_no_scale(q, k, v, windows, heads, scale):
    return _orig_attention(q, k, v, windows, heads, 1.0)


def _pool_adjacent(z):
    return z.reshape(-1, 4, z.shape[1]).max(axis=1)


def _unroll_coarse_first(H, W, L):
    HL, WL = H >> L, W >> L
    pos = np.empty(H * W, dtype=np.int64)
    for y in range(H):
        for x in range(W):
            outer = 0
            for k in reversed(range(L)):
                outer = outer * 4 + 2 * ((y >> k) & 1) + ((x >> k) & 1)
            pos[y * W + x] = outer * (HL * WL) + (y >> L) * WL + (x >> L)
    return pos


_orig_rope = ob.apply_rope
_orig_attention = ob.attention

def _stack_levels_kept(x, blocks, specs, levels, taps):
    # forgets that a 2x2 pool consumes one unroll level
    from oracle import stack as ost
    H, W = specs[0]["grid_h"], specs[0]["grid_w"]
    t = im.unroll(np.asarray(x, dtype=np.float64), H, W, levels)
    feats = []
    for i, (w, sp) in enumerate(zip(blocks, specs)):
        t = ob.block_forward(t, w, sp)["y"]
        if sp["q_stride"] == 4:
            H, W = H // 2, W // 2
        if i in taps:
            feats.append(im.reroll(t, H, W, levels))
    return feats


from oracle import stack as ost  # noqa: E402

MUTATIONS = [
    ("layer_norm unbiased variance", ob, "layer_norm", _ln_unbiased, pins.test_layer_norm_closed_form),
    ("layer_norm eps outside sqrt", ob, "layer_norm", _ln_eps_outside, pins.test_layer_norm_closed_form),
    ("softmax without max shift", ob, "softmax_rows", _softmax_unshifted, pins.test_softmax_rows_sum_to_one_and_shift_invariant),
    ("rope rotation sign", ob, "apply_rope", _rope_wrong_sign, pins.test_rope_properties),
    ("rope pairs split by halves", ob, "apply_rope", _rope_half_split, pins.test_rope_properties),
    ("gelu erf replaced by tanh form", ob, "gelu_erf", _gelu_erf_as_tanh, pins.test_gelu_erf_closed_form),
    ("contiguous mask units", im, "mask_unit_windows", _mask_unit_contiguous, pins.test_block_vs_brute_on_tiny_config),
    ("attention scale dropped", ob, "attention", _attention_no_scale, pins.test_attention_vs_torch_sdpa),
    ("pool over adjacent rows", ob, "pool4", _pool_adjacent, pins.test_pool4_definition),
    ("unroll coarse level first", im, "unroll_positions", _unroll_coarse_first, pins.test_mask_unit_is_spatial_block_and_pool_is_2x2_cell),
    ("stack keeps unroll levels after a pool", ost, "stack_forward", _stack_levels_kept,
     pins.test_stack_pooled_features_independent_of_unroll_depth),
]


from oracle import stem as ostem  # noqa: E402

_orig_conv2d = ostem.conv2d


def _weight_layout_ignored(weight, layout):
    # reads an OHWI weight as if it were OIHW (a reshape, no transpose)
    w = np.asarray(weight, dtype=np.float64)
    return w.reshape(w.shape[0], w.shape[3], w.shape[1], w.shape[2])


def _conv_flipped(P, w, stride, pad):
    # true convolution (kernel flipped) instead of the cross-correlation
    return _orig_conv2d(P, w[:, :, ::-1, ::-1], stride, pad)


def _conv_pad_one_side(P, w, stride, pad):
    # zero padding only after the image instead of around it
    B, C, H, W = P.shape
    Pp = np.zeros((B, C, H + pad, W + pad))
    Pp[:, :, :H, :W] = P
    return _orig_conv2d(Pp, w, stride, 0)[:, :, :(H + 2 * pad - w.shape[2]) // stride + 1,
                                          :(W + 2 * pad - w.shape[3]) // stride + 1]


def _bucket_identity(out_h, out_w, mode, side):
    y, x = np.divmod(np.arange(out_h * out_w), out_w)
    if mode == "bucket":
        return y * side + x
    return _orig_pos_rows(out_h, out_w, mode, side)


def _tile_by_block(out_h, out_w, mode, side):
    y, x = np.divmod(np.arange(out_h * out_w), out_w)
    if mode == "tile":
        return (y // (out_h // side)) * side + x // (out_w // side)
    return _orig_pos_rows(out_h, out_w, mode, side)


_orig_pos_rows = ostem.pos_rows

MUTATIONS += [
    ("stem OHWI weight read as OIHW", ostem, "weight_oihw", _weight_layout_ignored,
     lambda: pins.test_stem_conv_matches_torch("hiera", dict(batch=2, in_h=30, in_w=26))),
    ("stem kernel flipped", ostem, "conv2d", _conv_flipped,
     lambda: pins.test_stem_one_hot_weight_selects_the_pixel("siglip")),
    ("stem padding on one side", ostem, "conv2d", _conv_pad_one_side,
     lambda: pins.test_stem_conv_matches_torch("hiera", dict(batch=2, in_h=30, in_w=26))),
    ("siglip bucket as identity", ostem, "pos_rows", _bucket_identity, pins.test_siglip_pos_buckets_as_printed),
    ("siglip bucket as identity (procedure)", ostem, "pos_rows", _bucket_identity,
     pins.test_siglip_pos_buckets_follow_the_bucketize_procedure),
    ("sam3 table stretched instead of tiled", ostem, "pos_rows", _tile_by_block, pins.test_sam3_pos_table_tiles_the_grid),
]


from oracle import quant as oquant  # noqa: E402


def _q8_unsigned(buf, rows, cols):
    # payload read as unsigned bytes
    q, sc = _orig_q8_from_bytes(buf, rows, cols)
    return q.view(np.uint8).astype(np.int16), sc


def _q8_scale_by_column(q, scale):
    q = np.asarray(q, dtype=np.float64)
    s = np.resize(np.asarray(scale, dtype=np.float64), q.shape[1])
    return q * s[None, :]


def _q8_scales_big_endian(buf, rows, cols):
    b = np.frombuffer(bytes(buf), dtype=np.uint8)
    q = b[:rows * cols].view(np.int8).reshape(rows, cols)
    return q.copy(), b[rows * cols:rows * cols + 2 * rows].view(">f2").copy()


_orig_q8_from_bytes = oquant.q8_row_from_bytes

MUTATIONS += [
    ("q8 payload unsigned", oquant, "q8_row_from_bytes", _q8_unsigned, pins.test_q8_row_bytes_layout_by_hand),
    ("q8 scale per column", oquant, "dequant_q8_row", _q8_scale_by_column, pins.test_q8_row_bytes_layout_by_hand),
    ("q8 scales big-endian", oquant, "q8_row_from_bytes", _q8_scales_big_endian, pins.test_q8_row_bytes_layout_by_hand),
]


def _rope_qkv_all(qkv, table, rows, dim, hd):
    # rotates v as well
    out = qkv.copy()
    for p in range(3):
        out[:, p * dim:(p + 1) * dim] = ob.apply_rope(qkv[:, p * dim:(p + 1) * dim], table, rows, hd)
    return out


def _rope_q_only(qkv, table, rows, dim, hd):
    out = qkv.copy()
    out[:, :dim] = ob.apply_rope(qkv[:, :dim], table, rows, hd)
    return out


def _rope_k_only(qkv, table, rows, dim, hd):
    out = qkv.copy()
    out[:, dim:2 * dim] = ob.apply_rope(qkv[:, dim:2 * dim], table, rows, hd)
    return out


def _rope_rows_transposed_in_windows(spec):
    # in-window row taken column-major (x * win_h + y) instead of raster
    n = np.arange(spec["grid_h"] * spec["grid_w"])
    y, x = n // spec["grid_w"], n % spec["grid_w"]
    if spec["mode"] == "spatial":
        return (x % spec["win_w"]) * spec["win_h"] + (y % spec["win_h"])
    return n


_orig_tower = ost.tower_forward


def _tower_post_ln_skipped(x, blocks, specs, pre_ln=None, post_ln=None, eps=1e-6):
    return _orig_tower(x, blocks, specs, pre_ln=pre_ln, post_ln=None, eps=eps)


def _tower_post_ln_before_last_block(x, blocks, specs, pre_ln=None, post_ln=None, eps=1e-6):
    t = _orig_tower(x, blocks[:-1], specs[:-1], pre_ln=pre_ln, post_ln=post_ln, eps=eps)
    return ob.block_forward(t, blocks[-1], specs[-1])["y"]


def _tower_pre_ln_skipped(x, blocks, specs, pre_ln=None, post_ln=None, eps=1e-6):
    return _orig_tower(x, blocks, specs, pre_ln=None, post_ln=post_ln, eps=eps)


MUTATIONS += [
    ("rope on v too (spatial)", ob, "rope_qk", _rope_qkv_all,
     lambda: pins.test_block_rope_vs_brute("spatial")),
    ("rope on v too (global)", ob, "rope_qk", _rope_qkv_all,
     lambda: pins.test_block_rope_leaves_v_and_cancels_under_a_common_rotation("global")),
    ("rope on q only (brute)", ob, "rope_qk", _rope_q_only,
     lambda: pins.test_block_rope_vs_brute("global")),
    ("rope on q only (common rotation)", ob, "rope_qk", _rope_q_only,
     lambda: pins.test_block_rope_leaves_v_and_cancels_under_a_common_rotation("spatial")),
    ("rope on k only", ob, "rope_qk", _rope_k_only,
     lambda: pins.test_block_rope_leaves_v_and_cancels_under_a_common_rotation("global")),
    ("rope rows column-major inside windows", ob, "rope_rows_for", _rope_rows_transposed_in_windows,
     lambda: pins.test_block_rope_vs_brute("spatial")),
    ("tower post_ln skipped", ost, "tower_forward", _tower_post_ln_skipped,
     pins.test_tower_post_layernorm_follows_the_last_block),
    ("tower post_ln before the last block", ost, "tower_forward", _tower_post_ln_before_last_block,
     pins.test_tower_post_layernorm_follows_the_last_block),
    ("tower pre_ln skipped", ost, "tower_forward", _tower_pre_ln_skipped,
     pins.test_tower_pre_layernorm_precedes_the_first_block),
]


# ---------------------------------------------------------- block composition
# A block with one step of the composition wired wrong (the tiny mask-unit
# configuration of the brute-force pin: fused qkv, no RoPE, q_stride 1).
def _block_wired(kind):
    def fwd(x, w, spec):
        assert spec.get("qkv", "fused") == "fused" and not spec.get("rope") and spec["q_stride"] == 1
        f64 = lambda a: np.asarray(a, dtype=np.float64)
        x = f64(x)
        D, heads = spec["dim_out"], spec["heads"]
        hd = D // heads
        scale = spec.get("scale") or hd ** -0.5
        gelu = ob.gelu_erf if spec["gelu"] == "erf" else ob.gelu_tanh
        wins = ob.windows_for(spec)
        seams = {k: [] for k in ("h", "qkv", "r", "ctx", "attn_branch", "x1", "h2", "u", "mlp_branch", "y")}
        for b in range(x.shape[0]):
            xb = x[b]
            h = xb if kind == "ln1 skipped" else ob.layer_norm(xb, f64(w["ln1_g"]), f64(w["ln1_b"]), spec["eps"])
            qkv = ob.linear(h, w["qkv_w"], f64(w["qkv_b"]))
            q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
            ctx = ob.attention(q, k, v, wins, heads, scale)
            attn_branch = ob.linear(ctx, w["o_w"], f64(w["o_b"]))
            x1 = attn_branch if kind == "attention residual dropped" else xb + attn_branch
            h2 = ob.layer_norm(xb if kind == "ln2 reads x" else x1, f64(w["ln2_g"]), f64(w["ln2_b"]), spec["eps"])
            pre = ob.linear(h2, w["fc1_w"], f64(w["fc1_b"]))
            u = pre if kind == "gelu skipped" else gelu(pre)
            mlp_branch = ob.linear(u, w["fc2_w"], f64(w["fc2_b"]))
            y = (xb if kind == "mlp residual from x" else x1) + mlp_branch
            for name, val in (("h", h), ("qkv", qkv), ("r", xb), ("ctx", ctx), ("attn_branch", attn_branch),
                              ("x1", x1), ("h2", h2), ("u", u), ("mlp_branch", mlp_branch), ("y", y)):
                seams[name].append(val)
        return {k: np.stack(v) for k, v in seams.items()}
    return fwd


MUTATIONS += [
    ("block: " + kind, ob, "block_forward", _block_wired(kind), pins.test_block_vs_brute_on_tiny_config)
    for kind in ("ln1 skipped", "attention residual dropped", "ln2 reads x", "gelu skipped", "mlp residual from x")
]


@pytest.mark.parametrize("label,mod,attr,bad,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, label, mod, attr, bad, pin):
    monkeypatch.setattr(mod, attr, bad)
    with pytest.raises((AssertionError, FloatingPointError)):
        with np.errstate(over="ignore", invalid="ignore"):
            pin()


def test_block_rewired_without_a_mistake_passes(monkeypatch):
    # the harness above, with every step wired as the pages have it, passes
    # the same pin: the planted mistakes, not the harness, make it fail
    monkeypatch.setattr(ob, "block_forward", _block_wired("none"))
    pins.test_block_vs_brute_on_tiny_config()
