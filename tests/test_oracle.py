"""Pins for the CPU oracle (no GPU). Each test ties one oracle function to
something other than itself: a value printed on the pages, a closed form, an
invariant, a library routine, or the pure-Python brute force."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import block as ob
from oracle import brute
from oracle import index_maps as im
from vision_transformer_encoder_vit_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(i=0):
    return np.random.default_rng(1000 + i)


# ---------------------------------------------------------------- LayerNorm

def test_layer_norm_closed_form():
    # gamma = 1, beta = 0: each row has mean 0 and (biased) variance
    # var / (var + eps), the closed form of the SAM3 layer_norm_rows step.
    x = _rng().normal(3.0, 2.0, (7, 112))
    eps = 1e-6
    y = ob.layer_norm(x, np.ones(112), np.zeros(112), eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)
    # a large eps shrinks the variance as the closed form says
    y2 = ob.layer_norm(x, np.ones(112), np.zeros(112), 4.0)
    np.testing.assert_allclose(y2.var(axis=1), var / (var + 4.0), rtol=1e-12)


def test_layer_norm_vs_torch_and_brute():
    r = _rng(1)
    x, g, b = r.normal(size=(5, 48)), 1 + 0.1 * r.normal(size=48), 0.1 * r.normal(size=48)
    y = ob.layer_norm(x, g, b, 1e-6)
    t = torch.nn.functional.layer_norm(torch.from_numpy(x), (48,), torch.from_numpy(g),
                                       torch.from_numpy(b), eps=1e-6).numpy()
    np.testing.assert_allclose(y, t, atol=1e-12)
    np.testing.assert_allclose(y, brute.layer_norm(x.tolist(), g.tolist(), b.tolist(), 1e-6), atol=1e-12)


# ------------------------------------------------------------------ Linear

def test_linear_vs_brute_and_orientation():
    r = _rng(2)
    x, w, b = r.normal(size=(4, 6)), r.normal(size=(3, 6)), r.normal(size=3)
    np.testing.assert_allclose(ob.linear(x, w, b), brute.linear(x.tolist(), w.tolist(), b.tolist()), atol=1e-12)
    # [out, in] orientation: a one-hot input row picks a column of w
    e = np.zeros((1, 6)); e[0, 4] = 1.0
    np.testing.assert_allclose(ob.linear(e, w, np.zeros(3))[0], w[:, 4], atol=0)


# -------------------------------------------------------------------- GELU

def test_gelu_tanh_page_values():
    rows = np.loadtxt(os.path.join(GOLDEN, "gelu_tanh_siglip.txt"))
    for x, want, tol in rows:
        got = ob.gelu_tanh(np.float64(x))
        if tol == 0:
            assert got == want
        else:
            assert abs(got - want) < tol, (x, got, want)
    for x, want, tol in rows:
        if tol:
            assert abs(brute.gelu_tanh(x) - want) < tol


def test_gelu_erf_closed_form():
    # GELU(u) = u * Phi(u); Phi from the host's math.erf.
    for u in (-6.0, -1.0, -0.3, 0.0, 0.5, 1.0, 2.5):
        phi = 0.5 * (1 + math.erf(u / math.sqrt(2)))
        assert abs(ob.gelu_erf(np.float64(u)) - u * phi) < 1e-15
    assert abs(ob.gelu_erf(np.float64(1.0)) - 0.8413447460685429) < 1e-12
    assert abs(ob.gelu_erf(np.float64(-1.0)) + 0.15865525393145707) < 1e-12
    u = np.linspace(-4, 4, 33)
    t = torch.nn.functional.gelu(torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(ob.gelu_erf(u), t, atol=1e-14)
    # the two GELU forms are different functions: they must not be swapped
    assert abs(ob.gelu_erf(np.float64(1.0)) - ob.gelu_tanh(np.float64(1.0))) > 1e-4


# ----------------------------------------------------------------- softmax

def test_softmax_rows_sum_to_one_and_shift_invariant():
    s = _rng(3).normal(0, 30, (9, 40))
    p = ob.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(ob.softmax_rows(s + 123.0), p, atol=1e-12)
    # scores as large as the SAM3 trunk's (~155) stay finite
    big = ob.softmax_rows(np.array([[155.0, 150.0, -20.0]]))
    assert np.all(np.isfinite(big)) and abs(big.sum() - 1) < 1e-12
    # beyond float64's exp range the row max must still be subtracted first
    huge = ob.softmax_rows(np.array([[1000.0, 1000.0 - math.log(3.0)]]))
    np.testing.assert_allclose(huge, [[0.75, 0.25]], atol=1e-12)


# --------------------------------------------------------------- attention

def test_attention_vs_torch_sdpa():
    r = _rng(4)
    N, D, H = 24, 32, 4
    q, k, v = r.normal(size=(N, D)), r.normal(size=(N, D)), r.normal(size=(N, D))
    ctx = ob.attention(q, k, v, [(np.arange(N), np.arange(N))], H, (D // H) ** -0.5)
    t = lambda a: torch.from_numpy(a).reshape(N, H, D // H).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).transpose(0, 1).reshape(N, D)
    np.testing.assert_allclose(ctx, ref.numpy(), atol=1e-12)


def test_attention_special_cases():
    r = _rng(5)
    N, D, H = 6, 8, 2
    q, v = r.normal(size=(N, D)), r.normal(size=(N, D))
    k_same = np.tile(r.normal(size=(1, D)), (N, 1))
    ctx = ob.attention(q, k_same, v, [(np.arange(N), np.arange(N))], H, 0.5)
    np.testing.assert_allclose(ctx, np.tile(v.mean(axis=0), (N, 1)), atol=1e-12)
    # a window with a single key returns that key's value row
    wins = [(np.array([i]), np.array([i])) for i in range(N)]
    ctx1 = ob.attention(q, r.normal(size=(N, D)), v, wins, H, 0.5)
    np.testing.assert_allclose(ctx1, v, atol=1e-15)


def test_attention_windows_vs_brute():
    r = _rng(6)
    N, D, H, nw = 16, 12, 3, 4
    q, k, v = r.normal(size=(N, D)), r.normal(size=(N, D)), r.normal(size=(N, D))
    wins = im.mask_unit_windows(N, nw, 1)
    ctx = ob.attention(q, k, v, wins, H, 0.7)
    hd = D // H
    for qi, ki in wins:
        for t in range(H):
            c = slice(t * hd, (t + 1) * hd)
            want = brute.attention_head(q[qi, c].tolist(), k[ki, c].tolist(), v[ki, c].tolist(), 0.7)
            np.testing.assert_allclose(ctx[qi, c], want, atol=1e-12)


# --------------------------------------------------------------------- RoPE

def test_rope_properties():
    hd, H, W = 64, 6, 5
    tab = synth.axial_rope_table(H, W, hd, 10000.0).astype(np.float64)
    r = _rng(7)
    q = r.normal(size=(H * W, 2 * hd))
    rows = np.arange(H * W)
    qr = ob.apply_rope(q, tab, rows, hd)
    # each rotated pair keeps its length (to the float32 table's cos^2+sin^2)
    np.testing.assert_allclose(qr[:, 0::2] ** 2 + qr[:, 1::2] ** 2, q[:, 0::2] ** 2 + q[:, 1::2] ** 2, rtol=1e-6)
    # table row 0 (position (0, 0)) is the identity
    np.testing.assert_allclose(qr[0], q[0], atol=1e-7)
    # <R_p a, R_p' b> depends only on p' - p per axis: shift both positions
    a, b = r.normal(size=(1, hd)), r.normal(size=(1, hd))
    def dot(p1, p2):
        return (ob.apply_rope(a, tab, np.array([p1]), hd) @ ob.apply_rope(b, tab, np.array([p2]), hd).T).item()
    pos = lambda y, x: y * W + x
    assert abs(dot(pos(0, 0), pos(2, 3)) - dot(pos(1, 1), pos(3, 4))) < 1e-5
    assert abs(dot(pos(0, 0), pos(2, 3)) - dot(pos(0, 0), pos(3, 2))) > 1e-4  # axes are distinct
    # the pair rotation direction: (1, 0) at angle theta goes to (cos, sin)
    e = np.zeros((1, hd)); e[0, 0] = 1.0
    out = ob.apply_rope(e, tab, np.array([pos(0, 1)]), hd)
    assert abs(out[0, 0] - math.cos(1.0)) < 1e-6 and abs(out[0, 1] - math.sin(1.0)) < 1e-6


def test_rope_rows_for_modes():
    spec = dict(grid_h=72, grid_w=72, mode="spatial", win_h=24, win_w=24)
    rows = ob.rope_rows_for(spec)
    assert rows.max() == 575 and rows[24] == 0 and rows[72] == 24
    spec["mode"] = "global"
    assert ob.rope_rows_for(spec)[5183] == 5183


# -------------------------------------------------------------- index maps

@pytest.mark.parametrize("H,W,L", [(8, 8, 2), (128, 128, 3), (64, 64, 2), (16, 32, 3), (4, 4, 0)])
def test_unroll_bijection_and_roundtrip(H, W, L):
    pos = im.unroll_positions(H, W, L)
    assert sorted(pos.tolist()) == list(range(H * W))
    payload = np.arange(H * W, dtype=np.int64).reshape(1, H * W, 1) * 3 + 7
    assert np.array_equal(im.reroll(im.unroll(payload, H, W, L), H, W, L), payload)


def test_mask_unit_is_spatial_block_and_pool_is_2x2_cell():
    H = W = 128
    L = 3
    N = H * W
    pos = im.unroll_positions(H, W, L)
    ys, xs = np.divmod(np.arange(N), W)
    n_w = (H >> L) * (W >> L)
    # window n mod n_w == the 8x8 spatial block index
    blk = (ys >> L) * (W >> L) + (xs >> L)
    assert np.array_equal(pos % n_w, blk)
    # every pool group is one 2x2 spatial cell
    inv = np.empty(N, dtype=np.int64)
    inv[pos] = np.arange(N)
    g = im.pool_groups(N)
    cells = (ys[inv[g]] >> 1) * (W >> 1) + (xs[inv[g]] >> 1)
    assert np.all(cells == cells[:, :1])
    # the pooled order is the (L-1)-level unroll of the half-size grid
    pooled_cell = cells[:, 0]
    want = im.unroll_positions(H // 2, W // 2, L - 1)
    assert np.array_equal(want[pooled_cell], np.arange(N // 4))


def test_hiera_stage_shape_contract():
    # 512^2 input, stride-4 patch embed, 3 unroll levels, 3 pools: the stage
    # grids, mask-unit sizes and widths listed on the pages.
    rows = np.loadtxt(os.path.join(GOLDEN, "hiera_stage_shapes.txt"), dtype=np.int64)
    side, L = 512 // 4, 3
    N = side * side
    n_w = (side >> L) ** 2
    payload = np.arange(N, dtype=np.int64).reshape(1, N, 1)
    tok = im.unroll(payload, side, side, L)[0, :, 0]
    ys, xs = np.divmod(tok, side)
    for stage, grid, dim, heads, win, mu in rows:
        assert grid * grid == len(tok)
        assert len(tok) // n_w == win
        assert dim % heads == 0 and dim // heads == 56
        # every window (n mod n_w) stays one spatial block of the stage grid
        cell = 1 << (L - stage)
        scale = side // grid
        by, bx = (ys // scale) // cell, (xs // scale) // cell
        for w in range(0, n_w, 37):
            sel = np.arange(w, len(tok), n_w)
            assert len(set(zip(by[sel].tolist(), bx[sel].tolist()))) == 1
        if stage < 3:
            g = im.pool_groups(len(tok))
            # max-pool of the token ids' coarse position: all four share it
            assert np.all((ys[g] // (2 * scale)) == (ys[g][:, :1] // (2 * scale)))
            tok, ys, xs = tok[g[:, 0]], ys[g[:, 0]], xs[g[:, 0]]


def test_spatial_windows():
    wins = im.spatial_windows(72, 72, 24, 24)
    assert len(wins) == 9 and all(len(w) == 576 for w in wins)
    assert sorted(np.concatenate(wins).tolist()) == list(range(72 * 72))
    w4 = wins[4]  # centre window
    ys, xs = np.divmod(w4, 72)
    assert ys.min() == 24 and ys.max() == 47 and xs.min() == 24 and xs.max() == 47
    assert w4[1] - w4[0] == 1 and w4[24] - w4[0] == 72


# -------------------------------------------------------------- pool4

def test_pool4_definition():
    z = _rng(8).normal(size=(16, 3))
    p = ob.pool4(z)
    for m in range(4):
        np.testing.assert_array_equal(p[m], np.max(z[[m, m + 4, m + 8, m + 12]], axis=0))


# ------------------------------------------------------- whole block (tiny)

def _as_lists(w):
    return {k: np.asarray(v, dtype=np.float64).tolist() for k, v in w.items()}


def test_block_vs_brute_on_tiny_config():
    spec = synth.CONFIGS["c1_tiny_f32"]
    inp = synth.make_inputs(spec, seed=0)
    seams = ob.block_forward(inp["x"], inp, spec)
    ctx, y = brute.block_forward_mask_unit(np.asarray(inp["x"][0], np.float64).tolist(),
                                            _as_lists(inp), spec["n_windows"], spec["heads"], spec["eps"])
    np.testing.assert_allclose(seams["ctx"][0], ctx, atol=1e-12)
    np.testing.assert_allclose(seams["y"][0], y, atol=1e-12)
    # residual structure: y = x1 + mlp_branch, x1 = x + attn_branch
    np.testing.assert_allclose(seams["x1"], inp["x"] + seams["attn_branch"], atol=1e-12)
    np.testing.assert_allclose(seams["y"], seams["x1"] + seams["mlp_branch"], atol=1e-12)


def test_block_tanh_separate_qkv_vs_brute():
    # SigLIP structure (separate q/k/v, tanh-GELU, global) on a tiny shape:
    # separate projections equal the fused one with stacked weights.
    spec = synth.derive(synth.CONFIGS["c4_siglip_b8"], batch=2, grid_h=2, grid_w=4,
                        dim_in=16, dim_out=16, heads=2, mlp=32, dtype="f32", scale=None)
    inp = synth.make_inputs(spec, seed=3)
    seams = ob.block_forward(inp["x"], inp, spec)
    fused = dict(inp)
    fused["qkv_w"] = np.concatenate([inp["q_w"], inp["k_w"], inp["v_w"]])
    fused["qkv_b"] = np.concatenate([inp["q_b"], inp["k_b"], inp["v_b"]])
    for b in range(2):
        ctx, y = brute.block_forward_mask_unit(np.asarray(inp["x"][b], np.float64).tolist(),
                                                _as_lists(fused), 1, 2, spec["eps"], gelu="tanh")
        np.testing.assert_allclose(seams["y"][b], y, atol=1e-12)
        np.testing.assert_allclose(seams["ctx"][b], ctx, atol=1e-12)


def test_block_frames_independent():
    # frames never attend to each other: frame f of a batched run equals the
    # single-frame run (SigLIP batched-vs-sequential property)
    spec = synth.derive(synth.CONFIGS["c4_siglip_b8"], batch=3, grid_h=2, grid_w=3,
                        dim_in=8, dim_out=8, heads=2, mlp=16, dtype="f32")
    inp = synth.make_inputs(spec, seed=4)
    all3 = ob.block_forward(inp["x"], inp, spec)["y"]
    one = ob.block_forward(inp["x"][1:2], inp, synth.derive(spec, batch=1))["y"]
    np.testing.assert_allclose(all3[1], one[0], atol=0)


def test_block_transition_vs_definition():
    # pooled transition on a tiny grid: q and the residual are 2x2-max-pooled
    # (after the projection), kv keep every token; compare against a direct
    # loop over the windows with the brute-force attention.
    spec = synth.derive(synth.CONFIGS["c3a_hiera_trans"], grid_h=8, grid_w=8,
                        dim_in=8, dim_out=16, heads=2, mlp=32, n_windows=4, dtype="f32")
    inp = synth.make_inputs(spec, seed=5)
    s = ob.block_forward(inp["x"], inp, spec)
    x = np.asarray(inp["x"][0], np.float64)
    h = brute.layer_norm(x.tolist(), inp["ln1_g"].tolist(), inp["ln1_b"].tolist(), spec["eps"])
    res = np.array(brute.linear(h, inp["res_w"].tolist(), inp["res_b"].tolist()))
    qkv = np.array(brute.linear(h, inp["qkv_w"].tolist(), inp["qkv_b"].tolist()))
    N, D = 64, 16
    r = np.maximum.reduce([res[s_ * 16:(s_ + 1) * 16] for s_ in range(4)])
    q = np.maximum.reduce([qkv[s_ * 16:(s_ + 1) * 16, :D] for s_ in range(4)])
    np.testing.assert_allclose(s["r"][0], r, atol=1e-12)
    np.testing.assert_allclose(s["q_pooled"][0], q, atol=1e-12)
    ctx = np.zeros((16, D))
    for w in range(4):
        qi, ki = np.arange(w, 16, 4), np.arange(w, N, 4)
        for t in range(2):
            c = slice(t * 8, t * 8 + 8)
            ctx[qi, c] = brute.attention_head(q[qi, c].tolist(), qkv[ki, D:2 * D][:, c].tolist(),
                                              qkv[ki, 2 * D:][:, c].tolist(), 8 ** -0.5)
    np.testing.assert_allclose(s["ctx"][0], ctx, atol=1e-12)


def test_block_rope_windowed_locality():
    # spatial windows: changing a token in one window leaves every other
    # window's output exactly unchanged
    spec = synth.derive(synth.CONFIGS["c5w_sam3_win"], grid_h=8, grid_w=8, win_h=4, win_w=4,
                        dim_in=16, dim_out=16, heads=1, mlp=32, dtype="f32")
    spec["dim_out"] = 16
    inp = synth.make_inputs(spec, seed=6)
    inp["rope"] = synth.axial_rope_table(4, 4, 16, 10000.0)
    y0 = ob.block_forward(inp["x"], inp, spec)["y"][0]
    x2 = inp["x"].copy()
    x2[0, 0] += 1.0  # token (0, 0): window 0
    y1 = ob.block_forward(x2, inp, spec)["y"][0]
    changed = np.where(np.any(y0 != y1, axis=1))[0]
    ys, xs = np.divmod(changed, 8)
    assert len(changed) == 16 and ys.max() < 4 and xs.max() < 4


def _random_angle_table(rows, pairs, seed):
    a = np.random.default_rng(seed).uniform(-np.pi, np.pi, (rows, pairs))
    return np.stack([np.cos(a), np.sin(a)], axis=-1)


def _sam3_tiny(mode):
    kw = dict(grid_h=4, grid_w=6, dim_in=16, dim_out=16, heads=2, mlp=32, dtype="f32")
    if mode == "spatial":
        spec = synth.derive(synth.CONFIGS["c5w_sam3_win"], win_h=2, win_w=3, **kw)
        rows = 6
    else:
        spec = synth.derive(synth.CONFIGS["c5g_sam3_global"], **kw)
        rows = 24
    inp = synth.make_inputs(spec, seed=12)
    inp["rope"] = _random_angle_table(rows, 4, 13)
    return spec, inp


@pytest.mark.parametrize("mode", ["spatial", "global"])
def test_block_rope_vs_brute(mode):
    # the SAM3 block with RoPE against the pure-Python loop (SAM3 apply_rope:
    # the q part and the k part of each head turn pair by pair, v does not),
    # with a table of random angles so every pair turns
    spec, inp = _sam3_tiny(mode)
    s = ob.block_forward(inp["x"], inp, spec)
    wh, ww = (spec["win_h"], spec["win_w"]) if mode == "spatial" else (0, 0)
    qkv, ctx, y = brute.block_forward_rope(np.asarray(inp["x"][0], np.float64).tolist(), _as_lists(inp),
                                           4, 6, wh, ww, spec["heads"], spec["eps"], inp["rope"].tolist())
    np.testing.assert_allclose(s["qkv"][0], qkv, atol=1e-12)
    np.testing.assert_allclose(s["ctx"][0], ctx, atol=1e-12)
    np.testing.assert_allclose(s["y"][0], y, atol=1e-12)


@pytest.mark.parametrize("mode", ["spatial", "global"])
def test_block_rope_leaves_v_and_cancels_under_a_common_rotation(mode):
    # v is the plain projection of h; q and k keep their pair lengths; and a
    # rotation that is the same at every position (a table whose rows are all
    # equal) must drop out of attention, because R q . R k = q . k for an
    # orthogonal R applied to both -- so ctx and y equal the block without
    # RoPE. Rotating v as well, or only one of q and k, breaks that.
    spec, inp = _sam3_tiny(mode)
    D = spec["dim_out"]
    s = ob.block_forward(inp["x"], inp, spec)
    h = brute.layer_norm(np.asarray(inp["x"][0], np.float64).tolist(), inp["ln1_g"].tolist(),
                         inp["ln1_b"].tolist(), spec["eps"])
    plain = np.array(brute.linear(h, inp["qkv_w"].tolist(), inp["qkv_b"].tolist()))
    np.testing.assert_allclose(s["qkv"][0][:, 2 * D:], plain[:, 2 * D:], atol=1e-12)
    for part in (slice(0, D), slice(D, 2 * D)):
        got, ref = s["qkv"][0][:, part], plain[:, part]
        np.testing.assert_allclose(got[:, 0::2] ** 2 + got[:, 1::2] ** 2,
                                   ref[:, 0::2] ** 2 + ref[:, 1::2] ** 2, rtol=1e-10)
        assert np.abs(got - ref).max() > 1e-3  # the part did turn
    common = dict(inp)
    common["rope"] = np.repeat(_random_angle_table(1, 4, 14), inp["rope"].shape[0], axis=0)
    with_rope = ob.block_forward(inp["x"], common, spec)
    no_rope = ob.block_forward(inp["x"], inp, dict(spec, rope=False))
    for k in ("ctx", "y"):
        np.testing.assert_allclose(with_rope[k], no_rope[k], atol=1e-12, err_msg=k)


def test_block_rows_equals_full_block():
    # the sampled-row evaluation used at full sizes is the same computation
    for name, kw in (("c3a_hiera_trans", dict(grid_h=8, grid_w=8, dim_in=8, dim_out=16, heads=2,
                                               mlp=32, n_windows=4)),
                     ("c5w_sam3_win", dict(grid_h=8, grid_w=8, win_h=4, win_w=4, dim_in=16,
                                           dim_out=16, heads=1, mlp=32)),
                     ("c4_siglip_b8", dict(batch=2, grid_h=3, grid_w=4, dim_in=16, dim_out=16,
                                           heads=2, mlp=32))):
        spec = synth.derive(synth.CONFIGS[name], dtype="f32", **kw)
        inp = synth.make_inputs(spec, seed=9)
        if spec["rope"]:
            inp["rope"] = synth.axial_rope_table(4, 4, 16, 10000.0)
        full = ob.block_forward(inp["x"], inp, spec)
        rows = np.array([0, 3, 5, 11])
        part = ob.block_forward_rows(inp["x"], inp, spec, rows)
        for k, v in part.items():
            np.testing.assert_allclose(v, full[k][:, rows], atol=1e-12, err_msg=k)


# ---- Hiera stage stack (oracle/stack.py) ----

def test_stack_shape_contract_512():
    # the plan's per-stage feature shapes at a 512x512 input (128x128 tokens)
    from oracle import stack as ost
    rows = np.loadtxt(os.path.join(GOLDEN, "hiera_stage_shapes.txt"), dtype=np.int64)
    specs, levels, taps = synth.hiera_stack(side=128)
    assert len(specs) == 24 and taps == [1, 4, 20, 23]
    assert [i for i, s in enumerate(specs) if s["q_stride"] == 4] == [2, 5, 21]
    for (stage, grid, dim, heads, win, mu), t in zip(rows, taps):
        sp = specs[t]
        assert (sp["dim_out"], sp["heads"]) == (dim, heads)
        assert (sp["mode"] == "mask_unit") == bool(mu)
        n_out = sp["grid_h"] * sp["grid_w"] // sp["q_stride"]
        assert n_out == grid * grid
        if mu:
            assert n_out // sp["n_windows"] == win
    # shapes through the oracle itself, on a 4x narrower grid with the same
    # stage structure (one block per stage)
    small, levels, taps = synth.hiera_stack(side=32, stage_blocks=(1, 1, 1, 1))
    x, blocks = synth.make_stack_inputs(small, seed=3)
    feats = ost.stack_forward(x, blocks, small, levels, taps)
    assert [f.shape for f in feats] == [(1, 32 * 32, 112), (1, 16 * 16, 224), (1, 8 * 8, 448), (1, 4 * 4, 896)]


def test_stack_global_blocks_do_not_see_token_order():
    # global attention and the row-wise steps are permutation-equivariant:
    # through unroll -> blocks -> reroll the stack must equal the same blocks
    # on raster-order tokens, exactly (float64, same arithmetic per row)
    from oracle import stack as ost
    base = synth.derive(synth.CONFIGS["c3b_hiera_s2"], grid_h=16, grid_w=16, dim_in=112, dim_out=112, heads=2,
                        mlp=224, dtype="f32")
    specs = [dict(base, name="g%d" % i) for i in range(3)]
    x, blocks = synth.make_stack_inputs(specs, seed=5)
    for levels in (1, 2, 3):
        f = ost.stack_forward(x, blocks, specs, levels, [0, 2])
        ref = x.astype(np.float64)
        outs = []
        for i, (w, sp) in enumerate(zip(blocks, specs)):
            ref = ob.block_forward(ref, w, sp)["y"]
            if i in (0, 2):
                outs.append(ref)
        for a, b in zip(f, outs):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_stack_pooled_features_independent_of_unroll_depth():
    # a global block with the 2x2 query pool: the pool groups are the 2x2
    # cells for any unroll depth >= 1 (finest level outermost), and the
    # feature is rerolled with one level fewer; so the raster-order feature
    # must not depend on the depth. A stack that forgot to drop the level
    # (or pooled the wrong groups) differs.
    from oracle import stack as ost
    sp = synth.derive(synth.CONFIGS["c3b_hiera_s2"], grid_h=16, grid_w=16, dim_in=112, dim_out=224, heads=4,
                      mlp=448, q_stride=4, dtype="f32")
    nxt = synth.derive(synth.CONFIGS["c3b_hiera_s2"], grid_h=8, grid_w=8, dim_in=224, dim_out=224, heads=4,
                       mlp=448, dtype="f32")
    specs = [dict(sp, name="p"), dict(nxt, name="q")]
    x, blocks = synth.make_stack_inputs(specs, seed=7)
    feats = [ost.stack_forward(x, blocks, specs, levels, [0, 1]) for levels in (1, 2, 3)]
    for other in feats[1:]:
        for a, b in zip(feats[0], other):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # and the pooled residual of the unrolled tokens, rerolled, is the 2x2
    # spatial max of the raster-order projection
    h_rast = ob.layer_norm(x[0].astype(np.float64), blocks[0]["ln1_g"].astype(np.float64),
                           blocks[0]["ln1_b"].astype(np.float64), sp["eps"])
    proj = ob.linear(h_rast, blocks[0]["res_w"], blocks[0]["res_b"].astype(np.float64)).reshape(16, 16, -1)
    pooled = proj.reshape(8, 2, 8, 2, -1).max(axis=(1, 3)).reshape(64, -1)
    t = im.unroll(x.astype(np.float64), 16, 16, 2)
    r = ob.block_forward(t, blocks[0], sp)["r"]
    np.testing.assert_allclose(im.reroll(r, 8, 8, 1)[0], pooled, rtol=1e-12, atol=1e-12)


def test_sam3_trunk_windows_stay_local_until_a_global_layer():
    # windowed layers never mix 24x24 windows, through any number of layers:
    # changing one token of window 0 leaves every other window's output
    # unchanged, exactly; one global layer spreads it everywhere
    from oracle import stack as ost
    specs = synth.sam3_trunk(grid=48, layers=3, global_layers=(), dim=64, heads=2, mlp=128)
    specs = [synth.derive(s, dtype="f32") for s in specs]
    x, blocks = synth.make_stack_inputs(specs, seed=11)
    g, b = synth.make_layernorm_params(64, 11)
    y0 = ost.tower_forward(x, blocks, specs, pre_ln=(g, b))
    x2 = x.copy()
    x2[0, 5 * 48 + 7, 3] += 1.0  # token (5, 7): window (0, 0); one channel (a uniform shift is what LN removes)
    y1 = ost.tower_forward(x2, blocks, specs, pre_ln=(g, b))
    win = np.zeros(48 * 48, dtype=bool)
    for t in range(48 * 48):
        win[t] = (t // 48) < 24 and (t % 48) < 24
    assert np.abs(y1[0, win] - y0[0, win]).max() > 1e-3
    assert np.array_equal(y1[0, ~win], y0[0, ~win])
    specs_g = synth.sam3_trunk(grid=48, layers=3, global_layers=(1,), dim=64, heads=2, mlp=128)
    specs_g = [synth.derive(s, dtype="f32") for s in specs_g]
    _, blocks_g = synth.make_stack_inputs(specs_g, seed=11)
    z0 = ost.tower_forward(x, blocks_g, specs_g, pre_ln=(g, b))
    z1 = ost.tower_forward(x2, blocks_g, specs_g, pre_ln=(g, b))
    assert np.all(np.abs(z1[0] - z0[0]).max(axis=-1) > 0)


def _tiny_tower(seed):
    specs = synth.siglip_tower(batch=2, grid=3, layers=2, dim=16, heads=2, mlp=32)
    specs = [synth.derive(s, dtype="f32") for s in specs]
    x, blocks = synth.make_stack_inputs(specs, seed=seed)
    g, b = synth.make_layernorm_params(16, seed)
    return specs, x, blocks, g, b


def test_tower_post_layernorm_follows_the_last_block():
    # SigLIP forward_frame: the blocks, then post_layernorm on their output.
    # Pinned against the pure-Python LayerNorm of the blocks' output, and by
    # the closed form: with gamma 1, beta 0 every output row has mean 0 and
    # variance var / (var + eps) of the last block's row.
    from oracle import stack as ost
    specs, x, blocks, g, b = _tiny_tower(21)
    out = ost.tower_forward(x, blocks, specs, post_ln=(g, b))
    t = x.astype(np.float64)
    for w, sp in zip(blocks, specs):
        t = ob.block_forward(t, w, sp)["y"]
    for f in range(2):
        np.testing.assert_allclose(out[f], brute.layer_norm(t[f].tolist(), g.tolist(), b.tolist(), 1e-6),
                                   atol=1e-12)
    unit = ost.tower_forward(x, blocks, specs, post_ln=(np.ones(16), np.zeros(16)))
    var = t.var(axis=-1)
    np.testing.assert_allclose(unit.mean(axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(unit.var(axis=-1), var / (var + 1e-6), rtol=1e-10)


def test_tower_pre_layernorm_precedes_the_first_block():
    # SAM3 trunk: ln_pre on the embedded tokens, then the blocks. The first
    # block must see the pure-Python LayerNorm of x.
    from oracle import stack as ost
    specs, x, blocks, g, b = _tiny_tower(22)
    out = ost.tower_forward(x, blocks, specs, pre_ln=(g, b))
    t = np.array([brute.layer_norm(x[f].astype(np.float64).tolist(), g.tolist(), b.tolist(), 1e-6)
                  for f in range(2)])
    for w, sp in zip(blocks, specs):
        t = ob.block_forward(t, w, sp)["y"]
    np.testing.assert_allclose(out, t, atol=1e-12)


# ---------------------------------------------------------------- patch-embedding stems

def _stem_small(kind, **kw):
    spec = dict(synth.STEMS[kind])
    spec.update(kw)
    return spec


@pytest.mark.parametrize("kind,kw", [
    ("hiera", dict(batch=2, in_h=30, in_w=26)),            # k7 s4 p3, NHWC, OHWI, ragged
    ("siglip", dict(batch=2, in_h=64, in_w=48, pos_side=4)),  # k16 s16, NCHW
    ("sam3", dict(in_h=70, in_w=56, pos_side=3)),          # k14 s14, no bias
])
def test_stem_conv_matches_torch(kind, kw):
    # the convolution against torch's conv2d (float64, CPU), the pixels and
    # weights brought to NCHW / OIHW by torch's own permute
    from oracle import stem
    spec = _stem_small(kind, dtype="f32", pos_mode="none", **kw)
    inp = synth.make_stem_inputs(spec, seed=5)
    P = torch.from_numpy(inp["pixels"]).double()
    W = torch.from_numpy(inp["weight"]).double()
    if spec["layout"] == "nhwc":
        P = P.permute(0, 3, 1, 2)
    if spec["weight_layout"] == "ohwi":
        W = W.permute(0, 3, 1, 2)
    b = torch.from_numpy(inp["bias"]).double() if spec["bias"] else None
    ref = torch.nn.functional.conv2d(P, W, b, stride=spec["stride"], padding=spec["pad"])
    B, O, oh, ow = ref.shape
    assert (oh, ow) == synth.stem_out_grid(spec)
    got = stem.patch_embed(inp, spec)
    np.testing.assert_allclose(got, ref.reshape(B, O, oh * ow).permute(0, 2, 1).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kind", ["hiera", "siglip"])
def test_stem_one_hot_weight_selects_the_pixel(kind):
    # a weight with a single 1 at (o, c, ky, kx) copies pixel
    # (c, y*s + ky - p, x*s + kx - p) into channel o of token (y, x), zero
    # where that falls in the padding; a transposed layout or a flipped
    # kernel picks another pixel
    from oracle import stem
    spec = _stem_small(kind, batch=1, in_h=21, in_w=19, dim=3, pos_mode="none", bias=False, dtype="f32")
    inp = synth.make_stem_inputs(spec, seed=6)
    C, k, s, p = spec["in_ch"], spec["kernel"], spec["stride"], spec["pad"]
    P = inp["pixels"][0] if spec["layout"] == "nchw" else inp["pixels"][0].transpose(2, 0, 1)
    oh, ow = synth.stem_out_grid(spec)
    for (o, c, ky, kx) in [(0, 0, 0, 0), (1, C - 1, k - 1, 2), (2, 1, 3, k - 1)]:
        w = np.zeros(inp["weight"].shape, dtype=np.float32)
        if spec["weight_layout"] == "oihw":
            w[o, c, ky, kx] = 1.0
        else:
            w[o, ky, kx, c] = 1.0
        got = stem.patch_embed(dict(inp, weight=w), spec)[0]
        for y in range(oh):
            for x in range(ow):
                py, px = y * s + ky - p, x * s + kx - p
                want = P[c, py, px] if 0 <= py < P.shape[1] and 0 <= px < P.shape[2] else 0.0
                assert got[y * ow + x, o] == want
                assert np.all(got[y * ow + x, [i for i in range(3) if i != o]] == 0.0)


def test_stem_shape_contracts():
    # 512^2 -> 128^2 Hiera tokens (the first stage grid of the plan's shape
    # table), 512^2 -> 32^2 = 1024 SigLIP tokens, 1008^2 -> 72^2 SAM3 tokens
    rows = np.loadtxt(os.path.join(GOLDEN, "hiera_stage_shapes.txt"), dtype=np.int64)
    assert synth.stem_out_grid(synth.STEMS["hiera"]) == (rows[0][1], rows[0][1])
    assert synth.STEMS["hiera"]["dim"] == rows[0][2]
    assert synth.stem_out_grid(synth.STEMS["siglip"]) == (32, 32)
    assert synth.stem_out_grid(synth.STEMS["sam3"]) == (72, 72)
    # and the towers the stems feed start from those grids
    assert synth.hiera_stack()[0][0]["grid_h"] == 128
    assert synth.siglip_tower()[0]["grid_h"] * synth.siglip_tower()[0]["grid_w"] == 1024
    assert synth.sam3_trunk()[0]["grid_h"] == 72


def test_siglip_pos_buckets_as_printed():
    from oracle import stem
    fx = np.loadtxt(os.path.join(GOLDEN, "siglip_pos_buckets.txt"), dtype=np.int64)
    rows = stem.pos_rows(32, 32, "bucket", 32)
    y, x = np.divmod(np.arange(1024), 32)
    np.testing.assert_array_equal(rows, fx[y, 1] * 32 + fx[x, 1])


def test_siglip_pos_buckets_follow_the_bucketize_procedure():
    # the procedure the SigLIP page describes: fractional coordinates
    # (i / 32) * (1 - 1e-6) in float32, bucketized against the boundaries
    # j / 32 (j = 1..31) with right=True (index of the first boundary > value)
    from oracle import stem
    n = 32
    frac = (np.arange(n, dtype=np.float32) / np.float32(n)) * np.float32(1 - 1e-6)
    bounds = np.arange(1, n, dtype=np.float32) / np.float32(n)
    b = np.searchsorted(bounds, frac, side="right")
    y, x = np.divmod(np.arange(n * n), n)
    np.testing.assert_array_equal(stem.pos_rows(n, n, "bucket", n), b[y] * n + b[x])


def test_sam3_pos_table_tiles_the_grid():
    # zero weights: every token is its table row; the 72x72 grid repeats the
    # 24x24 table with period 24 on both axes, and the first 24x24 block is
    # the table in raster order
    from oracle import stem
    spec = dict(synth.STEMS["sam3"])
    inp = synth.make_stem_inputs(spec, seed=7)
    inp["weight"] = np.zeros_like(inp["weight"])
    out = stem.patch_embed(inp, spec)[0].reshape(72, 72, 1024)
    pos = inp["pos"].astype(np.float64).reshape(24, 24, 1024)
    np.testing.assert_array_equal(out[:24, :24], pos)
    np.testing.assert_array_equal(out[24:, :], out[:-24, :])
    np.testing.assert_array_equal(out[:, 24:], out[:, :-24])


# ---------------------------------------------------------------- q8_row weights

def test_q8_row_bytes_layout_by_hand():
    # 2 x 3 payload, row-major, then two little-endian float16 scales
    # (0x3800 = 0.5, 0x2000 = 2^-7)
    from oracle import quant
    payload = bytes([1, 0xFE, 0x7F, 0x80, 0x00, 0x05])  # 1, -2, 127 / -128, 0, 5
    scales = bytes([0x00, 0x38, 0x00, 0x20])
    q, s = quant.q8_row_from_bytes(payload + scales, 2, 3)
    w = quant.dequant_q8_row(q, s)
    np.testing.assert_array_equal(w, [[0.5, -1.0, 63.5], [-1.0, 0.0, 5.0 / 128.0]])
    with pytest.raises(ValueError):
        quant.q8_row_from_bytes(payload + scales[:3], 2, 3)


def test_q8_row_dequant_within_half_step():
    # the synthetic quantizer then the oracle's dequantization: every element
    # within half a scale step of the float matrix (plus the float16 rounding
    # of the scale, at most 2^-11 relative of the row maximum)
    from oracle import quant
    w = _rng(20).normal(0.0, 0.02, (96, 200)).astype(np.float32)
    q, s = synth.quantize_q8_row(w)
    assert q.dtype == np.int8 and s.dtype == np.float16 and np.abs(q.astype(int)).max() <= 127
    d = quant.dequant_q8_row(q, s)
    step = s.astype(np.float64)[:, None]
    amax = np.abs(w).max(axis=1, keepdims=True)
    assert np.all(np.abs(d - w) <= step / 2 + amax * 2.0 ** -10)
    # and the per-row maximum is hit to within that bound
    np.testing.assert_allclose(np.abs(d).max(axis=1), amax[:, 0], rtol=2e-3)
