"""Seeded synthetic inputs for the encoder block: shapes, draws and tables.

This module holds no arithmetic of the block itself. It is the one piece that
both the HIP path's tests/benchmark and the CPU oracle read: it decides the
shapes of the workloads and draws the random tensors, and both sides consume
exactly the arrays it returns.

Draws: numpy PCG64 (``default_rng``), one independent stream per tensor,
keyed by (seed, fixed tensor id), so adding or dropping an optional tensor
never shifts another tensor's values. Distributions: token inputs N(0, 1);
weight matrices N(0, 0.02); biases N(0, 0.01); LayerNorm gamma 1 + N(0, 0.1)
and beta N(0, 0.1). Values are drawn in float64, cast to float32, and for the
bf16 workloads the matrices and the token input are then rounded to the
nearest bf16 (ties to even), so both sides see identical bf16-representable
numbers. Vectors (biases, LN parameters) and RoPE tables stay float32.

Workloads (token grids, widths, heads, windows and GELU forms follow the
pages: the Hiera plan's stage table, the SigLIP constants, the SAM3 trunk
constants):

  c1_tiny_f32      1 x 8x8 tokens, D 112, 2 heads, 4 mask units of 16, MLP 448,
                   float32 end to end
  c2_hiera_s0      1 x 128x128, D 112, 2 heads, 256 mask units of 64, MLP 448
  c3a_hiera_trans  1 x 64x64 -> 32x32, D 112 -> 224, 4 heads, 64 mask units
                   (64 kv / 16 pooled q), residual proj + 2x2 max-pool, MLP 896
  c3b_hiera_s2     1 x 32x32, D 448, 8 heads, global, MLP 1792
  c4_siglip_b8     8 x 32x32, D 768, 12 heads (scale 1/8), separate q/k/v,
                   global per frame, MLP 3072, tanh-GELU
  c5w_sam3_win     1 x 72x72, D 1024, 16 heads, 24x24 windows, axial RoPE
                   (in-window table, 576 rows), MLP 4736
  c5g_sam3_global  as c5w with global attention and a 5184-row RoPE table
"""
import numpy as np

_TENSOR_IDS = {
    "x": 0, "ln1_g": 1, "ln1_b": 2, "res_w": 3, "res_b": 4,
    "qkv_w": 5, "qkv_b": 6, "q_w": 7, "q_b": 8, "k_w": 9, "k_b": 10,
    "v_w": 11, "v_b": 12, "o_w": 13, "o_b": 14, "ln2_g": 15, "ln2_b": 16,
    "fc1_w": 17, "fc1_b": 18, "fc2_w": 19, "fc2_b": 20,
}


def _spec(name, **kw):
    base = dict(name=name, batch=1, n_windows=1, win_h=0, win_w=0, q_stride=1,
                gelu="erf", eps=1e-6, scale=None, rope=False, theta=10000.0,
                qkv="fused", dtype="bf16")
    base.update(kw)
    return base


CONFIGS = {
    "c1_tiny_f32": _spec("c1_tiny_f32", grid_h=8, grid_w=8, dim_in=112,
                         dim_out=112, heads=2, mlp=448, mode="mask_unit",
                         n_windows=4, dtype="f32"),
    "c2_hiera_s0": _spec("c2_hiera_s0", grid_h=128, grid_w=128, dim_in=112,
                         dim_out=112, heads=2, mlp=448, mode="mask_unit",
                         n_windows=256),
    "c3a_hiera_trans": _spec("c3a_hiera_trans", grid_h=64, grid_w=64,
                             dim_in=112, dim_out=224, heads=4, mlp=896,
                             mode="mask_unit", n_windows=64, q_stride=4),
    "c3b_hiera_s2": _spec("c3b_hiera_s2", grid_h=32, grid_w=32, dim_in=448,
                          dim_out=448, heads=8, mlp=1792, mode="global"),
    "c4_siglip_b8": _spec("c4_siglip_b8", batch=8, grid_h=32, grid_w=32,
                          dim_in=768, dim_out=768, heads=12, mlp=3072,
                          mode="global", gelu="tanh", scale=0.125,
                          qkv="separate"),
    "c5w_sam3_win": _spec("c5w_sam3_win", grid_h=72, grid_w=72, dim_in=1024,
                          dim_out=1024, heads=16, mlp=4736, mode="spatial",
                          win_h=24, win_w=24, rope=True),
    "c5g_sam3_global": _spec("c5g_sam3_global", grid_h=72, grid_w=72,
                             dim_in=1024, dim_out=1024, heads=16, mlp=4736,
                             mode="global", rope=True),
}


def derive(base, **changes):
    """A copy of a workload spec with some fields changed (for smaller parity
    cases of the same structure)."""
    s = dict(base)
    s.update(changes)
    return s


def bf16_round(a):
    """Round float32 values to the nearest bfloat16 (ties to even) and return
    them as float32. Inputs here are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a):
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def axial_rope_table(grid_h, grid_w, head_dim, theta):
    """(cos, sin) table [grid_h*grid_w, head_dim/2, 2] for 2-D axial RoPE.

    The SAM3 trunk loads this table as a stored per-layer tensor; its layout
    (32 pairs per 64-wide head, first half of the pairs from the x position,
    second half from the y position) is stated with ``apply_rope`` on the SAM3
    page. The frequencies are the plain reading for base theta: pair j of each
    half turns at theta^(-4j/head_dim), j < head_dim/4. Row y*grid_w + x."""
    quarter = head_dim // 4
    freqs = theta ** (-(np.arange(quarter, dtype=np.float64) * 4.0) / head_dim)
    n = np.arange(grid_h * grid_w)
    ys, xs = n // grid_w, n % grid_w
    ang = np.concatenate([np.outer(xs, freqs), np.outer(ys, freqs)], axis=1)
    tab = np.stack([np.cos(ang), np.sin(ang)], axis=-1)
    return tab.astype(np.float32)


def tensor_shapes(spec):
    """Name -> shape of every input tensor of one block (PyTorch Linear
    layout [out, in] for matrices)."""
    B, N = spec["batch"], spec["grid_h"] * spec["grid_w"]
    Di, Do, M = spec["dim_in"], spec["dim_out"], spec["mlp"]
    s = {"x": (B, N, Di), "ln1_g": (Di,), "ln1_b": (Di,)}
    if spec["q_stride"] == 4:
        s.update(res_w=(Do, Di), res_b=(Do,))
    if spec["qkv"] == "separate":
        for p in "qkv":
            s[p + "_w"] = (Do, Di)
            s[p + "_b"] = (Do,)
    else:
        s.update(qkv_w=(3 * Do, Di), qkv_b=(3 * Do,))
    s.update(o_w=(Do, Do), o_b=(Do,), ln2_g=(Do,), ln2_b=(Do,),
             fc1_w=(M, Do), fc1_b=(M,), fc2_w=(Do, M), fc2_b=(Do,))
    return s


def make_inputs(spec, seed=0, qk_gain=1.0):
    """Draw every input of one block as float32 numpy arrays (bf16-rounded
    where the workload is bf16). ``qk_gain`` scales the query and key weight
    rows after drawing (the sharp-softmax stress variant); 1.0 is the plain
    workload. Adds the RoPE table under "rope" when the workload uses it."""
    out = {}
    bf16 = spec["dtype"] == "bf16"
    Do = spec["dim_out"]
    for name, shape in tensor_shapes(spec).items():
        rng = np.random.default_rng([seed, _TENSOR_IDS[name]])
        if name == "x":
            a = rng.standard_normal(shape)
        elif name.endswith("_w"):
            a = rng.normal(0.0, 0.02, shape)
        elif name.endswith("_g"):
            a = 1.0 + rng.normal(0.0, 0.1, shape)
        elif name.endswith("_b") and name.startswith("ln"):
            a = rng.normal(0.0, 0.1, shape)
        else:
            a = rng.normal(0.0, 0.01, shape)
        if qk_gain != 1.0:
            if name == "qkv_w":
                a[:2 * Do] *= qk_gain
            elif name in ("q_w", "k_w"):
                a *= qk_gain
        a = a.astype(np.float32)
        if bf16 and (name == "x" or name.endswith("_w")):
            a = bf16_round(a)
        out[name] = a
    if spec["rope"]:
        hd = Do // spec["heads"]
        if spec["mode"] == "spatial":
            out["rope"] = axial_rope_table(spec["win_h"], spec["win_w"], hd, spec["theta"])
        else:
            out["rope"] = axial_rope_table(spec["grid_h"], spec["grid_w"], hd, spec["theta"])
    return out


# Hiera stage stack (the Hiera plan's "Architecture Summary"): 24 blocks in
# four stages; stage s has width 112*2^s, 2^(s+1) heads of 56, mask units of
# 64/4^s tokens (mask-unit attention in stages 0-1, global in 2-3); the first
# block of stages 1-3 is a transition (projection + 2x2 max-pool, q_stride 4);
# features are taken after the last block of each stage. MLP ratio 4.
HIERA_STAGE_BLOCKS = (2, 3, 16, 3)
HIERA_UNROLL_LEVELS = 3


def hiera_stack(side=128, batch=1, stage_blocks=HIERA_STAGE_BLOCKS, dtype="bf16"):
    """Block specs of a Hiera stage stack on a side x side token grid (128 at a
    512x512 input), the unroll levels and the feature taps (block indices)."""
    specs, taps = [], []
    dim, grid = 112, side
    for stage, nb in enumerate(stage_blocks):
        for j in range(nb):
            trans = stage > 0 and j == 0
            d_in = dim // 2 if trans else dim
            g_in = grid * 2 if trans else grid
            mask_unit = stage < 2
            window = 64 // 4 ** stage  # tokens per mask unit at this stage's grid
            sp = _spec("hiera_b%d" % len(specs), batch=batch, grid_h=g_in, grid_w=g_in,
                       dim_in=d_in, dim_out=dim, heads=2 ** (stage + 1), mlp=4 * dim,
                       mode="mask_unit" if mask_unit else "global",
                       n_windows=(grid * grid) // window if mask_unit else 1,
                       q_stride=4 if trans else 1, dtype=dtype)
            specs.append(sp)
        taps.append(len(specs) - 1)
        dim, grid = dim * 2, grid // 2
    return specs, HIERA_UNROLL_LEVELS, taps


def make_stack_inputs(specs, seed=0):
    """Raster-order token input of the first block and every block's weights
    (block i draws with seed (seed, i) through make_inputs)."""
    blocks = []
    x = None
    for i, sp in enumerate(specs):
        w = make_inputs(sp, seed=seed * 1000 + i)
        if i == 0:
            x = w["x"]
        del w["x"]
        blocks.append(w)
    return x, blocks


# SAM3 ViT trunk (SAM3 page, trunk constants and block loop): LayerNorm
# ln_pre, then 32 blocks of width 1024, 16 heads, MLP 4736, 24x24 windows
# with in-window RoPE except layers 7, 15, 23, 31 (global, grid RoPE).
SAM3_GLOBAL_LAYERS = (7, 15, 23, 31)


def sam3_trunk(grid=72, win=24, layers=32, global_layers=SAM3_GLOBAL_LAYERS, dim=1024, heads=16, mlp=4736):
    """Block specs of a SAM3-style trunk (ln_pre comes before block 0)."""
    specs = []
    for l in range(layers):
        base = CONFIGS["c5g_sam3_global"] if l in global_layers else CONFIGS["c5w_sam3_win"]
        kw = dict(name="sam3_l%d" % l, grid_h=grid, grid_w=grid, dim_in=dim, dim_out=dim, heads=heads, mlp=mlp)
        if l not in global_layers:
            kw.update(win_h=win, win_w=win)
        specs.append(derive(base, **kw))
    return specs


# SigLIP tower (SigLIP page, ``forward_frame``): 12 pre-LN blocks of width 768,
# then the final post_layernorm; frames batched.
def siglip_tower(batch=8, grid=32, layers=12, dim=768, heads=12, mlp=3072):
    return [derive(CONFIGS["c4_siglip_b8"], name="siglip_l%d" % l, batch=batch, grid_h=grid, grid_w=grid,
                   dim_in=dim, dim_out=dim, heads=heads, mlp=mlp) for l in range(layers)]


def make_layernorm_params(dim, seed):
    """gamma 1 + N(0, 0.1), beta N(0, 0.1) (as the blocks' LayerNorms), float32;
    streams keyed by (seed, 100) and (seed, 101)."""
    g = 1.0 + np.random.default_rng([seed, 100]).normal(0.0, 0.1, (dim,))
    b = np.random.default_rng([seed, 101]).normal(0.0, 0.1, (dim,))
    return g.astype(np.float32), b.astype(np.float32)


def out_tokens(spec):
    """Tokens per frame leaving the block (4x fewer at a pooled transition)."""
    return spec["grid_h"] * spec["grid_w"] // spec["q_stride"]


# Patch-embedding stems: the step that turns pixels into the token grid the
# blocks consume. Hiera (Hiera plan, "Architecture Summary"): 4-channel NHWC
# pixels, Conv2d 4 -> 112, 7x7, stride 4 (padding 3, the one that keeps the
# 512 -> 128 shape contract symmetric), weight stored (112, 7, 7, 4), plus a
# learned position table of one row per token. SigLIP (SigLIP page,
# ``embed_frame``): NCHW frames, Conv 3 -> 768, 16x16, stride 16 with bias,
# plus a 32x32 position table looked up by bucketized coordinates. SAM3
# (SAM3 page, trunk patch step): 3 x 1008 x 1008, Conv 3 -> 1024, 14x14,
# stride 14 without bias, plus a 24x24 table tiled over the 72x72 grid.
STEMS = {
    "hiera": dict(name="hiera_stem", batch=1, in_h=512, in_w=512, in_ch=4, layout="nhwc", kernel=7, stride=4,
                  pad=3, dim=112, weight_layout="ohwi", bias=True, pos_mode="rows", pos_side=0, dtype="bf16"),
    "siglip": dict(name="siglip_stem", batch=8, in_h=512, in_w=512, in_ch=3, layout="nchw", kernel=16, stride=16,
                   pad=0, dim=768, weight_layout="oihw", bias=True, pos_mode="bucket", pos_side=32, dtype="bf16"),
    "sam3": dict(name="sam3_stem", batch=1, in_h=1008, in_w=1008, in_ch=3, layout="nchw", kernel=14, stride=14,
                 pad=0, dim=1024, weight_layout="oihw", bias=False, pos_mode="tile", pos_side=24, dtype="bf16"),
}

_STEM_IDS = {"pixels": 40, "weight": 41, "bias": 42, "pos": 43}


def stem_out_grid(spec):
    """(out_h, out_w) of the convolution: floor((in + 2 pad - kernel) / stride) + 1."""
    k, s, p = spec["kernel"], spec["stride"], spec["pad"]
    return (spec["in_h"] + 2 * p - k) // s + 1, (spec["in_w"] + 2 * p - k) // s + 1


def stem_shapes(spec):
    B, C, k, D = spec["batch"], spec["in_ch"], spec["kernel"], spec["dim"]
    oh, ow = stem_out_grid(spec)
    pix = (B, C, spec["in_h"], spec["in_w"]) if spec["layout"] == "nchw" else (B, spec["in_h"], spec["in_w"], C)
    w = (D, C, k, k) if spec["weight_layout"] == "oihw" else (D, k, k, C)
    rows = oh * ow if spec["pos_mode"] == "rows" else spec["pos_side"] ** 2
    shapes = {"pixels": pix, "weight": w, "pos": (rows, D)}
    if spec["bias"]:
        shapes["bias"] = (D,)
    if spec["pos_mode"] == "none":
        del shapes["pos"]
    return shapes


def make_stem_inputs(spec, seed=0):
    """Pixels U(-1, 1) (the normalised range the towers feed), weight
    N(0, 0.02), bias N(0, 0.01), position table N(0, 0.02); float32, with
    pixels and weight rounded to bf16 for the bf16 stems."""
    out = {}
    for name, shape in stem_shapes(spec).items():
        rng = np.random.default_rng([seed, _STEM_IDS[name]])
        if name == "pixels":
            a = rng.uniform(-1.0, 1.0, shape)
        elif name == "weight":
            a = rng.normal(0.0, 0.02, shape)
        elif name == "bias":
            a = rng.normal(0.0, 0.01, shape)
        else:
            a = rng.normal(0.0, 0.02, shape)
        a = a.astype(np.float32)
        if spec["dtype"] == "bf16" and name in ("pixels", "weight"):
            a = bf16_round(a)
        out[name] = a
    return out


# q8_row weights (the SAM3 page's quantized tensor type: one int8 per element
# and a float16 scale per row). Synthetic checkpoints are made the way a
# converter would: per row, scale = max|w| / 127 rounded to float16, payload
# = w / scale rounded to the nearest integer and clipped to [-127, 127].
def quantize_q8_row(w):
    w = np.asarray(w, dtype=np.float64)
    amax = np.abs(w).max(axis=1)
    scale = np.where(amax > 0, amax / 127.0, 1.0).astype(np.float16)
    q = np.clip(np.rint(w / scale.astype(np.float64)[:, None]), -127, 127).astype(np.int8)
    return q, scale


def make_q8_inputs(spec, seed=0, qk_gain=1.0):
    """make_inputs with every weight matrix "<name>_w" replaced by its int8
    payload and a float16 row scale under "<name>_s"."""
    out = make_inputs(spec, seed, qk_gain)
    for name in [k for k in out if k.endswith("_w")]:
        out[name], out[name[:-2] + "_s"] = quantize_q8_row(out[name])
    return out
