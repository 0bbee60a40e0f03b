"""Algorithmic work of one encoder block: FLOPs of the dense contractions and
the minimum HBM bytes of the bandwidth-bound steps.

Conventions (the work the method must do; padding and layout costs are not
counted): a GEMM M x N x K is 2*M*N*K FLOPs; attention is 4*n_q*n_kv*hd per
(frame, window, head) (QK^T plus PV); a LayerNorm moves each activation once
in and once out; a 4x pool reads four rows and writes one.

Cross-check: the SigLIP page gives about 213 GFLOP for one 512x512 frame
through the 12-block tower plus its patch embedding; ``siglip_tower_gflop``
gives 213.7 with these conventions (tests/test_work.py).
"""

DTYPE_BYTES = {"bf16": 2, "f32": 4}


def gemm_flops(m, n, k):
    return 2.0 * m * n * k


def _tokens(spec):
    n_in = spec["grid_h"] * spec["grid_w"]
    return n_in, n_in // spec["q_stride"]


def gemms(spec):
    """Name -> (M, N, K) of every GEMM in one block forward."""
    B = spec["batch"]
    n_in, n_out = _tokens(spec)
    Di, Do, F = spec["dim_in"], spec["dim_out"], spec["mlp"]
    g = {"qkv": (B * n_in, 3 * Do, Di)}
    if spec["q_stride"] == 4:
        g["res"] = (B * n_in, Do, Di)
    g.update(proj=(B * n_out, Do, Do), fc1=(B * n_out, F, Do), fc2=(B * n_out, Do, F))
    return g


def attention_units(spec):
    """(count, n_q, n_kv) of the (frame, window, head) attention units."""
    B, H = spec["batch"], spec["heads"]
    n_in, n_out = _tokens(spec)
    if spec["mode"] == "mask_unit":
        nw = spec["n_windows"]
        return B * nw * H, n_out // nw, n_in // nw
    if spec["mode"] == "spatial":
        nw = n_in // (spec["win_h"] * spec["win_w"])
        return B * nw * H, n_in // nw, n_in // nw
    return B * H, n_out, n_in


def attention_flops(spec):
    cnt, nq, nkv = attention_units(spec)
    return 4.0 * cnt * nq * nkv * (spec["dim_out"] // spec["heads"])


def block_flops(spec):
    return sum(gemm_flops(*v) for v in gemms(spec).values()) + attention_flops(spec)


def layernorm_bytes(rows, dim, dtype):
    """One read and one write of every activation (gamma/beta are negligible
    and shared by all rows)."""
    return 2.0 * rows * dim * DTYPE_BYTES[dtype]


def attention_bytes(spec):
    """Minimum HBM traffic of the attention step: q, k, v read once (the
    q_stride-4 form reads all four pooled query rows), ctx written once."""
    e = DTYPE_BYTES[spec["dtype"]]
    B = spec["batch"]
    n_in, n_out = _tokens(spec)
    D = spec["dim_out"]
    return float(e * B * (3 * n_in * D + n_out * D))


def gemm_bytes(m, n, k, dtype, extra_rows_in=0):
    """Minimum HBM traffic of one GEMM: A and W read once, C written once
    (plus any residual rows read by the epilogue)."""
    e = DTYPE_BYTES[dtype]
    return float(e * (m * k + n * k + m * n + extra_rows_in * n))


def block_min_bytes(spec):
    """Minimum HBM traffic of a whole block: x read once, y written once,
    every weight matrix and vector read once."""
    from . import synth
    e = DTYPE_BYTES[spec["dtype"]]
    total = 0.0
    for name, shape in synth.tensor_shapes(spec).items():
        n = 1
        for s in shape:
            n *= s
        total += n * (e if (name == "x" or name.endswith("_w")) else 4)
    total += spec["batch"] * synth.out_tokens(spec) * spec["dim_out"] * e  # y
    return total


def block_tokens(spec):
    return spec["batch"] * spec["grid_h"] * spec["grid_w"]


def siglip_tower_gflop():
    """12 SigLIP-B/16 blocks plus the k16 s16 patch embedding on one 512x512
    frame (1024 tokens, width 768, 12 heads of 64, MLP 3072)."""
    spec = dict(batch=1, grid_h=32, grid_w=32, dim_in=768, dim_out=768, heads=12,
                mlp=3072, mode="global", q_stride=1, n_windows=1)
    embed = gemm_flops(1024, 768, 3 * 16 * 16)
    return (12 * block_flops(spec) + embed) / 1e9


def stage_work(spec, residual_in_qkv=False):
    """Algorithmic FLOPs and minimum HBM bytes of each stage."""
    e = DTYPE_BYTES[spec["dtype"]]
    B = spec["batch"]
    n_in = spec["grid_h"] * spec["grid_w"]
    m_in, m_out = B * n_in, B * n_in // spec["q_stride"]
    Di, Do = spec["dim_in"], spec["dim_out"]
    g = gemms(spec)
    w = {"ln1": (0.0, layernorm_bytes(m_in, Di, spec["dtype"])),
         "ln2": (0.0, layernorm_bytes(m_out, Do, spec["dtype"]))}
    w["qkv"] = (gemm_flops(*g["qkv"]), gemm_bytes(*g["qkv"], spec["dtype"]))
    if "res" in g:
        # projection of every input row, 4x max-pooled: h and W_res read
        # once, the pooled rows written once
        w["residual"] = (gemm_flops(*g["res"]), e * (m_in * Di + Do * Di + m_out * Do))
    else:
        w["residual"] = (0.0, 0.0)
    if residual_in_qkv and "res" in g:
        # the qkv GEMM also computes the pooled residual projection: its
        # stage carries that work (h is read once for both)
        f, by = w["qkv"]
        w["qkv"] = (f + w["residual"][0], by + e * (Do * Di + m_out * Do))
        w["residual"] = (0.0, 0.0)
    w["attn"] = (attention_flops(spec), attention_bytes(spec))
    w["proj"] = (gemm_flops(*g["proj"]), gemm_bytes(*g["proj"], spec["dtype"], extra_rows_in=m_out))
    w["fc1"] = (gemm_flops(*g["fc1"]), gemm_bytes(*g["fc1"], spec["dtype"]))
    w["fc2"] = (gemm_flops(*g["fc2"]), gemm_bytes(*g["fc2"], spec["dtype"], extra_rows_in=m_out))
    # whole block in one kernel: x in, y out, every weight once
    w["fused"] = (block_flops(spec), block_min_bytes(spec))
    return w
