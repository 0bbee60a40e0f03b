"""Helpers for the GPU parity tests: move synthetic inputs to the device,
run the block through the C ABI, and measure errors against the oracle."""
import numpy as np
import torch

from vision_transformer_encoder_vit_amd import binding as vb
from vision_transformer_encoder_vit_amd import synth

# rel = max|got - ref| / max|ref| (the GPU-vs-CPU gate form on the SAM3
# page's attention test); bf16 path 2e-2; fp32 path 1e-4 in both rel and
# absolute terms.
BF16_REL = 2e-2
F32_TOL = 1e-4


def torch_dtype(spec):
    return torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32


def to_device(inp, spec):
    dt = torch_dtype(spec)
    dev = {}
    for k, a in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        if (k == "x" or k.endswith("_w")) and a.dtype != np.int8:
            t = t.to(dt)  # exact: the values are already representable in dt
        # int8 payloads and float16 row scales of q8_row weights stay as they are
        dev[k] = t.to("cuda")
    return dev


def seam_shapes(spec):
    B = spec["batch"]
    n_in = spec["grid_h"] * spec["grid_w"]
    n_out = n_in // spec["q_stride"]
    Di, Do, F = spec["dim_in"], spec["dim_out"], spec["mlp"]
    s = {"h": (B, n_in, Di), "qkv": (B, n_in, 3 * Do), "r": (B, n_out, Do), "ctx": (B, n_out, Do),
         "attn_branch": (B, n_out, Do), "x1": (B, n_out, Do), "h2": (B, n_out, Do),
         "u": (B, n_out, F), "mlp_branch": (B, n_out, Do)}
    if spec["q_stride"] == 4:
        s["q_pooled"] = (B, n_out, Do)
    return s


def run_block(spec, dev, seams=True, x=None, out=None):
    """Run one block forward on the GPU; returns (y tensor, seam tensors)."""
    plan = vb.Plan(vb.desc_from_spec(spec))
    dt = torch_dtype(spec)
    x = dev["x"] if x is None else x
    B, n_out = spec["batch"], synth.out_tokens(spec)
    y = torch.empty((B, n_out, spec["dim_out"]), dtype=dt, device="cuda") if out is None else out
    ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
    w = vb.weights_struct(dev)
    bufs = {}
    if seams:
        bufs = {k: torch.empty(s, dtype=dt, device="cuda") for k, s in seam_shapes(spec).items()}
        plan.forward_seams(w, x, y, bufs, ws)
    else:
        plan.forward(w, x, y, ws)
    torch.cuda.synchronize()
    plan.close()
    return y, bufs


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    d = np.abs(got - ref)
    denom = np.abs(ref).max()
    return float(d.max()), float(d.max() / denom) if denom > 0 else float(d.max())


def check(name, got, ref, spec):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name + ": non-finite values"
    mx, rel = errors(got, ref)
    if spec["dtype"] == "bf16":
        assert rel <= BF16_REL, "%s: rel %.3e > %.0e (max abs %.3e)" % (name, rel, BF16_REL, mx)
    else:
        assert mx <= F32_TOL and rel <= F32_TOL, "%s: max abs %.3e rel %.3e > %.0e" % (name, mx, rel, F32_TOL)
    return mx, rel
