"""vit_block_forward_static (the entry point that allocates nothing: its
workspace is the library's own device scratch) against vit_block_forward
with a caller workspace, through the C ABI: bit-identical outputs on two
calls in a row, the second on a smaller block, and a block whose workspace
exceeds the scratch refused before any launch."""
import numpy as np
import pytest
import torch

from tests import gpu_util as gu
from vision_transformer_encoder_vit_amd import binding as vb
from vision_transformer_encoder_vit_amd import synth

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


def _both(spec, seed):
    inp = synth.make_inputs(spec, seed=seed)
    dev = gu.to_device(inp, spec)
    plan = vb.Plan(vb.desc_from_spec(spec))
    assert plan.workspace_bytes <= vb.VIT_STATIC_SCRATCH_BYTES
    w = vb.weights_struct(dev)
    shape = (spec["batch"], synth.out_tokens(spec), spec["dim_out"])
    y_ref = torch.empty(shape, dtype=gu.torch_dtype(spec), device="cuda")
    ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
    plan.forward(w, dev["x"], y_ref, ws)
    y = torch.full(shape, float("nan"), dtype=gu.torch_dtype(spec), device="cuda")
    plan.forward_static(w, dev["x"], y)
    torch.cuda.synchronize()
    plan.close()
    return y, y_ref


def test_static_scratch_forward_equals_workspace_forward():
    # the SAM3 windowed block at full size (148 MiB of workspace), then a
    # smaller global block with a key split (its partials in the scratch)
    cases = [("c5w_sam3_win", C["c5w_sam3_win"]), ("c3b_hiera_s2", C["c3b_hiera_s2"])]
    for i, (name, spec) in enumerate(cases):
        print("case", name, flush=True)
        y, y_ref = _both(spec, seed=10 + i)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), name


def test_static_scratch_refuses_a_larger_workspace():
    spec = synth.derive(C["c4_siglip_b8"], batch=16)
    plan = vb.Plan(vb.desc_from_spec(spec))
    assert plan.workspace_bytes > vb.VIT_STATIC_SCRATCH_BYTES
    dev = gu.to_device(synth.make_inputs(synth.derive(spec, batch=1), seed=0), spec)
    x = torch.zeros((16, 1024, 768), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros_like(x)
    with pytest.raises(vb.VitError) as err:
        plan.forward_static(vb.weights_struct(dev), x, y)
    assert err.value.status == vb.VIT_ERR_WORKSPACE and "static scratch" in str(err.value)
    assert torch.count_nonzero(y) == 0
    plan.close()
