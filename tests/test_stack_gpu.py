"""Hiera stage stack on the GPU (vit_stack_* through the C ABI) against the
float64 stack oracle: Unroll once, the blocks in order, Reroll at each
stage end."""
import numpy as np
import pytest
import torch

from oracle import stack as ost
from tests import gpu_util as gu
from vision_transformer_encoder_vit_amd import binding as vb
from vision_transformer_encoder_vit_amd import synth

pytestmark = pytest.mark.gpu


def _run_stack(specs, levels, taps, x, blocks):
    dt = gu.torch_dtype(specs[0])
    dev_w = [gu.to_device(w, sp) for w, sp in zip(blocks, specs)]
    weights = [vb.weights_struct(w) for w in dev_w]
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()
    st = vb.Stack([vb.desc_from_spec(s) for s in specs], levels, taps)
    feats = []
    for t in taps:
        sp = specs[t]
        feats.append(torch.empty((sp["batch"], synth.out_tokens(sp), sp["dim_out"]), dtype=dt, device="cuda"))
    ws = torch.empty(st.workspace_bytes, dtype=torch.uint8, device="cuda")
    st.forward(weights, xd, feats, ws)
    torch.cuda.synchronize()
    st.close()
    return feats, dev_w, xd


@pytest.mark.parametrize("side,stage_blocks", [(32, (2, 2, 2, 2)), (128, synth.HIERA_STAGE_BLOCKS)],
                         ids=["32x32_8blocks", "hiera_512_24blocks"])
def test_stack_vs_oracle(side, stage_blocks):
    specs, levels, taps = synth.hiera_stack(side=side, stage_blocks=stage_blocks)
    print("case stack", side, stage_blocks, flush=True)
    x, blocks = synth.make_stack_inputs(specs, seed=0)
    feats, _, _ = _run_stack(specs, levels, taps, x, blocks)
    ref = ost.stack_forward(x, blocks, specs, levels, taps)
    for k, (got, want) in enumerate(zip(feats, ref)):
        g = gu.to64(got)
        assert g.shape == want.shape and np.all(np.isfinite(g))
        # Gate of a stack of bf16 blocks (a reading): the bf16 roundings of
        # the residual stream add up over the blocks, and each transition
        # replaces the stream by a projection about 5x smaller, so errors
        # made before it grow relative to what follows (measured: norm-wise
        # 3e-3 after 2 blocks, ~6e-3 after the first transition, ~1.2e-2
        # after the second and third, whether 8 or 24 blocks). Taken: the
        # tower gate form of the SigLIP page (cosine >= 0.9999 per output)
        # and the single block's 2e-2 applied norm-wise.
        a, b = g.ravel(), want.ravel()
        cos = float(a @ b / np.sqrt((a @ a) * (b @ b)))
        nrel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
        mrel = float(np.abs(a - b).max() / np.abs(b).max())
        print("feature %d (after block %d): cos %.7f norm-rel %.2e max-rel %.2e" % (k, taps[k], cos, nrel, mrel))
        assert cos >= 0.9999 and nrel <= 2e-2 and mrel <= STACK_MAX_REL, (k, cos, nrel, mrel)


def test_stack_equals_chained_single_calls():
    # the native stack is exactly vit_unroll -> vit_block_forward per block ->
    # vit_reroll at the taps, bit for bit
    specs, levels, taps = synth.hiera_stack(side=32, stage_blocks=(1, 2, 2, 1))
    x, blocks = synth.make_stack_inputs(specs, seed=1)
    feats, dev_w, xd = _run_stack(specs, levels, taps, x, blocks)
    H = W = specs[0]["grid_h"]
    cur = torch.empty_like(xd)
    vb.vit_unroll(xd, cur, H, W, levels)
    k = 0
    for i, (sp, w) in enumerate(zip(specs, dev_w)):
        plan = vb.Plan(vb.desc_from_spec(sp))
        out = torch.empty((sp["batch"], synth.out_tokens(sp), sp["dim_out"]), dtype=xd.dtype, device="cuda")
        ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
        plan.forward(vb.weights_struct(w), cur, out, ws)
        plan.close()
        cur = out
        if sp["q_stride"] == 4:
            levels -= 1
            H, W = H // 2, W // 2
        if i in taps:
            f = torch.empty_like(cur)
            vb.vit_reroll(cur, f, H, W, levels)
            torch.cuda.synchronize()
            assert torch.equal(f.view(torch.int16), feats[k].view(torch.int16)), i
            k += 1


def _tower_gpu(specs, x, blocks, pre_ln=None, post_ln=None):
    """vit_layernorm (ln_pre) -> vit_stack (levels 0, one tap) -> vit_layernorm (post_ln)."""
    dt = gu.torch_dtype(specs[0])
    dev_w = [gu.to_device(w, sp) for w, sp in zip(blocks, specs)]
    weights = [vb.weights_struct(w) for w in dev_w]
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()
    if pre_ln is not None:
        g, b = (torch.from_numpy(a).cuda() for a in pre_ln)
        vb.vit_layernorm(xd, xd, g, b, specs[0]["eps"])
    st = vb.Stack([vb.desc_from_spec(s) for s in specs], 0, [len(specs) - 1])
    last = specs[-1]
    y = torch.empty((last["batch"], synth.out_tokens(last), last["dim_out"]), dtype=dt, device="cuda")
    ws = torch.empty(st.workspace_bytes, dtype=torch.uint8, device="cuda")
    st.forward(weights, xd, [y], ws)
    if post_ln is not None:
        g, b = (torch.from_numpy(a).cuda() for a in post_ln)
        vb.vit_layernorm(y, y, g, b, last["eps"])
    torch.cuda.synchronize()
    st.close()
    return gu.to64(y)


# Element-wise bound of a stack or tower output: max|got - ref| / max|ref|
# (the block's rel form). A block holds it to 2e-2; through a chain of bf16
# blocks the per-block roundings add up, so the chain takes twice that.
STACK_MAX_REL = 4e-2


def _tower_gate(name, got, want):
    a, b = got.ravel(), want.ravel()
    cos = float(a @ b / np.sqrt((a @ a) * (b @ b)))
    nrel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    mrel = float(np.abs(a - b).max() / np.abs(b).max())
    print("%s: cos %.7f norm-rel %.2e max-rel %.2e" % (name, cos, nrel, mrel))
    assert np.all(np.isfinite(got)) and cos >= 0.9999 and nrel <= 2e-2 and mrel <= STACK_MAX_REL, \
        (name, cos, nrel, mrel)


def test_sam3_trunk_reduced_vs_oracle():
    # ln_pre, then windowed layers with in-window RoPE and two global layers
    # with grid RoPE (the SAM3 trunk pattern at 48x48 tokens, width 256)
    specs = synth.sam3_trunk(grid=48, layers=8, global_layers=(3, 7), dim=256, heads=4, mlp=1024)
    x, blocks = synth.make_stack_inputs(specs, seed=2)
    ln = synth.make_layernorm_params(256, 2)
    got = _tower_gpu(specs, x, blocks, pre_ln=ln)
    _tower_gate("sam3 trunk 8 layers", got, ost.tower_forward(x, blocks, specs, pre_ln=ln))


def test_sam3_trunk_full_grid_vs_oracle():
    # the SAM3 trunk at its real grid and width (72x72 tokens, D 1024, 16
    # heads): ln_pre, two windowed layers (24x24 windows, in-window RoPE), a
    # global layer (grid RoPE) and a windowed layer, every output element
    # against the oracle
    specs = synth.sam3_trunk(grid=72, layers=4, global_layers=(2,))
    print("case sam3 trunk 72x72 4 layers", flush=True)
    x, blocks = synth.make_stack_inputs(specs, seed=5)
    ln = synth.make_layernorm_params(1024, 5)
    got = _tower_gpu(specs, x, blocks, pre_ln=ln)
    _tower_gate("sam3 trunk 72x72 x 4 layers", got, ost.tower_forward(x, blocks, specs, pre_ln=ln))


def test_siglip_tower_batch8_vs_oracle():
    # the SigLIP tower on a batch of 8 frames (12 blocks + post_layernorm);
    # frames never mix, so the oracle evaluates two of them (0 and 5)
    specs = synth.siglip_tower(batch=8)
    print("case siglip tower batch 8", flush=True)
    x, blocks = synth.make_stack_inputs(specs, seed=6)
    ln = synth.make_layernorm_params(768, 6)
    got = _tower_gpu(specs, x, blocks, post_ln=ln)
    two = [synth.derive(s, batch=2) for s in specs]
    want = ost.tower_forward(x[[0, 5]], blocks, two, post_ln=ln)
    for i, f in enumerate((0, 5)):
        _tower_gate("siglip tower batch 8, frame %d" % f, got[f], want[i])


def test_siglip_tower_full_frame_vs_oracle():
    # the SigLIP tower at full size for one frame: 12 blocks + post_layernorm
    specs = synth.siglip_tower(batch=1)
    x, blocks = synth.make_stack_inputs(specs, seed=3)
    ln = synth.make_layernorm_params(768, 3)
    got = _tower_gpu(specs, x, blocks, post_ln=ln)
    _tower_gate("siglip tower 12 layers", got, ost.tower_forward(x, blocks, specs, post_ln=ln))


def _embed_gpu(stem, sin):
    dt = gu.torch_dtype(stem)
    oh, ow = synth.stem_out_grid(stem)
    desc = vb.stem_desc_from_spec(stem)
    tok = torch.empty((stem["batch"], oh * ow, stem["dim"]), dtype=dt, device="cuda")
    ws = torch.empty(vb.vit_patch_embed_workspace_size(desc), dtype=torch.uint8, device="cuda")
    vb.vit_patch_embed(desc, torch.from_numpy(sin["pixels"]).cuda(), torch.from_numpy(sin["weight"]).to(dt).cuda(),
                       torch.from_numpy(sin["bias"]).cuda() if "bias" in sin else None,
                       torch.from_numpy(sin["pos"]).cuda(), tok, ws)
    return tok


@pytest.mark.parametrize("kind", ["siglip", "sam3", "hiera"])
def test_tower_from_pixels(kind):
    # stem -> (ln_pre) -> blocks -> (post_layernorm), all on the GPU, against
    # the stem oracle feeding the tower / stack oracle. SigLIP: one full
    # frame and all 12 layers; SAM3: a 336x336 image (24x24 tokens, 12x12
    # windows) into a narrowed 8-layer trunk; Hiera: the 512x512 backbone.
    from oracle import stem as ostem
    print("case tower from pixels", kind, flush=True)
    if kind == "siglip":
        stem = dict(synth.STEMS["siglip"], batch=1)
        specs, levels, taps = synth.siglip_tower(batch=1), 0, [11]
        pre, post = None, synth.make_layernorm_params(768, 4)
    elif kind == "sam3":
        stem = dict(synth.STEMS["sam3"], in_h=336, in_w=336, dim=256, pos_side=12)
        specs = synth.sam3_trunk(grid=24, win=12, layers=8, global_layers=(3, 7), dim=256, heads=4, mlp=1024)
        levels, taps = 0, [7]
        pre, post = synth.make_layernorm_params(256, 4), None
    else:
        stem = synth.STEMS["hiera"]
        specs, levels, taps = synth.hiera_stack()
        pre = post = None
    sin = synth.make_stem_inputs(stem, seed=4)
    _, blocks = synth.make_stack_inputs(specs, seed=4)
    tok = _embed_gpu(stem, sin)
    x_ref = ostem.patch_embed(sin, stem)
    if kind == "hiera":
        dt = gu.torch_dtype(specs[0])
        dev_w = [gu.to_device(w, sp) for w, sp in zip(blocks, specs)]
        st = vb.Stack([vb.desc_from_spec(s) for s in specs], levels, taps)
        feats = [torch.empty((1, synth.out_tokens(specs[t]), specs[t]["dim_out"]), dtype=dt, device="cuda")
                 for t in taps]
        ws = torch.empty(st.workspace_bytes, dtype=torch.uint8, device="cuda")
        st.forward([vb.weights_struct(w) for w in dev_w], tok, feats, ws)
        torch.cuda.synchronize()
        st.close()
        ref = ost.stack_forward(x_ref, blocks, specs, levels, taps)
        for k, (f, r) in enumerate(zip(feats, ref)):
            _tower_gate("hiera from pixels, feature %d" % k, gu.to64(f), r)
    else:
        got = _tower_gpu(specs, gu.to64(tok), blocks, pre_ln=pre, post_ln=post)
        _tower_gate("%s from pixels" % kind, got, ost.tower_forward(x_ref, blocks, specs, pre_ln=pre, post_ln=post))


def test_stack_batch_of_two_frames():
    # two frames through an 8-block Hiera stack: each frame's features equal
    # the oracle's, and frame 1 equals a one-frame run of its own input
    specs, levels, taps = synth.hiera_stack(side=32, batch=2, stage_blocks=(2, 2, 2, 2))
    print("case stack batch 2", flush=True)
    x, blocks = synth.make_stack_inputs(specs, seed=7)
    feats, _, _ = _run_stack(specs, levels, taps, x, blocks)
    ref = ost.stack_forward(x, blocks, specs, levels, taps)
    for k, (f, r) in enumerate(zip(feats, ref)):
        _tower_gate("batch-2 stack feature %d" % k, gu.to64(f), r)
    one = [synth.derive(s, batch=1) for s in specs]
    feats1, _, _ = _run_stack(one, levels, taps, x[1:], blocks)
    for f2, f1 in zip(feats, feats1):
        assert torch.equal(f2[1:].view(torch.int16), f1.view(torch.int16))


def test_stack_forward_is_graph_capturable():
    # the stack forward allocates nothing and never synchronises: captured
    # into a HIP graph, every replay equals the eager features bit for bit
    specs, levels, taps = synth.hiera_stack(side=32, stage_blocks=(2, 2, 2, 2))
    x, blocks = synth.make_stack_inputs(specs, seed=8)
    eager, dev_w, xd = _run_stack(specs, levels, taps, x, blocks)
    weights = [vb.weights_struct(w) for w in dev_w]
    st = vb.Stack([vb.desc_from_spec(s) for s in specs], levels, taps)
    feats = [torch.empty_like(f) for f in eager]
    ws = torch.empty(st.workspace_bytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        st.forward(weights, xd, feats, ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st.forward(weights, xd, feats, ws, stream=s)
    torch.cuda.synchronize()
    for i in range(3):
        for f in feats:
            f.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for f, e in zip(feats, eager):
            assert torch.equal(f.view(torch.int16), e.view(torch.int16)), i
    st.close()
