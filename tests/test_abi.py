"""The C ABI on the CPU (no kernel is launched): the library loads, exports
every entry point the header declares, and rejects bad arguments with the
documented status before touching any buffer."""
import ctypes
import os
import re

import pytest

from vision_transformer_encoder_vit_amd import binding as vb
from vision_transformer_encoder_vit_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "vit_block.h")).read()
    names = set(re.findall(r"^\s*(?:vit_status|const char\*)\s+(vit_\w+)\s*\(", hdr, re.M))
    assert len(names) >= 10
    for n in names:
        assert hasattr(vb.lib, n), n


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(vb.vit_block_desc) == 20 * 4
    assert ctypes.sizeof(vb.vit_block_weights) == 29 * 8
    assert ctypes.sizeof(vb.vit_block_seams) == 10 * 8
    assert ctypes.sizeof(vb.vit_patch_embed_desc) == 13 * 4


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_create_every_workload(name):
    p = vb.Plan(vb.desc_from_spec(synth.CONFIGS[name]))
    assert p.workspace_bytes > 0 and p.workspace_bytes % 256 == 0
    p.close()


def _desc(**kw):
    d = vb.desc_from_spec(synth.CONFIGS["c5w_sam3_win"])
    for k, v in kw.items():
        setattr(d, k, v)
    return d


BAD = [
    (dict(batch=0), vb.VIT_ERR_INVALID_ARG, "batch"),
    (dict(grid_h=0), vb.VIT_ERR_INVALID_ARG, "grid"),
    (dict(dim_in=1020, dim_out=1020), vb.VIT_ERR_INVALID_ARG, "multiples of 8"),
    (dict(heads=6), vb.VIT_ERR_INVALID_ARG, "heads"),
    (dict(heads=8), vb.VIT_ERR_UNSUPPORTED, "head_dim 128"),
    (dict(heads=256), vb.VIT_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(q_stride=2), vb.VIT_ERR_INVALID_ARG, "q_stride"),
    (dict(dim_in=512), vb.VIT_ERR_INVALID_ARG, "residual projection"),
    (dict(win_h=25), vb.VIT_ERR_INVALID_ARG, "tile"),
    (dict(attn_mode=7), vb.VIT_ERR_INVALID_ARG, "attn_mode"),
    (dict(gelu=5), vb.VIT_ERR_INVALID_ARG, "gelu"),
    (dict(rope_rows=5184), vb.VIT_ERR_INVALID_ARG, "rope_rows"),
    (dict(attn_mode=vb.VIT_ATTN_MASK_UNIT, n_windows=9), vb.VIT_ERR_UNSUPPORTED, "RoPE"),
    (dict(ln_eps=0.0), vb.VIT_ERR_INVALID_ARG, "ln_eps"),
    (dict(ln_eps=float("nan")), vb.VIT_ERR_INVALID_ARG, "ln_eps"),
    (dict(attn_scale=-1.0), vb.VIT_ERR_INVALID_ARG, "attn_scale"),
    (dict(act_dtype=9), vb.VIT_ERR_INVALID_ARG, "act_dtype"),
    (dict(rope=0, q_stride=4, dim_in=512), vb.VIT_ERR_UNSUPPORTED, "SPATIAL"),
    (dict(weight_format=3), vb.VIT_ERR_INVALID_ARG, "weight_format"),
]


@pytest.mark.parametrize("kw,status,msg", BAD, ids=[str(b[0]) for b in BAD])
def test_create_rejects(kw, status, msg):
    h = ctypes.c_void_p()
    st = vb.lib.vit_block_create(ctypes.byref(_desc(**kw)), ctypes.byref(h))
    assert st == status, (st, vb.last_error())
    assert msg in vb.last_error()


def test_create_null_arguments():
    h = ctypes.c_void_p()
    assert vb.lib.vit_block_create(None, ctypes.byref(h)) == vb.VIT_ERR_INVALID_ARG
    assert vb.lib.vit_block_create(ctypes.byref(_desc()), None) == vb.VIT_ERR_INVALID_ARG


class FakeBuf:
    """A stand-in with a data_ptr(): validation fails before any access."""

    def __init__(self, addr, n=1 << 30):
        self.addr, self.n = addr, n

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def _weights(spec, misalign=None, drop=None):
    w = vb.vit_block_weights()
    addr = 0x100000
    for name in synth.tensor_shapes(spec):
        if name == "x":
            continue
        addr += 0x10000
        setattr(w, vb.WEIGHT_NAMES[name], addr + (4 if name == misalign else 0))
    if spec["rope"]:
        w.rope_table = 0x900000
    if drop:
        setattr(w, drop, None)
    return w


def _forward(spec, w, x, y, ws, ws_bytes):
    p = vb.Plan(vb.desc_from_spec(spec))
    st = vb.lib.vit_block_forward(p.handle, ctypes.byref(w), ctypes.c_void_p(x), ctypes.c_void_p(y),
                                  ctypes.c_void_p(ws), ws_bytes, None)
    need = p.workspace_bytes
    p.close()
    return st, need


def test_forward_rejects_before_launch():
    spec = synth.CONFIGS["c5w_sam3_win"]
    X, Y, WS = 0x10000000, 0x20000000, 0x30000000
    st, need = _forward(spec, _weights(spec, drop="w_fc1"), X, Y, WS, 1 << 30)
    assert st == vb.VIT_ERR_INVALID_ARG and "w_fc1" in vb.last_error()
    st, _ = _forward(spec, _weights(spec, drop="rope_table"), X, Y, WS, 1 << 30)
    assert st == vb.VIT_ERR_INVALID_ARG and "rope_table" in vb.last_error()
    st, _ = _forward(spec, _weights(spec, misalign="fc2_b"), X, Y, WS, 1 << 30)
    assert st == vb.VIT_ERR_INVALID_ARG and "aligned" in vb.last_error()
    st, _ = _forward(spec, _weights(spec), X, Y, WS, need - 256)
    assert st == vb.VIT_ERR_WORKSPACE
    st, _ = _forward(spec, _weights(spec), X, Y, 0, need)
    assert st == vb.VIT_ERR_WORKSPACE
    st, _ = _forward(spec, _weights(spec), X, X + 4096, WS, need)
    assert st == vb.VIT_ERR_INVALID_ARG and "overlap" in vb.last_error()
    st, _ = _forward(spec, _weights(spec), X, Y, Y + 4096, need)
    assert st == vb.VIT_ERR_INVALID_ARG and "workspace overlaps" in vb.last_error()
    st, _ = _forward(spec, _weights(spec), X + 8, Y, WS, need)
    assert st == vb.VIT_ERR_INVALID_ARG
    st, _ = _forward(spec, _weights(spec), 0, Y, WS, need)
    assert st == vb.VIT_ERR_INVALID_ARG
    trans = synth.CONFIGS["c3a_hiera_trans"]
    st, _ = _forward(trans, _weights(trans), X, X, WS, 1 << 30)
    assert st == vb.VIT_ERR_INVALID_ARG and "q_stride" in vb.last_error()
    st, _ = _forward(trans, _weights(trans, drop="w_res"), X, Y, WS, 1 << 30)
    assert st == vb.VIT_ERR_INVALID_ARG and "w_res" in vb.last_error()
    sep = synth.CONFIGS["c4_siglip_b8"]
    st, _ = _forward(sep, _weights(sep, drop="w_k"), X, Y, WS, 1 << 30)
    assert st == vb.VIT_ERR_INVALID_ARG and "w_k" in vb.last_error()


def test_seams_null_struct():
    spec = synth.CONFIGS["c2_hiera_s0"]
    p = vb.Plan(vb.desc_from_spec(spec))
    st = vb.lib.vit_block_forward_seams(p.handle, ctypes.byref(_weights(spec)), ctypes.c_void_p(0x10000000),
                                        ctypes.c_void_p(0x20000000), None, ctypes.c_void_p(0x30000000),
                                        p.workspace_bytes, None)
    assert st == vb.VIT_ERR_INVALID_ARG
    p.close()


def test_single_step_validation():
    L = vb.lib
    P = ctypes.c_void_p(0x10000)
    Q = ctypes.c_void_p(0x90000)
    assert L.vit_layernorm(P, Q, P, P, 4, 12, 1e-6, vb.VIT_DTYPE_BF16, None) == vb.VIT_ERR_INVALID_ARG
    assert L.vit_layernorm(P, Q, P, P, 4, 16, 0.0, vb.VIT_DTYPE_BF16, None) == vb.VIT_ERR_INVALID_ARG
    assert L.vit_layernorm(P, Q, P, P, 4, 16, 1e-6, 3, None) == vb.VIT_ERR_INVALID_ARG
    assert L.vit_layernorm(None, None, None, None, 0, 16, 1e-6, vb.VIT_DTYPE_BF16, None) == vb.VIT_OK  # empty
    assert L.vit_unroll(P, Q, 1, 12, 12, 3, 16, vb.VIT_DTYPE_BF16, None) == vb.VIT_ERR_INVALID_ARG
    assert L.vit_unroll(P, Q, 1, 16, 16, 9, 16, vb.VIT_DTYPE_BF16, None) == vb.VIT_ERR_INVALID_ARG
    assert L.vit_reroll(P, Q, 1, 16, 16, 2, 12, vb.VIT_DTYPE_BF16, None) == vb.VIT_ERR_INVALID_ARG
    assert L.vit_unroll(P, P, 1, 16, 16, 2, 16, vb.VIT_DTYPE_BF16, None) == vb.VIT_ERR_INVALID_ARG  # overlap
    assert L.vit_unroll(None, None, 0, 16, 16, 2, 16, vb.VIT_DTYPE_BF16, None) == vb.VIT_OK  # empty
    assert L.vit_pool4(P, 16, Q, 16, 1, 6, 16, vb.VIT_DTYPE_BF16, None) == vb.VIT_ERR_INVALID_ARG
    assert L.vit_pool4(P, 8, Q, 16, 1, 8, 16, vb.VIT_DTYPE_BF16, None) == vb.VIT_ERR_INVALID_ARG
    assert L.vit_pool4(None, 16, None, 16, 1, 0, 16, vb.VIT_DTYPE_BF16, None) == vb.VIT_OK


def test_stage_mask():
    names = vb.STAGES
    m = vb.Plan(vb.desc_from_spec(synth.CONFIGS["c2_hiera_s0"])).stage_mask()
    assert m == 1 << names.index("fused")
    m = vb.Plan(vb.desc_from_spec(synth.CONFIGS["c5w_sam3_win"])).stage_mask()
    assert not m >> names.index("residual") & 1 and m >> names.index("attn") & 1
    assert not m >> names.index("fused") & 1
    # a bf16 transition: the qkv GEMM also computes the pooled residual
    m = vb.Plan(vb.desc_from_spec(synth.CONFIGS["c3a_hiera_trans"])).stage_mask()
    assert not m >> names.index("residual") & 1 and m >> names.index("qkv") & 1
    # fp32 (VALU GEMM), or a qkv epilogue that writes V^T for global
    # attention: a residual stage of its own
    m = vb.Plan(vb.desc_from_spec(synth.derive(synth.CONFIGS["c3a_hiera_trans"], dtype="f32"))).stage_mask()
    assert m >> names.index("residual") & 1
    m = vb.Plan(vb.desc_from_spec(synth.derive(synth.CONFIGS["c3b_hiera_s2"], grid_h=32, grid_w=32, dim_in=224,
                                                dim_out=448, q_stride=4))).stage_mask()
    assert m >> names.index("residual") & 1


def _stack_descs(**kw):
    specs, levels, taps = synth.hiera_stack(**kw)
    return [vb.desc_from_spec(s) for s in specs], levels, taps


def test_stack_create_hiera_512():
    descs, levels, taps = _stack_descs()
    st = vb.Stack(descs, levels, taps)
    # two activation buffers of the largest token tensor (16384 x 224 bf16
    # entering/leaving block 2 is the largest) plus a block workspace
    assert st.workspace_bytes >= 2 * 16384 * 224 * 2
    st.close()


def test_stack_create_rejects():
    descs, levels, taps = _stack_descs(side=32, stage_blocks=(1, 1, 1, 1))
    cases = [
        (dict(levels=3, taps=[1, 0]), "taps must be increasing"),
        (dict(levels=3, taps=[4]), "taps must be increasing"),
        (dict(levels=2, taps=taps), "none left"),          # three pools, two levels
        (dict(levels=6, taps=taps), "not divisible"),      # 32x32 grid, 2^6
    ]
    for kw, msg in cases:
        with pytest.raises(vb.VitError) as e:
            vb.Stack(descs, kw["levels"], kw["taps"])
        assert msg in str(e.value), (kw, str(e.value))
    bad = list(descs)
    d = vb.desc_from_spec(synth.derive(synth.hiera_stack(side=32, stage_blocks=(1, 1, 1, 1))[0][1], dim_in=112 + 8))
    bad[1] = d
    with pytest.raises(vb.VitError) as e:
        vb.Stack(bad, levels, taps)
    assert "does not take block 0" in str(e.value)
    with pytest.raises(vb.VitError):
        vb.Stack([], levels, [])


@pytest.mark.parametrize("kind", sorted(synth.STEMS))
def test_patch_embed_workspace_every_stem(kind):
    spec = synth.STEMS[kind]
    n = vb.vit_patch_embed_workspace_size(vb.stem_desc_from_spec(spec))
    oh, ow = synth.stem_out_grid(spec)
    K = spec["in_ch"] * spec["kernel"] ** 2
    Kp = -(-K // 64) * 64
    a = -(-(spec["batch"] * oh * ow * Kp * 2) // 256) * 256
    w = 0 if K == Kp else -(-(spec["dim"] * Kp * 2) // 256) * 256
    assert n == a + w and n % 256 == 0


@pytest.mark.parametrize("kw,msg", [
    (dict(batch=0), "batch"),
    (dict(kernel=0), "kernel"),
    (dict(pad=7), "pad"),
    (dict(stride=0), "stride"),
    (dict(dim=100), "dim"),
    (dict(in_h=3, pad=0), "fit"),
    (dict(pixel_layout=5), "layout"),
    (dict(weight_layout=2), "layout"),
    (dict(pos_mode=9), "pos_mode"),
    (dict(act_dtype=7), "dtype"),
])
def test_patch_embed_rejects(kw, msg):
    d = vb.stem_desc_from_spec(synth.STEMS["hiera"])
    for k, v in kw.items():
        setattr(d, k, v)
    n = ctypes.c_size_t()
    assert vb.lib.vit_patch_embed_workspace_size(ctypes.byref(d), ctypes.byref(n)) == vb.VIT_ERR_INVALID_ARG
    assert msg in vb.last_error()


def test_patch_embed_rejects_before_launch():
    L = vb.lib
    d = vb.stem_desc_from_spec(synth.STEMS["siglip"])
    need = vb.vit_patch_embed_workspace_size(d)
    PX, W, B, POS, T, WS = (ctypes.c_void_p(a) for a in (0x10000000, 0x20000000, 0x21000000, 0x22000000,
                                                          0x30000000, 0x40000000))
    call = lambda *a: L.vit_patch_embed(ctypes.byref(d), *a)
    assert call(PX, W, B, None, T, WS, need, None) == vb.VIT_ERR_INVALID_ARG and "pos" in vb.last_error()
    assert call(None, W, B, POS, T, WS, need, None) == vb.VIT_ERR_INVALID_ARG
    assert call(PX, W, B, POS, T, WS, need - 256, None) == vb.VIT_ERR_WORKSPACE
    assert call(PX, W, B, POS, T, None, need, None) == vb.VIT_ERR_WORKSPACE
    assert call(PX, W, ctypes.c_void_p(0x21000004), POS, T, WS, need, None) == vb.VIT_ERR_INVALID_ARG
    assert call(PX, W, B, POS, ctypes.c_void_p(0x10000000 + 4096), WS, need, None) == vb.VIT_ERR_INVALID_ARG
    assert "overlap" in vb.last_error()
    # the bucketized table needs the grid to be pos_side x pos_side
    d.pos_side = 16
    assert call(PX, W, B, POS, T, WS, need, None) == vb.VIT_ERR_INVALID_ARG and "BUCKET" in vb.last_error()


def test_q8_forward_needs_every_scale():
    # int8 weights: each matrix needs its float16 row scales
    for name, drop in [("c5w_sam3_win", "s_qkv"), ("c5w_sam3_win", "s_fc2"), ("c4_siglip_b8", "s_k")]:
        spec = dict(synth.CONFIGS[name], weights="q8_row")
        w = _weights(spec)
        for k, f in [("qkv_s", "s_qkv"), ("q_s", "s_q"), ("k_s", "s_k"), ("v_s", "s_v"), ("o_s", "s_o"),
                     ("fc1_s", "s_fc1"), ("fc2_s", "s_fc2")]:
            setattr(w, f, 0xA00000 + 0x1000 * len(k))
        setattr(w, drop, None)
        st, _ = _forward(spec, w, 0x10000000, 0x20000000, 0x30000000, 1 << 30)
        assert st == vb.VIT_ERR_INVALID_ARG and drop in vb.last_error(), (name, drop, vb.last_error())
    # the workspace grows by the act_dtype copies of the payloads (read by
    # the step kernels), and the single-kernel mask-unit path takes the int8
    # payloads directly
    spec = synth.CONFIGS["c2_hiera_s0"]
    p8, pb = vb.Plan(vb.desc_from_spec(dict(spec, weights="q8_row"))), vb.Plan(vb.desc_from_spec(spec))
    D, F = spec["dim_out"], spec["mlp"]
    mats = [(3 * D, D), (D, D), (F, D), (D, F)]
    assert p8.workspace_bytes - pb.workspace_bytes >= sum(2 * r * c for r, c in mats)
    assert pb.stage_mask() == p8.stage_mask() == 1 << vb.STAGES.index("fused")
    p8.close()
    pb.close()


def test_library_binds_torchs_hip_runtime():
    # the binding loads torch first, so the library resolves torch's runtime
    ours = vb._runtime_file(vb.lib)
    assert ours is not None and ours == vb._runtime_file(ctypes.CDLL(vb._torch_runtime_path()))


def test_second_hip_runtime_fails_loudly():
    # a process that mapped another libamdhip64 before torch (the system one
    # from /opt/rocm) would run the library in a context without torch's
    # memory and streams; the import must refuse instead of crashing later
    import subprocess
    import sys
    import glob
    other = sorted(glob.glob("/opt/rocm*/lib/libamdhip64.so.*"))
    if not other:
        pytest.skip("no system HIP runtime to map")
    code = ("import ctypes; ctypes.CDLL(%r); import sys; sys.path.insert(0, %r)\n"
            "try:\n    import vision_transformer_encoder_vit_amd.binding\nexcept ImportError as e:\n"
            "    print('REFUSED', e); raise SystemExit(0)\nraise SystemExit(3)\n") % (other[0], ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "REFUSED" in r.stdout and "HIP runtime" in r.stdout, r.stdout + r.stderr


def test_workspace_has_no_partials_for_a_split_inside_the_workgroup():
    # the 1024-token Hiera stage-2 block splits its keys four ways among the
    # waves of one workgroup: its workspace is the block's activations (h,
    # qkv, ctx, x1, h2, u and V^T, bf16), with no fp32 split partials
    spec = synth.CONFIGS["c3b_hiera_s2"]
    m, d, f = 1024, 448, 1792
    acts = 2 * m * (d + 3 * d + d + d + d + f + d)
    p = vb.Plan(vb.desc_from_spec(spec))
    try:
        assert p.workspace_bytes == acts
    finally:
        p.close()
    # a pooled 4096-key window splits over workgroups: fp32 partials (O and
    # the row max / sum per head) for each of its splits come on top
    pooled = synth.derive(spec, grid_h=64, grid_w=64, dim_in=448, dim_out=448, q_stride=4)
    p = vb.Plan(vb.desc_from_spec(pooled))
    try:
        mi, mo = 4096, 1024
        acts = 2 * (mi * (d + 3 * d + d) + mo * (d + d + d + d + f) + mi * d)
        assert p.workspace_bytes > acts + 2 * 4 * mo * d
    finally:
        p.close()
