"""ctypes binding of libvitblock.so (include/vit_block.h), same names.

Argument marshalling only: tensors are passed as raw device pointers, the
stream as torch's current HIP stream. Every step of the block runs in the
library's HIP kernels; there is no other implementation behind these calls.
Importing this module raises if the built library is missing.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvitblock.so")

VIT_OK, VIT_ERR_INVALID_ARG, VIT_ERR_UNSUPPORTED, VIT_ERR_WORKSPACE, VIT_ERR_DEVICE = range(5)
VIT_STATIC_SCRATCH_BYTES = 256 << 20  # include/vit_block.h
VIT_DTYPE_F32, VIT_DTYPE_BF16 = 0, 1
VIT_ATTN_GLOBAL, VIT_ATTN_MASK_UNIT, VIT_ATTN_SPATIAL = 0, 1, 2
VIT_GELU_ERF, VIT_GELU_TANH = 0, 1
VIT_QKV_FUSED, VIT_QKV_SEPARATE = 0, 1
VIT_ROPE_NONE, VIT_ROPE_AXIAL_TABLE = 0, 1
VIT_WEIGHTS_ACT, VIT_WEIGHTS_Q8_ROW = 0, 1
VIT_PIXELS_NCHW, VIT_PIXELS_NHWC = 0, 1
VIT_CONV_OIHW, VIT_CONV_OHWI = 0, 1
VIT_POS_NONE, VIT_POS_ROWS, VIT_POS_BUCKET, VIT_POS_TILE = 0, 1, 2, 3
STAGES = ["ln1", "qkv", "residual", "attn", "proj", "ln2", "fc1", "fc2", "fused"]
VIT_NSTAGES = len(STAGES)

_i32, _f32, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class vit_block_desc(ctypes.Structure):
    _fields_ = [("batch", _i32), ("grid_h", _i32), ("grid_w", _i32), ("dim_in", _i32),
                ("dim_out", _i32), ("heads", _i32), ("mlp_hidden", _i32), ("attn_mode", _i32),
                ("n_windows", _i32), ("win_h", _i32), ("win_w", _i32), ("q_stride", _i32),
                ("gelu", _i32), ("qkv_layout", _i32), ("rope", _i32), ("rope_rows", _i32),
                ("ln_eps", _f32), ("attn_scale", _f32), ("act_dtype", _i32), ("weight_format", _i32)]


WEIGHT_FIELDS = ["ln1_gamma", "ln1_beta", "w_res", "b_res", "w_qkv", "b_qkv", "w_q", "b_q",
                 "w_k", "b_k", "w_v", "b_v", "w_o", "b_o", "ln2_gamma", "ln2_beta", "w_fc1",
                 "b_fc1", "w_fc2", "b_fc2", "rope_table", "s_res", "s_qkv", "s_q", "s_k", "s_v", "s_o",
                 "s_fc1", "s_fc2"]


class vit_block_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in WEIGHT_FIELDS]


SEAM_FIELDS = ["h", "qkv", "q_pooled", "r", "ctx", "attn_branch", "x1", "h2", "u", "mlp_branch"]


class vit_block_seams(ctypes.Structure):
    _fields_ = [(n, _vp) for n in SEAM_FIELDS]


class vit_patch_embed_desc(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("batch", "in_h", "in_w", "in_ch", "pixel_layout", "kernel", "stride", "pad",
                                     "dim", "weight_layout", "pos_mode", "pos_side", "act_dtype")]


class VitError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("vit status %d: %s" % (status, msg))
        self.status = status


def hip_runtimes_mapped():
    """Distinct HIP runtime libraries (libamdhip64*) mapped into this
    process, as real paths. Two of them means two HIP contexts: device memory
    and streams of one are invalid in the other."""
    found = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and os.path.basename(parts[5]).startswith("libamdhip64"):
                found.add(os.path.realpath(parts[5]))
    return sorted(found)


def _torch_runtime_path():
    import torch
    p = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    return p if os.path.exists(p) else "libamdhip64.so.7"


def _runtime_file(handle):
    """Real path of the file that holds the hipGetDevice this library handle
    resolves (dlsym searches the handle's own dependency scope)."""
    addr = ctypes.cast(handle.hipGetDevice, ctypes.c_void_p).value
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            lo, hi = (int(v, 16) for v in parts[0].split("-"))
            if lo <= addr < hi and len(parts) >= 6:
                return os.path.realpath(parts[5])
    return None


def _load():
    # torch ships its own HIP runtime under the same soname as the system's
    # (libamdhip64.so.7). Importing torch first makes this library bind to
    # that already-loaded runtime, so torch's device memory and streams and
    # this library's kernels live in one HIP context. Loading the library
    # first would pull in a second runtime that sees no device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("libvitblock.so is not built (run vision_transformer_encoder_vit_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    ours, torchs = _runtime_file(lib), _runtime_file(ctypes.CDLL(_torch_runtime_path()))
    if ours is None or ours != torchs:
        raise ImportError("libvitblock.so must share torch's HIP runtime, but it resolved %s while torch uses %s "
                          "(mapped: %s); load torch before anything that links libamdhip64 (this library "
                          "included)" % (ours, torchs, ", ".join(hip_runtimes_mapped())))
    P = ctypes.POINTER
    sig = {
        "vit_block_create": [P(vit_block_desc), P(_vp)],
        "vit_block_workspace_size": [_vp, P(ctypes.c_size_t)],
        "vit_block_forward": [_vp, P(vit_block_weights), _vp, _vp, _vp, ctypes.c_size_t, _vp],
        "vit_block_forward_static": [_vp, P(vit_block_weights), _vp, _vp, _vp],
        "vit_block_forward_seams": [_vp, P(vit_block_weights), _vp, _vp, P(vit_block_seams), _vp,
                                    ctypes.c_size_t, _vp],
        "vit_block_forward_timed": [_vp, P(vit_block_weights), _vp, _vp, _vp, ctypes.c_size_t, _vp,
                                    P(_vp), _i32],
        "vit_block_stage_mask": [_vp, P(ctypes.c_uint32)],
        "vit_block_destroy": [_vp],
        "vit_layernorm": [_vp, _vp, _vp, _vp, ctypes.c_int64, _i32, _f32, _i32, _vp],
        "vit_unroll": [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp],
        "vit_reroll": [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp],
        "vit_pool4": [_vp, ctypes.c_int64, _vp, ctypes.c_int64, _i32, _i32, _i32, _i32, _vp],
        "vit_stack_create": [P(vit_block_desc), _i32, _i32, P(_i32), _i32, P(_vp)],
        "vit_stack_workspace_size": [_vp, P(ctypes.c_size_t)],
        "vit_stack_forward": [_vp, P(vit_block_weights), _vp, P(_vp), _vp, ctypes.c_size_t, _vp],
        "vit_stack_destroy": [_vp],
        "vit_patch_embed_workspace_size": [P(vit_patch_embed_desc), P(ctypes.c_size_t)],
        "vit_patch_embed": [P(vit_patch_embed_desc), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.vit_last_error.argtypes = []
    lib.vit_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def check(status):
    if status != VIT_OK:
        raise VitError(status, lib.vit_last_error().decode())


def last_error():
    return lib.vit_last_error().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def desc_from_spec(spec):
    """vit_block_desc for a workload spec (see synth.CONFIGS)."""
    mode = {"global": VIT_ATTN_GLOBAL, "mask_unit": VIT_ATTN_MASK_UNIT,
            "spatial": VIT_ATTN_SPATIAL}[spec["mode"]]
    n = spec["grid_h"] * spec["grid_w"]
    rope_rows = 0
    if spec.get("rope"):
        rope_rows = spec["win_h"] * spec["win_w"] if spec["mode"] == "spatial" else n
    return vit_block_desc(
        batch=spec["batch"], grid_h=spec["grid_h"], grid_w=spec["grid_w"], dim_in=spec["dim_in"],
        dim_out=spec["dim_out"], heads=spec["heads"], mlp_hidden=spec["mlp"], attn_mode=mode,
        n_windows=spec.get("n_windows", 1), win_h=spec.get("win_h", 0), win_w=spec.get("win_w", 0),
        q_stride=spec["q_stride"],
        gelu=VIT_GELU_ERF if spec["gelu"] == "erf" else VIT_GELU_TANH,
        qkv_layout=VIT_QKV_SEPARATE if spec.get("qkv") == "separate" else VIT_QKV_FUSED,
        rope=VIT_ROPE_AXIAL_TABLE if spec.get("rope") else VIT_ROPE_NONE, rope_rows=rope_rows,
        ln_eps=spec["eps"], attn_scale=spec.get("scale") or 0.0,
        act_dtype=VIT_DTYPE_BF16 if spec["dtype"] == "bf16" else VIT_DTYPE_F32,
        weight_format=VIT_WEIGHTS_Q8_ROW if spec.get("weights") == "q8_row" else VIT_WEIGHTS_ACT)


# names of the synthetic input dict -> vit_block_weights members
WEIGHT_NAMES = {"ln1_g": "ln1_gamma", "ln1_b": "ln1_beta", "res_w": "w_res", "res_b": "b_res",
                "qkv_w": "w_qkv", "qkv_b": "b_qkv", "q_w": "w_q", "q_b": "b_q", "k_w": "w_k",
                "k_b": "b_k", "v_w": "w_v", "v_b": "b_v", "o_w": "w_o", "o_b": "b_o",
                "ln2_g": "ln2_gamma", "ln2_b": "ln2_beta", "fc1_w": "w_fc1", "fc1_b": "b_fc1",
                "fc2_w": "w_fc2", "fc2_b": "b_fc2", "rope": "rope_table", "res_s": "s_res", "qkv_s": "s_qkv",
                "q_s": "s_q", "k_s": "s_k", "v_s": "s_v", "o_s": "s_o", "fc1_s": "s_fc1", "fc2_s": "s_fc2"}


def weights_struct(tensors):
    """vit_block_weights from a dict of device tensors keyed by WEIGHT_NAMES."""
    w = vit_block_weights()
    for k, t in tensors.items():
        if k in WEIGHT_NAMES:
            setattr(w, WEIGHT_NAMES[k], t.data_ptr())
    return w


class Plan:
    """A created vit_block plan (vit_block_create / vit_block_destroy)."""

    def __init__(self, desc):
        self.desc = desc
        h = ctypes.c_void_p()
        check(lib.vit_block_create(ctypes.byref(desc), ctypes.byref(h)))
        self.handle = h
        n = ctypes.c_size_t()
        check(lib.vit_block_workspace_size(h, ctypes.byref(n)))
        self.workspace_bytes = n.value

    def stage_mask(self):
        m = ctypes.c_uint32()
        check(lib.vit_block_stage_mask(self.handle, ctypes.byref(m)))
        return m.value

    def forward(self, weights, x, y, workspace, stream=None):
        check(lib.vit_block_forward(self.handle, ctypes.byref(weights), _ptr(x), _ptr(y),
                                    _ptr(workspace), workspace.numel() * workspace.element_size()
                                    if workspace is not None else 0, _stream(stream)))

    def forward_static(self, weights, x, y, stream=None):
        """vit_block_forward_static: the workspace is the library's own
        device scratch (no allocation; calls on one GPU must not overlap)."""
        check(lib.vit_block_forward_static(self.handle, ctypes.byref(weights), _ptr(x), _ptr(y), _stream(stream)))

    def forward_timed(self, weights, x, y, workspace, events, stream=None):
        """events: a ctypes array of 2 * VIT_NSTAGES hipEvent_t handles."""
        check(lib.vit_block_forward_timed(self.handle, ctypes.byref(weights), _ptr(x), _ptr(y),
                                          _ptr(workspace), workspace.numel() * workspace.element_size()
                                          if workspace is not None else 0, _stream(stream), events,
                                          len(events)))

    def forward_seams(self, weights, x, y, seams, workspace, stream=None):
        s = vit_block_seams()
        for k, t in seams.items():
            setattr(s, k, t.data_ptr())
        check(lib.vit_block_forward_seams(self.handle, ctypes.byref(weights), _ptr(x), _ptr(y),
                                          ctypes.byref(s), _ptr(workspace),
                                          workspace.numel() * workspace.element_size()
                                          if workspace is not None else 0, _stream(stream)))

    def close(self):
        if self.handle is not None:
            lib.vit_block_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Stack:
    """A created vit_stack plan: blocks applied in order to one token grid,
    unrolled once and rerolled after each tap (vit_stack_create)."""

    def __init__(self, descs, unroll_levels, taps):
        arr = (vit_block_desc * len(descs))(*descs)
        t = (_i32 * max(len(taps), 1))(*taps)
        h = ctypes.c_void_p()
        check(lib.vit_stack_create(arr, len(descs), unroll_levels, t, len(taps), ctypes.byref(h)))
        self.handle = h
        self.n_blocks, self.n_taps = len(descs), len(taps)
        n = ctypes.c_size_t()
        check(lib.vit_stack_workspace_size(h, ctypes.byref(n)))
        self.workspace_bytes = n.value

    def forward(self, weights, x, features, workspace, stream=None):
        """weights: list of vit_block_weights (one per block); features: list
        of output tensors (one per tap)."""
        w = (vit_block_weights * self.n_blocks)(*weights)
        f = (_vp * max(self.n_taps, 1))(*[t.data_ptr() for t in features])
        check(lib.vit_stack_forward(self.handle, w, _ptr(x), f, _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))

    def close(self):
        if self.handle is not None:
            lib.vit_stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _dt(t):
    import torch
    if t.dtype == torch.bfloat16:
        return VIT_DTYPE_BF16
    if t.dtype == torch.float32:
        return VIT_DTYPE_F32
    raise TypeError("tensor dtype must be bfloat16 or float32")


def vit_layernorm(x, y, gamma, beta, eps, stream=None):
    dim = x.shape[-1]
    check(lib.vit_layernorm(_ptr(x), _ptr(y), _ptr(gamma), _ptr(beta), x.numel() // dim, dim,
                            eps, _dt(x), _stream(stream)))


def vit_unroll(x, y, grid_h, grid_w, levels, stream=None):
    check(lib.vit_unroll(_ptr(x), _ptr(y), x.shape[0], grid_h, grid_w, levels, x.shape[-1],
                         _dt(x), _stream(stream)))


def vit_reroll(x, y, grid_h, grid_w, levels, stream=None):
    check(lib.vit_reroll(_ptr(x), _ptr(y), x.shape[0], grid_h, grid_w, levels, x.shape[-1],
                         _dt(x), _stream(stream)))


def vit_pool4(x, y, channels=None, stream=None):
    """x [B, tokens, row_stride_x] (the first `channels` columns pooled),
    y [B, tokens/4, row_stride_y]."""
    c = channels or x.shape[-1]
    check(lib.vit_pool4(_ptr(x), x.shape[-1], _ptr(y), y.shape[-1], x.shape[0], x.shape[1], c,
                        _dt(x), _stream(stream)))


_POS = {"none": VIT_POS_NONE, "rows": VIT_POS_ROWS, "bucket": VIT_POS_BUCKET, "tile": VIT_POS_TILE}


def stem_desc_from_spec(spec):
    """vit_patch_embed_desc of a stem spec (as the input generator writes them)."""
    return vit_patch_embed_desc(
        batch=spec["batch"], in_h=spec["in_h"], in_w=spec["in_w"], in_ch=spec["in_ch"],
        pixel_layout=VIT_PIXELS_NHWC if spec["layout"] == "nhwc" else VIT_PIXELS_NCHW,
        kernel=spec["kernel"], stride=spec["stride"], pad=spec["pad"], dim=spec["dim"],
        weight_layout=VIT_CONV_OHWI if spec["weight_layout"] == "ohwi" else VIT_CONV_OIHW,
        pos_mode=_POS[spec["pos_mode"]], pos_side=spec["pos_side"],
        act_dtype=VIT_DTYPE_BF16 if spec["dtype"] == "bf16" else VIT_DTYPE_F32)


def vit_patch_embed_workspace_size(desc):
    n = ctypes.c_size_t()
    check(lib.vit_patch_embed_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def vit_patch_embed(desc, pixels, weight, bias, pos, tokens, workspace, stream=None):
    check(lib.vit_patch_embed(ctypes.byref(desc), _ptr(pixels), _ptr(weight), _ptr(bias), _ptr(pos), _ptr(tokens),
                              _ptr(workspace), workspace.numel() * workspace.element_size()
                              if workspace is not None else 0, _stream(stream)))
