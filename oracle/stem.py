"""Patch-embedding stems, float64 numpy oracle (test infrastructure: only
tests/, the smoke check and the benchmark's CPU baseline may import it).

A stem turns pixels into the token grid the blocks consume: a strided
convolution with kernel k, stride s and zero padding p, its output flattened
in raster order (token t = y * out_w + x, one row of `dim` channels per
token), then a learned position table added row by row:

  out[b, y*out_w + x, o] = bias[o]
      + sum_{c, ky, kx} w[o, c, ky, kx] * P[b, c, y*s + ky - p, x*s + kx - p]
      + pos[row(y, x), o]                 (P = 0 outside the image)

Position rows, per stem:
  rows   -- row t (Hiera plan: a learned (1, N, C) table, interpolated to the
            token count at load time, added after the patch embedding)
  bucket -- row b(y) * side + b(x) with b(i) = max(i - 1, 0) (SigLIP page,
            ``embed_frame``: the NaViT bucketize at the full-mask geometry
            puts coordinates 0 and 1 in bucket 0 and never uses bucket 31)
  tile   -- row (y mod side) * side + (x mod side) (SAM3 page, trunk: the
            24 x 24 table repeated over the 72 x 72 grid)

Pixel layouts NCHW (SigLIP, SAM3) and NHWC (Hiera, channels last at the
boundary); weight layouts OIHW (SigLIP and SAM3 checkpoints) and OHWI (the
Hiera converter's transposed form).

Pins (tests/test_oracle.py): torch's conv2d in float64 on both layouts;
a one-hot weight selects exactly the pixel the definition names; the shape
contracts (512 -> 128 x 128 Hiera tokens, 512 -> 32 x 32 SigLIP, 1008 ->
72 x 72 SAM3); the SigLIP buckets against the page's printed bucket list and
against the bucketize procedure the page describes; the SAM3 table tiling.
"""
import numpy as np


def to_nchw(pixels, layout):
    p = np.asarray(pixels, dtype=np.float64)
    return p if layout == "nchw" else p.transpose(0, 3, 1, 2)


def weight_oihw(weight, layout):
    w = np.asarray(weight, dtype=np.float64)
    return w if layout == "oihw" else w.transpose(0, 3, 1, 2)


def conv2d(P, w, stride, pad):
    """P [B, C, H, W], w [O, C, k, k] -> [B, O, out_h, out_w]: the sum over
    kernel offsets (ky, kx) of the strided pixel slices times w[:, :, ky, kx]."""
    B, C, H, W = P.shape
    O, _, k, _ = w.shape
    oh, ow = (H + 2 * pad - k) // stride + 1, (W + 2 * pad - k) // stride + 1
    Pp = np.zeros((B, C, H + 2 * pad, W + 2 * pad))
    Pp[:, :, pad:pad + H, pad:pad + W] = P
    out = np.zeros((B, O, oh, ow))
    for ky in range(k):
        for kx in range(k):
            sl = Pp[:, :, ky:ky + stride * (oh - 1) + 1:stride, kx:kx + stride * (ow - 1) + 1:stride]
            out += np.einsum("bchw,oc->bohw", sl, w[:, :, ky, kx])
    return out


def pos_rows(out_h, out_w, mode, side):
    """Table row of every token (raster order)."""
    y, x = np.divmod(np.arange(out_h * out_w), out_w)
    if mode == "rows":
        return y * out_w + x
    if mode == "bucket":
        return np.maximum(y - 1, 0) * side + np.maximum(x - 1, 0)
    if mode == "tile":
        return (y % side) * side + (x % side)
    raise ValueError(mode)


def patch_embed(inputs, spec):
    """inputs: dict with pixels, weight, optional bias and pos (as drawn by
    the input generator); returns tokens [B, out_h*out_w, dim] in float64."""
    P = to_nchw(inputs["pixels"], spec["layout"])
    w = weight_oihw(inputs["weight"], spec["weight_layout"])
    y = conv2d(P, w, spec["stride"], spec["pad"])
    B, O, oh, ow = y.shape
    t = y.reshape(B, O, oh * ow).transpose(0, 2, 1)
    if inputs.get("bias") is not None:
        t = t + np.asarray(inputs["bias"], dtype=np.float64)
    if spec["pos_mode"] != "none":
        t = t + np.asarray(inputs["pos"], dtype=np.float64)[pos_rows(oh, ow, spec["pos_mode"], spec["pos_side"])]
    return t
